"""Parity of the HIP path (through the C ABI) against the fp64 CPU oracle.

Bit-exact: INT8 codes, block scales, the K mean, integer Q.K^T tiles and the
key-block selection (near-ties counted).  Floating point: the fp32 output
within max-abs 2e-3 and rel-L2 1e-3 of the oracle; bf16 output equal to the
round-to-nearest-even of the fp32 output.
"""
import numpy as np
import pytest

from oracle import sla_oracle as O
from sparse_linear_attention_sagesla_amd.inputs import WORKLOADS, make_inputs, random_bf16

from gpu_util import (ATOL, REL_L2, assert_parity, bf16_bits_of, errors, rne_bf16,
                      selection_mismatches, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sla = pytest.importorskip("sparse_linear_attention_sagesla_amd")


def _case(name, Q, K, V):
    print(f"[case] {name} shape={tuple(Q.shape)}", flush=True)
    return to_dev(Q), to_dev(K), to_dev(V)


@pytest.fixture(scope="module")
def tiny():
    Q, K, V = make_inputs("tiny")
    return Q, K, V


# ---------------------------------------------------------------- quantiser
@pytest.mark.parametrize("N", [2048, 2000, 1, 65, 127])
def test_quantize_bit_exact(tiny, N):
    Q, K, V = tiny
    Q, K = Q[:, :, :N], K[:, :, :N]
    q, k, _ = _case(f"quantize N={N}", Q, K, V[:, :, :N])
    q8, k8, sq, sk, mu = (x.cpu().numpy() for x in sla.quantize_qk(q, k))
    for h in range(Q.shape[1]):
        oq8, ok8, osq, osk, omu = O.quantize_qk(Q[0, h], K[0, h], 64)
        assert np.array_equal(mu[0, h].view(np.uint32), omu.view(np.uint32))
        assert np.array_equal(sq[0, h].view(np.uint32), osq.view(np.uint32))
        assert np.array_equal(sk[0, h].view(np.uint32), osk.view(np.uint32))
        assert np.array_equal(q8[0, h], oq8)
        assert np.array_equal(k8[0, h], ok8)


def test_quantize_zero_block_and_outliers():
    N = 256
    Q = random_bf16((1, 1, N, 128), 5)
    K = random_bf16((1, 1, N, 128), 6, offset=3.0)
    Q[0, 0, 64:128] = 0                       # an all-zero block: scale 0, codes 0
    K[0, 0, :, 7] = random_bf16((N,), 7, scale=40.0)   # one large channel
    q, k, _ = _case("quantize zero block", Q, K, K)
    q8, k8, sq, sk, mu = (x.cpu().numpy() for x in sla.quantize_qk(q, k))
    oq8, ok8, osq, osk, omu = O.quantize_qk(Q[0, 0], K[0, 0], 64)
    assert sq[0, 0, 1] == 0 and not q8[0, 0, 64:128].any()
    assert np.array_equal(q8[0, 0], oq8) and np.array_equal(k8[0, 0], ok8)
    assert np.array_equal(sq[0, 0], osq) and np.array_equal(sk[0, 0], osk)
    assert np.array_equal(mu[0, 0], omu)


# ---------------------------------------------------------------- selection
@pytest.mark.parametrize("N,keep", [(2048, 0.1), (2048, 0.5), (2048, 1.0), (2000, 0.1),
                                    (1, 0.1), (4160, 0.03), (2048, 1e-6)])
def test_block_select_matches_oracle(tiny, N, keep):
    Q, K, V = tiny
    if N > 2048:
        Q = random_bf16((1, 2, N, 128), 8)
        K = random_bf16((1, 2, N, 128), 9)
    Q, K = Q[:, :, :N], K[:, :, :N]
    q, k, _ = _case(f"select N={N} keep={keep}", Q, K, K)
    idx, mask = sla.block_select(q, k, keep, with_mask=True)
    idx, mask = idx.cpu().numpy(), mask.cpu().numpy().view(np.uint32)
    nb = O.n_blocks(N, 64)
    kk = O.topk_count(nb, keep)
    for h in range(Q.shape[1]):
        oidx, s = O.select_head(Q[0, h], K[0, h], 64, keep)
        rows, excused, bad = selection_mismatches(idx[0, h], oidx, s, kk)
        print(f"[select] head {h}: rows differing {rows}, near-ties {excused}, other {bad}")
        assert bad == 0
        assert np.array_equal(idx[0, h], oidx)          # fp64 scores agree bit for bit
        assert (np.diff(idx[0, h], axis=1) > 0).all()
        bits = np.unpackbits(mask[0, h].view(np.uint8), bitorder="little", axis=1)[:, :nb]
        assert np.array_equal(bits.astype(bool), O.block_mask(oidx, nb))


def test_block_select_exact_ties_keep_lower_index():
    N = 64 * 16
    Q = random_bf16((1, 1, N, 128), 10, offset=0.25)
    K = random_bf16((1, 1, N, 128), 11)
    for dup in (3, 7, 12):
        K[0, 0, dup * 64:(dup + 1) * 64] = K[0, 0, 64:128]   # blocks 3, 7, 12 == block 1
    q, k, _ = _case("select exact ties", Q, K, K)
    for keep in (1 / 16, 3 / 16, 0.5):
        idx = sla.block_select(q, k, keep).cpu().numpy()
        oidx, _ = O.select_head(Q[0, 0], K[0, 0], 64, keep)
        assert np.array_equal(idx[0, 0], oidx)
    Qz = np.zeros_like(Q)                                    # all scores tie at 0
    qz, _, _ = _case("select all-zero queries", Qz, K, K)
    idx = sla.block_select(qz, k, 0.25).cpu().numpy()
    assert (idx[0, 0] == np.arange(4)).all()


@pytest.mark.parametrize("keep,phi", [(0.1, "elu1"), (0.3, "relu")])
def test_rows_handed_back_to_the_exact_selection(keep, phi):
    """Query blocks whose Q is zero score every key block 0; the filtered
    top-k hands such rows to the exact kernel (which keeps the lowest
    indices) while the rows around them stay with the filter.  Checked through
    the selection, the forward (whose walk schedule is built from the filter's
    lists before those rows are redone, then rebuilt) and the forked forward."""
    N = 64 * 40 - 11
    Q, K, V = (random_bf16((1, 2, N, 128), s) for s in (41, 42, 43))
    zero = {0: (5, 17, 39), 1: (0, 2, 3, 30)}   # block 39 is the ragged last one
    for h, blocks in zero.items():
        for i in blocks:
            Q[0, h, 64 * i:64 * (i + 1)] = 0
    q, k, v = _case(f"handed-back rows keep={keep} {phi}", Q, K, V)
    idx = sla.block_select(q, k, keep).cpu().numpy()
    out = sla.attention(q, k, v, keep, phi, torch.float32).cpu().numpy()
    side = torch.cuda.Stream()
    outf = sla.attention(q, k, v, keep, phi, torch.float32, side_stream=side)
    torch.cuda.synchronize()
    assert np.array_equal(outf.cpu().numpy(), out)
    kk = O.topk_count(O.n_blocks(N, 64), keep)
    for h in range(2):
        oidx, _ = O.select_head(Q[0, h], K[0, h], 64, keep)
        assert np.array_equal(idx[0, h], oidx)
        for i in zero[h]:
            assert (oidx[i] == np.arange(kk)).all()
        r = O.sla_forward_head(Q[0, h], K[0, h], V[0, h], 64, keep, phi)
        assert_parity(out[0, h], r["out"], what=f"handed-back rows h{h}")


# --------------------------------------------------------- integer QK tiles
def test_int8_accumulators_bit_exact_all_tiles(tiny):
    """Every integer tile of the tiny workload against the oracle's integer
    product of the oracle's own codes."""
    Q, K, _ = tiny
    q, k, _ = _case("debug qk", Q, K, K)
    q8, k8, *_ = sla.quantize_qk(q, k)
    nb = 32
    pairs = np.array([(0, h, i, j) for h in range(2) for i in range(nb) for j in range(nb)], np.int32)
    acc = sla.debug_qk_i32(q8, k8, 2048, torch.from_numpy(pairs)).cpu().numpy()
    codes = [O.quantize_qk(Q[0, h], K[0, h], 64)[:2] for h in range(2)]
    for p, (_, h, i, j) in enumerate(pairs):
        want = O.qk_accumulator(codes[h][0], codes[h][1], i, j, 64)
        assert np.array_equal(acc[p], want), f"tile (h={h}, i={i}, j={j})"


# ---------------------------------------------------------------- forward
def _oracle_out(Q, K, V, keep, phi, h, blocks=None):
    return O.sla_forward_head(Q[0, h], K[0, h], V[0, h], 64, keep, phi, query_blocks=blocks)


@pytest.mark.parametrize("keep,phi", [(0.1, "elu1"), (0.1, "none"), (1.0, "none"),
                                      (0.0, "elu1"), (0.0, "relu"), (0.2, "relu"),
                                      (0.5, "elu1"), (1.0, "elu1")])
def test_attention_parity_tiny(tiny, keep, phi):
    Q, K, V = tiny
    q, k, v = _case(f"attention tiny keep={keep} phi={phi}", Q, K, V)
    out, lin = sla.attention(q, k, v, keep, phi, torch.float32, return_linear=True)
    outb = sla.attention(q, k, v, keep, phi, torch.bfloat16)
    out, lin = out.cpu().numpy(), lin.cpu().numpy()
    for h in range(2):
        r = _oracle_out(Q, K, V, keep, phi, h)
        assert_parity(out[0, h], r["out"], what=f"h{h} out")
        if phi != "none":
            scale = max(np.abs(r["out_linear"]).max(), 1e-30)
            ma, rel = errors(lin[0, h], r["out_linear"])
            print(f"[parity] h{h} linear: max-abs {ma:.3e} (|O_l| max {scale:.3e}) rel-L2 {rel:.3e}")
            assert ma <= 1e-3 * scale + 1e-6 and rel <= 1e-3
    assert np.array_equal(bf16_bits_of(outb), rne_bf16(out))


@pytest.mark.parametrize("N", [2000, 1000, 64, 65, 1])
def test_attention_parity_ragged(N):
    Q, K, V = (random_bf16((1, 2, N, 128), s, scale=1.5) for s in (21, 22, 23))
    q, k, v = _case(f"attention ragged N={N}", Q, K, V)
    for keep, phi in ((0.1, "elu1"), (0.3, "none"), (0.0, "elu1")):
        out, lin = sla.attention(q, k, v, keep, phi, torch.float32, return_linear=True)
        out, lin = out.cpu().numpy(), lin.cpu().numpy()
        for h in range(2):
            r = _oracle_out(Q, K, V, keep, phi, h)
            assert_parity(out[0, h], r["out"], what=f"N={N} keep={keep} {phi} h{h}")
            assert np.isfinite(out).all()


def test_linear_branch_with_structured_values():
    """V correlated with K makes the kept blocks' share of the linear branch
    large, so a wrong subtraction of the kept blocks would show."""
    wl = WORKLOADS["tiny"]
    Q, K, _ = make_inputs(wl)
    from sparse_linear_attention_sagesla_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits
    V = f32_to_bf16_bits(np.tanh(bf16_bits_to_f32(K)) + np.float32(1.0))
    q, k, v = _case("structured V", Q, K, V)
    for keep, phi in ((0.1, "elu1"), (0.25, "relu"), (0.6, "elu1")):
        out, lin = sla.attention(q, k, v, keep, phi, torch.float32, return_linear=True)
        out, lin = out.cpu().numpy(), lin.cpu().numpy()
        for h in range(2):
            r = _oracle_out(Q, K, V, keep, phi, h)
            assert_parity(out[0, h], r["out"], what=f"structured keep={keep} {phi} h{h}")
            assert_parity(lin[0, h], r["out_linear"], atol=1e-3, rel_l2=1e-3,
                          what=f"structured linear keep={keep} {phi} h{h}")


def test_small_magnitude_values(tiny):
    """V of magnitude 1e-4 (most entries below fp16's normal range once
    staged): the staging keeps an absolute precision of 2^-25, far below the
    output's scale, so the relative bar still holds."""
    from sparse_linear_attention_sagesla_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits
    Q, K, V = tiny
    V = f32_to_bf16_bits(bf16_bits_to_f32(V) * np.float32(1e-4))
    q, k, v = _case("small V", Q, K, V)
    for keep, phi in ((0.1, "elu1"), (1.0, "none")):
        out = sla.attention(q, k, v, keep, phi, torch.float32).cpu().numpy()
        for h in range(2):
            r = _oracle_out(Q, K, V, keep, phi, h)
            assert_parity(out[0, h], r["out"], atol=2e-7, what=f"small V keep={keep} {phi} h{h}")


def test_attention_deterministic(tiny):
    Q, K, V = tiny
    q, k, v = _case("determinism", Q, K, V)
    a = sla.attention(q, k, v, 0.1, "elu1", torch.float32)
    b = sla.attention(q, k, v, 0.1, "elu1", torch.float32)
    assert torch.equal(a, b)


def test_batched_heads_match_single_calls():
    B, H, N = 2, 3, 640
    Q, K, V = (random_bf16((B, H, N, 128), s) for s in (31, 32, 33))
    q, k, v = _case("batch", Q, K, V)
    out = sla.attention(q, k, v, 0.2, "elu1", torch.float32).cpu().numpy()
    for b in range(B):
        for h in range(H):
            r = O.sla_forward_head(Q[b, h], K[b, h], V[b, h], 64, 0.2, "elu1")
            assert_parity(out[b, h], r["out"], what=f"b{b} h{h}")


def _sweep_configs(n=12, seed=2024):
    """Seeded mixed configurations: batch and head counts, ragged lengths from one
    token to a few thousand, keep fractions from 0 to 1 crossed with every
    feature map (keep 0 only with a feature map: without one nothing is
    computed), input scales and a channel offset (exercising the K mean
    smoothing)."""
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        out.append(dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)),
                        N=int(rng.integers(1, 2601)),
                        keep=(0.0, 0.03, 0.1, 0.37, 0.8, 1.0)[c % 6],
                        phi=("elu1", "relu", "none")[(c + c // 6) % 3],
                        scale=float(rng.choice([0.5, 1.5, 3.0])),
                        offset=float(rng.choice([0.0, 2.0])), seed=100 + 3 * c))
    return out


@pytest.mark.parametrize("cfg", _sweep_configs(), ids=lambda c: f"B{c['B']}H{c['H']}N{c['N']}k{c['keep']}{c['phi']}")
def test_attention_parity_config_sweep(cfg):
    B, H, N = cfg["B"], cfg["H"], cfg["N"]
    Q, K, V = (random_bf16((B, H, N, 128), cfg["seed"] + i, scale=cfg["scale"],
                           offset=cfg["offset"] if i < 2 else 0.0) for i in range(3))
    q, k, v = _case(f"sweep {cfg}", Q, K, V)
    out = sla.attention(q, k, v, cfg["keep"], cfg["phi"], torch.float32)
    outb = sla.attention(q, k, v, cfg["keep"], cfg["phi"], torch.bfloat16)
    out = out.cpu().numpy()
    assert np.isfinite(out).all()
    for b in range(B):
        for h in range(H):
            r = O.sla_forward_head(Q[b, h], K[b, h], V[b, h], 64, cfg["keep"], cfg["phi"])
            assert_parity(out[b, h], r["out"], what=f"b{b} h{h}")
    assert np.array_equal(bf16_bits_of(outb), rne_bf16(out))
