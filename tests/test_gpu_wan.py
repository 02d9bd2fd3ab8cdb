"""Parity at the full Wan attention shapes, in the launch configuration the
benchmark times (all heads of the workload in one call).

The whole output is computed on the GPU; the oracle recomputes sampled query
blocks one by one (first, middle, ragged last and one random block of three
heads) and the whole selection and INT8 codes of those heads.  The bf16 output
that the benchmark times must equal the round-to-nearest-even of the fp32
output everywhere that is checked.
"""
import numpy as np
import pytest

from oracle import sla_oracle as O
from sparse_linear_attention_sagesla_amd.inputs import WORKLOADS, make_inputs

from gpu_util import assert_parity, bf16_bits_of, errors, rne_bf16, selection_mismatches, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sla = pytest.importorskip("sparse_linear_attention_sagesla_amd")

_cache = {}


def _inputs(name):
    if name not in _cache:
        _cache.clear()
        print(f"[case] generating {name}", flush=True)
        Q, K, V = make_inputs(name)
        _cache[name] = (Q, K, V, to_dev(Q), to_dev(K), to_dev(V))
    return _cache[name]


def _sample_blocks(nb, seed):
    rng = np.random.default_rng(seed)
    return sorted({0, nb // 2, nb - 1, int(rng.integers(1, nb - 1))})


CASES = [("wan13b480", 0.10, "elu1"), ("wan14b480", 0.10, "elu1"), ("wan14b720", 0.10, "elu1"),
         ("sweep", 0.0, "elu1"), ("sweep", 0.05, "elu1"), ("sweep", 0.20, "elu1"),
         ("sweep", 1.0, "none")]


@pytest.mark.parametrize("name,keep,phi", CASES)
def test_wan_sampled_parity(name, keep, phi):
    wl = WORKLOADS[name]
    Q, K, V, q, k, v = _inputs(name)
    print(f"[case] {name} keep={keep} phi={phi} shape={tuple(q.shape)}", flush=True)
    out32, lin = sla.attention(q, k, v, keep, phi, torch.float32, return_linear=True)
    out16 = sla.attention(q, k, v, keep, phi, torch.bfloat16)
    torch.cuda.synchronize()
    nb = O.n_blocks(wl.N, 64)
    heads = sorted({0, wl.H // 2, wl.H - 1})
    for h in heads:
        blocks = _sample_blocks(nb, 100 * h + int(keep * 100))
        r = O.sla_forward_head(Q[0, h], K[0, h], V[0, h], 64, keep, phi, query_blocks=blocks)
        rows = torch.from_numpy(r["rows"]).cuda()
        got = out32[0, h].index_select(0, rows).cpu().numpy()
        assert_parity(got, r["out"], what=f"{name} keep={keep} h{h} blocks {blocks}")
        gl = lin[0, h].index_select(0, rows).cpu().numpy()
        ma, rel = errors(gl, r["out_linear"])
        print(f"[parity] linear branch: max-abs {ma:.3e} rel-L2 {rel:.3e} "
              f"(|O_l| max {np.abs(r['out_linear']).max():.3e})", flush=True)
        assert ma <= 2e-4 + 1e-3 * np.abs(r["out_linear"]).max()
        got16 = bf16_bits_of(out16[0, h].index_select(0, rows))
        assert np.array_equal(got16, rne_bf16(got))


@pytest.mark.parametrize("name", ["wan13b480", "wan14b720", "sweep"])
def test_wan_selection_and_codes_bit_exact(name):
    wl = WORKLOADS[name]
    Q, K, V, q, k, v = _inputs(name)
    keep = 0.05 if name == "sweep" else 0.10
    idx = sla.block_select(q, k, keep).cpu().numpy()
    q8, k8, sq, sk, mu = sla.quantize_qk(q, k)
    nb = O.n_blocks(wl.N, 64)
    kk = O.topk_count(nb, keep)
    for h in (0, wl.H - 1):
        oidx, s = O.select_head(Q[0, h], K[0, h], 64, keep)
        rows, excused, bad = selection_mismatches(idx[0, h], oidx, s, kk)
        print(f"[select] {name} h{h}: rows differing {rows}, near-ties {excused}, other {bad}")
        assert bad == 0
        assert np.array_equal(idx[0, h], oidx)
        oq8, ok8, osq, osk, omu = O.quantize_qk(Q[0, h], K[0, h], 64)
        assert np.array_equal(q8[0, h].cpu().numpy(), oq8)
        assert np.array_equal(k8[0, h].cpu().numpy(), ok8)
        assert np.array_equal(sq[0, h].cpu().numpy(), osq)
        assert np.array_equal(sk[0, h].cpu().numpy(), osk)
        assert np.array_equal(mu[0, h].cpu().numpy(), omu)


def test_wan_int8_accumulators_sampled():
    """Integer tiles of the GPU codes against the oracle's integer product of
    the oracle's own codes (the codes themselves must agree bit for bit)."""
    name = "wan14b720"
    wl = WORKLOADS[name]
    Q, K, V, q, k, v = _inputs(name)
    q8, k8, *_ = sla.quantize_qk(q, k)
    nb = O.n_blocks(wl.N, 64)
    rng = np.random.default_rng(9)
    heads = [0, 17, wl.H - 1]
    codes = {}
    for h in heads:
        oq8, ok8, *_ = O.quantize_qk(Q[0, h], K[0, h], 64)
        assert np.array_equal(q8[0, h].cpu().numpy(), oq8)
        assert np.array_equal(k8[0, h].cpu().numpy(), ok8)
        codes[h] = (oq8, ok8)
    P = 3000
    pairs = np.stack([np.zeros(P, np.int32), rng.choice(heads, P), rng.integers(0, nb, P),
                      rng.integers(0, nb, P)], axis=1).astype(np.int32)
    pairs[:8, 2] = nb - 1                       # the ragged tail block, both roles
    pairs[8:16, 3] = nb - 1
    acc = sla.debug_qk_i32(q8, k8, wl.N, torch.from_numpy(pairs)).cpu().numpy()
    for p, (_, h, i, j) in enumerate(pairs):
        want = O.qk_accumulator(codes[h][0], codes[h][1], i, j, 64)
        assert np.array_equal(acc[p], want), f"tile (h={h}, i={i}, j={j})"
