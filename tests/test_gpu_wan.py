"""Parity at the full Wan attention shapes, in the launch configuration the
benchmark times (all heads of the workload in one call).

The whole output is computed on the GPU and must be finite everywhere; the
oracle recomputes at least 32 sampled query blocks spread over every head
(first, middle, ragged last and random blocks), the selection of every head,
and the INT8 codes of four heads, whose integer Q.K^T tiles are compared on
10^4 sampled (query block, key block) pairs per workload.  The bf16 output
that the benchmark times must equal the round-to-nearest-even of the fp32
output everywhere that is checked.  The oracle runs in a pool of worker
processes, each regenerating its head from the seeded generator.
"""
import numpy as np
import pytest

from oracle import sla_oracle as O
from sparse_linear_attention_sagesla_amd.inputs import WORKLOADS, make_inputs

import oracle_jobs
from gpu_util import assert_parity, bf16_bits_of, errors, oracle_pool, rne_bf16, to_dev

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


@pytest.fixture(scope="module")
def pool():
    ex, _ = oracle_pool()
    yield ex
    ex.shutdown()


def _sample(nb, H, seed, at_least=32):
    """{head: query blocks}, at least `at_least` blocks over all H heads: the
    heads take in turn the first, middle, ragged last or a seeded random block,
    and seeded random ones make up the rest."""
    rng = np.random.default_rng(seed)
    per = -(-at_least // H)
    out = {}
    for h in range(H):
        picks = {(0, nb // 2, nb - 1, int(rng.integers(1, nb - 1)))[h % 4]}
        while len(picks) < per:
            picks.add(int(rng.integers(0, nb)))
        out[h] = sorted(picks)
    return out


CASES = [("wan13b480", 0.10, "elu1"), ("wan14b480", 0.10, "elu1"), ("wan14b720", 0.10, "elu1"),
         ("sweep", 0.0, "elu1"), ("sweep", 0.05, "elu1"), ("sweep", 0.20, "elu1"),
         ("sweep", 1.0, "none")]


@pytest.mark.parametrize("name,keep,phi", CASES)
def test_wan_sampled_parity(pool, name, keep, phi):
    wl = WORKLOADS[name]
    Q, K, V, q, k, v = _inputs(name)
    print(f"[case] {name} keep={keep} phi={phi} shape={tuple(q.shape)}", flush=True)
    nb = O.n_blocks(wl.N, 64)
    sample = _sample(nb, wl.H, 7 + int(keep * 100))
    jobs = pool.map(oracle_jobs.sampled_blocks,
                    [(name, h, keep, phi, b) for h, b in sample.items()])
    out32, lin = sla.attention(q, k, v, keep, phi, torch.float32, return_linear=True)
    out16 = sla.attention(q, k, v, keep, phi, torch.bfloat16)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out32).all()) and bool(torch.isfinite(out16).all())
    got, want, glin, wlin, nblocks = [], [], [], [], 0
    for h, r in jobs:
        rows = torch.from_numpy(r["rows"]).cuda()
        g = out32[0, h].index_select(0, rows).cpu().numpy()
        got.append(g)
        want.append(r["out"])
        glin.append(lin[0, h].index_select(0, rows).cpu().numpy())
        wlin.append(r["out_linear"])
        assert np.array_equal(bf16_bits_of(out16[0, h].index_select(0, rows)), rne_bf16(g))
        nblocks += len(sample[h])
    assert nblocks >= 32
    assert_parity(np.concatenate(got), np.concatenate(want),
                  what=f"{name} keep={keep}: {nblocks} query blocks over {wl.H} heads")
    ma, rel = errors(np.concatenate(glin), np.concatenate(wlin))
    lmax = max(float(np.abs(w).max()) for w in wlin)
    print(f"[parity] linear branch: max-abs {ma:.3e} rel-L2 {rel:.3e} (|O_l| max {lmax:.3e})",
          flush=True)
    assert ma <= 2e-4 + 1e-3 * lmax


SELECT = [("wan13b480", 0.10), ("wan14b480", 0.10), ("wan14b720", 0.10), ("sweep", 0.05)]


@pytest.mark.parametrize("name,keep", SELECT)
def test_wan_selection_and_codes_bit_exact(pool, name, keep):
    """The selection of every head (R6 near-ties counted, none expected) and
    the codes, scales and K mean of four heads, bit for bit."""
    wl = WORKLOADS[name]
    Q, K, V, q, k, v = _inputs(name)
    idx = sla.block_select(q, k, keep).cpu().numpy()
    res = list(pool.map(oracle_jobs.selection_against,
                        [(name, h, keep, idx[0, h]) for h in range(wl.H)]))
    rows = sum(r[1] for r in res)
    excused = sum(r[2] for r in res)
    bad = sum(r[3] for r in res)
    print(f"[select] {name}: {wl.H} heads, rows differing {rows}, near-ties {excused}, "
          f"other {bad}", flush=True)
    assert bad == 0
    assert all(r[4] for r in res)
    q8, k8, sq, sk, mu = (x.cpu().numpy() for x in sla.quantize_qk(q, k))
    heads = sorted({0, wl.H // 3, 2 * wl.H // 3, wl.H - 1})
    for h, oq8, ok8, osq, osk, omu in pool.map(oracle_jobs.codes, [(name, h) for h in heads]):
        assert np.array_equal(q8[0, h], oq8) and np.array_equal(k8[0, h], ok8)
        assert np.array_equal(sq[0, h].view(np.uint32), osq.view(np.uint32))
        assert np.array_equal(sk[0, h].view(np.uint32), osk.view(np.uint32))
        assert np.array_equal(mu[0, h].view(np.uint32), omu.view(np.uint32))


@pytest.mark.parametrize("name", ["wan13b480", "wan14b480", "wan14b720", "sweep"])
def test_wan_int8_accumulators_sampled(pool, name):
    """10^4 integer tiles of the GPU codes, through the attention kernel's
    INT8 matrix-core path, against the exact integer product of the oracle's
    codes (which must equal the GPU's bit for bit)."""
    wl = WORKLOADS[name]
    Q, K, V, q, k, v = _inputs(name)
    q8, k8, *_ = sla.quantize_qk(q, k)
    nb = O.n_blocks(wl.N, 64)
    heads = sorted({0, wl.H // 3, 2 * wl.H // 3, wl.H - 1})
    codes = {}
    for h, oq8, ok8, *_ in pool.map(oracle_jobs.codes, [(name, h) for h in heads]):
        assert np.array_equal(q8[0, h].cpu().numpy(), oq8)
        assert np.array_equal(k8[0, h].cpu().numpy(), ok8)
        codes[h] = (oq8, ok8)
    rng = np.random.default_rng(9)
    P = 10000
    pairs = np.stack([np.zeros(P, np.int32), rng.choice(heads, P), rng.integers(0, nb, P),
                      rng.integers(0, nb, P)], axis=1).astype(np.int32)
    pairs[:8, 2] = nb - 1                       # the ragged tail block, both roles
    pairs[8:16, 3] = nb - 1
    acc = sla.debug_qk_i32(q8, k8, wl.N, torch.from_numpy(pairs)).cpu().numpy()
    for p, (_, h, i, j) in enumerate(pairs):
        want = O.qk_accumulator(codes[h][0], codes[h][1], i, j, 64)
        assert np.array_equal(acc[p], want), f"tile (h={h}, i={i}, j={j})"
    print(f"[tiles] {name}: {P} tiles bit-exact", flush=True)
