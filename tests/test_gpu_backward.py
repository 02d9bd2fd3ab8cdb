"""Parity of the backward (sla_attention_bwd, through the C ABI) against the
fp64 oracle's sla_backward_head, on seeded inputs spanning several tiles with
a ragged last block.

Tolerance, from the arithmetic: every product on the GPU side has bf16
operands (the inputs are bf16 already; P, dS, phi(Q)/den, phi(K) and G - W
are rounded once, unit roundoff u = 2^-9) and fp32 accumulation; P also
carries the forward's fp16 rounding (2^-11).  A gradient entry is a sum of
such products, so its error is about u times the sum of the absolute values
of its terms (one rounding dominates: the bf16 P or dS); softmax-gradient
rows sum to zero, so those sums can exceed the entry itself.  The bound used
is rel-L2 <= 4u = 7.8e-3 (per tensor) and max-abs <= 8u times the tensor's
largest entry, plus an absolute floor of 1e-5 for tensors that vanish
exactly (one token: its softmax gradient cancels to zero in exact arithmetic,
to ~1e-7 in fp32).  Measured: rel-L2 1.3e-3 to 3.1e-3, max-abs at most 2.1u
of the largest entry.
"""
import numpy as np
import pytest

from oracle import sla_oracle as O
from sparse_linear_attention_sagesla_amd.inputs import make_dout, make_inputs, random_bf16

import oracle_jobs
from gpu_util import errors, oracle_pool, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sla = pytest.importorskip("sparse_linear_attention_sagesla_amd")

U_BF16 = 2.0 ** -9
REL = 4 * U_BF16
MAXREL = 8 * U_BF16


ATOL_FLOOR = 1e-5


def _check(name, got, want):
    max_abs, rel = errors(got, want)
    scale = float(np.abs(want).max())
    print(f"[bwd] {name}: max-abs {max_abs:.3e} (max |ref| {scale:.3e}) rel-L2 {rel:.3e}", flush=True)
    bound = MAXREL * scale + ATOL_FLOOR
    assert max_abs <= bound, f"{name}: max-abs {max_abs:.3e} > {bound:.3e}"
    if scale > ATOL_FLOOR:
        assert rel <= REL, f"{name}: rel-L2 {rel:.3e} > {REL:.3e}"


def _run(Q, K, V, G, keep, phi, grad_dtype=torch.float32):
    print(f"[case] bwd shape={tuple(Q.shape)} keep={keep} phi={phi}", flush=True)
    q, k, v, g = (to_dev(x) for x in (Q, K, V, G))
    dq, dk, dv = sla.attention_bwd(q, k, v, g, keep=keep, phi=phi, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return [x.float().cpu().numpy() for x in (dq, dk, dv)]


def _compare(Q, K, V, G, keep, phi, tag):
    got = _run(Q, K, V, G, keep, phi)
    for b in range(Q.shape[0]):
        for h in range(Q.shape[1]):
            r = O.sla_backward_head(Q[b, h], K[b, h], V[b, h], G[b, h], block=64, keep=keep,
                                    phi_kind=phi)
            for i, name in enumerate(("dq", "dk", "dv")):
                _check(f"{tag} b{b} h{h} {name}", got[i][b, h], r[name])


@pytest.mark.parametrize("keep,phi", [(0.3, "elu1"), (0.3, "relu"), (0.3, "none"),
                                      (0.0, "elu1"), (1.0, "elu1"), (0.6, "elu1")])
def test_backward_parity_ragged(keep, phi):
    N = 64 * 9 - 23  # nine blocks, the last with 41 rows
    Q, K, V, G = (random_bf16((1, 2, N, 128), s) for s in (101, 102, 103, 104))
    _compare(Q, K, V, G, keep, phi, f"ragged keep={keep} {phi}")


@pytest.mark.parametrize("keep,phi", [(0.3, "elu1"), (1.0, "relu")])
def test_backward_parity_batched(keep, phi):
    # B = 2, H = 3: every (batch, head) slice of the key and query sides
    N = 64 * 6 - 9
    Q, K, V, G = (random_bf16((2, 3, N, 128), s) for s in (131, 132, 133, 134))
    _compare(Q, K, V, G, keep, phi, f"batched keep={keep} {phi}")


def test_backward_parity_tiny_workload():
    Q, K, V = make_inputs("tiny")
    G = make_dout("tiny")
    _compare(Q, K, V, G, 0.1, "elu1", "tiny")


@pytest.mark.parametrize("N", [1, 64, 130])
def test_backward_small_shapes(N):
    Q, K, V, G = (random_bf16((1, 1, N, 128), s) for s in (111, 112, 113, 114))
    _compare(Q, K, V, G, 0.5, "elu1", f"N={N}")


def test_backward_bf16_grads_round_the_fp32_ones():
    N = 64 * 5 - 7
    Q, K, V, G = (random_bf16((1, 2, N, 128), s) for s in (121, 122, 123, 124))
    f32 = _run(Q, K, V, G, 0.4, "elu1", torch.float32)
    b16 = _run(Q, K, V, G, 0.4, "elu1", torch.bfloat16)
    for a, b in zip(f32, b16):
        # bf16 output is the round-to-nearest-even of the same fp32 value
        r = torch.from_numpy(a).to(torch.bfloat16).float().numpy()
        assert np.array_equal(r, b)


def test_backward_parity_many_blocks():
    """150 query blocks (ragged last block), one head, every gradient entry."""
    from sparse_linear_attention_sagesla_amd.inputs import Workload, make_head
    wl = Workload("mid", 1, 1, 64 * 150 - 37, None, 7001)
    Q, K, V = (x[None, None] for x in make_head(wl, 0, 0))
    G = random_bf16(Q.shape, 131)
    _compare(Q, K, V, G, 0.1, "elu1", "mid")


@pytest.fixture(scope="module")
def wan720():
    from sparse_linear_attention_sagesla_amd.inputs import WORKLOADS
    wl = WORKLOADS["wan14b720"]
    Q, K, V = make_inputs(wl)
    G = make_dout(wl)
    print(f"[case] bwd wan14b720 shape={tuple(Q.shape)}", flush=True)
    q, k, v, g = (to_dev(x) for x in (Q, K, V, G))
    dq, dk, dv = sla.attention_bwd(q, k, v, g, keep=0.1, phi="elu1", grad_dtype=torch.float32)
    torch.cuda.synchronize()
    return Q, K, V, G, (q, k, v, g), (dq, dk, dv)


def test_backward_wan720_sampled_dq(wan720):
    """Full Wan-14B-720p shape: dQ of sampled query blocks (the last one ragged)
    against the oracle, which needs only those blocks for their dQ rows."""
    Q, K, V, G, _, (dq, _, _) = wan720
    nb = O.n_blocks(Q.shape[2], 64)
    for h in (0, 23):
        blocks = [0, 517, nb - 1]
        r = O.sla_backward_head(Q[0, h], K[0, h], V[0, h], G[0, h], block=64, keep=0.1,
                                phi_kind="elu1", query_blocks=blocks)
        rows = np.concatenate([np.arange(i * 64, min(Q.shape[2], (i + 1) * 64)) for i in blocks])
        _check(f"wan720 h{h} dq rows of {blocks}", dq[0, h, rows].cpu().numpy(), r["dq"][rows])


def test_backward_wan720_dv_rows_sum_to_twice_dout(wan720):
    """Every row's softmax weights and linear weights each sum to one, so the
    dV rows of a head sum to twice the dO rows (no row of this shape has an
    empty or vanishing linear branch).  The per-channel sums of N = 75600
    fp32 gradient rows carry independent, unbiased (round-to-nearest)
    errors of a few u times the entries, so the bound is 8u * rms(dV) *
    sqrt(N) * 4 (four standard deviations of such a sum)."""
    Q, K, V, G, _, (_, _, dv) = wan720
    dvs = dv.double().sum(dim=2).cpu().numpy()           # [B, H, d]
    want = 2.0 * O.bf16_to_f64(G).sum(axis=2)            # [B, H, d]
    rms = float(dv.double().pow(2).mean().sqrt())
    bound = 8 * U_BF16 * rms * np.sqrt(Q.shape[2]) * 4
    err = float(np.abs(dvs - want).max())
    print(f"[bwd] wan720 dv row sums: max err {err:.3e} bound {bound:.3e}", flush=True)
    assert err <= bound


def test_backward_is_deterministic(wan720):
    _, _, _, _, (q, k, v, g), (dq, dk, dv) = wan720
    dq2, dk2, dv2 = sla.attention_bwd(q, k, v, g, keep=0.1, phi="elu1", grad_dtype=torch.float32)
    torch.cuda.synchronize()
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a, b)


def test_backward_wan720_no_linear_sampled_key_blocks(wan720):
    """Full Wan-14B-720p shape without the linear branch (phi = none, keep
    0.1), in the benchmark's launch configuration (all heads in one call):
    dK and dV of sampled key blocks (first, middle, ragged last) of one head
    against the oracle, summed over the query blocks that keep them (the only
    contributions to those rows), split over a pool of oracle workers; and in
    every head the dK rows sum to zero (softmax-gradient rows do) and the dV
    rows to the dO rows (softmax weights sum to one), within four standard
    deviations of the rounding of N = 75600 fp32 rows (the dV bound above)."""
    Q, K, V, G, (q, k, v, g), _ = wan720
    print("[case] bwd wan14b720 phi=none", flush=True)
    dq, dk, dv = sla.attention_bwd(q, k, v, g, keep=0.1, phi="none", grad_dtype=torch.float32)
    torch.cuda.synchronize()
    N = Q.shape[2]
    rms_k = float(dk.double().pow(2).mean().sqrt())
    rms_v = float(dv.double().pow(2).mean().sqrt())
    err_k = float(dk.double().sum(dim=2).abs().max())
    want_v = O.bf16_to_f64(G).sum(axis=2)
    err_v = float(np.abs(dv.double().sum(dim=2).cpu().numpy() - want_v).max())
    bk, bv = (8 * U_BF16 * r * np.sqrt(N) * 4 for r in (rms_k, rms_v))
    print(f"[bwd] wan720 phi=none: dK row sums max {err_k:.3e} (bound {bk:.3e}), dV row sums "
          f"max err {err_v:.3e} (bound {bv:.3e})", flush=True)
    assert err_k <= bk and err_v <= bv
    h = 7
    nb = O.n_blocks(N, 64)
    key_blocks = [0, 591, nb - 1]
    idx = sla.block_select(q[:, h:h + 1], k[:, h:h + 1], 0.1)[0, 0].cpu().numpy()
    column = sorted({i for i in range(nb) if set(idx[i].tolist()) & set(key_blocks)})
    ex, n = oracle_pool()
    try:
        chunks = [column[c::n] for c in range(n) if column[c::n]]
        parts = list(ex.map(oracle_jobs.backward_key_share,
                            [("wan14b720", h, 0.1, "none", key_blocks, c) for c in chunks]))
    finally:
        ex.shutdown()
    want_k = sum(p[0] for p in parts)
    want_v = sum(p[1] for p in parts)
    rows = np.concatenate([np.arange(j * 64, min(N, (j + 1) * 64)) for j in key_blocks])
    print(f"[bwd] wan720 phi=none h{h}: key blocks {key_blocks}, {len(column)} query blocks "
          f"keep them, {len(chunks)} oracle jobs", flush=True)
    _check(f"wan720 phi=none h{h} dk rows of {key_blocks}", dk[0, h, rows].cpu().numpy(), want_k)
    _check(f"wan720 phi=none h{h} dv rows of {key_blocks}", dv[0, h, rows].cpu().numpy(), want_v)
