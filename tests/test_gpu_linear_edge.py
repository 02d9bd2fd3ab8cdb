"""Linear branch on rows whose unselected keys carry little of the phi weight.

The linear branch is phi(q)^T H_U / phi(q)^T z_U over the unselected keys U
(tutorial "TurboDiffusion技术架构解析：稀疏线性注意力应用实战" §2.1, linear
attention, normalised).  When the kept blocks hold almost all of a row's phi
weight, the unselected share f = phi(q)^T z_U / phi(q)^T z_all is small and
any form that gets H_U and z_U as whole-head sums minus the kept share must
not lose them in rounding.  The inputs (``peaked_inputs``) give every query
block the same kept key blocks and set f through the weight of the others:

* ReLU with negative cold keys: f = 0 exactly (every unselected weight is 0),
  so the linear output must be exactly 0;
* ReLU / elu+1 with f around 1e-3, 6e-3 and 3e-2, and V with mean 1, so a
  lost complement shows as an O(1) error;
* rows with phi(q) = 0 (ReLU, negative query rows): linear output exactly 0.

Each case runs at the tiny shape (32 blocks, keep 0.1: 4 kept) and on sampled
query blocks of one head of the Wan-14B-720p shape (1182 blocks, 119 kept).
"""
import math

import numpy as np
import pytest

from oracle import sla_oracle as O
from sparse_linear_attention_sagesla_amd.inputs import peaked_inputs

from gpu_util import assert_parity, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sla = pytest.importorskip("sparse_linear_attention_sagesla_amd")

HOT = 2.0
SPREAD = {"relu": 0.25, "elu1": 0.05}   # relative spread of the K entries


def _cold_for(f: float, phi: str, nb: int, k: int) -> float:
    """Magnitude of the cold key rows that puts the unselected share near f."""
    if f == 0.0:
        return -1.0
    ratio = k * f / ((nb - k) * (1.0 - f))          # cold weight / hot weight per key
    if phi == "relu":
        return HOT * ratio
    # elu+1: hot features average HOT + 1; a cold entry c (1 + s E) averages
    # exp(c + c^2 s^2 / 2), so solve c + c^2 s^2 / 2 = log(ratio (HOT + 1))
    s2 = SPREAD[phi] ** 2
    L = math.log(ratio * (HOT + 1.0))
    return (-1.0 + math.sqrt(1.0 + 2.0 * s2 * L)) / s2


def _unselected_share(Q, K, idx, phi, blocks, block=64):
    """min and max over the valid rows of the sampled blocks of
    f = phi(q).z_U / phi(q).z_all (rows with phi(q).z_all = 0 skipped)."""
    N = Q.shape[0]
    fk = O.phi(O.bf16_to_f64(K), phi)
    z_all = fk.sum(0)
    out = []
    for i in blocks:
        kept = np.zeros(N, bool)
        for j in idx[i]:
            kept[j * block:(j + 1) * block] = True
        z_u = fk[~kept].sum(0)
        fq = O.phi(O.bf16_to_f64(Q[i * block:min(N, (i + 1) * block)]), phi)
        den = fq @ z_all
        ok = den > 0
        out.append((fq @ z_u)[ok] / den[ok])
    f = np.concatenate(out)
    return float(f.min()), float(f.max())


def _run(N, hot_blocks, phi, f, blocks, neg_rows=0, seed=0):
    nb = O.n_blocks(N, 64)
    k = O.topk_count(nb, 0.1)
    assert len(hot_blocks) == k
    cold = _cold_for(f, phi, nb, k)
    Q, K, V = peaked_inputs(N, hot_blocks, HOT, cold, seed=seed + 17, neg_rows=neg_rows,
                            k_spread=SPREAD[phi])
    print(f"[case] N={N} phi={phi} f~{f} cold={cold:.4g} neg_rows={neg_rows}", flush=True)
    q, k_, v = (to_dev(x[None, None]) for x in (Q, K, V))
    out, lin = sla.attention(q, k_, v, 0.1, phi, torch.float32, return_linear=True)
    outb = sla.attention(q, k_, v, 0.1, phi, torch.bfloat16)
    torch.cuda.synchronize()
    out, lin = out[0, 0].cpu().numpy(), lin[0, 0].cpu().numpy()
    assert np.isfinite(out).all() and np.isfinite(lin).all()
    r = O.sla_forward_head(Q, K, V, 64, 0.1, phi, query_blocks=blocks)
    assert all(sorted(r["idx"][i].tolist()) == sorted(hot_blocks) for i in blocks)
    fmin, fmax = _unselected_share(Q, K, r["idx"], phi, blocks)
    print(f"[case] unselected share f in [{fmin:.3e}, {fmax:.3e}]", flush=True)
    if f == 0.0:
        assert fmax == 0.0
    else:
        assert f / 3 <= fmin and fmax <= 3 * f
    rows = r["rows"]
    assert_parity(out[rows], r["out"], what=f"{phi} f~{f} out")
    assert_parity(lin[rows], r["out_linear"], what=f"{phi} f~{f} linear branch")
    zero = r["out_linear"] == 0.0
    if zero.any():
        # rows whose unselected weights all vanish: exactly zero on the GPU too
        assert (lin[rows][zero] == 0.0).all()
    from gpu_util import bf16_bits_of, rne_bf16
    assert np.array_equal(bf16_bits_of(outb)[0, 0], rne_bf16(out))
    return fmin, fmax


TINY_HOT = [2, 9, 17, 30]


@pytest.mark.parametrize("phi,f", [("relu", 0.0), ("relu", 1e-3), ("relu", 6e-3), ("relu", 3e-2),
                                   ("elu1", 1e-3), ("elu1", 6e-3), ("elu1", 3e-2),
                                   ("relu", 0.3), ("elu1", 0.3)])
def test_small_unselected_share_tiny(phi, f):
    _run(2048, TINY_HOT, phi, f, list(range(32)))


@pytest.mark.parametrize("f", [0.0, 6e-3])
def test_zero_feature_rows_tiny(f):
    # the first 16 rows of every block have phi(q) = 0 under ReLU
    _run(2048, TINY_HOT, "relu", f, list(range(32)), neg_rows=16)


WAN_N = 21 * 45 * 80
WAN_HOT = list(range(0, 1190, 10))          # 119 blocks: 0, 10, ..., 1180
WAN_BLOCKS = [0, 5, 590, 1181]              # first, inside, middle, ragged last


@pytest.mark.parametrize("phi,f", [("relu", 0.0), ("relu", 1e-3), ("elu1", 6e-3), ("elu1", 3e-2)])
def test_small_unselected_share_wan720_head(phi, f):
    _run(WAN_N, WAN_HOT, phi, f, WAN_BLOCKS, seed=5)
