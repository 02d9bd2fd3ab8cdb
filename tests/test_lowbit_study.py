"""Tolerance study for a lower-bit variant of the forward (CPU, fp64 emulation).

The pages cite INT8/INT4 SageAttention; gfx950 has no INT4 matrix-core
instruction (its double-rate low-precision MFMA takes FP8/FP6/FP4 with block
scales), so the candidate is e4m3 FP8 for the operands of P.V and of the
linear branch's kept share.  This emulates the oracle's forward with e4m3
rounding (round to nearest even, 3 mantissa bits, subnormals below 2^-6,
saturating at 448) of V, of P, or of phi(K), on the tiny workload, and checks
the conclusion the design draws: FP8 V or P misses the forward's bar
(max-abs 2e-3, rel-L2 1e-3) by one to two orders of magnitude, FP8 phi(K)
alone stays inside it.
"""
import math

import numpy as np
import pytest

from oracle import sla_oracle as O
from sparse_linear_attention_sagesla_amd.inputs import make_inputs


def e4m3(x):
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    out = np.zeros_like(x)
    nz = a > 0
    e = np.maximum(np.floor(np.log2(a[nz])), -6.0)
    q = 2.0 ** (e - 3)
    out[nz] = np.sign(x[nz]) * np.minimum(np.round(a[nz] / q) * q, 448.0)
    return out


def test_e4m3_rounding_grid():
    assert e4m3([1.0, 1.0625, 1.125, 1.1875, 448.0, 500.0, -3.3])[:6].tolist() == \
        [1.0, 1.0, 1.125, 1.25, 448.0, 448.0]            # ties to even; saturation
    assert e4m3([2.0 ** -9, 2.0 ** -10])[0] == 2.0 ** -9  # smallest subnormal


def _forward(Qb, Kb, Vb, keep, mode):
    N = Qb.shape[0]
    r = O.sla_forward_head(Qb, Kb, Vb, 64, keep, "elu1")
    idx = r["idx"]
    q8, k8, sq, sk, _ = O.quantize_qk(Qb, Kb, 64)
    q, k, v = O.bf16_to_f64(Qb), O.bf16_to_f64(Kb), O.bf16_to_f64(Vb)
    v8 = e4m3(v) if "V" in mode else v
    fk = O.phi(k, "elu1")
    fk8 = e4m3(fk) if "F" in mode else fk
    H, z = fk.T @ v, fk.sum(0)
    outs = []
    for i in range(O.n_blocks(N, 64)):
        rows = np.arange(64 * i, min(N, 64 * i + 64))
        sel = idx[i]
        S = np.concatenate([np.arange(64 * j, min(N, 64 * j + 64)) for j in sel])
        lg, _ = O.block_logits(i, sel, q8, k8, sq, sk, N, 64, 128)
        p = np.exp(lg - lg.max(1, keepdims=True))
        l = p.sum(1, keepdims=True)
        o_s = ((e4m3(p) if "P" in mode else p) @ v8[S]) / l
        fq = O.phi(q[rows], "elu1")
        M, zm = fk8[S].T @ v8[S], fk8[S].sum(0)
        outs.append(o_s + (fq @ (H - M)) / (fq @ (z - zm))[:, None])
    got, want = np.concatenate(outs), r["out"]
    return float(np.abs(got - want).max()), float(np.linalg.norm(got - want) / np.linalg.norm(want))


@pytest.mark.parametrize("mode,inside", [("V", False), ("P", False), ("F", True)])
def test_fp8_operand_error_against_the_forward_bar(mode, inside):
    Q, K, V = make_inputs("tiny")
    for h in range(Q.shape[1]):
        max_abs, rel = _forward(Q[0, h], K[0, h], V[0, h], 0.1, mode)
        print(f"[lowbit] tiny h{h} e4m3[{mode}]: max-abs {max_abs:.2e} rel-L2 {rel:.2e}")
        if inside:
            assert max_abs <= 2e-3 and rel <= 1e-3
        else:
            assert max_abs > 20 * 2e-3 and rel > 5 * 1e-3
