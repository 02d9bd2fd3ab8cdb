"""The opt-in lower-bit forward (sla_attention_fwd_lowbit): the linear branch's
phi(K) as FP8 e4m3 codes with a power-of-two scale per key block.

Its contract is parity with the oracle's FP8 option (``phi_k_fp8=True``: the
same per-block scale and round-to-nearest-even e4m3 rounding) at the forward's
tolerance, max-abs 2e-3 and rel-L2 1e-3 on the fp32 output, with the bf16
output the round-to-nearest-even of the fp32 one.  The distance to the exact
forward is printed for the record (the rounding of phi(K) is a change of the
computed function, not an error of the kernel).
"""
import numpy as np
import pytest

from oracle import sla_oracle as O
from sparse_linear_attention_sagesla_amd.inputs import make_inputs, peaked_inputs, random_bf16

from gpu_util import assert_parity, bf16_bits_of, errors, rne_bf16, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sla = pytest.importorskip("sparse_linear_attention_sagesla_amd")


@pytest.fixture(scope="module")
def tiny():
    return make_inputs("tiny")


def _check(Q, K, V, keep, phi, what, blocks=None):
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    print(f"[case] lowbit {what} shape={tuple(q.shape)} keep={keep} {phi}", flush=True)
    out, lin = sla.attention(q, k, v, keep, phi, torch.float32, return_linear=True, lowbit=True)
    out16 = sla.attention(q, k, v, keep, phi, torch.bfloat16, lowbit=True)
    torch.cuda.synchronize()
    out, lin = out.cpu().numpy(), lin.cpu().numpy()
    assert np.isfinite(out).all()
    for b in range(Q.shape[0]):
        for h in range(Q.shape[1]):
            r = O.sla_forward_head(Q[b, h], K[b, h], V[b, h], 64, keep, phi, query_blocks=blocks,
                                   phi_k_fp8=True)
            rows = r["rows"]
            assert_parity(out[b, h][rows], r["out"], what=f"lowbit {what} b{b} h{h}")
            assert_parity(lin[b, h][rows], r["out_linear"], what=f"lowbit {what} linear b{b} h{h}")
            e = O.sla_forward_head(Q[b, h], K[b, h], V[b, h], 64, keep, phi, query_blocks=blocks)
            ma, rel = errors(out[b, h][rows], e["out"])
            print(f"[lowbit] {what} b{b} h{h}: against the exact forward max-abs {ma:.3e} "
                  f"rel-L2 {rel:.3e}", flush=True)
    assert np.array_equal(bf16_bits_of(out16), rne_bf16(out))


@pytest.mark.parametrize("keep,phi", [(0.1, "elu1"), (0.2, "relu"), (0.0, "elu1"), (0.6, "elu1")])
def test_lowbit_parity_tiny(tiny, keep, phi):
    Q, K, V = tiny
    _check(Q, K, V, keep, phi, "tiny")


@pytest.mark.parametrize("N", [1, 65, 1000])
def test_lowbit_ragged(N):
    Q, K, V = (random_bf16((1, 2, N, 128), 80 + s, scale=1.5) for s in range(3))
    _check(Q, K, V, 0.1, "elu1", f"N={N}")


@pytest.mark.parametrize("phi,cold", [("relu", -1.0), ("relu", 2.86e-4), ("elu1", -6.0)])
def test_lowbit_small_unselected_share(phi, cold):
    # every query block keeps blocks 2, 9, 17, 30; the others weigh little (or nothing)
    Q, K, V = peaked_inputs(2048, [2, 9, 17, 30], 2.0, cold, seed=23,
                            k_spread=0.25 if phi == "relu" else 0.05)
    _check(Q[None, None], K[None, None], V[None, None], 0.1, phi, f"peaked cold={cold}")


def test_lowbit_wan720_head_sampled():
    Q, K, V = make_inputs("wan14b720", heads=[0])
    _check(Q, K, V, 0.1, "elu1", "wan14b720 head 0", blocks=[0, 5, 591, 1181])
