"""The training path: sla_attention_fwd_train (the forward, plus the residuals
its backward needs) and sla_attention_bwd_saved (the backward that reads them
instead of re-walking the kept tiles), through the C ABI.

The training forward's output must equal the plain forward's bit for bit, its
linear-branch residual must equal the forward's out_linear bit for bit, and
the softmax residual plus the linear one must give the output up to the
roundings of the product and the sum.  The saved backward is held to the same parity bar against the
fp64 oracle as the recomputing backward (the tolerance derivation is in
test_gpu_backward.py), and must stay close to the recomputing backward, from
which it differs only in how the linear output and D are formed.
"""
import numpy as np
import pytest

from oracle import sla_oracle as O
from sparse_linear_attention_sagesla_amd.inputs import make_dout, make_inputs, random_bf16

from gpu_util import errors, to_dev
from test_gpu_backward import _check

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sla = pytest.importorskip("sparse_linear_attention_sagesla_amd")

CASES = [(0.3, "elu1"), (0.3, "relu"), (0.3, "none"), (0.0, "elu1"), (1.0, "elu1"), (0.6, "elu1")]


def _views(res, B, H, N, keep, phi):
    """stats [B,H,N,2], os [B,H,N,128], ol (or None) inside the residual buffer,
    at the offsets the header documents (256-byte aligned pieces)."""
    up = lambda n: (n + 255) // 256 * 256
    nb = O.n_blocks(N, 64)
    k = O.topk_count(nb, keep)
    lin = phi != "none" and k < nb
    f = res.view(torch.uint8)
    o1 = up(B * H * N * 2 * 4)
    o2 = o1 + up(B * H * N * 128 * 4)
    stats = f[:B * H * N * 8].view(torch.float32).view(B, H, N, 2)
    os_ = f[o1:o1 + B * H * N * 512].view(torch.float32).view(B, H, N, 128)
    ol = f[o2:o2 + B * H * N * 512].view(torch.float32).view(B, H, N, 128) if lin else None
    return stats, os_, ol


def test_train_residuals_hold_the_forwards_codes_and_selection():
    """The staging a training forward leaves for the backward (INT8 codes and
    scales, kept lists), at the documented offsets, equals what the stand-alone
    entry points sla_quantize_qk and sla_block_select return, bit for bit."""
    B, H, N, keep = 1, 2, 64 * 9 - 23, 0.3   # 9 blocks, 3 kept: subtraction form
    Q, K, V = (random_bf16((B, H, N, 128), s) for s in (221, 222, 223))
    q, k, v = (to_dev(x) for x in (Q, K, V))
    print(f"[case] train residual staging N={N} keep={keep}", flush=True)
    _, res = sla.attention_train(q, k, v, keep, "elu1", torch.float32)
    q8, k8, sq, sk, _ = sla.quantize_qk(q, k)
    idx = sla.block_select(q, k, keep)
    torch.cuda.synchronize()
    up = lambda n: (n + 255) // 256 * 256
    nb = O.n_blocks(N, 64)
    kk = O.topk_count(nb, keep)
    assert nb - kk > kk
    off = (up(B * H * N * 8) + 2 * up(B * H * N * 512) + up(B * H * nb * 128 * 128 * 2)
           + up(B * H * nb * 128 * 4))
    f = res.view(torch.uint8)

    def take(nbytes, dtype, shape):
        nonlocal off
        t = f[off:off + nbytes].view(dtype).view(*shape)
        off += up(nbytes)
        return t

    codes = B * H * nb * 64 * 128
    r_q8 = take(codes, torch.int8, (B, H, nb * 64, 128))
    r_sq = take(B * H * nb * 4, torch.float32, (B, H, nb))
    r_k8 = take(codes, torch.int8, (B, H, nb * 64, 128))
    r_sk = take(B * H * nb * 4, torch.float32, (B, H, nb))
    r_idx = take(B * H * nb * kk * 4, torch.int32, (B, H, nb, kk))
    assert torch.equal(r_q8, q8) and torch.equal(r_k8, k8)
    assert torch.equal(r_sq, sq) and torch.equal(r_sk, sk)
    assert torch.equal(r_idx, idx)


@pytest.mark.parametrize("keep,phi", CASES)
def test_train_forward_output_and_residuals(keep, phi):
    N = 64 * 9 - 23
    Q, K, V = (random_bf16((1, 2, N, 128), s) for s in (201, 202, 203))
    q, k, v = (to_dev(x) for x in (Q, K, V))
    print(f"[case] train fwd N={N} keep={keep} phi={phi}", flush=True)
    out_t, res = sla.attention_train(q, k, v, keep, phi, torch.float32)
    out16_t, _ = sla.attention_train(q, k, v, keep, phi, torch.bfloat16)
    out, lin = sla.attention(q, k, v, keep, phi, torch.float32, return_linear=True)
    out16 = sla.attention(q, k, v, keep, phi, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(out_t, out) and torch.equal(out16_t, out16)
    stats, os_, ol = _views(res, 1, 2, N, keep, phi)
    nb = O.n_blocks(N, 64)
    kk = O.topk_count(nb, keep)
    if ol is not None:
        assert torch.equal(ol, lin)
        total, mag = os_ + ol, os_.abs() + ol.abs()
    else:
        total, mag = os_, os_.abs()
    # the kernel forms out = o * (1/l) + O_l with one fused rounding, the
    # residual o * (1/l) separately: they differ by at most the two roundings
    assert bool(((total - out).abs() <= 2.0 ** -23 * mag).all())
    if kk > 0:
        assert bool((stats[..., 1] > 0).all()) and bool(torch.isfinite(stats[..., 0]).all())
    else:
        assert bool((stats[..., 1] == 0).all()) and bool(torch.isinf(stats[..., 0]).all())
        assert not bool(os_.any())


def _saved(Q, K, V, G, keep, phi, grad_dtype=torch.float32):
    q, k, v, g = (to_dev(x) for x in (Q, K, V, G))
    print(f"[case] saved bwd shape={tuple(Q.shape)} keep={keep} phi={phi}", flush=True)
    _, res = sla.attention_train(q, k, v, keep, phi)
    dq, dk, dv = sla.attention_bwd(q, k, v, g, keep=keep, phi=phi, grad_dtype=grad_dtype, residuals=res)
    torch.cuda.synchronize()
    return [x.float().cpu().numpy() for x in (dq, dk, dv)]


def _compare(Q, K, V, G, keep, phi, tag):
    got = _saved(Q, K, V, G, keep, phi)
    for b in range(Q.shape[0]):
        for h in range(Q.shape[1]):
            r = O.sla_backward_head(Q[b, h], K[b, h], V[b, h], G[b, h], block=64, keep=keep, phi_kind=phi)
            for i, name in enumerate(("dq", "dk", "dv")):
                _check(f"saved {tag} b{b} h{h} {name}", got[i][b, h], r[name])


@pytest.mark.parametrize("keep,phi", CASES)
def test_saved_backward_parity_ragged(keep, phi):
    N = 64 * 9 - 23
    Q, K, V, G = (random_bf16((1, 2, N, 128), s) for s in (101, 102, 103, 104))
    _compare(Q, K, V, G, keep, phi, f"ragged keep={keep} {phi}")


def test_saved_backward_parity_batched():
    # B = 2, H = 3: the residuals' per-(batch, head) slices
    N = 64 * 6 - 9
    Q, K, V, G = (random_bf16((2, 3, N, 128), s) for s in (141, 142, 143, 144))
    _compare(Q, K, V, G, 0.3, "elu1", "batched")


def test_saved_backward_parity_tiny_workload():
    Q, K, V = make_inputs("tiny")
    G = make_dout("tiny")
    _compare(Q, K, V, G, 0.1, "elu1", "tiny")


@pytest.mark.parametrize("N", [1, 64, 130])
def test_saved_backward_small_shapes(N):
    Q, K, V, G = (random_bf16((1, 1, N, 128), s) for s in (111, 112, 113, 114))
    _compare(Q, K, V, G, 0.3, "elu1", f"N={N}")


@pytest.mark.parametrize("keep,phi", [(0.3, "elu1"), (0.3, "relu"), (0.3, "none"), (0.1, "elu1")])
def test_saved_backward_close_to_recomputing_backward(keep, phi):
    """Same gradients as sla_attention_bwd up to the linear output's and D's
    rounding: well inside the oracle bar (7.8e-3)."""
    N = 64 * 20 - 5
    Q, K, V, G = (random_bf16((1, 2, N, 128), s) for s in (141, 142, 143, 144))
    q, k, v, g = (to_dev(x) for x in (Q, K, V, G))
    ref = sla.attention_bwd(q, k, v, g, keep=keep, phi=phi, grad_dtype=torch.float32)
    got = _saved(Q, K, V, G, keep, phi)
    for i, name in enumerate(("dq", "dk", "dv")):
        ma, rel = errors(got[i], ref[i].cpu().numpy())
        print(f"[bwd] saved vs recomputed keep={keep} {phi} {name}: max-abs {ma:.3e} rel-L2 {rel:.3e}",
              flush=True)
        assert rel <= 2e-3


def test_saved_backward_bf16_grads_round_the_fp32_ones():
    N = 64 * 5 - 7
    Q, K, V, G = (random_bf16((1, 2, N, 128), s) for s in (121, 122, 123, 124))
    f32 = _saved(Q, K, V, G, 0.4, "elu1", torch.float32)
    b16 = _saved(Q, K, V, G, 0.4, "elu1", torch.bfloat16)
    for a, b in zip(f32, b16):
        assert np.array_equal(torch.from_numpy(a).to(torch.bfloat16).float().numpy(), b)


def test_saved_backward_wan720_sampled_dq_and_deterministic():
    """Full Wan-14B-720p shape: dQ of sampled query blocks (the last one
    ragged) of two heads against the oracle, and two calls bit-identical."""
    from sparse_linear_attention_sagesla_amd.inputs import WORKLOADS
    wl = WORKLOADS["wan14b720"]
    Q, K, V = make_inputs(wl)
    G = make_dout(wl)
    print(f"[case] saved bwd wan14b720 shape={tuple(Q.shape)}", flush=True)
    q, k, v, g = (to_dev(x) for x in (Q, K, V, G))
    _, res = sla.attention_train(q, k, v, 0.1, "elu1")
    dq, dk, dv = sla.attention_bwd(q, k, v, g, keep=0.1, phi="elu1", grad_dtype=torch.float32, residuals=res)
    dq2, dk2, dv2 = sla.attention_bwd(q, k, v, g, keep=0.1, phi="elu1", grad_dtype=torch.float32,
                                      residuals=res)
    torch.cuda.synchronize()
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a, b)
    nb = O.n_blocks(Q.shape[2], 64)
    for h in (0, 23):
        blocks = [0, 517, nb - 1]
        r = O.sla_backward_head(Q[0, h], K[0, h], V[0, h], G[0, h], block=64, keep=0.1,
                                phi_kind="elu1", query_blocks=blocks)
        rows = np.concatenate([np.arange(i * 64, min(Q.shape[2], (i + 1) * 64)) for i in blocks])
        _check(f"saved wan720 h{h} dq rows of {blocks}", dq[0, h, rows].cpu().numpy(), r["dq"][rows])
