"""Parity of the W8A8 path (through the C ABI) against the fp64 oracle.

Bit-exact: INT8 codes and scales of the per-row quantiser and of the
FusedNorm (with its fp32 mean and 1/std).  GEMM: the fp32 output within
4 fp32 ulps (relative 2^-22) of |acc * sx * sw| + |bias| per element -- the
integer sum is exact, then at most three fp32 roundings (the int32 -> fp32
conversion, two products, the bias add); bf16 output equal to the
round-to-nearest-even of the fp32 output.
"""
import numpy as np
import pytest

from oracle import w8a8_oracle as W
from sparse_linear_attention_sagesla_amd.inputs import random_bf16

from gpu_util import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
sla = pytest.importorskip("sparse_linear_attention_sagesla_amd")


def _dev2d(bits):
    return to_dev(bits)


@pytest.mark.parametrize("rows,K", [(7, 64), (33, 1536), (5, 5120), (3, 13824), (2, 16384)])
def test_rowquant_bit_exact(rows, K):
    print(f"[case] rowquant rows={rows} K={K}", flush=True)
    xb = random_bf16((rows, K), 200 + K, scale=0.02)
    xb[0] = 0                                        # an all-zero row: scale 0
    xb[-1, 3] = np.uint16(0x4780)                    # one large entry (65536)
    codes, scale = (t.cpu().numpy() for t in sla.rowquant_i8(_dev2d(xb)))
    oc, os_ = W.quantize_rows(W.bf16_to_f32(xb))
    assert np.array_equal(scale.view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(codes, oc)


@pytest.mark.parametrize("K,affine", [(128, False), (1536, True), (5120, True), (5120, False)])
def test_fused_norm_bit_exact(K, affine):
    rows = 24
    print(f"[case] fused norm rows={rows} K={K} affine={affine}", flush=True)
    xb = random_bf16((rows, K), 300 + K, scale=2.0, offset=0.3)
    xb[1] = xb[1, 0]                                  # a constant row: var 0
    g = b = None
    if affine:
        rng = np.random.default_rng(K)
        g = (1.0 + 0.2 * rng.standard_normal(K)).astype(np.float32)
        b = (0.1 * rng.standard_normal(K)).astype(np.float32)
    codes, scale, mean, rstd = sla.fused_norm_i8(
        _dev2d(xb), None if g is None else torch.from_numpy(g).cuda(),
        None if b is None else torch.from_numpy(b).cuda(), 1e-6)
    codes, scale, mean, rstd = (t.cpu().numpy() for t in (codes, scale, mean, rstd))
    oc, os_, om, orstd = W.fused_norm_quant(xb, 1e-6, g, b)
    assert np.array_equal(mean.view(np.uint32), om.view(np.uint32))
    assert np.array_equal(rstd.view(np.uint32), orstd.view(np.uint32))
    assert np.array_equal(scale.view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(codes, oc)


def _gemm_case(M, N, K, bias, seed):
    rng = np.random.default_rng(seed)
    x8 = rng.integers(-127, 128, (M, K)).astype(np.int8)
    w8 = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sx = (rng.random(M) * 0.05 + 1e-3).astype(np.float32)
    sw = (rng.random(N) * 0.01 + 1e-4).astype(np.float32)
    bv = rng.standard_normal(N).astype(np.float32) if bias else None
    return x8, sx, w8, sw, bv


def _run_gemm(x8, sx, w8, sw, bv, dtype):
    d = lambda a: torch.from_numpy(a).cuda()
    y = sla.w8a8_linear(d(x8), d(sx), d(w8), d(sw), None if bv is None else d(bv), out_dtype=dtype)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("M,N,K,bias", [(300, 260, 128, True), (256, 256, 384, False),
                                        (513, 516, 5120, True), (1, 4, 128, False),
                                        (700, 1024, 1536, True), (129, 64, 13824, False)])
def test_gemm_parity(M, N, K, bias):
    print(f"[case] gemm M={M} N={N} K={K} bias={bias}", flush=True)
    x8, sx, w8, sw, bv = _gemm_case(M, N, K, bias, M + N + K)
    y = _run_gemm(x8, sx, w8, sw, bv, torch.float32).cpu().numpy()
    want = W.w8a8_linear(x8, sx, w8, sw, bv)
    mag = np.abs(W.w8a8_linear(x8, sx, w8, sw)) + (np.abs(bv)[None, :] if bv is not None else 0.0)
    err = np.abs(y - want)
    print(f"[gemm] max err / magnitude {float((err / np.maximum(mag, 1e-30)).max()):.3e}", flush=True)
    assert np.all(err <= 2.0 ** -22 * mag)
    yb = _run_gemm(x8, sx, w8, sw, bv, torch.bfloat16)
    assert torch.equal(torch.from_numpy(y).to(torch.bfloat16), yb.cpu())


def test_fused_norm_then_linear_end_to_end():
    """A Wan-14B-shaped layer slice: FusedNorm on 1000 tokens of width 5120,
    weights [5120, 5120] quantised per output channel, the W8A8 product."""
    M, K, N = 1000, 5120, 5120
    print(f"[case] end to end M={M} K={K} N={N}", flush=True)
    xb = random_bf16((M, K), 41, scale=1.5)
    wb = random_bf16((N, K), 42, scale=0.02)
    c, s, _, _ = sla.fused_norm_i8(_dev2d(xb))
    w8, sw = sla.rowquant_i8(_dev2d(wb))
    y = sla.w8a8_linear(c, s, w8, sw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    oc, os_, _, _ = W.fused_norm_quant(xb, 1e-6)
    ow8, osw = W.quantize_rows(W.bf16_to_f32(wb))
    assert np.array_equal(c.cpu().numpy(), oc) and np.array_equal(w8.cpu().numpy(), ow8)
    rows = np.arange(0, M, 37)
    want = W.w8a8_linear(oc[rows], os_[rows], ow8, osw)
    got = y.cpu().numpy()[rows]
    assert np.all(np.abs(got - want) <= 2.0 ** -22 * np.abs(want) + 1e-30)


def test_gemm_full_ffn_shape_sampled():
    """Wan-14B-720p FFN up-projection shape (M = 75600 tokens, K = 5120,
    N = 13824), sampled rows against the oracle."""
    M, N, K = 75600, 13824, 5120
    print(f"[case] gemm full M={M} N={N} K={K}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(5)
    x8 = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda", generator=g)
    w8 = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda", generator=g)
    sx = torch.rand(M, device="cuda", generator=g) * 0.05 + 1e-3
    sw = torch.rand(N, device="cuda", generator=g) * 0.01 + 1e-4
    y = sla.w8a8_linear(x8, sx, w8, sw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 40000, M - 81, M - 1])
    xs, ws = x8[rows].cpu().numpy(), w8.cpu().numpy()
    want = W.w8a8_linear(xs, sx[rows].cpu().numpy(), ws, sw.cpu().numpy())
    got = y[rows].cpu().numpy()
    assert np.all(np.abs(got - want) <= 2.0 ** -22 * np.abs(want) + 1e-30)
