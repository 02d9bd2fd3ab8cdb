"""Pins of the W8A8 / FusedNorm oracle against facts outside it: torch's
LayerNorm in fp64, closed forms, a brute-force integer product, and
hand-checked quantiser values."""
import numpy as np
import pytest

from oracle import w8a8_oracle as W
from oracle import sla_oracle as O
from sparse_linear_attention_sagesla_amd.inputs import f32_to_bf16_bits, random_bf16


def test_quantize_rows_hand_values():
    x = np.array([[1.0, -2.0, 0.5, 127.0],        # a = 127: scale 1, codes = rint(x)
                  [0.0, 0.0, 0.0, 0.0],           # a = 0: scale 0, codes 0
                  [2.5, -0.5, 1.5, -3.0]], np.float32)  # a = 3: inv = 127/3
    codes, scales = W.quantize_rows(x)
    assert scales.tolist() == [1.0, 0.0, np.float32(3.0) / np.float32(127.0)]
    assert codes[0].tolist() == [1, -2, 0, 127]          # 0.5 ties to even 0
    assert codes[1].tolist() == [0, 0, 0, 0]
    inv = np.float32(127.0) / np.float32(3.0)
    want = [int(np.rint(np.float32(v * inv))) for v in x[2]]
    assert codes[2].tolist() == want and codes[2, 3] == -127


def test_layer_norm_matches_torch_fp64():
    torch = pytest.importorskip("torch")
    xb = random_bf16((7, 320), 3, scale=2.0, offset=0.7)
    g = (1.0 + 0.1 * np.random.default_rng(1).standard_normal(320)).astype(np.float32)
    b = (0.05 * np.random.default_rng(2).standard_normal(320)).astype(np.float32)
    mu, rstd, y = W.layer_norm_rows(xb, 1e-6, g, b)
    x64 = torch.tensor(O.bf16_to_f64(xb))
    ref = torch.nn.functional.layer_norm(x64, (320,), torch.tensor(g, dtype=torch.float64),
                                         torch.tensor(b, dtype=torch.float64), eps=1e-6).numpy()
    np.testing.assert_allclose(y, ref, rtol=0, atol=4e-6 * np.abs(ref).max())
    np.testing.assert_allclose(mu, x64.mean(1).numpy(), rtol=1e-7)
    np.testing.assert_allclose(rstd, 1 / np.sqrt(x64.var(1, unbiased=False).numpy() + 1e-6), rtol=1e-7)


def test_layer_norm_closed_forms_and_shift_invariance():
    K = 256
    const = f32_to_bf16_bits(np.full((2, K), 3.25, np.float32))
    mu, rstd, y = W.layer_norm_rows(const, 1e-6, None, np.full(K, 0.5, np.float32))
    assert mu.tolist() == [3.25, 3.25]
    assert np.all(rstd == np.float32(1.0 / np.sqrt(np.float64(np.float32(1e-6)))))
    assert np.all(y == np.float32(0.5))                  # zero deviation: y = beta
    # +-1 alternating row: mean 0, var 1
    alt = f32_to_bf16_bits(np.tile(np.array([1.0, -1.0], np.float32), (1, K // 2)))
    mu, rstd, y = W.layer_norm_rows(alt, 0.0)
    assert mu[0] == 0.0 and rstd[0] == 1.0 and np.array_equal(np.abs(y), np.ones((1, K), np.float32))
    # shifting every value (on a grid where bf16 holds x and x + 4 exactly)
    # leaves the normalised row unchanged
    x = (np.random.default_rng(9).integers(-128, 128, (3, K)) / 32.0).astype(np.float32)
    xb = f32_to_bf16_bits(x)
    shifted = f32_to_bf16_bits(x + np.float32(4.0))
    assert np.array_equal(O.bf16_to_f32(xb), x)
    assert np.array_equal(O.bf16_to_f32(shifted) - np.float32(4.0), x)
    _, _, y0 = W.layer_norm_rows(xb, 1e-6)
    _, _, y1 = W.layer_norm_rows(shifted, 1e-6)
    np.testing.assert_allclose(y0, y1, atol=2e-6)


def test_linear_matches_integer_loop_and_scales():
    rng = np.random.default_rng(4)
    x8 = rng.integers(-127, 128, (5, 96)).astype(np.int8)
    w8 = rng.integers(-127, 128, (3, 96)).astype(np.int8)
    sx = rng.random(5).astype(np.float32)
    sw = rng.random(3).astype(np.float32)
    bias = rng.standard_normal(3).astype(np.float32)
    y = W.w8a8_linear(x8, sx, w8, sw, bias)
    for m in range(5):
        for n in range(3):
            acc = sum(int(x8[m, k]) * int(w8[n, k]) for k in range(96))
            assert y[m, n] == acc * float(sx[m]) * float(sw[n]) + float(bias[n])


def test_w8a8_approximates_the_float_linear_layer():
    """Dequantised codes are within half a step of the inputs (plus the fp32
    rounding of scale and inverse scale, relative 2^-22 of the row maximum),
    so the W8A8 product is within the first-order bound of the float one."""
    xb = random_bf16((16, 512), 5)
    wb = random_bf16((24, 512), 6, scale=0.05)
    x, w = O.bf16_to_f32(xb), O.bf16_to_f32(wb)
    x8, sx = W.quantize_rows(x)
    w8, sw = W.quantize_rows(w)
    assert np.all(np.abs(x8 * sx[:, None].astype(np.float64) - x) <= 0.5 * sx[:, None] * (1 + 1e-4))
    y = W.w8a8_linear(x8, sx, w8, sw)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    bound = 0.5 * (sx[:, None] * np.abs(w).sum(1)[None, :] + sw[None, :] * np.abs(x).sum(1)[:, None]) \
        + 0.25 * sx[:, None] * sw[None, :] * 512
    assert np.all(np.abs(y - ref) <= bound)


def test_fused_norm_quant_codes_reconstruct_the_normalised_rows():
    xb = random_bf16((6, 640), 8, scale=3.0, offset=-1.0)
    codes, scales, mu, rstd = W.fused_norm_quant(xb, 1e-6)
    _, _, y = W.layer_norm_rows(xb, 1e-6)
    assert np.all(np.abs(codes * scales[:, None].astype(np.float64) - y) <= 0.5 * scales[:, None] * (1 + 1e-4))
    assert np.all(np.abs(codes).max(1) == 127)
