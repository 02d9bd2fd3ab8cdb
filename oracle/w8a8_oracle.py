"""Plain fp64 CPU oracle for the W8A8 INT8 linear layer and FusedNorm.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the HIP product path
never calls it and shares no code with it.

Sources (web pages on TurboDiffusion; citations name the page and section):

* [NEWS] TurboDiffusion news summary (jiqiren.org.cn), the opening component
         list, item 3: model parameters and activations are quantised to 8
         bits to speed up the linear layers and compress the model.
* [COM]  "清华开源TurboDiffusion加速框架..." (commentary), section
         "步数蒸馏与W8A8量化：在压缩与精度间找到平衡": weights and activations go
         from 16-bit floats to 8-bit integers and run on the GPU's INT8 units.
* [BLOG] "TurboDiffusion：让可视化视频生成效率提升200倍的加速引擎", section
         "1. 计算资源优化：CPU Offload与混合精度计算": W8A8 comes with a fused
         normalisation operator (FusedNorm), under 1% precision loss.

The pages give no granularity, rounding or normalisation formula.  Readings
(the plainest ones the rest supports):

 1. Weights W [N, K]: one symmetric INT8 scale per output channel (row), the
    same quantiser as the attention codes (``quantize_blocks`` with one row
    per block): a = max|w|, scale = fp32(a/127), code = clamp(rint_even(
    fp32(w * fp32(127/a))), +-127); a = 0 gives scale 0 and zero codes.
 2. Activations X [M, K]: one scale per token (row), the same quantiser.
 3. Linear: y[m, n] = (sum_k x8[m, k] w8[n, k]) * sx[m] * sw[n] + bias[n],
    the integer sum exact.
 4. FusedNorm: the LayerNorm in front of a Wan block's linear layers, fused
    with the activation quantisation: per token, mu = mean(x), var =
    mean((x - mu)^2), rstd = 1/sqrt(var + eps); y = (x - mu) * rstd, then the
    optional per-channel affine y * gamma + beta (which also expresses an
    adaptive-norm modulation (1 + scale, shift)); then reading 2 on y.  The
    steps that decide the INT8 codes are fixed in fp32: mu = fp32(mean in
    exact arithmetic), rstd = fp32(1/sqrt(var + eps)) with var formed
    exactly from the fp32 mu, t = fp32(x - mu), t = fp32(t * rstd),
    y = fp32(fp32(t * gamma) + beta).
"""
from __future__ import annotations

import math

import numpy as np

from oracle.sla_oracle import bf16_to_f32, quantize_blocks


def quantize_rows(x32: np.ndarray):
    """Per-row symmetric INT8 codes [R, K] and scales fp32 [R] (readings 1-2)."""
    x32 = np.asarray(x32, dtype=np.float32)
    return quantize_blocks(x32, 1)


def layer_norm_rows(x_bits: np.ndarray, eps: float, gamma=None, beta=None):
    """(mu fp32 [M], rstd fp32 [M], y fp32 [M, K]) of reading 4.

    mu: the exact row sum (math.fsum of the fp32 values), divided by K in
    fp64, rounded to fp32.  var: math.fsum of the fp64 squares of (x - mu)
    (x - mu itself exact in fp64), / K in fp64; rstd = fp32(1 / sqrt(var +
    eps)) in fp64.
    """
    x = bf16_to_f32(x_bits)
    M, K = x.shape
    mu = np.empty(M, np.float32)
    rstd = np.empty(M, np.float32)
    for m in range(M):
        row = x[m].astype(np.float64)
        mu[m] = np.float32(math.fsum(row.tolist()) / K)
        dev = row - np.float64(mu[m])
        var = math.fsum((dev * dev).tolist()) / K
        rstd[m] = np.float32(1.0 / math.sqrt(var + float(np.float32(eps))))
    t = (x - mu[:, None]).astype(np.float32)
    t = (t * rstd[:, None]).astype(np.float32)
    if gamma is not None:
        t = (t * np.asarray(gamma, np.float32)[None, :]).astype(np.float32)
    if beta is not None:
        t = (t + np.asarray(beta, np.float32)[None, :]).astype(np.float32)
    return mu, rstd, t


def fused_norm_quant(x_bits: np.ndarray, eps: float = 1e-6, gamma=None, beta=None):
    """FusedNorm: LayerNorm (+ affine) then per-token INT8 (reading 4).

    Returns (codes int8 [M, K], scales fp32 [M], mu, rstd)."""
    mu, rstd, y = layer_norm_rows(x_bits, eps, gamma, beta)
    codes, scales = quantize_rows(y)
    return codes, scales, mu, rstd


def w8a8_linear(x8, sx, w8, sw, bias=None) -> np.ndarray:
    """y = (x8 w8^T) * sx * sw + bias in fp64 (reading 3); the integer
    products summed exactly (int64)."""
    acc = np.asarray(x8, np.int64) @ np.asarray(w8, np.int64).T
    y = acc.astype(np.float64) * np.asarray(sx, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    return y
