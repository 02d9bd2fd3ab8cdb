"""Seeded synthetic inputs for the SageSLA attention forward.

This module only draws random numbers and rounds them to bfloat16; it holds
none of the attention arithmetic.  Both the HIP path (tests, bench) and the
CPU oracle consume what it produces, so the two sides always see the same bits.

Workloads (attention shapes of the Wan2.1 video DiT that the TurboDiffusion
pages accelerate; the pages measure real video generation, which needs model
weights, so these generators stand in for it):

* ``tiny``       B=1, H=2,  N=2048, d=128.  Each of Q, K, V is a rank-8
                 matrix (N x 8 @ 8 x 128, entries N(0,1)) plus 0.5*N(0,1) noise.
* ``wan13b480``  B=1, H=12, d=128, N=32760 tokens on a 21x30x52 latent grid.
* ``wan14b480``  B=1, H=40, same grid.
* ``wan14b720``  B=1, H=40, d=128, N=75600 tokens on a 21x45x80 latent grid.
* ``sweep``      the 720p shape with +8 added to channels 5, 37, 69, 101 of
                 both Q and K (outlier channels that exercise K smoothing).

For the grid workloads Q and K are independent trilinear-smooth random
fields (iid N(0,1) lattice every 4 tokens along each grid axis, interpolated
trilinearly, each channel scaled to unit empirical std over the grid) plus
0.3*N(0,1) noise; V is N(0,1).  Token order is t-major: n = (t*Hg + h)*W + w.

Every tensor is returned as uint16 bfloat16 bit patterns (round to nearest
even from float32), shape [B, H, N, d].
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

D_HEAD = 128
OUTLIER_CHANNELS = (5, 37, 69, 101)
OUTLIER_OFFSET = 8.0


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    grid: tuple | None          # (T, Hg, W) latent grid or None for the rank-8 recipe
    seed: int
    keep: tuple = (0.10,)       # keep fractions this workload is run at
    outliers: bool = False
    block: int = 64
    d: int = D_HEAD
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 2048, None, 1001),
    "wan13b480": Workload("wan13b480", 1, 12, 21 * 30 * 52, (21, 30, 52), 2001),
    "wan14b480": Workload("wan14b480", 1, 40, 21 * 30 * 52, (21, 30, 52), 3001),
    "wan14b720": Workload("wan14b720", 1, 40, 21 * 45 * 80, (21, 45, 80), 4001),
    "sweep": Workload("sweep", 1, 40, 21 * 45 * 80, (21, 45, 80), 5001,
                      keep=(0.0, 0.05, 0.20, 1.0), outliers=True),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _head_streams(seed: int, b: int, h: int):
    ss = np.random.SeedSequence([seed, b, h])
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(3)]


# Every step below is element-wise float32 arithmetic in a fixed order (no
# matrix products), so the bits do not depend on the BLAS library, its thread
# count or the threads that call it.

def _rank8(rng: np.random.Generator, N: int, d: int) -> np.ndarray:
    U = rng.standard_normal((N, 8), dtype=np.float32)
    A = rng.standard_normal((8, d), dtype=np.float32)
    E = rng.standard_normal((N, d), dtype=np.float32)
    x = U[:, 0:1] * A[0]
    for r in range(1, 8):
        x = x + U[:, r:r + 1] * A[r]
    return x + np.float32(0.5) * E


def _interp_axis(x: np.ndarray, n: int, axis: int, spacing: int = 4) -> np.ndarray:
    """Linear interpolation along `axis` from a lattice every `spacing` samples
    to n samples: sample t = (1 - f) x[i] + f x[i + 1], i = t // spacing,
    f = (t % spacing) / spacing."""
    t = np.arange(n)
    f = ((t % spacing) / spacing).astype(np.float32)
    shape = [1] * x.ndim
    shape[axis] = n
    a = np.take(x, t // spacing, axis=axis)
    b = np.take(x, t // spacing + 1, axis=axis)
    return a * (np.float32(1.0) - f).reshape(shape) + b * f.reshape(shape)


def _smooth_field(rng: np.random.Generator, grid, d: int) -> np.ndarray:
    T, Hg, W = grid
    m = [(n - 1) // 4 + 2 for n in grid]
    lat = rng.standard_normal((m[0], m[1], m[2], d), dtype=np.float32)
    # separable trilinear interpolation: along W, then Hg, then T
    f = _interp_axis(lat, W, 2)
    f = _interp_axis(f, Hg, 1)
    f = _interp_axis(f, T, 0)
    f = f.reshape(T * Hg * W, d)
    std = f.std(axis=0, dtype=np.float64).astype(np.float32)
    return f / std


def make_head(wl: Workload, b: int, h: int):
    """Q, K, V of one (batch, head) as uint16 bf16 bits, each [N, d]."""
    rq, rk, rv = _head_streams(wl.seed, b, h)
    N, d = wl.N, wl.d
    if wl.grid is None:
        q, k, v = _rank8(rq, N, d), _rank8(rk, N, d), _rank8(rv, N, d)
    else:
        assert wl.grid[0] * wl.grid[1] * wl.grid[2] == N
        q = _smooth_field(rq, wl.grid, d) + np.float32(0.3) * rq.standard_normal((N, d), dtype=np.float32)
        k = _smooth_field(rk, wl.grid, d) + np.float32(0.3) * rk.standard_normal((N, d), dtype=np.float32)
        v = rv.standard_normal((N, d), dtype=np.float32)
    if wl.outliers:
        for c in OUTLIER_CHANNELS:
            q[:, c] += np.float32(OUTLIER_OFFSET)
            k[:, c] += np.float32(OUTLIER_OFFSET)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def make_inputs(wl: Workload | str, heads=None, threads: int | None = None):
    """Q, K, V as uint16 bf16 bits [B, H', N, d] for the listed heads (default: all)."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    heads = list(range(wl.H)) if heads is None else list(heads)
    shape = (wl.B, len(heads), wl.N, wl.d)
    Q = np.empty(shape, np.uint16)
    K = np.empty(shape, np.uint16)
    V = np.empty(shape, np.uint16)
    jobs = [(b, hi, h) for b in range(wl.B) for hi, h in enumerate(heads)]

    def run(job):
        b, hi, h = job
        Q[b, hi], K[b, hi], V[b, hi] = make_head(wl, b, h)

    threads = threads or min(16, os.cpu_count() or 1, len(jobs))
    if threads <= 1:
        for j in jobs:
            run(j)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(run, jobs))
    return Q, K, V


def make_dout(wl: Workload | str, heads=None) -> np.ndarray:
    """Output gradient dO for the backward, N(0,1) bf16 bits [B, H', N, d].

    Drawn from its own stream per (batch, head), so adding it changes none of
    Q, K, V.
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    heads = list(range(wl.H)) if heads is None else list(heads)
    out = np.empty((wl.B, len(heads), wl.N, wl.d), np.uint16)
    for b in range(wl.B):
        for hi, h in enumerate(heads):
            rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, b, h, 9])))
            out[b, hi] = f32_to_bf16_bits(rng.standard_normal((wl.N, wl.d), dtype=np.float32))
    return out


def peaked_inputs(N: int, hot_blocks, hot: float, cold: float, seed: int,
                  neg_rows: int = 0, k_spread: float = 0.25, block: int = 64, d: int = D_HEAD):
    """Q, K, V bf16 bits [N, d] with a fixed block structure (edge-case tests).

    With E a standard normal clipped to [-3, 3] (so 1 + E/4 lies in
    [0.25, 1.75]): Q = 1 + E/4, except the first ``neg_rows`` rows of every
    block, which are -(1 + E/4); K rows of the blocks in ``hot_blocks`` are
    hot * (1 + s E) and all other K rows cold * (1 + s E), s = ``k_spread``
    (K draws its own E); V = 1 + N(0,1)/2.
    Every query block then sees the hot key blocks above all others, and
    ``cold`` sets how much the other blocks weigh against them.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 91])))

    def e(shape):
        return np.clip(rng.standard_normal(shape, dtype=np.float32), -3.0, 3.0)

    q = np.float32(1.0) + np.float32(0.25) * e((N, d))
    if neg_rows:
        blk_row = np.arange(N) % block
        q[blk_row < neg_rows] *= np.float32(-1.0)
    rows_hot = np.zeros(N, dtype=bool)
    for j in hot_blocks:
        rows_hot[j * block:min(N, (j + 1) * block)] = True
    mag = np.where(rows_hot, np.float32(hot), np.float32(cold)).astype(np.float32)
    k = mag[:, None] * (np.float32(1.0) + np.float32(k_spread) * e((N, d)))
    v = np.float32(1.0) + np.float32(0.5) * rng.standard_normal((N, d), dtype=np.float32)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def random_bf16(shape, seed: int, scale: float = 1.0, offset: float = 0.0) -> np.ndarray:
    """Plain N(offset, scale^2) bf16 bits, for edge-case tests."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 77])))
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale) + np.float32(offset)
    return f32_to_bf16_bits(x)
