"""The error bound of the filtered block top-k (CPU, no GPU needed).

The GPU selection approximates each block score s_ij = sum_c qbar_ic kbar_jc
by three bf16 products of hi/lo splits (x_h = bf16(x), x_l = bf16(x - x_h),
round to nearest even) accumulated in fp32, and trusts that the approximation
stays within E_i = 2^-12 |qbar_i| max_j |kbar_j| of the exact fp64 score, the
oracle's.  This test emulates that arithmetic in numpy -- the products are
exact in fp32, the 384 of them summed in fp32 in two different orders -- and
checks the distance against a quarter of the kernel's bound on smooth-field
block means and on adversarial ones (magnitudes from 2^-20 to 2^20 within a
row, heavy cancellation).  It checks the argument behind the kernel, not the
kernel itself: that is the GPU selection tests' job (bit-exact kept lists).
"""
import numpy as np


def bf16_rne(x32):
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def split(x32):
    h = bf16_rne(x32)
    lo = bf16_rne((x32 - h).astype(np.float32))
    return h, lo


def approx_scores(q, k, order):
    """[rows, cols] fp32 sums of the three split products, in `order`."""
    qh, ql = split(q)
    kh, kl = split(k)
    terms = [qh[:, None, :] * kh[None, :, :], qh[:, None, :] * kl[None, :, :],
             ql[:, None, :] * kh[None, :, :]]              # exact in fp32
    t = np.concatenate(terms, axis=2).astype(np.float32)    # [rows, cols, 384]
    if order == "reversed":
        t = t[:, :, ::-1]
    acc = np.zeros(t.shape[:2], np.float32)
    for c in range(t.shape[2]):
        acc = (acc + t[:, :, c]).astype(np.float32)
    return acc


def exact_scores(q, k):
    return q.astype(np.float64) @ k.astype(np.float64).T


def check(q, k):
    E = 2.0 ** -12 * np.linalg.norm(q.astype(np.float64), axis=1)[:, None] * \
        np.linalg.norm(k.astype(np.float64), axis=1).max()
    ref = exact_scores(q, k)
    worst = 0.0
    for order in ("forward", "reversed"):
        err = np.abs(approx_scores(q, k, order).astype(np.float64) - ref)
        worst = max(worst, float((err / E).max()))
    print(f"[bound] largest |s~ - s| / E: {worst:.3e}")
    assert worst <= 0.25


def test_bound_on_smooth_block_means():
    rng = np.random.default_rng(3)
    q = (rng.standard_normal((24, 128)) * 0.3).astype(np.float32)
    k = (rng.standard_normal((200, 128)) * 0.3 + 0.05).astype(np.float32)
    check(q, k)


def test_bound_with_mixed_magnitudes_and_cancellation():
    rng = np.random.default_rng(4)
    mag = 2.0 ** rng.integers(-20, 21, size=(16, 128))
    q = (rng.standard_normal((16, 128)) * mag).astype(np.float32)
    k = (rng.standard_normal((150, 128)) * 2.0 ** rng.integers(-20, 21, size=(150, 128))).astype(np.float32)
    k[:50] = -k[50:100] * (1 + 2.0 ** -10)                  # near-cancelling pairs
    k[100:] = q[rng.integers(0, 16, 50)] * -1.0 + 2.0 ** -30  # rows anti-aligned with queries
    check(q, k)
