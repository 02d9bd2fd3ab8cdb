"""Plain fp64 CPU oracle for the SageSLA attention forward.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the HIP product path
never calls it and shares no code with it.

Sources (web pages on TurboDiffusion; citations name the page and section):

* [TUT]  "TurboDiffusion技术架构解析：稀疏线性注意力应用实战" (tutorial),
         §2.1 "SageAttention与稀疏线性注意力机制": the standard attention
         formula softmax(QK^T/sqrt(d))V, the linear-attention form
         phi(Q)(phi(K)^T V) with phi = ReLU or elu+1, and SLA's top-k key
         selection T_k; §3.2 API example: attention_type="sagesla",
         sla_topk=0.1; §5.3: sla_topk=0.15 for more detail.
* [COM]  "清华开源TurboDiffusion加速框架：视频生成提升200倍，迈入秒级时代"
         (commentary), section "SageAttention与稀疏计算": SageAttention runs
         attention with low-bit integer (INT8) arithmetic; SLA skips about
         90% of attention connections, keeps about 10%, and is built on top
         of SageAttention.
* [DIG]  "TurboDiffusion" tool digest, section "使用方式与安装": SageSLA is the
         SageAttention-based fast SLA forward pass; section "训练": SLA is
         trained white-box, aligned to the full-attention model.
* [NEWS] TurboDiffusion news summary (jiqiren.org.cn), section "方法论": full
         attention is replaced by SLA and the pretrained model is fine-tuned
         to the sparsity.

What the oracle computes, per (batch, head), with blocks of ``block`` tokens
(Nb = ceil(N / block), the last block may be ragged; only valid rows count):

 1. K channel mean mu (fp64 sums, rows then blocks ascending, one fp64 divide,
    rounded to fp32) -- the K smoothing of low-bit SageAttention.
 2. Block-mean-pooled qbar, kbar of the raw inputs (fp64 sums, rounded to fp32).
 3. Block scores s_ij = sum_c qbar_ic kbar_jc in fp64 (c ascending); each query
    block keeps the k = topk_count(Nb, keep) highest-scoring key blocks, equal
    scores going to the lower key-block index [TUT §2.1 T_k; COM].
 4. Per-block symmetric INT8 quantisation of Q and of K - mu, computed in fp32
    exactly as specified in ``quantize_blocks`` [COM].
 5. Softmax branch: exact softmax attention of each query over the valid keys
    of its selected blocks, logits = (int8 dot product) * sq * sk / sqrt(d)
    [TUT §2.1 standard attention, restricted to the selected blocks].
 6. Linear branch over the valid keys of the unselected blocks U:
    phi(q)^T H_U / phi(q)^T z_U with H_U = sum_u phi(k_u) v_u^T and
    z_U = sum_u phi(k_u); zero when U is empty or the denominator is zero
    [TUT §2.1 linear attention, normalised].
 7. Output = softmax branch + linear branch.
 8. Backward (``sla_backward_head``): dQ, dK, dV of that output for a given
    output gradient, the selection held fixed, the INT8 rounding passed
    straight through [NEWS 方法论: SLA is fine-tuned into the model].
 9. Lower-bit option (``phi_k_fp8``): the linear branch's key features
    phi(K) rounded to FP8 (e4m3) with one power-of-two scale per key block,
    as a lower-bit variant of the low-bit attention arithmetic [COM: INT8 /
    INT4 SageAttention]; see ``phi_k_e4m3_blocks``.

The pages print the SLA formula as phi(Q)(T_k[phi(K)]^T V), which has no
softmax part; read together with the description of SLA as low-rank
approximation plus key-token selection [TUT §2.1] and with the kept ~10% being
computed by SageAttention [COM], this oracle takes the two-branch reading
above.  Everything is fp64 except the quantiser, whose fp32 steps are part of
its definition so that codes, scales and integer accumulators are comparable
bit for bit.
"""
from __future__ import annotations

import math

import numpy as np

PHI_NONE, PHI_ELU1, PHI_RELU = 0, 1, 2
_PHI_NAMES = {"none": PHI_NONE, "elu1": PHI_ELU1, "relu": PHI_RELU}


def phi_code(phi) -> int:
    if isinstance(phi, str):
        return _PHI_NAMES[phi]
    return int(phi)


# --------------------------------------------------------------------------
# sizes
# --------------------------------------------------------------------------
def topk_count(n_blocks: int, keep: float) -> int:
    """Number of key blocks each query block keeps.

    The pages give the keep fraction as "top k%" / sla_topk=0.1 [TUT §2.1,
    §3.2] and "about 10% kept" [COM] but not the rounding.  Reading: round up
    (keep at least the requested fraction), at least one block when keep > 0,
    with a 1e-9 guard so 0.1*30 = 3.0000000000000004 counts as 3.
    """
    if keep <= 0.0:
        return 0
    if keep >= 1.0:
        return n_blocks
    return min(n_blocks, max(1, int(math.ceil(keep * n_blocks - 1e-9))))


def n_blocks(N: int, block: int) -> int:
    return (N + block - 1) // block


def block_rows(N: int, block: int) -> np.ndarray:
    """Valid row count of every block (block, except possibly the last)."""
    nb = n_blocks(N, block)
    rows = np.full(nb, block, dtype=np.int64)
    rows[-1] = N - (nb - 1) * block
    return rows


# --------------------------------------------------------------------------
# element helpers
# --------------------------------------------------------------------------
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32, exact (bf16 is the top half of fp32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


def phi(x: np.ndarray, kind) -> np.ndarray:
    """Feature map of the linear branch [TUT §2.1]: elu+1 or ReLU, fp64."""
    kind = phi_code(kind)
    x = np.asarray(x, dtype=np.float64)
    if kind == PHI_ELU1:
        return np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))
    if kind == PHI_RELU:
        return np.maximum(x, 0.0)
    raise ValueError("phi 'none' has no feature map")


# --------------------------------------------------------------------------
# 1-2: block sums, pooled means, K channel mean
# --------------------------------------------------------------------------
def block_sums(x64: np.ndarray, block: int) -> np.ndarray:
    """fp64 per-block, per-channel sums over the valid rows, rows ascending.

    ``np.cumsum`` adds strictly in order, so the last cumulative row is the
    sequential sum row 0 + row 1 + ... of the block.
    """
    N, d = x64.shape
    out = np.empty((n_blocks(N, block), d), dtype=np.float64)
    for i in range(out.shape[0]):
        out[i] = np.cumsum(x64[i * block:min(N, (i + 1) * block)], axis=0)[-1]
    return out


def pooled_means(x_bits: np.ndarray, block: int) -> np.ndarray:
    """Block means fp32((sum over valid rows) / rows), from the raw bf16 input."""
    x64 = bf16_to_f64(x_bits)
    sums = block_sums(x64, block)
    rows = block_rows(x64.shape[0], block).astype(np.float64)
    return (sums / rows[:, None]).astype(np.float32)


def key_channel_mean(k_bits: np.ndarray, block: int) -> np.ndarray:
    """K smoothing mean mu_c = fp32((sum over blocks of block sums) / N).

    Block sums are added blocks ascending (cumsum), then one fp64 division.
    """
    k64 = bf16_to_f64(k_bits)
    sums = block_sums(k64, block)
    total = np.cumsum(sums, axis=0)[-1]
    return (total / float(k64.shape[0])).astype(np.float32)


# --------------------------------------------------------------------------
# 4: INT8 quantisation (fp32 definition)
# --------------------------------------------------------------------------
def quantize_blocks(x32: np.ndarray, block: int):
    """Symmetric per-block INT8 codes of an fp32 [N, d] matrix.

    Low-bit SageAttention quantises Q and K to INT8 [COM]; the pages do not
    give the granularity or rounding.  Reading: one scale per block of rows
    (all d channels), in fp32:
        a     = max |x| over the block's valid rows and all channels
        scale = fp32(a / 127),  inv = fp32(127 / a)
        code  = clamp(round_half_even(fp32(x * inv)), -127, 127)
    A block with a = 0 gets scale 0 and all-zero codes.  Rows past N (the pad
    of the ragged last block) get code 0.  Returns codes int8 [Nb*block, d]
    and scales fp32 [Nb].
    """
    x32 = np.asarray(x32, dtype=np.float32)
    N, d = x32.shape
    nb = n_blocks(N, block)
    codes = np.zeros((nb * block, d), dtype=np.int8)
    scales = np.zeros(nb, dtype=np.float32)
    f127 = np.float32(127.0)
    for i in range(nb):
        xb = x32[i * block:min(N, (i + 1) * block)]
        a = np.float32(np.max(np.abs(xb)))
        if a == np.float32(0.0):
            continue
        scales[i] = a / f127
        inv = f127 / a
        y = (xb * inv).astype(np.float32)
        c = np.clip(np.rint(y), -127.0, 127.0)
        codes[i * block:i * block + xb.shape[0]] = c.astype(np.int8)
    return codes, scales


def quantize_qk(q_bits: np.ndarray, k_bits: np.ndarray, block: int, smooth: bool = True):
    """INT8 codes and scales of Q and of K - mu (mu: K channel mean).

    x_Q = fp32(Q); x_K = fp32(K) - mu as one fp32 subtraction.  With
    ``smooth=False`` the mean is not subtracted (used only to show its effect).
    Returns (q8, k8, q_scale, k_scale, mu).
    """
    q32 = bf16_to_f32(q_bits)
    k32 = bf16_to_f32(k_bits)
    mu = key_channel_mean(k_bits, block)
    kx = (k32 - mu[None, :]).astype(np.float32) if smooth else k32
    q8, sq = quantize_blocks(q32, block)
    k8, sk = quantize_blocks(kx, block)
    return q8, k8, sq, sk, mu


# --------------------------------------------------------------------------
# 3: block scores and top-k selection
# --------------------------------------------------------------------------
def block_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """s_ij = sum_c qbar_ic * kbar_jc in fp64, channels added in ascending order.

    The product of two fp32 values is exact in fp64, so each step rounds once.
    The pages do not name the ranking score; this takes the plainest one, the
    dot product of the block means of raw Q and K (scaling by 1/sqrt(d) or a
    softmax over a row would not change the ranking).
    """
    qb = np.asarray(qbar, dtype=np.float32).astype(np.float64)
    kb = np.asarray(kbar, dtype=np.float32).astype(np.float64)
    s = np.zeros((qb.shape[0], kb.shape[0]), dtype=np.float64)
    for c in range(qb.shape[1]):
        s += np.multiply.outer(qb[:, c], kb[:, c])
    return s


def select_blocks(scores: np.ndarray, k: int) -> np.ndarray:
    """Top-k key blocks of every row: score descending, ties to the lower index.

    A stable sort of the negated scores orders by score descending and keeps
    equal scores in index order; the first k are kept, returned ascending.
    """
    order = np.argsort(-scores, axis=1, kind="stable")[:, :k]
    return np.sort(order, axis=1).astype(np.int32)


def block_mask(idx: np.ndarray, nb: int) -> np.ndarray:
    m = np.zeros((idx.shape[0], nb), dtype=bool)
    for i in range(idx.shape[0]):
        m[i, idx[i]] = True
    return m


def select_head(q_bits, k_bits, block: int, keep: float):
    """(idx [Nb, k] int32 ascending, scores fp64 [Nb, Nb]) for one head."""
    qbar = pooled_means(q_bits, block)
    kbar = pooled_means(k_bits, block)
    s = block_scores(qbar, kbar)
    k = topk_count(s.shape[1], keep)
    return select_blocks(s, k), s


# --------------------------------------------------------------------------
# 9: FP8 (e4m3) key features for the lower-bit option
# --------------------------------------------------------------------------
def round_e4m3(x: np.ndarray) -> np.ndarray:
    """Round to the nearest FP8 e4m3 value, ties to the even mantissa.

    e4m3: sign, 4 exponent bits (bias 7), 3 mantissa bits; normal values
    (1 + m/8) 2^(e-7) for e = 1..15 up to 448, subnormals (m/8) 2^-6.  The
    spacing in [2^e, 2^(e+1)) is 2^(e-3), and 2^-9 below 2^-6.  Inputs here
    are non-negative and below 448 (no overflow handling needed)."""
    a = np.asarray(x, dtype=np.float64)
    e = np.floor(np.log2(np.maximum(np.abs(a), 2.0 ** -6)))
    q = 2.0 ** (e - 3)
    return np.sign(a) * np.round(np.abs(a) / q) * q      # np.round: half to even


def phi_k_e4m3_blocks(fk: np.ndarray, block: int) -> np.ndarray:
    """phi(K) [N, d] rounded to e4m3 with one power-of-two scale per block.

    Per block of `block` rows: m = the largest feature of the block (valid
    rows, all channels); with e = floor(log2 m), the features are scaled by
    2^(7-e) (so the largest lands in [128, 256), inside e4m3's range),
    rounded to e4m3 and scaled back.  A block whose features are all zero
    stays zero."""
    fk = np.asarray(fk, dtype=np.float64)
    out = np.zeros_like(fk)
    for i in range(n_blocks(fk.shape[0], block)):
        b = fk[i * block:(i + 1) * block]
        m = float(b.max())
        if m <= 0.0:
            continue
        s = 7 - math.floor(math.log2(m))
        out[i * block:(i + 1) * block] = round_e4m3(b * 2.0 ** s) * 2.0 ** -s
    return out


# --------------------------------------------------------------------------
# 5-7: the two branches and their sum
# --------------------------------------------------------------------------
def _rows_of(blocks, N: int, block: int) -> np.ndarray:
    if len(blocks) == 0:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([np.arange(j * block, min(N, (j + 1) * block)) for j in blocks])


def block_logits(i, sel, q8, k8, sq, sk, N, block, d, q64=None, k64=None):
    """Logits of query block i against the valid keys of blocks ``sel``.

    acc * sq_i * sk_j / sqrt(d), acc the exact integer dot product of the INT8
    codes (an fp64 matrix product: every partial sum is an integer below 2^53,
    so it is exact in any order); with ``q64``/``k64`` given, QK^T/sqrt(d) of
    those fp64 matrices instead.  Returns (logits, acc or None).
    """
    qrows = np.arange(i * block, min(N, (i + 1) * block))
    krows = _rows_of(sel, N, block)
    if q64 is None:
        acc = q8[qrows].astype(np.float64) @ k8[krows].astype(np.float64).T
        kscale = np.repeat(sk[np.asarray(sel)].astype(np.float64),
                           [min(N, (j + 1) * block) - j * block for j in sel])
        return acc * float(sq[i]) * kscale[None, :] / math.sqrt(d), acc
    return (q64[qrows] @ k64[krows].T) / math.sqrt(d), None


def softmax_branch_block(i, sel, q8, k8, sq, sk, v64, N, block, d,
                         q64=None, k64=None):
    """Softmax attention of query block i over the valid keys of blocks ``sel``.

    Logits from ``block_logits`` (INT8, or exact with ``q64``/``k64``).
    Returns (out [rows, d], acc or None).
    """
    qrows = np.arange(i * block, min(N, (i + 1) * block))
    krows = _rows_of(sel, N, block)
    if krows.size == 0:
        return np.zeros((qrows.size, v64.shape[1])), None
    logits, acc = block_logits(i, sel, q8, k8, sq, sk, N, block, d, q64, k64)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    return (p @ v64[krows]) / p.sum(axis=1, keepdims=True), acc


def linear_branch_block(i, sel, q64, k64, v64, N, block, phi_kind, fk_all=None):
    """Normalised linear attention of query block i over the unselected blocks.

    Direct sums over U = valid rows of every key block not in ``sel``:
        out = phi(Q_i) H_U / (phi(Q_i) z_U),  H_U = phi(K_U)^T V_U,  z_U = sum phi(K_U)
    phi acts on the raw inputs [TUT §2.1].  Rows whose U is empty or whose
    denominator is zero get 0.  ``fk_all`` [N, d], when given, replaces
    phi(K) (the lower-bit option's rounded features).
    """
    nb = n_blocks(N, block)
    qrows = np.arange(i * block, min(N, (i + 1) * block))
    unsel = np.setdiff1d(np.arange(nb), np.asarray(sel, dtype=np.int64))
    urows = _rows_of(unsel, N, block)
    out = np.zeros((qrows.size, v64.shape[1]))
    if urows.size == 0:
        return out
    fk = phi(k64[urows], phi_kind) if fk_all is None else fk_all[urows]
    H = fk.T @ v64[urows]
    z = fk.sum(axis=0)
    fq = phi(q64[qrows], phi_kind)
    num = fq @ H
    den = fq @ z
    ok = den != 0.0
    out[ok] = num[ok] / den[ok, None]
    return out


def sla_forward_head(q_bits, k_bits, v_bits, block: int = 64, keep: float = 0.1,
                     phi_kind="elu1", query_blocks=None, quantize: bool = True,
                     smooth: bool = True, idx=None, phi_k_fp8: bool = False):
    """SageSLA forward of one (batch, head); inputs are bf16 bits [N, d].

    ``query_blocks`` restricts the output to those query blocks (the selection,
    mean and quantisation still use the whole head).  ``quantize=False``
    replaces the INT8 logits with exact fp64 ones; ``idx`` overrides the
    selection (for constructed masks); ``phi_k_fp8`` takes the linear
    branch's phi(K) rounded to e4m3 per key block (``phi_k_e4m3_blocks``).
    Returns a dict with
    out / out_softmax / out_linear (fp64, rows of the requested blocks in
    order), rows, idx, scores, q8, k8, q_scale, k_scale, mu.
    """
    phi_kind = phi_code(phi_kind)
    q_bits = np.asarray(q_bits)
    N, d = q_bits.shape
    nb = n_blocks(N, block)
    k = topk_count(nb, keep)
    if k == 0 and phi_kind == PHI_NONE:
        raise ValueError("keep = 0 with phi = none computes nothing")
    scores = None
    if idx is None:
        idx, scores = select_head(q_bits, k_bits, block, keep)
    q8, k8, sq, sk, mu = quantize_qk(q_bits, k_bits, block, smooth=smooth)
    q64, k64, v64 = bf16_to_f64(q_bits), bf16_to_f64(k_bits), bf16_to_f64(v_bits)
    fk_all = None
    if phi_k_fp8 and phi_kind != PHI_NONE:
        fk_all = phi_k_e4m3_blocks(phi(k64, phi_kind), block)
    qb = list(range(nb)) if query_blocks is None else list(query_blocks)
    outs_s, outs_l, rows = [], [], []
    for i in qb:
        sel = np.asarray(idx[i])
        os_, _ = softmax_branch_block(i, sel, q8, k8, sq, sk, v64, N, block, d,
                                      q64=None if quantize else q64,
                                      k64=None if quantize else k64)
        outs_s.append(os_)
        if phi_kind != PHI_NONE:
            outs_l.append(linear_branch_block(i, sel, q64, k64, v64, N, block, phi_kind, fk_all))
        else:
            outs_l.append(np.zeros_like(os_))
        rows.append(np.arange(i * block, min(N, (i + 1) * block)))
    o_s = np.concatenate(outs_s)
    o_l = np.concatenate(outs_l)
    return {"out": o_s + o_l, "out_softmax": o_s, "out_linear": o_l,
            "rows": np.concatenate(rows), "idx": idx, "scores": scores,
            "q8": q8, "k8": k8, "q_scale": sq, "k_scale": sk, "mu": mu}


def qk_accumulator(q8, k8, i: int, j: int, block: int) -> np.ndarray:
    """Integer Q.K^T tile of query block i and key block j (pad rows included)."""
    a = q8[i * block:(i + 1) * block].astype(np.int64)
    b = k8[j * block:(j + 1) * block].astype(np.int64)
    return a @ b.T


# --------------------------------------------------------------------------
# 8: backward (trainable SLA)
# --------------------------------------------------------------------------
def phi_grad(x: np.ndarray, kind) -> np.ndarray:
    """Derivative of the feature map: elu+1 -> 1 (x > 0) or exp(x); ReLU -> 1 (x > 0) or 0.

    At x = 0 both take the left-hand value (exp(0) = 1 for elu+1, 0 for ReLU).
    """
    kind = phi_code(kind)
    x = np.asarray(x, dtype=np.float64)
    if kind == PHI_ELU1:
        return np.where(x > 0.0, 1.0, np.exp(np.minimum(x, 0.0)))
    if kind == PHI_RELU:
        return np.where(x > 0.0, 1.0, 0.0)
    raise ValueError("phi 'none' has no feature map")


def softmax_branch_grad_block(i, sel, q64, k64, v64, do64, N, block, logits):
    """Gradients of the softmax branch of query block i (fp64).

    ``logits`` [rows_i, keys of sel] are the forward's logits.  With P the row
    softmax, O_s = P V and the loss gradient dO:
        dP = dO V^T,  D = rowsum(dO * O_s),  dL = P * (dP - D)
        dQ_i += dL K / sqrt(d),  dK += dL^T Q_i / sqrt(d),  dV += P^T dO.
    The logits are differentiated as QK^T/sqrt(d) of the real-valued inputs:
    the INT8 rounding passes the gradient straight through, and the K mean
    subtracted before coding adds the same amount to every logit of a row,
    which the softmax cancels.  Returns (qrows, krows, dq_i, dk_rows, dv_rows).
    """
    d = q64.shape[1]
    qrows = np.arange(i * block, min(N, (i + 1) * block))
    krows = _rows_of(sel, N, block)
    if krows.size == 0:
        z = np.zeros((0, d))
        return qrows, krows, np.zeros((qrows.size, d)), z, z
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    p = e / e.sum(axis=1, keepdims=True)
    g = do64[qrows]
    o_s = p @ v64[krows]
    dp = g @ v64[krows].T
    dl = p * (dp - (g * o_s).sum(axis=1, keepdims=True))
    s = 1.0 / math.sqrt(d)
    return qrows, krows, (dl @ k64[krows]) * s, (dl.T @ q64[qrows]) * s, p.T @ g


def linear_branch_grad_block(i, sel, q64, k64, v64, do64, N, block, phi_kind):
    """Gradients of the linear branch of query block i (fp64).

    Forward: O_l = num / den, num = phi(Q_i) H_U, den = phi(Q_i) z_U over the
    unselected rows U.  With g = dO:
        dnum = g / den,  dden = -(g . O_l) / den
        dphi(Q_i) = dnum H_U^T + dden z_U^T
        dH_U = phi(Q_i)^T dnum,  dz_U = phi(Q_i)^T dden
        dphi(K_u) = V_u dH_U^T + dz_U,  dV_u = phi(K_u) dH_U
    and dX = dphi(X) * phi'(X).  Rows whose forward output is 0 (U empty or a
    zero denominator) pass no gradient.  Returns (qrows, urows, dq_i, dk_u, dv_u).
    """
    d = q64.shape[1]
    nb = n_blocks(N, block)
    qrows = np.arange(i * block, min(N, (i + 1) * block))
    unsel = np.setdiff1d(np.arange(nb), np.asarray(sel, dtype=np.int64))
    urows = _rows_of(unsel, N, block)
    dq = np.zeros((qrows.size, d))
    if urows.size == 0:
        z = np.zeros((0, d))
        return qrows, urows, dq, z, z
    fk = phi(k64[urows], phi_kind)
    H = fk.T @ v64[urows]
    z = fk.sum(axis=0)
    fq = phi(q64[qrows], phi_kind)
    num = fq @ H
    den = fq @ z
    ok = den != 0.0
    g = np.where(ok[:, None], do64[qrows], 0.0)
    safe = np.where(ok, den, 1.0)
    o_l = num / safe[:, None]
    dnum = g / safe[:, None]
    dden = -(g * o_l).sum(axis=1) / safe
    dfq = dnum @ H.T + np.outer(dden, z)
    dq = dfq * phi_grad(q64[qrows], phi_kind)
    dH = fq.T @ dnum
    dz = fq.T @ dden
    dfk = v64[urows] @ dH.T + dz[None, :]
    dk = dfk * phi_grad(k64[urows], phi_kind)
    dv = fk @ dH
    return qrows, urows, dq, dk, dv


def sla_backward_head(q_bits, k_bits, v_bits, do_bits, block: int = 64, keep: float = 0.1,
                      phi_kind="elu1", quantize: bool = True, smooth: bool = True, idx=None,
                      query_blocks=None):
    """Gradients (dQ, dK, dV) of the SageSLA forward of one (batch, head).

    SLA is trained: full attention is swapped for it and the model fine-tuned
    [NEWS 方法论], with white-box alignment to full attention [DIG 训练],
    so the forward has a gradient.  The selection is a fixed mask (top-k has
    none); the softmax branch uses the forward's logits (INT8 or, with
    ``quantize=False``, exact) and differentiates them as exact QK^T/sqrt(d);
    the linear branch is differentiated exactly.  Inputs are bf16 bits [N, d];
    ``do_bits`` is the loss gradient of the output.  ``query_blocks``
    restricts the sum to those query blocks' contributions (their dQ rows are
    then complete; dK and dV hold only their share).  Returns a dict with
    dq, dk, dv (fp64 [N, d]) and idx.
    """
    phi_kind = phi_code(phi_kind)
    q_bits = np.asarray(q_bits)
    N, d = q_bits.shape
    nb = n_blocks(N, block)
    k = topk_count(nb, keep)
    if k == 0 and phi_kind == PHI_NONE:
        raise ValueError("keep = 0 with phi = none computes nothing")
    if idx is None:
        idx, _ = select_head(q_bits, k_bits, block, keep)
    q8, k8, sq, sk, _ = quantize_qk(q_bits, k_bits, block, smooth=smooth)
    q64, k64, v64 = bf16_to_f64(q_bits), bf16_to_f64(k_bits), bf16_to_f64(v_bits)
    do64 = bf16_to_f64(do_bits)
    dq = np.zeros((N, d))
    dk = np.zeros((N, d))
    dv = np.zeros((N, d))
    for i in (range(nb) if query_blocks is None else query_blocks):
        sel = np.asarray(idx[i])
        if sel.size:
            logits, _ = block_logits(i, sel, q8, k8, sq, sk, N, block, d,
                                     None if quantize else q64, None if quantize else k64)
            qr, kr, a, b, c = softmax_branch_grad_block(i, sel, q64, k64, v64, do64, N, block,
                                                        logits)
            dq[qr] += a
            dk[kr] += b
            dv[kr] += c
        if phi_kind != PHI_NONE:
            qr, ur, a, b, c = linear_branch_grad_block(i, sel, q64, k64, v64, do64, N, block,
                                                       phi_kind)
            dq[qr] += a
            dk[ur] += b
            dv[ur] += c
    return {"dq": dq, "dk": dk, "dv": dv, "idx": idx}
