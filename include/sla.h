/*
 * sla.h -- C ABI of libsla.so, the MI355X (gfx950) SageSLA attention forward.
 *
 * SageSLA is the SageAttention-based fast forward pass of sparse-linear
 * attention (SLA): tool digest "TurboDiffusion", section "使用方式与安装".
 * Each query block of `block` tokens keeps its top `keep` fraction of key
 * blocks (the pipeline knob sla_topk=0.1 of tutorial "TurboDiffusion技术架构解析：
 * 稀疏线性注意力应用实战" §3.2; "about 10% kept" in commentary "清华开源
 * TurboDiffusion加速框架：视频生成提升200倍，迈入秒级时代", section
 * "SageAttention与稀疏计算") and runs exact softmax attention softmax(QK^T/sqrt(d))V
 * on them (tutorial §2.1, standard attention) with Q.K^T on INT8 codes
 * (commentary, same section: low-bit SageAttention).  The remaining key blocks
 * are summarised by normalised linear attention phi(Q)(phi(K)^T V) with phi =
 * elu+1 or ReLU (tutorial §2.1, linear attention), and the two outputs are
 * summed.
 *
 * Conventions shared by every entry point
 *  - Tensors are device pointers (memory from hipMalloc / torch on the GPU),
 *    contiguous row-major [B, H, N, d] with d fastest, 16-byte aligned.
 *    bf16 tensors are passed as raw 16-bit patterns (`const void*`).
 *  - Supported shapes: block == 64 and d == 128 (SLA_ERR_UNSUPPORTED
 *    otherwise); B, H, N >= 1; N <= 2^20; 0 <= keep <= 1.
 *  - Blocks: Nb = ceil(N / 64); the last block may be ragged; rows past N
 *    ("pad rows") never take part in any sum, maximum or softmax.
 *  - The caller allocates and owns every buffer, including the workspace
 *    (size from sla_workspace_bytes, or sla_workspace_size per operation).
 *    The library allocates no device memory and keeps no global mutable
 *    state, so it may be called from several threads; calls on different
 *    streams are independent as long as their workspaces differ.
 *  - All work of a call is enqueued on `stream` (a hipStream_t; NULL = the
 *    default stream), in order, and the call returns without synchronising;
 *    a call is capturable in a HIP graph, its first call included.
 *    Arguments are validated before anything is enqueued: on any error
 *    status nothing has been enqueued.  SLA_ERR_DEVICE reports a failed
 *    kernel launch (hipGetLastError) or attribute set.
 *  - Outputs must not alias inputs or the workspace.
 *  - Numeric range: inputs must be finite.  V is staged in fp16, so |V| must
 *    stay below 65504; entries below 2^-14 in magnitude keep an absolute
 *    precision of 2^-25.  The linear branch stages phi(K)/16 in fp16
 *    (phi(K) up to 2^20; elu+1 features below 2^-20, i.e. K entries below
 *    about -13.8, count as zero) and phi(q) scaled per row so that its
 *    largest feature lies in [1, 2) (the branch is a ratio, so the factor
 *    cancels); features below 2^-24 of a row's largest count as zero.
 */
#ifndef SLA_H_
#define SLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SLA_BLOCK 64
#define SLA_HEAD_DIM 128
#define SLA_MAX_TOKENS (1 << 20)
#define SLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

typedef enum sla_status {
  SLA_OK = 0,
  SLA_ERR_INVALID_ARG = 1, /* null pointer, bad size, keep outside [0,1], ... */
  SLA_ERR_UNSUPPORTED = 2, /* valid request this build does not implement     */
  SLA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required      */
  SLA_ERR_DEVICE = 4,      /* a HIP call or kernel launch failed              */
  SLA_ERR_SCRATCH = 5      /* shape needs more than sla_attention_fwd_noalloc's
                              static scratch (SLA_NOALLOC_SCRATCH_BYTES)       */
} sla_status;

typedef enum sla_phi {
  SLA_PHI_NONE = 0, /* linear branch off                          */
  SLA_PHI_ELU1 = 1, /* phi(x) = x + 1 for x > 0, exp(x) otherwise */
  SLA_PHI_RELU = 2  /* phi(x) = max(x, 0)                         */
} sla_phi;

typedef enum sla_out_dtype {
  SLA_OUT_BF16 = 0, /* bf16 output, round-to-nearest-even of the fp32 result */
  SLA_OUT_F32 = 1   /* fp32 output                                           */
} sla_out_dtype;

typedef enum sla_op {
  SLA_OP_QUANTIZE = 0,
  SLA_OP_SELECT = 1,
  SLA_OP_ATTENTION = 2,
  SLA_OP_ATTENTION_BWD = 3
} sla_op;

/* Number of key blocks every query block keeps: 0 if keep <= 0, n_blocks if
 * keep >= 1, else min(n_blocks, max(1, ceil(keep * n_blocks - 1e-9))).  The
 * pages give the fraction (sla_topk, "top k%") but not the rounding; this
 * rounds up so at least the requested fraction is kept.  Pure host function;
 * returns -1 if n_blocks < 1 or keep is NaN. */
int32_t sla_topk_count(int32_t n_blocks, double keep);

/* Workspace bytes of the SageSLA forward for this shape, keep and phi (an
 * sla_phi): enough for each of sla_quantize_qk, sla_block_select and
 * sla_attention_fwd on the same B, H, N.  Pure host function; returns 0 when
 * the arguments are not a valid sla_attention_fwd call (as it validates
 * them), so 0 never sizes a usable workspace. */
size_t sla_workspace_bytes(int B, int H, int N, int d, int block, double keep,
                           int phi);

/* Workspace bytes `op` needs for this shape, written to *bytes.  `keep` and
 * `phi` matter only for SLA_OP_ATTENTION and SLA_OP_ATTENTION_BWD (pass 0
 * otherwise).  Pure host function; validates like the op itself. */
sla_status sla_workspace_size(int op, int B, int H, int N, int d, int block,
                              double keep, int phi, size_t *bytes);

/* Per-block INT8 quantisation of Q and of mean-smoothed K (low-bit
 * SageAttention, commentary section "SageAttention与稀疏计算"; the K channel
 * mean is subtracted before quantising, which leaves each softmax row
 * unchanged since q.(k - mu) = q.k - q.mu is constant along the row).
 *   q, k      bf16 [B,H,N,128]                                    (in)
 *   k_mean    fp32 [B,H,128]: mu_c = fp32((sum over all N rows of K[.,c],
 *             fp64, rows ascending within blocks, blocks ascending) / N)  (out)
 *   q_i8,k_i8 int8 [B,H,Nb*64,128]; pad rows are 0                  (out)
 *   q_scale,k_scale fp32 [B,H,Nb]                                   (out)
 * Per block, on x = fp32(Q) or x = fp32(K) - mu (one fp32 subtraction):
 *   a = max |x| over valid rows and all channels; scale = fp32(a/127);
 *   code = clamp(rint_half_even(fp32(x * fp32(127/a))), -127, 127);
 *   a == 0 gives scale 0 and zero codes.
 * Workspace: sla_workspace_size(SLA_OP_QUANTIZE, ...). */
sla_status sla_quantize_qk(const void *q, const void *k, int B, int H, int N,
                           int d, int block, int8_t *q_i8, int8_t *k_i8,
                           float *q_scale, float *k_scale, float *k_mean,
                           void *ws, size_t ws_bytes, void *stream);

/* Key-block selection T_k (tutorial §2.1): for every query block i, the
 * k = sla_topk_count(Nb, keep) key blocks j with the largest score
 *   s_ij = sum_c qbar_ic * kbar_jc   (fp64, channels ascending),
 * where qbar/kbar are the fp32-rounded block means of the raw Q and K
 * (fp64 row sums / valid rows).  Equal scores go to the lower j.
 *   kblock_idx  int32 [B,H,Nb,k], ascending within each row           (out)
 *   kblock_mask uint32 [B,H,Nb,ceil(Nb/32)] bit j%32 of word j/32 set iff j
 *               is kept; may be NULL                                  (out)
 * keep must be > 0 (k >= 1).  Workspace: SLA_OP_SELECT. */
sla_status sla_block_select(const void *q, const void *k, int B, int H, int N,
                            int d, int block, double keep, int32_t *kblock_idx,
                            uint32_t *kblock_mask, void *ws, size_t ws_bytes,
                            void *stream);

/* The SageSLA forward.  For query t of block i with kept set S_i:
 *   softmax branch: softmax over the valid keys u of S_i of
 *       acc_tu * q_scale_i * k_scale_j / sqrt(128)   (acc: exact int32 dot
 *       product of the INT8 codes), applied to V (P and V in fp16 on the
 *       matrix cores, fp32 accumulation, normaliser summed from the fp16 P);
 *       zero when k == 0;
 *   linear branch (phi != NONE): over the valid keys U of the other blocks,
 *       phi(q)^T (sum_U phi(k_u) v_u^T) / phi(q)^T (sum_U phi(k_u)), phi on
 *       the raw Q and K; zero when U is empty or the denominator vanishes;
 *   out = softmax branch + linear branch.
 *   q, k, v     bf16 [B,H,N,128]                                       (in)
 *   keep        kept fraction, 0..1; keep == 0 requires phi != NONE
 *   phi         sla_phi
 *   out         [B,H,N,128], bf16 or fp32 per out_dtype                 (out)
 * Workspace: sla_workspace_bytes (holds codes, selection, fp16 staging and
 * the linear state, about 3 bytes per element of Q).  Every stage runs on
 * `stream`, in the order listed under sla_stage. */
sla_status sla_attention_fwd(const void *q, const void *k, const void *v,
                             int B, int H, int N, int d, int block, double keep,
                             int phi, void *out, int out_dtype, void *ws,
                             size_t ws_bytes, void *stream);

/* Stages of sla_attention_fwd, all on the caller's stream in the order
 * STATS, TOPK, SCHEDULE, KMEAN, LINEAR_PREP, LINEAR_FINAL, SPARSE.  The INT8
 * coding is folded into STATS (Q) and LINEAR_PREP (K), so QUANTIZE, the
 * coding as a pass of its own (sla_quantize_qk), records nothing here. */
typedef enum sla_stage {
  SLA_STAGE_STATS = 0,        /* fp64 block sums, pooled block means of Q and K,  */
                              /* INT8 codes and scales of Q                       */
  SLA_STAGE_KMEAN = 1,        /* K channel mean                                   */
  SLA_STAGE_QUANTIZE = 2,     /* INT8 coding on its own: not run by this call     */
  SLA_STAGE_TOPK = 3,         /* block scores and top-k key-block selection       */
  SLA_STAGE_LINEAR_PREP = 4,  /* fp16 staging of V and phi(K), partial phi(K)^T V,*/
                              /* INT8 codes and scales of smoothed K              */
  SLA_STAGE_LINEAR_FINAL = 5, /* whole-head phi(K)^T V and sum phi(K)             */
  SLA_STAGE_SPARSE = 6,       /* block-sparse attention + linear branch + combine */
  SLA_STAGE_SCHEDULE = 7,     /* aligned key-block walks of query-block groups    */
  SLA_N_STAGES = 8
} sla_stage;

/* Options of sla_attention_fwd_ex (bit flags). */
#define SLA_OPT_PHI_K_FP8 1 /* lower-bit option, see sla_attention_fwd_lowbit */

/* sla_attention_fwd with optional extras, for tests and measurement:
 *   out_linear    fp32 [B,H,N,128], the linear branch alone, or NULL   (out)
 *   stage_events  NULL, or 2 * SLA_N_STAGES caller-created HIP events
 *                 (hipEvent_t, same device; any entry may be NULL):
 *                 stage_events[2*s] is recorded on `stream` just before
 *                 stage s and stage_events[2*s+1] just after.  Stages a
 *                 call skips (selection and schedule when keep == 0, the
 *                 schedule when the linear branch takes the direct form,
 *                 linear stages when phi == NONE, QUANTIZE always) record
 *                 nothing.
 *   options       0, or SLA_OPT_PHI_K_FP8 (other bits: SLA_ERR_INVALID_ARG)
 * With NULL, NULL, 0 it is exactly sla_attention_fwd.  Same arguments,
 * ownership and errors; a failed hipEventRecord gives SLA_ERR_DEVICE. */
sla_status sla_attention_fwd_ex(const void *q, const void *k, const void *v,
                                int B, int H, int N, int d, int block,
                                double keep, int phi, void *out, int out_dtype,
                                float *out_linear, void *ws, size_t ws_bytes,
                                void *stream, void *const *stage_events,
                                int options);

/* sla_attention_fwd with the selection on a second stream: after the
 * statistics pass (on `stream`), the block scores, the top-k selection and the
 * walk schedule run on `side` while the K mean and the linear staging run on
 * `stream`; `stream` waits for `side` before the attention kernel.  `side` is
 * a caller-owned HIP stream of the same device (hipStream_t; NULL or equal to
 * `stream`: exactly sla_attention_fwd).  The call creates two HIP events and
 * releases them (the runtime frees them once the work they mark is done); it
 * allocates no device memory.  The output equals sla_attention_fwd's bit for
 * bit (the same kernels on the same data).  Work left on `side` after the
 * call: none that `stream` does not wait for.  Same arguments, ownership and
 * errors as sla_attention_fwd; a failed event or stream call gives
 * SLA_ERR_DEVICE. */
sla_status sla_attention_fwd_fork(const void *q, const void *k, const void *v,
                                  int B, int H, int N, int d, int block,
                                  double keep, int phi, void *out,
                                  int out_dtype, void *ws, size_t ws_bytes,
                                  void *stream, void *side);

/* The forward with a lower-bit linear branch, an opt-in variant with its own
 * accuracy (the pages run SLA on low-bit INT8/INT4 SageAttention: commentary
 * "清华开源TurboDiffusion加速框架", section "SageAttention与稀疏计算").  The
 * linear branch's key features phi(K) are kept as FP8 e4m3 codes with one
 * power-of-two scale per 64-key block: the block's largest feature m is
 * scaled by 2^(7 - floor(log2 m)) into [128, 256) and every feature rounded
 * to nearest-even e4m3 (three mantissa bits, subnormals below 2^-6).  The
 * whole-head sums and the kept blocks' share use the same rounded features,
 * so the result is the exact forward with phi(K) replaced by its rounded
 * value (bit-level rounding decisions can differ from an fp64 evaluation of
 * phi only where phi lies within an fp32 rounding of an e4m3 midpoint).  It
 * moves 32 instead of 40 KB per kept (query block, key block) pair.  The
 * softmax branch is unchanged.  Same arguments, workspace, ownership and
 * errors as sla_attention_fwd. */
sla_status sla_attention_fwd_lowbit(const void *q, const void *k,
                                    const void *v, int B, int H, int N, int d,
                                    int block, double keep, int phi, void *out,
                                    int out_dtype, void *ws, size_t ws_bytes,
                                    void *stream);

/* sla_attention_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the workspace is a static device array of the library,
 * SLA_NOALLOC_SCRATCH_BYTES (64 MiB) on each device, which that device holds
 * until the process ends.  The call itself allocates nothing; the caller
 * passes inputs and output as for sla_attention_fwd (same arguments,
 * numerics and errors, bit-identical output).  Shapes whose workspace
 * (sla_workspace_bytes) exceeds the scratch are rejected with
 * SLA_ERR_SCRATCH before anything is enqueued (e.g. B*H = 2 at N = 2048 needs
 * 6.4 MiB, one head at N = 32760 28.6 MiB).  Every call on a device shares its
 * scratch and nothing in it needs to start at zero; calls that overlap on one
 * device (other streams, other threads) race on it, so the caller orders
 * them.  The first call on a device looks up the scratch's device address
 * (kept per device for the life of the process). */
sla_status sla_attention_fwd_noalloc(const void *q, const void *k,
                                     const void *v, int B, int H, int N, int d,
                                     int block, double keep, int phi, void *out,
                                     int out_dtype, void *stream);

/* Gradients of sla_attention_fwd (same q, k, v, keep, phi) for the output
 * gradient dout.  SLA is fine-tuned into the model it accelerates (news
 * summary, section "方法论"; tool digest, section "训练"), so the forward is
 * differentiated:
 *   - the kept lists are those of the forward and are held fixed;
 *   - softmax branch: P are the forward's weights (INT8 logits, fp16 P,
 *     1/l from the fp16 sum) and the logits are differentiated as
 *     QK^T/sqrt(128) of the real Q and K (the INT8 rounding passes the
 *     gradient straight through; the K mean shifts a row's logits equally
 *     and has no gradient):  dP = dout V^T, D = rowsum(dout * O_softmax),
 *     dS = P (dP - D);  dQ += dS K / sqrt(128), dK += dS^T Q / sqrt(128),
 *     dV += P^T dout;
 *   - linear branch: exact, with phi'(x) = 1 for x > 0, else exp(x) (elu+1)
 *     or 0 (ReLU); rows whose forward linear output is zero pass nothing.
 * The selection, codes and linear state are recomputed (nothing is carried
 * over from a forward call).  The linear branch is taken in the subtraction
 * form for every keep < 1.
 *   q, k, v, dout bf16 [B,H,N,128]                                     (in)
 *   dq, dk, dv    [B,H,N,128], bf16 or fp32 per grad_dtype (sla_out_dtype)
 *                 (out; every element written)
 * Arithmetic: INT8 matrix cores for the logits, bf16 matrix cores with fp32
 * accumulation for every other product (P and dS rounded to bf16), fp32
 * elsewhere.  Workspace: SLA_OP_ATTENTION_BWD (about 13 bytes per element of
 * Q at keep 0.1).  All work runs on `stream`.  Errors as sla_attention_fwd;
 * dout and the three outputs must be 16-byte aligned. */
sla_status sla_attention_bwd(const void *q, const void *k, const void *v,
                             const void *dout, int B, int H, int N, int d,
                             int block, double keep, int phi, void *dq,
                             void *dk, void *dv, int grad_dtype, void *ws,
                             size_t ws_bytes, void *stream);

/* Stages of sla_attention_bwd, all on the caller's stream in this order. */
typedef enum sla_bwd_stage {
  SLA_BWD_STAGE_FWD_STAGING = 0, /* the forward's statistics, selection, walk
                                    schedule, K mean and linear staging           */
  SLA_BWD_STAGE_TRANSPOSE = 1,   /* K^T, dO^T per block                           */
  SLA_BWD_STAGE_COLUMNS = 2,     /* per key block, the query blocks keeping it    */
  SLA_BWD_STAGE_QUERY = 3,       /* query side: dQ, row statistics                */
  SLA_BWD_STAGE_GRAD_H = 4,      /* whole-head linear-gradient sums               */
  SLA_BWD_STAGE_KEY = 5,         /* key side: dK, dV                              */
  SLA_BWD_N_STAGES = 6
} sla_bwd_stage;

/* sla_attention_bwd that also records caller-created HIP events (hipEvent_t,
 * same device) on `stream` around its stages: stage_events[2*s] just before
 * stage s and stage_events[2*s+1] just after.  stage_events is NULL or holds
 * 2 * SLA_BWD_N_STAGES entries, any of which may be NULL; stages a call skips
 * (COLUMNS when keep == 0, GRAD_H without the linear branch) record nothing.
 * Same arguments, ownership and errors as sla_attention_bwd; a failed
 * hipEventRecord gives SLA_ERR_DEVICE. */
sla_status sla_attention_bwd_timed(const void *q, const void *k, const void *v,
                                   const void *dout, int B, int H, int N, int d,
                                   int block, double keep, int phi, void *dq,
                                   void *dk, void *dv, int grad_dtype, void *ws,
                                   size_t ws_bytes, void *stream,
                                   void *const *stage_events);

/* ---- Training: a forward that keeps what the backward needs ----------------
 * SLA is fine-tuned into the model it accelerates (news summary, section
 * "方法论"), so a training step runs the forward and then the backward on the
 * same q, k, v.  sla_attention_fwd_train is sla_attention_fwd that also
 * writes, into a caller-owned residual buffer, what the backward's query side
 * would otherwise recompute with a second pass over the kept tiles, and the
 * forward's staging that the backward would otherwise rebuild:
 *   stats  fp32 [B,H,N,2]   per row: log2-domain maximum of the logits (+inf
 *                           for a row without kept keys) and 1/l
 *   os     fp32 [B,H,N,128] the softmax branch's normalised output
 *   ol     fp32 [B,H,N,128] the linear branch's output          (linear only)
 *   m      bf16 [B,H,Nb,128,128] per query block the kept tiles' share
 *                           M = sum phi(K_j)^T V_j (phi(K)/16 scale, row =
 *                           phi channel)            (subtraction form only)
 *   zm     fp32 [B,H,Nb,128] the kept share of sum phi(K)/16 (same)
 *   then, except in the direct form, when k > 0:
 *   codes  q8 int8 [B,H,Nb*64,128], sq fp32 [B,H,Nb],
 *                           k8 int8 [B,H,Nb*64,128], sk fp32 [B,H,Nb] (as
 *                           sla_quantize_qk), idx int32 [B,H,Nb,k] (as
 *                           sla_block_select), and the query-block groups'
 *                           aligned walks int32 [B,H,ceil(Nb/4),k,4]
 *   and, with the linear branch: hb bf16 [B,H,128,128] H = sum phi(K)^T V
 *                           (phi(K)/16 scale, row = phi channel), z fp32
 *                           [B,H,128] sum phi(K)/16
 * each piece 256-byte aligned, in this order; the subtraction form is taken
 * when the unselected key blocks outnumber the kept ones (Nb - k > k), the
 * direct form otherwise (with the linear branch on).
 * sla_train_residual_bytes gives the size (0 for invalid arguments). */
size_t sla_train_residual_bytes(int B, int H, int N, int d, int block,
                                double keep, int phi);

/* Same arguments, validation, ownership and errors as sla_attention_fwd, plus
 * the residual buffer (device memory, 16-byte aligned, at least
 * sla_train_residual_bytes; SLA_ERR_INVALID_ARG otherwise), every byte of
 * which the call writes for valid rows.  Exact mode only (no lower-bit
 * option).  The output equals sla_attention_fwd's bit for bit. */
sla_status sla_attention_fwd_train(const void *q, const void *k,
                                   const void *v, int B, int H, int N, int d,
                                   int block, double keep, int phi, void *out,
                                   int out_dtype, void *resid,
                                   size_t resid_bytes, void *ws,
                                   size_t ws_bytes, void *stream);

/* sla_attention_bwd for the residuals of a sla_attention_fwd_train call on the
 * same q, k, v, keep and phi (resid, resid_bytes as given to it): the query
 * side takes the forward's row statistics, outputs and kept share from them
 * instead of walking the kept tiles a second time, and the forward's codes,
 * selection, walks and linear state replace the backward's own staging.  Gradients equal
 * sla_attention_bwd's to rounding (the linear output comes from the forward's
 * fp32 H - M instead of a bf16-staged recomputation).  In the direct form
 * (Nb - k <= k) the residuals hold no kept share and the call computes as
 * sla_attention_bwd.  stage_events as sla_attention_bwd_timed (NULL: none).
 * Errors as sla_attention_bwd; a null, misaligned or short resid gives
 * SLA_ERR_INVALID_ARG. */
sla_status sla_attention_bwd_saved(const void *q, const void *k, const void *v,
                                   const void *dout, const void *resid,
                                   size_t resid_bytes, int B, int H, int N,
                                   int d, int block, double keep, int phi,
                                   void *dq, void *dk, void *dv, int grad_dtype,
                                   void *ws, size_t ws_bytes, void *stream,
                                   void *const *stage_events);

/* ---- W8A8 INT8 linear layers and FusedNorm ----------------------------------
 * Weights and activations of the linear layers quantised to 8 bits for the
 * INT8 units (news summary, opening component list; commentary, section
 * "步数蒸馏与W8A8量化"), with a fused normalisation in front of them (blog,
 * section "1. 计算资源优化：CPU Offload与混合精度计算").  The quantiser is the one
 * of sla_quantize_qk applied per row: a = max|x| over the row, scale =
 * fp32(a/127), code = clamp(rint_half_even(fp32(x * fp32(127/a))), +-127),
 * a == 0 giving scale 0 and zero codes.  Row lengths K: multiples of 64,
 * 64 <= K <= 16384.  All pointers are device pointers, 16-byte aligned; work
 * is enqueued on `stream`; no workspace. */

/* Per-row INT8 codes of a bf16 [rows, K] matrix: a weight matrix [N, K] per
 * output channel, or activations [M, K] per token.
 *   x      bf16 [rows, K]                                            (in)
 *   codes  int8 [rows, K]; scale fp32 [rows]                         (out) */
sla_status sla_rowquant_i8(const void *x, int rows, int K, int8_t *codes,
                           float *scale, void *stream);

/* FusedNorm: LayerNorm of every row of x, an optional per-channel affine
 * (which also expresses adaptive-norm modulation: gamma = 1 + scale, beta =
 * shift), then the per-row INT8 codes of the result, in one pass.
 *   mu = fp32(sum(x)/K) with the sum in fp64; var = sum((x - mu)^2)/K in fp64;
 *   rstd = fp32(1/sqrt(var + eps)); then in fp32, in this order:
 *   y = x - mu; y = y * rstd; y = y * gamma[k]; y = y + beta[k].
 *   x            bf16 [rows, K]                                      (in)
 *   gamma, beta  fp32 [K] each, or NULL (omitted step)               (in)
 *   eps          > 0 (Wan's LayerNorm uses 1e-6)
 *   codes int8 [rows, K], scale fp32 [rows]                          (out)
 *   mean, rstd   fp32 [rows] each, or NULL                           (out) */
sla_status sla_fused_norm_i8(const void *x, int rows, int K, const float *gamma,
                             const float *beta, float eps, int8_t *codes,
                             float *scale, float *mean, float *rstd,
                             void *stream);

/* W8A8 linear layer: y[m][n] = (sum_k x8[m][k] * w8[n][k]) * x_scale[m] *
 * w_scale[n] + bias[n], the integer sum exact (int32), the rest fp32.
 *   x8 int8 [M, K], x_scale fp32 [M]; w8 int8 [N, K], w_scale fp32 [N] (in)
 *   bias fp32 [N] or NULL                                             (in)
 *   y [M, N], bf16 (round to nearest even) or fp32 per out_dtype       (out)
 * K must be a multiple of 128 (128 <= K <= 16384) and N of 4; M * K and
 * N * K below 2^31.  x8, w8, y, both scale arrays and bias are 16-byte
 * aligned (SLA_ERR_INVALID_ARG otherwise). */
sla_status sla_w8a8_linear(const int8_t *x8, const float *x_scale,
                           const int8_t *w8, const float *w_scale,
                           const float *bias, int M, int N, int K, void *y,
                           int out_dtype, void *stream);

/* Integer Q.K^T tiles from the attention kernel's INT8 matrix-core path, for
 * checking accumulators bit for bit.  pairs: int32 [n_pairs,4] device array
 * of (b, h, query block i, key block j); acc: int32 [n_pairs,64,64],
 * acc[p][r][c] = sum_e q_i8[b,h,64i+r,e] * k_i8[b,h,64j+c,e] (pad rows
 * included).  No workspace. */
sla_status sla_debug_qk_i32(const int8_t *q_i8, const int8_t *k_i8, int B,
                            int H, int N, int d, int block,
                            const int32_t *pairs, int n_pairs, int32_t *acc,
                            void *stream);

/* Static string naming a status code. */
const char *sla_status_string(int status);

/* ABI version: major * 10000 + minor * 100 + patch. */
int sla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SLA_H_ */
