// Internal declarations shared by the libsla host code and its HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace sla {

constexpr int kBlk = 64;        // tokens per query / key block
constexpr int kD = 128;         // head dimension
constexpr int kLinChunks = 24;  // key-block chunks per head in the linear-state reduction
constexpr int kMaxTokens = 1 << 20;  // largest N the entry points accept
constexpr int kGroup = 4;            // query blocks whose key-block walks are aligned
constexpr float kPhiScale = 0.0625f;  // phi(Q), phi(K) are staged in fp16 as phi/16
constexpr int kMaxRowK = 16384;       // longest row of the W8A8 quantisers

enum Phi { kPhiNone = 0, kPhiElu1 = 1, kPhiRelu = 2 };

// Lets `func` take up to `bytes` of dynamic LDS.  Set before every launch that
// needs it, so the library holds no state of its own.
inline hipError_t allow_lds(const void* func, int bytes) {
  return hipFuncSetAttribute(func, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

struct Shape {
  int B, H, N;
  int BH;   // B * H
  int Nb;   // ceil(N / 64)
  int Np;   // Nb * 64 (rows of the padded code / staging buffers)
  int k;    // kept key blocks per query block
};

// Device buffers carved out of the caller's workspace (null when unused).
struct Workspace {
  double* ksum = nullptr;     // [BH, Nb, D]   fp64 K block sums (for the K mean)
  float* qbar = nullptr;      // [BH, Nb, D]   fp32 Q block means
  float* kbar = nullptr;      // [BH, D, Nb]   fp32 K block means, channel-major
  // the filtered top-k (where it runs: Nb <= 1728; null otherwise)
  uint16_t* ksplit = nullptr; // [BH, ceil(Nb/16), 4, 2, 64, 8] bf16 splits of kbar
  uint8_t* kflag = nullptr;   // [BH, Nb]      key block mean out of the filter's range
  float* kbar_rm = nullptr;   // [BH, Nb, D]   fp32 K block means, row-major
  float* knorm = nullptr;     // [BH, Nb]      upper bound of each K block mean's 2-norm
  float* topk_scores = nullptr;  // [BH, Nb, Nb] approximate scores, then [BH, Nb, 8] row maxima
  uint32_t* redo = nullptr;   // [1 + BH * Nb] rows handed to the exact top-k: count, rows
  float* mu = nullptr;        // [BH, D]       K channel mean
  int8_t* q8 = nullptr;       // [BH, Np, D]   INT8 codes
  int8_t* k8 = nullptr;       // [BH, Np, D]
  float* sq = nullptr;        // [BH, Nb]      block scales
  float* sk = nullptr;        // [BH, Nb]
  int32_t* idx = nullptr;     // [BH, Nb, k]   kept key blocks, ascending
  int32_t* sched = nullptr;   // [BH, ceil(Nb/kGroup), k, kGroup] aligned walks of query-block
                              // groups: key block, -1 for none
  uint16_t* fk16 = nullptr;   // [BH, Nb, D, 64] fp16 phi(K)/16 per block, [channel][permuted key]
  uint16_t* v16 = nullptr;    // [BH, Nb, D, 64] fp16 V per block, [channel][permuted key]
  float* zb = nullptr;        // [BH, Nb, D]   fp32 per-block sum of phi(K)/16 over the keys
  float* fkscale = nullptr;   // [BH, Nb]      FP8 phi(K) tiles (lower-bit option): code -> phi/16
  float* hpart = nullptr;     // [BH, kLinChunks, D, D] partial phi(K)^T V
  double* zpart = nullptr;    // [BH, kLinChunks, D]    partial sums of the block sums zb
  float* hf = nullptr;        // [BH, 4, 8, 2, 64, 4] fp32 H = sum phi(K)/16 ^T V in the
                              // attention kernel's M^T register layout (see sla_sparse.hip)
  double* z64 = nullptr;      // [BH, D] fp64 sum of zb over all key blocks
  uint16_t* h16t = nullptr;   // [BH, D(out), D(in)] fp16 H^T * 2^-s      (backward)
  float* hscale = nullptr;    // [BH] 2^s                                  (backward)
  float* z = nullptr;         // [BH, D] fp32 sum phi(K)/16               (backward)
};

// Extra device buffers of the backward (null when unused).
struct BwdWorkspace {
  uint16_t* hb = nullptr;     // [BH, D, D]     bf16 H row-major (staged scale, phi/16)
  uint16_t* kt = nullptr;     // [BH, Nb, D, 64] bf16 K^T per block, [channel][permuted key]
  uint16_t* dot = nullptr;    // [BH, Nb, D, 64] bf16 dO^T per block
  uint16_t* fqs = nullptr;    // [BH, Nb, D, 64] bf16 (phi(Q)/den)^T per block
  float* stats = nullptr;     // [BH, Nb, kBwdStatFloats] per row: log2 max, 1/l, D (row
                              // order), u (permuted order)
  uint32_t* maskT = nullptr;  // [BH, Nb, ceil(Nb/32)] query blocks keeping each key block
  int32_t* coff = nullptr;    // [BH, Nb + 1] column starts in cidx (per head)
  int32_t* cidx = nullptr;    // [BH, Nb * k] query blocks per key block (group order)
  float* gpart = nullptr;     // [BH, kGradChunks, D, D] partial G
  float* gzpart = nullptr;    // [BH, kGradChunks, D]    partial g_z
  float* G = nullptr;         // [BH, D, D] sum of (phi(Q)/den)^T dO over all rows
  float* gz = nullptr;        // [BH, D]    sum of (phi(Q)/den)^T u
};
constexpr int kGradChunks = 32;  // query-block chunks per head in the G reduction
constexpr int kBwdStatFloats = 4 * kBlk;  // per query block: four rows of 64 statistics

// Stage launchers (all enqueue on `s`, return the launch status).
// Block means and K block sums; also Q's INT8 codes and scales when q8 is set.
hipError_t launch_block_stats(const uint16_t* q, const uint16_t* k, const Shape& sh,
                              double* ksum, float* qbar, float* kbar, int8_t* q8, float* sq,
                              uint16_t* ksplit, uint8_t* kflag, float* kbar_rm, float* knorm,
                              hipStream_t s);
hipError_t launch_key_mean(const double* ksum, const Shape& sh, float* mu, hipStream_t s);
hipError_t launch_quantize(const uint16_t* q, const uint16_t* k, const float* mu,
                           const Shape& sh, int8_t* q8, int8_t* k8, float* sq, float* sk,
                           bool k_only, hipStream_t s);
// The filtered top-k's buffers (all null: the exact kernel selects every row).
struct TopkFilter {
  float* scores = nullptr;
  const uint16_t* ksplit = nullptr;
  const uint8_t* kflag = nullptr;
  const float* kbar_rm = nullptr;
  const float* knorm = nullptr;
  uint32_t* redo = nullptr;
};
// Bytes of TopkFilter::scores for BH heads of Nb blocks; 0 where the filter does not run.
size_t topk_filter_bytes(int BH, int Nb);
// Kept lists (and the optional bitmask): the filtered passes and then the
// exact kernel on the rows they hand over where `f` is set and the filter
// applies, else the exact kernel on every row.
hipError_t launch_block_topk(const float* qbar, const float* kbar, const TopkFilter& f,
                             const Shape& sh, int32_t* idx, uint32_t* mask, hipStream_t s);
// The same selection in two parts, for callers that build the walk schedule
// in between: the first pass (the filtered kernels where they apply, else the
// exact kernel on every row; *handed_back is the hand-back list, or null when
// the exact kernel already did everything), then the exact kernel on that list.
hipError_t launch_block_topk_first(const float* qbar, const float* kbar, const TopkFilter& f,
                                   const Shape& sh, int32_t* idx, uint32_t* mask, hipStream_t s,
                                   const uint32_t** handed_back);
hipError_t launch_block_topk_redo(const float* qbar, const float* kbar, const TopkFilter& f,
                                  const Shape& sh, int32_t* idx, uint32_t* mask, hipStream_t s);
size_t topk_lds_bytes(int Nb, int* rows_per_group);
// fp8: stage phi(K) as e4m3 codes (8 KB per block, a head's blocks at the
// start of its fk16 slice) with per-block decode scales in fkscale.
hipError_t launch_linear_prep(const uint16_t* k, const uint16_t* v, const Shape& sh, int phi,
                              bool reduce, uint16_t* fk16, uint16_t* v16, float* zb, float* hpart,
                              double* zpart, const float* mu, int8_t* k8, float* sk, bool fp8,
                              float* fkscale, hipStream_t s);
// Whole-head linear state from the chunk partials.  The forward takes hf and
// z64; the backward z, h16t, hscale and hb (bf16 H row-major); null outputs
// are skipped.
hipError_t launch_linear_final(float* hpart, const double* zpart, const Shape& sh, float* hf,
                               double* z64, float* z, uint16_t* h16t, float* hscale,
                               uint16_t* hb, hipStream_t s);
// Linear-branch form: with few unselected blocks (Nb - k <= k) the branch is
// summed directly over them; otherwise as whole-head sums minus the kept share.
inline bool linear_direct(const Shape& sh) { return sh.Nb - sh.k <= sh.k; }
// Aligned walks of the query-block groups from the kept lists (ws.sched);
// needed by launch_sparse_fwd unless the linear branch takes the direct form.
hipError_t launch_group_schedule(const int32_t* idx, const Shape& sh, int32_t* sched,
                                 hipStream_t s, const uint32_t* only_if = nullptr);
// What a training forward keeps for the backward (sla_attention_fwd_train);
// m and zm only in the subtraction form.
struct TrainResiduals {
  float* stats = nullptr;   // [BH, N, 2] log2-domain row maximum (+inf: no weights), 1/l
  float* os = nullptr;      // [BH, N, 128] normalised softmax-branch output
  float* ol = nullptr;      // [BH, N, 128] linear-branch output
  uint16_t* m = nullptr;    // [BH, Nb, 128, 128] bf16 kept share M, staged scale (phi/16)
  float* zm = nullptr;      // [BH, Nb, 128] kept share of z, staged scale
  // the forward's staging, taken over by the backward (null in the direct form)
  int8_t* q8 = nullptr;     // [BH, Np, 128] INT8 codes of Q and K, scales per block
  float* sq = nullptr;      // [BH, Nb]
  int8_t* k8 = nullptr;     // [BH, Np, 128]
  float* sk = nullptr;      // [BH, Nb]
  int32_t* idx = nullptr;   // [BH, Nb, k] kept key blocks
  int32_t* sched = nullptr; // [BH, ceil(Nb/kGroup), k, kGroup] aligned walks
  uint16_t* hb = nullptr;   // [BH, 128, 128] bf16 H row-major, staged scale  (linear only)
  float* z = nullptr;       // [BH, 128] fp32 sum of phi(K)/16              (linear only)
};
hipError_t launch_sparse_fwd(const uint16_t* q, const Workspace& ws, const Shape& sh, int phi,
                             void* out, int out_f32, float* out_linear, bool fp8,
                             const TrainResiduals* res, hipStream_t s);
// Backward launchers.
// Per block: K^T, dO^T as bf16 [channel][permuted row] (either may be null).
hipError_t launch_transpose_blocks(const uint16_t* k, const uint16_t* dout, const Shape& sh,
                                   uint16_t* kt, uint16_t* dot, hipStream_t s);
// Column lists: for every key block, the query blocks whose kept list holds it.
hipError_t launch_column_lists(const int32_t* idx, const Shape& sh, uint32_t* maskT,
                               int32_t* coff, int32_t* cidx, hipStream_t s);
// Query side of the backward; with `res` (a training forward's residuals) the
// forward's statistics, outputs and kept share are read instead of recomputed.
hipError_t launch_bwd_q(const uint16_t* q, const uint16_t* v, const uint16_t* dout,
                        const Workspace& ws, const BwdWorkspace& bw, const Shape& sh, int phi,
                        void* dq, int grad_f32, const TrainResiduals* res, hipStream_t s);
// G = sum over all rows of (phi(Q)/den)^T dO and g_z (from bwd_q's outputs).
hipError_t launch_grad_h(const BwdWorkspace& bw, const Shape& sh, hipStream_t s);
hipError_t launch_bwd_kv(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                         const Workspace& ws, const BwdWorkspace& bw, const Shape& sh, int phi,
                         void* dk, void* dv, int grad_f32, hipStream_t s);
// W8A8: per-row INT8 codes of a bf16 [rows, K] matrix, LayerNorm-ed first
// (and scaled/shifted per channel) when norm is set; and the INT8 GEMM.
hipError_t launch_rowquant(const uint16_t* x, int rows, int K, bool norm, const float* gamma,
                           const float* beta, float eps, int8_t* codes, float* scale, float* mu,
                           float* rstd, hipStream_t s);
hipError_t launch_w8a8_gemm(const int8_t* x8, const float* sx, const int8_t* w8, const float* sw,
                            const float* bias, int M, int N, int K, void* y, int out_f32,
                            hipStream_t s);
hipError_t launch_debug_qk(const int8_t* q8, const int8_t* k8, const Shape& sh,
                           const int32_t* pairs, int n_pairs, int32_t* acc, hipStream_t s);

}  // namespace sla
