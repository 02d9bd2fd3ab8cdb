// C ABI of libsla.so: argument validation, workspace carving and the launch
// sequence of the SageSLA forward.  Nothing is enqueued unless every argument
// checks out; kernels run on the caller's stream without host synchronisation.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/sla.h"
#include "sla_internal.h"

namespace {

using sla::Shape;
using sla::Workspace;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static_assert(SLA_MAX_TOKENS == sla::kMaxTokens, "token limit differs between the header and the kernels");

sla_status check_shape(int B, int H, int N, int d, int block) {
  if (B < 1 || H < 1 || N < 1) return SLA_ERR_INVALID_ARG;
  if (d != SLA_HEAD_DIM || block != SLA_BLOCK) return SLA_ERR_UNSUPPORTED;
  if (N > SLA_MAX_TOKENS) return SLA_ERR_UNSUPPORTED;
  if ((long long)B * H > (1 << 20)) return SLA_ERR_UNSUPPORTED;
  return SLA_OK;
}

Shape make_shape(int B, int H, int N, int k) {
  Shape s;
  s.B = B;
  s.H = H;
  s.N = N;
  s.BH = B * H;
  s.Nb = (N + SLA_BLOCK - 1) / SLA_BLOCK;
  s.Np = s.Nb * SLA_BLOCK;
  s.k = k;
  return s;
}

// Carves the workspace for `op`; with base == nullptr only the size is computed.
// The backward's extra buffers go to `bw`.
sla::TopkFilter topk_filter(const Workspace& w) {
  sla::TopkFilter f;
  f.scores = w.topk_scores;
  f.ksplit = w.ksplit;
  f.kflag = w.kflag;
  f.kbar_rm = w.kbar_rm;
  f.knorm = w.knorm;
  f.redo = w.redo;
  return f;
}

size_t carve(int op, const Shape& s, int phi, unsigned char* base, Workspace* w,
             sla::BwdWorkspace* bw = nullptr) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> unsigned char* {
    unsigned char* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  const size_t BH = (size_t)s.BH, Nb = (size_t)s.Nb, Np = (size_t)s.Np, D = SLA_HEAD_DIM;
  Workspace tmp;
  Workspace& ws = w ? *w : tmp;
  ws.ksum = reinterpret_cast<double*>(take(BH * Nb * D * sizeof(double)));
  ws.qbar = reinterpret_cast<float*>(take(BH * Nb * D * sizeof(float)));
  ws.kbar = reinterpret_cast<float*>(take(BH * Nb * D * sizeof(float)));
  if (const size_t fb = sla::topk_filter_bytes(s.BH, s.Nb)) {
    ws.ksplit = reinterpret_cast<uint16_t*>(take(BH * ((Nb + 15) / 16) * 4 * 2 * 512 * sizeof(uint16_t)));
    ws.kflag = take(BH * Nb);
    ws.kbar_rm = reinterpret_cast<float*>(take(BH * Nb * D * sizeof(float)));
    ws.knorm = reinterpret_cast<float*>(take(BH * Nb * sizeof(float)));
    ws.redo = reinterpret_cast<uint32_t*>(take((1 + BH * Nb) * sizeof(uint32_t)));
    ws.topk_scores = reinterpret_cast<float*>(take(fb));
  }
  if (op == SLA_OP_ATTENTION_BWD) {
    // the forward's buffers in the subtraction form, then the backward's
    const bool lin = phi != SLA_PHI_NONE && s.k < s.Nb;
    ws.mu = reinterpret_cast<float*>(take(BH * D * sizeof(float)));
    ws.q8 = reinterpret_cast<int8_t*>(take(BH * Np * D));
    ws.k8 = reinterpret_cast<int8_t*>(take(BH * Np * D));
    ws.sq = reinterpret_cast<float*>(take(BH * Nb * sizeof(float)));
    ws.sk = reinterpret_cast<float*>(take(BH * Nb * sizeof(float)));
    ws.idx = reinterpret_cast<int32_t*>(take(BH * Nb * (size_t)(s.k > 0 ? s.k : 1) * sizeof(int32_t)));
    ws.v16 = reinterpret_cast<uint16_t*>(take(BH * Np * D * sizeof(uint16_t)));
    if (s.k > 0)
      ws.sched = reinterpret_cast<int32_t*>(
          take(BH * (size_t)((s.Nb + sla::kGroup - 1) / sla::kGroup) * s.k * sla::kGroup * sizeof(int32_t)));
    sla::BwdWorkspace tb;
    sla::BwdWorkspace& b = bw ? *bw : tb;
    if (lin) {
      ws.fk16 = reinterpret_cast<uint16_t*>(take(BH * Np * D * sizeof(uint16_t)));
      ws.zb = reinterpret_cast<float*>(take(BH * Nb * D * sizeof(float)));
      ws.hpart = reinterpret_cast<float*>(take(BH * sla::kLinChunks * D * D * sizeof(float)));
      ws.zpart = reinterpret_cast<double*>(take(BH * sla::kLinChunks * D * sizeof(double)));
      ws.h16t = reinterpret_cast<uint16_t*>(take(BH * D * D * sizeof(uint16_t)));
      ws.hscale = reinterpret_cast<float*>(take(BH * sizeof(float)));
      ws.z = reinterpret_cast<float*>(take(BH * D * sizeof(float)));
      b.hb = reinterpret_cast<uint16_t*>(take(BH * D * D * sizeof(uint16_t)));
      b.fqs = reinterpret_cast<uint16_t*>(take(BH * Np * D * sizeof(uint16_t)));
      b.gpart = reinterpret_cast<float*>(take(BH * sla::kGradChunks * D * D * sizeof(float)));
      b.gzpart = reinterpret_cast<float*>(take(BH * sla::kGradChunks * D * sizeof(float)));
      b.G = reinterpret_cast<float*>(take(BH * D * D * sizeof(float)));
      b.gz = reinterpret_cast<float*>(take(BH * D * sizeof(float)));
    }
    b.kt = reinterpret_cast<uint16_t*>(take(BH * Np * D * sizeof(uint16_t)));
    b.dot = reinterpret_cast<uint16_t*>(take(BH * Np * D * sizeof(uint16_t)));
    b.stats = reinterpret_cast<float*>(take(BH * Nb * sla::kBwdStatFloats * sizeof(float)));
    if (s.k > 0) {
      b.maskT = reinterpret_cast<uint32_t*>(take(BH * Nb * (size_t)((s.Nb + 31) / 32) * sizeof(uint32_t)));
      b.coff = reinterpret_cast<int32_t*>(take(BH * (Nb + 1) * sizeof(int32_t)));
      b.cidx = reinterpret_cast<int32_t*>(take(BH * Nb * (size_t)s.k * sizeof(int32_t)));
    }
  }
  if (op == SLA_OP_ATTENTION) {
    ws.mu = reinterpret_cast<float*>(take(BH * D * sizeof(float)));
    ws.q8 = reinterpret_cast<int8_t*>(take(BH * Np * D));
    ws.k8 = reinterpret_cast<int8_t*>(take(BH * Np * D));
    ws.sq = reinterpret_cast<float*>(take(BH * Nb * sizeof(float)));
    ws.sk = reinterpret_cast<float*>(take(BH * Nb * sizeof(float)));
    ws.idx = reinterpret_cast<int32_t*>(take(BH * Nb * (size_t)(s.k > 0 ? s.k : 1) * sizeof(int32_t)));
    ws.v16 = reinterpret_cast<uint16_t*>(take(BH * Np * D * sizeof(uint16_t)));
    const bool direct = phi != SLA_PHI_NONE && s.k < s.Nb && sla::linear_direct(s);
    if (!direct && s.k > 0)
      ws.sched = reinterpret_cast<int32_t*>(
          take(BH * (size_t)((s.Nb + sla::kGroup - 1) / sla::kGroup) * s.k * sla::kGroup * sizeof(int32_t)));
    if (direct) {
      ws.fk16 = reinterpret_cast<uint16_t*>(take(BH * Np * D * sizeof(uint16_t)));
      ws.zb = reinterpret_cast<float*>(take(BH * Nb * D * sizeof(float)));
      ws.fkscale = reinterpret_cast<float*>(take(BH * Nb * sizeof(float)));
    } else if (phi != SLA_PHI_NONE && s.k < s.Nb) {
      ws.fk16 = reinterpret_cast<uint16_t*>(take(BH * Np * D * sizeof(uint16_t)));
      ws.zb = reinterpret_cast<float*>(take(BH * Nb * D * sizeof(float)));
      ws.fkscale = reinterpret_cast<float*>(take(BH * Nb * sizeof(float)));
      ws.hpart = reinterpret_cast<float*>(take(BH * sla::kLinChunks * D * D * sizeof(float)));
      ws.zpart = reinterpret_cast<double*>(take(BH * sla::kLinChunks * D * sizeof(double)));
      ws.hf = reinterpret_cast<float*>(take(BH * D * D * sizeof(float)));
      ws.z64 = reinterpret_cast<double*>(take(BH * D * sizeof(double)));
    }
  }
  return off;
}

sla_status device_status(hipError_t e) { return e == hipSuccess ? SLA_OK : SLA_ERR_DEVICE; }

// The workspace of sla_attention_fwd_noalloc: a static device array, one copy
// per device, alive until the process ends.  In host code its name is only a
// stand-in; kernels get the device address that hipGetSymbolAddress returns,
// looked up once per device (with that device current) and kept here.
static_assert(SLA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[SLA_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// Argument checks of the forward that come before the workspace.
sla_status check_fwd_args(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                          int block, double keep, int phi, const void* out, int out_dtype,
                          const float* out_linear) {
  sla_status st = check_shape(B, H, N, d, block);
  if (st != SLA_OK) return st;
  if (!q || !k || !v || !out) return SLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (out_linear && !aligned16(out_linear)))
    return SLA_ERR_INVALID_ARG;
  if (std::isnan(keep) || keep < 0.0 || keep > 1.0) return SLA_ERR_INVALID_ARG;
  if (phi < SLA_PHI_NONE || phi > SLA_PHI_RELU) return SLA_ERR_INVALID_ARG;
  if (out_dtype != SLA_OUT_BF16 && out_dtype != SLA_OUT_F32) return SLA_ERR_INVALID_ARG;
  const int Nb = (N + SLA_BLOCK - 1) / SLA_BLOCK;
  const int kk = sla_topk_count(Nb, keep);
  if (kk == 0 && phi == SLA_PHI_NONE) return SLA_ERR_INVALID_ARG;
  int R = 1;
  if (kk > 0 && sla::topk_lds_bytes(Nb, &R) > 160 * 1024) return SLA_ERR_UNSUPPORTED;
  return SLA_OK;
}

// A training forward's residuals in the caller's buffer (256-byte aligned
// pieces): per-row statistics and softmax output, the linear output, and in
// the subtraction form the kept share M and z_M per query block, then the
// forward's staging that the backward takes over (INT8 codes and scales,
// kept lists and walks when k > 0; H in bf16 and z with the linear branch).
// Returns the bytes needed; fills *r when base is set.
size_t carve_residuals(const Shape& s, int phi_eff, bool direct, unsigned char* base,
                       sla::TrainResiduals* r) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    unsigned char* p = base ? base + off : nullptr;
    off += (bytes + 255) & ~size_t(255);
    return p;
  };
  const size_t BH = s.BH, N = s.N, Nb = s.Nb, D = SLA_HEAD_DIM;
  sla::TrainResiduals t;
  t.stats = reinterpret_cast<float*>(take(BH * N * 2 * sizeof(float)));
  t.os = reinterpret_cast<float*>(take(BH * N * D * sizeof(float)));
  if (phi_eff != SLA_PHI_NONE) {
    t.ol = reinterpret_cast<float*>(take(BH * N * D * sizeof(float)));
    if (!direct) {
      t.m = reinterpret_cast<uint16_t*>(take(BH * Nb * D * D * sizeof(uint16_t)));
      t.zm = reinterpret_cast<float*>(take(BH * Nb * D * sizeof(float)));
    }
  }
  if (!direct) {
    const size_t Np = s.Np, K = s.k > 0 ? s.k : 0;
    if (K > 0) {
      t.q8 = reinterpret_cast<int8_t*>(take(BH * Np * D));
      t.sq = reinterpret_cast<float*>(take(BH * Nb * sizeof(float)));
      t.k8 = reinterpret_cast<int8_t*>(take(BH * Np * D));
      t.sk = reinterpret_cast<float*>(take(BH * Nb * sizeof(float)));
      t.idx = reinterpret_cast<int32_t*>(take(BH * Nb * K * sizeof(int32_t)));
      t.sched = reinterpret_cast<int32_t*>(
          take(BH * (size_t)((s.Nb + sla::kGroup - 1) / sla::kGroup) * K * sla::kGroup * sizeof(int32_t)));
    }
    if (phi_eff != SLA_PHI_NONE) {
      t.hb = reinterpret_cast<uint16_t*>(take(BH * D * D * sizeof(uint16_t)));
      t.z = reinterpret_cast<float*>(take(BH * D * sizeof(float)));
    }
  }
  if (r) *r = t;
  return off;
}

}  // namespace

extern "C" {

int32_t sla_topk_count(int32_t n_blocks, double keep) {
  if (n_blocks < 1 || std::isnan(keep)) return -1;
  if (keep <= 0.0) return 0;
  if (keep >= 1.0) return n_blocks;
  const double c = std::ceil(keep * (double)n_blocks - 1e-9);
  int32_t k = (int32_t)c;
  if (k < 1) k = 1;
  if (k > n_blocks) k = n_blocks;
  return k;
}

sla_status sla_workspace_size(int op, int B, int H, int N, int d, int block, double keep,
                              int phi, size_t* bytes) {
  if (!bytes) return SLA_ERR_INVALID_ARG;
  *bytes = 0;
  const sla_status st = check_shape(B, H, N, d, block);
  if (st != SLA_OK) return st;
  if (op < SLA_OP_QUANTIZE || op > SLA_OP_ATTENTION_BWD) return SLA_ERR_INVALID_ARG;
  int k = 0;
  if (op == SLA_OP_ATTENTION || op == SLA_OP_ATTENTION_BWD) {
    if (std::isnan(keep) || keep < 0.0 || keep > 1.0) return SLA_ERR_INVALID_ARG;
    if (phi < SLA_PHI_NONE || phi > SLA_PHI_RELU) return SLA_ERR_INVALID_ARG;
    k = sla_topk_count((N + SLA_BLOCK - 1) / SLA_BLOCK, keep);
  }
  *bytes = carve(op, make_shape(B, H, N, k), phi, nullptr, nullptr);
  return SLA_OK;
}

size_t sla_workspace_bytes(int B, int H, int N, int d, int block, double keep, int phi) {
  size_t bytes = 0;
  if (sla_workspace_size(SLA_OP_ATTENTION, B, H, N, d, block, keep, phi, &bytes) != SLA_OK) return 0;
  if (phi == SLA_PHI_NONE && sla_topk_count((N + SLA_BLOCK - 1) / SLA_BLOCK, keep) == 0) return 0;
  return bytes;
}

sla_status sla_quantize_qk(const void* q, const void* k, int B, int H, int N, int d, int block,
                           int8_t* q_i8, int8_t* k_i8, float* q_scale, float* k_scale,
                           float* k_mean, void* ws, size_t ws_bytes, void* stream) {
  sla_status st = check_shape(B, H, N, d, block);
  if (st != SLA_OK) return st;
  if (!q || !k || !q_i8 || !k_i8 || !q_scale || !k_scale || !k_mean) return SLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_i8) || !aligned16(k_i8))
    return SLA_ERR_INVALID_ARG;
  const Shape s = make_shape(B, H, N, 0);
  const size_t need = carve(SLA_OP_QUANTIZE, s, SLA_PHI_NONE, nullptr, nullptr);
  if (!ws || ws_bytes < need || !aligned16(ws)) return SLA_ERR_WORKSPACE;
  Workspace w;
  carve(SLA_OP_QUANTIZE, s, SLA_PHI_NONE, static_cast<unsigned char*>(ws), &w);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const auto* qb = static_cast<const uint16_t*>(q);
  const auto* kb = static_cast<const uint16_t*>(k);
  hipError_t e = sla::launch_block_stats(qb, kb, s, w.ksum, w.qbar, w.kbar, q_i8, q_scale, nullptr, nullptr, nullptr, nullptr, hs);
  if (e == hipSuccess) e = sla::launch_key_mean(w.ksum, s, k_mean, hs);
  if (e == hipSuccess)
    e = sla::launch_quantize(qb, kb, k_mean, s, q_i8, k_i8, q_scale, k_scale, true, hs);
  return device_status(e);
}

sla_status sla_block_select(const void* q, const void* k, int B, int H, int N, int d, int block,
                            double keep, int32_t* kblock_idx, uint32_t* kblock_mask, void* ws,
                            size_t ws_bytes, void* stream) {
  sla_status st = check_shape(B, H, N, d, block);
  if (st != SLA_OK) return st;
  if (!q || !k || !kblock_idx) return SLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k)) return SLA_ERR_INVALID_ARG;
  if (std::isnan(keep) || keep <= 0.0 || keep > 1.0) return SLA_ERR_INVALID_ARG;
  const int Nb = (N + SLA_BLOCK - 1) / SLA_BLOCK;
  const Shape s = make_shape(B, H, N, sla_topk_count(Nb, keep));
  int R = 1;
  if (sla::topk_lds_bytes(Nb, &R) > 160 * 1024) return SLA_ERR_UNSUPPORTED;
  const size_t need = carve(SLA_OP_SELECT, s, SLA_PHI_NONE, nullptr, nullptr);
  if (!ws || ws_bytes < need || !aligned16(ws)) return SLA_ERR_WORKSPACE;
  Workspace w;
  carve(SLA_OP_SELECT, s, SLA_PHI_NONE, static_cast<unsigned char*>(ws), &w);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const auto* qb = static_cast<const uint16_t*>(q);
  const auto* kb = static_cast<const uint16_t*>(k);
  hipError_t e = sla::launch_block_stats(qb, kb, s, w.ksum, w.qbar, w.kbar, nullptr, nullptr, w.ksplit, w.kflag, w.kbar_rm, w.knorm, hs);
  if (e == hipSuccess)
    e = sla::launch_block_topk(w.qbar, w.kbar, topk_filter(w), s, kblock_idx, kblock_mask, hs);
  return device_status(e);
}

}  // extern "C"

namespace {

// The forward; with `res` it also writes a training forward's residuals.
// The forward.  With `side` (a second caller-owned stream, other than
// `stream`), the selection (block scores, top-k, walk schedule) runs on it,
// forked after the statistics pass and joined before the attention kernel,
// concurrently with the K mean and the linear staging on `stream`.
sla_status fwd_impl(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                    int block, double keep, int phi, void* out, int out_dtype, float* out_linear,
                    void* ws, size_t ws_bytes, void* stream, void* const* stage_events, int options,
                    const sla::TrainResiduals* res, void* side = nullptr) {
  const sla_status st =
      check_fwd_args(q, k, v, B, H, N, d, block, keep, phi, out, out_dtype, out_linear);
  if (st != SLA_OK) return st;
  if (options & ~SLA_OPT_PHI_K_FP8) return SLA_ERR_INVALID_ARG;
  const bool fp8 = (options & SLA_OPT_PHI_K_FP8) != 0;
  const int Nb = (N + SLA_BLOCK - 1) / SLA_BLOCK;
  const int kk = sla_topk_count(Nb, keep);
  const Shape s = make_shape(B, H, N, kk);
  const size_t need = carve(SLA_OP_ATTENTION, s, phi, nullptr, nullptr);
  if (!ws || ws_bytes < need || !aligned16(ws)) return SLA_ERR_WORKSPACE;
  Workspace w;
  carve(SLA_OP_ATTENTION, s, phi, static_cast<unsigned char*>(ws), &w);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const auto* qb = static_cast<const uint16_t*>(q);
  const auto* kb = static_cast<const uint16_t*>(k);
  const auto* vb = static_cast<const uint16_t*>(v);
  // the linear branch exists only when some key block is left out
  const int phi_eff = (kk < Nb) ? phi : SLA_PHI_NONE;
  const bool direct = phi_eff != SLA_PHI_NONE && sla::linear_direct(s);
  // a training forward writes the codes, kept lists and walks into the
  // residuals, where the backward takes them over
  if (res && res->q8) {
    w.q8 = res->q8;
    w.sq = res->sq;
    w.k8 = res->k8;
    w.sk = res->sk;
    w.idx = res->idx;
    w.sched = res->sched;
  }
  hipError_t e = hipSuccess;
  // runs one stage on the caller's stream between its two optional events
  auto stage = [&](int id, auto&& launch) {
    if (e != hipSuccess) return;
    if (stage_events && stage_events[2 * id])
      e = hipEventRecord(static_cast<hipEvent_t>(stage_events[2 * id]), hs);
    if (e == hipSuccess) e = launch();
    if (e == hipSuccess && stage_events && stage_events[2 * id + 1])
      e = hipEventRecord(static_cast<hipEvent_t>(stage_events[2 * id + 1]), hs);
  };
  // the selection's stream, and the fork and join events when it is `side`
  hipStream_t sel = hs;
  hipEvent_t fork = nullptr, join = nullptr;
  if (side && side != stream && kk > 0) {
    sel = static_cast<hipStream_t>(side);
    e = hipEventCreateWithFlags(&fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&join, hipEventDisableTiming);
  }
  if (kk > 0) {
    stage(SLA_STAGE_STATS, [&] {
      return sla::launch_block_stats(qb, kb, s, w.ksum, w.qbar, w.kbar, w.q8, w.sq, w.ksplit, w.kflag, w.kbar_rm, w.knorm, hs);
    });
    if (fork && e == hipSuccess) {
      e = hipEventRecord(fork, hs);
      if (e == hipSuccess) e = hipStreamWaitEvent(sel, fork, 0);
    }
    // the selection; rows the filtered top-k hands back to the exact kernel
    // (none on smooth inputs) are redone after the walk schedule, which is
    // then rebuilt only if there were any, so that the exact kernel's grid
    // does not wait for the CUs in front of the schedule
    const uint32_t* handed_back = nullptr;
    stage(SLA_STAGE_TOPK, [&] {
      return sla::launch_block_topk_first(w.qbar, w.kbar, topk_filter(w), s, w.idx, nullptr, sel,
                                          &handed_back);
    });
    // the aligned walks of the query-block groups, from the kept lists alone
    stage(SLA_STAGE_SCHEDULE, [&] {
      hipError_t r = direct ? hipSuccess : sla::launch_group_schedule(w.idx, s, w.sched, sel);
      if (r == hipSuccess && handed_back) {
        r = sla::launch_block_topk_redo(w.qbar, w.kbar, topk_filter(w), s, w.idx, nullptr, sel);
        if (r == hipSuccess && !direct) r = sla::launch_group_schedule(w.idx, s, w.sched, sel, handed_back);
      }
      return r;
    });
    if (join && e == hipSuccess) e = hipEventRecord(join, sel);
    stage(SLA_STAGE_KMEAN, [&] { return sla::launch_key_mean(w.ksum, s, w.mu, hs); });
  }
  // Q is coded by the statistics pass and K by the staging pass (one read of
  // each), so the QUANTIZE stage does not run here
  stage(SLA_STAGE_LINEAR_PREP, [&] {
    return sla::launch_linear_prep(kb, vb, s, phi_eff, !direct, w.fk16, w.v16, w.zb, w.hpart,
                                   w.zpart, w.mu, kk > 0 ? w.k8 : nullptr, w.sk, fp8, w.fkscale, hs);
  });
  if (phi_eff != SLA_PHI_NONE && !direct)
    stage(SLA_STAGE_LINEAR_FINAL, [&] {
      return sla::launch_linear_final(w.hpart, w.zpart, s, w.hf, w.z64, res ? res->z : nullptr,
                                      nullptr, nullptr, res ? res->hb : nullptr, hs);
    });
  if (join && e == hipSuccess) e = hipStreamWaitEvent(hs, join, 0);
  stage(SLA_STAGE_SPARSE, [&] {
    return sla::launch_sparse_fwd(qb, w, s, phi_eff, out, out_dtype == SLA_OUT_F32 ? 1 : 0,
                                  out_linear, fp8, res, hs);
  });
  // released by the runtime once the recorded work has completed
  if (fork) hipEventDestroy(fork);
  if (join) hipEventDestroy(join);
  return device_status(e);
}

}  // namespace

extern "C" {

sla_status sla_attention_fwd_ex(const void* q, const void* k, const void* v, int B, int H, int N,
                                int d, int block, double keep, int phi, void* out, int out_dtype,
                                float* out_linear, void* ws, size_t ws_bytes, void* stream,
                                void* const* stage_events, int options) {
  return fwd_impl(q, k, v, B, H, N, d, block, keep, phi, out, out_dtype, out_linear, ws, ws_bytes,
                  stream, stage_events, options, nullptr);
}

size_t sla_train_residual_bytes(int B, int H, int N, int d, int block, double keep, int phi) {
  if (check_shape(B, H, N, d, block) != SLA_OK) return 0;
  if (std::isnan(keep) || keep < 0.0 || keep > 1.0 || phi < SLA_PHI_NONE || phi > SLA_PHI_RELU) return 0;
  const int Nb = (N + SLA_BLOCK - 1) / SLA_BLOCK;
  const int kk = sla_topk_count(Nb, keep);
  if (kk == 0 && phi == SLA_PHI_NONE) return 0;
  const Shape s = make_shape(B, H, N, kk);
  const int phi_eff = (kk < Nb) ? phi : SLA_PHI_NONE;
  return carve_residuals(s, phi_eff, phi_eff != SLA_PHI_NONE && sla::linear_direct(s), nullptr, nullptr);
}

sla_status sla_attention_fwd_train(const void* q, const void* k, const void* v, int B, int H, int N,
                                   int d, int block, double keep, int phi, void* out, int out_dtype,
                                   void* resid, size_t resid_bytes, void* ws, size_t ws_bytes,
                                   void* stream) {
  const sla_status st = check_fwd_args(q, k, v, B, H, N, d, block, keep, phi, out, out_dtype, nullptr);
  if (st != SLA_OK) return st;
  const size_t need = sla_train_residual_bytes(B, H, N, d, block, keep, phi);
  if (!resid || !aligned16(resid) || resid_bytes < need) return SLA_ERR_INVALID_ARG;
  const int Nb = (N + SLA_BLOCK - 1) / SLA_BLOCK;
  const int kk = sla_topk_count(Nb, keep);
  const Shape s = make_shape(B, H, N, kk);
  const int phi_eff = (kk < Nb) ? phi : SLA_PHI_NONE;
  sla::TrainResiduals r;
  carve_residuals(s, phi_eff, phi_eff != SLA_PHI_NONE && sla::linear_direct(s),
                  static_cast<unsigned char*>(resid), &r);
  return fwd_impl(q, k, v, B, H, N, d, block, keep, phi, out, out_dtype, r.ol, ws, ws_bytes, stream,
                  nullptr, 0, &r);
}

sla_status sla_attention_fwd_fork(const void* q, const void* k, const void* v, int B, int H, int N,
                                  int d, int block, double keep, int phi, void* out, int out_dtype,
                                  void* ws, size_t ws_bytes, void* stream, void* side) {
  return fwd_impl(q, k, v, B, H, N, d, block, keep, phi, out, out_dtype, nullptr, ws, ws_bytes,
                  stream, nullptr, 0, nullptr, side);
}

sla_status sla_attention_fwd(const void* q, const void* k, const void* v, int B, int H, int N,
                             int d, int block, double keep, int phi, void* out, int out_dtype,
                             void* ws, size_t ws_bytes, void* stream) {
  return sla_attention_fwd_ex(q, k, v, B, H, N, d, block, keep, phi, out, out_dtype, nullptr, ws,
                              ws_bytes, stream, nullptr, 0);
}

sla_status sla_attention_fwd_lowbit(const void* q, const void* k, const void* v, int B, int H,
                                    int N, int d, int block, double keep, int phi, void* out,
                                    int out_dtype, void* ws, size_t ws_bytes, void* stream) {
  return sla_attention_fwd_ex(q, k, v, B, H, N, d, block, keep, phi, out, out_dtype, nullptr, ws,
                              ws_bytes, stream, nullptr, SLA_OPT_PHI_K_FP8);
}

sla_status sla_attention_fwd_noalloc(const void* q, const void* k, const void* v, int B, int H,
                                     int N, int d, int block, double keep, int phi, void* out,
                                     int out_dtype, void* stream) {
  const sla_status st = check_fwd_args(q, k, v, B, H, N, d, block, keep, phi, out, out_dtype, nullptr);
  if (st != SLA_OK) return st;
  const size_t need = sla_workspace_bytes(B, H, N, d, block, keep, phi);
  if (need == 0 || need > SLA_NOALLOC_SCRATCH_BYTES) return SLA_ERR_SCRATCH;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return SLA_ERR_DEVICE;
  return sla_attention_fwd_ex(q, k, v, B, H, N, d, block, keep, phi, out, out_dtype, nullptr, ws,
                              SLA_NOALLOC_SCRATCH_BYTES, stream, nullptr, 0);
}

}  // extern "C"

namespace {

// The backward; with `resid` (a training forward's residuals) the query side
// reads the forward's statistics, outputs and kept share instead of
// recomputing them (not in the direct form, whose forward keeps no kept share).
sla_status bwd_impl(const void* q, const void* k, const void* v, const void* dout,
                    const void* resid, size_t resid_bytes, int B, int H, int N, int d, int block,
                    double keep, int phi, void* dq, void* dk, void* dv, int grad_dtype, void* ws,
                    size_t ws_bytes, void* stream, void* const* stage_events) {
  sla_status st = check_shape(B, H, N, d, block);
  if (st != SLA_OK) return st;
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return SLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv))
    return SLA_ERR_INVALID_ARG;
  if (std::isnan(keep) || keep < 0.0 || keep > 1.0) return SLA_ERR_INVALID_ARG;
  if (phi < SLA_PHI_NONE || phi > SLA_PHI_RELU) return SLA_ERR_INVALID_ARG;
  if (grad_dtype != SLA_OUT_BF16 && grad_dtype != SLA_OUT_F32) return SLA_ERR_INVALID_ARG;
  const int Nb = (N + SLA_BLOCK - 1) / SLA_BLOCK;
  const int kk = sla_topk_count(Nb, keep);
  if (kk == 0 && phi == SLA_PHI_NONE) return SLA_ERR_INVALID_ARG;
  int R = 1;
  if (kk > 0 && sla::topk_lds_bytes(Nb, &R) > 160 * 1024) return SLA_ERR_UNSUPPORTED;
  const Shape s = make_shape(B, H, N, kk);
  const size_t need = carve(SLA_OP_ATTENTION_BWD, s, phi, nullptr, nullptr);
  if (!ws || ws_bytes < need || !aligned16(ws)) return SLA_ERR_WORKSPACE;
  Workspace w;
  sla::BwdWorkspace bw;
  carve(SLA_OP_ATTENTION_BWD, s, phi, static_cast<unsigned char*>(ws), &w, &bw);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const auto* qb = static_cast<const uint16_t*>(q);
  const auto* kb = static_cast<const uint16_t*>(k);
  const auto* vb = static_cast<const uint16_t*>(v);
  const auto* gb = static_cast<const uint16_t*>(dout);
  const int phi_eff = (kk < Nb) ? phi : SLA_PHI_NONE;
  const int f32 = grad_dtype == SLA_OUT_F32 ? 1 : 0;
  sla::TrainResiduals r;
  const sla::TrainResiduals* res = nullptr;
  if (resid) {
    if (!aligned16(resid) || resid_bytes < sla_train_residual_bytes(B, H, N, d, block, keep, phi))
      return SLA_ERR_INVALID_ARG;
    const bool direct = phi_eff != SLA_PHI_NONE && sla::linear_direct(s);
    carve_residuals(s, phi_eff, direct, static_cast<unsigned char*>(const_cast<void*>(resid)), &r);
    if (!direct) res = &r;
  }
  hipError_t e = hipSuccess;
  auto run = [&](auto&& launch) {
    if (e == hipSuccess) e = launch();
  };
  auto mark = [&](int id, int end) {
    if (e == hipSuccess && stage_events && stage_events[2 * id + end])
      e = hipEventRecord(static_cast<hipEvent_t>(stage_events[2 * id + end]), hs);
  };
  // the forward's staging: codes, selection, walk schedule, linear state (a
  // training forward's residuals hold them)
  mark(SLA_BWD_STAGE_FWD_STAGING, 0);
  if (res) {
    if (kk > 0) {
      w.q8 = r.q8;
      w.sq = r.sq;
      w.k8 = r.k8;
      w.sk = r.sk;
      w.idx = r.idx;
      w.sched = r.sched;
    }
    if (phi_eff != SLA_PHI_NONE) {
      w.z = r.z;
      bw.hb = r.hb;
    }
  } else if (kk > 0) {
    run([&] { return sla::launch_block_stats(qb, kb, s, w.ksum, w.qbar, w.kbar, w.q8, w.sq, w.ksplit, w.kflag, w.kbar_rm, w.knorm, hs); });
    const uint32_t* handed_back = nullptr;
    run([&] {
      return sla::launch_block_topk_first(w.qbar, w.kbar, topk_filter(w), s, w.idx, nullptr, hs, &handed_back);
    });
    run([&] { return sla::launch_group_schedule(w.idx, s, w.sched, hs); });
    if (handed_back) {
      run([&] { return sla::launch_block_topk_redo(w.qbar, w.kbar, topk_filter(w), s, w.idx, nullptr, hs); });
      run([&] { return sla::launch_group_schedule(w.idx, s, w.sched, hs, handed_back); });
    }
    run([&] { return sla::launch_key_mean(w.ksum, s, w.mu, hs); });
  }
  if (!res)
    run([&] {
      return sla::launch_linear_prep(kb, vb, s, phi_eff, true, w.fk16, w.v16, w.zb, w.hpart, w.zpart,
                                     w.mu, kk > 0 ? w.k8 : nullptr, w.sk, false, nullptr, hs);
    });
  if (!res && phi_eff != SLA_PHI_NONE)
    run([&] {
      return sla::launch_linear_final(w.hpart, w.zpart, s, nullptr, nullptr, w.z, w.h16t, w.hscale,
                                      bw.hb, hs);
    });
  mark(SLA_BWD_STAGE_FWD_STAGING, 1);
  // the backward's own staging
  mark(SLA_BWD_STAGE_TRANSPOSE, 0);
  run([&] { return sla::launch_transpose_blocks(kk > 0 ? kb : nullptr, gb, s, bw.kt, bw.dot, hs); });
  mark(SLA_BWD_STAGE_TRANSPOSE, 1);
  if (kk > 0) {
    mark(SLA_BWD_STAGE_COLUMNS, 0);
    run([&] { return sla::launch_column_lists(w.idx, s, bw.maskT, bw.coff, bw.cidx, hs); });
    mark(SLA_BWD_STAGE_COLUMNS, 1);
  }
  mark(SLA_BWD_STAGE_QUERY, 0);
  run([&] { return sla::launch_bwd_q(qb, vb, gb, w, bw, s, phi_eff, dq, f32, res, hs); });
  mark(SLA_BWD_STAGE_QUERY, 1);
  if (phi_eff != SLA_PHI_NONE) {
    mark(SLA_BWD_STAGE_GRAD_H, 0);
    run([&] { return sla::launch_grad_h(bw, s, hs); });
    mark(SLA_BWD_STAGE_GRAD_H, 1);
  }
  mark(SLA_BWD_STAGE_KEY, 0);
  run([&] { return sla::launch_bwd_kv(qb, kb, vb, gb, w, bw, s, phi_eff, dk, dv, f32, hs); });
  mark(SLA_BWD_STAGE_KEY, 1);
  return device_status(e);
}

}  // namespace

extern "C" {

sla_status sla_attention_bwd_timed(const void* q, const void* k, const void* v, const void* dout,
                                   int B, int H, int N, int d, int block, double keep, int phi,
                                   void* dq, void* dk, void* dv, int grad_dtype, void* ws,
                                   size_t ws_bytes, void* stream, void* const* stage_events) {
  return bwd_impl(q, k, v, dout, nullptr, 0, B, H, N, d, block, keep, phi, dq, dk, dv, grad_dtype, ws,
                  ws_bytes, stream, stage_events);
}

sla_status sla_attention_bwd_saved(const void* q, const void* k, const void* v, const void* dout,
                                   const void* resid, size_t resid_bytes, int B, int H, int N, int d,
                                   int block, double keep, int phi, void* dq, void* dk, void* dv,
                                   int grad_dtype, void* ws, size_t ws_bytes, void* stream,
                                   void* const* stage_events) {
  if (!resid) return SLA_ERR_INVALID_ARG;
  return bwd_impl(q, k, v, dout, resid, resid_bytes, B, H, N, d, block, keep, phi, dq, dk, dv,
                  grad_dtype, ws, ws_bytes, stream, stage_events);
}

sla_status sla_attention_bwd(const void* q, const void* k, const void* v, const void* dout,
                             int B, int H, int N, int d, int block, double keep, int phi,
                             void* dq, void* dk, void* dv, int grad_dtype, void* ws,
                             size_t ws_bytes, void* stream) {
  return sla_attention_bwd_timed(q, k, v, dout, B, H, N, d, block, keep, phi, dq, dk, dv,
                                 grad_dtype, ws, ws_bytes, stream, nullptr);
}

sla_status sla_rowquant_i8(const void* x, int rows, int K, int8_t* codes, float* scale,
                           void* stream) {
  if (!x || !codes || !scale || rows < 1) return SLA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(codes)) return SLA_ERR_INVALID_ARG;
  if (K < 64 || K > sla::kMaxRowK || K % 64 != 0) return SLA_ERR_UNSUPPORTED;
  return device_status(sla::launch_rowquant(static_cast<const uint16_t*>(x), rows, K, false, nullptr,
                                            nullptr, 0.0f, codes, scale, nullptr, nullptr,
                                            static_cast<hipStream_t>(stream)));
}

sla_status sla_fused_norm_i8(const void* x, int rows, int K, const float* gamma, const float* beta,
                             float eps, int8_t* codes, float* scale, float* mean, float* rstd,
                             void* stream) {
  if (!x || !codes || !scale || rows < 1) return SLA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(codes) || (gamma && !aligned16(gamma)) || (beta && !aligned16(beta)))
    return SLA_ERR_INVALID_ARG;
  if (!(eps > 0.0f) || std::isinf(eps)) return SLA_ERR_INVALID_ARG;
  if (K < 64 || K > sla::kMaxRowK || K % 64 != 0) return SLA_ERR_UNSUPPORTED;
  return device_status(sla::launch_rowquant(static_cast<const uint16_t*>(x), rows, K, true, gamma,
                                            beta, eps, codes, scale, mean, rstd,
                                            static_cast<hipStream_t>(stream)));
}

sla_status sla_w8a8_linear(const int8_t* x8, const float* x_scale, const int8_t* w8,
                           const float* w_scale, const float* bias, int M, int N, int K, void* y,
                           int out_dtype, void* stream) {
  if (!x8 || !x_scale || !w8 || !w_scale || !y || M < 1 || N < 1) return SLA_ERR_INVALID_ARG;
  if (!aligned16(x8) || !aligned16(w8) || !aligned16(x_scale) || !aligned16(w_scale) ||
      !aligned16(y) || (bias && !aligned16(bias)))
    return SLA_ERR_INVALID_ARG;
  if (out_dtype != SLA_OUT_BF16 && out_dtype != SLA_OUT_F32) return SLA_ERR_INVALID_ARG;
  if (K < 128 || K > sla::kMaxRowK || K % 128 != 0 || N % 4 != 0) return SLA_ERR_UNSUPPORTED;
  if ((long long)M * K >= (1LL << 31) || (long long)N * K >= (1LL << 31)) return SLA_ERR_UNSUPPORTED;
  return device_status(sla::launch_w8a8_gemm(x8, x_scale, w8, w_scale, bias, M, N, K, y,
                                             out_dtype == SLA_OUT_F32 ? 1 : 0,
                                             static_cast<hipStream_t>(stream)));
}

sla_status sla_debug_qk_i32(const int8_t* q_i8, const int8_t* k_i8, int B, int H, int N, int d,
                            int block, const int32_t* pairs, int n_pairs, int32_t* acc,
                            void* stream) {
  sla_status st = check_shape(B, H, N, d, block);
  if (st != SLA_OK) return st;
  if (!q_i8 || !k_i8 || !pairs || !acc || n_pairs < 0) return SLA_ERR_INVALID_ARG;
  if (!aligned16(q_i8) || !aligned16(k_i8)) return SLA_ERR_INVALID_ARG;
  if (n_pairs == 0) return SLA_OK;
  const Shape s = make_shape(B, H, N, 0);
  return device_status(sla::launch_debug_qk(q_i8, k_i8, s, pairs, n_pairs, acc,
                                            static_cast<hipStream_t>(stream)));
}

const char* sla_status_string(int status) {
  switch (status) {
    case SLA_OK: return "SLA_OK";
    case SLA_ERR_INVALID_ARG: return "SLA_ERR_INVALID_ARG: invalid argument";
    case SLA_ERR_UNSUPPORTED: return "SLA_ERR_UNSUPPORTED: shape or option not supported";
    case SLA_ERR_WORKSPACE: return "SLA_ERR_WORKSPACE: workspace missing or too small";
    case SLA_ERR_DEVICE: return "SLA_ERR_DEVICE: HIP launch failed";
    case SLA_ERR_SCRATCH:
      return "SLA_ERR_SCRATCH: shape needs more workspace than the 64 MiB static scratch";
    default: return "unknown sla_status";
  }
}

int sla_version(void) { return 20100; }

}  // extern "C"
