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
      ws.zpart = reinterpret_cast<float*>(take(BH * sla::kLinChunks * D * sizeof(float)));
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
    b.qt = reinterpret_cast<uint16_t*>(take(BH * Np * D * sizeof(uint16_t)));
    b.dot = reinterpret_cast<uint16_t*>(take(BH * Np * D * sizeof(uint16_t)));
    b.stats = reinterpret_cast<float*>(take(BH * Nb * 256 * sizeof(float)));
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
      ws.uidx = reinterpret_cast<int32_t*>(take(BH * Nb * (size_t)(s.Nb - s.k) * sizeof(int32_t)));
      ws.fk16 = reinterpret_cast<uint16_t*>(take(BH * Np * D * sizeof(uint16_t)));
      ws.zb = reinterpret_cast<float*>(take(BH * Nb * D * sizeof(float)));
    } else if (phi != SLA_PHI_NONE && s.k < s.Nb) {
      ws.fk16 = reinterpret_cast<uint16_t*>(take(BH * Np * D * sizeof(uint16_t)));
      ws.zb = reinterpret_cast<float*>(take(BH * Nb * D * sizeof(float)));
      ws.hpart = reinterpret_cast<float*>(take(BH * sla::kLinChunks * D * D * sizeof(float)));
      ws.zpart = reinterpret_cast<float*>(take(BH * sla::kLinChunks * D * sizeof(float)));
      ws.h16t = reinterpret_cast<uint16_t*>(take(BH * D * D * sizeof(uint16_t)));
      ws.hscale = reinterpret_cast<float*>(take(BH * sizeof(float)));
      ws.z = reinterpret_cast<float*>(take(BH * D * sizeof(float)));
    }
  }
  return off;
}

sla_status device_status(hipError_t e) { return e == hipSuccess ? SLA_OK : SLA_ERR_DEVICE; }

// A side stream per device (non-blocking, default priority) on which the block
// scores run while the caller's stream stages the linear branch: the fork and
// the join are event edges, so the call stays asynchronous and capturable.
// The fork/join sequence of a call is enqueued under the lock, so concurrent
// calls never interleave their uses of the two events.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

hipError_t side_stream(SideStream** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  SideStream& ss = g_side[dev];
  if (!ss.stream) {
    e = hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming);
    if (e != hipSuccess) return e;
  }
  *out = &ss;
  return hipSuccess;
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
  hipError_t e = sla::launch_block_stats(qb, kb, s, w.ksum, w.qbar, w.kbar, q_i8, q_scale, hs);
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
  hipError_t e = sla::launch_block_stats(qb, kb, s, w.ksum, w.qbar, w.kbar, nullptr, nullptr, hs);
  if (e == hipSuccess)
    e = sla::launch_block_topk(w.qbar, w.kbar, s, kblock_idx, kblock_mask, nullptr, hs);
  return device_status(e);
}

sla_status sla_attention_fwd_timed(const void* q, const void* k, const void* v, int B, int H,
                                   int N, int d, int block, double keep, int phi, void* out,
                                   int out_dtype, float* out_linear, void* ws, size_t ws_bytes,
                                   void* stream, void* const* stage_events) {
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
  hipError_t e = hipSuccess;
  // runs one stage between its two optional events, on stream `on`
  auto stage_on = [&](hipStream_t on, int id, auto&& launch) {
    if (e != hipSuccess) return;
    if (stage_events && stage_events[2 * id])
      e = hipEventRecord(static_cast<hipEvent_t>(stage_events[2 * id]), on);
    if (e == hipSuccess) e = launch();
    if (e == hipSuccess && stage_events && stage_events[2 * id + 1])
      e = hipEventRecord(static_cast<hipEvent_t>(stage_events[2 * id + 1]), on);
  };
  auto stage = [&](int id, auto&& launch) { stage_on(hs, id, launch); };
  std::unique_lock<std::mutex> side_lock(g_side_mu, std::defer_lock);
  SideStream* side = nullptr;
  // with stage events every stage runs on the caller's stream, one after
  // another, so that each is timed alone
  const bool fork = stage_events == nullptr;
  if (kk > 0) {
    stage(SLA_STAGE_STATS, [&] {
      return sla::launch_block_stats(qb, kb, s, w.ksum, w.qbar, w.kbar, w.q8, w.sq, hs);
    });
    // fork: the block scores and top-k need only the block means
    hipStream_t sel = hs;
    if (fork) {
      side_lock.lock();
      if (e == hipSuccess) e = side_stream(&side);
      if (e == hipSuccess) e = hipEventRecord(side->fork, hs);
      if (e == hipSuccess) e = hipStreamWaitEvent(side->stream, side->fork, 0);
      if (e == hipSuccess) sel = side->stream;
    }
    stage_on(sel, SLA_STAGE_TOPK, [&] {
      return sla::launch_block_topk(w.qbar, w.kbar, s, w.idx, nullptr, direct ? w.uidx : nullptr, sel);
    });
    // then the walk schedule, which needs only the kept lists
    if (!direct)
      stage_on(sel, SLA_STAGE_SCHEDULE,
               [&] { return sla::launch_group_schedule(w.idx, s, w.sched, sel); });
    if (fork && e == hipSuccess) e = hipEventRecord(side->join, side->stream);
    stage(SLA_STAGE_KMEAN, [&] { return sla::launch_key_mean(w.ksum, s, w.mu, hs); });
  }
  // Q is coded by the statistics pass and K by the staging pass (one read of
  // each), so the QUANTIZE stage does not run here
  stage(SLA_STAGE_LINEAR_PREP, [&] {
    return sla::launch_linear_prep(kb, vb, s, phi_eff, !direct, w.fk16, w.v16, w.zb, w.hpart,
                                   w.zpart, w.mu, kk > 0 ? w.k8 : nullptr, w.sk, hs);
  });
  if (phi_eff != SLA_PHI_NONE && !direct)
    stage(SLA_STAGE_LINEAR_FINAL,
          [&] { return sla::launch_linear_final(w.hpart, w.zpart, s, w.h16t, w.hscale, w.z, hs); });
  if (kk > 0 && fork) {
    // join before the attention kernel
    if (e == hipSuccess) e = hipStreamWaitEvent(hs, side->join, 0);
    side_lock.unlock();
  }
  stage(SLA_STAGE_SPARSE, [&] {
    return sla::launch_sparse_fwd(qb, w, s, phi_eff, out, out_dtype == SLA_OUT_F32 ? 1 : 0,
                                  out_linear, hs);
  });
  return device_status(e);
}

sla_status sla_attention_fwd(const void* q, const void* k, const void* v, int B, int H, int N,
                             int d, int block, double keep, int phi, void* out, int out_dtype,
                             float* out_linear, void* ws, size_t ws_bytes, void* stream) {
  return sla_attention_fwd_timed(q, k, v, B, H, N, d, block, keep, phi, out, out_dtype, out_linear,
                                 ws, ws_bytes, stream, nullptr);
}

sla_status sla_attention_bwd_timed(const void* q, const void* k, const void* v, const void* dout,
                                   int B, int H, int N, int d, int block, double keep, int phi,
                                   void* dq, void* dk, void* dv, int grad_dtype, void* ws,
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
  hipError_t e = hipSuccess;
  auto run = [&](auto&& launch) {
    if (e == hipSuccess) e = launch();
  };
  auto mark = [&](int id, int end) {
    if (e == hipSuccess && stage_events && stage_events[2 * id + end])
      e = hipEventRecord(static_cast<hipEvent_t>(stage_events[2 * id + end]), hs);
  };
  // the forward's staging: codes, selection, walk schedule, linear state
  mark(SLA_BWD_STAGE_FWD_STAGING, 0);
  if (kk > 0) {
    run([&] { return sla::launch_block_stats(qb, kb, s, w.ksum, w.qbar, w.kbar, w.q8, w.sq, hs); });
    run([&] { return sla::launch_block_topk(w.qbar, w.kbar, s, w.idx, nullptr, nullptr, hs); });
    run([&] { return sla::launch_group_schedule(w.idx, s, w.sched, hs); });
    run([&] { return sla::launch_key_mean(w.ksum, s, w.mu, hs); });
  }
  run([&] {
    return sla::launch_linear_prep(kb, vb, s, phi_eff, true, w.fk16, w.v16, w.zb, w.hpart, w.zpart,
                                   w.mu, kk > 0 ? w.k8 : nullptr, w.sk, hs);
  });
  if (phi_eff != SLA_PHI_NONE)
    run([&] {
      return sla::launch_linear_final(w.hpart, w.zpart, s, w.h16t, w.hscale, w.z, hs, bw.hb);
    });
  mark(SLA_BWD_STAGE_FWD_STAGING, 1);
  // the backward's own staging
  mark(SLA_BWD_STAGE_TRANSPOSE, 0);
  run([&] { return sla::launch_transpose_blocks(kk > 0 ? kb : nullptr, kk > 0 ? qb : nullptr, gb, s,
                                                bw.kt, bw.qt, bw.dot, hs); });
  mark(SLA_BWD_STAGE_TRANSPOSE, 1);
  if (kk > 0) {
    mark(SLA_BWD_STAGE_COLUMNS, 0);
    run([&] { return sla::launch_column_lists(w.idx, s, bw.maskT, bw.coff, bw.cidx, hs); });
    mark(SLA_BWD_STAGE_COLUMNS, 1);
  }
  mark(SLA_BWD_STAGE_QUERY, 0);
  run([&] { return sla::launch_bwd_q(qb, vb, gb, w, bw, s, phi_eff, dq, f32, hs); });
  mark(SLA_BWD_STAGE_QUERY, 1);
  if (phi_eff != SLA_PHI_NONE) {
    mark(SLA_BWD_STAGE_GRAD_H, 0);
    run([&] { return sla::launch_grad_h(bw, s, hs); });
    mark(SLA_BWD_STAGE_GRAD_H, 1);
  }
  mark(SLA_BWD_STAGE_KEY, 0);
  run([&] { return sla::launch_bwd_kv(kb, vb, gb, w, bw, s, phi_eff, dk, dv, f32, hs); });
  mark(SLA_BWD_STAGE_KEY, 1);
  return device_status(e);
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
    default: return "unknown sla_status";
  }
}

int sla_version(void) { return 10300; }

}  // extern "C"
