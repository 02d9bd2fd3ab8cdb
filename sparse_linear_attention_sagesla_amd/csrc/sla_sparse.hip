// Block-sparse SageSLA attention kernel for gfx950 (CDNA4).
//
// One workgroup = one 64-row query block of one (b,h); four waves, each
// owning 16 query rows.  The workgroup walks a list of key blocks (tiles).
// Per tile, staged in LDS by direct global->LDS 16-byte loads, double-buffered
// so the next tile streams in while this one is computed:
//   K8_j   int8 [64 keys][128]      (8 KB)   -> S^T = K8_j Q8_i^T     (INT8 MFMA)
//   V_j    fp16 [128][64 perm keys] (16 KB)  -> O^T += V_j^T P^T      (fp16 MFMA)
//   phiK_j fp16 [128][64 perm keys] (16 KB)  -> M^T += V_j^T phiK_j   (fp16 MFMA)
// Scores are computed transposed (keys x queries) so each lane ends up holding
// one query's values for 16 keys; in that layout the exponentiated scores P are
// already the B operand of the P.V product and never leave registers, and the
// online-softmax statistics are per lane.  The V fragments read for P.V are
// also the A operand of the linear branch's M^T = sum V_j^T phiK_j, of which
// each wave owns 32 phi channels.
//
// Softmax branch (tutorial "TurboDiffusion技术架构解析：稀疏线性注意力应用实战"
// §2.1 standard attention, on INT8 codes as in low-bit SageAttention): logits
// acc * sq_i * sk_j / sqrt(128) in the log2 domain, online max/sum in fp32,
// P rounded to fp16 with the normaliser summed from the rounded P.  The running
// maximum is exact, so the largest weight of a row is exactly 1 in fp16 (no
// rounding error on the dominant term of a peaked row); the accumulators are
// rescaled only in tiles where some row's maximum rises.
// Linear branch (same section, linear attention with phi = elu+1 / ReLU),
// normalised, over the unselected blocks, in one of two forms:
//   subtraction: numerator phi(Q)(H - M), denominator phi(Q)(z - z_M), with
//                H, z the whole-head sums and M = sum phi(K_j)^T V_j,
//                z_M = sum of the block sums of phi(K_j) over the kept tiles
//                (kept tiles carry both branches);
//   direct:      M, z_M summed over the unselected tiles, walked after the
//                kept ones (used when they are no more than the kept ones);
//                numerator phi(Q)M, denominator phi(Q)z_M.
// M is the query block's, shared by its four waves: at the end it is stored
// once in LDS (fp16, power-of-two scaled) and multiplied by each wave's phi(Q).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "sla_internal.h"

namespace sla {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) unsigned char lds_byte;
typedef __attribute__((address_space(3))) const v4i lds_v4i;
typedef __attribute__((address_space(3))) const half8 lds_half8;

constexpr int kK8Bytes = kBlk * kD;          // 8 KB
constexpr int kF16TileBytes = kBlk * kD * 2; // 16 KB
constexpr int kVOff = kK8Bytes;                       // V tile offset in a stage
constexpr int kFOff = kK8Bytes + kF16TileBytes;       // phi(K) tile offset in a stage
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInvSqrtD = 0.08838834764831845f;  // 1/sqrt(128)

enum Mode { kSoftOnly = 0, kSubtract = 1, kDirect = 2 };

__device__ __forceinline__ float phi_apply(float x, int phi) {
  if (phi == kPhiElu1) return x > 0.0f ? x + 1.0f : __expf(x);
  return fmaxf(x, 0.0f);
}

// LDS layout.  The staged tiles have 128-byte rows and keep 16-byte chunk ch
// of row r at chunk ch ^ ((r >> 1) & 7); the final M^T (256-byte rows) keeps
// chunk ch of row r at ch ^ (r & 15).  A 16-lane read group (16 consecutive
// rows, same chunk) then touches 16 distinct 4-bank groups of the 64-bank LDS.
struct LaneOffsets {
  int rd8;    // read byte offset of (row l16, chunk g) in a staged tile; chunk g+4: ^64
  int rdK;    // rd8 in rows 32w.. of the stage's phi(K) tile (w = this wave)
  int rdM;    // read byte offset of (row l16, chunk g) in M^T; chunk g+4cc: ^(64cc)
  int ld8;    // global byte offset (within the tile) this lane fetches
  int zo;     // byte offset of this lane's phi channel 32w + (lane & 31) in a block sum
};

__device__ __forceinline__ LaneOffsets lane_offsets(int wave, int lane) {
  LaneOffsets o;
  const int l16 = lane & 15, g = lane >> 4;
  o.rd8 = l16 * 128 + ((g ^ ((l16 >> 1) & 7)) << 4);
  o.rdK = kFOff + 4096 * wave + o.rd8;  // bit 6 of the base is 0, so ^64 still picks chunk g+4
  o.rdM = l16 * 256 + ((g ^ l16) << 4);
  // LDS-direct loads: wave w, instruction m fills LDS chunks 256m + 64w + lane
  const int row = 8 * wave + (lane >> 3);             // + 32m
  const int ch = (lane & 7) ^ ((row >> 1) & 7);
  o.ld8 = row * 128 + ch * 16;                        // + 4096m
  o.zo = 4 * (32 * wave + (lane & 31));
  return o;
}

// Buffer resource over one head's slice of a staging tensor (the per-head slice
// is below 2^31 bytes, so tile offsets fit the 32-bit buffer offsets; reads
// past `bytes` return zero instead of faulting).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from rsrc[voff + soff] into LDS at ldst + 16 * lane.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                           lds_byte* ldst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3)))*)ldst, 16,
                                           voff, soff, 0, 0);
}

struct TileSrc {
  __amdgpu_buffer_rsrc_t k8, v16, fk16, zb;  // this head's slices
};

// Issues this wave's share of a tile's LDS-direct loads into `st` (kW waves
// per workgroup; each instruction round of the workgroup moves kW KB).
template <bool kK8, bool kFK, int kW = 4>
__device__ __forceinline__ void issue_tile(lds_byte* st, const TileSrc& src, int j, int wave,
                                           const LaneOffsets& lo) {
  constexpr int kRound = kW * 1024;
#pragma unroll
  for (int m = 0; m < kF16TileBytes / kRound; ++m)
    lds_load16(src.v16, lo.ld8, j * kF16TileBytes + kRound * m, st + kVOff + kRound * m + 1024 * wave);
  if (kK8) {
#pragma unroll
    for (int m = 0; m < kK8Bytes / kRound; ++m)
      lds_load16(src.k8, lo.ld8, j * kK8Bytes + kRound * m, st + kRound * m + 1024 * wave);
  }
  if (kFK) {
#pragma unroll
    for (int m = 0; m < kF16TileBytes / kRound; ++m)
      lds_load16(src.fk16, lo.ld8, j * kF16TileBytes + kRound * m, st + kFOff + kRound * m + 1024 * wave);
  }
}

// This lane's channel of key block j's phi(K) block sum.
__device__ __forceinline__ float load_zb(const TileSrc& src, int j, const LaneOffsets& lo) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(src.zb, lo.zo, j * (kD * 4), 0));
}

// S^T tile (64 keys x 16 queries of this wave) from the staged K8 tile.
// s[kt][r] = sum_e K8[16kt+4g+r][e] * Q8[query l16][e]
__device__ __forceinline__ void qk_tile(const lds_byte* st, const v4i qf[2], int rd8, v4i s[4]) {
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    s[kt] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int dc = 0; dc < 2; ++dc) {
      const v4i a = *(lds_v4i*)(st + kt * 2048 + (rd8 ^ (64 * dc)));
      s[kt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, qf[dc], s[kt], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void load_q8_frag(const int8_t* q8, size_t bh, int Np, int row, int g,
                                             v4i qf[2]) {
  const int8_t* p = q8 + ((size_t)bh * Np + row) * kD + 16 * g;
  qf[0] = *reinterpret_cast<const v4i*>(p);
  qf[1] = *reinterpret_cast<const v4i*>(p + 64);
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier for LDS hand-offs.  Unlike __syncthreads() it carries no
// release fence, whose vmcnt(0) would also wait for the tile loads issued
// ahead; each wave has already waited for its own share of the tile being
// handed over, and its LDS reads are complete (lgkmcnt(0)) before it arrives.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Reads a value the kernel never writes through the constant address space, so
// a wave-uniform address becomes a scalar load: it is counted by lgkmcnt and
// waiting for it does not drain the tile loads in flight.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* p, size_t i) {
  typedef const __attribute__((address_space(4))) T cT;
  return ((cT*)p)[i];
}

struct SparseArgs {
  const uint16_t* q;
  const int8_t* q8;
  const int8_t* k8;
  const float* sq;
  const float* sk;
  const int32_t* idx;
  const int32_t* uidx;
  const int32_t* sched;
  const uint16_t* fk16;
  const uint16_t* v16;
  const float* zb;
  const uint16_t* h16t;
  const float* hscale;
  const float* z;
  int N, Nb, Np, k;
  int phi;        // feature map for phi(Q)
  void* out;
  int out_f32;
  float* out_linear;
};

struct State {
  v4f o[8];       // O^T accumulator (softmax numerator), d = 16dt + 4g + r
  v4f mk[8][2];   // M^T accumulator (linear branch, kept or unselected share):
                  // row d = 16dt + 4g + r, phi channel 32w + 16x + l16
  float m_run;    // running log2-domain maximum (this lane's query)
  float l_part;   // this lane's share of the softmax normaliser
  float zk;       // z_M, phi channel 32w + (lane & 31)
};

// Maximum over the four 16-lane rows of the wave (lanes l, l^16, l^32, l^48).
// Each permlane swap hands every lane its partner's value in one of the two
// results, so max of the pair is the exchange-and-reduce step without LDS.
__device__ __forceinline__ int rows_max(int x) {
  const auto a = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  x = max((int)a[0], (int)a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
  return max((int)b[0], (int)b[1]);
}

// One tile's computation from stage `st`.  kMask: the tile is the ragged last
// key block (keys >= kvalid are padding and get weight 0).
template <bool kSoft, bool kLin, bool kMask>
__device__ __forceinline__ void compute_tile(State& S, const lds_byte* st, const v4i qf[2],
                                             const LaneOffsets& lo, float cs, float zj,
                                             int kvalid, int g) {
  half8 pf[2], fk[2][2];
  const half2v ones = {(_Float16)1.0f, (_Float16)1.0f};
  if (kSoft) {
    v4i s[4];
    qk_tile(st, qf, lo.rd8, s);
    if (kMask) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * kt + 4 * g + r >= kvalid) s[kt][r] = INT32_MIN;
    }
    int mi = s[0][0];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mi = max(mi, s[kt][r]);
    mi = rows_max(mi);
    const float mx = (float)mi * cs;  // cs >= 0, so this is the tile's largest logit
    const bool up = mx > S.m_run;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(up) != 0, 0)) {
      const float m_new = up ? mx : S.m_run;
      const float alpha = __builtin_amdgcn_exp2f(S.m_run - m_new);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) S.o[dt] *= alpha;
      S.l_part *= alpha;
      S.m_run = m_new;
    }
    const float nm = -S.m_run;
    float ls = S.l_part;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        float2v p;
        p.x = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s[kt][r], cs, nm));
        p.y = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s[kt][r + 1], cs, nm));
        if (kMask) {
          if (16 * kt + 4 * g + r >= kvalid) p.x = 0.0f;
          if (16 * kt + 4 * g + r + 1 >= kvalid) p.y = 0.0f;
        }
        const half2v ph = __builtin_convertvector(p, half2v);  // RNE
        pf[kt >> 1][4 * (kt & 1) + r] = ph.x;
        pf[kt >> 1][4 * (kt & 1) + r + 1] = ph.y;
        ls = __builtin_amdgcn_fdot2(ph, ones, ls, false);
      }
    }
    S.l_part = ls;
  }
  if (kLin) {
    // B operands phiK[key][channel] for this wave's channels 32w + 16x + l16
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int c = 0; c < 2; ++c) fk[x][c] = *(lds_half8*)(st + 2048 * x + (lo.rdK ^ (64 * c)));
    S.zk += zj;
  }
  // The products below are most of the tile's matrix-core work.  The wave
  // running them gets issue priority over the other workgroup's wave on this
  // SIMD, whose softmax steps then fill the issue slots between them.
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const half8 av = *(lds_half8*)(st + kVOff + dt * 2048 + (lo.rd8 ^ (64 * c)));
      if (kSoft) S.o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pf[c], S.o[dt], 0, 0, 0);
      if (kLin) {
#pragma unroll
        for (int x = 0; x < 2; ++x)
          S.mk[dt][x] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, fk[x][c], S.mk[dt][x], 0, 0, 0);
      }
    }
  }
  __builtin_amdgcn_s_setprio(0);
}

// Walks `n` tiles listed in `list` through the two LDS stages.
template <bool kSoft, bool kLin>
__device__ __forceinline__ void run_tiles(State& S, lds_byte* smem, int stage_bytes,
                                          const int32_t* list, int n, int stride,
                                          const SparseArgs& a,
                                          const TileSrc& src, size_t bh, const v4i qf[2],
                                          const LaneOffsets& lo, float qscale, int wave, int g) {
  if (n <= 0) return;
  // wave-uniform key block of tile p (kept in scalar registers), clamped so a
  // malformed list cannot address outside the staging buffers
  auto block_of = [&](int p) {
    return min(max(ld_uniform(list, (size_t)p * stride), 0), a.Nb - 1);
  };
  int j = block_of(0);
  issue_tile<kSoft, kLin>(smem, src, j, wave, lo);
  float zc = kLin ? load_zb(src, j, lo) : 0.0f;
  // lists are ascending, so only the last tile can be the ragged key block;
  // it is peeled off so the loop carries one compute variant
  const int nm = n - 1;
  for (int p = 0; p < nm; p += 2) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int pp = p + half;
      if (pp < nm) {
        lds_byte* cur = smem + half * stage_bytes;
        lds_byte* nxt = smem + (1 - half) * stage_bytes;
        const int jn = block_of(pp + 1);
        wait_loads();
        lds_barrier();  // tile pp is in LDS; every wave is done with tile pp-1
        issue_tile<kSoft, kLin>(nxt, src, jn, wave, lo);
        const float zn = kLin ? load_zb(src, jn, lo) : 0.0f;
        const float cs = kSoft ? qscale * ld_uniform(a.sk, bh * a.Nb + j) : 0.0f;
        compute_tile<kSoft, kLin, false>(S, cur, qf, lo, cs, zc, kBlk, g);
        j = jn;
        zc = zn;
      }
    }
  }
  {
    const float cs = kSoft ? qscale * ld_uniform(a.sk, bh * a.Nb + j) : 0.0f;
    const int kvalid = a.N - j * kBlk;
    const lds_byte* cur = smem + (nm & 1) * stage_bytes;
    wait_loads();
    lds_barrier();
    if (kSoft && kvalid < kBlk)
      compute_tile<kSoft, kLin, true>(S, cur, qf, lo, cs, zc, kvalid, g);
    else
      compute_tile<kSoft, kLin, false>(S, cur, qf, lo, cs, zc, kvalid, g);
  }
  lds_barrier();  // the stages may be refilled by a following walk
}

// Walks this block's column of its group schedule (key block of step s at
// col[s * kGroup]) through the two LDS stages.  A step's entry, and then the
// INT8 scale of its key block, are read with scalar loads when its tile is
// issued, a tile ahead of their use; reading entries earlier (a step further
// ahead, or 64-step chunks in registers) measured slower.
template <bool kLin>
__device__ __forceinline__ void run_sched(State& S, lds_byte* smem, int stage_bytes,
                                          const int32_t* col, int n, const SparseArgs& a,
                                          const TileSrc& src, size_t bh, const v4i qf[2],
                                          const LaneOffsets& lo, float qscale, int wave, int g) {
  if (n <= 0) return;
  auto block_of = [&](int p) { return min(max(ld_uniform(col, (size_t)p * kGroup), 0), a.Nb - 1); };
  auto scale_of = [&](int j) { return ld_uniform(a.sk, bh * a.Nb + j); };
  int j = block_of(0);
  issue_tile<true, kLin>(smem, src, j, wave, lo);
  float zc = kLin ? load_zb(src, j, lo) : 0.0f;
  float sc = scale_of(j);
  // the schedule puts a ragged key block only in the last step, which is
  // peeled off so the loop carries one compute variant
  const int nm = n - 1;
  for (int p = 0; p < nm; p += 2) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int pp = p + half;
      if (pp < nm) {
        lds_byte* cur = smem + half * stage_bytes;
        lds_byte* nxt = smem + (1 - half) * stage_bytes;
        wait_loads();
        lds_barrier();  // tile pp is in LDS; every wave is done with tile pp-1
        const int jn = block_of(pp + 1);
        issue_tile<true, kLin>(nxt, src, jn, wave, lo);
        const float zn = kLin ? load_zb(src, jn, lo) : 0.0f;
        const float sn = scale_of(jn);
        compute_tile<true, kLin, false>(S, cur, qf, lo, qscale * sc, zc, kBlk, g);
        j = jn;
        zc = zn;
        sc = sn;
      }
    }
  }
  const float c = qscale * sc;
  const int kvalid = a.N - j * kBlk;
  const lds_byte* cur = smem + (nm & 1) * stage_bytes;
  wait_loads();
  lds_barrier();
  if (kvalid < kBlk)
    compute_tile<true, kLin, true>(S, cur, qf, lo, c, zc, kvalid, g);
  else
    compute_tile<true, kLin, false>(S, cur, qf, lo, c, zc, kvalid, g);
}

// fp16 phi(Q)/16 of this lane's query, channels 32cc + 8g + e (B operand of
// the phi(Q)H and phi(Q)M products).
__device__ __forceinline__ void load_phi_q(const SparseArgs& a, size_t bh, int qrow, bool qvalid,
                                           int g, half8 fq[4]) {
  const uint16_t* qp = a.q + ((size_t)bh * a.N + (qvalid ? qrow : 0)) * kD + 8 * g;
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    const uint4 u = *reinterpret_cast<const uint4*>(qp + 32 * cc);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t bits = (e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16);
      const float x = __uint_as_float(bits);
      fq[cc][e] = qvalid ? (_Float16)(phi_apply(x, a.phi) * kPhiScale) : (_Float16)0.0f;
    }
  }
}

// Per-lane query state: INT8 codes (B operand of S^T), accumulators.
__device__ __forceinline__ void init_query(const SparseArgs& a, size_t bh, int qrow, int g,
                                           v4i qf[2], State& S) {
  load_q8_frag(a.q8, bh, a.Np, qrow, g, qf);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    S.o[dt] = v4f{0.f, 0.f, 0.f, 0.f};
    S.mk[dt][0] = v4f{0.f, 0.f, 0.f, 0.f};
    S.mk[dt][1] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  S.m_run = -INFINITY;
  S.l_part = 0.0f;
  S.zk = 0.0f;
}

// Maximum over the 64 lanes of a wave (DPP within rows, permlane across rows).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0xB1, 0xF, 0xF, true));   // lane ^ 1
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x4E, 0xF, 0xF, true));   // lane ^ 2
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x141, 0xF, 0xF, true));  // 8-lane mirror
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x140, 0xF, 0xF, true));  // 16-lane mirror
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = max((uint32_t)a[0], (uint32_t)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max((uint32_t)b[0], (uint32_t)b[1]);
}

// The head's linear state for the subtraction form, staged in LDS after the
// tiles are done: H^T (fp16, 128 rows of 256 bytes, chunk c of row r kept at
// c ^ (r & 15) like M^T, so the same lane offsets read it) at kHOff and z
// (fp32 [128]) after it.  LDS-direct loads, so they fly while M^T is formed.
constexpr int kHOff = 40 * 1024;
__device__ __forceinline__ void issue_linear_state(const SparseArgs& a, size_t bh, lds_byte* smem,
                                                   int wave, int lane) {
  const __amdgpu_buffer_rsrc_t hr = head_rsrc(a.h16t + bh * kD * kD, (size_t)kD * kD * 2);
  const int r = 4 * wave + (lane >> 4);  // row within each 16-row round
  const int voff = r * 256 + (((lane & 15) ^ (r & 15)) << 4);
#pragma unroll
  for (int m = 0; m < 8; ++m) lds_load16(hr, voff, 4096 * m, smem + kHOff + 4096 * m + 1024 * wave);
  if (wave == 0) {
    // lanes 32.. read past z and write zeros after it
    const __amdgpu_buffer_rsrc_t zr = head_rsrc(a.z + bh * kD, (size_t)kD * 4);
    lds_load16(zr, 16 * lane, 0, smem + kHOff + kD * kD * 2);
  }
}

// The linear branch's share phi(Q) M for this lane's query (O^T layout, d =
// 16dt + 4g + r) and phi(Q) z_M.  The workgroup's four waves hold M^T by
// channel slices; M^T goes through LDS once as fp16 scaled by 2^-s so that
// max|M| 2^-s lies in [2^14, 2^15), and comes back as A operands.
__device__ __forceinline__ void linear_share(const State& S, lds_byte* smem, const half8 fq[4],
                                             const LaneOffsets& lo, int wave, int lane,
                                             v4f num[8], float& den,
                                             const SparseArgs* stage_state = nullptr,
                                             size_t bh = 0) {
  constexpr int kZOff = kD * kD * 2;             // z_M, fp32 [128]
  constexpr int kRedOff = kZOff + kD * 4;        // per-wave maxima
  const int g = lane >> 4, l16 = lane & 15;
  float mx = 0.0f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(S.mk[dt][x][r]));
  const uint32_t wm = wave_max_u32(__float_as_uint(mx));  // non-negative floats order as integers
  lds_barrier();  // every wave is done with the tile stages
  if (stage_state) issue_linear_state(*stage_state, bh, smem, wave, lane);
  if (lane == 0) *(__attribute__((address_space(3))) uint32_t*)(smem + kRedOff + 4 * wave) = wm;
  if (lane < 32) *(__attribute__((address_space(3))) float*)(smem + kZOff + 4 * (32 * wave + lane)) = S.zk;
  lds_barrier();
  uint32_t m4 = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    m4 = max(m4, *(__attribute__((address_space(3))) const uint32_t*)(smem + kRedOff + 4 * w));
  const float mall = __uint_as_float(m4);
  const int sh = mall > 0.0f ? ilogbf(mall) - 14 : 0;
  const float down = ldexpf(1.0f, -sh);
  typedef __attribute__((address_space(3))) _Float16 lds_h;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * dt + 4 * g + r;
        const int ch = (4 * wave + 2 * x + (l16 >> 3)) ^ (row & 15);
        *(lds_h*)(smem + row * 256 + ch * 16 + 2 * (l16 & 7)) = (_Float16)(S.mk[dt][x][r] * down);
      }
  lds_barrier();
  const float up = ldexpf(1.0f, sh);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const half8 am = *(lds_half8*)(smem + 4096 * dt + (lo.rdM ^ (64 * cc)));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(am, fq[cc], acc, 0, 0, 0);
    }
    num[dt] = acc * up;
  }
  float d = 0.0f;
#pragma unroll
  for (int cc = 0; cc < 4; ++cc)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      d += (float)fq[cc][e] * *(__attribute__((address_space(3))) const float*)(smem + kZOff + 4 * (32 * cc + 8 * g + e));
  d += __shfl_xor(d, 16);
  den = d + __shfl_xor(d, 32);
}

// Linear output in the subtraction form, from the kept share (nm, dm) that
// linear_share returns: (phi(Q)H - phi(Q)M) / (phi(Q)z - phi(Q)z_M).  Returns
// 1/den, 0 when the denominator is lost in rounding; den is in the staged
// scale (phi/16 on both sides: 1/256 of the true denominator).  kStaged: H^T
// and z come from LDS (issue_linear_state), else straight from memory.
template <bool kStaged>
__device__ __forceinline__ float linear_subtract_out(const SparseArgs& a, size_t bh, int g,
                                                     const lds_byte* smem, const LaneOffsets& lo,
                                                     const half8 fq[4], const v4f nm[8], float dm,
                                                     v4f ol[8]) {
  const float hs = a.hscale[bh];
  if (kStaged) {
    wait_loads();
    lds_barrier();  // the staged H^T and z are in
  }
  typedef __attribute__((address_space(3))) const float lds_f;
  const float* zz = a.z + bh * kD;
  float dz = 0.0f;
#pragma unroll
  for (int cc = 0; cc < 4; ++cc)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      dz += (float)fq[cc][e] * (kStaged ? *(lds_f*)(smem + kHOff + kD * kD * 2 + 4 * (32 * cc + 8 * g + e))
                                        : zz[32 * cc + 8 * g + e]);
  dz += __shfl_xor(dz, 16);
  dz += __shfl_xor(dz, 32);
  // whole head minus the kept share; a denominator lost in rounding counts as 0
  const float den = dz - dm;
  const float inv_den = den > 1e-6f * dz ? 1.0f / den : 0.0f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    v4f num = v4f{0.f, 0.f, 0.f, 0.f};
    const _Float16* hrow = reinterpret_cast<const _Float16*>(a.h16t) + bh * kD * kD +
                           (size_t)(16 * dt + (lo.rdM >> 8)) * kD + 8 * g;  // row 16dt + l16
    half8 ah[4];  // the row's four fragments, loaded together
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
      ah[cc] = kStaged ? *(lds_half8*)(smem + kHOff + 4096 * dt + (lo.rdM ^ (64 * cc)))
                       : *reinterpret_cast<const half8*>(hrow + 32 * cc);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) num = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[cc], fq[cc], num, 0, 0, 0);
    ol[dt] = (num * hs - nm[dt]) * inv_den;
  }
  return inv_den;
}

// Normalise, add the linear branch, store this lane's query row.
template <int kMode>
__device__ __forceinline__ void finish_query(const State& S, const SparseArgs& a, size_t bh,
                                             int qrow, bool qvalid, lds_byte* smem,
                                             const LaneOffsets& lo, int wave, int lane) {
  constexpr bool kLinAny = kMode != kSoftOnly;
  const int g = lane >> 4;
  float l = S.l_part + __shfl_xor(S.l_part, 16);
  l += __shfl_xor(l, 32);
  const float inv_l = (a.k > 0 && l > 0.0f) ? 1.0f / l : 0.0f;

  v4f ol[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) ol[dt] = v4f{0.f, 0.f, 0.f, 0.f};
  if (kLinAny) {
    half8 fq[4];
    load_phi_q(a, bh, qrow, qvalid, g, fq);
    v4f nm[8];
    float dm;
    linear_share(S, smem, fq, lo, wave, lane, nm, dm, kMode == kSubtract ? &a : nullptr, bh);
    if (kMode == kDirect) {
      // numerator and denominator summed over the unselected blocks
      const float inv_den = dm > 0.0f ? 1.0f / dm : 0.0f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) ol[dt] = nm[dt] * inv_den;
    } else {
      linear_subtract_out<true>(a, bh, g, smem, lo, fq, nm, dm, ol);
    }
  }

  if (qvalid) {
    const size_t orow = (bh * a.N + qrow) * kD;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const v4f res = S.o[dt] * inv_l + ol[dt];
      const int c0 = 16 * dt + 4 * g;
      if (a.out_f32) {
        *reinterpret_cast<v4f*>(reinterpret_cast<float*>(a.out) + orow + c0) = res;
      } else {
        uint32_t w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t b0 = __float_as_uint(res[2 * h]);
          const uint32_t b1 = __float_as_uint(res[2 * h + 1]);
          const uint32_t r0 = (b0 + 0x7fffu + ((b0 >> 16) & 1u)) >> 16;
          const uint32_t r1 = (b1 + 0x7fffu + ((b1 >> 16) & 1u)) >> 16;
          w[h] = r0 | (r1 << 16);
        }
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + orow + c0) = make_uint2(w[0], w[1]);
      }
      if (a.out_linear) *reinterpret_cast<v4f*>(a.out_linear + orow + c0) = ol[dt];
    }
  }
}

__device__ __forceinline__ TileSrc head_sources(const SparseArgs& a, size_t bh, bool lin) {
  TileSrc src;
  const size_t k8_head = (size_t)a.Np * kD, f16_head = (size_t)a.Np * kD * 2;
  src.k8 = head_rsrc(a.k8 + bh * k8_head, k8_head);
  src.v16 = head_rsrc(a.v16 + bh * (size_t)a.Np * kD, f16_head);
  src.fk16 = head_rsrc(lin ? a.fk16 + bh * (size_t)a.Np * kD : a.v16, f16_head);
  src.zb = head_rsrc(lin ? a.zb + bh * (size_t)a.Nb * kD : reinterpret_cast<const float*>(a.v16),
                     (size_t)a.Nb * kD * 4);
  return src;
}

// One workgroup per query block.  Workgroups x, x+8, ..., x+8(kGroup-1) of a
// head (same XCD, dispatched together) take the query blocks of one group.
template <int kMode>
__global__ __launch_bounds__(256, 2) void sparse_fwd_kernel(SparseArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  lds_byte* smem = (lds_byte*)smem_raw;
  constexpr bool kLinAny = kMode != kSoftOnly;
  constexpr int stage_bytes = kK8Bytes + kF16TileBytes + (kLinAny ? kF16TileBytes : 0);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int x = blockIdx.x;
  const int span = 8 * kGroup;
  const int full = gridDim.x - gridDim.x % span;
  const int i = x < full ? x - x % span + kGroup * (x & 7) + (x % span) / 8 : x;
  if (i >= a.Nb) return;  // a missing member of the last group
  const size_t bh = blockIdx.y;
  const LaneOffsets lo = lane_offsets(wave, lane);

  const int qrow = i * kBlk + 16 * wave + l16;  // this lane's query row
  const bool qvalid = qrow < a.N;
  v4i qf[2];
  State S;
  init_query(a, bh, qrow, g, qf, S);
  const float qscale = a.sq[bh * a.Nb + i] * (kInvSqrtD * kLog2e);
  const TileSrc src = head_sources(a, bh, kLinAny);

  if (kMode != kDirect) {
    const int ngroups = (a.Nb + kGroup - 1) / kGroup;
    const int32_t* col = a.sched + (bh * ngroups + i / kGroup) * (size_t)a.k * kGroup + i % kGroup;
    run_sched<kLinAny>(S, smem, stage_bytes, col, a.k, a, src, bh, qf, lo, qscale, wave, g);
  } else {
    const int nu = a.Nb - a.k;
    const int32_t* sel = a.idx + (bh * a.Nb + i) * (size_t)a.k;
    const int32_t* usel = a.uidx + (bh * a.Nb + i) * (size_t)nu;
    run_tiles<true, false>(S, smem, stage_bytes, sel, a.k, 1, a, src, bh, qf, lo, qscale, wave, g);
    run_tiles<false, true>(S, smem, stage_bytes, usel, nu, 1, a, src, bh, qf, lo, qscale, wave, g);
  }
  finish_query<kMode>(S, a, bh, qrow, qvalid, smem, lo, wave, lane);
}

// ---------------------------------------------------------------------------
// Query-block groups.  The kGroup consecutive query blocks of a group each
// keep k key blocks.  Their walks are aligned so that a key block kept by
// several of them is visited by all of those in the same step; the group's
// workgroups run side by side on one XCD, so such a tile is fetched from
// memory once and the other requests find it in L2.  The order of tiles
// changes the result only by rounding (online softmax and the sums are
// order-free).
//
// The schedule is built greedily, step by step: each step repeatedly takes the
// remaining key block with the most owners among the group members still free
// in that step (lowest index on ties), until every member has one.  When no
// remaining block fits the free members, the lowest free member takes, alone,
// its remaining block with the fewest owners (lowest index on ties); the block
// stays pending for its other owners.  Every member gets exactly k blocks.
// A ragged last key block (N not a multiple of 64) is kept out of the greedy
// and placed in the last step of every member that keeps it.
// ---------------------------------------------------------------------------


// LDS bytes of the schedule kernel: one owner byte per key block (rounded to
// words) and the union of the group's kept blocks as (block << 8 | owners).
inline size_t group_schedule_lds(int Nb, int k, int G) {
  const size_t words = ((size_t)Nb + 3) / 4;
  const size_t cap = std::min<size_t>((size_t)Nb, (size_t)G * k);
  return 4 * (words + 2 * cap);  // owner bytes, union, union sorted by owner set
}

// Schedule entries: the key block, -1 for none.  The schedule depends only on
// the kept lists, so it is built as soon as the selection is done.
struct SchedOut {
  int32_t* p;
  __device__ __forceinline__ void put(size_t i, int j) const { p[i] = j; }
};

// The union of a group's kept blocks, entry = block << 8 | remaining owners,
// held by one wave in kSchedRegs registers per lane when it fits, else in LDS
// (UnionLds: visit(f) calls f(entry) on every entry of this lane; f returns
// true when it changed the entry).
constexpr int kSchedRegs = 8;
struct UnionLds {
  uint32_t* e;
  int n, lane;
  template <typename F>
  __device__ __forceinline__ void visit(F f) {
    for (int i = lane; i < n; i += 64) {
      uint32_t v = e[i];
      if (f(v)) e[i] = v;
    }
  }
};

// The greedy steps over the union (see the group comment above); writes the
// key block of every member and step to out[s * kG + u].
template <int kG, typename Ent>
__device__ __forceinline__ void greedy_steps(Ent& ent, int k, uint32_t full, uint32_t last_busy, int lane,
                                             const SchedOut& out) {
  for (int s = 0; s < k; ++s) {
    uint32_t freem = s == k - 1 ? full & ~last_busy : full;
    while (freem) {
      // most owners among the free members, then lowest block (keys are unique)
      uint32_t best = 0u;
      ent.visit([&](uint32_t& v) {
        const uint32_t m = v & 0xffu;
        if (m && !(m & ~freem)) best = max(best, ((uint32_t)__popc(m) << 24) | (0xffffffu - (v >> 8)));
        return false;
      });
      best = wave_max_u32(best);
      uint32_t take = 0xffu;  // owners this pick may serve
      if (!best) {
        // the lowest free member alone, with its block of fewest owners
        take = 1u << __builtin_ctz(freem);
        ent.visit([&](uint32_t& v) {
          const uint32_t m = v & 0xffu;
          if (m & take) best = max(best, ((uint32_t)(kG + 1 - __popc(m)) << 24) | (0xffffffu - (v >> 8)));
          return false;
        });
        best = wave_max_u32(best);
        if (!best) {  // not reached for well-formed lists: the member has no block left
          if (lane == 0) out.put((size_t)s * kG + __builtin_ctz(freem), 0);
          freem &= ~take;
          continue;
        }
      }
      const uint32_t j = 0xffffffu - (best & 0xffffffu);
      // the lane holding block j removes the served owners; all lanes learn them
      uint32_t m = 0u;
      ent.visit([&](uint32_t& v) {
        if (v && (v >> 8) == j) {
          m = v & take & 0xffu;
          v &= ~m;
          return true;
        }
        return false;
      });
      m = wave_max_u32(m);
      if (!m) m = take & freem & (0u - (take & freem));  // not reached; keeps the loop finite
      if (lane < kG && ((m >> lane) & 1u)) out.put((size_t)s * kG + lane, (int32_t)j);
      freem &= ~m;
    }
  }
}

// The same greedy with the union in registers: one pass over the entries
// finds the pick and the lane holding it, which alone updates the entry.
template <int kG, int kR>
__device__ __forceinline__ void greedy_steps_regs(uint32_t (&u)[kR], int k, uint32_t full, uint32_t last_busy,
                                                  int lane,
                                                  const SchedOut& out) {
  for (int s = 0; s < k; ++s) {
    uint32_t freem = s == k - 1 ? full & ~last_busy : full;
    while (freem) {
      uint32_t best = 0u, take = 0xffu;
      int slot = 0;
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const uint32_t m = u[r] & 0xffu;
        const uint32_t key =
            (m && !(m & ~freem)) ? ((uint32_t)__popc(m) << 24) | (0xffffffu - (u[r] >> 8)) : 0u;
        if (key > best) best = key, slot = r;
      }
      uint32_t top = wave_max_u32(best);
      if (!top) {
        // the lowest free member alone, with its block of fewest owners
        take = 1u << __builtin_ctz(freem);
#pragma unroll
        for (int r = 0; r < kR; ++r) {
          const uint32_t m = u[r] & 0xffu;
          const uint32_t key =
              (m & take) ? ((uint32_t)(kG + 1 - __popc(m)) << 24) | (0xffffffu - (u[r] >> 8)) : 0u;
          if (key > best) best = key, slot = r;
        }
        top = wave_max_u32(best);
        if (!top) {  // not reached for well-formed lists: the member has no block left
          if (lane == 0) out.put((size_t)s * kG + __builtin_ctz(freem), 0);
          freem &= ~take;
          continue;
        }
      }
      const int holder = __builtin_ctzll(__ballot(best == top));  // keys are unique
      uint32_t mine = 0u;
      if (lane == holder) {
#pragma unroll
        for (int r = 0; r < kR; ++r)
          if (r == slot) {
            mine = u[r] & take & 0xffu;
            u[r] &= ~mine;
          }
      }
      uint32_t m = (uint32_t)__builtin_amdgcn_readlane((int)mine, holder);
      if (!m) m = take & freem & (0u - (take & freem));  // not reached; keeps the loop finite
      const uint32_t j = 0xffffffu - (top & 0xffffffu);
      if (lane < kG && ((m >> lane) & 1u)) out.put((size_t)s * kG + lane, (int32_t)j);
      freem &= ~m;
    }
  }
}

// Groups of four: the same greedy over per-owner-set queues.  The union is
// sorted (stably, so by block within a set) into 15 queues, one per owner set;
// lane L < 15 holds the head of queue L, so a pick is one wave-wide maximum
// over the heads whose set is free.  Returns false, leaving the schedule to
// the general greedy, when a step would need a block split between steps.
__device__ __forceinline__ bool greedy_queues4(const uint32_t* uni, int n, uint32_t* q, int k,
                                               uint32_t full, uint32_t last_busy, int lane,
                                               const SchedOut& out) {
  constexpr uint32_t kSets[16] = {15, 7, 11, 13, 14, 3, 5, 6, 9, 10, 12, 1, 2, 4, 8, 0};
  const uint64_t below = (1ull << lane) - 1ull;
  // queue sizes and stable positions (all counts are wave-uniform)
  int cnt[16];
#pragma unroll
  for (int t = 0; t < 15; ++t) cnt[t] = 0;
  for (int base = 0; base < n; base += 64) {
    const int e = base + lane;
    const uint32_t m = e < n ? uni[e] & 0xffu : 0u;
#pragma unroll
    for (int t = 0; t < 15; ++t) cnt[t] += __popcll(__ballot(m == kSets[t]));
  }
  int off[16], mine_head = 0, mine_end = 0;
  int run = 0;
#pragma unroll
  for (int t = 0; t < 15; ++t) {
    off[t] = run;
    if (lane == t) mine_head = run, mine_end = run + cnt[t];
    run += cnt[t];
  }
  for (int base = 0; base < n; base += 64) {
    const int e = base + lane;
    const uint32_t v = e < n ? uni[e] : 0u, m = v & 0xffu;
#pragma unroll
    for (int t = 0; t < 15; ++t) {
      const uint64_t bal = __ballot(m == kSets[t]);
      if (m == kSets[t]) q[off[t] + __popcll(bal & below)] = v >> 8;
      off[t] += __popcll(bal);
    }
  }
  __syncthreads();
  uint32_t set = 0u;
#pragma unroll
  for (int t = 0; t < 15; ++t)
    if (lane == t) set = kSets[t];
  const uint32_t size = (uint32_t)__popc(set);
  uint32_t hj = mine_head < mine_end ? q[mine_head] : 0xffffffu;

  for (int s = 0; s < k; ++s) {
    uint32_t freem = s == k - 1 ? full & ~last_busy : full;
    while (freem) {
      // most owners among the free members, then lowest block
      const bool ok = set && !(set & ~freem) && mine_head < mine_end;
      const uint32_t key = ok ? (size << 24) | (0xffffffu - hj) : 0u;
      const uint32_t top = wave_max_u32(key);
      if (!top) return false;
      const int holder = __builtin_ctzll(__ballot(key == top));
      const uint32_t bm = (uint32_t)__builtin_amdgcn_readlane((int)set, holder);
      const int32_t bj = (int32_t)(0xffffffu - (top & 0xffffffu));
      if (lane == holder) {
        ++mine_head;
        hj = mine_head < mine_end ? q[mine_head] : 0xffffffu;
      }
      if (lane < 4 && ((bm >> lane) & 1u)) out.put((size_t)s * 4 + lane, bj);
      freem &= ~bm;
    }
  }
  return true;
}

// One wave per group: sched[((bh, grp, s) * kG) + u] = key block of member u
// (query block kG*grp + u) in step s.  Members past the last block get -1.
template <int kG>
__global__ __launch_bounds__(64) void group_schedule_kernel(const int32_t* __restrict__ idx,
                                                            int Nb, int k, int ragged,
                                                            int32_t* __restrict__ sched) {
  extern __shared__ uint32_t gsm[];
  const int lane = threadIdx.x;
  const int grp = blockIdx.x;
  const size_t bh = blockIdx.y;
  const int ngroups = (Nb + kG - 1) / kG;
  const int first = grp * kG;
  const int members = min(kG, Nb - first);
  const uint32_t full = (1u << members) - 1u;
  const int words = (Nb + 3) / 4;
  uint32_t* own = gsm;          // owner byte of key block j: byte j&3 of word j>>2
  uint32_t* uni = gsm + words;  // union, ascending key block
  const SchedOut out{sched + (bh * ngroups + grp) * (size_t)k * kG};
  auto clampj = [&](int j) { return min(max(j, 0), Nb - 1); };

  for (int w = lane; w < words; w += 64) own[w] = 0u;
  __syncthreads();
  for (int u = 0; u < members; ++u) {
    const int32_t* l = idx + (bh * Nb + first + u) * (size_t)k;
    for (int t = lane; t < k; t += 64) {
      const int j = clampj(l[t]);
      atomicOr(&own[j >> 2], (1u << u) << (8 * (j & 3)));
    }
  }
  __syncthreads();
  int n = 0;
  for (int base = 0; base < Nb; base += 64) {
    const int j = base + lane;
    const uint32_t m = j < Nb ? (own[j >> 2] >> (8 * (j & 3))) & 0xffu : 0u;
    const uint64_t bal = __ballot(m != 0u);
    const int pos = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (m) uni[pos] = ((uint32_t)j << 8) | m;
    n += __popcll(bal);
  }
  __syncthreads();
  if (lane >= members && lane < kG)
    for (int s = 0; s < k; ++s) out.put((size_t)s * kG + lane, -1);
  // A ragged last key block goes to the last step of every member that keeps
  // it, so the attention kernel masks padding only in its peeled last step.
  uint32_t last_busy = 0u;
  if (ragged && n > 0 && k > 0) {
    const uint32_t v = uni[n - 1];  // the union is ascending
    if ((int)(v >> 8) == Nb - 1) {
      last_busy = v & 0xffu;
      __syncthreads();
      if (lane == 0) uni[n - 1] = v & ~0xffu;  // no owners left for the greedy
      if (lane < kG && ((last_busy >> lane) & 1u)) out.put((size_t)(k - 1) * kG + lane, Nb - 1);
      __syncthreads();
    }
  }

  if (kG == 4 && greedy_queues4(uni, n, uni + n, k, full, last_busy, lane, out)) return;
  if (n <= 64 * kSchedRegs) {
    // the union fits in registers: kSchedRegs entries per lane, 0 = empty
    uint32_t u[kSchedRegs];
#pragma unroll
    for (int r = 0; r < kSchedRegs; ++r) u[r] = lane + 64 * r < n ? uni[lane + 64 * r] : 0u;
    greedy_steps_regs<kG>(u, k, full, last_busy, lane, out);
  } else {
    UnionLds ent{uni, n, lane};
    greedy_steps<kG>(ent, k, full, last_busy, lane, out);
  }
}

// Integer S tiles for (b, h, i, j) pairs through the same staging and INT8
// matrix-core path as the attention kernel.
__global__ __launch_bounds__(256) void debug_qk_kernel(const int8_t* __restrict__ q8,
                                                       const int8_t* __restrict__ k8, int B, int H,
                                                       int Np, const int32_t* __restrict__ pairs,
                                                       int32_t* __restrict__ acc) {
  __shared__ __align__(16) unsigned char lk_raw[kK8Bytes];
  lds_byte* lk = (lds_byte*)lk_raw;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int p = blockIdx.x;
  const int b = pairs[4 * p], h = pairs[4 * p + 1], i = pairs[4 * p + 2], j = pairs[4 * p + 3];
  if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= Np / kBlk || j < 0 || j >= Np / kBlk)
    return;  // out-of-range pair: its acc tile is left untouched (uniform per workgroup)
  const size_t bh = (size_t)b * H + h;
  const LaneOffsets lo = lane_offsets(wave, lane);
  const size_t k8_head = (size_t)Np * kD;
  const __amdgpu_buffer_rsrc_t r = head_rsrc(k8 + bh * k8_head, k8_head);
#pragma unroll
  for (int m = 0; m < 2; ++m) lds_load16(r, lo.ld8, j * kK8Bytes + 4096 * m, lk + 4096 * m + 1024 * wave);
  wait_loads();
  __syncthreads();
  v4i qf[2];
  load_q8_frag(q8, bh, Np, i * kBlk + 16 * wave + l16, g, qf);
  v4i s[4];
  qk_tile(lk, qf, lo.rd8, s);
  int32_t* dst = acc + (size_t)p * kBlk * kBlk + (size_t)(16 * wave + l16) * kBlk;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[16 * kt + 4 * g + r] = s[kt][r];
}

// ---------------------------------------------------------------------------
// Backward.  Gradient of the forward above for a given dO, with the kept lists
// held fixed (top-k has no gradient) and the INT8 rounding of the logits
// passed straight through: the logits are differentiated as QK^T/sqrt(d) of
// the real Q and K, while the weights P are the forward's own.  With O_s the
// softmax output and O_l = num/den the linear one:
//   dP = dO V^T,  D = rowsum(dO * O_s),  dS = P * (dP - D)
//   dQ += dS K / sqrt(d),  dK += dS^T Q / sqrt(d),  dV += P^T dO
//   u = -rowsum(dO * O_l),  dphi(Q) = (dO (H - M)^T + u (z - z_M)) / den
//   dphi(K_u) = (dH_U) V_u + dz_U,  dV_u += phi(K_u)^T-side: phi(K_u) dH_U
// over the unselected keys u, where dH_U and dz_U of a key block are the sums,
// over the query blocks that leave it out, of phi(Q)^T dO / den and
// phi(Q)^T u / den.  Those are formed as the whole-head sums G, g_z minus the
// sums W_j, w_j over the query blocks that keep block j.
//
// Query side: one workgroup per query block, in the forward's grouped walks.
// Sweep 1 is the forward (statistics, O_s, M); then D, u and dphi(Q); sweep 2
// re-walks the kept tiles (INT8 K codes, V rows, K^T) for dQ += dS K.  It
// leaves, per query row, the log2 maximum, 1/l, D and u, and phi(Q)/den
// transposed per block, for the key side.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) const v4f lds_v4f;

constexpr int kBwdVOff = kK8Bytes;                        // V rows [64 keys][128] bf16
constexpr int kBwdKtOff = kK8Bytes + kF16TileBytes;       // K^T [128][64 perm keys] bf16
constexpr int kBwdStage = kK8Bytes + 2 * kF16TileBytes;   // 40 KB
constexpr int kMRowOff = 33 * 1024;                       // M row-major, after linear_share's area
static_assert(kHOff + kD * kD * 2 + 1024 <= 2 * (kK8Bytes + 2 * kF16TileBytes),
              "staged linear state exceeds the forward stages");
constexpr int kZOffShared = kD * kD * 2;                  // z_M as linear_share leaves it (fp32 [128])

// Position of row t of a block in the permuted order of the transposed tiles
// (inside each 32-row half: rows 4g..4g+3 at 8g.., rows 16+4g.. at 8g+4..).
__device__ __forceinline__ int perm_row(int t) {
  const int r = t & 31;
  return 32 * (t >> 5) + 8 * ((r & 15) >> 2) + (r & 3) + 4 * (r >> 4);
}
constexpr float kSqrtD = 11.313708498984761f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float phi_slope(float x, int phi) {
  if (phi == kPhiElu1) return x > 0.0f ? 1.0f : __expf(x);
  return x > 0.0f ? 1.0f : 0.0f;
}

// 16 bytes of a 256-byte row, read as 8 bf16 at 16-byte chunk `chunk`, from a
// tile whose row r keeps chunk ch at ch ^ (r & 15).
__device__ __forceinline__ bf16x8 lds_row_frag(const lds_byte* base, int row, int chunk) {
  return *(lds_bf16x8*)(base + row * 256 + ((chunk ^ (row & 15)) << 4));
}

// Byte offset a lane fetches when a wave moves rounds of 1 KB of a tile with
// 256-byte rows into LDS so that row r keeps chunk ch at ch ^ (r & 15).
__device__ __forceinline__ int row256_ld(int wave, int lane) {
  const int r = 4 * wave + (lane >> 4);
  return r * 256 + ((((lane & 15) ^ r) & 15) << 4);
}

// Stores 4 consecutive channels of one row (bf16 with round to nearest even,
// or fp32).
__device__ __forceinline__ void store_row4(void* base, size_t off, v4f x, int f32) {
  if (f32) {
    *reinterpret_cast<v4f*>(reinterpret_cast<float*>(base) + off) = x;
  } else {
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t b0 = __float_as_uint(x[2 * h]);
      const uint32_t b1 = __float_as_uint(x[2 * h + 1]);
      const uint32_t r0 = (b0 + 0x7fffu + ((b0 >> 16) & 1u)) >> 16;
      const uint32_t r1 = (b1 + 0x7fffu + ((b1 >> 16) & 1u)) >> 16;
      w[h] = r0 | (r1 << 16);
    }
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + off) = make_uint2(w[0], w[1]);
  }
}

__device__ __forceinline__ void store_one(void* base, size_t off, float x, int f32) {
  if (f32) {
    reinterpret_cast<float*>(base)[off] = x;
  } else {
    const uint32_t b = __float_as_uint(x);
    reinterpret_cast<uint16_t*>(base)[off] = (uint16_t)((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
  }
}

struct BwdQArgs {
  SparseArgs f;           // forward inputs: raw Q, codes, schedule, linear staging
  const uint16_t* v;      // V bf16 [BH, N, D]
  const uint16_t* kt;     // K^T bf16 per block [BH, Nb, D, 64 permuted keys]
  const uint16_t* dout;   // dO bf16 [BH, N, D]
  const uint16_t* hb;     // H bf16 row-major [BH, D(phi), D(v)], staged scale (phi/16)
  float* stats;           // [BH, Nb, 4, 64]: log2 max, 1/l, D (row order), u (permuted)
  uint16_t* fqs;          // (phi(Q)/den)^T bf16 per block [BH, Nb, D, 64 permuted rows]
  void* dq;
  int grad_f32;
};

struct BwdQSrc {
  __amdgpu_buffer_rsrc_t k8, v, kt;
};

__device__ __forceinline__ void issue_bwd_q_tile(lds_byte* st, const BwdQSrc& src, int j, int wave,
                                                 const LaneOffsets& lo, int vld) {
#pragma unroll
  for (int m = 0; m < 4; ++m)
    lds_load16(src.v, vld, j * kF16TileBytes + 4096 * m, st + kBwdVOff + 4096 * m + 1024 * wave);
#pragma unroll
  for (int m = 0; m < 2; ++m)
    lds_load16(src.k8, lo.ld8, j * kK8Bytes + 4096 * m, st + 4096 * m + 1024 * wave);
#pragma unroll
  for (int m = 0; m < 4; ++m)
    lds_load16(src.kt, lo.ld8, j * kF16TileBytes + 4096 * m, st + kBwdKtOff + 4096 * m + 1024 * wave);
}

// One kept tile of sweep 2: S^T from the codes, the forward's fp16 weights,
// dP^T = V dO^T, dS^T, and dQ^T += K^T dS^T.
template <bool kMask>
__device__ __forceinline__ void bwd_q_tile(const lds_byte* st, const v4i qf[2], const bf16x8 gf[4],
                                           const LaneOffsets& lo, float cs, float m_fin,
                                           float inv_l, float Dt, int kvalid, int g, int l16,
                                           v4f dqa[8]) {
  v4i s[4];
  qk_tile(st, qf, lo.rd8, s);
  v4f dp[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    dp[kt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      dp[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_row_frag(st + kBwdVOff, 16 * kt + l16, 4 * ks + g),
                                                       gf[ks], dp[kt], 0, 0, 0);
  }
  bf16x8 dsf[2];
  const float nm = -m_fin;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float p = (float)(_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf((float)s[kt][r], cs, nm));
      if (kMask && 16 * kt + 4 * g + r >= kvalid) p = 0.0f;
      dsf[kt >> 1][4 * (kt & 1) + r] = (__bf16)(p * inv_l * (dp[kt][r] - Dt));
    }
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16x8 ak = *(lds_bf16x8*)(st + kBwdKtOff + ct * 2048 + (lo.rd8 ^ (64 * c)));
      dqa[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, dsf[c], dqa[ct], 0, 0, 0);
    }
}

template <bool kLin>
__global__ __launch_bounds__(256, 2) void bwd_q_kernel(BwdQArgs b) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  lds_byte* smem = (lds_byte*)smem_raw;
  const SparseArgs& a = b.f;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int x = blockIdx.x;
  const int span = 8 * kGroup;
  const int full = gridDim.x - gridDim.x % span;
  const int i = x < full ? x - x % span + kGroup * (x & 7) + (x % span) / 8 : x;
  if (i >= a.Nb) return;  // a missing member of the last group
  const size_t bh = blockIdx.y;
  const LaneOffsets lo = lane_offsets(wave, lane);
  const int qrow = i * kBlk + 16 * wave + l16;
  const bool qvalid = qrow < a.N;
  v4i qf[2];
  State S;
  init_query(a, bh, qrow, g, qf, S);
  const float qscale = a.sq[bh * a.Nb + i] * (kInvSqrtD * kLog2e);
  const int ngroups = (a.Nb + kGroup - 1) / kGroup;
  const int32_t* col =
      a.k > 0 ? a.sched + (bh * ngroups + i / kGroup) * (size_t)a.k * kGroup + i % kGroup : nullptr;
  run_sched<kLin>(S, smem, kBwdStage, col, a.k, a, head_sources(a, bh, kLin), bh, qf, lo, qscale,
                  wave, g);

  // softmax statistics of this lane's query and D = dO . O_s
  float l = S.l_part + __shfl_xor(S.l_part, 16);
  l += __shfl_xor(l, 32);
  const float inv_l = (a.k > 0 && l > 0.0f && qvalid) ? 1.0f / l : 0.0f;
  const float m_fin = inv_l > 0.0f ? S.m_run : INFINITY;  // rows without weights get P = 0
  const uint16_t* dorow = b.dout + ((size_t)bh * a.N + (qvalid ? qrow : 0)) * kD;
  v4f go[8];  // dO in the O^T layout, channel 16dt + 4g + r
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const uint2 w = *reinterpret_cast<const uint2*>(dorow + 16 * dt + 4 * g);
    go[dt] = qvalid ? v4f{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)}
                    : v4f{0.f, 0.f, 0.f, 0.f};
  }
  float dpart = 0.0f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) dpart += go[dt][r] * S.o[dt][r];
  dpart += __shfl_xor(dpart, 16);
  dpart += __shfl_xor(dpart, 32);
  const float Dt = dpart * inv_l;

  // dO of this lane's query as B operands (channels 32ks + 8g + e)
  bf16x8 gf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint4 w = *reinterpret_cast<const uint4*>(dorow + 32 * ks + 8 * g);
    gf[ks] = qvalid ? __builtin_bit_cast(bf16x8, w) : bf16x8{};
  }

  v4f dqa[8];  // dQ^T, channel 16ct + 4g + r, in units of 1/sqrt(d)
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) dqa[ct] = v4f{0.f, 0.f, 0.f, 0.f};
  float u = 0.0f;
  const int tl = 16 * wave + l16;  // row within the block
  if (kLin) {
    half8 fq[4];
    load_phi_q(a, bh, qrow, qvalid, g, fq);
    v4f nm[8];
    float dm;
    linear_share(S, smem, fq, lo, wave, lane, nm, dm);
    v4f ol[8];
    const float inv_den = linear_subtract_out<false>(a, bh, g, smem, lo, fq, nm, dm, ol);
    float up = 0.0f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) up += go[dt][r] * ol[dt][r];
    up += __shfl_xor(up, 16);
    up += __shfl_xor(up, 32);
    u = qvalid ? -up : 0.0f;
    // M (kept share, staged scale) row-major as bf16: row c = 32w + 16x + l16
    // holds M[c][16dt + 4g + r]
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int xx = 0; xx < 2; ++xx) {
        const int c = 32 * wave + 16 * xx + l16;
        bf16x8 w4;
#pragma unroll
        for (int r = 0; r < 4; ++r) w4[r] = (__bf16)S.mk[dt][xx][r];
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 h4 = {w4[0], w4[1], w4[2], w4[3]};
        *(__attribute__((address_space(3))) bf16x4*)(smem + kMRowOff + c * 256 +
                                                     (((2 * dt + (g >> 1)) ^ l16) << 4) + 8 * (g & 1)) = h4;
      }
    lds_barrier();
    // dphi(Q)^T[c][t] = ((H - M) dO^T)[c][t] + u (z - z_M)[c], in the staged
    // scale: the true value is that times inv_den / 16
    const __bf16* hrow = reinterpret_cast<const __bf16*>(b.hb) + bh * kD * kD;
    const float* zz = a.z + bh * kD;
    const uint16_t* qrowp = a.q + ((size_t)bh * a.N + (qvalid ? qrow : 0)) * kD;
    const float fscale = inv_den * (1.0f / 256.0f);  // phi(Q) -> phi(Q)/den (true scale)
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      v4f ah = v4f{0.f, 0.f, 0.f, 0.f}, am = v4f{0.f, 0.f, 0.f, 0.f};
      bf16x8 hv[4];  // the row's four fragments, loaded together
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        hv[ks] = *reinterpret_cast<const bf16x8*>(hrow + (16 * ct + l16) * kD + 32 * ks + 8 * g);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        ah = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hv[ks], gf[ks], ah, 0, 0, 0);
        am = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_row_frag(smem + kMRowOff, 16 * ct + l16, 4 * ks + g),
                                                     gf[ks], am, 0, 0, 0);
      }
      const uint2 qw = *reinterpret_cast<const uint2*>(qrowp + 16 * ct + 4 * g);
      const float qv[4] = {bf16_lo(qw.x), bf16_hi(qw.x), bf16_lo(qw.y), bf16_hi(qw.y)};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = 16 * ct + 4 * g + r;
        const float zi = zz[c] - *(__attribute__((address_space(3))) const float*)(smem + kZOffShared + 4 * c);
        const float dphi = (ah[r] - am[r] + u * zi) * (inv_den * 0.0625f);
        dqa[ct][r] = qvalid ? dphi * phi_slope(qv[r], a.phi) * kSqrtD : 0.0f;
        // phi(Q)/den, transposed into [c][permuted row] (region of M^T, now free)
        const float fv = qvalid ? phi_apply(qv[r], a.phi) * fscale : 0.0f;
        *(__attribute__((address_space(3))) __bf16*)(smem + c * 128 + 2 * perm_row(tl)) = (__bf16)fv;
      }
    }
    lds_barrier();
    // the block's (phi(Q)/den)^T: 16 KB, 16 bytes per thread per step
    uint16_t* dst = b.fqs + ((size_t)bh * a.Nb + i) * (kD * kBlk);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int off = 16 * (t + 256 * m);
      *reinterpret_cast<v4i*>(reinterpret_cast<unsigned char*>(dst) + off) = *(lds_v4i*)(smem + off);
    }
  }
  if (lane < 16) {
    float* st4 = b.stats + ((size_t)bh * a.Nb + i) * 256;
    st4[tl] = m_fin;
    st4[64 + tl] = inv_l;
    st4[128 + tl] = Dt;
    st4[192 + perm_row(tl)] = u;
  }

  // sweep 2: dQ += dS K over the kept tiles
  if (a.k > 0) {
    lds_barrier();  // LDS is reused for the tile stages
    BwdQSrc src;
    const size_t k8_head = (size_t)a.Np * kD;
    src.k8 = head_rsrc(a.k8 + bh * k8_head, k8_head);
    src.v = head_rsrc(b.v + bh * (size_t)a.N * kD, (size_t)a.N * kD * 2);
    src.kt = head_rsrc(b.kt + bh * (size_t)a.Np * kD, (size_t)a.Np * kD * 2);
    const int vld = row256_ld(wave, lane);
    auto block_of = [&](int p) { return min(max(ld_uniform(col, (size_t)p * kGroup), 0), a.Nb - 1); };
    auto scale_of = [&](int j) { return ld_uniform(a.sk, bh * a.Nb + j); };
    int j = block_of(0);
    issue_bwd_q_tile(smem, src, j, wave, lo, vld);
    float sc = scale_of(j);
    const int nm1 = a.k - 1;
    for (int p = 0; p < nm1; p += 2) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int pp = p + half;
        if (pp < nm1) {
          lds_byte* cur = smem + half * kBwdStage;
          lds_byte* nxt = smem + (1 - half) * kBwdStage;
          wait_loads();
          lds_barrier();
          const int jn = block_of(pp + 1);
          issue_bwd_q_tile(nxt, src, jn, wave, lo, vld);
          const float sn = scale_of(jn);
          bwd_q_tile<false>(cur, qf, gf, lo, qscale * sc, m_fin, inv_l, Dt, kBlk, g, l16, dqa);
          j = jn;
          sc = sn;
        }
      }
    }
    const int kvalid = a.N - j * kBlk;
    const lds_byte* cur = smem + (nm1 & 1) * kBwdStage;
    wait_loads();
    lds_barrier();
    if (kvalid < kBlk)
      bwd_q_tile<true>(cur, qf, gf, lo, qscale * sc, m_fin, inv_l, Dt, kvalid, g, l16, dqa);
    else
      bwd_q_tile<false>(cur, qf, gf, lo, qscale * sc, m_fin, inv_l, Dt, kBlk, g, l16, dqa);
  }
  if (qvalid) {
    const size_t orow = (bh * a.N + qrow) * kD;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) store_row4(b.dq, orow + 16 * ct + 4 * g, dqa[ct] * kInvSqrtD, b.grad_f32);
  }
}

// ---------------------------------------------------------------------------
// Key side: one workgroup per key block j (four waves, 16 keys each), walking
// the query blocks that keep j (shared with the group's other key blocks first).  Per query block i it stages the
// INT8 Q codes, dO rows, dO^T, Q^T, (phi(Q)/den)^T and the row statistics:
//   S, P (the forward's weights), dP = dO V^T, dS
//   dV += P^T dO,  dK += dS^T Q,  W += (phi(Q)/den)^T dO,  w += (phi(Q)/den)^T u
// then the linear gradient through G - W and g_z - w.
// ---------------------------------------------------------------------------
constexpr int kKvDoOff = kK8Bytes;                        // dO rows [64][128] bf16
constexpr int kKvDotOff = kK8Bytes + kF16TileBytes;       // dO^T [128][64 perm] bf16
constexpr int kKvQtOff = kK8Bytes + 2 * kF16TileBytes;    // Q^T
constexpr int kKvFqOff = kK8Bytes + 3 * kF16TileBytes;    // (phi(Q)/den)^T
constexpr int kKvStOff = kK8Bytes + 4 * kF16TileBytes;    // 4 x 64 fp32 statistics
constexpr int kKvStage = kKvStOff + 1024;                  // 73 KB

struct BwdKvArgs {
  const int8_t* q8;
  const int8_t* k8;
  const float* sq;
  const float* sk;
  const uint16_t* kin;    // K bf16 [BH, N, D]
  const uint16_t* v;      // V bf16 [BH, N, D]
  const uint16_t* dout;   // dO bf16 [BH, N, D]
  const uint16_t* qt;     // Q^T bf16 per block
  const uint16_t* dot;    // dO^T bf16 per block
  const uint16_t* fqs;    // (phi(Q)/den)^T bf16 per block
  const float* stats;     // [BH, Nb, 4, 64]
  const int32_t* coff;    // [BH, Nb + 1] column starts within the head's list
  const int32_t* cidx;    // [BH, Nb * k] query blocks keeping each key block
  const float* G;         // [BH, D, D] sum over all query blocks of (phi(Q)/den)^T dO
  const float* gz;        // [BH, D]    sum of (phi(Q)/den)^T u
  int N, Nb, Np, k, phi;
  void* dk;
  void* dv;
  int grad_f32;
};

struct BwdKvSrc {
  __amdgpu_buffer_rsrc_t q8, dout, dot, qt, fqs, stats;
};

template <bool kLin>
__device__ __forceinline__ void issue_kv_tile(lds_byte* st, const BwdKvSrc& src, int i, int wave,
                                              const LaneOffsets& lo, int vld, int lane) {
#pragma unroll
  for (int m = 0; m < 4; ++m)
    lds_load16(src.dout, vld, i * kF16TileBytes + 4096 * m, st + kKvDoOff + 4096 * m + 1024 * wave);
#pragma unroll
  for (int m = 0; m < 2; ++m)
    lds_load16(src.q8, lo.ld8, i * kK8Bytes + 4096 * m, st + 4096 * m + 1024 * wave);
#pragma unroll
  for (int m = 0; m < 4; ++m)
    lds_load16(src.dot, lo.ld8, i * kF16TileBytes + 4096 * m, st + kKvDotOff + 4096 * m + 1024 * wave);
#pragma unroll
  for (int m = 0; m < 4; ++m)
    lds_load16(src.qt, lo.ld8, i * kF16TileBytes + 4096 * m, st + kKvQtOff + 4096 * m + 1024 * wave);
  if (kLin) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
      lds_load16(src.fqs, lo.ld8, i * kF16TileBytes + 4096 * m, st + kKvFqOff + 4096 * m + 1024 * wave);
  }
  if (wave == 0) lds_load16(src.stats, 16 * lane, i * 1024, st + kKvStOff);
}

struct KvAcc {
  v4f dv[8];     // dV[key 4g + r][e 16et + l16]
  v4f dk[8];     // dK[key 4g + r][c 16ct + l16] (units of 1/sqrt(d))
  v4f w[2][8];   // W[c = 32w + 16mt + 4g + r][e = 16et + l16]
  v4f wz[2];     // w[c] in the lanes with l16 == 0
};

template <bool kLin>
__device__ __forceinline__ void kv_tile(const lds_byte* st, const v4i kf[2], const bf16x8 vf[4],
                                        const LaneOffsets& lo, float cs, int wave, int g, int l16,
                                        KvAcc& A) {
  v4i s[4];
  qk_tile(st, kf, lo.rd8, s);  // s[tt][r] = S[row 16tt + 4g + r][key l16]
  v4f dp[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    dp[tt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      dp[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_row_frag(st + kKvDoOff, 16 * tt + l16, 4 * ks + g),
                                                       vf[ks], dp[tt], 0, 0, 0);
  }
  bf16x8 pa[2], dsa[2];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const v4f mr = *(lds_v4f*)(st + kKvStOff + 4 * (16 * tt + 4 * g));
    const v4f il = *(lds_v4f*)(st + kKvStOff + 256 + 4 * (16 * tt + 4 * g));
    const v4f dd = *(lds_v4f*)(st + kKvStOff + 512 + 4 * (16 * tt + 4 * g));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p =
          (float)(_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf((float)s[tt][r], cs, -mr[r])) * il[r];
      pa[tt >> 1][4 * (tt & 1) + r] = (__bf16)p;
      dsa[tt >> 1][4 * (tt & 1) + r] = (__bf16)(p * (dp[tt][r] - dd[r]));
    }
  }
  bf16x8 af[2][2], ub[2];
  if (kLin) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        af[mt][c] = *(lds_bf16x8*)(st + kKvFqOff + (2 * wave + mt) * 2048 + (lo.rd8 ^ (64 * c)));
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const v4f u0 = *(lds_v4f*)(st + kKvStOff + 768 + 4 * (32 * c + 8 * g));
      const v4f u1 = *(lds_v4f*)(st + kKvStOff + 768 + 4 * (32 * c + 8 * g + 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ub[c][e] = l16 == 0 ? (__bf16)u0[e] : (__bf16)0.0f;
        ub[c][4 + e] = l16 == 0 ? (__bf16)u1[e] : (__bf16)0.0f;
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int et = 0; et < 8; ++et) {
      const bf16x8 bo = *(lds_bf16x8*)(st + kKvDotOff + et * 2048 + (lo.rd8 ^ (64 * c)));
      A.dv[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[c], bo, A.dv[et], 0, 0, 0);
      if (kLin) {
        A.w[0][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[0][c], bo, A.w[0][et], 0, 0, 0);
        A.w[1][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[1][c], bo, A.w[1][et], 0, 0, 0);
      }
    }
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const bf16x8 bq = *(lds_bf16x8*)(st + kKvQtOff + ct * 2048 + (lo.rd8 ^ (64 * c)));
      A.dk[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dsa[c], bq, A.dk[ct], 0, 0, 0);
    }
    if (kLin) {
      A.wz[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[0][c], ub[c], A.wz[0], 0, 0, 0);
      A.wz[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[1][c], ub[c], A.wz[1], 0, 0, 0);
    }
  }
}

template <bool kLin>
__global__ __launch_bounds__(256, 1) void bwd_kv_kernel(BwdKvArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  lds_byte* smem = (lds_byte*)smem_raw;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  // workgroups x, x+8, x+16, x+24 (one XCD, dispatched together) take four
  // consecutive key blocks, whose columns overlap, so their staged query
  // blocks meet in that XCD's L2
  const int x = blockIdx.x;
  const int span = 8 * kGroup;
  const int full = gridDim.x - gridDim.x % span;
  const int j = x < full ? x - x % span + kGroup * (x & 7) + (x % span) / 8 : x;
  const size_t bh = blockIdx.y;
  const LaneOffsets lo = lane_offsets(wave, lane);
  const int krow = j * kBlk + 16 * wave + l16;  // this lane's key as a B/A operand row
  const bool kvalid = krow < a.N;
  v4i kf[2];
  load_q8_frag(a.k8, bh, a.Np, krow, g, kf);
  const uint16_t* vrow = a.v + ((size_t)bh * a.N + (kvalid ? krow : 0)) * kD;
  bf16x8 vf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint4 w = *reinterpret_cast<const uint4*>(vrow + 32 * ks + 8 * g);
    vf[ks] = kvalid ? __builtin_bit_cast(bf16x8, w) : bf16x8{};
  }
  KvAcc A;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    A.dv[e] = v4f{0.f, 0.f, 0.f, 0.f};
    A.dk[e] = v4f{0.f, 0.f, 0.f, 0.f};
    A.w[0][e] = v4f{0.f, 0.f, 0.f, 0.f};
    A.w[1][e] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  A.wz[0] = A.wz[1] = v4f{0.f, 0.f, 0.f, 0.f};

  // this key block's column, clamped to the head's list
  const int c0 = a.coff ? min(max(a.coff[bh * (a.Nb + 1) + j], 0), a.Nb * a.k) : 0;
  const int n = a.coff ? min(a.coff[bh * (a.Nb + 1) + j + 1], a.Nb * a.k) - c0 : 0;
  if (n > 0) {
    const int32_t* list = a.cidx + bh * (size_t)a.Nb * a.k + c0;
    BwdKvSrc src;
    const size_t f16_head = (size_t)a.Np * kD * 2;
    src.q8 = head_rsrc(a.q8 + bh * (size_t)a.Np * kD, (size_t)a.Np * kD);
    src.dout = head_rsrc(a.dout + bh * (size_t)a.N * kD, (size_t)a.N * kD * 2);
    src.dot = head_rsrc(a.dot + bh * (size_t)a.Np * kD, f16_head);
    src.qt = head_rsrc(a.qt + bh * (size_t)a.Np * kD, f16_head);
    src.fqs = head_rsrc(kLin ? a.fqs + bh * (size_t)a.Np * kD : a.qt, f16_head);
    src.stats = head_rsrc(a.stats + bh * (size_t)a.Nb * 256, (size_t)a.Nb * 1024);
    const int vld = row256_ld(wave, lane);
    const float ks = a.sk[bh * a.Nb + j] * (kInvSqrtD * kLog2e);
    auto block_of = [&](int p) { return min(max(ld_uniform(list, (size_t)p), 0), a.Nb - 1); };
    int i = block_of(0);
    issue_kv_tile<kLin>(smem, src, i, wave, lo, vld, lane);
    float si = ld_uniform(a.sq, bh * a.Nb + i);
    for (int p = 0; p < n; p += 2) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int pp = p + half;
        if (pp < n) {
          lds_byte* cur = smem + half * kKvStage;
          lds_byte* nxt = smem + (1 - half) * kKvStage;
          wait_loads();
          lds_barrier();  // block pp is in LDS; every wave is done with block pp-1
          int in = i;
          float sn = si;
          if (pp + 1 < n) {
            in = block_of(pp + 1);
            issue_kv_tile<kLin>(nxt, src, in, wave, lo, vld, lane);
            sn = ld_uniform(a.sq, bh * a.Nb + in);
          }
          kv_tile<kLin>(cur, kf, vf, lo, si * ks, wave, g, l16, A);
          i = in;
          si = sn;
        }
      }
    }
  }

  // linear gradient through G - W and g_z - w
  v4f dfk[8], dvl[8];
  constexpr int kGaOff = 0, kGbOff = 32 * 1024, kGzOff = 64 * 1024;
  if (kLin) {
    lds_barrier();  // every wave is done with the stages
    const float* Gh = a.G + bh * kD * kD;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int et = 0; et < 8; ++et)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = 32 * wave + 16 * mt + 4 * g + r;
          const int e = 16 * et + l16;
          const __bf16 gv = (__bf16)(Gh[c * kD + e] - A.w[mt][et][r]);
          *(__attribute__((address_space(3))) __bf16*)(smem + kGaOff + c * 256 +
                                                      ((((e >> 3) ^ (c & 15)) & 15) << 4) + 2 * (e & 7)) = gv;
          *(__attribute__((address_space(3))) __bf16*)(smem + kGbOff + e * 256 +
                                                      ((((c >> 3) ^ (e & 15)) & 15) << 4) + 2 * (c & 7)) = gv;
        }
    if (l16 == 0) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = 32 * wave + 16 * mt + 4 * g + r;
          *(__attribute__((address_space(3))) float*)(smem + kGzOff + 4 * c) = a.gz[bh * kD + c] - A.wz[mt][r];
        }
    }
    lds_barrier();
    // phi(K) of this lane's key as A operands (channels 32ks + 8g + e)
    const uint16_t* krp = a.kin + ((size_t)bh * a.N + (kvalid ? krow : 0)) * kD;
    bf16x8 fk[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 w = *reinterpret_cast<const uint4*>(krp + 32 * ks + 8 * g);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xv = (e & 1) ? bf16_hi(ww[e >> 1]) : bf16_lo(ww[e >> 1]);
        fk[ks][e] = kvalid ? (__bf16)phi_apply(xv, a.phi) : (__bf16)0.0f;
      }
    }
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      dfk[ct] = v4f{0.f, 0.f, 0.f, 0.f};
      dvl[ct] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        dfk[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[ks], lds_row_frag(smem + kGaOff, 16 * ct + l16, 4 * ks + g),
                                                          dfk[ct], 0, 0, 0);
        dvl[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fk[ks], lds_row_frag(smem + kGbOff, 16 * ct + l16, 4 * ks + g),
                                                          dvl[ct], 0, 0, 0);
      }
    }
  }
  // outputs: lane holds keys 16w + 4g + r, channel 16ct + l16
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int kr = j * kBlk + 16 * wave + 4 * g + r;
    if (kr >= a.N) continue;
    const size_t orow = (bh * a.N + kr) * kD;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const int c = 16 * ct + l16;
      float dkv = A.dk[ct][r] * kInvSqrtD;
      float dvv = A.dv[ct][r];
      if (kLin) {
        const uint16_t kb = a.kin[orow + c];
        const float gzh = *(__attribute__((address_space(3))) const float*)(smem + kGzOff + 4 * c);
        dkv += (dfk[ct][r] + gzh) * phi_slope(bf16_lo(kb), a.phi);
        dvv += dvl[ct][r];
      }
      store_one(a.dk, orow + c, dkv, a.grad_f32);
      store_one(a.dv, orow + c, dvv, a.grad_f32);
    }
  }
}

template <int kMode>
hipError_t launch_mode(const SparseArgs& a, const Shape& sh, hipStream_t s) {
  constexpr size_t stage = (size_t)kK8Bytes + kF16TileBytes + (kMode != kSoftOnly ? kF16TileBytes : 0);
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(sparse_fwd_kernel<kMode>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)(2 * stage));
  });
  // grouped walks need every member's workgroup, so the block count is rounded up
  const int slots = kMode == kDirect ? sh.Nb : kGroup * ((sh.Nb + kGroup - 1) / kGroup);
  sparse_fwd_kernel<kMode><<<dim3(slots, sh.BH), 256, 2 * stage, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_fwd(const uint16_t* q, const Workspace& ws, const Shape& sh, int phi,
                             void* out, int out_f32, float* out_linear, hipStream_t s) {
  SparseArgs a;
  a.q = q;
  a.q8 = ws.q8;
  a.k8 = ws.k8;
  a.sq = ws.sq;
  a.sk = ws.sk;
  a.idx = ws.idx;
  a.uidx = ws.uidx;
  a.sched = ws.sched;
  a.fk16 = ws.fk16;
  a.v16 = ws.v16;
  a.zb = ws.zb;
  a.h16t = ws.h16t;
  a.hscale = ws.hscale;
  a.z = ws.z;
  a.N = sh.N;
  a.Nb = sh.Nb;
  a.Np = sh.Np;
  a.k = sh.k;
  a.phi = phi;
  a.out = out;
  a.out_f32 = out_f32;
  a.out_linear = out_linear;
  const bool lin = phi != kPhiNone && sh.k < sh.Nb;
  if (lin && linear_direct(sh)) return launch_mode<kDirect>(a, sh, s);
  if (!lin) return launch_mode<kSoftOnly>(a, sh, s);
  return launch_mode<kSubtract>(a, sh, s);
}

hipError_t launch_bwd_q(const uint16_t* q, const uint16_t* v, const uint16_t* dout,
                        const Workspace& ws, const BwdWorkspace& bw, const Shape& sh, int phi,
                        void* dq, int grad_f32, hipStream_t s) {
  BwdQArgs b;
  SparseArgs& a = b.f;
  a = SparseArgs{};
  a.q = q;
  a.q8 = ws.q8;
  a.k8 = ws.k8;
  a.sq = ws.sq;
  a.sk = ws.sk;
  a.sched = ws.sched;
  a.fk16 = ws.fk16;
  a.v16 = ws.v16;
  a.zb = ws.zb;
  a.h16t = ws.h16t;
  a.hscale = ws.hscale;
  a.z = ws.z;
  a.N = sh.N;
  a.Nb = sh.Nb;
  a.Np = sh.Np;
  a.k = sh.k;
  a.phi = phi;
  b.v = v;
  b.kt = bw.kt;
  b.dout = dout;
  b.hb = bw.hb;
  b.stats = bw.stats;
  b.fqs = bw.fqs;
  b.dq = dq;
  b.grad_f32 = grad_f32;
  const bool lin = phi != kPhiNone && sh.k < sh.Nb;
  const int slots = kGroup * ((sh.Nb + kGroup - 1) / kGroup);
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_q_kernel<true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kBwdStage);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_q_kernel<false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kBwdStage);
  });
  if (lin)
    bwd_q_kernel<true><<<dim3(slots, sh.BH), 256, 2 * kBwdStage, s>>>(b);
  else
    bwd_q_kernel<false><<<dim3(slots, sh.BH), 256, 2 * kBwdStage, s>>>(b);
  return hipGetLastError();
}

hipError_t launch_bwd_kv(const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                         const Workspace& ws, const BwdWorkspace& bw, const Shape& sh, int phi,
                         void* dk, void* dv, int grad_f32, hipStream_t s) {
  BwdKvArgs a;
  a.q8 = ws.q8;
  a.k8 = ws.k8;
  a.sq = ws.sq;
  a.sk = ws.sk;
  a.kin = k;
  a.v = v;
  a.dout = dout;
  a.qt = bw.qt;
  a.dot = bw.dot;
  a.fqs = bw.fqs;
  a.stats = bw.stats;
  a.coff = sh.k > 0 ? bw.coff : nullptr;
  a.cidx = bw.cidx;
  a.G = bw.G;
  a.gz = bw.gz;
  a.N = sh.N;
  a.Nb = sh.Nb;
  a.Np = sh.Np;
  a.k = sh.k;
  a.phi = phi;
  a.dk = dk;
  a.dv = dv;
  a.grad_f32 = grad_f32;
  const bool lin = phi != kPhiNone && sh.k < sh.Nb;
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_kv_kernel<true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kKvStage);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_kv_kernel<false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kKvStage);
  });
  if (lin)
    bwd_kv_kernel<true><<<dim3(sh.Nb, sh.BH), 256, 2 * kKvStage, s>>>(a);
  else
    bwd_kv_kernel<false><<<dim3(sh.Nb, sh.BH), 256, 2 * kKvStage, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_group_schedule(const int32_t* idx, const Shape& sh, int32_t* sched,
                                 hipStream_t s) {
  if (sh.k <= 0) return hipSuccess;
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(group_schedule_kernel<kGroup>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  });
  const int ngroups = (sh.Nb + kGroup - 1) / kGroup;
  group_schedule_kernel<kGroup><<<dim3(ngroups, sh.BH), 64, group_schedule_lds(sh.Nb, sh.k, kGroup), s>>>(
      idx, sh.Nb, sh.k, sh.N != sh.Nb * kBlk ? 1 : 0, sched);
  return hipGetLastError();
}

hipError_t launch_debug_qk(const int8_t* q8, const int8_t* k8, const Shape& sh,
                           const int32_t* pairs, int n_pairs, int32_t* acc, hipStream_t s) {
  debug_qk_kernel<<<n_pairs, 256, 0, s>>>(q8, k8, sh.B, sh.H, sh.Np, pairs, acc);
  return hipGetLastError();
}

}  // namespace sla
