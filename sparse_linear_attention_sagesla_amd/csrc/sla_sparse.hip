// Block-sparse SageSLA attention kernel for gfx950 (CDNA4).
//
// One workgroup = one 64-row query block of one (b,h); four waves, each
// owning 16 query rows.  The workgroup walks a list of key blocks (tiles).
// Per tile, staged in LDS by direct global->LDS 16-byte loads, double-buffered
// so the next tile streams in while this one is computed:
//   K8_j   int8 [64 keys][128]      (8 KB)   -> S^T = K8_j Q8_i^T     (INT8 MFMA)
//   V_j    fp16 [128][64 perm keys] (16 KB)  -> O^T += V_j^T P^T      (fp16 MFMA)
//   phiK_j fp16 [128][64 perm keys] (16 KB)  -> M^T += V_j^T phiK_j   (fp16 MFMA)
//          (lower-bit option: e4m3 codes, 8 KB, turned into fp16 with the
//          block's decode scale as they are read)
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
// normalised, over the unselected blocks U, in one of two forms:
//   subtraction: H_U = H - M and z_U = z - z_M, with H, z the whole-head sums
//                and M = sum phi(K_j)^T V_j, z_M = sum of the block sums of
//                phi(K_j) over the kept tiles (kept tiles carry both
//                branches); the differences are taken in fp32 (H, M) and
//                fp64 (z, z_M) before anything is rounded to fp16, so their
//                rounding is relative to the complement itself;
//   direct:      M, z_M summed over the unselected tiles, walked after the
//                kept ones (used when they are no more than the kept ones).
// The subtraction form still divides the rounding of the whole-head sums by
// the unselected share f = phi(q)z_U / phi(q)z of a row's weight; a query
// block with a valid row below kMinUnselectedShare falls back to the direct
// walk, which is exact in form (a complement whose weights are all zero gives
// a zero denominator and a zero output, as for the oracle).
// The complement's sums are the query block's, shared by its four waves: at
// the end they are stored once in LDS (fp16, power-of-two scaled) and
// multiplied by each wave's phi(Q).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "sla_internal.h"

namespace sla {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const u32x2 lds_u32x2;
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
// The FP8 phi(K) tile has 64-byte rows (one channel, 64 permuted keys) and
// keeps 16-byte chunk ch of row r at ch ^ ((r >> 2) & 3); a 16-lane read group
// (16 consecutive rows, same 8 bytes) then spreads over 16 distinct 4-bank
// groups.
struct LaneOffsets {
  int rd8;    // read byte offset of (row l16, chunk g) in a staged tile; chunk g+4: ^64
  int rdK;    // rd8 in rows 32w.. of the stage's phi(K) tile (w = this wave)
  int rdF;    // FP8 phi(K): bytes 8g.. of row 32w + l16 (row + 16: +1024; keys + 32: ^32)
  int rdM;    // read byte offset of (row l16, chunk g) in M^T; chunk g+4cc: ^(64cc)
  int ld8;    // global byte offset (within the tile) this lane fetches
  int ldF;    // the same for the FP8 phi(K) tile (64-byte rows)
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
  const int frow = 32 * wave + l16;
  o.rdF = kFOff + frow * 64 + (((g >> 1) ^ ((frow >> 2) & 3)) << 4) + 8 * (g & 1);
  const int lrow = 16 * wave + (lane >> 2);           // + 64m
  o.ldF = lrow * 64 + (((lane & 3) ^ ((lrow >> 2) & 3)) << 4);
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
// per workgroup; each instruction round of the workgroup moves kW KB).  kF8:
// the phi(K) tile is the 8 KB FP8 one.
template <bool kK8, bool kFK, bool kF8 = false, int kW = 4>
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
  if (kFK && kF8) {
#pragma unroll
    for (int m = 0; m < kK8Bytes / kRound; ++m)
      lds_load16(src.fk16, lo.ldF, j * kK8Bytes + kRound * m, st + kFOff + kRound * m + 1024 * wave);
  } else if (kFK) {
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
  const int32_t* sched;
  const uint16_t* fk16;
  const uint16_t* v16;
  const float* zb;
  const float* fkscale;   // FP8 phi(K) decode scale per key block (lower-bit option)
  const float* hf;        // whole-head H in the M^T register layout (forward)
  const double* z64;      // whole-head sum of the block sums zb (forward)
  const uint16_t* h16t;   // (backward)
  const float* hscale;    // (backward)
  const float* z;         // (backward)
  int N, Nb, Np, k;
  int phi;        // feature map for phi(Q)
  void* out;
  int out_f32;
  float* out_linear;
  // what a training forward keeps for the backward (null otherwise)
  float* res_stats;     // [BH, N, 2] per row: log2-domain maximum, 1/l
  float* res_os;        // [BH, N, 128] softmax branch's normalised output
  uint16_t* res_m;      // [BH, Nb, 128, 128] bf16 kept share M (staged scale), row = phi channel
  float* res_zm;        // [BH, Nb, 128] kept share of z (staged scale)
};

struct State {
  v4f o[8];       // O^T accumulator (softmax numerator), d = 16dt + 4g + r
  v4f mk[8][2];   // M^T accumulator (linear branch, kept or unselected share):
                  // row d = 16dt + 4g + r, phi channel 32w + 16x + l16
  float m_run;    // running log2-domain maximum (this lane's query)
  float l_part;   // this lane's share of the softmax normaliser
  double zk;      // z_M, phi channel 32w + (lane & 31), summed in fp64
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
template <bool kSoft, bool kLin, bool kMask, bool kF8 = false>
__device__ __forceinline__ void compute_tile(State& S, const lds_byte* st, const v4i qf[2],
                                             const LaneOffsets& lo, float cs, float zj,
                                             int kvalid, int g, float fs = 0.0f) {
  half8 pf[2], fk[2][2];
  const half2v ones = {(_Float16)1.0f, (_Float16)1.0f};
  if (kSoft) {
    v4i s[4];
    // The score products gate everything else in the tile: the wave running
    // them gets issue priority over the other workgroup's wave on this SIMD,
    // whose P.V and M products then fill the slots between them.
    __builtin_amdgcn_s_setprio(1);
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
    __builtin_amdgcn_s_setprio(0);
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
      for (int c = 0; c < 2; ++c) {
        if constexpr (kF8) {
          // 8 e4m3 codes, decoded to fp16 with the block's scale fs
          const u32x2 u = *(lds_u32x2*)(st + ((lo.rdF + 1024 * x) ^ (32 * c)));
          const half2v h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(u.x, fs, false);
          const half2v h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(u.x, fs, true);
          const half2v h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(u.y, fs, false);
          const half2v h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(u.y, fs, true);
          fk[x][c] = half8{h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
        } else {
          fk[x][c] = *(lds_half8*)(st + 2048 * x + (lo.rdK ^ (64 * c)));
        }
      }
    S.zk += (double)zj;
  }
  __builtin_amdgcn_s_setprio(0);  // the products below run at normal priority
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
}

// Key blocks of an ascending list, one per call (wave-uniform, in scalar
// registers), clamped so a malformed list cannot address outside the staging
// buffers.
struct ListWalk {
  const int32_t* list;
  int Nb, p;
  __device__ __forceinline__ int operator()() {
    return min(max(ld_uniform(list, (size_t)p++), 0), Nb - 1);
  }
};

// The key blocks an ascending list of k leaves out, ascending, one per call:
// a merge of 0..Nb-1 against the list.  Every call advances, so a malformed
// list still ends the walk (clamped to the last block).
struct ComplementWalk {
  const int32_t* sel;
  int k, Nb, p, kv, j;
  __device__ __forceinline__ ComplementWalk(const int32_t* s, int k_, int nb)
      : sel(s), k(k_), Nb(nb), p(0), j(-1) {
    kv = k > 0 ? ld_uniform(sel, 0) : Nb;
  }
  __device__ __forceinline__ int operator()() {
    ++j;
    while (j == kv) {
      ++j;
      ++p;
      kv = p < k ? ld_uniform(sel, (size_t)p) : Nb;
    }
    return min(j, Nb - 1);
  }
};

// Walks `n` tiles, the key block of each from `next` (called once per tile,
// in order), through the two LDS stages.
template <bool kSoft, bool kLin, bool kF8, typename Next>
__device__ __forceinline__ void run_tiles(State& S, lds_byte* smem, int stage_bytes, Next next,
                                          int n, const SparseArgs& a,
                                          const TileSrc& src, size_t bh, const v4i qf[2],
                                          const LaneOffsets& lo, float qscale, int wave, int g) {
  if (n <= 0) return;
  auto fscale_of = [&](int j) { return kF8 ? ld_uniform(a.fkscale, bh * a.Nb + j) : 0.0f; };
  int j = next();
  issue_tile<kSoft, kLin, kF8>(smem, src, j, wave, lo);
  float zc = kLin ? load_zb(src, j, lo) : 0.0f;
  float fc = kLin ? fscale_of(j) : 0.0f;
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
        const int jn = next();
        wait_loads();
        lds_barrier();  // tile pp is in LDS; every wave is done with tile pp-1
        issue_tile<kSoft, kLin, kF8>(nxt, src, jn, wave, lo);
        const float zn = kLin ? load_zb(src, jn, lo) : 0.0f;
        const float fn = kLin ? fscale_of(jn) : 0.0f;
        const float cs = kSoft ? qscale * ld_uniform(a.sk, bh * a.Nb + j) : 0.0f;
        compute_tile<kSoft, kLin, false, kF8>(S, cur, qf, lo, cs, zc, kBlk, g, fc);
        j = jn;
        zc = zn;
        fc = fn;
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
      compute_tile<kSoft, kLin, true, kF8>(S, cur, qf, lo, cs, zc, kvalid, g, fc);
    else
      compute_tile<kSoft, kLin, false, kF8>(S, cur, qf, lo, cs, zc, kvalid, g, fc);
  }
  lds_barrier();  // the stages may be refilled by a following walk
}

// Walks this block's column of its group schedule (key block of step s at
// col[s * kGroup]) through the two LDS stages.  A step's entry, and then the
// INT8 scale of its key block, are read with scalar loads when its tile is
// issued, a tile ahead of their use; reading entries earlier (a step further
// ahead, or 64-step chunks in registers) measured slower.
template <bool kLin, bool kF8 = false>
__device__ __forceinline__ void run_sched(State& S, lds_byte* smem, int stage_bytes,
                                          const int32_t* col, int n, const SparseArgs& a,
                                          const TileSrc& src, size_t bh, const v4i qf[2],
                                          const LaneOffsets& lo, float qscale, int wave, int g) {
  if (n <= 0) return;
  auto block_of = [&](int p) { return min(max(ld_uniform(col, (size_t)p * kGroup), 0), a.Nb - 1); };
  auto scale_of = [&](int j) { return ld_uniform(a.sk, bh * a.Nb + j); };
  auto fscale_of = [&](int j) { return kF8 ? ld_uniform(a.fkscale, bh * a.Nb + j) : 0.0f; };
  int j = block_of(0);
  issue_tile<true, kLin, kF8>(smem, src, j, wave, lo);
  float zc = kLin ? load_zb(src, j, lo) : 0.0f;
  float sc = scale_of(j);
  float fc = fscale_of(j);
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
        issue_tile<true, kLin, kF8>(nxt, src, jn, wave, lo);
        const float zn = kLin ? load_zb(src, jn, lo) : 0.0f;
        const float sn = scale_of(jn);
        const float fn = fscale_of(jn);
        compute_tile<true, kLin, false, kF8>(S, cur, qf, lo, qscale * sc, zc, kBlk, g, fc);
        j = jn;
        zc = zn;
        sc = sn;
        fc = fn;
      }
    }
  }
  const float c = qscale * sc;
  const int kvalid = a.N - j * kBlk;
  const lds_byte* cur = smem + (nm & 1) * stage_bytes;
  wait_loads();
  lds_barrier();
  if (kvalid < kBlk)
    compute_tile<true, kLin, true, kF8>(S, cur, qf, lo, c, zc, kvalid, g, fc);
  else
    compute_tile<true, kLin, false, kF8>(S, cur, qf, lo, c, zc, kvalid, g, fc);
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
  S.zk = 0.0;
}

// fp16 phi(Q) of this lane's query for the forward's linear branch, channels
// 32cc + 8g + e (B operand of the products with the complement's sums), scaled
// per row so that the row's largest feature lies in [1, 2).  The branch is a
// ratio of two sums that are both linear in phi(q), so the factor cancels; it
// keeps every row's features in fp16 range.  An elu+1 row whose entries are
// all <= 0 takes exp(q - max q) (its largest feature exp(max q) scaled to 1),
// so a row far below zero keeps its features.
__device__ __forceinline__ void load_phi_q_row(const SparseArgs& a, size_t bh, int qrow,
                                               bool qvalid, int g, half8 fq[4]) {
  const uint16_t* qp = a.q + ((size_t)bh * a.N + (qvalid ? qrow : 0)) * kD + 8 * g;
  float x[4][8];
  float xm = -INFINITY;
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    const uint4 u = *reinterpret_cast<const uint4*>(qp + 32 * cc);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[cc][e] = __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
      xm = fmaxf(xm, x[cc][e]);
    }
  }
  xm = fmaxf(xm, __shfl_xor(xm, 16));  // the row's 128 channels sit in lanes l16 + 16g
  xm = fmaxf(xm, __shfl_xor(xm, 32));
  const bool shifted = a.phi == kPhiElu1 && xm <= 0.0f;
  const float fm = phi_apply(xm, a.phi);
  const float sc = fm > 0.0f ? ldexpf(1.0f, -ilogbf(fm)) : 0.0f;
#pragma unroll
  for (int cc = 0; cc < 4; ++cc)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = shifted ? __expf(x[cc][e] - xm) : phi_apply(x[cc][e], a.phi) * sc;
      fq[cc][e] = qvalid ? (_Float16)f : (_Float16)0.0f;
    }
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

typedef __attribute__((address_space(3))) float lds_float;
typedef __attribute__((address_space(3))) uint32_t lds_u32;

// Largest |x| of this lane's share of a matrix held in the M^T register layout.
__device__ __forceinline__ float lane_absmax(const v4f x[8][2]) {
  float mx = 0.0f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(x[dt][c][r]));
  return mx;
}

// Power-of-two shift s that puts max * 2^-s in [2^14, 2^15) (0 for max = 0).
__device__ __forceinline__ int stage_shift(float mx) { return mx > 0.0f ? ilogbf(mx) - 14 : 0; }

// Stores the workgroup's 128x128 X^T, which the four waves hold in the M^T
// register layout (row d = 16dt + 4g + r, column 32w + 16x + l16), in LDS at
// [0, 32 KB) as fp16 times `down` (256-byte rows, chunk c of row r at
// c ^ (r & 15)).
__device__ __forceinline__ void store_xt(const v4f x[8][2], lds_byte* smem, float down, int wave,
                                         int lane) {
  typedef __attribute__((address_space(3))) _Float16 lds_h;
  const int g = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * dt + 4 * g + r;
        const int ch = (4 * wave + 2 * c + (l16 >> 3)) ^ (row & 15);
        *(lds_h*)(smem + row * 256 + ch * 16 + 2 * (l16 & 7)) = (_Float16)(x[dt][c][r] * down);
      }
}

// phi(Q) X for this lane's query (O^T layout, d = 16dt + 4g + r) from the
// staged X^T, times `up`.
__device__ __forceinline__ void apply_xt(const lds_byte* smem, const LaneOffsets& lo,
                                         const half8 fq[4], float up, v4f num[8]) {
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
}

// phi(Q) M and phi(Q) z_M for this lane's query (O^T layout) from the
// accumulated M^T and z_M: M^T goes through LDS once as fp16 (power-of-two
// scaled) and comes back as A operands; z_M is left in LDS at kZOff as fp32.
constexpr int kZOff = kD * kD * 2;             // z_M, fp32 [128]
constexpr int kRedOff = kZOff + kD * 4;        // per-wave maxima
__device__ __forceinline__ void linear_share(const State& S, lds_byte* smem, const half8 fq[4],
                                             const LaneOffsets& lo, int wave, int lane,
                                             v4f num[8], float& den) {
  const int g = lane >> 4;
  const uint32_t wm = wave_max_u32(__float_as_uint(lane_absmax(S.mk)));  // non-negative floats order as integers
  lds_barrier();  // every wave is done with the tile stages
  if (lane == 0) *(lds_u32*)(smem + kRedOff + 4 * wave) = wm;
  if (lane < 32) *(lds_float*)(smem + kZOff + 4 * (32 * wave + lane)) = (float)S.zk;
  lds_barrier();
  uint32_t m4 = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) m4 = max(m4, *(const lds_u32*)(smem + kRedOff + 4 * w));
  const int sh = stage_shift(__uint_as_float(m4));
  store_xt(S.mk, smem, ldexpf(1.0f, -sh), wave, lane);
  lds_barrier();
  apply_xt(smem, lo, fq, ldexpf(1.0f, sh), num);
  float d = 0.0f;
#pragma unroll
  for (int cc = 0; cc < 4; ++cc)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      d += (float)fq[cc][e] * *(const lds_float*)(smem + kZOff + 4 * (32 * cc + 8 * g + e));
  d += __shfl_xor(d, 16);
  den = d + __shfl_xor(d, 32);
}

// Linear output of the backward's query side in the subtraction form, from
// the kept share (nm, dm) that linear_share returns: (phi(Q)H - phi(Q)M) /
// (phi(Q)z - phi(Q)z_M), with H^T fp16-scaled and z from the backward's
// linear state.  Returns 1/den, 0 when the denominator is lost in rounding;
// den is in the staged scale (phi/16 on both sides: 1/256 of the true one).
__device__ __forceinline__ float linear_subtract_out(const SparseArgs& a, size_t bh, int g,
                                                     const LaneOffsets& lo, const half8 fq[4],
                                                     const v4f nm[8], float dm, v4f ol[8]) {
  const float hs = a.hscale[bh];
  const float* zz = a.z + bh * kD;
  float dz = 0.0f;
#pragma unroll
  for (int cc = 0; cc < 4; ++cc)
#pragma unroll
    for (int e = 0; e < 8; ++e) dz += (float)fq[cc][e] * zz[32 * cc + 8 * g + e];
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
    for (int cc = 0; cc < 4; ++cc) ah[cc] = *reinterpret_cast<const half8*>(hrow + 32 * cc);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) num = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[cc], fq[cc], num, 0, 0, 0);
    ol[dt] = (num * hs - nm[dt]) * inv_den;
  }
  return inv_den;
}

// Smallest unselected share f = phi(q)z_U / phi(q)z of a valid row that the
// subtraction form serves; a query block with a row below it takes the
// direct walk.  With f >= 1/16 the whole-head and kept sums' fp32 rounding
// (a relative 2^-24 per term, over a few hundred sequential sums) stays
// below about 4e-4 of the branch's value scale.
constexpr float kMinUnselectedShare = 1.0f / 16.0f;

// Epilogue LDS of the subtraction form (the tile stages are free by then):
// [0, 32 KB) the complement's H_U^T, then z_U and z (fp32 [128] each), then
// per-wave words (maxima, fallback flags).
constexpr int kEpZU = kD * kD * 2;
constexpr int kEpZ = kEpZU + kD * 4;
constexpr int kEpRed = kEpZ + kD * 4;

// The kept tiles' share of the linear state of query block i, as a training
// forward keeps it for the backward: M = sum phi(K_j)^T V_j over the kept
// tiles, row-major bf16 (row = phi channel 32w + 16x + l16, this lane's four
// entries 16dt + 4g + r of each row), and z_M per channel (fp32).
__device__ __forceinline__ void save_kept_share(const State& S, const SparseArgs& a, size_t bh, int i,
                                                int wave, int lane) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const int g = lane >> 4, l16 = lane & 15;
  uint16_t* mb = a.res_m + (bh * a.Nb + i) * (size_t)(kD * kD);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int c = 32 * wave + 16 * x + l16;
      const bf16x4 h4 = {(__bf16)S.mk[dt][x][0], (__bf16)S.mk[dt][x][1], (__bf16)S.mk[dt][x][2],
                         (__bf16)S.mk[dt][x][3]};
      *reinterpret_cast<bf16x4*>(mb + (size_t)c * kD + 16 * dt + 4 * g) = h4;
    }
  if (lane < 32) a.res_zm[(bh * a.Nb + i) * kD + 32 * wave + lane] = (float)S.zk;
}

// A training forward's per-row residuals: the softmax statistics (log2-domain
// maximum, +inf for a row without weights, and 1/l) and the normalised
// softmax output.
__device__ __forceinline__ void save_row(const State& S, const SparseArgs& a, size_t bh, int qrow,
                                         bool qvalid, float inv_l, int g) {
  if (!qvalid) return;
  const size_t row = bh * a.N + qrow;
  if (g == 0) {
    a.res_stats[2 * row] = inv_l > 0.0f ? S.m_run : INFINITY;
    a.res_stats[2 * row + 1] = inv_l;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    *reinterpret_cast<v4f*>(a.res_os + row * kD + 16 * dt + 4 * g) = S.o[dt] * inv_l;
}

// Normalise, add the linear branch, store this lane's query row.
template <int kMode, bool kF8>
__device__ __forceinline__ void finish_query(State& S, const SparseArgs& a, size_t bh, int i,
                                             int qrow, bool qvalid, lds_byte* smem, int stage_bytes,
                                             const TileSrc& src, const v4i qf[2],
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
    load_phi_q_row(a, bh, qrow, qvalid, g, fq);
    bool direct = kMode == kDirect;
    if (kMode == kSubtract) {
      if (!kF8 && a.res_m) save_kept_share(S, a, bh, i, wave, lane);
      // whole-head sums: z (fp64, this lane's channel 32w + (lane & 31)) and
      // H in this lane's M^T fragments, loaded together
      const double zh = a.z64[bh * kD + 32 * wave + (lane & 31)];
      const v4f* hp = reinterpret_cast<const v4f*>(a.hf) + (bh * 4 + wave) * (16 * 64) + lane;
      v4f hr[8][2];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int c = 0; c < 2; ++c) hr[dt][c] = hp[(2 * dt + c) * 64];
      const float zu = (float)fmax(zh - S.zk, 0.0);  // z_U, one rounding of the fp64 difference
      lds_barrier();  // every wave is done with the tile stages
      if (lane < 32) {
        *(lds_float*)(smem + kEpZU + 4 * (32 * wave + lane)) = zu;
        *(lds_float*)(smem + kEpZ + 4 * (32 * wave + lane)) = (float)zh;
      }
      lds_barrier();
      float du = 0.0f, dz = 0.0f;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = 32 * cc + 8 * g + e;
          const float f = (float)fq[cc][e];
          du += f * *(const lds_float*)(smem + kEpZU + 4 * c);
          dz += f * *(const lds_float*)(smem + kEpZ + 4 * c);
        }
      du += __shfl_xor(du, 16);
      du += __shfl_xor(du, 32);
      dz += __shfl_xor(dz, 16);
      dz += __shfl_xor(dz, 32);
      const bool need = qvalid && dz > 0.0f && du < kMinUnselectedShare * dz;
      // H_U = H - M, taken in fp32 before anything is rounded to fp16
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int c = 0; c < 2; ++c) S.mk[dt][c] = hr[dt][c] - S.mk[dt][c];
      const uint32_t wm = wave_max_u32(__float_as_uint(lane_absmax(S.mk)));
      const uint32_t wneed = __builtin_amdgcn_ballot_w64(need) != 0 ? 1u : 0u;
      if (lane == 0) {
        *(lds_u32*)(smem + kEpRed + 4 * wave) = wm;
        *(lds_u32*)(smem + kEpRed + 16 + 4 * wave) = wneed;
      }
      lds_barrier();
      uint32_t m4 = 0, any = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        m4 = max(m4, *(const lds_u32*)(smem + kEpRed + 4 * w));
        any |= *(const lds_u32*)(smem + kEpRed + 16 + 4 * w);
      }
      if (!any) {
        const int sh = stage_shift(__uint_as_float(m4));
        store_xt(S.mk, smem, ldexpf(1.0f, -sh), wave, lane);
        lds_barrier();
        v4f num[8];
        apply_xt(smem, lo, fq, ldexpf(1.0f, sh), num);
        const float inv_den = du > 0.0f ? 1.0f / du : 0.0f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) ol[dt] = num[dt] * inv_den;
      } else {
        // a row's unselected share is too small for the subtraction: sum the
        // complement directly
        direct = true;
        lds_barrier();  // every wave has read the words above; the stages are refilled next
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) S.mk[dt][0] = S.mk[dt][1] = v4f{0.f, 0.f, 0.f, 0.f};
        S.zk = 0.0;
        const int32_t* sel = a.idx + (bh * a.Nb + i) * (size_t)a.k;
        run_tiles<false, true, kF8>(S, smem, stage_bytes, ComplementWalk(sel, a.k, a.Nb),
                                    a.Nb - a.k, a, src, bh, qf, lo, 0.0f, wave, g);
      }
    }
    if (direct) {
      // numerator and denominator summed over the unselected blocks
      v4f nm[8];
      float dm;
      linear_share(S, smem, fq, lo, wave, lane, nm, dm);
      const float inv_den = dm > 0.0f ? 1.0f / dm : 0.0f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) ol[dt] = nm[dt] * inv_den;
    }
  }

  if (!kF8 && a.res_stats) save_row(S, a, bh, qrow, qvalid, inv_l, g);  // training: exact mode only
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
template <int kMode, bool kF8>
__global__ __launch_bounds__(256, 2) void sparse_fwd_kernel(SparseArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  lds_byte* smem = (lds_byte*)smem_raw;
  constexpr bool kLinAny = kMode != kSoftOnly;
  constexpr int stage_bytes =
      kK8Bytes + kF16TileBytes + (kLinAny ? (kF8 ? kK8Bytes : kF16TileBytes) : 0);
  const int t = threadIdx.x;
  const int lane = t & 63;
  // wave-uniform in a scalar register: the LDS destinations of the tile loads
  // (M0) are then computed with scalar arithmetic
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
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
    run_sched<kLinAny, kF8>(S, smem, stage_bytes, col, a.k, a, src, bh, qf, lo, qscale, wave, g);
  } else {
    const int32_t* sel = a.idx + (bh * a.Nb + i) * (size_t)a.k;
    run_tiles<true, false, false>(S, smem, stage_bytes, ListWalk{sel, a.Nb, 0}, a.k, a, src, bh,
                                  qf, lo, qscale, wave, g);
    run_tiles<false, true, kF8>(S, smem, stage_bytes, ComplementWalk(sel, a.k, a.Nb), a.Nb - a.k,
                                a, src, bh, qf, lo, qscale, wave, g);
  }
  finish_query<kMode, kF8>(S, a, bh, i, qrow, qvalid, smem, stage_bytes, src, qf, lo, wave, lane);
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
// sorted (stably, so by block within a set) into 15 queues, one per owner set
// (queue t holds the set kSets[t]); the lane holding queue t's head finds a
// pick as one maximum over the heads whose set is free.
constexpr uint32_t kSets[16] = {15, 7, 11, 13, 14, 3, 5, 6, 9, 10, 12, 1, 2, 4, 8, 0};
constexpr uint64_t kSetsPacked = 0x08421ca9653edb7full;  // kSets[t] in bits 4t..4t+3

// The queues of a union uni[0, n) at q (by the whole wave); returns queue
// t_of's range [head, end) of q.
__device__ __forceinline__ void queue_layout(const uint32_t* uni, int n, uint32_t* q, int lane, int t_of,
                                             int& mine_head, int& mine_end) {
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
  int off[16];
  int run = 0;
  mine_head = mine_end = 0;
#pragma unroll
  for (int t = 0; t < 15; ++t) {
    off[t] = run;
    if (t_of == t) mine_head = run, mine_end = run + cnt[t];
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
}

// One group per wave: lane L < 15 holds the head of queue L, so a pick is one
// wave-wide maximum.  Returns false, leaving the schedule to the general
// greedy, when a step would need a block split between steps.
__device__ __forceinline__ bool greedy_queues4(const uint32_t* uni, int n, uint32_t* q, int k,
                                               uint32_t full, uint32_t last_busy, int lane,
                                               const SchedOut& out) {
  int mine_head, mine_end;
  queue_layout(uni, n, q, lane, lane, mine_head, mine_end);
  __syncthreads();
  const uint32_t set = lane < 15 ? (uint32_t)(kSetsPacked >> (4 * lane)) & 15u : 0u;
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
// The union of group grp's kept blocks (one wave; the workgroup is that
// wave): own = owner byte of key block j in byte j&3 of word j>>2, then uni =
// the union, ascending key block, entry = block << 8 | owners.  Writes -1 for
// members past the last query block and the ragged last key block's last
// step; returns the union's size, the members and the members busy with the
// ragged block in the last step.
template <int kG>
__device__ __forceinline__ int group_union(const int32_t* __restrict__ idx, size_t bh, int Nb, int k,
                                           int grp, int ragged, uint32_t* own, uint32_t* uni, int lane,
                                           const SchedOut& out, uint32_t& full, uint32_t& last_busy) {
  const int first = grp * kG;
  const int members = min(kG, Nb - first);
  full = (1u << members) - 1u;
  const int words = (Nb + 3) / 4;
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
  last_busy = 0u;
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
  return n;
}

// The general greedy over a group's union (registers when it fits, else LDS).
template <int kG>
__device__ __forceinline__ void greedy_general(uint32_t* uni, int n, int k, uint32_t full, uint32_t last_busy,
                                               int lane, const SchedOut& out) {
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

// One wave per group: sched[((bh, grp, s) * kG) + u] = key block of member u
// (query block kG*grp + u) in step s.  Members past the last block get -1.
template <int kG>
__global__ __launch_bounds__(64) void group_schedule_kernel(const int32_t* __restrict__ idx,
                                                            int Nb, int k, int ragged,
                                                            int32_t* __restrict__ sched,
                                                            const uint32_t* __restrict__ only_if) {
  if (only_if && only_if[0] == 0u) return;  // a rebuild with nothing to rebuild
  extern __shared__ uint32_t gsm[];
  const int lane = threadIdx.x;
  const int grp = blockIdx.x;
  const size_t bh = blockIdx.y;
  const int ngroups = (Nb + kG - 1) / kG;
  const int words = (Nb + 3) / 4;
  uint32_t* own = gsm;
  uint32_t* uni = gsm + words;
  const SchedOut out{sched + (bh * ngroups + grp) * (size_t)k * kG};
  uint32_t full, last_busy;
  const int n = group_union<kG>(idx, bh, Nb, k, grp, ragged, own, uni, lane, out, full, last_busy);
  if (kG == 4 && greedy_queues4(uni, n, uni + n, k, full, last_busy, lane, out)) return;
  greedy_general<kG>(uni, n, k, full, last_busy, lane, out);
}

// Maximum over the 16 lanes of each row of the wave (DPP only).
__device__ __forceinline__ uint32_t row_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0xB1, 0xF, 0xF, true));   // lane ^ 1
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x4E, 0xF, 0xF, true));   // lane ^ 2
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x141, 0xF, 0xF, true));  // 8-lane mirror
  return max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x140, 0xF, 0xF, true));  // 16-lane mirror
}

// LDS words of the four-group kernel: owner bytes and a union (rebuilt for
// each group in turn), and the four groups' queues.
inline size_t group_schedule_x4_lds(int Nb, int k) {
  const size_t cap = std::min<size_t>((size_t)Nb, (size_t)kGroup * k);
  return 4 * (((size_t)Nb + 3) / 4 + 5 * cap);
}

// Four groups of four per wave: the union and queues of each are built by the
// whole wave in turn, then row r (lanes 16r..16r+15) runs the queue greedy of
// group 4 * blockIdx.x + r, lane 16r + t holding the head of queue t, so one
// pick is a 16-lane maximum and serves the four groups at once.  A group whose
// walk would need a block split between steps is then redone by the general
// greedy (the same schedule as the one-group kernel gives).
__global__ __launch_bounds__(64) void group_schedule_x4_kernel(const int32_t* __restrict__ idx, int Nb,
                                                               int k, int ragged,
                                                               int32_t* __restrict__ sched,
                                                               const uint32_t* __restrict__ only_if) {
  if (only_if && only_if[0] == 0u) return;  // a rebuild with nothing to rebuild
  extern __shared__ uint32_t gsm[];
  const int lane = threadIdx.x, row = lane >> 4, l16 = lane & 15;
  const size_t bh = blockIdx.y;
  const int ngroups = (Nb + kGroup - 1) / kGroup;
  const int words = (Nb + 3) / 4;
  const int cap = min(Nb, kGroup * k);
  uint32_t* own = gsm;
  uint32_t* uni = gsm + words;
  uint32_t* queues = uni + cap;
  auto out_of = [&](int grp) { return SchedOut{sched + (bh * ngroups + grp) * (size_t)k * kGroup}; };
  int head = 0, end = 0;
  uint32_t full = 0u, last_busy = 0u;  // this row's group (none: full = 0)
  for (int q = 0; q < 4; ++q) {
    const int grp = 4 * blockIdx.x + q;
    if (grp >= ngroups) break;
    uint32_t f, lb;
    const int n = group_union<kGroup>(idx, bh, Nb, k, grp, ragged, own, uni, lane, out_of(grp), f, lb);
    int h, e;
    queue_layout(uni, n, queues + q * cap, lane, l16, h, e);
    if (row == q) head = h, end = e, full = f, last_busy = lb;
    __syncthreads();  // own and uni are rebuilt for the next group
  }
  const uint32_t* myq = queues + row * cap;
  const uint32_t set = l16 < 15 ? (uint32_t)(kSetsPacked >> (4 * l16)) & 15u : 0u;
  const uint32_t size = (uint32_t)__popc(set);
  uint32_t hj = head < end ? myq[head] : 0xffffffu;
  const SchedOut out = out_of(min(4 * (int)blockIdx.x + row, ngroups - 1));  // written only with a group
  bool failed = false;  // row-uniform
  for (int s = 0; s < k; ++s) {
    uint32_t freem = failed ? 0u : s == k - 1 ? full & ~last_busy : full;
    while (__ballot(freem != 0u)) {
      // most owners among the free members, then lowest block
      const bool ok = set && !(set & ~freem) && head < end;
      const uint32_t key = ok ? (size << 24) | (0xffffffu - hj) : 0u;
      const uint32_t top = row_max_u32(key);
      const bool pick = top != 0u;
      if (!pick && freem) failed = true;
      const uint32_t rowbits = (uint32_t)(__ballot(pick && key == top) >> (16 * row)) & 0xffffu;
      const int h = pick ? __builtin_ctz(rowbits) : 0;
      const uint32_t bm = pick ? (uint32_t)(kSetsPacked >> (4 * h)) & 15u : 0u;
      if (pick && l16 == h) {
        ++head;
        hj = head < end ? myq[head] : 0xffffffu;
      }
      if (l16 < 4 && ((bm >> l16) & 1u)) out.put((size_t)s * 4 + l16, (int32_t)(0xffffffu - (top & 0xffffffu)));
      freem = pick ? freem & ~bm : 0u;
    }
  }
  const uint64_t redo = __ballot(failed && l16 == 0);
  for (int q = 0; q < 4; ++q) {
    if (!((redo >> (16 * q)) & 1ull)) continue;
    const int grp = 4 * blockIdx.x + q;
    __syncthreads();
    uint32_t f, lb;
    const int n = group_union<kGroup>(idx, bh, Nb, k, grp, ragged, own, uni, lane, out_of(grp), f, lb);
    greedy_general<kGroup>(uni, n, k, f, lb, lane, out_of(grp));
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
static_assert(kRedOff + 16 <= kMRowOff, "linear_share's LDS area overlaps the row-major M");
constexpr int kZOffShared = kZOff;                        // z_M as linear_share leaves it (fp32 [128])

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
  // a training forward's residuals (the saved form; null otherwise)
  const float* res_stats;   // [BH, N, 2] log2-domain row maximum, 1/l
  const float* res_os;      // [BH, N, D] normalised softmax-branch output
  const float* res_ol;      // [BH, N, D] linear-branch output
  const uint16_t* res_m;    // [BH, Nb, D, D] bf16 kept share M (staged scale)
  const float* res_zm;      // [BH, Nb, D] kept share of z (staged scale)
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

// kSaved: the forward's statistics, outputs and kept share come from a
// training forward's residuals instead of a first sweep over the kept tiles.
template <bool kLin, bool kSaved>
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
  if (!kSaved)
    run_sched<kLin>(S, smem, kBwdStage, col, a.k, a, head_sources(a, bh, kLin), bh, qf, lo, qscale,
                    wave, g);

  // softmax statistics of this lane's query and D = dO . O_s
  const size_t rrow = (size_t)bh * a.N + (qvalid ? qrow : 0);
  float inv_l, m_fin;
  if (kSaved) {
    inv_l = (a.k > 0 && qvalid) ? b.res_stats[2 * rrow + 1] : 0.0f;
    m_fin = inv_l > 0.0f ? b.res_stats[2 * rrow] : INFINITY;
  } else {
    float l = S.l_part + __shfl_xor(S.l_part, 16);
    l += __shfl_xor(l, 32);
    inv_l = (a.k > 0 && l > 0.0f && qvalid) ? 1.0f / l : 0.0f;
    m_fin = inv_l > 0.0f ? S.m_run : INFINITY;  // rows without weights get P = 0
  }
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
  for (int dt = 0; dt < 8; ++dt) {
    const v4f os = !kSaved ? S.o[dt]
                   : qvalid ? *reinterpret_cast<const v4f*>(b.res_os + rrow * kD + 16 * dt + 4 * g)
                            : v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r) dpart += go[dt][r] * os[r];
  }
  dpart += __shfl_xor(dpart, 16);
  dpart += __shfl_xor(dpart, 32);
  const float Dt = kSaved ? (inv_l > 0.0f ? dpart : 0.0f) : dpart * inv_l;

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
    const float* zmb = kSaved ? b.res_zm + ((size_t)bh * a.Nb + i) * kD : nullptr;
    v4f ol[8];
    float inv_den;
    if (kSaved) {
      // (phi(Q)z - phi(Q)z_M) in the staged scale, as linear_subtract_out
      // forms it, and the forward's linear output
      const float* zz0 = a.z + bh * kD;
      float dz = 0.0f, dm = 0.0f;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = 32 * cc + 8 * g + e;
          dz += (float)fq[cc][e] * zz0[c];
          dm += (float)fq[cc][e] * zmb[c];
        }
      dz += __shfl_xor(dz, 16);
      dz += __shfl_xor(dz, 32);
      dm += __shfl_xor(dm, 16);
      dm += __shfl_xor(dm, 32);
      const float den = dz - dm;
      inv_den = den > 1e-6f * dz ? 1.0f / den : 0.0f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        ol[dt] = qvalid ? *reinterpret_cast<const v4f*>(b.res_ol + rrow * kD + 16 * dt + 4 * g)
                        : v4f{0.f, 0.f, 0.f, 0.f};
    } else {
      v4f nm[8];
      float dm;
      linear_share(S, smem, fq, lo, wave, lane, nm, dm);
      inv_den = linear_subtract_out(a, bh, g, lo, fq, nm, dm, ol);
    }
    float up = 0.0f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) up += go[dt][r] * ol[dt][r];
    up += __shfl_xor(up, 16);
    up += __shfl_xor(up, 32);
    u = qvalid ? -up : 0.0f;
    // M (kept share, staged scale) row-major as bf16: row c = 32w + 16x + l16
    // holds M[c][16dt + 4g + r] (the saved form reads it from the residuals)
#pragma unroll
    for (int dt = 0; dt < 8 && !kSaved; ++dt)
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
      bf16x8 hv[4], mv[4];  // the row's four fragments of H (and saved M), loaded together
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        hv[ks] = *reinterpret_cast<const bf16x8*>(hrow + (16 * ct + l16) * kD + 32 * ks + 8 * g);
        if (kSaved)
          mv[ks] = *reinterpret_cast<const bf16x8*>(b.res_m + ((size_t)bh * a.Nb + i) * (kD * kD) +
                                                    (16 * ct + l16) * kD + 32 * ks + 8 * g);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        ah = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hv[ks], gf[ks], ah, 0, 0, 0);
        am = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            kSaved ? mv[ks] : lds_row_frag(smem + kMRowOff, 16 * ct + l16, 4 * ks + g), gf[ks], am, 0, 0, 0);
      }
      const uint2 qw = *reinterpret_cast<const uint2*>(qrowp + 16 * ct + 4 * g);
      const float qv[4] = {bf16_lo(qw.x), bf16_hi(qw.x), bf16_lo(qw.y), bf16_hi(qw.y)};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = 16 * ct + 4 * g + r;
        const float zi =
            zz[c] - (kSaved ? zmb[c] : *(__attribute__((address_space(3))) const float*)(smem + kZOffShared + 4 * c));
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
    float* st4 = b.stats + ((size_t)bh * a.Nb + i) * kBwdStatFloats;
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
// Key side: one workgroup per key block j, walking the query blocks that keep
// j (shared with the group's other key blocks first); the waves and their
// roles are described at kv_waves.  Per query block i it stages the INT8 Q
// codes, the dO and Q rows, (phi(Q)/den)^T and the row statistics:
//   S, P (the forward's weights), dP = dO V^T, dS
//   dV += P^T dO,  dK += dS^T Q,  W += (phi(Q)/den)^T dO,  w += (phi(Q)/den)^T u
// then the linear gradient through G - W and g_z - w.  dV, W and dK contract
// over the query rows and take dO and Q column-wise: those operands come from
// the row-major tiles through transposing LDS reads.
// ---------------------------------------------------------------------------
constexpr int kKvDoOff = kK8Bytes;                        // dO rows [64][128] bf16
constexpr int kKvQOff = kK8Bytes + kF16TileBytes;         // Q rows [64][128] bf16
constexpr int kKvFqOff = kK8Bytes + 2 * kF16TileBytes;    // (phi(Q)/den)^T [128][64 perm] bf16
constexpr int kKvStOff = kK8Bytes + 3 * kF16TileBytes;    // 4 x 64 fp32 statistics
constexpr int kKvStatBytes = 4 * kBwdStatFloats;
constexpr int kKvStage = kKvStOff + kKvStatBytes;         // 57 KB

// 256-byte-row tiles of the key side keep 16-byte chunk ch of row r at
// ch ^ kv_swz(r), so that neither of the two read shapes meets a bank
// conflict: a transposing read (per half wave: 8 consecutive rows from a
// multiple of 8, one 32-byte segment each) needs the segment index distinct
// over each aligned 8 rows; a 16-byte row fragment read (per half wave: rows
// 16tt..16tt+15, an aligned pair of chunks) spreads over 512 bytes of banks,
// so it needs the segment index distinct over the even and over the odd
// rows of 16.  (r & 7) ^ (r >> 3 & 1) is both.
__device__ __forceinline__ int kv_swz(int r) { return ((r & 7) ^ ((r >> 3) & 1)) << 1; }

// Byte offset a lane fetches when wave w moves its 1 KB (4 rows, 4w..4w+3 of
// the workgroup's round; a round of W waves covers 4W rows) of such a tile
// into LDS.
__device__ __forceinline__ int kv_row_ld(int wave, int lane) {
  const int r = 4 * wave + (lane >> 4);
  return r * 256 + (((lane & 15) ^ kv_swz(r)) << 4);
}

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// Transposing read of 16-bit data: in each 16-lane group, lane i receives
// element i % 4 of the 8-byte pieces addressed by lanes i/4, i/4 + 4, i/4 + 8,
// i/4 + 12 (in that order).
__device__ __forceinline__ v4s tr_read(const lds_byte* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p);
}

// Matrix-core fragment of a row-major tile X [64 rows][128 channels] taken
// column-wise: lane (l16, g) gets X[row][n0 + l16] for the eight rows
// 32c + 4g + e and 32c + 16 + 4g + e (e = 0..3) -- the k slots a score tile's
// rows occupy.  `off` is the lane's offset for channels n0.. (kv_tr_off).
__device__ __forceinline__ bf16x8 tr_frag(const lds_byte* tile, int c, int off) {
  const v4s lo = tr_read(tile + (32 * c) * 256 + off);
  const v4s hi = tr_read(tile + (32 * c + 16) * 256 + off);
  const v4s both[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8, both);
}

// The lane's byte offset for tr_frag over channels 16t..16t+15: it addresses
// row 4g + l16/4 (+ 32c + 16h), channels 16t + 4 (l16 % 4)..
__device__ __forceinline__ int kv_tr_off(int lane, int t) {
  const int l16 = lane & 15, g = lane >> 4;
  const int x = 4 * g + (l16 >> 2);
  const int pos = (2 * t + ((l16 & 3) >> 1)) ^ kv_swz(x);
  return x * 256 + (pos << 4) + 8 * (l16 & 1);
}

struct BwdKvArgs {
  const int8_t* q8;
  const int8_t* k8;
  const float* sq;
  const float* sk;
  const uint16_t* q;      // Q bf16 [BH, N, D]
  const uint16_t* kin;    // K bf16 [BH, N, D]
  const uint16_t* v;      // V bf16 [BH, N, D]
  const uint16_t* dout;   // dO bf16 [BH, N, D]
  const uint16_t* fqs;    // (phi(Q)/den)^T bf16 per block [BH, Nb, D, 64 permuted rows]
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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor over `bytes` bytes at `base` (the layout the buffer
// resource builtin produces: raw, stride 0, 32-bit data format).
__device__ __forceinline__ u32x4 kv_rsrc(const void* base, size_t bytes) {
  const unsigned long long b = (unsigned long long)base;
  return u32x4{(unsigned)b, (unsigned)(b >> 32) & 0xffffu, (unsigned)bytes, 0x00020000u};
}

// 16 bytes per lane from rsrc[voff] into LDS at lds + 16 * lane.  Issued from
// inline assembly because the compiler makes every transposing LDS read wait
// for all outstanding global->LDS loads (it cannot tell that they fill the
// other stage), which would serialise each tile's math behind the next
// tile's loads.  The instruction has no register results; the loads are
// awaited explicitly (wait_loads + lds_barrier) before their stage is read,
// and M0 is restored, so the compiler's view of every register stays valid.
__device__ __forceinline__ void kv_dma16(u32x4 rsrc, int voff, const lds_byte* lds) {
  // the stage address is wave-uniform; say so, also inside lane-masked code
  const unsigned la = __builtin_amdgcn_readfirstlane((unsigned)(size_t)lds);
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(la)
      : "memory");
}

struct BwdKvSrc {
  u32x4 q8, dout, q, fqs, stats;
};

// The key side runs 4 score waves (softmax branch) and, with the linear
// branch, 4 linear waves (W, w) per workgroup: two waves per SIMD, so the
// vector work of one overlaps the matrix-core work of the other.
template <bool kLin>
constexpr int kv_waves() { return kLin ? 8 : 4; }
// global->LDS load instructions per wave per staged block (every wave the same)
template <bool kLin>
constexpr int kv_loads() { return kLin ? 8 : 11; }
constexpr int kKvStages = 2;   // staged query blocks: one in use, one in flight
// dS hand-over slots (with the linear branch), two sets used by alternate
// blocks: for each of the two 16-byte halves, 16 bytes per lane of the 4
// score waves (lane-contiguous, so each access is free of bank conflicts).
// The score waves write block p's dS into set p % 2 during block p; the
// linear waves read it at the start of block p + 1, after the walk's
// barrier, and set p % 2 is written again only after the next barrier, so
// the hand-over needs no barrier of its own.
constexpr int kKvDsOff = kKvStages * kKvStage;
constexpr int kKvDsHalf = 4 * 64 * 16;

// The lane's LDS offsets of a score wave, fixed for the kernel.
struct KvLane {
  int rd8;      // INT8 Q tile (128-byte rows), as LaneOffsets::rd8
  int rf[4];    // dO row fragment: row l16, chunk 4ks + g (+ 4096 tt for rows 16tt..)
  int tr[8];    // tr_frag offsets for channels 16t..
};

__device__ __forceinline__ KvLane kv_lane(int lane) {
  const int l16 = lane & 15, g = lane >> 4;
  KvLane o;
  o.rd8 = l16 * 128 + ((g ^ ((l16 >> 1) & 7)) << 4);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) o.rf[ks] = l16 * 256 + (((4 * ks + g) ^ kv_swz(l16)) << 4);
#pragma unroll
  for (int t = 0; t < 8; ++t) o.tr[t] = kv_tr_off(lane, t);
  return o;
}

// Global fetch offsets of a wave's share of the staging (W waves; a round of
// the workgroup moves W KB): in the 128-byte-row tiles (INT8 codes,
// (phi(Q)/den)^T; row 8w + lane/8 of each round) and in the 256-byte-row tiles
// (dO, Q; row 4w + lane/16 of each round).
struct KvLoad {
  int ld8, rld;
};

__device__ __forceinline__ KvLoad kv_load_offsets(int wave, int lane) {
  const int row = 8 * wave + (lane >> 3);
  return KvLoad{row * 128 + (((lane & 7) ^ ((row >> 1) & 7)) << 4), kv_row_ld(wave, lane)};
}

// Issues this wave's share of query block i's staging into `st`.  The raw
// dO and Q rows are addressed through the lane offset, so the buffer's range
// check covers the rows past N (they read as zero).
template <bool kLin>
__device__ __forceinline__ void issue_kv_tile(lds_byte* st, const BwdKvSrc& src, int i, int wave,
                                              const KvLoad& ko, int lane) {
  constexpr int kW = kv_waves<kLin>();
  constexpr int kRound = 1024 * kW;
  const int rows = i * kF16TileBytes + ko.rld;
#pragma unroll
  for (int m = 0; m < kF16TileBytes / kRound; ++m)
    kv_dma16(src.dout, rows + kRound * m, st + kKvDoOff + kRound * m + 1024 * wave);
#pragma unroll
  for (int m = 0; m < kK8Bytes / kRound; ++m)
    kv_dma16(src.q8, i * kK8Bytes + kRound * m + ko.ld8, st + kRound * m + 1024 * wave);
#pragma unroll
  for (int m = 0; m < kF16TileBytes / kRound; ++m)
    kv_dma16(src.q, rows + kRound * m, st + kKvQOff + kRound * m + 1024 * wave);
  if (kLin) {
#pragma unroll
    for (int m = 0; m < kF16TileBytes / kRound; ++m)
      kv_dma16(src.fqs, i * kF16TileBytes + kRound * m + ko.ld8, st + kKvFqOff + kRound * m + 1024 * wave);
  }
  // the statistics, 1024 / kW bytes per wave
  constexpr int kSt = kKvStatBytes / kW;
  if (lane < kSt / 16) kv_dma16(src.stats, i * kKvStatBytes + kSt * wave + 16 * lane, st + kKvStOff + kSt * wave);
}
static_assert(kF16TileBytes / 8192 * 3 + kK8Bytes / 8192 + 1 == kv_loads<true>(), "load count (8 waves)");
static_assert(kF16TileBytes / 4096 * 2 + kK8Bytes / 4096 + 1 == kv_loads<false>(), "load count (4 waves)");

// Waits until at most n of this wave's global->LDS loads are outstanding.
template <int n>
__device__ __forceinline__ void wait_loads_but() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
}

// The walk over the key block's column (n query blocks from `list`), the same
// loads, waits and barriers in every wave: a ring of kKvStages stages, block
// p in stage p % kKvStages, the next kKvStages - 1 blocks in flight while p is
// computed by tile(stage, scale of block p).
template <bool kLin, typename Tile>
__device__ __forceinline__ void kv_walk(lds_byte* smem, const BwdKvSrc& src, const int32_t* list,
                                        int n, const float* sq_head, int Nb, int wave, int lane,
                                        Tile&& tile) {
  const KvLoad ko = kv_load_offsets(wave, lane);
  auto block_of = [&](int p) { return min(max(ld_uniform(list, (size_t)p), 0), Nb - 1); };
  auto scale_of = [&](int p) { return ld_uniform(sq_head, (size_t)block_of(p)); };
  float sc[kKvStages];
#pragma unroll
  for (int q = 0; q < kKvStages - 1; ++q) {
    if (q < n) issue_kv_tile<kLin>(smem + q * kKvStage, src, block_of(q), wave, ko, lane);
    sc[q] = q < n ? scale_of(q) : 0.0f;
  }
  int stage = 0;
  for (int p = 0; p < n; ++p) {
    if (kKvStages > 2 && p + kKvStages - 2 < n)
      wait_loads_but<(kKvStages - 2) * kv_loads<kLin>()>();  // later blocks stay in flight
    else
      wait_loads();
    lds_barrier();  // block p is in LDS; every wave is done with block p-1
    const int pn = p + kKvStages - 1;
    sc[kKvStages - 1] = 0.0f;
    if (pn < n) {
      const int sn = stage == 0 ? kKvStages - 1 : stage - 1;  // pn's stage: block p-1's
      issue_kv_tile<kLin>(smem + sn * kKvStage, src, block_of(pn), wave, ko, lane);
      sc[kKvStages - 1] = scale_of(pn);
    }
    tile(smem + stage * kKvStage, sc[0], p);
#pragma unroll
    for (int q = 0; q < kKvStages - 1; ++q) sc[q] = sc[q + 1];
    stage = stage == kKvStages - 1 ? 0 : stage + 1;
  }
}

// One staged query block for a score wave (16 keys): S, P, dP, dS, then
// dV += P^T dO and, unless kSplit, dK += dS^T Q.  kSplit: dS goes to this
// lane's slot of `ds` (the block's slot set), and the linear wave on the same
// SIMD takes dK one block later.
template <bool kSplit>
__device__ __forceinline__ void kv_score_tile(const lds_byte* st, const v4i kf[2], const bf16x8 vf[4],
                                              const KvLane& kl, float cs, int g, v4f dv[8],
                                              v4f dk[8], lds_byte* ds) {
  v4i s[4];
  qk_tile(st, kf, kl.rd8, s);  // s[tt][r] = S[row 16tt + 4g + r][key l16]
  v4f dp[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    dp[tt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      dp[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          *(lds_bf16x8*)(st + kKvDoOff + 4096 * tt + kl.rf[ks]), vf[ks], dp[tt], 0, 0, 0);
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
  if (kSplit) {
    *(__attribute__((address_space(3))) bf16x8*)ds = dsa[0];
    *(__attribute__((address_space(3))) bf16x8*)(ds + kKvDsHalf) = dsa[1];
  }
  // per 32-row step c: the column-wise dO fragments (dV) and Q fragments (dK),
  // read kAhead fragments ahead of the products that take them
  constexpr int kF = kSplit ? 8 : 16;
  constexpr int kAhead = 6;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    bf16x8 F[kF];
#pragma unroll
    for (int f = 0; f < kAhead; ++f) F[f] = tr_frag(st + (f < 8 ? kKvDoOff : kKvQOff), c, kl.tr[f & 7]);
#pragma unroll
    for (int f = 0; f < kF; ++f) {
      if (f + kAhead < kF)
        F[f + kAhead] = tr_frag(st + (f + kAhead < 8 ? kKvDoOff : kKvQOff), c, kl.tr[(f + kAhead) & 7]);
      if (f < 8)
        dv[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[c], F[f], dv[f], 0, 0, 0);
      else
        dk[f - 8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dsa[c], F[f], dk[f - 8], 0, 0, 0);
    }
  }
}

// dK += dS^T Q for the 16 keys of the score wave on this SIMD, from its dS
// slots at `ds` and the Q fragments bq held since that block was staged.
__device__ __forceinline__ void kv_dk8(const bf16x8 bq[2][8], const lds_byte* ds, v4f dk[8]) {
  const bf16x8 dsa[2] = {*(lds_bf16x8*)ds, *(lds_bf16x8*)(ds + kKvDsHalf)};
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int q = 0; q < 8; ++q) dk[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dsa[c], bq[c][q], dk[q], 0, 0, 0);
}

// One staged query block p for a linear wave (phi channels 32 lw..32 lw + 31):
// first the softmax branch's dK of block p - 1 (its dS and Q fragments are
// ready by now), then W += (phi(Q)/den)^T dO and w += (phi(Q)/den)^T u, and
// last block p's Q fragments into bq for the next call.
__device__ __forceinline__ void kv_linear_tile(const lds_byte* st, const KvLane& kl, int lw, int g,
                                               int l16, int p, v4f w[2][8], v4f wz[2], v4f dk[8],
                                               bf16x8 bq[2][8], const lds_byte* ds) {
  if (p > 0) kv_dk8(bq, ds + ((p - 1) & 1) * 2 * kKvDsHalf, dk);
  bf16x8 af[2][2], ub[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int c = 0; c < 2; ++c)
      af[mt][c] = *(lds_bf16x8*)(st + kKvFqOff + (2 * lw + mt) * 2048 + (kl.rd8 ^ (64 * c)));
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
  constexpr int kAhead = 4;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    bf16x8 F[8];
#pragma unroll
    for (int f = 0; f < kAhead; ++f) F[f] = tr_frag(st + kKvDoOff, c, kl.tr[f]);
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      if (f + kAhead < 8) F[f + kAhead] = tr_frag(st + kKvDoOff, c, kl.tr[f + kAhead]);
      w[0][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[0][c], F[f], w[0][f], 0, 0, 0);
      w[1][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[1][c], F[f], w[1][f], 0, 0, 0);
    }
    wz[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[0][c], ub[c], wz[0], 0, 0, 0);
    wz[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[1][c], ub[c], wz[1], 0, 0, 0);
  }
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int q = 0; q < 8; ++q) bq[c][q] = tr_frag(st + kKvQOff, c, kl.tr[q]);
}

// LDS of the linear gradient (after the walk): G - W as bf16 both row-major
// (rows = phi channel) and transposed, and g_z - w in fp32.
constexpr int kGaOff = 0, kGbOff = 32 * 1024, kGzOff = 64 * 1024;
static_assert(kGzOff + 4 * kD <= kKvStages * kKvStage, "the linear gradient's LDS fits the stages");
template <bool kLin>
constexpr int kv_lds_bytes() { return kKvStages * kKvStage + (kLin ? 4 * kKvDsHalf : 0); }
static_assert(kv_lds_bytes<true>() <= 160 * 1024, "the key side's LDS fits one CU");

// Score wave: the keys 16 wave.. of block j; dV (and, without the linear
// branch, dK).
template <bool kLin>
__device__ __forceinline__ void kv_score_role(const BwdKvArgs& a, lds_byte* smem, const BwdKvSrc& src,
                                              const int32_t* list, int n, int j, size_t bh, int wave,
                                              int lane) {
  const int g = lane >> 4, l16 = lane & 15;
  const KvLane kl = kv_lane(lane);
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
  v4f dv[8], dk[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) dv[e] = dk[e] = v4f{0.f, 0.f, 0.f, 0.f};
  const float ks = n > 0 ? a.sk[bh * a.Nb + j] * (kInvSqrtD * kLog2e) : 0.0f;
  lds_byte* ds = smem + kKvDsOff + 16 * (64 * wave + lane);
  kv_walk<kLin>(smem, src, list, n, a.sq + bh * a.Nb, a.Nb, wave, lane, [&](const lds_byte* st, float si, int p) {
    kv_score_tile<kLin>(st, kf, vf, kl, si * ks, g, dv, dk, ds + (p & 1) * 2 * kKvDsHalf);
  });

  // the linear branch's share of dV: phi(K) (G - W), G - W written by the
  // linear waves
  v4f dvl[8];
  if (kLin) {
    lds_barrier();  // every wave is done with the stages
    lds_barrier();  // the linear waves have written G - W and g_z - w
    // phi(K) of this lane's key as A operands (channels 32q + 8g + e)
    const uint16_t* krp = a.kin + ((size_t)bh * a.N + (kvalid ? krow : 0)) * kD;
    bf16x8 fk[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 w = *reinterpret_cast<const uint4*>(krp + 32 * q + 8 * g);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xv = (e & 1) ? bf16_hi(ww[e >> 1]) : bf16_lo(ww[e >> 1]);
        fk[q][e] = kvalid ? (__bf16)phi_apply(xv, a.phi) : (__bf16)0.0f;
      }
    }
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      dvl[ct] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        dvl[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fk[q], lds_row_frag(smem + kGbOff, 16 * ct + l16, 4 * q + g),
                                                          dvl[ct], 0, 0, 0);
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
      store_one(a.dv, orow + c, kLin ? dv[ct][r] + dvl[ct][r] : dv[ct][r], a.grad_f32);
      if (!kLin) store_one(a.dk, orow + c, dk[ct][r] * kInvSqrtD, a.grad_f32);
    }
  }
}

// Linear wave lw = wave - 4: W and w over phi channels 32 lw.., the softmax
// branch's dK of score wave lw's keys, then G - W and g_z - w into LDS and
// the keys' whole dK.
__device__ __forceinline__ void kv_linear_role(const BwdKvArgs& a, lds_byte* smem, const BwdKvSrc& src,
                                               const int32_t* list, int n, int j, size_t bh, int wave,
                                               int lane) {
  const int g = lane >> 4, l16 = lane & 15;
  const int lw = wave - 4;
  const KvLane kl = kv_lane(lane);
  v4f w[2][8], wz[2], dk[8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    wz[mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int et = 0; et < 8; ++et) w[mt][et] = v4f{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) dk[ct] = v4f{0.f, 0.f, 0.f, 0.f};
  const lds_byte* ds = smem + kKvDsOff + 16 * (64 * lw + lane);
  bf16x8 bq[2][8];
  kv_walk<true>(smem, src, list, n, a.sq + bh * a.Nb, a.Nb, wave, lane, [&](const lds_byte* st, float, int p) {
    kv_linear_tile(st, kl, lw, g, l16, p, w, wz, dk, bq, ds);
  });
  lds_barrier();  // every wave is done with the stages; the last block's dS is in LDS
  if (n > 0) kv_dk8(bq, ds + ((n - 1) & 1) * 2 * kKvDsHalf, dk);
  const float* Gh = a.G + bh * kD * kD;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int et = 0; et < 8; ++et)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = 32 * lw + 16 * mt + 4 * g + r;
        const int e = 16 * et + l16;
        const __bf16 gv = (__bf16)(Gh[c * kD + e] - w[mt][et][r]);
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
        const int c = 32 * lw + 16 * mt + 4 * g + r;
        *(__attribute__((address_space(3))) float*)(smem + kGzOff + 4 * c) = a.gz[bh * kD + c] - wz[mt][r];
      }
  }
  lds_barrier();  // G - W and g_z - w are in LDS
  // the linear branch's share of dK: (V (G - W)^T + g_z - w) phi'(K) for the
  // keys 16 lw..
  const int krow = j * kBlk + 16 * lw + l16;
  const bool kvalid = krow < a.N;
  const uint16_t* vrow = a.v + ((size_t)bh * a.N + (kvalid ? krow : 0)) * kD;
  bf16x8 vf[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 u = *reinterpret_cast<const uint4*>(vrow + 32 * q + 8 * g);
    vf[q] = kvalid ? __builtin_bit_cast(bf16x8, u) : bf16x8{};
  }
  v4f dfk[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    dfk[ct] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      dfk[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[q], lds_row_frag(smem + kGaOff, 16 * ct + l16, 4 * q + g),
                                                        dfk[ct], 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int kr = j * kBlk + 16 * lw + 4 * g + r;
    if (kr >= a.N) continue;
    const size_t orow = (bh * a.N + kr) * kD;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const int c = 16 * ct + l16;
      const uint16_t kb = a.kin[orow + c];
      const float gzh = *(__attribute__((address_space(3))) const float*)(smem + kGzOff + 4 * c);
      store_one(a.dk, orow + c, dk[ct][r] * kInvSqrtD + (dfk[ct][r] + gzh) * phi_slope(bf16_lo(kb), a.phi),
                a.grad_f32);
    }
  }
}

template <bool kLin>
__global__ __launch_bounds__(kv_waves<kLin>() * 64, 1) void bwd_kv_kernel(BwdKvArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  lds_byte* smem = (lds_byte*)smem_raw;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // workgroups x, x+8, x+16, x+24 (one XCD, dispatched together) take four
  // consecutive key blocks, whose columns overlap, so their staged query
  // blocks meet in that XCD's L2
  const int x = blockIdx.x;
  const int span = 8 * kGroup;
  const int full = gridDim.x - gridDim.x % span;
  const int j = x < full ? x - x % span + kGroup * (x & 7) + (x % span) / 8 : x;
  const size_t bh = blockIdx.y;
  // this key block's column, clamped to the head's list
  const int c0 = a.coff ? min(max(a.coff[bh * (a.Nb + 1) + j], 0), a.Nb * a.k) : 0;
  const int n = a.coff ? min(a.coff[bh * (a.Nb + 1) + j + 1], a.Nb * a.k) - c0 : 0;
  const int32_t* list = a.cidx ? a.cidx + bh * (size_t)a.Nb * a.k + c0 : nullptr;
  BwdKvSrc src;
  src.q8 = kv_rsrc(a.q8 + bh * (size_t)a.Np * kD, (size_t)a.Np * kD);
  src.dout = kv_rsrc(a.dout + bh * (size_t)a.N * kD, (size_t)a.N * kD * 2);
  src.q = kv_rsrc(a.q + bh * (size_t)a.N * kD, (size_t)a.N * kD * 2);
  src.fqs = kv_rsrc(kLin ? a.fqs + bh * (size_t)a.Np * kD : a.q, (size_t)a.Np * kD * 2);
  src.stats = kv_rsrc(a.stats + bh * (size_t)a.Nb * kBwdStatFloats, (size_t)a.Nb * kKvStatBytes);
  if (!kLin || wave < 4)
    kv_score_role<kLin>(a, smem, src, list, max(n, 0), j, bh, wave, lane);
  else
    kv_linear_role(a, smem, src, list, max(n, 0), j, bh, wave, lane);
}

template <int kMode, bool kF8 = false>
hipError_t launch_mode(const SparseArgs& a, const Shape& sh, hipStream_t s) {
  constexpr size_t stage = (size_t)kK8Bytes + kF16TileBytes +
                           (kMode != kSoftOnly ? (kF8 ? kK8Bytes : kF16TileBytes) : 0);
  const hipError_t e =
      allow_lds(reinterpret_cast<const void*>(sparse_fwd_kernel<kMode, kF8>), (int)(2 * stage));
  if (e != hipSuccess) return e;
  // grouped walks need every member's workgroup, so the block count is rounded up
  const int slots = kMode == kDirect ? sh.Nb : kGroup * ((sh.Nb + kGroup - 1) / kGroup);
  sparse_fwd_kernel<kMode, kF8><<<dim3(slots, sh.BH), 256, 2 * stage, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_fwd(const uint16_t* q, const Workspace& ws, const Shape& sh, int phi,
                             void* out, int out_f32, float* out_linear, bool fp8,
                             const TrainResiduals* res, hipStream_t s) {
  SparseArgs a;
  a.res_stats = res ? res->stats : nullptr;
  a.res_os = res ? res->os : nullptr;
  a.res_m = res ? res->m : nullptr;
  a.res_zm = res ? res->zm : nullptr;
  a.q = q;
  a.q8 = ws.q8;
  a.k8 = ws.k8;
  a.sq = ws.sq;
  a.sk = ws.sk;
  a.idx = ws.idx;
  a.sched = ws.sched;
  a.fk16 = ws.fk16;
  a.v16 = ws.v16;
  a.zb = ws.zb;
  a.fkscale = ws.fkscale;
  a.hf = ws.hf;
  a.z64 = ws.z64;
  a.h16t = nullptr;
  a.hscale = nullptr;
  a.z = nullptr;
  a.N = sh.N;
  a.Nb = sh.Nb;
  a.Np = sh.Np;
  a.k = sh.k;
  a.phi = phi;
  a.out = out;
  a.out_f32 = out_f32;
  a.out_linear = out_linear;
  const bool lin = phi != kPhiNone && sh.k < sh.Nb;
  if (!lin) return launch_mode<kSoftOnly>(a, sh, s);
  if (linear_direct(sh))
    return fp8 ? launch_mode<kDirect, true>(a, sh, s) : launch_mode<kDirect>(a, sh, s);
  return fp8 ? launch_mode<kSubtract, true>(a, sh, s) : launch_mode<kSubtract>(a, sh, s);
}

hipError_t launch_bwd_q(const uint16_t* q, const uint16_t* v, const uint16_t* dout,
                        const Workspace& ws, const BwdWorkspace& bw, const Shape& sh, int phi,
                        void* dq, int grad_f32, const TrainResiduals* res, hipStream_t s) {
  BwdQArgs b;
  b.res_stats = res ? res->stats : nullptr;
  b.res_os = res ? res->os : nullptr;
  b.res_ol = res ? res->ol : nullptr;
  b.res_m = res ? res->m : nullptr;
  b.res_zm = res ? res->zm : nullptr;
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
  auto launch = [&](auto kernel) {
    const hipError_t e = allow_lds(reinterpret_cast<const void*>(kernel), 2 * kBwdStage);
    if (e != hipSuccess) return e;
    kernel<<<dim3(slots, sh.BH), 256, 2 * kBwdStage, s>>>(b);
    return hipGetLastError();
  };
  if (res) return lin ? launch(bwd_q_kernel<true, true>) : launch(bwd_q_kernel<false, true>);
  return lin ? launch(bwd_q_kernel<true, false>) : launch(bwd_q_kernel<false, false>);
}

hipError_t launch_bwd_kv(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                         const Workspace& ws, const BwdWorkspace& bw, const Shape& sh, int phi,
                         void* dk, void* dv, int grad_f32, hipStream_t s) {
  BwdKvArgs a;
  a.q8 = ws.q8;
  a.k8 = ws.k8;
  a.sq = ws.sq;
  a.sk = ws.sk;
  a.q = q;
  a.kin = k;
  a.v = v;
  a.dout = dout;
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
  auto launch = [&](auto kernel, int threads, int lds) {
    const hipError_t e = allow_lds(reinterpret_cast<const void*>(kernel), lds);
    if (e != hipSuccess) return e;
    kernel<<<dim3(sh.Nb, sh.BH), threads, lds, s>>>(a);
    return hipGetLastError();
  };
  return lin ? launch(bwd_kv_kernel<true>, 64 * kv_waves<true>(), kv_lds_bytes<true>())
             : launch(bwd_kv_kernel<false>, 64 * kv_waves<false>(), kv_lds_bytes<false>());
}

hipError_t launch_group_schedule(const int32_t* idx, const Shape& sh, int32_t* sched,
                                 hipStream_t s, const uint32_t* only_if) {
  if (sh.k <= 0) return hipSuccess;
  const int ngroups = (sh.Nb + kGroup - 1) / kGroup;
  const int ragged = sh.N != sh.Nb * kBlk ? 1 : 0;
  const size_t lds4 = group_schedule_x4_lds(sh.Nb, sh.k);
  if (lds4 <= 32 * 1024) {
    const hipError_t e = allow_lds(reinterpret_cast<const void*>(group_schedule_x4_kernel), (int)lds4);
    if (e != hipSuccess) return e;
    group_schedule_x4_kernel<<<dim3((ngroups + 3) / 4, sh.BH), 64, lds4, s>>>(idx, sh.Nb, sh.k, ragged, sched,
                                                                            only_if);
    return hipGetLastError();
  }
  const size_t lds = group_schedule_lds(sh.Nb, sh.k, kGroup);
  const hipError_t e = allow_lds(reinterpret_cast<const void*>(group_schedule_kernel<kGroup>), (int)lds);
  if (e != hipSuccess) return e;
  group_schedule_kernel<kGroup><<<dim3(ngroups, sh.BH), 64, lds, s>>>(idx, sh.Nb, sh.k, ragged, sched, only_if);
  return hipGetLastError();
}

hipError_t launch_debug_qk(const int8_t* q8, const int8_t* k8, const Shape& sh,
                           const int32_t* pairs, int n_pairs, int32_t* acc, hipStream_t s) {
  debug_qk_kernel<<<n_pairs, 256, 0, s>>>(q8, k8, sh.B, sh.H, sh.Np, pairs, acc);
  return hipGetLastError();
}

}  // namespace sla
