// Bandwidth-bound stages of the SageSLA forward on gfx950:
//   block statistics (fp64 block sums, pooled means), K channel mean,
//   INT8 quantisation of Q and smoothed K, block scores + top-k selection,
//   and the linear-branch staging / global state.
//
// This translation unit is compiled with -ffp-contract=off: the quantiser and
// the statistics must reproduce a fixed fp32/fp64 operation order bit for bit.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "sla_internal.h"
#include "sla_quant.h"

namespace sla {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float phi_apply(float x, int phi) {
  if (phi == kPhiElu1) return x > 0.0f ? x + 1.0f : __expf(x);
  return fmaxf(x, 0.0f);
}

// ---------------------------------------------------------------------------
// Block statistics, and the Q quantiser.  One workgroup per (block, b*h):
// lane t loads rows t/16 + 16m (m < 4), channels 8*(t%16).. of Q and K (one
// read of each), then
//   * Q's INT8 codes and scale (the quantiser's arithmetic, code_row8), when
//     q8 is set;
//   * through LDS, lane c < 128 adds Q channel c and lane 128 + c K channel c
//     over the valid rows in ascending order in fp64.
// Outputs: Q/K block means rounded to fp32 (K channel-major, for the block
// scores) and the fp64 K block sums (for the K channel mean).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void block_stats_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, int N, int Nb,
    double* __restrict__ ksum, float* __restrict__ qbar, float* __restrict__ kbar,
    int8_t* __restrict__ q8, float* __restrict__ sq) {
  __shared__ __align__(16) uint16_t tile[2][kBlk][kD];  // bf16 Q, K rows of the block
  __shared__ float red[4];
  const int t = threadIdx.x;
  const int blk = blockIdx.x;
  const int bh = blockIdx.y;
  const int cc = t & 15;
  const int rr = t >> 4;
  const int rows = min(kBlk, N - blk * kBlk);
  const size_t row0 = (size_t)bh * N + (size_t)blk * kBlk;
  uint4 uq[4], uk[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int r = rr + 16 * m;
    uq[m] = uk[m] = make_uint4(0u, 0u, 0u, 0u);
    if (r < rows) {
      uq[m] = *reinterpret_cast<const uint4*>(q + (row0 + r) * kD + cc * 8);
      uk[m] = *reinterpret_cast<const uint4*>(k + (row0 + r) * kD + cc * 8);
    }
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int r = rr + 16 * m;
    *reinterpret_cast<uint4*>(&tile[0][r][cc * 8]) = uq[m];
    *reinterpret_cast<uint4*>(&tile[1][r][cc * 8]) = uk[m];
  }
  float amax = 0.0f;
  float x[4][8];
  if (q8) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      unpack_bf16x8(uq[m], x[m]);  // pad rows are 0
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[m][e]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if ((t & 63) == 0) red[t >> 6] = amax;
  }
  __syncthreads();
  {
    // sums in ascending row order
    const int tensor = t >> 7, c = t & 127;
    double acc = 0.0;
    for (int r = 0; r < rows; ++r) acc += (double)bf16_to_f32(tile[tensor][r][c]);
    const float mean = (float)(acc / (double)rows);
    if (tensor == 0) {
      qbar[((size_t)bh * Nb + blk) * kD + c] = mean;
    } else {
      // channel-major, so the scoring pass reads consecutive key blocks
      kbar[((size_t)bh * kD + c) * Nb + blk] = mean;
      ksum[((size_t)bh * Nb + blk) * kD + c] = acc;
    }
  }
  if (!q8) return;
  float scale, inv;
  const bool any = code_scale(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])), scale, inv);
  int8_t* dst = q8 + ((size_t)bh * Nb * kBlk + (size_t)blk * kBlk) * kD + cc * 8;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int r = rr + 16 * m;
    *reinterpret_cast<uint2*>(dst + (size_t)r * kD) = code_row8(x[m], inv, any && r < rows);
  }
  if (t == 0) sq[(size_t)bh * Nb + blk] = scale;
}

// K channel mean: blocks ascending, one fp64 division by N, rounded to fp32.
// Loads are issued 32 at a time so the dependent additions do not wait on
// one memory round trip each.
__global__ __launch_bounds__(128) void key_mean_kernel(const double* __restrict__ ksum,
                                                       int N, int Nb, float* __restrict__ mu) {
  const int c = threadIdx.x;
  const int bh = blockIdx.x;
  const double* p = ksum + (size_t)bh * Nb * kD + c;
  double s = 0.0;
  int i = 0;
  for (; i + 32 <= Nb; i += 32) {
    double v[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) v[u] = p[(size_t)(i + u) * kD];
#pragma unroll
    for (int u = 0; u < 32; ++u) s += v[u];
  }
  for (; i < Nb; ++i) s += p[(size_t)i * kD];
  mu[(size_t)bh * kD + c] = (float)(s / (double)N);
}

// ---------------------------------------------------------------------------
// INT8 quantiser.  One workgroup per (block, b*h, tensor) (tensor 0 = Q,
// 1 = K - mu; `first` skips Q when the statistics pass has coded it).  Lane t owns
// channels 8*(t%16).. of rows t/16 + 16m.  a = max|x| over valid rows;
// scale = a/127, inv = 127/a (IEEE fp32 division); code = rint(x*inv)
// clamped to [-127,127]; pad rows are written as 0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quantize_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const float* __restrict__ mu, int N, int Nb, int8_t* __restrict__ q8,
    int8_t* __restrict__ k8, float* __restrict__ sq, float* __restrict__ sk, int first) {
  __shared__ float red[4];
  const int t = threadIdx.x;
  const int blk = blockIdx.x;
  const int bh = blockIdx.y;
  const bool isk = blockIdx.z + first == 1;
  const int cc = t & 15;
  const int rr = t >> 4;
  const int rows = min(kBlk, N - blk * kBlk);
  const uint16_t* src = (isk ? k : q) + ((size_t)bh * N + (size_t)blk * kBlk) * kD;
  // the block's valid rows as a buffer, so rows past them read as zero and the
  // four loads are issued together without a condition
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(src), 0, rows * kD * 2, 0x00020000);
  float m8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) m8[e] = isk ? mu[(size_t)bh * kD + cc * 8 + e] : 0.0f;
  uint4 u[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
    u[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                         rs, ((rr + 16 * m) * kD + cc * 8) * 2, 0, 0));
  float x[4][8];
  float amax = 0.0f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const bool valid = rr + 16 * m < rows;
    unpack_bf16x8(u[m], x[m]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[m][e] = valid ? x[m][e] - m8[e] : 0.0f;
      amax = fmaxf(amax, fabsf(x[m][e]));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  float scale, inv;
  const bool any = code_scale(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])), scale, inv);
  int8_t* dst = (isk ? k8 : q8) + ((size_t)bh * Nb * kBlk + (size_t)blk * kBlk) * kD + cc * 8;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int r = rr + 16 * m;
    *reinterpret_cast<uint2*>(dst + (size_t)r * kD) = code_row8(x[m], inv, any && r < rows);
  }
  if (t == 0) (isk ? sk : sq)[(size_t)bh * Nb + blk] = scale;
}

// ---------------------------------------------------------------------------
// Block scores and top-k.  A workgroup owns R query blocks of one (b,h).
// Phase 1: lane t computes s_ij = sum_c qbar_ic kbar_jc for the key blocks
// j = t + 256u of a pass and all R rows (fp64 fma, channels ascending; the
// fp32 x fp32 product is exact in fp64 so each step rounds once) and keeps the
// scores in LDS.  kbar is channel-major, so a wave's loads of one channel are
// contiguous; qbar goes through LDS as fp64 [channel][row] and is read a
// chunk of channels at a time into registers.
// Phase 2, one wave per row: the scores are spread over kBins buckets by the
// monotone map floor((s - min) * kBins / (max - min)); one histogram and a
// suffix scan find the bucket B holding the k-th largest score.  Scores in
// buckets above B are kept; inside B the candidates are ranked exactly by
// (score descending, index ascending) to find the last kept one (Ts, Tj).
// Then j is kept iff s_j > Ts or (s_j == Ts and j <= Tj), written ascending.
// ---------------------------------------------------------------------------
constexpr int kBins = 1024;

template <int R>
__global__ __launch_bounds__(256) void block_topk_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int Nb, int k,
    int32_t* __restrict__ idx, uint32_t* __restrict__ mask, int32_t* __restrict__ uidx) {
  extern __shared__ __align__(16) unsigned char smem[];
  double* qs = reinterpret_cast<double*>(smem);                              // [128][R]
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem + R * kD * 8);           // [4][kBins]
  double* cand_s = reinterpret_cast<double*>(smem + R * kD * 8 + 4 * kBins * 4);   // [4][64]
  int* cand_j = reinterpret_cast<int*>(smem + R * kD * 8 + 4 * kBins * 4 + 4 * 64 * 8);  // [4][64]
  double* sc = reinterpret_cast<double*>(smem + R * kD * 8 + 4 * kBins * 4 + 4 * 64 * 12);  // [R][Nb]
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int bh = blockIdx.y;
  const int i0 = blockIdx.x * R;
  const float* kb = kbar + (size_t)bh * kD * Nb;  // [128][Nb]

  for (int e = t; e < R * kD; e += 256) {
    const int r = e % R, c = e / R;
    const int i = min(i0 + r, Nb - 1);
    qs[e] = (double)qbar[((size_t)bh * Nb + i) * kD + c];
  }
  __syncthreads();

  constexpr int kSlots = 5;       // key blocks per lane and pass
  constexpr int kCh = R >= 8 ? 4 : 8;  // channels per register chunk of qbar
  // this head's kbar slice (below 2^31 bytes); reads past it return 0
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(kb), 0, (int)((size_t)kD * Nb * 4), 0x00020000);
  for (int base = 0; base < Nb; base += 256 * kSlots) {
    double acc[kSlots][R];
    int voff[kSlots];
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
      voff[u] = 4 * min(base + 256 * u + t, Nb - 1);
#pragma unroll
      for (int r = 0; r < R; ++r) acc[u][r] = 0.0;
    }
    for (int c0 = 0; c0 < kD; c0 += kCh) {
      // all loads of the chunk first, so they are in flight together
      float kv[kSlots][kCh];
#pragma unroll
      for (int u = 0; u < kSlots; ++u)
#pragma unroll
        for (int e = 0; e < kCh; ++e)
          kv[u][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(kr, voff[u], 4 * (c0 + e) * Nb, 0));
      double qd[kCh][R];
#pragma unroll
      for (int e = 0; e < kCh; ++e)
#pragma unroll
        for (int r = 0; r < R; ++r) qd[e][r] = qs[(c0 + e) * R + r];
#pragma unroll
      for (int u = 0; u < kSlots; ++u)
#pragma unroll
        for (int e = 0; e < kCh; ++e) {
          const double kd = (double)kv[u][e];
#pragma unroll
          for (int r = 0; r < R; ++r) acc[u][r] = fma(qd[e][r], kd, acc[u][r]);
        }
    }
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {
      const int j = base + 256 * u + t;
      if (j < Nb) {
#pragma unroll
        for (int r = 0; r < R; ++r) sc[(size_t)r * Nb + j] = acc[u][r];
      }
    }
  }
  __syncthreads();

  uint32_t* h = hist + wave * kBins;
  double* cs = cand_s + wave * 64;
  int* cj = cand_j + wave * 64;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = wave; r < R; r += 4) {
    const int i = i0 + r;
    if (i >= Nb) break;  // wave-uniform; no block barrier follows
    const double* sr = sc + (size_t)r * Nb;
    double mn = INFINITY, mx = -INFINITY;
    for (int j = lane; j < Nb; j += 64) {
      mn = fmin(mn, sr[j]);
      mx = fmax(mx, sr[j]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      mn = fmin(mn, __shfl_xor(mn, off));
      mx = fmax(mx, __shfl_xor(mx, off));
    }
    double Ts;
    int Tj;
    if (!(mx > mn)) {
      // every score equal: the k lowest indices
      Ts = mx;
      Tj = k - 1;
    } else {
      double scale = (double)kBins / (mx - mn);
      if (!(scale < 1e300)) scale = 1e300;
      auto bucket = [&](double v) { return (int)fmin((v - mn) * scale, (double)(kBins - 1)); };
#pragma unroll
      for (int q = 0; q < kBins / 64; ++q) h[lane * (kBins / 64) + q] = 0;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      for (int j = lane; j < Nb; j += 64) atomicAdd(&h[bucket(sr[j])], 1u);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      // lane l owns buckets kBins-1-16l .. kBins-16-16l (descending)
      constexpr int kPer = kBins / 64;
      uint32_t cnt[kPer];
      uint32_t local = 0;
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        cnt[q] = h[kBins - 1 - kPer * lane - q];
        local += cnt[q];
      }
      uint32_t incl = local;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      uint32_t before = incl - local;
      int B = -1;
      uint32_t need = 0, nc = 0;
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        if (B < 0 && before < (uint32_t)k && before + cnt[q] >= (uint32_t)k) {
          B = kBins - 1 - kPer * lane - q;
          need = (uint32_t)k - before;
          nc = cnt[q];
        }
        before += cnt[q];
      }
      const uint64_t found = __ballot(B >= 0);
      const int src = __ffsll((unsigned long long)found) - 1;
      B = __shfl(B, src);
      need = __shfl(need, src);
      nc = __shfl(nc, src);
      // the need-th best candidate of bucket B by (score desc, index asc)
      Ts = 0.0;
      Tj = 0;
      if (nc <= 64) {
        uint32_t base = 0;
        for (int jb = 0; jb < Nb; jb += 64) {
          const int j = jb + lane;
          const bool in = j < Nb && bucket(sr[j]) == B;
          const uint64_t bb = __ballot(in);
          if (in) {
            const uint32_t pos = base + (uint32_t)__popcll(bb & lt_mask);
            cs[pos] = sr[j];
            cj[pos] = j;
          }
          base += (uint32_t)__popcll(bb);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
        __builtin_amdgcn_wave_barrier();
        bool mine = false;
        double my_s = 0.0;
        int my_j = 0;
        if ((uint32_t)lane < nc) {
          my_s = cs[lane];
          my_j = cj[lane];
          uint32_t rank = 0;
          for (uint32_t c = 0; c < nc; ++c)
            rank += (cs[c] > my_s || (cs[c] == my_s && cj[c] < my_j)) ? 1u : 0u;
          mine = rank == need - 1;
        }
        const int who = __ffsll((unsigned long long)__ballot(mine)) - 1;
        Ts = __shfl(my_s, who);
        Tj = __shfl(my_j, who);
      } else {
        // large tie groups: rank every member of bucket B against all others
        bool mine = false;
        double my_s = 0.0;
        int my_j = 0;
        for (int jb = 0; jb < Nb; jb += 64) {
          const int j = jb + lane;
          if (j < Nb && bucket(sr[j]) == B) {
            uint32_t rank = 0;
            for (int u = 0; u < Nb; ++u) {
              const double v = sr[u];
              if (bucket(v) == B) rank += (v > sr[j] || (v == sr[j] && u < j)) ? 1u : 0u;
            }
            if (rank == need - 1) {
              mine = true;
              my_s = sr[j];
              my_j = j;
            }
          }
        }
        const int who = __ffsll((unsigned long long)__ballot(mine)) - 1;
        Ts = __shfl(my_s, who);
        Tj = __shfl(my_j, who);
      }
    }
    int32_t* out = idx + ((size_t)bh * Nb + i) * k;
    uint32_t* mrow = mask ? mask + ((size_t)bh * Nb + i) * ((Nb + 31) / 32) : nullptr;
    int32_t* urow = uidx ? uidx + ((size_t)bh * Nb + i) * (Nb - k) : nullptr;
    uint32_t base = 0, ubase = 0;
    for (int jb = 0; jb < Nb; jb += 64) {
      const int j = jb + lane;
      const bool valid = j < Nb;
      const double v = valid ? sr[j] : -INFINITY;
      const bool sel = valid && (v > Ts || (v == Ts && j <= Tj));
      const uint64_t sb = __ballot(sel);
      const uint32_t pos = base + (uint32_t)__popcll(sb & lt_mask);
      if (sel && pos < (uint32_t)k) out[pos] = j;
      if (mrow) {
        const int w0 = jb >> 5;
        if (lane == 0) mrow[w0] = (uint32_t)sb;
        if (lane == 1 && w0 + 1 < (Nb + 31) / 32) mrow[w0 + 1] = (uint32_t)(sb >> 32);
      }
      if (urow) {
        const uint64_t ub = __ballot(valid && !sel);
        const uint32_t upos = ubase + (uint32_t)__popcll(ub & lt_mask);
        if (valid && !sel && upos < (uint32_t)(Nb - k)) urow[upos] = j;
        ubase += (uint32_t)__popcll(ub);
      }
      base += (uint32_t)__popcll(sb);
    }
  }
}

// ---------------------------------------------------------------------------
// Linear-branch staging.  A workgroup walks a contiguous chunk of key blocks
// of one (b,h).  For every block it
//   * writes V and phi(K)/16 as fp16 in the per-block layout
//     [channel][permuted key] that the attention kernel reads as matrix-core
//     operands (pad keys 0),
//   * writes the block's sum of phi(K)/16 over its keys (fp32, per channel),
//   * accumulates H = sum phi(K)^T V and z = sum phi(K) for the chunk
//     (fp16 operands, fp32 accumulation, blocks in ascending order),
//   * when k8 is set, writes the INT8 codes and scale of the smoothed block
//     K - mu (the quantiser's arithmetic, code_row8).
// Permuted key order inside each 32-key half: position 8g+s holds key
// 4g+s (s<4) or 16+4g+(s-4) (s>=4), matching the transposed score tiles
// that feed the P.V product.
// kMode: 0 = V staging only, 1 = V and phi(K) staging and block sums, 2 =
// staging plus the H, z partial sums.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int perm_pos(int key) {
  const int h = key >> 5, r = key & 31;
  return 32 * h + 8 * ((r & 15) >> 2) + (r & 3) + 4 * (r >> 4);
}

// LDS transpose tiles: row c (a channel) holds the 64 positions in 8 chunks of
// 8 fp16, rows padded to 72 and chunk P stored at P ^ ((c >> 4) & 7).  Rows 8
// apart (the transposed writes) and consecutive rows (the matrix-core and row
// reads) then spread over the 64 banks.
constexpr int kTRow = kBlk + 8;
__device__ __forceinline__ int tpos(int c, int pos) {
  return c * kTRow + ((((pos >> 3) ^ (c >> 4)) & 7) << 3) + (pos & 7);
}

template <int kMode>
__global__ __launch_bounds__(256) void linear_prep_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int N, int Nb, int phi,
    uint16_t* __restrict__ fk16, uint16_t* __restrict__ v16, float* __restrict__ zb,
    float* __restrict__ hpart, float* __restrict__ zpart, const float* __restrict__ mu,
    int8_t* __restrict__ k8, float* __restrict__ sk) {
  // LDS: transposed tiles [128 channels][64 positions] fp16 (see tpos)
  __shared__ __align__(16) _Float16 fkT[kD * kTRow];
  __shared__ __align__(16) _Float16 vT[kD * kTRow];
  __shared__ float red[4];
  constexpr bool kLinear = kMode >= 1;
  constexpr bool kReduce = kMode >= 2;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int chunk = blockIdx.x;
  const int bh = blockIdx.y;
  const int j0 = (int)(((long long)chunk * Nb) / kLinChunks);
  const int j1 = (int)(((long long)(chunk + 1) * Nb) / kLinChunks);
  // lane t: keys 4a..4a+3, channels 8cc..8cc+7
  const int a = t >> 4;
  const int cc = t & 15;

  float4v acc[2][8];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 8; ++y) acc[x][y] = float4v{0.f, 0.f, 0.f, 0.f};
  float zacc = 0.0f;
  const bool quant = k8 != nullptr;  // workgroup-uniform
  const bool needk = kLinear || quant;
  float m8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) m8[e] = quant ? mu[(size_t)bh * kD + cc * 8 + e] : 0.0f;

  // raw bf16 rows 4a+m, channels 8cc.. of block j (pad rows 0)
  auto load_raw = [&](int j, uint4* rv, uint4* rk) {
    const int rows = min(kBlk, N - j * kBlk);
    const size_t row0 = (size_t)bh * N + (size_t)j * kBlk;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r = 4 * a + m;
      rv[m] = rk[m] = make_uint4(0u, 0u, 0u, 0u);
      if (r < rows) {
        rv[m] = *reinterpret_cast<const uint4*>(v + (row0 + r) * kD + cc * 8);
        if (needk) rk[m] = *reinterpret_cast<const uint4*>(k + (row0 + r) * kD + cc * 8);
      }
    }
  };
  for (int j = j0; j < j1; ++j) {
    const int rows = min(kBlk, N - j * kBlk);
    uint4 rv[4], rk[4];
    load_raw(j, rv, rk);
    _Float16 fv[4][8], vv[4][8];
    float amax = 0.0f;  // max |K - mu| over this lane's valid rows
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r = 4 * a + m;
      float xv[8], xk[8];
      unpack_bf16x8(rv[m], xv);
      unpack_bf16x8(rk[m], xk);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        vv[m][e] = (_Float16)xv[e];
        if (kLinear) fv[m][e] = (r < rows) ? (_Float16)(phi_apply(xk[e], phi) * kPhiScale) : (_Float16)0.0f;
        if (quant && r < rows) amax = fmaxf(amax, fabsf(xk[e] - m8[e]));
      }
    }
    if (quant) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
      if (lane == 0) red[wave] = amax;
    }
    // transposed LDS writes: 4 consecutive keys -> 4 consecutive positions
    const int p0 = perm_pos(4 * a);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = cc * 8 + e;
      half4 hv = {vv[0][e], vv[1][e], vv[2][e], vv[3][e]};
      *reinterpret_cast<half4*>(&vT[tpos(c, p0)]) = hv;
      if (kLinear) {
        half4 hf = {fv[0][e], fv[1][e], fv[2][e], fv[3][e]};
        *reinterpret_cast<half4*>(&fkT[tpos(c, p0)]) = hf;
      }
    }
    __syncthreads();
    if (quant) {
      float scale, inv;
      const bool any = code_scale(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])), scale, inv);
      int8_t* dst = k8 + ((size_t)bh * Nb + j) * kBlk * kD + cc * 8;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = 4 * a + m;
        float xq[8];  // K - mu, recomputed from the raw row still in registers
        unpack_bf16x8(rk[m], xq);
#pragma unroll
        for (int e = 0; e < 8; ++e) xq[e] = xq[e] - m8[e];
        *reinterpret_cast<uint2*>(dst + (size_t)r * kD) = code_row8(xq, inv, any && r < rows);
      }
      if (t == 0) sk[(size_t)bh * Nb + j] = scale;
    }
    // V (and phi(K)) staging copy-out: 16 KB contiguous per block, 16-byte
    // chunk q = 8c + P
    {
      const size_t blk = ((size_t)bh * Nb + j) * kD * kBlk;
      uint4* dstv = reinterpret_cast<uint4*>(v16 + blk);
      uint4* dstf = reinterpret_cast<uint4*>(fk16 + blk);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int q = t + 256 * m;
        dstv[q] = *reinterpret_cast<const uint4*>(&vT[tpos(q >> 3, 8 * (q & 7))]);
        if (kLinear) dstf[q] = *reinterpret_cast<const uint4*>(&fkT[tpos(q >> 3, 8 * (q & 7))]);
      }
    }
    // per-block sum of phi(K)/16 over the keys, channel t
    if (kLinear && t < kD) {
      float zj = 0.0f;
      for (int p = 0; p < kBlk / 8; ++p) {
        const half8 hv = *reinterpret_cast<const half8*>(&fkT[tpos(t, 8 * p)]);
#pragma unroll
        for (int e = 0; e < 8; ++e) zj += (float)hv[e];
      }
      zb[((size_t)bh * Nb + j) * kD + t] = zj;
      if (kReduce) zacc += zj;
    }
    if (kReduce) {
      // H[c][e] += sum_pos fkT[c][pos] vT[e][pos]; wave owns c-tiles 2w, 2w+1
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        half8 af[2], bf[8];
#pragma unroll
        for (int x = 0; x < 2; ++x)
          af[x] = *reinterpret_cast<const half8*>(&fkT[tpos(16 * (2 * wave + x) + l16, 32 * kc + 8 * g)]);
#pragma unroll
        for (int y = 0; y < 8; ++y)
          bf[y] = *reinterpret_cast<const half8*>(&vT[tpos(16 * y + l16, 32 * kc + 8 * g)]);
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int y = 0; y < 8; ++y)
            acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[x], bf[y], acc[x][y], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  if (kReduce) {
    float* hp = hpart + ((size_t)bh * kLinChunks + chunk) * kD * kD;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 8; ++y)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          hp[(size_t)(16 * (2 * wave + x) + 4 * g + r) * kD + 16 * y + l16] = acc[x][y][r];
    if (t < kD) zpart[((size_t)bh * kLinChunks + chunk) * kD + t] = zacc;
  }
}

// Whole-head linear state, step 1: H (and z) as the chunk partials added in
// chunk order.  Workgroup (bh, y) owns H elements [1024y, 1024y + 1024) and
// writes the sum over chunk 0's slot (it alone reads and writes that range).
__global__ __launch_bounds__(256) void linear_sum_kernel(float* __restrict__ hpart,
                                                         const float* __restrict__ zpart,
                                                         float* __restrict__ z) {
  const int t = threadIdx.x;
  const int bh = blockIdx.x;
  float* hp = hpart + (size_t)bh * kLinChunks * kD * kD;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = blockIdx.y * 1024 + t + 256 * m;
    float v[kLinChunks];
#pragma unroll
    for (int c = 0; c < kLinChunks; ++c) v[c] = hp[(size_t)c * kD * kD + e];
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kLinChunks; ++c) s += v[c];
    hp[e] = s;
  }
  if (blockIdx.y == 0 && t < kD) {
    float v[kLinChunks];
#pragma unroll
    for (int c = 0; c < kLinChunks; ++c) v[c] = zpart[((size_t)bh * kLinChunks + c) * kD + t];
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kLinChunks; ++c) s += v[c];
    z[(size_t)bh * kD + t] = s;
  }
}

// Step 2: store H^T as fp16 scaled by 2^-s so that max|H| * 2^-s lies in
// [2^14, 2^15), plus 2^s; with hb set, also H itself (row-major, unscaled)
// as bf16 for the backward.
__global__ __launch_bounds__(256) void linear_cvt_kernel(const float* __restrict__ hpart,
                                                         uint16_t* __restrict__ h16t,
                                                         float* __restrict__ hscale,
                                                         uint16_t* __restrict__ hb) {
  __shared__ float red[4];
  const int t = threadIdx.x;
  const int bh = blockIdx.x;
  const float* hs = hpart + (size_t)bh * kLinChunks * kD * kD;
  float hv[64];
  float mx = 0.0f;
#pragma unroll
  for (int m = 0; m < 64; ++m) {
    hv[m] = hs[t + 256 * m];
    mx = fmaxf(mx, fabsf(hv[m]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((t & 63) == 0) red[t >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  int s = 0;
  if (mx > 0.0f) s = ilogbf(mx) - 14;
  const float down = ldexpf(1.0f, -s);
  if (t == 0) hscale[bh] = ldexpf(1.0f, s);
  _Float16* out = reinterpret_cast<_Float16*>(h16t) + (size_t)bh * kD * kD;
#pragma unroll
  for (int m = 0; m < 64; ++m) {
    const int e = t + 256 * m;       // H[c][o] with c = e / 128, o = e % 128
    const int c = e >> 7, o = e & 127;
    out[(size_t)o * kD + c] = (_Float16)(hv[m] * down);
  }
  if (hb) {
    __bf16* ob = reinterpret_cast<__bf16*>(hb) + (size_t)bh * kD * kD;
#pragma unroll
    for (int m = 0; m < 64; ++m) ob[t + 256 * m] = (__bf16)hv[m];
  }
}

}  // namespace

hipError_t launch_block_stats(const uint16_t* q, const uint16_t* k, const Shape& sh,
                              double* ksum, float* qbar, float* kbar, int8_t* q8, float* sq,
                              hipStream_t s) {
  dim3 grid(sh.Nb, sh.BH);
  block_stats_kernel<<<grid, 256, 0, s>>>(q, k, sh.N, sh.Nb, ksum, qbar, kbar, q8, sq);
  return hipGetLastError();
}

hipError_t launch_key_mean(const double* ksum, const Shape& sh, float* mu, hipStream_t s) {
  key_mean_kernel<<<sh.BH, 128, 0, s>>>(ksum, sh.N, sh.Nb, mu);
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* q, const uint16_t* k, const float* mu,
                           const Shape& sh, int8_t* q8, int8_t* k8, float* sq, float* sk,
                           bool k_only, hipStream_t s) {
  dim3 grid(sh.Nb, sh.BH, k_only ? 1 : 2);
  quantize_kernel<<<grid, 256, 0, s>>>(q, k, mu, sh.N, sh.Nb, q8, k8, sq, sk, k_only ? 1 : 0);
  return hipGetLastError();
}

size_t topk_lds_bytes(int Nb, int* rows_per_group) {
  auto bytes = [&](int R) {
    return (size_t)R * Nb * 8 + (size_t)R * kD * 8 + 4 * kBins * 4 + 4 * 64 * 12;
  };
  int R = 8;
  while (R > 1 && bytes(R) > 96 * 1024) R >>= 1;
  if (rows_per_group) *rows_per_group = R;
  return bytes(R);
}

hipError_t launch_block_topk(const float* qbar, const float* kbar, const Shape& sh,
                             int32_t* idx, uint32_t* mask, int32_t* uidx, hipStream_t s) {
  int R = 1;
  const size_t lds = topk_lds_bytes(sh.Nb, &R);
  static std::once_flag once;
  std::call_once(once, [] {
    const int big = 160 * 1024;
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(block_topk_kernel<1>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, big);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(block_topk_kernel<2>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, big);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(block_topk_kernel<4>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, big);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(block_topk_kernel<8>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, big);
  });
  dim3 grid((sh.Nb + R - 1) / R, sh.BH);
  switch (R) {
    case 8: block_topk_kernel<8><<<grid, 256, lds, s>>>(qbar, kbar, sh.Nb, sh.k, idx, mask, uidx); break;
    case 4: block_topk_kernel<4><<<grid, 256, lds, s>>>(qbar, kbar, sh.Nb, sh.k, idx, mask, uidx); break;
    case 2: block_topk_kernel<2><<<grid, 256, lds, s>>>(qbar, kbar, sh.Nb, sh.k, idx, mask, uidx); break;
    default: block_topk_kernel<1><<<grid, 256, lds, s>>>(qbar, kbar, sh.Nb, sh.k, idx, mask, uidx); break;
  }
  return hipGetLastError();
}

hipError_t launch_linear_prep(const uint16_t* k, const uint16_t* v, const Shape& sh, int phi,
                              bool reduce, uint16_t* fk16, uint16_t* v16, float* zb, float* hpart,
                              float* zpart, const float* mu, int8_t* k8, float* sk, hipStream_t s) {
  dim3 grid(kLinChunks, sh.BH);
  if (phi == kPhiNone)
    linear_prep_kernel<0><<<grid, 256, 0, s>>>(k, v, sh.N, sh.Nb, phi, fk16, v16, zb, hpart, zpart, mu, k8, sk);
  else if (!reduce)
    linear_prep_kernel<1><<<grid, 256, 0, s>>>(k, v, sh.N, sh.Nb, phi, fk16, v16, zb, hpart, zpart, mu, k8, sk);
  else
    linear_prep_kernel<2><<<grid, 256, 0, s>>>(k, v, sh.N, sh.Nb, phi, fk16, v16, zb, hpart, zpart, mu, k8, sk);
  return hipGetLastError();
}

hipError_t launch_linear_final(float* hpart, const float* zpart, const Shape& sh,
                               uint16_t* h16t, float* hscale, float* z, hipStream_t s,
                               uint16_t* hb) {
  linear_sum_kernel<<<dim3(sh.BH, kD * kD / 1024), 256, 0, s>>>(hpart, zpart, z);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  linear_cvt_kernel<<<sh.BH, 256, 0, s>>>(hpart, h16t, hscale, hb);
  return hipGetLastError();
}

}  // namespace sla
