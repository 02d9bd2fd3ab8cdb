// Bandwidth-bound stages of the SageSLA forward on gfx950:
//   block statistics (fp64 block sums, pooled means), K channel mean,
//   INT8 quantisation of Q and smoothed K, block scores + top-k selection,
//   and the linear-branch staging / global state.
//
// This translation unit is compiled with -ffp-contract=off: the quantiser and
// the statistics must reproduce a fixed fp32/fp64 operation order bit for bit.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "sla_internal.h"
#include "sla_quant.h"

namespace sla {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float phi_apply(float x, int phi) {
  if (phi == kPhiElu1) return x > 0.0f ? x + 1.0f : __expf(x);
  return fmaxf(x, 0.0f);
}

// bf16 splits of the fp32 block means for the filtered top-k (below): x =
// x_h + x_l + e with x_h = bf16(x) and x_l = bf16(x - x_h) (the difference is
// exact in fp32), |e| <= 2^-18 |x|.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void split_bf16(float x, __bf16& h, __bf16& l) {
  h = (__bf16)x;
  l = (__bf16)(x - (float)h);
}

__device__ __forceinline__ float next_up(float x) {  // the least float above a finite x
  if (x == 0.0f) return __uint_as_float(1u);
  const uint32_t u = __float_as_uint(x);
  return __uint_as_float(x > 0.0f ? u + 1u : u - 1u);
}

// A non-zero mean outside [2^-60, 2^60] (or not finite) is outside the
// filtered top-k's range: its rows take the exact kernel.
__device__ __forceinline__ bool out_of_range(float x) {
  const float a = fabsf(x);
  return a != 0.0f && !(a >= 0x1p-60f && a <= 0x1p60f);
}

// Layout of the K splits: per head, per tile of 16 key blocks, per k-step s
// of 32 channels, the hi and lo operands as the 64 lanes of the matrix core
// hold them (lane 16g + n: key block 16 tile + n, channels 32s + 8g ..
// 32s + 8g + 7), 1 KB each.
constexpr int kSplitTileElems = 4 * 2 * 512;  // bf16 per tile
__device__ __forceinline__ size_t ksplit_index(int bh, int Nb, int j, int c) {
  const int tl = j >> 4, n = j & 15, s = c >> 5, g = (c >> 3) & 3, e = c & 7;
  return ((size_t)bh * ((Nb + 15) >> 4) + tl) * kSplitTileElems + (size_t)s * 2 * 512 + (16 * g + n) * 8 + e;
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
    int8_t* __restrict__ q8, float* __restrict__ sq, uint16_t* __restrict__ ksplit,
    uint8_t* __restrict__ kflag, float* __restrict__ kbar_rm, float* __restrict__ knorm) {
  __shared__ __align__(16) uint16_t tile[2][kBlk][kD];  // bf16 Q, K rows of the block
  __shared__ float red[4];
  __shared__ double nsq[2];
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
  bool kbad = false;
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
      if (ksplit) {
        __bf16 h, l;
        split_bf16(mean, h, l);
        uint16_t* d = ksplit + ksplit_index(bh, Nb, blk, c);
        d[0] = __builtin_bit_cast(uint16_t, h);
        d[512] = __builtin_bit_cast(uint16_t, l);
        kbad = out_of_range(mean);
        kbar_rm[((size_t)bh * Nb + blk) * kD + c] = mean;  // row-major, for the filter's fp64 scores
        // the block's squared norm (fp64), over the two waves holding K
        double q2 = (double)mean * (double)mean;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) q2 += __shfl_xor(q2, off);
        if ((t & 63) == 0) nsq[(t >> 6) - 2] = q2;
      }
    }
  }
  if (ksplit) {
    const int any_bad = __syncthreads_or(kbad ? 1 : 0);
    if (t == 0) {
      kflag[(size_t)bh * Nb + blk] = any_bad ? 1 : 0;
      knorm[(size_t)bh * Nb + blk] = next_up((float)sqrt(nsq[0] + nsq[1]));  // an upper bound
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

// Rows i0 .. i0 + R - 1 of head bh (the workgroup's 256 threads, `smem` its LDS).
template <int R>
__device__ __forceinline__ void topk_rows(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                          int Nb, int k, int32_t* __restrict__ idx,
                                          uint32_t* __restrict__ mask, int bh, int i0,
                                          unsigned char* smem) {
  double* qs = reinterpret_cast<double*>(smem);                              // [128][R]
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem + R * kD * 8);           // [4][kBins]
  double* cand_s = reinterpret_cast<double*>(smem + R * kD * 8 + 4 * kBins * 4);   // [4][64]
  int* cand_j = reinterpret_cast<int*>(smem + R * kD * 8 + 4 * kBins * 4 + 4 * 64 * 8);  // [4][64]
  double* sc = reinterpret_cast<double*>(smem + R * kD * 8 + 4 * kBins * 4 + 4 * 64 * 12);  // [R][Nb]
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
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
    uint32_t base = 0;
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
      base += (uint32_t)__popcll(sb);
    }
  }
}

// One workgroup per R rows; or, with `list` (a count, then packed rows bh *
// Nb + i), the rows the filtered pass handed back, one at a time per
// workgroup over a small grid (R = 1), so that a pass with nothing to redo
// costs a few microseconds.
template <int R>
__global__ __launch_bounds__(256) void block_topk_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int Nb, int k,
    int32_t* __restrict__ idx, uint32_t* __restrict__ mask, const uint32_t* __restrict__ list) {
  extern __shared__ __align__(16) unsigned char smem[];
  if (!list) {
    topk_rows<R>(qbar, kbar, Nb, k, idx, mask, blockIdx.y, blockIdx.x * R, smem);
    return;
  }
  const uint32_t n = list[0];
  for (uint32_t e = blockIdx.x; e < n; e += gridDim.x) {
    const uint32_t row = list[1 + e];
    topk_rows<R>(qbar, kbar, Nb, k, idx, mask, (int)(row / (uint32_t)Nb), (int)(row % (uint32_t)Nb), smem);
    __syncthreads();  // the LDS serves the next row
  }
}

// ---------------------------------------------------------------------------
// Filtered block top-k: the same kept lists as block_topk_kernel, with the
// fp64 scores computed only for the key blocks whose fate they decide.
// block_scores_approx_kernel (matrix cores, 64 query blocks per workgroup):
// with the bf16 splits x = x_h + x_l + e of the means (split_bf16; the K ones
// written by the statistics pass), the approximate score s~_ij = sum_c q_h k_h
// + q_h k_l + q_l k_h takes exact bf16 products with fp32 accumulation.  The
// dropped terms (q_l k_l and the e parts) are below 2^-16.4 sum|q||k|, the
// fp32 accumulation of the 384 products below 2^-14.4 sum|q||k| even with
// truncating adds, and sum|q||k| <= |q_i| |k_j| (Cauchy-Schwarz; the norms
// rounded up), so the exact fp64 score s_ij of block_topk_kernel lies within
// E_i = 2^-12 |q_i| max_j |k_j| + 2^-100 of s~_ij for every key block j of
// row i.  (Inside the range of out_of_range no product overflows, and
// denormal products are covered by the 2^-100.)  It writes s~ (fp32 [Nb][Nb]
// per head) and, per row and wave, |q_i| times the largest |k_j| of the
// wave's key blocks (NaN when a mean of the row or of those key blocks is out
// of range).
// block_topk_approx_select_kernel (one wave per row): T = the k-th largest s~
// (the histogram of block_topk_kernel on s~).  At least k key blocks have s >=
// T - E and fewer than k have s > T + E, so the k-th largest s lies in
// [T - E, T + E]: key blocks with s~ > T + 2E are kept, those with s~ < T - 2E
// are not, and the ones in between (a handful on smooth inputs) get their fp64
// score, computed as block_topk_kernel does, and are ranked by (score desc,
// index asc) for the places the certain ones leave.  A row with more than 64
// such key blocks or more than 64 approximate scores in the threshold bucket
// (large groups of equal scores), or with means out of range, is appended to
// a list instead, and block_topk_kernel (list mode) selects it afterwards.
// ---------------------------------------------------------------------------
constexpr int kSRows = 64;   // query blocks per scoring workgroup (four row tiles)
constexpr int kSWaves = 8;   // waves per scoring workgroup
constexpr int kFSlots = 27;  // key blocks per lane of a row held in registers (Nb <= 1728)
constexpr int kBWaves = 4;   // rows per selecting workgroup (one wave each)
constexpr int kRedoGrid = 512;  // workgroups of the exact kernel over the hand-back list

__global__ __launch_bounds__(64 * kSWaves) void block_scores_approx_kernel(
    const float* __restrict__ qbar, const uint16_t* __restrict__ ksplit,
    const uint8_t* __restrict__ kflag, const float* __restrict__ knorm, int Nb,
    float* __restrict__ scores, float* __restrict__ amaxp, uint32_t* __restrict__ redo) {
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) redo[0] = 0;  // the hand-back list
  // the workgroup's A operands in LDS as the matrix core's lanes hold them:
  // [row tile][k-step][hi, lo][64 lanes][8 bf16], lane 16g + l16 = row
  // 16 rt + l16, channels 32s + 8g ..; then the rows' norms and range flags
  __shared__ __align__(16) unsigned char alds[4 * 4 * 2 * 1024];
  __shared__ float qnorm[kSRows];
  __shared__ uint32_t qflag[kSRows];
  const int t = threadIdx.x;
  // the wave index in a scalar register: tile offsets are uniform
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63, g = lane >> 4, l16 = lane & 15;
  const int bh = blockIdx.y;
  const int i0 = blockIdx.x * kSRows;
  const int ntiles = (Nb + 15) >> 4;
  typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

  {
    // thread t: row t / 8, channels 16 (t % 8) .. + 15 (two 8-channel groups)
    const int r = t >> 3, c0 = 16 * (t & 7);
    const int iq = min(i0 + r, Nb - 1);
    const float* qp = qbar + ((size_t)bh * Nb + iq) * kD + c0;
    bool bad = false;
    double n2 = 0.0;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const float4v u0 = *reinterpret_cast<const float4v*>(qp + 8 * hf);
      const float4v u1 = *reinterpret_cast<const float4v*>(qp + 8 * hf + 4);
      const float x[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
      bf16x8 h8, l8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bad |= out_of_range(x[e]);
        n2 += (double)x[e] * (double)x[e];
        __bf16 h, l;
        split_bf16(x[e], h, l);
        h8[e] = h;
        l8[e] = l;
      }
      const int c = c0 + 8 * hf, s = c >> 5, gg = (c >> 3) & 3, rt = r >> 4;
      unsigned char* dst = alds + ((rt * 4 + s) * 2) * 1024 + (16 * gg + (r & 15)) * 16;
      *(lds_bf16x8*)dst = h8;
      *(lds_bf16x8*)(dst + 1024) = l8;
    }
    // the row's eight threads are consecutive lanes
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
      n2 += __shfl_xor(n2, off);
      bad |= __shfl_xor(bad ? 1 : 0, off) != 0;
    }
    if ((t & 7) == 0) {
      qnorm[r] = next_up((float)sqrt(n2));  // an upper bound
      qflag[r] = bad ? 1u : 0u;
    }
  }
  __syncthreads();

  // B operands of tile t: 8 whole 16-byte loads per lane from the split layout
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(ksplit) + (size_t)bh * ntiles * kSplitTileElems, 0,
      ntiles * kSplitTileElems * 2, 0x00020000);
  float kmax = 0.0f;
  bool kbad = false;
  for (int tile = wave; tile < ntiles; tile += kSWaves) {
    v4i kv[8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
      kv[m] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                          sr, 16 * lane, (tile * kSplitTileElems + 512 * m) * 2, 0));
    const int j = 16 * tile + l16;
    if (j < Nb) {
      kbad |= kflag[(size_t)bh * Nb + j] != 0;
      kmax = fmaxf(kmax, knorm[(size_t)bh * Nb + j]);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      float4v acc = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const unsigned char* ap = alds + ((rt * 4 + s) * 2) * 1024 + 16 * lane;
        const bf16x8 ah = *(const lds_bf16x8*)ap;
        const bf16x8 al = *(const lds_bf16x8*)(ap + 1024);
        const bf16x8 bh8 = __builtin_bit_cast(bf16x8, kv[2 * s]);
        const bf16x8 bl8 = __builtin_bit_cast(bf16x8, kv[2 * s + 1]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh8, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl8, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh8, acc, 0, 0, 0);
      }
      // the lane holds rows 16 rt + 4g + r of key block j
      if (j < Nb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = i0 + 16 * rt + 4 * g + r;
          if (i < Nb) scores[((size_t)bh * Nb + i) * Nb + j] = acc[r];
        }
      }
    }
  }
  // per row and wave: |q_i| max |k_j| over the wave's key blocks (rounded
  // up), NaN when the row's means or any of those K means are out of range
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) kmax = fmaxf(kmax, __shfl_xor(kmax, off));
  const bool kbw = __builtin_amdgcn_ballot_w64(kbad) != 0;
  const int i = i0 + lane;
  if (i < Nb)
    amaxp[((size_t)bh * Nb + i) * kSWaves + wave] =
        (qflag[lane] || kbw) ? __builtin_nanf("") : next_up(qnorm[lane] * kmax);
}

// fp32 bounds of a window [lo, hi] given in fp64: for every fp32 x,
// lo <= x <= hi exactly when lo32 <= x <= hi32, and x > hi exactly when x > hi32.
__device__ __forceinline__ void window_f32(double lo, double hi, float& lo32, float& hi32) {
  lo32 = (float)lo;
  if ((double)lo32 < lo) lo32 = next_up(lo32);
  hi32 = (float)hi;
  if ((double)hi32 > hi) hi32 = -next_up(-hi32);
}

__global__ __launch_bounds__(64 * kBWaves) void block_topk_approx_select_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar_rm,
    const float* __restrict__ scores, const float* __restrict__ amaxp, int Nb, int k,
    int32_t* __restrict__ idx, uint32_t* __restrict__ mask, uint32_t* __restrict__ redo) {
  __shared__ uint32_t hist_all[kBWaves][kBins];
  __shared__ double cand_s_all[kBWaves][64];
  __shared__ int cand_j_all[kBWaves][64];
  const int t = threadIdx.x;
  // the wave index in a scalar register: the row and its q-bar are uniform
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int bh = blockIdx.y;
  const int i = blockIdx.x * kBWaves + wave;
  if (i >= Nb) return;  // no workgroup barrier in this kernel
  uint32_t* h = hist_all[wave];
  double* cs = cand_s_all[wave];
  int* cj = cand_j_all[wave];
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int mwords = (Nb + 31) / 32;
  const int nslots = (Nb + 63) >> 6;  // <= kFSlots
  const size_t row = (size_t)bh * Nb + i;
  int32_t* out = idx + row * k;
  uint32_t* mrow = mask ? mask + row * mwords : nullptr;
  if (k >= Nb) {  // every key block
    for (int j = lane; j < Nb; j += 64) out[j] = j;
    if (mrow)
      for (int w = lane; w < mwords; w += 64)
        mrow[w] = (w + 1) * 32 <= Nb ? 0xffffffffu : ((1u << (Nb - 32 * w)) - 1u);
    return;
  }
  // the row's approximate scores in registers (key block 64u + lane in slot u)
  const float* srow = scores + row * Nb;
  float v[kFSlots];
#pragma unroll
  for (int u = 0; u < kFSlots; ++u) {
    if (u >= nslots) continue;
    const int j = 64 * u + lane;
    v[u] = j < Nb ? srow[j] : 0.0f;
  }
  float am = lane < kSWaves ? amaxp[row * kSWaves + lane] : 0.0f;
  bool bad = __builtin_amdgcn_ballot_w64(am != am) != 0;  // a NaN partial: out of range
#pragma unroll
  for (int off = 1; off < kSWaves; off <<= 1) am = fmaxf(am, __shfl_xor(am, off));
  am = __shfl(am, 0);
  float mnf = INFINITY, mxf = -INFINITY;
#pragma unroll
  for (int u = 0; u < kFSlots; ++u) {
    if (u >= nslots) continue;
    if (64 * u + lane < Nb) {
      mnf = fminf(mnf, v[u]);
      mxf = fmaxf(mxf, v[u]);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mnf = fminf(mnf, __shfl_xor(mnf, off));
    mxf = fmaxf(mxf, __shfl_xor(mxf, off));
  }
  bad |= !(mxf > mnf);  // equal approximate scores: the exact kernel
  double T = 0.0;
  if (!bad) {
    // a monotone map of the scores onto the buckets (fp32 rounding keeps the
    // order, and the same map serves the histogram and the gather)
    float scale = (float)kBins / (mxf - mnf);
    if (!(scale < 1e30f)) scale = 1e30f;
    auto bucket = [&](float x) { return (int)fminf((x - mnf) * scale, (float)(kBins - 1)); };
#pragma unroll
    for (int q = 0; q < kBins / 64; ++q) h[lane * (kBins / 64) + q] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < kFSlots; ++u) {
      if (u >= nslots) continue;
      if (64 * u + lane < Nb) atomicAdd(&h[bucket(v[u])], 1u);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    __builtin_amdgcn_wave_barrier();
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
      const uint32_t x = __shfl_up(incl, off);
      if (lane >= off) incl += x;
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
    const int src = __ffsll((unsigned long long)__ballot(B >= 0)) - 1;
    B = __shfl(B, src);
    need = __shfl(need, src);
    nc = __shfl(nc, src);
    bad |= nc > 64;
    if (!bad) {
      // the need-th largest approximate score of bucket B (cs as scratch)
      uint32_t base = 0;
#pragma unroll
      for (int u = 0; u < kFSlots; ++u) {
        if (u >= nslots) continue;
        const bool in = 64 * u + lane < Nb && bucket(v[u]) == B;
        const uint64_t bb = __ballot(in);
        if (in) cs[base + (uint32_t)__popcll(bb & lt_mask)] = (double)v[u];
        base += (uint32_t)__popcll(bb);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
      __builtin_amdgcn_wave_barrier();
      bool mine = false;
      double my_s = 0.0;
      if ((uint32_t)lane < nc) {
        my_s = cs[lane];
        uint32_t rank = 0;
        for (uint32_t c = 0; c < nc; ++c)
          rank += (cs[c] > my_s || (cs[c] == my_s && c < (uint32_t)lane)) ? 1u : 0u;
        mine = rank == need - 1;
      }
      T = __shfl(my_s, __ffsll((unsigned long long)__ballot(mine)) - 1);
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
      __builtin_amdgcn_wave_barrier();  // cs is reused below
    }
  }
  // the window [T - 2E, T + 2E], widened so that its fp64 rounding stays outside
  const double E = 0x1p-12 * (double)am + 0x1p-100;
  float lo, hi;
  window_f32(T - 2.0 * E * (1.0 + 0x1p-30), T + 2.0 * E * (1.0 + 0x1p-30), lo, hi);
  uint32_t n_in = 0, n_amb = 0;
  if (!bad) {
#pragma unroll
    for (int u = 0; u < kFSlots; ++u) {
      if (u >= nslots) continue;
      const int j = 64 * u + lane;
      const float x = v[u];
      const bool amb = j < Nb && x >= lo && x <= hi;
      const uint64_t ba = __ballot(amb);
      const uint32_t pos = n_amb + (uint32_t)__popcll(ba & lt_mask);
      if (amb && pos < 64) cj[pos] = j;
      n_amb += (uint32_t)__popcll(ba);
      n_in += (uint32_t)__popcll(__ballot(j < Nb && x > hi));
    }
    // >= 1 and <= n_amb places for the listed ones by the bound
    bad |= n_amb > 64 || n_in >= (uint32_t)k || (uint32_t)k - n_in > n_amb;
  }
  if (bad) {
    if (lane == 0) redo[1 + atomicAdd(redo, 1u)] = (uint32_t)row;
    return;
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  __builtin_amdgcn_wave_barrier();
  // fp64 scores of the listed key blocks in block_topk_kernel's order
  // (channels ascending, one rounding per step), from the row-major k-bar:
  // a lane's 128 means in 16-byte loads, 32 channels in flight at a time
  const float* qr = qbar + row * kD;
  double my_s = 0.0;
  int my_j = 0;
  if ((uint32_t)lane < n_amb) {
    my_j = cj[lane];
    const float4v* kp = reinterpret_cast<const float4v*>(kbar_rm + ((size_t)bh * Nb + my_j) * kD);
    for (int c0 = 0; c0 < kD; c0 += 32) {
      float4v kv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) kv[e] = kp[c0 / 4 + e];
#pragma unroll
      for (int e = 0; e < 32; ++e) my_s = fma((double)qr[c0 + e], (double)kv[e >> 2][e & 3], my_s);
    }
    cs[lane] = my_s;
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  __builtin_amdgcn_wave_barrier();
  const uint32_t need = (uint32_t)k - n_in;
  bool mine = false;
  if ((uint32_t)lane < n_amb) {
    uint32_t rank = 0;
    for (uint32_t c = 0; c < n_amb; ++c)
      rank += (cs[c] > my_s || (cs[c] == my_s && cj[c] < my_j)) ? 1u : 0u;
    mine = rank == need - 1;
  }
  const int who = __ffsll((unsigned long long)__ballot(mine)) - 1;
  const double Ts = __shfl(my_s, who);
  const int Tj = __shfl(my_j, who);
  uint32_t base = 0, abase = 0;
#pragma unroll
  for (int u = 0; u < kFSlots; ++u) {
    if (u >= nslots) continue;
    const int jb = 64 * u;
    const int j = jb + lane;
    const bool valid = j < Nb;
    const float x = v[u];
    const bool amb = valid && x >= lo && x <= hi;
    const uint64_t ba = __ballot(amb);
    bool sel = valid && x > hi;
    if (amb) {
      const double ex = cs[abase + (uint32_t)__popcll(ba & lt_mask)];
      sel = ex > Ts || (ex == Ts && j <= Tj);
    }
    abase += (uint32_t)__popcll(ba);
    const uint64_t sb = __ballot(sel);
    const uint32_t pos = base + (uint32_t)__popcll(sb & lt_mask);
    if (sel && pos < (uint32_t)k) out[pos] = j;
    if (mrow) {
      const int w0 = jb >> 5;
      if (lane == 0) mrow[w0] = (uint32_t)sb;
      if (lane == 1 && w0 + 1 < mwords) mrow[w0 + 1] = (uint32_t)(sb >> 32);
    }
    base += (uint32_t)__popcll(sb);
  }
}

// ---------------------------------------------------------------------------
// Linear-branch staging.  A workgroup walks a contiguous chunk of key blocks
// of one (b,h).  For every block it
//   * writes V and phi(K)/16 as fp16 in the per-block layout
//     [channel][permuted key] that the attention kernel reads as matrix-core
//     operands (pad keys 0),
//   * writes the block's sum of phi(K)/16 over its keys (fp32, per channel),
//   * accumulates H = sum phi(K)^T V for the chunk (fp16 operands, fp32
//     accumulation, blocks in ascending order) and the chunk's sum of those
//     block sums in fp64,
//   * when k8 is set, writes the INT8 codes and scale of the smoothed block
//     K - mu (the quantiser's arithmetic, code_row8).
// Permuted key order inside each 32-key half: position 8g+s holds key
// 4g+s (s<4) or 16+4g+(s-4) (s>=4), matching the transposed score tiles
// that feed the P.V product.
// kMode: 0 = V staging only, 1 = V and phi(K) staging and block sums, 2 =
// staging plus the H, z partial sums.
// kF8 (lower-bit option): phi(K) is staged as FP8 e4m3 codes, [channel][64
// permuted keys] in 64-byte rows (8 KB per block), with one power-of-two
// scale per block: the block's largest feature m is scaled by 2^(7 - ilogb m)
// into [128, 256) and every feature is rounded to nearest-even e4m3;
// fkscale[block] = 2^(-(7 - ilogb m)) / 16 turns a code back into the fp16
// staging scale (phi/16).  The block sums, the H partials and the attention
// kernel all use the same decoded values.
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

template <int kMode, bool kF8>
__global__ __launch_bounds__(256) void linear_prep_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int N, int Nb, int phi,
    uint16_t* __restrict__ fk16, uint16_t* __restrict__ v16, float* __restrict__ zb,
    float* __restrict__ hpart, double* __restrict__ zpart, const float* __restrict__ mu,
    int8_t* __restrict__ k8, float* __restrict__ sk, float* __restrict__ fkscale) {
  // LDS: transposed tiles [128 channels][64 positions] fp16 (see tpos); with
  // kF8 also the codes, 16 words per channel, word w of channel c kept at
  // w ^ ((c >> 3) & 15) (the transposed writes of 16 channels 8 apart then
  // hit 16 banks)
  __shared__ __align__(16) _Float16 fkT[kD * kTRow];
  __shared__ __align__(16) _Float16 vT[kD * kTRow];
  __shared__ __align__(16) uint32_t fk8T[kF8 ? kD * 16 : 4];
  __shared__ float red[4];
  __shared__ float red8[4];
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
  double zacc = 0.0;
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
    float pf[4][8];     // kF8: phi(K) in fp32 (pad rows 0)
    float amax = 0.0f;  // max |K - mu| over this lane's valid rows
    float pmax = 0.0f;  // kF8: largest feature of this lane's valid rows
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r = 4 * a + m;
      float xv[8], xk[8];
      unpack_bf16x8(rv[m], xv);
      unpack_bf16x8(rk[m], xk);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        vv[m][e] = (_Float16)xv[e];
        if (kLinear && !kF8) fv[m][e] = (r < rows) ? (_Float16)(phi_apply(xk[e], phi) * kPhiScale) : (_Float16)0.0f;
        if (kF8) {
          pf[m][e] = (r < rows) ? phi_apply(xk[e], phi) : 0.0f;
          pmax = fmaxf(pmax, pf[m][e]);
        }
        if (quant && r < rows) amax = fmaxf(amax, fabsf(xk[e] - m8[e]));
      }
    }
    if (quant) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
      if (lane == 0) red[wave] = amax;
    }
    if (kF8) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) pmax = fmaxf(pmax, __shfl_xor(pmax, off));
      if (lane == 0) red8[wave] = pmax;
    }
    // transposed LDS writes: 4 consecutive keys -> 4 consecutive positions
    const int p0 = perm_pos(4 * a);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = cc * 8 + e;
      half4 hv = {vv[0][e], vv[1][e], vv[2][e], vv[3][e]};
      *reinterpret_cast<half4*>(&vT[tpos(c, p0)]) = hv;
      if (kLinear && !kF8) {
        half4 hf = {fv[0][e], fv[1][e], fv[2][e], fv[3][e]};
        *reinterpret_cast<half4*>(&fkT[tpos(c, p0)]) = hf;
      }
    }
    if constexpr (kF8) {
      __syncthreads();  // the block's largest feature is in red8
      const float bm = fmaxf(fmaxf(red8[0], red8[1]), fmaxf(red8[2], red8[3]));
      const int sh = bm > 0.0f ? 7 - ilogbf(bm) : 0;
      const float up = ldexpf(1.0f, sh);        // largest feature -> [128, 256)
      const float dq = ldexpf(1.0f, -sh - 4);   // code -> phi / 16
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = cc * 8 + e;
        uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(pf[0][e] * up, pf[1][e] * up, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(pf[2][e] * up, pf[3][e] * up, w, true);
        fk8T[c * 16 + ((p0 >> 2) ^ cc)] = w;
        const half2v lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, dq, false);
        const half2v hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, dq, true);
        half4 hf = {lo.x, lo.y, hi.x, hi.y};
        *reinterpret_cast<half4*>(&fkT[tpos(c, p0)]) = hf;
      }
      if (t == 0) fkscale[(size_t)bh * Nb + j] = dq;
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
        if (kLinear && !kF8) dstf[q] = *reinterpret_cast<const uint4*>(&fkT[tpos(q >> 3, 8 * (q & 7))]);
      }
      if (kF8) {
        // codes: 8 KB per block, 16-byte chunk q = 4c + k in linear order; a
        // head's blocks start at its fp16 staging slice (the first half of it)
        uint4* dst8 = reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(fk16 + (size_t)bh * Nb * kD * kBlk) +
                                               (size_t)j * kD * kBlk);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int q = t + 256 * m;
          const int r = q >> 2, sw = (r >> 3) & 15;
          // words 4k..4k+3 of row r sit at (4k + i) ^ sw
          const uint4 u = reinterpret_cast<const uint4*>(fk8T)[r * 4 + ((q & 3) ^ (sw >> 2))];
          uint32_t w[4] = {u.x, u.y, u.z, u.w};
          if (sw & 1) {
            const uint32_t t0 = w[0], t2 = w[2];
            w[0] = w[1], w[1] = t0, w[2] = w[3], w[3] = t2;
          }
          if (sw & 2) {
            const uint32_t t0 = w[0], t1 = w[1];
            w[0] = w[2], w[1] = w[3], w[2] = t0, w[3] = t1;
          }
          dst8[q] = make_uint4(w[0], w[1], w[2], w[3]);
        }
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
      if (kReduce) zacc += (double)zj;
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

// Position of H[c][d] (c: phi channel, d: value channel) in the attention
// kernel's M^T register layout: wave w = c / 32 holds phi channels 32w + 16x +
// l16 of value rows 16dt + 4g + r in lane 16g + l16, register (dt, x, r).
__device__ __forceinline__ int h_frag_index(int c, int d) {
  const int w = c >> 5, x = (c >> 4) & 1, l16 = c & 15;
  const int dt = d >> 4, g = (d >> 2) & 3, r = d & 3;
  return ((((w * 8 + dt) * 2 + x) * 64 + 16 * g + l16) << 2) + r;
}

// Whole-head linear state, step 1: H as the chunk partials added in chunk
// order, and the fp64 sum of the chunk sums of the block sums zb.  Workgroup
// (bh, y) owns H elements [1024y, 1024y + 1024) and writes the sum over chunk
// 0's slot (it alone reads and writes that range) and, with hf set, into the
// fragment layout.
__global__ __launch_bounds__(256) void linear_sum_kernel(float* __restrict__ hpart,
                                                         const double* __restrict__ zpart,
                                                         float* __restrict__ hf,
                                                         double* __restrict__ z64,
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
    if (hf) hf[(size_t)bh * kD * kD + h_frag_index(e >> 7, e & 127)] = s;
  }
  if (blockIdx.y == 0 && t < kD) {
    double v[kLinChunks];
#pragma unroll
    for (int c = 0; c < kLinChunks; ++c) v[c] = zpart[((size_t)bh * kLinChunks + c) * kD + t];
    double s = 0.0;
#pragma unroll
    for (int c = 0; c < kLinChunks; ++c) s += v[c];
    if (z64) z64[(size_t)bh * kD + t] = s;
    if (z) z[(size_t)bh * kD + t] = (float)s;
  }
}

// Step 2 (backward): store H^T as fp16 scaled by 2^-s so that max|H| * 2^-s
// lies in [2^14, 2^15), plus 2^s; with hb set, also H itself (row-major,
// unscaled) as bf16.
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
  if (t == 0 && hscale) hscale[bh] = ldexpf(1.0f, s);
  if (h16t) {
    _Float16* out = reinterpret_cast<_Float16*>(h16t) + (size_t)bh * kD * kD;
#pragma unroll
    for (int m = 0; m < 64; ++m) {
      const int e = t + 256 * m;     // H[c][o] with c = e / 128, o = e % 128
      const int c = e >> 7, o = e & 127;
      out[(size_t)o * kD + c] = (_Float16)(hv[m] * down);
    }
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
                              uint16_t* ksplit, uint8_t* kflag, float* kbar_rm, float* knorm,
                              hipStream_t s) {
  dim3 grid(sh.Nb, sh.BH);
  block_stats_kernel<<<grid, 256, 0, s>>>(q, k, sh.N, sh.Nb, ksum, qbar, kbar, q8, sq, ksplit, kflag,
                                          kbar_rm, knorm);
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

// LDS bytes of block_topk_kernel<R>.
static size_t topk_bytes(int Nb, int R) {
  return (size_t)R * Nb * 8 + (size_t)R * kD * 8 + 4 * kBins * 4 + 4 * 64 * 12;
}

size_t topk_lds_bytes(int Nb, int* rows_per_group) {
  int R = 8;
  while (R > 1 && topk_bytes(Nb, R) > 96 * 1024) R >>= 1;
  if (rows_per_group) *rows_per_group = R;
  return topk_bytes(Nb, R);
}

// Bytes of the filtered top-k's approximate scores and row maxima, 0 where
// it does not run (rows too long for its registers).
size_t topk_filter_bytes(int BH, int Nb) {
  if (Nb > 64 * kFSlots) return 0;
  return (size_t)BH * Nb * ((size_t)Nb + kSWaves) * 4;
}

static bool filter_applies(const TopkFilter& f, const Shape& sh) {
  return f.scores && f.ksplit && f.kflag && f.kbar_rm && f.knorm && f.redo && sh.Nb <= 64 * kFSlots;
}

hipError_t launch_block_topk_first(const float* qbar, const float* kbar, const TopkFilter& f,
                                   const Shape& sh, int32_t* idx, uint32_t* mask, hipStream_t s,
                                   const uint32_t** handed_back) {
  *handed_back = nullptr;
  if (filter_applies(f, sh)) {
    float* amaxp = f.scores + (size_t)sh.BH * sh.Nb * sh.Nb;
    block_scores_approx_kernel<<<dim3((sh.Nb + kSRows - 1) / kSRows, sh.BH), 64 * kSWaves, 0, s>>>(
        qbar, f.ksplit, f.kflag, f.knorm, sh.Nb, f.scores, amaxp, f.redo);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    block_topk_approx_select_kernel<<<dim3((sh.Nb + kBWaves - 1) / kBWaves, sh.BH), 64 * kBWaves, 0, s>>>(
        qbar, f.kbar_rm, f.scores, amaxp, sh.Nb, sh.k, idx, mask, f.redo);
    e = hipGetLastError();
    if (e == hipSuccess) *handed_back = f.redo;
    return e;
  }
  int R = 1;
  const size_t lds = topk_lds_bytes(sh.Nb, &R);
  const void* fn = R == 8   ? reinterpret_cast<const void*>(block_topk_kernel<8>)
                   : R == 4 ? reinterpret_cast<const void*>(block_topk_kernel<4>)
                   : R == 2 ? reinterpret_cast<const void*>(block_topk_kernel<2>)
                            : reinterpret_cast<const void*>(block_topk_kernel<1>);
  const hipError_t e = allow_lds(fn, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((sh.Nb + R - 1) / R, sh.BH);
  switch (R) {
    case 8: block_topk_kernel<8><<<grid, 256, lds, s>>>(qbar, kbar, sh.Nb, sh.k, idx, mask, nullptr); break;
    case 4: block_topk_kernel<4><<<grid, 256, lds, s>>>(qbar, kbar, sh.Nb, sh.k, idx, mask, nullptr); break;
    case 2: block_topk_kernel<2><<<grid, 256, lds, s>>>(qbar, kbar, sh.Nb, sh.k, idx, mask, nullptr); break;
    default: block_topk_kernel<1><<<grid, 256, lds, s>>>(qbar, kbar, sh.Nb, sh.k, idx, mask, nullptr); break;
  }
  return hipGetLastError();
}

hipError_t launch_block_topk_redo(const float* qbar, const float* kbar, const TopkFilter& f,
                                  const Shape& sh, int32_t* idx, uint32_t* mask, hipStream_t s) {
  const size_t lds1 = topk_bytes(sh.Nb, 1);
  const hipError_t e = allow_lds(reinterpret_cast<const void*>(block_topk_kernel<1>), (int)lds1);
  if (e != hipSuccess) return e;
  block_topk_kernel<1><<<kRedoGrid, 256, lds1, s>>>(qbar, kbar, sh.Nb, sh.k, idx, mask, f.redo);
  return hipGetLastError();
}

hipError_t launch_block_topk(const float* qbar, const float* kbar, const TopkFilter& f,
                             const Shape& sh, int32_t* idx, uint32_t* mask, hipStream_t s) {
  const uint32_t* list = nullptr;
  const hipError_t e = launch_block_topk_first(qbar, kbar, f, sh, idx, mask, s, &list);
  if (e != hipSuccess || !list) return e;
  return launch_block_topk_redo(qbar, kbar, f, sh, idx, mask, s);
}

hipError_t launch_linear_prep(const uint16_t* k, const uint16_t* v, const Shape& sh, int phi,
                              bool reduce, uint16_t* fk16, uint16_t* v16, float* zb, float* hpart,
                              double* zpart, const float* mu, int8_t* k8, float* sk, bool fp8,
                              float* fkscale, hipStream_t s) {
  dim3 grid(kLinChunks, sh.BH);
#define SLA_PREP(M, F8)                                                                         \
  linear_prep_kernel<M, F8><<<grid, 256, 0, s>>>(k, v, sh.N, sh.Nb, phi, fk16, v16, zb, hpart, \
                                                 zpart, mu, k8, sk, fkscale)
  if (phi == kPhiNone)
    SLA_PREP(0, false);
  else if (!reduce)
    fp8 ? SLA_PREP(1, true) : SLA_PREP(1, false);
  else
    fp8 ? SLA_PREP(2, true) : SLA_PREP(2, false);
#undef SLA_PREP
  return hipGetLastError();
}

hipError_t launch_linear_final(float* hpart, const double* zpart, const Shape& sh, float* hf,
                               double* z64, float* z, uint16_t* h16t, float* hscale,
                               uint16_t* hb, hipStream_t s) {
  linear_sum_kernel<<<dim3(sh.BH, kD * kD / 1024), 256, 0, s>>>(hpart, zpart, hf, z64, z);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (!h16t && !hb)) return e;
  linear_cvt_kernel<<<sh.BH, 256, 0, s>>>(hpart, h16t, hscale, hb);
  return hipGetLastError();
}

}  // namespace sla
