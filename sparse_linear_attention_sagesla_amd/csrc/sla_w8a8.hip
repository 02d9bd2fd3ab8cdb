// W8A8 INT8 linear layers and FusedNorm for gfx950 (CDNA4).
//
// Weights and activations are quantised to 8 bits to run the linear layers on
// the INT8 units (news summary, opening component list; commentary, section
// "步数蒸馏与W8A8量化"), with a fused normalisation operator in front
// (blog, section "1. 计算资源优化：CPU Offload与混合精度计算").
//
//   rowquant_kernel<norm>  one wave per row: per-row INT8 codes and scale of
//                          a bf16 matrix (weights per output channel, or plain
//                          activations per token); with `norm`, the row is first
//                          LayerNorm-ed (fp64 mean and variance, fp32 steps as
//                          fixed below) and optionally scaled and shifted per
//                          channel (the FusedNorm).
//   w8a8_gemm_kernel       y[m][n] = (sum_k x8[m][k] w8[n][k]) * sx[m] * sw[n] + b[n]:
//                          256 x 256 output tile per workgroup (eight waves of
//                          128 x 64, two per SIMD), K in steps of 128 through two LDS stages
//                          filled by direct global->LDS loads, 32x32x32 INT8
//                          MFMA with int32 accumulation, XCD-grouped tile order.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "sla_internal.h"
#include "sla_quant.h"

namespace sla {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_byte;
typedef __attribute__((address_space(3))) const v4i lds_v4i;

constexpr int kRowWaves = 4;                   // rows per workgroup (one wave each)
constexpr int kRowChunks = kMaxRowK / (8 * 64); // 8-value chunks per lane, longest rows

// ---------------------------------------------------------------------------
// Per-row quantiser / FusedNorm: one wave per row.  Lane l holds the 8-value
// chunks 8 (l + 64 c) .. + 7 of the row as packed bf16 (c < kC, the kernel
// is instantiated for a few chunk counts so short rows need few registers) and
// unpacks them in each pass: the sums, the normalised maximum, the codes.
// LayerNorm: mu = fp32(sum_k x / K) with the sum in fp64; var = (sum_k
// (x - mu)^2) / K in fp64 (x - mu exact in fp64, squares accumulated by fma);
// each lane keeps four partial sums (element e of a chunk into sum e % 4) so
// the fp64 additions do not form one long dependent chain.
// rstd = fp32(1 / sqrt(var + eps)) in fp64; then, in fp32 and in this order,
// t = x - mu, t = t * rstd, t = t * gamma, t = t + beta (gamma, beta optional).
// ---------------------------------------------------------------------------
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

typedef __attribute__((address_space(3))) const v4f lds_v4f;

// gamma (1 where absent) and beta (0 where absent) staged in LDS: lds_g[k],
// lds_g[K + k].  Multiplying by 1 and adding 0 change no code: t * 1 = t, and
// t + 0 differs from t only for t = -0, whose code is 0 either way.
template <bool kNorm, bool kAffine>
__device__ __forceinline__ void norm_chunk(const uint4& u, int k0, int K, float mu, float rstd,
                                           const __attribute__((address_space(3))) float* lds_g,
                                           float* y) {
  unpack_bf16x8(u, y);
  if (kNorm) {
    v4f g[2], b[2];
    if (kAffine) {
      g[0] = *(lds_v4f*)(lds_g + k0);
      g[1] = *(lds_v4f*)(lds_g + k0 + 4);
      b[0] = *(lds_v4f*)(lds_g + K + k0);
      b[1] = *(lds_v4f*)(lds_g + K + k0 + 4);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float t = y[e] - mu;
      t = t * rstd;
      if (kAffine) {
        t = t * g[e >> 2][e & 3];
        t = t + b[e >> 2][e & 3];
      }
      y[e] = t;
    }
  }
}

// Tells the compiler the packed row may have changed, so that each pass
// unpacks it again instead of keeping every converted value alive across
// passes (which does not fit in registers).
template <int kC>
__device__ __forceinline__ void launder(uint4 (&u)[kC]) {
#pragma unroll
  for (int c = 0; c < kC; ++c) asm volatile("" : "+v"(u[c].x), "+v"(u[c].y), "+v"(u[c].z), "+v"(u[c].w));
}

// One row's chunks, as packed bf16: buffer loads over the row's K values, which
// return zero past its end, so every load is issued unconditionally and all of
// them are in flight together.
template <int kC>
__device__ __forceinline__ void load_row(const uint16_t* __restrict__ xr, int K, int lane,
                                         uint4 (&u)[kC]) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(xr), 0, 2 * K, 0x00020000);
#pragma unroll
  for (int c = 0; c < kC; ++c)
    u[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, 16 * (lane + 64 * c), 0, 0));
}

template <bool kNorm, bool kAffine, int kC>
__device__ __forceinline__ void quant_row(uint4 (&u)[kC], size_t row, int K, int lane,
                                          const __attribute__((address_space(3))) float* lds_g,
                                          float eps,
                                          int8_t* __restrict__ codes, float* __restrict__ scale,
                                          float* __restrict__ mu_out, float* __restrict__ rstd_out) {
  float mu = 0.0f, rstd = 1.0f;
  if (kNorm) {
    double s[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      float v[8];
      unpack_bf16x8(u[c], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e & 3] += (double)v[e];
    }
    mu = (float)(wave_sum_f64((s[0] + s[1]) + (s[2] + s[3])) / (double)K);
    launder(u);
    double q[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      if (8 * (lane + 64 * c) < K) {
        float v[8];
        unpack_bf16x8(u[c], v);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double d = (double)v[e] - (double)mu;
          q[e & 3] = __builtin_fma(d, d, q[e & 3]);
        }
      }
    }
    rstd = (float)(1.0 / sqrt(wave_sum_f64((q[0] + q[1]) + (q[2] + q[3])) / (double)K + (double)eps));
    launder(u);
    if (lane == 0) {
      if (mu_out) mu_out[row] = mu;
      if (rstd_out) rstd_out[row] = rstd;
    }
  }
  float a = 0.0f;
#pragma unroll
  for (int c = 0; c < kC; ++c) {
    const int k0 = 8 * (lane + 64 * c);
    if (k0 < K) {
      float y[8];
      norm_chunk<kNorm, kAffine>(u[c], k0, K, mu, rstd, lds_g, y);
#pragma unroll
      for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(y[e]));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  float sc, inv;
  const bool live = code_scale(a, sc, inv);
  launder(u);
  int8_t* cr = codes + row * (size_t)K;
#pragma unroll
  for (int c = 0; c < kC; ++c) {
    const int k0 = 8 * (lane + 64 * c);
    if (k0 < K) {
      float y[8];
      norm_chunk<kNorm, kAffine>(u[c], k0, K, mu, rstd, lds_g, y);
      *reinterpret_cast<uint2*>(cr + k0) = code_row8(y, inv, live);
    }
  }
  if (lane == 0) scale[row] = sc;
}

// One wave per row.
template <bool kNorm, bool kAffine, int kC>
__global__ __launch_bounds__(64 * kRowWaves) void rowquant_kernel(
    const uint16_t* __restrict__ x, int rows, int K, const float* __restrict__ gamma,
    const float* __restrict__ beta, float eps, int8_t* __restrict__ codes,
    float* __restrict__ scale, float* __restrict__ mu_out, float* __restrict__ rstd_out) {
  extern __shared__ float rq_lds[];
  const auto lds_g = (const __attribute__((address_space(3))) float*)rq_lds;
  const int lane = threadIdx.x & 63;
  if (kAffine) {
    for (int k = threadIdx.x; k < K; k += 64 * kRowWaves) {
      rq_lds[k] = gamma ? gamma[k] : 1.0f;
      rq_lds[K + k] = beta ? beta[k] : 0.0f;
    }
    __syncthreads();
  }
  // the row index as a scalar, so the row's buffer descriptor is one too
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const size_t row = (size_t)blockIdx.x * kRowWaves + wave;
  if (row >= (size_t)rows) return;
  uint4 u[kC];
  load_row(x + row * (size_t)K, K, lane, u);
  quant_row<kNorm, kAffine>(u, row, K, lane, lds_g, eps, codes, scale, mu_out, rstd_out);
}

// ---------------------------------------------------------------------------
// INT8 GEMM.  C tile [n][m] = W8 rows (A operand) x X8 rows (B operand): the
// 32x32 accumulator of a lane holds column m = lane & 31 and rows
// n = 8j + 4 (lane >> 5) + i (j, i < 4), i.e. four consecutive output
// channels of one token, stored as one 8- or 16-byte write.
// LDS stage: A rows (256 x 128 bytes), then B rows; 16-byte chunk c of row r
// kept at c ^ ((r >> 1) & 7), so the 16 rows a quarter-wave reads at one chunk
// cover all 64 banks.
// ---------------------------------------------------------------------------
constexpr int kGT = 256;                 // output tile edge (n and m)
constexpr int kGK = 128;                 // K per stage
constexpr int kGStageHalf = kGT * kGK;   // 32 KB: one operand's stage
constexpr int kGStage = 2 * kGStageHalf; // 64 KB
constexpr int kGStages = 2;
constexpr int kGWaves = 8;               // two per SIMD
constexpr int kGOutRow = 2 * 128 + 16;   // LDS row of a wave's bf16 output (padded)
constexpr int kGOutWave = 64 * kGOutRow; // a wave's 64 x 128 output in LDS
constexpr int kGLds = kGStages * kGStage > kGWaves * kGOutWave ? kGStages * kGStage : kGWaves * kGOutWave;
constexpr int kGScaleOff = kGLds;               // the tile's w scales, x scales, bias (1 KB each)
constexpr int kGLdsTotal = kGLds + 3 * 1024;
constexpr int kGroupM = 8;               // m tiles per group of the tile order

struct GemmArgs {
  const int8_t* x8;   // [M, K]
  const float* sx;    // [M]
  const int8_t* w8;   // [N, K]
  const float* sw;    // [N]
  const float* bias;  // [N] or null
  void* y;            // [M, N] bf16 or fp32
  int M, N, K;
  int Mt, Nt;         // tile counts
  int per_xcd;        // tiles per XCD slot range
  int out_f32;
};

__device__ __forceinline__ void gemm_load(__amdgpu_buffer_rsrc_t r, int voff, int soff, lds_byte* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3)))*)dst, 16, voff,
                                           soff, 0, 0);
}

__device__ __forceinline__ void gemm_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__global__ __launch_bounds__(64 * kGWaves, 1) void w8a8_gemm_kernel(GemmArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  lds_byte* smem = (lds_byte*)smem_raw;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  // XCD-grouped tile order: workgroup x runs on XCD x % 8; each XCD takes a
  // contiguous range of the grouped order (kGroupM m tiles x all n tiles,
  // m fastest), so the tiles it runs together share operand rows in its L2
  const int x = blockIdx.x;
  const int tid = (x & 7) * a.per_xcd + (x >> 3);
  if (tid >= a.Mt * a.Nt) return;
  const int group = tid / (kGroupM * a.Nt);
  const int first_m = group * kGroupM;
  const int gsize = min(a.Mt - first_m, kGroupM);
  const int in_group = tid % (kGroupM * a.Nt);
  const int mt = first_m + in_group % gsize;
  const int nt = in_group / gsize;
  const int m0 = mt * kGT, n0 = nt * kGT;

  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(a.w8 + (size_t)n0 * a.K), 0, (int)min((size_t)(a.N - n0) * a.K, (size_t)0x7fffffff), 0x00020000);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(a.x8 + (size_t)m0 * a.K), 0, (int)min((size_t)(a.M - m0) * a.K, (size_t)0x7fffffff), 0x00020000);
  // this lane's load offsets: instruction i of wave w fills rows 8(4w + i) +
  // lane/8 (1 KB), stored chunk lane % 8, fetched chunk (lane % 8) ^ ((row >> 1) & 7)
  int voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * (4 * wave + i) + (lane >> 3);
    voff[i] = row * a.K + 16 * ((lane & 7) ^ ((row >> 1) & 7));
  }
  auto issue = [&](lds_byte* st, int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) gemm_load(rw, voff[i], k0, st + 1024 * (4 * wave + i));
#pragma unroll
    for (int i = 0; i < 4; ++i) gemm_load(rx, voff[i], k0, st + kGStageHalf + 1024 * (4 * wave + i));
  };

  // the epilogue's scales and bias for this tile go to LDS with the first stage,
  // so it reads them there instead of waiting on memory (entries past N or M
  // read as zero)
  {
    auto scale_rsrc = [](const float* p, int count) {
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0, 4 * min(count, kGT), 0x00020000);
    };
    if (wave == 0) gemm_load(scale_rsrc(a.sw + n0, a.N - n0), 16 * lane, 0, smem + kGScaleOff);
    if (wave == 1) gemm_load(scale_rsrc(a.sx + m0, a.M - m0), 16 * lane, 0, smem + kGScaleOff + 1024);
    if (wave == 2 && a.bias) gemm_load(scale_rsrc(a.bias + n0, a.N - n0), 16 * lane, 0, smem + kGScaleOff + 2048);
  }

  // wave w: output rows n in [128 (w & 1), +128), columns m in [64 (w >> 1), +64)
  const int wn = 128 * (wave & 1), wm = 64 * (wave >> 1);
  const int r32 = lane & 31, khalf = lane >> 5;
  v16i acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16i{};

  auto compute = [&](const lds_byte* st) {
#pragma unroll
    for (int kk = 0; kk < kGK / 32; ++kk) {
      const int c = khalf + 2 * kk;
      v4i af[4], bf[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rn = wn + 32 * i + r32;
        af[i] = *(lds_v4i*)(st + rn * kGK + ((c ^ ((rn >> 1) & 7)) << 4));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int rm = wm + 32 * j + r32;
        bf[j] = *(lds_v4i*)(st + kGStageHalf + rm * kGK + ((c ^ ((rm >> 1) & 7)) << 4));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };

  const int steps = a.K / kGK;  // K is a multiple of 128
  issue(smem, 0);
  // unrolled by the stage count so every stage address is a constant offset
  for (int p0 = 0; p0 < steps; p0 += kGStages) {
#pragma unroll
    for (int ph = 0; ph < kGStages; ++ph) {
      const int p = p0 + ph;
      if (p < steps) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        gemm_barrier();  // stage p is in; every wave is done with stage p-1
        if (p + 1 < steps) issue(smem + ((ph + 1) % kGStages) * kGStage, (p + 1) * kGK);
        compute(smem + ph * kGStage);
      }
    }
  }

  // epilogue: y = acc * sx[m] * sw[n] + bias[n].  bf16 output goes through
  // LDS (each wave's 64 tokens x 128 channels as rows) so that the stores are
  // whole 256-byte row segments; fp32 output is stored from the registers.
  gemm_barrier();  // every wave is done with the stages
  lds_byte* my = smem + wave * kGOutWave;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = m0 + wm + 32 * j + r32;
    typedef __attribute__((address_space(3))) const float lds_f;
    const float sxm = *(lds_f*)(smem + kGScaleOff + 1024 + 4 * (wm + 32 * j + r32));  // 0 past M
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = 32 * i + 8 * q + 4 * khalf;  // channel within the wave's 128
        const int n = n0 + wn + nl;
        v4f yv = v4f{0.f, 0.f, 0.f, 0.f};
        if (n < a.N) {
          const v4f swv = *(lds_v4f*)(smem + kGScaleOff + 4 * (wn + nl));
#pragma unroll
          for (int e = 0; e < 4; ++e) yv[e] = (float)acc[i][j][4 * q + e] * sxm * swv[e];
          if (a.bias) yv += *(lds_v4f*)(smem + kGScaleOff + 2048 + 4 * (wn + nl));
        }
        if (a.out_f32) {
          if (m < a.M && n < a.N)
            *reinterpret_cast<v4f*>(reinterpret_cast<float*>(a.y) + (size_t)m * a.N + n) = yv;
        } else {
          uint32_t w[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t b0 = __float_as_uint(yv[2 * h]);
            const uint32_t b1 = __float_as_uint(yv[2 * h + 1]);
            const uint32_t r0 = (b0 + 0x7fffu + ((b0 >> 16) & 1u)) >> 16;
            const uint32_t r1 = (b1 + 0x7fffu + ((b1 >> 16) & 1u)) >> 16;
            w[h] = r0 | (r1 << 16);
          }
          typedef unsigned int v2u __attribute__((ext_vector_type(2)));
          *(__attribute__((address_space(3))) v2u*)(my + (32 * j + r32) * kGOutRow + 2 * nl) =
              v2u{w[0], w[1]};
        }
      }
    }
  }
  if (!a.out_f32) {
    // this wave's rows back out: 16 lanes x 16 bytes per row, four rows per step
    // (the wave reads only what it wrote, so no workgroup barrier is needed)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int cl = lane & 15;
    const int n = n0 + wn + 8 * cl;
#pragma unroll
    for (int s4 = 0; s4 < 16; ++s4) {
      const int r = 4 * s4 + (lane >> 4);
      const int m = m0 + wm + r;
      const v4i v = *(lds_v4i*)(my + r * kGOutRow + 16 * cl);
      if (m < a.M) {
        uint16_t* dst = reinterpret_cast<uint16_t*>(a.y) + (size_t)m * a.N + n;
        if (n + 8 <= a.N)
          *reinterpret_cast<v4i*>(dst) = v;
        else if (n < a.N)
          *reinterpret_cast<uint2*>(dst) = make_uint2((uint32_t)v[0], (uint32_t)v[1]);
      }
    }
  }
}

}  // namespace

hipError_t launch_rowquant(const uint16_t* x, int rows, int K, bool norm, const float* gamma,
                           const float* beta, float eps, int8_t* codes, float* scale, float* mu,
                           float* rstd, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int blocks = (rows + kRowWaves - 1) / kRowWaves;
  const int chunks = (K + 511) / 512;  // 8-value chunks per lane
  const size_t affine_lds = 8 * (size_t)K;  // gamma and beta as fp32
  auto go = [&](auto kc) -> hipError_t {
    constexpr int C = decltype(kc)::value;
    if (norm && (gamma || beta)) {
      const hipError_t e = allow_lds(reinterpret_cast<const void*>(rowquant_kernel<true, true, C>),
                                     (int)affine_lds);
      if (e != hipSuccess) return e;
      rowquant_kernel<true, true, C><<<blocks, 64 * kRowWaves, affine_lds, s>>>(
          x, rows, K, gamma, beta, eps, codes, scale, mu, rstd);
    } else if (norm) {
      rowquant_kernel<true, false, C><<<blocks, 64 * kRowWaves, 0, s>>>(
          x, rows, K, nullptr, nullptr, eps, codes, scale, mu, rstd);
    } else {
      rowquant_kernel<false, false, C><<<blocks, 64 * kRowWaves, 0, s>>>(
          x, rows, K, nullptr, nullptr, 0.0f, codes, scale, nullptr, nullptr);
    }
    return hipSuccess;
  };
  hipError_t e;
  if (chunks <= 2) e = go(std::integral_constant<int, 2>());
  else if (chunks <= 4) e = go(std::integral_constant<int, 4>());
  else if (chunks <= 8) e = go(std::integral_constant<int, 8>());
  else if (chunks <= 10) e = go(std::integral_constant<int, 10>());
  else if (chunks <= 16) e = go(std::integral_constant<int, 16>());
  else if (chunks <= 24) e = go(std::integral_constant<int, 24>());
  else e = go(std::integral_constant<int, kRowChunks>());
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t launch_w8a8_gemm(const int8_t* x8, const float* sx, const int8_t* w8, const float* sw,
                            const float* bias, int M, int N, int K, void* y, int out_f32,
                            hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  GemmArgs a;
  a.x8 = x8;
  a.sx = sx;
  a.w8 = w8;
  a.sw = sw;
  a.bias = bias;
  a.y = y;
  a.M = M;
  a.N = N;
  a.K = K;
  a.Mt = (M + kGT - 1) / kGT;
  a.Nt = (N + kGT - 1) / kGT;
  const int tiles = a.Mt * a.Nt;
  a.per_xcd = (tiles + 7) / 8;
  a.out_f32 = out_f32;
  const hipError_t e = allow_lds(reinterpret_cast<const void*>(w8a8_gemm_kernel), kGLdsTotal);
  if (e != hipSuccess) return e;
  w8a8_gemm_kernel<<<8 * a.per_xcd, 64 * kGWaves, kGLdsTotal, s>>>(a);
  return hipGetLastError();
}

}  // namespace sla
