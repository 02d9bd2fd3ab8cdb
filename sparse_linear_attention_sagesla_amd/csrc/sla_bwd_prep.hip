// Staging kernels of the SageSLA backward for gfx950: per-block transposes,
// the column lists (for every key block, the query blocks that keep it) and
// the whole-head linear-gradient sums G and g_z.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "sla_internal.h"

namespace sla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Position of row t of a block in the permuted order of the transposed tiles:
// inside each 32-row half, rows 4g..4g+3 go to 8g.. and rows 16+4g.. to 8g+4..
// (the order in which a score tile's rows meet the matrix-core k slots).
__device__ __forceinline__ int perm_row(int t) {
  const int r = t & 31;
  return 32 * (t >> 5) + 8 * ((r & 15) >> 2) + (r & 3) + 4 * (r >> 4);
}

// Row held at permuted position p (inverse of perm_row).
__device__ __forceinline__ int row_at(int p) {
  const int h = p >> 5, q = p & 31;
  return 32 * h + 16 * ((q >> 2) & 1) + 4 * (q >> 3) + (q & 3);
}

// x [BH, N, 128] bf16 rows -> out [BH, Nb, 128, 64] bf16, out[c][p] =
// x[64 blk + row_at(p)][c], rows past N as 0.  blockIdx.z picks the tensor.
constexpr int kTPitch = 136;  // LDS row pitch in bf16 (272 bytes)

__global__ __launch_bounds__(256) void transpose_blocks_kernel(const uint16_t* __restrict__ x0,
                                                               const uint16_t* __restrict__ x1,
                                                               uint16_t* __restrict__ o0,
                                                               uint16_t* __restrict__ o1, int N,
                                                               int Nb) {
  __shared__ __align__(16) uint16_t tile[kBlk * kTPitch];
  const uint16_t* x = blockIdx.z == 0 ? x0 : x1;
  uint16_t* o = blockIdx.z == 0 ? o0 : o1;
  if (!x || !o) return;
  const int t = threadIdx.x;
  const int blk = blockIdx.x;
  const size_t bh = blockIdx.y;
  const uint16_t* src = x + ((size_t)bh * N + (size_t)blk * kBlk) * kD;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int q = t + 256 * m;  // 16-byte chunk: row q / 16, channels 8 (q % 16)..
    const int row = q >> 4, c8 = (q & 15) * 8;
    uint4 w = make_uint4(0, 0, 0, 0);
    if (blk * kBlk + row < N) w = *reinterpret_cast<const uint4*>(src + (size_t)row * kD + c8);
    *reinterpret_cast<uint4*>(tile + row * kTPitch + c8) = w;
  }
  __syncthreads();
  uint16_t* dst = o + ((size_t)bh * Nb + blk) * (kD * kBlk);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int q = t + 256 * m;  // output chunk: channel q / 8, positions 8 (q % 8)..
    const int c = q >> 3, p0 = (q & 7) * 8;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = tile[row_at(p0 + 2 * e) * kTPitch + c];
      const uint32_t hi = tile[row_at(p0 + 2 * e + 1) * kTPitch + c];
      w[e] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4*>(dst + (size_t)c * kBlk + p0) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* __restrict__ p, size_t n) {
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256) p[e] = 0u;
}

// Bit i of maskT[bh][j] row is set when query block i keeps key block j.
__global__ __launch_bounds__(256) void column_mark_kernel(const int32_t* __restrict__ idx, int Nb,
                                                          int k, int W, size_t total,
                                                          uint32_t* __restrict__ maskT) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const size_t row = e / (size_t)k;  // bh * Nb + i
  const int i = (int)(row % (size_t)Nb);
  const size_t bh = row / (size_t)Nb;
  const int j = idx[e];
  if (j < 0 || j >= Nb) return;
  atomicOr(&maskT[(bh * Nb + j) * (size_t)W + (i >> 5)], 1u << (i & 31));
}

// Column starts: coff[bh][j] = number of (i, j') with j' < j, coff[bh][Nb] = total.
// One workgroup of 1024 threads per head; thread t counts columns
// [t * per, t * per + per).
__global__ __launch_bounds__(1024) void column_offsets_kernel(const uint32_t* __restrict__ maskT,
                                                              int Nb, int W,
                                                              int32_t* __restrict__ coff) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const size_t bh = blockIdx.x;
  const int per = (Nb + 1023) / 1024;
  int cnt = 0;
  for (int j = t * per; j < min(Nb, t * per + per); ++j) {
    const uint32_t* row = maskT + (bh * Nb + j) * (size_t)W;
    for (int w = 0; w < W; ++w) cnt += __popc(row[w]);
  }
  part[t] = cnt;
  __syncthreads();
  // inclusive scan of the per-thread counts (Hillis-Steele over 1024 entries)
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = part[t] - cnt;
  int32_t* co = coff + bh * (size_t)(Nb + 1);
  for (int j = t * per; j < min(Nb, t * per + per); ++j) {
    co[j] = run;
    const uint32_t* row = maskT + (bh * Nb + j) * (size_t)W;
    for (int w = 0; w < W; ++w) run += __popc(row[w]);
  }
  if (t == 1023) co[Nb] = part[1023];
}

// The column lists: one wave per key block.  The key side runs the kGroup
// consecutive key blocks of a group side by side on one XCD, so a column is
// ordered to meet its group mates: first the query blocks that all of the
// group keep, then those kept by three of them, two, and this one alone,
// ascending within each class.  The shared prefix is then walked in step by
// every member and each staged query block is fetched once for all of them.
static_assert(kGroup == 4, "the owner count below is a 4-input bit-sliced adder");
__global__ __launch_bounds__(256) void column_fill_kernel(const uint32_t* __restrict__ maskT,
                                                          const int32_t* __restrict__ coff, int Nb,
                                                          int W, int k,
                                                          int32_t* __restrict__ cidx) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const size_t bh = blockIdx.y;
  if (j >= Nb) return;
  const int j0 = j - j % kGroup;
  const uint32_t* row = maskT + (bh * Nb + j) * (size_t)W;
  int32_t* out = cidx + bh * (size_t)Nb * k + coff[bh * (size_t)(Nb + 1) + j];
  int base = 0;
  for (int cls = kGroup; cls >= 1; --cls) {
    for (int w0 = 0; w0 < W; w0 += 64) {
      uint32_t word = 0u;
      if (w0 + lane < W) {
        // owners per query block among the group's members, as a bit-sliced count
        uint32_t m[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          m[u] = j0 + u < Nb ? maskT[(bh * Nb + j0 + u) * (size_t)W + w0 + lane] : 0u;
        const uint32_t s0 = m[0] ^ m[1], c0 = m[0] & m[1];
        const uint32_t s1 = m[2] ^ m[3], c1 = m[2] & m[3];
        const uint32_t b0 = s0 ^ s1, cr = s0 & s1;
        const uint32_t b1 = c0 ^ c1 ^ cr;
        const uint32_t b2 = (c0 & c1) | ((c0 ^ c1) & cr);
        const uint32_t n4 = b2;
        const uint32_t n3 = ~b2 & b1 & b0;
        const uint32_t n2 = ~b2 & b1 & ~b0;
        const uint32_t n1 = ~b2 & ~b1 & b0;
        const uint32_t sel = cls == 4 ? n4 : cls == 3 ? n3 : cls == 2 ? n2 : n1;
        word = row[w0 + lane] & sel;
      }
      const int c = __popc(word);
      int incl = c;  // inclusive scan over the wave
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      int pos = base + incl - c;
      while (word) {
        const int b = __ffs(word) - 1;
        out[pos++] = 32 * (w0 + lane) + b;
        word &= word - 1;
      }
      base += __shfl(incl, 63);
    }
  }
}

// Partial G and g_z over a chunk of query blocks: wave w owns phi channels
// 32w..32w+31; the operands are read straight from the per-block transposed
// tiles ([channel][permuted row], 128-byte rows).
__global__ __launch_bounds__(256) void grad_h_partial_kernel(const uint16_t* __restrict__ fqs,
                                                             const uint16_t* __restrict__ dot,
                                                             const float* __restrict__ stats,
                                                             int Nb, float* __restrict__ gpart,
                                                             float* __restrict__ gzpart) {
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6, g = lane >> 4, l16 = lane & 15;
  const int ch = blockIdx.x;
  const size_t bh = blockIdx.y;
  v4f w[2][8], wz[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    wz[mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int et = 0; et < 8; ++et) w[mt][et] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  const int i0 = (int)((long long)Nb * ch / kGradChunks);
  const int i1 = (int)((long long)Nb * (ch + 1) / kGradChunks);
  for (int i = i0; i < i1; ++i) {
    const size_t base = ((size_t)bh * Nb + i) * (kD * kBlk);
    const uint16_t* fb = fqs + base;
    const uint16_t* db = dot + base;
    const float* ub = stats + ((size_t)bh * Nb + i) * kBwdStatFloats + 192;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      // every operand of this half block first, unconditionally, so the loads
      // are in flight together
      bf16x8 af[2], bo[8];
      v4f uq[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        af[mt] = *reinterpret_cast<const bf16x8*>(fb + (32 * wave + 16 * mt + l16) * kBlk + 32 * c + 8 * g);
#pragma unroll
      for (int et = 0; et < 8; ++et)
        bo[et] = *reinterpret_cast<const bf16x8*>(db + (16 * et + l16) * kBlk + 32 * c + 8 * g);
#pragma unroll
      for (int h = 0; h < 2; ++h) uq[h] = *reinterpret_cast<const v4f*>(ub + 32 * c + 8 * g + 4 * h);
#pragma unroll
      for (int et = 0; et < 8; ++et) {
        w[0][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[0], bo[et], w[0][et], 0, 0, 0);
        w[1][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[1], bo[et], w[1][et], 0, 0, 0);
      }
      bf16x8 uv;
#pragma unroll
      for (int e = 0; e < 8; ++e) uv[e] = l16 == 0 ? (__bf16)uq[e >> 2][e & 3] : (__bf16)0.0f;
      wz[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[0], uv, wz[0], 0, 0, 0);
      wz[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[1], uv, wz[1], 0, 0, 0);
    }
  }
  float* gp = gpart + ((size_t)bh * kGradChunks + ch) * kD * kD;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int et = 0; et < 8; ++et)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        gp[(32 * wave + 16 * mt + 4 * g + r) * kD + 16 * et + l16] = w[mt][et][r];
  if (l16 == 0) {
    float* zp = gzpart + ((size_t)bh * kGradChunks + ch) * kD;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) zp[32 * wave + 16 * mt + 4 * g + r] = wz[mt][r];
  }
}

// G, g_z: the chunk partials added in chunk order.
__global__ __launch_bounds__(256) void grad_h_final_kernel(const float* __restrict__ gpart,
                                                           const float* __restrict__ gzpart,
                                                           float* __restrict__ G,
                                                           float* __restrict__ gz) {
  const int t = threadIdx.x;
  const size_t bh = blockIdx.x;
  const float* gp = gpart + bh * kGradChunks * kD * kD;
  for (int e = blockIdx.y * 1024 + t; e < blockIdx.y * 1024 + 1024; e += 256) {
    float s = 0.0f;
    for (int c = 0; c < kGradChunks; ++c) s += gp[(size_t)c * kD * kD + e];
    G[bh * kD * kD + e] = s;
  }
  if (blockIdx.y == 0 && t < kD) {
    float s = 0.0f;
    for (int c = 0; c < kGradChunks; ++c) s += gzpart[(bh * kGradChunks + c) * kD + t];
    gz[bh * kD + t] = s;
  }
}

}  // namespace

hipError_t launch_transpose_blocks(const uint16_t* k, const uint16_t* dout, const Shape& sh,
                                   uint16_t* kt, uint16_t* dot, hipStream_t s) {
  transpose_blocks_kernel<<<dim3(sh.Nb, sh.BH, 2), 256, 0, s>>>(k, dout, kt, dot, sh.N, sh.Nb);
  return hipGetLastError();
}

hipError_t launch_column_lists(const int32_t* idx, const Shape& sh, uint32_t* maskT,
                               int32_t* coff, int32_t* cidx, hipStream_t s) {
  if (sh.k <= 0) return hipSuccess;
  const int W = (sh.Nb + 31) / 32;
  const size_t words = (size_t)sh.BH * sh.Nb * W;
  fill_u32_kernel<<<(unsigned)std::min<size_t>((words + 255) / 256, 4096), 256, 0, s>>>(maskT, words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t total = (size_t)sh.BH * sh.Nb * sh.k;
  column_mark_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(idx, sh.Nb, sh.k, W, total, maskT);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  column_offsets_kernel<<<sh.BH, 1024, 0, s>>>(maskT, sh.Nb, W, coff);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  column_fill_kernel<<<dim3((sh.Nb + 3) / 4, sh.BH), 256, 0, s>>>(maskT, coff, sh.Nb, W, sh.k, cidx);
  return hipGetLastError();
}

hipError_t launch_grad_h(const BwdWorkspace& bw, const Shape& sh, hipStream_t s) {
  grad_h_partial_kernel<<<dim3(kGradChunks, sh.BH), 256, 0, s>>>(bw.fqs, bw.dot, bw.stats, sh.Nb,
                                                                  bw.gpart, bw.gzpart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  grad_h_final_kernel<<<dim3(sh.BH, kD * kD / 1024), 256, 0, s>>>(bw.gpart, bw.gzpart, bw.G, bw.gz);
  return hipGetLastError();
}

}  // namespace sla
