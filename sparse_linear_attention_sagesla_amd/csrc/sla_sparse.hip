// Block-sparse SageSLA attention kernel for gfx950 (CDNA4).
//
// One workgroup = one 64-row query block of one (b,h); four waves, each
// owning 16 query rows.  The workgroup walks the query block's kept key
// blocks (ascending).  Per kept block j, staged in LDS (double-buffered):
//   K8_j   int8 [64 keys][128]      (8 KB)   -> S^T = K8_j Q8_i^T     (INT8 MFMA)
//   phiK_j fp16 [64 keys][128]      (16 KB)  -> G^T = phiK_j phiQ_i^T (fp16 MFMA)
//   V_j    fp16 [128][64 perm keys] (16 KB)  -> O^T += V_j^T P^T, A^T += V_j^T G^T
// Scores are computed transposed (keys x queries) so each lane ends up holding
// one query's values for 16 keys; in that layout the exponentiated scores P and
// the linear weights G are already the B operand of the next product and never
// leave registers, and the online-softmax statistics are per lane.
//
// Softmax branch (tutorial "TurboDiffusion技术架构解析：稀疏线性注意力应用实战"
// §2.1 standard attention, on INT8 codes as in low-bit SageAttention): logits
// acc * sq_i * sk_j / sqrt(128) taken in the log2 domain, online max/sum in
// fp32, P rounded to fp16 with the normaliser summed from the rounded P.
// Linear branch (same section, linear attention with phi = elu+1 / ReLU),
// normalised, over the unselected blocks: numerator phi(Q)H - A and
// denominator phi(Q)z - r, where H, z are the whole-head sums and A, r the
// kept blocks' share accumulated in this loop.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "sla_internal.h"

namespace sla {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));

constexpr int kK8Bytes = kBlk * kD;          // 8 KB
constexpr int kF16TileBytes = kBlk * kD * 2; // 16 KB
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInvSqrtD = 0.08838834764831845f;  // 1/sqrt(128)

// LDS byte offsets of one 16-byte chunk, XOR-swizzled by row to spread banks.
__device__ __forceinline__ int k8_off(int row, int ch) {      // 64 rows x 8 chunks
  return (row * 8 + (ch ^ (row & 7))) * 16;
}
__device__ __forceinline__ int f16row_off(int row, int ch) {  // 64 rows x 16 chunks
  return (row * 16 + (ch ^ (row & 7))) * 16;
}
__device__ __forceinline__ int vt_off(int row, int ch) {      // 128 rows x 8 chunks
  return (row * 8 + (ch ^ (row & 7))) * 16;
}

__device__ __forceinline__ float phi_apply(float x, int phi) {
  if (phi == kPhiElu1) return x > 0.0f ? x + 1.0f : __expf(x);
  return fmaxf(x, 0.0f);
}

struct TileRegs {
  uint4 k8[2];
  uint4 fk[4];
  uint4 v[4];
};

// Global -> registers for one key block: INT8 codes (softmax tiles), fp16
// phi(K)/16 (tiles that feed the linear branch) and fp16 V (always).
__device__ __forceinline__ void load_tile(TileRegs& r, const int8_t* k8, const uint16_t* fk16,
                                          const uint16_t* v16, size_t bh, int Np, int Nb, int j,
                                          bool soft, bool lin, int t) {
  if (soft) {
    const uint4* ks = reinterpret_cast<const uint4*>(k8 + ((size_t)bh * Np + (size_t)j * kBlk) * kD);
    r.k8[0] = ks[t];
    r.k8[1] = ks[t + 256];
  }
  const uint4* vs = reinterpret_cast<const uint4*>(v16 + ((size_t)bh * Nb + j) * kD * kBlk);
#pragma unroll
  for (int m = 0; m < 4; ++m) r.v[m] = vs[t + 256 * m];
  if (lin) {
    const uint4* fs = reinterpret_cast<const uint4*>(fk16 + ((size_t)bh * Np + (size_t)j * kBlk) * kD);
#pragma unroll
    for (int m = 0; m < 4; ++m) r.fk[m] = fs[t + 256 * m];
  }
}

__device__ __forceinline__ void store_tile(const TileRegs& r, unsigned char* st, bool soft,
                                           bool lin, int t) {
  unsigned char* lk = st;
  unsigned char* lv = st + kK8Bytes;
  unsigned char* lf = st + kK8Bytes + kF16TileBytes;
  if (soft) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int gi = t + 256 * m;
      *reinterpret_cast<uint4*>(lk + k8_off(gi >> 3, gi & 7)) = r.k8[m];
    }
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int gi = t + 256 * m;
    *reinterpret_cast<uint4*>(lv + vt_off(gi >> 3, gi & 7)) = r.v[m];
  }
  if (lin) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int gi = t + 256 * m;
      *reinterpret_cast<uint4*>(lf + f16row_off(gi >> 4, gi & 15)) = r.fk[m];
    }
  }
}

// S^T tile (64 keys x 16 queries of this wave) from the staged K8 tile.
// s[kt][r] = sum_e K8[16kt+4g+r][e] * Q8[query l16][e]
__device__ __forceinline__ void qk_tile(const unsigned char* lk, const v4i qf[2], int l16, int g,
                                        v4i s[4]) {
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    s[kt] = v4i{0, 0, 0, 0};
    const int row = 16 * kt + l16;
#pragma unroll
    for (int dc = 0; dc < 2; ++dc) {
      const v4i a = *reinterpret_cast<const v4i*>(lk + k8_off(row, 4 * dc + g));
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

struct SparseArgs {
  const uint16_t* q;
  const int8_t* q8;
  const int8_t* k8;
  const float* sq;
  const float* sk;
  const int32_t* idx;
  const int32_t* uidx;
  const uint16_t* fk16;
  const uint16_t* v16;
  const uint16_t* h16t;
  const float* hscale;
  const float* z;
  int N, Nb, Np, k;
  int phi;        // feature map for phi(Q) (0 = linear branch off)
  int lin;        // linear branch has a non-empty complement
  int direct;     // linear branch summed directly over the unselected blocks
  void* out;
  int out_f32;
  float* out_linear;
};

// Tiles of a query block: p < k are its kept key blocks (softmax branch; in
// the subtraction form they also give the kept share of the linear branch);
// with the direct form, p >= k walk the unselected blocks (linear branch only).
__global__ __launch_bounds__(256, 2) void sparse_fwd_kernel(SparseArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int i = blockIdx.x;
  const size_t bh = blockIdx.y;
  const bool lin = a.phi != kPhiNone && a.lin;
  const bool direct = lin && a.direct;
  const int nu = direct ? a.Nb - a.k : 0;
  const int ntiles = a.k + nu;
  const int stage_bytes = kK8Bytes + kF16TileBytes + (lin ? kF16TileBytes : 0);

  const int qrow = i * kBlk + 16 * wave + l16;  // this lane's query row
  const bool qvalid = qrow < a.N;

  v4i qf[2];
  load_q8_frag(a.q8, bh, a.Np, qrow, g, qf);

  half8 fq[4];
  if (lin) {
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

  v4f o[8], acc_l[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    o[dt] = v4f{0.f, 0.f, 0.f, 0.f};
    acc_l[dt] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  float m_run = -INFINITY, l_part = 0.0f, r_part = 0.0f;
  const float qscale = a.sq[bh * a.Nb + i] * (kInvSqrtD * kLog2e);
  const int32_t* sel = a.idx + (bh * a.Nb + i) * (size_t)a.k;
  const int32_t* usel = direct ? a.uidx + (bh * a.Nb + i) * (size_t)nu : nullptr;

  // key block of tile p, clamped so a malformed index list cannot read outside
  // the staging buffers
  auto tile_block = [&](int p) {
    const int j = p < a.k ? sel[p] : usel[p - a.k];
    return min(max(j, 0), a.Nb - 1);
  };
  auto tile_lin = [&](int p) { return lin && (direct ? p >= a.k : true); };

  TileRegs regs;
  if (ntiles > 0) {
    load_tile(regs, a.k8, a.fk16, a.v16, bh, a.Np, a.Nb, tile_block(0), 0 < a.k, tile_lin(0), t);
    store_tile(regs, smem, 0 < a.k, tile_lin(0), t);
  }
  __syncthreads();

  for (int p = 0; p < ntiles; ++p) {
    const int j = tile_block(p);
    const bool soft = p < a.k;
    const bool plin = tile_lin(p);
    const bool more = p + 1 < ntiles;
    if (more)
      load_tile(regs, a.k8, a.fk16, a.v16, bh, a.Np, a.Nb, tile_block(p + 1), p + 1 < a.k,
                tile_lin(p + 1), t);
    const unsigned char* st = smem + (p & 1) * stage_bytes;
    const unsigned char* lk = st;
    const unsigned char* lv = st + kK8Bytes;
    const unsigned char* lf = st + kK8Bytes + kF16TileBytes;

    // ---- softmax branch scores of a kept block
    half8 pf[2];
    if (soft) {
      v4i s[4];
      qk_tile(lk, qf, l16, g, s);
      const float cs = qscale * a.sk[bh * a.Nb + j];
      const int kvalid = a.N - j * kBlk;  // keys >= kvalid are pad rows
      float x[4][4];
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = 16 * kt + 4 * g + r;
          x[kt][r] = key < kvalid ? (float)s[kt][r] * cs : -INFINITY;
          mx = fmaxf(mx, x[kt][r]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);
      m_run = m_new;
      float psum = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const _Float16 ph = (_Float16)exp2f(x[kt][r] - m_new);
          pf[kt >> 1][4 * (kt & 1) + r] = ph;
          psum += (float)ph;
        }
      l_part = l_part * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
    }

    // ---- linear-branch weights G^T = phiK phiQ^T of this block
    half8 gf[2];
    if (plin) {
      v4f gt[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        gt[kt] = v4f{0.f, 0.f, 0.f, 0.f};
        const int row = 16 * kt + l16;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const half8 af = *reinterpret_cast<const half8*>(lf + f16row_off(row, 4 * cc + g));
          gt[kt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, fq[cc], gt[kt], 0, 0, 0);
        }
      }
      float gsum = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const _Float16 gh = (_Float16)gt[kt][r];
          gf[kt >> 1][4 * (kt & 1) + r] = gh;
          gsum += (float)gh;
        }
      r_part += gsum;
    }

    // ---- O^T += V^T P^T and A^T += V^T G^T
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int row = 16 * dt + l16;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const half8 av = *reinterpret_cast<const half8*>(lv + vt_off(row, 4 * c + g));
        if (soft) o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pf[c], o[dt], 0, 0, 0);
        if (plin) acc_l[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, gf[c], acc_l[dt], 0, 0, 0);
      }
    }

    if (more) store_tile(regs, smem + ((p + 1) & 1) * stage_bytes, p + 1 < a.k, tile_lin(p + 1), t);
    __syncthreads();
  }

  // ---- epilogue: normalise, add the linear branch, store
  float l = l_part + __shfl_xor(l_part, 16);
  l += __shfl_xor(l, 32);
  const float inv_l = (a.k > 0 && l > 0.0f) ? 1.0f / l : 0.0f;

  v4f ol[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) ol[dt] = v4f{0.f, 0.f, 0.f, 0.f};
  if (lin) {
    float r = r_part + __shfl_xor(r_part, 16);
    r += __shfl_xor(r, 32);
    if (direct) {
      // numerator and denominator summed over the unselected blocks
      const float inv_den = r > 0.0f ? 1.0f / r : 0.0f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) ol[dt] = acc_l[dt] * inv_den;
    } else {
      const _Float16* ht = reinterpret_cast<const _Float16*>(a.h16t) + bh * kD * kD;
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
      const float den = dz - r;
      const float inv_den = den > 1e-6f * dz ? 1.0f / den : 0.0f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        v4f num = v4f{0.f, 0.f, 0.f, 0.f};
        const _Float16* hrow = ht + (size_t)(16 * dt + l16) * kD + 8 * g;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const half8 ah = *reinterpret_cast<const half8*>(hrow + 32 * cc);
          num = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, fq[cc], num, 0, 0, 0);
        }
        ol[dt] = (num * hs - acc_l[dt]) * inv_den;
      }
    }
  }

  if (qvalid) {
    const size_t orow = (bh * a.N + qrow) * kD;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const v4f res = o[dt] * inv_l + ol[dt];
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

// Integer S tiles for (b, h, i, j) pairs through the same staging and INT8
// matrix-core path as the attention kernel.
__global__ __launch_bounds__(256) void debug_qk_kernel(const int8_t* __restrict__ q8,
                                                       const int8_t* __restrict__ k8, int B, int H,
                                                       int Np, const int32_t* __restrict__ pairs,
                                                       int32_t* __restrict__ acc) {
  __shared__ __align__(16) unsigned char lk[kK8Bytes];
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
  const uint4* ks = reinterpret_cast<const uint4*>(k8 + (bh * Np + (size_t)j * kBlk) * kD);
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int gi = t + 256 * m;
    *reinterpret_cast<uint4*>(lk + k8_off(gi >> 3, gi & 7)) = ks[gi];
  }
  __syncthreads();
  v4i qf[2];
  load_q8_frag(q8, bh, Np, i * kBlk + 16 * wave + l16, g, qf);
  v4i s[4];
  qk_tile(lk, qf, l16, g, s);
  int32_t* dst = acc + (size_t)p * kBlk * kBlk + (size_t)(16 * wave + l16) * kBlk;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[16 * kt + 4 * g + r] = s[kt][r];
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
  a.fk16 = ws.fk16;
  a.v16 = ws.v16;
  a.h16t = ws.h16t;
  a.hscale = ws.hscale;
  a.z = ws.z;
  a.N = sh.N;
  a.Nb = sh.Nb;
  a.Np = sh.Np;
  a.k = sh.k;
  a.phi = phi;
  a.lin = (phi != kPhiNone && sh.k < sh.Nb) ? 1 : 0;
  a.direct = linear_direct(sh) ? 1 : 0;
  a.out = out;
  a.out_f32 = out_f32;
  a.out_linear = out_linear;
  const size_t stage = (size_t)kK8Bytes + kF16TileBytes + (phi != kPhiNone ? kF16TileBytes : 0);
  const size_t lds = 2 * stage;
  static std::once_flag once;
  std::call_once(once, [] {
    hipFuncSetAttribute(reinterpret_cast<const void*>(sparse_fwd_kernel),
                        hipFuncAttributeMaxDynamicSharedMemorySize, 2 * (kK8Bytes + 2 * kF16TileBytes));
  });
  dim3 grid(sh.Nb, sh.BH);
  sparse_fwd_kernel<<<grid, 256, lds, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_debug_qk(const int8_t* q8, const int8_t* k8, const Shape& sh,
                           const int32_t* pairs, int n_pairs, int32_t* acc, hipStream_t s) {
  debug_qk_kernel<<<n_pairs, 256, 0, s>>>(q8, k8, sh.B, sh.H, sh.Np, pairs, acc);
  return hipGetLastError();
}

}  // namespace sla
