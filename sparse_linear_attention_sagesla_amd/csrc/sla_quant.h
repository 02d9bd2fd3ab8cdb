// The INT8 quantiser shared by every coding site of the library (attention
// codes of Q and K, W8A8 weights and activations): per group of values with
// a = max|x|, scale = fp32(a/127), inv = fp32(127/a) (IEEE fp32 divisions),
// code = clamp(rint(fp32(x * inv)), +-127); a = 0 gives scale 0 and codes 0.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace sla {

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// 8 consecutive bf16 values packed in a uint4 -> 8 floats.
__device__ __forceinline__ void unpack_bf16x8(const uint4& u, float* x) {
  x[0] = __uint_as_float(u.x << 16);
  x[1] = __uint_as_float(u.x & 0xffff0000u);
  x[2] = __uint_as_float(u.y << 16);
  x[3] = __uint_as_float(u.y & 0xffff0000u);
  x[4] = __uint_as_float(u.z << 16);
  x[5] = __uint_as_float(u.z & 0xffff0000u);
  x[6] = __uint_as_float(u.w << 16);
  x[7] = __uint_as_float(u.w & 0xffff0000u);
}

// scale = a/127 and inv = 127/a, or 0 and 0 for a == 0.  Returns a > 0.
__device__ __forceinline__ bool code_scale(float a, float& scale, float& inv) {
  scale = 0.0f;
  inv = 0.0f;
  if (a > 0.0f) {
    scale = a / 127.0f;
    inv = 127.0f / a;
  }
  return a > 0.0f;
}

// Codes of 8 consecutive values: clamp(rint(x * inv), +-127), little-endian
// bytes; 0 unless `live`.
__device__ __forceinline__ uint2 code_row8(const float* x, float inv, bool live) {
  uint32_t w[2] = {0u, 0u};
  if (live) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float y = rintf(x[e] * inv);
      y = fminf(fmaxf(y, -127.0f), 127.0f);
      const uint32_t b = (uint32_t)(int32_t)y & 0xffu;
      w[e >> 2] |= b << (8 * (e & 3));
    }
  }
  return make_uint2(w[0], w[1]);
}

}  // namespace sla
