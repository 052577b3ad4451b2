// Device helpers shared by the gfx950 kernels of libgdn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kChunk = 64;        // steps per checkpoint
constexpr float kNormEps = 1e-6f; // inside the square root of the L2 norm
constexpr float kClamp = 20.0f;   // upper bound of the softplus argument

// bf16 storage type (raw bits).
struct bf16 {
  uint16_t x;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) {
  return __uint_as_float(static_cast<uint32_t>(v.x) << 16);
}

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// Round to nearest, ties to even; NaN stays NaN.
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return bf16{static_cast<uint16_t>((u >> 16) | 0x40u)};
  u += 0x7fffu + ((u >> 16) & 1u);
  return bf16{static_cast<uint16_t>(u >> 16)};
}

// Unpack 16 bytes of storage into fp32 values.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void unpack(uint4 u, float* out) {
    out[0] = __uint_as_float(u.x);
    out[1] = __uint_as_float(u.y);
    out[2] = __uint_as_float(u.z);
    out[3] = __uint_as_float(u.w);
  }
};
template <> struct Vec16<bf16> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void unpack(uint4 u, float* out) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

// DPP lane exchange within a row of 16 lanes.
template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Sum over the 16 lanes of a DPP row.  Every lane of the row ends with the
// same bits: each stage adds a value to its partner's value (a + b == b + a).
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<kQuadXor1>(v);
  v += dpp<kQuadXor2>(v);
  v += dpp<kRowHalfMirror>(v);
  v += dpp<kRowMirror>(v);
  return v;
}

__device__ __forceinline__ float softplus_f(float x) {
  return x > 0.f ? x + log1pf(expf(-x)) : log1pf(expf(x));
}
__device__ __forceinline__ float sigmoid_f(float x) {
  if (x >= 0.f) return 1.f / (1.f + expf(-x));
  float e = expf(x);
  return e / (1.f + e);
}

}  // namespace gdn
