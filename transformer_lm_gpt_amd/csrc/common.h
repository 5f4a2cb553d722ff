// Device-side building blocks shared by the gfx950 kernels: operand types,
// the 16x16 MFMA tile traits, bf16 rounding and wavefront reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gpt {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

// 16x16 output tile MFMA on one wavefront.
//   A fragment: lane l holds row (l & 15), contraction indices of group (l >> 4).
//   B fragment: lane l holds column (l & 15), contraction indices of group (l >> 4).
//   C: lane l holds rows 4*(l >> 4) + i (i = 0..3) of column (l & 15).
// KG = contraction elements per lane per instruction, KPI = contraction length
// of one instruction (4 groups of KG).
template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int KG = 8;
  static constexpr int KPI = 32;
  typedef bf16x8 frag;
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int KG = 1;
  static constexpr int KPI = 4;
  typedef float frag;
  __device__ static inline f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

template <typename T> __device__ inline T from_f32(float x);
template <> __device__ inline float from_f32<float>(float x) { return x; }
template <> __device__ inline bf16 from_f32<bf16>(float x) { return (bf16)x; }  // round to nearest even

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(bf16 x) { return (float)x; }

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}
// Reductions over the 16 lanes that share (lane >> 4): the columns of a C tile row.
__device__ inline float row16_sum(float v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ inline float row16_max(float v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

// Exact GELU u * Phi(u) and its derivative Phi(u) + u phi(u), with the device erf.
__device__ inline float gelu_f(float u) { return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f)); }
__device__ inline float gelu_grad_f(float u) {
  float cdf = 0.5f * (1.0f + erff(u * 0.70710678118654752f));
  float pdf = 0.39894228040143268f * __expf(-0.5f * u * u);
  return cdf + u * pdf;
}

}  // namespace gpt
