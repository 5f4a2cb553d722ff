// Device-side building blocks shared by the gfx950 kernels: operand types,
// the 16x16 MFMA tile traits, bf16 rounding and wavefront reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

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
// Standard normal CDF Phi(u) = (1 + erf(u / sqrt 2)) / 2 and density phi(u) from one
// exponential, with erf from Abramowitz and Stegun, Handbook of Mathematical
// Functions, formula 7.1.26: for z >= 0, 1 - erf(z) = t (a1 + t (a2 + t (a3 + t (a4 +
// t a5)))) exp(-z^2), t = 1 / (1 + p z), absolute error at most 1.5e-7. The
// coefficients below are the published ones halved, so the polynomial gives
// (1 - erf(z)) / 2 directly; exp(-z^2) with z = |u|/sqrt 2 is exp(-u^2/2).
__device__ inline void normal_cdf_pdf(float u, float& cdf, float& pdf) {
  const float z = fabsf(u) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * z);
  const float e = __builtin_amdgcn_exp2f(-0.72134752044448170f * u * u);   // exp(-u^2 / 2)
  const float q = t * (0.127414796f + t * (-0.142248368f + t * (0.7107068705f + t * (-0.7265760135f + t * 0.5307027145f))));
  const float tail = q * e;                                               // (1 - erf(z)) / 2
  cdf = u >= 0.f ? 1.0f - tail : tail;
  pdf = 0.39894228040143268f * e;
}
// GELU(u) = u Phi(u) and its derivative Phi(u) + u phi(u).
__device__ inline float gelu_f(float u) {
  float c, d;
  normal_cdf_pdf(u, c, d);
  return u * c;
}
__device__ inline float gelu_grad_f(float u) {
  float c, d;
  normal_cdf_pdf(u, c, d);
  return c + u * d;
}
// Both from one evaluation of Phi and phi: the forward epilogue saves GELU'(u) for
// the backward, which then only multiplies by it.
__device__ inline void gelu_and_grad(float u, float& g, float& dg) {
  float c, d;
  normal_cdf_pdf(u, c, d);
  g = u * c;
  dg = c + u * d;
}

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, SC 2011): ten rounds, each taking
// the 32x32 -> 64-bit products of counter words 0 and 2 with the two round
// multipliers and forming (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
// lo(M0 c0)); the key advances by the two Weyl increments between rounds.
__device__ inline u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                      uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; r++) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // one v_mad_u64_u32 per product instead of a mul_lo / mul_hi pair
    const uint64_t p0 = (uint64_t)c0 * 0xD2511F53ull, p1 = (uint64_t)c2 * 0xCD9E8D57ull;
    c0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    c2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
  }
  return (u32x4){c0, c1, c2, c3};
}

// Dropout multipliers (scale when kept, 0 when dropped) of columns 4*grp .. 4*grp+3
// of `row` at `site`.
__device__ inline f32x4 drop_mult4(const DropArgs& a, uint32_t site, uint32_t row, uint32_t grp) {
  const u32x4 w = philox4x32_10(grp, row, site, a.call, a.k0, a.k1);
  f32x4 m;
#pragma unroll
  for (int i = 0; i < 4; i++) m[i] = w[i] >= a.thr ? a.scale : 0.f;
  return m;
}
// The multiplier of one element (row, col).
__device__ inline float drop_mult1(const DropArgs& a, uint32_t site, uint32_t row, uint32_t col) {
  const u32x4 w = philox4x32_10(col >> 2, row, site, a.call, a.k0, a.k1);
  const uint32_t j = col & 3;
  const uint32_t x = j == 0 ? w[0] : (j == 1 ? w[1] : (j == 2 ? w[2] : w[3]));
  return x >= a.thr ? a.scale : 0.f;
}

}  // namespace gpt
