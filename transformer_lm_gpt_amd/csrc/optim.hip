// Global gradient norm, clip coefficient and the single-pass AdamW update.
//
// Clipping at a global L2 norm of 1.0 ("Building microGPT from scratch",
// single-GPU parameter list) and AdamW with decoupled weight decay and betas
// (nanoGPT run log, section 2.1; the microGPT page for the Adam constants).
// The norm is reduced in a fixed order (per-block partials, then one block in
// double precision), so it is bitwise reproducible. The step counter, the clip
// coefficient and the bias corrections stay on the device; a non-finite norm
// skips the update without a host round trip.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace gpt {

// The gradient norm's per-block partial sums for gpt_adamw_step_noalloc, which takes
// no workspace for them: one file-scope array per GPU, alive until the process ends.
// Host code never passes `scratch` itself (in host code the name is a stand-in, not
// the device address): noalloc_norm_scratch() looks up each device's address once,
// with that device current, and hands that out.
static __device__ __align__(256) float scratch[NOALLOC_SCRATCH_FLOATS];

hipError_t noalloc_norm_scratch(int device, float** out) {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static float* ptr[MAX_DEVICES] = {};
  if (device < 0 || device >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[device]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != device ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (e2 != hipSuccess) return e2;
    if (!p) return hipErrorInvalidSymbol;
    ptr[device] = (float*)p;
  }
  *out = ptr[device];
  return hipSuccess;
}

__global__ __launch_bounds__(256) void sumsq_partial_kernel(const float* __restrict__ g, size_t n4,
                                                            float* __restrict__ part) {
  __shared__ float red[4];
  const f32x4* g4 = (const f32x4*)g;
  float s = 0.f;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    f32x4 v = g4[i];
    s += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = ((red[0] + red[1]) + red[2]) + red[3];
}

hipError_t launch_sumsq_partial(const float* g, size_t n, float* part, hipStream_t s) {
  // n is a multiple of 4 (the flat layout pads to 64 elements).
  hipLaunchKernelGGL(sumsq_partial_kernel, dim3(NORM_BLOCKS), dim3(256), 0, s, g, n / 4, part);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void opt_prepare_kernel(const float* __restrict__ part, OptState* st, float clip,
                                                          float beta1, float beta2, float* norm_out) {
  __shared__ double red[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < NORM_BLOCKS; i += 256) s += (double)part[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double norm = sqrt(red[0]);
    const float nf = (float)norm;
    st->norm = nf;
    if (norm_out) *norm_out = nf;
    if (st->bad_ids) {   // gradients of out-of-range ids: no update (reported at sync)
      st->skip = 1;
      st->coef = 0.f;
      return;
    }
    if (!isfinite(norm)) {
      st->skip = 1;
      st->nonfinite = 1;
      st->coef = 0.f;
      return;
    }
    st->skip = 0;
    double coef = 1.0;
    if (clip > 0.f) coef = fmin(1.0, (double)clip / (norm + 1e-6));
    st->coef = (float)coef;
    const int64_t t = st->t + 1;
    st->t = t;
    st->bc1 = (float)(1.0 - pow((double)beta1, (double)t));
    st->bc2 = (float)(1.0 - pow((double)beta2, (double)t));
  }
}

hipError_t launch_opt_prepare(const float* part, OptState* st, float clip, float beta1, float beta2,
                              float* norm_out, hipStream_t s) {
  hipLaunchKernelGGL(opt_prepare_kernel, dim3(1), dim3(256), 0, s, part, st, clip, beta1, beta2, norm_out);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void check_ids_kernel(const int32_t* __restrict__ ids, int n, int V, OptState* st) {
  bool bad = false;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) bad |= (uint32_t)ids[i] >= (uint32_t)V;
  if (bad) st->bad_ids = 1;   // the same value from every offending lane
}

hipError_t launch_check_ids(const int32_t* ids, int n, int V, OptState* st, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = std::min((n + 255) / 256, 256);
  hipLaunchKernelGGL(check_ids_kernel, dim3(blocks), dim3(256), 0, s, ids, n, V, st);
  return hipGetLastError();
}

// One pass over the flat buffers, four elements per thread per iteration.
__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ p, const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v,
                                                    bf16* __restrict__ shadow, size_t n4, size_t n_decay,
                                                    const OptState* __restrict__ st, float lr, float beta1,
                                                    float beta2, float eps, float wd) {
  if (st->skip) return;
  const float coef = st->coef;
  const float inv_bc1 = 1.f / st->bc1;
  const float inv_bc2 = 1.f / st->bc2;
  const float decay = 1.f - lr * wd;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    // every byte is touched once: streaming loads and stores keep the caches out of it
    f32x4 pv = __builtin_nontemporal_load((f32x4*)p + i);
    const f32x4 gv = __builtin_nontemporal_load((const f32x4*)g + i);
    f32x4 mv = __builtin_nontemporal_load((f32x4*)m + i);
    f32x4 vv = __builtin_nontemporal_load((f32x4*)v + i);
    const bool dec = i * 4 < n_decay;   // n_decay is a multiple of 64
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const float gg = gv[e] * coef;
      mv[e] = beta1 * mv[e] + (1.f - beta1) * gg;
      vv[e] = beta2 * vv[e] + (1.f - beta2) * gg * gg;
      const float mhat = mv[e] * inv_bc1;
      const float vhat = vv[e] * inv_bc2;
      float pe = dec ? pv[e] * decay : pv[e];
      pv[e] = pe - lr * mhat / (sqrtf(vhat) + eps);
    }
    __builtin_nontemporal_store(pv, (f32x4*)p + i);
    __builtin_nontemporal_store(mv, (f32x4*)m + i);
    __builtin_nontemporal_store(vv, (f32x4*)v + i);
    if (shadow) {
      bf16x4 sv;
#pragma unroll
      for (int e = 0; e < 4; e++) sv[e] = (bf16)pv[e];
      __builtin_nontemporal_store(__builtin_bit_cast(u32x2, sv), (u32x2*)shadow + i);
    }
  }
}

hipError_t launch_adamw(float* p, const float* g, float* m, float* v, void* shadow_bf16, size_t n, size_t n_decay,
                        const OptState* st, float lr, float beta1, float beta2, float eps, float wd,
                        hipStream_t s) {
  const size_t n4 = n / 4;
  unsigned blocks = (unsigned)std::min<size_t>((n4 + 255) / 256, 65536);
  hipLaunchKernelGGL(adamw_kernel, dim3(blocks), dim3(256), 0, s, p, g, m, v, (bf16*)shadow_bf16, n4, n_decay, st,
                     lr, beta1, beta2, eps, wd);
  return hipGetLastError();
}

}  // namespace gpt
