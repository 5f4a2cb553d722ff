// Row-wise, HBM-bound kernels of the step: embedding gather, LayerNorm forward
// and backward, deterministic column sums (bias and LayerNorm parameter
// gradients), the fused softmax cross-entropy forward+backward and the loss mean.
#include "common.h"
#include "kernels.h"

namespace gpt {

// ----------------------------------------------------------------------------- embedding
// Token embedding plus learned position embedding ("Building microGPT from
// scratch", model-core section: token/pos embedding, no rotary), then the
// embedding dropout when da.on (nanoGPT run log, sections 2.1 and 2.2).
__global__ void embed_fwd_kernel(const float* __restrict__ wte, const float* __restrict__ wpe,
                                 const int32_t* __restrict__ tok, float* __restrict__ x0, int M, int T, int d,
                                 int Vp, DropArgs da) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t total = (int64_t)M * d;
  if (i >= total) return;
  int m = (int)(i / d), c = (int)(i % d);
  const int id = tok[m];
  // an id outside the table poisons the row instead of reading out of bounds
  float v = (id >= 0 && id < Vp) ? wte[(int64_t)id * d + c] + wpe[(int64_t)(m % T) * d + c] : __builtin_nanf("");
  if (da.on) v *= drop_mult1(da, 0, m, c);
  x0[i] = v;
}

// The same, four columns per thread (d a multiple of 4, 16-byte aligned tables).
__global__ void embed_fwd4_kernel(const float* __restrict__ wte, const float* __restrict__ wpe,
                                  const int32_t* __restrict__ tok, float* __restrict__ x0, int M, int T, int d,
                                  int Vp, DropArgs da) {
  const int d4 = d >> 2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)M * d4) return;
  const int m = (int)(i / d4), c = (int)(i % d4) * 4;
  const int id = tok[m];
  f32x4 v;
  if (id >= 0 && id < Vp) {
    v = *(const f32x4*)(wte + (int64_t)id * d + c) + *(const f32x4*)(wpe + (int64_t)(m % T) * d + c);
  } else {
    const float nan = __builtin_nanf("");
    v = (f32x4){nan, nan, nan, nan};
  }
  if (da.on) v *= drop_mult4(da, 0, m, c >> 2);
  *(f32x4*)(x0 + (int64_t)m * d + c) = v;
}

hipError_t launch_embed_fwd(const float* wte, const float* wpe, const int32_t* tok, float* x0, int M, int T,
                            int d, int Vp, const DropArgs& da, hipStream_t s) {
  if (d % 4 == 0 && (uintptr_t)wte % 16 == 0 && (uintptr_t)wpe % 16 == 0 && (uintptr_t)x0 % 16 == 0) {
    const int64_t n4 = (int64_t)M * (d / 4);
    hipLaunchKernelGGL(embed_fwd4_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, wte, wpe, tok, x0, M,
                       T, d, Vp, da);
    return hipGetLastError();
  }
  int64_t total = (int64_t)M * d;
  hipLaunchKernelGGL(embed_fwd_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, wte, wpe, tok,
                     x0, M, T, d, Vp, da);
  return hipGetLastError();
}

// dst = src * mask(site) over an fp32 [M, d] array, four columns per thread.
__global__ void dropout_rows_kernel(const float* src, float* dst, int M, int d4, DropArgs da, uint32_t site) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)M * d4) return;
  const int m = (int)(i / d4), g = (int)(i % d4);
  ((f32x4*)dst)[i] = ((const f32x4*)src)[i] * drop_mult4(da, site, m, g);
}

hipError_t launch_dropout_rows(const float* src, float* dst, int M, int d, const DropArgs& da, uint32_t site,
                               hipStream_t s) {
  if (d % 4 != 0 || (uintptr_t)src % 16 != 0 || (uintptr_t)dst % 16 != 0) return hipErrorInvalidValue;
  const int64_t n4 = (int64_t)M * (d / 4);
  hipLaunchKernelGGL(dropout_rows_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, src, dst, M, d / 4,
                     da, site);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- LayerNorm
// One wavefront per row: mean, biased variance, rstd = 1/sqrt(var + 1e-5).
template <typename T>
__global__ __launch_bounds__(256) void ln_fwd_kernel(const float* __restrict__ x, const float* __restrict__ g,
                                                     const float* __restrict__ b, T* __restrict__ y,
                                                     float* __restrict__ mean, float* __restrict__ rstd, int M,
                                                     int d) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float* xr = x + (int64_t)row * d;
  float s = 0.f;
  for (int c = lane; c < d; c += 64) s += xr[c];
  const float mu = wave_sum(s) / d;
  float v = 0.f;
  for (int c = lane; c < d; c += 64) {
    float t = xr[c] - mu;
    v += t * t;
  }
  const float rs = 1.0f / sqrtf(wave_sum(v) / d + 1e-5f);
  T* yr = y + (int64_t)row * d;
  for (int c = lane; c < d; c += 64) yr[c] = from_f32<T>((xr[c] - mu) * rs * g[c] + b[c]);
  if (lane == 0) {
    mean[row] = mu;
    rstd[row] = rs;
  }
}

// The same with the row held in registers: each lane owns NCH float4 column groups
// (d a multiple of 4, at most 256 * NCH), so x is read once, as 16-byte vectors.
template <typename T, int NCH>
__global__ __launch_bounds__(256) void ln_fwd_vec_kernel(const float* __restrict__ x, const float* __restrict__ g,
                                                         const float* __restrict__ b, T* __restrict__ y,
                                                         float* __restrict__ mean, float* __restrict__ rstd, int M,
                                                         int d) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const int d4 = d >> 2;
  const f32x4* xr = (const f32x4*)(x + (int64_t)row * d);
  f32x4 xv[NCH];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; j++) {
    const int c4 = j * 64 + lane;
    xv[j] = c4 < d4 ? xr[c4] : (f32x4){0.f, 0.f, 0.f, 0.f};
    s += (xv[j][0] + xv[j][1]) + (xv[j][2] + xv[j][3]);
  }
  const float mu = wave_sum(s) / d;
  float v = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; j++)
    if (j * 64 + lane < d4)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const float t = xv[j][e] - mu;
        v += t * t;
      }
  const float rs = 1.0f / sqrtf(wave_sum(v) / d + 1e-5f);
#pragma unroll
  for (int j = 0; j < NCH; j++) {
    const int c4 = j * 64 + lane;
    if (c4 >= d4) continue;
    const f32x4 gv = ((const f32x4*)g)[c4], bv = ((const f32x4*)b)[c4];
    f32x4 o;
#pragma unroll
    for (int e = 0; e < 4; e++) o[e] = (xv[j][e] - mu) * rs * gv[e] + bv[e];
    if constexpr (sizeof(T) == 2) {
      bf16x4 ob;
#pragma unroll
      for (int e = 0; e < 4; e++) ob[e] = (bf16)o[e];
      ((bf16x4*)(y + (int64_t)row * d))[c4] = ob;
    } else {
      ((f32x4*)(y + (int64_t)row * d))[c4] = o;
    }
  }
  if (lane == 0) {
    mean[row] = mu;
    rstd[row] = rs;
  }
}

template <typename T>
static hipError_t ln_fwd_t(const float* x, const float* g, const float* b, T* y, float* mean, float* rstd, int M,
                           int d, hipStream_t s) {
  dim3 grid((M + 3) / 4);
  const bool vec = d % 4 == 0 && ((uintptr_t)x | (uintptr_t)g | (uintptr_t)b) % 16 == 0 &&
                   (uintptr_t)y % (4 * sizeof(T)) == 0;
  switch (vec ? (d / 4 + 63) / 64 : 0) {
#define LNF(N) \
  case N: hipLaunchKernelGGL((ln_fwd_vec_kernel<T, N>), grid, dim3(256), 0, s, x, g, b, y, mean, rstd, M, d); break;
    LNF(1) LNF(2) LNF(3) LNF(4)
#undef LNF
    default: hipLaunchKernelGGL(ln_fwd_kernel<T>, grid, dim3(256), 0, s, x, g, b, y, mean, rstd, M, d);
  }
  return hipGetLastError();
}

hipError_t launch_layernorm_fwd(const float* x, const float* g, const float* b, void* y, bool bf16_out,
                                float* mean, float* rstd, int M, int d, hipStream_t s) {
  if (bf16_out) return ln_fwd_t<bf16>(x, g, b, (bf16*)y, mean, rstd, M, d, s);
  return ln_fwd_t<float>(x, g, b, (float*)y, mean, rstd, M, d, s);
}

// Weightless RMSNorm (the microGPT block): y = x / sqrt(mean(x^2) + 1e-5). One
// wavefront per row, d a multiple of 4; writes mean = 0 and rstd so that the
// LayerNorm backward's xhat = (x - mean) rstd is this norm's output.
template <typename T>
__global__ __launch_bounds__(256) void rms_fwd_kernel(const float* __restrict__ x, T* __restrict__ y,
                                                      float* __restrict__ mean, float* __restrict__ rstd, int M, int d) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const int d4 = d >> 2;
  const f32x4* xr = (const f32x4*)(x + (int64_t)row * d);
  float s = 0.f;
  for (int c4 = lane; c4 < d4; c4 += 64) {
    const f32x4 v = xr[c4];
    s += (v[0] * v[0] + v[1] * v[1]) + (v[2] * v[2] + v[3] * v[3]);
  }
  const float rs = 1.0f / sqrtf(wave_sum(s) / d + 1e-5f);
  for (int c4 = lane; c4 < d4; c4 += 64) {
    const f32x4 v = xr[c4];
    if constexpr (sizeof(T) == 2) {
      bf16x4 ob;
#pragma unroll
      for (int e = 0; e < 4; e++) ob[e] = (bf16)(v[e] * rs);
      ((bf16x4*)(y + (int64_t)row * d))[c4] = ob;
    } else {
      ((f32x4*)(y + (int64_t)row * d))[c4] = v * rs;
    }
  }
  if (lane == 0) {
    mean[row] = 0.f;
    rstd[row] = rs;
  }
}

hipError_t launch_rmsnorm_fwd(const float* x, void* y, bool bf16_out, float* mean, float* rstd, int M, int d,
                              hipStream_t s) {
  if (d % 4 != 0 || (uintptr_t)x % 16 != 0 || (uintptr_t)y % (bf16_out ? 8 : 16) != 0) return hipErrorInvalidValue;
  dim3 grid((M + 3) / 4);
  if (bf16_out)
    hipLaunchKernelGGL(rms_fwd_kernel<bf16>, grid, dim3(256), 0, s, x, (bf16*)y, mean, rstd, M, d);
  else
    hipLaunchKernelGGL(rms_fwd_kernel<float>, grid, dim3(256), 0, s, x, (float*)y, mean, rstd, M, d);
  return hipGetLastError();
}

// Backward: with xhat = (x - mu) rstd and gh = dy * g,
//   dx = rstd (gh - mean(gh) - xhat mean(gh xhat)) + dres.
// dy arrives in the operand type T (bf16 from the input-gradient GEMMs in bf16
// mode, fp32 otherwise); everything else is fp32.
// One wavefront per row, LN_BWD_ROWS rows per workgroup. Each lane owns
// NCH float4 column groups and keeps its column partials of dy*xhat, dy and
// dres in registers; the four waves are combined in LDS in a fixed order and
// written as one partial row per workgroup (reduced later by colsum_final).
// The dres column sum is the bias gradient of the projection whose output
// feeds this residual, so it comes for free here.
// With DROP, the dres column sums take dres times the mask of site_in (the
// gradient of the dropped branch output whose add fed this residual) and dx_op
// holds dx times the mask of site_out (the operand of the branch below); a
// negative site leaves that side unmasked.
// With RMS (the weightless RMSNorm, mean = 0 saved): gh = dy, no mean(gh) term,
// and no gain or shift partials.
constexpr int LN_MAX_D = 1024;
template <typename T, int NCH, bool DROP, bool RMS = false>
__global__ __launch_bounds__(256) void ln_bwd_kernel(const T* __restrict__ dy, const float* __restrict__ x,
                                                     const float* __restrict__ mean,
                                                     const float* __restrict__ rstd, const float* __restrict__ g,
                                                     const float* dres, float* dx, T* dx_op,
                                                     float* __restrict__ part_g, float* __restrict__ part_b,
                                                     float* __restrict__ part_r, int M, int d, DropArgs da,
                                                     int site_in, int site_out) {
  __shared__ f32x4 red[4][LN_MAX_D / 4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int d4 = d >> 2;
  f32x4 gg[NCH], pg[NCH], pb[NCH], pr[NCH];
#pragma unroll
  for (int j = 0; j < NCH; j++) {
    const int c4 = j * 64 + lane;
    gg[j] = RMS ? (f32x4){1.f, 1.f, 1.f, 1.f} : (c4 < d4 ? ((const f32x4*)g)[c4] : (f32x4){0.f, 0.f, 0.f, 0.f});
    pg[j] = pb[j] = pr[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  const int row0 = blockIdx.x * LN_BWD_ROWS;
  // the next row's x, dy and dres are requested before this row's reductions run
  f32x4 xn[NCH], dyn[NCH], rn[NCH];
  auto fetch = [&](int row) {
    const int64_t o4 = (int64_t)row * d4;
#pragma unroll
    for (int j = 0; j < NCH; j++) {
      const int c4 = j * 64 + lane;
      const bool in = c4 < d4;
      xn[j] = in ? ((const f32x4*)x)[o4 + c4] : (f32x4){0.f, 0.f, 0.f, 0.f};
      if constexpr (sizeof(T) == 2) {
        if (in) {
          const bf16x4 t = ((const bf16x4*)dy)[o4 + c4];
          dyn[j] = (f32x4){(float)t[0], (float)t[1], (float)t[2], (float)t[3]};
        } else {
          dyn[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
      } else {
        dyn[j] = in ? ((const f32x4*)dy)[o4 + c4] : (f32x4){0.f, 0.f, 0.f, 0.f};
      }
      rn[j] = in && dres ? ((const f32x4*)dres)[o4 + c4] : (f32x4){0.f, 0.f, 0.f, 0.f};
    }
  };
  if (row0 + w < M) fetch(row0 + w);
  for (int r = w; r < LN_BWD_ROWS; r += 4) {
    const int row = row0 + r;
    if (row >= M) break;
    const int64_t o4 = (int64_t)row * d4;
    const float mu = mean[row], rs = rstd[row];
    f32x4 xh[NCH], dyv[NCH], rv[NCH];
#pragma unroll
    for (int j = 0; j < NCH; j++) {
      xh[j] = xn[j];
      dyv[j] = dyn[j];
      rv[j] = rn[j];
    }
    if (r + 4 < LN_BWD_ROWS && row + 4 < M) fetch(row + 4);
    float sa = 0.f, sbb = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; j++) {
      const int c4 = j * 64 + lane;
      if (c4 < d4) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
          xh[j][e] = (xh[j][e] - mu) * rs;
          const float gh = dyv[j][e] * gg[j][e];
          sa += gh;
          sbb += gh * xh[j][e];
          pg[j][e] += dyv[j][e] * xh[j][e];
          pb[j][e] += dyv[j][e];
        }
      }
    }
    const float a = RMS ? 0.f : wave_sum(sa) / d;
    const float bb = wave_sum(sbb) / d;
#pragma unroll
    for (int j = 0; j < NCH; j++) {
      const int c4 = j * 64 + lane;
      if (c4 < d4) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          v[e] = rs * (dyv[j][e] * gg[j][e] - a - xh[j][e] * bb) + rv[j][e];
          if constexpr (!DROP) pr[j][e] += rv[j][e];
        }
        if constexpr (DROP) pr[j] += site_in >= 0 ? rv[j] * drop_mult4(da, site_in, row, c4) : rv[j];
        ((f32x4*)dx)[o4 + c4] = v;
        if (DROP && site_out >= 0) v *= drop_mult4(da, site_out, row, c4);
        if (dx_op) {
          if constexpr (sizeof(T) == 2) {
            bf16x4 vb;
#pragma unroll
            for (int e = 0; e < 4; e++) vb[e] = (bf16)v[e];
            ((bf16x4*)dx_op)[o4 + c4] = vb;
          } else {
            ((f32x4*)dx_op)[o4 + c4] = v;
          }
        }
      }
    }
  }
  // fixed-order combine of the four waves, one quantity at a time
  float* const outs[3] = {part_g, part_b, part_r};
#pragma unroll
  for (int q = RMS ? 2 : 0; q < 3; q++) {
    if (q == 2 && !part_r) break;
#pragma unroll
    for (int j = 0; j < NCH; j++) {
      const int c4 = j * 64 + lane;
      if (c4 < d4) red[w][c4] = q == 0 ? pg[j] : (q == 1 ? pb[j] : pr[j]);
    }
    __syncthreads();
    for (int c4 = threadIdx.x; c4 < d4; c4 += 256) {
      f32x4 t = red[0][c4];
#pragma unroll
      for (int ww = 1; ww < 4; ww++) t += red[ww][c4];
      ((f32x4*)outs[q])[(int64_t)blockIdx.x * d4 + c4] = t;
    }
    __syncthreads();
  }
}

template <typename T, bool DROP, bool RMS = false>
static hipError_t ln_bwd_t(const void* dy, const float* x, const float* mean, const float* rstd, const float* g,
                           const float* dres, float* dx, void* dx_op, float* pg, float* pb, float* pr, int M, int d,
                           const DropArgs& da, int si, int so, hipStream_t s) {
  dim3 grid((M + LN_BWD_ROWS - 1) / LN_BWD_ROWS);
  const int nch = (d / 4 + 63) / 64;
  switch (nch) {
#define LNB(N) \
  case N: hipLaunchKernelGGL((ln_bwd_kernel<T, N, DROP, RMS>), grid, dim3(256), 0, s, (const T*)dy, x, mean, rstd, g, dres, dx, (T*)dx_op, pg, pb, pr, M, d, da, si, so); break;
    LNB(1) LNB(2) LNB(3) LNB(4)
#undef LNB
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_layernorm_bwd(const void* dy, const float* x, const float* mean, const float* rstd,
                                const float* g, const float* dres, float* dx, void* dx_op, bool bf16_out,
                                float* part_g, float* part_b, float* part_r, int M, int d, const DropArgs& da,
                                int site_in, int site_out, hipStream_t s) {
  if (d > LN_MAX_D || d % 4 != 0) return hipErrorInvalidValue;
  const bool drop = da.on && (site_in >= 0 || site_out >= 0);
  if (!g) {   // weightless RMSNorm
    if (bf16_out)
      return drop ? ln_bwd_t<bf16, true, true>(dy, x, mean, rstd, g, dres, dx, dx_op, part_g, part_b, part_r, M, d,
                                               da, site_in, site_out, s)
                  : ln_bwd_t<bf16, false, true>(dy, x, mean, rstd, g, dres, dx, dx_op, part_g, part_b, part_r, M, d,
                                                da, site_in, site_out, s);
    return drop ? ln_bwd_t<float, true, true>(dy, x, mean, rstd, g, dres, dx, dx_op, part_g, part_b, part_r, M, d,
                                              da, site_in, site_out, s)
                : ln_bwd_t<float, false, true>(dy, x, mean, rstd, g, dres, dx, dx_op, part_g, part_b, part_r, M, d,
                                               da, site_in, site_out, s);
  }
  if (bf16_out)
    return drop ? ln_bwd_t<bf16, true>(dy, x, mean, rstd, g, dres, dx, dx_op, part_g, part_b, part_r, M, d, da,
                                       site_in, site_out, s)
                : ln_bwd_t<bf16, false>(dy, x, mean, rstd, g, dres, dx, dx_op, part_g, part_b, part_r, M, d, da,
                                        site_in, site_out, s);
  return drop ? ln_bwd_t<float, true>(dy, x, mean, rstd, g, dres, dx, dx_op, part_g, part_b, part_r, M, d, da,
                                      site_in, site_out, s)
              : ln_bwd_t<float, false>(dy, x, mean, rstd, g, dres, dx, dx_op, part_g, part_b, part_r, M, d, da,
                                       site_in, site_out, s);
}

// ----------------------------------------------------------------------------- column sums
template <typename T>
__global__ void colsum_partial_kernel(const T* __restrict__ X, int64_t ldx, int M, int N, float* __restrict__ part) {
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= N) return;
  const int r0 = blockIdx.y * COLSUM_ROWS;
  const int r1 = min(M, r0 + COLSUM_ROWS);
  float s = 0.f;
  for (int r = r0; r < r1; r++) s += to_f32(X[(int64_t)r * ldx + col]);
  part[(int64_t)blockIdx.y * N + col] = s;
}

hipError_t launch_colsum_partial(const void* X, bool bf16_in, int64_t ldx, int M, int N, float* part,
                                 hipStream_t s) {
  dim3 grid((N + 255) / 256, (M + COLSUM_ROWS - 1) / COLSUM_ROWS);
  if (bf16_in)
    hipLaunchKernelGGL(colsum_partial_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)X, ldx, M, N, part);
  else
    hipLaunchKernelGGL(colsum_partial_kernel<float>, grid, dim3(256), 0, s, (const float*)X, ldx, M, N, part);
  return hipGetLastError();
}

// RED_COLS (64) columns per workgroup, 16 row groups: each thread sums every 16th
// partial row of its four columns in order, then the 16 group sums are added in a
// fixed order. A workgroup finds its job by binary search over first_blk.
__global__ __launch_bounds__(256) void reduce_jobs_kernel(const RedJob* __restrict__ jobs, int njobs,
                                                          const float* __restrict__ part, float* __restrict__ grads,
                                                          RedRows rows, float beta) {
  __shared__ f32x4 red[16][17];
  __shared__ int job;
  if (threadIdx.x == 0) {
    int lo = 0, hi = njobs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (jobs[mid].first_blk <= (int)blockIdx.x) lo = mid;
      else hi = mid - 1;
    }
    job = lo;
  }
  __syncthreads();
  const RedJob J = jobs[job];
  const int nblk = rows.nblk[J.rows_kind];
  const float* pp = part + J.part;
  const int cl = threadIdx.x & 15, grp = threadIdx.x >> 4;
  const int col = ((int)blockIdx.x - J.first_blk) * RED_COLS + 4 * cl;
  const int64_t n = J.n;
  f32x4 s = (f32x4){0.f, 0.f, 0.f, 0.f};
  if ((n & 3) == 0 && (J.part & 3) == 0) {
    if (col < n) {
      const float* q = pp + col;
      int r = grp;
      for (; r + 48 < nblk; r += 64) {   // four rows in flight, added in row order
        const f32x4 a = *(const f32x4*)(q + r * n), b = *(const f32x4*)(q + (r + 16) * n);
        const f32x4 c = *(const f32x4*)(q + (r + 32) * n), d = *(const f32x4*)(q + (r + 48) * n);
        s += a;
        s += b;
        s += c;
        s += d;
      }
      for (; r < nblk; r += 16) s += *(const f32x4*)(q + r * n);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; e++)
      if (col + e < n)
        for (int r = grp; r < nblk; r += 16) s[e] += pp[r * n + col + e];
  }
  red[grp][cl] = s;
  __syncthreads();
  if (grp == 0) {
    f32x4 t = red[0][cl];
#pragma unroll
    for (int q = 1; q < 16; q++) t += red[q][cl];
    float* dst = grads + J.dst;
#pragma unroll
    for (int e = 0; e < 4; e++)
      if (col + e < n) dst[col + e] = (beta != 0.f ? beta * dst[col + e] : 0.f) + t[e];
  }
}

hipError_t launch_reduce_jobs(const RedJob* jobs, int njobs, int total_blk, const float* part, float* grads,
                              RedRows rows, float beta, hipStream_t s) {
  if (njobs <= 0 || total_blk <= 0) return hipSuccess;
  hipLaunchKernelGGL(reduce_jobs_kernel, dim3(total_blk), dim3(256), 0, s, jobs, njobs, part, grads, rows, beta);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- cross-entropy
// Per row m of logits z: lse = log sum_j exp(z_j) over all Vp columns,
// loss_m = lse - z[y_m]; the row is then overwritten by its gradient
// (softmax - onehot(y)) * grad_scale ("Building microGPT from scratch",
// training-loop section: -log probs[target], averaged over positions).
template <typename T>
__global__ __launch_bounds__(256) void xent_kernel(T* z, int64_t ldz, const int32_t* __restrict__ y,
                                                   float* __restrict__ row_loss, int Vp, float grad_scale) {
  __shared__ float red_m[4], red_s[4];
  __shared__ float s_lse, s_zt;
  const int row = blockIdx.x;
  T* zr = z + (int64_t)row * ldz;
  const int tgt = y[row];
  float m = -INFINITY, s = 0.f;
  for (int c = threadIdx.x; c < Vp; c += 256) {
    float v = to_f32(zr[c]);
    if (v > m) {
      s = s * __expf(m - v) + 1.f;
      m = v;
    } else {
      s += __expf(v - m);
    }
  }
  // wave combine of (m, s)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float m2 = __shfl_xor(m, o, WAVE), s2 = __shfl_xor(s, o, WAVE);
    float mm = fmaxf(m, m2);
    s = (m == -INFINITY ? 0.f : s * __expf(m - mm)) + (m2 == -INFINITY ? 0.f : s2 * __expf(m2 - mm));
    m = mm;
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red_m[w] = m;
    red_s[w] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float mm = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
    float ss = 0.f;
    for (int i = 0; i < 4; i++) ss += red_m[i] == -INFINITY ? 0.f : red_s[i] * __expf(red_m[i] - mm);
    float lse = mm + logf(ss);
    s_lse = lse;
    const bool ok = tgt >= 0 && tgt < Vp;   // an id outside the table yields a NaN loss
    float zt = ok ? to_f32(zr[tgt]) : __builtin_nanf("");
    s_zt = zt;
    row_loss[row] = lse - zt;
  }
  __syncthreads();
  const float lse = s_lse;
  for (int c = threadIdx.x; c < Vp; c += 256) {
    float p = __expf(to_f32(zr[c]) - lse);
    zr[c] = from_f32<T>((p - (c == tgt ? 1.f : 0.f)) * grad_scale);
  }
}

// bf16 rows of up to 8192 NV columns held in registers: each of 1024 threads keeps
// NV 16-byte vectors of the row, forms the max and the sum of exp relative to its
// own max, the (max, sum) pairs are merged over the row, and the gradient is
// written from the registers: one read and one write of the row, and registers
// small enough for two rows in flight per CU.
template <int NV>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(8, 8))) void xent_reg_kernel(bf16* z, int64_t ldz, const int32_t* __restrict__ y,
                                                        float* __restrict__ row_loss, int Vp, float grad_scale) {
  constexpr float L2E = 1.4426950408889634f;
  __shared__ float red_m[16], red_s[16];
  __shared__ float s_m, s_s;
  const int row = blockIdx.x, tid = threadIdx.x, w = tid >> 6;
  bf16* zr = z + (int64_t)row * ldz;
  const int tgt = y[row];
  const int nv = Vp / 8;
  bf16x8 v[NV];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < NV; j++) {
    const int i = tid + 1024 * j;
    if (i < nv) {
      // the row is read once and overwritten once: streaming accesses
      v[j] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const u32x4*)(zr + 8 * i)));
#pragma unroll
      for (int e = 0; e < 8; e++) m = fmaxf(m, (float)v[j][e]);
    }
  }
  float s = 0.f;
  const float ml = m * L2E;
#pragma unroll
  for (int j = 0; j < NV; j++)
    if (tid + 1024 * j < nv)
#pragma unroll
      for (int e = 0; e < 8; e++) s += __builtin_amdgcn_exp2f(__builtin_fmaf((float)v[j][e], L2E, -ml));
  // merge (max, sum) pairs: s is relative to m
  auto merge = [](float& m, float& s, float m2, float s2) {
    const float mm = fmaxf(m, m2);
    s = (m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f((m - mm) * L2E)) +
        (m2 == -INFINITY ? 0.f : s2 * __builtin_amdgcn_exp2f((m2 - mm) * L2E));
    m = mm;
  };
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) merge(m, s, __shfl_xor(m, o, WAVE), __shfl_xor(s, o, WAVE));
  if ((tid & 63) == 0) {
    red_m[w] = m;
    red_s[w] = s;
  }
  __syncthreads();
  if (tid == 0) {
    float mm = red_m[0], ss = red_s[0];
    for (int i = 1; i < 16; i++) merge(mm, ss, red_m[i], red_s[i]);
    s_m = mm;
    s_s = ss;
    const bool ok = tgt >= 0 && tgt < Vp;   // an id outside the table yields a NaN loss
    row_loss[row] = mm + logf(ss) - (ok ? (float)zr[tgt] : __builtin_nanf(""));
  }
  __syncthreads();
  const float mrow = s_m * L2E, inv = grad_scale / s_s;
#pragma unroll
  for (int j = 0; j < NV; j++) {
    const int i = tid + 1024 * j;
    if (i < nv) {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        float g = __builtin_amdgcn_exp2f(__builtin_fmaf((float)v[j][e], L2E, -mrow)) * inv;
        if (8 * i + e == tgt) g -= grad_scale;
        o[e] = (bf16)g;
      }
      __builtin_nontemporal_store(__builtin_bit_cast(u32x4, o), (u32x4*)(zr + 8 * i));
    }
  }
}

hipError_t launch_xent(void* z, bool bf16_z, int64_t ldz, const int32_t* y, float* row_loss, int M, int Vp,
                       float grad_scale, hipStream_t s) {
  if (bf16_z && Vp % 8 == 0 && ldz % 8 == 0 && (uintptr_t)z % 16 == 0 && Vp <= 8 * 8192) {
    const int nv = (Vp / 8 + 1023) / 1024;
    switch (nv) {
#define XR(N) \
  case N: hipLaunchKernelGGL((xent_reg_kernel<N>), dim3(M), dim3(1024), 0, s, (bf16*)z, ldz, y, row_loss, Vp, grad_scale); break;
      XR(1) XR(2) XR(3) XR(4) XR(5) XR(6) XR(7) XR(8)
#undef XR
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (bf16_z)
    hipLaunchKernelGGL(xent_kernel<bf16>, dim3(M), dim3(256), 0, s, (bf16*)z, ldz, y, row_loss, Vp, grad_scale);
  else
    hipLaunchKernelGGL(xent_kernel<float>, dim3(M), dim3(256), 0, s, (float*)z, ldz, y, row_loss, Vp,
                       grad_scale);
  return hipGetLastError();
}

__global__ __launch_bounds__(1024) void mean_kernel(const float* __restrict__ x, int M, float* out) {
  __shared__ float red[16];
  float s = 0.f;
  if ((M & 3) == 0 && ((uintptr_t)x & 15) == 0) {
    for (int i = threadIdx.x; i < (M >> 2); i += 1024) {
      const f32x4 v = ((const f32x4*)x)[i];
      s += (v[0] + v[1]) + (v[2] + v[3]);
    }
  } else {
    for (int i = threadIdx.x; i < M; i += 1024) s += x[i];
  }
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int i = 0; i < 16; i++) t += red[i];
    *out = t / (float)M;
  }
}

hipError_t launch_mean(const float* row_loss, int M, float* out, hipStream_t s) {
  hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(1024), 0, s, row_loss, M, out);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- small utilities
// 64 x 64 tiles of every 2-D weight, transposed through LDS with coalesced reads
// and writes; the tensor of a tile is found by binary search over first_tile.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16* __restrict__ src, bf16* __restrict__ dst,
                                                             const TransposeEntry* __restrict__ table, int n) {
  __shared__ bf16 t[64][65];
  const int64_t tile = blockIdx.x;
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (table[mid].first_tile <= tile) lo = mid;
    else hi = mid - 1;
  }
  const TransposeEntry e = table[lo];
  const int64_t local = tile - e.first_tile;
  const int64_t tiles_c = (e.cols + 63) / 64;
  const int64_t r0 = (local / tiles_c) * 64, c0 = (local % tiles_c) * 64;
  const bf16* s0 = src + e.offset;
  bf16* d0 = dst + e.offset;
  if (r0 + 64 <= e.rows && c0 + 64 <= e.cols && e.rows % 8 == 0 && e.cols % 8 == 0 &&
      ((uintptr_t)s0 | (uintptr_t)d0) % 16 == 0) {
    // whole tile, 16-byte rows: each thread moves two runs of 8 elements each way
    __shared__ uint16_t u[64][66];
#pragma unroll
    for (int k = 0; k < 2; k++) {
      const int i = threadIdx.x + 256 * k, rr = i >> 3, cu = (i & 7) * 8;
      const uint4 v = *(const uint4*)(s0 + (r0 + rr) * e.cols + c0 + cu);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; q++) {
        u[rr][cu + 2 * q] = (uint16_t)(w[q] & 0xFFFFu);
        u[rr][cu + 2 * q + 1] = (uint16_t)(w[q] >> 16);
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; k++) {
      const int i = threadIdx.x + 256 * k, cc = i >> 3, ru = (i & 7) * 8;
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; q++) w[q] = (uint32_t)u[ru + 2 * q][cc] | ((uint32_t)u[ru + 2 * q + 1][cc] << 16);
      *(uint4*)(d0 + (c0 + cc) * e.rows + r0 + ru) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    return;
  }
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int rr = i >> 6, cc = i & 63;
    if (r0 + rr < e.rows && c0 + cc < e.cols) t[rr][cc] = s0[(r0 + rr) * e.cols + c0 + cc];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int cc = i >> 6, rr = i & 63;
    if (r0 + rr < e.rows && c0 + cc < e.cols) d0[(c0 + cc) * e.rows + r0 + rr] = t[rr][cc];
  }
}

hipError_t launch_transpose_bf16(const void* src, void* dst, const TransposeEntry* d_table, int n_entries,
                                 int64_t total_tiles, hipStream_t s) {
  if (total_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)total_tiles), dim3(256), 0, s, (const bf16*)src,
                     (bf16*)dst, d_table, n_entries);
  return hipGetLastError();
}

__global__ void cast_bf16_kernel(const float* __restrict__ src, bf16* __restrict__ dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = (bf16)src[i];
}
hipError_t launch_cast_bf16(const float* src, void* dst, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(cast_bf16_kernel, dim3(blocks), dim3(256), 0, s, src, (bf16*)dst, n);
  return hipGetLastError();
}

__global__ void zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}
hipError_t launch_zero(void* p, size_t n_words, hipStream_t s) {
  if (n_words == 0) return hipSuccess;
  unsigned blocks = (unsigned)std::min<size_t>((n_words + 255) / 256, 65536);
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, s, (uint32_t*)p, n_words);
  return hipGetLastError();
}

template <typename T>
__global__ void rows_to_f32_kernel(const T* __restrict__ src, int64_t ld, int M, int N, float* __restrict__ dst) {
  const int64_t total = (int64_t)M * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / N, n = i % N;
    dst[i] = to_f32(src[m * ld + n]);
  }
}
hipError_t launch_rows_to_f32(const void* src, bool bf16_src, int64_t ld, int M, int N, float* dst, hipStream_t s) {
  const int64_t total = (int64_t)M * N;
  if (total == 0) return hipSuccess;
  unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
  if (bf16_src)
    hipLaunchKernelGGL(rows_to_f32_kernel<bf16>, dim3(blocks), dim3(256), 0, s, (const bf16*)src, ld, M, N, dst);
  else
    hipLaunchKernelGGL(rows_to_f32_kernel<float>, dim3(blocks), dim3(256), 0, s, (const float*)src, ld, M, N, dst);
  return hipGetLastError();
}

}  // namespace gpt
