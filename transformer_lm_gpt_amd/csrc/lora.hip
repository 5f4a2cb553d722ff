// Low-rank adapters on the q and v projections (the fine-tuning article on
// blog.hotdry.top, LoRA section): W0 stays frozen and only A [r, d] and
// B [d, r] train, the branch adding s B A x with s = lora_alpha / r. The
// article's merge of B A into W0 is how the forward runs here: after every
// update the q and v row blocks of the GEMM operand weight become
// W0 + s B A, so the forward and the input gradients use the base path's GEMMs
// unchanged. The adapters' gradients follow from the q (or v) weight gradient
// dW = dq^T a that the base path's weight-gradient GEMM forms:
//   dB = s dW A^T   ([d, r]),   dA = s B^T dW   ([r, d]).
// Both are fixed-order fp32 reductions with no atomics.
#include "common.h"
#include "kernels.h"

namespace gpt {

// Columns are taken four at a time: lane c of a wavefront holds columns
// 4c + 256i .. 4c + 256i + 3 for i < ceil(d / 256) (d is a multiple of 4 and at
// most 1024, so at most four float4 per lane).
constexpr int LORA_MAX_RANK = 64;
constexpr int LORA_MAX_NI = 4;

__device__ inline f32x4 ld4(const float* p) { return *(const f32x4*)p; }

// W_eff[n, k] = W0[n, k] + s * sum_j B[n, j] A[j, k], one wavefront per row n of
// one job (blockIdx.y), written as fp32 and/or bf16 (round to nearest even).
__global__ __launch_bounds__(256) void lora_merge_kernel(const LoraJob* __restrict__ jobs, int d, int r,
                                                          float s) {
  const LoraJob jb = jobs[blockIdx.y];
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (n >= d) return;
  f32x4 acc[LORA_MAX_NI];
#pragma unroll
  for (int i = 0; i < LORA_MAX_NI; i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float* Brow = jb.B + (size_t)n * r;
  for (int j = 0; j < r; j++) {
    const float b = Brow[j];
    const float* Arow = jb.A + (size_t)j * d;
#pragma unroll
    for (int i = 0; i < LORA_MAX_NI; i++) {
      const int k = 4 * lane + 256 * i;
      if (k < d) acc[i] += b * ld4(Arow + k);
    }
  }
#pragma unroll
  for (int i = 0; i < LORA_MAX_NI; i++) {
    const int k = 4 * lane + 256 * i;
    if (k >= d) continue;
    const size_t e = (size_t)n * d + k;
    const f32x4 w = ld4(jb.W0 + e) + s * acc[i];
    if (jb.weff) *(f32x4*)(jb.weff + e) = w;
    if (jb.weff_bf16) {
      bf16x4 o;
      o[0] = (bf16)w[0]; o[1] = (bf16)w[1]; o[2] = (bf16)w[2]; o[3] = (bf16)w[3];
      *(bf16x4*)((bf16*)jb.weff_bf16 + e) = o;
    }
  }
}

// dB[n, j] = beta * dB[n, j] + s * sum_k dW[n, k] A[j, k]: one wavefront per four rows
// n of one job (each row of A is read once for the four); the rows of dW stay in
// registers, and per j and row the 64 lanes reduce in a fixed order (lane j keeps
// the sum, lanes < r store).
constexpr int LORA_B_ROWS = 4;
__global__ __launch_bounds__(256) void lora_grad_b_kernel(const LoraJob* __restrict__ jobs, int d, int r, float s,
                                                          float beta) {
  const LoraJob jb = jobs[blockIdx.y];
  const int n0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * LORA_B_ROWS, lane = threadIdx.x & 63;
  if (n0 >= d) return;
  f32x4 w[LORA_B_ROWS][LORA_MAX_NI];
#pragma unroll
  for (int q = 0; q < LORA_B_ROWS; q++)
#pragma unroll
    for (int i = 0; i < LORA_MAX_NI; i++) {
      const int k = 4 * lane + 256 * i;
      w[q][i] = k < d && n0 + q < d ? ld4(jb.dW + (size_t)(n0 + q) * d + k) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  float mine[LORA_B_ROWS];
#pragma unroll
  for (int q = 0; q < LORA_B_ROWS; q++) mine[q] = 0.f;
  for (int j = 0; j < r; j++) {
    const float* Arow = jb.A + (size_t)j * d;
    f32x4 a[LORA_MAX_NI];
#pragma unroll
    for (int i = 0; i < LORA_MAX_NI; i++) {
      const int k = 4 * lane + 256 * i;
      a[i] = k < d ? ld4(Arow + k) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int q = 0; q < LORA_B_ROWS; q++) {
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < LORA_MAX_NI; i++)
        if (4 * lane + 256 * i < d)
          p += (w[q][i][0] * a[i][0] + w[q][i][1] * a[i][1]) + (w[q][i][2] * a[i][2] + w[q][i][3] * a[i][3]);
      p = wave_sum(p);
      if (lane == j) mine[q] = p;
    }
  }
#pragma unroll
  for (int q = 0; q < LORA_B_ROWS; q++) {
    if (lane < r && n0 + q < d) {
      float* o = jb.dB + (size_t)(n0 + q) * r + lane;
      *o = (beta != 0.f ? beta * *o : 0.f) + s * mine[q];
    }
  }
}

// dA[j, k] = beta * dA[j, k] + s * sum_n B[n, j] dW[n, k]: a workgroup takes 256
// columns of one job and eight ranks (blockIdx.z), its four wavefronts a quarter of
// the rows each (in order, loads fetched eight rows ahead), with those ranks' column
// of B staged in LDS (zero past r); the quarters are added in wavefront order.
constexpr int LORA_JC = 8;
typedef const f32x4 __attribute__((address_space(1)))* gf32x4p;   // global memory
__global__ __launch_bounds__(256) void lora_grad_a_kernel(const LoraJob* __restrict__ jobs, int d, int r, float s,
                                                          float beta) {
  __shared__ f32x4 part[3][LORA_JC][64];
  __shared__ f32x4 bsh[1024 * LORA_JC / 4];   // B[n, j0 .. j0 + 8) for every row n (d <= 1024)
  const LoraJob jb = jobs[blockIdx.y];
  const float* dW = jb.dW;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int k = blockIdx.x * 256 + 4 * lane;
  const bool live = k < d;
  const int rows = (d + 3) / 4, n0 = wv * rows, n1 = min(d, n0 + rows);
  {
    const int j0 = blockIdx.z * LORA_JC;
    float* bs = (float*)bsh;
    for (int e = threadIdx.x; e < d * LORA_JC; e += 256) {
      const int n = e / LORA_JC, j = j0 + e % LORA_JC;
      bs[e] = j < r ? jb.B[(size_t)n * r + j] : 0.f;
    }
    __syncthreads();
    f32x4 acc[LORA_JC];
#pragma unroll
    for (int i = 0; i < LORA_JC; i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (live) {
      for (int nb = n0; nb < n1; nb += 8) {
        f32x4 w[8];
#pragma unroll
        for (int u = 0; u < 8; u++)
          w[u] = nb + u < n1 ? *(gf32x4p)(dW + (size_t)(nb + u) * d + k) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 8; u++) {
          const int n = min(nb + u, d - 1);   // rows past n1 carry w = 0
          const f32x4 b0 = bsh[n * 2], b1 = bsh[n * 2 + 1];
          acc[0] += b0[0] * w[u]; acc[1] += b0[1] * w[u]; acc[2] += b0[2] * w[u]; acc[3] += b0[3] * w[u];
          acc[4] += b1[0] * w[u]; acc[5] += b1[1] * w[u]; acc[6] += b1[2] * w[u]; acc[7] += b1[3] * w[u];
        }
      }
    }
    if (wv > 0) {
#pragma unroll
      for (int i = 0; i < LORA_JC; i++) part[wv - 1][i][lane] = acc[i];
    }
    __syncthreads();
    if (wv == 0 && live) {
#pragma unroll
      for (int i = 0; i < LORA_JC; i++) {
        if (j0 + i >= r) continue;
        const f32x4 t = ((acc[i] + part[0][i][lane]) + part[1][i][lane]) + part[2][i][lane];
        f32x4* o = (f32x4*)(jb.dA + (size_t)(j0 + i) * d + k);
        *o = (beta != 0.f ? beta * *o : f32x4{0.f, 0.f, 0.f, 0.f}) + s * t;
      }
    }
  }
}

hipError_t launch_lora_merge(const LoraJob* jobs, int njobs, int d, int r, float s, hipStream_t st) {
  if (njobs <= 0) return hipSuccess;
  if (r < 1 || r > LORA_MAX_RANK || d < 1) return hipErrorInvalidValue;
  if (d % 4 != 0 || d > 256 * LORA_MAX_NI) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lora_merge_kernel, dim3((d + 3) / 4, njobs), dim3(256), 0, st, jobs, d, r, s);
  return hipGetLastError();
}

hipError_t launch_lora_grad(const LoraJob* jobs, int njobs, int d, int r, float s, float beta, hipStream_t st) {
  if (njobs <= 0) return hipSuccess;
  if (r < 1 || r > LORA_MAX_RANK || d < 1 || d % 4 != 0 || d > 256 * LORA_MAX_NI) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lora_grad_b_kernel, dim3((d + 4 * LORA_B_ROWS - 1) / (4 * LORA_B_ROWS), njobs), dim3(256), 0, st,
                     jobs, d, r, s, beta);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lora_grad_a_kernel, dim3((d + 255) / 256, njobs, (r + LORA_JC - 1) / LORA_JC), dim3(256), 0, st,
                     jobs, d, r, s, beta);
  return hipGetLastError();
}

}  // namespace gpt
