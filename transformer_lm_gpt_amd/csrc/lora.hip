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

// W_eff[n, k] = W0[n, k] + s * sum_j B[n, j] A[j, k] for one d x d block per job
// (blockIdx.z), written as fp32 and/or bf16 (round to nearest even).
__global__ __launch_bounds__(256) void lora_merge_kernel(const LoraJob* __restrict__ jobs, int d, int r,
                                                          float s) {
  const LoraJob& jb = jobs[blockIdx.z];
  const int n = blockIdx.y;
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= d) return;
  const float* Brow = jb.B + (size_t)n * r;
  float acc = 0.f;
  for (int j = 0; j < r; j++) acc = fmaf(Brow[j], jb.A[(size_t)j * d + k], acc);
  const size_t e = (size_t)n * d + k;
  const float w = jb.W0[e] + s * acc;
  if (jb.weff) jb.weff[e] = w;
  if (jb.weff_bf16) ((bf16*)jb.weff_bf16)[e] = (bf16)w;
}

// dB[n, j] = beta * dB[n, j] + s * sum_k dW[n, k] A[j, k]: one workgroup per row n
// of one job; each thread takes columns k = t, t + 256, ...; per j the four
// wavefronts reduce in a fixed order.
constexpr int LORA_MAX_RANK = 64;
__global__ __launch_bounds__(256) void lora_grad_b_kernel(const LoraJob* __restrict__ jobs, int d, int r, float s,
                                                          float beta) {
  __shared__ float red[4][LORA_MAX_RANK];
  const LoraJob& jb = jobs[blockIdx.y];
  const int n = blockIdx.x;
  const int t = threadIdx.x, wv = t >> 6;
  const float* dWrow = jb.dW + (size_t)n * d;
  for (int j = 0; j < r; j++) {
    const float* Arow = jb.A + (size_t)j * d;
    float p = 0.f;
    for (int k = t; k < d; k += 256) p = fmaf(dWrow[k], Arow[k], p);
    p = wave_sum(p);
    if ((t & 63) == 0) red[wv][j] = p;
  }
  __syncthreads();
  if (t < r) {
    const float sum = ((red[0][t] + red[1][t]) + red[2][t]) + red[3][t];
    float* o = jb.dB + (size_t)n * r + t;
    *o = (beta != 0.f ? beta * *o : 0.f) + s * sum;
  }
}

// dA[j, k] = beta * dA[j, k] + s * sum_n B[n, j] dW[n, k]: one thread per column k
// walks the d rows in order, eight ranks at a time.
__global__ __launch_bounds__(64) void lora_grad_a_kernel(const LoraJob* __restrict__ jobs, int d, int r, float s,
                                                         float beta) {
  const LoraJob& jb = jobs[blockIdx.y];
  const int k = blockIdx.x * 64 + threadIdx.x;
  if (k >= d) return;
  for (int j0 = 0; j0 < r; j0 += 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = 0.f;
    for (int n = 0; n < d; n++) {
      const float w = jb.dW[(size_t)n * d + k];
      const float* Brow = jb.B + (size_t)n * r + j0;
#pragma unroll
      for (int i = 0; i < 8; i++)
        if (j0 + i < r) acc[i] = fmaf(Brow[i], w, acc[i]);
    }
#pragma unroll
    for (int i = 0; i < 8; i++) {
      if (j0 + i < r) {
        float* o = jb.dA + (size_t)(j0 + i) * d + k;
        *o = (beta != 0.f ? beta * *o : 0.f) + s * acc[i];
      }
    }
  }
}

hipError_t launch_lora_merge(const LoraJob* jobs, int njobs, int d, int r, float s, hipStream_t st) {
  if (njobs <= 0) return hipSuccess;
  if (r < 1 || r > LORA_MAX_RANK || d < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lora_merge_kernel, dim3((d + 255) / 256, d, njobs), dim3(256), 0, st, jobs, d, r, s);
  return hipGetLastError();
}

hipError_t launch_lora_grad(const LoraJob* jobs, int njobs, int d, int r, float s, float beta, hipStream_t st) {
  if (njobs <= 0) return hipSuccess;
  if (r < 1 || r > LORA_MAX_RANK || d < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lora_grad_b_kernel, dim3(d, njobs), dim3(256), 0, st, jobs, d, r, s, beta);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lora_grad_a_kernel, dim3((d + 63) / 64, njobs), dim3(64), 0, st, jobs, d, r, s, beta);
  return hipGetLastError();
}

}  // namespace gpt
