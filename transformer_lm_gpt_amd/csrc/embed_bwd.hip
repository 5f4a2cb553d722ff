// Embedding backward, deterministic.
//
// x0[b, t] = wte[tok[b, t]] + wpe[t], so
//   dwpe[t]  = sum_b dx0[b, t]
//   dwte[id] += sum over positions m with tok[m] == id of dx0[m]
// (the second adds to the lm_head contribution of the tied embedding).
// Repeated ids are frequent (Zipf-distributed tokens put about an eighth of all
// positions on one id), so the scatter is done without float atomics: the
// (id, position) pairs are sorted in LDS by one workgroup, the sorted list is
// cut into fixed chunks whose same-id runs are summed in order, and every
// distinct id then adds its run sums in order. The summation order depends only
// on the token ids, never on scheduling.
#include "common.h"
#include "kernels.h"

namespace gpt {

constexpr int PIECE = 32;          // sorted positions per chunk
constexpr int SORT_MAX = 32768;    // keys sorted in one workgroup's LDS

static int ceil_log2(int x) {
  int s = 0;
  while ((1 << s) < x) s++;
  return s;
}

int embed_bwd_sort_size(int M) { return 1 << ceil_log2(M < 16 ? 16 : M); }

__global__ void wpe_grad_kernel(const float* __restrict__ dx0, float* __restrict__ dwpe, float beta, int B, int T,
                                int d) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;   // over T*d
  if (i >= T * d) return;
  float s = 0.f;
  for (int b = 0; b < B; b++) s += dx0[(int64_t)b * T * d + i];
  dwpe[i] = (beta != 0.f ? beta * dwpe[i] : 0.f) + s;
}

// Bitonic sort of n (a power of two, at least 16) keys (id << shift) | position in
// LDS. Distances j >= 16 run as LDS passes over the n/2 compare-exchange pairs;
// the four distances below 16 of every stage run in registers, each thread holding
// 16 consecutive keys, so only about half the passes need a barrier.
__device__ inline void cas(uint32_t& a, uint32_t& b, bool up) {
  if ((a > b) == up) {
    const uint32_t t = a;
    a = b;
    b = t;
  }
}

__global__ __launch_bounds__(1024) void sort_keys_kernel(const int32_t* __restrict__ tok, int M, int shift, int n,
                                                         uint32_t* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint32_t sk[];
  for (int i = threadIdx.x; i < n; i += 1024)
    sk[i] = i < M ? (((uint32_t)tok[i]) << shift) | (uint32_t)i : 0xFFFFFFFFu;
  __syncthreads();
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j >= 16; j >>= 1) {
      int lj = 0;
      while ((1 << lj) < j) lj++;
      for (int q = threadIdx.x; q < (n >> 1); q += 1024) {
        const int i = ((q >> lj) << (lj + 1)) | (q & (j - 1));   // i has bit lj clear; partner i + j
        uint32_t a = sk[i], b = sk[i + j];
        cas(a, b, (i & k) == 0);
        sk[i] = a;
        sk[i + j] = b;
      }
      __syncthreads();
    }
    // distances 8, 4, 2, 1 (those below k) inside each thread's 16 consecutive keys
    for (int base = threadIdx.x * 16; base < n; base += 1024 * 16) {
      uint32_t v[16];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const uint4 w = *(const uint4*)(sk + base + 4 * q);
        v[4 * q] = w.x;
        v[4 * q + 1] = w.y;
        v[4 * q + 2] = w.z;
        v[4 * q + 3] = w.w;
      }
      const bool up = (base & k) == 0;                          // the same for all 16 when k >= 16
#pragma unroll
      for (int j = 8; j >= 1; j >>= 1) {
        if (j >= k) continue;
#pragma unroll
        for (int e = 0; e < 16; e++)
          if ((e & j) == 0) cas(v[e], v[e + j], k >= 16 ? up : (((base + e) & k) == 0));
      }
#pragma unroll
      for (int q = 0; q < 4; q++) *(uint4*)(sk + base + 4 * q) = make_uint4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < M; i += 1024) out[i] = sk[i];
}

// Stable LSD radix sort of the same keys by id, 4 bits per pass, for M <= RADIX_MAX
// (two key buffers and the per-thread digit counters fit in LDS). The keys start
// in position order and positions are unique, so the result equals the bitonic
// sort's. Thread t owns the KPT consecutive keys from t*KPT. Each pass: every
// thread counts its digits in its own LDS row of sixteen 16-bit counters; the
// rows, read as eight 32-bit words holding two counters each, are scanned over
// the wavefront (the counters never exceed M < 2^16, so the pairs add without
// carries) and then over the wavefronts; each thread turns its row into the
// destination of its first key of each digit and scatters its keys in order.
constexpr int RADIX_MAX = 15360;
constexpr int RADIX_THREADS = 1024;
constexpr int RADIX_KPT = RADIX_MAX / RADIX_THREADS;

__device__ inline uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

__global__ __launch_bounds__(RADIX_THREADS) void radix_sort_keys_kernel(const int32_t* __restrict__ tok, int M,
                                                                        int shift, int passes,
                                                                        uint32_t* __restrict__ out) {
  __shared__ uint32_t buf[2][RADIX_MAX];
  __shared__ uint32_t cnt[RADIX_THREADS][8];      // digit 2q in the low half of word q, 2q+1 in the high half
  __shared__ uint32_t wtot[RADIX_THREADS / 64][8];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int kpt = (M + RADIX_THREADS - 1) / RADIX_THREADS;
  const int k0 = t * kpt, k1 = min(M, k0 + kpt);
  for (int i = t; i < M; i += RADIX_THREADS) buf[0][i] = (((uint32_t)tok[i]) << shift) | (uint32_t)i;
  __syncthreads();
  for (int p = 0; p < passes; p++) {
    const uint32_t* src = buf[p & 1];
    uint32_t* dst = buf[(p & 1) ^ 1];
    const int dsh = shift + 4 * p;
#pragma unroll
    for (int q = 0; q < 8; q++) cnt[t][q] = 0u;
    for (int j = k0; j < k1; j++) {
      const uint32_t dg = (src[j] >> dsh) & 15u;
      cnt[t][dg >> 1] += 1u << ((dg & 1u) << 4);
    }
    // exclusive prefix of the counters over the threads before t
    uint32_t c[8], inc[8];
#pragma unroll
    for (int q = 0; q < 8; q++) {
      c[q] = cnt[t][q];
      inc[q] = wave_incl_scan(c[q]);
    }
    if (lane == 63)
#pragma unroll
      for (int q = 0; q < 8; q++) wtot[w][q] = inc[q];
    __syncthreads();
    uint32_t before[8], total[8];
#pragma unroll
    for (int q = 0; q < 8; q++) before[q] = total[q] = 0u;
    for (int v = 0; v < RADIX_THREADS / 64; v++)
#pragma unroll
      for (int q = 0; q < 8; q++) {
        const uint32_t x = wtot[v][q];
        total[q] += x;
        if (v < w) before[q] += x;
      }
    // destination of this thread's first key of each digit: the digit's base (an
    // exclusive scan of the sixteen totals, in digit order) plus the keys of that
    // digit in earlier threads
    uint32_t base = 0u, first[8];
#pragma unroll
    for (int q = 0; q < 8; q++) {
      const uint32_t mine = before[q] + inc[q] - c[q];
      const uint32_t lo = base + (mine & 0xFFFFu);
      base += total[q] & 0xFFFFu;
      const uint32_t hi = base + (mine >> 16);
      base += total[q] >> 16;
      first[q] = lo | (hi << 16);
    }
#pragma unroll
    for (int q = 0; q < 8; q++) cnt[t][q] = first[q];
    for (int j = k0; j < k1; j++) {
      const uint32_t k = src[j];
      const uint32_t dg = (k >> dsh) & 15u, sh = (dg & 1u) << 4;
      const uint32_t word = cnt[t][dg >> 1];
      dst[(word >> sh) & 0xFFFFu] = k;
      cnt[t][dg >> 1] = word + (1u << sh);
    }
    __syncthreads();
  }
  const uint32_t* res = buf[passes & 1];
  for (int i = t; i < M; i += RADIX_THREADS) out[i] = res[i];
}

// One workgroup per chunk of PIECE sorted positions: walks them in order and
// writes the sum of every same-id run to piece_sums[first position of the run].
__global__ __launch_bounds__(256) void piece_sum_kernel(const uint32_t* __restrict__ keys, const float* __restrict__ dx0,
                                                        float* __restrict__ piece_sums, int M, int shift, int d) {
  const int i0 = blockIdx.x * PIECE;
  const int i1 = min(M, i0 + PIECE);
  const uint32_t mask = (1u << shift) - 1u;
  for (int c = threadIdx.x; c < d; c += 256) {
    int start = i0;
    uint32_t cur = keys[i0] >> shift;
    float s = 0.f;
    for (int i = i0; i < i1; i++) {
      const uint32_t k = keys[i];
      const uint32_t id = k >> shift;
      if (id != cur) {
        piece_sums[(int64_t)start * d + c] = s;
        s = 0.f;
        start = i;
        cur = id;
      }
      s += dx0[(int64_t)(k & mask) * d + c];
    }
    piece_sums[(int64_t)start * d + c] = s;
  }
}

// One workgroup per sorted position; those that start an id's run add the run's
// chunk sums, in order, into dwte[id].
__global__ __launch_bounds__(256) void segment_add_kernel(const uint32_t* __restrict__ keys,
                                                          const float* __restrict__ piece_sums,
                                                          float* __restrict__ dwte, int M, int shift, int d,
                                                          int Vp) {
  const int i = blockIdx.x;
  const uint32_t id = keys[i] >> shift;
  if (i > 0 && (keys[i - 1] >> shift) == id) return;
  if (id >= (uint32_t)Vp) return;   // ids outside the table are dropped, never written
  // pieces of this run start at i and at every chunk boundary inside the run
  for (int c = threadIdx.x; c < d; c += 256) {
    float s = piece_sums[(int64_t)i * d + c];
    for (int j = (i / PIECE + 1) * PIECE; j < M && (keys[j] >> shift) == id; j += PIECE)
      s += piece_sums[(int64_t)j * d + c];
    dwte[(int64_t)id * d + c] += s;
  }
}

hipError_t launch_embed_bwd(const float* dx0, const int32_t* tok, float* dwte, float* dwpe, float beta_wpe, int B,
                            int T, int d, int Vp, EmbedBwdScratch scr, hipStream_t s) {
  const int M = B * T;
  const int shift = ceil_log2(M < 2 ? 2 : M);
  const int n = 1 << ceil_log2(M < 16 ? 16 : M);   // sort size: at least one thread's 16 keys
  if (n > SORT_MAX || ((uint64_t)Vp << shift) > 0xFFFFFFFFull) return hipErrorInvalidValue;
  hipLaunchKernelGGL(wpe_grad_kernel, dim3((T * d + 255) / 256), dim3(256), 0, s, dx0, dwpe, beta_wpe, B, T, d);
  if (M <= RADIX_MAX) {
    const int passes = (ceil_log2(Vp < 2 ? 2 : Vp) + 3) / 4;
    hipLaunchKernelGGL(radix_sort_keys_kernel, dim3(1), dim3(RADIX_THREADS), 0, s, tok, M, shift, passes, scr.keys);
    hipLaunchKernelGGL(piece_sum_kernel, dim3((M + PIECE - 1) / PIECE), dim3(256), 0, s, (const uint32_t*)scr.keys,
                       dx0, scr.piece_sums, M, shift, d);
    hipLaunchKernelGGL(segment_add_kernel, dim3(M), dim3(256), 0, s, (const uint32_t*)scr.keys,
                       (const float*)scr.piece_sums, dwte, M, shift, d, Vp);
    return hipGetLastError();
  }
  const size_t lds = (size_t)n * sizeof(uint32_t);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)sort_keys_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(sort_keys_kernel, dim3(1), dim3(1024), lds, s, tok, M, shift, n, scr.keys);
  hipLaunchKernelGGL(piece_sum_kernel, dim3((M + PIECE - 1) / PIECE), dim3(256), 0, s, (const uint32_t*)scr.keys,
                     dx0, scr.piece_sums, M, shift, d);
  hipLaunchKernelGGL(segment_add_kernel, dim3(M), dim3(256), 0, s, (const uint32_t*)scr.keys,
                     (const float*)scr.piece_sums, dwte, M, shift, d, Vp);
  return hipGetLastError();
}

}  // namespace gpt
