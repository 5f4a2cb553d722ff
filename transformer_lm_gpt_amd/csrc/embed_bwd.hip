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

// four elements of dwpe per thread (T*d is a multiple of 4: d is)
__global__ void wpe_grad_kernel(const float* __restrict__ dx0, float* __restrict__ dwpe, float beta, int B, int T,
                                int d) {
  const int i = 4 * (blockIdx.x * blockDim.x + threadIdx.x);   // over T*d
  if (i >= T * d) return;
  const int64_t td = (int64_t)T * d;
  f32x4 s = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int b = 0; b < B; b++) s += *(const f32x4*)(dx0 + b * td + i);
  f32x4* dst = (f32x4*)(dwpe + i);
  *dst = beta != 0.f ? beta * *dst + s : s;
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
// The chunk's rows are all fetched before the in-order walk (four columns per
// thread), so the walk waits on one round of loads, not on PIECE.
__global__ __launch_bounds__(256) void piece_sum_kernel(const uint32_t* __restrict__ keys, const float* __restrict__ dx0,
                                                        float* __restrict__ piece_sums, int M, int shift, int d) {
  __shared__ uint32_t ks[PIECE];
  const int i0 = blockIdx.x * PIECE;
  const int n = min(M - i0, PIECE);
  if ((int)threadIdx.x < n) ks[threadIdx.x] = keys[i0 + threadIdx.x];
  __syncthreads();
  const uint32_t mask = (1u << shift) - 1u;
  for (int c = 4 * threadIdx.x; c < d; c += 4 * 256) {
    f32x4 x[PIECE];
#pragma unroll
    for (int i = 0; i < PIECE; i++)
      if (i < n) x[i] = *(const f32x4*)(dx0 + (int64_t)(ks[i] & mask) * d + c);
    int start = 0;
    uint32_t cur = ks[0] >> shift;
    f32x4 sum = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < PIECE; i++) {
      if (i < n) {
        const uint32_t id = ks[i] >> shift;
        if (id != cur) {
          *(f32x4*)(piece_sums + (int64_t)(i0 + start) * d + c) = sum;
          sum = (f32x4){0.f, 0.f, 0.f, 0.f};
          start = i;
          cur = id;
        }
        sum += x[i];
      }
    }
    *(f32x4*)(piece_sums + (int64_t)(i0 + start) * d + c) = sum;
  }
}

// Every run of one id adds its chunk sums (at the run's first position and at each
// chunk boundary inside the run), in order, into dwte[id]. A workgroup covers
// SEG_POS sorted positions and takes the run starts among them one after another,
// four columns per thread; the chunk sums of a long run (the most frequent ids)
// are fetched four at a time.
constexpr int SEG_POS = 16;
__global__ __launch_bounds__(256) void segment_add_kernel(const uint32_t* __restrict__ keys,
                                                          const float* __restrict__ piece_sums,
                                                          float* __restrict__ dwte, int M, int shift, int d,
                                                          int Vp) {
  __shared__ uint32_t ids[SEG_POS + 1];   // ids[0]: the id before the first position (none: ~0)
  __shared__ int lasts[SEG_POS];          // a run's last chunk boundary (its first position if none)
  const int i0 = blockIdx.x * SEG_POS;
  const int n = min(M - i0, SEG_POS);
  if ((int)threadIdx.x <= n)
    ids[threadIdx.x] = threadIdx.x == 0 ? (i0 > 0 ? keys[i0 - 1] >> shift : ~0u) : keys[i0 + threadIdx.x - 1] >> shift;
  __syncthreads();
  if ((int)threadIdx.x < n) {
    const uint32_t id = ids[threadIdx.x + 1];
    const int first = i0 + threadIdx.x;
    int last = first;
    if (id != ids[threadIdx.x]) {
      // the run ends before the first sorted position e with another id (binary search)
      int lo = first + 1, hi = M;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((keys[mid] >> shift) == id) lo = mid + 1;
        else hi = mid;
      }
      last = max(first, (lo - 1) / PIECE * PIECE);
    }
    lasts[threadIdx.x] = last;
  }
  __syncthreads();
  for (int i = 0; i < n; i++) {
    const uint32_t id = ids[i + 1];
    if (id == ids[i] || id >= (uint32_t)Vp) continue;   // not a run start, or outside the table (dropped)
    const int first = i0 + i, last = lasts[i];
    for (int c = 4 * threadIdx.x; c < d; c += 4 * 256) {
      const float* ps = piece_sums + c;
      f32x4 sum = *(const f32x4*)(ps + (int64_t)first * d);
      int j = (first / PIECE + 1) * PIECE;
      for (; j + 3 * PIECE <= last; j += 4 * PIECE) {
        const f32x4 a = *(const f32x4*)(ps + (int64_t)j * d), b = *(const f32x4*)(ps + (int64_t)(j + PIECE) * d);
        const f32x4 e = *(const f32x4*)(ps + (int64_t)(j + 2 * PIECE) * d);
        const f32x4 f = *(const f32x4*)(ps + (int64_t)(j + 3 * PIECE) * d);
        sum += a;
        sum += b;
        sum += e;
        sum += f;
      }
      for (; j <= last; j += PIECE) sum += *(const f32x4*)(ps + (int64_t)j * d);
      f32x4* dst = (f32x4*)(dwte + (int64_t)id * d + c);
      *dst = *dst + sum;
    }
  }
}

hipError_t launch_embed_bwd(const float* dx0, const int32_t* tok, float* dwte, float* dwpe, float beta_wpe, int B,
                            int T, int d, int Vp, EmbedBwdScratch scr, hipStream_t s) {
  const int M = B * T;
  const int shift = ceil_log2(M < 2 ? 2 : M);
  const int n = 1 << ceil_log2(M < 16 ? 16 : M);   // sort size: at least one thread's 16 keys
  if (n > SORT_MAX || ((uint64_t)Vp << shift) > 0xFFFFFFFFull) return hipErrorInvalidValue;
  // four columns per access
  if (d % 4 != 0 || (uintptr_t)dx0 % 16 != 0 || (uintptr_t)dwte % 16 != 0 || (uintptr_t)scr.piece_sums % 16 != 0)
    return hipErrorInvalidValue;
  if ((uintptr_t)dwpe % 16 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(wpe_grad_kernel, dim3((T * d / 4 + 255) / 256), dim3(256), 0, s, dx0, dwpe, beta_wpe, B, T, d);
  if (M <= RADIX_MAX) {
    const int passes = (ceil_log2(Vp < 2 ? 2 : Vp) + 3) / 4;
    hipLaunchKernelGGL(radix_sort_keys_kernel, dim3(1), dim3(RADIX_THREADS), 0, s, tok, M, shift, passes, scr.keys);
    hipLaunchKernelGGL(piece_sum_kernel, dim3((M + PIECE - 1) / PIECE), dim3(256), 0, s, (const uint32_t*)scr.keys,
                       dx0, scr.piece_sums, M, shift, d);
    hipLaunchKernelGGL(segment_add_kernel, dim3((M + SEG_POS - 1) / SEG_POS), dim3(256), 0, s, (const uint32_t*)scr.keys,
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
  hipLaunchKernelGGL(segment_add_kernel, dim3((M + SEG_POS - 1) / SEG_POS), dim3(256), 0, s, (const uint32_t*)scr.keys,
                     (const float*)scr.piece_sums, dwte, M, shift, d, Vp);
  return hipGetLastError();
}

}  // namespace gpt
