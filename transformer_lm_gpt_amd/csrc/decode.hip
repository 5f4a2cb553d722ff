// Inference with a key/value cache: one new token per sequence against the keys
// and values of every earlier position ("GPT training and inference from scratch
// with nanoGPT", section 4; the microGPT page's single-GPU inference section: the
// cache grows by one position per generated token), and the token draw
// (temperature, top-k cut, softmax, one uniform per row).
//
// Cache layout: per layer [B_max * T_max, 2 * d] in operand type, row b * T_max + t,
// keys in columns [0, d) and values in [d, 2d), head h at columns h * hd of each.
#include <cstdlib>

#include "common.h"
#include "kernels.h"

namespace gpt {

// x[b, :] = wte[tok[b], :] + wpe[pos, :] (NaN for an id outside the table), pos read
// from device memory and clamped to the table's Tmax rows.
__global__ void embed_pos_kernel(const float* __restrict__ wte, const float* __restrict__ wpe,
                                 const int32_t* __restrict__ tok, float* __restrict__ x, int B, int d, int Vp,
                                 const int* __restrict__ pos_p, int Tmax) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * d) return;
  const int b = i / d, c = i % d;
  const int id = tok[b];
  const int pos = min(max(*pos_p, 0), Tmax - 1);
  x[i] = (id >= 0 && id < Vp) ? wte[(int64_t)id * d + c] + wpe[(int64_t)pos * d + c] : __builtin_nanf("");
}

hipError_t launch_embed_pos(const float* wte, const float* wpe, const int32_t* tok, float* x, int B, int d, int Vp,
                            const int* pos, int Tmax, hipStream_t s) {
  if (!pos || Tmax < 1) return hipErrorInvalidValue;
  const int n = B * d;
  hipLaunchKernelGGL(embed_pos_kernel, dim3((n + 255) / 256), dim3(256), 0, s, wte, wpe, tok, x, B, d, Vp, pos, Tmax);
  return hipGetLastError();
}

__global__ void set_i32_kernel(int* p, int v) {
  if (threadIdx.x == 0) *p = v;
}

hipError_t launch_set_i32(int* p, int v, hipStream_t s) {
  hipLaunchKernelGGL(set_i32_kernel, dim3(1), dim3(64), 0, s, p, v);
  return hipGetLastError();
}

// cache[b * Tmax + pos0 + t, c] = qkv[b * T + t, d + c] for c < 2d: the keys and values
// of T new positions of every sequence.
template <typename T>
__global__ void kv_append_kernel(const T* __restrict__ qkv, T* __restrict__ cache, int B, int Tn, int Tmax,
                                 int pos0, int d) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_row = 2 * (int64_t)d;
  if (i >= (int64_t)B * Tn * per_row) return;
  const int64_t r = i / per_row;
  const int c = (int)(i % per_row);
  const int b = (int)(r / Tn), t = (int)(r % Tn);
  cache[((int64_t)b * Tmax + pos0 + t) * per_row + c] = qkv[r * 3 * d + d + c];
}

hipError_t launch_kv_append(const void* qkv, bool bf16_ops, void* cache, int B, int T, int Tmax, int pos0, int d,
                            hipStream_t s) {
  if (pos0 < 0 || pos0 + T > Tmax) return hipErrorInvalidValue;
  const int64_t n = (int64_t)B * T * 2 * d;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (bf16_ops)
    hipLaunchKernelGGL(kv_append_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)qkv, (bf16*)cache, B, T, Tmax,
                       pos0, d);
  else
    hipLaunchKernelGGL(kv_append_kernel<float>, grid, dim3(256), 0, s, (const float*)qkv, (float*)cache, B, T,
                       Tmax, pos0, d);
  return hipGetLastError();
}

// One query per (sequence, head) against keys 0 .. len-1, len = *pos + 1 read from
// device memory (clamped to [1, Tmax]):
// s_j = q . k_j / sqrt(hd), p = softmax(s), o = sum_j p_j v_j. One workgroup of 256
// per (b, h); the scores of all keys sit in LDS (len <= DEC_MAX_T). Keys and values
// 0 .. len-2 come from the cache; those of the new position len-1 are read from this
// step's qkv row, and the workgroup also stores them (its head's columns) into the
// cache row len-1 for later steps, which no workgroup of this launch reads. For the value sum
// with 16-byte rows, thread t takes 8 columns (t mod hd/8) of every (256 / (hd/8))-th
// key, and the per-slot partial vectors are added in slot order; otherwise each
// wavefront takes every fourth key with a lane per column.
constexpr int DEC_MAX_T = 8192;

// GPT_DECODE_ATTN_VEC=0: the bf16 decode attention on attn_decode_kernel (for comparisons).
static bool decode_attn_vec() {
  static int on = -1;
  if (on < 0) {
    const char* e = std::getenv("GPT_DECODE_ATTN_VEC");
    on = (e && e[0] == '0') ? 0 : 1;
  }
  return on == 1;
}
template <typename T>
__global__ __launch_bounds__(256) void attn_decode_kernel(const T* __restrict__ qkv, T* __restrict__ cache,
                                                          T* __restrict__ out, int H, int hd, int Tmax,
                                                          const int* __restrict__ pos, float scale) {
  const int len = min(max(*pos + 1, 1), Tmax);
  __shared__ float sc[DEC_MAX_T];
  __shared__ float qs[64];
  __shared__ float red[4][64];
  __shared__ float vred[256 * 8];
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int d = H * hd;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const T* qrow = qkv + (int64_t)b * 3 * d + h * hd;   // this head's q; its k at + d, v at + 2d
  T* kb = cache + (int64_t)b * Tmax * 2 * d + h * hd;
  if (tid < hd) {
    qs[tid] = to_f32(qrow[tid]);
    kb[(int64_t)(len - 1) * 2 * d + tid] = qrow[d + tid];
    kb[(int64_t)(len - 1) * 2 * d + d + tid] = qrow[2 * d + tid];
  }
  __syncthreads();
  float mx = -INFINITY;
  const bool vec = sizeof(T) == 2 && hd % 8 == 0;   // 16-byte key reads (rows 16-byte aligned)
  for (int j = tid; j < len; j += 256) {
    const T* kr = j == len - 1 ? qrow + d : kb + (int64_t)j * 2 * d;
    float s = 0.f;
    if (vec) {
      for (int c8 = 0; c8 < hd; c8 += 8) {
        const bf16x8 kv = *(const bf16x8*)(kr + c8);
#pragma unroll
        for (int e = 0; e < 8; e++) s += qs[c8 + e] * (float)kv[e];
      }
    } else {
      for (int c = 0; c < hd; c++) s += qs[c] * to_f32(kr[c]);
    }
    s *= scale;
    sc[j] = s;
    mx = fmaxf(mx, s);
  }
  mx = wave_max(mx);
  if (lane == 0) red[0][w] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  __syncthreads();
  float sum = 0.f;
  for (int j = tid; j < len; j += 256) {
    const float p = __expf(sc[j] - mx);
    sc[j] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  if (lane == 0) red[0][w] = sum;
  __syncthreads();
  sum = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
  __syncthreads();
  if (vec) {
    const int nch = hd / 8, slots = 256 / nch;       // 8-column chunks, keys per round
    const int ch = tid % nch, slot = tid / nch;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; e++) acc[e] = 0.f;
    if (slot < slots) {
      const T* vb = kb + d + ch * 8;
#pragma unroll 4
      for (int j = slot; j < len; j += slots) {
        const bf16x8 v = *(const bf16x8*)(j == len - 1 ? qrow + 2 * d + ch * 8 : vb + (int64_t)j * 2 * d);
        const float pj = sc[j];
#pragma unroll
        for (int e = 0; e < 8; e++) acc[e] += pj * (float)v[e];
      }
#pragma unroll
      for (int e = 0; e < 8; e++) vred[slot * hd + ch * 8 + e] = acc[e];
    }
    __syncthreads();
    if (tid < hd) {
      float t = 0.f;
      for (int q = 0; q < slots; q++) t += vred[q * hd + tid];
      out[(int64_t)b * d + h * hd + tid] = from_f32<T>(t / sum);
    }
    return;
  }
  float o = 0.f;
  if (lane < hd) {
    const T* vb = kb + d + lane;
    for (int j = w; j < len; j += 4) o += sc[j] * to_f32(j == len - 1 ? qrow[2 * d + lane] : vb[(int64_t)j * 2 * d]);
  }
  red[w][lane] = o;
  __syncthreads();
  if (tid < hd) {
    const float t = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
    out[(int64_t)b * d + h * hd + tid] = from_f32<T>(t / sum);
  }
}

// The bf16 kernel for head_dim HD (32 or 64), with every global load of a workgroup
// issued before the first reduction: each thread's value chunks of up to NVP keys of
// its slot, and the key rows of two scores per thread. The arithmetic and its order
// are those of attn_decode_kernel (dot products over 8-column chunks in column order;
// value sums per slot in key order, then over the slots in order), so the output is
// the same.
template <int HD>
__global__ __launch_bounds__(256) void attn_decode_vec_kernel(const bf16* __restrict__ qkv, bf16* __restrict__ cache,
                                                              bf16* __restrict__ out, int H, int Tmax,
                                                              const int* __restrict__ pos, float scale) {
  constexpr int NCH = HD / 8, SLOTS = 256 / NCH, NVP = 512 / SLOTS;
  __shared__ float sc[DEC_MAX_T];
  __shared__ float red[4];
  __shared__ float vred[SLOTS * HD];
  const int len = min(max(*pos + 1, 1), Tmax);
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int d = H * HD;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ch = tid % NCH, slot = tid / NCH;
  const bf16* qrow = qkv + (int64_t)b * 3 * d + h * HD;
  bf16* kb = cache + (int64_t)b * Tmax * 2 * d + h * HD;
  auto krow = [&](int j) { return j == len - 1 ? qrow + d : kb + (int64_t)j * 2 * d; };
  auto vrow = [&](int j) { return j == len - 1 ? qrow + 2 * d : kb + d + (int64_t)j * 2 * d; };
  bf16x8 vp[NVP];
#pragma unroll
  for (int i = 0; i < NVP; i++) {
    const int j = slot + SLOTS * i;
    vp[i] = j < len ? *(const bf16x8*)(vrow(j) + ch * 8) : (bf16x8){};
  }
  bf16x8 qv[NCH], k0[NCH], k1[NCH];
#pragma unroll
  for (int c = 0; c < NCH; c++) qv[c] = *(const bf16x8*)(qrow + c * 8);
  const int j0 = tid, j1 = tid + 256;
#pragma unroll
  for (int c = 0; c < NCH; c++) {
    k0[c] = j0 < len ? *(const bf16x8*)(krow(j0) + c * 8) : (bf16x8){};
    k1[c] = j1 < len ? *(const bf16x8*)(krow(j1) + c * 8) : (bf16x8){};
  }
  if (tid < HD) {                                    // this position's key and value into the cache
    kb[(int64_t)(len - 1) * 2 * d + tid] = qrow[d + tid];
    kb[(int64_t)(len - 1) * 2 * d + d + tid] = qrow[2 * d + tid];
  }
  auto dot = [&](const bf16x8 (&k)[NCH]) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; c++)
#pragma unroll
      for (int e = 0; e < 8; e++) s += (float)qv[c][e] * (float)k[c][e];
    return s * scale;
  };
  float mx = -INFINITY;
  if (j0 < len) {
    const float s = dot(k0);
    sc[j0] = s;
    mx = s;
  }
  if (j1 < len) {
    const float s = dot(k1);
    sc[j1] = s;
    mx = fmaxf(mx, s);
  }
  for (int j = tid + 512; j < len; j += 256) {        // beyond 512 keys: loaded as they come
    bf16x8 kr[NCH];
#pragma unroll
    for (int c = 0; c < NCH; c++) kr[c] = *(const bf16x8*)(krow(j) + c * 8);
    const float s = dot(kr);
    sc[j] = s;
    mx = fmaxf(mx, s);
  }
  mx = wave_max(mx);
  if (lane == 0) red[w] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float sum = 0.f;
  for (int j = tid; j < len; j += 256) {
    const float p = __expf(sc[j] - mx);
    sc[j] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  if (lane == 0) red[w] = sum;
  __syncthreads();
  sum = (red[0] + red[1]) + (red[2] + red[3]);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; e++) acc[e] = 0.f;
#pragma unroll
  for (int i = 0; i < NVP; i++) {
    const int j = slot + SLOTS * i;
    if (j < len) {
      const float pj = sc[j];
#pragma unroll
      for (int e = 0; e < 8; e++) acc[e] += pj * (float)vp[i][e];
    }
  }
  for (int j = slot + SLOTS * NVP; j < len; j += SLOTS) {
    const bf16x8 v = *(const bf16x8*)(vrow(j) + ch * 8);
    const float pj = sc[j];
#pragma unroll
    for (int e = 0; e < 8; e++) acc[e] += pj * (float)v[e];
  }
#pragma unroll
  for (int e = 0; e < 8; e++) vred[slot * HD + ch * 8 + e] = acc[e];
  __syncthreads();
  if (tid < HD) {
    float t = 0.f;
    for (int q = 0; q < SLOTS; q++) t += vred[q * HD + tid];
    out[(int64_t)b * d + h * HD + tid] = from_f32<bf16>(t / sum);
  }
}

hipError_t launch_attn_decode(const void* qkv, void* cache, void* out, bool bf16_ops, int B, int H, int hd,
                              int Tmax, const int* pos, hipStream_t s) {
  if (hd <= 0 || hd > 64 || !pos || Tmax < 1 || Tmax > DEC_MAX_T) return hipErrorInvalidValue;
  const float scale = 1.0f / sqrtf((float)hd);
  const bool aligned = ((uintptr_t)qkv | (uintptr_t)cache) % 16 == 0;
  if (bf16_ops && aligned && (hd == 64 || hd == 32) && decode_attn_vec()) {
    if (hd == 64)
      hipLaunchKernelGGL(attn_decode_vec_kernel<64>, dim3(B * H), dim3(256), 0, s, (const bf16*)qkv, (bf16*)cache,
                         (bf16*)out, H, Tmax, pos, scale);
    else
      hipLaunchKernelGGL(attn_decode_vec_kernel<32>, dim3(B * H), dim3(256), 0, s, (const bf16*)qkv, (bf16*)cache,
                         (bf16*)out, H, Tmax, pos, scale);
    return hipGetLastError();
  }
  if (bf16_ops)
    hipLaunchKernelGGL(attn_decode_kernel<bf16>, dim3(B * H), dim3(256), 0, s, (const bf16*)qkv, (bf16*)cache,
                       (bf16*)out, H, hd, Tmax, pos, scale);
  else
    hipLaunchKernelGGL(attn_decode_kernel<float>, dim3(B * H), dim3(256), 0, s, (const float*)qkv,
                       (float*)cache, (float*)out, H, hd, Tmax, pos, scale);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- sampling
// One workgroup of 1024 per row. temperature <= 0: the argmax, lowest index on ties.
// Otherwise: the candidates are the logits >= the k-th largest (found exactly by a
// four-pass radix select on order-preserving integer keys; all V when top_k <= 0 or
// >= V), weighted by exp((z - max) / temperature); each wavefront owns a contiguous
// segment of indices, the segment sums are added in order, and the token is the first
// index whose running sum exceeds u times the total.
constexpr int SAMPLE_THREADS = 1024;
constexpr int SAMPLE_REG = 50;                        // logits per thread kept in registers (V <= 51,200)

__device__ inline uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // ascending floats -> ascending keys
}

__global__ __launch_bounds__(SAMPLE_THREADS) void sample_kernel(const float* __restrict__ logits, int64_t ld, int V,
                                                                float temperature, int top_k,
                                                                const float* __restrict__ uniform,
                                                                int32_t* __restrict__ out) {
  constexpr int NW = SAMPLE_THREADS / 64;
  constexpr int UNR = 8;                              // loads in flight per thread in the strided passes
  __shared__ uint32_t hist[NW][256];                  // one histogram per wavefront
  __shared__ float fred[NW];
  __shared__ int ired[NW];
  __shared__ uint32_t sel[2];                         // prefix of the k-th key, count still needed
  __shared__ float csum[NW][64];                      // weight sum of each lane's run
  __shared__ int answer;                              // the wavefront whose segment holds the draw
  __shared__ uint32_t wsuf[4];                        // bins counted by each quarter of the histogram
  const float* z = logits + (int64_t)blockIdx.x * ld;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  // Thread tid takes the logits tid + j * SAMPLE_THREADS: the first SAMPLE_REG of them
  // stay in registers for the maximum and the radix passes (every vocabulary up to
  // SAMPLE_REG * SAMPLE_THREADS), the rest are read again from memory in each pass.
  float zr[SAMPLE_REG];
#pragma unroll
  for (int j = 0; j < SAMPLE_REG; j++) {
    const int i = tid + j * SAMPLE_THREADS;
    zr[j] = i < V ? z[i] : -INFINITY;
  }
  auto each = [&](auto&& f) {                         // f(value, index), indices ascending
#pragma unroll
    for (int j = 0; j < SAMPLE_REG; j++)
      if (tid + j * SAMPLE_THREADS < V) f(zr[j], tid + j * SAMPLE_THREADS);
    for (int i = tid + SAMPLE_REG * SAMPLE_THREADS; i < V; i += SAMPLE_THREADS) f(z[i], i);
  };

  // maximum, with its lowest index (indices rise within a thread: the first maximum stays)
  float mx = -INFINITY;
  int mi = 0x7fffffff;
  each([&](float v, int i) {
    if (v > mx) {
      mx = v;
      mi = i;
    }
  });
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(mx, o, 64);
    const int i2 = __shfl_xor(mi, o, 64);
    if (v2 > mx || (v2 == mx && i2 < mi)) {
      mx = v2;
      mi = i2;
    }
  }
  if (lane == 0) {
    fred[w] = mx;
    ired[w] = mi;
  }
  __syncthreads();
  if (tid == 0) {
    float m = fred[0];
    int k = ired[0];
    for (int q = 1; q < NW; q++)
      if (fred[q] > m || (fred[q] == m && ired[q] < k)) {
        m = fred[q];
        k = ired[q];
      }
    fred[0] = m;
    ired[0] = k;
  }
  __syncthreads();
  mx = fred[0];
  __syncthreads();                                    // fred is written again below
  if (temperature <= 0.f) {
    if (tid == 0) out[blockIdx.x] = ired[0];
    return;
  }

  // k-th largest key (radix select, most significant byte first)
  uint32_t kth = 0;                                   // keys >= kth are candidates
  if (top_k > 0 && top_k < V) {
    if (tid == 0) {
      sel[0] = 0;
      sel[1] = (uint32_t)top_k;
    }
    for (int pass = 0; pass < 4; pass++) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < NW * 256; i += SAMPLE_THREADS) hist[i / 256][i % 256] = 0;
      __syncthreads();
      const uint32_t prefix = sel[0];
      const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
      each([&](float v, int) {
        const uint32_t key = order_key(v);
        if ((key & hi_mask) == prefix) atomicAdd(&hist[w][(key >> shift) & 255u], 1u);
      });
      __syncthreads();
      if (tid < 256) {
        uint32_t c = 0;
#pragma unroll
        for (int q = 0; q < NW; q++) c += hist[q][tid];
        hist[0][tid] = c;
      }
      __syncthreads();
      // the bin holding the need-th largest key: the one whose suffix count (bins at or
      // above it) reaches `need` while the suffix above it does not; every bin in parallel
      const uint32_t need = sel[1];
      // suffix counts (bins at or above each bin) by a scan over the four wavefronts
      // that hold the 256 bins, then their totals
      uint32_t c = 0, suf = 0;
      if (tid < 256) {
        c = suf = hist[0][tid];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t t = __shfl_down(suf, o, 64);
          if (lane + o < 64) suf += t;
        }
        if (lane == 0) wsuf[w] = suf;
      }
      __syncthreads();
      if (tid < 256) {
        uint32_t incl = suf;
        for (int q = w + 1; q < 4; q++) incl += wsuf[q];
        const uint32_t above = incl - c;
        if (above < need && incl >= need) {
          sel[0] = prefix | ((uint32_t)tid << shift);
          sel[1] = need - above;
        }
      }
      __syncthreads();
    }
    kth = sel[0];
  }

  // weights exp((z - max) / temperature) of the candidates, summed in index order:
  // wavefront w owns the segment [w S, (w + 1) S) and its lane l the run
  // [w S + l CH, w S + (l + 1) CH) (S = 64 CH, CH a multiple of 4), summed in order by
  // that lane; runs add up across lanes, segments across wavefronts
  const float inv_t = 1.0f / temperature;
  const int CH = ((V + NW - 1) / NW + 255) / 256 * 4;
  const int s0 = min(V, w * 64 * CH), s1 = min(V, s0 + 64 * CH);
  const int a0 = min(s1, s0 + lane * CH), a1 = min(s1, a0 + CH);
  auto weight = [&](float v) -> float { return order_key(v) >= kth ? __expf((v - mx) * inv_t) : 0.f; };
  float cs = 0.f;
  if (a1 - a0 == CH && ((uintptr_t)z & 15) == 0) {   // whole run of an aligned row: 16-byte loads
    for (int i = a0; i < a1; i += 4 * UNR) {
      f32x4 v[UNR];
#pragma unroll
      for (int u = 0; u < UNR; u++) v[u] = i + 4 * u < a1 ? *(const f32x4*)(z + i + 4 * u) : (f32x4){-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int u = 0; u < UNR; u++)
#pragma unroll
        for (int e = 0; e < 4; e++) cs += i + 4 * u < a1 ? weight(v[u][e]) : 0.f;
    }
  } else {
    for (int i = a0; i < a1; i++) cs += weight(z[i]);
  }
  csum[w][lane] = cs;
  const float wtot = wave_sum(cs);
  if (lane == 0) fred[w] = wtot;
  if (tid == 0) answer = -1;
  __syncthreads();
  float start = 0.f, total = 0.f;
  for (int q = 0; q < NW; q++) {
    if (q < w) start += fred[q];
    total += fred[q];
  }
  const float target = uniform[blockIdx.x] * total;
  // the segment holding the target is the last non-empty one that starts at or before it
  if (lane == 0 && wtot > 0.f && start <= target) atomicMax(&answer, w);
  __syncthreads();
  if (w != answer) return;
  float incl = cs;                                    // runs before this lane's, in lane order
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  const float lstart = start + incl - cs;
  const uint64_t claim = __ballot(cs > 0.f && lstart <= target);
  if (lane != 63 - __builtin_clzll(claim)) return;    // the last non-empty run starting at or before it
  // the run's weights added in index order, sixteen logits fetched at a time
  float acc = lstart;
  int pick = -1, last = -1;
  for (int i = a0; i < a1 && pick < 0; i += 16) {
    float v[16];
#pragma unroll
    for (int e = 0; e < 16; e++) v[e] = i + e < a1 ? z[i + e] : -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; e++) {
      const float wi = i + e < a1 ? weight(v[e]) : 0.f;
      if (pick < 0 && wi > 0.f) {
        last = i + e;
        acc += wi;
        if (acc > target) pick = i + e;
      }
    }
  }
  out[blockIdx.x] = pick >= 0 ? pick : last;          // rounding can leave the target past the run's sum
}

hipError_t launch_sample(const float* logits, int64_t ld, int B, int V, float temperature, int top_k,
                         const float* uniform, int32_t* out, hipStream_t s) {
  if (B < 1 || V < 1 || ld < V) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sample_kernel, dim3(B), dim3(SAMPLE_THREADS), 0, s, logits, ld, V, temperature, top_k, uniform,
                     out);
  return hipGetLastError();
}

}  // namespace gpt
