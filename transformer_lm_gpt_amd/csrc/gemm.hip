// Tiled MFMA GEMM for gfx950 with fused epilogues.
//
// Every linear layer of the step (QKV, attention output, MLP up and down, the
// tied lm_head) and each of their two backward products runs here:
//   forward  C = X W^T      A k-contiguous, B k-contiguous
//   dgrad    dX = dY W      A k-contiguous, B n-contiguous
//   wgrad    dW = dY^T X    A m-contiguous, B n-contiguous
// A 256-thread workgroup computes a 128x128 tile; its four wavefronts each own
// a 64x64 quadrant made of 4x4 MFMA 16x16 tiles. The contraction advances in
// slices of BK (64 for bf16, 16 for fp32) staged through two LDS buffers: the
// next slice is fetched into registers while the current one feeds the MFMAs.
// LDS tiles are stored as [BK/KG][rows + pad][KG], so that one MFMA operand
// fragment (KG contraction-consecutive values of one row) is one LDS read.
// Operands that arrive m-contiguous are transposed in registers on the way in.
#include "common.h"
#include "kernels.h"

namespace gpt {

constexpr int BM = 128, BN = 128;

template <typename T> struct GemmCfg;
template <> struct GemmCfg<bf16> {
  static constexpr int BK = 64;
  static constexpr int PAD = 1;                      // rows of KG elements (16 bytes)
  static constexpr int tile_elems(int rows) { return (BK / 8) * (rows + PAD) * 8; }
};
template <> struct GemmCfg<float> {
  static constexpr int BK = 16;
  static constexpr int PAD = 16;                     // floats
  static constexpr int tile_elems(int rows) { return BK * (rows + PAD); }
};

// ----------------------------------------------------------------------------- tile loaders
// Load a ROWS x BK slice starting at (row0, k0) of a logical [nrows, K] operand.
template <typename T, bool KC> struct Loader;

// bf16, k-contiguous: 16-byte vectors of 8 consecutive k.
template <> struct Loader<bf16, true> {
  static constexpr int NV = BM * 64 / 8 / 256;   // 4 vectors per thread
  bf16x8 r[NV];
  __device__ void load(const bf16* __restrict__ src, int64_t ld, int row0, int nrows, int k0, int K, bool vec) {
#pragma unroll
    for (int j = 0; j < NV; j++) {
      int i = threadIdx.x + 256 * j;
      int row = i >> 3, g = i & 7;
      int gr = row0 + row, gk = k0 + g * 8;
      if (vec && gr < nrows && gk + 8 <= K) {
        r[j] = *(const bf16x8*)(src + (int64_t)gr * ld + gk);
      } else {
#pragma unroll
        for (int e = 0; e < 8; e++)
          r[j][e] = (gr < nrows && gk + e < K) ? src[(int64_t)gr * ld + gk + e] : (bf16)0.0f;
      }
    }
  }
  __device__ void store(bf16* lds) const {
#pragma unroll
    for (int j = 0; j < NV; j++) {
      int i = threadIdx.x + 256 * j;
      int row = i >> 3, g = i & 7;
      *(bf16x8*)(lds + (g * (BM + 1) + row) * 8) = r[j];
    }
  }
};

// bf16, m-contiguous: each pair of threads owns an 8(k) x 8(m) block; a thread
// loads 4 k-rows of 8 m and writes 8 half-fragments of 4 k.
template <> struct Loader<bf16, false> {
  bf16x8 r[4];
  __device__ void load(const bf16* __restrict__ src, int64_t ld, int row0, int nrows, int k0, int K, bool vec) {
    int b = threadIdx.x >> 1, half = threadIdx.x & 1;
    int kb = b / (BM / 8), mb = b % (BM / 8);
    int gm = row0 + mb * 8;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      int gk = k0 + kb * 8 + half * 4 + q;
      if (vec && gk < K && gm + 8 <= nrows) {
        r[q] = *(const bf16x8*)(src + (int64_t)gk * ld + gm);
      } else {
#pragma unroll
        for (int e = 0; e < 8; e++)
          r[q][e] = (gk < K && gm + e < nrows) ? src[(int64_t)gk * ld + gm + e] : (bf16)0.0f;
      }
    }
  }
  __device__ void store(bf16* lds) const {
    int b = threadIdx.x >> 1, half = threadIdx.x & 1;
    int kb = b / (BM / 8), mb = b % (BM / 8);
#pragma unroll
    for (int j = 0; j < 8; j++) {
      bf16x4 w;
      w[0] = r[0][j]; w[1] = r[1][j]; w[2] = r[2][j]; w[3] = r[3][j];
      *(bf16x4*)(lds + (kb * (BM + 1) + mb * 8 + j) * 8 + half * 4) = w;
    }
  }
};

// fp32, k-contiguous: float4 of 4 consecutive k, scattered into 4 LDS rows.
template <> struct Loader<float, true> {
  static constexpr int NV = BM * 16 / 4 / 256;   // 2
  f32x4 r[NV];
  __device__ void load(const float* __restrict__ src, int64_t ld, int row0, int nrows, int k0, int K, bool vec) {
#pragma unroll
    for (int j = 0; j < NV; j++) {
      int i = threadIdx.x + 256 * j;
      int row = i >> 2, kq = i & 3;
      int gr = row0 + row, gk = k0 + kq * 4;
      if (vec && gr < nrows && gk + 4 <= K) {
        r[j] = *(const f32x4*)(src + (int64_t)gr * ld + gk);
      } else {
#pragma unroll
        for (int e = 0; e < 4; e++) r[j][e] = (gr < nrows && gk + e < K) ? src[(int64_t)gr * ld + gk + e] : 0.0f;
      }
    }
  }
  __device__ void store(float* lds) const {
    constexpr int S = BM + GemmCfg<float>::PAD;
#pragma unroll
    for (int j = 0; j < NV; j++) {
      int i = threadIdx.x + 256 * j;
      int row = i >> 2, kq = i & 3;
#pragma unroll
      for (int e = 0; e < 4; e++) lds[(kq * 4 + e) * S + row] = r[j][e];
    }
  }
};

// fp32, m-contiguous: float4 of 4 consecutive m.
template <> struct Loader<float, false> {
  static constexpr int NV = 2;
  f32x4 r[NV];
  __device__ void load(const float* __restrict__ src, int64_t ld, int row0, int nrows, int k0, int K, bool vec) {
#pragma unroll
    for (int j = 0; j < NV; j++) {
      int i = threadIdx.x + 256 * j;
      int k = i >> 5, mq = i & 31;
      int gk = k0 + k, gm = row0 + mq * 4;
      if (vec && gk < K && gm + 4 <= nrows) {
        r[j] = *(const f32x4*)(src + (int64_t)gk * ld + gm);
      } else {
#pragma unroll
        for (int e = 0; e < 4; e++) r[j][e] = (gk < K && gm + e < nrows) ? src[(int64_t)gk * ld + gm + e] : 0.0f;
      }
    }
  }
  __device__ void store(float* lds) const {
    constexpr int S = BM + GemmCfg<float>::PAD;
#pragma unroll
    for (int j = 0; j < NV; j++) {
      int i = threadIdx.x + 256 * j;
      int k = i >> 5, mq = i & 31;
      *(f32x4*)(lds + k * S + mq * 4) = r[j];
    }
  }
};

// One MFMA operand fragment for rows row (lane & 15 already added) and k-step kk.
__device__ inline bf16x8 frag_at(const bf16* lds, int kk, int row) {
  int g = kk * 4 + (threadIdx.x & 63) / 16;
  return *(const bf16x8*)(lds + (g * (BM + 1) + row) * 8);
}
__device__ inline float frag_at(const float* lds, int kk, int row) {
  int k = kk * 4 + (threadIdx.x & 63) / 16;
  return lds[k * (BM + GemmCfg<float>::PAD) + row];
}

struct GemmArgs {
  const void* A; int64_t lda;
  const void* B; int64_t ldb;
  void* C; int64_t ldc;
  int M, N, K;
  const float* bias;
  const float* resid; int64_t ldr;
  float* aux; int64_t ldaux;
  float beta;
  int a_vec, b_vec;
};

template <typename T, bool AK, bool BK_, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs p) {
  typedef GemmCfg<T> Cfg;
  constexpr int BK = Cfg::BK;
  constexpr int TILE = Cfg::tile_elems(BM);
  constexpr int KSTEPS = BK / Mfma<T>::KPI;
  __shared__ __attribute__((aligned(16))) T smem[2 * 2 * TILE];
  // buffer i of A at smem + i*TILE, of B at smem + (2 + i)*TILE

  const T* A = (const T*)p.A;
  const T* B = (const T*)p.B;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  Loader<T, AK> la;
  Loader<T, BK_> lb;
  const int nk = (p.K + BK - 1) / BK;
  la.load(A, p.lda, m0, p.M, 0, p.K, p.a_vec);
  lb.load(B, p.ldb, n0, p.N, 0, p.K, p.b_vec);
  la.store(smem);
  lb.store(smem + 2 * TILE);
  __syncthreads();

  for (int kt = 0; kt < nk; kt++) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      la.load(A, p.lda, m0, p.M, (kt + 1) * BK, p.K, p.a_vec);
      lb.load(B, p.ldb, n0, p.N, (kt + 1) * BK, p.K, p.b_vec);
    }
#pragma unroll
    for (int kk = 0; kk < KSTEPS; kk++) {
      typename Mfma<T>::frag af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; i++) af[i] = frag_at(smem + cur * TILE, kk, wm * 64 + i * 16 + (lane & 15));
#pragma unroll
      for (int j = 0; j < 4; j++) bfr[j] = frag_at(smem + (2 + cur) * TILE, kk, wn * 64 + j * 16 + (lane & 15));
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = Mfma<T>::mma(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) {
      la.store(smem + (cur ^ 1) * TILE);
      lb.store(smem + (2 + (cur ^ 1)) * TILE);
    }
    __syncthreads();
  }

  // Epilogue: lane holds rows 4*(lane>>4)+e of column (lane&15) in each 16x16 tile.
#pragma unroll
  for (int i = 0; i < 4; i++) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int col = n0 + wn * 64 + j * 16 + (lane & 15);
      if (col >= p.N) continue;
      float bias = 0.f;
      if (EPI == EPI_BIAS || EPI == EPI_BIAS_RESID || EPI == EPI_BIAS_GELU) bias = p.bias[col];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int row = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + e;
        if (row >= p.M) continue;
        float v = acc[i][j][e];
        const int64_t ci = (int64_t)row * p.ldc + col;
        if constexpr (EPI == EPI_STORE) {
          ((T*)p.C)[ci] = from_f32<T>(v);
        } else if constexpr (EPI == EPI_BIAS) {
          ((T*)p.C)[ci] = from_f32<T>(v + bias);
        } else if constexpr (EPI == EPI_BIAS_RESID) {
          ((float*)p.C)[ci] = p.resid[(int64_t)row * p.ldr + col] + (v + bias);
        } else if constexpr (EPI == EPI_BIAS_GELU) {
          float u = v + bias;
          p.aux[(int64_t)row * p.ldaux + col] = u;
          ((T*)p.C)[ci] = from_f32<T>(gelu_f(u));
        } else if constexpr (EPI == EPI_F32) {
          ((float*)p.C)[ci] = v;
        } else if constexpr (EPI == EPI_GELU_BWD) {
          ((T*)p.C)[ci] = from_f32<T>(v * gelu_grad_f(p.aux[(int64_t)row * p.ldaux + col]));
        } else {  // EPI_ACC
          float* c = (float*)p.C + ci;
          *c = (p.beta != 0.f ? p.beta * *c : 0.f) + v;
        }
      }
    }
  }
}

template <typename T, bool AK, bool BK_>
static hipError_t dispatch_epi(const GemmArgs& a, int epi, dim3 grid, hipStream_t s) {
  switch (epi) {
#define GPT_EPI_CASE(E) \
  case E: hipLaunchKernelGGL((gemm_kernel<T, AK, BK_, E>), grid, dim3(256), 0, s, a); break;
    GPT_EPI_CASE(EPI_STORE)
    GPT_EPI_CASE(EPI_BIAS)
    GPT_EPI_CASE(EPI_BIAS_RESID)
    GPT_EPI_CASE(EPI_BIAS_GELU)
    GPT_EPI_CASE(EPI_F32)
    GPT_EPI_CASE(EPI_GELU_BWD)
    GPT_EPI_CASE(EPI_ACC)
#undef GPT_EPI_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t dispatch_layout(const GemmDesc& d, const GemmArgs& a, dim3 grid, hipStream_t s) {
  if (d.a_kc && d.b_kc) return dispatch_epi<T, true, true>(a, d.epi, grid, s);
  if (d.a_kc && !d.b_kc) return dispatch_epi<T, true, false>(a, d.epi, grid, s);
  if (!d.a_kc && !d.b_kc) return dispatch_epi<T, false, false>(a, d.epi, grid, s);
  return hipErrorInvalidValue;  // m-contiguous A with k-contiguous B is not used by the step
}

hipError_t launch_gemm(const GemmDesc& d, bool bf16_operands, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0) return hipSuccess;
  GemmArgs a;
  a.A = d.A; a.lda = d.lda; a.B = d.B; a.ldb = d.ldb; a.C = d.C; a.ldc = d.ldc;
  a.M = d.M; a.N = d.N; a.K = d.K; a.bias = d.bias; a.resid = d.resid; a.ldr = d.ldr;
  a.aux = d.aux; a.ldaux = d.ldaux; a.beta = d.beta;
  const int vw = bf16_operands ? 8 : 4;               // elements per 16-byte vector
  a.a_vec = (d.lda % vw == 0) && ((uintptr_t)d.A % 16 == 0);
  a.b_vec = (d.ldb % vw == 0) && ((uintptr_t)d.B % 16 == 0);
  dim3 grid((d.N + BN - 1) / BN, (d.M + BM - 1) / BM);
  if (bf16_operands) return dispatch_layout<bf16>(d, a, grid, s);
  return dispatch_layout<float>(d, a, grid, s);
}

}  // namespace gpt
