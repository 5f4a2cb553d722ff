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
#include <cstdlib>
#include <type_traits>

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
  void* aux; int64_t ldaux;   // operand type
  float beta;
  int a_vec, b_vec;
  int c_vec;           // C / aux / resid rows allow 16-column vector access
  int kchunk;          // contraction length per split (gridDim.z splits)
  float* part;         // split partials [gridDim.z, M, N] (EPI_ACC with gridDim.z > 1)
  float* colsum;       // EPI_GELU_BWD: per-tile-row column sums [tiles_m, N], or NULL
  DropArgs drop;       // EPI_BIAS_RESID_DROP: the branch output's dropout mask
  uint32_t drop_site;
  // workgroups [stagger_lo, stagger_hi) sleep stagger_iters x 2048 cycles before
  // their first load (the second workgroup of each CU in the first round, so the
  // two tiles of a CU reach their epilogues apart)
  int stagger_lo = 0, stagger_hi = 0, stagger_iters = 0;
  int krot = 0;        // rotate each tile's k-slice order by its position in the launch
  int* bump = nullptr; // few-rows kernel: block 0 adds one to *bump (no block reads it)
  // few-rows kernel with the normalization fused in front: A = norm(nx) (rows of K
  // fp32, gain ng and shift nb for the LayerNorm), computed into LDS
  const float* nx = nullptr;
  const float* ng = nullptr;
  const float* nb = nullptr;
};

// Epilogues that add a residual (with or without dropout on the branch) and those with a bias.
template <int EPI> constexpr bool epi_resid() { return EPI == EPI_BIAS_RESID || EPI == EPI_BIAS_RESID_DROP; }
template <int EPI> constexpr bool epi_has_bias() {
  return EPI == EPI_BIAS || epi_resid<EPI>() || EPI == EPI_BIAS_GELU || EPI == EPI_BIAS_RELU;
}
// Epilogues that scale by the activation's derivative at the saved input (and can sum columns).
template <int EPI> constexpr bool epi_act_bwd() { return EPI == EPI_GELU_BWD || EPI == EPI_RELU_BWD; }

template <int EPI>
__device__ inline float epi_bias(const GemmArgs& p, int col) {
  if constexpr (epi_has_bias<EPI>()) return p.bias[col];
  return 0.f;
}

// The branch mask of one output element, kept out of line: the element epilogues
// below are unrolled over whole tiles, and inlined generator rounds for every element
// would be scheduled together and spill.
__device__ __noinline__ float drop_mult_elem(const DropArgs& a, uint32_t site, uint32_t row, uint32_t col) {
  return drop_mult1(a, site, row, col);
}

// One output element: the fused epilogue of every GEMM of the step.
template <typename T, int EPI>
__device__ inline void epi_store(const GemmArgs& p, int row, int col, float v, float bias) {
  const int64_t ci = (int64_t)row * p.ldc + col;
  if constexpr (EPI == EPI_STORE) {
    ((T*)p.C)[ci] = from_f32<T>(v);
  } else if constexpr (EPI == EPI_BIAS) {
    ((T*)p.C)[ci] = from_f32<T>(v + bias);
  } else if constexpr (EPI == EPI_BIAS_RESID) {
    ((float*)p.C)[ci] = p.resid[(int64_t)row * p.ldr + col] + (v + bias);
  } else if constexpr (EPI == EPI_BIAS_RESID_DROP) {
    ((float*)p.C)[ci] = p.resid[(int64_t)row * p.ldr + col] + (v + bias) * drop_mult_elem(p.drop, p.drop_site, row, col);
  } else if constexpr (EPI == EPI_BIAS_GELU) {
    float g, dg;
    gelu_and_grad(v + bias, g, dg);
    ((T*)p.aux)[(int64_t)row * p.ldaux + col] = from_f32<T>(dg);
    ((T*)p.C)[ci] = from_f32<T>(g);
  } else if constexpr (EPI == EPI_F32) {
    ((float*)p.C)[ci] = v;
  } else if constexpr (EPI == EPI_BIAS_RELU) {
    const float u = v + bias;
    ((T*)p.aux)[(int64_t)row * p.ldaux + col] = from_f32<T>(u);
    ((T*)p.C)[ci] = from_f32<T>(fmaxf(u, 0.f));
  } else if constexpr (EPI == EPI_GELU_BWD) {
    ((T*)p.C)[ci] = from_f32<T>(v * to_f32(((const T*)p.aux)[(int64_t)row * p.ldaux + col]));
  } else if constexpr (EPI == EPI_RELU_BWD) {
    ((T*)p.C)[ci] = from_f32<T>(to_f32(((const T*)p.aux)[(int64_t)row * p.ldaux + col]) > 0.f ? v : 0.f);
  } else {  // EPI_ACC
    if (gridDim.z > 1) {
      p.part[((int64_t)blockIdx.z * p.M + row) * p.N + col] = v;
    } else {
      float* c = (float*)p.C + ci;
      *c = (p.beta != 0.f ? p.beta * *c : 0.f) + v;
    }
  }
}

// Global inputs of the vector epilogue (the residual, or the saved GELU'(u) / ReLU
// input) for sixteen columns, loaded ahead of the tile's parked accumulators so the loads of the next 16-row
// block are in flight while the current one is stored.
template <int EPI>
struct EpiPre {
  static constexpr bool ON = epi_resid<EPI>() || epi_act_bwd<EPI>();
  f32x4 r[epi_resid<EPI>() ? 4 : 1];
  bf16x8 u[epi_act_bwd<EPI>() ? 2 : 1];
  __device__ inline void load(const GemmArgs& p, int row, int col0) {
    if constexpr (epi_resid<EPI>()) {
      const float* src = p.resid + (int64_t)row * p.ldr + col0;
#pragma unroll
      for (int q = 0; q < 4; q++) r[q] = *(const f32x4*)(src + 4 * q);
    } else if constexpr (epi_act_bwd<EPI>()) {
      const bf16* src = (const bf16*)p.aux + (int64_t)row * p.ldaux + col0;
#pragma unroll
      for (int q = 0; q < 2; q++) u[q] = *(const bf16x8*)(src + 8 * q);
    }
  }
};

// Sixteen consecutive output columns col0.. of one row: vector loads and stores
// when the run is inside the matrix and aligned, element-wise otherwise. pre, if
// given, holds this run's residual or saved GELU'(u) / ReLU input, loaded by EpiPre::load.
// With EPI_GELU_BWD the final fp32 values are also added into sum16 (the bias
// gradient's column sums); other epilogues leave it alone.
template <int EPI>
__device__ inline void epi_store16(const GemmArgs& p, int row, int col0, const float (&v)[16], bool vec,
                                   float (&sum16)[16], const EpiPre<EPI>* pre = nullptr,
                                   const f32x4* bias16 = nullptr) {
  if (!vec) {
#pragma unroll
    for (int c = 0; c < 16; c++)
      if (col0 + c < p.N) {
        epi_store<bf16, EPI>(p, row, col0 + c, v[c], epi_bias<EPI>(p, col0 + c));
        if constexpr (EPI == EPI_GELU_BWD)
          sum16[c] += v[c] * (float)((const bf16*)p.aux)[(int64_t)row * p.ldaux + col0 + c];
        if constexpr (EPI == EPI_RELU_BWD)
          sum16[c] += (float)((const bf16*)p.aux)[(int64_t)row * p.ldaux + col0 + c] > 0.f ? v[c] : 0.f;
      }
    return;
  }
  const int64_t ci = (int64_t)row * p.ldc + col0;
  float x[16];
#pragma unroll
  for (int c = 0; c < 16; c++) x[c] = v[c];
  if constexpr (epi_has_bias<EPI>()) {
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const f32x4 b = bias16 ? bias16[q] : *(const f32x4*)(p.bias + col0 + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; e++) x[4 * q + e] += b[e];
    }
  }
  if constexpr (EPI == EPI_STORE || EPI == EPI_BIAS) {
#pragma unroll
    for (int q = 0; q < 2; q++) {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; e++) o[e] = (bf16)x[8 * q + e];
      *(bf16x8*)((bf16*)p.C + ci + 8 * q) = o;
    }
  } else if constexpr (epi_resid<EPI>()) {
    const float* r = p.resid + (int64_t)row * p.ldr + col0;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const f32x4 rv = pre ? pre->r[q] : *(const f32x4*)(r + 4 * q);
      f32x4 o;
      if constexpr (EPI == EPI_BIAS_RESID_DROP) {
        // the opaque copy of the row keeps each mask block after the stores before it:
        // hoisted together, the blocks of every pass spill the parked accumulators
        uint32_t mrow = (uint32_t)row;
        asm volatile("" : "+v"(mrow)::"memory");
        const f32x4 mk = drop_mult4(p.drop, p.drop_site, mrow, (col0 >> 2) + q);
#pragma unroll
        for (int e = 0; e < 4; e++) o[e] = rv[e] + x[4 * q + e] * mk[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; e++) o[e] = rv[e] + x[4 * q + e];
      }
      *(f32x4*)((float*)p.C + ci + 4 * q) = o;
    }
  } else if constexpr (EPI == EPI_BIAS_GELU) {
    bf16* dgp = (bf16*)p.aux + (int64_t)row * p.ldaux + col0;
#pragma unroll
    for (int q = 0; q < 2; q++) {
      bf16x8 dgo, o;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        float g, dg;
        gelu_and_grad(x[8 * q + e], g, dg);
        dgo[e] = (bf16)dg;
        o[e] = (bf16)g;
      }
      *(bf16x8*)(dgp + 8 * q) = dgo;
      *(bf16x8*)((bf16*)p.C + ci + 8 * q) = o;
    }
  } else if constexpr (EPI == EPI_BIAS_RELU) {
    bf16* u = (bf16*)p.aux + (int64_t)row * p.ldaux + col0;
#pragma unroll
    for (int q = 0; q < 2; q++) {
      bf16x8 uo, o;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        uo[e] = (bf16)x[8 * q + e];
        o[e] = (bf16)fmaxf(x[8 * q + e], 0.f);
      }
      *(bf16x8*)(u + 8 * q) = uo;
      *(bf16x8*)((bf16*)p.C + ci + 8 * q) = o;
    }
  } else if constexpr (EPI == EPI_RELU_BWD) {
    const bf16* u = (const bf16*)p.aux + (int64_t)row * p.ldaux + col0;
#pragma unroll
    for (int q = 0; q < 2; q++) {
      const bf16x8 uv = pre ? pre->u[q] : *(const bf16x8*)(u + 8 * q);
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const float y = (float)uv[e] > 0.f ? x[8 * q + e] : 0.f;
        o[e] = (bf16)y;
        sum16[8 * q + e] += y;
      }
      *(bf16x8*)((bf16*)p.C + ci + 8 * q) = o;
    }
  } else if constexpr (EPI == EPI_F32) {
#pragma unroll
    for (int q = 0; q < 4; q++) *(f32x4*)((float*)p.C + ci + 4 * q) = (f32x4){x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
  } else if constexpr (EPI == EPI_GELU_BWD) {
    const bf16* u = (const bf16*)p.aux + (int64_t)row * p.ldaux + col0;
#pragma unroll
    for (int q = 0; q < 2; q++) {
      const bf16x8 uv = pre ? pre->u[q] : *(const bf16x8*)(u + 8 * q);
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const float y = x[8 * q + e] * (float)uv[e];
        o[e] = (bf16)y;
        sum16[8 * q + e] += y;
      }
      *(bf16x8*)((bf16*)p.C + ci + 8 * q) = o;
    }
  } else {  // EPI_ACC
    if (gridDim.z > 1) {
      float* d = p.part + ((int64_t)blockIdx.z * p.M + row) * p.N + col0;
#pragma unroll
      for (int q = 0; q < 4; q++) *(f32x4*)(d + 4 * q) = (f32x4){x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
    } else {
      float* c = (float*)p.C + ci;
#pragma unroll
      for (int q = 0; q < 4; q++) {
        f32x4 o = (f32x4){x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
        if (p.beta != 0.f) o += *(const f32x4*)(c + 4 * q);
        *(f32x4*)(c + 4 * q) = o;
      }
    }
  }
}

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
  const int kb = blockIdx.z * p.kchunk;
  const int ke = min(p.K, kb + p.kchunk);
  const int nk = (ke - kb + BK - 1) / BK;
  la.load(A, p.lda, m0, p.M, kb, ke, p.a_vec);
  lb.load(B, p.ldb, n0, p.N, kb, ke, p.b_vec);
  la.store(smem);
  lb.store(smem + 2 * TILE);
  __syncthreads();

  for (int kt = 0; kt < nk; kt++) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      la.load(A, p.lda, m0, p.M, kb + (kt + 1) * BK, ke, p.a_vec);
      lb.load(B, p.ldb, n0, p.N, kb + (kt + 1) * BK, ke, p.b_vec);
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
      const float bias = epi_bias<EPI>(p, col);
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int row = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + e;
        if (row < p.M) epi_store<T, EPI>(p, row, col, acc[i][j][e], bias);
      }
    }
  }
}

// ----------------------------------------------------------------------------- pipelined bf16 (global -> LDS)
// BM_ x BN_ tile, BK = 32, STAGES LDS buffers filled straight from global memory
// (global_load_lds, 16 bytes per lane, a wavefront's 64 lanes land on 1 KB of
// consecutive LDS), so loads for STAGES-1 future k-slices are in flight while a
// slice is multiplied. Requires K (and the split length) to be a multiple of 32;
// rows past the edge are clamped to a valid address and masked at the store.
//
// k-contiguous operand, per stage [ROWS][4 units of 8 k]; unit u of row r sits at
// r*4 + (u ^ ((r >> 1) & 3)). Measured on gfx950, this XOR keeps the MFMA fragment
// reads (16 consecutive rows of one unit column) at the full ds_read_b128 rate,
// where the unswizzled layout or an XOR with (r >> 2) loses about a fifth.
// m-contiguous operand, per stage [32 k][ROWS/8 units of 8 m]; unit mu of row k
// sits at k*(ROWS/8) + (mu ^ swz(k)). It is read with ds_read_tr16_b64: in each
// 16-lane group, lane q reads 4 m at (k0 + q/4, m0 + 4*(q%4)) and receives 4 k of
// column m0 + q, which is one half of an MFMA fragment.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ inline int mc_swz(int k) { return 2 * (k & 3) + 8 * ((k >> 3) & 1); }

// The loaders below fill LDS with buffer loads (MUBUF LDS DMA) over a resource whose
// base is the tile's first row (k-contiguous) or column (m-contiguous), so every
// per-lane byte offset fits 32 bits. The buffer form matters to the compiler: with a
// FLAT-encoded LDS DMA (global_load_lds) in a loop, its wait-count pass must assume
// LDS accesses complete out of order and waits for every LDS read in flight before
// each use, where the buffer form keeps the counts exact and lets fragment reads
// overlap the MFMAs.
__device__ inline __amdgpu_buffer_rsrc_t tile_rsrc(const bf16* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}

// rmax: rows of the operand from the tile's first row on (>= 1); rows past it are
// clamped to the last one (their products are masked at the store).
template <int ROWS, int NW>
__device__ inline void dma_kc(__amdgpu_buffer_rsrc_t src, int64_t ld, int rmax, int k0, char* lds, int wave,
                              int lane) {
  constexpr int CHUNKS = ROWS * 32 * 2 / 1024;   // 1 KB per wavefront instruction
  static_assert(ROWS % 16 == 0 && CHUNKS % NW == 0, "k-contiguous tile shape");
#pragma unroll
  for (int i = 0; i < CHUNKS / NW; i++) {
    const int ch = wave + NW * i;
    const int r = ch * 16 + (lane >> 2);
    const int u = (lane & 3) ^ ((r >> 1) & 3);
    const int gr = min(r, rmax - 1);
    const uint32_t off = (uint32_t)(((int64_t)gr * ld + k0 + 8 * u) * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void*)(lds + ch * 1024), 16, off, 0, 0, 0);
  }
}

// m-contiguous: the resource starts at the tile's first column; mmax = columns from
// it on (a multiple of 8, >= 8), the last 8-column unit standing in for those past it.
template <int ROWS, int NW>
__device__ inline void dma_mc(__amdgpu_buffer_rsrc_t src, int64_t ld, int mmax, int k0, char* lds, int wave,
                              int lane) {
  constexpr int UPR = ROWS / 8;                  // 16-byte units per k-row
  constexpr int RPC = 64 / UPR;                  // k-rows per 1 KB chunk
  constexpr int CHUNKS = 32 / RPC;
  static_assert(64 % UPR == 0 && 32 % RPC == 0 && CHUNKS % NW == 0, "m-contiguous tile shape");
#pragma unroll
  for (int i = 0; i < CHUNKS / NW; i++) {
    const int ch = wave + NW * i;
    const int k = ch * RPC + lane / UPR;
    const int mu = (lane % UPR) ^ mc_swz(k);
    const int gm = min(8 * mu, mmax - 8);
    const uint32_t off = (uint32_t)(((int64_t)(k0 + k) * ld + gm) * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void*)(lds + ch * 1024), 16, off, 0, 0, 0);
  }
}

// 64-wide k-slices of a k-contiguous operand: a row is 128 bytes = 8 units, unit u of
// row r at r*8 + (u ^ ((r >> 1) & 7)); a 1 KB wavefront instruction covers 8 rows, one
// whole 128-byte line per row (half the requests per byte of the 32-wide slices).
template <int ROWS, int NW>
__device__ inline void dma_kc64(__amdgpu_buffer_rsrc_t src, int64_t ld, int rmax, int k0, char* lds, int wave,
                                int lane) {
  constexpr int CHUNKS = ROWS * 64 * 2 / 1024;
  static_assert(ROWS % 16 == 0 && CHUNKS % NW == 0, "k-contiguous tile shape");
#pragma unroll
  for (int i = 0; i < CHUNKS / NW; i++) {
    const int ch = wave + NW * i;
    const int r = ch * 8 + (lane >> 3);
    const int u = (lane & 7) ^ ((r >> 1) & 7);
    const int gr = min(r, rmax - 1);
    const uint32_t off = (uint32_t)(((int64_t)gr * ld + k0 + 8 * u) * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void*)(lds + ch * 1024), 16, off, 0, 0, 0);
  }
}
// fragment of the h-th 32-wide half of a 64-wide slice
__device__ inline bf16x8 frag_kc64(const char* lds, int r, int h) {
  const int u = (4 * h + ((threadIdx.x & 63) >> 4)) ^ ((r >> 1) & 7);
  return *(const bf16x8*)(lds + (r * 8 + u) * 16);
}

// MFMA fragment (8 consecutive k = 8*(lane>>4) .. +7 of one row) from a stage buffer.
template <int ROWS>
__device__ inline bf16x8 frag_kc(const char* lds, int r) {
  const int u = ((threadIdx.x & 63) >> 4) ^ ((r >> 1) & 3);
  return *(const bf16x8*)(lds + (r * 4 + u) * 16);
}
template <int ROWS>
__device__ inline bf16x8 frag_mc(const char* lds, int mbase) {
  constexpr int UPR = ROWS / 8;
  const int lane = threadIdx.x & 63;
  const int q = lane & 15, g = lane >> 4;
  const int mu = (mbase >> 3) + ((q & 3) >> 1);
  s16x4 h[2];
#pragma unroll
  for (int hh = 0; hh < 2; hh++) {
    const int k = 8 * g + 4 * hh + (q >> 2);
    const char* a = lds + (k * UPR + (mu ^ mc_swz(k))) * 16 + (q & 1) * 8;
    h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a));
  }
  bf16x8 f;
  __builtin_memcpy(&f, h, 16);
  return f;
}

// Grouped tile order: runs of 8 tile-rows, column by column, so that tiles in
// flight together share A and B panels in L2.
__device__ inline void tile_coords(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GM = 8;
  const int group = GM * tiles_n;
  const int first_m = (t / group) * GM;
  const int gsz = min(tiles_m - first_m, GM);
  tm = first_m + (t % group) % gsz;
  tn = (t % group) / gsz;
}

// Epilogue of one BM_ x BN_ tile whose wavefronts (WM_ x WN_ of them, TM x TN each)
// hold their sums in acc: the fused epilogue, or the raw fp32 sums parked in `park`
// (BM_ x BN_, row-major) when it is given. Ends with a barrier, so the LDS may be
// reused by the caller. PF_OK: the epilogue's global inputs may be loaded one
// 16-row block ahead (registers allow it).
// RB: 16-row blocks per round. A round parks RB blocks of the wave's quadrant and
// its lanes take 16-column items of them, so RB is chosen to make the items a
// multiple of 64 (with 96-wide wave tiles one block gives 96 items: a second pass
// with half the lanes idle; two give 192, three full passes).
template <int BN_, int WM_, int WN_, int TM, int TN, int EPI, bool PF_OK, int RB = 1>
__device__ __forceinline__ void tile_epilogue(const GemmArgs& p, char* smem, int tm, int m0, int n0,
                                              f32x4 (&acc)[TM / 16][TN / 16], float* park) {
  constexpr int NW = WM_ * WN_;
  constexpr int FM = TM / 16, FN = TN / 16;
  static_assert(FM % RB == 0, "whole rounds of row blocks");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN_, wn = wave % WN_;
  // Epilogue through LDS: each wave parks RB 16-row blocks of its TM x TN quadrant,
  // then a lane handles 16 contiguous columns of one row (TN/16 such groups per
  // row, so 64 lanes cover the round in one or more passes), so bias, residual and
  // saved derivative inputs are read and outputs written as vectors.
  constexpr int ELD = TN + 4;
  constexpr int CG = TN / 16, ROWS = 16 * RB, ITEMS = ROWS * CG, PASSES = (ITEMS + 63) / 64;
  // epilogue inputs of round i (item it = lane + 64*ps: row er, columns ec..)
  // (the fp32 residual of two blocks does not fit beside the accumulators of two
  // workgroups per CU: the 32-wide-slice residual kernel loads it in place)
  constexpr bool PF = EpiPre<EPI>::ON && PF_OK;
  EpiPre<EPI> pre[PF ? 2 : 1][PASSES];
  auto prefetch = [&](int i, EpiPre<EPI> (&dst)[PASSES]) {
#pragma unroll
    for (int ps = 0; ps < PASSES; ps++) {
      const int it = lane + 64 * ps;
      if (ITEMS % 64 != 0 && it >= ITEMS) break;
      const int row = m0 + wm * TM + i * ROWS + it / CG, col0 = n0 + wn * TN + (it % CG) * 16;
      if (row < p.M && col0 + 16 <= p.N && p.c_vec) dst[ps].load(p, row, col0);
    }
  };
  if constexpr (PF)
    if (!park) prefetch(0, pre[0]);
  // the bias of an item's 16 columns is the same in every round
  constexpr bool PB = epi_has_bias<EPI>();
  f32x4 bias16[PB ? PASSES : 1][4];
  if constexpr (PB) {
#pragma unroll
    for (int ps = 0; ps < PASSES; ps++) {
      const int it = lane + 64 * ps;
      if (ITEMS % 64 != 0 && it >= ITEMS) break;
      const int col0 = n0 + wn * TN + (it % CG) * 16;
      if (!park && col0 + 16 <= p.N && p.c_vec)
#pragma unroll
        for (int q = 0; q < 4; q++) bias16[ps][q] = *(const f32x4*)(p.bias + col0 + 4 * q);
    }
  }
  // Every wave is done with the stage buffers: their LDS reads have returned, and
  // the last k-slices waited for all global->LDS loads. A plain s_barrier, so the
  // epilogue loads just issued stay in flight.
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  float* scr = (float*)smem + wave * ROWS * ELD;
  // fused bias gradient (GELU backward): this lane's column sums of its items
  constexpr bool CS = epi_act_bwd<EPI>();
  const bool colsum = CS && p.colsum && !park;
  float cs[PASSES][16];
#pragma unroll
  for (int ps = 0; ps < PASSES; ps++)
#pragma unroll
    for (int e = 0; e < 16; e++) cs[ps][e] = 0.f;
#pragma unroll
  for (int i = 0; i < FM / RB; i++) {
    if constexpr (PF)
      if (!park && i + 1 < FM / RB) prefetch(i + 1, pre[(i + 1) & 1]);
#pragma unroll
    for (int r = 0; r < RB; r++)
#pragma unroll
      for (int j = 0; j < FN; j++)
#pragma unroll
        for (int e = 0; e < 4; e++)
          scr[(16 * r + 4 * (lane >> 4) + e) * ELD + j * 16 + (lane & 15)] = acc[i * RB + r][j][e];
#pragma unroll
    for (int ps = 0; ps < PASSES; ps++) {
      const int it = lane + 64 * ps;
      if (ITEMS % 64 != 0 && it >= ITEMS) break;
      const int er = it / CG, ec = (it % CG) * 16;
      float v[16];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const f32x4 t = *(const f32x4*)(scr + er * ELD + ec + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; e++) v[4 * q + e] = t[e];
      }
      const int rt = wm * TM + i * ROWS + er;    // row within the tile
      if (park) {
        float* d = park + (int64_t)rt * BN_ + wn * TN + ec;
#pragma unroll
        for (int q = 0; q < 4; q++) *(f32x4*)(d + 4 * q) = (f32x4){v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
      } else {
        const int row = m0 + rt, col0 = n0 + wn * TN + ec;
        if (row < p.M && col0 < p.N)
          epi_store16<EPI>(p, row, col0, v, (col0 + 16 <= p.N) && p.c_vec, cs[ps], PF ? &pre[i & 1][ps] : nullptr,
                           PB ? bias16[ps] : nullptr);
      }
    }
  }
  if constexpr (CS) {
    if (colsum) {
      // rows of each wave's items through its own scratch, then the WM waves that
      // share a column range in a fixed order, into one partial row per tile row
      float* red = (float*)smem + NW * ROWS * ELD;   // [WM_][BN_]
#pragma unroll
      for (int ps = 0; ps < PASSES; ps++) {
        const int it = lane + 64 * ps;
        if (ITEMS % 64 != 0 && it >= ITEMS) break;
        const int er = it / CG, ec = (it % CG) * 16;
#pragma unroll
        for (int e = 0; e < 16; e++) scr[er * ELD + ec + e] = cs[ps][e];
      }
      for (int c = lane; c < TN; c += 64) {
        float t = 0.f;
#pragma unroll
        for (int r = 0; r < ROWS; r++) t += scr[r * ELD + c];
        red[wm * BN_ + wn * TN + c] = t;
      }
      __syncthreads();
      for (int c = threadIdx.x; c < BN_; c += 64 * NW) {
        float t = red[c];
#pragma unroll
        for (int q = 1; q < WM_; q++) t += red[q * BN_ + c];
        if (n0 + c < p.N) p.colsum[(int64_t)tm * p.N + n0 + c] = t;
      }
    }
  }
  __syncthreads();
}

// One output tile over k-slices [s0, s1) of 32. With park == nullptr the fused
// epilogue is applied; otherwise the raw fp32 sums go to park (BM_ x BN_, row-major).
// Ends with a barrier, so the LDS may be reused by the caller.
// KS: k per slice, 32, or 64 when both operands are k-contiguous (s0, s1 count
// slices of KS).
template <int BM_, int BN_, int WM_, int WN_, int STAGES, bool AK, bool BK_, int EPI, int KS = 32>
__device__ __forceinline__ void dma_tile(const GemmArgs& p, char* smem, int tm, int tn, int s0, int s1,
                                         float* park, int rot = 0) {
  static_assert(KS == 32 || (KS == 64 && AK && BK_), "64-wide slices need k-contiguous operands");
  constexpr int NW = WM_ * WN_;
  constexpr int TM = BM_ / WM_, TN = BN_ / WN_;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int AB = BM_ * KS * 2, BB = BN_ * KS * 2, SB = AB + BB;
  constexpr int LPS = (AB + BB) / 1024 / NW;     // load instructions per stage per wave
  const int m0 = tm * BM_, n0 = tn * BN_;
  const bf16* A = (const bf16*)p.A;
  const bf16* B = (const bf16*)p.B;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN_, wn = wave % WN_;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int nk = s1 - s0;
  // resources from the tile's first row (k-contiguous) or column (m-contiguous)
  const __amdgpu_buffer_rsrc_t ra = tile_rsrc(AK ? A + (int64_t)m0 * p.lda : A + m0);
  const __amdgpu_buffer_rsrc_t rb = tile_rsrc(BK_ ? B + (int64_t)n0 * p.ldb : B + n0);
  const int am = p.M - m0, bn = p.N - n0;
  auto issue = [&](int t) {
    char* st = smem + (t % STAGES) * SB;
    // rot: this tile's first k-slice (the tiles of a launch then walk the shared operand
    // rows at different k instead of all at once)
    const int tr = t + rot < nk ? t + rot : t + rot - nk;
    const int k0 = (s0 + tr) * KS;
    if constexpr (KS == 64) {
      dma_kc64<BM_, NW>(ra, p.lda, am, k0, st, wave, lane);
      dma_kc64<BN_, NW>(rb, p.ldb, bn, k0, st + AB, wave, lane);
    } else {
      if constexpr (AK) dma_kc<BM_, NW>(ra, p.lda, am, k0, st, wave, lane);
      else dma_mc<BM_, NW>(ra, p.lda, am, k0, st, wave, lane);
      if constexpr (BK_) dma_kc<BN_, NW>(rb, p.ldb, bn, k0, st + AB, wave, lane);
      else dma_mc<BN_, NW>(rb, p.ldb, bn, k0, st + AB, wave, lane);
    }
  };

#pragma unroll
  for (int t = 0; t < STAGES - 1; t++)
    if (t < nk) issue(t);

  for (int t = 0; t < nk; t++) {
    // A plain s_barrier: __syncthreads() would also wait for every global->LDS
    // load still in flight, which would serialise the pipeline. LDS reads of the
    // previous slice are complete (their MFMAs consumed them) before the barrier.
    if (t + STAGES - 2 < nk) {
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((STAGES - 2) * LPS) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    if (t + STAGES - 1 < nk) issue(t + STAGES - 1);
    const char* As = smem + (t % STAGES) * SB;
    const char* Bs = As + AB;
#pragma unroll
    for (int h = 0; h < KS / 32; h++) {
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; i++) {
        const int r = wm * TM + i * 16;
        if constexpr (KS == 64) af[i] = frag_kc64(As, r + (lane & 15), h);
        else if constexpr (AK) af[i] = frag_kc<BM_>(As, r + (lane & 15));
        else af[i] = frag_mc<BM_>(As, r);
      }
#pragma unroll
      for (int j = 0; j < FN; j++) {
        const int r = wn * TN + j * 16;
        if constexpr (KS == 64) bfr[j] = frag_kc64(Bs, r + (lane & 15), h);
        else if constexpr (BK_) bfr[j] = frag_kc<BN_>(Bs, r + (lane & 15));
        else bfr[j] = frag_mc<BN_>(Bs, r);
      }
#pragma unroll
      for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) acc[i][j] = Mfma<bf16>::mma(af[i], bfr[j], acc[i][j]);
    }
  }

  // two row blocks per epilogue round when one leaves lanes idle and the scratch fits the stages
  constexpr int CGE = TN / 16;
  constexpr bool RB2 = CGE % 4 != 0 && (2 * CGE) % 4 == 0 && FM % 2 == 0 &&
                       (NW * 32 * (TN + 4) + WM_ * BN_) * 4 <= STAGES * SB;
  tile_epilogue<BN_, WM_, WN_, TM, TN, EPI, !(epi_resid<EPI>() && KS == 32), RB2 ? 2 : 1>(p, smem, tm, m0, n0, acc,
                                                                                          park);
}


// The 192-wide, 32-wide-slice kernels and the 96 x 192 kernel run two workgroups per
// CU (their LDS rings allow it); the register budget is held to that occupancy so the
// epilogue's prefetched inputs cannot push them to one.
template <int BM_, int BN_, int WM_, int WN_, int STAGES, bool AK, bool BK_, int EPI, int KS = 32>
__global__ __launch_bounds__(64 * WM_ * WN_) __attribute__((amdgpu_waves_per_eu((KS == 32 && BM_ == 192) || BM_ == 96 ? 2 : 1)))
void gemm_dma_kernel(GemmArgs p) {
  constexpr int SB = (BM_ + BN_) * KS * 2;
  static_assert(STAGES * SB >= (WM_ * WN_ * 16 * (BN_ / WN_ + 4) + WM_ * BN_) * 4, "epilogue scratch fits the stages");
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * SB];
  if ((int)blockIdx.x >= p.stagger_lo && (int)blockIdx.x < p.stagger_hi)
    for (int i = 0; i < p.stagger_iters; i++) __builtin_amdgcn_s_sleep(32);
  const int tiles_m = (p.M + BM_ - 1) / BM_, tiles_n = (p.N + BN_ - 1) / BN_;
  const int total = tiles_m * tiles_n;
  // the hardware deals workgroups round-robin to the 8 XCDs; give each XCD a
  // contiguous run of tiles
  int bid = blockIdx.x;
  if (total % 8 == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  int tm, tn;
  tile_coords(bid, tiles_m, tiles_n, tm, tn);
  const int s0 = blockIdx.z * (p.kchunk / KS);
  const int s1 = min(p.K, (int)(blockIdx.z + 1) * p.kchunk) / KS;
  const int rot = p.krot && gridDim.z == 1 ? (int)((int64_t)bid * (s1 - s0) / total) : 0;
  dma_tile<BM_, BN_, WM_, WN_, STAGES, AK, BK_, EPI, KS>(p, smem, tm, tn, s0, s1, nullptr, rot);
}

// Stream-K: gridDim.x workgroups share the tiles x (K/32) slice-units evenly, each a
// contiguous range; a tile cut between workgroups is parked as fp32 partial sums
// (slot = tile * maxseg + segment) and finished by sk_fixup_kernel in a fixed order.
__device__ inline int sk_owner(long long x, int W, long long U) { return (int)(((x + 1) * W - 1) / U); }

template <int BM_, int BN_, int WM_, int WN_, int STAGES, bool AK, bool BK_, int EPI>
__global__ __launch_bounds__(64 * WM_ * WN_) void gemm_sk_kernel(GemmArgs p, float* ws, int maxseg) {
  constexpr int SB = (BM_ + BN_) * 32 * 2;
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * SB];
  const int tiles_m = (p.M + BM_ - 1) / BM_, tiles_n = (p.N + BN_ - 1) / BN_;
  const int KI = p.K / 32;
  const int W = gridDim.x, w = blockIdx.x;
  const long long U = (long long)tiles_m * tiles_n * KI;
  const long long beg = (long long)w * U / W, end = (long long)(w + 1) * U / W;
  for (long long x = beg; x < end;) {
    const int t = (int)(x / KI);
    const int s0 = (int)(x - (long long)t * KI);
    const int s1 = (int)min((long long)KI, end - (long long)t * KI);
    const int first = sk_owner((long long)t * KI, W, U);
    const int last = sk_owner((long long)t * KI + KI - 1, W, U);
    float* park = nullptr;
    if (first != last) park = ws + ((int64_t)t * maxseg + (w - first)) * (BM_ * BN_);
    int tm, tn;
    tile_coords(t, tiles_m, tiles_n, tm, tn);
    dma_tile<BM_, BN_, WM_, WN_, STAGES, AK, BK_, EPI>(p, smem, tm, tn, s0, s1, park);
    x = (long long)t * KI + s1;
  }
}

// One workgroup per 16 rows of a split tile (blockIdx.y picks the rows), one
// thread per 16-column run: sums the tile's parked partials in segment order and
// applies the epilogue.
template <int BM_, int BN_, int EPI>
__global__ __launch_bounds__(256) void sk_fixup_kernel(GemmArgs p, const float* __restrict__ ws, int maxseg, int W) {
  static_assert(BN_ == 256, "one thread per 16 columns of a 256-wide tile row");
  const int tiles_m = (p.M + BM_ - 1) / BM_, tiles_n = (p.N + BN_ - 1) / BN_;
  const int KI = p.K / 32;
  const long long U = (long long)tiles_m * tiles_n * KI;
  const int t = blockIdx.x;
  const int first = sk_owner((long long)t * KI, W, U);
  const int nseg = sk_owner((long long)t * KI + KI - 1, W, U) - first + 1;
  if (nseg == 1) return;
  int tm, tn;
  tile_coords(t, tiles_m, tiles_n, tm, tn);
  const int r = blockIdx.y * 16 + (threadIdx.x >> 4), c0 = (threadIdx.x & 15) * 16;
  const int row = tm * BM_ + r, col0 = tn * BN_ + c0;
  if (row >= p.M || col0 >= p.N) return;
  const float* src = ws + (int64_t)t * maxseg * (BM_ * BN_) + r * BN_ + c0;
  float v[16];
#pragma unroll
  for (int e = 0; e < 16; e++) v[e] = 0.f;
  for (int sg = 0; sg < nseg; sg++) {
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
      const f32x4 x = *(const f32x4*)(src + (int64_t)sg * (BM_ * BN_) + 4 * q4);
#pragma unroll
      for (int e = 0; e < 4; e++) v[4 * q4 + e] += x[e];
    }
  }
  float unused[16];
  epi_store16<EPI>(p, row, col0, v, p.c_vec && col0 + 16 <= p.N, unused);
}


template <int BM_, int BN_, int WM_, int WN_, int STAGES, bool AK, bool BK_, int KS = 32>
static hipError_t dma_epi(const GemmArgs& a, int epi, int splits, hipStream_t s) {
  const int total = ((a.M + BM_ - 1) / BM_) * ((a.N + BN_ - 1) / BN_);
  dim3 grid(total, 1, splits);
  switch (epi) {
#define GPT_DMA_CASE(E)                                                                                              \
  case E:                                                                                                            \
    hipLaunchKernelGGL((gemm_dma_kernel<BM_, BN_, WM_, WN_, STAGES, AK, BK_, E, KS>), grid, dim3(64 * WM_ * WN_), 0, \
                       s, a);                                                                                        \
    break;
    GPT_DMA_CASE(EPI_STORE)
    GPT_DMA_CASE(EPI_BIAS)
    GPT_DMA_CASE(EPI_BIAS_RESID)
    GPT_DMA_CASE(EPI_BIAS_GELU)
    GPT_DMA_CASE(EPI_F32)
    GPT_DMA_CASE(EPI_GELU_BWD)
    GPT_DMA_CASE(EPI_ACC)
    GPT_DMA_CASE(EPI_BIAS_RESID_DROP)
    GPT_DMA_CASE(EPI_BIAS_RELU)
    GPT_DMA_CASE(EPI_RELU_BWD)
#undef GPT_DMA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BM_, int BN_, int WM_, int WN_, int STAGES, bool AK, bool BK_>
static hipError_t sk_epi(const GemmArgs& a, int epi, int W, float* ws, int maxseg, hipStream_t s) {
  const int tiles = ((a.M + BM_ - 1) / BM_) * ((a.N + BN_ - 1) / BN_);
  switch (epi) {
#define GPT_SK_CASE(E)                                                                                             \
  case E:                                                                                                          \
    hipLaunchKernelGGL((gemm_sk_kernel<BM_, BN_, WM_, WN_, STAGES, AK, BK_, E>), dim3(W), dim3(64 * WM_ * WN_), 0, \
                       s, a, ws, maxseg);                                                                          \
    hipLaunchKernelGGL((sk_fixup_kernel<BM_, BN_, E>), dim3(tiles, BM_ / 16), dim3(256), 0, s, a,                 \
                       (const float*)ws, maxseg, W);                                                               \
    break;
    GPT_SK_CASE(EPI_STORE)
    GPT_SK_CASE(EPI_BIAS)
    GPT_SK_CASE(EPI_BIAS_RESID)
    GPT_SK_CASE(EPI_BIAS_GELU)
    GPT_SK_CASE(EPI_F32)
    GPT_SK_CASE(EPI_GELU_BWD)
    GPT_SK_CASE(EPI_ACC)
    GPT_SK_CASE(EPI_BIAS_RESID_DROP)
    GPT_SK_CASE(EPI_BIAS_RELU)
    GPT_SK_CASE(EPI_RELU_BWD)
#undef GPT_SK_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BM_, int BN_, int WM_, int WN_, int STAGES>
static hipError_t sk_layout(const GemmDesc& d, const GemmArgs& a, int W, float* ws, int maxseg, hipStream_t s) {
  if (d.a_kc && d.b_kc) return sk_epi<BM_, BN_, WM_, WN_, STAGES, true, true>(a, d.epi, W, ws, maxseg, s);
  if (d.a_kc && !d.b_kc) return sk_epi<BM_, BN_, WM_, WN_, STAGES, true, false>(a, d.epi, W, ws, maxseg, s);
  if (!d.a_kc && !d.b_kc) return sk_epi<BM_, BN_, WM_, WN_, STAGES, false, false>(a, d.epi, W, ws, maxseg, s);
  return hipErrorInvalidValue;
}

template <int BM_, int BN_, int WM_, int WN_, int STAGES>
static hipError_t dma_layout(const GemmDesc& d, const GemmArgs& a, int splits, hipStream_t s) {
  if (d.a_kc && d.b_kc) return dma_epi<BM_, BN_, WM_, WN_, STAGES, true, true>(a, d.epi, splits, s);
  if (d.a_kc && !d.b_kc) return dma_epi<BM_, BN_, WM_, WN_, STAGES, true, false>(a, d.epi, splits, s);
  if (!d.a_kc && !d.b_kc) return dma_epi<BM_, BN_, WM_, WN_, STAGES, false, false>(a, d.epi, splits, s);
  return hipErrorInvalidValue;
}

// C[m, n] = beta * C[m, n] + sum_z part[z, m, n], z in order.
__global__ void splitk_reduce_kernel(const float* __restrict__ part, int S, int M, int N, float* C, int64_t ldc,
                                     float beta) {
  const int64_t total = (int64_t)M * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    float s = 0.f;
    for (int z = 0; z < S; z++) s += part[(int64_t)z * total + i];
    const int64_t m = i / N, n = i % N;
    float* c = C + m * ldc + n;
    *c = (beta != 0.f ? beta * *c : 0.f) + s;
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
    GPT_EPI_CASE(EPI_BIAS_RESID_DROP)
    GPT_EPI_CASE(EPI_BIAS_RELU)
    GPT_EPI_CASE(EPI_RELU_BWD)
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

static int num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      n = cus;
    else
      n = 256;
  }
  return n;
}

// ----------------------------------------------------------------------------- grouped weight gradients
__device__ inline int find_problem(const WgradProblem* __restrict__ pr, int np, int t) {
  int lo = 0, hi = np - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pr[mid].first_tile <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__device__ inline GemmArgs problem_args(const WgradProblem& pr, int K, float beta) {
  GemmArgs p;
  p.A = pr.A; p.lda = pr.lda; p.B = pr.B; p.ldb = pr.ldb; p.C = pr.C; p.ldc = pr.ldc;
  p.M = pr.M; p.N = pr.N; p.K = K;
  p.bias = nullptr; p.resid = nullptr; p.ldr = 0; p.aux = nullptr; p.ldaux = 0;
  p.beta = beta; p.a_vec = 1; p.b_vec = 1; p.c_vec = pr.c_vec; p.kchunk = K; p.part = nullptr; p.colsum = nullptr;
  return p;
}

// Stream-K partial tiles: workgroup w parks at most two (the tile its range starts
// in, slot 0, and the one it ends in, slot 1).
__device__ inline int group_slot(int w, int r, int W, long long U, int KI) {
  const long long beg = (long long)w * U / W;
  return 2 * w + (r == (int)(beg / KI) ? 0 : 1);
}

template <int BM_, int BN_, int WM_, int WN_, int STAGES>
__global__ __launch_bounds__(64 * WM_ * WN_) void gemm_group_kernel(const WgradProblem* __restrict__ probs, int nprob,
                                                                    int total, int dp_tiles, int K, float beta,
                                                                    float* __restrict__ ws) {
  constexpr int SB = (BM_ + BN_) * 32 * 2;
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * SB];
  const int W = gridDim.x, w = blockIdx.x, KI = K / 32;
  auto run = [&](int t, int s0, int s1, float* park) {
    const WgradProblem pr = probs[find_problem(probs, nprob, t)];
    const GemmArgs p = problem_args(pr, K, beta);
    int tm, tn;
    tile_coords(t - pr.first_tile, pr.tiles_m, pr.tiles_n, tm, tn);
    dma_tile<BM_, BN_, WM_, WN_, STAGES, false, false, EPI_ACC>(p, smem, tm, tn, s0, s1, park);
  };
  // whole tiles, one round of W at a time; workgroups are dealt round-robin to the 8
  // XCDs, so give each XCD a contiguous run of the round's tiles (they share A or B
  // panels in that XCD's L2)
  const int lw = W % 8 == 0 ? (w & 7) * (W >> 3) + (w >> 3) : w;
  for (int t = lw; t < dp_tiles; t += W) run(t, 0, KI, nullptr);
  const int rem = total - dp_tiles;
  if (rem == 0) return;
  const long long U = (long long)rem * KI;
  const long long beg = (long long)w * U / W, end = (long long)(w + 1) * U / W;
  for (long long x = beg; x < end;) {
    const int r = (int)(x / KI);
    const int s0 = (int)(x - (long long)r * KI);
    const int s1 = (int)min((long long)KI, end - (long long)r * KI);
    const bool split = sk_owner((long long)r * KI, W, U) != sk_owner((long long)r * KI + KI - 1, W, U);
    run(dp_tiles + r, s0, s1, split ? ws + (int64_t)group_slot(w, r, W, U, KI) * (BM_ * BN_) : nullptr);
    x = (long long)r * KI + s1;
  }
}

// One workgroup per 16 rows of a split leftover tile: its parked partials summed in
// owner order, then C = beta * C + sum.
template <int BM_, int BN_>
__global__ __launch_bounds__(256) void group_fixup_kernel(const WgradProblem* __restrict__ probs, int nprob,
                                                          int total, int dp_tiles, int K, float beta,
                                                          const float* __restrict__ ws, int W) {
  static_assert(BN_ == 256, "one thread per 16 columns of a 256-wide tile row");
  const int KI = K / 32, rem = total - dp_tiles;
  const long long U = (long long)rem * KI;
  const int r = blockIdx.x;
  const int first = sk_owner((long long)r * KI, W, U), last = sk_owner((long long)r * KI + KI - 1, W, U);
  if (first == last) return;
  const int t = dp_tiles + r;
  const WgradProblem pr = probs[find_problem(probs, nprob, t)];
  const GemmArgs p = problem_args(pr, K, beta);
  int tm, tn;
  tile_coords(t - pr.first_tile, pr.tiles_m, pr.tiles_n, tm, tn);
  const int rr = blockIdx.y * 16 + (threadIdx.x >> 4), c0 = (threadIdx.x & 15) * 16;
  const int row = tm * BM_ + rr, col0 = tn * BN_ + c0;
  if (row >= p.M || col0 >= p.N) return;
  float v[16];
#pragma unroll
  for (int e = 0; e < 16; e++) v[e] = 0.f;
  for (int o = first; o <= last; o++) {
    if ((long long)o * U / W == (long long)(o + 1) * U / W) continue;   // a workgroup with no units
    const float* src = ws + (int64_t)group_slot(o, r, W, U, KI) * (BM_ * BN_) + rr * BN_ + c0;
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
      const f32x4 x = *(const f32x4*)(src + 4 * q4);
#pragma unroll
      for (int e = 0; e < 4; e++) v[4 * q4 + e] += x[e];
    }
  }
  float unused[16];
  epi_store16<EPI_ACC>(p, row, col0, v, p.c_vec && col0 + 16 <= p.N, unused);
}

// ----------------------------------------------------------------------------- wide tiles
// A (2 TM) x (2 TN) tile on four wavefronts of TM x TN (the grouped weight gradients
// use 256 x 256 tiles of 128 x 128), one workgroup per CU, with the accumulators held
// in the accumulation registers for the whole k-loop. 128 x 128 wavefront tiles read
// 16 KB of fragments per 32-wide slice for 64 MFMAs, half the LDS traffic per MFMA
// of 64 x 64 ones. (On k-contiguous operands this schedule measured slower than the
// 192 x 192 kernels with two workgroups per CU: with one, each tile's pipeline fill
// and output stores stand between k-loops.)
// The LDS latency is hidden inside each wavefront, with few registers: a slice runs
// row block by row block (FN MFMAs on one A fragment each); the A fragment of row
// block i+2 is read during row block i into a small ring (crossing into the next
// slice at the end), and the next slice's B fragments are read into a second set, a
// share of them per row block. One barrier per slice publishes the next slice's
// stage and frees the stage the next load overwrites; loads run STAGES - 2 slices
// ahead of the slice being read.

// One 16 x 16 x 32 bf16 MFMA accumulating into acc, which the constraint keeps in
// the accumulation registers for the whole k-loop (the compiler otherwise moves the
// accumulators between register files around the loop's blocks). Volatile: the
// MFMAs keep the order written; LDS reads are still scheduled between them.
__device__ __forceinline__ void mfma_agpr(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// After the last mfma_agpr of a tile and before its accumulators are read: the
// compiler cannot see the MFMA inside the asm, so the wait states between an MFMA
// writing a register and a plain read of it are spent here (24 > the 18 an 8-pass
// MFMA needs), and each accumulator is passed through an empty asm after them, so
// no read of it can be scheduled before the wait.
template <int FM, int FN>
__device__ __forceinline__ void mfma_agpr_drain(f32x4 (&acc)[FM][FN]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < FM; i++)
#pragma unroll
    for (int j = 0; j < FN; j++) asm volatile("" : "+a"(acc[i][j]));
}

template <int TM, int TN, bool AK, bool BK_, int STAGES, int AHEAD = 3>
__device__ __forceinline__ void wide_mainloop(const GemmArgs& p, char* smem, int m0, int n0, int s0, int s1,
                                              f32x4 (&acc)[TM / 16][TN / 16]) {
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int BM_ = 2 * TM, BN_ = 2 * TN, NW = 4, KS = 32;
  constexpr int AB = BM_ * KS * 2, SB = AB + BN_ * KS * 2;
  constexpr int LPS = SB / 1024 / NW;              // load instructions per stage per wavefront
  // A fragments are read AHEAD row blocks early into a ring of RING (a multiple of
  // FM's divisor so the ring wraps into the next slice in phase); the next slice's B
  // fragments are read during the first half of the slice, BPR per row block.
  constexpr int RING = FM % (AHEAD + 1) == 0 ? AHEAD + 1 : FM;
  constexpr int BPR = (2 * FN + FM - 1) / FM;
  static_assert(STAGES >= 3, "a stage is read while one is loaded and one is being freed");
  static_assert(FM % RING == 0 && RING > AHEAD && FM >= AHEAD, "the A ring wraps into the next slice in phase");
  const bf16* A = (const bf16*)p.A;
  const bf16* B = (const bf16*)p.B;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const __amdgpu_buffer_rsrc_t ra = tile_rsrc(AK ? A + (int64_t)m0 * p.lda : A + m0);
  const __amdgpu_buffer_rsrc_t rb = tile_rsrc(BK_ ? B + (int64_t)n0 * p.ldb : B + n0);
  const int am = p.M - m0, bn = p.N - n0;
  auto issue_to = [&](char* st, int t) {
    const int k0 = (s0 + t) * KS;
    if constexpr (AK) dma_kc<BM_, NW>(ra, p.lda, am, k0, st, wave, lane);
    else dma_mc<BM_, NW>(ra, p.lda, am, k0, st, wave, lane);
    if constexpr (BK_) dma_kc<BN_, NW>(rb, p.ldb, bn, k0, st + AB, wave, lane);
    else dma_mc<BN_, NW>(rb, p.ldb, bn, k0, st + AB, wave, lane);
  };
  auto afrag = [&](const char* st, int i) {
    if constexpr (AK) return frag_kc<BM_>(st, wm * TM + i * 16 + (lane & 15));
    else return frag_mc<BM_>(st, wm * TM + i * 16);
  };
  auto bfrag = [&](const char* st, int j) {
    if constexpr (BK_) return frag_kc<BN_>(st + AB, wn * TN + j * 16 + (lane & 15));
    else return frag_mc<BN_>(st + AB, wn * TN + j * 16);
  };
  const int nk = s1 - s0;
#pragma unroll
  for (int t = 0; t < STAGES - 1; t++)
    if (t < nk) issue_to(smem + t * SB, t);
  // stage 0 is in LDS for every wavefront
  if (nk >= STAGES - 1) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((STAGES - 2) * LPS) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  bf16x8 fa[RING], fb0[FN], fb1[FN];
#pragma unroll
  for (int i = 0; i < AHEAD; i++) fa[i] = afrag(smem, i);
#pragma unroll
  for (int j = 0; j < FN; j++) fb0[j] = bfrag(smem, j);
  // Slice t: its B fragments are in fb_c, rows 0 .. AHEAD-1 of A in the ring. The
  // steady state (a later slice exists and the slice STAGES - 1 ahead is to be
  // loaded) has no branches, so the accumulators stay in their registers through it.
  // The three stages a slice touches (the one loaded, the two read) are distinct and
  // passed as restrict pointers: the compiler can then tell that the fragment reads
  // do not touch the stage being loaded (otherwise it waits for every load in flight
  // before each transposing read).
  auto slice_in = [&](auto steady_c, int t, bf16x8 (&fb_c)[FN], bf16x8 (&fb_n)[FN], char* __restrict__ dst,
                      const char* __restrict__ cur, const char* __restrict__ nxt) {
    constexpr bool STEADY = decltype(steady_c)::value;
    const bool more = STEADY || t + 1 < nk;
    if (STEADY) {
      // this wavefront's loads of slice t+1 have landed; after the barrier every
      // wavefront's have, and every wavefront has consumed its reads of slice t-1,
      // whose stage the next load overwrites
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((STAGES - 3) * LPS) : "memory");
      issue_to(dst, t + STAGES - 1);
    } else if (more) {
      if (t + STAGES - 2 < nk) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((STAGES - 3) * LPS) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      if (t + STAGES - 1 < nk) issue_to(dst, t + STAGES - 1);
    }
#pragma unroll
    for (int i = 0; i < FM; i++) {
      __builtin_amdgcn_sched_barrier(0);
      if (i + AHEAD < FM) fa[(i + AHEAD) % RING] = afrag(cur, i + AHEAD);
      else if (more) fa[(i + AHEAD) % RING] = afrag(nxt, i + AHEAD - FM);
      if (more)
#pragma unroll
        for (int j = i * BPR; j < (i + 1) * BPR && j < FN; j++) fb_n[j] = bfrag(nxt, j);
#pragma unroll
      for (int j = 0; j < FN; j++) mfma_agpr(acc[i][j], fa[i % RING], fb_c[j]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto slice = [&](auto steady_c, int t, bf16x8 (&fb_c)[FN], bf16x8 (&fb_n)[FN]) {
    slice_in(steady_c, t, fb_c, fb_n, smem + ((t + STAGES - 1) % STAGES) * SB, smem + (t % STAGES) * SB,
             smem + ((t + 1) % STAGES) * SB);
  };
  using steady = std::integral_constant<bool, true>;
  using edge = std::integral_constant<bool, false>;
  int t = 0;
  for (; t + STAGES < nk; t += 2) {   // both slices steady: t + 1 + STAGES - 1 < nk
    slice(steady{}, t, fb0, fb1);
    slice(steady{}, t + 1, fb1, fb0);
  }
  for (; t + 1 < nk; t += 2) {
    slice(edge{}, t, fb0, fb1);
    slice(edge{}, t + 1, fb1, fb0);
  }
  if (t < nk) slice(edge{}, t, fb0, fb1);
  mfma_agpr_drain<FM, FN>(acc);
}

// All weight gradients of a micro-batch on wide tiles: the grouped launch of
// gemm_group_kernel with 256 x 256 tiles on four wavefronts of 128 x 128.
template <int STAGES>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_group_wide_kernel(const WgradProblem* __restrict__ probs, int nprob, int total, int dp_tiles, int K,
                            float beta, float* __restrict__ ws) {
  constexpr int SB = 2 * 256 * 32 * 2;
  static_assert(STAGES * SB >= 4 * 16 * (128 + 4) * 4, "epilogue scratch fits the stages");
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * SB];
  const int W = gridDim.x, w = blockIdx.x, KI = K / 32;
  auto run = [&](int t, int s0, int s1, float* park) {
    const WgradProblem pr = probs[find_problem(probs, nprob, t)];
    const GemmArgs p = problem_args(pr, K, beta);
    int tm, tn;
    tile_coords(t - pr.first_tile, pr.tiles_m, pr.tiles_n, tm, tn);
    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
      for (int j = 0; j < 8; j++) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
    wide_mainloop<128, 128, false, false, STAGES>(p, smem, tm * 256, tn * 256, s0, s1, acc);
    tile_epilogue<256, 2, 2, 128, 128, EPI_ACC, true>(p, smem, tm, tm * 256, tn * 256, acc, park);
  };
  const int lw = W % 8 == 0 ? (w & 7) * (W >> 3) + (w >> 3) : w;
  for (int t = lw; t < dp_tiles; t += W) run(t, 0, KI, nullptr);
  const int rem = total - dp_tiles;
  if (rem == 0) return;
  const long long U = (long long)rem * KI;
  const long long beg = (long long)w * U / W, end = (long long)(w + 1) * U / W;
  for (long long x = beg; x < end;) {
    const int r = (int)(x / KI);
    const int s0 = (int)(x - (long long)r * KI);
    const int s1 = (int)min((long long)KI, end - (long long)r * KI);
    const bool split = sk_owner((long long)r * KI, W, U) != sk_owner((long long)r * KI + KI - 1, W, U);
    run(dp_tiles + r, s0, s1, split ? ws + (int64_t)group_slot(w, r, W, U, KI) * (256 * 256) : nullptr);
    x = (long long)r * KI + s1;
  }
}

static int num_cus();

// ----------------------------------------------------------------------------- few output rows
// The epilogue inputs of a few-rows tile (lane: column n0 + (lane & 15), rows 4g..4g+3),
// loaded by the wavefront that stores the tile at the start of the kernel, so that
// their latency overlaps the weight stream instead of following the reduction.
template <int EPI>
struct SkinnyEpiIn {
  float bias = 0.f;
  f32x4 res = (f32x4){0.f, 0.f, 0.f, 0.f};
  __device__ inline void load(const GemmArgs& p, int col, int g) {
    if (col >= p.N) return;
    bias = epi_bias<EPI>(p, col);
    if constexpr (EPI == EPI_BIAS_RESID) {
#pragma unroll
      for (int i = 0; i < 4; i++)
        if (4 * g + i < p.M) res[i] = p.resid[(int64_t)(4 * g + i) * p.ldr + col];
    }
  }
  __device__ inline void store(const GemmArgs& p, int col, int g, const f32x4& t) const {
    if (col >= p.N) return;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int row = 4 * g + i;
      if (row >= p.M) continue;
      if constexpr (EPI == EPI_BIAS_RESID) ((float*)p.C)[(int64_t)row * p.ldc + col] = res[i] + (t[i] + bias);
      else epi_store<bf16, EPI>(p, row, col, t[i], bias);
    }
  }
};

// M <= 16 (one token per sequence while decoding): the weight operand streams from
// HBM once and nothing is worth staging. One workgroup of NW wavefronts per 16 output
// columns; wavefront w multiplies every NW-th 32-wide k-slice with fragments read
// straight from global memory (A: the M rows, zero past M; B: 16 weight rows), and
// the NW partial tiles are added in LDS in a fixed order before the element epilogue
// (bias, residual, GELU, store). NW = 16 for outputs of up to 4 column groups per CU;
// wider outputs (the lm_head) take NW = 4, so that more workgroups are resident per CU
// (21.4 against 23.2 us for the GPT-2 lm_head at 12 rows). Measured and dropped: every
// k-slice of a wavefront loaded before its first MFMA (+15 us per decode step).
template <int EPI, int NW>
__global__ __launch_bounds__(64 * NW) void gemm_skinny_kernel(GemmArgs p) {
  __shared__ f32x4 part[NW][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16;
  if (p.bump && blockIdx.x == 0 && threadIdx.x == 0) *p.bump += 1;
  const bool arow = r < p.M, brow = n0 + r < p.N;
  const bf16* ap = (const bf16*)p.A + (int64_t)(arow ? r : 0) * p.lda + g * 8;
  const bf16* bp = (const bf16*)p.B + (int64_t)(brow ? n0 + r : 0) * p.ldb + g * 8;
  SkinnyEpiIn<EPI> ein;
  if (w == 0) ein.load(p, n0 + r, g);
  f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
  const int nk = p.K / 32;
#pragma unroll 4
  for (int kt = w; kt < nk; kt += NW) {
    const bf16x8 af = arow ? *(const bf16x8*)(ap + kt * 32) : (bf16x8){};
    const bf16x8 bfr = brow ? *(const bf16x8*)(bp + kt * 32) : (bf16x8){};
    acc = Mfma<bf16>::mma(af, bfr, acc);
  }
  part[w][lane] = acc;
  __syncthreads();
  if (w == 0) {
    f32x4 t = part[0][lane];
#pragma unroll
    for (int q = 1; q < NW; q++) t += part[q][lane];
    ein.store(p, n0 + r, g, t);                       // lane holds rows 4g + i of column r
  }
}

// The same product with A = norm(x) computed by every workgroup from the M rows of x
// (fp32, K columns): NORM 1 is the LayerNorm (x - mean) / sqrt(var + 1e-5) * g + b,
// NORM 2 the weightless RMSNorm x / sqrt(mean(x^2) + 1e-5), each as the row kernels
// compute it, rounded to bf16. A wavefront's weight fragments are loaded before the
// normalization, so the weight stream is in flight while the rows are normalized into
// LDS (wavefront w takes row w); the k-loop then reads A from LDS. K <= 16 * 32 * SKN_S.
constexpr int SKN_S = 2;
constexpr int SKN_MAXK = 16 * 32 * SKN_S;
template <int EPI, int NORM>
__global__ __launch_bounds__(1024) void gemm_skinny_norm_kernel(GemmArgs p) {
  __shared__ f32x4 part[16][64];
  __shared__ __attribute__((aligned(16))) bf16 an[16 * (SKN_MAXK + 8)];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int K = p.K, ka = K + 8;                     // LDS row stride: 16 bytes of padding
  if (p.bump && blockIdx.x == 0 && threadIdx.x == 0) *p.bump += 1;
  const bool brow = n0 + r < p.N;
  const bf16* bp = (const bf16*)p.B + (int64_t)(brow ? n0 + r : 0) * p.ldb + g * 8;
  SkinnyEpiIn<EPI> ein;
  if (w == 0) ein.load(p, n0 + r, g);
  const int nk = K / 32;
  bf16x8 bfr[SKN_S];
#pragma unroll
  for (int i = 0; i < SKN_S; i++) {
    const int kt = w + 16 * i;
    bfr[i] = brow && kt < nk ? *(const bf16x8*)(bp + kt * 32) : (bf16x8){};
  }
  {
    bf16* arow = an + w * ka;
    const int K4 = K >> 2;
    if (w < p.M) {
      const f32x4* xr = (const f32x4*)(p.nx + (int64_t)w * K);
      f32x4 xv[SKN_MAXK / 256];
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < SKN_MAXK / 256; j++) {
        const int c4 = j * 64 + lane;
        xv[j] = c4 < K4 ? xr[c4] : (f32x4){0.f, 0.f, 0.f, 0.f};
        if constexpr (NORM == 1) s += (xv[j][0] + xv[j][1]) + (xv[j][2] + xv[j][3]);
        else s += (xv[j][0] * xv[j][0] + xv[j][1] * xv[j][1]) + (xv[j][2] * xv[j][2] + xv[j][3] * xv[j][3]);
      }
      float mu = 0.f, rs;
      if constexpr (NORM == 1) {
        mu = wave_sum(s) / K;
        float v = 0.f;
#pragma unroll
        for (int j = 0; j < SKN_MAXK / 256; j++)
          if (j * 64 + lane < K4)
#pragma unroll
            for (int e = 0; e < 4; e++) {
              const float t = xv[j][e] - mu;
              v += t * t;
            }
        rs = 1.0f / sqrtf(wave_sum(v) / K + 1e-5f);
      } else {
        rs = 1.0f / sqrtf(wave_sum(s) / K + 1e-5f);
      }
#pragma unroll
      for (int j = 0; j < SKN_MAXK / 256; j++) {
        const int c4 = j * 64 + lane;
        if (c4 >= K4) continue;
        bf16x4 ob;
        if constexpr (NORM == 1) {
          const f32x4 gv = ((const f32x4*)p.ng)[c4], bv = ((const f32x4*)p.nb)[c4];
#pragma unroll
          for (int e = 0; e < 4; e++) ob[e] = (bf16)((xv[j][e] - mu) * rs * gv[e] + bv[e]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; e++) ob[e] = (bf16)(xv[j][e] * rs);
        }
        *(bf16x4*)(arow + 4 * c4) = ob;
      }
    } else {                                          // rows past M: zeros
      for (int c4 = lane; c4 < K4; c4 += 64) *(bf16x4*)(arow + 4 * c4) = (bf16x4){};
    }
  }
  __syncthreads();
  f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < SKN_S; i++) {
    const int kt = w + 16 * i;
    if (kt < nk) acc = Mfma<bf16>::mma(*(const bf16x8*)(an + r * ka + kt * 32 + g * 8), bfr[i], acc);
  }
  part[w][lane] = acc;
  __syncthreads();
  if (w == 0) {
    f32x4 t = part[0][lane];
#pragma unroll
    for (int q = 1; q < 16; q++) t += part[q][lane];
    ein.store(p, n0 + r, g, t);
  }
}

__global__ void bump_kernel(int* c) {
  if (threadIdx.x == 0) *c += 1;
}

template <int NORM>
static hipError_t skinny_norm_epi(const GemmArgs& a, int epi, hipStream_t s) {
  const dim3 grid((a.N + 15) / 16);
  switch (epi) {
#define GPT_SKINNY_CASE(E) \
  case E: hipLaunchKernelGGL((gemm_skinny_norm_kernel<E, NORM>), grid, dim3(1024), 0, s, a); break;
    GPT_SKINNY_CASE(EPI_BIAS)
    GPT_SKINNY_CASE(EPI_BIAS_GELU)
    GPT_SKINNY_CASE(EPI_BIAS_RELU)
#undef GPT_SKINNY_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// GPT_SKINNY_NW4=0: every few-rows product on 16-wavefront workgroups (for comparisons).
static bool skinny_nw4() {
  static int on = -1;
  if (on < 0) {
    const char* e = std::getenv("GPT_SKINNY_NW4");
    on = (e && e[0] == '0') ? 0 : 1;
  }
  return on == 1;
}

static hipError_t skinny_epi(const GemmArgs& a, int epi, hipStream_t s) {
  const dim3 grid((a.N + 15) / 16);
  const bool nw4 = skinny_nw4() && (int)grid.x > 4 * num_cus();
  switch (epi) {
#define GPT_SKINNY_CASE(E)                                                                  \
  case E:                                                                                   \
    if (nw4) hipLaunchKernelGGL((gemm_skinny_kernel<E, 4>), grid, dim3(256), 0, s, a);     \
    else hipLaunchKernelGGL((gemm_skinny_kernel<E, 16>), grid, dim3(1024), 0, s, a);       \
    break;
    GPT_SKINNY_CASE(EPI_STORE)
    GPT_SKINNY_CASE(EPI_BIAS)
    GPT_SKINNY_CASE(EPI_BIAS_RESID)
    GPT_SKINNY_CASE(EPI_BIAS_GELU)
    GPT_SKINNY_CASE(EPI_BIAS_RELU)
    GPT_SKINNY_CASE(EPI_F32)
#undef GPT_SKINNY_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool wgrad_group_ok(int M, int N, int64_t lda, int64_t ldb, int64_t ldc) {
  return M >= 8 && N >= 8 && M % 8 == 0 && N % 8 == 0 && lda % 8 == 0 && ldb % 8 == 0 && ldc >= N;
}
int wgrad_group_tiles(int M, int N) { return ((M + 255) / 256) * ((N + 255) / 256); }
// two parked 256 x 256 partial tiles per workgroup, for up to 256 workgroups
size_t wgrad_group_ws_floats() { return (size_t)2 * 256 * 256 * 256; }

// GPT_GEMM_WIDE=0 selects the 16-wavefront grouped kernel (for comparisons).
static bool wgrad_wide() {
  static int on = -1;
  if (on < 0) {
    const char* e = std::getenv("GPT_GEMM_WIDE");
    on = (e && e[0] == '0') ? 0 : 1;
  }
  return on == 1;
}

hipError_t launch_wgrad_group(const WgradProblem* probs, int nprob, int total_tiles, int K, float beta, float* ws,
                              size_t ws_floats, hipStream_t s) {
  if (nprob <= 0 || total_tiles <= 0 || K <= 0) return hipSuccess;
  const int W = (int)std::min<size_t>(num_cus(), ws_floats / (2 * 256 * 256));   // one workgroup per CU
  if (K % 32 != 0 || W < 1) return hipErrorInvalidValue;
  const int dp = total_tiles / W * W, rem = total_tiles - dp;
  // 16 wavefronts of 64 x 64 per 256 x 256 tile: four per SIMD hide the transposing LDS
  // reads and the global->LDS waits better than eight of 128 x 64 (-6 % per launch)
  if (wgrad_wide())
    hipLaunchKernelGGL((gemm_group_wide_kernel<4>), dim3(W), dim3(256), 0, s, probs, nprob, total_tiles, dp, K, beta,
                       ws);
  else
    hipLaunchKernelGGL((gemm_group_kernel<256, 256, 4, 4, 4>), dim3(W), dim3(1024), 0, s, probs, nprob, total_tiles,
                       dp, K, beta, ws);
  if (rem > 0)
    hipLaunchKernelGGL((group_fixup_kernel<256, 256>), dim3(rem, 16), dim3(256), 0, s, probs, nprob, total_tiles, dp,
                       K, beta, (const float*)ws, W);
  return hipGetLastError();
}

// The pipelined kernels load 16-byte vectors straight into LDS with no edge
// handling along k: they need bf16, K a multiple of 32, aligned operands and, for
// m-contiguous operands, a row count that is a multiple of 8.
static bool pipelined_ok(const GemmDesc& d, bool bf16_operands) {
  auto vec_ok = [&](const void* ptr, int64_t ld) { return (ld % 8 == 0) && ((uintptr_t)ptr % 16 == 0); };
  return bf16_operands && d.M >= 256 && d.N >= 256 && d.K % 32 == 0 && vec_ok(d.A, d.lda) && vec_ok(d.B, d.ldb) &&
         (d.a_kc || d.M % 8 == 0) && (d.b_kc || d.N % 8 == 0);
}
// Both operands k-contiguous (every GEMM of the step except the weight
// gradients): 192 x 192 tiles on four wavefronts, three stages. For 12288-row
// outputs with 768, 2304 or 3072 columns these come in whole multiples of 256
// tiles, where 256 x 256 tiles leave part of the last wave of CUs idle.
static bool use_k192(const GemmDesc& d, bool bf16_operands) {
  return pipelined_ok(d, bf16_operands) && d.a_kc && d.b_kc && d.epi != EPI_ACC;
}

// Rows per tile of the launch use_k192 picks (K <= 4096, K a multiple of 64): 96 x 192
// tiles, two workgroups per CU, when one 192 x 192 tile per CU or fewer would cover the
// output, or when the 96-row tiles fill the last round of two workgroups per CU clearly
// better (the QKV projection: 768 tiles of 192 rows are 1.5 rounds, 1,536 of 96 rows are
// 3); else 192 x 192. Measured per launch at M 12,288, K 768: QKV (N 2,304) 55.0 -> 52.8 us
// on 96-row tiles; MLP up (N 3,072, two whole rounds either way) 88 -> 93 us and the
// lm_head (N 50,304) slower, so they keep 192 rows. The fused column sums write one
// partial row per tile row.
static int k192_tile_rows(const GemmDesc& d) {
  if (d.K % 64 != 0 || d.K > 4096) return 192;
  const int64_t t192 = (int64_t)((d.M + 191) / 192) * ((d.N + 191) / 192);
  if (t192 <= num_cus()) return 96;
  const int64_t t96 = (int64_t)((d.M + 95) / 96) * ((d.N + 191) / 192);
  const int64_t slots = 2 * (int64_t)num_cus();
  // last-round fill of each tiling, in 1/100
  const int64_t f192 = 100 * t192 / (((t192 + slots - 1) / slots) * slots);
  const int64_t f96 = 100 * t96 / (((t96 + slots - 1) / slots) * slots);
  return f96 >= f192 + 20 ? 96 : 192;
}

int gemm_colsum_rows(const GemmDesc& d, bool bf16_operands) {
  if ((d.epi != EPI_GELU_BWD && d.epi != EPI_RELU_BWD) || !use_k192(d, bf16_operands)) return 0;
  const int r = k192_tile_rows(d);
  return (d.M + r - 1) / r;
}

// The start delay (n x 2048 cycles) of the second workgroup per CU in the
// 192 x 192 two-workgroup kernels (launches of several rounds; the 96 x 192 launches
// take none). The first round's two workgroups of a CU otherwise finish
// their k-loops together and run their epilogues side by side; offset, one's
// epilogue overlaps the other's MFMAs. Measured on the GPT-2 step (whole-step
// A/B in one session): n = 4..10 took 0.3 ms off 72.3 ms, n >= 12 less. The
// workgroups dealt to the second slot are [num_cus, 2 num_cus): probed on gfx950,
// every CU of a 512-workgroup grid of two workgroups per CU held one from each
// half. GPT_GEMM_STAGGER=n overrides (for comparisons).
static int gemm_stagger() {
  static int n = -1;
  if (n < 0) {
    const char* e = std::getenv("GPT_GEMM_STAGGER");
    n = e ? std::max(0, std::min(64, std::atoi(e))) : 6;
  }
  return n;
}

// Each tile of a 192-wide launch walks its k-slices starting at its own position in
// the launch (tile i of T starts at slice i * nk / T and wraps around), so the tiles
// that share an operand panel do not all request the same rows at the same moment.
// Measured on the GPT-2 step (whole-step A/B, each pair in one session): 68.8 -> 67.1
// and 69.5 -> 68.2 ms, most of it in the lm_head forward and the 768-column residual
// GEMMs. The same rotation of the grouped weight-gradient tiles measured slower (68.6-68.9
// against 68.2 ms), so that launch keeps the plain order. The fp32 sums of a
// tile are taken in the rotated order (fixed per tile, so the result is deterministic).
// GPT_GEMM_KROT=0 restores the plain order (for comparisons).
static int gemm_krot() {
  static int on = -1;
  if (on < 0) {
    const char* e = std::getenv("GPT_GEMM_KROT");
    on = (e && e[0] == '0') ? 0 : 1;
  }
  return on;
}

// few rows, both operands k-contiguous, aligned 16-byte fragments
static bool skinny_ok(const GemmDesc& d, bool bf16_operands) {
  const int vw = bf16_operands ? 8 : 4;
  auto vec_ok = [&](const void* ptr, int64_t ld) { return (ld % vw == 0) && ((uintptr_t)ptr % 16 == 0); };
  return bf16_operands && d.M >= 1 && d.M <= 16 && d.a_kc && d.b_kc && d.K % 32 == 0 && d.K > 0 &&
         (d.norm || vec_ok(d.A, d.lda)) && vec_ok(d.B, d.ldb) &&
         (d.epi == EPI_STORE || d.epi == EPI_BIAS || d.epi == EPI_BIAS_RESID || d.epi == EPI_BIAS_GELU ||
          d.epi == EPI_BIAS_RELU || d.epi == EPI_F32);
}

bool gemm_norm_fusable(const GemmDesc& d, bool bf16_operands) {
  return (d.norm == 1 || d.norm == 2) && skinny_ok(d, bf16_operands) && d.K <= SKN_MAXK && d.K % 4 == 0 &&
         (d.epi == EPI_BIAS || d.epi == EPI_BIAS_GELU || d.epi == EPI_BIAS_RELU) && d.norm_x &&
         (uintptr_t)d.norm_x % 16 == 0 &&
         (d.norm == 2 || (d.norm_g && d.norm_b && ((uintptr_t)d.norm_g | (uintptr_t)d.norm_b) % 16 == 0));
}

hipError_t launch_gemm(const GemmDesc& d, bool bf16_operands, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0) {
    if (d.bump) hipLaunchKernelGGL(bump_kernel, dim3(1), dim3(64), 0, s, d.bump);
    return hipGetLastError();
  }
  if (d.colsum && gemm_colsum_rows(d, bf16_operands) == 0) return hipErrorInvalidValue;
  GemmArgs a;
  a.colsum = d.colsum;
  a.A = d.A; a.lda = d.lda; a.B = d.B; a.ldb = d.ldb; a.C = d.C; a.ldc = d.ldc;
  a.M = d.M; a.N = d.N; a.K = d.K; a.bias = d.bias; a.resid = d.resid; a.ldr = d.ldr;
  a.aux = d.aux; a.ldaux = d.ldaux; a.beta = d.beta;
  a.drop = d.drop; a.drop_site = d.drop_site;
  const int vw = bf16_operands ? 8 : 4;               // elements per 16-byte vector
  auto vec_ok = [&](const void* ptr, int64_t ld) { return (ld % vw == 0) && ((uintptr_t)ptr % 16 == 0); };
  a.a_vec = vec_ok(d.A, d.lda);
  a.b_vec = vec_ok(d.B, d.ldb);
  {
    // vector epilogue: 16-byte aligned rows for every matrix the epilogue touches
    bool cv = ((uintptr_t)d.C % 16 == 0) && (d.ldc % 8 == 0);
    if (d.resid) cv = cv && ((uintptr_t)d.resid % 16 == 0) && (d.ldr % 4 == 0);
    if (d.aux) cv = cv && ((uintptr_t)d.aux % 16 == 0) && (d.ldaux % 8 == 0);
    if (d.bias) cv = cv && ((uintptr_t)d.bias % 16 == 0);
    if (d.epi == EPI_ACC && d.split_ws) cv = cv && (d.N % 4 == 0) && ((uintptr_t)d.split_ws % 16 == 0);
    a.c_vec = cv;
  }
  if (d.norm) {
    if (!gemm_norm_fusable(d, bf16_operands)) return hipErrorInvalidValue;
    a.bump = d.bump;
    a.nx = d.norm_x; a.ng = d.norm_g; a.nb = d.norm_b;
    return d.norm == 1 ? skinny_norm_epi<1>(a, d.epi, s) : skinny_norm_epi<2>(a, d.epi, s);
  }
  // few rows, both operands k-contiguous, aligned 16-byte fragments
  if (skinny_ok(d, bf16_operands)) {
    a.bump = d.bump;
    return skinny_epi(a, d.epi, s);
  }
  if (d.bump) {
    GemmDesc e = d;
    e.bump = nullptr;
    const hipError_t r = launch_gemm(e, bf16_operands, s);
    if (r != hipSuccess) return r;
    hipLaunchKernelGGL(bump_kernel, dim3(1), dim3(64), 0, s, d.bump);
    return hipGetLastError();
  }
  const bool pipelined = pipelined_ok(d, bf16_operands);
  const int TBM = pipelined ? 256 : BM, TBN = pipelined ? 256 : BN;
  const int tiles = ((d.M + TBM - 1) / TBM) * ((d.N + TBN - 1) / TBN);
  const int BKt = bf16_operands ? GemmCfg<bf16>::BK : GemmCfg<float>::BK;
  a.kchunk = d.K > 0 ? d.K : 1;
  a.part = nullptr;
  // Split the contraction when the output has too few tiles to fill the chip
  // (weight gradients: small outputs, K = B*T); partials are reduced in order.
  int S = 1;
  if (d.epi == EPI_ACC && d.split_ws) {
    const int want = (512 + tiles - 1) / tiles;
    const int by_k = d.K / (4 * BKt);
    const int64_t mn = (int64_t)d.M * d.N;
    const int by_ws = (int)std::min<int64_t>(64, (int64_t)(d.split_ws_floats / (size_t)mn));
    S = std::max(1, std::min(want, std::min(by_k, by_ws)));
    if (S > 1) {
      const int kc = ((d.K + S - 1) / S + BKt - 1) / BKt * BKt;   // a multiple of 64 (bf16) or 16
      S = (d.K + kc - 1) / kc;
      a.kchunk = kc;
      a.part = d.split_ws;
    }
  }
  hipError_t e;
  // Stream-K over the whole chip for long contractions with too few output tiles
  // (weight gradients, K = B*T; the lm_head input gradient, K = vocab): every CU
  // gets the same number of k-slices. Measured on gfx950 it loses to one tile per
  // workgroup when K <= 3072, where parking partial tiles costs more than it saves.
  if (use_k192(d, bf16_operands)) {
    // 96 x 192 tiles where k192_tile_rows picks them (the step's N = 768 launches: the
    // out-projection and MLP down-projection forwards with their residual epilogue, the
    // fc, qkv and out-projection input gradients; and the QKV projection): two workgroups
    // of 4 wavefronts of 48 x 96 per CU over 64-wide k-slices (half the memory requests
    // per byte) in two stages of 36 KB. With one 192 x 192 tile per CU every tile
    // finished its k-loop at once and its stores stood alone; with two workgroups per CU
    // the two interleave (measured: 66.58 -> 66.18 ms per step, the residual launches
    // 6.55 -> 6.23 ms). These launches take no staggered start: their tiles are all
    // resident from the start (or nearly), so a delayed second workgroup only lengthens
    // the launch (delays of 0, 1, 2, 3, 4 and 6 units: 65.60-65.64, 65.66-65.68,
    // 65.70-65.75, 65.83-65.89, 65.96-65.99 and 66.32-66.34 ms per step). Otherwise one
    // 192 x 192 tile per CU or fewer (the lm_head input gradient, K = 50,304) runs 8
    // wavefronts of 96 x 48 over 64-wide slices, which hide more latency than 4 of
    // 96 x 96 when the CU holds no second workgroup; more tiles run 32-wide slices in
    // three stages, which leave room for two workgroups per CU.
    const int t192 = ((d.M + 191) / 192) * ((d.N + 191) / 192);
    a.krot = gemm_krot();
    if (k192_tile_rows(d) == 96) return dma_epi<96, 192, 2, 2, 2, true, true, 64>(a, d.epi, 1, s);
    if (t192 <= num_cus() && d.K % 64 == 0) return dma_epi<192, 192, 2, 4, 2, true, true, 64>(a, d.epi, 1, s);
    a.stagger_lo = num_cus();
    a.stagger_hi = 2 * num_cus();
    a.stagger_iters = gemm_stagger();
    return dma_epi<192, 192, 2, 2, 3, true, true>(a, d.epi, 1, s);
  }
  a.colsum = nullptr;
  if (pipelined && tiles < 2 * num_cus() && d.K >= 8192 && d.split_ws) {
    const long long KI = d.K / 32;
    const long long U = (long long)tiles * KI;
    const int W = (int)std::min<long long>(num_cus(), U);
    const long long per = U / W;
    const int maxseg = per > 0 ? (int)((KI + per - 1) / per + 1) : 1;
    const size_t need = (size_t)tiles * maxseg * 256 * 256;
    if (per >= 4 && need <= d.split_ws_floats) {
      a.kchunk = d.K;
      a.part = nullptr;
      return sk_layout<256, 256, 2, 4, 4>(d, a, W, d.split_ws, maxseg, s);
    }
  }
  if (pipelined) {
    e = dma_layout<256, 256, 2, 4, 4>(d, a, S, s);
  } else {
    dim3 grid((d.N + BN - 1) / BN, (d.M + BM - 1) / BM, S);
    e = bf16_operands ? dispatch_layout<bf16>(d, a, grid, s) : dispatch_layout<float>(d, a, grid, s);
  }
  if (e != hipSuccess || S == 1) return e;
  const int64_t total = (int64_t)d.M * d.N;
  const unsigned blocks = (unsigned)std::min<int64_t>((total + 255) / 256, 8192);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s, (const float*)d.split_ws, S, d.M, d.N,
                     (float*)d.C, d.ldc, d.beta);
  return hipGetLastError();
}

}  // namespace gpt
