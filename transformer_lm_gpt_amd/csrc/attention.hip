// Causal multi-head attention on MFMA for gfx950.
//
// What is computed ("Building microGPT from scratch", model-core section: QKV
// projection, scaled dot product, softmax, weighted V; head width n_embd/n_head
// as in the nanoGPT run log, section 2.2): for every (batch, head)
//   S = Q K^T / sqrt(hd),  S[i, j] = -inf for j > i,  P = softmax_rows(S),  O = P V,
// keeping lse_i = log sum_j exp(S[i, j]) for the backward, and its gradients
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  D_i = sum_c dO[i, c] O[i, c],
//   dQ = dS K / sqrt(hd),  dK = dS^T Q / sqrt(hd).
//
// Layout: qkv is [B*T, 3*d] with q | k | v and head h at columns h*hd; O and dO
// are [B*T, d]; lse and D are fp32 [B*H, T].
//
// Forward: one workgroup per (64-query tile, batch*head); its four wavefronts
// own 16 queries each and stream 64-key tiles of K and V through LDS with an
// online softmax (running max and sum per row, rescaling the O accumulator).
// Backward: the score tile is recomputed from Q, K and lse. dK and dV are
// accumulated per 64-key tile over the query tiles at or after it; dQ is
// accumulated per 64-query tile over the key tiles at or before it. Both run
// without atomics, so the result is deterministic.
#include "common.h"
#include "kernels.h"

namespace gpt {

// LDS tile of ROWS rows by a contraction dimension, stored [kdim/KG][ROWS+PADR][KG]
// so that one MFMA fragment is one contiguous read.
template <typename T, int ROWS, int PADR>
struct Tile {
  static constexpr int KG = Mfma<T>::KG;
  static constexpr int size(int kdim) { return (kdim / KG) * (ROWS + PADR) * KG; }
  __device__ static inline int idx(int kappa, int r) { return ((kappa / KG) * (ROWS + PADR) + r) * KG + (kappa % KG); }
  __device__ static inline typename Mfma<T>::frag frag(const T* t, int kk, int r) {
    const int g = kk * 4 + ((threadIdx.x & 63) >> 4);
    return *(const typename Mfma<T>::frag*)(t + (g * (ROWS + PADR) + r) * KG);
  }
};

template <typename T> struct AttnPad {
  static constexpr int big = Mfma<T>::KG == 8 ? 1 : 16;   // 64-row tiles
};

// Per-lane A-operand fragments of rows `row` (lane & 15 included) of a row-major
// [*, ld] source at column offset col0, zero beyond hd or past nrows.
template <typename T, int HDP>
__device__ inline void load_row_frags(typename Mfma<T>::frag (&f)[HDP / Mfma<T>::KPI], const T* src, int64_t ld,
                                      int row, int nrows, int col0, int hd) {
  constexpr int KG = Mfma<T>::KG;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int kk = 0; kk < HDP / Mfma<T>::KPI; kk++) {
    if constexpr (KG == 1) {
      const int c = kk * 4 + (lane >> 4);
      f[kk] = (row < nrows && c < hd) ? src[(int64_t)row * ld + col0 + c] : 0.f;
    } else {
#pragma unroll
      for (int e = 0; e < KG; e++) {
        const int c = (kk * 4 + (lane >> 4)) * KG + e;
        f[kk][e] = (row < nrows && c < hd) ? src[(int64_t)row * ld + col0 + c] : (T)0.0f;
      }
    }
  }
}

// ----------------------------------------------------------------------------- forward
template <typename T, int HDP>
__global__ __launch_bounds__(256) void attn_fwd_kernel(const T* __restrict__ qkv, T* __restrict__ o,
                                                       float* __restrict__ lse, int Tn, int H, int hd,
                                                       float scale) {
  constexpr int KPI = Mfma<T>::KPI;
  constexpr int PB = AttnPad<T>::big;
  typedef Tile<T, 64, PB> KT;     // contraction c, rows = keys
  typedef Tile<T, HDP, PB> VT;    // contraction key, rows = c
  typedef Tile<T, 16, 0> PT;      // contraction key, rows = 16 queries
  __shared__ __attribute__((aligned(16))) T Ks[KT::size(HDP)];
  __shared__ __attribute__((aligned(16))) T Vs[VT::size(64)];
  __shared__ __attribute__((aligned(16))) T Ps[4][PT::size(64)];

  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int q0 = blockIdx.x * 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int d = H * hd;
  const int64_t ld = 3 * (int64_t)d;
  const T* base = qkv + (int64_t)b * Tn * ld;

  typename Mfma<T>::frag qf[HDP / KPI];
  load_row_frags<T, HDP>(qf, base, ld, q0 + w * 16 + (lane & 15), Tn, h * hd, hd);

  f32x4 oacc[HDP / 16];
#pragma unroll
  for (int cb = 0; cb < HDP / 16; cb++) oacc[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float mrow[4], lrow[4];
#pragma unroll
  for (int e = 0; e < 4; e++) {
    mrow[e] = -INFINITY;
    lrow[e] = 0.f;
  }

  const int q_last = min(q0 + 63, Tn - 1);
  const int ntiles = q_last / 64 + 1;
  for (int kt = 0; kt < ntiles; kt++) {
    const int k0 = kt * 64;
    for (int i = threadIdx.x; i < 64 * HDP; i += 256) {
      const int key = i / HDP, c = i % HDP;
      const int gk = k0 + key;
      T kv = (T)0.0f, vv = (T)0.0f;
      if (gk < Tn && c < hd) {
        kv = base[(int64_t)gk * ld + d + h * hd + c];
        vv = base[(int64_t)gk * ld + 2 * d + h * hd + c];
      }
      Ks[KT::idx(c, key)] = kv;
      Vs[VT::idx(key, c)] = vv;
    }
    __syncthreads();

    f32x4 s[4];
#pragma unroll
    for (int nb = 0; nb < 4; nb++) {
      s[nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < HDP / KPI; kk++) s[nb] = Mfma<T>::mma(qf[kk], KT::frag(Ks, kk, nb * 16 + (lane & 15)), s[nb]);
    }
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const int qi = q0 + w * 16 + (lane >> 4) * 4 + e;
      float mx = -INFINITY;
#pragma unroll
      for (int nb = 0; nb < 4; nb++) {
        const int kj = k0 + nb * 16 + (lane & 15);
        const float v = (kj <= qi && kj < Tn) ? s[nb][e] * scale : -INFINITY;
        s[nb][e] = v;
        mx = fmaxf(mx, v);
      }
      mx = row16_max(mx);
      const float mnew = fmaxf(mrow[e], mx);
      const float alpha = (mrow[e] == -INFINITY) ? 0.f : __expf(mrow[e] - mnew);
      float rs = 0.f;
#pragma unroll
      for (int nb = 0; nb < 4; nb++) {
        const float p = (s[nb][e] == -INFINITY) ? 0.f : __expf(s[nb][e] - mnew);
        rs += p;
        Ps[w][PT::idx(nb * 16 + (lane & 15), (lane >> 4) * 4 + e)] = from_f32<T>(p);
      }
      rs = row16_sum(rs);
      lrow[e] = lrow[e] * alpha + rs;
      mrow[e] = mnew;
#pragma unroll
      for (int cb = 0; cb < HDP / 16; cb++) oacc[cb][e] *= alpha;
    }
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < HDP / 16; cb++) {
#pragma unroll
      for (int kk = 0; kk < 64 / KPI; kk++)
        oacc[cb] = Mfma<T>::mma(PT::frag(Ps[w], kk, lane & 15), VT::frag(Vs, kk, cb * 16 + (lane & 15)), oacc[cb]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int e = 0; e < 4; e++) {
    const int qi = q0 + w * 16 + (lane >> 4) * 4 + e;
    if (qi >= Tn) continue;
    const float inv = 1.f / lrow[e];
#pragma unroll
    for (int cb = 0; cb < HDP / 16; cb++) {
      const int c = cb * 16 + (lane & 15);
      if (c < hd) o[((int64_t)b * Tn + qi) * d + h * hd + c] = from_f32<T>(oacc[cb][e] * inv);
    }
    if ((lane & 15) == 0) lse[(int64_t)bh * Tn + qi] = mrow[e] + logf(lrow[e]);
  }
}

// ----------------------------------------------------------------------------- backward
// D[b*H + h, t] = sum_c dO[b, t, h, c] O[b, t, h, c]; one thread per (b, t, h), heads
// fastest so that a wavefront reads whole rows; 16-byte loads when hd allows.
template <typename T>
__global__ void attn_bwd_D_kernel(const T* __restrict__ o, const T* __restrict__ dout, float* __restrict__ D,
                                  int B, int Tn, int H, int hd) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;   // over B*T*H, h fastest
  if (i >= B * H * Tn) return;
  const int h = i % H, bt = i / H, t = bt % Tn, b = bt / Tn;
  const int64_t off = (int64_t)bt * H * hd + h * hd;
  constexpr int VW = 16 / sizeof(T);
  float s = 0.f;
  if (hd % VW == 0) {
    typedef T vec __attribute__((ext_vector_type(VW)));
    for (int c = 0; c < hd; c += VW) {
      const vec a = *(const vec*)(dout + off + c);
      const vec bv = *(const vec*)(o + off + c);
#pragma unroll
      for (int e = 0; e < VW; e++) s += to_f32(a[e]) * to_f32(bv[e]);
    }
  } else {
    for (int c = 0; c < hd; c++) s += to_f32(dout[off + c]) * to_f32(o[off + c]);
  }
  D[((int64_t)b * H + h) * Tn + t] = s;
}

template <typename T, int HDP>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(const T* __restrict__ qkv, const T* __restrict__ dout,
                                                            const float* __restrict__ lse,
                                                            const float* __restrict__ Dv, T* __restrict__ dqkv,
                                                            int Tn, int H, int hd, float scale) {
  constexpr int KPI = Mfma<T>::KPI;
  constexpr int PB = AttnPad<T>::big;
  typedef Tile<T, 64, PB> NT;     // contraction c, rows = queries
  typedef Tile<T, HDP, PB> TT;    // contraction query, rows = c
  typedef Tile<T, 16, 0> WT;      // contraction query, rows = 16 keys of a wave
  __shared__ __attribute__((aligned(16))) T Qs1[NT::size(HDP)];
  __shared__ __attribute__((aligned(16))) T dOs1[NT::size(HDP)];
  __shared__ __attribute__((aligned(16))) T Qs2[TT::size(64)];
  __shared__ __attribute__((aligned(16))) T dOs2[TT::size(64)];
  __shared__ __attribute__((aligned(16))) T PTs[4][WT::size(64)];
  __shared__ __attribute__((aligned(16))) T dSTs[4][WT::size(64)];
  __shared__ float ls[64], Ds[64];

  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int k0 = blockIdx.x * 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int d = H * hd;
  const int64_t ld = 3 * (int64_t)d;
  const T* base = qkv + (int64_t)b * Tn * ld;
  const T* dob = dout + (int64_t)b * Tn * d;

  typename Mfma<T>::frag kf[HDP / KPI], vf[HDP / KPI];
  const int krow = k0 + w * 16 + (lane & 15);
  load_row_frags<T, HDP>(kf, base, ld, krow, Tn, d + h * hd, hd);
  load_row_frags<T, HDP>(vf, base, ld, krow, Tn, 2 * d + h * hd, hd);

  f32x4 dk[HDP / 16], dv[HDP / 16];
#pragma unroll
  for (int cb = 0; cb < HDP / 16; cb++) {
    dk[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    dv[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  const int nqt = (Tn + 63) / 64;
  for (int qt = blockIdx.x; qt < nqt; qt++) {
    const int q0 = qt * 64;
    for (int i = threadIdx.x; i < 64 * HDP; i += 256) {
      const int r = i / HDP, c = i % HDP;
      const int gq = q0 + r;
      T qv = (T)0.0f, dov = (T)0.0f;
      if (gq < Tn && c < hd) {
        qv = base[(int64_t)gq * ld + h * hd + c];
        dov = dob[(int64_t)gq * d + h * hd + c];
      }
      Qs1[NT::idx(c, r)] = qv;
      dOs1[NT::idx(c, r)] = dov;
      Qs2[TT::idx(r, c)] = qv;
      dOs2[TT::idx(r, c)] = dov;
    }
    if (threadIdx.x < 64) {
      const int gq = q0 + threadIdx.x;
      ls[threadIdx.x] = gq < Tn ? lse[(int64_t)bh * Tn + gq] : 0.f;
      Ds[threadIdx.x] = gq < Tn ? Dv[(int64_t)bh * Tn + gq] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < 4; nb++) {
      f32x4 st = (f32x4){0.f, 0.f, 0.f, 0.f}, dpt = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < HDP / KPI; kk++) {
        st = Mfma<T>::mma(kf[kk], NT::frag(Qs1, kk, nb * 16 + (lane & 15)), st);
        dpt = Mfma<T>::mma(vf[kk], NT::frag(dOs1, kk, nb * 16 + (lane & 15)), dpt);
      }
      const int ql = nb * 16 + (lane & 15);
      const int q = q0 + ql;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int key = k0 + w * 16 + (lane >> 4) * 4 + e;
        const float p = (key <= q && q < Tn) ? __expf(st[e] * scale - ls[ql]) : 0.f;
        const float ds = p * (dpt[e] - Ds[ql]);
        PTs[w][WT::idx(ql, (lane >> 4) * 4 + e)] = from_f32<T>(p);
        dSTs[w][WT::idx(ql, (lane >> 4) * 4 + e)] = from_f32<T>(ds);
      }
    }
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < HDP / 16; cb++) {
#pragma unroll
      for (int kk = 0; kk < 64 / KPI; kk++) {
        dv[cb] = Mfma<T>::mma(WT::frag(PTs[w], kk, lane & 15), TT::frag(dOs2, kk, cb * 16 + (lane & 15)), dv[cb]);
        dk[cb] = Mfma<T>::mma(WT::frag(dSTs[w], kk, lane & 15), TT::frag(Qs2, kk, cb * 16 + (lane & 15)), dk[cb]);
      }
    }
    __syncthreads();
  }

  T* db = dqkv + (int64_t)b * Tn * ld;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const int key = k0 + w * 16 + (lane >> 4) * 4 + e;
    if (key >= Tn) continue;
#pragma unroll
    for (int cb = 0; cb < HDP / 16; cb++) {
      const int c = cb * 16 + (lane & 15);
      if (c < hd) {
        db[(int64_t)key * ld + d + h * hd + c] = from_f32<T>(dk[cb][e] * scale);
        db[(int64_t)key * ld + 2 * d + h * hd + c] = from_f32<T>(dv[cb][e]);
      }
    }
  }
}

template <typename T, int HDP>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(const T* __restrict__ qkv, const T* __restrict__ dout,
                                                          const float* __restrict__ lse,
                                                          const float* __restrict__ Dv, T* __restrict__ dqkv,
                                                          int Tn, int H, int hd, float scale) {
  constexpr int KPI = Mfma<T>::KPI;
  constexpr int PB = AttnPad<T>::big;
  typedef Tile<T, 64, PB> NT;     // contraction c, rows = keys
  typedef Tile<T, HDP, PB> TT;    // contraction key, rows = c
  typedef Tile<T, 16, 0> WT;      // contraction key, rows = 16 queries of a wave
  __shared__ __attribute__((aligned(16))) T Ks1[NT::size(HDP)];
  __shared__ __attribute__((aligned(16))) T Vs1[NT::size(HDP)];
  __shared__ __attribute__((aligned(16))) T Ks2[TT::size(64)];
  __shared__ __attribute__((aligned(16))) T dSs[4][WT::size(64)];

  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int q0 = blockIdx.x * 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int d = H * hd;
  const int64_t ld = 3 * (int64_t)d;
  const T* base = qkv + (int64_t)b * Tn * ld;
  const T* dob = dout + (int64_t)b * Tn * d;

  typename Mfma<T>::frag qf[HDP / KPI], dof[HDP / KPI];
  const int qrow = q0 + w * 16 + (lane & 15);
  load_row_frags<T, HDP>(qf, base, ld, qrow, Tn, h * hd, hd);
  load_row_frags<T, HDP>(dof, dob, d, qrow, Tn, h * hd, hd);
  float lsr[4], Dr[4];
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const int qi = q0 + w * 16 + (lane >> 4) * 4 + e;
    lsr[e] = qi < Tn ? lse[(int64_t)bh * Tn + qi] : 0.f;
    Dr[e] = qi < Tn ? Dv[(int64_t)bh * Tn + qi] : 0.f;
  }
  f32x4 dq[HDP / 16];
#pragma unroll
  for (int cb = 0; cb < HDP / 16; cb++) dq[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int q_last = min(q0 + 63, Tn - 1);
  const int ntiles = q_last / 64 + 1;
  for (int kt = 0; kt < ntiles; kt++) {
    const int k0 = kt * 64;
    for (int i = threadIdx.x; i < 64 * HDP; i += 256) {
      const int r = i / HDP, c = i % HDP;
      const int gk = k0 + r;
      T kv = (T)0.0f, vv = (T)0.0f;
      if (gk < Tn && c < hd) {
        kv = base[(int64_t)gk * ld + d + h * hd + c];
        vv = base[(int64_t)gk * ld + 2 * d + h * hd + c];
      }
      Ks1[NT::idx(c, r)] = kv;
      Vs1[NT::idx(c, r)] = vv;
      Ks2[TT::idx(r, c)] = kv;
    }
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < 4; nb++) {
      f32x4 s = (f32x4){0.f, 0.f, 0.f, 0.f}, dp = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < HDP / KPI; kk++) {
        s = Mfma<T>::mma(qf[kk], NT::frag(Ks1, kk, nb * 16 + (lane & 15)), s);
        dp = Mfma<T>::mma(dof[kk], NT::frag(Vs1, kk, nb * 16 + (lane & 15)), dp);
      }
      const int kl = nb * 16 + (lane & 15);
      const int key = k0 + kl;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int qi = q0 + w * 16 + (lane >> 4) * 4 + e;
        const float p = (key <= qi && key < Tn && qi < Tn) ? __expf(s[e] * scale - lsr[e]) : 0.f;
        dSs[w][WT::idx(kl, (lane >> 4) * 4 + e)] = from_f32<T>(p * (dp[e] - Dr[e]));
      }
    }
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < HDP / 16; cb++) {
#pragma unroll
      for (int kk = 0; kk < 64 / KPI; kk++)
        dq[cb] = Mfma<T>::mma(WT::frag(dSs[w], kk, lane & 15), TT::frag(Ks2, kk, cb * 16 + (lane & 15)), dq[cb]);
    }
    __syncthreads();
  }

  T* db = dqkv + (int64_t)b * Tn * ld;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const int qi = q0 + w * 16 + (lane >> 4) * 4 + e;
    if (qi >= Tn) continue;
#pragma unroll
    for (int cb = 0; cb < HDP / 16; cb++) {
      const int c = cb * 16 + (lane & 15);
      if (c < hd) db[(int64_t)qi * ld + h * hd + c] = from_f32<T>(dq[cb][e] * scale);
    }
  }
}

// ----------------------------------------------------------------------------- launchers
template <typename T, int HDP>
static hipError_t fwd_t(const void* qkv, void* o, float* lse, int B, int Tn, int H, int hd, hipStream_t s) {
  dim3 grid((Tn + 63) / 64, B * H);
  const float scale = 1.0f / sqrtf((float)hd);
  hipLaunchKernelGGL((attn_fwd_kernel<T, HDP>), grid, dim3(256), 0, s, (const T*)qkv, (T*)o, lse, Tn, H, hd, scale);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const void* qkv, void* o, float* lse, bool bf16_ops, int B, int T, int H, int hd,
                           hipStream_t s) {
  if (hd <= 0 || hd > 64) return hipErrorInvalidValue;
  if (bf16_ops) return hd <= 32 ? fwd_t<bf16, 32>(qkv, o, lse, B, T, H, hd, s) : fwd_t<bf16, 64>(qkv, o, lse, B, T, H, hd, s);
  return hd <= 32 ? fwd_t<float, 32>(qkv, o, lse, B, T, H, hd, s) : fwd_t<float, 64>(qkv, o, lse, B, T, H, hd, s);
}

template <typename T, int HDP>
static hipError_t bwd_t(const void* qkv, const void* o, const void* dout, const float* lse, float* D, void* dqkv,
                        int B, int Tn, int H, int hd, hipStream_t s) {
  const float scale = 1.0f / sqrtf((float)hd);
  const int n = B * H * Tn;
  hipLaunchKernelGGL(attn_bwd_D_kernel<T>, dim3((n + 255) / 256), dim3(256), 0, s, (const T*)o, (const T*)dout, D,
                     B, Tn, H, hd);
  dim3 grid((Tn + 63) / 64, B * H);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, HDP>), grid, dim3(256), 0, s, (const T*)qkv, (const T*)dout, lse,
                     (const float*)D, (T*)dqkv, Tn, H, hd, scale);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, HDP>), grid, dim3(256), 0, s, (const T*)qkv, (const T*)dout, lse,
                     (const float*)D, (T*)dqkv, Tn, H, hd, scale);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const void* qkv, const void* o, const void* dout, const float* lse, float* D,
                           void* dqkv, bool bf16_ops, int B, int T, int H, int hd, hipStream_t s) {
  if (hd <= 0 || hd > 64) return hipErrorInvalidValue;
  if (bf16_ops)
    return hd <= 32 ? bwd_t<bf16, 32>(qkv, o, dout, lse, D, dqkv, B, T, H, hd, s)
                    : bwd_t<bf16, 64>(qkv, o, dout, lse, D, dqkv, B, T, H, hd, s);
  return hd <= 32 ? bwd_t<float, 32>(qkv, o, dout, lse, D, dqkv, B, T, H, hd, s)
                  : bwd_t<float, 64>(qkv, o, dout, lse, D, dqkv, B, T, H, hd, s);
}

}  // namespace gpt
