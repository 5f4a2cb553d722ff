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
// Forward: one workgroup per (query tile, batch*head); its four wavefronts own
// 16 queries each (fp32: 64-query tiles) or 32 each (bf16: 128-query tiles) and
// stream 64-key tiles of K and V through LDS with an online softmax (running max
// and sum per row, rescaling the O accumulator).
// Backward: the score tile is recomputed from Q, K and lse. dK and dV are
// accumulated per 64-key tile over the query tiles at or after it; dQ is
// accumulated per 64-query tile over the key tiles at or before it. Both run
// without atomics, so the result is deterministic.
//
// Dropout on the probabilities (nanoGPT run log, sections 2.1 and 2.2), in the
// DROP instantiations: with Z the mask times 1/(1-p), O = (P o Z) V, and the
// backward takes dV = (P o Z)^T dO, dS = P o (Z o dP - D); D = rowsum(dO o O) still
// equals sum_j P_ij Z_ij dP_ij. The softmax statistics (m, l, lse) are those of
// the undropped P. Z is recomputed from the counter-based generator, never stored.
#include "common.h"
#include "kernels.h"

namespace gpt {

typedef short s16x4 __attribute__((ext_vector_type(4)));

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
template <typename T, int HDP, bool DROP>
__global__ __launch_bounds__(256) void attn_fwd_kernel(const T* __restrict__ qkv, T* __restrict__ o,
                                                       float* __restrict__ lse, int Tn, int H, int hd,
                                                       float scale, DropArgs da, uint32_t site) {
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
        float p = (s[nb][e] == -INFINITY) ? 0.f : __expf(s[nb][e] - mnew);
        rs += p;
        if constexpr (DROP) p *= drop_mult1(da, site, (uint32_t)(bh * Tn + qi), k0 + nb * 16 + (lane & 15));
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

template <typename T, int HDP, bool DROP>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(const T* __restrict__ qkv, const T* __restrict__ dout,
                                                            const float* __restrict__ lse,
                                                            const float* __restrict__ Dv, T* __restrict__ dqkv,
                                                            int Tn, int H, int hd, float scale, DropArgs da,
                                                            uint32_t site) {
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
        const float mk = DROP ? drop_mult1(da, site, (uint32_t)(bh * Tn + q), key) : 1.f;
        const float ds = p * (dpt[e] * mk - Ds[ql]);
        PTs[w][WT::idx(ql, (lane >> 4) * 4 + e)] = from_f32<T>(DROP ? p * mk : p);
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

template <typename T, int HDP, bool DROP>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(const T* __restrict__ qkv, const T* __restrict__ dout,
                                                          const float* __restrict__ lse,
                                                          const float* __restrict__ Dv, T* __restrict__ dqkv,
                                                          int Tn, int H, int hd, float scale, DropArgs da,
                                                          uint32_t site) {
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
        const float mk = DROP ? drop_mult1(da, site, (uint32_t)(bh * Tn + qi), key) : 1.f;
        dSs[w][WT::idx(kl, (lane >> 4) * 4 + e)] = from_f32<T>(p * (dp[e] * mk - Dr[e]));
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

// ----------------------------------------------------------------------------- bf16, register-resident P
// Transposed formulation for bf16 with head_dim HDP in {32, 64}. A wavefront owns
// 16 columns (queries, or keys in the dK/dV kernel); a 64-row tile of the other
// side streams through LDS. Scores are produced as S^T = K Q^T, so the MFMA
// output layout puts four keys of one query in each lane. Two such 16-key
// blocks are exactly the B operand of the next MFMA (Vt P^T, K^T dS^T, ...) when
// the A operand reads its keys in the same order, which the 16-lane transposing
// LDS read gives. So P and dS never leave registers, the row statistics need two
// cross-lane steps, and the output rescale needs none.
//
// LDS tiles are [64 rows][HDP] bf16 with 16-byte units XOR-swizzled by row. For
// head_dim 64 the XOR is r & 7: measured on gfx950 it keeps the 16-row fragment
// reads at the rate of the (r >> 1) & 7 swizzle and lifts the transposing reads
// from about 109 to 132 bytes per clock per CU.
template <int HDP>
struct ATile {
  static constexpr int UR = HDP / 8;                  // 16-byte units per row
  __device__ static inline int swz(int r) { return UR == 8 ? (r & 7) : ((r >> 1) & 3); }
  __device__ static inline int unit(int r, int u) { return r * UR + (u ^ swz(r)); }
  // 8 consecutive columns u*8.. of row r (an A or B fragment along the row)
  __device__ static inline bf16x8 row_frag(const bf16* t, int r, int u) {
    return *(const bf16x8*)(t + unit(r, u) * 8);
  }
  // 16-lane transposed read: lane j of each group gets rows k0..k0+3 of column c0 + j
  __device__ static inline s16x4 tr(const bf16* t, int k0, int c0) {
    const int q = threadIdx.x & 15;
    const int r = k0 + (q >> 2), c = c0 + 4 * (q & 3);
    const bf16* a = t + unit(r, c >> 3) * 8 + (c & 4);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(a));
  }
};

__device__ inline bf16x8 cat4(s16x4 lo, s16x4 hi) {
  s16x4 h[2] = {lo, hi};
  bf16x8 f;
  __builtin_memcpy(&f, h, 16);
  return f;
}
__device__ inline bf16x8 pack_p(const f32x4& lo, const f32x4& hi) {
  bf16x8 f;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    f[i] = (bf16)lo[i];
    f[4 + i] = (bf16)hi[i];
  }
  return f;
}

// Buffer resource over `bytes` bytes from `base`: loads at or past the end read as
// zero, so rows past the sequence need no branch.
__device__ inline __amdgpu_buffer_rsrc_t range_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// A 64-row tile (rows row0.., columns col0..col0+HDP of a row-major [rows, ld]
// bf16 source) staged through registers: each thread holds HDP/32 16-byte units.
template <int HDP>
struct TileRegs {
  static constexpr int NU = 64 * HDP / 8 / 256;
  bf16x8 v[NU];
  __device__ inline void load(__amdgpu_buffer_rsrc_t src, int ld, int row0, int col0) {
#pragma unroll
    for (int j = 0; j < NU; j++) {
      const int idx = threadIdx.x + 256 * j;
      const int r = idx / (HDP / 8), u = idx % (HDP / 8);
      const int off = ((row0 + r) * ld + col0 + u * 8) * 2;
      v[j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(src, off, 0, 0));
    }
  }
  __device__ inline void store(bf16* t) const {
#pragma unroll
    for (int j = 0; j < NU; j++) {
      const int idx = threadIdx.x + 256 * j;
      const int r = idx / (HDP / 8), u = idx % (HDP / 8);
      *(bf16x8*)(t + ATile<HDP>::unit(r, u) * 8) = v[j];
    }
  }
};

constexpr float LOG2E_F = 1.4426950408889634f;
constexpr float RESCALE_LAG = 8.f;   // log2 units: the forward's running max may lag by up to 2^8
constexpr float LN2_F = 0.6931471805599453f;

// Reductions over the four lanes l, l^16, l^32, l^48 that hold one column's four
// 4-row groups of an MFMA output block. Every lane gets the same bits.
__device__ inline float group_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float group_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Inclusive prefix sum along each 16-lane row with DPP row shifts (a lane whose
// source is outside its row adds 0): lane 15 of every row ends with the row total.
__device__ inline float row16_total(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, false));   // row_shr:1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, false));   // row_shr:2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false));   // row_shr:4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, false));   // row_shr:8
  return v;
}

// Column sums of a wave's CB x 4 accumulator values (hd column cb*16 + 4g + i, one
// query or key per lane & 15) over its 16 rows and then over the four waves in a
// fixed order, into dst[c] for c < HDP (bias gradient partials).
template <int HDP>
__device__ inline void block_colsum(const f32x4 (&acc)[HDP / 16], float mul, float* red, float* dst) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4;
#pragma unroll
  for (int cb = 0; cb < HDP / 16; cb++)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float t = row16_total(acc[cb][i] * mul);
      if ((lane & 15) == 15) red[w * HDP + cb * 16 + 4 * g + i] = t;
    }
  __syncthreads();
  if (threadIdx.x < HDP) {
    float t = red[threadIdx.x];
#pragma unroll
    for (int q = 1; q < 4; q++) t += red[q * HDP + threadIdx.x];
    dst[threadIdx.x] = t;
  }
}

// The forward with 128 queries per workgroup, 32 per wavefront. Each K fragment and
// each transposed V fragment read from LDS feeds the MFMAs of two 16-query halves
// (register blocking on the query side), which halves the LDS read bytes per score
// (with 16 queries per wavefront every 16 queries read the whole 64 x hd K and V
// tiles). Wavefront w owns queries 128 QB + 32 w + 16 hh + (lane & 15), which lie in
// the 64-query block sb = 2 QB + w/2: key tiles before sb are fully visible, tile sb
// is the diagonal one, later tiles are skipped (the wavefront only helps stage them).
// Per query the arithmetic, and its order, is that of 16 queries per wavefront.
// The exponentials run in base 2 with the 1/sqrt(hd) scale folded in: with
// c = log2(e)/sqrt(hd), exp(S*scale - x) = exp2(S*c - x*log2(e)), one FMA and one
// v_exp per score. Only the diagonal tile of a causal block needs the mask.
// Without dropout only (DROP = false; da and site are unused): the dropout forward is
// attn_fwd_v2 below.
template <int HDP, bool DROP>
__global__ __launch_bounds__(256) void attn_fwd_v3(const bf16* __restrict__ qkv, bf16* __restrict__ o,
                                                   float* __restrict__ lse, int Tn, int H, float scale, DropArgs da,
                                                   uint32_t site) {
  static_assert(!DROP, "the dropout forward is attn_fwd_v2");
  typedef ATile<HDP> AT;
  constexpr int KK = HDP / 32, CB = HDP / 16;
  __shared__ __attribute__((aligned(16))) bf16 Ks[64 * HDP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[64 * HDP];
  const int nkt = (Tn + 63) / 64;
  const int nQB = (Tn + 127) / 128;
  const int QB = nQB - 1 - blockIdx.y;                // longest first
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4;
  const int d = H * HDP;
  const int64_t ld = 3 * (int64_t)d;
  const bf16* base = qkv + (int64_t)b * Tn * ld;
  const int sb = 2 * QB + (w >> 1);                   // this wavefront's 64-query block
  const int q0w = QB * 128 + w * 32;                  // its first query
  const bool active = q0w < Tn;                       // wave-uniform: some query is in range
  int q[2];
  q[0] = q0w + (lane & 15);
  q[1] = q[0] + 16;
  const float c = scale * LOG2E_F;
  bf16x8 qf[2][KK];
#pragma unroll
  for (int hh = 0; hh < 2; hh++)
#pragma unroll
    for (int kk = 0; kk < KK; kk++)
      qf[hh][kk] = q[hh] < Tn ? *(const bf16x8*)(base + (int64_t)q[hh] * ld + h * HDP + kk * 32 + g * 8)
                              : (bf16x8){};
  f32x4 ot[2][CB];
  // running sums of the bf16-rounded P, from one MFMA of a ones fragment against
  // each P fragment (every entry of the output block holds its query's sum)
  f32x4 lt[2];
  float m[2];
#pragma unroll
  for (int hh = 0; hh < 2; hh++) {
#pragma unroll
    for (int cb = 0; cb < CB; cb++) ot[hh][cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    lt[hh] = (f32x4){0.f, 0.f, 0.f, 0.f};
    m[hh] = -INFINITY;
  }
  const bf16x8 ones = (bf16x8){(bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f,
                               (bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f};
  const int last = min(2 * QB + 1, nkt - 1);          // the block's last key tile

  const auto src = range_rsrc(base, (int64_t)Tn * ld * 2);
  TileRegs<HDP> kr, vr;
  kr.load(src, (int)ld, 0, d + h * HDP);
  vr.load(src, (int)ld, 0, 2 * d + h * HDP);
  for (int kt = 0; kt <= last; kt++) {
    __syncthreads();
    kr.store(Ks);
    vr.store(Vs);
    __syncthreads();
    if (kt < last) {
      kr.load(src, (int)ld, (kt + 1) * 64, d + h * HDP);
      vr.load(src, (int)ld, (kt + 1) * 64, 2 * d + h * HDP);
    }
    if (!active || kt > sb) continue;                 // wave-uniform
    f32x4 st[2][4];
#pragma unroll
    for (int nb = 0; nb < 4; nb++) {
      st[0][nb] = st[1][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; kk++) {
        const bf16x8 kf = AT::row_frag(Ks, nb * 16 + (lane & 15), kk * 4 + g);
        st[0][nb] = Mfma<bf16>::mma(kf, qf[0][kk], st[0][nb]);
        st[1][nb] = Mfma<bf16>::mma(kf, qf[1][kk], st[1][nb]);
      }
    }
    if (kt == sb) {                                   // keys after the query, or past Tn
#pragma unroll
      for (int hh = 0; hh < 2; hh++) {
        const int lim = q[hh] - kt * 64;
#pragma unroll
        for (int nb = 0; nb < 4; nb++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int kl = nb * 16 + 4 * g + i;
            if (kl > lim || kt * 64 + kl >= Tn) st[hh][nb][i] = -INFINITY;
          }
      }
    }
#pragma unroll
    for (int hh = 0; hh < 2; hh++) {
      float mx = st[hh][0][0];
#pragma unroll
      for (int nb = 0; nb < 4; nb++)
#pragma unroll
        for (int i = 0; i < 4; i++) mx = fmaxf(mx, st[hh][nb][i]);
      // the running max moves only when a row's max grows by more than 2^RESCALE_LAG
      // (and on the first tile): until then P = exp2(S c - m) stays below 2^8, which bf16
      // and the fp32 sums hold at full relative precision, and the sums and the output
      // carry the same stale m, so the result is the same; most tiles skip the rescale
      const float mt = group_max(mx) * c;            // finite: key 0 is always visible
      if (__any(mt > m[hh] + RESCALE_LAG)) {
        const float mnew = fmaxf(m[hh], mt);
        const float alpha = __builtin_amdgcn_exp2f(m[hh] - mnew);
        lt[hh] *= alpha;
#pragma unroll
        for (int cb = 0; cb < CB; cb++) ot[hh][cb] *= alpha;
        m[hh] = mnew;
      }
#pragma unroll
      for (int nb = 0; nb < 4; nb++)
#pragma unroll
        for (int i = 0; i < 4; i++) st[hh][nb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[hh][nb][i], c, -m[hh]));
    }
#pragma unroll
    for (int kp = 0; kp < 2; kp++) {
      bf16x8 pf[2];
#pragma unroll
      for (int hh = 0; hh < 2; hh++) {
        pf[hh] = pack_p(st[hh][2 * kp], st[hh][2 * kp + 1]);
        lt[hh] = Mfma<bf16>::mma(ones, pf[hh], lt[hh]);
      }
#pragma unroll
      for (int cb = 0; cb < CB; cb++) {
        const bf16x8 vf = cat4(AT::tr(Vs, 32 * kp + 4 * g, cb * 16), AT::tr(Vs, 32 * kp + 16 + 4 * g, cb * 16));
        ot[0][cb] = Mfma<bf16>::mma(vf, pf[0], ot[0][cb]);
        ot[1][cb] = Mfma<bf16>::mma(vf, pf[1], ot[1][cb]);
      }
    }
  }
#pragma unroll
  for (int hh = 0; hh < 2; hh++) {
    if (q[hh] < Tn) {
      const float l = lt[hh][0];
      const float inv = 1.f / l;
      bf16* orow = o + ((int64_t)b * Tn + q[hh]) * d + h * HDP;
#pragma unroll
      for (int cb = 0; cb < CB; cb++) {
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; i++) v[i] = (bf16)(ot[hh][cb][i] * inv);
        *(bf16x4*)(orow + cb * 16 + 4 * g) = v;
      }
      if (g == 0) lse[(int64_t)bh * Tn + q[hh]] = (m[hh] + log2f(l)) * LN2_F;
    }
  }
}

// The dropout forward: 64-query workgroups, 16 queries per wavefront. With the
// generator's state, 32 queries per wavefront (attn_fwd_v3) would leave two
// wavefronts per SIMD instead of four. Per query the arithmetic, and its order, is
// that of attn_fwd_v3, so a rate that keeps every element reproduces the undropped
// result bit for bit. DROP = true only.
template <int HDP, bool DROP>
__global__ __launch_bounds__(256) void attn_fwd_v2(const bf16* __restrict__ qkv, bf16* __restrict__ o,
                                                   float* __restrict__ lse, int Tn, int H, float scale, DropArgs da,
                                                   uint32_t site) {
  static_assert(DROP, "the forward without dropout is attn_fwd_v3");
  typedef ATile<HDP> AT;
  constexpr int KK = HDP / 32, CB = HDP / 16;
  __shared__ __attribute__((aligned(16))) bf16 Ks[64 * HDP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[64 * HDP];
  const int nqb = (Tn + 63) / 64;
  // (batch*head) varies fastest, so every block of a query-block index is issued
  // before any shorter one (longest first keeps the tail short) and one head's
  // blocks share an XCD's L2 (workgroups go round-robin over the 8 XCDs)
  const int qb = nqb - 1 - blockIdx.y;
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4;
  const int d = H * HDP;
  const int64_t ld = 3 * (int64_t)d;
  const bf16* base = qkv + (int64_t)b * Tn * ld;
  const int q = qb * 64 + w * 16 + (lane & 15);      // this lane's query
  const float c = scale * LOG2E_F;
  bf16x8 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; kk++)
    qf[kk] = q < Tn ? *(const bf16x8*)(base + (int64_t)q * ld + h * HDP + kk * 32 + g * 8) : (bf16x8){};
  f32x4 ot[CB];
#pragma unroll
  for (int cb = 0; cb < CB; cb++) ot[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;   // running max of S*c over the keys seen (same in the four lanes of a query)
  // The running sum of exp2(S*c - m) comes from the matrix cores: an A fragment of
  // ones times a P fragment gives, in each of the four entries, the sum of the
  // fragment's 32 (bf16-rounded) probabilities of this lane's query. That moves 16
  // VALU adds per tile (the forward is VALU-bound) to two MFMAs, and normalizes O by
  // the sum of the probabilities before the mask (the mask multiplies only the P that
  // weights V).
  f32x4 lt = (f32x4){0.f, 0.f, 0.f, 0.f};
  const bf16x8 ones = (bf16x8){(bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f,
                               (bf16)1.f, (bf16)1.f, (bf16)1.f, (bf16)1.f};

  const auto src = range_rsrc(base, (int64_t)Tn * ld * 2);
  TileRegs<HDP> kr, vr;
  kr.load(src, (int)ld, 0, d + h * HDP);
  vr.load(src, (int)ld, 0, 2 * d + h * HDP);
  for (int kt = 0; kt <= qb; kt++) {
    __syncthreads();
    kr.store(Ks);
    vr.store(Vs);
    __syncthreads();
    if (kt < qb) {
      kr.load(src, (int)ld, (kt + 1) * 64, d + h * HDP);
      vr.load(src, (int)ld, (kt + 1) * 64, 2 * d + h * HDP);
    }
    f32x4 st[4];
#pragma unroll
    for (int nb = 0; nb < 4; nb++) {
      st[nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; kk++)
        st[nb] = Mfma<bf16>::mma(AT::row_frag(Ks, nb * 16 + (lane & 15), kk * 4 + g), qf[kk], st[nb]);
    }
    if (kt == qb) {                                   // keys after the query, or past Tn
      const int lim = q - kt * 64;
#pragma unroll
      for (int nb = 0; nb < 4; nb++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int kl = nb * 16 + 4 * g + i;
          if (kl > lim || kt * 64 + kl >= Tn) st[nb][i] = -INFINITY;
        }
    }
    float mx = st[0][0];
#pragma unroll
    for (int nb = 0; nb < 4; nb++)
#pragma unroll
      for (int i = 0; i < 4; i++) mx = fmaxf(mx, st[nb][i]);
    // The running max is moved only when a row's max grows by more than 2^RESCALE_LAG
    // over it (and on the first tile): until then P = exp2(S c - m) stays below 2^8,
    // which bf16 and the fp32 sums hold at full relative precision, and l and the
    // output carry the same stale m, so the result is the same. Most tiles then skip
    // the rescale of the output accumulators.
    const float mt = group_max(mx) * c;              // finite: key 0 is always visible
    if (__any(mt > m + RESCALE_LAG)) {
      const float mnew = fmaxf(m, mt);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      lt *= alpha;
#pragma unroll
      for (int cb = 0; cb < CB; cb++) ot[cb] *= alpha;
      m = mnew;
    }
#pragma unroll
    for (int nb = 0; nb < 4; nb++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[nb][i], c, -m));
        st[nb][i] = p;
      }
    // the row sum takes the undropped P; this lane's four keys of a block share one
    // Philox block
#pragma unroll
    for (int kp = 0; kp < 2; kp++) lt = Mfma<bf16>::mma(ones, pack_p(st[2 * kp], st[2 * kp + 1]), lt);
#pragma unroll
    for (int nb = 0; nb < 4; nb++) st[nb] *= drop_mult4(da, site, (uint32_t)(bh * Tn + q), kt * 16 + nb * 4 + g);
#pragma unroll
    for (int kp = 0; kp < 2; kp++) {
      const bf16x8 pf = pack_p(st[2 * kp], st[2 * kp + 1]);
#pragma unroll
      for (int cb = 0; cb < CB; cb++) {
        const bf16x8 vf = cat4(AT::tr(Vs, 32 * kp + 4 * g, cb * 16), AT::tr(Vs, 32 * kp + 16 + 4 * g, cb * 16));
        ot[cb] = Mfma<bf16>::mma(vf, pf, ot[cb]);
      }
    }
  }
  const float l = lt[0];
  if (q < Tn) {
    const float inv = 1.f / l;
    bf16* orow = o + ((int64_t)b * Tn + q) * d + h * HDP;
#pragma unroll
    for (int cb = 0; cb < CB; cb++) {
      bf16x4 v;
#pragma unroll
      for (int i = 0; i < 4; i++) v[i] = (bf16)(ot[cb][i] * inv);
      *(bf16x4*)(orow + cb * 16 + 4 * g) = v;
    }
    if (g == 0) lse[(int64_t)bh * Tn + q] = (m + log2f(l)) * LN2_F;
  }
}

// dQ for a 64-query block; also writes D = rowsum(dO * O) for these queries,
// which the dK/dV kernel (launched after) reads.
template <int HDP, bool DROP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void attn_bwd_dq_v2(const bf16* __restrict__ qkv, const bf16* __restrict__ o,
                                                      const bf16* __restrict__ dout, const float* __restrict__ lse,
                                                      float* __restrict__ Dv, bf16* __restrict__ dqkv, int Tn, int H,
                                                      float scale, float* __restrict__ bias_part, DropArgs da,
                                                      uint32_t site) {
  typedef ATile<HDP> AT;
  constexpr int KK = HDP / 32, CB = HDP / 16;
  __shared__ __attribute__((aligned(16))) bf16 Ks[64 * HDP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[64 * HDP];
  const int nqb = (Tn + 63) / 64;
  const int qb = nqb - 1 - blockIdx.y;                // longest first, as in the forward
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4;
  const int d = H * HDP;
  const int64_t ld = 3 * (int64_t)d;
  const bf16* base = qkv + (int64_t)b * Tn * ld;
  const int q = qb * 64 + w * 16 + (lane & 15);
  const float c = scale * LOG2E_F;
  bf16x8 qf[KK], dof[KK];
  float Dq = 0.f;
#pragma unroll
  for (int kk = 0; kk < KK; kk++) {
    const int col = kk * 32 + g * 8;
    if (q < Tn) {
      qf[kk] = *(const bf16x8*)(base + (int64_t)q * ld + h * HDP + col);
      dof[kk] = *(const bf16x8*)(dout + ((int64_t)b * Tn + q) * d + h * HDP + col);
      const bf16x8 ov = *(const bf16x8*)(o + ((int64_t)b * Tn + q) * d + h * HDP + col);
#pragma unroll
      for (int e = 0; e < 8; e++) Dq += (float)dof[kk][e] * (float)ov[e];
    } else {
      qf[kk] = (bf16x8){};
      dof[kk] = (bf16x8){};
    }
  }
  Dq = group_sum(Dq);
  // lse in base-2 units; +inf past Tn makes every P of such a query exactly 0
  const float lq = q < Tn ? lse[(int64_t)bh * Tn + q] * LOG2E_F : INFINITY;
  if (q < Tn && g == 0) Dv[(int64_t)bh * Tn + q] = Dq;

  f32x4 dqt[CB];
#pragma unroll
  for (int cb = 0; cb < CB; cb++) dqt[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const auto src = range_rsrc(base, (int64_t)Tn * ld * 2);
  TileRegs<HDP> kr, vr;
  kr.load(src, (int)ld, 0, d + h * HDP);
  vr.load(src, (int)ld, 0, 2 * d + h * HDP);
  for (int kt = 0; kt <= qb; kt++) {
    __syncthreads();
    kr.store(Ks);
    vr.store(Vs);
    __syncthreads();
    if (kt < qb) {
      kr.load(src, (int)ld, (kt + 1) * 64, d + h * HDP);
      vr.load(src, (int)ld, (kt + 1) * 64, 2 * d + h * HDP);
    }
    f32x4 st[4], ds[4];
#pragma unroll
    for (int nb = 0; nb < 4; nb++) {
      // the dP accumulator starts at -D, so the MFMAs leave dP - D
      f32x4 dpt = (f32x4){-Dq, -Dq, -Dq, -Dq};
      st[nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; kk++) {
        st[nb] = Mfma<bf16>::mma(AT::row_frag(Ks, nb * 16 + (lane & 15), kk * 4 + g), qf[kk], st[nb]);
        dpt = Mfma<bf16>::mma(AT::row_frag(Vs, nb * 16 + (lane & 15), kk * 4 + g), dof[kk], dpt);
      }
      if constexpr (DROP) {
        // Z dP - D from t = dP - D as Z t + (Z D - D): at Z = 1 the inner term is exactly
        // 0 and the result is t itself, bit for bit; at Z = 0 it is -D
        const f32x4 mk = drop_mult4(da, site, (uint32_t)(bh * Tn + q), kt * 16 + nb * 4 + g);
#pragma unroll
        for (int i = 0; i < 4; i++) dpt[i] = __builtin_fmaf(mk[i], dpt[i], __builtin_fmaf(mk[i], Dq, -Dq));
      }
      ds[nb] = dpt;
    }
    if (kt == qb) {                                   // diagonal tile: local keys <= q - k0 are visible
      const int lim = q - kt * 64;
#pragma unroll
      for (int nb = 0; nb < 4; nb++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float p = nb * 16 + 4 * g + i <= lim ? __builtin_amdgcn_exp2f(__builtin_fmaf(st[nb][i], c, -lq)) : 0.f;
          ds[nb][i] *= p;
        }
    } else {
#pragma unroll
      for (int nb = 0; nb < 4; nb++)
#pragma unroll
        for (int i = 0; i < 4; i++) ds[nb][i] *= __builtin_amdgcn_exp2f(__builtin_fmaf(st[nb][i], c, -lq));
    }
#pragma unroll
    for (int kp = 0; kp < 2; kp++) {
      const bf16x8 df = pack_p(ds[2 * kp], ds[2 * kp + 1]);
#pragma unroll
      for (int cb = 0; cb < CB; cb++) {
        const bf16x8 kf = cat4(AT::tr(Ks, 32 * kp + 4 * g, cb * 16), AT::tr(Ks, 32 * kp + 16 + 4 * g, cb * 16));
        dqt[cb] = Mfma<bf16>::mma(kf, df, dqt[cb]);
      }
    }
  }
  if (q < Tn) {
    bf16* row = dqkv + ((int64_t)b * Tn + q) * ld + h * HDP;
#pragma unroll
    for (int cb = 0; cb < CB; cb++) {
      bf16x4 v;
#pragma unroll
      for (int i = 0; i < 4; i++) v[i] = (bf16)(dqt[cb][i] * scale);
      *(bf16x4*)(row + cb * 16 + 4 * g) = v;
    }
  }
  // queries past Tn have P = 0, so their dq is 0 and adds nothing here
  if (bias_part) {
    __syncthreads();                                  // the K/V tiles are free: reuse them for the reduction
    block_colsum<HDP>(dqt, scale, (float*)Ks, bias_part + ((int64_t)b * nqb + qb) * ld + h * HDP);
  }
}

// A quad of lanes (j = lane & 3) each holding one Philox block b_j: lane j gets
// the words b_0[j], b_1[j], b_2[j], b_3[j]. In round r, lane i offers its word
// (i + r) & 3 and lane j reads lane (j - r) & 3 (a fixed quad permutation), which
// offers exactly word j.
__device__ inline uint32_t sel4(const u32x4& v, int k) {
  return k == 0 ? v[0] : (k == 1 ? v[1] : (k == 2 ? v[2] : v[3]));
}
__device__ inline u32x4 quad_transpose(const u32x4& b) {
  const int j = threadIdx.x & 3;
  u32x4 out;
  out[0] = out[1] = out[2] = out[3] = 0u;
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const uint32_t send = sel4(b, (j + r) & 3);
    // quad_perm selectors [(0-r)&3, (1-r)&3, (2-r)&3, (3-r)&3]: lane j reads lane (j - r) & 3
    uint32_t got = send;
    if (r == 1) got = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x93, 0xf, 0xf, false);
    if (r == 2) got = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x4E, 0xf, 0xf, false);
    if (r == 3) got = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x39, 0xf, 0xf, false);
    const int i = (j - r) & 3;
#pragma unroll
    for (int k = 0; k < 4; k++) out[k] = i == k ? got : out[k];
  }
  return out;
}

// dK and dV for a 64-key block over the query tiles at or after it.
template <int HDP, bool DROP>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_v2(const bf16* __restrict__ qkv, const bf16* __restrict__ dout,
                                                        const float* __restrict__ lse, const float* __restrict__ Dv,
                                                        bf16* __restrict__ dqkv, int Tn, int H, float scale,
                                                        float* __restrict__ bias_part, DropArgs da, uint32_t site) {
  typedef ATile<HDP> AT;
  constexpr int KK = HDP / 32, CB = HDP / 16;
  __shared__ __attribute__((aligned(16))) bf16 Qs2[2][64 * HDP];   // double-buffered Q and dO tiles
  __shared__ __attribute__((aligned(16))) bf16 dOs2[2][64 * HDP];
  __shared__ __attribute__((aligned(16))) float ls2[2][64];
  __shared__ __attribute__((aligned(16))) float Ds2[2][64];
  const int nb_t = (Tn + 63) / 64;
  const int kb = blockIdx.y;                          // key blocks near 0 see the most queries: first
  const int bh = blockIdx.x, b = bh / H, h = bh % H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4;
  const int d = H * HDP;
  const int64_t ld = 3 * (int64_t)d;
  const bf16* base = qkv + (int64_t)b * Tn * ld;
  const bf16* dob = dout + (int64_t)b * Tn * d;
  const int key = kb * 64 + w * 16 + (lane & 15);    // this lane's key (B-operand column)
  const float c = scale * LOG2E_F;
  bf16x8 kf[KK], vf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; kk++) {
    const int col = kk * 32 + g * 8;
    kf[kk] = key < Tn ? *(const bf16x8*)(base + (int64_t)key * ld + d + h * HDP + col) : (bf16x8){};
    vf[kk] = key < Tn ? *(const bf16x8*)(base + (int64_t)key * ld + 2 * d + h * HDP + col) : (bf16x8){};
  }
  f32x4 dkt[CB], dvt[CB];
#pragma unroll
  for (int cb = 0; cb < CB; cb++) {
    dkt[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    dvt[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  // lse (base-2 units, +inf past Tn so those queries get P = 0) and D of the next
  // query tile, held by the first wavefront until the tile is stored to LDS
  const auto lsrc = range_rsrc(lse + (int64_t)bh * Tn, (int64_t)Tn * 4);
  const auto dsrc = range_rsrc(Dv + (int64_t)bh * Tn, (int64_t)Tn * 4);
  auto stats = [&](int gq, float& lv, float& dv) {
    lv = gq < Tn ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(lsrc, gq * 4, 0, 0)) * LOG2E_F : INFINITY;
    dv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(dsrc, gq * 4, 0, 0));
  };
  float lnext = 0.f, dnext = 0.f;
  if (threadIdx.x < 64) stats(kb * 64 + threadIdx.x, lnext, dnext);
  const auto qsrc = range_rsrc(base, (int64_t)Tn * ld * 2);
  const auto dosrc = range_rsrc(dob, (int64_t)Tn * d * 2);
  // query tile qt goes to buffer (qt - kb) & 1 during step qt - 1 (one barrier per step)
  TileRegs<HDP> qr, dr;
  auto put = [&](int buf) {
    qr.store(Qs2[buf]);
    dr.store(dOs2[buf]);
    if (threadIdx.x < 64) {
      ls2[buf][threadIdx.x] = lnext;
      Ds2[buf][threadIdx.x] = dnext;
    }
  };
  qr.load(qsrc, (int)ld, kb * 64, h * HDP);
  dr.load(dosrc, d, kb * 64, h * HDP);
  put(0);
  if (kb + 1 < nb_t) {
    qr.load(qsrc, (int)ld, kb * 64 + 64, h * HDP);
    dr.load(dosrc, d, kb * 64 + 64, h * HDP);
    if (threadIdx.x < 64) stats(kb * 64 + 64 + threadIdx.x, lnext, dnext);
  }
  __syncthreads();
  for (int qt = kb; qt < nb_t; qt++) {
    const int q0 = qt * 64, cur = (qt - kb) & 1;
    const bf16* Qs = Qs2[cur];
    const bf16* dOs = dOs2[cur];
    const float* ls = ls2[cur];
    const float* Ds = Ds2[cur];
    if (qt + 1 < nb_t) {
      // buffer cur ^ 1 was last read in step qt - 1, which ended with a barrier
      put(cur ^ 1);
      if (qt + 2 < nb_t) {
        qr.load(qsrc, (int)ld, q0 + 128, h * HDP);
        dr.load(dosrc, d, q0 + 128, h * HDP);
        if (threadIdx.x < 64) stats(q0 + 128 + threadIdx.x, lnext, dnext);
      }
    }
    f32x4 p[4], ds[4], mk[DROP ? 4 : 1];
#pragma unroll
    for (int nb = 0; nb < 4; nb++) {
      f32x4 dp = (f32x4){0.f, 0.f, 0.f, 0.f};
      p[nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; kk++) {
        p[nb] = Mfma<bf16>::mma(AT::row_frag(Qs, nb * 16 + (lane & 15), kk * 4 + g), kf[kk], p[nb]);
        dp = Mfma<bf16>::mma(AT::row_frag(dOs, nb * 16 + (lane & 15), kk * 4 + g), vf[kk], dp);
      }
      p[nb] = __builtin_elementwise_fma(p[nb], (f32x4){c, c, c, c}, -*(const f32x4*)(ls + nb * 16 + 4 * g));
      if constexpr (DROP) {
        // this lane holds queries q0 + nb*16 + 4g + i of one key: lane j of the quad
        // makes the block of query i = j (the quad's four keys are one counter's
        // words), then the quad trades words
        const uint32_t qrow = (uint32_t)(bh * Tn + q0 + nb * 16 + 4 * g + (lane & 3));
        const u32x4 wv = quad_transpose(philox4x32_10((uint32_t)key >> 2, qrow, site, da.call, da.k0, da.k1));
#pragma unroll
        for (int i = 0; i < 4; i++) mk[nb][i] = wv[i] >= da.thr ? da.scale : 0.f;
        dp *= mk[nb];
      }
      ds[nb] = dp - *(const f32x4*)(Ds + nb * 16 + 4 * g);
    }
    if (qt == kb) {                                   // diagonal tile: local queries >= key - q0 see the key
      const int lim = key - q0;
#pragma unroll
      for (int nb = 0; nb < 4; nb++)
#pragma unroll
        for (int i = 0; i < 4; i++) p[nb][i] = nb * 16 + 4 * g + i >= lim ? __builtin_amdgcn_exp2f(p[nb][i]) : 0.f;
    } else {
#pragma unroll
      for (int nb = 0; nb < 4; nb++)
#pragma unroll
        for (int i = 0; i < 4; i++) p[nb][i] = __builtin_amdgcn_exp2f(p[nb][i]);
    }
#pragma unroll
    for (int nb = 0; nb < 4; nb++) ds[nb] *= p[nb];
    if constexpr (DROP) {
#pragma unroll
      for (int nb = 0; nb < 4; nb++) p[nb] *= mk[nb];
    }
#pragma unroll
    for (int qp = 0; qp < 2; qp++) {
      const bf16x8 pf = pack_p(p[2 * qp], p[2 * qp + 1]);
      const bf16x8 df = pack_p(ds[2 * qp], ds[2 * qp + 1]);
#pragma unroll
      for (int cb = 0; cb < CB; cb++) {
        const bf16x8 dof = cat4(AT::tr(dOs, 32 * qp + 4 * g, cb * 16), AT::tr(dOs, 32 * qp + 16 + 4 * g, cb * 16));
        dvt[cb] = Mfma<bf16>::mma(dof, pf, dvt[cb]);
        const bf16x8 qf = cat4(AT::tr(Qs, 32 * qp + 4 * g, cb * 16), AT::tr(Qs, 32 * qp + 16 + 4 * g, cb * 16));
        dkt[cb] = Mfma<bf16>::mma(qf, df, dkt[cb]);
      }
    }
    __syncthreads();   // tile qt + 1 is visible; buffer cur is free
  }
  if (key < Tn) {
    bf16* row = dqkv + ((int64_t)b * Tn + key) * ld + h * HDP;
#pragma unroll
    for (int cb = 0; cb < CB; cb++) {
      bf16x4 vk, vv;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        vk[i] = (bf16)(dkt[cb][i] * scale);
        vv[i] = (bf16)dvt[cb][i];
      }
      *(bf16x4*)(row + d + cb * 16 + 4 * g) = vk;
      *(bf16x4*)(row + 2 * d + cb * 16 + 4 * g) = vv;
    }
  }
  // keys past Tn see no query with P != 0, so their dk and dv are 0
  if (bias_part) {
    float* dst = bias_part + ((int64_t)b * nb_t + kb) * ld + h * HDP;
    block_colsum<HDP>(dkt, scale, (float*)Qs2[0], dst + d);
    __syncthreads();
    block_colsum<HDP>(dvt, 1.f, (float*)Qs2[0], dst + 2 * d);
  }
}

// ----------------------------------------------------------------------------- launchers
template <typename T, int HDP, bool DROP>
static hipError_t fwd_t(const void* qkv, void* o, float* lse, int B, int Tn, int H, int hd, const DropArgs& da,
                        uint32_t site, hipStream_t s) {
  dim3 grid((Tn + 63) / 64, B * H);
  const float scale = 1.0f / sqrtf((float)hd);
  hipLaunchKernelGGL((attn_fwd_kernel<T, HDP, DROP>), grid, dim3(256), 0, s, (const T*)qkv, (T*)o, lse, Tn, H, hd,
                     scale, da, site);
  return hipGetLastError();
}

template <bool DROP>
static hipError_t fwd_any(const void* qkv, void* o, float* lse, bool bf16_ops, int B, int T, int H, int hd,
                          const DropArgs& da, uint32_t site, hipStream_t s) {
  if (bf16_ops && (hd == 32 || hd == 64)) {
    if ((int64_t)T * 3 * H * hd * 2 > INT32_MAX) return hipErrorInvalidValue;   // 32-bit buffer offsets per sequence
    const float scale = 1.0f / sqrtf((float)hd);
    if (DROP) {
      dim3 grid(B * H, (T + 63) / 64);
      if (hd == 64)
        hipLaunchKernelGGL((attn_fwd_v2<64, true>), grid, dim3(256), 0, s, (const bf16*)qkv, (bf16*)o, lse, T, H,
                           scale, da, site);
      else
        hipLaunchKernelGGL((attn_fwd_v2<32, true>), grid, dim3(256), 0, s, (const bf16*)qkv, (bf16*)o, lse, T, H,
                           scale, da, site);
    } else {
      dim3 grid(B * H, (T + 127) / 128);
      if (hd == 64)
        hipLaunchKernelGGL((attn_fwd_v3<64, false>), grid, dim3(256), 0, s, (const bf16*)qkv, (bf16*)o, lse, T, H,
                           scale, da, site);
      else
        hipLaunchKernelGGL((attn_fwd_v3<32, false>), grid, dim3(256), 0, s, (const bf16*)qkv, (bf16*)o, lse, T, H,
                           scale, da, site);
    }
    return hipGetLastError();
  }
  if (bf16_ops)
    return hd <= 32 ? fwd_t<bf16, 32, DROP>(qkv, o, lse, B, T, H, hd, da, site, s)
                    : fwd_t<bf16, 64, DROP>(qkv, o, lse, B, T, H, hd, da, site, s);
  return hd <= 32 ? fwd_t<float, 32, DROP>(qkv, o, lse, B, T, H, hd, da, site, s)
                  : fwd_t<float, 64, DROP>(qkv, o, lse, B, T, H, hd, da, site, s);
}

hipError_t launch_attn_fwd(const void* qkv, void* o, float* lse, bool bf16_ops, int B, int T, int H, int hd,
                           const DropArgs& da, uint32_t site, hipStream_t s) {
  if (hd <= 0 || hd > 64) return hipErrorInvalidValue;
  return da.on ? fwd_any<true>(qkv, o, lse, bf16_ops, B, T, H, hd, da, site, s)
               : fwd_any<false>(qkv, o, lse, bf16_ops, B, T, H, hd, da, site, s);
}

template <typename T, int HDP, bool DROP>
static hipError_t bwd_t(const void* qkv, const void* o, const void* dout, const float* lse, float* D, void* dqkv,
                        int B, int Tn, int H, int hd, const DropArgs& da, uint32_t site, hipStream_t s) {
  const float scale = 1.0f / sqrtf((float)hd);
  const int n = B * H * Tn;
  hipLaunchKernelGGL(attn_bwd_D_kernel<T>, dim3((n + 255) / 256), dim3(256), 0, s, (const T*)o, (const T*)dout, D,
                     B, Tn, H, hd);
  dim3 grid((Tn + 63) / 64, B * H);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, HDP, DROP>), grid, dim3(256), 0, s, (const T*)qkv, (const T*)dout,
                     lse, (const float*)D, (T*)dqkv, Tn, H, hd, scale, da, site);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, HDP, DROP>), grid, dim3(256), 0, s, (const T*)qkv, (const T*)dout, lse,
                     (const float*)D, (T*)dqkv, Tn, H, hd, scale, da, site);
  return hipGetLastError();
}

int attn_bwd_colsum_rows(bool bf16_ops, int B, int T, int hd) {
  return bf16_ops && (hd == 32 || hd == 64) ? B * ((T + 63) / 64) : 0;
}

template <bool DROP>
static hipError_t bwd_any(const void* qkv, const void* o, const void* dout, const float* lse, float* D, void* dqkv,
                          bool bf16_ops, int B, int T, int H, int hd, float* bias_part, const DropArgs& da,
                          uint32_t site, hipStream_t s) {
  if (bf16_ops && (hd == 32 || hd == 64)) {
    if ((int64_t)T * 3 * H * hd * 2 > INT32_MAX) return hipErrorInvalidValue;   // 32-bit buffer offsets per sequence
    dim3 grid(B * H, (T + 63) / 64);
    const float scale = 1.0f / sqrtf((float)hd);
    if (hd == 64) {
      hipLaunchKernelGGL((attn_bwd_dq_v2<64, DROP>), grid, dim3(256), 0, s, (const bf16*)qkv, (const bf16*)o,
                         (const bf16*)dout, lse, D, (bf16*)dqkv, T, H, scale, bias_part, da, site);
      hipLaunchKernelGGL((attn_bwd_dkdv_v2<64, DROP>), grid, dim3(256), 0, s, (const bf16*)qkv, (const bf16*)dout,
                         lse, (const float*)D, (bf16*)dqkv, T, H, scale, bias_part, da, site);
    } else {
      hipLaunchKernelGGL((attn_bwd_dq_v2<32, DROP>), grid, dim3(256), 0, s, (const bf16*)qkv, (const bf16*)o,
                         (const bf16*)dout, lse, D, (bf16*)dqkv, T, H, scale, bias_part, da, site);
      hipLaunchKernelGGL((attn_bwd_dkdv_v2<32, DROP>), grid, dim3(256), 0, s, (const bf16*)qkv, (const bf16*)dout,
                         lse, (const float*)D, (bf16*)dqkv, T, H, scale, bias_part, da, site);
    }
    return hipGetLastError();
  }
  if (bf16_ops)
    return hd <= 32 ? bwd_t<bf16, 32, DROP>(qkv, o, dout, lse, D, dqkv, B, T, H, hd, da, site, s)
                    : bwd_t<bf16, 64, DROP>(qkv, o, dout, lse, D, dqkv, B, T, H, hd, da, site, s);
  return hd <= 32 ? bwd_t<float, 32, DROP>(qkv, o, dout, lse, D, dqkv, B, T, H, hd, da, site, s)
                  : bwd_t<float, 64, DROP>(qkv, o, dout, lse, D, dqkv, B, T, H, hd, da, site, s);
}

hipError_t launch_attn_bwd(const void* qkv, const void* o, const void* dout, const float* lse, float* D,
                           void* dqkv, bool bf16_ops, int B, int T, int H, int hd, float* bias_part,
                           const DropArgs& da, uint32_t site, hipStream_t s) {
  if (hd <= 0 || hd > 64) return hipErrorInvalidValue;
  if (bias_part && attn_bwd_colsum_rows(bf16_ops, B, T, hd) == 0) return hipErrorInvalidValue;
  return da.on ? bwd_any<true>(qkv, o, dout, lse, D, dqkv, bf16_ops, B, T, H, hd, bias_part, da, site, s)
               : bwd_any<false>(qkv, o, dout, lse, D, dqkv, bf16_ops, B, T, H, hd, bias_part, da, site, s);
}

}  // namespace gpt
