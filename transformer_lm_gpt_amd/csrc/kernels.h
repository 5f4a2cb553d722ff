// Host-side launchers of the gfx950 kernels. Each returns hipSuccess or the
// launch error; shapes are validated by the runtime before the call.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gpt {

// Dropout masks from the counter-based generator Philox4x32-10 (Salmon, Moraes,
// Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011), as the
// nanoGPT run log (sections 2.1 and 2.2) uses dropout: on the embedding output,
// the attention probabilities and each residual branch before its add. Element
// (row, col) of a site's tensor takes word col % 4 of the block at counter
// (col / 4, row, site, call) under the key (k0, k1); it is kept when that word is
// >= thr, and a kept value is multiplied by `scale`, a dropped one by 0.
// Rows and columns: token row b*T + t by channel for the embedding and branch
// outputs; row (b*H + h)*T + i by key j for the attention probabilities.
struct DropArgs {
  uint32_t k0, k1;   // key: the seed's low and high words
  uint32_t call;     // forward counter
  uint32_t thr;      // floor(p * 2^32)
  float scale;       // 1 / (1 - p), rounded to fp32
  int32_t on;        // 0: no dropout (no mask is evaluated)
};
// Site numbers: the embedding output, then per layer l the attention
// probabilities, the attention branch output and the MLP branch output.
inline uint32_t site_embed() { return 0; }
inline uint32_t site_attn_prob(int l) { return 3u * l + 1; }
inline uint32_t site_attn_out(int l) { return 3u * l + 2; }
inline uint32_t site_mlp_out(int l) { return 3u * l + 3; }

enum Epilogue {
  EPI_STORE = 0,       // C(T)   = acc
  EPI_BIAS = 1,        // C(T)   = acc + bias[n]
  EPI_BIAS_RESID = 2,  // C(f32) = resid[m, n] + acc + bias[n]
  EPI_BIAS_GELU = 3,   // u = acc + bias[n]: aux(T) = gelu'(u) (saved for EPI_GELU_BWD);  C(T) = gelu(u)
  EPI_F32 = 4,         // C(f32) = acc
  EPI_GELU_BWD = 5,    // C(T)   = acc * aux[m, n], aux = gelu'(u) from EPI_BIAS_GELU (operand type T)
  EPI_ACC = 6,         // C(f32) = beta * C + acc   (beta is 0 or 1; C is not read when 0)
  EPI_BIAS_RESID_DROP = 7,  // C(f32) = resid[m, n] + mask(drop_site, m, n) * (acc + bias[n])
  EPI_BIAS_RELU = 8,   // aux(T) = u = acc + bias[n];  C(T) = max(u, 0)
  EPI_RELU_BWD = 9,    // C(T)   = acc * (aux[m, n] > 0)   (aux in operand type T)
};

// C[m, n] = sum_k A(m, k) B(n, k) followed by the epilogue, where
//   A(m, k) = a_kc ? A[m * lda + k] : A[k * lda + m]
//   B(n, k) = b_kc ? B[n * ldb + k] : B[k * ldb + n]
// T is the operand type (float or bf16), selected by `bf16_operands`.
struct GemmDesc {
  const void* A; int64_t lda; bool a_kc;
  const void* B; int64_t ldb; bool b_kc;
  void* C; int64_t ldc;
  int M, N, K;
  int epi;
  const float* bias;
  const float* resid; int64_t ldr;
  void* aux; int64_t ldaux;
  float beta;
  float* split_ws; size_t split_ws_floats;   // optional split-K workspace (EPI_ACC only)
  // optional, EPI_GELU_BWD only: per-tile-row column sums of C (fp32, before
  // rounding) into colsum[r * N + n], r < gemm_colsum_rows(...)
  float* colsum;
  // EPI_BIAS_RESID_DROP only: the branch output's mask (rows m and columns n of C)
  DropArgs drop;
  uint32_t drop_site;
  // optional: a device counter the call adds one to once its product is written
  // (the decode step's cache position); in the same launch when the product takes
  // the few-rows kernel, else by a one-thread launch after it
  int* bump;
  // optional (norm 1: LayerNorm with gain norm_g and shift norm_b, eps 1e-5; norm 2:
  // weightless RMSNorm): A is not read; the product takes A = norm(norm_x) over
  // rows of K fp32, computed inside the launch. Only where gemm_norm_fusable holds.
  int norm;
  const float* norm_x;
  const float* norm_g;
  const float* norm_b;
};

hipError_t launch_gemm(const GemmDesc& d, bool bf16_operands, hipStream_t s);
// Whether launch_gemm takes `d` with its normalization fused (bf16 operands, M <= 16,
// K <= 1024, a bias epilogue); otherwise the caller normalizes A itself.
bool gemm_norm_fusable(const GemmDesc& d, bool bf16_operands);
// Partial rows the fused column sum of `d` writes, or 0 when the kernel chosen for
// `d` cannot fuse it (then colsum must be NULL and the caller sums C itself).
int gemm_colsum_rows(const GemmDesc& d, bool bf16_operands);

// Grouped weight gradients, all sharing the contraction length K (the tokens):
// for each problem, C[m, n] = beta * C[m, n] + sum_k A[k * lda + m] * B[k * ldb + n]
// (bf16 operands, both m-contiguous; fp32 C). One launch covers every problem:
// whole 256 x 256 tiles are dealt round-robin to one workgroup per CU, and the
// tiles left over after the last full round are shared stream-K style, their
// partial sums reduced in a fixed order by a second kernel.
struct WgradProblem {
  const void* A; int64_t lda;
  const void* B; int64_t ldb;
  float* C; int64_t ldc;
  int32_t M, N;
  int32_t tiles_m, tiles_n;
  int32_t first_tile;   // tiles of the problems before this one
  int32_t c_vec;        // C rows allow 16-column vector access
};
// Whether a problem of this shape can join the grouped launch (pointers 16-byte aligned).
bool wgrad_group_ok(int M, int N, int64_t lda, int64_t ldb, int64_t ldc);
// Tiles of a problem in the grouped launch.
int wgrad_group_tiles(int M, int N);
// Partial-sum workspace (floats) for the full grouped launch (fewer workgroups run
// with less).
size_t wgrad_group_ws_floats();
hipError_t launch_wgrad_group(const WgradProblem* probs, int nprob, int total_tiles, int K, float beta, float* ws,
                              size_t ws_floats, hipStream_t s);

// x0[m, :] = wte[tok[m], :] + wpe[m % T, :]   (fp32), times the embedding
// site's dropout mask when da.on. Ids outside [0, Vp) produce NaN rows instead of
// out-of-bounds reads.
hipError_t launch_embed_fwd(const float* wte, const float* wpe, const int32_t* tok, float* x0,
                            int M, int T, int d, int Vp, const DropArgs& da, hipStream_t s);
// dst[m, :] = src[m, :] * mask(site, m, :) for an fp32 [M, d] array (dst may be
// src). d must be a multiple of 4 and both pointers 16-byte aligned.
hipError_t launch_dropout_rows(const float* src, float* dst, int M, int d, const DropArgs& da, uint32_t site,
                               hipStream_t s);

// y = LN(x) with gain g, shift b; writes y as operand type, mean and rstd (fp32 [M]).
hipError_t launch_layernorm_fwd(const float* x, const float* g, const float* b, void* y, bool bf16_out,
                                float* mean, float* rstd, int M, int d, hipStream_t s);

// Weightless RMSNorm y = x / sqrt(mean(x^2) + 1e-5) (operand type); writes mean = 0 and
// rstd, so launch_layernorm_bwd with g = NULL is its backward. d a multiple of 4.
hipError_t launch_rmsnorm_fwd(const float* x, void* y, bool bf16_out, float* mean, float* rstd, int M, int d,
                              hipStream_t s);

// dx = dres + LN backward of dy; writes dx (fp32) and optionally its operand-type copy
// dx_op. dy is in the operand type (bf16 when bf16_out, else fp32); per-block partial column sums of dy * xhat, dy and dres (dres may be NULL,
// then part_r is unused) into part_g / part_b / part_r ([nblk, d] each,
// nblk = ceil(M / LN_BWD_ROWS)). dx may alias dres. d must be a multiple of 4.
// With da.on, the dres column sums take dres * mask(site_in) when site_in >= 0,
// and dx_op holds dx * mask(site_out) when site_out >= 0 (dx itself is unmasked).
// g = NULL: the backward of the weightless RMSNorm (part_g and part_b unused).
constexpr int LN_BWD_ROWS = 16;
hipError_t launch_layernorm_bwd(const void* dy, const float* x, const float* mean, const float* rstd,
                                const float* g, const float* dres, float* dx, void* dx_op, bool bf16_out,
                                float* part_g, float* part_b, float* part_r, int M, int d, const DropArgs& da,
                                int site_in, int site_out, hipStream_t s);

// Column sums of an [M, N] matrix (fp32 or bf16) into per-block partials [nblk, N].
constexpr int COLSUM_ROWS = 64;
hipError_t launch_colsum_partial(const void* X, bool bf16_in, int64_t ldx, int M, int N, float* part,
                                 hipStream_t s);
// Deferred column-sum reductions: job j adds the sum of its partial rows,
// part[r, n] for r < nblk (fixed order), into dst: dst[n] = beta * dst[n] + sum.
// All jobs of one backward run in a single launch of total_blk workgroups
// (RED_COLS columns each); first_blk numbers them, ascending.
struct RedJob {
  int64_t part;       // float offset of the [nblk, n] partials in the partial area
  int64_t dst;        // float offset of the destination in the gradient array
  int32_t n;          // columns
  int32_t rows_kind;  // index into RedRows: which producer wrote the partials
  int32_t first_blk;
  int32_t pad;
};
constexpr int RED_KINDS = 3;
constexpr int RED_COLS = 64;   // columns of one reduction job per workgroup
struct RedRows {
  int32_t nblk[RED_KINDS];   // partial rows written by each kind of producer in this backward
};
hipError_t launch_reduce_jobs(const RedJob* jobs, int njobs, int total_blk, const float* part, float* grads,
                              RedRows rows, float beta, hipStream_t s);

// Row-wise softmax cross-entropy over Vp columns of z (operand type, row stride ldz).
// Writes row_loss[m] = lse - z[m, y[m]] and overwrites z with
// (softmax - onehot(y)) * grad_scale.
hipError_t launch_xent(void* z, bool bf16_z, int64_t ldz, const int32_t* y, float* row_loss,
                       int M, int Vp, float grad_scale, hipStream_t s);
// out = sum(row_loss) / M (single block, fixed order).
hipError_t launch_mean(const float* row_loss, int M, float* out, hipStream_t s);

// Causal attention forward. qkv: [B*T, 3*d] (q | k | v, head h at columns h*hd);
// o: [B*T, d]; lse: fp32 [B*H, T].
// With da.on, O = (P * mask(site)) V; lse stays that of the undropped P.
hipError_t launch_attn_fwd(const void* qkv, void* o, float* lse, bool bf16_ops, int B, int T, int H,
                           int hd, const DropArgs& da, uint32_t site, hipStream_t s);
// Attention backward: D = rowsum(dO * O), then dK/dV and dQ into dqkv [B*T, 3*d].
// bias_part (optional): the qkv bias gradient's partial column sums of dqkv (fp32,
// before rounding), one row per (sequence, 64-row block): [attn_bwd_colsum_rows(), 3 H hd].
// Must be NULL when attn_bwd_colsum_rows() is 0 for the same arguments.
// With da.on (the forward's mask): dV = (P * Z)^T dO and dS = P * (Z * dP - D), Z the
// mask; D = rowsum(dO * O) is unchanged.
hipError_t launch_attn_bwd(const void* qkv, const void* o, const void* dout, const float* lse,
                           float* Dbuf, void* dqkv, bool bf16_ops, int B, int T, int H, int hd,
                           float* bias_part, const DropArgs& da, uint32_t site, hipStream_t s);
int attn_bwd_colsum_rows(bool bf16_ops, int B, int T, int hd);

// Embedding backward: dwpe[t] = beta * dwpe[t] + sum_b dx0[b, t]; dwte[tok] += rows of dx0,
// summed deterministically (stable sort by id, fixed-order segment sums). Works on four
// columns at a time: d must be a multiple of 4 and dx0, dwte, dwpe and piece_sums
// 16-byte aligned, else hipErrorInvalidValue before any launch.
struct EmbedBwdScratch {
  uint32_t* keys;       // [sort_n]
  float* piece_sums;    // [M, d]
};
int embed_bwd_sort_size(int M);   // power of two >= M
hipError_t launch_embed_bwd(const float* dx0, const int32_t* tok, float* dwte, float* dwpe, float beta_wpe,
                            int B, int T, int d, int Vp, EmbedBwdScratch scr, hipStream_t s);

// ---- inference with a key/value cache (decode.hip)
// x[b, :] = wte[tok[b], :] + wpe[pos, :] for B single-token rows; pos is read from
// device memory when the kernel runs (clamped to [0, Tmax)).
hipError_t launch_embed_pos(const float* wte, const float* wpe, const int32_t* tok, float* x, int B, int d, int Vp,
                            const int* pos, int Tmax, hipStream_t s);
// *p = v, as a kernel (stream-ordered; recordable in a graph, unlike a memset).
hipError_t launch_set_i32(int* p, int v, hipStream_t s);
// Copies the keys and values (columns d .. 3d) of qkv [B*T, 3d] into cache rows
// b * Tmax + pos0 + t ([B_max * Tmax, 2d], operand type). pos0 + T <= Tmax.
hipError_t launch_kv_append(const void* qkv, bool bf16_ops, void* cache, int B, int T, int Tmax, int pos0, int d,
                            hipStream_t s);
// Causal attention of one new query per sequence (q, k, v in qkv [B, 3d]) against
// positions 0 .. len-1, len = *pos + 1 read from device memory when the kernel runs
// (clamped to [1, Tmax]): 0 .. len-2 from the cache, len-1 from qkv, whose k and v the
// call also stores into cache position len-1. out [B, d]. Tmax <= 8192.
hipError_t launch_attn_decode(const void* qkv, void* cache, void* out, bool bf16_ops, int B, int H, int hd,
                              int Tmax, const int* pos, hipStream_t s);
// One token per row of fp32 logits [B, ld] over V columns: the argmax (lowest index
// on ties) when temperature <= 0, else a draw with uniform[b] from the softmax of
// logits / temperature over the logits >= the top_k-th largest (all when top_k <= 0
// or >= V), by inverse CDF in index order.
hipError_t launch_sample(const float* logits, int64_t ld, int B, int V, float temperature, int top_k,
                         const float* uniform, int32_t* out, hipStream_t s);

// Sum of squares of n floats into per-block partials [NORM_BLOCKS].
constexpr int NORM_BLOCKS = 1024;
hipError_t launch_sumsq_partial(const float* g, size_t n, float* part, hipStream_t s);
// Floats of the static device array behind gpt_adamw_step_noalloc (4 KB per GPU).
constexpr size_t NOALLOC_SCRATCH_FLOATS = 1024;
// Device address of that array on `device` (looked up once per device, with the
// device made current for the lookup).
hipError_t noalloc_norm_scratch(int device, float** out);

// Device state used by the optimizer (lives in the workspace).
struct OptState {
  int64_t t;            // completed steps
  float norm;           // last gradient norm (pre-clip)
  float coef;           // clip coefficient applied
  float bc1, bc2;       // 1 - beta^t for the pending step
  int32_t skip;         // 1 if the pending step is skipped (non-finite norm or bad ids)
  int32_t nonfinite;    // sticky flag read by the host at sync
  int32_t bad_ids;      // sticky: a checked token or target id was outside [0, vocab_size)
  int32_t pad;
};
// Sets st->bad_ids when any of the n ids lies outside [0, V) (a checking pass in
// front of the embedding gather; ids are only read).
hipError_t launch_check_ids(const int32_t* ids, int n, int V, OptState* st, hipStream_t s);
// Reduces the partials to the norm, decides skip/coef, advances t, sets bias corrections.
hipError_t launch_opt_prepare(const float* part, OptState* st, float clip, float beta1, float beta2,
                              float* norm_out, hipStream_t s);
// AdamW over n elements; elements [0, n_decay) decay. Writes the bf16 shadow if non-null.
hipError_t launch_adamw(float* p, const float* g, float* m, float* v, void* shadow_bf16, size_t n,
                        size_t n_decay, const OptState* st, float lr, float beta1, float beta2, float eps,
                        float wd, hipStream_t s);
// Transposed bf16 copies of 2-D tensors: for every entry {offset, rows, cols} of the
// device table, dst[offset + c * rows + r] = src[offset + r * cols + c].
struct TransposeEntry {
  int64_t offset, rows, cols, first_tile;   // first_tile: prefix sum of 64x64 tiles
};
hipError_t launch_transpose_bf16(const void* src, void* dst, const TransposeEntry* d_table, int n_entries,
                                 int64_t total_tiles, hipStream_t s);
// bf16 copy of n fp32 values.
hipError_t launch_cast_bf16(const float* src, void* dst, size_t n, hipStream_t s);

// Low-rank adapters: one job per adapted d x d block (the q or v rows of one
// layer's qkv weight). A [r, d], B [d, r], W0 and dW [d, d] row-major fp32.
struct LoraJob {
  const float* A;
  const float* B;
  const float* W0;      // frozen base block
  const float* dW;      // the block's weight gradient dq^T a (input of the adapter gradients)
  float* dA;
  float* dB;
  float* weff;          // fp32 merged block, or NULL
  void* weff_bf16;      // bf16 merged block, or NULL
};
// weff = W0 + s B A for every job; 1 <= r <= 64.
hipError_t launch_lora_merge(const LoraJob* jobs, int njobs, int d, int r, float s, hipStream_t st);
// dB = beta dB + s dW A^T and dA = beta dA + s B^T dW for every job (beta 0 or 1;
// the outputs are not read when it is 0); 1 <= r <= 64.
hipError_t launch_lora_grad(const LoraJob* jobs, int njobs, int d, int r, float s, float beta, hipStream_t st);
// Zero n 32-bit words with a fill kernel (safe inside captured graphs).
hipError_t launch_zero(void* p, size_t n_words, hipStream_t s);
// dst[m * N + n] = float(src[m * ld + n]) for an [M, N] block of operand type.
hipError_t launch_rows_to_f32(const void* src, bool bf16_src, int64_t ld, int M, int N, float* dst, hipStream_t s);

}  // namespace gpt
