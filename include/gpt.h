/*
 * gpt.h - C ABI of the MI355X (gfx950) GPT training-step library, libgpt.so.
 *
 * One training step of a GPT-2-style causal language model: token plus learned
 * position embedding, pre-LayerNorm decoder blocks (causal multi-head
 * attention, 4x GELU MLP, residual adds), final LayerNorm, lm_head tied to the
 * token embedding, softmax cross-entropy over the (padded) vocabulary, the full
 * backward pass with gradient accumulation, and an AdamW update with decoupled
 * weight decay and global-norm gradient clipping.
 *
 * Passages that define the operations (the nanoGPT pages):
 *   - "Building microGPT from scratch" (blog.hotdry.top), model-core section:
 *     embeddings, QKV projection, scaled dot-product, softmax, weighted V,
 *     output projection, the 4x MLP, residual plus norm; training-loop
 *     section: causal next-token loss averaged over positions, backward,
 *     Adam with (beta1, beta2, eps), gradient clipping at 1.0.
 *   - nanoGPT run log (wmrh.cn), section 2.1: AdamW with weight decay 0.1 and
 *     betas 0.9/0.95; section 3.1: gradient accumulation adds micro-batch
 *     gradients before one update (effective batch = batch x steps).
 *   - nanoGPT README translation (oa0.com): the GPT-2 124M model at block 1024.
 *   - Dropout: the nanoGPT run log, sections 2.1 and 2.2 (rate 0.1, or 0.0 on
 *     large data) and the microGPT page's parameter list (0.2 for the
 *     Shakespeare character model).
 *   - LoRA: the fine-tuning article (blog.hotdry.top), LoRA section: W0
 *     frozen, low-rank A and B on the q and v projections, the branch B A x
 *     scaled by lora_alpha / r, only A and B trained, B A mergeable into W0.
 *
 * Conventions
 *   - All device pointers are plain HIP device addresses. The library never
 *     allocates device memory: the caller allocates the buffers whose sizes
 *     gpt_get_sizes() reports and hands them over with gpt_bind(), together
 *     with the HIP stream every call is enqueued on. Calls are asynchronous
 *     on that stream unless stated otherwise.
 *   - Every function returns GPT_OK (0) or a negative GPT_E_* code; the
 *     message is available from gpt_last_error(). No exception crosses the ABI.
 *     An error is sticky: later calls on the handle return it until
 *     gpt_sync() reports and clears it.
 *   - One handle must not be used from several host threads at once.
 *   - Layout: parameters, gradients and both Adam moments are flat fp32 arrays
 *     with identical offsets (gpt_tensor_info_at). Every linear weight is
 *     stored [out, in] row-major and acts as y = x W^T + b. All 2-D tensors
 *     (the decayed ones) come first, then all 1-D tensors, then the LoRA
 *     adapters when lora_rank > 0; every tensor starts at a multiple of 64
 *     elements and the gaps are zero.
 */
#ifndef GPT_MI355X_H
#define GPT_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define GPT_OK              0
#define GPT_E_INVAL        -1  /* bad argument, config or shape                      */
#define GPT_E_SEQ_TOO_LONG -2  /* T > block_size or B > batch                        */
#define GPT_E_STATE        -3  /* call out of order (backward with no forward, ...)  */
#define GPT_E_UNSUPPORTED  -4  /* valid request this build does not implement        */
#define GPT_E_HIP          -5  /* HIP runtime or launch error                        */
#define GPT_E_NONFINITE    -6  /* non-finite loss or gradient norm: update skipped   */

#define GPT_PREC_FP32 0        /* every GEMM operand fp32                            */
#define GPT_F_KV_CACHE 1u      /* gpt_config.flags: reserve the key/value cache of
                                  gpt_prefill / gpt_decode in the workspace           */
#define GPT_F_MICROGPT 2u      /* gpt_config.flags: the microGPT block ("Building
                                  microGPT from scratch", model-core section):
                                  weightless RMSNorm y = x / sqrt(mean(x^2) + 1e-5)
                                  where the LayerNorms are, ReLU instead of GELU, no
                                  biases and an lm_head [padded_vocab, n_embd] of its
                                  own (tensors wte, wpe, h<l>.attn.w (q|k|v rows),
                                  h<l>.proj.w, h<l>.fc.w, h<l>.fcproj.w, lm_head; all
                                  decayed)                                           */
#define GPT_F_DEBUG_CHECKS 4u  /* gpt_config.flags: check every token id (gpt_forward_loss,
                                  gpt_forward_logits, gpt_prefill, gpt_decode) and target
                                  id (gpt_forward_loss) against [0, vocab_size) on the
                                  device before the embedding gather reads them (the
                                  fine-tuning article, data paragraph, and the nanoGPT
                                  README translation's OpenWebText preparation: the
                                  ids are GPT-2 BPE ids stored as uint16, of a
                                  50,257-token vocabulary). An id outside
                                  that range sets a sticky device flag: the next
                                  gpt_adamw_step is skipped (parameters, moments and the
                                  step counter untouched) and the next gpt_sync returns
                                  GPT_E_INVAL. Nothing reads outside the tables either
                                  way: without the flag an id in [vocab_size,
                                  padded_vocab) is an ordinary padded row and an id
                                  outside [0, padded_vocab) yields NaN rows and a NaN
                                  loss (GPT_E_NONFINITE at the step). One extra launch
                                  of M threads per call.                               */
#define GPT_PREC_BF16 1        /* GEMM/attention operands bf16, everything else fp32 */

typedef struct gpt_model gpt_model;

typedef struct gpt_config {
  int32_t vocab_size;    /* ids in tokens/targets are < vocab_size                  */
  int32_t padded_vocab;  /* rows of wte and softmax width, >= vocab_size            */
  int32_t n_layer;
  int32_t n_head;
  int32_t n_embd;        /* multiple of n_head; head_dim = n_embd / n_head <= 64    */
  int32_t block_size;    /* maximum T (rows of wpe)                                 */
  int32_t batch;         /* maximum micro-batch B per gpt_forward_loss call         */
  int32_t grad_accum;    /* A: backward scales the micro-batch mean loss by 1/A     */
  int32_t precision;     /* GPT_PREC_FP32 or GPT_PREC_BF16                          */
  float   dropout;       /* p in [0, 1): see gpt_set_dropout_seed                   */
  uint32_t flags;        /* GPT_F_KV_CACHE | GPT_F_MICROGPT | GPT_F_DEBUG_CHECKS    */
  int32_t lora_rank;     /* r in [0, 64]; r > 0 adds low-rank adapters (fine-tuning
                            article, LoRA section) to the q and v projections of
                            every block: tensors h<l>.lora_q.A [r, n_embd],
                            h<l>.lora_q.B [n_embd, r] and the same for v, after all
                            base tensors; q = a W0_q^T + b_q + (alpha / r) (a A^T) B^T.
                            Then only the adapters train: gpt_backward forms their
                            gradients alone (the gradients of every other tensor are
                            left undefined: that part of the array is scratch), and
                            gpt_adamw_step's norm, clip and update cover them alone.
                            The base weights stay as loaded; the GEMMs read the
                            merged W0 + (alpha / r) B A, rebuilt by gpt_init_state
                            and after every update. 0: no adapters.               */
  float   lora_alpha;    /* the branch scale is lora_alpha / lora_rank (finite,
                            nonzero when lora_rank > 0; ignored otherwise)         */
} gpt_config;

typedef struct gpt_sizes {
  size_t n_params;         /* scalars of every tensor, adapters included (no gaps)  */
  size_t n_flat;           /* elements of the flat param/grad/m/v arrays            */
  size_t param_bytes;      /* fp32 master weights                                    */
  size_t grad_bytes;       /* fp32 gradients                                         */
  size_t m_bytes, v_bytes; /* fp32 Adam moments                                      */
  size_t shadow_bytes;     /* bf16 copies of the weights (0 in fp32 mode)            */
  size_t activation_bytes; /* saved forward activations                              */
  size_t workspace_bytes;  /* backward scratch, reductions, device state             */
} gpt_sizes;

typedef struct gpt_tensor_info {
  char    name[48];        /* e.g. "wte", "h3.fc.w", "lnf.b"                         */
  size_t  offset;          /* element offset in the flat arrays                      */
  int32_t ndim;            /* 1 or 2                                                 */
  int64_t shape[2];        /* [rows, cols] for 2-D, [n, 1] for 1-D                   */
  int32_t decay;           /* 1 if weight decay applies                              */
} gpt_tensor_info;

typedef struct gpt_buffers {
  void* params;       /* fp32 [n_flat]                        read/write            */
  void* grads;        /* fp32 [n_flat]                        written by backward   */
  void* m;            /* fp32 [n_flat]                        Adam first moment     */
  void* v;            /* fp32 [n_flat]                        Adam second moment    */
  void* shadow;       /* bf16 [2 * n_flat] (NULL in fp32 mode): the weights as GEMM
                         input, then at offset n_flat each 2-D weight transposed
                         ([in, out] at the tensor's own offset)                    */
  void* activations;  /* activation_bytes, 256-byte aligned                          */
  void* workspace;    /* workspace_bytes, 256-byte aligned                           */
} gpt_buffers;

/* Validates the configuration and plans every layout. Touches no GPU.
 * On failure *out is NULL and gpt_last_error(NULL) holds the reason. */
int gpt_create(const gpt_config* cfg, gpt_model** out);
void gpt_destroy(gpt_model* h);

/* Thread-local message for the last failed call (h may be NULL for gpt_create). */
const char* gpt_last_error(const gpt_model* h);

int gpt_get_sizes(const gpt_model* h, gpt_sizes* out);
int gpt_num_tensors(const gpt_model* h);
int gpt_tensor_info_at(const gpt_model* h, int i, gpt_tensor_info* out);

/* Binds caller-owned device buffers (see gpt_buffers) and the HIP stream
 * (hipStream_t, NULL = default stream). Buffers must stay alive and unmoved
 * until gpt_destroy or the next gpt_bind. */
int gpt_bind(gpt_model* h, const gpt_buffers* bufs, void* hip_stream);

/* Call after writing weights into `params`: refreshes the bf16 shadow (and,
 * with LoRA adapters, the merged qkv weights W0 + (alpha / r) B A), zeroes
 * gradients, both moments and the step counter. */
int gpt_init_state(gpt_model* h);

/* Call after writing new weights into `params` mid-training (a host load of a
 * checkpoint's weights, a manual edit): rebuilds what is derived from them, the
 * bf16 shadow and its transposed half and, with LoRA adapters, the merged qkv
 * weights W0 + (alpha / r) B A, and nothing else. Gradients, both Adam moments
 * and the step counter are left as they are (gpt_init_state resets them). A
 * pending forward is invalidated: its saved activations belong to the old
 * weights, so gpt_backward returns GPT_E_STATE until the next gpt_forward_loss.
 * GPT_E_STATE if no buffers are bound. */
int gpt_params_loaded(gpt_model* h);

/* Forward of one micro-batch and the loss.
 * d_tokens, d_targets: int32 [B, T] row-major on the device, ids in
 * [0, vocab_size) (checked on the device only with GPT_F_DEBUG_CHECKS);
 * 1 <= B <= batch, 1 <= T <= block_size. The tokens are
 * copied, so the caller may reuse them after the call returns.
 * d_loss (nullable): receives the fp32 mean over the B*T positions of
 * -log softmax(logits)[target]. The loss gradient is formed in the same pass
 * and kept for gpt_backward. */
int gpt_forward_loss(gpt_model* h, const int32_t* d_tokens, const int32_t* d_targets,
                     int32_t B, int32_t T, float* d_loss);

/* Dropout (config.dropout = p > 0) in gpt_forward_loss and the backward that
 * follows it; gpt_forward_logits never drops. Inverted dropout at four kinds of
 * site: the embedding output (site 0) and, in layer l, the attention
 * probabilities (3l+1), the attention branch output before its residual add
 * (3l+2) and the MLP branch output before its add (3l+3). Element (row, col)
 * of a site's tensor takes word col % 4 of Philox4x32-10 (Salmon, Moraes, Dror
 * and Shaw, SC 2011) at counter (col / 4, row, site, n) under the key
 * (seed low 32 bits, seed high 32 bits); it is dropped when that word is below
 * floor(p * 2^32) and otherwise multiplied by 1 / (1 - p) rounded to float.
 * Rows and columns: token row b*T + t by channel for the embedding and the
 * branch outputs, row (b*n_head + h)*T + i by key j for the probabilities of
 * query i, with T the call's sequence length. n is the forward counter: each
 * gpt_forward_loss uses the current value and then adds one (with or without
 * dropout). This call sets the seed and the next forward's counter; both start
 * at 0. Host-only, no GPU work; returns GPT_E_INVAL for a NULL handle. */
int gpt_set_dropout_seed(gpt_model* h, uint64_t seed, uint32_t counter);

/* Forward only, up to the logits, copied as fp32 [B, T, padded_vocab] into
 * d_logits. Does not disturb a pending backward's saved state only if no
 * forward_loss is pending; it invalidates it otherwise. */
int gpt_forward_logits(gpt_model* h, const int32_t* d_tokens, int32_t B, int32_t T,
                       float* d_logits);

/* Generation with a key/value cache ("GPT training and inference from scratch
 * with nanoGPT" (adg.csdn.net), section 4: sampling with temperature and top_k;
 * "Building microGPT from scratch", single-GPU inference section: the cache
 * grows by one position per generated token). Needs GPT_F_KV_CACHE at create;
 * the cache holds every layer's keys and values for batch x block_size
 * positions in the workspace. No dropout. A pending backward is invalidated.
 *
 * gpt_prefill: forward over prompts d_tokens int32 [B, T] (device); keeps the
 * keys and values of positions 0..T-1 and writes the fp32 logits of position
 * T-1 of every sequence to d_logits [B, padded_vocab]. Resets the cache.
 * gpt_decode: one token per sequence, d_tokens int32 [B] with the B of the
 * last prefill, at the next position; appends its keys and values and writes
 * fp32 logits [B, padded_vocab]. The logits equal the last row of a full
 * forward over the sequence so far (up to rounding). GPT_E_STATE without a
 * prefill, GPT_E_SEQ_TOO_LONG once block_size positions are cached. The ids are
 * read and the logits written by the step's kernels, in stream order (d_tokens
 * may be rewritten once the call's work has run). A call whose d_tokens,
 * d_logits and batch repeat the previous call's replays a graph of the step,
 * recorded by the library at the first repeat (the position is kept on the
 * device); any other call launches the kernels one by one. The results are the
 * same either way. The graph holds the bound buffers' addresses: gpt_bind drops it.
 * gpt_sample: one token per row of fp32 logits [B, padded_vocab] into
 * d_tokens_out int32 [B]. temperature <= 0: the argmax, lowest index on ties
 * (d_uniform may be NULL). Otherwise the candidates are the logits >= the
 * top_k-th largest (every column when top_k <= 0 or >= padded_vocab; ties at
 * the cut stay in), weighted by exp((z - max z) / temperature), and the token
 * is the first index whose running weight, summed in index order, exceeds
 * d_uniform[b] (in [0, 1)) times the total. */
int gpt_prefill(gpt_model* h, const int32_t* d_tokens, int32_t B, int32_t T, float* d_logits);
int gpt_decode(gpt_model* h, const int32_t* d_tokens, float* d_logits);
int gpt_sample(gpt_model* h, const float* d_logits, int32_t B, float temperature, int32_t top_k,
               const float* d_uniform, int32_t* d_tokens_out);

/* Backward of the last gpt_forward_loss. Adds d(loss / grad_accum) into the
 * gradients; the first backward after gpt_init_state, gpt_zero_grad or
 * gpt_adamw_step overwrites them instead. */
int gpt_backward(gpt_model* h);

/* Makes the next backward overwrite the gradients (no kernel runs). */
int gpt_zero_grad(gpt_model* h);

/* Global L2 norm n of all gradients; coef = min(1, clip / (n + 1e-6)) if
 * clip > 0 else 1; t += 1; for every element: g' = coef g,
 * m = beta1 m + (1 - beta1) g', v = beta2 v + (1 - beta2) g'^2,
 * p = p (1 - lr wd) [decayed tensors only] - lr (m / (1 - beta1^t)) /
 * (sqrt(v / (1 - beta2^t)) + eps); then refreshes both bf16 shadows. With
 * LoRA adapters (config.lora_rank > 0) "all" is the adapters alone, and the
 * merged qkv weights are rebuilt from the updated A and B.
 * d_grad_norm (nullable) receives n (before clipping). If n is not finite the
 * update is skipped on the device, t is not advanced, and the next gpt_sync
 * returns GPT_E_NONFINITE. */
int gpt_adamw_step(gpt_model* h, float lr, float beta1, float beta2, float eps,
                   float weight_decay, float clip, float* d_grad_norm);

/* gpt_adamw_step for callers that cannot allocate device memory or hand over
 * scratch (code under HIP graph capture, tight serving or training loops,
 * harnesses that forbid hipMalloc): the same update, the same kernels and a
 * bitwise identical result, but the gradient norm's per-block partial sums live
 * in a file-scope device array of the library (4 KB per GPU, kept until the
 * process ends) instead of the bound workspace. The partials do not grow with
 * the model: every size gpt_create accepts fits; a build whose partial count
 * exceeded the array would return GPT_E_UNSUPPORTED. The array is looked up once
 * per device on the first call there. Calls nothing that allocates. Every call on
 * one GPU shares that GPU's array, which keeps the last call's partials (each
 * call overwrites all of them before reading): calls that overlap on one GPU
 * (several streams or threads) race and must be serialized by the caller. */
int gpt_adamw_step_noalloc(gpt_model* h, float lr, float beta1, float beta2, float eps,
                           float weight_decay, float clip, float* d_grad_norm);

/* Waits for the stream, then reports a pending sticky error, a device-side
 * out-of-range id flag (GPT_E_INVAL, GPT_F_DEBUG_CHECKS only), a device-side
 * non-finite flag (GPT_E_NONFINITE) or GPT_OK, and clears them. */
int gpt_sync(gpt_model* h);

/* Synchronous: the device step counter t. */
int gpt_get_step(gpt_model* h, int64_t* t);

/* Synchronous copy of a saved activation into caller memory on the device.
 * what: "x" (fp32 [M, d] residual input of block `layer`, layer == n_layer
 * is the input of the final LayerNorm), "qkv" ([M, 3d], operand type),
 * "attn" ([M, d], operand type), "lse" (fp32 [B, H, T]), "u" (what the MLP
 * backward reads: GELU'(u) of the GELU block's pre-activation u, or u itself for
 * the ReLU block; [M, 4d], operand type), "h" (the activation's output, [M, 4d],
 * operand type). bytes
 * must equal the size of the request. */
int gpt_debug_copy(gpt_model* h, const char* what, int32_t layer, void* d_dst, size_t bytes);

/* Kernel timing hook used by benchmarks: while enabled, every launch of the
 * named kernel family ("lm_head_fwd", "gemm", "attn_fwd", "attn_bwd",
 * "xent", "adamw") is bracketed by HIP events on the bound stream.
 * gpt_timer_read synchronizes and returns the summed milliseconds and the
 * number of launches since enable. */
int gpt_timer_enable(gpt_model* h, const char* family);
int gpt_timer_disable(gpt_model* h);
int gpt_timer_read(gpt_model* h, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* GPT_MI355X_H */
