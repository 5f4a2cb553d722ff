// C ABI of the GPT training step (see include/gpt.h): configuration checks,
// the flat parameter layout, the activation and workspace plans, and the
// launch sequences of forward, backward and AdamW on the bound HIP stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "../../include/gpt.h"
#include "kernels.h"

using namespace gpt;

namespace {

thread_local std::string g_create_error;

constexpr size_t ALIGN_ELEMS = 64;     // tensor offsets in the flat arrays
constexpr size_t ALIGN_BYTES = 256;    // arena slices

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Tensor {
  std::string name;
  size_t offset;
  int ndim;
  int64_t rows, cols;
  int decay;
  size_t numel() const { return (size_t)rows * (size_t)cols; }
};

struct Slice {
  size_t off = 0, bytes = 0;
};

struct Planner {
  size_t total = 0;
  Slice take(size_t bytes) {
    Slice s;
    s.off = total;
    s.bytes = bytes;
    total = round_up(total + bytes, ALIGN_BYTES);
    return s;
  }
};

struct LayerAct {
  Slice x, xmid, ln1, ln1_mean, ln1_rstd, qkv, att, lse, ln2, ln2_mean, ln2_rstd, u, h;
};

struct Timer {
  bool on = false;
  std::string family;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> events;
  size_t used = 0;
};

}  // namespace

enum { RED_LN = 0, RED_QKV = 1, RED_FC = 2 };   // rows_kind of the deferred reductions

struct gpt_model {
  gpt_config cfg;
  bool bf16;
  int d, H, hd, L, V, Vp, Tmax, Bmax, A;
  int64_t ldz;
  size_t op_size;  // bytes per operand element
  std::vector<Tensor> tensors;
  size_t n_params = 0, n_flat = 0, n_decay = 0;
  // activations
  std::vector<LayerAct> layers;
  Slice x_final, lnf, lnf_mean, lnf_rstd, logits, row_loss, tokens, targets;
  size_t act_bytes = 0;
  // workspace
  Slice dres, dln, du, dO, dqkv, attnD, red, emb_keys, emb_piece, norm_part, opt, split, ttable, rtable;
  // bf16: operand copies of the residual-stream gradients, d x_l (l = 0..L) and
  // d xmid_l, and per-layer du and dqkv, kept for the weight gradients that run
  // together at the end of the backward
  Slice rx, rm, wtable;
  // fp32 mode with dropout: the masked copy of a residual-stream gradient that the
  // branch below reads as its GEMM operand
  Slice dxm;
  // GPT_F_KV_CACHE: keys and values of every layer, [B_max * T_max, 2d] operand type each
  Slice kv;
  size_t kv_stride = 0;   // bytes per layer
  Slice kvpos;            // the next decode position (int32), on the device: the decode kernels read it
  size_t layer_stride_du = 0, layer_stride_dqkv = 0, resid_stride = 0;   // bytes
  std::vector<WgradProblem> wprobs;   // host copy of the grouped weight-gradient table
  int wtiles = 0;
  bool wgroup = false;                // every weight gradient can join the grouped launch
  size_t split_floats = 0;
  std::vector<TransposeEntry> tentries;   // 2-D weights whose transposed shadow the dgrads read
  int64_t ttiles = 0;
  // bias and LayerNorm-parameter gradients: partial column sums written during the
  // backward, reduced by one launch at its end
  std::vector<RedJob> rjobs;
  std::map<std::string, int64_t> rpart;   // destination tensor -> float offset of its partials in `red`
  int rblocks = 0;
  bool tables_ready = false;              // device copies of the two tables are in this workspace
  size_t ws_bytes = 0;
  // binding
  gpt_buffers buf{};
  bool bound = false;
  hipStream_t stream = nullptr;
  // dropout: key, threshold and scale (drop.call unused), the next forward's
  // counter, and the masks of the forward that the pending backward belongs to
  DropArgs drop{};
  uint32_t drop_call = 0;
  DropArgs drop_fwd{};
  int kv_len = 0, kv_B = 0;   // cached positions per sequence and sequences, after gpt_prefill
  // the decode step recorded as a graph, with the pointers and batch it was recorded for
  struct {
    hipStream_t cap = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    const int32_t* tok = nullptr;
    const float* out = nullptr;
    int B = 0;
    bool off = false;   // the graph API failed once: direct launches from then on
  } dg;
  // GPT_F_MICROGPT: weightless RMSNorm, ReLU, no biases, an lm_head of its own
  bool micro = false;
  std::string head = "wte";   // the tensor the logits are taken against
  Slice zbias;                // zeros standing in for the absent biases (4d floats)
  // LoRA adapters on the q and v rows of every qkv weight: rank, branch scale
  // alpha / r, first flat element of the adapters (they end the flat arrays), one
  // job per adapted block, and in fp32 mode the merged qkv weights [L][3d][d]
  int lora_r = 0;
  float lora_s = 0.f;
  size_t lora_off = 0;
  std::vector<LoraJob> ljobs;
  Slice ltable, weff;
  // state
  bool grads_fresh = true;
  bool fwd_pending = false;
  int cur_B = 0, cur_T = 0;
  int sticky = GPT_OK;
  std::string err;
  Timer timer;
};

// ----------------------------------------------------------------------------- helpers
namespace {

int fail(gpt_model* h, int code, const std::string& msg) {
  if (h) {
    if (h->sticky == GPT_OK) h->sticky = code;
    h->err = msg;
  }
  g_create_error = msg;
  return code;
}

int hip_check(gpt_model* h, hipError_t e, const char* what) {
  if (e == hipSuccess) return GPT_OK;
  return fail(h, GPT_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

const Tensor* find(const gpt_model* h, const std::string& name) {
  for (const auto& t : h->tensors)
    if (t.name == name) return &t;
  return nullptr;
}

float* P(gpt_model* h, const std::string& name) { return (float*)h->buf.params + find(h, name)->offset; }
float* G(gpt_model* h, const std::string& name) { return (float*)h->buf.grads + find(h, name)->offset; }
// Weight as a GEMM operand: the bf16 shadow in bf16 mode, the fp32 master otherwise.
// With adapters, the qkv weights are the merged W0 + s B A: written into the shadow
// in bf16 mode, kept in the workspace in fp32 mode.
const void* Wop(gpt_model* h, const std::string& name) {
  const Tensor* t = find(h, name);
  if (h->bf16) return (const uint16_t*)h->buf.shadow + t->offset;
  const size_t n = name.size();
  if (h->lora_r && n > 7 && name.compare(n - 7, 7, ".attn.w") == 0) {
    const int l = std::atoi(name.c_str() + 1);   // "h<l>.attn.w"
    return (const float*)((char*)h->buf.workspace + h->weff.off) + (size_t)l * 3 * h->d * h->d;
  }
  return (const float*)h->buf.params + t->offset;
}

// Transposed weight ([in, out]) for the input-gradient GEMMs; bf16 mode only.
const void* WopT(gpt_model* h, const std::string& name) {
  return (const uint16_t*)h->buf.shadow + h->n_flat + find(h, name)->offset;
}

template <typename X = void>
X* act(gpt_model* h, const Slice& s) { return (X*)((char*)h->buf.activations + s.off); }
template <typename X = void>
X* ws(gpt_model* h, const Slice& s) { return (X*)((char*)h->buf.workspace + s.off); }

// Launch wrapper: brackets the call with events when the timer is on for `family`.
template <typename F>
int run(gpt_model* h, const char* family, const char* what, F&& f) {
  Timer& tm = h->timer;
  const bool timed = tm.on && (tm.family == family || (tm.family == "gemm" && std::strncmp(family, "gemm", 4) == 0) ||
                               (tm.family == "gemm" && std::strcmp(family, "lm_head_fwd") == 0));
  if (timed) {
    if (tm.used == tm.events.size()) {
      hipEvent_t a, b;
      if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess)
        return fail(h, GPT_E_HIP, "hipEventCreate failed");
      tm.events.push_back({a, b});
    }
    hipEventRecord(tm.events[tm.used].first, h->stream);
  }
  hipError_t e = f();
  if (timed) {
    hipEventRecord(tm.events[tm.used].second, h->stream);
    tm.used++;
  }
  return hip_check(h, e, what);
}

// GEMM launch with the shared split / stream-K workspace attached.
hipError_t gemm(gpt_model* h, GemmDesc g, bool bf) {
  g.split_ws = (float*)((char*)h->buf.workspace + h->split.off);
  g.split_ws_floats = h->split_floats;
  return launch_gemm(g, bf, h->stream);
}

hipError_t transpose_shadow(gpt_model* h) {
  return launch_transpose_bf16(h->buf.shadow, (uint16_t*)h->buf.shadow + h->n_flat,
                               (const TransposeEntry*)((char*)h->buf.workspace + h->ttable.off), (int)h->tentries.size(),
                               h->ttiles, h->stream);
}

#define RUN(fam, what, call)                                     \
  do {                                                           \
    int rc__ = run(h, fam, what, [&]() { return (call); });      \
    if (rc__ != GPT_OK) return rc__;                             \
  } while (0)

GemmDesc gemm_desc(const void* A, int64_t lda, bool a_kc, const void* B, int64_t ldb, bool b_kc, void* C,
                   int64_t ldc, int M, int N, int K, int epi) {
  GemmDesc d;
  std::memset(&d, 0, sizeof(d));
  d.split_ws = nullptr;
  d.split_ws_floats = 0;
  d.A = A; d.lda = lda; d.a_kc = a_kc;
  d.B = B; d.ldb = ldb; d.b_kc = b_kc;
  d.C = C; d.ldc = ldc; d.M = M; d.N = N; d.K = K; d.epi = epi;
  return d;
}

int check_usable(gpt_model* h) {
  if (!h) return GPT_E_INVAL;
  if (h->sticky != GPT_OK) return h->sticky;
  if (!h->bound) return fail(h, GPT_E_STATE, "buffers are not bound (call gpt_bind)");
  return GPT_OK;
}

void plan(gpt_model* h) {
  const int d = h->d, L = h->L, Vp = h->Vp;
  // ---- parameters: 2-D tensors first (decayed), then 1-D tensors
  size_t off = 0;
  auto add = [&](const std::string& name, int64_t rows, int64_t cols, int ndim, int decay) {
    Tensor t{name, off, ndim, rows, cols, decay};
    h->tensors.push_back(t);
    h->n_params += t.numel();
    off = round_up(off + t.numel(), ALIGN_ELEMS);
  };
  add("wte", Vp, d, 2, 1);
  add("wpe", h->Tmax, d, 2, 1);
  for (int l = 0; l < L; l++) {
    const std::string p = "h" + std::to_string(l) + ".";
    add(p + "attn.w", 3 * d, d, 2, 1);
    add(p + "proj.w", d, d, 2, 1);
    add(p + "fc.w", 4 * d, d, 2, 1);
    add(p + "fcproj.w", d, 4 * d, 2, 1);
  }
  if (h->micro) add("lm_head", Vp, d, 2, 1);
  h->n_decay = off;
  for (int l = 0; l < L && !h->micro; l++) {
    const std::string p = "h" + std::to_string(l) + ".";
    add(p + "ln1.g", d, 1, 1, 0);
    add(p + "ln1.b", d, 1, 1, 0);
    add(p + "attn.b", 3 * d, 1, 1, 0);
    add(p + "proj.b", d, 1, 1, 0);
    add(p + "ln2.g", d, 1, 1, 0);
    add(p + "ln2.b", d, 1, 1, 0);
    add(p + "fc.b", 4 * d, 1, 1, 0);
    add(p + "fcproj.b", d, 1, 1, 0);
  }
  if (!h->micro) {
    add("lnf.g", d, 1, 1, 0);
    add("lnf.b", d, 1, 1, 0);
  }
  // the adapters end the flat arrays, so the optimizer's range is one contiguous run
  h->lora_off = off;
  for (int l = 0; l < L && h->lora_r; l++) {
    const std::string p = "h" + std::to_string(l) + ".";
    for (const char* t : {"q", "v"}) {
      add(p + "lora_" + t + ".A", h->lora_r, d, 2, 1);
      add(p + "lora_" + t + ".B", d, h->lora_r, 2, 1);
    }
  }
  h->n_flat = round_up(off, 256);

  // ---- activations for the largest micro-batch
  const size_t M = (size_t)h->Bmax * h->Tmax;
  const size_t ob = h->op_size, fb = 4;
  const size_t bht = (size_t)h->Bmax * h->H * h->Tmax;
  Planner a;
  h->layers.resize(L);
  for (int l = 0; l < L; l++) {
    LayerAct& la = h->layers[l];
    la.x = a.take(M * d * fb);
    la.xmid = a.take(M * d * fb);
    la.ln1 = a.take(M * d * ob);
    la.ln1_mean = a.take(M * fb);
    la.ln1_rstd = a.take(M * fb);
    la.qkv = a.take(M * 3 * d * ob);
    la.att = a.take(M * d * ob);
    la.lse = a.take(bht * fb);
    la.ln2 = a.take(M * d * ob);
    la.ln2_mean = a.take(M * fb);
    la.ln2_rstd = a.take(M * fb);
    la.u = a.take(M * 4 * d * ob);   // GELU'(u) (GELU block) or u (ReLU block), for the MLP backward
    la.h = a.take(M * 4 * d * ob);
  }
  h->x_final = a.take(M * d * fb);
  h->lnf = a.take(M * d * ob);
  h->lnf_mean = a.take(M * fb);
  h->lnf_rstd = a.take(M * fb);
  h->ldz = (int64_t)round_up((size_t)Vp, 64);
  h->logits = a.take(M * (size_t)h->ldz * ob);
  h->row_loss = a.take(M * fb);
  h->tokens = a.take(M * 4);
  h->targets = a.take(M * 4);
  h->act_bytes = a.total;

  // ---- workspace
  Planner w;
  h->dres = w.take(M * d * fb);

  h->dln = w.take(M * d * ob);   // the LayerNorm backward's dy, in the operand type
  const size_t per_layer = h->bf16 ? (size_t)L : 1;
  h->layer_stride_du = h->bf16 ? M * 4 * d * ob : 0;
  h->layer_stride_dqkv = h->bf16 ? M * 3 * d * ob : 0;
  h->resid_stride = M * d * ob;
  h->du = w.take(per_layer * M * 4 * d * ob);
  h->rx = w.take(h->bf16 ? (L + 1) * M * d * ob : 0);
  h->rm = w.take(h->bf16 ? L * M * d * ob : 0);
  h->dO = w.take(M * d * ob);
  h->dqkv = w.take(per_layer * M * 3 * d * ob);
  h->dxm = w.take(!h->bf16 && h->cfg.dropout > 0.f ? M * d * fb : 0);
  h->kv_stride = (h->cfg.flags & GPT_F_KV_CACHE) ? M * 2 * d * ob : 0;
  h->kv = w.take((size_t)L * h->kv_stride);
  h->kvpos = w.take((h->cfg.flags & GPT_F_KV_CACHE) ? 4 : 0);
  h->attnD = w.take(bht * fb);
  const size_t ln_blk = (M + LN_BWD_ROWS - 1) / LN_BWD_ROWS;
  const size_t cs_blk = (M + COLSUM_ROWS - 1) / COLSUM_ROWS;
  size_t red_floats = 0;
  auto red_job = [&](const std::string& dst, int kind) {
    const Tensor* t = find(h, dst);
    RedJob j{(int64_t)red_floats, (int64_t)t->offset, (int32_t)t->numel(), kind, h->rblocks, 0};
    h->rjobs.push_back(j);
    h->rpart[dst] = j.part;
    const size_t rows = kind == RED_LN ? ln_blk
                        : kind == RED_QKV ? std::max(cs_blk, (size_t)h->Bmax * ((h->Tmax + 63) / 64))
                                          : cs_blk;
    red_floats += rows * t->numel();
    h->rblocks += (int)((t->numel() + RED_COLS - 1) / RED_COLS);
  };
  // kinds: RED_LN LayerNorm backward partials, RED_QKV and RED_FC the qkv and fc
  // bias column sums (from the GEMM epilogue or a column-sum pass)
  if (!h->micro) {   // the microGPT block has no bias or norm parameter
    red_job("lnf.g", RED_LN);
    red_job("lnf.b", RED_LN);
    for (int l = 0; l < h->L; l++) {
      const std::string p = "h" + std::to_string(l) + ".";
      for (const char* n : {"ln1.g", "ln1.b", "proj.b", "ln2.g", "ln2.b", "fcproj.b"}) red_job(p + n, RED_LN);
      red_job(p + "fc.b", RED_FC);
      red_job(p + "attn.b", RED_QKV);
    }
  }
  h->red = w.take(red_floats * fb);
  h->rtable = w.take(h->rjobs.size() * sizeof(RedJob));
  h->emb_keys = w.take((size_t)embed_bwd_sort_size((int)M) * 4);
  h->emb_piece = w.take(M * d * fb);
  h->norm_part = w.take(NORM_BLOCKS * fb);
  // split-K partials, or stream-K partial tiles of 256 x 256 (at most about
  // CUs + 2 * tiles of them for the < 512-tile GEMMs that use stream-K)
  h->split_floats = 16 * (size_t)d * d + 4096;
  if (M >= 256 && d >= 256) h->split_floats = std::max(h->split_floats, (size_t)1664 * 256 * 256);
  if (h->bf16) h->split_floats = std::max(h->split_floats, wgrad_group_ws_floats());
  h->split = w.take(h->split_floats * fb);
  for (const Tensor& t : h->tensors) {
    if (t.ndim != 2 || t.name == "wpe" || t.name.find(".lora_") != std::string::npos) continue;
    TransposeEntry e{(int64_t)t.offset, t.rows, t.cols, h->ttiles};
    h->tentries.push_back(e);
    h->ttiles += ((t.rows + 63) / 64) * ((t.cols + 63) / 64);
  }
  h->ttable = w.take(h->tentries.size() * sizeof(TransposeEntry));
  h->opt = w.take(sizeof(OptState));
  h->zbias = w.take(4 * (size_t)d * fb);
  h->weff = w.take(h->lora_r && !h->bf16 ? (size_t)L * 3 * d * d * fb : 0);
  h->ltable = w.take(h->lora_r ? 2 * (size_t)L * sizeof(LoraJob) : 0);
  // the weight gradients as one grouped launch: wte (tied lm_head), then per layer
  // fcproj.w, fc.w, proj.w, attn.w; operands are [tokens, features] (m-contiguous)
  if (h->bf16) {
    const int64_t Vp = h->Vp, D = d;
    bool ok = wgrad_group_ok(h->Vp, d, h->ldz, D, D) && h->split_floats >= wgrad_group_ws_floats();
    ok = ok && wgrad_group_ok(d, 4 * d, D, 4 * D, 4 * D) && wgrad_group_ok(4 * d, d, 4 * D, D, D);
    ok = ok && wgrad_group_ok(d, d, D, D, D) && wgrad_group_ok(3 * d, d, 3 * D, D, D);
    // with adapters: the q and v row blocks of each qkv weight gradient only
    if (h->lora_r)
      ok = wgrad_group_ok(d, d, 3 * D, D, D) && d % 8 == 0 && h->split_floats >= wgrad_group_ws_floats();
    h->wgroup = ok;
    (void)Vp;
    h->wtable = w.take((4 * (size_t)L + 1) * sizeof(WgradProblem));
  }
  h->ws_bytes = w.total;
}

float* red_part(gpt_model* h, const std::string& dst) {
  return (float*)((char*)h->buf.workspace + h->red.off) + h->rpart.at(dst);
}

// Partial column sums of X into the partials of bias `dst` (reduced at the end of the backward).
int colsum(gpt_model* h, const void* X, bool bf16_in, int64_t ldx, int M, int N, const std::string& dst) {
  RUN("colsum", "colsum_partial", launch_colsum_partial(X, bf16_in, ldx, M, N, red_part(h, dst), h->stream));
  return GPT_OK;
}

// LayerNorm backward into dres (in place when dres is given); writes the partial
// column sums of the gain and shift gradients and, when `resid_bias` names a
// tensor, of the incoming residual gradient (the bias gradient of that projection).
// With dropout, site_in names the mask of the branch whose output was added into
// this residual (its bias gradient sums the masked dres) and site_out the mask that
// the operand copy dx_op carries (-1: none).
int ln_bwd(gpt_model* h, const void* dy, const float* x, const float* mean, const float* rstd,
           const std::string& gname, const std::string& bname, const float* dres, const char* resid_bias, void* dx_op,
           int M, int site_in = -1, int site_out = -1) {
  // the microGPT block: weightless RMSNorm (g = NULL), and no bias to take column sums for
  float* pr = resid_bias && !h->micro ? red_part(h, resid_bias) : nullptr;
  const float* g = h->micro ? nullptr : P(h, gname);
  float* pg = h->micro ? nullptr : red_part(h, gname);
  float* pb = h->micro ? nullptr : red_part(h, bname);
  RUN("layernorm", "layernorm_bwd",
      launch_layernorm_bwd(dy, x, mean, rstd, g, dres, ws<float>(h, h->dres), dx_op, h->bf16, pg, pb, pr, M, h->d,
                           h->drop_fwd, site_in, site_out, h->stream));
  return GPT_OK;
}

// The block's norm in front of a GEMM: LayerNorm with gain and shift `name`.g / .b,
// or the microGPT block's weightless RMSNorm.
int norm_fwd(gpt_model* h, const float* x, const std::string& name, void* y, float* mean, float* rstd, int M) {
  if (h->micro)
    RUN("layernorm", "rms_fwd", launch_rmsnorm_fwd(x, y, h->bf16, mean, rstd, M, h->d, h->stream));
  else
    RUN("layernorm", "ln_fwd",
        launch_layernorm_fwd(x, P(h, name + ".g"), P(h, name + ".b"), y, h->bf16, mean, rstd, M, h->d, h->stream));
  return GPT_OK;
}
// A linear layer's bias, or zeros for the microGPT block.
const float* bias_of(gpt_model* h, const std::string& name) { return h->micro ? ws<float>(h, h->zbias) : P(h, name); }

// bf16 operand slots of the backward (see gpt_model)
void* rx_slot(gpt_model* h, int l) { return (char*)ws(h, h->rx) + (size_t)l * h->resid_stride; }
void* rm_slot(gpt_model* h, int l) { return (char*)ws(h, h->rm) + (size_t)l * h->resid_stride; }
void* du_slot(gpt_model* h, int l) { return (char*)ws(h, h->du) + (size_t)l * h->layer_stride_du; }
void* dqkv_slot(gpt_model* h, int l) { return (char*)ws(h, h->dqkv) + (size_t)l * h->layer_stride_dqkv; }
void* kv_slot(gpt_model* h, int l) { return (char*)ws(h, h->kv) + (size_t)l * h->kv_stride; }

// The grouped weight-gradient problems with this binding's addresses.
void build_wgrad_table(gpt_model* h) {
  h->wprobs.clear();
  h->wtiles = 0;
  const int d = h->d;
  auto add = [&](const void* A, int64_t lda, const void* B, int64_t ldb, float* C, int Mo, int No) {
    WgradProblem q;
    q.A = A; q.lda = lda; q.B = B; q.ldb = ldb; q.C = C; q.ldc = No;
    q.M = Mo; q.N = No;
    q.tiles_m = (Mo + 255) / 256; q.tiles_n = (No + 255) / 256;
    q.first_tile = h->wtiles;
    q.c_vec = (No % 8 == 0) ? 1 : 0;
    h->wtiles += wgrad_group_tiles(Mo, No);
    h->wprobs.push_back(q);
  };
  if (h->lora_r) {
    // adapters: dW of the q and v row blocks, the input of the adapter gradients
    for (int l = h->L - 1; l >= 0; l--) {
      const LayerAct& la = h->layers[l];
      const std::string w = "h" + std::to_string(l) + ".attn.w";
      add(dqkv_slot(h, l), 3 * d, act(h, la.ln1), d, G(h, w), d, d);
      add((char*)dqkv_slot(h, l) + 2 * (size_t)d * h->op_size, 3 * d, act(h, la.ln1), d, G(h, w) + 2 * (size_t)d * d,
          d, d);
    }
    return;
  }
  add(act(h, h->logits), h->ldz, act(h, h->lnf), d, G(h, h->head), h->Vp, d);
  for (int l = h->L - 1; l >= 0; l--) {
    const LayerAct& la = h->layers[l];
    const std::string p = "h" + std::to_string(l) + ".";
    add(rx_slot(h, l + 1), d, act(h, la.h), 4 * d, G(h, p + "fcproj.w"), d, 4 * d);
    add(du_slot(h, l), 4 * d, act(h, la.ln2), d, G(h, p + "fc.w"), 4 * d, d);
    add(rm_slot(h, l), d, act(h, la.att), d, G(h, p + "proj.w"), d, d);
    add(dqkv_slot(h, l), 3 * d, act(h, la.ln1), d, G(h, p + "attn.w"), 3 * d, d);
  }
}

// The adapter jobs with this binding's addresses: layer l's q block, then its v block.
void build_lora_jobs(gpt_model* h) {
  h->ljobs.clear();
  const size_t d = h->d;
  for (int l = 0; l < h->L; l++) {
    const std::string p = "h" + std::to_string(l) + ".";
    const size_t attn = find(h, p + "attn.w")->offset;
    for (int t = 0; t < 2; t++) {
      const std::string a = p + (t ? "lora_v" : "lora_q");
      const size_t row0 = t ? 2 * d : 0;   // first row of the block in the [3d, d] weight
      LoraJob j;
      j.A = P(h, a + ".A");
      j.B = P(h, a + ".B");
      j.W0 = (const float*)h->buf.params + attn + row0 * d;
      j.dW = (const float*)h->buf.grads + attn + row0 * d;
      j.dA = G(h, a + ".A");
      j.dB = G(h, a + ".B");
      j.weff = h->bf16 ? nullptr : (float*)((char*)h->buf.workspace + h->weff.off) + ((size_t)l * 3 * d + row0) * d;
      j.weff_bf16 = h->bf16 ? (void*)((uint16_t*)h->buf.shadow + attn + row0 * d) : nullptr;
      h->ljobs.push_back(j);
    }
  }
}

// Copies the transpose and reduction tables into the bound workspace (once per bind).
int upload_tables(gpt_model* h) {
  if (h->tables_ready) return GPT_OK;
  hipError_t e = hipMemcpyAsync(ws(h, h->rtable), h->rjobs.data(), h->rjobs.size() * sizeof(RedJob),
                                hipMemcpyHostToDevice, h->stream);
  if (e == hipSuccess && h->bf16)
    e = hipMemcpyAsync(ws(h, h->ttable), h->tentries.data(), h->tentries.size() * sizeof(TransposeEntry),
                       hipMemcpyHostToDevice, h->stream);
  if (e == hipSuccess && h->bf16) {
    build_wgrad_table(h);
    e = hipMemcpyAsync(ws(h, h->wtable), h->wprobs.data(), h->wprobs.size() * sizeof(WgradProblem),
                       hipMemcpyHostToDevice, h->stream);
  }
  if (e == hipSuccess && h->lora_r) {
    build_lora_jobs(h);
    e = hipMemcpyAsync(ws(h, h->ltable), h->ljobs.data(), h->ljobs.size() * sizeof(LoraJob), hipMemcpyHostToDevice,
                       h->stream);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
  if (e != hipSuccess) return hip_check(h, e, "upload tables");
  h->tables_ready = true;
  return GPT_OK;
}

// The merged qkv weights W0 + s B A (fp32 workspace copy or bf16 shadow rows).
int lora_merge(gpt_model* h) {
  RUN("lora", "lora_merge",
      launch_lora_merge(ws<LoraJob>(h, h->ltable), 2 * h->L, h->d, h->lora_r, h->lora_s, h->stream));
  return GPT_OK;
}

// Forward up to the logits for B x T tokens already copied into the arena, with
// the dropout masks of `da` (da.on = 0: none).
int forward_to_logits(gpt_model* h, int B, int T, const DropArgs& da) {
  const int d = h->d, M = B * T;
  const bool bf = h->bf16;
  hipStream_t s = h->stream;
  const int32_t* tok = act<int32_t>(h, h->tokens);
  const int resid_epi = da.on ? EPI_BIAS_RESID_DROP : EPI_BIAS_RESID;
  RUN("embed", "embed_fwd",
      launch_embed_fwd(P(h, "wte"), P(h, "wpe"), tok, act<float>(h, h->layers[0].x), M, T, d, h->Vp, da, s));
  for (int l = 0; l < h->L; l++) {
    const LayerAct& la = h->layers[l];
    const std::string p = "h" + std::to_string(l) + ".";
    float* x = act<float>(h, la.x);
    float* xmid = act<float>(h, la.xmid);
    float* xnext = (l + 1 < h->L) ? act<float>(h, h->layers[l + 1].x) : act<float>(h, h->x_final);
    int rc;
    if ((rc = norm_fwd(h, x, p + "ln1", act(h, la.ln1), act<float>(h, la.ln1_mean), act<float>(h, la.ln1_rstd), M)))
      return rc;
    {
      GemmDesc g = gemm_desc(act(h, la.ln1), d, true, Wop(h, p + "attn.w"), d, true, act(h, la.qkv), 3 * d, M,
                             3 * d, d, EPI_BIAS);
      g.bias = bias_of(h, p + "attn.b");
      RUN("gemm_fwd", "qkv_fwd", gemm(h, g, bf));
    }
    RUN("attn_fwd", "attn_fwd",
        launch_attn_fwd(act(h, la.qkv), act(h, la.att), act<float>(h, la.lse), bf, B, T, h->H, h->hd, da,
                        site_attn_prob(l), s));
    {
      GemmDesc g = gemm_desc(act(h, la.att), d, true, Wop(h, p + "proj.w"), d, true, xmid, d, M, d, d, resid_epi);
      g.bias = bias_of(h, p + "proj.b");
      g.resid = x;
      g.ldr = d;
      g.drop = da;
      g.drop_site = site_attn_out(l);
      RUN("gemm_fwd", "proj_fwd", gemm(h, g, bf));
    }
    if ((rc = norm_fwd(h, xmid, p + "ln2", act(h, la.ln2), act<float>(h, la.ln2_mean), act<float>(h, la.ln2_rstd),
                       M)))
      return rc;
    {
      GemmDesc g = gemm_desc(act(h, la.ln2), d, true, Wop(h, p + "fc.w"), d, true, act(h, la.h), 4 * d, M, 4 * d,
                             d, h->micro ? EPI_BIAS_RELU : EPI_BIAS_GELU);
      g.bias = bias_of(h, p + "fc.b");
      g.aux = act(h, la.u);
      g.ldaux = 4 * d;
      RUN("gemm_fwd", "fc_fwd", gemm(h, g, bf));
    }
    {
      GemmDesc g = gemm_desc(act(h, la.h), 4 * d, true, Wop(h, p + "fcproj.w"), 4 * d, true, xnext, d, M, d,
                             4 * d, resid_epi);
      g.bias = bias_of(h, p + "fcproj.b");
      g.resid = xmid;
      g.ldr = d;
      g.drop = da;
      g.drop_site = site_mlp_out(l);
      RUN("gemm_fwd", "fcproj_fwd", gemm(h, g, bf));
    }
  }
  {
    int rc = norm_fwd(h, act<float>(h, h->x_final), "lnf", act(h, h->lnf), act<float>(h, h->lnf_mean),
                      act<float>(h, h->lnf_rstd), M);
    if (rc) return rc;
  }
  {
    GemmDesc g = gemm_desc(act(h, h->lnf), d, true, Wop(h, h->head), d, true, act(h, h->logits), h->ldz, M, h->Vp, d,
                           EPI_STORE);
    RUN("lm_head_fwd", "lm_head_fwd", gemm(h, g, bf));
  }
  return GPT_OK;
}

int copy_ids(gpt_model* h, const int32_t* src, const Slice& dst, int M) {
  return hip_check(h, hipMemcpyAsync(act(h, dst), src, (size_t)M * 4, hipMemcpyDeviceToDevice, h->stream),
                   "copy token ids");
}

// GPT_F_DEBUG_CHECKS: ids of the arena copy checked against [0, vocab_size) before use.
int check_ids(gpt_model* h, const Slice& ids, int n) {
  if (!(h->cfg.flags & GPT_F_DEBUG_CHECKS)) return GPT_OK;
  RUN("check", "check_ids", launch_check_ids(act<int32_t>(h, ids), n, h->V, ws<OptState>(h, h->opt), h->stream));
  return GPT_OK;
}

int check_shape(gpt_model* h, int B, int T) {
  if (B < 1 || T < 1) return fail(h, GPT_E_INVAL, "B and T must be >= 1");
  if (B > h->Bmax || T > h->Tmax)
    return fail(h, GPT_E_SEQ_TOO_LONG, "B " + std::to_string(B) + " x T " + std::to_string(T) +
                                           " exceeds batch " + std::to_string(h->Bmax) + " x block_size " +
                                           std::to_string(h->Tmax));
  return GPT_OK;
}

}  // namespace

// ----------------------------------------------------------------------------- ABI
extern "C" {

const char* gpt_last_error(const gpt_model* h) {
  if (h) return h->err.c_str();
  return g_create_error.c_str();
}

int gpt_create(const gpt_config* cfg, gpt_model** out) {
  if (!out) return fail(nullptr, GPT_E_INVAL, "out is NULL");
  *out = nullptr;
  if (!cfg) return fail(nullptr, GPT_E_INVAL, "cfg is NULL");
  const gpt_config& c = *cfg;
  if (c.vocab_size < 1 || c.padded_vocab < c.vocab_size) return fail(nullptr, GPT_E_INVAL, "need 1 <= vocab_size <= padded_vocab");
  if (c.n_layer < 1 || c.n_head < 1 || c.n_embd < 1 || c.block_size < 1 || c.batch < 1 || c.grad_accum < 1)
    return fail(nullptr, GPT_E_INVAL, "n_layer, n_head, n_embd, block_size, batch and grad_accum must be >= 1");
  if (c.n_embd % c.n_head != 0) return fail(nullptr, GPT_E_INVAL, "n_embd must be a multiple of n_head");
  if (c.n_embd / c.n_head > 64) return fail(nullptr, GPT_E_UNSUPPORTED, "head_dim above 64 is not implemented");
  if (c.n_embd > 1024) return fail(nullptr, GPT_E_UNSUPPORTED, "n_embd above 1024 is not implemented");
  if (c.n_embd % 4 != 0) return fail(nullptr, GPT_E_UNSUPPORTED, "n_embd must be a multiple of 4");
  if (c.precision != GPT_PREC_FP32 && c.precision != GPT_PREC_BF16) return fail(nullptr, GPT_E_INVAL, "unknown precision");
  if (!(c.dropout >= 0.0f && c.dropout < 1.0f)) return fail(nullptr, GPT_E_INVAL, "dropout must be in [0, 1)");
  if (c.flags & ~(uint32_t)(GPT_F_KV_CACHE | GPT_F_MICROGPT | GPT_F_DEBUG_CHECKS))
    return fail(nullptr, GPT_E_INVAL, "unknown flags");
  if (c.lora_rank < 0 || c.lora_rank > 64) return fail(nullptr, GPT_E_INVAL, "lora_rank must be in [0, 64]");
  if (c.lora_rank > 0 && !(std::isfinite(c.lora_alpha) && c.lora_alpha != 0.0f))
    return fail(nullptr, GPT_E_INVAL, "lora_alpha must be finite and nonzero");
  const int64_t M = (int64_t)c.batch * c.block_size;
  if (M > 32768) return fail(nullptr, GPT_E_UNSUPPORTED, "batch * block_size above 32768 is not implemented");
  {
    int sh = 0;
    while ((1ll << sh) < (M < 2 ? 2 : M)) sh++;
    if (((uint64_t)c.padded_vocab << sh) > 0xFFFFFFFFull)
      return fail(nullptr, GPT_E_UNSUPPORTED, "padded_vocab * batch * block_size too large for the embedding sort");
  }
  gpt_model* h = new gpt_model();
  h->cfg = c;
  h->bf16 = c.precision == GPT_PREC_BF16;
  h->d = c.n_embd;
  h->H = c.n_head;
  h->hd = c.n_embd / c.n_head;
  h->L = c.n_layer;
  h->V = c.vocab_size;
  h->Vp = c.padded_vocab;
  h->Tmax = c.block_size;
  h->Bmax = c.batch;
  h->A = c.grad_accum;
  h->micro = (c.flags & GPT_F_MICROGPT) != 0;
  h->head = h->micro ? "lm_head" : "wte";
  h->op_size = h->bf16 ? 2 : 4;
  h->lora_r = c.lora_rank;
  h->lora_s = c.lora_rank > 0 ? c.lora_alpha / (float)c.lora_rank : 0.f;
  // keep an element when its Philox word >= floor(p 2^32); scale kept ones by 1/(1-p)
  h->drop.on = c.dropout > 0.0f ? 1 : 0;
  h->drop.thr = (uint32_t)std::floor((double)c.dropout * 4294967296.0);
  h->drop.scale = (float)(1.0 / (1.0 - (double)c.dropout));
  plan(h);
  *out = h;
  return GPT_OK;
}

void gpt_destroy(gpt_model* h) {
  if (!h) return;
  for (auto& e : h->timer.events) {
    hipEventDestroy(e.first);
    hipEventDestroy(e.second);
  }
  if (h->dg.exec) (void)hipGraphExecDestroy(h->dg.exec);
  if (h->dg.graph) (void)hipGraphDestroy(h->dg.graph);
  if (h->dg.cap) (void)hipStreamDestroy(h->dg.cap);
  delete h;
}

int gpt_get_sizes(const gpt_model* h, gpt_sizes* out) {
  if (!h || !out) return GPT_E_INVAL;
  out->n_params = h->n_params;
  out->n_flat = h->n_flat;
  out->param_bytes = out->grad_bytes = out->m_bytes = out->v_bytes = h->n_flat * 4;
  out->shadow_bytes = h->bf16 ? h->n_flat * 2 * 2 : 0;
  out->activation_bytes = h->act_bytes;
  out->workspace_bytes = h->ws_bytes;
  return GPT_OK;
}

int gpt_num_tensors(const gpt_model* h) { return h ? (int)h->tensors.size() : GPT_E_INVAL; }

int gpt_tensor_info_at(const gpt_model* h, int i, gpt_tensor_info* out) {
  if (!h || !out || i < 0 || i >= (int)h->tensors.size()) return GPT_E_INVAL;
  const Tensor& t = h->tensors[i];
  std::memset(out, 0, sizeof(*out));
  std::snprintf(out->name, sizeof(out->name), "%s", t.name.c_str());
  out->offset = t.offset;
  out->ndim = t.ndim;
  out->shape[0] = t.rows;
  out->shape[1] = t.cols;
  out->decay = t.decay;
  return GPT_OK;
}

int gpt_bind(gpt_model* h, const gpt_buffers* bufs, void* hip_stream) {
  if (!h || !bufs) return fail(h, GPT_E_INVAL, "NULL handle or buffers");
  if (!bufs->params || !bufs->grads || !bufs->m || !bufs->v || !bufs->activations || !bufs->workspace ||
      (h->bf16 && !bufs->shadow))
    return fail(h, GPT_E_INVAL, "a required buffer is NULL");
  const void* ptrs[] = {bufs->params, bufs->grads, bufs->m, bufs->v, bufs->activations, bufs->workspace};
  for (const void* p : ptrs)
    if ((uintptr_t)p % ALIGN_BYTES != 0) return fail(h, GPT_E_INVAL, "buffers must be 256-byte aligned");
  if (h->bf16 && (uintptr_t)bufs->shadow % ALIGN_BYTES != 0) return fail(h, GPT_E_INVAL, "shadow must be 256-byte aligned");
  h->buf = *bufs;
  h->stream = (hipStream_t)hip_stream;
  h->bound = true;
  // a recorded decode step holds the old buffers' addresses
  if (h->dg.exec) (void)hipGraphExecDestroy(h->dg.exec);
  if (h->dg.graph) (void)hipGraphDestroy(h->dg.graph);
  h->dg.exec = nullptr;
  h->dg.graph = nullptr;
  h->dg.tok = nullptr;
  h->dg.out = nullptr;
  h->tables_ready = false;
  h->fwd_pending = false;
  h->grads_fresh = true;
  return GPT_OK;
}

// Everything derived from the fp32 weights: the bf16 shadow and its transposed half,
// and with adapters the merged qkv weights.
static int refresh_derived(gpt_model* h) {
  int rc;
  hipStream_t s = h->stream;
  if (h->bf16) {
    RUN("init", "bf16 shadow", launch_cast_bf16((const float*)h->buf.params, h->buf.shadow, h->n_flat, s));
    if ((rc = upload_tables(h))) return rc;
    if (h->lora_r && (rc = lora_merge(h))) return rc;
    RUN("init", "transposed shadow", transpose_shadow(h));
  } else if (h->lora_r) {
    if ((rc = upload_tables(h))) return rc;
    const size_t dd = (size_t)h->d * h->d;
    for (int l = 0; l < h->L; l++)   // the k rows stay W0; the merge rewrites q and v
      RUN("init", "qkv weight copy",
          hipMemcpyAsync(ws<float>(h, h->weff) + (size_t)l * 3 * dd, P(h, "h" + std::to_string(l) + ".attn.w"),
                         3 * dd * 4, hipMemcpyDeviceToDevice, s));
    if ((rc = lora_merge(h))) return rc;
  }
  return GPT_OK;
}

int gpt_init_state(gpt_model* h) {
  int rc = check_usable(h);
  if (rc) return rc;
  hipStream_t s = h->stream;
  RUN("init", "zero grads", launch_zero(h->buf.grads, h->n_flat, s));
  RUN("init", "zero m", launch_zero(h->buf.m, h->n_flat, s));
  RUN("init", "zero v", launch_zero(h->buf.v, h->n_flat, s));
  RUN("init", "zero optimizer state", launch_zero(ws(h, h->opt), sizeof(OptState) / 4, s));
  RUN("init", "zero stand-in biases", launch_zero(ws(h, h->zbias), 4 * (size_t)h->d, s));
  if ((rc = refresh_derived(h))) return rc;
  h->grads_fresh = true;
  h->fwd_pending = false;
  return GPT_OK;
}

int gpt_params_loaded(gpt_model* h) {
  int rc = check_usable(h);
  if (rc) return rc;
  if ((rc = refresh_derived(h))) return rc;
  h->fwd_pending = false;
  return GPT_OK;
}

int gpt_forward_loss(gpt_model* h, const int32_t* d_tokens, const int32_t* d_targets, int32_t B, int32_t T,
                     float* d_loss) {
  int rc = check_usable(h);
  if (rc) return rc;
  if (!d_tokens || !d_targets) return fail(h, GPT_E_INVAL, "NULL token or target pointer");
  if ((rc = check_shape(h, B, T))) return rc;
  const int M = B * T;
  if ((rc = copy_ids(h, d_tokens, h->tokens, M))) return rc;
  if ((rc = copy_ids(h, d_targets, h->targets, M))) return rc;
  if ((rc = check_ids(h, h->tokens, M)) || (rc = check_ids(h, h->targets, M))) return rc;
  h->fwd_pending = false;
  DropArgs da = h->drop;
  da.call = h->drop_call++;                        // advances with or without dropout
  h->drop_fwd = da;
  if ((rc = forward_to_logits(h, B, T, da))) return rc;
  const float scale = (float)(1.0 / ((double)M * (double)h->A));
  RUN("xent", "xent", launch_xent(act(h, h->logits), h->bf16, h->ldz, act<int32_t>(h, h->targets),
                                   act<float>(h, h->row_loss), M, h->Vp, scale, h->stream));
  if (d_loss) RUN("xent", "loss_mean", launch_mean(act<float>(h, h->row_loss), M, d_loss, h->stream));
  h->fwd_pending = true;
  h->cur_B = B;
  h->cur_T = T;
  return GPT_OK;
}

int gpt_prefill(gpt_model* h, const int32_t* d_tokens, int32_t B, int32_t T, float* d_logits) {
  int rc = check_usable(h);
  if (rc) return rc;
  if (!(h->cfg.flags & GPT_F_KV_CACHE)) return fail(h, GPT_E_UNSUPPORTED, "create the model with GPT_F_KV_CACHE to decode");
  if (!d_tokens || !d_logits) return fail(h, GPT_E_INVAL, "NULL pointer");
  if ((rc = check_shape(h, B, T))) return rc;
  h->fwd_pending = false;
  h->kv_len = 0;
  if ((rc = copy_ids(h, d_tokens, h->tokens, B * T))) return rc;
  if ((rc = check_ids(h, h->tokens, B * T))) return rc;
  const DropArgs none{};
  if ((rc = forward_to_logits(h, B, T, none))) return rc;
  // the last position of every sequence: rows b*T + T-1 of the logits
  const char* last = (const char*)act(h, h->logits) + (size_t)(T - 1) * h->ldz * h->op_size;
  RUN("copy", "logits_to_f32", launch_rows_to_f32(last, h->bf16, (int64_t)T * h->ldz, B, h->Vp, d_logits, h->stream));
  for (int l = 0; l < h->L; l++)
    RUN("decode", "kv_append",
        launch_kv_append(act(h, h->layers[l].qkv), h->bf16, kv_slot(h, l), B, T, h->Tmax, 0, h->d, h->stream));
  RUN("decode", "kv_position", launch_set_i32(ws<int>(h, h->kvpos), T, h->stream));
  h->kv_len = T;
  h->kv_B = B;
  return GPT_OK;
}

}  // extern "C"

namespace {

// The launches of one decode step on h->stream: token ids read from d_tokens, fp32
// logits written to d_logits [B, Vp], the position taken from (and, by the lm_head
// launch, advanced in) the device counter kvpos. Nothing here depends on the host's
// copy of the position, so a recording of these launches serves every step.
// GPT_DECODE_FUSE_NORM=0: the decode step's normalizations as launches of their own
// (for comparisons).
bool decode_fuse_norm() {
  static int on = -1;
  if (on < 0) {
    const char* e = std::getenv("GPT_DECODE_FUSE_NORM");
    on = (e && e[0] == '0') ? 0 : 1;
  }
  return on == 1;
}

int decode_launches(gpt_model* h, const int32_t* d_tokens, float* d_logits) {
  const int B = h->kv_B, d = h->d;
  const bool bf = h->bf16;
  hipStream_t s = h->stream;
  int* pos = ws<int>(h, h->kvpos);
  int rc;
  if (h->cfg.flags & GPT_F_DEBUG_CHECKS)
    RUN("check", "check_ids", launch_check_ids(d_tokens, B, h->V, ws<OptState>(h, h->opt), s));
  // B single-token rows through the layer-0 activation slots
  const LayerAct& a = h->layers[0];
  float* x = act<float>(h, a.x);
  float* xmid = act<float>(h, a.xmid);
  RUN("decode", "embed", launch_embed_pos(P(h, "wte"), P(h, "wpe"), d_tokens, x, B, d, h->Vp, pos, h->Tmax, s));
  // The normalization in front of the qkv and MLP-up products runs inside their
  // launch where the few-rows kernel allows it (its output is not kept: nothing
  // reads it after a decode step), else as a launch of its own.
  auto normed_gemm = [&](const float* xin, const std::string& ln, const Slice& y, const Slice& mean,
                         const Slice& rstd, GemmDesc g, const char* what) -> int {
    g.norm = h->micro ? 2 : 1;
    g.norm_x = xin;
    g.norm_g = h->micro ? nullptr : P(h, ln + ".g");
    g.norm_b = h->micro ? nullptr : P(h, ln + ".b");
    if (!decode_fuse_norm() || !gemm_norm_fusable(g, bf)) {
      g.norm = 0;
      int r;
      if ((r = norm_fwd(h, xin, ln, act(h, y), act<float>(h, mean), act<float>(h, rstd), B))) return r;
    }
    RUN("decode", what, gemm(h, g, bf));
    return GPT_OK;
  };
  for (int l = 0; l < h->L; l++) {
    const std::string p = "h" + std::to_string(l) + ".";
    {
      GemmDesc g = gemm_desc(act(h, a.ln1), d, true, Wop(h, p + "attn.w"), d, true, act(h, a.qkv), 3 * d, B, 3 * d, d,
                             EPI_BIAS);
      g.bias = bias_of(h, p + "attn.b");
      if ((rc = normed_gemm(x, p + "ln1", a.ln1, a.ln1_mean, a.ln1_rstd, g, "qkv"))) return rc;
    }
    // the attention stores this position's keys and values into the cache itself
    RUN("decode", "attn",
        launch_attn_decode(act(h, a.qkv), kv_slot(h, l), act(h, a.att), bf, B, h->H, h->hd, h->Tmax, pos, s));
    {
      GemmDesc g = gemm_desc(act(h, a.att), d, true, Wop(h, p + "proj.w"), d, true, xmid, d, B, d, d, EPI_BIAS_RESID);
      g.bias = bias_of(h, p + "proj.b");
      g.resid = x;
      g.ldr = d;
      RUN("decode", "proj", gemm(h, g, bf));
    }
    {
      GemmDesc g = gemm_desc(act(h, a.ln2), d, true, Wop(h, p + "fc.w"), d, true, act(h, a.h), 4 * d, B, 4 * d, d,
                             h->micro ? EPI_BIAS_RELU : EPI_BIAS_GELU);
      g.bias = bias_of(h, p + "fc.b");
      g.aux = act(h, a.u);
      g.ldaux = 4 * d;
      if ((rc = normed_gemm(xmid, p + "ln2", a.ln2, a.ln2_mean, a.ln2_rstd, g, "fc"))) return rc;
    }
    {
      GemmDesc g = gemm_desc(act(h, a.h), 4 * d, true, Wop(h, p + "fcproj.w"), 4 * d, true, x, d, B, d, 4 * d,
                             EPI_BIAS_RESID);
      g.bias = bias_of(h, p + "fcproj.b");
      g.resid = xmid;
      g.ldr = d;
      RUN("decode", "fcproj", gemm(h, g, bf));
    }
  }
  if ((rc = norm_fwd(h, x, "lnf", act(h, h->lnf), act<float>(h, h->lnf_mean), act<float>(h, h->lnf_rstd), B)))
    return rc;
  {
    // fp32 logits straight into the caller's rows (the fp32 accumulators, not a
    // rounded operand-type copy); the same launch advances the position
    GemmDesc g = gemm_desc(act(h, h->lnf), d, true, Wop(h, h->head), d, true, d_logits, h->Vp, B, h->Vp, d,
                           bf ? EPI_F32 : EPI_STORE);
    g.bump = pos;
    RUN("decode", "lm_head", gemm(h, g, bf));
  }
  return GPT_OK;
}

// GPT_DECODE_GRAPH=0: every decode step launched one kernel at a time (for comparisons).
bool decode_graph_on() {
  static int on = -1;
  if (on < 0) {
    const char* e = std::getenv("GPT_DECODE_GRAPH");
    on = (e && e[0] == '0') ? 0 : 1;
  }
  return on == 1;
}

void drop_decode_graph(gpt_model* h) {
  if (h->dg.exec) (void)hipGraphExecDestroy(h->dg.exec);
  if (h->dg.graph) (void)hipGraphDestroy(h->dg.graph);
  h->dg.exec = nullptr;
  h->dg.graph = nullptr;
}

// Records decode_launches on the library's own capture stream (the caller's stream
// may be the null stream, which cannot be captured) and instantiates the graph. A
// failure of the graph API itself is not an error of the step: the model then stops
// recording (dg.off) and the step runs as direct launches. Returns whether a graph
// is ready, or a GPT_E_* code for an error of the launches themselves.
int record_decode_graph(gpt_model* h, const int32_t* d_tokens, float* d_logits, bool* ready) {
  *ready = false;
  if (!h->dg.cap && hipStreamCreateWithFlags(&h->dg.cap, hipStreamNonBlocking) != hipSuccess) {
    (void)hipGetLastError();
    h->dg.cap = nullptr;
    h->dg.off = true;
    return GPT_OK;
  }
  if (hipStreamBeginCapture(h->dg.cap, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    (void)hipGetLastError();
    h->dg.off = true;
    return GPT_OK;
  }
  hipStream_t user = h->stream;
  h->stream = h->dg.cap;
  const int rc = decode_launches(h, d_tokens, d_logits);
  h->stream = user;
  hipGraph_t g = nullptr;
  const hipError_t e = hipStreamEndCapture(h->dg.cap, &g);
  if (rc != GPT_OK || e != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    (void)hipGetLastError();
    if (rc != GPT_OK) return rc;
    h->dg.off = true;
    return GPT_OK;
  }
  hipGraphExec_t x = nullptr;
  if (hipGraphInstantiate(&x, g, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipGraphDestroy(g);
    h->dg.off = true;
    return GPT_OK;
  }
  h->dg.graph = g;
  h->dg.exec = x;
  *ready = true;
  return GPT_OK;
}

}  // namespace

extern "C" {

int gpt_decode(gpt_model* h, const int32_t* d_tokens, float* d_logits) {
  int rc = check_usable(h);
  if (rc) return rc;
  if (!(h->cfg.flags & GPT_F_KV_CACHE)) return fail(h, GPT_E_UNSUPPORTED, "create the model with GPT_F_KV_CACHE to decode");
  if (!d_tokens || !d_logits) return fail(h, GPT_E_INVAL, "NULL pointer");
  if (h->kv_len < 1) return fail(h, GPT_E_STATE, "gpt_decode needs a preceding gpt_prefill");
  if (h->kv_len >= h->Tmax) return fail(h, GPT_E_SEQ_TOO_LONG, "the cache holds block_size positions already");
  h->fwd_pending = false;
  // A call with the previous call's token and logits pointers and batch replays the
  // recorded step (recorded at the first such repeat); any other call runs the
  // launches directly and becomes the new reference.
  const bool repeat = h->dg.tok == d_tokens && h->dg.out == d_logits && h->dg.B == h->kv_B;
  bool ready = h->dg.exec != nullptr;
  if (repeat && !ready && decode_graph_on() && !h->timer.on && !h->dg.off &&
      (rc = record_decode_graph(h, d_tokens, d_logits, &ready)))
    return rc;
  if (repeat && ready && !h->timer.on) {
    if ((rc = hip_check(h, hipGraphLaunch(h->dg.exec, h->stream), "decode graph launch"))) return rc;
  } else if (repeat) {
    if ((rc = decode_launches(h, d_tokens, d_logits))) return rc;
  } else {
    drop_decode_graph(h);
    h->dg.tok = d_tokens;
    h->dg.out = d_logits;
    h->dg.B = h->kv_B;
    if ((rc = decode_launches(h, d_tokens, d_logits))) return rc;
  }
  h->kv_len++;
  return GPT_OK;
}

int gpt_sample(gpt_model* h, const float* d_logits, int32_t B, float temperature, int32_t top_k,
               const float* d_uniform, int32_t* d_tokens_out) {
  int rc = check_usable(h);
  if (rc) return rc;
  if (!d_logits || !d_tokens_out || (temperature > 0.f && !d_uniform)) return fail(h, GPT_E_INVAL, "NULL pointer");
  if (B < 1) return fail(h, GPT_E_INVAL, "B must be >= 1");
  if (!(temperature == temperature)) return fail(h, GPT_E_INVAL, "temperature is NaN");
  RUN("decode", "sample",
      launch_sample(d_logits, h->Vp, B, h->Vp, temperature, top_k, d_uniform, d_tokens_out, h->stream));
  return GPT_OK;
}

int gpt_forward_logits(gpt_model* h, const int32_t* d_tokens, int32_t B, int32_t T, float* d_logits) {
  int rc = check_usable(h);
  if (rc) return rc;
  if (!d_tokens || !d_logits) return fail(h, GPT_E_INVAL, "NULL pointer");
  if ((rc = check_shape(h, B, T))) return rc;
  const int M = B * T;
  h->fwd_pending = false;
  if ((rc = copy_ids(h, d_tokens, h->tokens, M))) return rc;
  if ((rc = check_ids(h, h->tokens, M))) return rc;
  const DropArgs none{};                           // inference: no dropout
  if ((rc = forward_to_logits(h, B, T, none))) return rc;
  RUN("copy", "logits_to_f32",
      launch_rows_to_f32(act(h, h->logits), h->bf16, h->ldz, M, h->Vp, d_logits, h->stream));
  return GPT_OK;
}

int gpt_backward(gpt_model* h) {
  int rc = check_usable(h);
  if (rc) return rc;
  if (!h->fwd_pending) return fail(h, GPT_E_STATE, "gpt_backward needs a preceding gpt_forward_loss");
  if ((rc = upload_tables(h))) return rc;
  const int B = h->cur_B, T = h->cur_T, M = B * T, d = h->d, L = h->L;
  RedRows rows;                                   // partial rows per producer kind, set as they run
  rows.nblk[RED_LN] = (M + LN_BWD_ROWS - 1) / LN_BWD_ROWS;
  rows.nblk[RED_QKV] = (M + COLSUM_ROWS - 1) / COLSUM_ROWS;
  rows.nblk[RED_FC] = (M + COLSUM_ROWS - 1) / COLSUM_ROWS;
  const bool bf = h->bf16;
  hipStream_t s = h->stream;
  const float beta = h->grads_fresh ? 0.f : 1.f;
  float* dres = ws<float>(h, h->dres);
  void* dln = ws(h, h->dln);   // input gradients into a LayerNorm backward (operand type)
  void* dO = ws(h, h->dO);
  const DropArgs& da = h->drop_fwd;
  const bool drop = da.on != 0;
  float* dxm = drop && !bf ? ws<float>(h, h->dxm) : nullptr;   // fp32: masked operand copies
  // In bf16 mode the weight gradients wait for the end of the backward (their
  // operands stay in per-layer slots); in fp32 mode each runs as soon as its
  // operands exist, before the residual gradient is overwritten.
  // With adapters only the qkv weight gradient is formed, as this micro-batch's
  // input to the adapter gradients (beta 0); the frozen tensors get none.
  const bool lora = h->lora_r > 0;
  auto wgrad_now = [&](const void* A, int64_t lda, const void* Bm, int64_t ldb, const std::string& w, int Mo,
                       int No, const char* what) {
    const size_t n = w.size();
    if (lora && !(n > 7 && w.compare(n - 7, 7, ".attn.w") == 0)) return GPT_OK;
    GemmDesc g = gemm_desc(A, lda, false, Bm, ldb, false, G(h, w), No, Mo, No, M, EPI_ACC);
    g.beta = lora ? 0.f : beta;
    RUN("gemm_wgrad", what, gemm(h, g, bf));
    return GPT_OK;
  };

  // lm_head (tied): dwte = dlogits^T lnf; dlnf = dlogits wte
  {
    if (!bf && (rc = wgrad_now(act(h, h->logits), h->ldz, act(h, h->lnf), d, h->head, h->Vp, d, "lm_head_wgrad")))
      return rc;
    GemmDesc g2 = bf ? gemm_desc(act(h, h->logits), h->ldz, true, WopT(h, h->head), h->Vp, true, dln, d, M, d, h->Vp, EPI_STORE)
                     : gemm_desc(act(h, h->logits), h->ldz, true, Wop(h, h->head), d, false, dln, d, M, d, h->Vp, EPI_F32);
    RUN("gemm_dgrad", "lm_head_dgrad", gemm(h, g2, bf));
  }
  if ((rc = ln_bwd(h, dln, act<float>(h, h->x_final), act<float>(h, h->lnf_mean), act<float>(h, h->lnf_rstd),
                   "lnf.g", "lnf.b", nullptr, nullptr, bf ? rx_slot(h, L) : (void*)dxm, M, -1,
                   (int)site_mlp_out(L - 1))))
    return rc;

  for (int l = L - 1; l >= 0; l--) {
    const LayerAct& la = h->layers[l];
    const std::string p = "h" + std::to_string(l) + ".";
    void* du = bf ? du_slot(h, l) : ws(h, h->du);
    void* dqkv = bf ? dqkv_slot(h, l) : ws(h, h->dqkv);
    // ---- MLP: x_{l+1} = xmid + drop(gelu(LN2(xmid) Wfc^T + bfc) Wp^T + bp) ; dres holds d x_{l+1}
    {
      // GEMM operand view of d x_{l+1} (times the MLP output mask with dropout)
      const void* dx = bf ? rx_slot(h, l + 1) : (dxm ? (const void*)dxm : (const void*)dres);
      const int act_bwd = h->micro ? EPI_RELU_BWD : EPI_GELU_BWD;
      GemmDesc g = bf ? gemm_desc(dx, d, true, WopT(h, p + "fcproj.w"), d, true, du, 4 * d, M, 4 * d, d, act_bwd)
                      : gemm_desc(dx, d, true, Wop(h, p + "fcproj.w"), 4 * d, false, du, 4 * d, M, 4 * d, d, act_bwd);
      g.aux = act(h, la.u);
      g.ldaux = 4 * d;
      const int fc_rows = h->micro ? 0 : gemm_colsum_rows(g, bf);   // fc.b gradient fused into this GEMM when possible
      if (fc_rows) g.colsum = red_part(h, p + "fc.b");
      rows.nblk[RED_FC] = fc_rows ? fc_rows : (M + COLSUM_ROWS - 1) / COLSUM_ROWS;
      RUN("gemm_dgrad", "fcproj_dgrad", gemm(h, g, bf));
      if (!bf && (rc = wgrad_now(dx, d, act(h, la.h), 4 * d, p + "fcproj.w", d, 4 * d, "fcproj_wgrad"))) return rc;
      GemmDesc g2 = bf ? gemm_desc(du, 4 * d, true, WopT(h, p + "fc.w"), 4 * d, true, dln, d, M, d, 4 * d, EPI_STORE)
                       : gemm_desc(du, 4 * d, true, Wop(h, p + "fc.w"), d, false, dln, d, M, d, 4 * d, EPI_F32);
      RUN("gemm_dgrad", "fc_dgrad", gemm(h, g2, bf));
      if (!bf && (rc = wgrad_now(du, 4 * d, act(h, la.ln2), d, p + "fc.w", 4 * d, d, "fc_wgrad"))) return rc;
      if (!h->micro && !lora && !fc_rows && (rc = colsum(h, du, bf, 4 * d, M, 4 * d, p + "fc.b"))) return rc;
      const std::string fcproj_b = p + "fcproj.b";
      if ((rc = ln_bwd(h, dln, act<float>(h, la.xmid), act<float>(h, la.ln2_mean), act<float>(h, la.ln2_rstd),
                       p + "ln2.g", p + "ln2.b", dres, fcproj_b.c_str(), bf ? rm_slot(h, l) : (void*)dxm, M,
                       (int)site_mlp_out(l), (int)site_attn_out(l))))
        return rc;
    }
    // ---- attention: xmid = x + drop(attn(LN1(x)) Wo^T + bo) ; dres now holds d xmid
    {
      // GEMM operand view of d xmid (times the attention output mask with dropout)
      const void* dx = bf ? rm_slot(h, l) : (dxm ? (const void*)dxm : (const void*)dres);
      GemmDesc g = bf ? gemm_desc(dx, d, true, WopT(h, p + "proj.w"), d, true, dO, d, M, d, d, EPI_STORE)
                      : gemm_desc(dx, d, true, Wop(h, p + "proj.w"), d, false, dO, d, M, d, d, EPI_STORE);
      RUN("gemm_dgrad", "proj_dgrad", gemm(h, g, bf));
      if (!bf && (rc = wgrad_now(dx, d, act(h, la.att), d, p + "proj.w", d, d, "proj_wgrad"))) return rc;
      const int qkv_rows = h->micro ? 0 : attn_bwd_colsum_rows(bf, B, T, h->hd);   // attn.b gradient fused into the kernels
      rows.nblk[RED_QKV] = qkv_rows ? qkv_rows : (M + COLSUM_ROWS - 1) / COLSUM_ROWS;
      RUN("attn_bwd", "attn_bwd",
          launch_attn_bwd(act(h, la.qkv), act(h, la.att), dO, act<float>(h, la.lse), ws<float>(h, h->attnD), dqkv, bf,
                          B, T, h->H, h->hd, qkv_rows ? red_part(h, p + "attn.b") : nullptr, da,
                          site_attn_prob(l), s));
      if (!bf && (rc = wgrad_now(dqkv, 3 * d, act(h, la.ln1), d, p + "attn.w", 3 * d, d, "qkv_wgrad"))) return rc;
      if (!h->micro && !lora && !qkv_rows && (rc = colsum(h, dqkv, bf, 3 * d, M, 3 * d, p + "attn.b"))) return rc;
      // d x_0 feeds only the embedding backward, which reads the fp32 copy; with
      // adapters the embeddings are frozen, so layer 0's input gradient (this GEMM
      // and the LayerNorm backward) has no reader
      if (lora && l == 0) continue;
      GemmDesc g2 = bf ? gemm_desc(dqkv, 3 * d, true, WopT(h, p + "attn.w"), 3 * d, true, dln, d, M, d, 3 * d, EPI_STORE)
                       : gemm_desc(dqkv, 3 * d, true, Wop(h, p + "attn.w"), d, false, dln, d, M, d, 3 * d, EPI_F32);
      RUN("gemm_dgrad", "qkv_dgrad", gemm(h, g2, bf));
      const std::string proj_b = p + "proj.b";
      void* xop = l == 0 ? nullptr : (bf ? rx_slot(h, l) : (void*)dxm);
      if ((rc = ln_bwd(h, dln, act<float>(h, la.x), act<float>(h, la.ln1_mean), act<float>(h, la.ln1_rstd),
                       p + "ln1.g", p + "ln1.b", dres, proj_b.c_str(), xop, M, (int)site_attn_out(l),
                       l > 0 ? (int)site_mlp_out(l - 1) : -1)))
        return rc;
    }
  }
  if (bf) {
    // every weight gradient of the micro-batch: one grouped launch when the shapes
    // allow it (K = B*T a multiple of 32), else one GEMM each
    if (h->wgroup && M % 32 == 0) {
      RUN("gemm_wgrad", "grouped_wgrad",
          launch_wgrad_group(ws<WgradProblem>(h, h->wtable), (int)h->wprobs.size(), h->wtiles, M, lora ? 0.f : beta,
                             (float*)((char*)h->buf.workspace + h->split.off), h->split_floats, s));
    } else {
      for (const WgradProblem& q : h->wprobs) {
        GemmDesc g = gemm_desc(q.A, q.lda, false, q.B, q.ldb, false, q.C, q.ldc, q.M, q.N, M, EPI_ACC);
        g.beta = lora ? 0.f : beta;
        RUN("gemm_wgrad", "wgrad", gemm(h, g, bf));
      }
    }
  }
  if (lora) {
    // the adapters' gradients from this micro-batch's q and v weight gradients; the
    // frozen biases, norms and embeddings take none
    RUN("lora", "lora_grad",
        launch_lora_grad(ws<LoraJob>(h, h->ltable), 2 * L, d, h->lora_r, h->lora_s, beta, s));
    h->grads_fresh = false;
    h->fwd_pending = false;
    return GPT_OK;
  }
  if (!h->rjobs.empty())
    RUN("colsum", "bias_and_ln_grads",
        launch_reduce_jobs(ws<RedJob>(h, h->rtable), (int)h->rjobs.size(), h->rblocks, ws<float>(h, h->red),
                           (float*)h->buf.grads, rows, beta, s));
  // ---- embeddings: dres holds d x0 (after the lm_head weight gradient: both write wte's gradient;
  // with an lm_head of its own, the embedding scatter is wte's only gradient and starts from zero)
  if (h->grads_fresh && h->micro)
    RUN("embed", "zero wte grad", launch_zero(G(h, "wte"), (size_t)h->Vp * d, s));
  if (h->grads_fresh && T < h->Tmax) {
    float* wpe_tail = G(h, "wpe") + (size_t)T * d;
    RUN("embed", "zero wpe tail", launch_zero(wpe_tail, (size_t)(h->Tmax - T) * d, s));
  }
  if (drop)   // x0 = drop(wte[tok] + wpe): the tables see d x0 times the embedding mask
    RUN("embed", "embed_dropout", launch_dropout_rows(dres, dres, M, d, da, site_embed(), s));
  EmbedBwdScratch scr{ws<uint32_t>(h, h->emb_keys), ws<float>(h, h->emb_piece)};
  RUN("embed", "embed_bwd",
      launch_embed_bwd(dres, act<int32_t>(h, h->tokens), G(h, "wte"), G(h, "wpe"), beta, B, T, d, h->Vp, scr, s));
  h->grads_fresh = false;
  h->fwd_pending = false;
  return GPT_OK;
}

int gpt_set_dropout_seed(gpt_model* h, uint64_t seed, uint32_t counter) {
  if (!h) return GPT_E_INVAL;
  h->drop.k0 = (uint32_t)(seed & 0xFFFFFFFFu);
  h->drop.k1 = (uint32_t)(seed >> 32);
  h->drop_call = counter;
  return GPT_OK;
}

int gpt_zero_grad(gpt_model* h) {
  if (!h) return GPT_E_INVAL;
  h->grads_fresh = true;
  return GPT_OK;
}

// The update of gpt_adamw_step with the gradient norm's partial sums in `part`
// (NORM_BLOCKS floats): the bound workspace, or the static array of the
// no-allocation variant.
static int adamw_step(gpt_model* h, float lr, float beta1, float beta2, float eps, float weight_decay, float clip,
                      float* d_grad_norm, float* part) {
  hipStream_t s = h->stream;
  int rc;
  OptState* st = ws<OptState>(h, h->opt);
  // With adapters the norm, the clip and the update cover the adapters alone (the
  // last, contiguous run of the flat arrays, all 2-D and decayed); the merged qkv
  // weights are rebuilt after the update.
  const size_t o = h->lora_r ? h->lora_off : 0;
  const size_t n = h->n_flat - o;
  const size_t n_decay = h->lora_r ? n : h->n_decay;
  RUN("adamw", "grad_sumsq", launch_sumsq_partial((const float*)h->buf.grads + o, n, part, s));
  RUN("adamw", "opt_prepare", launch_opt_prepare(part, st, clip, beta1, beta2, d_grad_norm, s));
  RUN("adamw", "adamw",
      launch_adamw((float*)h->buf.params + o, (const float*)h->buf.grads + o, (float*)h->buf.m + o,
                   (float*)h->buf.v + o, h->bf16 && !h->lora_r ? h->buf.shadow : nullptr, n, n_decay, st, lr, beta1,
                   beta2, eps, weight_decay, s));
  if (h->lora_r && (rc = lora_merge(h))) return rc;
  if (h->bf16) RUN("adamw", "transposed shadow", transpose_shadow(h));
  h->grads_fresh = true;
  return GPT_OK;
}

static int adamw_check(gpt_model* h, float lr, float beta1, float beta2, float eps, float weight_decay, float clip) {
  int rc = check_usable(h);
  if (rc) return rc;
  if (!(beta1 >= 0.f && beta1 < 1.f && beta2 >= 0.f && beta2 < 1.f && eps >= 0.f && std::isfinite(lr) &&
        std::isfinite(weight_decay) && std::isfinite(clip)))
    return fail(h, GPT_E_INVAL, "invalid AdamW hyper-parameters");
  if (h->grads_fresh) return fail(h, GPT_E_STATE, "gpt_adamw_step needs at least one gpt_backward since the last step");
  return GPT_OK;
}

int gpt_adamw_step(gpt_model* h, float lr, float beta1, float beta2, float eps, float weight_decay, float clip,
                   float* d_grad_norm) {
  int rc = adamw_check(h, lr, beta1, beta2, eps, weight_decay, clip);
  if (rc) return rc;
  return adamw_step(h, lr, beta1, beta2, eps, weight_decay, clip, d_grad_norm, ws<float>(h, h->norm_part));
}

int gpt_adamw_step_noalloc(gpt_model* h, float lr, float beta1, float beta2, float eps, float weight_decay,
                           float clip, float* d_grad_norm) {
  int rc = adamw_check(h, lr, beta1, beta2, eps, weight_decay, clip);
  if (rc) return rc;
  static_assert(NORM_BLOCKS <= NOALLOC_SCRATCH_FLOATS, "the norm's partials fit the static scratch");
  const size_t need = NORM_BLOCKS;   // partial sums of the norm, whatever the model's size
  if (need > NOALLOC_SCRATCH_FLOATS)
    return fail(h, GPT_E_UNSUPPORTED, "gradient-norm partials (" + std::to_string(need) +
                                          " floats) exceed the static scratch (" +
                                          std::to_string(NOALLOC_SCRATCH_FLOATS) + " floats)");
  hipDevice_t dev = 0;
  hipError_t e = hipStreamGetDevice(h->stream, &dev);
  if (e != hipSuccess) return hip_check(h, e, "hipStreamGetDevice");
  float* part = nullptr;
  if ((e = noalloc_norm_scratch((int)dev, &part)) != hipSuccess) return hip_check(h, e, "static scratch address");
  return adamw_step(h, lr, beta1, beta2, eps, weight_decay, clip, d_grad_norm, part);
}

int gpt_sync(gpt_model* h) {
  if (!h) return GPT_E_INVAL;
  hipError_t e = hipStreamSynchronize(h->stream);
  int rc = h->sticky;
  h->sticky = GPT_OK;
  if (e != hipSuccess) return fail(h, GPT_E_HIP, std::string("hipStreamSynchronize: ") + hipGetErrorString(e));
  if (rc != GPT_OK) return rc;
  if (h->bound) {
    OptState st;
    e = hipMemcpy(&st, ws(h, h->opt), sizeof(st), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(h, GPT_E_HIP, std::string("read optimizer state: ") + hipGetErrorString(e));
    if (st.bad_ids) {
      const int32_t zero2[2] = {0, 0};   // bad_ids and nonfinite: the ids explain a NaN loss
      static_assert(offsetof(OptState, bad_ids) == offsetof(OptState, nonfinite) + 4, "flag order");
      e = hipMemcpy((char*)ws(h, h->opt) + offsetof(OptState, nonfinite), zero2, 8, hipMemcpyHostToDevice);
      if (e != hipSuccess) return fail(h, GPT_E_HIP, std::string("clear id flag: ") + hipGetErrorString(e));
      h->err = "a token or target id lies outside [0, vocab_size): the AdamW update was skipped";
      return GPT_E_INVAL;
    }
    if (st.nonfinite) {
      int32_t zero = 0;
      e = hipMemcpy((char*)ws(h, h->opt) + offsetof(OptState, nonfinite), &zero, 4, hipMemcpyHostToDevice);
      h->err = "non-finite gradient norm: the AdamW update was skipped";
      return GPT_E_NONFINITE;
    }
  }
  return GPT_OK;
}

int gpt_get_step(gpt_model* h, int64_t* t) {
  int rc = check_usable(h);
  if (rc) return rc;
  if (!t) return fail(h, GPT_E_INVAL, "NULL output");
  OptState st;
  hipError_t e = hipStreamSynchronize(h->stream);
  if (e == hipSuccess) e = hipMemcpy(&st, ws(h, h->opt), sizeof(st), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_check(h, e, "read optimizer state");
  *t = st.t;
  return GPT_OK;
}

int gpt_debug_copy(gpt_model* h, const char* what, int32_t layer, void* d_dst, size_t bytes) {
  int rc = check_usable(h);
  if (rc) return rc;
  if (!what || !d_dst) return fail(h, GPT_E_INVAL, "NULL argument");
  const size_t M = (size_t)h->cur_B * h->cur_T;
  const std::string w(what);
  const void* src = nullptr;
  size_t n = 0;
  const size_t d = h->d;
  if (w == "x") {
    if (layer < 0 || layer > h->L) return fail(h, GPT_E_INVAL, "layer out of range");
    src = layer == h->L ? act(h, h->x_final) : act(h, h->layers[layer].x);
    n = M * d * 4;
  } else if (w == "qkv" || w == "attn" || w == "h" || w == "lse" || w == "u") {
    if (layer < 0 || layer >= h->L) return fail(h, GPT_E_INVAL, "layer out of range");
    const LayerAct& la = h->layers[layer];
    if (w == "qkv") { src = act(h, la.qkv); n = M * 3 * d * h->op_size; }
    if (w == "attn") { src = act(h, la.att); n = M * d * h->op_size; }
    if (w == "h") { src = act(h, la.h); n = M * 4 * d * h->op_size; }
    if (w == "u") { src = act(h, la.u); n = M * 4 * d * h->op_size; }
    if (w == "lse") { src = act(h, la.lse); n = (size_t)h->cur_B * h->H * h->cur_T * 4; }
  } else {
    return fail(h, GPT_E_INVAL, "unknown activation '" + w + "'");
  }
  if (M == 0) return fail(h, GPT_E_STATE, "no forward has run");
  if (bytes != n) return fail(h, GPT_E_INVAL, "size mismatch: expected " + std::to_string(n) + " bytes");
  hipError_t e = hipMemcpyAsync(d_dst, src, n, hipMemcpyDeviceToDevice, h->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
  return hip_check(h, e, "debug copy");
}

int gpt_timer_enable(gpt_model* h, const char* family) {
  if (!h || !family) return GPT_E_INVAL;
  h->timer.on = true;
  h->timer.family = family;
  h->timer.used = 0;
  return GPT_OK;
}

int gpt_timer_disable(gpt_model* h) {
  if (!h) return GPT_E_INVAL;
  h->timer.on = false;
  return GPT_OK;
}

int gpt_timer_read(gpt_model* h, double* total_ms, int64_t* launches) {
  if (!h || !total_ms || !launches) return GPT_E_INVAL;
  hipError_t e = hipStreamSynchronize(h->stream);
  if (e != hipSuccess) return hip_check(h, e, "timer sync");
  double tot = 0.0;
  for (size_t i = 0; i < h->timer.used; i++) {
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, h->timer.events[i].first, h->timer.events[i].second);
    if (e != hipSuccess) return hip_check(h, e, "hipEventElapsedTime");
    tot += ms;
  }
  *total_ms = tot;
  *launches = (int64_t)h->timer.used;
  return GPT_OK;
}

}  // extern "C"
