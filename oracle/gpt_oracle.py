"""CPU oracle for one GPT-2-style training step.  TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and bench's cpu_baseline leg may import this
module. The product path (the HIP library and its binding) never does, and this
module imports nothing from it. It is plain NumPy, float64 by default, with a
hand-written backward; it loops over the sequences of a micro-batch so that a
whole GPT-2 124M micro-batch fits in memory.

What it computes, and the passage each part follows (the nanoGPT pages):
  * embedding: token embedding plus learned position embedding, no rotary
    ("Building microGPT from scratch", model-core section).
  * block: norm before attention and before the MLP, residual adds around both
    (same section, "residual + norm"); LayerNorm with affine gain/shift and the
    exact erf GELU in a 4x MLP, as the GPT-2 configuration asks.
  * attention: QKV projection, scaled dot product over heads of width
    n_embd / n_head, causal mask, softmax, weighted V, output projection (same
    section; the nanoGPT run log, section 2.2, for head width).
  * head: final LayerNorm then logits against the tied token embedding.
  * loss: mean over every position of -log softmax(logits)[target]
    (microGPT page, training-loop section).
  * gradient accumulation: gradients of several micro-batches are added and the
    effective batch is batch x steps (run log, section 3.1); each micro-batch
    loss is scaled by 1/A so the update sees the mean.
  * clipping at global L2 norm ``clip`` (microGPT page, single-GPU parameters).
  * AdamW: Adam moments with bias correction and decoupled weight decay on the
    2-D tensors (run log, section 2.1: wd 0.1, betas 0.9/0.95; microGPT page:
    betas 0.85/0.99, eps 1e-8).

  * dropout (the nanoGPT run log, section 2.2; the microGPT page's parameter
    list): inverted dropout on the embedding output, on the attention
    probabilities and on the output of each residual branch before its add, the
    kept values scaled by 1 / (1 - p). The masks come from the counter-based
    generator Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random
    numbers: as easy as 1, 2, 3", SC 2011), keyed by a 64-bit seed; see
    ``dropout_keep`` for which counter names which element.

  * generation (nanoGPT practical guide on adg.csdn.net, section 4; the microGPT
    page's single-GPU inference section): logits divided by a temperature, an
    optional top-k cut, a draw from the softmax, one token appended at a time.
    ``generate`` recomputes the whole forward for every new token: that is the
    definition a decoder with a key/value cache has to reproduce.

  * the microGPT variant (configuration variant "microgpt"; same page, model-core
    section): weightless RMSNorm, ReLU instead of GELU, no biases, an lm_head of
    its own. Its norms sit where the GPT-2 block has them (before attention,
    before the MLP and before the head), with eps 1e-5.

  * LoRA (configuration fields lora_rank r > 0 and lora_alpha; the fine-tuning
    article on blog.hotdry.top, LoRA section): the q and v projections of every
    block gain a low-rank branch, q = a W0_q^T + b_q + s (a A_q^T) B_q^T with
    A [r, n_embd], B [n_embd, r] and s = lora_alpha / r; only the A and B
    tensors are trained, every other tensor stays frozen; the merged weight
    W0 + s B A gives the same forward.

Readings where the pages are silent: LayerNorm eps 1e-5 with the biased
variance; attention scale 1/sqrt(head_dim); the softmax runs over all padded
vocabulary columns; the clip coefficient is min(1, clip / (norm + 1e-6)) and
clip <= 0 disables it; decay applies to every 2-D tensor (both embeddings and
all linear weights) and to no bias or LayerNorm parameter; Adam's step count
starts at 1.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np
from scipy.special import erf

LN_EPS = 1e-5
CLIP_EPS = 1e-6


# --------------------------------------------------------------------------- layout

def variant_of(cfg) -> str:
    return getattr(cfg, "variant", "gpt2")


def param_shapes(cfg, variant: str | None = None) -> List[Tuple[str, Tuple[int, ...]]]:
    """Trainable tensors. Linear weights are [out, in] and act as y = x W^T + b.

    variant "gpt2": LayerNorm gain/shift, biased linears, tied head.
    variant "microgpt": the microGPT block ("Building microGPT from scratch",
    model-core section: weightless RMSNorm, ReLU, no biases, an lm_head of its
    own). Its q, k and v matrices are the three row blocks of attn.w, its output
    matrix is proj.w and its two MLP matrices fc.w and fcproj.w.
    (Default: the configuration's own variant.)
    """
    variant = variant_of(cfg) if variant is None else variant
    V, d, T, L = cfg.padded_vocab, cfg.n_embd, cfg.block_size, cfg.n_layer
    out: List[Tuple[str, Tuple[int, ...]]] = [("wte", (V, d)), ("wpe", (T, d))]
    for l in range(L):
        p = f"h{l}."
        if variant == "gpt2":
            out += [(p + "ln1.g", (d,)), (p + "ln1.b", (d,)),
                    (p + "attn.w", (3 * d, d)), (p + "attn.b", (3 * d,)),
                    (p + "proj.w", (d, d)), (p + "proj.b", (d,)),
                    (p + "ln2.g", (d,)), (p + "ln2.b", (d,)),
                    (p + "fc.w", (4 * d, d)), (p + "fc.b", (4 * d,)),
                    (p + "fcproj.w", (d, 4 * d)), (p + "fcproj.b", (d,))]
        elif variant == "microgpt":
            out += [(p + "attn.w", (3 * d, d)), (p + "proj.w", (d, d)),
                    (p + "fc.w", (4 * d, d)), (p + "fcproj.w", (d, 4 * d))]
        else:
            raise ValueError(variant)
    if variant == "gpt2":
        out += [("lnf.g", (d,)), ("lnf.b", (d,))]
    else:
        out += [("lm_head", (V, d))]
    r, _ = lora_of(cfg)
    for l in range(L):
        for t in ("q", "v"):
            out += [(f"h{l}.lora_{t}.A", (r, d)), (f"h{l}.lora_{t}.B", (d, r))] if r else []
    return out


def lora_of(cfg) -> Tuple[int, float]:
    """(rank r, branch scale lora_alpha / r), or (0, 0.0) without adapters.

    The fine-tuning article (LoRA section) names lora_alpha as the scaling factor;
    the scale applied to B A is alpha / r, as in the LoRA paper (Hu et al., 2021).
    """
    r = int(getattr(cfg, "lora_rank", 0) or 0)
    return (r, float(cfg.lora_alpha) / r) if r > 0 else (0, 0.0)


def trainable(cfg, name: str) -> bool:
    """With adapters only their A and B tensors train (the article freezes W0 and
    updates the low-rank matrices alone); otherwise every tensor does."""
    return ".lora_" in name if lora_of(cfg)[0] else True


def n_params(cfg, variant: str | None = None) -> int:
    return int(sum(int(np.prod(s)) for _, s in param_shapes(cfg, variant)))


def decays(name: str, shape) -> bool:
    """Weight decay applies to 2-D tensors only."""
    return len(shape) == 2


# --------------------------------------------------------------------------- dropout masks

_PHILOX_M = (0xD2511F53, 0xCD9E8D57)    # round multipliers of Philox4x32
_PHILOX_W = (0x9E3779B9, 0xBB67AE85)    # key increments (golden ratio, sqrt(3) - 1)
_U32 = np.uint64(0xFFFFFFFF)


def philox4x32(counter, key, rounds: int = 10):
    """Philox4x32-R of Salmon et al. (SC 2011): four 32-bit counter words and a
    two-word key to four 32-bit outputs.

    counter: uint array [..., 4]; key: two ints. Each round takes the 32x32->64
    products of counter words 0 and 2 with the two multipliers, and forms the new
    counter (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the
    key advances by the two Weyl increments between rounds. Returns uint64 [..., 4]
    holding 32-bit values.
    """
    c = np.asarray(counter, dtype=np.uint64)
    c0, c1, c2, c3 = (c[..., i] for i in range(4))
    k0, k1 = np.uint64(int(key[0]) & 0xFFFFFFFF), np.uint64(int(key[1]) & 0xFFFFFFFF)
    for r in range(rounds):
        if r:
            k0 = (k0 + np.uint64(_PHILOX_W[0])) & _U32
            k1 = (k1 + np.uint64(_PHILOX_W[1])) & _U32
        p0 = np.uint64(_PHILOX_M[0]) * c0       # < 2^64: exact in uint64
        p1 = np.uint64(_PHILOX_M[1]) * c2
        c0, c1, c2, c3 = (p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & _U32, (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & _U32
    return np.stack([c0, c1, c2, c3], axis=-1)


class Dropout:
    """Dropout rate p, the generator's 64-bit seed and the forward counter.

    An element is dropped when its 32-bit Philox word is below
    thr = floor(p * 2^32), so it is kept with probability 1 - thr / 2^32, and
    kept values are multiplied by scale = 1 / (1 - p) rounded to float32.
    ``call`` numbers the forward passes: each micro-batch forward uses the
    current value and then advances it (``next_call``).
    """

    def __init__(self, p: float, seed: int, call: int = 0):
        if not 0.0 <= p < 1.0:
            raise ValueError("dropout must be in [0, 1)")
        self.p = float(np.float32(p))
        self.seed = int(seed) & 0xFFFFFFFFFFFFFFFF
        self.call = int(call) & 0xFFFFFFFF
        self.thr = int(math.floor(self.p * 4294967296.0))
        self.scale = float(np.float32(1.0 / (1.0 - self.p)))

    def next_call(self) -> int:
        c = self.call
        self.call = (self.call + 1) & 0xFFFFFFFF
        return c


# Sites: 0 is the embedding output; layer l owns 3l+1 (attention probabilities),
# 3l+2 (attention branch output) and 3l+3 (MLP branch output).
def site_embed() -> int: return 0
def site_attn_prob(l: int) -> int: return 3 * l + 1
def site_attn_out(l: int) -> int: return 3 * l + 2
def site_mlp_out(l: int) -> int: return 3 * l + 3


def dropout_keep(drop: Dropout, call: int, site: int, rows, ncols: int) -> np.ndarray:
    """Keep mask [len(rows), ncols] of one site for one forward.

    Element (row, col) takes word col mod 4 of Philox4x32-10 at counter
    (col div 4, row, site, call) under the key (seed low word, seed high word).
    Rows and columns are those of the site's tensor: token rows b*T + t and
    channel columns for the embedding and branch outputs, and rows
    (b*H + h)*T + i by key columns j for the attention probabilities, with T the
    micro-batch's sequence length.
    """
    rows = np.asarray(rows, dtype=np.uint64)
    groups = np.arange((ncols + 3) // 4, dtype=np.uint64)
    ctr = np.empty((len(rows), len(groups), 4), dtype=np.uint64)
    ctr[..., 0] = groups[None, :]
    ctr[..., 1] = rows[:, None]
    ctr[..., 2] = site
    ctr[..., 3] = call
    words = philox4x32(ctr, (drop.seed & 0xFFFFFFFF, drop.seed >> 32)).reshape(len(rows), -1)[:, :ncols]
    return words >= np.uint64(drop.thr)


def _zmask(drop, call, site, rows, ncols, dtype):
    """Keep mask times the scale, as a multiplier in ``dtype``."""
    return dropout_keep(drop, call, site, rows, ncols).astype(dtype) * dtype(drop.scale)


# --------------------------------------------------------------------------- pieces

def layernorm_fwd(x, g, b):
    mu = x.mean(axis=-1, keepdims=True)
    xc = x - mu
    var = (xc * xc).mean(axis=-1, keepdims=True)     # biased variance
    rstd = 1.0 / np.sqrt(var + LN_EPS)
    xhat = xc * rstd
    return xhat * g + b, (xhat, rstd)


def layernorm_bwd(dy, cache, g):
    xhat, rstd = cache
    dg = (dy * xhat).sum(axis=0)
    db = dy.sum(axis=0)
    gh = dy * g
    dx = rstd * (gh - gh.mean(axis=-1, keepdims=True)
                 - xhat * (gh * xhat).mean(axis=-1, keepdims=True))
    return dx, dg, db


def rmsnorm_fwd(x):
    """Weightless RMSNorm: x / sqrt(mean(x^2) + eps) (the microGPT block's norm)."""
    rstd = 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + LN_EPS)
    xhat = x * rstd
    return xhat, (xhat, rstd)


def rmsnorm_bwd(dy, cache):
    xhat, rstd = cache
    return rstd * (dy - xhat * (dy * xhat).mean(axis=-1, keepdims=True))


def relu(u):
    return np.maximum(u, 0.0)


def relu_grad(u):
    return (u > 0.0).astype(u.dtype)


def gelu(u):
    """Exact GELU: u * Phi(u) with the standard normal CDF Phi."""
    return 0.5 * u * (1.0 + erf(u / math.sqrt(2.0)))


def gelu_grad(u):
    """d/du [u Phi(u)] = Phi(u) + u phi(u)."""
    cdf = 0.5 * (1.0 + erf(u / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * u * u) / math.sqrt(2.0 * math.pi)
    return cdf + u * pdf


def softmax_rows(s):
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def attention_fwd(q, k, v, z=None):
    """Causal attention for one sequence. q, k, v: [H, T, hd] -> O [H, T, hd], P.

    z, if given, is the dropout multiplier [H, T, T] applied to the
    probabilities after the softmax: O = (P * z) V. P is returned undropped.
    """
    T, hd = q.shape[1], q.shape[2]
    s = np.matmul(q, np.swapaxes(k, 1, 2)) / math.sqrt(hd)
    future = np.triu(np.ones((T, T), dtype=bool), 1)     # key j > query i
    s = np.where(future[None], -np.inf, s)
    p = softmax_rows(s)
    return np.matmul(p if z is None else p * z, v), p


def attention_bwd(dout, q, k, v, p, z=None):
    hd = q.shape[2]
    sc = 1.0 / math.sqrt(hd)
    pd = p if z is None else p * z
    dv = np.matmul(np.swapaxes(pd, 1, 2), dout)
    dp = np.matmul(dout, np.swapaxes(v, 1, 2))          # gradient of P * z
    if z is not None:
        dp = dp * z                                      # gradient of P
    ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))
    dq = np.matmul(ds, k) * sc
    dk = np.matmul(np.swapaxes(ds, 1, 2), q) * sc
    return dq, dk, dv


def xent_rows(z, y):
    """Per-row -log softmax(z)[y] and the softmax itself."""
    m = z.max(axis=-1, keepdims=True)
    e = np.exp(z - m)
    ssum = e.sum(axis=-1, keepdims=True)
    lse = (m + np.log(ssum))[:, 0]
    loss = lse - z[np.arange(len(y)), y]
    return loss, e / ssum


# --------------------------------------------------------------------------- model

def _as(params: Dict[str, np.ndarray], dtype) -> Dict[str, np.ndarray]:
    return {k: np.asarray(v, dtype=dtype) for k, v in params.items()}


def forward_sequence(P, tok, cfg, drop=None, b=0):
    """Forward pass of one sequence (tok: int [T]). Returns logits [T, Vp] and a cache.

    drop: None, or (Dropout, call) to apply dropout as sequence b of its
    micro-batch (which fixes the mask rows).
    """
    T = len(tok)
    d, H, L = cfg.n_embd, cfg.n_head, cfg.n_layer
    hd = d // H
    dt = P["wte"].dtype.type
    micro = variant_of(cfg) == "microgpt"
    r_lora, s_lora = lora_of(cfg)
    # microGPT: weightless RMSNorm, ReLU, no biases, its own lm_head
    norm = (lambda x, name: rmsnorm_fwd(x)) if micro else (lambda x, name: layernorm_fwd(x, P[name + ".g"], P[name + ".b"]))
    act = relu if micro else gelu
    bias = (lambda name: 0.0) if micro else (lambda name: P[name])
    if drop is not None:
        dr, call = drop
        tok_rows = b * T + np.arange(T)
        zm = lambda site: _zmask(dr, call, site, tok_rows, d, dt)
        head_rows = lambda: ((b * H + np.arange(H))[:, None] * T + np.arange(T)[None, :]).reshape(-1)
    x = P["wte"][tok] + P["wpe"][:T]
    ze = None
    if drop is not None:
        ze = zm(site_embed())
        x = x * ze
    layers = []
    for l in range(L):
        p = f"h{l}."
        a, c1 = norm(x, p + "ln1")
        qkv = a @ P[p + "attn.w"].T + bias(p + "attn.b")
        lo = None
        if r_lora:
            # low-rank branches on the q and v columns: s (a A^T) B^T
            uq = a @ P[p + "lora_q.A"].T
            uv = a @ P[p + "lora_v.A"].T
            qkv[:, :d] += s_lora * (uq @ P[p + "lora_q.B"].T)
            qkv[:, 2 * d:] += s_lora * (uv @ P[p + "lora_v.B"].T)
            lo = (uq, uv)
        q, k, v = (qkv[:, i * d:(i + 1) * d].reshape(T, H, hd).transpose(1, 0, 2) for i in range(3))
        zp = za = zo = None
        if drop is not None:
            zp = _zmask(dr, call, site_attn_prob(l), head_rows(), T, dt).reshape(H, T, T)
            za = zm(site_attn_out(l))
            zo = zm(site_mlp_out(l))
        o, pr = attention_fwd(q, k, v, zp)
        o2 = o.transpose(1, 0, 2).reshape(T, d)
        y1 = o2 @ P[p + "proj.w"].T + bias(p + "proj.b")
        x1 = x + (y1 if za is None else y1 * za)
        b2, c2 = norm(x1, p + "ln2")
        u = b2 @ P[p + "fc.w"].T + bias(p + "fc.b")
        h = act(u)
        y2 = h @ P[p + "fcproj.w"].T + bias(p + "fcproj.b")
        x2 = x1 + (y2 if zo is None else y2 * zo)
        layers.append((a, c1, q, k, v, pr, o2, b2, c2, u, h, zp, za, zo, lo))
        x = x2
    xf, cf = norm(x, "lnf")
    z = xf @ P["lm_head" if micro else "wte"].T
    return z, (tok, layers, xf, cf, ze)


def backward_sequence(P, cache, dz, cfg, G):
    """Adds the gradients of one sequence (given dL/dlogits) into G."""
    tok, layers, xf, cf, ze = cache
    T = len(tok)
    d, H, L = cfg.n_embd, cfg.n_head, cfg.n_layer
    hd = d // H
    micro = variant_of(cfg) == "microgpt"
    head = "lm_head" if micro else "wte"
    s_lora = lora_of(cfg)[1]

    def norm_bwd(dy, c, name):
        if micro:
            return rmsnorm_bwd(dy, c)
        dxn, dgn, dbn = layernorm_bwd(dy, c, P[name + ".g"])
        G[name + ".g"] += dgn
        G[name + ".b"] += dbn
        return dxn

    def add_bias(name, g):
        if not micro:
            G[name] += g.sum(axis=0)

    act_grad = relu_grad if micro else gelu_grad
    G[head] += dz.T @ xf
    dxf = dz @ P[head]
    dx = norm_bwd(dxf, cf, "lnf")
    for l in reversed(range(L)):
        p = f"h{l}."
        a, c1, q, k, v, pr, o2, b2, c2, u, h, zp, za, zo, lo = layers[l]
        # MLP: x2 = x1 + drop(gelu(LN2(x1) Wfc^T + bfc) Wp^T + bp)
        dy2 = dx if zo is None else dx * zo
        G[p + "fcproj.w"] += dy2.T @ h
        add_bias(p + "fcproj.b", dy2)
        du = (dy2 @ P[p + "fcproj.w"]) * act_grad(u)
        G[p + "fc.w"] += du.T @ b2
        add_bias(p + "fc.b", du)
        db2 = du @ P[p + "fc.w"]
        dx1 = dx + norm_bwd(db2, c2, p + "ln2")
        # attention: x1 = x + drop(attn(LN1(x)) Wo^T + bo)
        dy1 = dx1 if za is None else dx1 * za
        G[p + "proj.w"] += dy1.T @ o2
        add_bias(p + "proj.b", dy1)
        do2 = dy1 @ P[p + "proj.w"]
        do = do2.reshape(T, H, hd).transpose(1, 0, 2)
        dq, dk, dv = attention_bwd(do, q, k, v, pr, zp)
        dqkv = np.concatenate([t.transpose(1, 0, 2).reshape(T, d) for t in (dq, dk, dv)], axis=1)
        G[p + "attn.w"] += dqkv.T @ a
        add_bias(p + "attn.b", dqkv)
        da = dqkv @ P[p + "attn.w"]
        if lo is not None:
            # q (or v) = ... + s u B^T with u = a A^T
            for t, uu, dt_ in (("q", lo[0], dqkv[:, :d]), ("v", lo[1], dqkv[:, 2 * d:])):
                G[p + f"lora_{t}.B"] += s_lora * (dt_.T @ uu)
                du_ = s_lora * (dt_ @ P[p + f"lora_{t}.B"])
                G[p + f"lora_{t}.A"] += du_.T @ a
                da = da + du_ @ P[p + f"lora_{t}.A"]
        dx = dx1 + norm_bwd(da, c1, p + "ln1")
    # x0 = drop(wte[tok] + wpe[:T]); repeated ids add up.
    if ze is not None:
        dx = dx * ze
    np.add.at(G["wte"], tok, dx)
    G["wpe"][:T] += dx


def logits(params, tokens, cfg, dtype=np.float64):
    P = _as(params, dtype)
    return np.stack([forward_sequence(P, np.asarray(t), cfg)[0] for t in tokens])


def microbatch(params, tokens, targets, cfg, grad_scale=None, dtype=np.float64,
               grads=None, rows=None, dropout=None, call=None):
    """Loss of one micro-batch and (optionally) its gradient.

    tokens, targets: int [B, T]. The loss is the mean over all B*T positions.
    When ``grad_scale`` is given, adds grad_scale * d(sum of row losses)/dθ
    into ``grads`` (created if None) and returns it; the caller picks
    grad_scale = 1 / (B * T * A) for A accumulated micro-batches.
    ``rows`` optionally limits the work to a subset of sequences (their
    per-position losses are still returned in place, others are NaN).
    ``dropout`` (a Dropout) applies dropout with forward counter ``call``
    (default: the next value of the Dropout's counter).
    """
    P = _as(params, dtype)
    tokens = np.asarray(tokens)
    targets = np.asarray(targets)
    B, T = tokens.shape
    if grad_scale is not None and grads is None:
        grads = {k: np.zeros_like(v) for k, v in P.items()}
    row_loss = np.full((B, T), np.nan, dtype=dtype)
    drop = None
    if dropout is not None:
        c = dropout.next_call() if call is None else call    # advances for p = 0 too
        if dropout.p > 0.0:
            drop = (dropout, c)
    for b in (range(B) if rows is None else rows):
        z, cache = forward_sequence(P, tokens[b], cfg, drop, b)
        ell, sm = xent_rows(z, targets[b])
        row_loss[b] = ell
        if grad_scale is not None:
            dz = sm
            dz[np.arange(T), targets[b]] -= 1.0
            dz *= grad_scale
            backward_sequence(P, cache, dz, cfg, grads)
    return row_loss, grads


def accumulate_grads(params, batches, cfg, dtype=np.float64, dropout=None, progress=None):
    """Mean loss over A micro-batches and the gradient of that mean.

    With a Dropout, micro-batch i takes the Dropout's next forward counter.
    progress (optional) is called with (i, loss_i) after each micro-batch; it
    only reports, it takes no part in the arithmetic.
    """
    A = len(batches)
    grads = None
    losses = []
    for i, (tok, tgt) in enumerate(batches):
        B, T = tok.shape
        rl, grads = microbatch(params, tok, tgt, cfg, grad_scale=1.0 / (B * T * A),
                               dtype=dtype, grads=grads, dropout=dropout)
        losses.append(float(rl.mean()))
        if progress is not None:
            progress(i, losses[-1])
    return losses, grads


def relu_gate_band(params, batches, cfg, rel_round: float = 2.0 ** -7, dtype=np.float64,
                   dropout=None, call0: int = 0):
    """How far the gradient of one step can move when the ReLU gates that lie within
    operand rounding of zero change side (the microGPT block: ReLU in the MLP,
    "Building microGPT from scratch", model-core section).

    A gate is ambiguous when |u| <= rel_round * sum_k |b_k| |W_jk|, with u = b W^T the
    pre-activation of MLP column j and b the normed input: rel_round = 2^-7 is the
    relative rounding of a product of two operands each rounded to bf16 (8
    significant bits, half an ulp each), so such a u may take either sign once its
    operands are rounded. Every ambiguous gate is flipped in the backward (the
    forward output ReLU(u) moves by at most |u|, within rounding, and is left alone)
    and the step's gradients are formed again. Returns ({tensor: ||G_flip - G|| /
    ||G||}, with "__all__" for the whole gradient vector, and the fraction of
    gates that are ambiguous). A rounded computation flips some subset of these
    gates; their effects add with random signs, so flipping all of them gives the
    scale of the deviation such flips cause. Uses the oracle's own values only.

    dropout / call0: a Dropout, and the forward counter of the first micro-batch
    (micro-batch i uses call0 + i), as accumulate_grads would draw them.
    """
    if variant_of(cfg) != "microgpt":
        raise ValueError("only the ReLU block has gates")
    P = _as(params, dtype)
    A = len(batches)
    G0 = {k: np.zeros_like(v) for k, v in P.items()}
    G1 = {k: np.zeros_like(v) for k, v in P.items()}
    amb_n = tot_n = 0
    for i, (tok, tgt) in enumerate(batches):
        tok, tgt = np.asarray(tok), np.asarray(tgt)
        B, T = tok.shape
        drop = (dropout, (call0 + i) & 0xFFFFFFFF) if dropout is not None and dropout.p > 0.0 else None
        for b in range(B):
            z, cache = forward_sequence(P, tok[b], cfg, drop, b)
            _, sm = xent_rows(z, tgt[b])
            dz = sm
            dz[np.arange(T), tgt[b]] -= 1.0
            dz *= 1.0 / (B * T * A)
            backward_sequence(P, cache, dz, cfg, G0)
            layers = []
            for l, lay in enumerate(cache[1]):
                b2, u = lay[7], lay[9]
                scale = np.abs(b2) @ np.abs(P[f"h{l}.fc.w"]).T
                amb = np.abs(u) <= rel_round * scale
                amb_n += int(amb.sum())
                tot_n += amb.size
                # the backward reads u only through the gate (u > 0): give every
                # ambiguous element the other side
                uf = np.where(amb, np.where(u > 0.0, -1.0, 1.0), u)
                layers.append(lay[:9] + (uf,) + lay[10:])
            backward_sequence(P, (cache[0], layers) + tuple(cache[2:]), dz, cfg, G1)
    band = {k: float(np.linalg.norm(G1[k] - G0[k]) / max(np.linalg.norm(G0[k]), 1e-300)) for k in P}
    num = math.sqrt(sum(float(np.sum(np.square(G1[k] - G0[k]))) for k in P))
    band["__all__"] = num / max(grad_norm(G0), 1e-300)
    return band, amb_n / max(tot_n, 1)


def grad_norm(grads) -> float:
    return math.sqrt(sum(float(np.sum(np.square(g, dtype=np.float64))) for g in grads.values()))


def clip_coef(norm: float, clip: float) -> float:
    if clip <= 0.0:
        return 1.0
    return min(1.0, clip / (norm + CLIP_EPS))


def adamw_update(params, grads, m, v, t, lr, beta1, beta2, eps, wd, coef, decay_mask, keys=None):
    """One AdamW update in place of the tensors ``keys`` (default: all of
    ``params``). t is the step number after increment (>= 1).

    Decoupled decay first: p <- p (1 - lr wd) for decayed tensors, then
    p <- p - lr * mhat / (sqrt(vhat) + eps) with bias-corrected moments.
    """
    bc1 = 1.0 - beta1 ** t
    bc2 = 1.0 - beta2 ** t
    for k in (params if keys is None else keys):
        g = grads[k] * coef
        m[k] = beta1 * m[k] + (1.0 - beta1) * g
        v[k] = beta2 * v[k] + (1.0 - beta2) * g * g
        mhat = m[k] / bc1
        vhat = v[k] / bc2
        if decay_mask[k]:
            params[k] = params[k] * (1.0 - lr * wd)
        params[k] = params[k] - lr * mhat / (np.sqrt(vhat) + eps)


class Trainer:
    """Full optimizer steps on the oracle: accumulate, clip, AdamW."""

    def __init__(self, params, cfg, dtype=np.float64, dropout=None):
        self.cfg = cfg
        self.dropout = dropout
        self.dtype = dtype
        self.p = _as(params, dtype)
        self.m = {k: np.zeros_like(v) for k, v in self.p.items()}
        self.v = {k: np.zeros_like(v) for k, v in self.p.items()}
        self.t = 0
        self.decay = {k: decays(k, v.shape) for k, v in self.p.items()}
        self.train = [k for k in self.p if trainable(cfg, k)]

    def step(self, batches, lr=None, beta1=None, beta2=None, eps=None, wd=None, clip=None, progress=None):
        c = self.cfg
        lr = c.lr if lr is None else lr
        beta1 = c.beta1 if beta1 is None else beta1
        beta2 = c.beta2 if beta2 is None else beta2
        eps = c.eps if eps is None else eps
        wd = c.weight_decay if wd is None else wd
        clip = c.grad_clip if clip is None else clip
        losses, grads = accumulate_grads(self.p, batches, c, self.dtype, self.dropout, progress)
        grads = {k: grads[k] for k in self.train}     # frozen tensors take no part
        norm = grad_norm(grads)
        coef = clip_coef(norm, clip)
        self.t += 1
        adamw_update(self.p, grads, self.m, self.v, self.t, lr, beta1, beta2, eps, wd,
                     coef, self.decay, keys=self.train)
        return {"losses": losses, "loss": float(np.mean(losses)), "grads": grads,
                "norm": norm, "coef": coef}


# --------------------------------------------------------------------------- generation

def sample_token(z, temperature: float, top_k: int, u: float) -> int:
    """One next token from a row of logits z [V] and a uniform u in [0, 1).

    temperature <= 0: the argmax, lowest index on ties. Otherwise the candidates
    are the logits >= the k-th largest value (all V when top_k <= 0 or >= V; ties
    at the cut stay in, as nanoGPT's sampler keeps them), weighted by
    exp((z_i - max z) / temperature); the token is the smallest index whose
    cumulative weight, summed in index order, exceeds u times the total.
    """
    z = np.asarray(z, dtype=np.float64)
    if temperature <= 0.0:
        return int(np.argmax(z))
    V = z.shape[0]
    cand = np.ones(V, dtype=bool)
    if 0 < top_k < V:
        kth = np.sort(z)[V - top_k]
        cand = z >= kth
    w = np.where(cand, np.exp((z - z.max()) / temperature), 0.0)
    c = np.cumsum(w)
    return int(np.searchsorted(c, u * c[-1], side="right"))


def generate(params, prompt, cfg, n_new: int, temperature: float, top_k: int, uniforms,
             dtype=np.float64):
    """Autoregressive generation by full recomputation, no cache.

    prompt: int [B, T0]; uniforms: [n_new, B] in [0, 1). Returns the tokens
    [B, T0 + n_new] and the logits of every generated position [n_new, B, Vp]
    (the last row of the forward over the sequence so far).
    """
    P = _as(params, dtype)
    seqs = [list(map(int, r)) for r in np.asarray(prompt)]
    zs = []
    for s in range(n_new):
        row = []
        for b, seq in enumerate(seqs):
            z, _ = forward_sequence(P, np.asarray(seq), cfg)
            row.append(z[-1])
            seq.append(sample_token(z[-1], temperature, top_k, float(uniforms[s][b])))
        zs.append(np.stack(row))
    return np.asarray(seqs), np.stack(zs)

