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

def param_shapes(cfg, variant: str = "gpt2") -> List[Tuple[str, Tuple[int, ...]]]:
    """Trainable tensors. Linear weights are [out, in] and act as y = x W^T + b.

    variant "gpt2": LayerNorm gain/shift, biased linears, tied head.
    variant "microgpt": the microGPT block (weightless RMSNorm, no biases,
    separate q/k/v/o matrices, untied lm_head) used only to check the page's
    printed parameter count.
    """
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
            out += [(p + "wq", (d, d)), (p + "wk", (d, d)), (p + "wv", (d, d)),
                    (p + "wo", (d, d)), (p + "fc1", (4 * d, d)), (p + "fc2", (d, 4 * d))]
        else:
            raise ValueError(variant)
    if variant == "gpt2":
        out += [("lnf.g", (d,)), ("lnf.b", (d,))]
    else:
        out += [("lm_head", (V, d))]
    return out


def n_params(cfg, variant: str = "gpt2") -> int:
    return int(sum(int(np.prod(s)) for _, s in param_shapes(cfg, variant)))


def decays(name: str, shape) -> bool:
    """Weight decay applies to 2-D tensors only."""
    return len(shape) == 2


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


def attention_fwd(q, k, v):
    """Causal attention for one sequence. q, k, v: [H, T, hd] -> O [H, T, hd], P."""
    T, hd = q.shape[1], q.shape[2]
    s = np.matmul(q, np.swapaxes(k, 1, 2)) / math.sqrt(hd)
    future = np.triu(np.ones((T, T), dtype=bool), 1)     # key j > query i
    s = np.where(future[None], -np.inf, s)
    p = softmax_rows(s)
    return np.matmul(p, v), p


def attention_bwd(dout, q, k, v, p):
    hd = q.shape[2]
    sc = 1.0 / math.sqrt(hd)
    dv = np.matmul(np.swapaxes(p, 1, 2), dout)
    dp = np.matmul(dout, np.swapaxes(v, 1, 2))
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


def forward_sequence(P, tok, cfg):
    """Forward pass of one sequence (tok: int [T]). Returns logits [T, Vp] and a cache."""
    T = len(tok)
    d, H, L = cfg.n_embd, cfg.n_head, cfg.n_layer
    hd = d // H
    x = P["wte"][tok] + P["wpe"][:T]
    layers = []
    for l in range(L):
        p = f"h{l}."
        a, c1 = layernorm_fwd(x, P[p + "ln1.g"], P[p + "ln1.b"])
        qkv = a @ P[p + "attn.w"].T + P[p + "attn.b"]
        q, k, v = (qkv[:, i * d:(i + 1) * d].reshape(T, H, hd).transpose(1, 0, 2) for i in range(3))
        o, pr = attention_fwd(q, k, v)
        o2 = o.transpose(1, 0, 2).reshape(T, d)
        x1 = x + o2 @ P[p + "proj.w"].T + P[p + "proj.b"]
        b2, c2 = layernorm_fwd(x1, P[p + "ln2.g"], P[p + "ln2.b"])
        u = b2 @ P[p + "fc.w"].T + P[p + "fc.b"]
        h = gelu(u)
        x2 = x1 + h @ P[p + "fcproj.w"].T + P[p + "fcproj.b"]
        layers.append((a, c1, q, k, v, pr, o2, b2, c2, u, h))
        x = x2
    xf, cf = layernorm_fwd(x, P["lnf.g"], P["lnf.b"])
    z = xf @ P["wte"].T
    return z, (tok, layers, xf, cf)


def backward_sequence(P, cache, dz, cfg, G):
    """Adds the gradients of one sequence (given dL/dlogits) into G."""
    tok, layers, xf, cf = cache
    T = len(tok)
    d, H, L = cfg.n_embd, cfg.n_head, cfg.n_layer
    hd = d // H
    G["wte"] += dz.T @ xf
    dxf = dz @ P["wte"]
    dx, dg, db = layernorm_bwd(dxf, cf, P["lnf.g"])
    G["lnf.g"] += dg
    G["lnf.b"] += db
    for l in reversed(range(L)):
        p = f"h{l}."
        a, c1, q, k, v, pr, o2, b2, c2, u, h = layers[l]
        # MLP: x2 = x1 + gelu(LN2(x1) Wfc^T + bfc) Wp^T + bp
        G[p + "fcproj.w"] += dx.T @ h
        G[p + "fcproj.b"] += dx.sum(axis=0)
        du = (dx @ P[p + "fcproj.w"]) * gelu_grad(u)
        G[p + "fc.w"] += du.T @ b2
        G[p + "fc.b"] += du.sum(axis=0)
        db2 = du @ P[p + "fc.w"]
        dln, dg, dbb = layernorm_bwd(db2, c2, P[p + "ln2.g"])
        G[p + "ln2.g"] += dg
        G[p + "ln2.b"] += dbb
        dx1 = dx + dln
        # attention: x1 = x + attn(LN1(x)) Wo^T + bo
        G[p + "proj.w"] += dx1.T @ o2
        G[p + "proj.b"] += dx1.sum(axis=0)
        do2 = dx1 @ P[p + "proj.w"]
        do = do2.reshape(T, H, hd).transpose(1, 0, 2)
        dq, dk, dv = attention_bwd(do, q, k, v, pr)
        dqkv = np.concatenate([t.transpose(1, 0, 2).reshape(T, d) for t in (dq, dk, dv)], axis=1)
        G[p + "attn.w"] += dqkv.T @ a
        G[p + "attn.b"] += dqkv.sum(axis=0)
        da = dqkv @ P[p + "attn.w"]
        dln, dg, dbb = layernorm_bwd(da, c1, P[p + "ln1.g"])
        G[p + "ln1.g"] += dg
        G[p + "ln1.b"] += dbb
        dx = dx1 + dln
    # x0 = wte[tok] + wpe[:T]; repeated ids add up.
    np.add.at(G["wte"], tok, dx)
    G["wpe"][:T] += dx


def logits(params, tokens, cfg, dtype=np.float64):
    P = _as(params, dtype)
    return np.stack([forward_sequence(P, np.asarray(t), cfg)[0] for t in tokens])


def microbatch(params, tokens, targets, cfg, grad_scale=None, dtype=np.float64,
               grads=None, rows=None):
    """Loss of one micro-batch and (optionally) its gradient.

    tokens, targets: int [B, T]. The loss is the mean over all B*T positions.
    When ``grad_scale`` is given, adds grad_scale * d(sum of row losses)/dθ
    into ``grads`` (created if None) and returns it; the caller picks
    grad_scale = 1 / (B * T * A) for A accumulated micro-batches.
    ``rows`` optionally limits the work to a subset of sequences (their
    per-position losses are still returned in place, others are NaN).
    """
    P = _as(params, dtype)
    tokens = np.asarray(tokens)
    targets = np.asarray(targets)
    B, T = tokens.shape
    if grad_scale is not None and grads is None:
        grads = {k: np.zeros_like(v) for k, v in P.items()}
    row_loss = np.full((B, T), np.nan, dtype=dtype)
    for b in (range(B) if rows is None else rows):
        z, cache = forward_sequence(P, tokens[b], cfg)
        ell, sm = xent_rows(z, targets[b])
        row_loss[b] = ell
        if grad_scale is not None:
            dz = sm
            dz[np.arange(T), targets[b]] -= 1.0
            dz *= grad_scale
            backward_sequence(P, cache, dz, cfg, grads)
    return row_loss, grads


def accumulate_grads(params, batches, cfg, dtype=np.float64):
    """Mean loss over A micro-batches and the gradient of that mean."""
    A = len(batches)
    grads = None
    losses = []
    for tok, tgt in batches:
        B, T = tok.shape
        rl, grads = microbatch(params, tok, tgt, cfg, grad_scale=1.0 / (B * T * A),
                               dtype=dtype, grads=grads)
        losses.append(float(rl.mean()))
    return losses, grads


def grad_norm(grads) -> float:
    return math.sqrt(sum(float(np.sum(np.square(g, dtype=np.float64))) for g in grads.values()))


def clip_coef(norm: float, clip: float) -> float:
    if clip <= 0.0:
        return 1.0
    return min(1.0, clip / (norm + CLIP_EPS))


def adamw_update(params, grads, m, v, t, lr, beta1, beta2, eps, wd, coef, decay_mask):
    """One AdamW update in place. t is the step number after increment (>= 1).

    Decoupled decay first: p <- p (1 - lr wd) for decayed tensors, then
    p <- p - lr * mhat / (sqrt(vhat) + eps) with bias-corrected moments.
    """
    bc1 = 1.0 - beta1 ** t
    bc2 = 1.0 - beta2 ** t
    for k in params:
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

    def __init__(self, params, cfg, dtype=np.float64):
        self.cfg = cfg
        self.dtype = dtype
        self.p = _as(params, dtype)
        self.m = {k: np.zeros_like(v) for k, v in self.p.items()}
        self.v = {k: np.zeros_like(v) for k, v in self.p.items()}
        self.t = 0
        self.decay = {k: decays(k, v.shape) for k, v in self.p.items()}

    def step(self, batches, lr=None, beta1=None, beta2=None, eps=None, wd=None, clip=None):
        c = self.cfg
        lr = c.lr if lr is None else lr
        beta1 = c.beta1 if beta1 is None else beta1
        beta2 = c.beta2 if beta2 is None else beta2
        eps = c.eps if eps is None else eps
        wd = c.weight_decay if wd is None else wd
        clip = c.grad_clip if clip is None else clip
        losses, grads = accumulate_grads(self.p, batches, c, self.dtype)
        norm = grad_norm(grads)
        coef = clip_coef(norm, clip)
        self.t += 1
        adamw_update(self.p, grads, self.m, self.v, self.t, lr, beta1, beta2, eps, wd,
                     coef, self.decay)
        return {"losses": losses, "loss": float(np.mean(losses)), "grads": grads,
                "norm": norm, "coef": coef}
