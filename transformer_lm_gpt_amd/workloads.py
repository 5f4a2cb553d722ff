"""Workload presets and seeded synthetic inputs for the GPT training step.

This module is shared by the HIP path's callers (tests, bench) and by the
checks that feed the CPU oracle. It holds no arithmetic of the method: only the
five configurations, the random weight initialisation and the synthetic token
streams. Both sides receive exactly the same float32 weights and int32 tokens.

Sources for the presets (the nanoGPT pages):
  * "Building microGPT from scratch" (blog.hotdry.top), model-core section:
    vocab 27, n_embd 16, 4 heads of dim 4, one layer, block 16, Gaussian init
    with std 0.08; training-loop section: Adam with betas 0.85/0.99, eps 1e-8,
    lr 1e-2.
  * nanoGPT README translation (oa0.com), the CPU quick-start run: 4 layers,
    4 heads, n_embd 128, block 64, batch 12, dropout 0, char vocab 65.
  * "GPT training and inference from scratch with nanoGPT" (adg.csdn.net) and
    the microGPT page's parameter table: the 6-layer, 6-head, 384-d
    Shakespeare-char model at block 256, batch 64.
  * nanoGPT run log (wmrh.cn) section 2.1: 12 layers, 8 heads, n_embd 512,
    block 512, batch 12, BPE vocab 50257, lr 6e-4, wd 0.1, betas 0.9/0.95.
  * "Fine-tuning pipelines for medium GPTs with nanoGPT, LoRA and multi-GPU"
    (blog.hotdry.top): GPT-2 small (12/12/768), block 1024, batch 12 per GPU
    with gradient accumulation; 50257-token BPE ids stored as uint16.
  * The run log, section 4.5: seed 1337.

The datasets behind these pages (names.txt, tinyshakespeare, OpenWebText) are
not available; seeded synthetic streams with the same vocabularies and shapes
stand in for them.
"""
from __future__ import annotations

import bisect
from dataclasses import dataclass, field, replace
from typing import Dict, List, Tuple

import numpy as np

SEED = 1337


@dataclass(frozen=True)
class GPTConfig:
    name: str
    vocab_size: int          # ids drawn from [0, vocab_size)
    padded_vocab: int        # rows of wte == softmax width
    n_layer: int
    n_head: int
    n_embd: int
    block_size: int
    batch: int               # micro-batch B
    grad_accum: int          # micro-batches per optimizer step A
    init_std: float
    resid_scaled: bool       # residual projections scaled by 1/sqrt(2 L)
    data: str                # "uniform" | "zipf_stream" | "markov_stream" | "zipf_batch"
    zipf_s: float = 0.0
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.99
    eps: float = 1e-8
    weight_decay: float = 0.1
    grad_clip: float = 1.0
    parity_steps: int = 1
    precisions: Tuple[str, ...] = ("bf16",)
    variant: str = "gpt2"    # "gpt2" | "microgpt" (weightless RMSNorm, ReLU, no biases, untied head)
    lora_rank: int = 0       # r > 0: low-rank adapters on the q and v projections, only they train
    lora_alpha: float = 16.0 # the adapters' branch is scaled by lora_alpha / r

    @property
    def head_dim(self) -> int:
        return self.n_embd // self.n_head

    def with_(self, **kw) -> "GPTConfig":
        return replace(self, **kw)


CONFIGS: Dict[str, GPTConfig] = {
    # microGPT-sized toy: uniform ids, fp32, 10 optimizer steps, constant lr,
    # no weight decay and no clipping (microGPT's Adam has neither).
    "tiny": GPTConfig("tiny", 27, 27, 1, 4, 16, 16, 4, 1, 0.08, False, "uniform",
                      lr=1e-2, beta1=0.85, beta2=0.99, eps=1e-8, weight_decay=0.0,
                      grad_clip=0.0, parity_steps=10, precisions=("fp32",)),
    # nanoGPT CPU run shape over a Zipf(1.1) char stream.
    "char_small": GPTConfig("char_small", 65, 65, 4, 4, 128, 64, 12, 1, 0.02, False,
                            "zipf_stream", zipf_s=1.1, lr=1e-3, beta1=0.9, beta2=0.99,
                            weight_decay=0.1, grad_clip=1.0, parity_steps=3,
                            precisions=("fp32", "bf16")),
    # Shakespeare-char baseline shape over an order-1 Markov char stream.
    "char_6l": GPTConfig("char_6l", 65, 65, 6, 6, 384, 256, 64, 1, 0.02, False,
                         "markov_stream", lr=1e-3, beta1=0.9, beta2=0.99,
                         weight_decay=0.1, grad_clip=1.0, parity_steps=3),
    # The run log's 12-layer, 512-wide BPE model at block 512.
    "bpe_12l_512": GPTConfig("bpe_12l_512", 50257, 50304, 12, 8, 512, 512, 12, 1, 0.02,
                             True, "zipf_batch", zipf_s=1.07, lr=6e-4, beta1=0.9,
                             beta2=0.95, weight_decay=0.1, grad_clip=1.0, parity_steps=1),
    # GPT-2 124M at T=1024, micro-batch 12, 5 accumulation steps.
    "gpt2_124m": GPTConfig("gpt2_124m", 50257, 50304, 12, 12, 768, 1024, 12, 5, 0.02,
                           True, "zipf_batch", zipf_s=1.07, lr=6e-4, beta1=0.9,
                           beta2=0.95, weight_decay=0.1, grad_clip=1.0, parity_steps=1),
}

ORDER = ["tiny", "char_small", "char_6l", "bpe_12l_512", "gpt2_124m"]

# The microGPT block ("Building microGPT from scratch", model-core section) at the
# page's own size (4,192 parameters) and at the char_small shape.
CONFIGS["micro"] = CONFIGS["tiny"].with_(name="micro", variant="microgpt")
CONFIGS["char_small_micro"] = CONFIGS["char_small"].with_(name="char_small_micro", variant="microgpt")
# the block at the GPT-2 124M shape, for throughput
CONFIGS["gpt2_124m_micro"] = CONFIGS["gpt2_124m"].with_(name="gpt2_124m_micro", variant="microgpt")
VARIANT_CONFIGS = ["micro", "char_small_micro", "gpt2_124m_micro"]
# LoRA fine-tuning (the fine-tuning article on blog.hotdry.top, LoRA section:
# adapters on the q and v projections, lora_alpha 16, r from 16 down) on the
# toy, the char_small shape and GPT-2 124M.
CONFIGS["tiny_lora"] = CONFIGS["tiny"].with_(name="tiny_lora", lora_rank=4, lora_alpha=16.0)
CONFIGS["char_small_lora"] = CONFIGS["char_small"].with_(name="char_small_lora", lora_rank=8, lora_alpha=16.0)
CONFIGS["gpt2_124m_lora"] = CONFIGS["gpt2_124m"].with_(name="gpt2_124m_lora", lora_rank=16, lora_alpha=16.0)
LORA_CONFIGS = ["tiny_lora", "char_small_lora", "gpt2_124m_lora"]


def rngs(seed: int = SEED) -> Tuple[np.random.Generator, np.random.Generator]:
    """(data stream, weight stream): two independent PCG64 generators."""
    data_ss, weight_ss = np.random.SeedSequence(seed).spawn(2)
    return np.random.Generator(np.random.PCG64(data_ss)), np.random.Generator(np.random.PCG64(weight_ss))


# --------------------------------------------------------------------------- weights

def tensor_table(cfg: GPTConfig) -> List[Tuple[str, Tuple[int, ...]]]:
    """Names and shapes of the trainable tensors, linear weights as [out, in]."""
    V, d, T, L = cfg.padded_vocab, cfg.n_embd, cfg.block_size, cfg.n_layer
    out = [("wte", (V, d)), ("wpe", (T, d))]
    if cfg.variant == "microgpt":
        for l in range(L):
            p = f"h{l}."
            out += [(p + "attn.w", (3 * d, d)), (p + "proj.w", (d, d)),
                    (p + "fc.w", (4 * d, d)), (p + "fcproj.w", (d, 4 * d))]
        return out + [("lm_head", (V, d))] + _lora_table(cfg)
    for l in range(L):
        p = f"h{l}."
        out += [(p + "ln1.g", (d,)), (p + "ln1.b", (d,)),
                (p + "attn.w", (3 * d, d)), (p + "attn.b", (3 * d,)),
                (p + "proj.w", (d, d)), (p + "proj.b", (d,)),
                (p + "ln2.g", (d,)), (p + "ln2.b", (d,)),
                (p + "fc.w", (4 * d, d)), (p + "fc.b", (4 * d,)),
                (p + "fcproj.w", (d, 4 * d)), (p + "fcproj.b", (d,))]
    out += [("lnf.g", (d,)), ("lnf.b", (d,))]
    return out + _lora_table(cfg)


def _lora_table(cfg: GPTConfig) -> List[Tuple[str, Tuple[int, ...]]]:
    """The adapters, after every base tensor: per block A [r, d] and B [d, r] for q, then v."""
    r, d = cfg.lora_rank, cfg.n_embd
    out: List[Tuple[str, Tuple[int, ...]]] = []
    for l in range(cfg.n_layer if r > 0 else 0):
        for t in ("q", "v"):
            out += [(f"h{l}.lora_{t}.A", (r, d)), (f"h{l}.lora_{t}.B", (d, r))]
    return out


def init_params(cfg: GPTConfig, rng: np.random.Generator | None = None,
                perturb: bool = False) -> Dict[str, np.ndarray]:
    """Float32 weights: matrices and embeddings N(0, std), residual projections
    optionally scaled by 1/sqrt(2 L), biases 0, LayerNorm gain 1 and shift 0.

    With ``perturb`` the biases, gains and shifts get small random values too, so
    that parity checks exercise every term (an all-zero bias hides a dropped add).
    Adapters: A is N(0, std) and B is 0 (so training starts from the base model),
    B N(0, std) too with ``perturb``.
    """
    if rng is None:
        rng = rngs()[1]
    params: Dict[str, np.ndarray] = {}
    for name, shape in tensor_table(cfg):
        leaf = name.split(".")[-1]
        if ".lora_" in name and leaf == "B" and not perturb:
            a = np.zeros(shape)
        elif len(shape) == 2:
            std = cfg.init_std
            if cfg.resid_scaled and (name.endswith("proj.w")):
                std = std / np.sqrt(2.0 * cfg.n_layer)
            a = rng.normal(0.0, std, size=shape)
        elif leaf == "g":
            a = np.ones(shape) + (rng.normal(0.0, 0.1, size=shape) if perturb else 0.0)
        else:
            a = rng.normal(0.0, 0.02, size=shape) if perturb else np.zeros(shape)
        params[name] = np.ascontiguousarray(a, dtype=np.float32)
    return params


# --------------------------------------------------------------------------- tokens

def zipf_cdf(n: int, s: float) -> np.ndarray:
    """CDF over ids 0..n-1 with p(id) proportional to (id + 1)^-s."""
    w = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(w)
    return c / c[-1]


def _draw(cdf: np.ndarray, u: np.ndarray) -> np.ndarray:
    return np.minimum(np.searchsorted(cdf, u, side="right"), len(cdf) - 1).astype(np.int32)


_STREAM_LEN = 1 << 20
_stream_cache: Dict[Tuple[str, int], np.ndarray] = {}


def token_stream(cfg: GPTConfig, seed: int = SEED) -> np.ndarray:
    """A long uint16-range id stream for the stream-backed presets (cached)."""
    key = (cfg.data + f":{cfg.vocab_size}:{cfg.zipf_s}", seed)
    if key in _stream_cache:
        return _stream_cache[key]
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    V = cfg.vocab_size
    if cfg.data == "zipf_stream":
        s = _draw(zipf_cdf(V, cfg.zipf_s), rng.random(_STREAM_LEN))
    elif cfg.data == "markov_stream":
        rows = rng.dirichlet(np.full(V, 0.1), size=V)
        cum = [list(np.cumsum(r) / np.sum(r)) for r in rows]
        u = rng.random(_STREAM_LEN).tolist()
        state = int(rng.integers(0, V))
        out = [0] * _STREAM_LEN
        for i in range(_STREAM_LEN):
            state = min(bisect.bisect_right(cum[state], u[i]), V - 1)
            out[i] = state
        s = np.asarray(out, dtype=np.int32)
    else:
        raise ValueError(cfg.data)
    _stream_cache[key] = s
    return s


def make_batch(cfg: GPTConfig, rng: np.random.Generator, B: int | None = None,
               T: int | None = None) -> Tuple[np.ndarray, np.ndarray]:
    """One micro-batch (tokens, targets), int32 [B, T]; targets are tokens shifted by one."""
    B = cfg.batch if B is None else B
    T = cfg.block_size if T is None else T
    V = cfg.vocab_size
    if cfg.data == "uniform":
        w = rng.integers(0, V, size=(B, T + 1)).astype(np.int32)
    elif cfg.data == "zipf_batch":
        w = _draw(zipf_cdf(V, cfg.zipf_s), rng.random((B, T + 1)))
    else:
        s = token_stream(cfg)
        offs = rng.integers(0, len(s) - T - 1, size=B)
        w = np.stack([s[o:o + T + 1] for o in offs]).astype(np.int32)
    return np.ascontiguousarray(w[:, :T]), np.ascontiguousarray(w[:, 1:])


def make_step_batches(cfg: GPTConfig, rng: np.random.Generator, A: int | None = None,
                      B: int | None = None, T: int | None = None):
    A = cfg.grad_accum if A is None else A
    return [make_batch(cfg, rng, B, T) for _ in range(A)]
