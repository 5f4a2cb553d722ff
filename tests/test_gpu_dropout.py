"""Dropout on the HIP path against the oracle: both sides draw every mask from
Philox4x32-10 under the same seed and forward counter, so the step is the same
function on both sides and the tolerances of the undropped step apply."""
import numpy as np
import pytest

from oracle import gpt_oracle as O
from transformer_lm_gpt_amd import workloads as W

from gpu_helpers import new_model, run_steps, say

pytestmark = pytest.mark.gpu

SEED = 0x5EED0123456789AB


@pytest.mark.parametrize("name,prec,p,steps,B,T,A", [
    ("tiny", "fp32", 0.1, 3, None, None, None),
    ("tiny", "fp32", 0.3, 2, 3, 11, 2),           # T not a multiple of 4: mask blocks straddle rows
    ("char_small", "fp32", 0.2, 2, None, None, None),
    ("char_small", "bf16", 0.2, 2, None, None, None),
    ("char_small", "bf16", 0.2, 2, 5, 37, 3),     # head_dim 32 register-resident kernels, ragged tile
    ("char_6l", "bf16", 0.1, 2, 8, None, 2),      # head_dim 64 register-resident kernels
    ("char_6l", "bf16", 0.2, 2, 2, 150, 2),       # ... with a ragged last tile
])
def test_dropout_step_parity(name, prec, p, steps, B, T, A):
    run_steps(name, prec, steps=steps, B=B, T=T, A=A, dropout=p, seed=SEED, counter=5)


def test_dropout_embedding_mask_bit_exact():
    """fp32: x0 = (wte[tok] + wpe) * z with one rounding per operation on both
    sides, so the embedding output, and with it the mask, matches bit for bit."""
    import torch
    cfg = W.CONFIGS["char_small"]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng)
    tok, tgt = W.make_batch(cfg, drng)
    d = O.Dropout(0.25, SEED, 9)
    gpu = new_model(cfg, "fp32", dropout=0.25)
    gpu.load_params(params)
    gpu.set_dropout_seed(SEED, 9)
    gpu.forward_loss(tok, tgt)
    B, T, C = tok.shape[0], tok.shape[1], cfg.n_embd
    x0 = gpu.debug("x", 0, (B, T, C), torch.float32).cpu().numpy().reshape(B * T, C)
    keep = O.dropout_keep(d, 9, O.site_embed(), np.arange(B * T), C)
    base = (params["wte"][tok] + params["wpe"][None, :T]).reshape(B * T, C)
    expect = np.where(keep, base * np.float32(d.scale), np.float32(0.0)).astype(np.float32)
    assert 0.2 < 1.0 - keep.mean() < 0.3
    assert np.array_equal(x0, expect)
    gpu.close()


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_dropout_tiny_rate_equals_no_dropout_bitwise(prec):
    """p = 1e-12 keeps every element (floor(p 2^32) = 0) with scale 1.0f, so the
    dropout kernels must reproduce the undropped path bit for bit: the masks sit
    where they multiply by exactly 1, and nothing else moves."""
    cfg = W.CONFIGS["char_6l"] if prec == "bf16" else W.CONFIGS["char_small"]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng, perturb=True)
    tok, tgt = W.make_batch(cfg, drng, B=4)
    out = []
    for p in (0.0, 1e-12):
        say(f"[dropout] {prec} p={p}")
        gpu = new_model(cfg, prec, dropout=p)
        gpu.load_params(params)
        loss = float(gpu.forward_loss(tok, tgt).item())
        gpu.backward()
        out.append((loss, gpu.grads()))
        gpu.close()
    assert out[0][0] == out[1][0]
    assert all(np.array_equal(out[0][1][k], out[1][1][k]) for k in out[0][1])


def test_dropout_counter_and_seed():
    """Each forward takes the next counter; resetting seed and counter repeats
    the masks exactly, and another seed changes them."""
    cfg = W.CONFIGS["char_small"]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng, perturb=True)
    tok, tgt = W.make_batch(cfg, drng, B=4)
    gpu = new_model(cfg, "bf16", dropout=0.2)
    gpu.load_params(params)
    gpu.set_dropout_seed(SEED, 3)
    a = float(gpu.forward_loss(tok, tgt).item())
    b = float(gpu.forward_loss(tok, tgt).item())
    gpu.set_dropout_seed(SEED, 3)
    a2 = float(gpu.forward_loss(tok, tgt).item())
    gpu.set_dropout_seed(SEED + 1, 3)
    c = float(gpu.forward_loss(tok, tgt).item())
    gpu.sync()
    assert a == a2 and a != b and a != c
    ref = O.microbatch(params, tok, tgt, cfg, dropout=O.Dropout(0.2, SEED, 4))[0].mean()
    assert abs(b - ref) / ref < 2e-2
    gpu.close()
