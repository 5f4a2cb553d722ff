"""Parity at the GPT-2 124M size, in the launch configuration the benchmark times
(B 12, T 1024, 5 micro-batches, bf16).

The oracle cannot run all 60 sequences of a step in float64 in test time, so:
  * the forward is checked on two sampled sequences of a real Zipf batch: their
    logits (and per-position losses recomputed from them) against the oracle's
    per-sequence forward;
  * a full optimizer step runs on micro-batches made of 12 identical copies of one
    sequence each (5 different sequences). The mean over identical copies equals
    the single-sequence value, so the oracle's step on five single-sequence
    micro-batches is the exact reference for the GPU's full-size step.
"""
import numpy as np
import pytest

from oracle import gpt_oracle as O
from transformer_lm_gpt_amd import workloads as W

from gpu_helpers import check_loss, check_tensors, new_model, rel, say

pytestmark = pytest.mark.gpu

NAME = "gpt2_124m"


def _lse_loss(z, y):
    z = z.astype(np.float64)
    m = z.max(-1, keepdims=True)
    lse = (m + np.log(np.exp(z - m).sum(-1, keepdims=True)))[..., 0]
    return lse - np.take_along_axis(z, y[..., None], -1)[..., 0]


@pytest.mark.timeout(900)
def test_gpt2_forward_sampled_sequences():
    cfg = W.CONFIGS[NAME]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng, perturb=True)
    tok, tgt = W.make_batch(cfg, drng)                  # [12, 1024], Zipf ids
    say(f"[fullsize] forward B={tok.shape[0]} T={tok.shape[1]} bf16")
    gpu = new_model(cfg, "bf16")
    gpu.load_params(params)
    loss = float(gpu.forward_loss(tok, tgt).item())
    z = gpu.forward_logits(tok)                          # fp32 [12, 1024, 50304]
    rows = [0, 11]
    zs = z[rows].cpu().numpy()
    # the fused cross-entropy agrees with the loss recomputed from the GPU's own logits
    zall = z.cpu().numpy()
    host_loss = float(_lse_loss(zall, tgt).mean())
    assert abs(loss - host_loss) < 1e-3 * host_loss, (loss, host_loss)
    del zall
    zr = O.logits(params, tok[rows], cfg)
    for i, b in enumerate(rows):
        r = rel(zs[i], zr[i])
        say(f"  sequence {b}: logits rel err {r:.2e}")
        assert r < 2e-2
        lg = _lse_loss(zs[i], tgt[b]).mean()
        lo = _lse_loss(zr[i], tgt[b]).mean()
        assert abs(lg - lo) / lo < 2e-2, (b, lg, lo)
    # argmax agrees wherever the oracle's top-2 gap is clear in bf16 terms
    top = np.sort(zr, -1)[..., -2:]
    clear = (top[..., 1] - top[..., 0]) > 0.05 * zr.std(-1)
    assert np.array_equal(np.argmax(zs, -1)[clear], np.argmax(zr, -1)[clear])
    gpu.close()


@pytest.mark.timeout(1200)
def test_gpt2_full_step_identical_copies():
    cfg = W.CONFIGS[NAME]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng, perturb=True)
    seqs = [W.make_batch(cfg, drng, B=1) for _ in range(cfg.grad_accum)]
    say(f"[fullsize] one step, {cfg.grad_accum} micro-batches of {cfg.batch} identical copies, bf16")
    gpu = new_model(cfg, "bf16")
    gpu.load_params(params)
    gl = []
    for tok1, tgt1 in seqs:
        tok = np.repeat(tok1, cfg.batch, axis=0)
        tgt = np.repeat(tgt1, cfg.batch, axis=0)
        gl.append(float(gpu.forward_loss(tok, tgt).item()))
        gpu.backward()
    g_gpu = gpu.grads()
    norm = float(gpu.adamw_step(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.grad_clip).item())
    gpu.sync()
    tr = O.Trainer(params, cfg)
    ref = tr.step(seqs)
    for a, b in zip(gl, ref["losses"]):
        check_loss(a, b, "bf16", "micro-batch loss")
    assert abs(norm - ref["norm"]) <= 3e-2 * ref["norm"], (norm, ref["norm"])
    wg = check_tensors(g_gpu, ref["grads"], "bf16", "grads")
    d = cfg.n_embd
    wp = check_tensors(gpu.params(), tr.p, "bf16", "params", d=d, key_bias_bound=2.0 * cfg.lr)
    m_gpu, v_gpu = gpu.moments()
    gmax = max(float(np.max(np.abs(g))) for g in ref["grads"].values())
    wm = check_tensors(m_gpu, tr.m, "bf16", "m", d=d, key_bias_bound=1e-3 * gmax)
    wv = check_tensors(v_gpu, tr.v, "bf16", "v", tol=6e-2, d=d, key_bias_bound=1e-6 * gmax * gmax)
    say(f"  loss {np.mean(gl):.5f} vs {ref['loss']:.5f}; worst grad {wg}; param {wp[0]:.2e} m {wm[0]:.2e} v {wv[0]:.2e}")
    gpu.close()


@pytest.mark.timeout(900)
def test_gpt2_forward_with_dropout_sampled_sequences():
    """Dropout 0.1 at the full size and launch configuration: the input of the final
    LayerNorm after all 12 dropped blocks, for two sampled sequences of a B 12 x T 1024
    micro-batch, against the oracle's forward of those sequences with the same masks
    (logits and per-position losses formed on the host from the GPU's activations)."""
    import torch
    cfg = W.CONFIGS[NAME]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng, perturb=True)
    tok, tgt = W.make_batch(cfg, drng)
    seed, call = 0x0DD5EED, 3
    say(f"[fullsize] forward with dropout 0.1, B={tok.shape[0]} T={tok.shape[1]} bf16")
    gpu = new_model(cfg, "bf16", dropout=0.1)
    gpu.load_params(params)
    gpu.set_dropout_seed(seed, call)
    gpu.forward_loss(tok, tgt)
    B, T, d = tok.shape[0], tok.shape[1], cfg.n_embd
    xL = gpu.debug("x", cfg.n_layer, (B, T, d), torch.float32).cpu().numpy()
    gpu.close()
    P = {k: v.astype(np.float64) for k, v in params.items()}
    drop = (O.Dropout(0.1, seed, call), call)
    for b in (0, B - 1):
        zr, _ = O.forward_sequence(P, tok[b], cfg, drop, b)
        xf, _ = O.layernorm_fwd(xL[b].astype(np.float64), P["lnf.g"], P["lnf.b"])
        zg = xf @ P["wte"].T
        r = rel(zg, zr)
        say(f"  sequence {b}: logits rel err {r:.2e}")
        assert r < 2e-2
        lg = _lse_loss(zg, tgt[b]).mean()
        lo = _lse_loss(zr, tgt[b]).mean()
        assert abs(lg - lo) / lo < 2e-2, (b, lg, lo)
