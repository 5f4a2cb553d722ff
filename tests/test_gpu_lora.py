"""LoRA adapters on the q and v projections (the fine-tuning article on
blog.hotdry.top, LoRA section) on the HIP path against the oracle.

The oracle runs the low-rank branch as written, q = a W0^T + b + s (a A^T) B^T;
the HIP path runs the merged weight W0 + s B A and forms the adapter gradients
from the q and v weight gradients. Both train A and B alone."""
import numpy as np
import pytest

from oracle import gpt_oracle as O
from transformer_lm_gpt_amd import workloads as W

from gpu_helpers import check_loss, check_tensors, new_model, rel, run_steps, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,prec,steps,B,T,A,perturb", [
    ("tiny_lora", "fp32", 10, None, None, None, True),
    ("tiny_lora", "fp32", 3, 3, 11, 2, True),           # ragged, two micro-batches
    ("tiny_lora", "fp32", 3, None, None, None, False),  # B = 0 at the start, as fine-tuning begins
    ("char_small_lora", "fp32", 3, None, None, None, True),
    ("char_small_lora", "bf16", 3, None, None, None, True),
    ("char_small_lora", "bf16", 1, 5, 37, 2, False),    # ragged, B = 0 at the start
])
def test_lora_step_parity(name, prec, steps, B, T, A, perturb):
    # From B = 0, bf16's first Adam step flips the sign of B's near-zero-gradient
    # elements (see check_zero_start); fp32 holds B to the usual relative bound. The
    # next step's dA = s B^T dW reads those flipped elements, so from there the two
    # bf16 trajectories part by design (5 % on one dA tensor at step 2, measured):
    # that case is held to its first step, and bf16 over several steps is checked
    # from a random B, where the loaded values dominate.
    zs = (".lora_q.B", ".lora_v.B") if prec == "bf16" and not perturb else ()
    run_steps(name, prec, steps=steps, B=B, T=T, A=A, perturb=perturb, zero_start=zs)


def test_lora_step_parity_with_dropout():
    run_steps("char_small_lora", "fp32", steps=1, dropout=0.1, seed=0x5EED, counter=2)
    run_steps("char_small_lora", "bf16", steps=1, dropout=0.1, seed=0x5EED, counter=2)


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_lora_base_frozen_and_zero_B_is_base(prec):
    """B = 0: the logits equal the base model's bitwise (the merged weight is W0
    exactly); after steps, every base tensor is bitwise what was loaded."""
    cfg = W.CONFIGS["char_small_lora"]
    base_cfg = cfg.with_(lora_rank=0)
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng, perturb=False)
    tok, tgt = W.make_batch(cfg, drng, B=4)
    say(f"[lora] zero B and frozen base, {prec}")
    g0 = new_model(base_cfg, prec)
    g0.load_params({k: v for k, v in params.items() if ".lora_" not in k})
    z0 = g0.forward_logits(tok).cpu().numpy()
    g0.close()
    g1 = new_model(cfg, prec)
    g1.load_params(params)
    z1 = g1.forward_logits(tok).cpu().numpy()
    assert np.array_equal(z0, z1)
    for _ in range(2):
        g1.forward_loss(tok, tgt)
        g1.backward()
        g1.adamw_step(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.grad_clip)
    g1.sync()
    after = g1.params()
    for k, v in params.items():
        if ".lora_" in k:
            assert not np.array_equal(after[k], v), k
        else:
            assert np.array_equal(after[k], v), k
    # the trained adapters change the model: the logits now match the oracle's
    z2 = g1.forward_logits(tok).cpu().numpy()
    zr = O.logits(after, tok, cfg)
    assert rel(z2, zr) < (1e-5 if prec == "fp32" else 2e-2)
    assert not np.array_equal(z2, z0)
    g1.close()


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_lora_decode_matches_full_forward(prec):
    from transformer_lm_gpt_amd.binding import GPT
    cfg = W.CONFIGS["char_small_lora"]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng, perturb=True)
    B, T0, steps = 3, 9, 4
    tok, _ = W.make_batch(cfg, drng, B=B, T=T0 + steps)
    say(f"[lora decode] {prec}")
    gpu = GPT(cfg, prec, kv_cache=True)
    gpu.load_params(params)
    tol = 1e-5 if prec == "fp32" else 2e-2
    z = gpu.prefill(tok[:, :T0]).cpu().numpy()
    assert rel(z, O.logits(params, tok[:, :T0], cfg)[:, -1]) < tol
    for s in range(steps):
        z = gpu.decode(tok[:, T0 + s]).cpu().numpy()
        zr = O.logits(params, tok[:, :T0 + s + 1], cfg)[:, -1]
        assert rel(z, zr) < tol, (s, rel(z, zr))
    gpu.close()


@pytest.mark.timeout(1200)
def test_gpt2_lora_full_step_identical_copies():
    """GPT-2 124M with rank-16 adapters in the benchmark's launch configuration
    (B 12, T 1024, 5 micro-batches, bf16): micro-batches of 12 identical copies of
    one sequence, so the oracle's step on the five single sequences is the exact
    reference."""
    cfg = W.CONFIGS["gpt2_124m_lora"]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng, perturb=True)
    seqs = [W.make_batch(cfg, drng, B=1) for _ in range(cfg.grad_accum)]
    say(f"[lora fullsize] one step, {cfg.grad_accum} micro-batches of {cfg.batch} identical copies, bf16")
    gpu = new_model(cfg, "bf16")
    gpu.load_params(params)
    gl = []
    for tok1, tgt1 in seqs:
        gl.append(float(gpu.forward_loss(np.repeat(tok1, cfg.batch, 0), np.repeat(tgt1, cfg.batch, 0)).item()))
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
    wp = check_tensors(gpu.params(), tr.p, "bf16", "params")
    m_gpu, v_gpu = gpu.moments()
    wm = check_tensors(m_gpu, tr.m, "bf16", "m")
    wv = check_tensors(v_gpu, tr.v, "bf16", "v", tol=6e-2)
    say(f"  loss {np.mean(gl):.5f} vs {ref['loss']:.5f}; worst grad {wg}; param {wp[0]:.2e} m {wm[0]:.2e} v {wv[0]:.2e}")
    gpu.close()


@pytest.mark.parametrize("rank,prec,steps", [
    (12, "fp32", 2),     # a full rank chunk of 8 and a partial one
    (5, "bf16", 1),      # one partial chunk
    (64, "fp32", 1),     # the largest rank the adapter kernels take
    (64, "bf16", 1),
])
def test_lora_rank_edges(rank, prec, steps):
    cfg = W.CONFIGS["char_small_lora"].with_(lora_rank=rank)
    run_steps("char_small_lora", prec, steps=steps, cfg=cfg)


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_lora_widest_rows(prec):
    # n_embd 1024: four float4 per lane in the merge and dB kernels, and B's rank
    # chunk for all 1024 rows filling the dA kernel's LDS stage
    cfg = W.CONFIGS["char_small_lora"].with_(n_layer=1, n_head=16, n_embd=1024, block_size=16, batch=2)
    run_steps("char_small_lora", prec, steps=1, cfg=cfg)


@pytest.mark.parametrize("prec,steps", [("fp32", 3), ("bf16", 1)])
def test_lora_on_the_microgpt_block(prec, steps):
    # Adapters on the microGPT block's bias-free q and v rows (untied head, RMSNorm,
    # ReLU). In bf16 the ReLU gates within rounding of 0 may flip (the layer-0 adapter
    # gradients collect every layer's flips): run_steps adds the oracle's gate band
    # (O.relu_gate_band) to each tensor's bound, as for the block without adapters.
    cfg = W.CONFIGS["char_small_micro"].with_(lora_rank=8, lora_alpha=16.0)
    run_steps("char_small_micro", prec, steps=steps, cfg=cfg)
