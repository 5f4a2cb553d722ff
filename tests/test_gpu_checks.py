"""Boundary behaviour on the GPU: GPT_F_DEBUG_CHECKS (token and target ids checked
against [0, vocab_size) on the device before the gather; the fine-tuning article's
data paragraph and the nanoGPT README translation store GPT-2 BPE ids of a
50,257-token vocabulary as uint16) and gpt_params_loaded (weights replaced
mid-training without resetting the optimizer)."""
import numpy as np
import pytest

from oracle import gpt_oracle as O
from transformer_lm_gpt_amd import workloads as W
from transformer_lm_gpt_amd.binding import GPTError

from gpu_helpers import check_loss, check_tensors, new_model, rel, say

pytestmark = pytest.mark.gpu

# char_small with a data vocabulary of 60 ids inside the 65-row table: id 60 is a
# padded row (valid memory, invalid id), which only the flag can tell apart
CFG = W.CONFIGS["char_small"].with_(vocab_size=60)


def _model(prec, debug_checks, **kw):
    from transformer_lm_gpt_amd.binding import GPT
    return GPT(CFG, prec, debug_checks=debug_checks, **kw)


def _batch(B=4):
    drng, wrng = W.rngs()
    params = W.init_params(CFG, wrng, perturb=True)
    tok, tgt = W.make_batch(CFG, drng, B=B)
    return params, tok % CFG.vocab_size, tgt % CFG.vocab_size


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
@pytest.mark.parametrize("where,bad", [("token", 60), ("target", 60), ("token", -1), ("target", 65),
                                        ("token", 2 ** 31 - 1)])
def test_debug_checks_reject_ids_outside_the_vocabulary(prec, where, bad):
    params, tok, tgt = _batch()
    tok, tgt = tok.copy(), tgt.copy()
    (tok if where == "token" else tgt)[1, 7] = bad
    say(f"[checks] {prec} {where} id {bad}")
    gpu = _model(prec, True)
    gpu.load_params(params)
    p0 = gpu.params()
    gpu.forward_loss(tok, tgt)
    gpu.backward()
    gpu.adamw_step(CFG.lr, CFG.beta1, CFG.beta2, CFG.eps, CFG.weight_decay, CFG.grad_clip)
    with pytest.raises(GPTError) as e:
        gpu.sync()
    assert e.value.code == -1 and "vocab_size" in str(e.value)
    # the update was skipped: parameters bitwise as loaded, moments zero, no step
    p1 = gpu.params()
    assert all(np.array_equal(p1[k], p0[k]) for k in p0)
    m, v = gpu.moments()
    assert all(not np.any(m[k]) and not np.any(v[k]) for k in m)
    assert gpu.step_count() == 0
    # the flag was cleared by the sync: a valid step goes through and matches the oracle
    good_tok, good_tgt = _batch()[1:]
    loss = float(gpu.forward_loss(good_tok, good_tgt).item())
    gpu.backward()
    gpu.adamw_step(CFG.lr, CFG.beta1, CFG.beta2, CFG.eps, CFG.weight_decay, CFG.grad_clip)
    gpu.sync()
    assert gpu.step_count() == 1
    ref = O.Trainer(params, CFG).step([(good_tok, good_tgt)])
    check_loss(loss, ref["loss"], prec)
    gpu.close()


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_debug_checks_cover_inference_calls(prec):
    params, tok, _ = _batch()
    bad = tok.copy()
    bad[0, 0] = CFG.vocab_size
    gpu = _model(prec, True, kv_cache=True)
    gpu.load_params(params)
    for call in (lambda: gpu.forward_logits(bad), lambda: gpu.prefill(bad)):
        call()
        with pytest.raises(GPTError) as e:
            gpu.sync()
        assert e.value.code == -1
    gpu.prefill(tok[:, :CFG.block_size // 2])
    gpu.sync()
    gpu.decode(np.full(tok.shape[0], CFG.vocab_size + 2, np.int32))
    with pytest.raises(GPTError) as e:
        gpu.sync()
    assert e.value.code == -1
    # valid ids leave the flag clear
    gpu.forward_logits(tok)
    gpu.sync()
    gpu.close()


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_without_the_flag_padded_ids_are_ordinary_rows(prec):
    """Without GPT_F_DEBUG_CHECKS an id in [vocab_size, padded_vocab) reads its padded
    row like any other: the step runs and matches the oracle, which indexes the same
    row (the table has padded_vocab rows)."""
    params, tok, tgt = _batch()
    tok, tgt = tok.copy(), tgt.copy()
    tok[2, 3] = CFG.vocab_size
    tgt[0, 5] = CFG.padded_vocab - 1
    gpu = _model(prec, False)
    gpu.load_params(params)
    loss = float(gpu.forward_loss(tok, tgt).item())
    gpu.backward()
    g = gpu.grads()
    gpu.adamw_step(CFG.lr, CFG.beta1, CFG.beta2, CFG.eps, CFG.weight_decay, CFG.grad_clip)
    gpu.sync()
    ref = O.Trainer(params, CFG).step([(tok, tgt)])
    check_loss(loss, ref["loss"], prec)
    check_tensors(g, ref["grads"], prec, "grads with padded ids")
    gpu.close()


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_params_loaded_keeps_gradients_moments_and_step(prec):
    """A step, then new weights written into the parameter buffer and announced with
    gpt_params_loaded: the moments and the step counter are kept bitwise, the forward
    uses the new weights (bf16 shadow refreshed), and the next step equals the oracle's
    step from the new weights with the old moments."""
    cfg = W.CONFIGS["char_small"]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng, perturb=True)
    b1 = [W.make_batch(cfg, drng)]
    b2 = [W.make_batch(cfg, drng)]
    gpu = new_model(cfg, prec)
    gpu.load_params(params)
    for tok, tgt in b1:
        gpu.forward_loss(tok, tgt)
        gpu.backward()
    gpu.adamw_step(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.grad_clip)
    gpu.sync()
    m0, v0 = gpu.moments()
    # new weights: the loaded ones with a fixed perturbation (not the trained ones)
    rng = np.random.default_rng(7)
    new = {k: (v + 0.01 * rng.standard_normal(v.shape)).astype(np.float32) for k, v in params.items()}
    gpu.forward_loss(*b2[0])             # pending, then made stale by the load
    gpu.load_params(new, reset_state=False)
    assert gpu.step_count() == 1
    m1, v1 = gpu.moments()
    assert all(np.array_equal(m1[k], m0[k]) and np.array_equal(v1[k], v0[k]) for k in m0)
    with pytest.raises(GPTError) as e:   # the forward before the load no longer has a backward
        gpu.backward()
    assert e.value.code == -3
    with pytest.raises(GPTError):        # the error is sticky until the sync reports it
        gpu.sync()
    z = gpu.forward_logits(b2[0][0]).cpu().numpy()
    assert rel(z, O.logits(new, b2[0][0], cfg)) < (1e-5 if prec == "fp32" else 2e-2)
    # second step on both sides from the new weights and the first step's moments
    tr = O.Trainer(params, cfg)
    tr.step(b1)
    tr.p = {k: v.astype(np.float64) for k, v in new.items()}
    tr.m = {k: v.astype(np.float64) for k, v in m0.items()}
    tr.v = {k: v.astype(np.float64) for k, v in v0.items()}
    for tok, tgt in b2:
        gpu.forward_loss(tok, tgt)
        gpu.backward()
    g = gpu.grads()
    gpu.adamw_step(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.grad_clip)
    gpu.sync()
    ref = tr.step(b2)
    assert gpu.step_count() == 2 and tr.t == 2
    check_tensors(g, ref["grads"], prec, "grads after reload")
    m2, _ = gpu.moments()
    check_tensors(m2, tr.m, prec, "m after reload", d=cfg.n_embd, key_bias_bound=1e-3 * max(
        float(np.max(np.abs(x))) for x in ref["grads"].values()))
    gpu.close()
