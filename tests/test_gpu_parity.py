"""The HIP path against the oracle on the same seeded inputs and weights.

Tolerances (from the step's stated bounds): loss within 1e-4 absolute in fp32
mode and 2e-2 relative in bf16 mode; every gradient, parameter and Adam first
moment within 1e-3 (fp32) or 3e-2 (bf16) in relative L2 norm per tensor; the
second moment, a square of the gradient, within twice that."""
import numpy as np
import pytest

from oracle import gpt_oracle as O
from transformer_lm_gpt_amd import workloads as W

from gpu_helpers import check_tensors, new_model, rel, run_steps, say

pytestmark = pytest.mark.gpu


# ----------------------------------------------------------------------------- forward pieces first

def _x_layers(params, tok, cfg):
    """Residual-stream inputs of every block (and of the final norm) for one sequence, from oracle pieces."""
    P = {k: v.astype(np.float64) for k, v in params.items()}
    T = len(tok)
    x = P["wte"][tok] + P["wpe"][:T]
    out = [x]
    for l in range(cfg.n_layer):
        p = f"h{l}."
        a, _ = O.layernorm_fwd(x, P[p + "ln1.g"], P[p + "ln1.b"])
        qkv = a @ P[p + "attn.w"].T + P[p + "attn.b"]
        d, H = cfg.n_embd, cfg.n_head
        q, k, v = (qkv[:, i * d:(i + 1) * d].reshape(T, H, d // H).transpose(1, 0, 2) for i in range(3))
        o, _ = O.attention_fwd(q, k, v)
        x1 = x + o.transpose(1, 0, 2).reshape(T, d) @ P[p + "proj.w"].T + P[p + "proj.b"]
        b2, _ = O.layernorm_fwd(x1, P[p + "ln2.g"], P[p + "ln2.b"])
        x = x1 + O.gelu(b2 @ P[p + "fc.w"].T + P[p + "fc.b"]) @ P[p + "fcproj.w"].T + P[p + "fcproj.b"]
        out.append(x)
    return out


@pytest.mark.parametrize("name,prec", [("tiny", "fp32"), ("char_small", "fp32"), ("char_small", "bf16")])
def test_forward_activations_and_logits(name, prec):
    import torch
    cfg = W.CONFIGS[name]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng, perturb=True)
    tok, tgt = W.make_batch(cfg, drng, B=2)
    say(f"[forward] {name} {prec} B=2 T={cfg.block_size}")
    gpu = new_model(cfg, prec)
    gpu.load_params(params)
    loss = float(gpu.forward_loss(tok, tgt).item())
    B, T, d = tok.shape[0], tok.shape[1], cfg.n_embd
    tol = 1e-5 if prec == "fp32" else 1e-2
    for b in range(B):
        xs = _x_layers(params, tok[b], cfg)
        for l in range(cfg.n_layer + 1):
            xg = gpu.debug("x", l, (B, T, d), torch.float32).cpu().numpy()[b]
            assert rel(xg, xs[l]) < tol, (l, rel(xg, xs[l]))
    z = gpu.forward_logits(tok).cpu().numpy()
    zr = O.logits(params, tok, cfg)
    assert rel(z, zr) < (1e-5 if prec == "fp32" else 2e-2)
    rl, _ = O.microbatch(params, tok, tgt, cfg)
    if prec == "fp32":
        assert abs(loss - rl.mean()) < 1e-4
    else:
        assert abs(loss - rl.mean()) / rl.mean() < 2e-2
    gpu.close()


def test_embedding_gather_bit_exact():
    import torch
    cfg = W.CONFIGS["char_small"]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng)
    tok, tgt = W.make_batch(cfg, drng)
    gpu = new_model(cfg, "fp32")
    gpu.load_params(params)
    gpu.forward_loss(tok, tgt)
    x0 = gpu.debug("x", 0, (cfg.batch, cfg.block_size, cfg.n_embd), torch.float32).cpu().numpy()
    expect = params["wte"][tok] + params["wpe"][None, :cfg.block_size]     # one fp32 add, same order
    assert np.array_equal(x0, expect)
    gpu.close()


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_causality_bitwise(prec):
    cfg = W.CONFIGS["char_small"]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng, perturb=True)
    tok, _ = W.make_batch(cfg, drng, B=3)
    gpu = new_model(cfg, prec)
    gpu.load_params(params)
    z0 = gpu.forward_logits(tok).cpu().numpy()
    t = 37
    tok2 = tok.copy()
    tok2[:, t + 1:] = (tok2[:, t + 1:] + 11) % cfg.vocab_size
    z1 = gpu.forward_logits(tok2).cpu().numpy()
    assert np.array_equal(z0[:, :t + 1], z1[:, :t + 1])
    assert not np.array_equal(z0[:, t + 1:], z1[:, t + 1:])
    gpu.close()


def test_argmax_exact_where_gap_is_clear():
    cfg = W.CONFIGS["char_small"]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng, perturb=True)
    params["wte"] *= 20.0                                  # spread the logits
    tok, _ = W.make_batch(cfg, drng, B=4)
    gpu = new_model(cfg, "fp32")
    gpu.load_params(params)
    z = gpu.forward_logits(tok).cpu().numpy()
    zr = O.logits(params, tok, cfg)
    top2 = np.sort(zr, axis=-1)[..., -2:]
    clear = (top2[..., 1] - top2[..., 0]) > 1e-3
    assert clear.mean() > 0.9
    assert np.array_equal(np.argmax(z, -1)[clear], np.argmax(zr, -1)[clear])
    gpu.close()


# ----------------------------------------------------------------------------- full steps

@pytest.mark.parametrize("name,prec", [
    ("tiny", "fp32"),
    ("char_small", "fp32"),
    ("char_small", "bf16"),
])
def test_step_parity_small(name, prec):
    run_steps(name, prec)


def test_step_parity_char_6l_bf16():
    run_steps("char_6l", "bf16")


@pytest.mark.timeout(900)
def test_step_parity_bpe_12l_bf16():
    run_steps("bpe_12l_512", "bf16")


@pytest.mark.parametrize("name,prec,B,T,A", [
    ("tiny", "fp32", 3, 11, 2),        # ragged: T below block_size, two micro-batches
    ("char_small", "bf16", 5, 37, 3),
    ("char_small", "fp32", 1, 1, 1),   # a single position
    ("char_6l", "bf16", 2, 150, 2),    # head_dim 64, three 64-row tiles, the last one ragged
])
def test_step_parity_ragged(name, prec, B, T, A):
    run_steps(name, prec, steps=2, B=B, T=T, A=A)


# ----------------------------------------------------------------------------- determinism and errors

def test_gradients_bitwise_deterministic():
    cfg = W.CONFIGS["char_small"]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng, perturb=True)
    tok, tgt = W.make_batch(cfg, drng)
    out = []
    for _ in range(2):
        gpu = new_model(cfg, "bf16")
        gpu.load_params(params)
        gpu.forward_loss(tok, tgt)
        gpu.backward()
        out.append(gpu.grads())
        gpu.close()
    assert all(np.array_equal(out[0][k], out[1][k]) for k in out[0])


def test_nonfinite_gradient_skips_update():
    from transformer_lm_gpt_amd.binding import GPTError
    cfg = W.CONFIGS["tiny"]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng)
    params["h0.fc.w"][0, 0] = np.inf
    tok, tgt = W.make_batch(cfg, drng)
    gpu = new_model(cfg, "fp32")
    gpu.load_params(params)
    gpu.forward_loss(tok, tgt)
    gpu.backward()
    gpu.adamw_step(1e-2, 0.9, 0.99, 1e-8, 0.0, 1.0)
    with pytest.raises(GPTError) as e:
        gpu.sync()
    assert e.value.code == -6
    after = gpu.params()
    assert all(np.array_equal(after[k], params[k]) for k in params)
    assert gpu.step_count() == 0
    gpu.close()


def test_call_order_and_shape_errors():
    from transformer_lm_gpt_amd.binding import GPTError
    cfg = W.CONFIGS["tiny"]
    drng, wrng = W.rngs()
    gpu = new_model(cfg, "fp32")
    gpu.load_params(W.init_params(cfg, wrng))
    with pytest.raises(GPTError) as e:
        gpu.backward()
    assert e.value.code == -3
    gpu.sync_code = None
    with pytest.raises(GPTError):
        gpu.sync()                       # reports and clears the sticky error
    tok, tgt = W.make_batch(cfg, drng, T=cfg.block_size)
    big = np.concatenate([tok, tok], axis=1)
    with pytest.raises(GPTError) as e:
        gpu.forward_loss(big, big)
    assert e.value.code == -2
    with pytest.raises(GPTError):
        gpu.sync()
    gpu.forward_loss(tok, tgt)
    gpu.backward()
    gpu.adamw_step(1e-2, 0.9, 0.99, 1e-8, 0.0, 1.0)
    with pytest.raises(GPTError) as e:
        gpu.adamw_step(1e-2, 0.9, 0.99, 1e-8, 0.0, 1.0)     # no backward since the last step
    assert e.value.code == -3
    gpu.close()
