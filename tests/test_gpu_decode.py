"""Generation on the HIP path: prefill, decode with the key/value cache and the
sampling kernel, against the oracle's full recomputation (``generate``) and its
``sample_token``. The decode logits must equal the last row of a full forward
over the sequence so far, at the forward's tolerances."""
import numpy as np
import pytest

from oracle import gpt_oracle as O
from transformer_lm_gpt_amd import workloads as W

from gpu_helpers import rel, say

pytestmark = pytest.mark.gpu


def _model(cfg, prec, **kw):
    from transformer_lm_gpt_amd.binding import GPT
    return GPT(cfg, prec, kv_cache=True, **kw)


@pytest.mark.parametrize("name,prec,B,T0,steps", [
    ("tiny", "fp32", 3, 5, 6),
    ("char_small", "fp32", 4, 20, 8),
    ("char_small", "bf16", 4, 20, 8),
    ("char_6l", "bf16", 3, 61, 6),        # head_dim 64; the prompt ends inside a 64-row tile
])
def test_prefill_and_decode_match_full_forward(name, prec, B, T0, steps):
    cfg = W.CONFIGS[name]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng, perturb=True)
    tok, _ = W.make_batch(cfg, drng, B=B, T=T0 + steps)
    say(f"[decode] {name} {prec} B={B} T0={T0} steps={steps}")
    gpu = _model(cfg, prec)
    gpu.load_params(params)
    tol = 1e-5 if prec == "fp32" else 2e-2
    z = gpu.prefill(tok[:, :T0]).cpu().numpy()
    zr = O.logits(params, tok[:, :T0], cfg)[:, -1]
    assert rel(z, zr) < tol, rel(z, zr)
    for s in range(steps):
        z = gpu.decode(tok[:, T0 + s]).cpu().numpy()
        zr = O.logits(params, tok[:, :T0 + s + 1], cfg)[:, -1]
        say(f"  step {s}: rel {rel(z, zr):.2e}")
        assert rel(z, zr) < tol, (s, rel(z, zr))
    gpu.close()


def test_decode_gpt2_124m_bf16():
    """The GPT-2 124M shapes: prefill 40 positions of two sequences, three decode steps."""
    cfg = W.CONFIGS["gpt2_124m"]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng)
    tok, _ = W.make_batch(cfg, drng, B=2, T=43)
    gpu = _model(cfg, "bf16")
    gpu.load_params(params)
    z = gpu.prefill(tok[:, :40]).cpu().numpy()
    assert rel(z, O.logits(params, tok[:, :40], cfg)[:, -1]) < 2e-2
    for s in range(3):
        z = gpu.decode(tok[:, 40 + s]).cpu().numpy()
        zr = O.logits(params, tok[:, :41 + s], cfg)[:, -1]
        say(f"  gpt2_124m step {s}: rel {rel(z, zr):.2e}")
        assert rel(z, zr) < 2e-2
    gpu.close()


@pytest.mark.parametrize("name,prec", [("char_6l", "bf16"), ("tiny", "fp32")])
def test_decode_graph_replays_equal_direct_launches(name, prec):
    """A decode call that repeats the previous call's token and logits pointers replays
    the recorded step; one whose pointers differ launches the kernels one by one. Both
    give the same logits, bit for bit, at every step. Each replay is followed by eager
    work (the sampler) and a host synchronization. A second prefill of another length
    moves the device position that the same recording then reads."""
    import ctypes as C
    import torch
    cfg = W.CONFIGS[name]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng, perturb=True)
    B, steps, lens = 3, 4, (min(21, cfg.block_size // 3), min(34, cfg.block_size // 2))
    tok, _ = W.make_batch(cfg, drng, B=B, T=max(lens) + steps)
    say(f"[decode graph] {name} {prec} B={B} prompts {lens}")
    gpu = _model(cfg, prec)
    gpu.load_params(params)
    recorded = {}
    for T0 in lens:                                   # the binding's fixed buffers: replays
        gpu.prefill(tok[:, :T0])
        zs = []
        for s in range(steps):
            z = gpu.decode(tok[:, T0 + s])
            gpu.sample(z, 0.0)
            gpu.sync()
            zs.append(z.cpu().numpy().copy())
        recorded[T0] = zs
    tb = gpu.decode_tokens()
    outs = [torch.empty_like(gpu._dec_out), torch.empty_like(gpu._dec_out)]
    tol = 1e-5 if prec == "fp32" else 2e-2
    for T0 in lens:                                   # alternating logits buffers: direct launches
        gpu.prefill(tok[:, :T0])
        for s in range(steps):
            tb.copy_(torch.from_numpy(np.ascontiguousarray(tok[:, T0 + s], dtype=np.int32)).to(tb.device))
            o = outs[s % 2]
            gpu._check(gpu.lib.gpt_decode(gpu.h, C.c_void_p(tb.data_ptr()), C.c_void_p(o.data_ptr())))
            zd = o.cpu().numpy()
            assert np.array_equal(zd, recorded[T0][s]), (T0, s, float(np.max(np.abs(zd - recorded[T0][s]))))
        zr = O.logits(params, tok[:, :T0 + steps], cfg)[:, -1]
        say(f"  prompt {T0}: {steps} steps equal; last step rel {rel(recorded[T0][-1], zr):.2e}")
        assert rel(recorded[T0][-1], zr) < tol
    gpu.close()


def test_greedy_generation_matches_oracle():
    """fp32, spread logits: the greedy tokens equal the oracle's wherever its top-1
    and top-2 logits are more than 1e-3 apart (after the first unclear step the
    sequences may part, so the comparison stops there)."""
    cfg = W.CONFIGS["char_small"]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng, perturb=True)
    params["wte"] *= 20.0
    tok, _ = W.make_batch(cfg, drng, B=4, T=12)
    n = 10
    seqs, zs = O.generate(params, tok, cfg, n, 0.0, 0, np.zeros((n, 4)))
    gpu = _model(cfg, "fp32")
    gpu.load_params(params)
    z = gpu.prefill(tok)
    got = []
    for s in range(n):
        t = gpu.sample(z, 0.0)
        got.append(t.cpu().numpy())
        if s + 1 < n:
            z = gpu.decode(t)
    got = np.stack(got, axis=1)
    clear_steps = 0
    for b in range(4):
        for s in range(n):
            top2 = np.sort(zs[s, b])[-2:]
            if top2[1] - top2[0] <= 1e-3:
                break
            assert got[b, s] == seqs[b, 12 + s], (b, s)
            clear_steps += 1
    assert clear_steps >= 30
    gpu.close()


@pytest.mark.parametrize("V", [50304, 60000, 65])   # 60000: past the logits the kernel keeps in registers
@pytest.mark.parametrize("temperature,top_k", [(0.0, 0), (1.0, 0), (0.8, 40), (1.5, 1), (1.0, 50304), (0.7, 3)])
def test_sample_kernel_against_oracle(temperature, top_k, V):
    """Same logits and uniforms on both sides. The token must be a candidate and its
    cumulative-weight interval (fp64) must hold u times the total up to 1e-5 of the
    total (the kernel sums about 50k weights in fp32); wherever u times the total lies
    farther than that from an interval edge, it must be the oracle's token exactly."""
    import torch
    rng = np.random.default_rng(21)
    B = 16
    z = (rng.standard_normal((B, V)) * 3.0).astype(np.float32)
    z[3, 100:110] = z[3].max()                         # ties at the maximum
    u = rng.random(B).astype(np.float32)
    gpu = _model(W.CONFIGS["char_small"].with_(vocab_size=V, padded_vocab=V), "fp32")
    got = gpu.sample(torch.from_numpy(z), temperature, top_k, u).cpu().numpy()
    exact = 0
    for b in range(B):
        want = O.sample_token(z[b], temperature, top_k, float(u[b]))
        if temperature <= 0:
            assert got[b] == want
            exact += 1
            continue
        zz = z[b].astype(np.float64)
        cand = np.ones(V, bool) if not (0 < top_k < V) else zz >= np.sort(zz)[V - top_k]
        assert cand[got[b]], (b, got[b])
        w = np.where(cand, np.exp((zz - zz.max()) / temperature), 0.0)
        c = np.cumsum(w)
        tgt = float(u[b]) * c[-1]
        lo = c[got[b]] - w[got[b]]
        assert lo - 1e-5 * c[-1] <= tgt <= c[got[b]] + 1e-5 * c[-1], (b, lo, tgt, c[got[b]])
        if min(abs(tgt - lo), abs(c[want] - tgt)) > 1e-5 * c[-1]:
            assert got[b] == want
            exact += 1
    assert exact >= B // 2                             # most draws land away from an edge
    gpu.close()


def test_decode_state_errors():
    from transformer_lm_gpt_amd.binding import GPT, GPTError
    cfg = W.CONFIGS["tiny"]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng)
    tok, _ = W.make_batch(cfg, drng, B=2, T=cfg.block_size)
    plain = GPT(cfg, "fp32")
    plain.load_params(params)
    with pytest.raises(GPTError) as e:
        plain.prefill(tok[:, :4])
    assert e.value.code == -4                          # no cache reserved
    plain.close()
    gpu = _model(cfg, "fp32")
    gpu.load_params(params)
    with pytest.raises(GPTError) as e:
        gpu.decode(tok[:, 0])
    assert e.value.code == -3                          # no prefill
    with pytest.raises(GPTError):
        gpu.sync()
    gpu.prefill(tok[:, :cfg.block_size - 1])
    gpu.decode(tok[:, cfg.block_size - 1])             # fills the last position
    with pytest.raises(GPTError) as e:
        gpu.decode(tok[:, 0])
    assert e.value.code == -2
    gpu.close()
