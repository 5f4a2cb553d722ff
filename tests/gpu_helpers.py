"""Shared helpers of the GPU tests: run the HIP path and the oracle on the same
seeded inputs and compare them."""
import sys

import numpy as np

from oracle import gpt_oracle as O
from transformer_lm_gpt_amd import workloads as W

TOL = {"fp32": {"loss_abs": 1e-4, "rel": 1e-3}, "bf16": {"loss_rel": 2e-2, "rel": 3e-2}}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    if nb == 0.0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def check_loss(gpu_loss, ref_loss, prec, what=""):
    if prec == "fp32":
        assert abs(gpu_loss - ref_loss) <= TOL["fp32"]["loss_abs"], (what, gpu_loss, ref_loss)
    else:
        assert abs(gpu_loss - ref_loss) / abs(ref_loss) <= TOL["bf16"]["loss_rel"], (what, gpu_loss, ref_loss)


def split_key_bias(t: dict, d: int) -> dict:
    """Splits every attn.b into its q, k and v parts. The key bias has an
    identically zero gradient (a per-query constant added to all scores leaves
    the softmax unchanged), so its Adam state and update are driven by rounding
    noise alone and are checked against a bound, not a relative error."""
    out = {}
    for k, v in t.items():
        if k.endswith("attn.b"):
            out[k + ".q"], out[k + ".k"], out[k + ".v"] = v[:d], v[d:2 * d], v[2 * d:]
        else:
            out[k] = v
    return out


def check_tensors(gpu: dict, ref: dict, prec, what="", tol=None, d=None, key_bias_bound=None):
    tol = TOL[prec]["rel"] if tol is None else tol
    if d is not None:
        gpu, ref = split_key_bias(gpu, d), split_key_bias(ref, d)
    keys = [k for k in ref if not (d is not None and k.endswith("attn.b.k"))]
    worst = max(((rel(gpu[k], ref[k]), k) for k in keys), key=lambda x: x[0])
    bad = {k: rel(gpu[k], ref[k]) for k in keys if rel(gpu[k], ref[k]) > tol}
    assert not bad, (what, bad)
    if d is not None and key_bias_bound is not None:
        for k in ref:
            if k.endswith("attn.b.k"):
                dev = float(np.max(np.abs(np.asarray(gpu[k], np.float64) - ref[k])))
                assert dev <= key_bias_bound, (what, k, dev, key_bias_bound)
    return worst


def new_model(cfg, prec, batch=None, grad_accum=None, dropout=0.0):
    from transformer_lm_gpt_amd.binding import GPT
    return GPT(cfg, prec, batch=batch, grad_accum=grad_accum, dropout=dropout)


def check_zero_start(gpu, ref, lr, steps, what=""):
    """Tensors that start at exactly zero (LoRA's B). Adam's first update is about
    lr * sign(g) per element, so an element whose gradient lies within rounding of 0
    may move the other way on the two sides, and with nothing loaded to dilute it
    such a flip dominates the tensor's relative error. Each element is held to the
    Adam step bound (|delta| <= 2 lr per step), and elements apart by more than lr / 2
    must be rare; m and v, checked to the usual tolerance, pin the update itself."""
    for k in ref:
        dev = np.abs(np.asarray(gpu[k], np.float64) - ref[k])
        assert float(dev.max()) <= 2.0 * lr * steps, (what, k, float(dev.max()))
        frac = float(np.mean(dev > 0.5 * lr))
        assert frac <= 0.02, (what, k, frac)


def run_steps(name, prec, steps=None, B=None, T=None, A=None, perturb=True, check_every=True, cfg=None,
              dropout=0.0, seed=0, counter=0, rel_tol=None, zero_start=()):
    """Runs `steps` optimizer steps on both sides and checks losses, gradients,
    and parameters/moments after every step. With dropout > 0 both sides draw
    their masks from the same seed and forward counter. Parameters whose names end
    with a suffix in `zero_start` start at zero and are checked by check_zero_start."""
    cfg = W.CONFIGS[name] if cfg is None else cfg
    steps = cfg.parity_steps if steps is None else steps
    A = cfg.grad_accum if A is None else A
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng, perturb=perturb)
    say(f"[parity] {name} {prec} steps={steps} B={B or cfg.batch} T={T or cfg.block_size} A={A} dropout={dropout}")
    gpu = new_model(cfg, prec, grad_accum=A, dropout=dropout)
    gpu.load_params(params)
    drop = None
    if dropout > 0.0:
        gpu.set_dropout_seed(seed, counter)
        drop = O.Dropout(dropout, seed, counter)
    tr = O.Trainer(params, cfg, dropout=drop)
    report = []
    for s in range(steps):
        batches = W.make_step_batches(cfg, drng, A=A, B=B, T=T)
        gl = []
        for tok, tgt in batches:
            gl.append(float(gpu.forward_loss(tok, tgt).item()))
            gpu.backward()
        g_gpu = gpu.grads()
        norm_gpu = gpu.adamw_step(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.grad_clip)
        gpu.sync()
        ref = tr.step(batches)
        for i, (a, b) in enumerate(zip(gl, ref["losses"])):
            check_loss(a, b, prec, f"step {s} micro {i}")
        tol = TOL[prec]["rel"] if rel_tol is None else rel_tol
        assert abs(float(norm_gpu.item()) - ref["norm"]) <= tol * ref["norm"], (float(norm_gpu.item()), ref["norm"])
        if check_every or s == 0:
            wg = check_tensors(g_gpu, ref["grads"], prec, f"grads step {s}", tol=tol)
        p_gpu = gpu.params()
        m_gpu, v_gpu = gpu.moments()
        d = cfg.n_embd
        # key bias: each noise-driven Adam step moves it by at most lr (|mhat| <= sqrt(vhat))
        zs = [k for k in tr.p if zero_start and k.endswith(tuple(zero_start))]
        check_zero_start({k: p_gpu[k] for k in zs}, {k: tr.p[k] for k in zs}, cfg.lr, s + 1, f"params step {s}")
        wp = check_tensors(p_gpu, {k: v for k, v in tr.p.items() if k not in zs}, prec, f"params step {s}", tol=tol,
                           d=d, key_bias_bound=2.0 * cfg.lr * (s + 1))
        gmax = max(float(np.max(np.abs(g))) for g in ref["grads"].values())
        wm = check_tensors(m_gpu, tr.m, prec, f"m step {s}", tol=tol, d=d, key_bias_bound=1e-3 * gmax)
        wv = check_tensors(v_gpu, tr.v, prec, f"v step {s}", tol=2 * tol, d=d, key_bias_bound=1e-6 * gmax * gmax)
        report.append((gl, ref["losses"], wg, wp, wm, wv))
        say(f"  step {s}: loss gpu {np.mean(gl):.6f} oracle {ref['loss']:.6f} worst grad {wg[0]:.2e} ({wg[1]}) "
            f"param {wp[0]:.2e} m {wm[0]:.2e} v {wv[0]:.2e}")
    assert gpu.step_count() == steps
    gpu.close()
    return report
