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


# Tables whose rows are separate vectors (one per token id or position): besides
# the tensor-wide norm, each row is held to the relative bound on its own, so that
# a few wrong rows cannot hide under the dense part of the gradient.
ROW_TABLES = ("wte", "wpe", "lm_head")
# Element-wise: |gpu - ref| <= MAX_ABS_K * tol * max|ref| for every element of a tensor.
MAX_ABS_K = 1.0
# Rows whose reference norm is below this fraction of the table's largest row norm
# are held to an absolute bound instead (tol times that floor): a row that receives
# nothing (a position past T) has no relative error to speak of.
ROW_FLOOR = 1e-6


def row_errors(g, r):
    """Per-row relative L2 errors of a 2-D table; rows with a reference norm below
    ROW_FLOOR of the largest row use the floor as their denominator."""
    g = np.asarray(g, np.float64).reshape(len(r), -1)
    r = np.asarray(r, np.float64).reshape(len(r), -1)
    nr = np.linalg.norm(r, axis=1)
    den = np.maximum(nr, ROW_FLOOR * float(nr.max()) if nr.size else 0.0)
    den = np.where(den > 0, den, 1.0)
    return np.linalg.norm(g - r, axis=1) / den


def max_abs_ratio(g, r):
    """max |g - r| / max |r| (0 for an all-zero reference that g matches)."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    dev = float(np.max(np.abs(g - r))) if r.size else 0.0
    m = float(np.max(np.abs(r))) if r.size else 0.0
    return dev / m if m > 0 else dev


MARGINS = {}   # what -> worst (tensor rel, row rel, max-abs ratio), for the run's report


def check_tensors(gpu: dict, ref: dict, prec, what="", tol=None, d=None, key_bias_bound=None, rows_of=None,
                  elem_floor=0.0, tol_extra=None, elementwise=True):
    """Per tensor: relative L2 <= tol, every element within
    max(MAX_ABS_K * tol * max|ref|, elem_floor), and for the embedding-like tables of
    ROW_TABLES every row's relative L2 <= tol. rows_of (optional): ids whose rows of
    wte are reported apart (the rows the embedding scatter writes).

    elem_floor is for parameters after AdamW: an element whose gradient lies within
    rounding of zero takes Adam's nearly sign-like step (about lr) in either
    direction on the two sides, so one element may differ by up to 2 lr per step
    whatever the tolerance; the tensor-wide norm still pins the update as a whole.

    tol_extra (optional, {tensor: band}): added to the bound of that tensor (see
    gate_band_tol).

    elementwise=False keeps only the tensor-wide bound: for the later steps of a
    multi-step run, where the two sides no longer start from the same weights (each
    Adam update moves the elements whose gradient is within rounding of zero by
    about lr either way), so single rows or elements compare two nearby
    trajectories rather than one function at one point."""
    tol = TOL[prec]["rel"] if tol is None else tol
    if d is not None:
        gpu, ref = split_key_bias(gpu, d), split_key_bias(ref, d)
    keys = [k for k in ref if not (d is not None and k.endswith("attn.b.k"))]
    tk = {k: tol + (tol_extra or {}).get(k.rsplit(".attn.b.", 1)[0] + ".attn.b" if ".attn.b." in k else k, 0.0)
          for k in keys}
    worst = max(((rel(gpu[k], ref[k]), k) for k in keys), key=lambda x: x[0])
    bad = {k: (rel(gpu[k], ref[k]), tk[k]) for k in keys if rel(gpu[k], ref[k]) > tk[k]}
    assert not bad, (what, bad)
    ma = {k: max_abs_ratio(gpu[k], ref[k]) for k in keys}
    lim = {k: max(MAX_ABS_K * tk[k], elem_floor / max(float(np.max(np.abs(ref[k]))), 1e-30)) for k in keys}
    bad = {k: (v, lim[k]) for k, v in ma.items() if v > lim[k]}
    assert not (bad and elementwise), (what, "element-wise", bad)
    worst_row = (0.0, "")
    for k in keys:
        if elementwise and k in ROW_TABLES and np.ndim(ref[k]) == 2:
            e = row_errors(gpu[k], ref[k])
            i = int(np.argmax(e))
            if e[i] > worst_row[0]:
                worst_row = (float(e[i]), f"{k}[{i}]")
            assert e[i] <= tk[k], (what, "row", k, i, float(e[i]), int(np.sum(e > tk[k])))
            if rows_of is not None and k == "wte":
                used = np.zeros(len(e), bool)
                used[np.unique(np.asarray(rows_of).reshape(-1))] = True
                say(f"  {what}: wte rows, scatter-written ids worst {float(e[used].max()):.2e}, "
                    f"other rows worst {float(e[~used].max()) if (~used).any() else 0.0:.2e}")
    wma = max(ma.items(), key=lambda x: x[1])
    MARGINS[what] = (worst, worst_row, wma)
    say(f"  {what}: worst rel {worst[0]:.2e} ({worst[1]}), worst row {worst_row[0]:.2e} ({worst_row[1]}), "
        f"worst max-abs {wma[1]:.2e} ({wma[0]})")
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


def gate_band_tol(cfg, prec, params, batches, drop):
    """Extra bound per tensor for the ReLU block in bf16: the oracle's own estimate
    (relu_gate_band) of how far the step's gradients move when the gates within
    operand rounding of zero change side. None for fp32 (rounding 2^-24 flips no gate
    the tolerance would see) and for blocks without ReLU."""
    if prec != "bf16" or getattr(cfg, "variant", "gpt2") != "microgpt":
        return None
    band, frac = O.relu_gate_band(params, batches, cfg, dropout=drop, call0=drop.call if drop is not None else 0)
    say(f"  gate band: {100 * frac:.2f} % of ReLU gates within bf16 rounding of 0; "
        f"largest band {max(band.items(), key=lambda x: x[1])}")
    return band


def run_steps(name, prec, steps=None, B=None, T=None, A=None, perturb=True, check_every=True, cfg=None,
              dropout=0.0, seed=0, counter=0, rel_tol=None, zero_start=()):
    """Runs `steps` optimizer steps on both sides and checks losses, gradients,
    and parameters/moments after every step. With dropout > 0 both sides draw
    their masks from the same seed and forward counter. Parameters whose names end
    with a suffix in `zero_start` start at zero and are checked by check_zero_start.
    The ReLU block in bf16 adds the oracle's gate band (gate_band_tol) to every
    tensor's bound."""
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
        band = gate_band_tol(cfg, prec, tr.p, batches, drop)
        ref = tr.step(batches)
        for i, (a, b) in enumerate(zip(gl, ref["losses"])):
            check_loss(a, b, prec, f"step {s} micro {i}")
        tol = TOL[prec]["rel"] if rel_tol is None else rel_tol
        ball = band["__all__"] if band else 0.0
        assert abs(float(norm_gpu.item()) - ref["norm"]) <= (tol + ball) * ref["norm"], (float(norm_gpu.item()),
                                                                                         ref["norm"])
        # m carries the clip coefficient, which moves with the whole gradient's norm
        mband = {k: v + ball for k, v in band.items()} if band else None
        vband = {k: 2 * v for k, v in mband.items()} if band else None
        if check_every or s == 0:
            ids = np.concatenate([np.asarray(t).reshape(-1) for t, _ in batches])
            wg = check_tensors(g_gpu, ref["grads"], prec, f"grads step {s}", tol=tol, rows_of=ids, tol_extra=band,
                               elementwise=s == 0)
        p_gpu = gpu.params()
        m_gpu, v_gpu = gpu.moments()
        d = cfg.n_embd
        # key bias: each noise-driven Adam step moves it by at most lr (|mhat| <= sqrt(vhat))
        zs = [k for k in tr.p if zero_start and k.endswith(tuple(zero_start))]
        check_zero_start({k: p_gpu[k] for k in zs}, {k: tr.p[k] for k in zs}, cfg.lr, s + 1, f"params step {s}")
        wp = check_tensors(p_gpu, {k: v for k, v in tr.p.items() if k not in zs}, prec, f"params step {s}", tol=tol,
                           d=d, key_bias_bound=2.0 * cfg.lr * (s + 1), elem_floor=2.0 * cfg.lr * (s + 1),
                           tol_extra=mband, elementwise=s == 0)
        gmax = max(float(np.max(np.abs(g))) for g in ref["grads"].values())
        wm = check_tensors(m_gpu, tr.m, prec, f"m step {s}", tol=tol, d=d, key_bias_bound=1e-3 * gmax,
                           tol_extra=mband, elementwise=s == 0)
        wv = check_tensors(v_gpu, tr.v, prec, f"v step {s}", tol=2 * tol, d=d, key_bias_bound=1e-6 * gmax * gmax,
                           tol_extra=vband, elementwise=s == 0)
        report.append((gl, ref["losses"], wg, wp, wm, wv))
        say(f"  step {s}: loss gpu {np.mean(gl):.6f} oracle {ref['loss']:.6f} worst grad {wg[0]:.2e} ({wg[1]}) "
            f"param {wp[0]:.2e} m {wm[0]:.2e} v {wv[0]:.2e}")
    assert gpu.step_count() == steps
    gpu.close()
    return report
