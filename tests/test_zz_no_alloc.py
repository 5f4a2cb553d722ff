"""gpt_adamw_step_noalloc, the AdamW update whose gradient-norm partials live in the
library's static device array, against gpt_adamw_step through the C ABI: two
models side by side, one per entry point, same weights and batches, compared
bitwise (same kernels in the same order). Two calls in a row on one GPU, the
second on a smaller model, so the second reads the array the first wrote."""
import numpy as np
import pytest

from transformer_lm_gpt_amd import workloads as W

from gpu_helpers import new_model, say

pytestmark = pytest.mark.gpu


def _pair_step(name, prec, steps):
    cfg = W.CONFIGS[name]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng, perturb=True)
    a, b = new_model(cfg, prec), new_model(cfg, prec)
    a.load_params(params)
    b.load_params(params)
    for s in range(steps):
        batches = W.make_step_batches(cfg, drng)
        for g in (a, b):
            for tok, tgt in batches:
                g.forward_loss(tok, tgt)
                g.backward()
        na = float(a.adamw_step(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.grad_clip).item())
        nb = float(b.adamw_step(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.grad_clip,
                                noalloc=True).item())
        a.sync()
        b.sync()
        assert na == nb, (name, s, na, nb)
    pa, pb = a.params(), b.params()
    (ma, va), (mb, vb) = a.moments(), b.moments()
    for k in pa:
        assert np.array_equal(pa[k], pb[k]) and np.array_equal(ma[k], mb[k]) and np.array_equal(va[k], vb[k]), k
    assert a.step_count() == b.step_count() == steps
    say(f"[noalloc] {name} {prec}: {steps} steps, norm {nb:.6f}, parameters and moments bitwise equal")
    a.close()
    b.close()


def test_noalloc_adamw_equals_the_workspace_entry_point():
    _pair_step("char_small", "bf16", 2)    # 0.8 M parameters
    _pair_step("tiny", "fp32", 2)          # then 4,000: a smaller gradient over the same array


def test_noalloc_adamw_errors_like_the_entry_point():
    from transformer_lm_gpt_amd.binding import GPTError
    cfg = W.CONFIGS["tiny"]
    g = new_model(cfg, "fp32")
    g.load_params(W.init_params(cfg, W.rngs()[1]))
    with pytest.raises(GPTError) as e:     # no backward since the last update
        g.adamw_step(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay, cfg.grad_clip, noalloc=True)
    assert e.value.code == -3
    g.close()
