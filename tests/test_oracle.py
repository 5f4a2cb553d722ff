"""Pins for the CPU oracle: page values, closed forms, invariants and finite
differences. None of these compares the oracle with itself."""
import json
import math
import os

import numpy as np
import pytest

from oracle import gpt_oracle as O
from transformer_lm_gpt_amd import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _cfg(**kw):
    base = W.CONFIGS["tiny"]
    return base.with_(**kw)


# --------------------------------------------------------------------------- parameter counts

EXPECTED_COUNTS = {"tiny": 4000, "char_small": 809856, "char_6l": 10770816,
                   "bpe_12l_512": 63847424, "gpt2_124m": 124475904}


@pytest.mark.parametrize("name", W.ORDER)
def test_param_count_closed_form(name):
    c = W.CONFIGS[name]
    V, d, T, L = c.padded_vocab, c.n_embd, c.block_size, c.n_layer
    closed = V * d + T * d + L * (12 * d * d + 13 * d) + 2 * d
    assert O.n_params(c) == closed == EXPECTED_COUNTS[name]


def test_param_count_page_values():
    g = _gold("page_values.json")
    mg = g["microgpt_param_count"]
    c = _cfg(vocab_size=27, padded_vocab=27, n_embd=16, n_head=4, n_layer=1, block_size=16)
    assert O.n_params(c, "microgpt") == mg["value"]
    e = g["bpe_wte_params"]
    wte = dict(O.param_shapes(_cfg(padded_vocab=50257, n_embd=512, n_layer=12, block_size=512)))["wte"]
    assert abs(np.prod(wte) - e["value_approx"]) <= e["rel_tol"] * e["value_approx"]
    a = g["attention_params_per_layer"]
    sh = dict(O.param_shapes(_cfg(n_embd=512, n_layer=1)))
    attn = np.prod(sh["h0.attn.w"]) + np.prod(sh["h0.proj.w"])
    assert abs(attn - a["value_approx"]) <= a["rel_tol"] * a["value_approx"]
    s = g["gpt2_small_params_millions"]
    c = W.CONFIGS["gpt2_124m"].with_(padded_vocab=50257)
    assert abs(O.n_params(c) / 1e6 - s["value_approx"]) <= s["rel_tol"] * s["value_approx"]


def test_generator_table_matches_oracle_layout():
    for name in W.ORDER:
        c = W.CONFIGS[name]
        assert W.tensor_table(c) == O.param_shapes(c)


# --------------------------------------------------------------------------- closed forms

def test_layernorm_closed_form():
    g = _gold("closed_forms.json")["layernorm_pm1"]
    y, _ = O.layernorm_fwd(np.array([g["x"]], float), np.ones(4), np.zeros(4))
    np.testing.assert_allclose(y[0], g["y"], rtol=0, atol=1e-15)


def test_gelu_table_values():
    g = _gold("closed_forms.json")["gelu_values"]
    np.testing.assert_allclose(O.gelu(np.array(g["u"])), g["gelu"], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(O.gelu_grad(np.array(g["u_grad"])), g["gelu_grad"], rtol=1e-14)


def test_gelu_grad_matches_difference_quotient():
    u = np.linspace(-6, 6, 97)
    h = 1e-6
    fd = (O.gelu(u + h) - O.gelu(u - h)) / (2 * h)
    np.testing.assert_allclose(O.gelu_grad(u), fd, atol=1e-8)


def test_gelu_is_exact_not_tanh():
    u = np.linspace(-5, 5, 20001)
    tanh = 0.5 * u * (1 + np.tanh(math.sqrt(2 / math.pi) * (u + 0.044715 * u ** 3)))
    diff = np.abs(O.gelu(u) - tanh)
    assert 4.0e-4 < diff.max() < 5.0e-4


def test_attention_worked_example():
    g = _gold("closed_forms.json")["attention_two_keys"]
    q, k, v = (np.array(g[n], float)[None] for n in ("q", "k", "v"))
    o, p = O.attention_fwd(q, k, v)
    np.testing.assert_allclose(o[0], g["out"], atol=1e-12)


def test_attention_T1_and_zero_query():
    rng = np.random.default_rng(0)
    v = rng.normal(size=(3, 1, 8))
    o, _ = O.attention_fwd(rng.normal(size=(3, 1, 8)), rng.normal(size=(3, 1, 8)), v)
    assert np.array_equal(o, v)
    T = 7
    v = rng.normal(size=(2, T, 8))
    o, p = O.attention_fwd(np.zeros((2, T, 8)), rng.normal(size=(2, T, 8)), v)
    expect = np.cumsum(v, axis=1) / np.arange(1, T + 1)[None, :, None]
    np.testing.assert_allclose(o, expect, atol=1e-13)


def test_attention_brute_force_loops():
    rng = np.random.default_rng(1)
    H, T, hd = 2, 4, 3
    q, k, v = (rng.normal(size=(H, T, hd)) for _ in range(3))
    o, p = O.attention_fwd(q, k, v)
    for h in range(H):
        for i in range(T):
            w = [math.exp(sum(q[h, i, c] * k[h, j, c] for c in range(hd)) / math.sqrt(hd)) for j in range(i + 1)]
            z = sum(w)
            for c in range(hd):
                assert abs(o[h, i, c] - sum(w[j] * v[h, j, c] for j in range(i + 1)) / z) < 1e-12
    assert np.all(p[:, np.triu_indices(T, 1)[0], np.triu_indices(T, 1)[1]] == 0)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-14)


def test_adam_constant_gradient_closed_form():
    g = _gold("closed_forms.json")["adam_constant_gradient"]
    P = {"w": np.array([[g["p0"]]])}
    m = {"w": np.zeros((1, 1))}
    v = {"w": np.zeros((1, 1))}
    for t in range(1, 4):
        O.adamw_update(P, {"w": np.array([[g["g"]]])}, m, v, t, g["lr"], g["beta1"], g["beta2"],
                       g["eps"], g["wd"], 1.0, {"w": True})
        assert abs(P["w"][0, 0] - g["p"][t - 1]) < 1e-12


def test_adam_step1_and_decay_mask():
    rng = np.random.default_rng(2)
    p0 = {"w": rng.normal(size=(3, 4)), "b": rng.normal(size=(4,))}
    gr = {"w": rng.normal(size=(3, 4)), "b": np.zeros(4)}
    P = {k: v.copy() for k, v in p0.items()}
    m = {k: np.zeros_like(v) for k, v in P.items()}
    vv = {k: np.zeros_like(v) for k, v in P.items()}
    lr, wd, eps = 0.01, 0.1, 1e-8
    mask = {k: O.decays(k, v.shape) for k, v in P.items()}
    O.adamw_update(P, gr, m, vv, 1, lr, 0.9, 0.95, eps, wd, 1.0, mask)
    np.testing.assert_allclose(P["w"], p0["w"] * (1 - lr * wd) - lr * gr["w"] / (np.abs(gr["w"]) + eps), rtol=1e-13)
    assert np.array_equal(P["b"], p0["b"])          # no decay on 1-D tensors, zero grad


def test_clip_closed_form():
    rng = np.random.default_rng(3)
    g = {"a": rng.normal(size=(10, 10)), "b": rng.normal(size=(7,))}
    n = O.grad_norm(g)
    assert abs(n - math.sqrt(sum((x ** 2).sum() for x in g.values()))) < 1e-12
    c = O.clip_coef(n, 1.0)
    clipped = math.sqrt(sum(((x * c) ** 2).sum() for x in g.values()))
    assert abs(clipped - n / (n + 1e-6)) < 1e-12
    assert O.clip_coef(n, 1e9) == 1.0
    assert O.clip_coef(n, 0.0) == 1.0


# --------------------------------------------------------------------------- model-level pins

def _setup(name, perturb=False, B=None, T=None, **kw):
    c = W.CONFIGS[name].with_(**kw) if kw else W.CONFIGS[name]
    drng, wrng = W.rngs()
    params = W.init_params(c, wrng, perturb=perturb)
    tok, tgt = W.make_batch(c, drng, B, T)
    return c, params, tok, tgt


@pytest.mark.parametrize("name,B", [("tiny", None), ("char_small", None), ("char_6l", 2), ("bpe_12l_512", 1)])
def test_initial_loss_near_log_vocab(name, B):
    c, params, tok, tgt = _setup(name, B=B)
    z = O.logits(params, tok, c)
    rl, _ = O.microbatch(params, tok, tgt, c)
    L0 = rl.mean()
    expect = math.log(c.padded_vocab) + 0.5 * z.var(axis=-1).mean()
    assert abs(L0 - expect) < 0.05, (L0, expect)


def test_initial_loss_page_value_bpe():
    g = _gold("page_values.json")["initial_loss_bpe"]
    c, params, tok, tgt = _setup("bpe_12l_512", B=1, T=128)
    rl, _ = O.microbatch(params, tok, tgt, c)
    assert abs(rl.mean() - g["value_approx"]) < g["abs_tol"]


def test_zero_wte_gives_log_vocab_and_uniform_dlogits():
    c, params, tok, tgt = _setup("tiny", perturb=True)
    params["wte"][:] = 0.0
    z = O.logits(params, tok, c)
    assert np.all(z == 0.0)
    rl, _ = O.microbatch(params, tok, tgt, c)
    assert np.allclose(rl, math.log(c.padded_vocab), rtol=0, atol=1e-14)
    ell, sm = O.xent_rows(z[0], tgt[0])
    dz = sm.copy()
    dz[np.arange(len(tgt[0])), tgt[0]] -= 1
    expect = np.full_like(dz, 1.0 / c.padded_vocab)
    expect[np.arange(len(tgt[0])), tgt[0]] -= 1
    np.testing.assert_allclose(dz, expect, atol=1e-15)


def test_dlogits_rows_sum_to_zero():
    c, params, tok, tgt = _setup("char_small", perturb=True, B=2)
    z = O.logits(params, tok, c)
    ell, sm = O.xent_rows(z[0], tgt[0])
    dz = sm.copy()
    dz[np.arange(len(tgt[0])), tgt[0]] -= 1
    assert np.abs(dz.sum(-1)).max() < 1e-14
    np.testing.assert_allclose(sm.sum(-1), 1.0, atol=1e-14)


def test_causality_bitwise():
    c, params, tok, tgt = _setup("char_small", perturb=True, B=2)
    z0 = O.logits(params, tok, c)
    t = 20
    tok2 = tok.copy()
    tok2[:, t + 1:] = (tok2[:, t + 1:] + 17) % c.vocab_size
    z1 = O.logits(params, tok2, c)
    assert np.array_equal(z0[:, :t + 1], z1[:, :t + 1])
    assert not np.array_equal(z0[:, t + 1:], z1[:, t + 1:])


def test_layernorm_invariants():
    rng = np.random.default_rng(4)
    x = rng.normal(size=(5, 32)) * 3 + 1
    y, cache = O.layernorm_fwd(x, np.ones(32), np.zeros(32))
    np.testing.assert_allclose(y.mean(-1), 0, atol=1e-14)
    np.testing.assert_allclose((y ** 2).mean(-1), 1 / (1 + 1e-5 / x.var(-1)), rtol=1e-12)
    dy = rng.normal(size=(5, 32))
    dx, dg, db = O.layernorm_bwd(dy, cache, np.ones(32))
    np.testing.assert_allclose(dx.sum(-1), 0, atol=1e-13)
    # orthogonal to xhat up to the eps term: sum(dx xhat) = rstd sum(dy xhat) eps / (var + eps)
    xhat, rstd = cache
    var = x.var(-1, keepdims=True)
    expect = (rstd * (dy * xhat).sum(-1, keepdims=True) * 1e-5 / (var + 1e-5))[:, 0]
    np.testing.assert_allclose((dx * xhat).sum(-1), expect, rtol=1e-6, atol=1e-15)
    np.testing.assert_allclose(dg, (dy * xhat).sum(0), rtol=1e-14)
    np.testing.assert_allclose(db, dy.sum(0), rtol=1e-14)


def _fd_check(c, params, tok, tgt, n_random=20, seed=5, dropout=None):
    P = {k: v.astype(np.float64) for k, v in params.items()}
    B, T = tok.shape
    call = 7            # one fixed forward counter: every evaluation sees the same masks
    _, G = O.microbatch(P, tok, tgt, c, grad_scale=1.0 / (B * T), dropout=dropout, call=call)

    def loss(Pp):
        return O.microbatch(Pp, tok, tgt, c, dropout=dropout, call=call)[0].mean()

    rng = np.random.default_rng(seed)
    h = 1e-5
    checked = 0
    for name, arr in P.items():
        flat = arr.reshape(-1)
        if arr.ndim == 1:
            idx = np.arange(flat.size)                     # every bias / gain / shift
        else:
            idx = rng.choice(flat.size, size=min(n_random, flat.size), replace=False)
            if name == "wte":                              # rows that are inputs and targets
                idx = np.unique(np.concatenate([idx, tok[0, :3] * arr.shape[1], tgt[0, :3] * arr.shape[1] + 1]))
        g = G[name].reshape(-1)
        scale = np.abs(g).max() + 1e-12
        for i in idx:
            old = flat[i]
            flat[i] = old + h
            lp = loss(P)
            flat[i] = old - h
            lm = loss(P)
            flat[i] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[i]) <= 1e-6 * scale + 1e-10, (name, int(i), fd, g[i])
            checked += 1
    return checked


def test_finite_difference_tiny():
    c, params, tok, tgt = _setup("tiny", perturb=True)
    assert _fd_check(c, params, tok, tgt) > 200


@pytest.mark.slow
def test_finite_difference_shrunk_char():
    c = W.CONFIGS["char_small"].with_(n_layer=2, n_embd=32, n_head=4, block_size=8, batch=2)
    drng, wrng = W.rngs()
    params = W.init_params(c, wrng, perturb=True)
    tok, tgt = W.make_batch(c, drng)
    assert _fd_check(c, params, tok, tgt, n_random=8) > 500


# --------------------------------------------------------------------------- dropout

def test_philox_known_answers():
    """Philox4x32-10 against the generator's published known-answer vectors."""
    for v in _gold("philox4x32_10_kat.json")["vectors"]:
        ctr = np.array([int(x, 16) for x in v["counter"]], dtype=np.uint64)
        key = [int(x, 16) for x in v["key"]]
        out = O.philox4x32(ctr, key)
        assert [int(x) for x in out] == [int(x, 16) for x in v["out"]]


def test_dropout_threshold_and_scale():
    d = O.Dropout(0.25, 1)
    assert d.thr == 1 << 30
    assert d.scale == float(np.float32(4.0 / 3.0))
    z = O.Dropout(0.0, 1)
    assert z.thr == 0 and z.scale == 1.0
    with pytest.raises(ValueError):
        O.Dropout(1.0, 1)


def test_dropout_keep_rate_unbiased_and_independent():
    """Kept fraction 1 - p, E[keep * scale] = 1 (inverted dropout), and masks of
    different sites, calls and seeds are independent (joint keep rate (1-p)^2)."""
    p = 0.3
    d = O.Dropout(p, 0x0123456789ABCDEF)
    rows = np.arange(1024)
    a = O.dropout_keep(d, 5, 2, rows, 1024)
    n = a.size
    sd = math.sqrt(p * (1 - p) / n)
    assert abs(a.mean() - (1 - p)) < 5 * sd
    z = a * d.scale
    assert abs(z.mean() - 1.0) < 5 * d.scale * sd
    for other in (O.dropout_keep(d, 5, 3, rows, 1024),                 # another site
                  O.dropout_keep(d, 6, 2, rows, 1024),                 # another forward
                  O.dropout_keep(O.Dropout(p, 0x0123456789ABCDEE), 5, 2, rows, 1024),   # another seed
                  O.dropout_keep(d, 5, 2, rows + 1024, 1024)):         # other rows
        both = (a & other).mean()
        assert abs(both - (1 - p) ** 2) < 5 * math.sqrt((1 - p) ** 2 * (1 - (1 - p) ** 2) / n)


def test_dropout_counter_layout_brute_force():
    """Element (row, col) takes word col % 4 of the block at counter (col // 4, row, site, call)."""
    d = O.Dropout(0.5, (7 << 32) | 9)
    rows = [0, 3, 70000]
    m = O.dropout_keep(d, 11, 4, rows, 10)
    for i, r in enumerate(rows):
        for c in range(10):
            w = O.philox4x32(np.array([c // 4, r, 4, 11], dtype=np.uint64), (9, 7))[c % 4]
            assert m[i, c] == (int(w) >= d.thr)


def test_dropout_zero_rate_is_bitwise_identity():
    c, params, tok, tgt = _setup("tiny", perturb=True)
    B, T = tok.shape
    l0, g0 = O.microbatch(params, tok, tgt, c, grad_scale=1.0 / (B * T))
    l1, g1 = O.microbatch(params, tok, tgt, c, grad_scale=1.0 / (B * T), dropout=O.Dropout(0.0, 3))
    assert np.array_equal(l0, l1)
    for k in g0:
        assert np.array_equal(g0[k], g1[k])


def test_attention_dropout_uniform_queries():
    """q = 0 makes every row of P uniform over the visible keys, so the dropped
    output is O_i = sum_{j<=i} z_ij v_j / (i + 1) with z = keep * scale."""
    H, T, hd = 2, 6, 4
    rng = np.random.default_rng(3)
    k = rng.normal(size=(H, T, hd))
    v = rng.normal(size=(H, T, hd))
    d = O.Dropout(0.4, 99)
    keep = O.dropout_keep(d, 0, 1, np.arange(H * T), T).reshape(H, T, T)
    z = keep * d.scale
    out, p = O.attention_fwd(np.zeros((H, T, hd)), k, v, z)
    for h in range(H):
        for i in range(T):
            expect = sum(z[h, i, j] * v[h, j] for j in range(i + 1)) / (i + 1)
            np.testing.assert_allclose(out[h, i], expect, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=1e-14)     # P itself is returned undropped


def test_finite_difference_tiny_with_dropout():
    """With the masks fixed (one forward counter), dropout is linear in each
    masked value, so central differences pin every mask in the backward."""
    c, params, tok, tgt = _setup("tiny", perturb=True)
    assert _fd_check(c, params, tok, tgt, dropout=O.Dropout(0.3, 0xDEADBEEF12345)) > 200


def test_dropout_changes_loss_and_advances_counter():
    c, params, tok, tgt = _setup("tiny", perturb=True)
    d = O.Dropout(0.2, 5, call=3)
    l1, _ = O.microbatch(params, tok, tgt, c, dropout=d)
    assert d.call == 4
    l2, _ = O.microbatch(params, tok, tgt, c, dropout=d)
    l0, _ = O.microbatch(params, tok, tgt, c)
    assert not np.array_equal(l1, l2) and not np.array_equal(l1, l0)
    l1b, _ = O.microbatch(params, tok, tgt, c, dropout=d, call=3)
    assert np.array_equal(l1, l1b)


# --------------------------------------------------------------------------- sampling

def test_sample_two_logit_closed_form():
    """z = (0, ln 3): softmax (1/4, 3/4) at temperature 1 and (1/10, 9/10) at 1/2."""
    z = np.array([0.0, math.log(3.0)])
    assert O.sample_token(z, 1.0, 0, 0.2) == 0 and O.sample_token(z, 1.0, 0, 0.3) == 1
    assert O.sample_token(z, 0.5, 0, 0.05) == 0 and O.sample_token(z, 0.5, 0, 0.15) == 1
    assert O.sample_token(z, 1.0, 0, 0.0) == 0 and O.sample_token(z, 1.0, 0, 0.999999) == 1


def test_sample_greedy_and_top1_are_argmax():
    rng = np.random.default_rng(8)
    for _ in range(50):
        z = rng.normal(size=97) * 3
        a = int(np.argmax(z))
        assert O.sample_token(z, 0.0, 0, 0.7) == a
        assert O.sample_token(z, 1.3, 1, float(rng.random())) == a
    assert O.sample_token(np.array([1.0, 5.0, 5.0, 2.0]), 0.0, 0, 0.5) == 1     # lowest index on ties


def test_sample_stratified_frequencies_match_softmax():
    """With stratified uniforms the token frequencies equal the probabilities of
    softmax(z / T) restricted to the top-k logits, up to the 1/N stratum width."""
    from scipy.special import softmax
    rng = np.random.default_rng(9)
    z = rng.normal(size=40) * 2
    N = 20000
    for temp, k in ((1.0, 0), (0.7, 10), (2.0, 3)):
        cnt = np.zeros(40)
        for i in range(N):
            cnt[O.sample_token(z, temp, k, (i + 0.5) / N)] += 1
        keep = np.argsort(-z)[:k] if k else np.arange(40)
        p = np.zeros(40)
        p[keep] = softmax(z[keep] / temp)
        assert np.abs(cnt / N - p).max() <= 1.0 / N + 1e-12
        assert np.all(cnt[np.setdiff1d(np.arange(40), keep)] == 0)


def test_sample_top_k_keeps_ties_at_the_cut():
    z = np.array([1.0, 2.0, 2.0, 0.0])
    picked = {O.sample_token(z, 1.0, 1, u) for u in (0.1, 0.9)}
    assert picked == {1, 2}


def test_generate_greedy_is_argmax_of_full_forward():
    c, params, tok, _ = _setup("tiny", perturb=True)
    prompt = tok[:2, :5]
    seqs, zs = O.generate(params, prompt, c, 4, 0.0, 0, np.zeros((4, 2)))
    assert seqs.shape == (2, 9) and np.array_equal(seqs[:, :5], prompt)
    for s in range(4):
        z_full = O.logits(params, seqs[:, :5 + s], c)[:, -1]
        np.testing.assert_allclose(zs[s], z_full, rtol=1e-12, atol=1e-12)
        assert np.array_equal(seqs[:, 5 + s], np.argmax(z_full, axis=-1))


def test_grad_accumulation_equals_big_batch():
    c, params, tok, tgt = _setup("char_small", perturb=True, B=4, T=16)
    _, g_big = O.accumulate_grads(params, [(tok, tgt)], c)
    _, g_acc = O.accumulate_grads(params, [(tok[:2], tgt[:2]), (tok[2:], tgt[2:])], c)
    for k in g_big:
        np.testing.assert_allclose(g_acc[k], g_big[k], rtol=1e-12, atol=1e-17)


# --------------------------------------------------------------------------- generators

def test_generators_deterministic():
    for name in ["tiny", "char_small", "char_6l", "gpt2_124m"]:
        c = W.CONFIGS[name]
        a = W.make_batch(c, W.rngs()[0], B=2, T=16)
        b = W.make_batch(c, W.rngs()[0], B=2, T=16)
        assert a[0].tobytes() == b[0].tobytes() and a[1].tobytes() == b[1].tobytes()
        assert np.array_equal(a[0][:, 1:], a[1][:, :-1])        # targets are the next tokens
        assert a[0].min() >= 0 and a[0].max() < c.vocab_size
    p1 = W.init_params(W.CONFIGS["char_small"], W.rngs()[1])
    p2 = W.init_params(W.CONFIGS["char_small"], W.rngs()[1])
    assert all(p1[k].tobytes() == p2[k].tobytes() for k in p1)


def test_zipf_head_mass():
    assert abs(W.zipf_cdf(65, 1.1)[0] - 0.250) < 0.001
    assert abs(W.zipf_cdf(50257, 1.07)[0] - 0.122) < 0.001
    c = W.CONFIGS["gpt2_124m"]
    tok, _ = W.make_batch(c, W.rngs()[0])
    assert abs((tok == 0).mean() - 0.122) < 0.01


def test_init_std_and_residual_scale():
    c = W.CONFIGS["gpt2_124m"].with_(padded_vocab=64, block_size=64)
    p = W.init_params(c, W.rngs()[1])
    assert abs(p["h0.fc.w"].std() - 0.02) < 5e-4
    assert abs(p["h0.fcproj.w"].std() - 0.02 / math.sqrt(24)) < 2e-4
    assert abs(p["h0.proj.w"].std() - 0.02 / math.sqrt(24)) < 3e-4
    assert np.all(p["h0.ln1.g"] == 1) and np.all(p["h0.attn.b"] == 0)


# --------------------------------------------------------------------------- the microGPT variant

def test_micro_param_count_is_the_page_value():
    g = _gold("page_values.json")["microgpt_param_count"]
    c = W.CONFIGS["micro"]
    assert O.n_params(c) == g["value"] == 4192
    assert W.tensor_table(c) == O.param_shapes(c)
    assert all(len(sh) == 2 for _, sh in O.param_shapes(c))          # every tensor decays


def test_rmsnorm_closed_form_and_invariants():
    """x = (1, -1, 1, -1): mean square 1, so y = x / sqrt(1 + 1e-5); x = (3, 4):
    mean square 12.5. The input gradient is orthogonal to xhat up to the eps term:
    sum(dx xhat) = rstd sum(dy xhat) eps / (ms + eps)."""
    y, _ = O.rmsnorm_fwd(np.array([[1.0, -1.0, 1.0, -1.0]]))
    np.testing.assert_allclose(y, [[x / math.sqrt(1 + 1e-5) for x in (1, -1, 1, -1)]], rtol=1e-15)
    y, _ = O.rmsnorm_fwd(np.array([[3.0, 4.0]]))
    np.testing.assert_allclose(y, [[3 / math.sqrt(12.5 + 1e-5), 4 / math.sqrt(12.5 + 1e-5)]], rtol=1e-15)
    rng = np.random.default_rng(11)
    x = rng.normal(size=(6, 24)) * 2 + 0.5
    dy = rng.normal(size=(6, 24))
    xh, cache = O.rmsnorm_fwd(x)
    dx = O.rmsnorm_bwd(dy, cache)
    ms = (x * x).mean(-1, keepdims=True)
    rstd = cache[1]
    expect = (rstd * (dy * xh).sum(-1, keepdims=True) * 1e-5 / (ms + 1e-5))[:, 0]
    np.testing.assert_allclose((dx * xh).sum(-1), expect, rtol=1e-6, atol=1e-15)


def test_micro_zero_head_gives_log_vocab():
    c = W.CONFIGS["micro"]
    drng, wrng = W.rngs()
    params = W.init_params(c, wrng)
    params["lm_head"][:] = 0.0
    tok, tgt = W.make_batch(c, drng)
    rl, _ = O.microbatch(params, tok, tgt, c)
    np.testing.assert_allclose(rl, math.log(c.padded_vocab), rtol=0, atol=1e-12)


def test_finite_difference_micro():
    c = W.CONFIGS["micro"]
    drng, wrng = W.rngs()
    params = W.init_params(c, wrng)
    tok, tgt = W.make_batch(c, drng)
    assert _fd_check(c, params, tok, tgt) > 100


def test_finite_difference_micro_with_dropout():
    c = W.CONFIGS["micro"]
    drng, wrng = W.rngs()
    params = W.init_params(c, wrng)
    tok, tgt = W.make_batch(c, drng)
    assert _fd_check(c, params, tok, tgt, dropout=O.Dropout(0.25, 77)) > 100


# --------------------------------------------------------------------------- LoRA adapters
# The fine-tuning article (blog.hotdry.top), LoRA section: W0 frozen, low-rank A and B
# on the q and v projections, h = W0 x + B A x scaled by lora_alpha / r, only A and B
# trained, and B A can be merged into W0.

@pytest.mark.parametrize("name", W.LORA_CONFIGS)
def test_lora_layout_and_count(name):
    c = W.CONFIGS[name]
    assert W.tensor_table(c) == O.param_shapes(c)
    base = O.n_params(c.with_(lora_rank=0))
    L, d, r = c.n_layer, c.n_embd, c.lora_rank
    assert O.n_params(c) - base == 4 * L * d * r          # A [r, d] and B [d, r], for q and v
    trained = [n for n, _ in O.param_shapes(c) if O.trainable(c, n)]
    assert len(trained) == 4 * L and all(".lora_" in n for n in trained)
    assert O.lora_of(c) == (r, c.lora_alpha / r)


def test_lora_zero_B_is_the_base_model_bitwise():
    c, params, tok, tgt = _setup("tiny_lora")               # B = 0, A random
    assert all(not np.any(params[f"h{l}.lora_{t}.B"]) for l in range(c.n_layer) for t in "qv")
    base = {k: v for k, v in params.items() if ".lora_" not in k}
    z = O.logits(params, tok, c)
    zb = O.logits(base, tok, c.with_(lora_rank=0))
    assert np.array_equal(z, zb)
    # with B = 0 the A gradient vanishes exactly (its only path runs through B)
    _, G = O.microbatch(params, tok, tgt, c, grad_scale=1.0 / tok.size)
    for l in range(c.n_layer):
        for t in "qv":
            assert not np.any(G[f"h{l}.lora_{t}.A"])
            assert np.any(G[f"h{l}.lora_{t}.B"])


@pytest.mark.parametrize("name,B", [("tiny_lora", None), ("char_small_lora", 2)])
def test_lora_equals_merged_weight(name, B):
    # the article's merge: W0 + s B A in the q and v row blocks gives the same model
    c, params, tok, tgt = _setup(name, perturb=True, B=B)
    r, s = O.lora_of(c)
    d = c.n_embd
    merged = {k: v.astype(np.float64).copy() for k, v in params.items() if ".lora_" not in k}
    for l in range(c.n_layer):
        w = merged[f"h{l}.attn.w"]
        for t, rows in (("q", slice(0, d)), ("v", slice(2 * d, 3 * d))):
            Bm = params[f"h{l}.lora_{t}.B"].astype(np.float64)
            Am = params[f"h{l}.lora_{t}.A"].astype(np.float64)
            w[rows] += s * (Bm @ Am)
    z = O.logits(params, tok, c)
    zm = O.logits(merged, tok, c.with_(lora_rank=0))
    assert np.max(np.abs(z - zm)) <= 1e-12 * np.max(np.abs(zm))
    assert np.max(np.abs(z - O.logits({k: v for k, v in params.items() if ".lora_" not in k}, tok,
                                      c.with_(lora_rank=0)))) > 1e-3   # the adapters do change the model


def test_finite_difference_tiny_lora():
    c, params, tok, tgt = _setup("tiny_lora", perturb=True)
    assert _fd_check(c, params, tok, tgt) > 250


def test_lora_first_step_closed_form_and_frozen_base():
    # B0 = 0: dA = 0, so A only decays, A1 = A0 (1 - lr wd); B1 = -lr c g / (c |g| + eps)
    # elementwise (the Adam step-1 closed form with clip coefficient c); nothing else moves.
    c = W.CONFIGS["tiny_lora"].with_(weight_decay=0.1, grad_clip=0.05)
    drng, wrng = W.rngs()
    params = W.init_params(c, wrng)
    batches = W.make_step_batches(c, drng)
    tr = O.Trainer(params, c)
    out = tr.step(batches)
    assert set(out["grads"]) == {n for n in params if ".lora_" in n}
    norm = math.sqrt(sum(float(np.sum(g.astype(np.float64) ** 2)) for g in out["grads"].values()))
    assert out["norm"] == pytest.approx(norm, rel=1e-12)
    coef = O.clip_coef(norm, c.grad_clip)
    assert coef < 1.0
    for k, p0 in params.items():
        p1 = tr.p[k]
        if ".lora_" not in k:
            assert np.array_equal(p1, p0.astype(np.float64)), k
        elif k.endswith(".A"):
            np.testing.assert_allclose(p1, p0.astype(np.float64) * (1.0 - c.lr * c.weight_decay), rtol=1e-15, atol=0)
        else:
            g = out["grads"][k]
            np.testing.assert_allclose(p1, -c.lr * coef * g / (coef * np.abs(g) + c.eps), rtol=1e-12, atol=1e-15)


# --------------------------------------------------------------------------- the ReLU gate band

def _micro_case(B=2):
    cfg = W.CONFIGS["micro"]
    drng, wrng = W.rngs()
    params = W.init_params(cfg, wrng)
    return cfg, params, [W.make_batch(cfg, drng, B=B)]


def test_gate_band_zero_rounding_flips_nothing():
    cfg, params, batches = _micro_case()
    band, frac = O.relu_gate_band(params, batches, cfg, rel_round=0.0)
    assert frac == 0.0 and all(v == 0.0 for v in band.values())


def test_gate_band_counts_the_gates_a_loop_finds():
    """The ambiguous fraction against a plain loop over every pre-activation of the
    one-layer toy: |u_mj| <= 2^-7 sum_k |b_mk W_jk|."""
    cfg, params, batches = _micro_case()
    _, frac = O.relu_gate_band(params, batches, cfg)
    P = {k: v.astype(np.float64) for k, v in params.items()}
    W_ = P["h0.fc.w"]
    amb = tot = 0
    for tok in batches[0][0]:
        _, cache = O.forward_sequence(P, tok, cfg)
        b2, u = cache[1][0][7], cache[1][0][9]
        for m in range(b2.shape[0]):
            for j in range(W_.shape[0]):
                s = sum(abs(b2[m, k] * W_[j, k]) for k in range(b2.shape[1]))
                amb += abs(u[m, j]) <= 2.0 ** -7 * s
                tot += 1
    assert amb > 0 and frac == amb / tot


def test_gate_band_all_flipped_is_the_complementary_gate():
    """With every gate ambiguous the band is the gradient formed with the other side
    of every gate, which the oracle's backward gives when fed -u."""
    cfg, params, batches = _micro_case()
    band, frac = O.relu_gate_band(params, batches, cfg, rel_round=1e30)
    assert frac == 1.0
    P = {k: v.astype(np.float64) for k, v in params.items()}
    tok, tgt = batches[0]
    B, T = tok.shape
    G0 = {k: np.zeros_like(v) for k, v in P.items()}
    G1 = {k: np.zeros_like(v) for k, v in P.items()}
    for b in range(B):
        z, cache = O.forward_sequence(P, tok[b], cfg)
        _, dz = O.xent_rows(z, tgt[b])
        dz[np.arange(T), tgt[b]] -= 1.0
        dz /= B * T
        O.backward_sequence(P, cache, dz, cfg, G0)
        neg = [lay[:9] + (-lay[9],) + lay[10:] for lay in cache[1]]
        O.backward_sequence(P, (cache[0], neg) + tuple(cache[2:]), dz, cfg, G1)
    for k in P:
        want = np.linalg.norm(G1[k] - G0[k]) / np.linalg.norm(G0[k])
        assert abs(band[k] - want) <= 1e-12 * max(1.0, want), k
    assert band["h0.fc.w"] > 0.1     # the flip is visible, not rounding noise


def test_gate_band_needs_the_relu_block():
    cfg = W.CONFIGS["tiny"]
    with pytest.raises(ValueError):
        O.relu_gate_band({}, [], cfg)
