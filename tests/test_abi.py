"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, plans the layout the oracle's table describes, and rejects bad input."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from oracle import gpt_oracle as O
from transformer_lm_gpt_amd import binding as Bd
from transformer_lm_gpt_amd import workloads as W

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "gpt.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gpt_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = Bd.load_library()
    declared = header_functions()
    assert len(declared) >= 19
    assert sorted(Bd.EXPORTS) == declared
    for name in declared:
        assert getattr(lib, name) is not None


def test_library_is_gfx950_only():
    # the shared object carries a gfx950 code object and no other GPU target
    blob = open(Bd.LIB_PATH, "rb").read()
    assert b"gfx950" in blob
    for other in (b"gfx942", b"gfx90a", b"gfx1100", b"sm_80"):
        assert other not in blob


def test_every_launch_stub_has_its_device_kernel():
    # each host launch stub (gpt::__device_stub__<kernel>) must find a kernel
    # descriptor of the same mangled name in the gfx950 code object; a library whose
    # host and device passes saw different versions of a kernel's signature builds
    # and loads, and fails only at the first launch of that kernel
    blob = open(Bd.LIB_PATH, "rb").read()
    stubs = set(re.findall(rb"_ZN3gpt(\d+)__device_stub__([A-Za-z0-9_]+)", blob))
    assert len(stubs) > 100
    missing = []
    for n, tail in stubs:
        name_len = int(n) - len("__device_stub__")
        name, rest = tail[:name_len], tail[name_len:]
        kernel = b"_ZN3gpt" + str(name_len).encode() + name + rest
        if kernel + b".kd" not in blob:
            missing.append(kernel.decode())
    assert not missing, missing


@pytest.mark.parametrize("name", W.ORDER + W.VARIANT_CONFIGS + W.LORA_CONFIGS)
@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_layout_matches_oracle(name, prec):
    cfg = W.CONFIGS[name]
    lay = Bd.Layout(cfg, prec)
    try:
        assert lay.sizes.n_params == O.n_params(cfg)
        table = {n: (shape, dec) for n, _, shape, dec in lay.tensors}
        oracle = {n: (s, O.decays(n, s)) for n, s in O.param_shapes(cfg)}
        assert table == oracle
        # offsets: 64-aligned, disjoint, decayed tensors first, then the 1-D tensors,
        # then the adapters (all after every base tensor)
        spans = sorted((off, off + int(np.prod(shape)), dec, ".lora_" in n) for n, off, shape, dec in lay.tensors)
        for (a0, a1, _, _), (b0, _, _, _) in zip(spans, spans[1:]):
            assert a1 <= b0
        assert all(off % 64 == 0 for _, off, _, _ in lay.tensors)
        kinds = [ad for _, _, _, ad in spans]
        assert kinds == sorted(kinds)
        decs = [dec for _, _, dec, ad in spans if not ad]
        assert decs == sorted(decs, reverse=True)
        assert all(dec for _, _, dec, ad in spans if ad)
        assert spans[-1][1] <= lay.sizes.n_flat and lay.sizes.n_flat % 256 == 0
        assert lay.sizes.shadow_bytes == (lay.sizes.n_flat * 4 if prec == "bf16" else 0)   # weights + transposed weights
        # round trip through the flat layout
        p = W.init_params(cfg, np.random.default_rng(0)) if cfg.padded_vocab < 1000 else None
        if p is not None:
            back = lay.unflatten(lay.flatten(p))
            assert all(np.array_equal(back[k], p[k]) for k in p)
    finally:
        lay.close()


def _raw(**kw):
    c = W.CONFIGS["tiny"]
    r = Bd.make_config(c, "fp32")
    for k, v in kw.items():
        setattr(r, k, v)
    return r


@pytest.mark.parametrize("kw,code", [
    (dict(n_embd=18), -1),                 # not a multiple of n_head
    (dict(n_head=0), -1),
    (dict(padded_vocab=10), -1),           # below vocab_size
    (dict(precision=7), -1),
    (dict(flags=8), -1),                   # unknown flag
    (dict(dropout=1.0), -1),               # dropout must be in [0, 1)
    (dict(dropout=-0.1), -1),
    (dict(dropout=float("nan")), -1),
    (dict(n_embd=512, n_head=4), -4),      # head_dim 128
    (dict(batch=4096, block_size=16), -4),  # M above the single-workgroup sort
    (dict(lora_rank=-1), -1),
    (dict(lora_rank=65), -1),              # above the adapter kernels' rank
    (dict(lora_rank=4, lora_alpha=0.0), -1),
    (dict(lora_rank=4, lora_alpha=float("inf")), -1),
])
def test_create_rejects(kw, code):
    lib = Bd.load_library()
    h = C.c_void_p()
    rc = lib.gpt_create(C.byref(_raw(**kw)), C.byref(h))
    assert rc == code
    assert not h.value
    assert len(lib.gpt_last_error(None)) > 0


def test_calls_before_bind_are_state_errors():
    lib = Bd.load_library()
    lay = Bd.Layout(W.CONFIGS["tiny"], "fp32")
    try:
        assert lib.gpt_backward(lay.h) == -3
        assert lib.gpt_forward_loss(lay.h, None, None, 1, 1, None) == -3
        assert b"bind" in lib.gpt_last_error(lay.h)
    finally:
        lay.close()
    lay = Bd.Layout(W.CONFIGS["tiny"], "bf16")
    try:
        assert lib.gpt_params_loaded(lay.h) == -3
        assert lib.gpt_params_loaded(None) == -1
    finally:
        lay.close()


@pytest.mark.parametrize("name", ["tiny", "char_small", "gpt2_124m"])
def test_debug_checks_flag_is_accepted_and_changes_no_layout(name):
    """GPT_F_DEBUG_CHECKS (4) is a valid flag: the id check reuses the optimizer's
    device state, so sizes and the tensor table are those of the plain model."""
    c = W.CONFIGS[name]
    plain = Bd.Layout(c, "bf16")
    chk = Bd.Layout(c, "bf16", debug_checks=True)
    try:
        assert chk.raw.flags & Bd.F_DEBUG_CHECKS
        for f in ("n_params", "n_flat", "shadow_bytes", "activation_bytes", "workspace_bytes"):
            assert getattr(chk.sizes, f) == getattr(plain.sizes, f), f
        assert chk.tensors == plain.tensors
    finally:
        chk.close()
        plain.close()


def test_bind_rejects_misaligned_and_null():
    lib = Bd.load_library()
    lay = Bd.Layout(W.CONFIGS["tiny"], "bf16")
    try:
        b = Bd.gpt_buffers(256, 512, 768, 1024, None, 1280, 1536)      # shadow missing in bf16 mode
        assert lib.gpt_bind(lay.h, C.byref(b), None) == -1
    finally:
        lay.close()
    lay = Bd.Layout(W.CONFIGS["tiny"], "fp32")
    try:
        b = Bd.gpt_buffers(256 + 4, 512, 768, 1024, None, 1280, 1536)  # misaligned params
        assert lib.gpt_bind(lay.h, C.byref(b), None) == -1
    finally:
        lay.close()


def test_dropout_config_and_seed_are_host_only():
    """A dropout rate in [0, 1) is accepted; the seed call touches no GPU. In fp32
    mode the workspace grows by one fp32 [M, d] array (the masked operand copy)."""
    lib = Bd.load_library()
    c = W.CONFIGS["char_small"]
    plain = Bd.Layout(c, "fp32")
    lay = Bd.Layout(c, "fp32", dropout=0.1)
    try:
        assert lib.gpt_set_dropout_seed(lay.h, 0xFFFFFFFFFFFFFFFF, 7) == 0
        assert lib.gpt_set_dropout_seed(None, 1, 0) == -1
        M = c.batch * c.block_size
        grow = lay.sizes.workspace_bytes - plain.sizes.workspace_bytes
        assert M * c.n_embd * 4 <= grow <= M * c.n_embd * 4 + 256
        assert lay.sizes.activation_bytes == plain.sizes.activation_bytes
    finally:
        lay.close()
        plain.close()


def test_kv_cache_flag_reserves_the_cache():
    """GPT_F_KV_CACHE adds n_layer arrays of [batch * block_size, 2 n_embd] operand
    elements to the workspace, and nothing else."""
    c = W.CONFIGS["char_small"]
    for prec, ob in (("fp32", 4), ("bf16", 2)):
        plain = Bd.Layout(c, prec)
        kv = Bd.Layout(c, prec, kv_cache=True)
        try:
            grow = kv.sizes.workspace_bytes - plain.sizes.workspace_bytes
            want = c.n_layer * c.batch * c.block_size * 2 * c.n_embd * ob
            assert want <= grow <= want + 256
            assert kv.sizes.activation_bytes == plain.sizes.activation_bytes
        finally:
            kv.close()
            plain.close()
