"""Thin ctypes binding of libgpt.so (include/gpt.h).

The binding only marshals arguments: PyTorch allocates the device buffers the
library asks for and supplies the HIP stream; every step of the training step
runs in the library's gfx950 kernels. If the library has not been built the
import of `load_library` fails loudly; there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, List, Optional, Tuple

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
# GPT_MI355X_LIB names another build of the library (to compare two builds side by side)
LIB_PATH = os.environ.get("GPT_MI355X_LIB") or os.path.join(PKG, "libgpt.so")

GPT_OK = 0
ERRORS = {-1: "GPT_E_INVAL", -2: "GPT_E_SEQ_TOO_LONG", -3: "GPT_E_STATE", -4: "GPT_E_UNSUPPORTED",
          -5: "GPT_E_HIP", -6: "GPT_E_NONFINITE"}
PREC = {"fp32": 0, "bf16": 1}

# Every symbol include/gpt.h declares.
EXPORTS = ["gpt_create", "gpt_destroy", "gpt_last_error", "gpt_get_sizes", "gpt_num_tensors",
           "gpt_tensor_info_at", "gpt_bind", "gpt_init_state", "gpt_params_loaded", "gpt_forward_loss",
           "gpt_forward_logits",
           "gpt_backward", "gpt_zero_grad", "gpt_set_dropout_seed", "gpt_adamw_step", "gpt_sync", "gpt_get_step",
           "gpt_prefill", "gpt_decode", "gpt_sample", "gpt_adamw_step_noalloc",
           "gpt_debug_copy", "gpt_timer_enable", "gpt_timer_disable", "gpt_timer_read"]


class GPTError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


class gpt_config(C.Structure):
    _fields_ = [("vocab_size", C.c_int32), ("padded_vocab", C.c_int32), ("n_layer", C.c_int32),
                ("n_head", C.c_int32), ("n_embd", C.c_int32), ("block_size", C.c_int32),
                ("batch", C.c_int32), ("grad_accum", C.c_int32), ("precision", C.c_int32),
                ("dropout", C.c_float), ("flags", C.c_uint32), ("lora_rank", C.c_int32),
                ("lora_alpha", C.c_float)]


class gpt_sizes(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in ("n_params", "n_flat", "param_bytes", "grad_bytes", "m_bytes",
                                          "v_bytes", "shadow_bytes", "activation_bytes", "workspace_bytes")]


class gpt_tensor_info(C.Structure):
    _fields_ = [("name", C.c_char * 48), ("offset", C.c_size_t), ("ndim", C.c_int32),
                ("shape", C.c_int64 * 2), ("decay", C.c_int32)]


class gpt_buffers(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("params", "grads", "m", "v", "shadow", "activations", "workspace")]


_lib: Optional[C.CDLL] = None


def load_library(path: str = LIB_PATH) -> C.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m transformer_lm_gpt_amd.build`")
    lib = C.CDLL(path)
    vp, i32, f32 = C.c_void_p, C.c_int32, C.c_float
    sig = {
        "gpt_create": (C.c_int, [C.POINTER(gpt_config), C.POINTER(vp)]),
        "gpt_destroy": (None, [vp]),
        "gpt_last_error": (C.c_char_p, [vp]),
        "gpt_get_sizes": (C.c_int, [vp, C.POINTER(gpt_sizes)]),
        "gpt_num_tensors": (C.c_int, [vp]),
        "gpt_tensor_info_at": (C.c_int, [vp, C.c_int, C.POINTER(gpt_tensor_info)]),
        "gpt_bind": (C.c_int, [vp, C.POINTER(gpt_buffers), vp]),
        "gpt_init_state": (C.c_int, [vp]),
        "gpt_params_loaded": (C.c_int, [vp]),
        "gpt_forward_loss": (C.c_int, [vp, vp, vp, i32, i32, vp]),
        "gpt_forward_logits": (C.c_int, [vp, vp, i32, i32, vp]),
        "gpt_backward": (C.c_int, [vp]),
        "gpt_zero_grad": (C.c_int, [vp]),
        "gpt_set_dropout_seed": (C.c_int, [vp, C.c_uint64, C.c_uint32]),
        "gpt_prefill": (C.c_int, [vp, vp, i32, i32, vp]),
        "gpt_decode": (C.c_int, [vp, vp, vp]),
        "gpt_sample": (C.c_int, [vp, vp, i32, f32, i32, vp, vp]),
        "gpt_adamw_step": (C.c_int, [vp, f32, f32, f32, f32, f32, f32, vp]),
        "gpt_adamw_step_noalloc": (C.c_int, [vp, f32, f32, f32, f32, f32, f32, vp]),
        "gpt_sync": (C.c_int, [vp]),
        "gpt_get_step": (C.c_int, [vp, C.POINTER(C.c_int64)]),
        "gpt_debug_copy": (C.c_int, [vp, C.c_char_p, i32, vp, C.c_size_t]),
        "gpt_timer_enable": (C.c_int, [vp, C.c_char_p]),
        "gpt_timer_disable": (C.c_int, [vp]),
        "gpt_timer_read": (C.c_int, [vp, C.POINTER(C.c_double), C.POINTER(C.c_int64)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


F_KV_CACHE = 1
F_MICROGPT = 2
F_DEBUG_CHECKS = 4


def make_config(cfg, precision: str, batch: Optional[int] = None, grad_accum: Optional[int] = None,
                dropout: float = 0.0, kv_cache: bool = False, debug_checks: bool = False) -> gpt_config:
    return gpt_config(cfg.vocab_size, cfg.padded_vocab, cfg.n_layer, cfg.n_head, cfg.n_embd, cfg.block_size,
                      cfg.batch if batch is None else batch,
                      cfg.grad_accum if grad_accum is None else grad_accum, PREC[precision], float(dropout),
                      (F_KV_CACHE if kv_cache else 0) | (F_MICROGPT if getattr(cfg, "variant", "gpt2") == "microgpt" else 0)
                      | (F_DEBUG_CHECKS if debug_checks else 0),
                      int(getattr(cfg, "lora_rank", 0)), float(getattr(cfg, "lora_alpha", 0.0)))


class Layout:
    """Host-side view of a configuration: sizes and the flat tensor table. Needs no GPU."""

    def __init__(self, cfg, precision: str = "bf16", batch: Optional[int] = None,
                 grad_accum: Optional[int] = None, raw: Optional[gpt_config] = None, dropout: float = 0.0,
                 kv_cache: bool = False, debug_checks: bool = False):
        self.lib = load_library()
        self.cfg = cfg
        self.precision = precision
        self.raw = raw if raw is not None else make_config(cfg, precision, batch, grad_accum, dropout, kv_cache,
                                                           debug_checks)
        h = C.c_void_p()
        rc = self.lib.gpt_create(C.byref(self.raw), C.byref(h))
        if rc != GPT_OK:
            raise GPTError(rc, self.lib.gpt_last_error(None).decode())
        self.h = h
        self.sizes = gpt_sizes()
        self._check(self.lib.gpt_get_sizes(h, C.byref(self.sizes)))
        self.tensors: List[Tuple[str, int, Tuple[int, ...], bool]] = []
        for i in range(self.lib.gpt_num_tensors(h)):
            ti = gpt_tensor_info()
            self._check(self.lib.gpt_tensor_info_at(h, i, C.byref(ti)))
            shape = (int(ti.shape[0]), int(ti.shape[1])) if ti.ndim == 2 else (int(ti.shape[0]),)
            self.tensors.append((ti.name.decode(), int(ti.offset), shape, bool(ti.decay)))

    def _check(self, rc: int):
        if rc != GPT_OK:
            msg = self.lib.gpt_last_error(self.h).decode() if getattr(self, "h", None) else ""
            raise GPTError(rc, msg)

    def flatten(self, params: Dict[str, np.ndarray]) -> np.ndarray:
        flat = np.zeros(self.sizes.n_flat, dtype=np.float32)
        for name, off, shape, _ in self.tensors:
            a = np.asarray(params[name], dtype=np.float32)
            if a.shape != shape:
                raise ValueError(f"{name}: shape {a.shape} != {shape}")
            flat[off:off + a.size] = a.reshape(-1)
        return flat

    def unflatten(self, flat: np.ndarray) -> Dict[str, np.ndarray]:
        return {name: flat[off:off + int(np.prod(shape))].reshape(shape).copy()
                for name, off, shape, _ in self.tensors}

    def close(self):
        if getattr(self, "h", None):
            self.lib.gpt_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class GPT(Layout):
    """One model bound to device buffers on the current torch device and stream."""

    def __init__(self, cfg, precision: str = "bf16", batch: Optional[int] = None,
                 grad_accum: Optional[int] = None, device: str = "cuda", dropout: float = 0.0,
                 kv_cache: bool = False, debug_checks: bool = False):
        import torch
        super().__init__(cfg, precision, batch, grad_accum, dropout=dropout, kv_cache=kv_cache,
                         debug_checks=debug_checks)
        self.torch = torch
        self.device = torch.device(device)
        s = self.sizes

        def alloc(nbytes):
            return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=self.device)

        self.buf = {"params": alloc(s.param_bytes), "grads": alloc(s.grad_bytes), "m": alloc(s.m_bytes),
                    "v": alloc(s.v_bytes), "activations": alloc(s.activation_bytes),
                    "workspace": alloc(s.workspace_bytes)}
        self.buf["shadow"] = alloc(s.shadow_bytes) if s.shadow_bytes else None
        b = gpt_buffers(*[self.buf[k].data_ptr() if self.buf[k] is not None else None
                          for k in ("params", "grads", "m", "v", "shadow", "activations", "workspace")])
        self.stream = torch.cuda.current_stream(self.device)
        self._check(self.lib.gpt_bind(self.h, C.byref(b), C.c_void_p(self.stream.cuda_stream)))
        self.loss_buf = torch.zeros(1, dtype=torch.float32, device=self.device)
        self.norm_buf = torch.zeros(1, dtype=torch.float32, device=self.device)
        self._dec_tok = self._dec_out = None   # decode's token and logits buffers

    # ---- weights and state
    def load_params(self, params: Dict[str, np.ndarray], reset_state: bool = True):
        """Copies the weights in; reset_state=False keeps gradients, moments and the
        step counter (gpt_params_loaded), True starts training afresh (gpt_init_state)."""
        flat = self.torch.from_numpy(self.flatten(params))
        self.buf["params"].view(self.torch.float32)[: flat.numel()].copy_(flat)
        self._check(self.lib.gpt_init_state(self.h) if reset_state else self.lib.gpt_params_loaded(self.h))

    def _flat(self, key: str) -> np.ndarray:
        self.sync()
        return self.buf[key].view(self.torch.float32)[: self.sizes.n_flat].cpu().numpy()

    def params(self) -> Dict[str, np.ndarray]:
        return self.unflatten(self._flat("params"))

    def grads(self) -> Dict[str, np.ndarray]:
        return self.unflatten(self._flat("grads"))

    def moments(self) -> Tuple[Dict[str, np.ndarray], Dict[str, np.ndarray]]:
        return self.unflatten(self._flat("m")), self.unflatten(self._flat("v"))

    def step_count(self) -> int:
        t = C.c_int64()
        self._check(self.lib.gpt_get_step(self.h, C.byref(t)))
        return int(t.value)

    # ---- the step
    def _ids(self, a):
        t = self.torch
        if isinstance(a, np.ndarray):
            a = t.from_numpy(np.ascontiguousarray(a, dtype=np.int32))
        if a.device != self.device:
            a = a.to(self.device)
        return a.to(t.int32).contiguous()

    def forward_loss(self, tokens, targets, loss_out=None):
        tok, tgt = self._ids(tokens), self._ids(targets)
        B, T = tok.shape
        out = self.loss_buf if loss_out is None else loss_out
        self._keep = (tok, tgt)
        self._check(self.lib.gpt_forward_loss(self.h, C.c_void_p(tok.data_ptr()), C.c_void_p(tgt.data_ptr()),
                                              B, T, C.c_void_p(out.data_ptr())))
        return out

    def forward_logits(self, tokens):
        tok = self._ids(tokens)
        B, T = tok.shape
        out = self.torch.empty((B, T, self.cfg.padded_vocab), dtype=self.torch.float32, device=self.device)
        self._check(self.lib.gpt_forward_logits(self.h, C.c_void_p(tok.data_ptr()), B, T,
                                                C.c_void_p(out.data_ptr())))
        return out

    def backward(self):
        self._check(self.lib.gpt_backward(self.h))

    # ---- generation with the key/value cache
    def prefill(self, tokens):
        tok = self._ids(tokens)
        B, T = tok.shape
        out = self.torch.empty((B, self.cfg.padded_vocab), dtype=self.torch.float32, device=self.device)
        self._keep_dec = tok
        self._check(self.lib.gpt_prefill(self.h, C.c_void_p(tok.data_ptr()), B, T, C.c_void_p(out.data_ptr())))
        self._kv_B = B
        return out

    def decode_tokens(self, B: Optional[int] = None):
        """The token buffer decode() reads, one id per sequence of the last prefill (or
        B): sample(..., out=gpu.decode_tokens()) draws straight into it, with no copy."""
        B = getattr(self, "_kv_B", None) if B is None else B
        if B is None:
            raise RuntimeError("decode_tokens() needs a preceding prefill or B")
        if self._dec_tok is None or self._dec_tok.numel() != B:
            t = self.torch
            self._dec_tok = t.zeros(B, dtype=t.int32, device=self.device)
            self._dec_out = t.empty((B, self.cfg.padded_vocab), dtype=t.float32, device=self.device)
        return self._dec_tok

    def decode(self, tokens):
        """One decode step. The ids go through one token buffer and the fp32 logits come
        back in one logits buffer, both kept by this object, so that every call passes the
        library the same pointers and it replays its recorded step. The returned logits
        are overwritten by the next decode: clone them to keep them."""
        tok = self._ids(tokens).reshape(-1)
        if tok.numel() != getattr(self, "_kv_B", tok.numel()):
            raise ValueError(f"decode takes one token per sequence of the last prefill ({self._kv_B}), "
                             f"got {tok.numel()}")
        buf = self.decode_tokens(tok.numel())   # without a prefill the library reports the state error
        if tok.data_ptr() != buf.data_ptr():
            buf.copy_(tok)
        self._check(self.lib.gpt_decode(self.h, C.c_void_p(buf.data_ptr()), C.c_void_p(self._dec_out.data_ptr())))
        return self._dec_out

    def sample(self, logits, temperature: float, top_k: int = 0, uniforms=None, out=None):
        t = self.torch
        z = logits.to(self.device, t.float32).contiguous()
        B = z.shape[0]
        u = None
        if isinstance(uniforms, t.Tensor):
            u = uniforms.to(self.device, t.float32).contiguous()
        elif uniforms is not None:
            u = t.as_tensor(np.asarray(uniforms, dtype=np.float32)).to(self.device).contiguous()
        if out is None:
            out = t.empty(B, dtype=t.int32, device=self.device)
        elif out.dtype != t.int32 or out.numel() != B or not out.is_contiguous() or out.device != z.device:
            raise ValueError("out must be a contiguous int32 device tensor of one token per row")
        self._keep_dec = (z, u)
        self._check(self.lib.gpt_sample(self.h, C.c_void_p(z.data_ptr()), B, float(temperature), int(top_k),
                                        C.c_void_p(u.data_ptr()) if u is not None else None,
                                        C.c_void_p(out.data_ptr())))
        return out

    def set_dropout_seed(self, seed: int, counter: int = 0):
        self._check(self.lib.gpt_set_dropout_seed(self.h, int(seed) & 0xFFFFFFFFFFFFFFFF, int(counter) & 0xFFFFFFFF))

    def zero_grad(self):
        self._check(self.lib.gpt_zero_grad(self.h))

    def adamw_step(self, lr, beta1, beta2, eps, weight_decay, clip, norm_out=None, noalloc=False):
        """noalloc=True: gpt_adamw_step_noalloc (the norm's partials in the library's
        static device array instead of the workspace)."""
        out = self.norm_buf if norm_out is None else norm_out
        f = self.lib.gpt_adamw_step_noalloc if noalloc else self.lib.gpt_adamw_step
        self._check(f(self.h, lr, beta1, beta2, eps, weight_decay, clip, C.c_void_p(out.data_ptr())))
        return out

    def sync(self):
        self._check(self.lib.gpt_sync(self.h))

    def debug(self, what: str, layer: int, shape, dtype):
        t = self.torch
        out = t.empty(shape, dtype=dtype, device=self.device)
        self._check(self.lib.gpt_debug_copy(self.h, what.encode(), layer, C.c_void_p(out.data_ptr()),
                                            out.numel() * out.element_size()))
        return out

    # ---- timing hook
    def timer_enable(self, family: str):
        self._check(self.lib.gpt_timer_enable(self.h, family.encode()))

    def timer_disable(self):
        self._check(self.lib.gpt_timer_disable(self.h))

    def timer_read(self) -> Tuple[float, int]:
        ms, n = C.c_double(), C.c_int64()
        self._check(self.lib.gpt_timer_read(self.h, C.byref(ms), C.byref(n)))
        return float(ms.value), int(n.value)
