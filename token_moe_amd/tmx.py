"""ctypes binding of libtmx.so -- argument marshalling only.

Same names as the C ABI (include/tmx.h). Tensors are passed as raw device
pointers (``tensor.data_ptr()``); torch is used by callers only to own device
memory and streams. Every compute step runs in the HIP library.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtmx.so")

TMX_OK, TMX_ERR_INVALID_ARG, TMX_ERR_UNSUPPORTED, TMX_ERR_OOM, TMX_ERR_DEVICE, TMX_ERR_STATE = range(6)
STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "OOM", 4: "DEVICE", 5: "STATE"}
TMX_F32, TMX_BF16, TMX_MXFP8 = 0, 1, 2
TMX_MIX, TMX_REVERT = 0, 1
TMX_BLOCK_TOKENMIXER_LARGE, TMX_BLOCK_RANKMIXER = 0, 1
TMX_PERM_ELEMENT, TMX_PERM_LANECOL, TMX_PERM_CURSOR = 0, 1, 2

EXPORTED = ("tmx_create", "tmx_destroy", "tmx_last_error", "tmx_load_weights",
            "tmx_block_stack_forward", "tmx_moe_route", "tmx_sublayer_forward", "tmx_debug_permute",
            "tmx_relu_route", "tmx_moe_buckets", "tmx_set_kernel_timing", "tmx_kernel_times",
            "tmx_sublayer_forward_noalloc", "tmx_set_model_io", "tmx_load_io_weights", "tmx_tokenize",
            "tmx_head", "tmx_model_forward")
KERNEL_KINDS = ("mlp_dense", "mlp_routed", "mlp_shared", "router", "bucket", "rmx_block", "f32", "tokenize",
                "head")


class TmxError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"tmx {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class tmx_config(ctypes.Structure):
    _fields_ = [
        ("B_max", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
        ("D", ctypes.c_int32), ("L", ctypes.c_int32),
        ("hidden_mix", ctypes.c_int32), ("hidden_rev", ctypes.c_int32),
        ("E", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("expert_hidden", ctypes.c_int32), ("shared_hidden", ctypes.c_int32),
        ("alpha", ctypes.c_float), ("eps", ctypes.c_float),
        ("inter_residual_gap", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("block", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libtmx.so (raises if it was never built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with `python -m token_moe_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.tmx_create.argtypes = [ctypes.POINTER(tmx_config), i32, ctypes.POINTER(vp)]
    lib.tmx_destroy.argtypes = [vp]
    lib.tmx_last_error.argtypes = [vp]
    lib.tmx_last_error.restype = ctypes.c_char_p
    lib.tmx_load_weights.argtypes = [vp, i32, i32, i32, vp, sz, vp]
    lib.tmx_block_stack_forward.argtypes = [vp, vp, vp, i32, vp]
    lib.tmx_moe_route.argtypes = [vp, i32, i32, vp, i32, vp, vp, vp]
    lib.tmx_sublayer_forward.argtypes = [vp, i32, i32, vp, vp, vp, vp, i32, vp]
    lib.tmx_sublayer_forward_noalloc.argtypes = [vp, i32, i32, vp, vp, vp, vp, i32, vp]
    lib.tmx_debug_permute.argtypes = [vp, vp, vp, i32, i32, i32, vp]
    lib.tmx_relu_route.argtypes = [vp, i32, vp, i32, vp, vp]
    lib.tmx_moe_buckets.argtypes = [vp, i32, i32, vp, i32, vp, vp, vp, vp]
    lib.tmx_set_kernel_timing.argtypes = [vp, i32]
    lib.tmx_set_model_io.argtypes = [vp, ctypes.POINTER(ctypes.c_int32), i32, i32, i32]
    lib.tmx_load_io_weights.argtypes = [vp, i32, vp, sz, vp]
    lib.tmx_tokenize.argtypes = [vp, vp, vp, i32, vp]
    lib.tmx_head.argtypes = [vp, vp, vp, i32, vp]
    lib.tmx_model_forward.argtypes = [vp, vp, vp, i32, vp]
    lib.tmx_kernel_times.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_longlong), i32]
    for name in EXPORTED:
        if name != "tmx_last_error":
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def make_config(B_max, T, H, D, L, hidden_mix=0, hidden_rev=0, E=0, top_k=0, expert_hidden=0,
                shared_hidden=0, alpha=0.0, eps=1e-6, inter_residual_gap=2, dtype=TMX_BF16,
                block=TMX_BLOCK_TOKENMIXER_LARGE) -> tmx_config:
    return tmx_config(B_max, T, H, D, L, hidden_mix, hidden_rev, E, top_k, expert_hidden,
                      shared_hidden, alpha, eps, inter_residual_gap, dtype, block)


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


class Context:
    """Owns one tmx_ctx. Methods mirror the C ABI one to one."""

    def __init__(self, cfg: tmx_config, device: int = 0):
        self.lib = load_library()
        self.cfg = cfg
        h = ctypes.c_void_p()
        st = self.lib.tmx_create(ctypes.byref(cfg), device, ctypes.byref(h))
        if st != TMX_OK:
            raise TmxError(st, self.lib.tmx_last_error(None).decode())
        self.h = h

    def _check(self, st: int):
        if st != TMX_OK:
            raise TmxError(st, self.lib.tmx_last_error(self.h).decode())

    def close(self):
        if getattr(self, "h", None):
            self.lib.tmx_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def load_weights(self, layer: int, sublayer: int, kind: int, src_ptr: int, nbytes: int, stream=None):
        self._check(self.lib.tmx_load_weights(self.h, layer, sublayer, kind, src_ptr, nbytes, _ptr(stream)))

    def block_stack_forward(self, x_in, x_out, B: int, stream=None):
        self._check(self.lib.tmx_block_stack_forward(self.h, _ptr(x_in), _ptr(x_out), B, _ptr(stream)))

    def moe_route(self, layer: int, sublayer: int, x, B: int, idx, gate, stream=None):
        self._check(self.lib.tmx_moe_route(self.h, layer, sublayer, _ptr(x), B, _ptr(idx), _ptr(gate),
                                           _ptr(stream)))

    def moe_buckets(self, layer: int, sublayer: int, x, B: int, xhat, counts, rows, stream=None):
        self._check(self.lib.tmx_moe_buckets(self.h, layer, sublayer, _ptr(x), B, _ptr(xhat), _ptr(counts),
                                             _ptr(rows), _ptr(stream)))

    def set_model_io(self, group_widths, tok_hidden: int, head_hidden: int):
        arr = (ctypes.c_int32 * len(group_widths))(*group_widths)
        self._check(self.lib.tmx_set_model_io(self.h, arr, len(group_widths), tok_hidden, head_hidden))

    def load_io_weights(self, kind: int, src_ptr: int, nbytes: int, stream=None):
        self._check(self.lib.tmx_load_io_weights(self.h, kind, src_ptr, nbytes, _ptr(stream)))

    def tokenize(self, emb, x_out, B: int, stream=None):
        self._check(self.lib.tmx_tokenize(self.h, _ptr(emb), _ptr(x_out), B, _ptr(stream)))

    def head(self, y, logits, B: int, stream=None):
        self._check(self.lib.tmx_head(self.h, _ptr(y), _ptr(logits), B, _ptr(stream)))

    def model_forward(self, emb, logits, B: int, stream=None):
        self._check(self.lib.tmx_model_forward(self.h, _ptr(emb), _ptr(logits), B, _ptr(stream)))

    def set_kernel_timing(self, enable: bool):
        self._check(self.lib.tmx_set_kernel_timing(self.h, 1 if enable else 0))

    def kernel_times(self):
        """{kernel name: (summed ms, launches)} since the previous call."""
        n = len(KERNEL_KINDS)
        ms = (ctypes.c_double * n)()
        cnt = (ctypes.c_longlong * n)()
        self._check(self.lib.tmx_kernel_times(self.h, ms, cnt, n))
        return {KERNEL_KINDS[i]: (ms[i], cnt[i]) for i in range(n) if cnt[i]}

    def relu_route(self, layer: int, s, B: int, gates, stream=None):
        self._check(self.lib.tmx_relu_route(self.h, layer, _ptr(s), B, _ptr(gates), _ptr(stream)))

    def sublayer_forward(self, layer: int, sublayer: int, x_in, resid, extra, x_out, B: int, stream=None):
        self._check(self.lib.tmx_sublayer_forward(self.h, layer, sublayer, _ptr(x_in), _ptr(resid),
                                                  _ptr(extra), _ptr(x_out), B, _ptr(stream)))

    def sublayer_forward_noalloc(self, layer: int, sublayer: int, x_in, resid, extra, x_out, B: int,
                                 stream=None):
        self._check(self.lib.tmx_sublayer_forward_noalloc(self.h, layer, sublayer, _ptr(x_in), _ptr(resid),
                                                          _ptr(extra), _ptr(x_out), B, _ptr(stream)))

    def debug_permute(self, x_in, x_out, B: int, inverse: int, form: int = 0, stream=None):
        self._check(self.lib.tmx_debug_permute(self.h, _ptr(x_in), _ptr(x_out), B, inverse, form,
                                               _ptr(stream)))
