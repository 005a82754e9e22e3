"""ctypes loader for libdd.so, with the C signatures of include/dd.h.

Argument marshalling only.  There is no fallback: if the library is missing
or fails to load, importing the package's operations raises.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdd.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "dd.h")

DD_OK = 0
DD_ERR_INVALID_ARG = 1
DD_ERR_UNSUPPORTED = 2
DD_ERR_WORKSPACE = 3
DD_ERR_HIP = 4
DD_ERR_ALLOC = 5
DD_F32 = 0
DD_BF16 = 1
DD_LOGITS = 0
DD_ALPHA = 1
DD_MAX_K = 4096
DD_STAGE_EVENTS = 7

c_int, c_int64, c_size_t, c_float, c_void_p, c_char_p = (
    ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p, ctypes.c_char_p)
P = c_void_p  # every pointer crosses as an address


class CtxConfig(ctypes.Structure):
    _fields_ = [("ring_slots", c_int), ("gather_cus", c_int), ("prefetch_wgs", c_int),
                ("prefetch_mode", c_int), ("k_rows", c_int), ("perturb_side_us", c_int),
                ("perturb_main_us", c_int), ("select_prefetch_slabs", c_int)]


class LayerStepArgs(ctypes.Structure):
    _fields_ = [
        ("L", c_int), ("B", c_int), ("H", c_int), ("D", c_int), ("k", c_int), ("dtype", c_int),
        ("n_max", c_int64), ("scale", c_float),
        ("lens", P),
        ("q", P), ("k_dev", P), ("k_host", P), ("v_host", P), ("pred", P),
        ("cur_idx", P), ("spec_idx", P), ("out", P), ("lse", P),
        ("stats", P),
        ("ring", P), ("ring_bytes", c_size_t),
        ("ws", P), ("ws_bytes", c_size_t),
        ("stream", P),
        ("timing", P),
        ("chunk", c_int), ("landmarks", P),
        ("out_spec", P), ("lse_spec", P),
        ("resident", P), ("resident_bytes", c_size_t), ("parity", c_int), ("reset", c_int),
    ]


_SIGNATURES = {
    "dd_last_error": (c_char_p, []),
    "dd_version": (c_int, []),
    "dd_host_alloc": (c_int, [c_size_t, ctypes.POINTER(c_void_p)]),
    "dd_host_free": (c_int, [P]),
    "dd_score": (c_int, [P, P, P, c_int, c_int, c_int, c_int, c_int64, c_int, c_float, c_int, P, P]),
    "dd_topk": (c_int, [P, P, c_int, c_int, c_int, c_int64, c_int, P, P]),
    "dd_gather": (c_int, [P, P, P, P, c_int, c_int, c_int, c_int, c_int64, c_int, P, P, P]),
    "dd_attn_workspace": (c_size_t, [c_int, c_int, c_int, c_int]),
    "dd_sparse_attn": (c_int, [P, c_int64, P, P, P, P, c_int, c_int, c_int, c_int, c_int, c_int,
                               c_float, P, P, P, c_size_t, P]),
    "dd_sparse_attn_noalloc": (c_int, [P, c_int64, P, P, P, P, c_int, c_int, c_int, c_int, c_int,
                                       c_int, c_float, P, P, P]),
    "dd_ctx_create": (c_int, [ctypes.POINTER(CtxConfig), ctypes.POINTER(c_void_p)]),
    "dd_ctx_destroy": (c_int, [P]),
    "dd_ring_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int]),
    "dd_layer_step_workspace": (c_size_t, [c_int, c_int, c_int, c_int64, c_int]),
    "dd_resident_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int64, c_int, c_int]),
    "dd_layer_step": (c_int, [P, ctypes.POINTER(LayerStepArgs)]),
    "dd_stream_copy": (c_int, [P, P, c_size_t, P]),
    "dd_stream_read": (c_int, [P, c_size_t, P, P]),
    "dd_gather_chunks": (c_int, [P, P, P, P, c_int, c_int, c_int, c_int, c_int, c_int64, c_int,
                                 P, P, P]),
    "dd_landmarks": (c_int, [P, P, c_int, c_int, c_int, c_int64, c_int, c_int, P, P]),
    "dd_kv_append": (c_int, [P, P, P, P, P, P, P, c_int, c_int, c_int, c_int64, c_int, c_int, P, P]),
}

_lib = None


def header_symbols(path: str = HEADER) -> list[str]:
    """Names of the functions include/dd.h declares with DD_API."""
    text = open(path).read()
    return re.findall(r"DD_API\s+[\w\s\*]+?\b(dd_\w+)\s*\(", text)


def load():
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                           "or python -m sparse_kv_retrieval_dual_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class DDError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dd status {code}: {msg}")
        self.code = code


def check(rc: int):
    if rc != DD_OK:
        raise DDError(rc, load().dd_last_error().decode(errors="replace"))
