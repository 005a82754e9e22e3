"""Predictive sparse-KV decode hot path on MI355X (gfx950).

The operations live in the HIP library libdd.so (C ABI in include/dd.h);
this package is its torch-facing binding.  torch is imported before the
library is loaded so that the process has a single HIP runtime.
"""
import torch  # noqa: F401  (must precede loading libdd.so)

from . import _lib
from .api import (  # noqa: F401
    Context,
    Decoder,
    PreparedStep,
    attn_workspace_bytes,
    gather,
    gather_chunks,
    host_empty,
    kv_append,
    kv_dtype,
    landmarks,
    layer_step_workspace_bytes,
    resident_bytes,
    ring_bytes,
    score,
    sparse_attn,
    sparse_attn_noalloc,
    stream_copy,
    stream_read,
    topk,
)
from ._lib import DD_MAX_K, DD_STAGE_EVENTS, DDError  # noqa: F401


def load():
    """Loads libdd.so now (raises if it is not built)."""
    return _lib.load()
