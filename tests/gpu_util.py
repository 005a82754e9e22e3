"""Helpers for the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch


def require_gpu():
    """Skips without a GPU; where a GPU is present a missing library is a failure."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_kv_retrieval_dual_amd as dd
    dd.load()  # raises if libdd.so is missing
    return dd


def announce(msg: str):
    """Names the case on stdout before a GPU step (flushed at once)."""
    sys.stdout.write(f"[case] {msg}\n")
    sys.stdout.flush()


def stored(t: torch.Tensor) -> np.ndarray:
    """Oracle view of stored K/V elements: bf16 -> int16 bit patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    return t.numpy()


def to_host(dd, t: torch.Tensor) -> torch.Tensor:
    """A pinned, device-mapped copy of t (dd_host_alloc)."""
    h = dd.host_empty(t.shape, t.dtype)
    h.copy_(t.cpu() if t.is_cuda else t)
    return h
