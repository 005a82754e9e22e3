"""HIP events as raw handles, for timing work that the library enqueues.

Measurement plumbing: dd_layer_step records caller-supplied hipEvent_t
handles between its stages (on the stream each stage runs on), and these
helpers create those handles and read the elapsed times.  The HIP runtime
is the one already loaded in the process (torch's).
"""
from __future__ import annotations

import ctypes

import torch  # noqa: F401  (loads the process's HIP runtime first)

_hip = None


def _rt():
    global _hip
    if _hip is None:
        h = ctypes.CDLL("libamdhip64.so.7")
        h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        h.hipEventCreate.restype = ctypes.c_int
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipEventDestroy.restype = ctypes.c_int
        h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventRecord.restype = ctypes.c_int
        h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        h.hipEventSynchronize.restype = ctypes.c_int
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventElapsedTime.restype = ctypes.c_int
        h.hipGetLastError.argtypes = []
        h.hipGetLastError.restype = ctypes.c_int
        _hip = h
    return _hip


def _ok(rc, what):
    if rc != 0:
        _rt().hipGetLastError()  # do not leave the error for the next runtime call
        raise RuntimeError(f"{what} failed with HIP error {rc}")


class EventSet:
    """n timing events; handles[i] is the raw hipEvent_t of event i."""

    def __init__(self, n: int):
        rt = _rt()
        self.handles = []
        for _ in range(n):
            e = ctypes.c_void_p()
            _ok(rt.hipEventCreate(ctypes.byref(e)), "hipEventCreate")
            self.handles.append(e.value)

    def record(self, i: int, stream=None):
        s = torch.cuda.current_stream() if stream is None else stream
        _ok(_rt().hipEventRecord(ctypes.c_void_p(self.handles[i]), ctypes.c_void_p(s.cuda_stream)),
            "hipEventRecord")

    def synchronize(self, i: int):
        _ok(_rt().hipEventSynchronize(ctypes.c_void_p(self.handles[i])), "hipEventSynchronize")

    def elapsed_ms(self, a: int, b: int) -> float:
        t = ctypes.c_float()
        _ok(_rt().hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(self.handles[a]),
                                      ctypes.c_void_p(self.handles[b])), "hipEventElapsedTime")
        return float(t.value)

    def close(self):
        for h in self.handles:
            _rt().hipEventDestroy(ctypes.c_void_p(h))
        self.handles = []
