"""Torch-facing binding of libdd: same operations and names as include/dd.h.

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory, streams and the host-side tensors.  Shapes
and dtypes are checked here so that a mistake raises a Python error before
anything is enqueued; the library checks its own contract again.
"""
from __future__ import annotations

import ctypes
import math
import weakref

import torch

from . import _lib as L

_DTYPE = {torch.float32: L.DD_F32, torch.bfloat16: L.DD_BF16}


def _lib():
    return L.load()


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _dev(t, name):
    _need(t.is_cuda, f"{name} must be a GPU tensor")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def kv_dtype(t: torch.Tensor) -> int:
    _need(t.dtype in _DTYPE, f"K/V dtype must be float32 or bfloat16, got {t.dtype}")
    return _DTYPE[t.dtype]


# --------------------------------------------------------------------------- host memory
def host_empty(shape, dtype: torch.dtype) -> torch.Tensor:
    """A CPU tensor over pinned, device-mapped memory from dd_host_alloc.

    Its address is also valid in kernels; the memory is freed with
    dd_host_free once the last tensor viewing it is gone.
    """
    shape = tuple(int(s) for s in shape)
    nbytes = math.prod(shape) * torch.empty((), dtype=dtype).element_size()
    if nbytes == 0:
        return torch.empty(shape, dtype=dtype)
    lib = _lib()
    ptr = ctypes.c_void_p()
    L.check(lib.dd_host_alloc(nbytes, ctypes.byref(ptr)))
    addr = ptr.value
    buf = (ctypes.c_uint8 * nbytes).from_address(addr)
    weakref.finalize(buf, lib.dd_host_free, ctypes.c_void_p(addr))
    return torch.frombuffer(buf, dtype=torch.uint8).view(dtype).reshape(shape)


# --------------------------------------------------------------------------- stages
def score(q, keys, lens, kind: str = "logits", scale: float = 0.0, out=None, stream=None):
    """dd_score.  q fp32 [B][H][Q][D]; keys [B][H][n_max][D]; lens int32 [B]."""
    _dev(q, "q"), _dev(keys, "keys"), _dev(lens, "lens")
    _need(q.dtype == torch.float32 and q.dim() == 4, "q must be fp32 [B][H][Q][D]")
    B, H, Q, D = q.shape
    _need(keys.dim() == 4 and keys.shape[0] == B and keys.shape[1] == H and keys.shape[3] == D,
          "keys must be [B][H][n_max][D]")
    _need(lens.dtype == torch.int32 and lens.numel() == B, "lens must be int32 [B]")
    n_max = keys.shape[2]
    if out is None:
        out = torch.empty(B, H, Q, n_max, dtype=torch.float32, device=q.device)
    _dev(out, "out")
    _need(out.shape == (B, H, Q, n_max) and out.dtype == torch.float32, "out must be fp32 [B][H][Q][n_max]")
    k_code = {"logits": L.DD_LOGITS, "alpha": L.DD_ALPHA}[kind]
    L.check(_lib().dd_score(_p(q), _p(keys), _p(lens), B, H, Q, D, n_max, kv_dtype(keys),
                            float(scale), k_code, _p(out), _stream(stream)))
    return out


def topk(scores, lens, k: int, out=None, stream=None):
    """dd_topk.  scores fp32 [B][H][Q][n_max] -> int32 [B][H][Q][k], ascending, -1 padded."""
    _dev(scores, "scores"), _dev(lens, "lens")
    _need(scores.dtype == torch.float32 and scores.dim() == 4, "scores must be fp32 [B][H][Q][n_max]")
    B, H, Q, n_max = scores.shape
    _need(lens.dtype == torch.int32 and lens.numel() == B, "lens must be int32 [B]")
    if out is None:
        out = torch.empty(B, H, Q, k, dtype=torch.int32, device=scores.device)
    _dev(out, "out")
    _need(out.shape == (B, H, Q, k) and out.dtype == torch.int32, "out must be int32 [B][H][Q][k]")
    L.check(_lib().dd_topk(_p(scores), _p(lens), B, H, Q, n_max, int(k), _p(out), _stream(stream)))
    return out


def gather(k_host, v_host, idx, cnt=None, k_out=None, v_out=None, stream=None):
    """dd_gather.  k_host/v_host pinned [B][H][n_max][D] (host_empty); idx int32 [B][H][m]."""
    ref = k_host if k_host is not None else v_host
    _need(ref is not None, "need at least one host plane")
    _dev(idx, "idx")
    _need(idx.dtype == torch.int32 and idx.dim() == 3, "idx must be int32 [B][H][m]")
    B, H, m = idx.shape
    _need(ref.dim() == 4 and ref.shape[0] == B and ref.shape[1] == H, "host planes must be [B][H][n_max][D]")
    n_max, D = ref.shape[2], ref.shape[3]
    dt = kv_dtype(ref)
    for t, name in ((k_host, "k_host"), (v_host, "v_host")):
        if t is not None:
            _need(not t.is_cuda and t.is_contiguous() and t.shape == ref.shape and t.dtype == ref.dtype,
                  f"{name} must be a contiguous host tensor like the other plane")
    if cnt is not None:
        _dev(cnt, "cnt")
        _need(cnt.dtype == torch.int32 and cnt.numel() == B * H, "cnt must be int32 [B][H]")
    if k_host is not None and k_out is None:
        k_out = torch.empty(B, H, m, D, dtype=ref.dtype, device=idx.device)
    if v_host is not None and v_out is None:
        v_out = torch.empty(B, H, m, D, dtype=ref.dtype, device=idx.device)
    for t, name in ((k_out, "k_out"), (v_out, "v_out")):
        if t is not None:
            _dev(t, name)
            _need(t.shape == (B, H, m, D) and t.dtype == ref.dtype, f"{name} must be [B][H][m][D]")
    L.check(_lib().dd_gather(_p(k_host), _p(v_host), _p(idx), _p(cnt), B, H, m, D, n_max, dt,
                             _p(k_out), _p(v_out), _stream(stream)))
    return k_out, v_out


def gather_chunks(k_host, v_host, idx, chunk: int, cnt=None, k_out=None, v_out=None, stream=None):
    """dd_gather_chunks.  idx int32 [B][H][m] chunk indices; rows out [B][H][m*chunk][D]."""
    ref = k_host if k_host is not None else v_host
    _need(ref is not None, "need at least one host plane")
    _dev(idx, "idx")
    _need(idx.dtype == torch.int32 and idx.dim() == 3, "idx must be int32 [B][H][m]")
    B, H, m = idx.shape
    _need(ref.dim() == 4 and ref.shape[0] == B and ref.shape[1] == H, "host planes must be [B][H][n_max][D]")
    n_max, D = ref.shape[2], ref.shape[3]
    dt = kv_dtype(ref)
    for t, name in ((k_host, "k_host"), (v_host, "v_host")):
        if t is not None:
            _need(not t.is_cuda and t.is_contiguous() and t.shape == ref.shape and t.dtype == ref.dtype,
                  f"{name} must be a contiguous host tensor like the other plane")
    if cnt is not None:
        _dev(cnt, "cnt")
        _need(cnt.dtype == torch.int32 and cnt.numel() == B * H, "cnt must be int32 [B][H]")
    rows = m * int(chunk)
    if k_host is not None and k_out is None:
        k_out = torch.empty(B, H, rows, D, dtype=ref.dtype, device=idx.device)
    if v_host is not None and v_out is None:
        v_out = torch.empty(B, H, rows, D, dtype=ref.dtype, device=idx.device)
    for t, name in ((k_out, "k_out"), (v_out, "v_out")):
        if t is not None:
            _dev(t, name)
            _need(t.shape == (B, H, rows, D) and t.dtype == ref.dtype,
                  f"{name} must be [B][H][m*chunk][D]")
    L.check(_lib().dd_gather_chunks(_p(k_host), _p(v_host), _p(idx), _p(cnt), B, H, m, int(chunk),
                                    D, n_max, dt, _p(k_out), _p(v_out), _stream(stream)))
    return k_out, v_out


def landmarks(keys, lens, chunk: int, out=None, stream=None):
    """dd_landmarks.  keys device [B][H][n_max][D]; returns fp32 [B][H][ceil(n_max/chunk)][D]."""
    _dev(keys, "keys"), _dev(lens, "lens")
    _need(keys.dim() == 4 and keys.is_contiguous(), "keys must be contiguous [B][H][n_max][D]")
    B, H, n_max, D = keys.shape
    _need(lens.dtype == torch.int32 and lens.numel() == B, "lens must be int32 [B]")
    nc = (n_max + int(chunk) - 1) // int(chunk)
    if out is None:
        out = torch.empty(B, H, nc, D, dtype=torch.float32, device=keys.device)
    _dev(out, "out")
    _need(out.shape == (B, H, nc, D) and out.dtype == torch.float32 and out.is_contiguous(),
          "out must be fp32 [B][H][ceil(n_max/chunk)][D]")
    L.check(_lib().dd_landmarks(_p(keys), _p(lens), B, H, D, n_max, int(chunk), kv_dtype(keys),
                                _p(out), _stream(stream)))
    return out


def kv_append(k_dev, k_host, v_host, new_k, new_v, lens, lens_out=None, chunk: int = 0,
              landmarks=None, stream=None):
    """dd_kv_append: the new token's K/V rows ([B][H][D], device) at row lens[b]."""
    _dev(k_dev, "k_dev"), _dev(new_k, "new_k"), _dev(new_v, "new_v"), _dev(lens, "lens")
    B, H, n_max, D = k_dev.shape
    dt = kv_dtype(k_dev)
    for t, name in ((k_host, "k_host"), (v_host, "v_host")):
        _need(not t.is_cuda and t.is_contiguous() and t.shape == k_dev.shape
              and t.dtype == k_dev.dtype, f"{name} must be a contiguous host tensor like k_dev")
    for t, name in ((new_k, "new_k"), (new_v, "new_v")):
        _need(t.shape == (B, H, D) and t.dtype == k_dev.dtype and t.is_contiguous(),
              f"{name} must be [B][H][D] of the cache dtype")
    _need(lens.dtype == torch.int32 and lens.numel() == B, "lens must be int32 [B]")
    if lens_out is not None:
        _dev(lens_out, "lens_out")
        _need(lens_out.dtype == torch.int32 and lens_out.numel() == B, "lens_out must be int32 [B]")
    if landmarks is not None:
        _dev(landmarks, "landmarks")
        _need(landmarks.shape == (B, H, (n_max + chunk - 1) // chunk, D)
              and landmarks.dtype == torch.float32, "landmarks must be fp32 [B][H][ceil(n_max/chunk)][D]")
    L.check(_lib().dd_kv_append(_p(k_dev), _p(k_host), _p(v_host), _p(new_k), _p(new_v), _p(lens),
                                _p(lens_out), B, H, D, n_max, dt, int(chunk) if landmarks is not None else 0,
                                _p(landmarks), _stream(stream)))
    return lens_out


def attn_workspace_bytes(B: int, H: int, k: int, D: int) -> int:
    return int(_lib().dd_attn_workspace(B, H, k, D))


def sparse_attn(q, k_rows, v_rows, pos=None, cnt=None, k: int | None = None, scale: float = 0.0,
                out=None, lse=None, with_lse: bool = True, ws=None, stream=None):
    """dd_sparse_attn.  q fp32 [B][H][D] or [B][H][2][D] (plane 0 attends)."""
    _dev(q, "q"), _dev(k_rows, "k_rows"), _dev(v_rows, "v_rows")
    _need(q.dtype == torch.float32, "q must be fp32")
    B, H, m, D = k_rows.shape
    _need(v_rows.shape == k_rows.shape and v_rows.dtype == k_rows.dtype, "k_rows/v_rows mismatch")
    if q.dim() == 3:
        _need(q.shape == (B, H, D), "q must be [B][H][D]")
        q_stride = D
    else:
        _need(q.dim() == 4 and q.shape[0] == B and q.shape[1] == H and q.shape[3] == D,
              "q must be [B][H][Q][D]")
        q_stride = q.shape[2] * D
    if pos is not None:
        _dev(pos, "pos")
        _need(pos.dtype == torch.int32 and pos.dim() == 3 and pos.shape[:2] == (B, H), "pos must be int32 [B][H][k]")
        kk = pos.shape[2] if k is None else int(k)
        _need(pos.shape[2] == kk, "pos must have k entries per (b, h)")
    else:
        kk = m if k is None else int(k)
    if cnt is not None:
        _dev(cnt, "cnt")
        _need(cnt.dtype == torch.int32 and cnt.numel() == B * H, "cnt must be int32 [B][H]")
    if out is None:
        out = torch.empty(B, H, D, dtype=torch.float32, device=q.device)
    if lse is None and with_lse:
        lse = torch.empty(B, H, dtype=torch.float32, device=q.device)
    need = attn_workspace_bytes(B, H, kk, D)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    L.check(_lib().dd_sparse_attn(_p(q), q_stride, _p(k_rows), _p(v_rows), _p(pos), _p(cnt), B, H,
                                  kk, m, D, kv_dtype(k_rows), float(scale), _p(out), _p(lse),
                                  _p(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                  _stream(stream)))
    return out, lse


def sparse_attn_noalloc(q, k_rows, v_rows, out, lse=None, pos=None, cnt=None,
                        k: int | None = None, scale: float = 0.0, stream=None):
    """dd_sparse_attn_noalloc: dd_sparse_attn with the library's own scratch.

    The caller passes the outputs (out fp32 [B][H][D], lse fp32 [B][H] or
    None); neither this wrapper nor the library allocates anything."""
    _dev(q, "q"), _dev(k_rows, "k_rows"), _dev(v_rows, "v_rows"), _dev(out, "out")
    _need(q.dtype == torch.float32, "q must be fp32")
    B, H, m, D = k_rows.shape
    _need(v_rows.shape == k_rows.shape and v_rows.dtype == k_rows.dtype, "k_rows/v_rows mismatch")
    if q.dim() == 3:
        _need(q.shape == (B, H, D), "q must be [B][H][D]")
        q_stride = D
    else:
        _need(q.dim() == 4 and q.shape[0] == B and q.shape[1] == H and q.shape[3] == D,
              "q must be [B][H][Q][D]")
        q_stride = q.shape[2] * D
    if pos is not None:
        _dev(pos, "pos")
        _need(pos.dtype == torch.int32 and pos.dim() == 3 and pos.shape[:2] == (B, H), "pos must be int32 [B][H][k]")
        kk = pos.shape[2] if k is None else int(k)
        _need(pos.shape[2] == kk, "pos must have k entries per (b, h)")
    else:
        kk = m if k is None else int(k)
    if cnt is not None:
        _dev(cnt, "cnt")
        _need(cnt.dtype == torch.int32 and cnt.numel() == B * H, "cnt must be int32 [B][H]")
    _need(out.shape == (B, H, D) and out.dtype == torch.float32, "out must be fp32 [B][H][D]")
    if lse is not None:
        _dev(lse, "lse")
        _need(lse.shape == (B, H) and lse.dtype == torch.float32, "lse must be fp32 [B][H]")
    L.check(_lib().dd_sparse_attn_noalloc(_p(q), q_stride, _p(k_rows), _p(v_rows), _p(pos),
                                          _p(cnt), B, H, kk, m, D, kv_dtype(k_rows), float(scale),
                                          _p(out), _p(lse), _stream(stream)))
    return out, lse


def stream_copy(src, dst, stream=None):
    """dd_stream_copy: device-to-device streaming copy of src's bytes into dst."""
    _dev(src, "src"), _dev(dst, "dst")
    n = src.numel() * src.element_size()
    _need(dst.numel() * dst.element_size() >= n, "dst too small")
    L.check(_lib().dd_stream_copy(_p(src), _p(dst), n, _stream(stream)))
    return dst


def stream_read(src, sink, stream=None):
    """dd_stream_read: a streaming read of src's bytes (sink: >= 256 device bytes)."""
    _dev(src, "src"), _dev(sink, "sink")
    n = src.numel() * src.element_size()
    _need(sink.numel() * sink.element_size() >= 256, "sink needs 256 bytes")
    L.check(_lib().dd_stream_read(_p(src), n, _p(sink), _stream(stream)))


# --------------------------------------------------------------------------- layer step
def ring_bytes(ring_slots: int, B: int, H: int, D: int, k: int, dtype: int) -> int:
    return int(_lib().dd_ring_bytes(ring_slots, B, H, D, k, dtype))


def resident_bytes(L: int, B: int, H: int, D: int, n_max: int, k: int, dtype: int) -> int:
    """dd_resident_bytes: state of rows kept across steps for L layers."""
    return int(_lib().dd_resident_bytes(L, B, H, D, n_max, k, dtype))


def layer_step_workspace_bytes(B: int, H: int, D: int, n_max: int, k: int) -> int:
    return int(_lib().dd_layer_step_workspace(B, H, D, n_max, k))


def _ptr_array(ts):
    arr = (ctypes.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = None if t is None else t.data_ptr()
    return arr


class Context:
    """dd_ctx: the side stream, events and ring configuration of the layer step."""

    PREFETCH_MODES = {"auto": 0, "side": 1, "fused": 2}
    K_ROWS = {"device": 0, "host": 1}

    def __init__(self, ring_slots: int = 2, gather_cus: int = 0, prefetch_wgs: int = 0,
                 prefetch: str = "auto", k_rows: str = "device", perturb_side_us: int = 0,
                 perturb_main_us: int = 0, select_prefetch_slabs: int = 0):
        lib = _lib()
        cfg = L.CtxConfig(ring_slots=int(ring_slots), gather_cus=int(gather_cus),
                          prefetch_wgs=int(prefetch_wgs),
                          prefetch_mode=self.PREFETCH_MODES[prefetch],
                          k_rows=self.K_ROWS[k_rows], perturb_side_us=int(perturb_side_us),
                          perturb_main_us=int(perturb_main_us),
                          select_prefetch_slabs=int(select_prefetch_slabs))
        h = ctypes.c_void_p()
        L.check(lib.dd_ctx_create(ctypes.byref(cfg), ctypes.byref(h)))
        self._h = h
        self.ring_slots = int(ring_slots)
        self.k_rows = k_rows
        self._ring = None
        self._ws = None
        self._fin = weakref.finalize(self, lib.dd_ctx_destroy, h)

    def close(self):
        self._fin()

    def _buffer(self, attr, nbytes, device):
        buf = getattr(self, attr)
        if buf is None or buf.numel() < nbytes or buf.device != device:
            buf = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
            setattr(self, attr, buf)
        return buf

    def layer_step(self, q, k_dev, k_host, v_host, lens, k: int, pred=None, scale: float = 0.0,
                   cur=None, spec=None, out=None, lse=None, stats=None, ring=None, ws=None,
                   timing=None, stream=None, chunk: int = 0, landmarks=None,
                   dual: bool = False, out_spec=None, lse_spec=None, resident=None,
                   parity: int = 0, reset: bool = False):
        """dd_layer_step over the layers given as lists (one tensor per layer).

        q[l] fp32 [B][H][2][D]; k_dev[l] device [B][H][n_max][D]; k_host[l], v_host[l]
        pinned host tensors of the same shape (k_host may be None, or hold None entries,
        when K rows come from k_dev: k_rows="device"); pred: None or a list whose entries are
        None or int32 [B][H][k].  Returns dict(cur, spec, out, lse, stats).
        chunk > 1: landmarks[l] fp32 [B][H][ceil(n_max/chunk)][D] are scored and
        pred / cur / spec hold k // chunk chunk indices per (b, h).
        dual: the speculated query also attends over the same rows (out_spec,
        lse_spec in the result).
        resident: None, or a device uint8 tensor of resident_bytes(...) bytes: rows
        kept across steps (each layer's own two slots, used in turn by parity 0 / 1;
        reset clears it first, for the first step of a sequence).
        `timing` is None or a sequence of L * DD_STAGE_EVENTS raw hipEvent_t handles.
        """
        step = self.prepare_step(q, k_dev, k_host, v_host, lens, k, scale=scale, cur=cur,
                                 spec=spec, out=out, lse=lse, stats=stats, ring=ring, ws=ws,
                                 chunk=chunk, landmarks=landmarks, dual=dual, out_spec=out_spec,
                                 lse_spec=lse_spec, resident=resident, parity=parity,
                                 reset=reset)
        return step.run(pred=pred, timing=timing, stream=stream)

    def prepare_step(self, q, k_dev, k_host, v_host, lens, k: int, scale: float = 0.0,
                     cur=None, spec=None, out=None, lse=None, stats=None, ring=None, ws=None,
                     chunk: int = 0, landmarks=None, dual: bool = False, out_spec=None,
                     lse_spec=None, resident=None, parity: int = 0, reset: bool = False):
        """The arguments of layer_step, checked and marshalled once: the
        returned PreparedStep runs dd_layer_step on them as often as needed,
        taking only the prediction (checked like layer_step's), the timing
        events and the stream per call.  The tensors given here (and the
        outputs allocated here) are used by every run; their contents may
        change between runs, their storage may not."""
        Lyr = len(q)
        if k_host is None:
            _need(self.k_rows == "device", "k_host is needed when K rows come from the host")
            k_host = [None] * len(k_dev)
        _need(Lyr == len(k_dev) == len(k_host) == len(v_host), "per-layer lists differ in length")
        B, H, two, D = q[0].shape
        _need(two == 2, "q must hold two query planes")
        n_max = k_dev[0].shape[2]
        dt = kv_dtype(k_dev[0])
        dev = q[0].device
        chunk = int(chunk)
        ks = k // chunk if chunk > 1 else k
        _need(chunk <= 1 or landmarks is not None and len(landmarks) == Lyr,
              "chunk > 1 needs one landmark tensor per layer")
        for l in range(Lyr):
            _dev(q[l], "q"), _dev(k_dev[l], "k_dev")
            _need(q[l].shape == (B, H, 2, D) and q[l].dtype == torch.float32, "q shape")
            _need(k_dev[l].shape == (B, H, n_max, D) and kv_dtype(k_dev[l]) == dt, "k_dev shape")
            _need(k_host[l] is not None or self.k_rows == "device",
                  "k_host is needed when K rows come from the host")
            for t in (k_host[l], v_host[l]):
                if t is None:
                    continue
                _need(not t.is_cuda and t.is_contiguous() and t.shape == (B, H, n_max, D)
                      and t.dtype == k_dev[l].dtype, "host K/V must be contiguous [B][H][n_max][D]")
            if chunk > 1:
                _dev(landmarks[l], "landmarks")
                _need(landmarks[l].shape == (B, H, (n_max + chunk - 1) // chunk, D)
                      and landmarks[l].dtype == torch.float32 and landmarks[l].is_contiguous(),
                      "landmarks must be fp32 [B][H][ceil(n_max/chunk)][D]")
        _dev(lens, "lens")
        _need(lens.dtype == torch.int32 and lens.numel() == B, "lens must be int32 [B]")
        if cur is None:
            cur = [torch.empty(B, H, ks, dtype=torch.int32, device=dev) for _ in range(Lyr)]
        if spec is None:
            spec = [torch.empty(B, H, ks, dtype=torch.int32, device=dev) for _ in range(Lyr)]
        if out is None:
            out = [torch.empty(B, H, D, dtype=torch.float32, device=dev) for _ in range(Lyr)]
        if lse is None:
            lse = [torch.empty(B, H, dtype=torch.float32, device=dev) for _ in range(Lyr)]
        dual = dual or out_spec is not None
        if dual and out_spec is None:
            out_spec = [torch.empty(B, H, D, dtype=torch.float32, device=dev) for _ in range(Lyr)]
        if dual and lse_spec is None:
            lse_spec = [torch.empty(B, H, dtype=torch.float32, device=dev) for _ in range(Lyr)]
        if stats is None:
            stats = torch.zeros(Lyr, 3, dtype=torch.int64, device=dev)
        rb = ring_bytes(self.ring_slots, B, H, D, k, dt)
        wb = layer_step_workspace_bytes(B, H, D, n_max, k)
        if resident is not None:
            _dev(resident, "resident")
            _need(resident.numel() * resident.element_size() >= resident_bytes(Lyr, B, H, D, n_max, k, dt),
                  "resident state too small (resident_bytes)")
        if ring is None and resident is None:
            ring = self._buffer("_ring", rb, dev)
        if ws is None:
            ws = self._buffer("_ws", wb, dev)
        keep = [_ptr_array(q), _ptr_array(k_dev), _ptr_array(k_host), _ptr_array(v_host),
                (ctypes.c_void_p * Lyr)(),
                _ptr_array(cur), _ptr_array(spec), _ptr_array(out),
                _ptr_array(lse) if lse is not None else None,
                _ptr_array(landmarks) if chunk > 1 else None,
                _ptr_array(out_spec) if dual else None,
                _ptr_array(lse_spec) if dual else None]
        a = L.LayerStepArgs(
            L=Lyr, B=B, H=H, D=D, k=int(k), dtype=dt, n_max=n_max, scale=float(scale),
            lens=lens.data_ptr(),
            q=ctypes.cast(keep[0], ctypes.c_void_p), k_dev=ctypes.cast(keep[1], ctypes.c_void_p),
            k_host=ctypes.cast(keep[2], ctypes.c_void_p), v_host=ctypes.cast(keep[3], ctypes.c_void_p),
            pred=None,
            cur_idx=ctypes.cast(keep[5], ctypes.c_void_p), spec_idx=ctypes.cast(keep[6], ctypes.c_void_p),
            out=ctypes.cast(keep[7], ctypes.c_void_p),
            lse=None if keep[8] is None else ctypes.cast(keep[8], ctypes.c_void_p),
            stats=stats.data_ptr(),
            ring=None if ring is None else ring.data_ptr(),
            ring_bytes=0 if ring is None else ring.numel() * ring.element_size(),
            ws=ws.data_ptr(), ws_bytes=ws.numel() * ws.element_size(),
            stream=None, timing=None, chunk=chunk,
            landmarks=None if keep[9] is None else ctypes.cast(keep[9], ctypes.c_void_p),
            out_spec=None if keep[10] is None else ctypes.cast(keep[10], ctypes.c_void_p),
            lse_spec=None if keep[11] is None else ctypes.cast(keep[11], ctypes.c_void_p),
            resident=None if resident is None else resident.data_ptr(),
            resident_bytes=0 if resident is None else resident.numel() * resident.element_size(),
            parity=int(parity), reset=1 if reset else 0,
        )
        res = {"cur": cur, "spec": spec, "out": out, "lse": lse, "stats": stats}
        if dual:
            res["out_spec"], res["lse_spec"] = out_spec, lse_spec
        # Tensors whose storage the marshalled pointers name stay referenced.
        held = (q, k_dev, k_host, v_host, lens, landmarks, ring, ws, resident)
        return PreparedStep(self, a, keep, res, (B, H, ks, Lyr), held)


class PreparedStep:
    """One dd_layer_step call's arguments, marshalled by Context.prepare_step."""

    def __init__(self, ctx, args, keep, result, shape, held):
        self._ctx = ctx
        self._a = args
        self._keep = keep
        self._pred_arr = keep[4]
        self._pred_ptr = ctypes.cast(keep[4], ctypes.c_void_p)
        self.result = result
        self._shape = shape
        self._held = held

    def run(self, pred=None, timing=None, stream=None):
        """dd_layer_step on the prepared arguments.  pred: None or a list of
        one int32 [B][H][k // chunk] device tensor (or None) per layer.
        `timing`: None or a sequence of L * DD_STAGE_EVENTS raw hipEvent_t
        handles.  Returns the result dict (the prepared output tensors)."""
        a = self._a
        B, H, ks, Lyr = self._shape
        if pred is None:
            a.pred = None
        else:
            _need(len(pred) == Lyr, "pred needs one entry per layer")
            arr = self._pred_arr
            for l in range(Lyr):
                p = pred[l]
                if p is None:
                    arr[l] = None
                    continue
                _dev(p, "pred")
                _need(p.shape == (B, H, ks) and p.dtype == torch.int32,
                      "pred must be int32 [B][H][k // chunk]")
                arr[l] = p.data_ptr()
            a.pred = self._pred_ptr
        tarr = None
        if timing is not None:
            tarr = (ctypes.c_void_p * len(timing))(*timing)
        a.timing = None if tarr is None else ctypes.cast(tarr, ctypes.c_void_p)
        a.stream = _stream(stream).value
        L.check(_lib().dd_layer_step(self._ctx._h, ctypes.byref(a)))
        return self.result


class Decoder:
    """A steady-state decode loop over the layer step (several real steps).

    Each step appends the new token's K/V rows of every layer (dd_kv_append,
    also updating chunk landmarks), then runs dd_layer_step for all layers
    with the previous step's speculated sets as the prediction, so the
    prediction is carried across real steps.  The caller owns the caches:
    per layer, device keys k_dev[l] and pinned host k_host[l] / v_host[l] of
    [B][H][n_max][D], with room to grow; lens (int32 [B], device) is the
    current length, and the class keeps its own copy.  resident: each layer
    keeps its selected rows across steps (dd_layer_step_args.resident), so a
    step fetches over the host link only rows its previous step did not
    bring in; the state is cleared on the first step.

    The outputs of a step (cur, spec, out, lse, stats) live in one of two
    buffer sets used in turn, so a step's results stay valid through the
    next step and are overwritten by the one after; clone what must live
    longer.  Each step's arguments are marshalled once per buffer set,
    parity and set of query tensors (prepared steps), so a loop that reuses
    its query tensors pays the argument checks only on its first steps.
    """

    def __init__(self, ctx: Context, k_dev, k_host, v_host, lens, k: int, chunk: int = 0,
                 resident: bool = False):
        self.ctx = ctx
        self.k_dev, self.k_host, self.v_host = list(k_dev), list(k_host), list(v_host)
        self.k = int(k)
        self.chunk = int(chunk) if chunk and chunk > 1 else 0
        self.L = len(self.k_dev)
        self._lens = [lens.clone(), torch.empty_like(lens)]
        self._cur = 0
        self.landmarks = None
        if self.chunk:
            self.landmarks = [landmarks(kd, self._lens[0], self.chunk) for kd in self.k_dev]
        self.pred = None
        self.history = []  # per step: stats [L][3] (device)
        self._bufs = [None, None]  # output sets, used in turn
        self._buf = 0
        self._plans = {}
        self.state = None
        self._parity, self._reset = 0, True
        if resident:
            kd = self.k_dev[0]
            B, H, n_max, D = kd.shape
            nb = resident_bytes(self.L, B, H, D, n_max, self.k, kv_dtype(kd))
            self.state = torch.empty(nb, dtype=torch.uint8, device=kd.device)

    @property
    def lens(self):
        return self._lens[self._cur]

    def step(self, q, new_k, new_v, stream=None):
        """q[l] fp32 [B][H][2][D] (current, speculated); new_k[l] / new_v[l] [B][H][D]."""
        src, dst = self._lens[self._cur], self._lens[1 - self._cur]
        for l in range(self.L):
            kv_append(self.k_dev[l], self.k_host[l], self.v_host[l], new_k[l], new_v[l], src,
                      lens_out=dst if l == self.L - 1 else None, chunk=self.chunk,
                      landmarks=None if self.landmarks is None else self.landmarks[l],
                      stream=stream)
        self._cur = 1 - self._cur
        q = list(q)
        b = self._buf
        key = (b, self._cur, self._parity, self._reset, tuple(t.data_ptr() for t in q))
        plan = self._plans.get(key)
        if plan is None:
            if len(self._plans) >= 16:  # query tensors that change every step
                self._plans.clear()
            o = self._bufs[b] or {}
            plan = self.ctx.prepare_step(q, self.k_dev, self.k_host, self.v_host, self.lens,
                                         self.k, cur=o.get("cur"), spec=o.get("spec"),
                                         out=o.get("out"), lse=o.get("lse"),
                                         stats=o.get("stats"), chunk=self.chunk,
                                         landmarks=self.landmarks, resident=self.state,
                                         parity=self._parity, reset=self._reset)
            self._bufs[b] = plan.result
            self._plans[key] = plan
        res = plan.run(pred=self.pred, stream=stream)
        if self.state is not None:
            self._parity, self._reset = 1 - self._parity, False
        # The next step reads this step's speculated sets from this buffer
        # set while it writes the other one.
        self.pred = res["spec"]
        self._buf = 1 - b
        self.history.append(res["stats"].clone())
        return res
