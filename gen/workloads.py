"""Seeded synthetic long-context decode inputs.

The shapes follow the decode workloads that the DualDecoder pages discuss:
Llama-2-7B (32 heads x 128) and Llama-2-13B (40 heads x 128) attention
layouts at 32K-128K contexts and up to 64 concurrent requests (paper-daily
summary, "experimental results" and "worked example" sections), batched
decoding of several requests (arXiv page, section 2.1).  The premise that a
decode step attends mostly to a small set of important past tokens (arXiv
page, section 2.2) is modelled by planting high-score keys; imperfect token
speculation (arXiv page, section 1) is modelled by a speculated query that is
only correlated with the current one.

Nothing here is a step of the method: the module draws random numbers,
plants structure and lays tensors out.  Scores, selections and attention are
computed elsewhere (the oracle and the HIP library), from these tensors.

Layout of one layer:
  q      fp32 [B][H][2][D]      plane 0 = current query, plane 1 = speculated
  k, v   dtype [B][H][n_max][D] rows past lens[b] are filler, never selected
  lens   int32 [B]
  planted int64 [B][H][P] planted row positions, -1 padded; planted_cnt [B][H]
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    cid: int            # workload number, used as the seed base
    L: int              # layers
    B: int              # requests in the decode batch
    H: int              # heads (query heads = KV heads, MHA)
    D: int              # head dimension
    n_max: int          # cached keys per (request, head) slab
    len_lo: int         # per-request context length, uniform in [len_lo, len_hi]
    len_hi: int
    dtype: str          # storage type of K and V: "f32" or "bf16"
    k: int              # rows selected per (request, head, query)
    rho: float          # speculated query = rho * q + rho_c * z
    rho_c: float
    plant: str          # "exact16" | "frac" | "zipf"
    plant_frac: float = 0.01

    def scaled(self, **kw) -> "Workload":
        """Same recipe at other sizes (for tests that must finish fast)."""
        w = replace(self, **kw)
        if "n_max" in kw and "len_hi" not in kw:
            w = replace(w, len_hi=min(w.len_hi, w.n_max), len_lo=min(w.len_lo, w.n_max))
        return w

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPE[self.dtype]


WORKLOADS = {
    # 1 layer, batch 1, 8 heads x 64, 4096 keys, fp32; 16 keys per head set to 4 q.
    "tiny": Workload("tiny", 1, 1, 1, 8, 64, 4096, 4096, 4096, "f32", 64, 0.9, 0.44, "exact16"),
    # Llama-2-7B shape, one layer, 32K context, bf16, 1% planted keys, top-128.
    "llama7b_32k_layer": Workload("llama7b_32k_layer", 2, 1, 1, 32, 128, 32768, 32768, 32768,
                                  "bf16", 128, 0.9, 0.44, "frac"),
    # Llama-2-7B shape, 32-layer decode step, batch 16, top-1024.
    "llama7b_32k_step": Workload("llama7b_32k_step", 3, 32, 16, 32, 128, 32768, 32768, 32768,
                                 "bf16", 1024, 0.9, 0.44, "frac"),
    # Llama-2-13B shape, 40 layers, batch 4, 128K context, Zipf(1.1) planted keys, top-2048.
    "llama13b_128k": Workload("llama13b_128k", 4, 40, 4, 40, 128, 131072, 131072, 131072,
                              "bf16", 2048, 0.8, 0.6, "zipf"),
    # 64 concurrent requests, ragged lengths uniform in [16384, 65536], top-512.
    "hiconc_64": Workload("hiconc_64", 5, 1, 64, 32, 128, 65536, 16384, 65536,
                          "bf16", 512, 0.9, 0.44, "frac"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def layer_seed(w: Workload, layer: int) -> int:
    return 1000 * w.cid + layer


def request_lens(w: Workload) -> torch.Tensor:
    """Per-request context lengths (int32, CPU), fixed per workload."""
    if w.len_lo == w.len_hi:
        return torch.full((w.B,), w.len_hi, dtype=torch.int32)
    g = torch.Generator().manual_seed(1000 * w.cid + 999)
    return torch.randint(w.len_lo, w.len_hi + 1, (w.B,), generator=g, dtype=torch.int64).to(torch.int32)


def _plant_count(w: Workload, n: int) -> int:
    if w.plant == "exact16":
        return min(16, n)
    return min(n, int(round(w.plant_frac * n)))


def make_layer(w: Workload, layer: int, device="cpu", k_out=None, v_out=None):
    """Draw one layer of inputs on `device`.

    If `k_out` / `v_out` are given (tensors [B][H][n_max][D] of the storage
    dtype, on any device, e.g. pinned host memory) the keys and values are
    written there one request at a time and are not returned whole; this keeps
    the peak footprint at one request's slab for the large workloads.
    """
    device = torch.device(device)
    g = torch.Generator(device=device).manual_seed(layer_seed(w, layer))
    B, H, D, n_max = w.B, w.H, w.D, w.n_max
    lens = request_lens(w)

    q = torch.randn(B, H, D, generator=g, device=device, dtype=torch.float32)
    z = torch.randn(B, H, D, generator=g, device=device, dtype=torch.float32)
    q_both = torch.stack([q, w.rho * q + w.rho_c * z], dim=2).contiguous()

    pmax = max(_plant_count(w, int(n)) for n in lens.tolist())
    planted = torch.full((B, H, max(pmax, 1)), -1, dtype=torch.int64)
    planted_cnt = torch.zeros(B, H, dtype=torch.int32)

    k_full = v_full = None
    if k_out is None:
        k_full = torch.empty(B, H, n_max, D, dtype=w.torch_dtype, device=device)
    if v_out is None:
        v_full = torch.empty(B, H, n_max, D, dtype=w.torch_dtype, device=device)

    for b in range(B):
        n = int(lens[b])
        kb = torch.randn(H, n_max, D, generator=g, device=device, dtype=torch.float32)
        vb = torch.randn(H, n_max, D, generator=g, device=device, dtype=torch.float32)
        cnt = _plant_count(w, n)
        if cnt > 0:
            # Positions uniform without replacement in [0, n), independent per head.
            key = torch.rand(H, n_max, generator=g, device=device)
            key[:, n:] = 2.0
            pos = torch.argsort(key, dim=1)[:, :cnt]                      # [H, cnt]
            qb = q[b]                                                     # [H, D]
            if w.plant == "exact16":
                rows = (4.0 * qb)[:, None, :].expand(H, cnt, D)
            else:
                noise = torch.randn(H, cnt, D, generator=g, device=device, dtype=torch.float32)
                if w.plant == "frac":
                    coef = torch.full((H, cnt), 4.0, device=device)
                else:  # zipf: rank r gets coefficient 4 - 1.1 ln(r) sqrt(D) / |q|^2
                    r = torch.arange(1, cnt + 1, device=device, dtype=torch.float32)
                    qn2 = (qb * qb).sum(dim=1, keepdim=True)              # [H, 1]
                    coef = 4.0 - 1.1 * torch.log(r)[None, :] * math.sqrt(D) / qn2
                rows = coef[:, :, None] * qb[:, None, :] + noise
            kb.scatter_(1, pos[:, :, None].expand(H, cnt, D), rows)
            planted[b, :, :cnt] = pos.cpu()
            planted_cnt[b, :] = cnt
        kb = kb.to(w.torch_dtype)
        vb = vb.to(w.torch_dtype)
        if k_out is not None:
            k_out[b].copy_(kb)
        else:
            k_full[b].copy_(kb)
        if v_out is not None:
            v_out[b].copy_(vb)
        else:
            v_full[b].copy_(vb)
        del kb, vb

    return {
        "q": q_both,
        "k": k_full,
        "v": v_full,
        "lens": lens.to(device),
        "planted": planted,
        "planted_cnt": planted_cnt,
    }


def decode_step_inputs(w: Workload, layer: int, step: int, q_prev: torch.Tensor, device="cpu"):
    """Inputs of decode step `step` (1, 2, ...) of one layer after the drawn
    layer (make_layer is step 0).

    The token decoded now is the one the previous step speculated, up to the
    same imperfection the workload gives speculation: q_cur = rho * q_spec(prev)
    + rho_c * z, and the new speculated query is rho * q_cur + rho_c * z'
    (arXiv page, section 1: the speculated token guides the next step's
    retrieval).  The new token's key and value rows are N(0, 1) in the
    storage type.  q_prev: fp32 [B][H][2][D] of the previous step.
    Returns (q [B][H][2][D] fp32, new_k [B][H][D], new_v [B][H][D]).
    """
    device = torch.device(device)
    g = torch.Generator(device=device).manual_seed(layer_seed(w, layer) * 7919 + step)
    B, H, D = w.B, w.H, w.D
    z = torch.randn(B, H, D, generator=g, device=device, dtype=torch.float32)
    z2 = torch.randn(B, H, D, generator=g, device=device, dtype=torch.float32)
    q_cur = w.rho * q_prev[:, :, 1].to(device) + w.rho_c * z
    q_spec = w.rho * q_cur + w.rho_c * z2
    q = torch.stack([q_cur, q_spec], dim=2).contiguous()
    new_k = torch.randn(B, H, D, generator=g, device=device, dtype=torch.float32).to(w.torch_dtype)
    new_v = torch.randn(B, H, D, generator=g, device=device, dtype=torch.float32).to(w.torch_dtype)
    return q, new_k.contiguous(), new_v.contiguous()


def tie_scores(rows: int, n: int, seed: int, nvalues: int = 5, device="cpu") -> torch.Tensor:
    """fp32 score rows drawn from a small value set, so that exact ties occur.

    The set contains both -0.0 and +0.0, and a negative value.
    """
    g = torch.Generator(device=device).manual_seed(seed)
    base = torch.tensor([-0.0, 0.0, 1.5, -2.25, 3.0, 0.75, -0.5][: max(nvalues, 2)],
                        dtype=torch.float32, device=device)
    pick = torch.randint(0, base.numel(), (rows, n), generator=g, device=device)
    return base[pick].contiguous()


def random_sorted_indices(rows: int, k: int, upper: torch.Tensor, seed: int,
                          fill: float = 1.0) -> torch.Tensor:
    """int32 [rows][k]: per row, up to k distinct ascending indices in [0, upper[row]).

    A fraction `fill` of the k slots is used; the rest are -1 at the end.
    """
    g = torch.Generator().manual_seed(seed)
    out = torch.full((rows, k), -1, dtype=torch.int32)
    for r in range(rows):
        n = int(upper[r])
        m = min(n, int(round(fill * k)))
        if m <= 0:
            continue
        sel = torch.randperm(n, generator=g)[:m].sort().values
        out[r, :m] = sel.to(torch.int32)
    return out


def bf16_bits(t: torch.Tensor) -> torch.Tensor:
    """The raw 16-bit patterns of a bfloat16 tensor, as int16 (a view)."""
    assert t.dtype == torch.bfloat16
    return t.view(torch.int16)


def random_tensor(shape, seed: int, dtype=torch.float32, scale: float = 1.0,
                  device="cpu") -> torch.Tensor:
    """Seeded N(0, scale^2) tensor, rounded to `dtype` (RNE for bf16)."""
    g = torch.Generator(device=device).manual_seed(seed)
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        t = t * scale
    return t.to(dtype)


def random_positions(rows: int, k: int, m: int, seed: int, invalid_frac: float = 0.0) -> torch.Tensor:
    """int32 [rows][k]: distinct row numbers in [0, m) per row, in random order;
    a fraction of entries is replaced by -1 or by m + something (out of range)."""
    g = torch.Generator().manual_seed(seed)
    out = torch.empty(rows, k, dtype=torch.int32)
    for r in range(rows):
        out[r] = torch.randperm(m, generator=g)[:k].to(torch.int32)
    if invalid_frac > 0:
        bad = torch.rand(rows, k, generator=g) < invalid_frac
        alt = torch.where(torch.rand(rows, k, generator=g) < 0.5, torch.tensor(-1),
                          torch.tensor(m) + torch.randint(0, 50, (rows, k), generator=g))
        out = torch.where(bad, alt.to(torch.int32), out)
    return out
