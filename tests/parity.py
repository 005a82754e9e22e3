"""Comparison rules shared by the parity tests (not collected by pytest).

Tolerances:
* index sets: identical, except that entries whose oracle logit lies within
  ln(1 + 1e-3) of the oracle's k-th largest logit may be exchanged (a relative
  gap of 1e-3 in attention weight);
* logits: per row, max |gpu - oracle| <= 1e-3 * max |oracle|;
* attention outputs: per (b, h), max_d |gpu - oracle| <= 1e-2 * max_d |oracle|,
  widened where the index sets legitimately differ by the largest change such
  an exchange can cause (computed from the oracle's own data).
"""
from __future__ import annotations

import math

import numpy as np

TIE_REL_GAP = 1e-3
TIE_LOGIT_GAP = math.log1p(TIE_REL_GAP)
SCORE_RTOL = 1e-3
ATTN_RTOL = 1e-2


def check_index_sets(gpu: np.ndarray, ref: np.ndarray, logits: np.ndarray,
                     lens: np.ndarray, k: int, exact: bool = False):
    """gpu, ref: int32 [rows][k]; logits: float64 [rows][n_max]; lens: [rows].

    Returns the list of rows whose sets differ (all within the tie band).
    """
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    rows = gpu.shape[0]
    differing = []
    for r in range(rows):
        n = int(lens[r])
        m = min(k, n)
        g = gpu[r]
        o = ref[r]
        assert np.all(g[m:] == -1), f"row {r}: padding past {m} is not -1: {g[m:m + 8]}"
        gv = g[:m]
        assert np.all((gv >= 0) & (gv < n)), f"row {r}: index out of [0,{n})"
        assert np.all(np.diff(gv) > 0), f"row {r}: not strictly ascending"
        if np.array_equal(gv, o[:m]):
            continue
        assert not exact, f"row {r}: index sets differ (exact comparison)\n gpu {gv[:16]}\n ref {o[:16]}"
        row = logits[r, :n]
        ordered = np.sort(row)[::-1]
        s_b = ordered[m - 1]
        diff = np.setxor1d(gv, o[:m])
        bad = diff[np.abs(row[diff] - s_b) > TIE_LOGIT_GAP]
        assert bad.size == 0, (
            f"row {r}: {bad.size} exchanged entries outside the tie band; "
            f"k-th logit {s_b}, offending logits {row[bad[:8]]}")
        differing.append(r)
    return differing


def check_logits(gpu: np.ndarray, ref: np.ndarray, lens: np.ndarray, pad_value=-np.inf):
    """gpu fp32, ref fp64, both [rows][n_max]."""
    for r in range(gpu.shape[0]):
        n = int(lens[r])
        g = gpu[r, :n].astype(np.float64)
        o = ref[r, :n]
        if n:
            scale = max(np.max(np.abs(o)), 1e-30)
            err = np.max(np.abs(g - o))
            assert err <= SCORE_RTOL * scale, f"row {r}: logit error {err} > {SCORE_RTOL} * {scale}"
        if pad_value is not None and n < gpu.shape[1]:
            tail = gpu[r, n:]
            if np.isneginf(pad_value):
                assert np.all(np.isneginf(tail)), f"row {r}: padding is not -inf"
            else:
                assert np.all(tail == pad_value), f"row {r}: padding is not {pad_value}"


def exchange_slack(logits_row: np.ndarray, ref_sel: np.ndarray, v_rows: np.ndarray,
                   k: int, o_ref: np.ndarray) -> float:
    """Largest change of the attention output caused by exchanging tie-band entries.

    logits_row: float64 [n] (current query); ref_sel: the oracle's set;
    v_rows: float64 [n][D] (all values of the row); o_ref: oracle output [D].
    """
    n = logits_row.shape[0]
    m = min(k, n)
    sel = ref_sel[:m]
    s_b = np.sort(logits_row)[::-1][m - 1]
    band = np.nonzero(np.abs(logits_row - s_b) <= TIE_LOGIT_GAP)[0]
    inside = np.intersect1d(band, sel)
    outside = np.setdiff1d(band, sel)
    swaps = min(inside.size, outside.size)
    if swaps == 0:
        return 0.0
    top = logits_row[sel].max()
    w = np.exp(logits_row - top)
    z = w[sel].sum()
    w_hi = w[band].max()
    w_lo = w[band].min()
    vmax = np.abs(v_rows[band]).max()
    dn = swaps * 2.0 * w_hi * vmax
    dz = swaps * (w_hi - w_lo)
    return float((dn + np.abs(o_ref).max() * dz) / max(z - swaps * w_hi, 1e-300))


def check_attention(gpu: np.ndarray, ref: np.ndarray, slack: np.ndarray | None = None,
                    rtol: float = ATTN_RTOL):
    """gpu fp32 [rows][D], ref fp64 [rows][D]; slack per row (or None)."""
    worst = 0.0
    for r in range(gpu.shape[0]):
        o = ref[r]
        scale = max(np.abs(o).max(), 1e-30)
        err = np.abs(gpu[r].astype(np.float64) - o).max()
        tol = rtol * scale + (0.0 if slack is None else float(slack[r]))
        assert err <= tol, f"row {r}: attention error {err} > {tol}"
        worst = max(worst, err / scale)
    return worst
