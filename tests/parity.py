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
import os
import threading

import numpy as np

TIE_REL_GAP = 1e-3
TIE_LOGIT_GAP = math.log1p(TIE_REL_GAP)
SCORE_RTOL = 1e-3
ATTN_RTOL = 1e-2

# Regression bounds, separate from the contract above: what fp32 accumulation
# actually reaches, with a margin.  A logit is a D-term fp32 dot product:
# its error is a few units of 2^-24 times sum_d |q_d K_d| (at most about
# 10 max|s| for the workloads' planted keys), about 1e-6 of max|s|.  An
# attention output moves by about the absolute error of the logits (each
# weight exp(s_i - m) changes by that factor) plus the fp32 sums over at most
# 128 entries per chunk and 32 chunk merges: a few 1e-6 of max|o|, 3e-6
# measured.  1e-5 (logits) and 1e-4 (attention) leave a 10x margin and still
# catch a path that loses precision, such as bf16 accumulation (about 4e-3).
SCORE_REGRESSION_RTOL = 1e-5
ATTN_REGRESSION_RTOL = 1e-4

# Worst achieved relative errors, per test (printed at the end of the run).
ACHIEVED: dict = {}
_ACHIEVED_LOCK = threading.Lock()


def _record(kind: str, value: float):
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    key = (test, kind)
    with _ACHIEVED_LOCK:
        ACHIEVED[key] = max(ACHIEVED.get(key, 0.0), float(value))


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
    """gpu fp32, ref fp64, both [rows][n_max].  Returns the worst relative error."""
    worst = 0.0
    for r in range(gpu.shape[0]):
        n = int(lens[r])
        g = gpu[r, :n].astype(np.float64)
        o = ref[r, :n]
        if n:
            scale = max(np.max(np.abs(o)), 1e-30)
            err = np.max(np.abs(g - o))
            assert err <= SCORE_RTOL * scale, f"row {r}: logit error {err} > {SCORE_RTOL} * {scale}"
            assert err <= SCORE_REGRESSION_RTOL * scale, (
                f"row {r}: logit error {err / scale:.3e} of max|s| is within the contract but "
                f"above the fp32 regression bound {SCORE_REGRESSION_RTOL}")
            worst = max(worst, err / scale)
        if pad_value is not None and n < gpu.shape[1]:
            tail = gpu[r, n:]
            if np.isneginf(pad_value):
                assert np.all(np.isneginf(tail)), f"row {r}: padding is not -inf"
            else:
                assert np.all(tail == pad_value), f"row {r}: padding is not {pad_value}"
    _record("logits", worst)
    return worst


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
                    rtol: float = ATTN_RTOL, regression: float | None = ATTN_REGRESSION_RTOL):
    """gpu fp32 [rows][D], ref fp64 [rows][D]; slack per row (or None).

    Every row must meet the contract (rtol, plus its exchange slack); rows
    whose sets match the oracle's (no slack) must also meet the fp32
    regression bound.  Returns the worst relative error of those rows.
    """
    worst = 0.0
    for r in range(gpu.shape[0]):
        o = ref[r]
        scale = max(np.abs(o).max(), 1e-30)
        err = np.abs(gpu[r].astype(np.float64) - o).max()
        sl = 0.0 if slack is None else float(slack[r])
        tol = rtol * scale + sl
        assert err <= tol, f"row {r}: attention error {err} > {tol}"
        if sl == 0.0:
            if regression is not None:
                assert err <= regression * scale, (
                    f"row {r}: attention error {err / scale:.3e} of max|o| is within the "
                    f"contract but above the fp32 regression bound {regression}")
            worst = max(worst, err / scale)
    _record("attention", worst)
    return worst
