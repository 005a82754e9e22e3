"""Plain CPU oracle for the predictive sparse-KV decode path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it, and it shares no code,
table or helper with that path.

What it computes, and where the pages define it:

* Scoring.  For each request b, head h and query j (0 = current token,
  1 = speculated next token) the scaled logits s_i = q_j . K_i / sqrt(d_k)
  over the request's valid keys, and the attention distribution
  alpha = softmax(s) (paper-daily summary of "DualDecoder: Accelerate Long
  Context LLM Inference by Predictive Prefetch", core-formulas section; the
  worked-example section applies it to every cached key of a layer).
* Selection.  I = argtopk(alpha, k), the k keys of largest weight (same
  core-formulas section; "Select" and "Top-k" boxes of Figure 1 on the arXiv
  page).  Ties go to the lower index and sets are returned in ascending
  index order.
* Prediction bookkeeping.  The speculated token's set from the previous
  step is the prediction P; the true set's entries missing from P are
  fetched on the critical path (arXiv page, section 1: the layer-aware
  transfer schedule corrects prediction misses on the critical path).
* Gather.  Selected K/V rows are copied from the host-resident full KV
  cache into a small GPU buffer (arXiv page, section 2.2 and Figure 1,
  "Sparse KV" / "Gather").
* Sparse attention.  Decode attention of the current query over only the
  selected rows ("Attention" box of Figure 1), written here as dense
  attention with every unselected logit masked to -inf.
* KV append.  Each decode step appends the new token's key and value rows to
  the cache (arXiv page, section 2.1), so a multi-step loop grows every
  request by one row per step.
* Chunk landmarks.  Selection may instead score compressed landmarks of
  chunks of adjacent entries and retrieve whole chunks (arXiv page, section
  2.2, on ShadowKV); a landmark is read as the mean key of its chunk.
* Rows kept across steps.  The host-link rows of a step whose layer still
  holds what its previous step brought in (that step's prediction and
  misses): the prediction and misses not among them (arXiv page, section 1:
  the predicted entries are prefetched so the step need not wait for them;
  reading: a row already on the GPU is not fetched again).

Arithmetic is float64 on exact upcasts of the stored fp32 or bf16 values.
Where the pages leave a point open, the reading used is stated next to the
code.  Every function is pinned by tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math

import numpy as np

F32 = "f32"
BF16 = "bf16"
F64 = "f64"  # values already exact in float64 (landmarks)


def upcast(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Stored K/V/score elements -> float64, exactly.

    bf16 is held as 16-bit integers (its bit pattern): the fp32 value with the
    same upper half has those bits followed by sixteen zero bits.
    """
    if dtype == BF16:
        bits = np.ascontiguousarray(stored).view(np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == F32:
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if dtype == F64:
        return np.asarray(stored, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def default_scale(D: int) -> float:
    """1/sqrt(d_k) with d_k = the head dimension.

    Reading: the worked example divides by sqrt(64) for a 4096-wide model with
    32 heads, whose head dimension is 128; the head dimension of the data is
    taken as d_k.
    """
    return 1.0 / math.sqrt(D)


def scaled_logits(q: np.ndarray, keys: np.ndarray, lens: np.ndarray, dtype: str,
                  scale: float | None = None) -> np.ndarray:
    """s[b,h,j,i] = scale * q[b,h,j] . K[b,h,i] for i < lens[b]; -inf beyond.

    q: fp32 [B][H][Q][D]; keys: stored [B][H][n_max][D]; returns float64
    [B][H][Q][n_max].
    """
    B, H, Q, D = q.shape
    n_max = keys.shape[2]
    sc = default_scale(D) if scale is None or scale <= 0 else float(scale)
    q64 = np.asarray(q, dtype=np.float32).astype(np.float64)
    out = np.full((B, H, Q, n_max), -np.inf, dtype=np.float64)
    for b in range(B):
        n = int(lens[b])
        for h in range(H):
            kf = upcast(keys[b, h, :n], dtype)                 # [n][D]
            for j in range(Q):
                out[b, h, j, :n] = (kf @ q64[b, h, j]) * sc
    return out


def attention_weights(s: np.ndarray, lens: np.ndarray) -> np.ndarray:
    """alpha = softmax(s) over each row's valid keys [0, lens[b]); 0 beyond.

    Reading: the softmax domain is the request's own cached keys.
    """
    B, H, Q, n_max = s.shape
    a = np.zeros_like(s, dtype=np.float64)
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        row = s[b, :, :, :n]
        m = row.max(axis=-1, keepdims=True)
        e = np.exp(row - m)
        a[b, :, :, :n] = e / e.sum(axis=-1, keepdims=True)
    return a


def select_topk(s: np.ndarray, lens: np.ndarray, k: int) -> np.ndarray:
    """I = the k largest entries of each row, as int32 [B][H][Q][k].

    A full sort by (value descending, index ascending): equal values go to the
    lower index.  The chosen indices are returned in ascending order; when a
    row holds fewer than k valid keys, all of them are returned and the
    remaining slots hold -1.  -0.0 and +0.0 are one value.
    """
    B, H, Q, n_max = s.shape
    out = np.full((B, H, Q, k), -1, dtype=np.int32)
    for b in range(B):
        n = int(lens[b])
        m = min(k, n)
        if m == 0:
            continue
        idx = np.arange(n)
        for h in range(H):
            for j in range(Q):
                row = np.asarray(s[b, h, j, :n], dtype=np.float64)
                if not np.all(np.isfinite(row)):
                    raise ValueError("scores must be finite on valid keys")
                row = np.where(row == 0.0, 0.0, row)           # -0.0 -> +0.0
                order = np.lexsort((idx, -row))                 # primary: -row
                out[b, h, j, :m] = np.sort(order[:m]).astype(np.int32)
    return out


def gather_rows(host: np.ndarray, idx: np.ndarray, cnt: np.ndarray | None = None,
                out: np.ndarray | None = None) -> np.ndarray:
    """rows[b,h,j] = host[b,h,idx[b,h,j]] as raw stored elements.

    host: [B][H][n_max][D] stored elements; idx: int32 [B][H][m].
    For j < cnt[b,h] (all j when cnt is None): an index outside [0, n_max)
    (e.g. -1 padding) gives an all-zero row.  Rows j >= cnt[b,h] are left as
    they were in `out` (zeros when `out` is None).
    """
    B, H, n_max, D = host.shape
    m = idx.shape[2]
    if out is None:
        out = np.zeros((B, H, m, D), dtype=host.dtype)
    for b in range(B):
        for h in range(H):
            lim = m if cnt is None else max(0, min(m, int(cnt[b, h])))
            for j in range(lim):
                i = int(idx[b, h, j])
                if 0 <= i < n_max:
                    out[b, h, j] = host[b, h, i]
                else:
                    out[b, h, j] = 0
    return out


def attend_rows(q: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, dtype: str,
                pos: np.ndarray | None = None, cnt: np.ndarray | None = None,
                k: int | None = None, scale: float | None = None):
    """Decode attention of one query per (b, h) over gathered rows.

    q: fp32 [B][H][D]; k_rows, v_rows: stored [B][H][m][D];
    pos: int32 [B][H][k] row of the j-th selected entry (None: row j).
    Entries j < cnt[b,h] (all k when cnt is None) take part; an entry whose
    row is outside [0, m) is skipped.  Returns (out fp64 [B][H][D],
    lse fp64 [B][H]); with no entry, out = 0 and lse = -inf.
    """
    B, H, m, D = k_rows.shape
    kk = k if k is not None else (pos.shape[2] if pos is not None else m)
    sc = default_scale(D) if scale is None or scale <= 0 else float(scale)
    q64 = np.asarray(q, dtype=np.float32).astype(np.float64)
    out = np.zeros((B, H, D), dtype=np.float64)
    lse = np.full((B, H), -np.inf, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            lim = kk if cnt is None else max(0, min(kk, int(cnt[b, h])))
            rows = []
            for j in range(lim):
                r = j if pos is None else int(pos[b, h, j])
                if 0 <= r < m:
                    rows.append(r)
            if not rows:
                continue
            kf = upcast(k_rows[b, h, rows], dtype)
            vf = upcast(v_rows[b, h, rows], dtype)
            z = (kf @ q64[b, h]) * sc
            mx = z.max()
            e = np.exp(z - mx)
            tot = e.sum()
            out[b, h] = (e / tot) @ vf
            lse[b, h] = mx + math.log(tot)
    return out, lse


def masked_attention(q_cur: np.ndarray, keys: np.ndarray, values: np.ndarray,
                     lens: np.ndarray, sel: np.ndarray, dtype: str,
                     scale: float | None = None):
    """Dense attention over all valid keys with unselected logits set to -inf.

    q_cur: fp32 [B][H][D]; keys/values: stored [B][H][n_max][D];
    sel: int32 [B][H][k] (ascending, -1 padded).  Returns (out, lse) in fp64.
    Reading: only the selected rows are attended; no recent-window or sink
    rows are added, since the pages name none.
    """
    B, H, n_max, D = keys.shape
    sc = default_scale(D) if scale is None or scale <= 0 else float(scale)
    q64 = np.asarray(q_cur, dtype=np.float32).astype(np.float64)
    out = np.zeros((B, H, D), dtype=np.float64)
    lse = np.full((B, H), -np.inf, dtype=np.float64)
    for b in range(B):
        n = int(lens[b])
        for h in range(H):
            chosen = [int(i) for i in sel[b, h] if 0 <= int(i) < n]
            if n == 0 or not chosen:
                continue
            z = (upcast(keys[b, h, :n], dtype) @ q64[b, h]) * sc
            mask = np.full(n, True)
            mask[chosen] = False
            z[mask] = -np.inf
            mx = z.max()
            e = np.exp(z - mx)                                   # exp(-inf) = 0
            tot = e.sum()
            out[b, h] = (e / tot) @ upcast(values[b, h, :n], dtype)
            lse[b, h] = mx + math.log(tot)
    return out, lse


def bookkeeping(cur: np.ndarray, pred: np.ndarray | None, n_max: int):
    """Misses of the true set against the prediction, and the slot row map.

    cur: int32 [B][H][k], the true (current-token) set, ascending, -1 padded.
    pred: int32 [B][H][k], the prediction P (the previous step's speculated
    set, same layout), or None for a step without a prediction.

    The layer slot holds 2k rows per (b, h): row p < k is the prefetched host
    row of pred[p] (zero if pred[p] is outside [0, n_max)); row k + t is the
    t-th miss.  Returns a dict with
      miss     int32 [B][H][k]: cur entries not in pred, ascending, -1 padded
      miss_cnt int32 [B][H]
      pos      int32 [B][H][k]: slot row of cur[j] (-1 where cur[j] is -1)
      hits     int32 [B][H]
      prefetched int32 [B][H]: pred entries that are fetched from the host
    """
    B, H, k = cur.shape
    miss = np.full((B, H, k), -1, dtype=np.int32)
    pos = np.full((B, H, k), -1, dtype=np.int32)
    miss_cnt = np.zeros((B, H), dtype=np.int32)
    hits = np.zeros((B, H), dtype=np.int32)
    prefetched = np.zeros((B, H), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            where = {}
            if pred is not None:
                for p in range(k):
                    v = int(pred[b, h, p])
                    if 0 <= v < n_max:
                        prefetched[b, h] += 1
                        where.setdefault(v, p)
            t = 0
            for j in range(k):
                c = int(cur[b, h, j])
                if c < 0:
                    continue
                if c in where:
                    pos[b, h, j] = where[c]
                    hits[b, h] += 1
                else:
                    miss[b, h, t] = c
                    pos[b, h, j] = k + t
                    t += 1
            miss_cnt[b, h] = t
    return {"miss": miss, "miss_cnt": miss_cnt, "pos": pos, "hits": hits,
            "prefetched": prefetched}


def resident_fetches(prev_pred, prev_miss, pred, miss, n_max: int) -> np.ndarray:
    """Rows a step reads over the host link when its layer keeps the rows of
    its previous step, int64 [B][H].

    The previous step's slot holds the keys of its prediction prev_pred
    (entries in [0, n_max)) and of its misses prev_miss (entries >= 0);
    either may be None (nothing held: the first step).  This step fetches
    every entry of its prediction pred (in [0, n_max); None: no prediction)
    and of its misses miss (>= 0) whose key that slot does not hold; the
    others are copied on the GPU.  All arrays are [B][H][k], -1 padded.
    Reading: a key held by the previous step is not fetched again (arXiv
    page, section 1, prefetch of the predicted entries; the pages do not
    discuss keeping rows across steps).
    """
    B, H, _ = miss.shape
    out = np.zeros((B, H), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            held = set()
            if prev_pred is not None:
                held.update(int(x) for x in prev_pred[b, h] if 0 <= x < n_max)
            if prev_miss is not None:
                held.update(int(x) for x in prev_miss[b, h] if x >= 0)
            n = 0
            if pred is not None:
                n += sum(1 for x in pred[b, h] if 0 <= x < n_max and int(x) not in held)
            n += sum(1 for x in miss[b, h] if x >= 0 and int(x) not in held)
            out[b, h] = n
    return out


def landmarks(keys: np.ndarray, lens: np.ndarray, chunk: int, dtype: str) -> np.ndarray:
    """Chunk landmarks, float64 [B][H][ceil(n_max / chunk)][D].

    Chunk e of (b, h) is rows [e*chunk, (e+1)*chunk); its landmark is the mean
    of those of its keys below lens[b], and zero when it has none.  Reading:
    the arXiv page (section 2.2) names compressed chunk landmarks without
    defining them; the mean key of the chunk is the plainest reading.
    """
    B, H, n_max, D = keys.shape
    nc = -(-n_max // chunk)
    out = np.zeros((B, H, nc, D), dtype=np.float64)
    for b in range(B):
        n = int(min(max(int(lens[b]), 0), n_max))
        kf = upcast(keys[b, :, :n], dtype)                      # [H][n][D]
        for e in range(-(-n // chunk)):
            lo, hi = e * chunk, min((e + 1) * chunk, n)
            out[b, :, e] = kf[:, lo:hi].sum(axis=1) / (hi - lo)
    return out


def append_rows(cache: np.ndarray, lens: np.ndarray, new_rows: np.ndarray):
    """The cache after appending one row per (b, h), and the new lengths.

    cache: stored [B][H][n_max][D]; new_rows: stored [B][H][D].  Row lens[b]
    of request b becomes new_rows[b] and its length grows by one; a request
    whose length is outside [0, n_max) is left as it is.
    """
    out = np.array(cache, copy=True)
    new_lens = np.array(lens, dtype=np.int64, copy=True)
    n_max = cache.shape[2]
    for b in range(cache.shape[0]):
        n = int(lens[b])
        if 0 <= n < n_max:
            out[b, :, n] = new_rows[b]
            new_lens[b] = n + 1
    return out, new_lens


def chunk_rows(sel: np.ndarray, lens: np.ndarray, chunk: int) -> np.ndarray:
    """Rows of the selected chunks: int32 [B][H][ks*chunk], ascending, -1 padded.

    Chunk c brings rows c*chunk .. c*chunk + chunk - 1, those below lens[b].
    """
    B, H, ks = sel.shape
    out = np.full((B, H, ks * chunk), -1, dtype=np.int32)
    for b in range(B):
        n = int(lens[b])
        for h in range(H):
            rows = [c * chunk + i for c in sorted(int(x) for x in sel[b, h] if x >= 0)
                    for i in range(chunk) if c * chunk + i < n]
            out[b, h, :len(rows)] = rows
    return out


def layer_step(q: np.ndarray, keys_dev: np.ndarray, keys_host: np.ndarray,
               values_host: np.ndarray, lens: np.ndarray, k: int, dtype: str,
               pred: np.ndarray | None = None, scale: float | None = None,
               chunk: int = 0, dual: bool = False):
    """One layer of the predictive decode step, end to end.

    Score both queries against every cached key, select each query's top-k,
    compare the true set with the prediction, and attend the current query
    over its own set.  Reading: the true set is always the one attended,
    because misses are fetched on the critical path, so `out` does not depend
    on `pred`; the speculated set is returned as the next step's prediction.

    chunk >= 1: selection by chunk landmarks instead.  Both queries score the
    landmarks (same scale), k // chunk chunks are selected per query (ties to
    the lower chunk), the prediction and the bookkeeping are in chunks, and
    the current query attends over the rows of its chunks (those below
    lens[b]).  chunk = 1 is the per-key step computed through landmarks.

    dual: the speculated query also attends, over the same rows as the
    current one (out_spec, lse_spec).  Reading: the dual-token pipeline runs
    the normal and the retrieval-guiding token through the same decoding flow
    (arXiv page, section 1); the rows in the layer buffer are the current
    token's, so those are the rows both attend.
    """
    if chunk >= 1:
        D = keys_dev.shape[3]
        sc = default_scale(D) if scale is None or scale <= 0 else float(scale)
        lm = landmarks(keys_dev, lens, chunk, dtype)
        nlen = np.array([-(-int(x) // chunk) if x > 0 else 0 for x in lens], dtype=np.int64)
        s = scaled_logits(q, lm, nlen, F64, sc)
        sel = select_topk(s, nlen, k // chunk)
        cur = np.ascontiguousarray(sel[:, :, 0])
        spec = np.ascontiguousarray(sel[:, :, 1])
        bk = bookkeeping(cur, pred, lm.shape[2])
        rows = chunk_rows(cur, lens, chunk)
        out, lse = masked_attention(q[:, :, 0], keys_host, values_host, lens, rows, dtype, sc)
        misses = int(bk["miss_cnt"].sum())
        stats = np.array([misses, int(bk["hits"].sum()),
                          int(bk["prefetched"].sum()) + misses], dtype=np.int64)
        extra = {}
        if dual:
            extra["out_spec"], extra["lse_spec"] = masked_attention(
                q[:, :, 1], keys_host, values_host, lens, rows, dtype, sc)
        return {"scores": s, "cur": cur, "spec": spec, "out": out, "lse": lse,
                "stats": stats, "landmarks": lm, "rows": rows, **extra, **bk}
    s = scaled_logits(q, keys_dev, lens, dtype, scale)
    sel = select_topk(s, lens, k)
    cur = np.ascontiguousarray(sel[:, :, 0])
    spec = np.ascontiguousarray(sel[:, :, 1])
    bk = bookkeeping(cur, pred, keys_dev.shape[2])
    out, lse = masked_attention(q[:, :, 0], keys_host, values_host, lens, cur, dtype, scale)
    misses = int(bk["miss_cnt"].sum())
    stats = np.array([misses, int(bk["hits"].sum()),
                      int(bk["prefetched"].sum()) + misses], dtype=np.int64)
    extra = {}
    if dual:
        extra["out_spec"], extra["lse_spec"] = masked_attention(
            q[:, :, 1], keys_host, values_host, lens, cur, dtype, scale)
    return {"scores": s, "cur": cur, "spec": spec, "out": out, "lse": lse,
            "stats": stats, **extra, **bk}
