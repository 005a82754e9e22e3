"""Benchmark of the predictive sparse-KV decode hot path on one MI355X.

One step = one dd_layer_step over one batch of the Llama-2-7B-shape
single-layer workload (batch 1, 32 heads x 128, 32768 cached keys, bf16 K/V,
top-128, current + speculated query): scoring of every key for both queries,
both top-k selections with the prediction bookkeeping, the prefetch of the
predicted V rows (inside the scoring kernel by default), the miss fetch and
the sparse attention.  The prediction is the speculated set of an untimed
first step, as in decode.  --workload times one layer of another workload.

Inputs are resident before the clock starts: keys in HBM, the full K/V in
pinned host memory.  The key copy rotates over several identical HBM copies
so that repeated steps cannot be served from the 256 MB Infinity Cache.

Prints one JSON line (see the fields at the end of main()).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "keys scored/s (% HBM peak) + gather GB/s + layer decode step µs, 7B-shape 32K"
HBM_PEAK_GBPS = 8000.0
# The host link the pages' cost model takes (a PCIe 5.0 x16 figure, arXiv
# page, section 2.2); the measured pinned copy is the other reference.
LINK_PAGES_GBPS = 64.0
PROFILES = os.path.join(ROOT, "profiles")


# The scoring kernel's source: its file and the headers it includes.
SCORE_SOURCES = ("score.hip", "dd_device.h", "gather_body.h", "gather_res.h")


def _progress(msg: str) -> None:
    """A line on stderr as each phase of the run ends (stdout holds only the
    JSON result)."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def _cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo (or "unknown")."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _source_hash(files) -> str:
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(ROOT, "sparse_kv_retrieval_dual_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _counter_traffic(kernel: str, sources, workload: str):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel source (else None)."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    if fields.get("source_sha256_16") != _source_hash(sources):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def decode_loop(dd, gen, w, lay, kh, vh, k_dev, lens, steps: int, chunk: int, dev,
                layers: int = 1, resident: bool = False, h2d_gbps: float = 0.0,
                prefetch_wgs: int = 0, prefetch: str = "auto"):
    """Real decode steps on the same cache: each appends the new token's K/V
    rows (dd_kv_append) and runs the layer step with the previous step's
    speculated set as the prediction.  The loop starts `steps` rows short of
    the workload's context (rows past the length are filler) and grows back
    to it.  Each step is timed alone (eager, events around it on the
    caller's stream), after a 1 GiB streaming copy that clears the keys from
    the 256 MB Infinity Cache.

    layers > 1: every step runs that many layers of the workload's shape.
    The layers share the cache tensors (their appends land on the same rows,
    which changes no amount of work) but each has its own query sequence,
    prediction and outputs.  resident: each layer keeps its selected rows
    across steps, so only rows its previous step did not bring in cross the
    host link.  prefetch / prefetch_wgs: the context's prefetch mode and
    workgroup count (0: the library's default)."""
    import numpy as np
    import torch
    from sparse_kv_retrieval_dual_amd.hipevents import EventSet

    N = layers
    start = torch.clamp(lens - steps, min=0).to(torch.int32)
    ctx = dd.Context(ring_slots=2, prefetch_wgs=prefetch_wgs, prefetch=prefetch)
    dec = dd.Decoder(ctx, [k_dev] * N, [kh] * N, [vh] * N, start, w.k, chunk=chunk,
                     resident=resident)
    q0 = lay["q"].cpu()
    res = ctx.layer_step([q0.to(dev)] * N, [k_dev] * N, [kh] * N, [vh] * N, dec.lens, w.k,
                         chunk=chunk, landmarks=dec.landmarks)
    dec.pred = [s.clone() for s in res["spec"]]
    inputs = []
    qs = [q0] * N
    for t in range(1, steps + 1):
        new = [gen.decode_step_inputs(w, l, t, qs[l]) for l in range(N)]
        qs = [x[0] for x in new]
        inputs.append(tuple([x[i].to(dev) for x in new] for i in range(3)))
    big = torch.empty(1 << 29, dtype=torch.uint8, device=dev)
    big2 = torch.empty_like(big)
    ev = EventSet(2)
    times = []
    # A decode loop writes each step's queries into the same buffers (so the
    # decoder's prepared steps are reused); the copy is outside the timing.
    qbuf = [torch.empty_like(x) for x in inputs[0][0]]
    for qd, nk, nv in inputs:
        dd.stream_copy(big, big2)
        for l in range(N):
            qbuf[l].copy_(qd[l])
        ev.record(0)
        dec.step(qbuf, nk, nv)
        ev.record(1)
        torch.cuda.synchronize()
        times.append(ev.elapsed_ms(0, 1) * 1e3)
    del big, big2
    c = max(chunk, 1)
    recall, link_rows = [], []
    for st in dec.history:
        a = st.cpu().numpy()
        m, h = int(a[:, 0].sum()), int(a[:, 1].sum())
        recall.append(h / max(m + h, 1))
        link_rows.append(int(a[:, 2].sum()))
    ctx.close()
    out = {"steps": steps, "layers": N, "resident": bool(resident), "chunk": c,
           "us_per_step_mean": float(np.mean(times)),
           "us_per_step_median": float(np.median(times)),
           "us_per_layer_median": float(np.median(times)) / N,
           "timing": "eager, one step at a time", "recall_per_step": recall,
           "host_rows_per_step": link_rows}
    if h2d_gbps > 0:
        # V rows only cross the link (K rows come from the scoring copy).
        row_b = w.D * w.elem_bytes * c
        tail = link_rows[len(link_rows) // 2:]
        out["host_bytes_per_step_late_half"] = float(np.mean(tail)) * row_b
        out["link_floor_us_late_half"] = float(np.mean(tail)) * row_b / (h2d_gbps * 1e9) * 1e6
        out["us_per_step_median_late_half"] = float(np.median(times[len(times) // 2:]))
    return out


def multi_layer(dd, w, lay, kh, vh, k_dev, lens, layers: int, h2d_gbps: float, dev,
                steps: int, prefetch: str, k_rows: str, chunk: int = 1, lm=None):
    """One decode step over `layers` layers of the workload's shape (the same
    queries and host cache serve every layer, the keys and landmarks rotate
    over the copies given; each layer keeps its own prediction and
    outputs): the multi-layer schedule, where layer l+1's prefetch overlaps
    layer l (on the side stream by default).  Eager steps, each bracketed by
    events on the caller's stream; the link floor is the host-link bytes the
    step moved (prefetched and missed rows) at the measured pinned-copy rate.
    chunk > 1: selection by the chunk landmarks lm (the stats count chunks)."""
    import numpy as np
    import torch
    from sparse_kv_retrieval_dual_amd.hipevents import EventSet

    N = layers
    ctx = dd.Context(ring_slots=2, prefetch=prefetch, k_rows=k_rows)
    q = lay["q"]
    # k_dev / lm: one tensor, or copies that the layers take in turn (so
    # that a later layer's scan is not served by the Infinity Cache).
    kd = k_dev if isinstance(k_dev, (list, tuple)) else [k_dev]
    lms = lm if isinstance(lm, (list, tuple)) else [lm]
    lists = ([q] * N, [kd[i % len(kd)] for i in range(N)], None if kh is None else [kh] * N,
             [vh] * N)
    ck = dict(chunk=chunk, landmarks=[lms[i % len(lms)] for i in range(N)]) if chunk > 1 else {}
    res = ctx.layer_step(*lists, lens, w.k, **ck)
    pred = [s.clone() for s in res["spec"]]
    stats = torch.zeros(N, 3, dtype=torch.int64, device=dev)
    plan = ctx.prepare_step(*lists, lens, w.k, cur=res["cur"], spec=res["spec"],
                            out=res["out"], lse=res["lse"], stats=stats, **ck)
    ev = EventSet(2)
    times = []
    for i in range(steps + 2):
        ev.record(0)
        plan.run(pred=pred)
        ev.record(1)
        torch.cuda.synchronize()
        if i >= 2:
            times.append(ev.elapsed_ms(0, 1) * 1e3)
    # The same step replayed from a HIP graph (checked against the eager
    # outputs on two replays first), as a decode loop would run it.
    t_graph, graph_note = None, None
    try:
        ref = [o.clone() for o in res["out"]]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            plan.run(pred=pred)
        for _ in range(2):
            for o in res["out"]:
                o.zero_()
            g.replay()
            torch.cuda.synchronize()
            if not all(torch.equal(a, b) for a, b in zip(res["out"], ref)):
                raise RuntimeError("graph replay differs from the eager step")
        gt = []
        for i in range(steps + 2):
            ev.record(0)
            g.replay()
            ev.record(1)
            torch.cuda.synchronize()
            if i >= 2:
                gt.append(ev.elapsed_ms(0, 1) * 1e3)
        t_graph = float(np.median(gt))
        del g
    except Exception as e:  # noqa: BLE001
        graph_note = f"graph replay unavailable: {e}"
    st = stats.cpu().numpy()
    ctx.close()
    t = float(np.median(times))
    planes = 1 if k_rows == "device" else 2
    link_bytes = int(st[:, 2].sum()) * max(chunk, 1) * w.D * w.elem_bytes * planes
    floor_us = link_bytes / (h2d_gbps * 1e9) * 1e6
    return {"layers": N, "prefetch": prefetch, "chunk": max(chunk, 1), "step_us_median": t,
            "per_layer_us": t / N,
            "timing": "eager, events around each whole step",
            "graph_step_us_median": t_graph,
            "graph_per_layer_us": None if t_graph is None else t_graph / N,
            "graph_note": graph_note,
            "link_bytes_per_step": link_bytes, "link_floor_us": floor_us,
            "frac_of_link_floor": floor_us / t,
            "misses": int(st[:, 0].sum()), "hits": int(st[:, 1].sum()),
            "recall": float(st[:, 1].sum() / max(st[:, 0].sum() + st[:, 1].sum(), 1))}


def components(dd, gen, w, kh, vh, h2d_gbps: float, dev, reps: int = 6):
    """The gather and the sparse attention measured alone at sizes where
    their own rate shows (inside the layer step the first runs beside the
    scorer and the second handles only k rows per head):

    gather: dd_gather of 4096 distinct random rows per head of K and V from
      the pinned host cache of this workload (row by row), and
      dd_gather_chunks of the same number of rows as 512 chunks of 8;
    attention: dd_sparse_attn over k = 1024 resident bf16 rows per head at
      the 32-layer 7B step's per-layer shape (16 requests x 32 heads x 128),
      ten calls back to back on two alternating copies of the rows (so they
      are not served from the Infinity Cache), time per call."""
    import numpy as np
    import torch
    from sparse_kv_retrieval_dual_amd.hipevents import EventSet

    B, H, D = w.B, w.H, w.D
    eb = w.elem_bytes
    g = torch.Generator().manual_seed(7)
    n = int(gen.request_lens(w).min().item())      # rows valid in every request
    m = min(4096, n)
    idx = torch.stack([torch.randperm(n, generator=g)[:m]
                       for _ in range(B * H)]).view(B, H, m).to(torch.int32).to(dev)
    ko = torch.empty(B, H, m, D, dtype=w.torch_dtype, device=dev)
    vo = torch.empty_like(ko)
    c = 8
    cidx = torch.stack([torch.randperm(n // c, generator=g)[:m // c]
                        for _ in range(B * H)]).view(B, H, m // c).to(torch.int32).to(dev)
    ev = EventSet(2)

    def timed(fn):
        fn()
        ts = []
        for _ in range(reps):
            ev.record(0)
            fn()
            ev.record(1)
            torch.cuda.synchronize()
            ts.append(ev.elapsed_ms(0, 1))
        return float(np.median(ts))

    gbytes = 2 * B * H * m * D * eb
    t_rows = timed(lambda: dd.gather(kh, vh, idx, k_out=ko, v_out=vo))
    t_chunks = timed(lambda: dd.gather_chunks(kh, vh, cidx, c, k_out=ko, v_out=vo))
    del ko, vo

    sw = gen.workload("llama7b_32k_step")
    aB, aH, ak, aD = sw.B, sw.H, sw.k, sw.D
    rows = [(torch.randn(aB, aH, ak, aD, device=dev).to(sw.torch_dtype),
             torch.randn(aB, aH, ak, aD, device=dev).to(sw.torch_dtype)) for _ in range(2)]
    q = torch.randn(aB, aH, 2, aD, device=dev)
    out = torch.empty(aB, aH, aD, dtype=torch.float32, device=dev)
    lse = torch.empty(aB, aH, dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, dd.attn_workspace_bytes(aB, aH, ak, aD)), dtype=torch.uint8, device=dev)
    abytes = 2 * aB * aH * ak * aD * sw.elem_bytes + aB * aH * aD * 4 * 2 + aB * aH * 4
    # Calls back to back between the events (the copies alternate), so that
    # the host's launch time is hidden behind the GPU's work.
    per = 10
    ts = []
    for i in range(reps + 2):
        ev.record(0)
        for j in range(per):
            kr, vr = rows[j % 2]
            dd.sparse_attn(q, kr, vr, k=ak, out=out, lse=lse, ws=ws)
        ev.record(1)
        torch.cuda.synchronize()
        if i >= 2:
            ts.append(ev.elapsed_ms(0, 1) / per)
    t_attn = float(np.median(ts))
    del rows
    return {
        "gather_rows": {"rows_per_head": m, "planes": 2, "bytes": gbytes, "us": t_rows * 1e3,
                        "GBps": gbytes / (t_rows * 1e-3) / 1e9,
                        "frac_of_h2d": gbytes / (t_rows * 1e-3) / 1e9 / h2d_gbps,
                        "frac_of_64GBps": gbytes / (t_rows * 1e-3) / 1e9 / LINK_PAGES_GBPS},
        "gather_chunks8": {"chunks_per_head": m // c, "planes": 2, "bytes": gbytes,
                           "us": t_chunks * 1e3, "GBps": gbytes / (t_chunks * 1e-3) / 1e9,
                           "frac_of_h2d": gbytes / (t_chunks * 1e-3) / 1e9 / h2d_gbps,
                           "frac_of_64GBps": gbytes / (t_chunks * 1e-3) / 1e9 / LINK_PAGES_GBPS},
        "sparse_attention": {"shape": f"B={aB} H={aH} k={ak} D={aD} {sw.dtype}",
                             "algorithmic_bytes": abytes, "us": t_attn * 1e3,
                             "GBps": abytes / (t_attn * 1e-3) / 1e9,
                             "frac": abytes / (t_attn * 1e-3) / 1e9 / HBM_PEAK_GBPS},
    }


def stage_inputs(dd, gen, w, dev, copies: int, k_host: bool = True):
    """One layer of the workload resident: keys in HBM (`copies` identical
    copies to rotate over), V (and K unless k_host is False: a step that
    reads K rows from HBM never reads the host K plane) in pinned host
    memory.  K and V are drawn one request at a time straight into their
    destinations, so a large workload never holds its whole V in HBM."""
    import torch

    kd = torch.empty(w.B, w.H, w.n_max, w.D, dtype=w.torch_dtype, device=dev)
    vh = dd.host_empty(kd.shape, kd.dtype)
    lay = gen.make_layer(w, 0, dev, k_out=kd, v_out=vh)
    torch.cuda.synchronize()
    kh = None
    if k_host:
        kh = dd.host_empty(kd.shape, kd.dtype)
        kh.copy_(kd)
    lay["k"] = kd
    k_copies = [kd] + [kd.clone() for _ in range(copies - 1)]
    torch.cuda.synchronize()
    return lay, kh, vh, k_copies


def one_workload(dd, gen, name: str, h2d_gbps: float, dev, steps: int = 6):
    """One layer step of a workload at its full per-layer shape: eager
    steps, each bracketed by events on the caller's stream (median), the
    same step replayed from a HIP graph, the
    scoring kernel's own duration from events its dispatch records, and the
    host-link bytes the step moved (prefetched and missed V rows) against
    the measured pinned-copy rate.  Keys rotate over two HBM copies when
    they fit the 256 MB Infinity Cache twice over, else one copy."""
    import gc

    import numpy as np
    import torch
    from sparse_kv_retrieval_dual_amd.hipevents import EventSet

    w = gen.workload(name)
    key_bytes = w.B * w.H * w.n_max * w.D * w.elem_bytes
    copies = 4 if key_bytes <= (64 << 20) else (2 if key_bytes <= (1 << 30) else 1)
    t0 = time.time()
    lay, kh, vh, k_copies = stage_inputs(dd, gen, w, dev, copies, k_host=False)
    lens = lay["lens"]
    t_stage = time.time() - t0
    ctx = dd.Context(ring_slots=2)
    q = lay["q"]
    res = ctx.layer_step([q], [k_copies[0]], None, [vh], lens, w.k)
    pred = [s_.clone() for s_ in res["spec"]]
    stats = torch.zeros(1, 3, dtype=torch.int64, device=dev)
    E = dd.DD_STAGE_EVENTS
    ev = EventSet(2 * (steps + 2))
    tev = EventSet(E * (steps + 2))
    plans = [ctx.prepare_step([q], [kc], None, [vh], lens, w.k, cur=res["cur"],
                              spec=res["spec"], out=res["out"], lse=res["lse"], stats=stats)
             for kc in k_copies]
    for i in range(steps + 2):
        ev.record(2 * i)
        t = [None] * E
        t[0], t[1] = tev.handles[E * i], tev.handles[E * i + 1]
        plans[i % len(plans)].run(pred=pred, timing=t)
        ev.record(2 * i + 1)
    torch.cuda.synchronize()
    step_us = float(np.median([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(2, steps + 2)])) * 1e3
    score_us = float(np.median([tev.elapsed_ms(E * i, E * i + 1) for i in range(2, steps + 2)])) * 1e3
    st = stats[0].cpu().tolist()
    # The same step replayed from a HIP graph (one step per key copy,
    # checked against the eager output first), as a decode loop runs it.
    graph_us, graph_note = None, None
    try:
        ref = res["out"][0].clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in range(len(k_copies)):
                plans[c].run(pred=pred)
        res["out"][0].zero_()
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(res["out"][0], ref):
            raise RuntimeError("graph replay differs from the eager step")
        gt = []
        for i in range(steps):
            ev.record(0)
            g.replay()
            ev.record(1)
            torch.cuda.synchronize()
            gt.append(ev.elapsed_ms(0, 1) * 1e3 / len(k_copies))
        graph_us = float(np.median(gt))
        del g
    except Exception as e:  # noqa: BLE001
        graph_note = f"graph replay unavailable: {e}"
    n_keys = int(lens.sum().item()) * w.H
    score_bytes = n_keys * (w.D * w.elem_bytes + 8)
    link_bytes = st[2] * w.D * w.elem_bytes
    floor_us = link_bytes / (h2d_gbps * 1e9) * 1e6
    ctx.close()
    out = {"B": w.B, "H": w.H, "context": w.n_max, "top_k": w.k, "kv_dtype": w.dtype,
           "ragged_lengths": w.len_lo != w.len_hi, "hbm_key_copies": len(k_copies),
           "layer_step_us": step_us, "keys_per_s": n_keys / (step_us * 1e-6),
           "score_us": score_us, "score_frac_of_hbm_peak":
               score_bytes / (score_us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
           "link_bytes": link_bytes, "link_floor_us": floor_us,
           "frac_of_link_floor": floor_us / step_us,
           "recall": st[1] / max(st[0] + st[1], 1), "misses": st[0],
           "timing": "eager, events around each step, median",
           "graph_layer_step_us": graph_us, "graph_keys_per_s":
               None if graph_us is None else n_keys / (graph_us * 1e-6),
           "graph_note": graph_note, "inputs_staged_s": t_stage}
    del lay, kh, vh, k_copies, res, pred, stats
    gc.collect()
    torch.cuda.empty_cache()
    return out


def gather_worked_example(dd, w, kh, vh, lens, h2d_gbps: float, dev, reps: int = 21):
    """dd_gather of exactly the transfer the worked example sizes: k = 128
    rows of K and V per head, 32 heads, bf16, head dim 128 = 2,097,152 B,
    from this workload's pinned host cache into HBM.  Each call is timed
    alone (events around it on the caller's stream; median)."""
    import numpy as np
    import torch
    from sparse_kv_retrieval_dual_amd.hipevents import EventSet

    B, H, D, m = w.B, w.H, w.D, 128
    g = torch.Generator().manual_seed(11)
    n = int(lens.min().item())
    idx = torch.stack([torch.randperm(n, generator=g)[:m].sort().values
                       for _ in range(B * H)]).view(B, H, m).to(torch.int32).to(dev)
    ko = torch.empty(B, H, m, D, dtype=w.torch_dtype, device=dev)
    vo = torch.empty_like(ko)
    nbytes = 2 * B * H * m * D * w.elem_bytes
    ev = EventSet(2)
    ts = []
    for i in range(reps + 1):
        ev.record(0)
        dd.gather(kh, vh, idx, k_out=ko, v_out=vo)
        ev.record(1)
        torch.cuda.synchronize()
        if i > 0:
            ts.append(ev.elapsed_ms(0, 1))
    t = float(np.median(ts))
    # The same call ten times back to back between two events: the rate once
    # the launch and the first host round trip are amortised.
    per = 10
    bts = []
    for i in range(6):
        ev.record(0)
        for _ in range(per):
            dd.gather(kh, vh, idx, k_out=ko, v_out=vo)
        ev.record(1)
        torch.cuda.synchronize()
        if i > 0:
            bts.append(ev.elapsed_ms(0, 1) / per)
    tb = float(np.median(bts))
    return {"bytes": nbytes, "rows": 2 * B * H * m, "us": t * 1e3,
            "GBps": nbytes / (t * 1e-3) / 1e9, "frac_of_h2d": nbytes / (t * 1e-3) / 1e9 / h2d_gbps,
            "timing": "one call alone, events around it, median of %d" % reps,
            "back_to_back_us": tb * 1e3, "back_to_back_GBps": nbytes / (tb * 1e-3) / 1e9,
            "back_to_back_frac_of_h2d": nbytes / (tb * 1e-3) / 1e9 / h2d_gbps,
            "frac_of_64GBps": nbytes / (t * 1e-3) / 1e9 / LINK_PAGES_GBPS,
            "back_to_back_frac_of_64GBps": nbytes / (tb * 1e-3) / 1e9 / LINK_PAGES_GBPS}


def hbm_read_rate(dd, dev, reps: int = 5, slice_bytes: int = 1 << 28):
    """Achievable HBM read rate: dd_stream_read (non-temporal loads, as the
    scorer's) of 1 GiB per call, median GB/s; and of slice_bytes per call
    (the scorer's key bytes at the 7B layer), four slices of the same buffer
    in turn so that the 256 MB Infinity Cache cannot serve a repeat, eight
    calls back to back between two events, median over reps of the per-call
    rate."""
    import numpy as np
    import torch
    from sparse_kv_retrieval_dual_amd.hipevents import EventSet

    big = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.empty(256, dtype=torch.uint8, device=dev)
    ev = EventSet(2)
    dd.stream_read(big, sink)
    rates, slice_rates = [], []
    for _ in range(reps):
        ev.record(0)
        dd.stream_read(big, sink)
        ev.record(1)
        torch.cuda.synchronize()
        rates.append(big.numel() / (ev.elapsed_ms(0, 1) * 1e-3) / 1e9)
    n_sl = big.numel() // slice_bytes
    slices = [big[i * slice_bytes:(i + 1) * slice_bytes] for i in range(n_sl)]
    for _ in range(reps):
        ev.record(0)
        for i in range(8):
            dd.stream_read(slices[i % n_sl], sink)
        ev.record(1)
        torch.cuda.synchronize()
        slice_rates.append(8 * slice_bytes / (ev.elapsed_ms(0, 1) * 1e-3) / 1e9)
    del big, slices
    return float(np.median(rates)), float(np.median(slice_rates))


def cpu_baseline(w, lay, budget_s: float):
    """The oracle as it stands, on the same workload, on the host's cores: a
    pool of threads runs oracle layer steps of one (request, head) each --
    its scoring, its full-sort top-k, its byte gather of the selected K and V
    rows and its dense-then-masked attention, each timed -- with BLAS held to
    one thread per call; heads are independent, so the layer is the sum of
    its heads.  Layers repeat until about budget_s seconds have passed.  The
    pool has one thread per core this process may run on, at most 16 (the
    host's share per GPU)."""
    import numpy as np
    import torch
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limiter = None
    # A batch of several requests is sampled down to its first request (the
    # oracle's fp64 copy of a whole batch would not fit in host memory).
    nb = 1

    def stored(t):  # the oracle's view of stored elements: bf16 as int16 bit patterns
        t = t[:nb].cpu().contiguous()
        return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.numpy()

    q = lay["q"][:nb].cpu().numpy()
    k16 = stored(lay["k"])
    v16 = stored(lay["v"])
    lens = lay["lens"][:nb].cpu().numpy()
    units = [(q[:, h:h + 1].copy(), k16[:, h:h + 1].copy(), v16[:, h:h + 1].copy())
             for h in range(w.H)]
    affinity = len(os.sched_getaffinity(0))
    threads = max(1, min(16, affinity))

    def run(u):
        qq, kk, vv = u
        t = [time.perf_counter()]
        s_ = oracle.scaled_logits(qq, kk, lens, w.dtype)
        t.append(time.perf_counter())
        sel = oracle.select_topk(s_, lens, w.k)
        t.append(time.perf_counter())
        cur = np.ascontiguousarray(sel[:, :, 0])
        oracle.gather_rows(kk, cur)
        oracle.gather_rows(vv, cur)
        t.append(time.perf_counter())
        oracle.masked_attention(qq[:, :, 0], kk, vv, lens, cur, w.dtype)
        t.append(time.perf_counter())
        return np.diff(t)

    reps, t0 = 0, time.perf_counter()
    stage = np.zeros(4)
    with ThreadPoolExecutor(threads) as ex:
        while True:
            for d in ex.map(run, units):
                stage += d
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    if limiter is not None:
        limiter.unregister()
    keys = int(np.sum(lens)) * w.H * reps
    names = ("score", "topk_full_sort", "gather", "masked_attention")
    per_layer = {n: float(x) / reps * 1e3 for n, x in zip(names, stage)}
    return {"value": keys / el, "unit": "keys/s", "cores": threads, "kind": "oracle",
            "affinity_cores": affinity, "cpu_model": _cpu_model(),
            "layer_step_ms_wall": el / reps * 1e3,
            "stage_thread_ms_per_layer": per_layer,
            "sample": f"{reps} oracle layer steps of {w.name} (B={nb} H={w.H} n={w.n_max} "
                      f"k={w.k}; fp64 scoring, full sort, byte gather of K and V, dense-masked "
                      f"attention), one (request, head) per task on {threads} threads, in "
                      f"{el:.1f} s; stage times are thread time summed over a layer's heads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama7b_32k_layer")
    ap.add_argument("--copies", type=int, default=4, help="HBM copies of the keys to rotate over")
    ap.add_argument("--ring", type=int, default=2)
    ap.add_argument("--gather-cus", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time the eager loop only")
    ap.add_argument("--prefetch-wgs", type=int, default=0)
    ap.add_argument("--prefetch", default="auto", choices=["auto", "side", "fused"])
    ap.add_argument("--select-prefetch-slabs", type=int, default=0,
                    help="slabs whose prefetch the selection kernel does (0: split by "
                         "sizes, -1: none)")
    ap.add_argument("--k-rows", default="device", choices=["device", "host"],
                    help="where attention reads the selected K rows")
    ap.add_argument("--chunk", type=int, default=0,
                    help="select by landmarks of chunks of this many keys (0: every key)")
    ap.add_argument("--dual", action="store_true",
                    help="the speculated query also attends over the selected rows")
    ap.add_argument("--no-components", action="store_true",
                    help="skip the stand-alone gather and attention measurements")
    ap.add_argument("--layers", type=int, default=1,
                    help="also time one step over this many layers of the workload's shape")
    ap.add_argument("--decode-steps", type=int, default=0,
                    help="also time this many real decode steps (KV append + layer step, "
                         "prediction carried), after the headline measurement; with "
                         "--layers, each step runs that many layers")
    ap.add_argument("--resident", action="store_true",
                    help="in the decode loop, also time it with each layer keeping its "
                         "selected rows across steps")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the one-layer steps of the other workloads and the "
                         "multi-layer 7B step")
    ap.add_argument("--workload-layers", type=int, default=32,
                    help="layers of the multi-layer 7B step in the workloads section")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(each GPU would run its own share of requests or heads independently).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gen
    import sparse_kv_retrieval_dual_amd as dd
    from sparse_kv_retrieval_dual_amd.hipevents import EventSet

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dd.load()
    dev = torch.device("cuda:0")
    w = gen.workload(args.workload)
    # A step is one layer step; a workload of L layers is timed on its first
    # layer (every layer has the same shapes and work).
    lay = gen.make_layer(w, 0, dev)
    lens = lay["lens"]
    kh = dd.host_empty(lay["k"].shape, lay["k"].dtype)
    vh = dd.host_empty(lay["v"].shape, lay["v"].dtype)
    kh.copy_(lay["k"].cpu())
    vh.copy_(lay["v"].cpu())
    k_copies = [lay["k"]] + [lay["k"].clone() for _ in range(args.copies - 1)]
    q = lay["q"]
    B, H, D, k = w.B, w.H, w.D, w.k
    n_keys = int(lens.sum().item()) * H
    eb = w.elem_bytes
    torch.cuda.synchronize()
    _progress(f"{w.name}: inputs resident ({n_keys} keys)")

    ctx = dd.Context(ring_slots=args.ring, gather_cus=args.gather_cus,
                     prefetch_wgs=args.prefetch_wgs, prefetch=args.prefetch, k_rows=args.k_rows,
                     select_prefetch_slabs=args.select_prefetch_slabs)
    chunk = args.chunk if args.chunk > 1 else 1
    ks = k // chunk                                      # entries selected per query
    # Landmarks are built once per cache (untimed here, measured below), one
    # per key copy so that they rotate like the keys.
    lm_copies = [dd.landmarks(kc, lens, chunk) for kc in k_copies] if chunk > 1 else None
    cur = [torch.empty(B, H, ks, dtype=torch.int32, device=dev)]
    spec = [torch.empty(B, H, ks, dtype=torch.int32, device=dev)]
    out = [torch.empty(B, H, D, dtype=torch.float32, device=dev)]
    lse = [torch.empty(B, H, dtype=torch.float32, device=dev)]
    out_spec = [torch.empty(B, H, D, dtype=torch.float32, device=dev)] if args.dual else None
    stats = torch.zeros(1, 3, dtype=torch.int64, device=dev)
    ring = torch.empty(dd.ring_bytes(args.ring, B, H, D, k, dd.kv_dtype(lay["k"])), dtype=torch.uint8, device=dev)
    ws = torch.empty(dd.layer_step_workspace_bytes(B, H, D, w.n_max, k), dtype=torch.uint8, device=dev)

    # One prepared step per (context, key copy): the arguments are checked
    # and marshalled once, and a step only passes its prediction, events and
    # stream (what a decode loop does; Context.layer_step redoes it all).
    plans = {}

    def step(i, pred, timing=None, c=None):
        cc = c or ctx
        key = (id(cc), i % len(k_copies))
        plan = plans.get(key)
        if plan is None:
            plan = cc.prepare_step([q], [k_copies[i % len(k_copies)]], [kh], [vh], lens, k,
                                   cur=cur, spec=spec, out=out, lse=lse, stats=stats,
                                   ring=ring, ws=ws, chunk=chunk if chunk > 1 else 0,
                                   landmarks=[lm_copies[i % len(lm_copies)]] if chunk > 1
                                   else None, out_spec=out_spec)
            plans[key] = plan
        plan.run(pred=pred, timing=timing)

    # Untimed first step without a prediction; its speculated set predicts the next.
    step(0, None)
    pred = [spec[0].clone()]
    for i in range(args.warmup):
        step(i, pred)
    torch.cuda.synchronize()
    ref_out = out[0].clone()

    # A decode loop replays the step from a HIP graph (one per key copy);
    # each graph is checked against the eager result on several replays with
    # eager work in between, else the eager loop is the headline.
    # One graph holds one full step per key copy, back to back (each step
    # still starts only after the previous one ended, as in decode).
    graph, graph_note = None, None
    S = len(k_copies)
    if not args.no_graph:
        try:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for c in range(S):
                    step(c, pred)
            for rep in range(3):
                out[0].zero_()
                g.replay()
                torch.cuda.synchronize()
                if not torch.equal(out[0], ref_out):
                    raise RuntimeError(f"graph replay {rep} differs from the eager step")
                step(rep, pred)
                torch.cuda.synchronize()
            graph = g
        except Exception as e:  # noqa: BLE001
            graph, graph_note = None, f"graph replay unavailable: {e}"

    K = args.steps
    E = dd.DD_STAGE_EVENTS
    bounds = EventSet(4)
    if graph is not None:
        reps = max(1, K // S)
        for i in range(max(1, args.warmup // S)):
            graph.replay()
        torch.cuda.synchronize()
        bounds.record(2)
        for i in range(reps):
            graph.replay()
        bounds.record(3)
        torch.cuda.synchronize()
        graph_ms = bounds.elapsed_ms(2, 3) / (reps * S)
        if not torch.equal(out[0], ref_out):
            raise RuntimeError("graph replays changed the output")

    # Eager timed region: K steps; the only events inside a step bracket the
    # scoring kernel (the dominant one), on the stream it runs on.
    score_ev = EventSet(2 * K)
    torch.cuda.synchronize()
    bounds.record(0)
    for i in range(K):
        t = [None] * E
        t[0], t[1] = score_ev.handles[2 * i], score_ev.handles[2 * i + 1]
        step(i, pred, timing=t)
    bounds.record(1)
    torch.cuda.synchronize()
    eager_ms = bounds.elapsed_ms(0, 1) / K
    ms_per_step = graph_ms if graph is not None else eager_ms
    t_score = float(np.mean([score_ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(K)]))
    _progress(f"timed {K} steps: {ms_per_step * 1e3:.1f} us per step")

    # Breakdown: the same steps again with every stage bracketed (the extra
    # event records make these steps slightly longer; not the headline).
    stage = EventSet(K * E)
    for i in range(K):
        step(i, pred, timing=stage.handles[i * E:(i + 1) * E])
    torch.cuda.synchronize()

    def avg(a, b):
        return float(np.mean([stage.elapsed_ms(i * E + a, i * E + b) for i in range(K)]))

    # Events 2-4 all follow the kernel that selects, does the bookkeeping and
    # attends; 5 and 6 bracket a side-stream prefetch (when there is one).
    t_select_attn = avg(1, 4)
    t_prefetch = avg(5, 6) if args.prefetch == "side" else None
    t_step_instr = avg(0, 4)
    steps_instr = np.array([stage.elapsed_ms(i * E, i * E + 4) for i in range(K)]) * 1e3
    st = stats[0].cpu().tolist()
    misses, hits, fetched = st
    n_sel = int(((lens + chunk - 1) // chunk).sum().item()) * H   # rows scored: keys or landmarks
    valid = int(torch.clamp((lens + chunk - 1) // chunk, max=ks).sum().item()) * H  # entries selected

    # Algorithmic bytes of the scorer per launch: every valid key row (or
    # fp32 landmark row) once (both queries), plus the two fp32 logits
    # written per row.
    row_b = D * eb if chunk == 1 else D * 4
    score_bytes = n_sel * row_b + n_sel * 2 * 4
    score_gbps = score_bytes / (t_score * 1e-3) / 1e9
    planes = 1 if args.k_rows == "device" else 2    # V rows only, or K and V
    prefetch_bytes = valid * chunk * planes * D * eb     # k rows per (b, h)
    # The prefetch runs on the side stream (own events) or inside the scoring
    # kernel (then its rate is bounded below by that kernel's duration).
    t_pf = t_prefetch if t_prefetch is not None else t_score
    prefetch_gbps = prefetch_bytes / (t_pf * 1e-3) / 1e9
    miss_bytes = misses * chunk * planes * D * eb

    # A cold step: the same step with no prediction, so every selected row
    # is fetched over the host link on the critical path (eager, events
    # around each step on the caller's stream).
    cold_ev = EventSet(2)
    cold_sc = EventSet(2)
    cold, cold_score = [], []
    for i in range(max(3, min(K, 20))):
        cold_ev.record(0)
        t = [None] * E
        t[0], t[1] = cold_sc.handles[0], cold_sc.handles[1]
        step(i, None, timing=t)
        cold_ev.record(1)
        torch.cuda.synchronize()
        cold.append(cold_ev.elapsed_ms(0, 1) * 1e3)
        cold_score.append(cold_sc.elapsed_ms(0, 1) * 1e3)
    step(0, pred)  # leaves the stats and outputs of a predicted step
    torch.cuda.synchronize()

    # The prefetch alone: the prediction's V rows (and K rows with K from the
    # host) gathered by a stand-alone dd_gather, each call timed alone.
    pf_ev = EventSet(2)
    pf_times = []
    pf_v = torch.empty(B, H, ks * chunk, D, dtype=w.torch_dtype, device=dev)
    pf_k = torch.empty_like(pf_v) if args.k_rows == "host" else None
    for i in range(8):
        pf_ev.record(0)
        if chunk > 1:
            dd.gather_chunks(kh if pf_k is not None else None, vh, pred[0], chunk,
                             k_out=pf_k, v_out=pf_v)
        else:
            dd.gather(kh if pf_k is not None else None, vh, pred[0], k_out=pf_k, v_out=pf_v)
        pf_ev.record(1)
        torch.cuda.synchronize()
        if i >= 2:
            pf_times.append(pf_ev.elapsed_ms(0, 1) * 1e3)
    del pf_v, pf_k
    t_prefetch_alone = float(np.median(pf_times))

    # The landmark build (once per cache, not per step), over the same copies.
    lm_info = None
    if chunk > 1:
        ev_lm = EventSet(2)
        for kc, lm in zip(k_copies, lm_copies):
            dd.landmarks(kc, lens, chunk, out=lm)
        reps = 4 * len(k_copies)
        ev_lm.record(0)
        for i in range(reps):
            dd.landmarks(k_copies[i % len(k_copies)], lens, chunk, out=lm_copies[i % len(lm_copies)])
        ev_lm.record(1)
        torch.cuda.synchronize()
        t_lm = ev_lm.elapsed_ms(0, 1) / reps
        lm_bytes = n_keys * D * eb + B * H * lm_copies[0].shape[2] * D * 4
        lm_info = {"us": t_lm * 1e3, "algorithmic_bytes": lm_bytes,
                   "GBps": lm_bytes / (t_lm * 1e-3) / 1e9,
                   "frac": lm_bytes / (t_lm * 1e-3) / 1e9 / HBM_PEAK_GBPS}

    # Reference rates measured in the same process.
    big = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    big2 = torch.empty_like(big)
    ev = EventSet(2)
    dd.stream_copy(big, big2)
    copies = []
    for _ in range(5):
        ev.record(0)
        dd.stream_copy(big, big2)
        ev.record(1)
        torch.cuda.synchronize()
        copies.append(2 * big.numel() / (ev.elapsed_ms(0, 1) * 1e-3) / 1e9)
    hbm_copy = float(np.median(copies))
    hpin = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    h2d = []
    for _ in range(5):
        ev.record(0)
        big.copy_(hpin, non_blocking=True)
        ev.record(1)
        torch.cuda.synchronize()
        h2d.append(big.numel() / (ev.elapsed_ms(0, 1) * 1e-3) / 1e9)
    h2d_gbps = float(np.median(h2d))
    del big, big2, hpin
    hbm_read, hbm_read_slice = hbm_read_rate(dd, dev)
    worked = (gather_worked_example(dd, w, kh, vh, lens, h2d_gbps, dev)
              if (B, H, D, w.dtype) == (1, 32, 128, "bf16") else None)
    comp = None if args.no_components else components(dd, gen, w, kh, vh, h2d_gbps, dev)
    _progress("reference rates and components done")

    # The same step with K and V rows both gathered from the host copy (the
    # pages' transfer: K rows of the selection cross the link too, and
    # attention reads the gathered K rows), timed the same way as the
    # headline when a graph is available, else eagerly.
    host_kv = None
    # Only at the 7B layer's shape: run as the main workload, hiconc_64 ended
    # in a host segmentation fault somewhere after its reference rates,
    # before its JSON line (cause not found), so this stage stays off for the
    # other shapes.
    if args.k_rows == "device" and chunk == 1 and w.name == "llama7b_32k_layer":
        hctx = dd.Context(ring_slots=args.ring, gather_cus=args.gather_cus,
                          prefetch_wgs=args.prefetch_wgs, prefetch=args.prefetch, k_rows="host")
        step(0, pred, c=hctx)
        torch.cuda.synchronize()
        hstats0 = stats[0].cpu().tolist()
        hev = EventSet(2)
        h_note = "eager"
        try:
            hg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(hg):
                for c_ in range(S):
                    step(c_, pred, c=hctx)
            hg.replay()
            torch.cuda.synchronize()
            hreps = max(1, K // S)
            hev.record(0)
            for i in range(hreps):
                hg.replay()
            hev.record(1)
            torch.cuda.synchronize()
            h_us = hev.elapsed_ms(0, 1) / (hreps * S) * 1e3
            h_note = f"hip-graph replay, {S} steps per graph"
            del hg
        except Exception:  # noqa: BLE001
            hts = []
            for i in range(K):
                hev.record(0)
                step(i, pred, c=hctx)
                hev.record(1)
                torch.cuda.synchronize()
                hts.append(hev.elapsed_ms(0, 1) * 1e3)
            h_us = float(np.median(hts))
        hlink = hstats0[2] * 2 * D * eb
        host_kv = {"layer_step_us": h_us, "keys_per_s": n_keys / (h_us * 1e-6), "timing": h_note,
                   "link_bytes": hlink,
                   "link_floor_us": hlink / (h2d_gbps * 1e9) * 1e6,
                   "note": "K and V rows of the prediction and the misses over the host link "
                           "(the pages' transfer); attention reads the gathered K rows"}
        hctx.close()
        step(0, pred)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, lay, args.cpu_seconds)
        _progress("cpu baseline done")

    traffic = _counter_traffic("score", SCORE_SOURCES, w.name) if chunk == 1 else None
    result = {
        "metric": METRIC,
        "value": n_keys / (ms_per_step * 1e-3),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "layers_timed": f"1 of {w.L}", "batch": B, "heads": H,
                   "head_dim": D, "context": w.n_max,
                   "top_k": k, "queries": 2, "kv_dtype": w.dtype, "accumulate": "f32",
                   "ring_slots": args.ring, "hbm_key_copies": len(k_copies),
                   "k_rows": args.k_rows, "chunk": chunk, "dual_token": bool(args.dual)},
        "roofline": {"bound": "hbm", "achieved": score_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": score_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic,
                     "kernel": "score", "algorithmic_bytes": score_bytes,
                     "avg_launch_us": t_score * 1e3},
        "cpu_baseline": cpu,
        "layer_step_us": ms_per_step * 1e3,
        "timing": (f"hip-graph replay, {S} steps per graph" if graph is not None else "eager"),
        "eager_layer_step_us": eager_ms * 1e3,
        "graph_note": graph_note,
        "stages_us": {"score": t_score * 1e3,
                      "select_bookkeeping_attention": t_select_attn * 1e3,
                      "prefetch_side_stream": None if t_prefetch is None else t_prefetch * 1e3,
                      "instrumented_step": t_step_instr * 1e3,
                      "instrumented_step_p10_p50_p90": [float(np.percentile(steps_instr, p))
                                                        for p in (10, 50, 90)]},
        "cold_layer_step_us": {"median": float(np.median(cold)),
                               "note": "eager, no prediction: every selected row over the "
                                       "host link on the critical path"},
        "score_keys_per_s": n_keys / (t_score * 1e-3),
        "score_frac_of_measured_hbm_read": score_gbps / hbm_read,
        "hbm_stream_read_GBps": hbm_read,
        "hbm_stream_read_256MiB_GBps": hbm_read_slice,
        "score_frac_of_256MiB_read": score_gbps / hbm_read_slice,
        "hbm_stream_read_note": ("dd_stream_read: 1 GiB per call (events around one call), and "
                                 "256 MiB per call (the scorer's key bytes at the 7B layer; "
                                 "8 calls back to back over 4 slices)"),
        "gather_GBps_lower_bound": prefetch_gbps,
        "gather_frac_of_h2d_lower_bound": prefetch_gbps / h2d_gbps,
        "gather_lower_bound_note": ("the step's prefetched bytes over the whole scoring kernel "
                                    "it rides in (or its side-stream span): a lower bound on "
                                    "the gather's rate; gather_worked_example and components "
                                    "time the gather alone"),
        "gather_worked_example": worked,
        "h2d_memcpy_GBps": h2d_gbps,
        "hbm_stream_copy_GBps": hbm_copy,
        "hbm_stream_copy_note": "1 GiB read + 1 GiB written per copy, both counted",
        "prediction": {"misses": misses, "hits": hits, "rows_fetched": fetched,
                       "recall": hits / max(valid, 1), "miss_bytes": miss_bytes,
                       "unit": "keys" if chunk == 1 else f"chunks of {chunk} keys"},
    }
    # Overlap: the stages measured alone (scoring without the prefetch, the
    # prefetch gather alone, the top-k + bookkeeping + attention kernel of a
    # predicted step) against the step, and the floors the step cannot beat.
    t_score_alone = float(np.median(cold_score))
    sum_stages = t_score_alone + t_prefetch_alone + t_select_attn * 1e3
    hbm_floor = score_bytes / (HBM_PEAK_GBPS * 1e9) * 1e6
    link_floor = (fetched * chunk * planes * D * eb) / (h2d_gbps * 1e9) * 1e6
    step_us = ms_per_step * 1e3
    result["overlap"] = {
        "eta": (sum_stages - step_us) / max(sum_stages - max(hbm_floor, link_floor), 1e-9),
        "definition": "(sum of stage times - step) / (sum of stage times - max(HBM floor, "
                      "host-link floor))",
        "sum_stages_us": sum_stages, "step_us": step_us,
        "stages_alone_us": {"score_without_prefetch": t_score_alone,
                            "prefetch_gather_alone": t_prefetch_alone,
                            "select_bookkeeping_attention": t_select_attn * 1e3},
        "hbm_floor_us": hbm_floor, "link_floor_us": link_floor,
        "step_frac_of_floor": max(hbm_floor, link_floor) / step_us}
    if host_kv is not None:
        result["k_rows_host"] = host_kv
    if comp is not None:
        result["components"] = comp
    if lm_info is not None:
        result["landmarks_build"] = lm_info
    if args.layers > 1:
        result["multi_layer"] = multi_layer(dd, w, lay, kh, vh, k_copies, lens, args.layers,
                                            h2d_gbps, dev, max(3, min(args.steps, 10)),
                                            "auto" if args.prefetch == "auto" else args.prefetch,
                                            args.k_rows, chunk, lm_copies)
    if args.decode_steps > 0:
        c0 = chunk if chunk > 1 else 0
        result["decode_loop"] = decode_loop(dd, gen, w, lay, kh, vh, k_copies[0], lens,
                                            args.decode_steps, c0, dev, layers=args.layers,
                                            h2d_gbps=h2d_gbps, prefetch_wgs=args.prefetch_wgs,
                                            prefetch=args.prefetch)
        if args.resident:
            result["decode_loop_resident"] = decode_loop(
                dd, gen, w, lay, kh, vh, k_copies[0], lens, args.decode_steps, c0, dev,
                layers=args.layers, resident=True, h2d_gbps=h2d_gbps,
                prefetch_wgs=args.prefetch_wgs, prefetch=args.prefetch)
    ctx.close()
    if not args.no_workloads and w.name == "llama7b_32k_layer":
        # Largest first, while the most host memory is free; a workload that
        # cannot be staged or run is recorded with its error, not fatal.
        import gc
        del k_copies, kh, vh, lay, lm_copies, ring, ws, cur, spec, out, lse, out_spec, pred
        graph = None
        gc.collect()
        torch.cuda.empty_cache()
        if hasattr(torch._C, "_host_emptyCache"):
            torch._C._host_emptyCache()  # the pinned buffer of the H2D reference
        wl = {}
        for name in ("hiconc_64", "llama13b_128k", "llama7b_32k_step", "tiny"):
            try:
                wl[name] = one_workload(dd, gen, name, h2d_gbps, dev)
                _progress(f"workload {name}: {wl[name]['layer_step_us']:.1f} us per layer step")
            except Exception as e:  # noqa: BLE001
                wl[name] = {"error": f"{type(e).__name__}: {e}"}
                _progress(f"workload {name}: {wl[name]['error']}")
            gc.collect()
            torch.cuda.empty_cache()
        # The multi-layer step of the 7B decode workload: layer l+1's prefetch
        # overlaps layer l (side stream), its layers sharing one layer's tensors.
        try:
            sw = gen.workload("llama7b_32k_step")
            slay, skh, svh, sk = stage_inputs(dd, gen, sw, dev, 1, k_host=False)
            ml = multi_layer(dd, sw, slay, skh, svh, sk[0], slay["lens"], args.workload_layers,
                             h2d_gbps, dev, 3, "side", "device")
            del slay, skh, svh, sk
            _progress("multi-layer step done")
        except Exception as e:  # noqa: BLE001
            ml = {"error": f"{type(e).__name__}: {e}"}
            _progress(f"multi-layer step: {ml['error']}")
        if "error" not in wl["llama7b_32k_step"]:
            wl["llama7b_32k_step"]["multi_layer"] = ml
        else:
            wl["llama7b_32k_step_multi_layer"] = ml
        result["workloads"] = wl
    print(json.dumps(result))


if __name__ == "__main__":
    main()
