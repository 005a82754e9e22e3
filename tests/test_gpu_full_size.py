"""Every workload at its full size, run the way bench.py runs the layer step
(ring of two slots, default prefetch placement and width, a cold step and
then a step predicted by the cold step's speculated sets).

The oracle checks every (request, head) slab of every distinct storage layer
one by one (a pool of threads runs the slabs); every slab is also checked
against properties that hold at any size: valid ascending sets, the planted
keys' place in the sets, prediction statistics recomputed from the returned
sets, bitwise independence of the prediction, bitwise equal results for
layers that share their storage, and the ring-slot rows.

The multi-layer workloads keep `m` distinct layers of storage and let layer
l use storage l mod m: every layer of its own would need 128 GiB of HBM keys
and 256 GiB of pinned host K/V (32 layers of batch 16 at 32K), or 200 GiB and
400 GiB (40 layers of batch 4 at 128K), more pinned memory than the host
gives one process.  The test prints m and the host's memory.
"""
import concurrent.futures as cf
import gc
import os
import time

import numpy as np
import pytest
import torch

import gen
import oracle
from tests import parity
from tests.gpu_util import announce, require_gpu, stored

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

# workload, distinct storage layers (every slab of each is checked)
FULL = [
    ("tiny", 1),
    ("llama7b_32k_layer", 1),
    ("llama7b_32k_step", 2),
    ("llama13b_128k", 2),
    ("hiconc_64", 1),
]


def _host_memory():
    """(MemTotal, MemAvailable) in GiB from /proc/meminfo, or (None, None)."""
    try:
        info = {}
        with open("/proc/meminfo") as f:
            for line in f:
                key, val = line.split(":", 1)
                info[key] = int(val.split()[0]) * 1024
        return info["MemTotal"] / 2**30, info.get("MemAvailable", 0) / 2**30
    except (OSError, KeyError, ValueError):
        return None, None


def _workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _log(t0, msg):
    announce(f"  {time.time() - t0:7.1f}s {msg}")


def _make(dd, w, m):
    """m layers of storage: keys in HBM, K and V in pinned host memory."""
    layers = []
    for l in range(m):
        kd = torch.empty(w.B, w.H, w.n_max, w.D, dtype=w.torch_dtype, device="cuda")
        vh = dd.host_empty(kd.shape, kd.dtype)
        lay = gen.make_layer(w, l, "cuda", k_out=kd, v_out=vh)
        torch.cuda.synchronize()
        kh = dd.host_empty(kd.shape, kd.dtype)
        kh.copy_(kd)
        layers.append({"q": lay["q"], "k_dev": kd, "k_host": kh, "v_host": vh,
                       "lens": lay["lens"],
                       "planted": lay["planted"].numpy(), "planted_cnt": lay["planted_cnt"].numpy()})
    return layers


def _check_sets(w, cur, lens):
    """Every row: count min(k, len), ascending, in range, -1 padding."""
    k = w.k
    m = np.minimum(np.repeat(lens, w.H), k).reshape(w.B, w.H)
    valid = cur >= 0
    assert np.array_equal(valid.sum(axis=2), m)
    col = np.arange(k)[None, None, :]
    assert np.all(valid == (col < m[:, :, None]))
    both = valid[:, :, 1:] & valid[:, :, :-1]
    assert np.all(np.diff(cur, axis=2)[both] > 0)
    assert np.all(cur < np.repeat(lens, w.H).reshape(w.B, w.H)[:, :, None])


def _check_planted(w, cur, lay):
    """The planted keys dominate every other key by tens of logit units, so
    each set holds all of them when they fit and only them when they do not."""
    for b in range(w.B):
        for h in range(w.H):
            c = int(lay["planted_cnt"][b, h])
            p = set(lay["planted"][b, h, :c].tolist())
            s = set(cur[b, h][cur[b, h] >= 0].tolist())
            if c <= w.k:
                assert p <= s, (b, h, len(p - s))
            else:
                assert s <= p, (b, h, len(s - p))


def _stats_from_sets(cur, pred):
    """[misses, hits, rows fetched] summed over slabs, from the sets alone."""
    k = cur.shape[-1]
    cur = cur.reshape(-1, k)
    pred = np.full_like(cur, -1) if pred is None else pred.reshape(-1, k)
    misses = hits = fetched = 0
    for c_row, p_row in zip(cur, pred):
        c = c_row[c_row >= 0]
        p = np.unique(p_row[p_row >= 0])
        hit = np.isin(c, p).sum()
        misses += c.size - hit
        hits += hit
        fetched += p.size + (c.size - hit)
    return [int(misses), int(hits), int(fetched)]


def _check_slab(w, lay, got, b, h, n, pred_l):
    """Oracle parity of one (layer, request, head) slab of n valid keys.

    got: the layer's results as NumPy arrays (q, cur, spec, out, lse)."""
    k, D = w.k, w.D
    q = got["q"][b, h][None, None]
    kk = stored(lay["k_host"][b, h])[None, None]
    vv = stored(lay["v_host"][b, h])[None, None]
    p = None if pred_l is None else pred_l[b, h][None, None]
    ref = oracle.layer_step(q, kk, kk, vv, np.array([n], np.int32), k, w.dtype, pred=p)
    s = ref["scores"]
    lens_row = np.array([n])
    cur = got["cur"][b, h][None]
    spec = got["spec"][b, h][None]
    diff = parity.check_index_sets(cur, ref["cur"].reshape(1, k), s[:, :, 0].reshape(1, -1), lens_row, k)
    parity.check_index_sets(spec, ref["spec"].reshape(1, k), s[:, :, 1].reshape(1, -1), lens_row, k)
    slack = np.zeros(1)
    swaps = 0
    if diff:
        m = min(k, n)
        swaps = np.setxor1d(cur[0, :m], ref["cur"][0, 0, :m]).size // 2
        vf = oracle.upcast(vv[0, 0, :n], w.dtype)
        slack[0] = parity.exchange_slack(s[0, 0, 0, :n], ref["cur"][0, 0], vf, k, ref["out"][0, 0])
    out = got["out"][b, h][None]
    worst = parity.check_attention(out, ref["out"].reshape(1, D), slack)
    gl = float(got["lse"][b, h])
    rl = float(ref["lse"][0, 0])
    # exchanging two entries of the tie band moves the log-sum-exp by at most
    # about twice the band width each
    assert abs(gl - rl) <= 1e-4 * max(1.0, abs(rl)) + swaps * 2.1e-3, (b, h, gl, rl)
    return worst, len(diff)


def _check_slot(w, ring, res, l, R, pred_l, lay, slabs, k_rows="device"):
    """Ring slot of layer l: row pos[j] of the slab holds host row cur[j] (V, and
    K when K rows come from the host)."""
    eb = w.elem_bytes
    BH, k, D = w.B * w.H, w.k, w.D
    slot_bytes = 2 * BH * 2 * k * D * eb
    base = (l % R) * slot_bytes
    slab_bytes = 2 * k * D * eb
    for b, h in slabs:
        bh = b * w.H + h
        cur = res["cur"][l][b, h].cpu().numpy()
        p = None if pred_l is None else pred_l[b, h][None, None]
        pos = oracle.bookkeeping(cur[None, None], p, w.n_max)["pos"][0, 0]
        koff = base + bh * slab_bytes
        voff = base + slot_bytes // 2 + bh * slab_bytes
        ks = ring[koff:koff + slab_bytes].cpu().numpy()
        vs = ring[voff:voff + slab_bytes].cpu().numpy()
        kh = stored(lay["k_host"][b, h]).view(np.uint8).reshape(w.n_max, D * eb)
        vh = stored(lay["v_host"][b, h]).view(np.uint8).reshape(w.n_max, D * eb)
        ks = ks.reshape(2 * k, D * eb)
        vs = vs.reshape(2 * k, D * eb)
        for j in np.nonzero(cur >= 0)[0]:
            if k_rows == "host":
                assert np.array_equal(ks[pos[j]], kh[cur[j]]), (l, b, h, j)
            assert np.array_equal(vs[pos[j]], vh[cur[j]]), (l, b, h, j)


@pytest.mark.parametrize("name,m", FULL)
def test_full_size_layer_step(name, m):
    dd = require_gpu()
    w = gen.workload(name)
    t0 = time.time()
    total, avail = _host_memory()
    per_layer = 2 * w.B * w.H * w.n_max * w.D * w.elem_bytes  # pinned K and V
    announce(f"full-size layer step {name}: L={w.L} B={w.B} H={w.H} D={w.D} n_max={w.n_max} "
             f"k={w.k} {w.dtype}, m={m} distinct storage layers; pinned K/V "
             f"{per_layer / 2**30:.1f} GiB per layer, {w.L * per_layer / 2**30:.0f} GiB for all "
             f"{w.L}; host memory " + ("unknown" if total is None else
                                         f"{total:.0f} GiB total, {avail:.0f} GiB available"))
    layers = _make(dd, w, m)
    _log(t0, "inputs ready")
    L, R = w.L, 2
    sel = [layers[l % m] for l in range(L)]
    lens = layers[0]["lens"]
    lens_np = lens.cpu().numpy()
    ctx = dd.Context(ring_slots=R)
    ring = torch.empty(dd.ring_bytes(R, w.B, w.H, w.D, w.k, dd.kv_dtype(sel[0]["k_dev"])),
                       dtype=torch.uint8, device="cuda")

    def run(pred):
        res = ctx.layer_step([d["q"] for d in sel], [d["k_dev"] for d in sel],
                             [d["k_host"] for d in sel], [d["v_host"] for d in sel], lens, w.k,
                             pred=pred, ring=ring)
        torch.cuda.synchronize()
        return res

    cold = run(None)
    _log(t0, "cold step done")
    pred = [s.clone() for s in cold["spec"]]
    hot = run(pred)
    _log(t0, "predicted step done")
    if L == 1:
        # K rows from the host copy instead of the device copy: the same bits
        hctx = dd.Context(ring_slots=R, k_rows="host")
        hring = torch.empty_like(ring)
        hres = hctx.layer_step([d["q"] for d in sel], [d["k_dev"] for d in sel],
                               [d["k_host"] for d in sel], [d["v_host"] for d in sel], lens, w.k,
                               pred=pred, ring=hring)
        torch.cuda.synchronize()
        for key in ("out", "lse", "cur", "spec", "stats"):
            if key == "stats":
                assert torch.equal(hres[key], hot[key])
            else:
                assert torch.equal(hres[key][0], hot[key][0]), key
        bh_pick = [(0, 0), (w.B - 1, w.H - 1)]
        _check_slot(w, hring, hres, 0, R, pred[0].cpu().numpy(), layers[0], bh_pick, "host")
        hctx.close()
        _log(t0, "K rows from the host copy: bitwise equal")

    for l in range(L):
        # the prediction never changes a result
        for key in ("out", "lse", "cur", "spec"):
            assert torch.equal(hot[key][l], cold[key][l]), (key, l)
        # layers sharing storage give bitwise equal results
        if l >= m:
            for key in ("out", "lse", "cur", "spec"):
                assert torch.equal(hot[key][l], hot[key][l % m]), (key, l)

    stats_cold = cold["stats"].cpu().numpy()
    stats_hot = hot["stats"].cpu().numpy()
    for l in range(min(L, m)):
        lay = layers[l]
        cur = hot["cur"][l].cpu().numpy()
        spec = hot["spec"][l].cpu().numpy()
        _check_sets(w, cur, lens_np)
        _check_sets(w, spec, lens_np)
        _check_planted(w, cur, lay)
        p = pred[l].cpu().numpy()
        assert stats_cold[l].tolist() == _stats_from_sets(cur, None), (l, stats_cold[l])
        assert stats_hot[l].tolist() == _stats_from_sets(cur, p), (l, stats_hot[l])
    for l in range(m, L):
        assert np.array_equal(stats_hot[l], stats_hot[l % m])
    _log(t0, f"properties hold on all slabs; predicted-step stats {stats_hot[0].tolist()}")

    worst = 0.0
    workers = _workers()
    for l in range(min(L, m)):
        lay = layers[l]
        slabs = [(b, h) for b in range(w.B) for h in range(w.H)]
        p = pred[l].cpu().numpy()
        got = {"q": lay["q"].cpu().numpy()}
        for key in ("cur", "spec", "out", "lse"):
            got[key] = hot[key][l].cpu().numpy()
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            futs = [ex.submit(_check_slab, w, lay, got, b, h, int(lens_np[b]), p)
                    for b, h in slabs]
            results = [f.result() for f in futs]
        worst = max([worst] + [r[0] for r in results])
        exchanged = sum(1 for r in results if r[1])
        # the last R layers still hold their rows in the ring
        corners = [(0, 0), (w.B - 1, w.H - 1), (int(np.argmin(lens_np)), 0)]
        for lr in range(max(0, L - R), L):
            if lr % m == l:
                _check_slot(w, ring, hot, lr, R, p, lay, corners)
        _log(t0, f"layer {l}: all {len(slabs)} slabs match the oracle ({workers} threads; "
                 f"{exchanged} with tie-band exchanges)")
    print(f"worst relative attention error {worst:.2e}")

    # the step as bench.py replays it: captured once, replayed twice
    if L == 1:
        g = torch.cuda.CUDAGraph()
        out_ref = [o.clone() for o in hot["out"]]
        bufs = {key: hot[key] for key in ("cur", "spec", "out", "lse", "stats")}
        with torch.cuda.graph(g):
            ctx.layer_step([d["q"] for d in sel], [d["k_dev"] for d in sel],
                           [d["k_host"] for d in sel], [d["v_host"] for d in sel], lens, w.k,
                           pred=pred, ring=ring, **bufs)
        for rep in range(2):
            for o in bufs["out"]:
                o.zero_()
            g.replay()
            torch.cuda.synchronize()
            for a, b_ in zip(bufs["out"], out_ref):
                assert torch.equal(a, b_), f"graph replay {rep}"
        del g
        _log(t0, "graph replays match")

    ctx.close()
    del layers, sel, cold, hot, pred, ring
    gc.collect()
    torch.cuda.empty_cache()
