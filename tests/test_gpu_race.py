"""Race detection for the layer step's two-stream schedule.

The prefetch of layer l runs on the side stream once its ring slot is free
(after the selection + attention kernel of layer l - R), and that kernel of
layer l waits for it (arXiv page, section 1: the layer-scoped manager
coordinates the asynchronous transfer with attention).  A missing or wrong
wait shows only under some timings, so the step is run with fixed stalls
inserted before every prefetch (side stream) or before every selection +
attention kernel (main stream), for R = 1, 2 and 3 slots, side and fused
prefetch, over 4 layers.  Every perturbed run must give the unperturbed
outputs, sets and statistics bit for bit.

The ring lies between two guard bands and every byte of it starts as a
canary: afterwards the guards are intact, every slot row a layer's step
wrote holds the right host row (its prediction's rows and its misses'), and
every row no step wrote still holds the canary.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from tests.gpu_util import announce, require_gpu, stored, to_host

pytestmark = pytest.mark.gpu

CANARY = 0xA5
GUARD = 4096


def _stage(dd, w):
    data = []
    for l in range(w.L):
        lay = gen.make_layer(w, l, "cpu")
        data.append({"q": lay["q"].cuda(), "k_dev": lay["k"].cuda(), "k": lay["k"], "v": lay["v"],
                     "k_host": to_host(dd, lay["k"]), "v_host": to_host(dd, lay["v"]),
                     "lens": lay["lens"]})
    return data


def _run(ctx, w, data, pred, ring=None, **kw):
    res = ctx.layer_step([d["q"] for d in data], [d["k_dev"] for d in data],
                         [d["k_host"] for d in data], [d["v_host"] for d in data],
                         data[0]["lens"].cuda(), w.k, pred=pred, ring=ring, **kw)
    torch.cuda.synchronize()
    return res


def _check_ring(w, data, res, pred, buf, R, k_rows):
    """Guards intact; rows written by the layers that used a slot hold their
    host rows (the last writer's); every other row holds the canary."""
    B, H, k, D, L = w.B, w.H, w.k, w.D, w.L
    eb = w.elem_bytes
    raw = buf.cpu().numpy()
    assert np.all(raw[:GUARD] == CANARY), "guard band before the ring overwritten"
    assert np.all(raw[-GUARD:] == CANARY), "guard band after the ring overwritten"
    ring = raw[GUARD:-GUARD]
    sb = 2 * B * H * 2 * k * D * eb
    row_b = D * eb
    for slot in range(min(R, L)):
        layers = [l for l in range(L) if l % R == slot]
        planes = ring[slot * sb:(slot + 1) * sb].reshape(2, B, H, 2 * k, row_b)
        for b in range(B):
            for h in range(H):
                written = set()
                for l in layers:
                    cur = res["cur"][l][b, h].cpu().numpy()
                    p = pred[l][b, h].cpu().numpy()
                    bk = oracle.bookkeeping(cur[None, None], p[None, None], w.n_max)
                    written |= {int(r) for r in range(k) if 0 <= p[r] < w.n_max}
                    written |= {k + t for t in range(int(bk["miss_cnt"][0, 0]))}
                last = layers[-1]
                cur = res["cur"][last][b, h].cpu().numpy()
                p = pred[last][b, h].cpu().numpy()
                pos = oracle.bookkeeping(cur[None, None], p[None, None], w.n_max)["pos"][0, 0]
                vh = stored(data[last]["v"][b, h]).view(np.uint8).reshape(w.n_max, row_b)
                kh = stored(data[last]["k"][b, h]).view(np.uint8).reshape(w.n_max, row_b)
                for j in np.nonzero(cur >= 0)[0]:
                    assert np.array_equal(planes[1, b, h, pos[j]], vh[cur[j]]), (slot, b, h, j)
                    if k_rows == "host":
                        assert np.array_equal(planes[0, b, h, pos[j]], kh[cur[j]]), (slot, b, h, j)
                untouched = [r for r in range(2 * k) if r not in written]
                assert np.all(planes[1, b, h, untouched] == CANARY), (slot, b, h, "V canary")
                if k_rows == "host":
                    assert np.all(planes[0, b, h, untouched] == CANARY), (slot, b, h, "K canary")
                else:
                    assert np.all(planes[0, b, h] == CANARY), (slot, b, h, "K plane written")


@pytest.mark.parametrize("mode,k_rows", [("side", "device"), ("fused", "device"),
                                         ("side", "host")])
def test_perturbed_streams_give_the_same_bits(mode, k_rows):
    dd = require_gpu()
    w = gen.workload("llama7b_32k_layer").scaled(L=4, B=2, H=4, n_max=6000, k=256)
    announce(f"race: prefetch={mode} k_rows={k_rows} L={w.L}")
    data = _stage(dd, w)
    base_ctx = dd.Context(ring_slots=2)
    cold = _run(base_ctx, w, data, None)
    pred = [s.clone() for s in cold["spec"]]
    base = _run(base_ctx, w, data, pred)
    base_ctx.close()
    for R in (1, 2, 3):
        nbytes = dd.ring_bytes(R, w.B, w.H, w.D, w.k, dd.kv_dtype(data[0]["k_dev"]))
        for side_us, main_us in ((0, 0), (40, 0), (0, 40), (40, 40)):
            if mode == "fused" and side_us:
                continue  # no side stream to stall
            announce(f"  R={R} stall side={side_us}us main={main_us}us")
            ctx = dd.Context(ring_slots=R, prefetch=mode, k_rows=k_rows,
                             perturb_side_us=side_us, perturb_main_us=main_us)
            buf = torch.full((nbytes + 2 * GUARD,), CANARY, dtype=torch.uint8, device="cuda")
            res = _run(ctx, w, data, pred, ring=buf[GUARD:GUARD + nbytes])
            for l in range(w.L):
                for key in ("out", "lse", "cur", "spec"):
                    assert torch.equal(res[key][l], base[key][l]), (R, side_us, main_us, key, l)
            assert torch.equal(res["stats"], base["stats"]), (R, side_us, main_us)
            _check_ring(w, data, res, pred, buf, R, k_rows)
            ctx.close()


def test_perturbed_streams_rows_kept_across_steps():
    """Rows kept across steps, prefetch on the side stream (every layer its
    own slots): two steps under stalls give the unperturbed bits."""
    dd = require_gpu()
    w = gen.workload("llama7b_32k_layer").scaled(L=4, B=2, H=4, n_max=6000, k=256)
    announce("race: rows kept across steps, side prefetch")
    data = _stage(dd, w)
    nb = dd.resident_bytes(w.L, w.B, w.H, w.D, w.n_max, w.k, dd.kv_dtype(data[0]["k_dev"]))
    results = {}
    for side_us, main_us in ((0, 0), (40, 0), (0, 40)):
        ctx = dd.Context(ring_slots=2, prefetch="side", perturb_side_us=side_us,
                         perturb_main_us=main_us)
        st = torch.empty(nb, dtype=torch.uint8, device="cuda")
        r0 = _run(ctx, w, data, None, resident=st, parity=0, reset=True)
        pred = [s.clone() for s in r0["spec"]]
        r1 = _run(ctx, w, data, pred, resident=st, parity=1)
        results[(side_us, main_us)] = (r0, r1)
        ctx.close()
    b0, b1 = results[(0, 0)]
    for key_, (r0, r1) in results.items():
        for l in range(w.L):
            for key in ("out", "lse", "cur", "spec"):
                assert torch.equal(r0[key][l], b0[key][l]), (key_, key, l)
                assert torch.equal(r1[key][l], b1[key][l]), (key_, key, l)
        assert torch.equal(r1["stats"], b1["stats"]), key_
