"""Parity of dd_layer_step with the oracle's layer step, its independence of
the prediction, the ring-slot contents, and the statistics."""
import numpy as np
import pytest
import torch

import gen
import oracle
from tests import parity
from tests.gpu_util import announce, require_gpu, stored, to_host

pytestmark = pytest.mark.gpu


def _stage(dd, w, layers):
    data = []
    for l in range(layers):
        lay = gen.make_layer(w, l, "cpu")
        data.append({
            "q": lay["q"], "k": lay["k"], "v": lay["v"], "lens": lay["lens"],
            "q_dev": lay["q"].cuda(), "k_dev": lay["k"].cuda(),
            "k_host": to_host(dd, lay["k"]), "v_host": to_host(dd, lay["v"]),
        })
    return data


def _run(dd, ctx, w, data, pred=None, ring=None, ws=None):
    res = ctx.layer_step([d["q_dev"] for d in data], [d["k_dev"] for d in data],
                         [d["k_host"] for d in data], [d["v_host"] for d in data],
                         data[0]["lens"].cuda(), w.k, pred=pred, ring=ring, ws=ws)
    torch.cuda.synchronize()
    return res


def _check_layer(w, d, res, l, pred_np=None):
    """Sets (tie rule), attention (with exchange slack) and statistics of layer l."""
    B, H, k = w.B, w.H, w.k
    ref = oracle.layer_step(d["q"].numpy(), stored(d["k"]), stored(d["k"]), stored(d["v"]),
                            d["lens"].numpy(), k, w.dtype, pred=pred_np)
    lens_rows = np.repeat(d["lens"].numpy(), H)
    s = ref["scores"]
    cur = res["cur"][l].cpu().numpy().reshape(B * H, k)
    spec = res["spec"][l].cpu().numpy().reshape(B * H, k)
    diff_cur = parity.check_index_sets(cur, ref["cur"].reshape(B * H, k), s[:, :, 0].reshape(B * H, -1), lens_rows, k)
    parity.check_index_sets(spec, ref["spec"].reshape(B * H, k), s[:, :, 1].reshape(B * H, -1), lens_rows, k)
    slack = np.zeros(B * H)
    vf = oracle.upcast(stored(d["v"]), w.dtype)
    for r in diff_cur:
        b, h = divmod(r, H)
        n = int(lens_rows[r])
        slack[r] = parity.exchange_slack(s[b, h, 0, :n], ref["cur"][b, h], vf[b, h, :n], k,
                                         ref["out"][b, h])
    got = res["out"][l].cpu().numpy().reshape(B * H, w.D)
    worst = parity.check_attention(got, ref["out"].reshape(B * H, w.D), slack)
    st = res["stats"][l].cpu().numpy()
    valid = int(np.minimum(d["lens"].numpy(), k).sum()) * H
    assert st[0] + st[1] == valid
    if not diff_cur:
        assert np.array_equal(st, ref["stats"]), (st, ref["stats"])
    return worst, ref


@pytest.mark.parametrize("name,kw,R", [
    ("tiny", {}, 2),
    ("llama7b_32k_layer", dict(H=4, n_max=8192), 2),
    ("llama7b_32k_step", dict(L=1, B=2, H=2, n_max=8192, k=1024), 1),
    ("llama13b_128k", dict(L=1, B=1, H=2, n_max=16384, k=2048), 2),
    ("hiconc_64", dict(B=3, H=2, n_max=20000, len_lo=300, len_hi=20000, k=512), 3),
    # the attention's other two lane shapes: bf16 rows of 64 (two entries per
    # lane) and fp32 rows of 128 (eight), with k over one 128-entry chunk
    ("llama7b_32k_layer", dict(B=2, H=3, D=64, n_max=3000, len_lo=2000, len_hi=3000), 2),
    ("tiny", dict(H=3, D=128, n_max=3000, len_lo=2500, len_hi=3000, k=192), 2),
    # selection sizes at the edges: one key, an odd count, one past a chunk
    ("llama7b_32k_layer", dict(B=2, H=3, n_max=5000, len_lo=1, len_hi=5000, k=1), 2),
    ("llama7b_32k_layer", dict(B=3, H=2, n_max=4099, len_lo=20, len_hi=4099, k=33), 1),
    ("hiconc_64", dict(B=2, H=2, n_max=6000, len_lo=100, len_hi=6000, k=129), 2),
])
def test_layer_step_matches_oracle(name, kw, R):
    dd = require_gpu()
    w = gen.workload(name).scaled(**kw)
    announce(f"layer_step {name} {kw} R={R}")
    data = _stage(dd, w, w.L)
    ctx = dd.Context(ring_slots=R)
    cold = _run(dd, ctx, w, data)
    for l in range(w.L):
        worst, ref = _check_layer(w, data[l], cold, l)
    # the oracle's own speculated set as the prediction: statistics must match
    pred = [torch.from_numpy(ref["spec"]).cuda()]
    hot = _run(dd, ctx, w, data, pred=pred)
    _check_layer(w, data[0], hot, 0, pred_np=ref["spec"])
    assert torch.equal(hot["out"][0], cold["out"][0])
    ctx.close()
    print(f"worst relative attention error {worst:.2e}")


@pytest.mark.parametrize("mode,R", [("side", 2), ("fused", 1), ("fused", 2)])
def test_layer_step_short_and_empty_requests(mode, R):
    """Requests of 0, 1, k - 1, k, k + 1 and n_max keys in one batch: a
    request of length n <= k selects all of its keys (then -1), an empty one
    selects nothing and attends to nothing (zero output, lse -inf), and a
    second step on the speculated sets (-1 entries included) agrees again."""
    dd = require_gpu()
    w = gen.workload("llama7b_32k_layer").scaled(L=2, B=6, H=2, n_max=3000, k=128)
    lens = torch.tensor([0, 1, w.k - 1, w.k, w.k + 1, w.n_max], dtype=torch.int32)
    announce(f"layer_step short and empty requests lens={lens.tolist()} mode={mode} R={R}")
    data = _stage(dd, w, w.L)
    for d in data:
        d["lens"] = lens
    ctx = dd.Context(ring_slots=R, prefetch=mode)
    cold = _run(dd, ctx, w, data)
    refs = []
    for l in range(w.L):
        _, ref = _check_layer(w, data[l], cold, l)
        refs.append(ref)
    for l in range(w.L):
        cur = cold["cur"][l].cpu().numpy()
        assert (cur[0] == -1).all()
        assert np.array_equal(cur[1, :, 0], [0] * w.H) and (cur[1, :, 1:] == -1).all()
        assert (cur[2, :, :w.k - 1] == np.arange(w.k - 1)).all() and (cur[2, :, w.k - 1] == -1).all()
        assert (cur[3] == np.arange(w.k)).all()
        assert (cold["out"][l][0] == 0).all()
        assert torch.isneginf(cold["lse"][l][0]).all()
    pred = [torch.from_numpy(r["spec"]).cuda() for r in refs]
    hot = _run(dd, ctx, w, data, pred=pred)
    for l in range(w.L):
        _check_layer(w, data[l], hot, l, pred_np=refs[l]["spec"])
        assert torch.equal(hot["out"][l], cold["out"][l])
    ctx.close()


def test_outputs_do_not_depend_on_prediction_or_ring():
    """Misses are fetched on the critical path, so any prediction (none,
    perfect, speculated, random, another request's) and any ring size give
    bitwise identical outputs; the slot holds the right rows."""
    dd = require_gpu()
    w = gen.workload("llama7b_32k_layer").scaled(L=3, B=2, H=4, n_max=6000, k=256)
    announce("layer_step prediction independence")
    data = _stage(dd, w, w.L)
    B, H, k = w.B, w.H, w.k
    base_ctx = dd.Context(ring_slots=2)
    base = _run(dd, base_ctx, w, data)
    rand = [gen.random_sorted_indices(B * H, k, torch.tensor([w.n_max] * (B * H)), seed=50 + l,
                                      fill=0.9).reshape(B, H, k).cuda() for l in range(w.L)]
    other = [c.flip(0).contiguous() for c in base["cur"]]  # request 1's set for request 0 and back
    g = torch.Generator().manual_seed(77)
    perm = torch.randperm(k, generator=g).cuda()
    shuffled = [c[:, :, perm].contiguous() for c in base["cur"]]  # out of order
    dups = [torch.cat([c[:, :, : k // 2], c[:, :, : k // 2]], dim=2).contiguous() for c in base["cur"]]
    preds = {"spec": base["spec"], "perfect": base["cur"], "random": rand, "other": other,
             "partial": [None, base["spec"][1], None], "shuffled": shuffled, "duplicated": dups}
    # Reading of the pages (prediction format): a prediction out of order or
    # with repeats may lose hits, never outputs; the slot rows stay right.
    unordered = {"shuffled", "duplicated"}
    # K rows from the device copy (the base) or the host copy: the same bytes,
    # so the same bits.
    for R, mode, k_rows in ((1, "side", "device"), (2, "side", "device"), (3, "side", "device"),
                            (1, "fused", "device"), (2, "fused", "device"), (2, "side", "host"),
                            (1, "fused", "host"), (2, "fused", "host")):
        ctx = dd.Context(ring_slots=R, prefetch=mode, prefetch_wgs=8 if R == 1 else 0,
                         k_rows=k_rows)
        ring = torch.zeros(dd.ring_bytes(R, B, H, w.D, k, 1), dtype=torch.uint8, device="cuda")
        for pname, pred in preds.items():
            announce(f"  R={R} prefetch={mode} k_rows={k_rows} pred={pname}")
            res = _run(dd, ctx, w, data, pred=pred, ring=ring)
            for l in range(w.L):
                assert torch.equal(res["out"][l], base["out"][l]), (R, pname, l)
                assert torch.equal(res["lse"][l], base["lse"][l]), (R, pname, l)
                assert torch.equal(res["cur"][l], base["cur"][l])
                assert torch.equal(res["spec"][l], base["spec"][l])
                cur_l = res["cur"][l].cpu().numpy()
                p_l = None if pred[l] is None else pred[l].cpu().numpy()
                st = res["stats"][l].cpu().numpy()
                for_sets = [(set(cur_l[b, h][cur_l[b, h] >= 0].tolist()),
                             set() if p_l is None else set(p_l[b, h][p_l[b, h] >= 0].tolist()))
                            for b in range(B) for h in range(H)]
                misses = sum(len(c - p) for c, p in for_sets)
                hits = sum(len(c & p) for c, p in for_sets)
                fetched = sum(len(p) for _, p in for_sets) + misses
                if pname in unordered:
                    assert st[0] + st[1] == misses + hits and st[1] <= hits, (R, pname, l, st)
                else:
                    assert st.tolist() == [misses, hits, fetched], (R, pname, l, st)
            # slot of the last layer: row pos[j] holds host row cur[j] (V, and K
            # when K rows come from the host)
            l = w.L - 1
            slot = l % R
            if pname in unordered:
                continue
            cur_l = res["cur"][l].cpu().numpy()
            p_l = None if pred[l] is None else pred[l].cpu().numpy()
            bk = oracle.bookkeeping(cur_l, p_l, w.n_max)
            eb = 2
            sb = 2 * B * H * 2 * k * w.D * eb
            ring_np = ring[slot * sb:(slot + 1) * sb].cpu().numpy()
            kslot = ring_np[:sb // 2].view(np.int16).reshape(B, H, 2 * k, w.D)
            vslot = ring_np[sb // 2:].view(np.int16).reshape(B, H, 2 * k, w.D)
            kh, vh = stored(data[l]["k_host"]), stored(data[l]["v_host"])
            for b in range(B):
                for h in range(H):
                    for j in range(k):
                        c = cur_l[b, h, j]
                        if c < 0:
                            continue
                        r = bk["pos"][b, h, j]
                        if k_rows == "host":
                            assert np.array_equal(kslot[b, h, r], kh[b, h, c])
                        assert np.array_equal(vslot[b, h, r], vh[b, h, c])
        ctx.close()
    base_ctx.close()


def test_layer_step_workspace_errors():
    dd = require_gpu()
    w = gen.workload("tiny")
    announce("layer_step workspace errors")
    data = _stage(dd, w, 1)
    ctx = dd.Context(ring_slots=2)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(dd.DDError) as e:
        _run(dd, ctx, w, data, ring=small)
    assert e.value.code == 3
    with pytest.raises(dd.DDError) as e:
        _run(dd, ctx, w, data, ws=small)
    assert e.value.code == 3
    ctx.close()


def test_prepared_step_matches_layer_step():
    """A prepared step run with a prediction, with none and with another one
    gives what layer_step gives for each, bit for bit (outputs, sets,
    statistics), and layer_step's outputs do not depend on the prediction."""
    dd = require_gpu()
    w = gen.workload("llama7b_32k_layer").scaled(L=2, B=2, H=4, n_max=5000, k=256)
    announce("prepared step against layer_step")
    data = []
    for l in range(w.L):
        lay = gen.make_layer(w, l, "cpu")
        data.append(dict(q=lay["q"].cuda(), k=lay["k"].cuda(), kh=to_host(dd, lay["k"]),
                         vh=to_host(dd, lay["v"]), lens=lay["lens"].cuda()))
    args = ([d["q"] for d in data], [d["k"] for d in data], [d["kh"] for d in data],
            [d["vh"] for d in data], data[0]["lens"], w.k)
    ctx = dd.Context(ring_slots=2)
    cold = ctx.layer_step(*args)
    pa = [s.clone() for s in cold["spec"]]
    pb = [torch.flip(s, dims=[2]).contiguous() for s in cold["cur"]]
    want = {}
    for name, p in (("a", pa), ("none", None), ("b", pb)):
        r = ctx.layer_step(*args, pred=p)
        torch.cuda.synchronize()
        want[name] = {k_: [t.clone() for t in r[k_]] for k_ in ("out", "lse", "cur", "spec")}
        want[name]["stats"] = r["stats"].clone()
    step = ctx.prepare_step(*args)
    for name, p in (("a", pa), ("none", None), ("b", pb), ("a", pa)):
        r = step.run(pred=p)
        torch.cuda.synchronize()
        for k_ in ("out", "lse", "cur", "spec"):
            for l in range(w.L):
                assert torch.equal(r[k_][l], want[name][k_][l]), (name, k_, l)
                assert torch.equal(r[k_][l], want["none"][k_][l]), (name, k_, l)
        assert torch.equal(r["stats"], want[name]["stats"]), name
    ctx.close()
