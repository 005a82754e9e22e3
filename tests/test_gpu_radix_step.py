"""Layer-step parity on rows that take the top-k radix path.

A current-query row goes to the radix path when its bound admits more
candidates than the candidate list holds (rows dominated by ties: every key
equal, or keys drawn from three vectors) or when it is longer than the
filter path handles (more than 131072 keys).  On that path the bookkeeping
walks the prediction list alongside the selection, numbering misses across
8192-key segments, and then attends.  A request shorter than k takes a third
path (every valid key selected) with its own lookup.

Tie-dominated keys use values whose dot products are exact in fp32 (entries
in {-1, -0.5, 0, 0.5, 1}, query entries multiples of 1/4): equal key rows
give bitwise equal scores on the GPU and exactly equal ones in the oracle,
so the lower-index rule decides both sets and they must be identical.

Each case runs with no prediction and with speculated, perfect, random,
other-request, shuffled and duplicated predictions, with the prefetch inside
the scoring kernel and on the side stream (K rows from the host copy), and
with rows kept across steps.  Checked: sets against the oracle, outputs
within the tolerance and bitwise independent of the prediction, statistics
equal to the oracle's bookkeeping, and every selected row of every slab in
its slot, byte for byte.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from tests import parity
from tests.gpu_util import announce, require_gpu, stored, to_host

pytestmark = pytest.mark.gpu

D = 128


def _nice_vectors(g, count):
    """count key rows with entries in {-1, -0.5, 0, 0.5, 1} (exact in bf16)."""
    return (torch.randint(-2, 3, (count, D), generator=g).to(torch.float32) * 0.5)


def _nice_query(g, shape):
    return torch.randint(-8, 9, shape, generator=g).to(torch.float32) * 0.25


def _make(B, H, n_max, lens, kinds, seed):
    """One layer: kinds[b][h] in {"equal", "three", "normal"}."""
    g = torch.Generator().manual_seed(seed)
    q = torch.empty(B, H, 2, D)
    k = torch.empty(B, H, n_max, D)
    v = torch.randn(B, H, n_max, D, generator=g)
    for b in range(B):
        for h in range(H):
            kind = kinds[b][h]
            if kind == "normal":
                qc = torch.randn(D, generator=g)
                q[b, h, 0] = qc
                q[b, h, 1] = 0.9 * qc + 0.44 * torch.randn(D, generator=g)
                kk = torch.randn(n_max, D, generator=g)
                n = int(lens[b])
                cnt = max(1, round(0.01 * n))
                pos = torch.randperm(n, generator=g)[:cnt]
                kk[pos] = 4.0 * qc + torch.randn(cnt, D, generator=g)
                k[b, h] = kk
            else:
                q[b, h] = _nice_query(g, (2, D))
                nv = 1 if kind == "equal" else 3
                vecs = _nice_vectors(g, nv)
                pick = torch.randint(0, nv, (n_max,), generator=g)
                k[b, h] = vecs[pick]
    kb = k.to(torch.bfloat16)
    vb = v.to(torch.bfloat16)
    return {"q": q.contiguous(), "k": kb.contiguous(), "v": vb.contiguous(),
            "lens": torch.tensor(lens, dtype=torch.int32)}


CASES = {
    # cached rows (n_max <= 32768): ties overflow the 2560-candidate list;
    # request 1 is shorter than k
    "cached_ties": dict(seed=11, B=2, H=4, n_max=32768, lens=[32768, 100], k=128,
                        kinds=[["equal", "three", "three", "normal"],
                               ["three", "equal", "normal", "three"]]),
    # longer rows: ties overflow the 8192-candidate list; n_max not a
    # multiple of 4 (no vector loads), ragged lengths
    "long_ties": dict(seed=12, B=2, H=2, n_max=40961, lens=[40961, 33001], k=1024,
                      kinds=[["three", "equal"], ["equal", "three"]]),
    # longer than the filter path takes: radix by length
    "over_filter": dict(seed=13, B=1, H=2, n_max=140000, lens=[140000], k=512,
                        kinds=[["normal", "three"]]),
}


def _oracle(lay, k, pred=None):
    ks = stored(lay["k"])
    return oracle.layer_step(lay["q"].numpy(), ks, ks, stored(lay["v"]), lay["lens"].numpy(), k,
                             "bf16", pred=pred)


def _check(case, lay, ref, res):
    """Sets, attention and the rows allowed to differ: only heads of
    continuous keys may exchange tie-band entries; tie-dominated heads must
    match exactly."""
    B, H, k = case["B"], case["H"], case["k"]
    lens_rows = np.repeat(lay["lens"].numpy(), H)
    s = ref["scores"]
    cur = res["cur"][0].cpu().numpy().reshape(B * H, k)
    spec = res["spec"][0].cpu().numpy().reshape(B * H, k)
    diff = parity.check_index_sets(cur, ref["cur"].reshape(B * H, k),
                                   s[:, :, 0].reshape(B * H, -1), lens_rows, k)
    dspec = parity.check_index_sets(spec, ref["spec"].reshape(B * H, k),
                                    s[:, :, 1].reshape(B * H, -1), lens_rows, k)
    for r in list(diff) + list(dspec):
        b, h = divmod(r, H)
        assert case["kinds"][b][h] == "normal", f"tie-dominated row {(b, h)} differs"
    slack = np.zeros(B * H)
    vf = oracle.upcast(stored(lay["v"]), "bf16")
    for r in diff:
        b, h = divmod(r, H)
        n = int(lens_rows[r])
        slack[r] = parity.exchange_slack(s[b, h, 0, :n], ref["cur"][b, h], vf[b, h, :n], k,
                                         ref["out"][b, h])
    parity.check_attention(res["out"][0].cpu().numpy().reshape(B * H, D),
                           ref["out"].reshape(B * H, D), slack)
    return diff


def _check_slot(case, lay, ring, R, cur, pred, k_rows):
    """Every selected row of every slab sits in its slot row, byte for byte."""
    B, H, k = case["B"], case["H"], case["k"]
    n_max = case["n_max"]
    bk = oracle.bookkeeping(cur, pred, n_max)
    sb = 2 * B * H * 2 * k * D * 2
    slot = ring[0:sb].cpu().numpy()  # layer 0 uses slot 0
    kslot = slot[:sb // 2].view(np.int16).reshape(B, H, 2 * k, D)
    vslot = slot[sb // 2:].view(np.int16).reshape(B, H, 2 * k, D)
    kh, vh = stored(lay["k"]), stored(lay["v"])
    for b in range(B):
        for h in range(H):
            sel = cur[b, h] >= 0
            c = cur[b, h][sel]
            r = bk["pos"][b, h][sel]
            assert np.array_equal(vslot[b, h, r], vh[b, h, c]), (b, h)
            if k_rows == "host":
                assert np.array_equal(kslot[b, h, r], kh[b, h, c]), (b, h)
    return bk


@pytest.mark.parametrize("name", list(CASES))
def test_radix_path_layer_step(name):
    dd = require_gpu()
    case = CASES[name]
    B, H, k, n_max = case["B"], case["H"], case["k"], case["n_max"]
    announce(f"radix-path layer step {name}: B={B} H={H} n_max={n_max} k={k}")
    lay = _make(B, H, n_max, case["lens"], case["kinds"], seed=case["seed"])
    q, kd = lay["q"].cuda(), lay["k"].cuda()
    kh, vh = to_host(dd, lay["k"]), to_host(dd, lay["v"])
    lens = lay["lens"].cuda()

    def run(ctx, pred, ring=None, **kw):
        res = ctx.layer_step([q], [kd], [kh], [vh], lens, k,
                             pred=None if pred is None else [pred], ring=ring, **kw)
        torch.cuda.synchronize()
        return res

    base_ctx = dd.Context(ring_slots=2)
    cold = run(base_ctx, None)
    ref = _oracle(lay, k)
    _check(case, lay, ref, cold)
    assert cold["stats"][0].tolist() == ref["stats"].tolist()

    spec = cold["spec"][0]
    cur = cold["cur"][0]
    perm = torch.randperm(k, generator=torch.Generator().manual_seed(5)).cuda()
    half = cur[:, :, : k // 2]
    preds = {
        "spec": spec.clone(),
        "perfect": cur.clone(),
        "random": gen.random_sorted_indices(B * H, k, torch.tensor([n_max] * (B * H)), seed=9,
                                            fill=0.8).reshape(B, H, k).cuda(),
        "other": cur.flip(0).contiguous(),
        "shuffled": spec[:, :, perm].contiguous(),
        "duplicated": torch.cat([half, half], dim=2).contiguous(),
    }
    cur_np = cur.cpu().numpy()
    for mode, R, k_rows in (("fused", 2, "device"), ("side", 1, "host")):
        ctx = dd.Context(ring_slots=R, prefetch=mode, k_rows=k_rows)
        ring = torch.zeros(dd.ring_bytes(R, B, H, D, k, 1), dtype=torch.uint8, device="cuda")
        for pname, pred in preds.items():
            announce(f"  prefetch={mode} R={R} k_rows={k_rows} pred={pname}")
            res = run(ctx, pred, ring)
            for key in ("out", "lse", "cur", "spec"):
                assert torch.equal(res[key][0], cold[key][0]), (pname, key)
            p_np = pred.cpu().numpy()
            bk = _check_slot(case, lay, ring, R, cur_np, p_np, k_rows)
            misses = int(bk["miss_cnt"].sum())
            want = [misses, int(bk["hits"].sum()), int(bk["prefetched"].sum()) + misses]
            assert res["stats"][0].tolist() == want, (mode, pname, res["stats"][0].tolist(), want)
        ctx.close()

    # the oracle's own step with a prediction: the same statistics
    ref_p = _oracle(lay, k, pred=preds["shuffled"].cpu().numpy())
    res = run(base_ctx, preds["shuffled"])
    assert res["stats"][0].tolist() == ref_p["stats"].tolist()

    # rows kept across steps: a first step, then one predicted by it
    st = torch.empty(dd.resident_bytes(1, B, H, D, n_max, k, 1), dtype=torch.uint8, device="cuda")
    rctx = dd.Context(ring_slots=2)
    r0 = run(rctx, None, resident=st, parity=0, reset=True)
    r1 = run(rctx, preds["shuffled"], resident=st, parity=1)
    for r in (r0, r1):
        for key in ("out", "lse", "cur", "spec"):
            assert torch.equal(r[key][0], cold[key][0]), key
    s1 = r1["stats"][0].tolist()
    assert s1[:2] == ref_p["stats"][:2].tolist(), (s1, ref_p["stats"])
    rctx.close()
    base_ctx.close()
