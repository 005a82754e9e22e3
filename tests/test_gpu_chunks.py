"""Selection by chunk landmarks: dd_landmarks, dd_gather_chunks and the layer
step with chunk > 1, against the oracle (landmarks, chunk_rows and
layer_step(chunk=c))."""
import numpy as np
import pytest
import torch

import gen
import oracle
from tests import parity
from tests.gpu_util import announce, require_gpu, stored, to_host

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24  # unit roundoff of fp32


@pytest.mark.parametrize("name,kw,c", [
    ("tiny", {}, 8),                                                       # fp32, D = 64
    ("llama7b_32k_layer", dict(H=3, n_max=5000), 16),                      # bf16, partial tail
    ("hiconc_64", dict(B=3, H=2, n_max=3000, len_lo=1, len_hi=3000), 8),   # ragged
    ("llama7b_32k_layer", dict(H=2, n_max=1000), 1),
    ("llama7b_32k_layer", dict(H=2, n_max=1000), 64),
])
def test_landmarks_match_oracle(name, kw, c):
    """fp32 sum of at most c terms in row order, then one division: the error
    is below (c + 1) u max |K| of the chunk (u = 2^-24)."""
    dd = require_gpu()
    w = gen.workload(name).scaled(**kw)
    announce(f"landmarks {name} {kw} chunk={c}")
    lay = gen.make_layer(w, 0, "cpu")
    lens = lay["lens"]
    got = dd.landmarks(lay["k"].cuda(), lens.cuda(), c).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    kst = stored(lay["k"])
    ref = oracle.landmarks(kst, lens.numpy(), c, w.dtype)
    assert got.shape == ref.shape
    kf = np.abs(oracle.upcast(kst, w.dtype))
    for b in range(w.B):
        n = int(lens[b])
        nc = -(-n // c)
        assert np.all(got[b, :, nc:] == 0)
        for e in range(nc):
            m = kf[b, :, e * c:min((e + 1) * c, n)].max()
            err = np.abs(got[b, :, e] - ref[b, :, e]).max()
            assert err <= (c + 1) * U32 * m, (b, e, err, m)


@pytest.mark.parametrize("c,planes", [(1, "kv"), (8, "kv"), (32, "v"), (64, "k")])
def test_gather_chunks_bytes(c, planes):
    """Byte-exact against the oracle's row gather of the expanded rows: a
    negative index and rows at or past n_max give zero rows, entries at or
    past cnt stay untouched."""
    dd = require_gpu()
    w = gen.workload("llama7b_32k_layer").scaled(B=2, H=3, n_max=1000)
    announce(f"gather_chunks chunk={c} planes={planes}")
    lay = gen.make_layer(w, 0, "cpu")
    kh, vh = to_host(dd, lay["k"]), to_host(dd, lay["v"])
    nc = -(-w.n_max // c)
    m = 24
    rng = np.random.default_rng(11 + c)
    idx = rng.integers(-1, nc + 1, size=(w.B, w.H, m)).astype(np.int32)
    idx[0, 0, 0] = nc - 1                       # the last, partial chunk
    cnt = rng.integers(0, m + 1, size=(w.B, w.H)).astype(np.int32)
    cnt[0, 0] = m
    rows_idx = np.where(idx[..., None] >= 0, idx[..., None] * c + np.arange(c), -1)
    rows_idx = rows_idx.reshape(w.B, w.H, m * c).astype(np.int64)
    rows_idx[rows_idx >= w.n_max] = -1
    sentinel = torch.full((w.B, w.H, m * c, w.D), 7, dtype=torch.int16).view(torch.bfloat16)
    k_out = sentinel.clone().cuda() if "k" in planes else None
    v_out = sentinel.clone().cuda() if "v" in planes else None
    dd.gather_chunks(kh if "k" in planes else None, vh if "v" in planes else None,
                     torch.from_numpy(idx).cuda(), c, cnt=torch.from_numpy(cnt).cuda(),
                     k_out=k_out, v_out=v_out)
    torch.cuda.synchronize()
    for plane, out, host in (("k", k_out, kh), ("v", v_out, vh)):
        if plane not in planes:
            continue
        want = oracle.gather_rows(stored(host), rows_idx, cnt * c, out=stored(sentinel).copy())
        assert np.array_equal(stored(out), want), plane


def _stage(dd, w, c, fixed_lens=None):
    data = []
    for l in range(w.L):
        lay = gen.make_layer(w, l, "cpu")
        if fixed_lens is not None:
            lay["lens"] = torch.tensor(fixed_lens, dtype=torch.int32)
        k_dev = lay["k"].cuda()
        lens = lay["lens"].cuda()
        data.append({"q": lay["q"], "k": lay["k"], "v": lay["v"], "lens": lay["lens"],
                     "q_dev": lay["q"].cuda(), "k_dev": k_dev,
                     "lm": dd.landmarks(k_dev, lens, c),
                     "k_host": to_host(dd, lay["k"]), "v_host": to_host(dd, lay["v"])})
    torch.cuda.synchronize()
    return data


def _run(ctx, w, data, c, pred=None, ring=None):
    res = ctx.layer_step([d["q_dev"] for d in data], [d["k_dev"] for d in data],
                         [d["k_host"] for d in data], [d["v_host"] for d in data],
                         data[0]["lens"].cuda(), w.k, pred=pred, ring=ring, chunk=c,
                         landmarks=[d["lm"] for d in data])
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("name,kw,c,R", [
    ("tiny", {}, 8, 2),
    ("llama7b_32k_layer", dict(H=4, n_max=8192), 8, 2),
    ("hiconc_64", dict(B=3, H=2, n_max=20000, len_lo=300, len_hi=20000, k=512), 16, 3),
    ("llama13b_128k", dict(L=1, B=1, H=2, n_max=16384, k=2048), 32, 2),
    ("llama7b_32k_step", dict(L=2, B=2, H=2, n_max=8192, k=1024), 64, 1),
    ("llama7b_32k_layer", dict(H=3, n_max=4096), 2, 2),
    ("hiconc_64", dict(B=3, H=2, n_max=3000, len_lo=100, len_hi=3000, k=128), 4, 2),
    # an empty request and requests of 1, 16 (= k/c chunks) less one key, 16
    # chunks, 16 chunks and one key, and n_max keys
    ("llama7b_32k_layer", dict(B=6, H=2, n_max=3000, k=128, lens=[0, 1, 127, 128, 129, 3000]),
     8, 2),
])
def test_chunk_layer_step_matches_oracle(name, kw, c, R):
    dd = require_gpu()
    kw = dict(kw)
    fixed = kw.pop("lens", None)
    w = gen.workload(name).scaled(**kw)
    announce(f"chunk layer_step {name} {kw} lens={fixed} chunk={c} R={R}")
    data = _stage(dd, w, c, fixed)
    B, H, ks = w.B, w.H, w.k // c
    ctx = dd.Context(ring_slots=R)
    ring = torch.zeros(dd.ring_bytes(R, B, H, w.D, w.k, dd.kv_dtype(data[0]["k_dev"])),
                       dtype=torch.uint8, device="cuda")
    cold = _run(ctx, w, data, c, ring=ring)
    pred = [s.clone() for s in cold["spec"]]
    hot = _run(ctx, w, data, c, pred=pred, ring=ring)
    hctx = dd.Context(ring_slots=R, k_rows="host")
    host = _run(hctx, w, data, c, pred=pred)
    sctx = dd.Context(ring_slots=R, prefetch="side")
    side = _run(sctx, w, data, c, pred=pred)
    sctx.close()
    worst = 0.0
    for l in range(w.L):
        d = data[l]
        # outputs do not depend on the prediction, on where K rows come from,
        # nor on where the prefetch runs
        for key in ("out", "lse", "cur", "spec"):
            assert torch.equal(hot[key][l], cold[key][l]), (key, l)
            assert torch.equal(host[key][l], hot[key][l]), (key, l)
            assert torch.equal(side[key][l], hot[key][l]), (key, l)
        lens = d["lens"].numpy()
        kst, vst = stored(d["k"]), stored(d["v"])
        ref = oracle.layer_step(d["q"].numpy(), kst, kst, vst, lens, w.k, w.dtype, chunk=c)
        nlen_rows = np.repeat(-(-lens // c), H)
        s = ref["scores"]
        cur = hot["cur"][l].cpu().numpy()
        spec = hot["spec"][l].cpu().numpy()
        parity.check_index_sets(cur.reshape(B * H, ks), ref["cur"].reshape(B * H, ks),
                                s[:, :, 0].reshape(B * H, -1), nlen_rows, ks)
        parity.check_index_sets(spec.reshape(B * H, ks), ref["spec"].reshape(B * H, ks),
                                s[:, :, 1].reshape(B * H, -1), nlen_rows, ks)
        # attention over the rows of the chunks the GPU chose (a valid top-k set)
        rows = oracle.chunk_rows(cur, lens, c)
        want, want_lse = oracle.masked_attention(d["q"][:, :, 0].numpy(), kst, vst, lens, rows,
                                                 w.dtype)
        got = hot["out"][l].cpu().numpy().reshape(B * H, w.D)
        worst = max(worst, parity.check_attention(got, want.reshape(B * H, w.D), np.zeros(B * H)))
        # statistics, in chunks
        p_np = pred[l].cpu().numpy()
        for res, p in ((cold, None), (hot, p_np)):
            bk = oracle.bookkeeping(cur, p, -(-w.n_max // c))
            misses = int(bk["miss_cnt"].sum())
            want_st = [misses, int(bk["hits"].sum()), int(bk["prefetched"].sum()) + misses]
            assert res["stats"][l].cpu().numpy().tolist() == want_st, (l, p is None)
    # the slot of the last layer holds the V rows of every selected chunk
    l = w.L - 1
    d = data[l]
    lens = d["lens"].numpy()
    cur = hot["cur"][l].cpu().numpy()
    bk = oracle.bookkeeping(cur, pred[l].cpu().numpy(), -(-w.n_max // c))
    eb = w.elem_bytes
    sb = 2 * B * H * 2 * w.k * w.D * eb
    vslot = ring[(l % R) * sb + sb // 2:(l % R + 1) * sb].cpu().numpy()
    vslot = vslot.view(np.uint8).reshape(B, H, 2 * w.k, w.D * eb)
    vh = stored(d["v_host"]).view(np.uint8).reshape(B, H, w.n_max, w.D * eb)
    for b, h in {(0, 0), (B - 1, H - 1)}:
        for j in range(ks):
            ch = int(cur[b, h, j])
            if ch < 0:
                continue
            p = int(bk["pos"][b, h, j])
            for i in range(c):
                r = ch * c + i
                if r < lens[b]:
                    assert np.array_equal(vslot[b, h, p * c + i], vh[b, h, r]), (b, h, j, i)
    ctx.close()
    hctx.close()
    print(f"worst relative attention error {worst:.2e}")


def test_chunk_ties_and_partial_tail_closed_form():
    """Keys are zero except the rows of the partial last chunk (48..51 of 52,
    chunk 8), which are 2q: that chunk's landmark scores 2|q|^2/sqrt(D) = 1
    and every other chunk exactly 0.  With k = 16 (two chunks) the current
    query takes chunk 6 and, among the tied zeros, chunk 0; the speculated
    query -q takes chunks 0 and 1.  Attention over rows 0-7 (logit 0) and
    48-51 (logit 1), V row i = i in column 0: (28 + 198 e) / (8 + 4 e).  With
    the prediction {0, 1}, chunk 0 hits and chunk 6 misses."""
    dd = require_gpu()
    announce("chunk closed form (ties, partial tail)")
    D, c, n, n_max = 64, 8, 52, 64
    qv = torch.zeros(D)
    qv[0] = 2.0
    q = torch.stack([qv, -qv])[None, None].contiguous().cuda()          # [1][1][2][D]
    keys = torch.zeros(1, 1, n_max, D)
    keys[0, 0, 48:52] = 2 * qv
    keys[0, 0, 52:] = 99.0                                              # padding
    vals = torch.zeros(1, 1, n_max, D)
    vals[0, 0, :, 0] = torch.arange(n_max, dtype=torch.float32)
    vals[0, 0, :, 1] = 1.0
    lens = torch.tensor([n], dtype=torch.int32).cuda()
    k_dev = keys.cuda()
    kh, vh = to_host(dd, keys), to_host(dd, vals)
    lm = dd.landmarks(k_dev, lens, c)
    ctx = dd.Context(ring_slots=1)
    res = ctx.layer_step([q], [k_dev], [kh], [vh], lens, 16, chunk=c, landmarks=[lm], dual=True)
    hot = ctx.layer_step([q], [k_dev], [kh], [vh], lens, 16, chunk=c, landmarks=[lm],
                         pred=[torch.tensor([[[0, 1]]], dtype=torch.int32).cuda()])
    torch.cuda.synchronize()
    assert res["cur"][0].cpu().tolist() == [[[0, 6]]]
    assert res["spec"][0].cpu().tolist() == [[[0, 1]]]
    e = float(np.e)
    out = res["out"][0][0, 0].cpu().numpy().astype(np.float64)
    assert abs(out[0] - (28 + 198 * e) / (8 + 4 * e)) < 1e-5
    assert abs(out[1] - 1.0) < 1e-6
    assert abs(float(res["lse"][0][0, 0]) - np.log(8 + 4 * e)) < 1e-5
    spec_out = res["out_spec"][0][0, 0].cpu().numpy().astype(np.float64)
    assert abs(spec_out[0] - (28 + 198 / e) / (8 + 4 / e)) < 1e-5
    assert hot["stats"][0].cpu().tolist() == [1, 1, 3]
    assert torch.equal(hot["out"][0], res["out"][0])
    ctx.close()


def test_chunk_layer_step_full_size_7b():
    """The 7B-shape layer at full size (32 heads x 32768 keys, k = 128) with
    8-key chunks, against the oracle on every head."""
    dd = require_gpu()
    w = gen.workload("llama7b_32k_layer")
    c = 8
    announce(f"chunk layer_step full size {w.name} chunk={c}")
    data = _stage(dd, w, c)
    ctx = dd.Context(ring_slots=2)
    cold = _run(ctx, w, data, c)
    hot = _run(ctx, w, data, c, pred=[s.clone() for s in cold["spec"]])
    for key in ("out", "lse", "cur", "spec"):
        assert torch.equal(hot[key][0], cold[key][0]), key
    d = data[0]
    lens = d["lens"].numpy()
    kst, vst = stored(d["k"]), stored(d["v"])
    ref = oracle.layer_step(d["q"].numpy(), kst, kst, vst, lens, w.k, w.dtype, chunk=c)
    B, H, ks = w.B, w.H, w.k // c
    nlen = np.repeat(-(-lens // c), H)
    cur = hot["cur"][0].cpu().numpy()
    parity.check_index_sets(cur.reshape(B * H, ks), ref["cur"].reshape(B * H, ks),
                            ref["scores"][:, :, 0].reshape(B * H, -1), nlen, ks)
    parity.check_index_sets(hot["spec"][0].cpu().numpy().reshape(B * H, ks),
                            ref["spec"].reshape(B * H, ks),
                            ref["scores"][:, :, 1].reshape(B * H, -1), nlen, ks)
    rows = oracle.chunk_rows(cur, lens, c)
    want, _ = oracle.masked_attention(d["q"][:, :, 0].numpy(), kst, vst, lens, rows, w.dtype)
    got = hot["out"][0].cpu().numpy().reshape(B * H, w.D)
    worst = parity.check_attention(got, want.reshape(B * H, w.D), np.zeros(B * H))
    ctx.close()
    print(f"worst relative attention error {worst:.2e}")


@pytest.mark.parametrize("name,kw,c,sel", [
    ("llama7b_32k_layer", dict(H=8, n_max=4096), 8, 0),
    ("llama7b_32k_layer", dict(H=8, n_max=4096), 8, 3),
    ("llama7b_32k_layer", dict(H=8, n_max=4096), 8, -1),   # all in the scoring kernel
    ("llama7b_32k_layer", dict(H=6, n_max=1000), 16, 0),
    ("llama7b_32k_layer", dict(H=32, n_max=32768), 8, 0),
    # ragged: some requests shorter than k rows (every chunk selected)
    ("hiconc_64", dict(B=4, H=2, n_max=4096, len_lo=1, len_hi=4096, k=128), 8, 0),
    ("hiconc_64", dict(B=4, H=2, n_max=4096, len_lo=1, len_hi=4096, k=128), 8, 5),
    ("llama7b_32k_layer", dict(H=8, n_max=4096), 2, 0),
    ("llama7b_32k_layer", dict(H=8, n_max=4096), 4, 3),
])
def test_selection_side_prefetch_matches_side_stream(name, kw, c, sel):
    """One layer with 256-byte V rows and k <= 128 rows: the prediction's rows
    are fetched by the selection kernel for the last slabs (by the layer's
    sizes: all slabs at the small shapes, 8 of 32 at the full 7B shape; or
    the last `sel`; none for -1) and by the scoring kernel for the rest.  Outputs,
    statistics and every slab's prefetched slot rows must equal those of a
    side-stream prefetch bit for bit, and the slot rows must hold the host
    rows of the prediction (zero rows for entries outside the cache, -1, and
    rows past the last key)."""
    dd = require_gpu()
    w = gen.workload(name).scaled(L=1, **kw)
    H, n_max = w.H, w.n_max
    announce(f"selection-side prefetch {name} {kw} chunk={c} slabs={sel}")
    data = _stage(dd, w, c)
    B, ks, k = w.B, w.k // c, w.k
    nc = -(-n_max // c)
    eb = w.elem_bytes
    nbytes = dd.ring_bytes(1, B, H, w.D, k, dd.kv_dtype(data[0]["k_dev"]))
    ctx0 = dd.Context(ring_slots=1)
    cold = _run(ctx0, w, data, c)
    ctx0.close()
    p = cold["spec"][0].cpu().numpy().copy()
    rng = np.random.default_rng(5 + c)
    for b in range(B):
        for h in range(H):
            p[b, h] = rng.permutation(p[b, h])
    p[0, 0, 0] = -1
    p[0, H - 1, 1] = nc + 3         # past the cache
    p[B - 1, H // 2, 2] = nc - 1    # the last, partial chunk
    pred = [torch.from_numpy(p).cuda()]
    out = {}
    for mode in ("fused", "side"):
        ctx = dd.Context(ring_slots=1, prefetch=mode, select_prefetch_slabs=sel)
        ring = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda")
        out[mode] = (_run(ctx, w, data, c, pred=pred, ring=ring), ring.cpu().numpy())
        ctx.close()
    (fr, fring), (sr, sring) = out["fused"], out["side"]
    for key in ("out", "lse", "cur", "spec", "stats"):
        got, want = fr[key], sr[key]
        if isinstance(got, list):
            got, want = got[0], want[0]
        assert torch.equal(got, want), key
    vplane = lambda raw: raw[nbytes // 2:].reshape(B, H, 2 * k, w.D * eb)
    fv, sv = vplane(fring), vplane(sring)
    assert np.array_equal(fv[:, :, :k], sv[:, :, :k]), "prediction rows differ"
    vh = stored(data[0]["v_host"]).view(np.uint8).reshape(B, H, n_max, w.D * eb)
    zero = np.zeros(w.D * eb, np.uint8)
    for b in range(B):
        for h in range(H):
            for j in range(ks):
                e = int(p[b, h, j])
                for i in range(c):
                    r = e * c + i
                    want = vh[b, h, r] if 0 <= e < nc and r < n_max else zero
                    assert np.array_equal(fv[b, h, j * c + i], want), (b, h, j, i)
