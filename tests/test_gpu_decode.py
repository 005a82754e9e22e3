"""The multi-step decode loop: dd_kv_append (rows and chunk landmarks) and
several real steps of dd_layer_step with the prediction carried across
steps, against the oracle's loop (append_rows, then layer_step with the
previous step's speculated set)."""
import numpy as np
import pytest
import torch

import gen
import oracle
from tests import parity
from tests.gpu_util import announce, require_gpu, stored, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,kw,chunk", [
    ("tiny", dict(H=3, n_max=300, len_lo=200, len_hi=200), 8),
    ("hiconc_64", dict(B=3, H=2, n_max=700, len_lo=100, len_hi=699, k=64), 16),
    ("llama7b_32k_layer", dict(B=2, H=2, n_max=512, len_lo=400, len_hi=400), 0),
])
def test_kv_append_rows_and_landmarks(name, kw, chunk):
    """Row lens[b] of the device keys and both host planes becomes the new
    row, nothing else changes, lens_out = lens + 1 (a full request stays),
    and the updated landmarks equal a rebuild of the grown cache bit for bit."""
    dd = require_gpu()
    w = gen.workload(name).scaled(**kw)
    announce(f"kv_append {name} {kw} chunk={chunk}")
    lay = gen.make_layer(w, 0, "cpu")
    lens = lay["lens"].clone()
    if w.B > 1:
        lens[-1] = w.n_max  # full: left unchanged
    k_dev = lay["k"].cuda()
    kh, vh = to_host(dd, lay["k"]), to_host(dd, lay["v"])
    lens_d = lens.cuda()
    lm = dd.landmarks(k_dev, lens_d, chunk) if chunk else None
    _, nk, nv = gen.decode_step_inputs(w, 0, 1, lay["q"])
    lens_out = torch.full_like(lens_d, -7)
    dd.kv_append(k_dev, kh, vh, nk.cuda(), nv.cuda(), lens_d, lens_out=lens_out, chunk=chunk,
                 landmarks=lm)
    torch.cuda.synchronize()
    want_k, want_lens = oracle.append_rows(stored(lay["k"]), lens.numpy(), stored(nk))
    want_v, _ = oracle.append_rows(stored(lay["v"]), lens.numpy(), stored(nv))
    assert lens_out.cpu().numpy().tolist() == want_lens.tolist()
    assert np.array_equal(stored(k_dev), want_k)
    assert np.array_equal(stored(kh), want_k)
    assert np.array_equal(stored(vh), want_v)
    if chunk:
        rebuilt = dd.landmarks(k_dev, lens_out, chunk)
        torch.cuda.synchronize()
        assert torch.equal(lm, rebuilt)


def _check_step(w, res, ref, lens, chunk, q_cur, kst, vst):
    """Sets within the tie band of the oracle's scores; attention against the
    oracle over the GPU's own (valid) set."""
    B, H = w.B, w.H
    c = max(chunk, 1)
    ks = w.k // c
    nlen = np.repeat(-(-lens // c), H)
    s = ref["scores"]
    cur = res["cur"][0].cpu().numpy()
    spec = res["spec"][0].cpu().numpy()
    d_cur = parity.check_index_sets(cur.reshape(B * H, ks), ref["cur"].reshape(B * H, ks),
                                    s[:, :, 0].reshape(B * H, -1), nlen, ks)
    d_spec = parity.check_index_sets(spec.reshape(B * H, ks), ref["spec"].reshape(B * H, ks),
                                     s[:, :, 1].reshape(B * H, -1), nlen, ks)
    rows = oracle.chunk_rows(cur, lens, c) if chunk else cur
    want, _ = oracle.masked_attention(q_cur, kst, vst, lens, rows, w.dtype)
    got = res["out"][0].cpu().numpy().reshape(B * H, w.D)
    parity.check_attention(got, want.reshape(B * H, w.D), np.zeros(B * H))
    return not d_cur and not d_spec


@pytest.mark.parametrize("name,kw,chunk,qbuf", [
    ("llama7b_32k_layer", dict(B=2, H=2, n_max=4096, len_lo=3000, len_hi=4000), 0, False),
    ("llama7b_32k_layer", dict(B=2, H=2, n_max=4096, len_lo=3000, len_hi=4000), 8, False),
    ("tiny", dict(n_max=2048, len_lo=1500, len_hi=1500), 0, False),
    # the queries written into one buffer each step: the decoder reuses its
    # prepared steps (and its two output sets) from the third step on
    ("llama7b_32k_layer", dict(B=2, H=2, n_max=4096, len_lo=3000, len_hi=4000), 0, True),
    ("llama7b_32k_layer", dict(B=2, H=2, n_max=4096, len_lo=3000, len_hi=4000), 8, True),
    # requests growing from below k (every key, or every chunk, selected) past it
    ("llama7b_32k_layer", dict(B=3, H=2, n_max=512, len_lo=125, len_hi=128), 0, False),
    ("llama7b_32k_layer", dict(B=3, H=2, n_max=512, len_lo=123, len_hi=128), 8, False),
])
def test_decode_loop_matches_oracle(name, kw, chunk, qbuf):
    """Four real steps: at each, the GPU's sets, attention and (where the sets
    agree) statistics match the oracle's loop on the same grown cache."""
    dd = require_gpu()
    w = gen.workload(name).scaled(**kw)
    announce(f"decode loop {name} {kw} chunk={chunk}")
    lay = gen.make_layer(w, 0, "cpu")
    lens = lay["lens"].numpy().astype(np.int64)
    k_dev = lay["k"].cuda()
    kh, vh = to_host(dd, lay["k"]), to_host(dd, lay["v"])
    ctx = dd.Context(ring_slots=2)
    dec = dd.Decoder(ctx, [k_dev], [kh], [vh], lay["lens"].cuda(), w.k, chunk=chunk)
    kst, vst = stored(lay["k"]), stored(lay["v"])
    q = lay["q"]
    # step 0: the layer as drawn, no prediction
    res = ctx.layer_step([q.cuda()], [k_dev], [kh], [vh], dec.lens, w.k, chunk=chunk,
                         landmarks=dec.landmarks)
    dec.pred = [s.clone() for s in res["spec"]]
    ref = oracle.layer_step(q.numpy(), kst, kst, vst, lens, w.k, w.dtype, chunk=chunk)
    same = _check_step(w, res, ref, lens, chunk, q[:, :, 0].numpy(), kst, vst)
    qd = q.cuda()
    prev = None
    for t in range(1, 5):
        q, nk, nv = gen.decode_step_inputs(w, 0, t, q)
        if qbuf:
            qd.copy_(q)
        else:
            qd = q.cuda()
        res = dec.step([qd], [nk.cuda()], [nv.cuda()])
        torch.cuda.synchronize()
        if prev is not None:  # the previous step's results are still intact
            assert torch.equal(prev[1], prev[0]["out"][0]), t
        prev = (res, res["out"][0].clone())
        kst, _ = oracle.append_rows(kst, lens, stored(nk))
        vst, lens = oracle.append_rows(vst, lens, stored(nv))
        assert dec.lens.cpu().numpy().tolist() == lens.tolist()
        ref = oracle.layer_step(q.numpy(), kst, kst, vst, lens, w.k, w.dtype, pred=ref["spec"],
                                chunk=chunk)
        same_now = _check_step(w, res, ref, lens, chunk, q[:, :, 0].numpy(), kst, vst)
        if same and same_now:  # the prediction (the previous spec) was the oracle's too
            assert res["stats"][0].cpu().numpy().tolist() == ref["stats"].tolist(), t
        same = same_now
    ctx.close()


@pytest.mark.parametrize("case", ["perfect", "dominant"])
def test_decode_loop_recall_closed_forms(case):
    """perfect: speculation equals the next token and new keys are zero (below
    the k-th score), so every true set was predicted (no misses).  dominant:
    each new key is 8 q_cur, above every planted key, so it joins every true
    set unpredicted: exactly one miss per (b, h)."""
    dd = require_gpu()
    w = gen.workload("llama7b_32k_layer").scaled(B=2, H=2, n_max=3000, rho=1.0, rho_c=0.0,
                                                 len_lo=2900, len_hi=2900)
    announce(f"decode loop recall {case}")
    lay = gen.make_layer(w, 0, "cpu")
    k_dev = lay["k"].cuda()
    kh, vh = to_host(dd, lay["k"]), to_host(dd, lay["v"])
    ctx = dd.Context(ring_slots=2)
    dec = dd.Decoder(ctx, [k_dev], [kh], [vh], lay["lens"].cuda(), w.k)
    q = lay["q"]
    res = ctx.layer_step([q.cuda()], [k_dev], [kh], [vh], dec.lens, w.k)
    dec.pred = [s.clone() for s in res["spec"]]
    for t in range(1, 4):
        q, nk, nv = gen.decode_step_inputs(w, 0, t, q)
        if case == "dominant":
            nk = (8.0 * q[:, :, 0]).to(nk.dtype).contiguous()
        else:
            nk = torch.zeros_like(nk)
        res = dec.step([q.cuda()], [nk.cuda()], [nv.cuda()])
        st = res["stats"][0].cpu().numpy().tolist()
        BH = w.B * w.H
        if case == "perfect":
            assert st[0] == 0 and st[1] == BH * w.k, (t, st)
        else:
            assert st[0] == BH and st[1] == BH * (w.k - 1), (t, st)
            n = int(dec.lens[0].item())
            assert torch.all(res["cur"][0][:, :, -1] == n - 1)
    ctx.close()
