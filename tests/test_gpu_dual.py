"""Dual-token attention in the layer step: the speculated query attends over
the same selected rows as the current one (each K/V row read once for both),
against the oracle's layer_step(dual=True); the current query's outputs stay
bitwise the same."""
import numpy as np
import pytest
import torch

import gen
import oracle
from tests import parity
from tests.gpu_util import announce, require_gpu, stored, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,kw,chunk", [
    ("tiny", {}, 0),
    ("llama7b_32k_layer", dict(H=4, n_max=8192), 0),
    ("llama13b_128k", dict(L=1, B=1, H=2, n_max=40000, k=2048), 0),   # long rows (not cached)
    ("hiconc_64", dict(B=3, H=2, n_max=20000, len_lo=300, len_hi=20000, k=512), 16),
    ("llama7b_32k_layer", dict(H=2, n_max=4096), 8),
    # an empty request (both outputs zero, both lse -inf) and requests of
    # 1, k - 1 and k + 1 keys
    ("llama7b_32k_layer", dict(B=4, H=2, n_max=3000, k=128, lens=[0, 1, 127, 129]), 0),
    ("llama7b_32k_layer", dict(B=4, H=2, n_max=3000, k=128, lens=[0, 1, 127, 1029]), 8),
])
def test_dual_token_attention(name, kw, chunk):
    dd = require_gpu()
    kw = dict(kw)
    fixed = kw.pop("lens", None)
    w = gen.workload(name).scaled(**kw)
    announce(f"dual-token attention {name} {kw} lens={fixed} chunk={chunk}")
    lay = gen.make_layer(w, 0, "cpu")
    if fixed is not None:
        lay["lens"] = torch.tensor(fixed, dtype=torch.int32)
    q, k_dev = lay["q"].cuda(), lay["k"].cuda()
    kh, vh = to_host(dd, lay["k"]), to_host(dd, lay["v"])
    lens = lay["lens"].cuda()
    lm = [dd.landmarks(k_dev, lens, chunk)] if chunk else None
    ctx = dd.Context(ring_slots=2)
    args = ([q], [k_dev], [kh], [vh], lens, w.k)
    cold = ctx.layer_step(*args, chunk=chunk, landmarks=lm)
    pred = [s.clone() for s in cold["spec"]]
    one = ctx.layer_step(*args, pred=pred, chunk=chunk, landmarks=lm)
    two = ctx.layer_step(*args, pred=pred, chunk=chunk, landmarks=lm, dual=True)
    torch.cuda.synchronize()
    for key in ("out", "lse", "cur", "spec", "stats"):
        a, b = one[key], two[key]
        assert torch.equal(a if key == "stats" else a[0], b if key == "stats" else b[0]), key
    B, H = w.B, w.H
    lens_np = lay["lens"].numpy()
    cur = two["cur"][0].cpu().numpy()
    rows = oracle.chunk_rows(cur, lens_np, chunk) if chunk else cur
    kst, vst = stored(lay["k"]), stored(lay["v"])
    want, want_lse = oracle.masked_attention(lay["q"][:, :, 1].numpy(), kst, vst, lens_np, rows,
                                             w.dtype)
    got = two["out_spec"][0].cpu().numpy().reshape(B * H, w.D)
    worst = parity.check_attention(got, want.reshape(B * H, w.D), np.zeros(B * H))
    got_lse = two["lse_spec"][0].cpu().numpy().reshape(-1).astype(np.float64)
    ref_lse = want_lse.reshape(-1)
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(got_lse), empty)
    assert np.all(np.abs(got_lse[~empty] - ref_lse[~empty])
                  <= 1e-4 * np.maximum(1.0, np.abs(ref_lse[~empty])))
    if empty.any():
        assert np.all(got[empty] == 0)
    ctx.close()
    print(f"worst relative error of the speculated query's attention {worst:.2e}")
