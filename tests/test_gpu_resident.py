"""Rows kept across decode steps (dd_layer_step_args.resident): a decode
loop where every layer keeps its own two slots gives, bit for bit, the sets,
outputs and hit / miss counts of the shared ring, and reads over the host
link exactly the rows the oracle's resident_fetches counts (whenever the
GPU's sets are the oracle's)."""
import numpy as np
import pytest
import torch

import gen
import oracle
from tests.gpu_util import announce, require_gpu, stored, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("prefetch", ["auto", "side"])
@pytest.mark.parametrize("name,kw,short", [
    ("llama7b_32k_layer", dict(B=2, H=2, n_max=4096, len_lo=3000, len_hi=4000), None),
    ("llama7b_32k_step", dict(L=2, B=2, H=2, n_max=4096, len_lo=3000, len_hi=4000, k=256), None),
    ("tiny", dict(n_max=2048, len_lo=1500, len_hi=1500), None),
    # request 0 shorter than k: its sets and predictions carry -1 padding
    ("llama7b_32k_layer", dict(B=2, H=2, n_max=4096, len_lo=3000, len_hi=4000), 60),
    # request 0 empty before the first append: it grows from 1 key
    ("llama7b_32k_layer", dict(B=2, H=2, n_max=4096, len_lo=3000, len_hi=4000), 0),
    # the other row sizes of the copy queues: 128 B (bf16, D = 64), 512 B (fp32, D = 128)
    ("llama7b_32k_layer", dict(B=2, H=2, D=64, n_max=4096, len_lo=3000, len_hi=4000), None),
    ("tiny", dict(H=4, D=128, n_max=2048, len_lo=1500, len_hi=1500), None),
])
def test_resident_decode_loop(name, kw, short, prefetch):
    dd = require_gpu()
    w = gen.workload(name).scaled(**kw)
    L = w.L
    announce(f"resident decode loop {name} {kw} short={short} prefetch={prefetch}")
    layers = [gen.make_layer(w, l, "cpu") for l in range(L)]
    if short is not None:  # rows past the new length are filler
        for lay in layers:
            lay["lens"][0] = short

    def caches():
        return ([lay["k"].cuda() for lay in layers], [to_host(dd, lay["k"]) for lay in layers],
                [to_host(dd, lay["v"]) for lay in layers])

    # auto: the kept-rows prefetch rides in each layer's scoring kernel;
    # side: it runs on the context's side stream.
    ctx = dd.Context(ring_slots=2, prefetch=prefetch)
    lens = layers[0]["lens"].cuda()
    plain = dd.Decoder(ctx, *caches(), lens, w.k)
    keep = dd.Decoder(ctx, *caches(), lens, w.k, resident=True)
    q = [lay["q"] for lay in layers]
    kst = [stored(lay["k"]) for lay in layers]
    vst = [stored(lay["v"]) for lay in layers]
    lens_np = layers[0]["lens"].numpy().astype(np.int64)
    pred_ref = [None] * L       # the oracle's prediction of each layer
    held = [None] * L           # the oracle's (prediction, misses) of the previous step
    agree = True                # the GPU's sets have been the oracle's at every step
    for t in range(1, 6):
        if t == 4:              # a reset mid-sequence: nothing is held any more
            keep._reset = True
            held = [None] * L
        new = [gen.decode_step_inputs(w, l, t, q[l]) for l in range(L)]
        q = [x[0] for x in new]
        args = ([x.cuda() for x in q], [x[1].cuda() for x in new], [x[2].cuda() for x in new])
        a = plain.step(*args)
        b = keep.step(*args)
        torch.cuda.synchronize()
        for l in range(L):
            for key in ("cur", "spec", "out", "lse"):
                assert torch.equal(a[key][l], b[key][l]), (t, l, key)
        sa, sb = a["stats"].cpu().numpy(), b["stats"].cpu().numpy()
        assert np.array_equal(sa[:, :2], sb[:, :2]), t
        assert sb[:, 2].sum() <= sa[:, 2].sum(), t
        # the oracle's loop: append, then the step with the previous spec set
        for l in range(L):
            kst[l], _ = oracle.append_rows(kst[l], lens_np, stored(new[l][1]))
            vst[l], grown = oracle.append_rows(vst[l], lens_np, stored(new[l][2]))
        lens_np = grown
        want = np.zeros(L, dtype=np.int64)
        for l in range(L):
            ref = oracle.layer_step(q[l].numpy(), kst[l], kst[l], vst[l], lens_np, w.k, w.dtype,
                                    pred=pred_ref[l])
            agree = agree and np.array_equal(b["cur"][l].cpu().numpy(), ref["cur"]) \
                and np.array_equal(b["spec"][l].cpu().numpy(), ref["spec"])
            pp, pm = held[l] if held[l] is not None else (None, None)
            want[l] = oracle.resident_fetches(pp, pm, pred_ref[l], ref["miss"], w.n_max).sum()
            held[l] = (pred_ref[l], ref["miss"])
            pred_ref[l] = ref["spec"]
        if agree:
            assert sb[:, 2].tolist() == want.tolist(), (t, sb[:, 2].tolist(), want.tolist())
        print(f"step {t}: host rows {int(sb[:, 2].sum())} kept-rows mode, "
              f"{int(sa[:, 2].sum())} ring; sets agree with the oracle: {agree}")
    ctx.close()


def test_resident_argument_errors():
    dd = require_gpu()
    announce("resident argument errors")
    w = gen.workload("tiny").scaled(n_max=512, len_lo=400, len_hi=400)
    lay = gen.make_layer(w, 0, "cpu")
    q, kd = lay["q"].cuda(), lay["k"].cuda()
    kh, vh = to_host(dd, lay["k"]), to_host(dd, lay["v"])
    lens = lay["lens"].cuda()
    B, H, n_max, D = kd.shape
    nb = dd.resident_bytes(1, B, H, D, n_max, w.k, dd.kv_dtype(kd))
    state = torch.empty(nb, dtype=torch.uint8, device="cuda")
    ctx = dd.Context(ring_slots=2)
    with pytest.raises(Exception, match="parity"):
        ctx.layer_step([q], [kd], [kh], [vh], lens, w.k, resident=state, parity=2, reset=True)
    lm = dd.landmarks(kd, lens, 8)
    with pytest.raises(Exception, match="chunk"):
        ctx.layer_step([q], [kd], [kh], [vh], lens, w.k, chunk=8, landmarks=[lm], resident=state,
                       reset=True)
    with pytest.raises(Exception, match="too small"):
        ctx.layer_step([q], [kd], [kh], [vh], lens, w.k, resident=state[:nb // 2], reset=True)
    hctx = dd.Context(ring_slots=2, k_rows="host")
    with pytest.raises(Exception, match="k_dev|DD_KROWS_DEVICE"):
        hctx.layer_step([q], [kd], [kh], [vh], lens, w.k, resident=state, reset=True)
    ctx.close()
    hctx.close()


def test_resident_step_graph_replays_match_eager():
    """A kept-rows step captured in a HIP graph (the prefetch rides in the
    scoring kernel): every replay, with eager work in between, reproduces the
    eager step's sets, outputs and host-row counts bitwise.  The state of the
    kept rows is restored before each run of the step (eagerly, between
    replays), so every run starts from the state the previous step left."""
    dd = require_gpu()
    announce("resident layer step graph capture and replay")
    w = gen.workload("llama7b_32k_step").scaled(L=2, B=2, H=4, n_max=8192, len_lo=6000,
                                                len_hi=8000, k=256)
    layers = [gen.make_layer(w, l, "cpu") for l in range(w.L)]
    kd = [d["k"].cuda() for d in layers]
    kh = [to_host(dd, d["k"]) for d in layers]
    vh = [to_host(dd, d["v"]) for d in layers]
    lens = layers[0]["lens"].cuda()
    B, H, D, k, n_max = w.B, w.H, w.D, w.k, w.n_max
    ctx = dd.Context(ring_slots=2)
    state = torch.empty(dd.resident_bytes(w.L, B, H, D, n_max, k, dd.kv_dtype(kd[0])),
                        dtype=torch.uint8, device="cuda")
    qs = [[d["q"].cuda() for d in layers]]
    for t in range(1, 3):  # queries of two later steps
        qs.append([gen.decode_step_inputs(w, l, t, qs[-1][l].cpu())[0].cuda() for l in range(w.L)])
    cur = [torch.empty(B, H, k, dtype=torch.int32, device="cuda") for _ in range(w.L)]
    spec = [torch.empty_like(c) for c in cur]
    out = [torch.empty(B, H, D, device="cuda") for _ in range(w.L)]
    lse = [torch.empty(B, H, device="cuda") for _ in range(w.L)]
    stats = torch.zeros(w.L, 3, dtype=torch.int64, device="cuda")

    def step(q, pred, parity, reset):
        ctx.layer_step(q, kd, kh, vh, lens, k, pred=pred, cur=cur, spec=spec, out=out, lse=lse,
                       stats=stats, resident=state, parity=parity, reset=reset)

    step(qs[0], None, 0, True)
    p1 = [s.clone() for s in spec]
    step(qs[1], p1, 1, False)
    p2 = [s.clone() for s in spec]
    before = state.clone()     # what the captured step starts from
    step(qs[2], p2, 0, False)  # the step that is captured, run eagerly first
    torch.cuda.synchronize()
    ref = [o.clone() for o in out] + [x.clone() for x in cur] + [x.clone() for x in spec] \
        + [stats.clone()]
    assert int(stats[:, 2].sum()) > 0 and int(stats[:, 0].sum()) > 0

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(qs[2], p2, 0, False)
    scratch = torch.empty(1 << 20, device="cuda")
    for rep in range(4):
        for o in out:
            o.zero_()
        stats.zero_()
        state.copy_(before)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in out] + [x.clone() for x in cur] + [x.clone() for x in spec] \
            + [stats.clone()]
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), f"replay {rep} differs"
        scratch.normal_()  # eager work between replays
        torch.cuda.synchronize()
    ctx.close()
