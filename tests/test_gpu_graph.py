"""The layer step captured in a HIP graph: every replay, with eager steps and
synchronizations in between, must reproduce the eager result bitwise."""
import pytest
import torch

import gen
from tests.gpu_util import announce, require_gpu, to_host

pytestmark = pytest.mark.gpu


def test_layer_step_graph_replays_match_eager():
    dd = require_gpu()
    announce("layer_step graph capture and replay")
    w = gen.workload("llama7b_32k_layer").scaled(L=2, B=2, H=4, n_max=8192, k=256)
    layers = [gen.make_layer(w, l, "cpu") for l in range(w.L)]
    q = [d["q"].cuda() for d in layers]
    kd = [d["k"].cuda() for d in layers]
    kh = [to_host(dd, d["k"]) for d in layers]
    vh = [to_host(dd, d["v"]) for d in layers]
    lens = layers[0]["lens"].cuda()
    B, H, D, k = w.B, w.H, w.D, w.k
    ctx = dd.Context(ring_slots=2)
    cur = [torch.empty(B, H, k, dtype=torch.int32, device="cuda") for _ in range(w.L)]
    spec = [torch.empty(B, H, k, dtype=torch.int32, device="cuda") for _ in range(w.L)]
    out = [torch.empty(B, H, D, device="cuda") for _ in range(w.L)]
    lse = [torch.empty(B, H, device="cuda") for _ in range(w.L)]
    stats = torch.zeros(w.L, 3, dtype=torch.int64, device="cuda")
    ring = torch.empty(dd.ring_bytes(2, B, H, D, k, 1), dtype=torch.uint8, device="cuda")
    ws = torch.empty(dd.layer_step_workspace_bytes(B, H, D, w.n_max, k), dtype=torch.uint8, device="cuda")

    def step(pred):
        ctx.layer_step(q, kd, kh, vh, lens, k, pred=pred, cur=cur, spec=spec, out=out, lse=lse,
                       stats=stats, ring=ring, ws=ws)

    step(None)
    pred = [s.clone() for s in spec]
    step(pred)
    torch.cuda.synchronize()
    ref = [o.clone() for o in out] + [x.clone() for x in cur] + [stats.clone()]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(pred)
    for rep in range(4):
        for o in out:
            o.zero_()
        stats.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in out] + [x.clone() for x in cur] + [stats.clone()]
        assert all(torch.equal(a, b) for a, b in zip(got, ref)), f"replay {rep} differs"
        step(None)  # eager work between replays
        torch.cuda.synchronize()
    ctx.close()
