"""dd_sparse_attn_noalloc against dd_sparse_attn: the entry point for
callers that cannot allocate keeps its chunk partials in the library's own
scratch array and must give the same bits as the workspace entry point.

Two calls in a row share the scratch (the second with a smaller input, so
stale partials from the first are left in it), then a size whose partials
exceed the scratch is refused with nothing enqueued."""
import pytest
import torch

import gen
from tests.gpu_util import announce, require_gpu

pytestmark = pytest.mark.gpu


def _inputs(B, H, k, m, D, dtype, seed):
    q = gen.random_tensor((B, H, 2, D), seed, torch.float32).cuda()
    kr = gen.random_tensor((B, H, m, D), seed + 1, dtype).cuda()
    vr = gen.random_tensor((B, H, m, D), seed + 2, dtype).cuda()
    pos = gen.random_positions(B * H, k, m, seed + 3, invalid_frac=0.05).reshape(B, H, k).cuda()
    cnt = torch.randint(0, k + 1, (B, H), generator=torch.Generator().manual_seed(seed + 4),
                        dtype=torch.int32).cuda()
    return q, kr, vr, pos, cnt


def _both(dd, q, kr, vr, pos, cnt, k):
    B, H, m, D = kr.shape
    ref_out, ref_lse = dd.sparse_attn(q, kr, vr, pos=pos, cnt=cnt, k=k)
    out = torch.full((B, H, D), float("nan"), device="cuda")
    lse = torch.full((B, H), float("nan"), device="cuda")
    dd.sparse_attn_noalloc(q, kr, vr, out, lse, pos=pos, cnt=cnt, k=k)
    torch.cuda.synchronize()
    return out, lse, ref_out, ref_lse


def test_noalloc_matches_workspace_entry_point():
    dd = require_gpu()
    # 1: 8 x 32 (b, h), k = 1024 (8 chunks, partials in the scratch: 1.1 MB)
    # 2: smaller, 2 x 8 (b, h), k = 512 (4 chunks), fp32 rows, D = 64
    # 3: 16 x 32 = 512 (b, h), k = 2048: one workgroup per (b, h), no partials
    for case, (B, H, k, m, D, dtype) in enumerate([(8, 32, 1024, 1400, 128, torch.bfloat16),
                                                   (2, 8, 512, 700, 64, torch.float32),
                                                   (16, 32, 2048, 2048, 128, torch.bfloat16)]):
        announce(f"noalloc attention call {case}: B={B} H={H} k={k} m={m} D={D} {dtype}")
        need = dd.attn_workspace_bytes(B, H, k, D)
        q, kr, vr, pos, cnt = _inputs(B, H, k, m, D, dtype, seed=100 + 10 * case)
        out, lse, ref_out, ref_lse = _both(dd, q, kr, vr, pos, cnt, k)
        assert torch.equal(out, ref_out), case
        assert torch.equal(lse, ref_lse), case
        print(f"call {case}: bitwise equal ({need} bytes of partials)")


def test_noalloc_refuses_sizes_beyond_its_scratch():
    dd = require_gpu()
    # 511 (b, h) x 32 chunks x 130 floats = 8.5 MB > 4 MiB
    B, H, k, m, D = 1, 511, 4096, 4096, 128
    announce("noalloc attention: oversize request is refused")
    q = torch.zeros(B, H, D, device="cuda")
    kr = torch.zeros(B, H, m, D, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros(B, H, D, device="cuda")
    with pytest.raises(dd.DDError) as e:
        dd.sparse_attn_noalloc(q, kr, kr, out, k=k)
    assert e.value.code == 3
    assert "scratch" in str(e.value)
