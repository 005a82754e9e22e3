"""Parity of each HIP stage (score, top-k, gather, sparse attention) with the
CPU oracle, through the C ABI, on seeded inputs that span several tiles,
ragged tails and the degenerate cases."""
import numpy as np
import pytest
import torch

import gen
import oracle
from tests import parity
from tests.gpu_util import announce, require_gpu, stored, to_host

pytestmark = pytest.mark.gpu


# --------------------------------------------------------------------------- score
SCORE_CASES = [
    # dtype, D, Q, n_max, lens
    ("bf16", 128, 2, 4096, [4096, 2049, 0]),
    ("bf16", 128, 1, 65, [65, 64, 63]),
    ("bf16", 64, 2, 4095, [4095, 1, 4000]),
    ("f32", 64, 2, 4096, [4096, 17, 3000]),
    ("f32", 128, 2, 1000, [1000, 999, 1]),
    ("f32", 128, 1, 64, [64, 5, 0]),
    ("bf16", 64, 1, 1, [1, 0, 1]),
    ("bf16", 128, 2, 40961, [40961, 20000, 513]),
]


@pytest.mark.parametrize("dtype,D,Q,n_max,lens", SCORE_CASES)
def test_score_logits(dtype, D, Q, n_max, lens):
    dd = require_gpu()
    announce(f"score logits {dtype} D={D} Q={Q} n_max={n_max} lens={lens}")
    B, H = len(lens), 3
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    keys = gen.random_tensor((B, H, n_max, D), seed=n_max + D, dtype=td)
    q = gen.random_tensor((B, H, Q, D), seed=7 + Q, scale=1.5)
    lens_t = torch.tensor(lens, dtype=torch.int32)
    got = dd.score(q.cuda(), keys.cuda(), lens_t.cuda()).cpu().numpy()
    torch.cuda.synchronize()
    ref = oracle.scaled_logits(q.numpy(), stored(keys), lens_t.numpy(), dtype)
    rows_g = got.reshape(B * H * Q, n_max)
    rows_r = ref.reshape(B * H * Q, n_max)
    row_lens = np.repeat(np.array(lens), H * Q)
    parity.check_logits(rows_g, rows_r, row_lens)


@pytest.mark.parametrize("dtype,D,n_max,lens", [("bf16", 128, 4096, [4096, 333]),
                                                 ("f32", 64, 700, [700, 1])])
def test_score_alpha(dtype, D, n_max, lens):
    dd = require_gpu()
    announce(f"score alpha {dtype} D={D} n_max={n_max}")
    B, H, Q = len(lens), 2, 2
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    keys = gen.random_tensor((B, H, n_max, D), seed=5, dtype=td)
    q = gen.random_tensor((B, H, Q, D), seed=6, scale=2.0)
    lens_t = torch.tensor(lens, dtype=torch.int32)
    got = dd.score(q.cuda(), keys.cuda(), lens_t.cuda(), kind="alpha").cpu().numpy().astype(np.float64)
    s = oracle.scaled_logits(q.numpy(), stored(keys), lens_t.numpy(), dtype)
    ref = oracle.attention_weights(s, lens_t.numpy())
    big = ref >= 1e-30
    rel = np.abs(got - ref)[big] / ref[big]
    assert rel.max() <= 1e-3, rel.max()
    assert np.all(np.abs(got - ref)[~big] <= 1e-33)
    for b, n in enumerate(lens):
        assert np.all(got[b, :, :, n:] == 0.0)
        assert np.allclose(got[b, :, :, :n].sum(-1), 1.0, atol=1e-4)


# --------------------------------------------------------------------------- top-k
def _topk_case(kind, rows_shape, n_max, seed):
    B, H, Q = rows_shape
    if kind == "normal":
        s = gen.random_tensor((B, H, Q, n_max), seed=seed, scale=3.0)
    elif kind == "ties":
        s = gen.tie_scores(B * H * Q, n_max, seed=seed, nvalues=5).reshape(B, H, Q, n_max)
    elif kind == "signedzero":
        # 20 positive keys, then 30 entries of +0 and 30 of -0 at random
        # places over a negative background: the k-th largest is a zero
        s = -1.0 - gen.random_tensor((B, H, Q, n_max), seed=seed, scale=1.0).abs()
        flat = s.view(B * H * Q, n_max)
        idx = gen.random_positions(B * H * Q, min(80, n_max), n_max, seed + 1).long()
        flat.scatter_(1, idx[:, :20], 1.0 + gen.random_tensor((B * H * Q, 20), seed=seed + 2).abs())
        flat.scatter_(1, idx[:, 20:50], 0.0)
        flat.scatter_(1, idx[:, 50:80], -0.0)
    elif kind == "allzero":
        s = torch.zeros(B, H, Q, n_max)
        s[..., ::2] = -0.0
    else:  # planted: a few large values over a tie-heavy background
        s = gen.tie_scores(B * H * Q, n_max, seed=seed, nvalues=3).reshape(B, H, Q, n_max)
        idx = gen.random_positions(B * H * Q, min(40, n_max), n_max, seed + 1).long()
        s.view(B * H * Q, n_max).scatter_(1, idx, 100.0)
    return s.contiguous()


TOPK_CASES = [
    # kind, (B, H, Q), n_max, lens, k
    ("normal", (2, 2, 2), 4096, [4096, 3000], 64),
    ("normal", (3, 1, 2), 65, [65, 64, 63], 7),
    ("normal", (2, 2, 1), 1000, [1000, 5], 128),
    ("normal", (1, 2, 2), 32768, [32768], 1024),
    ("normal", (2, 1, 2), 40961, [40961, 36001], 2048),
    ("normal", (1, 2, 1), 131072, [131072], 2048),
    ("normal", (2, 2, 2), 300, [300, 299], 300),
    ("normal", (1, 1, 1), 10, [10], 4096),
    ("ties", (2, 2, 2), 4096, [4096, 4000], 100),
    ("ties", (1, 2, 2), 40961, [40961], 3000),
    ("ties", (2, 1, 1), 37, [37, 36], 5),
    ("allzero", (1, 1, 2), 5000, [5000], 33),
    # +0 and -0 (equal scores, one key) tied at the k-th largest: the
    # lower index wins whatever the sign
    ("signedzero", (2, 2, 2), 8192, [8192, 5000], 40),
    ("signedzero", (2, 2, 2), 8192, [8192, 5000], 30),
    ("signedzero", (1, 2, 2), 40961, [40961], 40),
    ("planted", (2, 2, 1), 20000, [20000, 16384], 40),
    ("planted", (1, 1, 2), 70000, [70000], 39),
    ("normal", (3, 1, 1), 50, [0, 1, 2], 1),
    # shapes of the split path: several 8192-key segments, ragged and unaligned rows
    ("normal", (2, 4, 2), 32768, [32768, 20001], 128),
    ("planted", (1, 2, 2), 65536, [65536], 200),
    ("normal", (1, 1, 2), 65536, [50000], 256),
    ("normal", (1, 2, 1), 9999, [9999], 50),
    ("normal", (2, 2, 2), 20000, [20000, 777], 1),
    ("ties", (1, 2, 2), 5000, [5000], 1),
]


@pytest.mark.parametrize("kind,shape,n_max,lens,k", TOPK_CASES)
def test_topk_exact(kind, shape, n_max, lens, k):
    """Both sides rank the same fp32 values, so the sets must be identical,
    including every tie (lower index wins)."""
    dd = require_gpu()
    announce(f"topk {kind} shape={shape} n_max={n_max} lens={lens} k={k}")
    s = _topk_case(kind, shape, n_max, seed=n_max + k)
    lens_t = torch.tensor(lens, dtype=torch.int32)
    ref = oracle.select_topk(s.numpy().astype(np.float64), lens_t.numpy(), k)
    got = dd.topk(s.cuda(), lens_t.cuda(), k).cpu().numpy()
    B, H, Q = shape
    for b in range(B):
        for h in range(H):
            for j in range(Q):
                assert np.array_equal(got[b, h, j], ref[b, h, j]), (
                    b, h, j, got[b, h, j][:10], ref[b, h, j][:10])


# --------------------------------------------------------------------------- gather
GATHER_CASES = [
    # dtype, D, n_max, m, with_cnt, invalid_frac
    ("bf16", 128, 5000, 128, False, 0.0),
    ("bf16", 128, 3000, 257, True, 0.1),
    ("bf16", 64, 999, 33, True, 0.2),
    ("f32", 64, 4096, 64, False, 0.05),
    ("f32", 128, 700, 100, True, 0.0),
]


@pytest.mark.parametrize("dtype,D,n_max,m,with_cnt,invalid_frac", GATHER_CASES)
def test_gather_bytes(dtype, D, n_max, m, with_cnt, invalid_frac):
    dd = require_gpu()
    announce(f"gather {dtype} D={D} n_max={n_max} m={m} cnt={with_cnt}")
    B, H = 2, 3
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    kh = to_host(dd, gen.random_tensor((B, H, n_max, D), seed=1, dtype=td))
    vh = to_host(dd, gen.random_tensor((B, H, n_max, D), seed=2, dtype=td))
    idx = gen.random_positions(B * H, m, n_max, seed=3, invalid_frac=invalid_frac).reshape(B, H, m)
    cnt = None
    if with_cnt:
        cnt = torch.tensor([[m, 0, 1], [m // 2, m + 5, -3]], dtype=torch.int32)
    sentinel = torch.full((B, H, m, D), 7.0).to(td)
    k_out, v_out = sentinel.clone().cuda(), sentinel.clone().cuda()
    dd.gather(kh, vh, idx.cuda(), None if cnt is None else cnt.cuda(), k_out=k_out, v_out=v_out)
    kr = oracle.gather_rows(stored(kh), idx.numpy(), None if cnt is None else cnt.numpy(),
                            out=stored(sentinel).copy())
    vr = oracle.gather_rows(stored(vh), idx.numpy(), None if cnt is None else cnt.numpy(),
                            out=stored(sentinel).copy())
    assert stored(k_out).tobytes() == kr.tobytes()
    assert stored(v_out).tobytes() == vr.tobytes()


def test_gather_worked_example_volume():
    """Top-128 rows of K and V at the 7B shape (32 heads x 128, bf16) move
    2,097,152 bytes, the paper-daily worked example's "about 2 MB"."""
    dd = require_gpu()
    announce("gather worked-example volume")
    B, H, D, n, k = 1, 32, 128, 32768, 128
    kh = to_host(dd, gen.random_tensor((B, H, n, D), seed=11, dtype=torch.bfloat16))
    vh = to_host(dd, gen.random_tensor((B, H, n, D), seed=12, dtype=torch.bfloat16))
    idx = gen.random_sorted_indices(H, k, torch.tensor([n] * H), seed=13).reshape(B, H, k)
    k_out, v_out = dd.gather(kh, vh, idx.cuda())
    assert k_out.numel() * 2 + v_out.numel() * 2 == 2097152
    assert stored(k_out).tobytes() == oracle.gather_rows(stored(kh), idx.numpy()).tobytes()
    assert stored(v_out).tobytes() == oracle.gather_rows(stored(vh), idx.numpy()).tobytes()


# --------------------------------------------------------------------------- attention
ATTN_CASES = [
    # dtype, D, k, m, invalid_frac, with_cnt
    ("bf16", 128, 128, 256, 0.0, False),
    ("bf16", 128, 1024, 2048, 0.05, False),
    ("bf16", 128, 129, 300, 0.1, True),
    ("bf16", 64, 512, 512, 0.0, True),
    ("f32", 64, 64, 128, 0.0, False),
    ("f32", 128, 300, 400, 0.02, True),
    ("bf16", 128, 1, 4, 0.0, False),
    ("bf16", 128, 2048, 4096, 0.0, False),
]


@pytest.mark.parametrize("dtype,D,k,m,invalid_frac,with_cnt", ATTN_CASES)
def test_sparse_attention(dtype, D, k, m, invalid_frac, with_cnt):
    dd = require_gpu()
    announce(f"attn {dtype} D={D} k={k} m={m} invalid={invalid_frac} cnt={with_cnt}")
    B, H = 2, 3
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    kr = gen.random_tensor((B, H, m, D), seed=k, dtype=td)
    vr = gen.random_tensor((B, H, m, D), seed=k + 1, dtype=td)
    q = gen.random_tensor((B, H, D), seed=k + 2, scale=2.0)
    pos = gen.random_positions(B * H, k, m, seed=k + 3, invalid_frac=invalid_frac).reshape(B, H, k)
    cnt = None
    if with_cnt:
        cnt = torch.tensor([[k, 0, 1], [k // 2, k + 9, k - 1]], dtype=torch.int32)
    out, lse = dd.sparse_attn(q.cuda(), kr.cuda(), vr.cuda(), pos=pos.cuda(),
                              cnt=None if cnt is None else cnt.cuda())
    ro, rl = oracle.attend_rows(q.numpy(), stored(kr), stored(vr), dtype, pos=pos.numpy(),
                                cnt=None if cnt is None else cnt.numpy(), k=k)
    got = out.cpu().numpy().reshape(B * H, D)
    worst = parity.check_attention(got, ro.reshape(B * H, D))
    gl = lse.cpu().numpy().reshape(-1)
    rl = rl.reshape(-1)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(gl), fin)
    assert np.all(np.abs(gl[fin] - rl[fin]) <= 1e-4 * np.maximum(1.0, np.abs(rl[fin])))
    assert np.all(got[~fin] == 0.0)
    print(f"worst relative attention error {worst:.2e}")


def test_attention_is_independent_of_row_placement():
    """The same entry list stored at other rows gives bitwise the same output."""
    dd = require_gpu()
    announce("attn placement invariance")
    B, H, D, k, m = 1, 4, 128, 700, 1400
    kr = gen.random_tensor((B, H, m, D), seed=31, dtype=torch.bfloat16)
    vr = gen.random_tensor((B, H, m, D), seed=32, dtype=torch.bfloat16)
    q = gen.random_tensor((B, H, D), seed=33)
    pos = gen.random_positions(B * H, k, m, seed=34).reshape(B, H, k)
    perm = torch.randperm(m, generator=torch.Generator().manual_seed(35))
    inv = torch.argsort(perm)
    kr2, vr2 = kr[:, :, perm].contiguous(), vr[:, :, perm].contiguous()   # row r moves to inv[r]
    pos2 = inv[pos.long()].to(torch.int32)
    o1, l1 = dd.sparse_attn(q.cuda(), kr.cuda(), vr.cuda(), pos=pos.cuda())
    o2, l2 = dd.sparse_attn(q.cuda(), kr2.cuda(), vr2.cuda(), pos=pos2.cuda())
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_attention_workspace_reuse():
    """One workspace, with what earlier calls of other sizes left in it,
    serves the next call: every result equals, bit for bit, that of the same
    call on a fresh workspace (the last case repeats the first after three
    others), for splits of one (b, h) over several workgroups and for one
    workgroup per (b, h)."""
    dd = require_gpu()
    announce("attn workspace reuse")
    D = 128
    cases = [(2, 3, 1024, 1100), (1, 5, 300, 300), (4, 8, 2048, 2048), (3, 2, 129, 200),
             (2, 3, 1024, 1100), (16, 40, 640, 640)]
    need = max(dd.attn_workspace_bytes(B, H, k, D) for B, H, k, _ in cases)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    for i, (B, H, k, m) in enumerate(cases):
        seed = 40 + 3 * (i % 4)
        kr = gen.random_tensor((B, H, m, D), seed=seed, dtype=torch.bfloat16).cuda()
        vr = gen.random_tensor((B, H, m, D), seed=seed + 1, dtype=torch.bfloat16).cuda()
        q = gen.random_tensor((B, H, D), seed=seed + 2).cuda()
        o1, l1 = dd.sparse_attn(q, kr, vr, k=k, ws=ws)
        o2, l2 = dd.sparse_attn(q, kr, vr, k=k)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), (B, H, k)


@pytest.mark.parametrize("big_b,big_h,k,m", [
    (4, 160, 1000, 1024),   # 640 (b, h): one 256-thread workgroup each
    (8, 160, 300, 320),     # 1280 (b, h): two groups, 3 chunks (one group idles in its second pass)
])
def test_attention_split_does_not_change_bits(big_b, big_h, k, m):
    """The same (b, h) rows give the same bits whether the batch around them
    is small (its chunks spread over several workgroups, merged by a second
    kernel) or large (one workgroup per (b, h), merged in LDS); both match
    the oracle."""
    dd = require_gpu()
    announce(f"attn split invariance B={big_b} H={big_h} k={k} m={m}")
    D = 128
    kr = gen.random_tensor((big_b, big_h, m, D), seed=71, dtype=torch.bfloat16)
    vr = gen.random_tensor((big_b, big_h, m, D), seed=72, dtype=torch.bfloat16)
    q = gen.random_tensor((big_b, big_h, D), seed=73, scale=2.0)
    pos = gen.random_positions(big_b * big_h, k, m, seed=74, invalid_frac=0.03).reshape(big_b, big_h, k)
    o_big, l_big = dd.sparse_attn(q.cuda(), kr.cuda(), vr.cuda(), pos=pos.cuda())
    sl = slice(0, 3)                   # 3 (b, h): split
    o_small, l_small = dd.sparse_attn(q[:1, sl].contiguous().cuda(), kr[:1, sl].contiguous().cuda(),
                                      vr[:1, sl].contiguous().cuda(), pos=pos[:1, sl].contiguous().cuda())
    torch.cuda.synchronize()
    assert torch.equal(o_big[:1, sl], o_small) and torch.equal(l_big[:1, sl], l_small)
    ro, _ = oracle.attend_rows(q[:1, sl].numpy(), stored(kr[:1, sl].contiguous()),
                               stored(vr[:1, sl].contiguous()), "bf16", pos=pos[:1, sl].numpy(), k=k)
    parity.check_attention(o_small.cpu().numpy().reshape(3, D), ro.reshape(3, D))
    # a sample of the large batch against the oracle too
    last = slice(big_h - 2, big_h)
    ro2, _ = oracle.attend_rows(q[-1:, last].numpy(), stored(kr[-1:, last].contiguous()),
                                stored(vr[-1:, last].contiguous()), "bf16", pos=pos[-1:, last].numpy(),
                                k=k)
    parity.check_attention(o_big[-1:, last].cpu().numpy().reshape(2, D), ro2.reshape(2, D))
