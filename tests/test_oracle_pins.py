"""Pins for the CPU oracle: each check ties it to something other than itself.

Closed forms, exact arithmetic (math.fsum of exact products), brute force on
tiny inputs, library routines for textbook special cases (torch's
scaled_dot_product_attention in float64), invariants, the structure the
input recipe plants, and the one number the pages print for this path (the
worked-example transfer size).
"""
import math
import os

import numpy as np
import pytest
import torch

import gen
import oracle
from tests import parity

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(t):
    """Stored form for the oracle: bf16 -> int16 bit patterns, fp32 -> float32."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    return t.numpy()


def _rand_keys(B, H, n, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn(B, H, n, D, generator=g)
    return k.to(torch.bfloat16 if dtype == "bf16" else torch.float32)


# --------------------------------------------------------------------------- upcast
def test_upcast_bf16_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3E20, 0x0000, 0x8000, 0x7F7F], dtype=np.uint16)
    got = oracle.upcast(bits, "bf16")
    want = [1.0, -2.0, 0.15625, 0.0, -0.0, (2 - 2 ** -7) * 2.0 ** 127]
    assert got.tolist() == want
    assert math.copysign(1.0, got[4]) == -1.0


def test_upcast_matches_torch_conversion():
    t = torch.randn(1000, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    assert np.array_equal(oracle.upcast(_bits(t), "bf16"), t.to(torch.float64).numpy())
    f = torch.randn(1000, generator=torch.Generator().manual_seed(4))
    assert np.array_equal(oracle.upcast(f.numpy(), "f32"), f.to(torch.float64).numpy())


# --------------------------------------------------------------------------- scoring
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_logits_match_exact_sums(dtype):
    """S5: every product of two fp32 values is exact in float64 and fsum rounds
    their sum correctly, so the exact scaled logit is known to within one
    rounding; the oracle's float64 matmul must agree to a few ulps of the
    absolute sum."""
    B, H, Q, D, n_max = 2, 3, 2, 8, 11
    keys = _rand_keys(B, H, n_max, D, dtype, 11)
    q = torch.randn(B, H, Q, D, generator=torch.Generator().manual_seed(12))
    lens = np.array([11, 6])
    scale = 0.3
    s = oracle.scaled_logits(q.numpy(), _bits(keys), lens, dtype, scale)
    kf = keys.to(torch.float64).numpy()
    qf = q.to(torch.float64).numpy()
    for b in range(B):
        for h in range(H):
            for j in range(Q):
                for i in range(n_max):
                    if i >= lens[b]:
                        assert s[b, h, j, i] == -np.inf
                        continue
                    prods = [float(qf[b, h, j, d]) * float(kf[b, h, i, d]) for d in range(D)]
                    exact = math.fsum(prods) * scale
                    bound = 1e-14 * scale * math.fsum(abs(p) for p in prods) + 1e-300
                    assert abs(s[b, h, j, i] - exact) <= bound


def test_default_scale_is_inverse_sqrt_head_dim():
    assert oracle.default_scale(128) == 1.0 / math.sqrt(128)
    assert oracle.default_scale(64) == 0.125
    q = np.zeros((1, 1, 1, 64), dtype=np.float32)
    q[..., 0] = 1.0
    keys = np.zeros((1, 1, 2, 64), dtype=np.float32)
    keys[0, 0, 0, 0] = 8.0
    s = oracle.scaled_logits(q, keys, np.array([2]), "f32")
    assert s[0, 0, 0].tolist() == [1.0, 0.0]
    s0 = oracle.scaled_logits(q, keys, np.array([2]), "f32", scale=0.0)   # <= 0 -> default
    assert s0[0, 0, 0].tolist() == [1.0, 0.0]


def test_alpha_sums_to_one_and_ratios():
    """S1 and the closed form alpha_i / alpha_j = exp(s_i - s_j)."""
    rng = np.random.default_rng(5)
    B, H, Q, n_max = 3, 2, 2, 50
    s = rng.normal(size=(B, H, Q, n_max)) * 4
    lens = np.array([50, 17, 1])
    for b in range(B):
        s[b, :, :, lens[b]:] = -np.inf
    a = oracle.attention_weights(s, lens)
    for b in range(B):
        n = lens[b]
        tot = a[b, :, :, :n].sum(axis=-1)
        assert np.all(np.abs(tot - 1.0) <= 1e-12)
        assert np.all(a[b, :, :, n:] == 0.0)
        for h in range(H):
            for j in range(Q):
                for i1, i2 in [(0, n - 1), (n // 2, 0)]:
                    want = math.exp(s[b, h, j, i1] - s[b, h, j, i2])
                    assert a[b, h, j, i1] / a[b, h, j, i2] == pytest.approx(want, rel=1e-12)


def test_hand_example_closed_form():
    """A four-key, two-dimensional example worked by hand from the formulas
    alpha = softmax(q K^T / sqrt(d_k)), I = argtopk(alpha, k)."""
    q = np.array([[[[1.0, 0.0], [0.0, 1.0]]]], dtype=np.float32)          # cur, spec
    keys = np.array([[[[2, 0], [0, 2], [1, 1], [-1, 0]]]], dtype=np.float32)
    vals = np.array([[[[1, 0], [0, 1], [1, 1], [2, 2]]]], dtype=np.float32)
    lens = np.array([4])
    r2 = math.sqrt(2.0)
    s = oracle.scaled_logits(q, keys, lens, "f32")
    assert s[0, 0, 0] == pytest.approx([2 / r2, 0.0, 1 / r2, -1 / r2], abs=1e-15)
    assert s[0, 0, 1] == pytest.approx([0.0, 2 / r2, 1 / r2, 0.0], abs=1e-15)
    sel = oracle.select_topk(s, lens, 2)
    assert sel[0, 0, 0].tolist() == [0, 2]
    assert sel[0, 0, 1].tolist() == [1, 2]
    out, lse = oracle.masked_attention(q[:, :, 0], keys, vals, lens, sel[:, :, 0], "f32")
    p2 = 1.0 / (1.0 + math.exp(1 / r2))                 # weight of key 2 against key 0
    assert out[0, 0] == pytest.approx([1.0, p2], abs=1e-15)
    assert lse[0, 0] == pytest.approx(math.log(math.exp(r2) + math.exp(1 / r2)), abs=1e-14)
    bk = oracle.bookkeeping(sel[:, :, 0], sel[:, :, 1], 4)
    assert bk["pos"][0, 0].tolist() == [2, 1]          # key 0 missed -> row k+0; key 2 hit at P[1]
    assert bk["miss"][0, 0].tolist() == [0, -1]
    assert int(bk["hits"][0, 0]) == 1 and int(bk["miss_cnt"][0, 0]) == 1


# --------------------------------------------------------------------------- selection
def _brute_topk(row, k):
    """i is chosen iff fewer than k entries beat it (larger, or equal and earlier)."""
    n = len(row)
    chosen = []
    for i in range(n):
        beats = sum(1 for j in range(n) if row[j] > row[i] or (row[j] == row[i] and j < i))
        if beats < k:
            chosen.append(i)
    return chosen


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_brute_force_with_ties(seed):
    """S4: rank-count definition on tiny rows drawn from a 5-value set (with
    -0.0 and +0.0), so exact ties are frequent."""
    rows, n = 4, 37
    t = gen.tie_scores(rows, n, seed=seed, nvalues=5).numpy().astype(np.float64)
    s = t.reshape(1, 1, rows, n)
    lens = np.array([n])
    for k in [1, 2, 5, 17, 36, 37, 40]:
        sel = oracle.select_topk(s, lens, k)
        for r in range(rows):
            want = _brute_topk([float(x) + 0.0 for x in t[r]], k)
            got = [int(i) for i in sel[0, 0, r] if i >= 0]
            assert got == want, (k, r)
            assert np.all(sel[0, 0, r, len(want):] == -1)


def test_topk_on_logits_equals_topk_on_alpha():
    """S2: softmax is increasing, so selecting on logits or on weights agrees."""
    rng = np.random.default_rng(9)
    B, H, Q, n_max = 2, 3, 2, 300
    s = rng.normal(size=(B, H, Q, n_max)) * 3
    lens = np.array([300, 123])
    for b in range(B):
        s[b, :, :, lens[b]:] = -np.inf
    a = oracle.attention_weights(s, lens)
    for k in [1, 10, 123, 200]:
        assert np.array_equal(oracle.select_topk(s, lens, k), oracle.select_topk(a, lens, k))


def test_topk_short_rows_pad_with_minus_one():
    s = np.array([[[[3.0, 1.0, 2.0, -np.inf]]]])
    sel = oracle.select_topk(s, np.array([3]), 5)
    assert sel[0, 0, 0].tolist() == [0, 1, 2, -1, -1]
    sel0 = oracle.select_topk(s, np.array([0]), 2)
    assert sel0[0, 0, 0].tolist() == [-1, -1]


# --------------------------------------------------------------------------- gather
def test_gather_is_identity_on_bytes():
    """S8: the gathered rows are the host rows, byte for byte."""
    keys = _rand_keys(2, 3, 40, 16, "bf16", 21)
    host = _bits(keys)
    idx = gen.random_sorted_indices(6, 9, torch.tensor([40] * 6), seed=3, fill=0.8).numpy().reshape(2, 3, 9)
    idx[0, 1, 2] = 45                                     # out of range -> zero row
    rows = oracle.gather_rows(host, idx)
    for b in range(2):
        for h in range(3):
            for j in range(9):
                i = idx[b, h, j]
                want = host[b, h, i] if 0 <= i < 40 else np.zeros(16, dtype=host.dtype)
                assert rows[b, h, j].tobytes() == want.tobytes()
    cnt = np.array([[3, 0, 9], [1, 2, 4]])
    pre = np.full((2, 3, 9, 16), 7, dtype=host.dtype)
    part = oracle.gather_rows(host, idx, cnt, out=pre.copy())
    for b in range(2):
        for h in range(3):
            assert np.all(part[b, h, cnt[b, h]:] == 7)
            assert np.array_equal(part[b, h, :cnt[b, h]], rows[b, h, :cnt[b, h]])


def test_gather_volume_matches_worked_example():
    """The worked example's transfer: top-128 rows of K and V at hidden size
    4096 in 2-byte elements is 2,097,152 bytes."""
    fields = {}
    with open(os.path.join(GOLDEN, "worked_example_transfer.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                name, value = line.split()
                fields[name] = int(value)
    H, D = 32, 128
    assert H * D == fields["hidden"]
    k = fields["selected_tokens"]
    host = np.zeros((1, H, 1024, D), dtype=np.int16)
    idx = np.tile(np.arange(k, dtype=np.int32), (1, H, 1))
    krows = oracle.gather_rows(host, idx)
    vrows = oracle.gather_rows(host, idx)
    assert krows.itemsize == fields["bytes_per_element"]
    assert krows.nbytes + vrows.nbytes == fields["transfer_bytes"]
    assert fields["selected_tokens"] * fields["kv_planes"] * fields["hidden"] * \
        fields["bytes_per_element"] == fields["transfer_bytes"]


# --------------------------------------------------------------------------- attention
def _sdpa(q, k, v, scale):
    """torch's textbook attention in float64 on the CPU (the library routine)."""
    qt = torch.from_numpy(q)[:, None, :]                 # [rows, 1, D]
    return torch.nn.functional.scaled_dot_product_attention(
        qt, torch.from_numpy(k), torch.from_numpy(v), scale=scale)[:, 0, :].numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_masked_attention_with_all_keys_is_dense_attention(dtype):
    """S3: with k = n the mask removes nothing and the result is plain attention."""
    B, H, n, D = 2, 3, 57, 16
    keys = _rand_keys(B, H, n, D, dtype, 31)
    vals = _rand_keys(B, H, n, D, dtype, 32)
    q = torch.randn(B, H, D, generator=torch.Generator().manual_seed(33)) * 2
    lens = np.array([n, n])
    sel = np.tile(np.arange(n, dtype=np.int32), (B, H, 1))
    out, lse = oracle.masked_attention(q.numpy(), _bits(keys), _bits(vals), lens, sel, dtype)
    kf = keys.to(torch.float64).numpy().reshape(B * H, n, D)
    vf = vals.to(torch.float64).numpy().reshape(B * H, n, D)
    qf = q.to(torch.float64).numpy().reshape(B * H, D)
    want = _sdpa(qf, kf, vf, 1 / math.sqrt(D))
    assert np.max(np.abs(out.reshape(B * H, D) - want)) <= 1e-12 * np.max(np.abs(want))
    z = np.einsum("rnd,rd->rn", kf, qf) / math.sqrt(D)
    want_lse = np.log(np.exp(z - z.max(1, keepdims=True)).sum(1)) + z.max(1)
    assert np.allclose(lse.reshape(-1), want_lse, rtol=1e-13, atol=0)


def test_attend_rows_is_dense_attention_over_the_rows():
    B, H, m, D = 2, 2, 30, 8
    kr = _rand_keys(B, H, m, D, "bf16", 41)
    vr = _rand_keys(B, H, m, D, "bf16", 42)
    q = torch.randn(B, H, D, generator=torch.Generator().manual_seed(43))
    out, _ = oracle.attend_rows(q.numpy(), _bits(kr), _bits(vr), "bf16")
    want = _sdpa(q.double().numpy().reshape(-1, D), kr.double().numpy().reshape(-1, m, D),
                 vr.double().numpy().reshape(-1, m, D), 1 / math.sqrt(D))
    assert np.max(np.abs(out.reshape(-1, D) - want)) <= 1e-12 * np.max(np.abs(want))


def test_attention_identities():
    """S7: one row -> that row exactly; equal logits -> mean; convex hull;
    row order does not matter; invalid rows are skipped; nothing -> 0, -inf."""
    rng = np.random.default_rng(7)
    D, m = 8, 12
    vr = rng.normal(size=(1, 1, m, D)).astype(np.float32)
    kr = rng.normal(size=(1, 1, m, D)).astype(np.float32)
    q = rng.normal(size=(1, 1, D)).astype(np.float32)
    one, _ = oracle.attend_rows(q, kr, vr, "f32", pos=np.array([[[5]]], dtype=np.int32))
    assert np.array_equal(one[0, 0], vr[0, 0, 5].astype(np.float64))
    # equal logits: q orthogonal to every key difference
    q0 = np.zeros((1, 1, D), dtype=np.float32)
    q0[0, 0, 0] = 1.0
    keq = kr.copy()
    keq[..., 0] = 0.5
    pos = np.array([[[0, 3, 7, 9]]], dtype=np.int32)
    mean, _ = oracle.attend_rows(q0, keq, vr, "f32", pos=pos)
    assert np.max(np.abs(mean[0, 0] - vr[0, 0, [0, 3, 7, 9]].astype(np.float64).mean(0))) <= 1e-15
    full, _ = oracle.attend_rows(q, kr, vr, "f32")
    assert np.all(full[0, 0] <= vr[0, 0].max(0) + 1e-15)
    assert np.all(full[0, 0] >= vr[0, 0].min(0) - 1e-15)
    perm = rng.permutation(m)
    shuffled, _ = oracle.attend_rows(q, kr[:, :, perm], vr[:, :, perm], "f32")
    assert np.max(np.abs(shuffled - full)) <= 1e-15 * np.abs(full).max()
    bad = np.array([[[2, -1, 40, 4]]], dtype=np.int32)
    skip, _ = oracle.attend_rows(q, kr, vr, "f32", pos=bad)
    keep, _ = oracle.attend_rows(q, kr, vr, "f32", pos=np.array([[[2, 4]]], dtype=np.int32))
    assert np.array_equal(skip, keep)
    empty, lse = oracle.attend_rows(q, kr, vr, "f32", pos=bad, cnt=np.array([[0]]))
    assert np.all(empty == 0) and lse[0, 0] == -np.inf


def test_masked_attention_equals_attention_over_gathered_rows():
    w = gen.workload("tiny").scaled(H=2, n_max=300)
    lay = gen.make_layer(w, 0)
    kh, vh = _bits(lay["k"]), _bits(lay["v"])
    lens = lay["lens"].numpy()
    s = oracle.scaled_logits(lay["q"].numpy(), kh, lens, w.dtype)
    sel = oracle.select_topk(s, lens, 20)[:, :, 0]
    o1, l1 = oracle.masked_attention(lay["q"][:, :, 0].numpy(), kh, vh, lens, sel, w.dtype)
    o2, l2 = oracle.attend_rows(lay["q"][:, :, 0].numpy(), oracle.gather_rows(kh, sel),
                                oracle.gather_rows(vh, sel), w.dtype)
    assert np.max(np.abs(o1 - o2)) <= 1e-13 * np.abs(o1).max()
    assert np.max(np.abs(l1 - l2)) <= 1e-13 * np.abs(l1).max()


# --------------------------------------------------------------------------- bookkeeping
@pytest.mark.parametrize("seed", range(4))
def test_bookkeeping_matches_set_arithmetic(seed):
    B, H, k, n = 2, 3, 16, 60
    rows = B * H
    cur = gen.random_sorted_indices(rows, k, torch.tensor([n] * rows), seed=seed, fill=0.9)
    pred = gen.random_sorted_indices(rows, k, torch.tensor([n] * rows), seed=100 + seed, fill=1.0)
    cur = cur.numpy().reshape(B, H, k)
    pred = pred.numpy().reshape(B, H, k)
    bk = oracle.bookkeeping(cur, pred, n)
    for b in range(B):
        for h in range(H):
            c = [int(x) for x in cur[b, h] if x >= 0]
            p = [int(x) for x in pred[b, h] if x >= 0]
            misses = sorted(set(c) - set(p))
            assert bk["miss"][b, h, :len(misses)].tolist() == misses
            assert np.all(bk["miss"][b, h, len(misses):] == -1)
            assert bk["miss_cnt"][b, h] == len(misses)
            assert bk["hits"][b, h] == len(set(c) & set(p))
            assert bk["prefetched"][b, h] == len(p)
            slot = list(pred[b, h]) + misses + [None] * (k - len(misses))
            for j, cj in enumerate(cur[b, h]):
                if cj < 0:
                    assert bk["pos"][b, h, j] == -1
                else:
                    assert slot[bk["pos"][b, h, j]] == cj


def test_bookkeeping_cold_and_perfect_prediction():
    cur = np.array([[[1, 4, 9, -1]]], dtype=np.int32)
    cold = oracle.bookkeeping(cur, None, 10)
    assert cold["pos"][0, 0].tolist() == [4, 5, 6, -1]
    assert cold["miss_cnt"][0, 0] == 3 and cold["prefetched"][0, 0] == 0
    hot = oracle.bookkeeping(cur, cur.copy(), 10)
    assert hot["pos"][0, 0].tolist() == [0, 1, 2, -1]
    assert hot["miss_cnt"][0, 0] == 0 and hot["hits"][0, 0] == 3
    out_of_range = oracle.bookkeeping(cur, np.array([[[4, 12, -1, -1]]], dtype=np.int32), 10)
    assert out_of_range["prefetched"][0, 0] == 1 and out_of_range["hits"][0, 0] == 1


# --------------------------------------------------------------------------- layer step
def _layer(w, layer=0):
    lay = gen.make_layer(w, layer)
    return lay, _bits(lay["k"]), _bits(lay["v"]), lay["lens"].numpy()


def test_layer_step_output_does_not_depend_on_prediction():
    w = gen.workload("llama7b_32k_layer").scaled(H=2, n_max=2048, k=32)
    lay, kh, vh, lens = _layer(w)
    q = lay["q"].numpy()
    cold = oracle.layer_step(q, kh, kh, vh, lens, w.k, w.dtype, pred=None)
    assert np.array_equal(cold["stats"], [cold["miss_cnt"].sum(), 0, cold["miss_cnt"].sum()])
    for pred in [cold["spec"], cold["cur"],
                 gen.random_sorted_indices(w.B * w.H, w.k, torch.tensor([2048] * 2), 5).numpy()
                 .reshape(w.B, w.H, w.k)]:
        hot = oracle.layer_step(q, kh, kh, vh, lens, w.k, w.dtype, pred=pred)
        assert np.array_equal(hot["out"], cold["out"])
        assert np.array_equal(hot["cur"], cold["cur"])
        assert hot["stats"][0] + hot["stats"][1] == np.sum(hot["cur"] >= 0)
    perfect = oracle.layer_step(q, kh, kh, vh, lens, w.k, w.dtype, pred=cold["cur"])
    assert perfect["stats"][0] == 0


def test_planted_tiny_workload():
    """S6, tiny workload at full size: the 16 keys set to 4 q have logit
    4 |q|^2 / 8 (about 32) against N(0,1) for the rest, so both queries select
    them and they carry all but 1e-6 of the current query's weight."""
    w = gen.workload("tiny")
    lay, kh, vh, lens = _layer(w)
    q = lay["q"].numpy()
    s = oracle.scaled_logits(q, kh, lens, w.dtype)
    a = oracle.attention_weights(s, lens)
    sel = oracle.select_topk(s, lens, w.k)
    for h in range(w.H):
        planted = set(lay["planted"][0, h, :16].tolist())
        assert planted <= set(sel[0, h, 0].tolist())
        assert planted <= set(sel[0, h, 1].tolist())
        assert a[0, h, 0, sorted(planted)].sum() >= 1 - 1e-6
        want = 4 * float(np.dot(q[0, h, 0].astype(np.float64), q[0, h, 0])) / 8
        assert s[0, h, 0, sorted(planted)] == pytest.approx(want, rel=1e-6)


@pytest.mark.parametrize("name,kw,relation", [
    ("llama7b_32k_layer", dict(H=3), "sel_in_planted"),           # k=128 < 328 planted
    ("llama7b_32k_step", dict(B=1, H=2), "planted_in_sel"),       # k=1024 > 328
    ("llama13b_128k", dict(B=1, H=1), "planted_in_sel"),          # k=2048 > 1311
    ("hiconc_64", dict(B=3, H=2), "by_len"),                      # ragged
])
def test_planted_structure(name, kw, relation):
    """S6: planted keys score about 4 |q|^2 / sqrt(D) = 45 (Zipf: 45 - 1.1 ln r,
    at least 37) against N(0, 1) for random keys, so the selected set and the
    planted set nest one inside the other."""
    w = gen.workload(name).scaled(**kw)
    lay, kh, _, lens = _layer(w)
    s = oracle.scaled_logits(lay["q"][:, :, :1].numpy(), kh, lens, w.dtype)
    sel = oracle.select_topk(s, lens, w.k)
    for b in range(w.B):
        for h in range(w.H):
            cnt = int(lay["planted_cnt"][b, h])
            planted = set(lay["planted"][b, h, :cnt].tolist())
            chosen = set(int(i) for i in sel[b, h, 0] if i >= 0)
            rel = relation
            if rel == "by_len":
                rel = "planted_in_sel" if cnt <= w.k else "sel_in_planted"
            if rel == "planted_in_sel":
                assert planted <= chosen
            else:
                assert chosen <= planted


# --------------------------------------------------------------------------- chunk landmarks
def test_landmarks_of_constant_chunks_and_partial_tail():
    """A chunk of equal keys has that key as its landmark, the last, partial
    chunk included (its mean is over its valid rows, not over the chunk
    size); chunks with no valid row are zero and rows past the length never
    count (they hold +-1e30 here)."""
    rng = np.random.default_rng(3)
    B, H, n_max, D, c = 2, 3, 40, 8, 8
    lens = np.array([37, 5])
    base = rng.standard_normal((B, H, n_max // c, D)).astype(np.float32)
    keys = np.repeat(base, c, axis=2).copy()
    keys[0, :, 37:] = 1e30
    keys[1, :, 5:] = -1e30
    lm = oracle.landmarks(keys, lens, c, oracle.F32)
    assert lm.shape == (B, H, 5, D)
    for b in range(B):
        nc = -(-int(lens[b]) // c)
        np.testing.assert_array_equal(lm[b, :, :nc], base[b, :, :nc].astype(np.float64))
        assert np.all(lm[b, :, nc:] == 0)


def test_landmarks_with_chunk_one_are_the_keys():
    w = gen.workload("llama7b_32k_layer").scaled(H=2, n_max=300)
    lay, kh, _, lens = _layer(w)
    lm = oracle.landmarks(kh, lens, 1, w.dtype)
    n = int(lens[0])
    np.testing.assert_array_equal(lm[0, :, :n], oracle.upcast(kh[0, :, :n], w.dtype))


def test_landmarks_weighted_by_counts_sum_to_the_keys():
    """sum over chunks of (valid rows) x landmark = the sum of all valid keys."""
    w = gen.workload("hiconc_64").scaled(B=3, H=2, n_max=700, len_lo=50, len_hi=700)
    lay, kh, _, lens = _layer(w)
    c = 16
    lm = oracle.landmarks(kh, lens, c, w.dtype)
    for b in range(w.B):
        n = int(lens[b])
        cnt = np.array([min(c, n - e * c) for e in range(-(-n // c))], dtype=np.float64)
        for h in range(w.H):
            kf = oracle.upcast(kh[b, h, :n], w.dtype)
            for d in range(0, w.D, 37):
                want = math.fsum(kf[:, d].tolist())
                got = math.fsum((cnt * lm[b, h, :len(cnt), d]).tolist())
                assert abs(got - want) <= 1e-9 * (1 + math.fsum(np.abs(kf[:, d]).tolist()))


def test_chunk_step_with_chunk_one_is_the_per_key_step():
    for name, kw in (("tiny", {}), ("hiconc_64", dict(B=2, H=2, n_max=600, len_lo=100, len_hi=600, k=64))):
        w = gen.workload(name).scaled(**kw)
        lay, kh, vh, lens = _layer(w)
        q = lay["q"].numpy()
        a = oracle.layer_step(q, kh, kh, vh, lens, w.k, w.dtype)
        b = oracle.layer_step(q, kh, kh, vh, lens, w.k, w.dtype, chunk=1)
        for key in ("cur", "spec", "out", "lse", "stats"):
            np.testing.assert_array_equal(a[key], b[key])


def test_chunk_selection_and_attention_closed_form():
    """Keys are zero except the partial last chunk (rows 12 and 13 of 14,
    chunk size 4), whose rows are 2q: its landmark scores 2|q|^2/sqrt(D) = 1
    and every other chunk 0.  With k = 8 (two chunks) the current query takes
    chunk 3 and, among the tied zeros, chunk 0; the speculated query -q takes
    chunks 0 and 1.  Attention over rows 0-3 (logit 0) and 12-13 (logit 1)
    with V row i = i in column 0 gives (0+1+2+3 + e(12+13)) / (4 + 2e)."""
    D, c, n = 4, 4, 14
    qv = np.array([1.0, 0.0, 0.0, 0.0], dtype=np.float32)
    q = np.stack([qv, -qv])[None, None]                      # [1][1][2][D]
    keys = np.zeros((1, 1, 16, D), dtype=np.float32)
    keys[0, 0, 12:14] = 2 * qv
    keys[0, 0, 14:] = 99.0                                   # padding
    vals = np.zeros((1, 1, 16, D), dtype=np.float32)
    vals[0, 0, :, 0] = np.arange(16)
    vals[0, 0, :, 1] = 1.0
    lens = np.array([n])
    r = oracle.layer_step(q, keys, keys, vals, lens, 8, oracle.F32, chunk=c)
    assert r["cur"].tolist() == [[[0, 3]]]
    assert r["spec"].tolist() == [[[0, 1]]]
    assert r["rows"][0, 0].tolist() == [0, 1, 2, 3, 12, 13, -1, -1]
    e = math.e
    assert abs(r["out"][0, 0, 0] - (6 + 25 * e) / (4 + 2 * e)) < 1e-12
    assert abs(r["out"][0, 0, 1] - 1.0) < 1e-12
    assert abs(r["lse"][0, 0] - math.log(4 + 2 * e)) < 1e-12
    # dual-token: the speculated query -q attends over the same rows {0-3, 12, 13}
    # (logits 0 and -1), not over its own chunks {0, 1}
    rd = oracle.layer_step(q, keys, keys, vals, lens, 8, oracle.F32, chunk=c, dual=True)
    assert abs(rd["out_spec"][0, 0, 0] - (6 + 25 / e) / (4 + 2 / e)) < 1e-12
    assert abs(rd["lse_spec"][0, 0] - math.log(4 + 2 / e)) < 1e-12
    np.testing.assert_array_equal(rd["out"], r["out"])
    # prediction = chunks {0, 1}: chunk 0 hits (slot rows 0..3), chunk 3 misses
    r2 = oracle.layer_step(q, keys, keys, vals, lens, 8, oracle.F32, chunk=c,
                           pred=np.array([[[0, 1]]], dtype=np.int32))
    assert r2["stats"].tolist() == [1, 1, 3]
    assert r2["pos"].tolist() == [[[0, 2]]]
    np.testing.assert_array_equal(r2["out"], r["out"])


def test_dual_token_attention_with_equal_queries_is_the_current_output():
    """With the speculated query equal to the current one, both attend over the
    same rows with the same logits: equal outputs, per key and by chunks."""
    w = gen.workload("llama7b_32k_layer").scaled(B=2, H=2, n_max=700, rho=1.0, rho_c=0.0,
                                                 len_lo=600, len_hi=700, k=64)
    lay, kh, vh, lens = _layer(w)
    for chunk in (0, 8):
        r = oracle.layer_step(lay["q"].numpy(), kh, kh, vh, lens, w.k, w.dtype, chunk=chunk,
                              dual=True)
        np.testing.assert_array_equal(r["out_spec"], r["out"])
        np.testing.assert_array_equal(r["lse_spec"], r["lse"])


# --------------------------------------------------------------------------- decode loop
def test_append_rows_writes_one_row_per_request():
    cache = np.arange(2 * 3 * 5 * 4, dtype=np.float32).reshape(2, 3, 5, 4)
    new = -np.ones((2, 3, 4), dtype=np.float32)
    out, lens = oracle.append_rows(cache, np.array([2, 5]), new)
    assert lens.tolist() == [3, 5]                    # request 1 is full
    assert np.all(out[0, :, 2] == -1)
    out[0, :, 2] = cache[0, :, 2]
    np.testing.assert_array_equal(out, cache)


def _loop(w, steps, new_key=None, chunk=0):
    """The oracle decode loop: append, then the layer step with the previous
    step's speculated set as the prediction."""
    lay, kh, vh, lens = _layer(w)
    q = lay["q"]
    ref = oracle.layer_step(q.numpy(), kh, kh, vh, lens, w.k, w.dtype, chunk=chunk)
    out = []
    for t in range(1, steps + 1):
        q, nk, nv = gen.decode_step_inputs(w, 0, t, q)
        if new_key is not None:
            nk = new_key(q).to(nk.dtype)
        kh, _ = oracle.append_rows(kh, lens, _stored(nk))
        vh, lens = oracle.append_rows(vh, lens, _stored(nv))
        ref = oracle.layer_step(q.numpy(), kh, kh, vh, lens, w.k, w.dtype, pred=ref["spec"],
                                chunk=chunk)
        out.append((ref, lens.copy()))
    return out


def _stored(t):
    t = t.contiguous()
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.numpy()


def test_decode_loop_perfect_speculation_has_full_recall():
    """With the speculated query equal to the current one and the next token
    equal to the speculated one, and zero new keys (below the k-th score), the
    true set of step t+1 is the speculated set of step t: no misses."""
    w = gen.workload("llama7b_32k_layer").scaled(B=2, H=2, n_max=3000, rho=1.0, rho_c=0.0,
                                                 len_lo=2900, len_hi=2900)
    for chunk in (0, 4):
        for t, (ref, lens) in enumerate(_loop(w, 3, new_key=lambda q: 0.0 * q[:, :, 0],
                                              chunk=chunk), start=1):
            st = ref["stats"]
            assert st[0] == 0 and st[1] == w.B * w.H * (w.k // max(chunk, 1)), (chunk, st)
            assert lens.tolist() == [2900 + t] * w.B


def test_decode_loop_new_dominant_key_is_exactly_one_miss():
    """A new key of 8 q_cur scores 8|q|^2/sqrt(D), above every planted key, so it
    joins each true set without being in the prediction (made before it
    existed): exactly one miss per (b, h) at every step."""
    w = gen.workload("llama7b_32k_layer").scaled(B=2, H=2, n_max=3000, rho=1.0, rho_c=0.0,
                                                 len_lo=2900, len_hi=2900)
    for ref, lens in _loop(w, 3, new_key=lambda q: 8.0 * q[:, :, 0]):
        st = ref["stats"]
        assert st[0] == w.B * w.H and st[1] == w.B * w.H * (w.k - 1), st
        n = int(lens[0])
        assert np.all(ref["cur"][:, :, -1] == n - 1)    # the new row, last in ascending order


# --------------------------------------------------------------------------- comparators
def test_tie_band_comparator_accepts_swaps_and_rejects_errors():
    logits = np.array([[5.0, 3.0, 3.0 + 5e-4, 1.0, 3.0 - 2e-3]])
    lens = np.array([5])
    ref = np.array([[0, 2]])
    parity.check_index_sets(np.array([[0, 2]]), ref, logits, lens, 2)
    assert parity.check_index_sets(np.array([[0, 1]]), ref, logits, lens, 2) == [0]
    with pytest.raises(AssertionError):
        parity.check_index_sets(np.array([[0, 4]]), ref, logits, lens, 2)
    with pytest.raises(AssertionError):
        parity.check_index_sets(np.array([[2, 0]]), ref, logits, lens, 2)


def test_resident_fetches_hand_example():
    """Previous slot holds prediction {1, 2, 3} (the -1 and the out-of-range
    9 hold nothing) and miss {7}; this step's prediction {2, 3, 4, 5} brings
    4 and 5 over the link, its misses {7, 8} bring 8: three rows."""
    n_max = 9
    prev_pred = np.array([[[1, 2, 3, -1, 9]]], dtype=np.int32)
    prev_miss = np.array([[[7, -1, -1, -1, -1]]], dtype=np.int32)
    pred = np.array([[[2, 3, 4, 5, -1]]], dtype=np.int32)
    miss = np.array([[[7, 8, -1, -1, -1]]], dtype=np.int32)
    assert oracle.resident_fetches(prev_pred, prev_miss, pred, miss, n_max).tolist() == [[3]]
    # nothing held before: every valid prediction entry and every miss
    assert oracle.resident_fetches(None, None, pred, miss, n_max).tolist() == [[6]]
    # no prediction this step: only the misses not held
    assert oracle.resident_fetches(prev_pred, prev_miss, None, miss, n_max).tolist() == [[1]]
    # the same prediction and misses again: nothing crosses the link
    assert oracle.resident_fetches(prev_pred, prev_miss, prev_pred, prev_miss, n_max).tolist() == [[0]]


def test_resident_fetches_cold_step_is_the_ring_count():
    """Without a previous step, the rows fetched are the prediction's valid
    entries plus the misses: the bookkeeping's prefetched + miss_cnt."""
    rng = np.random.default_rng(5)
    B, H, k, n_max = 2, 3, 16, 64
    cur = np.sort(np.stack([[rng.choice(n_max, k, replace=False) for _ in range(H)]
                            for _ in range(B)]), axis=2).astype(np.int32)
    pred = np.sort(np.stack([[rng.choice(n_max, k, replace=False) for _ in range(H)]
                             for _ in range(B)]), axis=2).astype(np.int32)
    bk = oracle.bookkeeping(cur, pred, n_max)
    got = oracle.resident_fetches(None, None, pred, bk["miss"], n_max)
    assert np.array_equal(got, bk["prefetched"] + bk["miss_cnt"])


def test_resident_fetches_match_a_brute_force_count():
    """Against a count by membership masks over all n_max keys."""
    rng = np.random.default_rng(6)
    B, H, k, n_max = 2, 2, 8, 24
    def draw():
        a = np.full((B, H, k), -1, dtype=np.int32)
        for b in range(B):
            for h in range(H):
                m = rng.integers(0, k + 1)
                a[b, h, :m] = np.sort(rng.choice(n_max, m, replace=False))
        return a
    for _ in range(20):
        pp, pm, p, m = draw(), draw(), draw(), draw()
        got = oracle.resident_fetches(pp, pm, p, m, n_max)
        for b in range(B):
            for h in range(H):
                held = np.zeros(n_max, dtype=bool)
                for x in list(pp[b, h]) + list(pm[b, h]):
                    if x >= 0:
                        held[x] = True
                want = sum(1 for x in p[b, h] if x >= 0 and not held[x]) + \
                    sum(1 for x in m[b, h] if x >= 0 and not held[x])
                assert got[b, h] == want
