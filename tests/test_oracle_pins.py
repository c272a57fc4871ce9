"""Pins for the fp64 oracle: what the pages print and what mathematics fixes.

None of these tests retypes the oracle's formulas: each compares the oracle
with a printed fixture, a closed form derived by hand, a special case that
reduces to a library routine, or the independent pure-Python brute force.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute, oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_matrix(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(x) for x in line.split()])
    return np.array(rows, dtype=bool)


def _three_doc_ids():
    lines = []
    with open(os.path.join(GOLDEN, "document_3doc_boundaries.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                lines.append([int(x) for x in line.split()])
    S = lines[0][0]
    doc = np.zeros(S, dtype=np.int32)
    for start, d in lines[1:]:
        doc[start:] = d
    return doc


# ---------------------------------------------------------------- masks
def test_sliding_window_printed_matrix():
    # crackedaicode "State the boundary precisely": the printed T=6, W=3 mask
    want = _read_matrix("sliding_window_T6_W3.txt")
    got = O.dense_mask("sliding_window", 6, 6, window=3)
    assert got.shape == (6, 6)
    assert np.array_equal(got, want)
    # "Build and apply the mask": the last row is [0,0,0,1,1,1]
    assert np.array_equal(got[-1], np.array([0, 0, 0, 1, 1, 1], bool))


def test_sliding_window_boundary_and_off_by_one():
    T, W = 40, 7
    m = O.dense_mask("sliding_window", T, T, window=W)
    for i in range(T):
        # allowed keys run from max(0, i - W + 1) through i inclusive
        assert np.flatnonzero(m[i]).tolist() == list(range(max(0, i - W + 1),
                                                          i + 1))
    # "i - j <= W would allow one extra earlier key": the wrong variant
    # differs from the mask in exactly one key on every row with i >= W
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    wrong = (i >= j) & (i - j <= W)
    diff = (wrong & ~m).sum(axis=1)
    assert np.all(diff[W:] == 1) and np.all(diff[:W] == 0)
    assert not (m & ~wrong).any()


@pytest.mark.parametrize("T", [1, 2, 5, 16, 33])
def test_sliding_window_special_cases(T):
    # W = 1 permits only self-attention; W >= T is the causal triangle
    assert np.array_equal(O.dense_mask("sliding_window", T, T, window=1),
                          np.eye(T, dtype=bool))
    tri = np.tril(np.ones((T, T), dtype=bool))
    for W in (T, T + 1, 5 * T):
        assert np.array_equal(O.dense_mask("sliding_window", T, T, window=W),
                              tri)
    assert np.array_equal(O.dense_mask("causal", T, T), tri)
    assert O.dense_mask("none", T, T).all()
    with pytest.raises(ValueError):
        O.dense_mask("sliding_window", T, T, window=0)


@pytest.mark.parametrize("T", [1, 2, 6, 17])
def test_local_window_is_the_symmetric_bound(T):
    # crackedaicode "State the boundary precisely": the symmetric variant
    # limits |i - j|. For square masks it is the causal
    # window together with its transpose, W = 1 is the identity, and W >= T
    # allows every pair.
    for W in (1, 2, 3, T, T + 4):
        loc = O.dense_mask("local_window", T, T, window=W)
        sw = O.dense_mask("sliding_window", T, T, window=W)
        assert np.array_equal(loc, loc.T)
        assert np.array_equal(loc, sw | sw.T)
        for i in range(T):
            assert np.flatnonzero(loc[i]).tolist() == list(
                range(max(0, i - W + 1), min(T, i + W)))
    assert np.array_equal(O.dense_mask("local_window", T, T, window=1),
                          np.eye(T, dtype=bool))
    assert O.dense_mask("local_window", T, T, window=T).all()
    with pytest.raises(ValueError):
        O.dense_mask("local_window", T, T, window=0)


def test_document_mask_is_block_diagonal_three_docs():
    # how-to "Mask 3": ids switch at 2048 and 5000 in an 8192 context
    doc = _three_doc_ids()
    S = len(doc)
    assert S == 8192
    starts = [0, 2048, 5000]
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([
        [0, 1, 2047, 2048, 2049, 4999, 5000, 5001, 8191],
        rng.integers(0, S, 64)]))
    m = O.dense_mask("document", S, S, doc_id=doc, rows=rows)
    for r, i in enumerate(rows):
        s = max(x for x in starts if x <= i)
        want = np.zeros(S, dtype=bool)
        want[s:i + 1] = True           # lower triangle inside its document
        assert np.array_equal(m[r], want), i


def test_document_mask_block_diagonal_small():
    lengths = [3, 5, 1, 7]
    doc = np.repeat(np.arange(4, dtype=np.int32), lengths)
    T = len(doc)
    m = O.dense_mask("document", T, T, doc_id=doc)
    want = np.zeros((T, T), dtype=bool)
    s = 0
    for L in lengths:
        want[s:s + L, s:s + L] = np.tril(np.ones((L, L), dtype=bool))
        s += L
    assert np.array_equal(m, want)


# --------------------------------------------------------- block counts
def _counts(bm):
    num = bm["kv_num_blocks"][0, 0].astype(int)
    full = bm["full_kv_num_blocks"][0, 0].astype(int)
    return num, full


def test_block_counts_closed_forms_small_configs():
    # c1: W = 64 over 256 tokens, 64-blocks. A block at block-distance k
    # holds pairs with i - j in [(k-1)*64 + 1, (k+1)*64 - 1]: k = 0 and 1 are
    # partial, k >= 2 empty -> 4 + 3 = 7 partial, 0 full.
    bm = O.create_block_mask("sliding_window", 1, 1, 256, 256, 64, 64,
                             window=64)
    num, full = _counts(bm)
    assert num.sum() == 7 and full.sum() == 0
    # causal with n blocks of equal size: n diagonal partial, n(n-1)/2 full
    for T, b in ((512, 128), (1024, 64), (8192, 128)):
        n = T // b
        bm = O.create_block_mask("causal", 1, 1, T, T, b, b)
        num, full = _counts(bm)
        assert num.sum() == n and full.sum() == n * (n - 1) // 2
        assert num.tolist() == [1] * n
        assert full.tolist() == list(range(n))


def test_block_counts_sliding_window_8k_seven_eighths_empty():
    # how-to "Mask 2" / "At a glance": W = 1024 over 8k leaves about 7/8 of
    # the blocks fully masked. Hand count with 128-blocks: row m has the
    # diagonal partial block, min(m, 7) full ones and one more partial block
    # at distance 8 when m >= 8.
    bm = O.create_block_mask("sliding_window", 1, 1, 8192, 8192, 128, 128,
                             window=1024)
    num, full = _counts(bm)
    n = 64
    assert num.tolist() == [1 + (m >= 8) for m in range(n)]
    assert full.tolist() == [min(m, 7) for m in range(n)]
    assert num.sum() == 120 and full.sum() == 420
    empty = n * n - num.sum() - full.sum()
    assert empty == 3556
    assert abs(empty / (n * n) - 7 / 8) < 0.01


@pytest.mark.slow
def test_block_counts_causal_16k_and_equal_docs_32k():
    bm = O.create_block_mask("causal", 1, 1, 16384, 16384, 128, 128)
    num, full = _counts(bm)
    assert num.sum() == 128 and full.sum() == 128 * 127 // 2
    # how-to "At a glance": 4 packed documents cost about 1/4 of one long
    # causal sequence. Equal documents of 8192 tokens = 64 blocks each:
    # 4 x (64 partial + 2016 full).
    doc = np.repeat(np.arange(4, dtype=np.int32), 8192)
    bm = O.create_block_mask("document", 1, 1, 32768, 32768, 128, 128,
                             doc_id=doc)
    num, full = _counts(bm)
    assert num.sum() == 256 and full.sum() == 8064
    causal_live = 256 + 256 * 255 // 2
    assert abs((num.sum() + full.sum()) / causal_live - 0.25) < 0.01


def test_block_mask_lists_are_permutations_and_partition():
    doc = np.repeat(np.arange(3, dtype=np.int32), [70, 101, 129])
    for kind, kw in (("causal", {}), ("sliding_window", {"window": 45}),
                     ("document", {"doc_id": doc}), ("none", {})):
        bm = O.create_block_mask(kind, 2, 3, 300, 300, 32, 64, **kw)
        nq, nk = bm["num_q_blocks"], bm["num_kv_blocks"]
        assert (nq, nk) == (10, 5)
        st = O.block_states(kind, 300, 300, 32, 64, **kw)
        for b in range(2):
            for h in range(3):
                for m in range(nq):
                    for key in ("kv_indices", "full_kv_indices"):
                        row = bm[key][b, h, m]
                        assert sorted(row.tolist()) == list(range(nk))
                    p = bm["kv_num_blocks"][b, h, m]
                    f = bm["full_kv_num_blocks"][b, h, m]
                    listed = set(bm["kv_indices"][b, h, m, :p].tolist())
                    flisted = set(bm["full_kv_indices"][b, h, m, :f].tolist())
                    assert not listed & flisted
                    assert listed == set(np.flatnonzero(st[m] == O.PARTIAL))
                    assert flisted == set(np.flatnonzero(st[m] == O.FULL))
        # ragged tiles (300 is not a multiple of 32 or 64) are never full
        assert not (st[-1] == O.FULL).any() and not (st[:, -1] == O.FULL).any()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_block_mask_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    for _ in range(6):
        ql = int(rng.integers(1, 40))
        kl = int(rng.integers(1, 40))
        bm_, bn_ = (int(x) for x in rng.choice([1, 2, 4, 8], size=2))
        W = int(rng.integers(1, 12))
        L = max(ql, kl)
        doc = np.sort(rng.integers(0, 4, size=L)).astype(np.int32)
        for kind in O.MASK_KINDS:
            sep = bool(rng.integers(0, 2))
            got = O.create_block_mask(kind, 1, 1, ql, kl, bm_, bn_, window=W,
                                      doc_id=doc, separate_full_blocks=sep)
            num, idx, fnum, fidx = brute.block_lists(
                kind, ql, kl, bm_, bn_, window=W, doc=doc.tolist(),
                separate_full_blocks=sep)
            assert got["kv_num_blocks"][0, 0].tolist() == num
            assert got["kv_indices"][0, 0].tolist() == idx
            if sep:
                assert got["full_kv_num_blocks"][0, 0].tolist() == fnum
                assert got["full_kv_indices"][0, 0].tolist() == fidx
            else:
                assert got["full_kv_num_blocks"] is None


def test_separate_full_blocks_false_lists_every_live_block():
    a = O.create_block_mask("causal", 1, 1, 512, 512, 128, 128)
    b = O.create_block_mask("causal", 1, 1, 512, 512, 128, 128,
                            separate_full_blocks=False)
    assert (b["kv_num_blocks"] == a["kv_num_blocks"]
            + a["full_kv_num_blocks"]).all()
    assert b["full_kv_indices"] is None


# ------------------------------------------------------------ attention
def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _mask_kw(kind, T, rng):
    if kind in ("sliding_window", "local_window"):
        return {"window": int(rng.integers(1, T + 2))}
    if kind == "document":
        return {"doc_id": np.sort(rng.integers(0, 3, T)).astype(np.int32)}
    return {}


def _nested(a):
    return a.tolist()


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("mask", O.MASK_KINDS)
@pytest.mark.parametrize("score", O.SCORE_KINDS)
def test_attention_matches_brute_force(seed, mask, score):
    rng = np.random.default_rng(100 * seed + 7)
    B, H, Hk, T, D = 1, 4, 2, 12, 5
    q = _rand(rng, B, H, T, D)
    k = _rand(rng, B, Hk, T, D)
    v = _rand(rng, B, Hk, T, D)
    kw = _mask_kw(mask, T, rng)
    cap = 1.7 if score == "softcap" else None
    o, l = O.attention(q, k, v, mask=mask, score=score, softcap=cap, **kw)
    bo, bl = brute.attention(_nested(q), _nested(k), _nested(v), mask=mask,
                             score=score, window=kw.get("window"),
                             doc=None if "doc_id" not in kw
                             else kw["doc_id"].tolist(), cap=cap)
    np.testing.assert_allclose(o, np.array(bo), rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, np.array(bl), rtol=0, atol=1e-12)


def test_row_chunks_match_brute_force():
    # The oracle evaluates the requested rows in chunks of at most
    # chunk_bytes of fp64 scores. Force three rows per chunk: every chunk
    # after the first (and a row subset whose chunk edges fall between
    # unevenly spaced rows) must give the one-chunk result, and the brute
    # force's values on those rows.
    rng = np.random.default_rng(4242)
    B, H, T, D = 1, 2, 13, 4
    q = _rand(rng, B, H, T, D)
    k = _rand(rng, B, H, T, D)
    v = _rand(rng, B, H, T, D)
    small = 8 * T * 3
    for mask, kw in (("causal", {}), ("sliding_window", {"window": 4})):
        bo, bl = brute.attention(_nested(q), _nested(k), _nested(v),
                                 mask=mask, window=kw.get("window"))
        bo, bl = np.array(bo), np.array(bl)
        for rows in (None, np.array([0, 2, 3, 5, 6, 7, 9, 11, 12])):
            o1, l1 = O.attention(q, k, v, mask=mask, rows=rows, **kw)
            oc, lc = O.attention(q, k, v, mask=mask, rows=rows,
                                 chunk_bytes=small, **kw)
            sel = np.arange(T) if rows is None else rows
            # (the matrix product may round differently per chunk shape)
            np.testing.assert_allclose(oc, o1, rtol=0, atol=1e-14)
            np.testing.assert_allclose(lc, l1, rtol=0, atol=1e-14)
            np.testing.assert_allclose(oc, bo[:, :, sel], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lc, bl[:, :, sel], rtol=0, atol=1e-12)


def test_per_batch_document_ids():
    # a batch of packed sequences: entry b uses its own ids. Brute force
    # (independent loops) agrees, each entry equals the shared-id
    # computation on its ids, and an entry that is one document is causal.
    rng = np.random.default_rng(77)
    B, H, T, D = 3, 2, 13, 4
    q = _rand(rng, B, H, T, D)
    k = _rand(rng, B, H, T, D)
    v = _rand(rng, B, H, T, D)
    doc = np.stack([np.sort(rng.integers(0, 3, T)),
                    np.sort(rng.integers(0, 5, T)),
                    np.zeros(T, dtype=np.int64)]).astype(np.int32)
    o, l = O.attention(q, k, v, mask="document", doc_id=doc)
    bo, bl = brute.attention(_nested(q), _nested(k), _nested(v),
                             mask="document", doc=doc.tolist())
    np.testing.assert_allclose(o, np.array(bo), rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, np.array(bl), rtol=0, atol=1e-12)
    for b in range(B):
        ob, lb = O.attention(q[b:b + 1], k[b:b + 1], v[b:b + 1],
                             mask="document", doc_id=doc[b])
        assert np.array_equal(o[b:b + 1], ob) and np.array_equal(l[b:b + 1], lb)
    oc, lc = O.attention(q[2:], k[2:], v[2:], mask="causal")
    np.testing.assert_allclose(o[2:], oc, rtol=0, atol=1e-14)
    # block masks: one set of rows per entry, each the entry's own mask
    bm = O.create_block_mask("document", B, H, T, T, 4, 4, doc_id=doc)
    assert bm["kv_num_blocks"].shape == (B, H, 4)
    for b in range(B):
        one = O.create_block_mask("document", 1, H, T, T, 4, 4, doc_id=doc[b])
        for key in ("kv_num_blocks", "kv_indices", "full_kv_num_blocks",
                    "full_kv_indices"):
            assert np.array_equal(bm[key][b], one[key][0])
        num, idx, fnum, fidx = brute.block_lists("document", T, T, 4, 4,
                                                 doc=doc[b].tolist())
        assert bm["kv_num_blocks"][b, 0].tolist() == num
        assert bm["full_kv_indices"][b, 1].tolist() == fidx


def test_attention_rectangular_and_row_subset():
    rng = np.random.default_rng(5)
    q = _rand(rng, 1, 2, 9, 4)
    k = _rand(rng, 1, 2, 14, 4)
    v = _rand(rng, 1, 2, 14, 3)
    for mask in ("causal", "none", "sliding_window"):
        kw = {"window": 3} if mask == "sliding_window" else {}
        o, l = O.attention(q, k, v, mask=mask, score="alibi", **kw)
        bo, bl = brute.attention(_nested(q), _nested(k), _nested(v),
                                 mask=mask, score="alibi",
                                 window=kw.get("window"))
        np.testing.assert_allclose(o, np.array(bo), atol=1e-12, rtol=0)
        np.testing.assert_allclose(l, np.array(bl), atol=1e-12, rtol=0)
        rows = np.array([8, 0, 3])
        os_, ls_ = O.attention(q, k, v, mask=mask, score="alibi", rows=rows,
                               **kw)
        np.testing.assert_array_equal(os_, o[:, :, rows])
        np.testing.assert_array_equal(ls_, l[:, :, rows])


def test_empty_rows_give_zero_and_minus_inf():
    # a query whose document starts after every key: no allowed key
    rng = np.random.default_rng(3)
    q = _rand(rng, 1, 1, 6, 4)
    k = _rand(rng, 1, 1, 6, 4)
    v = _rand(rng, 1, 1, 6, 4)
    o, l = O.attention(q, k[:, :, :2], v[:, :, :2], mask="sliding_window",
                       window=2)
    assert np.isneginf(l[0, 0, 3:]).all() and (o[0, 0, 3:] == 0).all()
    assert np.isfinite(l[0, 0, :3]).all()


def test_sdpa_library_cross_check():
    # torch's CPU scaled_dot_product_attention (fp64) with a boolean mask,
    # and with ALiBi as an additive float mask, is the same definition
    rng = np.random.default_rng(11)
    B, H, T, D = 2, 3, 37, 8
    q = _rand(rng, B, H, T, D)
    k = _rand(rng, B, H, T, D)
    v = _rand(rng, B, H, T, D)
    doc = np.sort(rng.integers(0, 4, T)).astype(np.int32)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    for mask, kw in (("causal", {}), ("sliding_window", {"window": 6}),
                     ("document", {"doc_id": doc}), ("none", {})):
        o, _ = O.attention(q, k, v, mask=mask, **kw)
        m = torch.from_numpy(O.dense_mask(mask, T, T, **kw))
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, attn_mask=m)
        np.testing.assert_allclose(o, ref.numpy(), atol=1e-12, rtol=0)
    # ALiBi, written here as the additive bias -slope_h * (i - j) on top of
    # the causal -inf mask
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    bias = np.stack([-(2.0 ** (-8.0 * (h + 1) / H)) * (i - j)
                     for h in range(H)])
    bias = np.where(i >= j, bias, -np.inf)[None]
    o, _ = O.attention(q, k, v, mask="causal", score="alibi")
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(bias))
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12, rtol=0)
    # grouped heads: torch repeats each key head over consecutive query heads
    kg, vg = tk[:, :1].contiguous(), tv[:, :1].contiguous()
    o, _ = O.attention(q, kg.numpy(), vg.numpy(), mask="causal")
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, kg, vg, is_causal=True, enable_gqa=True)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12, rtol=0)
    # explicit scale
    o, _ = O.attention(q, k, v, mask="none", scale=0.3)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv,
                                                           scale=0.3)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12, rtol=0)


def _n_allowed(mask, T, kw):
    i = np.arange(T)
    if mask == "none":
        return np.full(T, T)
    if mask == "causal":
        return i + 1
    if mask == "sliding_window":
        return np.minimum(i + 1, kw["window"])
    if mask == "local_window":
        # W - 1 keys on each side of the diagonal, cut at both sequence ends
        return (np.minimum(i, kw["window"] - 1)
                + np.minimum(T - 1 - i, kw["window"] - 1) + 1)
    doc = kw["doc_id"]
    start = np.array([np.flatnonzero(doc == doc[t])[0] for t in range(T)])
    return i - start + 1


@pytest.mark.parametrize("mask", O.MASK_KINDS)
def test_rows_sum_to_one_and_uniform_weights(mask):
    rng = np.random.default_rng(21)
    B, H, T, D = 1, 2, 29, 6
    kw = _mask_kw(mask, T, rng)
    q = _rand(rng, B, H, T, D)
    k = _rand(rng, B, H, T, D)
    # V = ones: every output row is exactly a convex combination of ones
    for score in O.SCORE_KINDS:
        o, _ = O.attention(q, k, np.ones((B, H, T, D)), mask=mask,
                           score=score, softcap=2.0, **kw)
        np.testing.assert_allclose(o, 1.0, atol=1e-13, rtol=0)
    # K = 0 and no score_mod: weights are uniform over the n_i allowed keys,
    # so LSE_i = ln n_i and O_i is the mean of the allowed values
    v = _rand(rng, B, H, T, D)
    o, l = O.attention(q, np.zeros((B, H, T, D)), v, mask=mask, **kw)
    n = _n_allowed(mask, T, kw)
    np.testing.assert_allclose(l[0, 0], np.log(n), atol=1e-13, rtol=0)
    allowed = O.dense_mask(mask, T, T, **kw)
    means = np.stack([v[0, 1][allowed[t]].mean(axis=0) for t in range(T)])
    np.testing.assert_allclose(o[0, 1], means, atol=1e-13, rtol=0)


def test_identity_values_expose_exact_zero_weights():
    # V = I (T <= D): O is the weight matrix itself, masked entries exactly 0
    rng = np.random.default_rng(4)
    T = 10
    q = _rand(rng, 1, 1, T, T)
    k = _rand(rng, 1, 1, T, T)
    v = np.eye(T)[None, None]
    o, _ = O.attention(q, k, v, mask="sliding_window", window=4)
    allowed = O.dense_mask("sliding_window", T, T, window=4)
    assert (o[0, 0][~allowed] == 0).all()
    assert (o[0, 0][allowed] > 0).all()
    np.testing.assert_allclose(o[0, 0].sum(axis=1), 1.0, atol=1e-14)


def test_alibi_closed_form():
    # K = 0, causal, ALiBi: s_ij = -slope_h (i - j), so
    # LSE_i = ln sum_{d=0..i} e^{-slope d} = ln((1 - e^{-slope (i+1)}) /
    #                                          (1 - e^{-slope}))
    B, H, T, D = 1, 8, 50, 4
    rng = np.random.default_rng(8)
    q = _rand(rng, B, H, T, D)
    o, l = O.attention(q, np.zeros((B, H, T, D)), np.ones((B, H, T, D)),
                       mask="causal", score="alibi")
    i = np.arange(T)
    for h in range(H):
        a = 2.0 ** (-8.0 * (h + 1) / H)
        want = np.log((1 - np.exp(-a * (i + 1))) / (1 - np.exp(-a)))
        np.testing.assert_allclose(l[0, h], want, atol=1e-12, rtol=0)
    # the slope schedule: head 0 of 8 heads has slope 1/2, the last 1/256
    assert O.alibi_slope(0, 8) == 0.5 and O.alibi_slope(7, 8) == 2.0 ** -8


@pytest.mark.parametrize("cap", [0.5, 3.0, 50.0])
def test_softcap_closed_form(cap):
    # q . k == a * b for every pair (Q = a e1, K = b e1):
    # LSE_i = cap * tanh(scale * a * b / cap) + ln n_i
    T, D, a, bb = 20, 16, 3.0, 2.5
    q = np.zeros((1, 1, T, D))
    q[..., 0] = a
    k = np.zeros((1, 1, T, D))
    k[..., 0] = bb
    v = np.random.default_rng(0).standard_normal((1, 1, T, D))
    _, l = O.attention(q, k, v, mask="causal", score="softcap", softcap=cap)
    scale = 1 / math.sqrt(D)
    want = cap * math.tanh(scale * a * bb / cap) + np.log(np.arange(T) + 1)
    np.testing.assert_allclose(l[0, 0], want, atol=1e-12, rtol=0)
    # cap -> infinity reduces to no score_mod
    o1, l1 = O.attention(q, k, v, mask="causal", score="softcap",
                         softcap=1e9)
    o0, l0 = O.attention(q, k, v, mask="causal")
    np.testing.assert_allclose(l1, l0, atol=1e-9)


@pytest.mark.parametrize("score", O.SCORE_KINDS)
def test_single_key_rows(score):
    # W = 1: every query sees only itself, O_i = v_i exactly and LSE_i is the
    # modified scaled score of the pair (i, i)
    rng = np.random.default_rng(9)
    B, H, T, D = 1, 2, 17, 8
    q = _rand(rng, B, H, T, D)
    k = _rand(rng, B, H, T, D)
    v = _rand(rng, B, H, T, D)
    o, l = O.attention(q, k, v, mask="sliding_window", window=1,
                       score=score, softcap=4.0)
    assert np.array_equal(o, v)
    s = (q * k).sum(-1) / math.sqrt(D)
    if score == "softcap":
        s = 4.0 * np.tanh(s / 4.0)
    np.testing.assert_allclose(l, s, atol=1e-13, rtol=0)


def test_masked_positions_do_not_matter():
    # crackedaicode "Build and apply the mask": changing a position outside
    # the window leaves that query's output unchanged (here bit-identical)
    rng = np.random.default_rng(12)
    B, H, T, D, W = 1, 2, 24, 8, 5
    q = _rand(rng, B, H, T, D)
    k = _rand(rng, B, H, T, D)
    v = _rand(rng, B, H, T, D)
    o, l = O.attention(q, k, v, mask="sliding_window", window=W)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 0] += 10.0
    v2[:, :, 0] -= 3.0
    o2, l2 = O.attention(q, k2, v2, mask="sliding_window", window=W)
    assert np.array_equal(o[:, :, W:], o2[:, :, W:])
    assert np.array_equal(l[:, :, W:], l2[:, :, W:])
    assert not np.array_equal(o[:, :, 0], o2[:, :, 0])
