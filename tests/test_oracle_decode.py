"""Pins of the oracle's paged decode step (``oracle.decode_paged``): it must
equal the separately pinned dense ``attention`` evaluated at the newest row
of each sequence, whatever the physical order of the pages, and satisfy
closed forms."""
import numpy as np
import pytest

from oracle import oracle as O


def _paged_case(rng, B=3, H=4, H_kv=2, D=5, page=4, lens=(9, 1, 13),
                pool_extra=3):
    n_pages = [-(-L // page) for L in lens]
    P = sum(n_pages) + pool_extra
    k_pages = rng.standard_normal((P, page, H_kv, D))
    v_pages = rng.standard_normal((P, page, H_kv, D))
    perm = rng.permutation(P)          # physical pages in shuffled order
    maxp = max(n_pages)
    table = np.full((B, maxp), -7, dtype=np.int32)   # unused slots: junk
    at = 0
    for b, n in enumerate(n_pages):
        table[b, :n] = perm[at:at + n]
        at += n
    q = rng.standard_normal((B, H, D))
    return q, k_pages, v_pages, table, np.array(lens, dtype=np.int32)


def _mask_kw(mask, rng, max_len, B):
    if mask in ("sliding_window", "local_window"):
        return {"window": 3}
    if mask == "document":
        return {"doc_id": np.sort(rng.integers(0, 3, (B, max_len)), axis=1)}
    return {}


@pytest.mark.parametrize("mask", O.MASK_KINDS)
@pytest.mark.parametrize("score", O.SCORE_KINDS)
def test_decode_equals_last_row_of_dense_attention(mask, score):
    rng = np.random.default_rng(hash((mask, score)) % 2**32)
    q, kp, vp, table, lens = _paged_case(rng)
    B, H, D = q.shape
    kw = _mask_kw(mask, rng, int(lens.max()), B)
    o, lse = O.decode_paged(q, kp, vp, table, lens, mask=mask, score=score,
                            softcap=2.5, **kw)
    for b in range(B):
        L = int(lens[b])
        # the same tokens laid out contiguously, the query at row L - 1
        k = np.stack([O.paged_rows(kp, table[b], L)])
        v = np.stack([O.paged_rows(vp, table[b], L)])
        qf = np.zeros((1, H, L, D))
        qf[0, :, L - 1] = q[b]
        doc = kw.get("doc_id")
        o_ref, l_ref = O.attention(
            qf, k, v, mask=mask, score=score, softcap=2.5,
            window=kw.get("window"),
            doc_id=None if doc is None else doc[b][:L], rows=[L - 1])
        np.testing.assert_allclose(o[b], o_ref[0, :, 0], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse[b], l_ref[0, :, 0], rtol=1e-13, atol=1e-13)


def test_paged_rows_is_the_gather_by_page_table():
    # pages laid out in order equal the contiguous cache; a table that
    # permutes the pool reads the same tokens
    rng = np.random.default_rng(1)
    L, page, Hk, D = 10, 4, 2, 3
    cache = rng.standard_normal((12, Hk, D))        # 3 pages, 2 rows spare
    pages = cache.reshape(3, page, Hk, D)
    got = O.paged_rows(pages, np.array([0, 1, 2]), L)
    np.testing.assert_array_equal(got, cache[:L].transpose(1, 0, 2))
    perm = np.array([2, 0, 1])
    pool = np.empty_like(pages)
    pool[perm] = pages
    np.testing.assert_array_equal(O.paged_rows(pool, perm, L), got)


def test_page_order_and_unused_rows_do_not_matter():
    rng = np.random.default_rng(2)
    q, kp, vp, table, lens = _paged_case(rng)
    o1, l1 = O.decode_paged(q, kp, vp, table, lens, mask="causal",
                            score="alibi")
    # move every page to another physical slot and remap the table
    P = kp.shape[0]
    perm = rng.permutation(P)
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    t2 = table.copy()
    valid = t2 >= 0
    t2[valid] = perm[t2[valid]]
    o2, l2 = O.decode_paged(q, kp2, vp2, t2, lens, mask="causal",
                            score="alibi")
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    # rows past each sequence's length are never read
    kp3, vp3 = kp.copy(), vp.copy()
    for b, L in enumerate(lens):
        page = kp.shape[1]
        last = table[b, (L - 1) // page]
        kp3[last, (L - 1) % page + 1:] = np.nan
        vp3[last, (L - 1) % page + 1:] = np.nan
    o3, l3 = O.decode_paged(q, kp3, vp3, table, lens, mask="causal",
                            score="alibi")
    np.testing.assert_array_equal(o1, o3)
    np.testing.assert_array_equal(l1, l3)


def test_decode_closed_forms():
    rng = np.random.default_rng(3)
    q, kp, vp, table, lens = _paged_case(rng)
    # V = 1: every output is 1
    o, _ = O.decode_paged(q, kp, np.ones_like(vp), table, lens)
    np.testing.assert_allclose(o, 1.0, atol=1e-15)
    # K = 0: uniform weights, LSE = ln(number of allowed keys)
    _, lse = O.decode_paged(q, np.zeros_like(kp), vp, table, lens)
    np.testing.assert_allclose(lse, np.log(lens)[:, None] * np.ones(4), atol=1e-15)
    _, lse = O.decode_paged(q, np.zeros_like(kp), vp, table, lens,
                            mask="sliding_window", window=3)
    np.testing.assert_allclose(lse, np.log(np.minimum(lens, 3))[:, None] * np.ones(4),
                               atol=1e-15)
    # window 1: the newest token's own value
    o, _ = O.decode_paged(q, kp, vp, table, lens, mask="sliding_window",
                          window=1)
    for b, L in enumerate(lens):
        last = O.paged_rows(vp, table[b], L)[:, L - 1]
        np.testing.assert_allclose(o[b], np.repeat(last, 2, axis=0), atol=1e-15)
    # an empty sequence gives O = 0, LSE = -inf
    lens0 = lens.copy()
    lens0[1] = 0
    o, lse = O.decode_paged(q, kp, vp, table, lens0)
    assert (o[1] == 0).all() and np.isneginf(lse[1]).all()
