"""Pins of the oracle's masked softmax over materialised scores: it equals
the weights of the separately pinned dense attention, reproduces the
minimum-select chain it replaces, and meets closed forms."""
import numpy as np
import pytest
import torch

from oracle import oracle as O


@pytest.mark.parametrize("mask", O.MASK_KINDS)
def test_masked_softmax_times_v_is_attention(mask):
    # P = masked_softmax(scale q k^T) gives attention's O = P v, for a chunk
    # of queries that starts after q_offset earlier tokens
    rng = np.random.default_rng(5)
    Q, K, D, off = 7, 12, 4, 5
    q = rng.standard_normal((1, 1, Q + off, D))
    k = rng.standard_normal((1, 1, K, D))
    v = rng.standard_normal((1, 1, K, D))
    kw = {"window": 3} if "window" in mask else {}
    if mask == "document":
        kw = {"doc_id": np.array([0, 0, 0, 1, 1, 1, 1, 2, 2, 2, 2, 2])}
    s = (q[0, 0, off:] @ k[0, 0].T) / np.sqrt(D)
    p = O.masked_softmax(s, mask, q_offset=off, **kw)
    o_ref, _ = O.attention(q, k, v, mask=mask, rows=np.arange(off, off + Q), **kw)
    np.testing.assert_allclose(p @ v[0, 0], o_ref[0, 0], atol=1e-13)


def test_masked_softmax_matches_the_minimum_select_chain():
    # torch's chain: where(mask, s, finfo(bf16).min) then softmax, in fp64
    rng = np.random.default_rng(6)
    s = rng.standard_normal((3, 9, 9)) * 5
    mask = np.tril(np.ones((9, 9), dtype=bool))
    t = torch.from_numpy(s)
    chain = torch.softmax(torch.where(torch.from_numpy(mask), t,
                                      torch.tensor(float(torch.finfo(torch.bfloat16).min),
                                                   dtype=torch.float64)), dim=-1)
    p = np.stack([O.masked_softmax(s[b], "causal") for b in range(3)])
    np.testing.assert_allclose(p, chain.numpy(), atol=1e-15)
    assert (p[:, ~mask] == 0).all() and (chain.numpy()[:, ~mask] == 0).all()


def test_masked_softmax_closed_forms():
    s = np.zeros((6, 6))
    # constant scores: uniform over the allowed keys (causal: 1/(i+1))
    p = O.masked_softmax(s, "causal")
    np.testing.assert_allclose(p, np.tril(np.ones((6, 6))) / np.arange(1, 7)[:, None])
    # rows sum to one; masked entries exactly zero
    rng = np.random.default_rng(7)
    s = rng.standard_normal((5, 11)) * 3
    p = O.masked_softmax(s, "sliding_window", q_offset=6, window=4)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-15)
    allowed = O.dense_mask("sliding_window", 11, 11, window=4)[6:]
    assert (p[~allowed] == 0).all() and (p[allowed] > 0).all()
    # a row with no allowed entry: zeros (offset pushes the window past K)
    p = O.masked_softmax(s, "sliding_window", q_offset=20, window=3)
    assert (p == 0).all()
    # single allowed entry: exactly one
    p = O.masked_softmax(s, "sliding_window", q_offset=0, window=1)
    np.testing.assert_array_equal(p, np.eye(5, 11))
