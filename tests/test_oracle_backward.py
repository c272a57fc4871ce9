"""Pins of the oracle's backward (dQ, dK, dV): central finite differences of
the oracle's own forward (an independent route: no formula in common with
the chain rule), torch fp64 autograd through a dense implementation built
from library ops, and special cases with closed forms."""
import numpy as np
import pytest
import torch

from oracle import oracle as O


def _case(rng, B=1, H=2, Hk=1, T=7, D=3):
    q = rng.standard_normal((B, H, T, D))
    k = rng.standard_normal((B, Hk, T, D))
    v = rng.standard_normal((B, Hk, T, D))
    do = rng.standard_normal((B, H, T, D))
    return q, k, v, do


def _kw(mask, T, rng):
    if mask in ("sliding_window", "local_window"):
        return {"window": 3}
    if mask == "document":
        return {"doc_id": np.sort(rng.integers(0, 3, T)).astype(np.int32)}
    return {}


@pytest.mark.parametrize("mask", O.MASK_KINDS)
@pytest.mark.parametrize("score", O.SCORE_KINDS)
def test_backward_matches_finite_differences(mask, score):
    rng = np.random.default_rng(hash((mask, score)) % 2**32)
    q, k, v, do = _case(rng)
    kw = _kw(mask, q.shape[2], rng)
    cap = 1.4

    def loss(q_, k_, v_):
        o, _ = O.attention(q_, k_, v_, mask=mask, score=score, softcap=cap,
                           **kw)
        return float((o * do).sum())

    grads = O.attention_backward(q, k, v, do, mask=mask, score=score,
                                 softcap=cap, **kw)
    eps = 1e-6
    for which, g in enumerate(grads):
        args = [q, k, v]
        fd = np.zeros_like(g)
        for idx in np.ndindex(g.shape):
            a = [x.copy() for x in args]
            a[which][idx] += eps
            up = loss(*a)
            a[which][idx] -= 2 * eps
            fd[idx] = (up - loss(*a)) / (2 * eps)
        np.testing.assert_allclose(g, fd, rtol=0, atol=1e-7)


def _torch_dense(q, k, v, mask_b, score, cap, slopes, scale):
    # dense masked attention from library ops, for autograd
    t = scale * torch.matmul(q, k.transpose(-1, -2))
    if score == "softcap":
        s = cap * torch.tanh(t / cap)
    elif score == "alibi":
        T, S = t.shape[-2:]
        dist = (torch.arange(T)[:, None] - torch.arange(S)[None, :]).double()
        s = t - slopes[:, None, None] * dist
    else:
        s = t
    s = s.masked_fill(~mask_b, float("-inf"))
    p = torch.softmax(s, dim=-1)
    p = torch.nan_to_num(p, nan=0.0)          # rows with no allowed key
    return torch.matmul(p, v)


@pytest.mark.parametrize("mask", ["causal", "document", "none",
                                  "sliding_window"])
@pytest.mark.parametrize("score", O.SCORE_KINDS)
def test_backward_matches_torch_autograd(mask, score):
    rng = np.random.default_rng(5)
    B, H, T, D = 1, 3, 9, 4
    q, k, v, do = _case(rng, B, H, H, T, D)
    kw = _kw(mask, T, rng)
    cap, scale = 2.0, 0.7
    dq, dk, dv = O.attention_backward(q, k, v, do, mask=mask, score=score,
                                      softcap=cap, scale=scale, **kw)
    allowed = torch.from_numpy(O.dense_mask(mask, T, T, **kw))
    slopes = torch.tensor([O.alibi_slope(h, H) for h in range(H)],
                          dtype=torch.float64)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = _torch_dense(tq, tk, tv, allowed, score, cap, slopes, scale)
    o.backward(torch.from_numpy(do))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=0, atol=1e-12)


def test_backward_special_cases():
    rng = np.random.default_rng(9)
    B, H, T, D = 1, 2, 8, 3
    q, k, v, do = _case(rng, B, H, H, T, D)
    # dO = 0: every gradient is 0
    for g in O.attention_backward(q, k, v, np.zeros_like(do), mask="causal"):
        assert not g.any()
    # W = 1: each row attends only to itself (P = I): dV = dO, dQ = dK = 0
    dq, dk, dv = O.attention_backward(q, k, v, do, mask="sliding_window",
                                      window=1)
    np.testing.assert_allclose(dv, do, atol=1e-15)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
    # K = 0, causal: uniform weights 1/(i+1); dV_j = sum_{i>=j} dO_i/(i+1)
    dq, dk, dv = O.attention_backward(q, np.zeros_like(k), v, do,
                                      mask="causal")
    w = 1.0 / np.arange(1, T + 1)
    want = np.stack([(do[0, 0, j:] * w[j:, None]).sum(axis=0)
                     for j in range(T)])
    np.testing.assert_allclose(dv[0, 0], want, atol=1e-14)
    # grouped heads: dK / dV of a key head sum over its query heads
    qg, kg, vg, dog = _case(rng, 1, 4, 2, T, D)
    dq1, dk1, dv1 = O.attention_backward(qg, kg, vg, dog, mask="causal")
    for hk in range(2):
        parts = [O.attention_backward(qg[:, h:h + 1], kg[:, hk:hk + 1],
                                      vg[:, hk:hk + 1], dog[:, h:h + 1],
                                      mask="causal") for h in (2 * hk, 2 * hk + 1)]
        np.testing.assert_allclose(dv1[:, hk], parts[0][2][:, 0] + parts[1][2][:, 0],
                                   atol=1e-13)


@pytest.mark.parametrize("mask", O.MASK_KINDS)
@pytest.mark.parametrize("score", O.SCORE_KINDS)
def test_backward_row_sample_matches_all_rows(mask, score):
    # rows=: the sampled rows' dQ equals those rows of the full gradient
    # (each row's dQ is a function of that row alone), and dK / dV of keys
    # seen only by sampled rows equal the full gradients; unsorted and
    # boundary rows
    rng = np.random.default_rng(7)
    q, k, v, do = _case(rng, B=2, H=4, Hk=2, T=11, D=5)
    kw = _kw(mask, q.shape[2], rng)
    full = O.attention_backward(q, k, v, do, mask=mask, score=score,
                                softcap=1.7, **kw)
    rows = np.array([10, 0, 3, 7])
    dq, _, _ = O.attention_backward(q, k, v, do, mask=mask, score=score,
                                    softcap=1.7, rows=rows, **kw)
    np.testing.assert_allclose(dq, full[0][:, :, rows], rtol=1e-12, atol=1e-14)
    # the last three keys: every row allowed to see them is in `tail`
    T = q.shape[2]
    cols = np.arange(T - 3, T)
    seen = O.mask_mod(mask, np.arange(T)[:, None], cols[None, :],
                      window=kw.get("window"), doc_id=kw.get("doc_id")).any(axis=1)
    tail = np.flatnonzero(seen)
    part = O.attention_backward(q, k, v, do, mask=mask, score=score,
                                softcap=1.7, rows=tail, **kw)
    for g, r in zip(part[1:], full[1:]):
        np.testing.assert_allclose(g[:, :, cols], r[:, :, cols], rtol=1e-12,
                                   atol=1e-14)
    with pytest.raises(ValueError):
        O.attention_backward(q, k, v, do, rows=[1, 1])
