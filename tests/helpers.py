"""Shared helpers for the GPU tests: device transfer, the oracle side of a
case, deterministic row samples and the comparison bar."""
from __future__ import annotations

import numpy as np
import torch

import workloads as WL
from oracle import oracle as O

# Output tolerances (max-abs, on O and on LSE) against the fp64 oracle.
TOL = {"bf16": 2e-2, "fp32": 1e-4}

MASK_ARG = {"none": "none", "causal": "causal",
            "sliding_window": "sliding_window", "document": "document"}


def torch_dtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def sample_rows(q_len, block, doc_id=None, n_random=64, seed=0):
    """Deterministic query-row sample: ends, block boundaries, document
    boundaries and seeded random rows."""
    rows = {0, 1, q_len - 1, q_len - 2}
    nqb = -(-q_len // block)
    step = max(1, nqb // 16)
    for m in range(0, nqb, step):
        rows.update({m * block, m * block + block - 1, m * block + block // 2})
    if doc_id is not None:
        starts = np.flatnonzero(np.diff(doc_id)) + 1
        for s in starts:
            rows.update({int(s) - 1, int(s), int(s) + 1})
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, q_len, n_random).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < q_len), dtype=np.int64)


def oracle_case(q, k, v, w: WL.Workload, doc=None, rows=None, score=None,
                cap=None):
    score = w.score if score is None else score
    cap = w.softcap if cap is None else cap
    return O.attention(q, k, v, mask=w.mask, score=score, scale=w.scale,
                       window=w.window, doc_id=doc, softcap=cap, rows=rows)


def assert_close(o_gpu, lse_gpu, o_ref, lse_ref, tol, what=""):
    o = o_gpu.detach().float().cpu().double().numpy()
    l = lse_gpu.detach().cpu().double().numpy()
    assert o.shape == o_ref.shape, (o.shape, o_ref.shape)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(l), fin), f"{what}: -inf rows differ"
    assert (l[~fin] == -np.inf).all()
    err_o = np.abs(o - o_ref).max() if o.size else 0.0
    err_l = np.abs(l[fin] - lse_ref[fin]).max() if fin.any() else 0.0
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    assert err_o <= tol, f"{what}: max |O - oracle| = {err_o:.3g} > {tol}"
    assert err_l <= tol, f"{what}: max |LSE - oracle| = {err_l:.3g} > {tol}"
    return err_o, err_l


def caller_lists(kind, mask, q_len, kv_len, block_m, block_n, window=None,
                 doc_id=None):
    """Index lists for BlockMask.from_kv_blocks, built on the host:
    "oracle": the oracle's create_block_mask arrays; "no_skip": every key
    block of every row listed as partial (no full list); "clamped": the
    oracle's arrays with out-of-range entries after each row's partial
    blocks and a partial count above NKVB (the kernels clamp the count and
    skip the entries). Returns (num, idx, fnum, fidx), fnum/fidx None for
    no_skip."""
    ref = O.create_block_mask(mask, 1, 1, q_len, kv_len, block_m, block_n,
                              window=window, doc_id=doc_id)
    nqb, nkvb = ref["kv_indices"].shape[2], ref["kv_indices"].shape[3]
    if kind == "no_skip":
        num = np.full((1, 1, nqb), nkvb, dtype=np.int32)
        idx = np.broadcast_to(np.arange(nkvb, dtype=np.int32),
                              (1, 1, nqb, nkvb)).copy()
        return num, idx, None, None
    num = ref["kv_num_blocks"].astype(np.int32).copy()
    idx = ref["kv_indices"].astype(np.int32).copy()
    fnum = ref["full_kv_num_blocks"].astype(np.int32).copy()
    fidx = ref["full_kv_indices"].astype(np.int32).copy()
    if kind == "clamped":
        bad = np.array([-1, nkvb, nkvb + 7, 2 ** 31 - 1, -(2 ** 31)],
                       dtype=np.int64)
        for m in range(nqb):
            c = int(num[0, 0, m])
            idx[0, 0, m, c:] = np.resize(bad, nkvb - c).astype(np.int32)
            num[0, 0, m] = nkvb + 3 + m
    return num, idx, fnum, fidx
