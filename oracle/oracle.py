"""Oracle: plain, slow, fp64 CPU definition of block-sparse masked attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The
product path (``block_sparse_masked_fa_amd``) never does, and this module
imports nothing from it: the two share no code. Inputs come from the caller
(the seeded generator in ``workloads.py``), already rounded to the dtype the
GPU sees; this module upcasts them to fp64 (exact for bf16 and fp32).

What is computed, and where the pages fix it
---------------------------------------------
* ``mask_mod(b, h, q_idx, kv_idx) -> bool``, True = the pair is allowed
  ("How to Use FlexAttention on Apple Silicon", section "The two hooks";
  tensorplay ``create_block_mask`` page, parameter ``mask_mod``).
  Built-ins:

  - causal, ``q_idx >= kv_idx`` (how-to, "Mask 1: causal");
  - sliding window, ``0 <= q_idx - kv_idx < W``: the window counts the
    diagonal, allowed keys run from ``max(0, i - W + 1)`` to ``i``
    (how-to, "Mask 2"; crackedaicode "Sliding-Window Self-Attention",
    section "State the boundary precisely");
  - document, causal and ``doc[q_idx] == doc[kv_idx]`` with one int32 id
    array indexed by both positions (how-to, "Mask 3: document-packed");
    a batch of packed sequences may give each entry b its own array
    ``doc[b]`` (mask_mod receives b, tensorplay page, parameter mask_mod);
  - local window, ``|q_idx - kv_idx| < W``: the symmetric variant, which the
    crackedaicode page mentions in passing as limiting |i - j| rather than
    i - j (same section);
  - none: every pair allowed (how-to, "The two hooks": either hook may be
    omitted).

* ``score_mod(score, b, h, q_idx, kv_idx) -> score`` on live positions
  (how-to, "The two hooks" and "Bonus: a score_mod for soft-capping"):

  - soft-cap ``cap * tanh(score / cap)`` (how-to, "Bonus");
  - ALiBi, an additive distance penalty ``score - slope_h * (q_idx - kv_idx)``
    with ``slope_h = 2**(-8 (h + 1) / H)``. The pages name ALiBi as an
    additive bias (how-to "The two hooks"; frontiernews "What Attention
    Patterns Does FlexAttention Support?") but print no formula; this is
    the geometric slope schedule of the ALiBi workload definition.

* Attention, per (b, h, i): scores ``s_j = score_mod(scale * q_i . k_j)``
  over every key (the dense form of crackedaicode, "A dense mask does not
  make the calculation sparse"); the mask keeps ``A_i = {j : mask_mod}``
  (the score_mod acts "on what survives", how-to "Bonus"); then the plain
  softmax ``w_j = exp(s_j - max_{A_i} s) / sum_{A_i} exp(s - max)`` over
  ``A_i``, ``O_i = sum_j w_j v_j``, and ``LSE_i = max + ln sum exp(s - max)``
  (natural log). A row with empty ``A_i`` gives ``O_i = 0`` and
  ``LSE_i = -inf``. No page states the logsumexp output, the scale, or the
  empty-row value: the scale is 1/sqrt(D) unless given (the API mirrors
  scaled_dot_product_attention, how-to FAQ "What tensor shape does
  flex_attention expect?"), and the rest are the plain readings above.

* Block mask (tensorplay ``create_block_mask``, parameters ``BLOCK_SIZE``
  and ``separate_full_blocks``; how-to "The two mistakes": only *fully*
  masked blocks can be skipped). For each query block m and key block n,
  count the allowed in-range pairs ``c`` of the tile: ``c == 0`` is empty,
  ``c == BM * BN`` is full, anything else is partial. A tile cut by the end
  of the sequence is never full. With ``separate_full_blocks`` the partial
  blocks go to ``kv_indices`` and the full ones to ``full_kv_indices``;
  without it every non-empty block is listed in ``kv_indices``. Each row of
  an index array lists its blocks in ascending n and then the remaining
  block numbers in ascending n, so every row is a permutation of
  ``0..NKVB-1`` (the pages fix no order or padding; this stable partition is
  the plain reading).

* Masked softmax over materialised scores (``masked_softmax``): the
  materialising fallback's compare / select / softmax chain as one
  operation (MLX pull request "Fuse the causal mask into the SDPA fallback
  softmax"). Pinned in ``tests/test_oracle_masked_softmax.py``.

* Decode over a paged cache (``decode_paged``): one new query token per
  sequence at the end of its cached keys, the key/value cache kept as pages
  with a per-sequence page table (frontiernews "What Attention Patterns
  Does FlexAttention Support?": PagedAttention, causal masking for
  language-model decoding, sliding-window decoders). Pinned in
  ``tests/test_oracle_decode.py`` against ``attention`` on the gathered
  rows, page-order invariance and closed forms.

Every function here is pinned by ``tests/test_oracle_pins.py`` against
what the pages print or what mathematics fixes (the T=6, W=3 mask printed
on the crackedaicode page, W=1 and W>=T special cases, block-diagonal
document masks, block-count closed forms, rows summing to one, closed-form
log-sum-exp values, single-key rows, a pure-Python brute force on tiny
inputs and torch's CPU scaled_dot_product_attention).
"""
from __future__ import annotations

import math

import numpy as np

MASK_KINDS = ("none", "causal", "sliding_window", "document", "local_window")
SCORE_KINDS = ("none", "softcap", "alibi")

EMPTY, PARTIAL, FULL = 0, 1, 2


def _as_f64(x) -> np.ndarray:
    """Exact upcast of a CPU tensor or array (bf16/fp32/fp64) to fp64."""
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# mask_mod built-ins
# --------------------------------------------------------------------------
def mask_mod(kind: str, q_idx, kv_idx, window=None, doc_id=None):
    """Evaluate a built-in mask_mod on broadcastable integer index arrays.

    The built-ins do not depend on the batch or head index."""
    i = np.asarray(q_idx, dtype=np.int64)
    j = np.asarray(kv_idx, dtype=np.int64)
    if kind == "none":
        return np.ones(np.broadcast(i, j).shape, dtype=bool)
    if kind == "causal":
        return i >= j
    if kind == "sliding_window":
        if window is None or int(window) < 1:
            raise ValueError("sliding window needs W >= 1")
        d = i - j
        return (d >= 0) & (d < int(window))
    if kind == "local_window":
        # symmetric local window: |i - j| limited instead of i - j
        # (crackedaicode "Sliding-Window Self-Attention", "State the
        # boundary precisely", last paragraph)
        if window is None or int(window) < 1:
            raise ValueError("local window needs W >= 1")
        return np.abs(i - j) < int(window)
    if kind == "document":
        if doc_id is None:
            raise ValueError("document mask needs doc_id")
        doc = np.asarray(doc_id, dtype=np.int64)
        return (i >= j) & (doc[i] == doc[j])
    raise ValueError(f"unknown mask kind {kind!r}")


def dense_mask(kind, q_len, kv_len, window=None, doc_id=None, rows=None):
    """bool [len(rows), kv_len] matrix of mask_mod over all keys."""
    rows = np.arange(q_len) if rows is None else np.asarray(rows)
    return mask_mod(kind, rows[:, None], np.arange(kv_len)[None, :],
                    window=window, doc_id=doc_id)


# --------------------------------------------------------------------------
# score_mod built-ins
# --------------------------------------------------------------------------
def alibi_slope(h: int, H: int) -> float:
    return 2.0 ** (-8.0 * (h + 1) / H)


def score_mod(kind: str, s, h, H, q_idx, kv_idx, softcap=None):
    """Apply a built-in score_mod to the scaled score ``s`` (fp64)."""
    if kind == "none":
        return s
    if kind == "softcap":
        if softcap is None or not (softcap > 0):
            raise ValueError("soft-cap needs cap > 0")
        return softcap * np.tanh(s / softcap)
    if kind == "alibi":
        i = np.asarray(q_idx, dtype=np.float64)
        j = np.asarray(kv_idx, dtype=np.float64)
        return s - alibi_slope(h, H) * (i - j)
    raise ValueError(f"unknown score kind {kind!r}")


# --------------------------------------------------------------------------
# create_block_mask
# --------------------------------------------------------------------------
def block_states(kind, q_len, kv_len, block_m, block_n, window=None,
                 doc_id=None):
    """int8 [NQB, NKVB]: EMPTY / PARTIAL / FULL from the exact count of
    allowed in-range pairs in each tile."""
    nqb = -(-q_len // block_m)
    nkvb = -(-kv_len // block_n)
    states = np.empty((nqb, nkvb), dtype=np.int8)
    area = block_m * block_n
    for m in range(nqb):
        rows = np.arange(m * block_m, min((m + 1) * block_m, q_len))
        allowed = dense_mask(kind, q_len, kv_len, window, doc_id, rows)
        padded = np.zeros((len(rows), nkvb * block_n), dtype=bool)
        padded[:, :kv_len] = allowed
        count = padded.reshape(len(rows), nkvb, block_n).sum(axis=(0, 2))
        states[m] = np.where(count == 0, EMPTY,
                             np.where(count == area, FULL, PARTIAL))
    return states


def _lists(selected: np.ndarray):
    """Row-wise stable partition: selected block numbers ascending, then
    the others ascending. Returns (num [NQB] int32, idx [NQB, NKVB] int32)."""
    nqb, nkvb = selected.shape
    num = selected.sum(axis=1).astype(np.int32)
    idx = np.empty((nqb, nkvb), dtype=np.int32)
    cols = np.arange(nkvb, dtype=np.int32)
    for m in range(nqb):
        idx[m] = np.concatenate([cols[selected[m]], cols[~selected[m]]])
    return num, idx


def create_block_mask(kind, B, H, q_len, kv_len, block_m, block_n=None,
                      window=None, doc_id=None, separate_full_blocks=True):
    """Block mask arrays as int32 numpy arrays.

    ``B``/``H`` of 1 broadcast one mask over every batch entry / head
    (``B=None, H=None`` on the how-to's "Mask 1: causal"). A 2-D ``doc_id``
    ``[B, L]`` gives each batch entry its own document ids (mask_mod takes the
    batch index, tensorplay page, parameter ``mask_mod``). Returns a dict
    with ``kv_num_blocks [B,H,NQB]``, ``kv_indices [B,H,NQB,NKVB]`` and,
    when ``separate_full_blocks``, ``full_kv_num_blocks`` and
    ``full_kv_indices`` of the same shapes (else ``None``)."""
    block_n = block_m if block_n is None else block_n
    if doc_id is not None and np.ndim(doc_id) == 2:
        # one id array per batch entry: the mask depends on b, so each entry
        # gets its own rows (no broadcast over the batch)
        if np.shape(doc_id)[0] != B:
            raise ValueError("per-batch doc_id needs one row per batch entry")
        parts = [create_block_mask(kind, 1, H, q_len, kv_len, block_m, block_n,
                                   window=window, doc_id=np.asarray(doc_id)[b],
                                   separate_full_blocks=separate_full_blocks)
                 for b in range(B)]
        out = {key: (None if parts[0][key] is None
                     else np.concatenate([pt[key] for pt in parts], axis=0))
               for key in ("kv_num_blocks", "kv_indices", "full_kv_num_blocks",
                           "full_kv_indices")}
        out["num_q_blocks"] = parts[0]["num_q_blocks"]
        out["num_kv_blocks"] = parts[0]["num_kv_blocks"]
        return out
    st = block_states(kind, q_len, kv_len, block_m, block_n, window, doc_id)
    if separate_full_blocks:
        num, idx = _lists(st == PARTIAL)
        fnum, fidx = _lists(st == FULL)
    else:
        num, idx = _lists(st != EMPTY)
        fnum = fidx = None

    def bcast(a):
        if a is None:
            return None
        return np.ascontiguousarray(
            np.broadcast_to(a, (B, H) + a.shape)).astype(np.int32)

    return {"kv_num_blocks": bcast(num), "kv_indices": bcast(idx),
            "full_kv_num_blocks": bcast(fnum), "full_kv_indices": bcast(fidx),
            "num_q_blocks": st.shape[0], "num_kv_blocks": st.shape[1]}


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------
def attention(q, k, v, mask="none", score="none", scale=None, window=None,
              doc_id=None, softcap=None, rows=None, chunk_bytes=1 << 28):
    """Dense masked softmax attention in fp64.

    ``q [B,H,Q,D]``, ``k``/``v [B,H_kv,KV,D]`` (H a multiple of H_kv; query
    head h reads key head ``h // (H // H_kv)``). ``doc_id``: ``[L]`` shared
    by every batch entry, or ``[B, L]`` per entry. ``rows``: optional query
    positions to evaluate (all by default). Returns
    ``O [B,H,len(rows),D]`` and ``LSE [B,H,len(rows)]`` in fp64."""
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, H, q_len, D = q.shape
    H_kv, kv_len = k.shape[1], k.shape[2]
    if H % H_kv:
        raise ValueError("H must be a multiple of H_kv")
    group = H // H_kv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rows = np.arange(q_len) if rows is None else np.asarray(rows, np.int64)
    out = np.zeros((B, H, len(rows), v.shape[3]))
    lse = np.full((B, H, len(rows)), -np.inf)
    cols = np.arange(kv_len)
    step = max(1, chunk_bytes // (8 * max(kv_len, 1)))
    for b in range(B):
        doc_b = (np.asarray(doc_id)[b]
                 if doc_id is not None and np.ndim(doc_id) == 2 else doc_id)
        for h in range(H):
            kb = k[b, h // group]
            vb = v[b, h // group]
            for r0 in range(0, len(rows), step):
                ri = rows[r0:r0 + step]
                s = scale * (q[b, h, ri] @ kb.T)
                s = score_mod(score, s, h, H, ri[:, None], cols[None, :],
                              softcap=softcap)
                allowed = mask_mod(mask, ri[:, None], cols[None, :],
                                   window=window, doc_id=doc_b)
                t = np.where(allowed, s, -np.inf)
                live = allowed.any(axis=1)
                mx = np.where(live, t.max(axis=1, initial=-np.inf), 0.0)
                w = np.exp(t - mx[:, None])
                denom = w.sum(axis=1)
                safe = np.where(live, denom, 1.0)
                out[b, h, r0:r0 + len(ri)] = np.where(
                    live[:, None], (w @ vb) / safe[:, None], 0.0)
                lse[b, h, r0:r0 + len(ri)] = np.where(
                    live, mx + np.log(safe), -np.inf)
    return out, lse


# --------------------------------------------------------------------------
# masked softmax over materialised scores
# --------------------------------------------------------------------------
def masked_softmax(scores, mask="causal", q_offset=0, window=None,
                   doc_id=None):
    """Softmax over the last axis of materialised scores with a built-in
    mask_mod folded in, fp64 (the fallback chain "compare, select the
    minimum, softmax" of the MLX pull request "Fuse the causal mask into the
    SDPA fallback softmax", as one operation).

    ``scores [..., Q, K]``: row i is query position ``q_idx = i + q_offset``
    (a prefill chunk that starts after ``q_offset`` earlier tokens), column j
    is ``kv_idx = j``. Allowed entries get ``exp(s - max) / sum exp(s - max)``
    over the row's allowed entries; masked entries are exactly 0 (the pull
    request's point: the masked minimum's exponential underflows to exact
    zero). A row with no allowed entry is all zeros."""
    s = _as_f64(scores)
    Q, K = s.shape[-2], s.shape[-1]
    rows = np.arange(Q)[:, None] + int(q_offset)
    cols = np.arange(K)[None, :]
    allowed = mask_mod(mask, rows, cols, window=window, doc_id=doc_id)
    z = np.where(allowed, s, -np.inf)
    live = allowed.any(axis=1)
    mx = np.where(live, z.max(axis=-1, initial=-np.inf), 0.0)
    w = np.exp(z - mx[..., None])
    den = w.sum(axis=-1, keepdims=True)
    return np.where(live[:, None], w / np.where(den > 0, den, 1.0), 0.0)


# --------------------------------------------------------------------------
# decode over a paged key/value cache
# --------------------------------------------------------------------------
def paged_rows(pages, table_b, length):
    """The first ``length`` token rows of one sequence from a paged cache.

    ``pages [P, page_size, H_kv, D]``: a pool of physical pages of
    ``page_size`` consecutive token rows (the key/value cache treated as
    pages, frontiernews "What Attention Patterns Does FlexAttention
    Support?", PagedAttention); ``table_b``: the sequence's page table,
    logical page p (tokens ``[p * page_size, (p + 1) * page_size)``) held in
    physical page ``table_b[p]``. Returns ``[H_kv, length, D]``."""
    page_size = pages.shape[1]
    n = -(-int(length) // page_size)
    rows = np.concatenate([_as_f64(pages[int(table_b[p])]) for p in range(n)],
                          axis=0) if n else np.zeros((0,) + tuple(pages.shape[2:]))
    return rows[:length].transpose(1, 0, 2)


def decode_paged(q, k_pages, v_pages, page_table, seq_lens, mask="causal",
                 score="none", scale=None, window=None, doc_id=None,
                 softcap=None):
    """One decode step over a paged cache, fp64.

    ``q [B, H, D]`` holds each sequence's newest token, already appended to
    the cache: sequence b has ``L_b = seq_lens[b]`` cached tokens (rows of
    ``k_pages`` / ``v_pages [P, page_size, H_kv, D]`` reached through
    ``page_table [B, max_pages]``) and its query sits at position
    ``q_idx = L_b - 1``. The attention is the plain definition above for
    that one row over keys ``kv_idx in [0, L_b)``: ``mask_mod(q_idx,
    kv_idx)``, ``score_mod`` with that q_idx and the query head h, the
    softmax over the allowed keys. ``doc_id``: ``[L]`` shared or ``[B, L]``
    per sequence, indexed by token position. Returns ``O [B, H, D]`` and
    ``LSE [B, H]``; a sequence with no allowed key (``L_b = 0``) gives 0 and
    -inf."""
    q = _as_f64(q)
    B, H, D = q.shape
    H_kv = k_pages.shape[2]
    group = H // H_kv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    table = np.asarray(page_table)
    lens = np.asarray(seq_lens)
    out = np.zeros((B, H, v_pages.shape[3]))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        L = int(lens[b])
        if L <= 0:
            continue
        kb = paged_rows(k_pages, table[b], L)
        vb = paged_rows(v_pages, table[b], L)
        doc_b = (np.asarray(doc_id)[b]
                 if doc_id is not None and np.ndim(doc_id) == 2 else doc_id)
        i = L - 1
        cols = np.arange(L)
        allowed = mask_mod(mask, i, cols, window=window, doc_id=doc_b)
        if not allowed.any():
            continue
        for h in range(H):
            t = scale * (kb[h // group] @ q[b, h])
            s = score_mod(score, t, h, H, i, cols, softcap=softcap)
            z = np.where(allowed, s, -np.inf)
            mx = z.max()
            w = np.exp(z - mx)
            den = w.sum()
            out[b, h] = (w @ vb[h // group]) / den
            lse[b, h] = mx + np.log(den)
    return out, lse


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------
def score_mod_grad(kind: str, s, softcap=None):
    """d score_mod / d s at the scaled score ``s`` (fp64): 1 for the additive
    mods, 1 - tanh(s / cap)**2 for the soft-cap (the derivative of
    cap * tanh(s / cap))."""
    if kind in ("none", "alibi"):
        return np.ones_like(s)
    if kind == "softcap":
        return 1.0 - np.tanh(s / softcap) ** 2
    raise ValueError(f"unknown score kind {kind!r}")


def attention_backward(q, k, v, do, mask="none", score="none", scale=None,
                       window=None, doc_id=None, softcap=None, rows=None):
    """Gradients (dQ, dK, dV) of ``O = attention(q, k, v, ...)`` for an
    upstream gradient ``do`` of O (LSE treated as not differentiated), in
    fp64, by the chain rule through the definition above:

        t = scale * q . k;  s = score_mod(t);  P = softmax over A_i of s;
        dV_j = sum_i P_ij dO_i;  dP_ij = dO_i . v_j;
        dS_ij = P_ij (dP_ij - sum_j' P_ij' dP_ij');
        dT = dS * score_mod'(t);  dQ_i = scale sum_j dT_ij k_j;
        dK_j = scale sum_i dT_ij q_i.

    Masked pairs have P = 0 and contribute nothing; a row with no allowed
    key has P = 0 everywhere. With grouped heads, dK / dV of a key head sum
    over the query heads that read it.

    ``rows``: optional distinct query-row indices. Row i's dQ depends on
    row i alone (its softmax, its dO), so then only those rows are
    evaluated: dQ is ``[B,H,len(rows),D]`` and dK, dV hold the sums over
    those rows only, which are the full gradients of every key j whose
    allowed rows all lie in ``rows``."""
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    do = _as_f64(do)
    B, H, q_len, D = q.shape
    H_kv, kv_len = k.shape[1], k.shape[2]
    group = H // H_kv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rows = np.arange(q_len) if rows is None else np.asarray(rows, np.int64)
    if len(np.unique(rows)) != len(rows):
        raise ValueError("rows must be distinct")
    dq = np.zeros((B, H, len(rows), D))
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    cols = np.arange(kv_len)
    for b in range(B):
        doc_b = (np.asarray(doc_id)[b]
                 if doc_id is not None and np.ndim(doc_id) == 2 else doc_id)
        allowed = mask_mod(mask, rows[:, None], cols[None, :], window=window,
                           doc_id=doc_b)
        live = allowed.any(axis=1)
        for h in range(H):
            hk = h // group
            t = scale * (q[b, h][rows] @ k[b, hk].T)
            s = score_mod(score, t, h, H, rows[:, None], cols[None, :],
                          softcap=softcap)
            z = np.where(allowed, s, -np.inf)
            mx = np.where(live, z.max(axis=1, initial=-np.inf), 0.0)
            w = np.exp(z - mx[:, None])
            den = np.where(live, w.sum(axis=1), 1.0)
            p = w / den[:, None]
            dp = do[b, h][rows] @ v[b, hk].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dt = ds * score_mod_grad(score, t, softcap=softcap)
            dq[b, h] = scale * (dt @ k[b, hk])
            dv[b, hk] += p.T @ do[b, h][rows]
            dk[b, hk] += scale * (dt.T @ q[b, h][rows])
    return dq, dk, dv
