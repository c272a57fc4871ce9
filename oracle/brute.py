"""Pure-Python brute force for tiny inputs (T <= 16 or so).

TEST INFRASTRUCTURE, like ``oracle.py``: only tests may call it. It is a
second, independent transcription of the same definitions (explicit loops,
``math`` only, no numpy) so that a slip in one of the two shows up as a
disagreement. The definitions and their sources are listed in the header
of ``oracle/oracle.py``.
"""
from __future__ import annotations

import math


def allowed(kind, i, j, window=None, doc=None):
    if kind == "none":
        return True
    if kind == "causal":
        return i >= j
    if kind == "sliding_window":
        return 0 <= i - j < window
    if kind == "local_window":
        return -window < i - j < window
    if kind == "document":
        return i >= j and doc[i] == doc[j]
    raise ValueError(kind)


def modified(kind, s, h, H, i, j, cap=None):
    if kind == "none":
        return s
    if kind == "softcap":
        return cap * math.tanh(s / cap)
    if kind == "alibi":
        return s - 2.0 ** (-8.0 * (h + 1) / H) * (i - j)
    raise ValueError(kind)


def attention(q, k, v, mask="none", score="none", scale=None, window=None,
              doc=None, cap=None):
    """q, k, v: nested lists [B][H][T][D] (k, v may have fewer heads).
    Returns (O, LSE) as nested lists."""
    B, H = len(q), len(q[0])
    Hk = len(k[0])
    D = len(q[0][0][0])
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    O, L = [], []
    for b in range(B):
        # doc: one id list for every batch entry, or a list of lists (one
        # per entry)
        doc_b = doc[b] if doc is not None and isinstance(doc[0], list) else doc
        Ob, Lb = [], []
        for h in range(H):
            hk = h // (H // Hk)
            Oh, Lh = [], []
            for i in range(len(q[b][h])):
                live = []
                for j in range(len(k[b][hk])):
                    if not allowed(mask, i, j, window, doc_b):
                        continue
                    dot = 0.0
                    for d in range(D):
                        dot += q[b][h][i][d] * k[b][hk][j][d]
                    live.append((j, modified(score, scale * dot, h, H, i, j,
                                             cap)))
                Dv = len(v[b][hk][0])
                if not live:
                    Oh.append([0.0] * Dv)
                    Lh.append(-math.inf)
                    continue
                mx = max(s for _, s in live)
                tot = sum(math.exp(s - mx) for _, s in live)
                row = [0.0] * Dv
                for j, s in live:
                    p = math.exp(s - mx) / tot
                    for d in range(Dv):
                        row[d] += p * v[b][hk][j][d]
                Oh.append(row)
                Lh.append(mx + math.log(tot))
            Ob.append(Oh)
            Lb.append(Lh)
        O.append(Ob)
        L.append(Lb)
    return O, L


def block_lists(kind, q_len, kv_len, bm, bn, window=None, doc=None,
                separate_full_blocks=True):
    """(num, idx, full_num, full_idx) for one (b, h) as Python lists."""
    nqb = (q_len + bm - 1) // bm
    nkvb = (kv_len + bn - 1) // bn
    num, idx, fnum, fidx = [], [], [], []
    for m in range(nqb):
        part, full = [], []
        for n in range(nkvb):
            c = 0
            for i in range(m * bm, min((m + 1) * bm, q_len)):
                for j in range(n * bn, min((n + 1) * bn, kv_len)):
                    if allowed(kind, i, j, window, doc):
                        c += 1
            if c == 0:
                continue
            if c == bm * bn and separate_full_blocks:
                full.append(n)
            else:
                part.append(n)
        num.append(len(part))
        idx.append(part + [n for n in range(nkvb) if n not in part])
        fnum.append(len(full))
        fidx.append(full + [n for n in range(nkvb) if n not in full])
    if not separate_full_blocks:
        return num, idx, None, None
    return num, idx, fnum, fidx
