"""Seeded synthetic workloads for block-sparse masked attention.

This module only draws inputs. It holds none of the attention arithmetic:
no mask predicate, no score modification, no softmax. The oracle (a CPU
reference used by the tests) and the HIP path both consume what it returns,
and neither of them is imported here.

The five workloads follow the shapes the pages use:

* ``c1``: small fp32 case, sliding window W=64 over 256 tokens, block 64.
* ``c2``: the create_block_mask example of the tensorplay API page
  (B=1, H=1, 8192 tokens, head dim 64, causal), in bf16.
* ``c3``: a 1k-token sliding window over an 8k context, as in the
  sliding-window section of the FlexAttention-on-Apple-Silicon how-to
  ("Mask 2"), batched as B=4, H=16, head dim 128.
* ``c4``: four packed documents (the how-to's "Mask 3" and its at-a-glance
  table), scaled to 32768 tokens, with the tanh soft-cap of its "Bonus"
  section at cap 50.
* ``c5``: causal attention with an ALiBi distance bias over 16384 tokens.

A sixth workload, ``decode_paged``, is one decode step per sequence over a
paged key/value cache (PagedAttention and language-model decoding in the
frontiernews article's list of supported patterns): 16 sequences with
seeded context lengths between 1024 and 32768 tokens, 32 query heads over 8
key heads, head dim 128, pages of 128 token rows scattered over the pool in
a seeded order, causal. See :class:`DecodeWorkload` and
:func:`make_paged_inputs`.

A seventh, ``softmax_fallback``, is the masked softmax of a materialising
attention fallback at the size the MLX pull request quotes (one chunk of
8192 query rows over 32768 keys, bf16 scores: 512 MiB), the last chunk of a
causal prefill (query offset 24576); see :func:`make_scores`.

Values are N(0, 1) from ``numpy.random.default_rng(seed)``, drawn as float32
in (B, H, S, D) order: the document lengths first (``c4`` only), then Q, K
and V. bf16 workloads are rounded to bf16 with round-to-nearest-even, and
both sides use those rounded values.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Workload", "CONFIGS", "get", "doc_lengths", "doc_ids",
           "draw_qkv", "make_inputs", "DecodeWorkload", "DECODE",
           "make_paged_inputs", "SoftmaxWorkload", "SOFTMAX", "make_scores"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str              # "bf16" or "fp32"
    B: int
    H: int
    H_kv: int
    q_len: int
    kv_len: int
    D: int
    mask: str               # "none" | "causal" | "sliding_window" | "document"
    block_m: int
    block_n: int
    seed: int
    window: Optional[int] = None
    n_docs: Optional[int] = None
    min_doc_len: Optional[int] = None
    score: str = "none"     # "none" | "softcap" | "alibi"
    softcap: Optional[float] = None

    @property
    def scale(self) -> float:
        # 1/sqrt(D), the SDPA default the pages' API mirrors.
        return 1.0 / float(np.sqrt(self.D))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "c1": Workload("c1", "fp32", 1, 2, 2, 256, 256, 64, "sliding_window",
                   64, 64, seed=0, window=64),
    "c2": Workload("c2", "bf16", 1, 1, 1, 8192, 8192, 64, "causal",
                   128, 128, seed=1),
    "c3": Workload("c3", "bf16", 4, 16, 16, 8192, 8192, 128,
                   "sliding_window", 128, 128, seed=2, window=1024),
    "c4": Workload("c4", "bf16", 1, 32, 32, 32768, 32768, 128, "document",
                   128, 128, seed=3, n_docs=4, min_doc_len=2048,
                   score="softcap", softcap=50.0),
    "c5": Workload("c5", "bf16", 2, 32, 32, 16384, 16384, 128, "causal",
                   128, 128, seed=4, score="alibi"),
}


def get(name: str) -> Workload:
    return CONFIGS[name]


def doc_lengths(rng: np.random.Generator, total: int, n_docs: int,
                min_len: int) -> np.ndarray:
    """Stick-breaking draw of ``n_docs`` lengths, each >= ``min_len``,
    summing to ``total``: the slack beyond the minimum is cut at
    ``n_docs - 1`` sorted uniform integer points."""
    extra = total - n_docs * min_len
    if extra < 0:
        raise ValueError("documents do not fit")
    cuts = np.sort(rng.integers(0, extra + 1, size=n_docs - 1))
    parts = np.diff(np.concatenate([[0], cuts, [extra]]))
    return (min_len + parts).astype(np.int64)


def doc_ids(lengths) -> np.ndarray:
    """int32 document id per token, consecutive runs in order."""
    lengths = np.asarray(lengths, dtype=np.int64)
    return np.repeat(np.arange(len(lengths), dtype=np.int32), lengths)


def draw_qkv(rng: np.random.Generator, w: Workload):
    """float32 Q [B,H,q_len,D], K and V [B,H_kv,kv_len,D], N(0,1)."""
    q = rng.standard_normal((w.B, w.H, w.q_len, w.D), dtype=np.float32)
    k = rng.standard_normal((w.B, w.H_kv, w.kv_len, w.D), dtype=np.float32)
    v = rng.standard_normal((w.B, w.H_kv, w.kv_len, w.D), dtype=np.float32)
    return q, k, v


def make_inputs(w: Workload):
    """Return ``(q, k, v, doc_id)`` as CPU torch tensors in the workload's
    dtype (bf16 values are RNE-rounded from the float32 draw) and
    ``doc_id`` as an int32 numpy array or ``None``."""
    import torch

    rng = np.random.default_rng(w.seed)
    doc = None
    if w.mask == "document":
        if w.q_len != w.kv_len:
            raise ValueError("document workloads use q_len == kv_len")
        doc = doc_ids(doc_lengths(rng, w.kv_len, w.n_docs, w.min_doc_len))
    q, k, v = draw_qkv(rng, w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qt, kt, vt = (torch.from_numpy(x).to(tdt) for x in (q, k, v))
    return qt, kt, vt, doc


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int                  # sequences
    H: int                  # query heads
    H_kv: int               # key / value heads
    D: int
    page_size: int
    min_len: int            # context lengths drawn uniformly in
    max_len: int            # [min_len, max_len]
    seed: int
    mask: str = "causal"
    window: Optional[int] = None
    score: str = "none"
    softcap: Optional[float] = None
    spare_pages: int = 7    # unused pages in the pool (poisoned)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))


DECODE = DecodeWorkload("decode_paged", B=16, H=32, H_kv=8, D=128,
                        page_size=128, min_len=1024, max_len=32768, seed=5)


def make_paged_inputs(w: DecodeWorkload, lens=None, poison=True):
    """Seeded paged cache for ``w``.

    Draws, in order: the context lengths (unless ``lens`` is given), each
    sequence's K and V token rows ``[L_b, H_kv, D]`` and its query
    ``[H, D]`` (float32 N(0, 1), then bf16 RNE), and a random permutation of
    the physical pages. Pages are filled in the order of the sequences and
    their logical pages; rows of a sequence's last page past its length,
    the spare pages and the unused page-table slots hold poison (NaN rows,
    index -1), which a correct reader never touches.

    Returns CPU tensors ``q [B, H, D]``, ``k_pages``, ``v_pages
    [P, page_size, H_kv, D]`` (bf16), ``page_table [B, max_pages]`` and
    ``seq_lens [B]`` (int32)."""
    import torch

    rng = np.random.default_rng(w.seed)
    if lens is None:
        lens = rng.integers(w.min_len, w.max_len + 1, size=w.B)
    lens = np.asarray(lens, dtype=np.int64)
    ps = w.page_size
    n_pages = [-(-int(L) // ps) for L in lens]
    P = sum(n_pages) + w.spare_pages
    max_pages = max(max(n_pages), 1)
    fill = np.nan if poison else 0.0
    kp = np.full((P, ps, w.H_kv, w.D), fill, dtype=np.float32)
    vp = np.full((P, ps, w.H_kv, w.D), fill, dtype=np.float32)
    q = np.empty((w.B, w.H, w.D), dtype=np.float32)
    perm = rng.permutation(P)
    table = np.full((w.B, max_pages), -1, dtype=np.int32)
    at = 0
    for b, L in enumerate(lens):
        L = int(L)
        k = rng.standard_normal((L, w.H_kv, w.D), dtype=np.float32)
        v = rng.standard_normal((L, w.H_kv, w.D), dtype=np.float32)
        q[b] = rng.standard_normal((w.H, w.D), dtype=np.float32)
        for lp in range(n_pages[b]):
            phys = int(perm[at])
            at += 1
            table[b, lp] = phys
            rows = slice(lp * ps, min(L, (lp + 1) * ps))
            n = rows.stop - rows.start
            kp[phys, :n] = k[rows]
            vp[phys, :n] = v[rows]
    to = lambda x: torch.from_numpy(x).to(torch.bfloat16)  # noqa: E731
    return (to(q), to(kp), to(vp), torch.from_numpy(table),
            torch.from_numpy(lens.astype(np.int32)))


@dataclasses.dataclass(frozen=True)
class SoftmaxWorkload:
    name: str
    BH: int                 # batch * heads
    q_len: int
    kv_len: int
    q_offset: int
    seed: int
    mask: str = "causal"
    window: Optional[int] = None
    spread: float = 2.0     # scores ~ N(0, spread^2)


SOFTMAX = SoftmaxWorkload("softmax_fallback", BH=1, q_len=8192, kv_len=32768,
                          q_offset=24576, seed=6)


def make_scores(w: SoftmaxWorkload):
    """Seeded bf16 scores ``[BH, q_len, kv_len]`` (CPU tensor), N(0,
    spread^2) drawn as float32 and rounded to bf16 (RNE)."""
    import torch

    rng = np.random.default_rng(w.seed)
    x = rng.standard_normal((w.BH, w.q_len, w.kv_len), dtype=np.float32)
    x *= np.float32(w.spread)
    return torch.from_numpy(x).to(torch.bfloat16)

