"""Python binding of libflexattn.so.

Thin marshalling over the C ABI (``include/flexattn.h``): torch provides the
device buffers and the current HIP stream, every computation runs in the HIP
kernels. Two layers:

* the raw entry points with the C names (``fa_block_mask_dims``,
  ``fa_create_block_mask``, ``fa_flex_attention_fwd``,
  ``fa_flex_attention_fwd_split``, ``fa_split_workspace_bytes``,
  ``fa_flex_attention_bwd``, ``fa_bwd_workspace_bytes``,
  ``fa_flex_attention_decode_paged``, ``fa_masked_softmax``), taking
  ctypes structs and integer device addresses;
* a FlexAttention-style convenience layer: ``create_block_mask(...)`` returns
  a :class:`BlockMask` holding its index tensors, and
  ``flex_attention(q, k, v, block_mask, score_mod)`` returns ``(O, LSE)``
  and ``flex_attention_backward(...)`` returns ``(dQ, dK, dV)``;
  ``flex_attention_decode_paged(...)`` runs one decode step per sequence
  over a paged key/value cache.
  The shapes follow scaled_dot_product_attention: (B, H, S, D).
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
from typing import Optional, Tuple, Union

import numpy as np
import torch

from . import _capi as C

__all__ = [
    "MaskMod", "ScoreMod", "causal", "sliding_window", "local_window",
    "document",
    "no_mask", "softcap", "alibi", "BlockMask", "create_block_mask",
    "flex_attention", "fa_block_mask_dims", "fa_create_block_mask",
    "fa_flex_attention_fwd", "fa_flex_attention_fwd_split",
    "fa_split_workspace_bytes", "auto_num_splits", "FlexAttnError",
    "flex_attention_backward", "fa_flex_attention_bwd",
    "fa_bwd_workspace_bytes", "auto_bwd_splits", "flex_attention_decode_paged",
    "fa_flex_attention_decode_paged", "auto_decode_splits",
    "masked_softmax", "fa_masked_softmax", "fwd_workspace",
    "fa_flex_attention_fwd_split_noalloc",
]

FlexAttnError = C.FlexAttnError


# ------------------------------------------------------------------ mods
@dataclasses.dataclass(frozen=True)
class MaskMod:
    """A built-in mask_mod. ``doc_id`` is an int32 tensor on the device:
    ``[L]`` shared by every batch entry, or ``[B, L]`` with one row per
    entry (a batch of packed sequences)."""
    kind: int
    window: int = 0
    doc_id: Optional[torch.Tensor] = None

    @property
    def per_batch(self) -> bool:
        return self.doc_id is not None and self.doc_id.dim() == 2

    def to_c(self) -> C.fa_mask_mod:
        doc = self.doc_id
        return C.fa_mask_mod(
            kind=self.kind, window=int(self.window),
            doc_id=doc.data_ptr() if doc is not None else None,
            doc_len=doc.shape[-1] if doc is not None else 0,
            doc_stride=doc.stride(0) if self.per_batch else 0)


def causal() -> MaskMod:
    return MaskMod(C.FA_MASK_CAUSAL)


def sliding_window(window: int) -> MaskMod:
    return MaskMod(C.FA_MASK_SLIDING_WINDOW, window=int(window))


def local_window(window: int) -> MaskMod:
    """|q_idx - kv_idx| < window (symmetric, not causal)."""
    return MaskMod(C.FA_MASK_LOCAL_WINDOW, window=int(window))


def document(doc_id: torch.Tensor) -> MaskMod:
    """Document mask: ``doc_id`` int32 ``[L]`` (one packed sequence layout
    for every batch entry) or ``[B, L]`` (one per entry)."""
    if doc_id.dtype != torch.int32 or doc_id.dim() not in (1, 2):
        raise ValueError("doc_id must be a 1-D or 2-D int32 tensor")
    return MaskMod(C.FA_MASK_DOCUMENT, doc_id=doc_id.contiguous())


def no_mask() -> MaskMod:
    return MaskMod(C.FA_MASK_NONE)


@dataclasses.dataclass(frozen=True)
class ScoreMod:
    kind: int
    cap: float = 0.0

    def to_c(self) -> C.fa_score_mod:
        return C.fa_score_mod(kind=self.kind, softcap=float(self.cap))


def softcap(cap: float) -> ScoreMod:
    return ScoreMod(C.FA_SCORE_SOFTCAP, float(cap))


def alibi() -> ScoreMod:
    return ScoreMod(C.FA_SCORE_ALIBI)


def _mask_from(spec, window=None, doc_id=None) -> MaskMod:
    if isinstance(spec, MaskMod):
        return spec
    if spec is None or spec == "none":
        return no_mask()
    if spec == "causal":
        return causal()
    if spec == "sliding_window":
        return sliding_window(window)
    if spec == "local_window":
        return local_window(window)
    if spec == "document":
        return document(doc_id)
    raise ValueError(f"unknown mask_mod {spec!r}")


def _score_from(spec) -> ScoreMod:
    if isinstance(spec, ScoreMod):
        return spec
    if spec is None or spec == "none":
        return ScoreMod(C.FA_SCORE_NONE)
    if spec == "alibi":
        return alibi()
    if isinstance(spec, tuple) and len(spec) == 2 and spec[0] == "softcap":
        return softcap(spec[1])
    raise ValueError(f"unknown score_mod {spec!r}")


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


# -------------------------------------------------------------- raw calls
def fa_block_mask_dims(q_len: int, kv_len: int, block_m: int,
                       block_n: int) -> Tuple[int, int]:
    nq, nk = ctypes.c_int32(), ctypes.c_int32()
    C.check(C.lib().fa_block_mask_dims(q_len, kv_len, block_m, block_n,
                                       ctypes.byref(nq), ctypes.byref(nk)),
            "fa_block_mask_dims")
    return nq.value, nk.value


def fa_create_block_mask(mask: C.fa_mask_mod, B: int, H: int, q_len: int,
                         kv_len: int, block_m: int, block_n: int,
                         separate_full_blocks: int, bm: C.fa_block_mask,
                         stream: Optional[int]) -> int:
    return C.lib().fa_create_block_mask(
        ctypes.byref(mask), B, H, q_len, kv_len, block_m, block_n,
        separate_full_blocks, ctypes.byref(bm), stream)


def fa_flex_attention_fwd(dtype: int, B: int, H: int, H_kv: int, q_len: int,
                          kv_len: int, D: int, q: int, q_stride, k: int,
                          k_stride, v: int, v_stride, scale: float,
                          bm: C.fa_block_mask, score: Optional[C.fa_score_mod],
                          o: int, lse: Optional[int],
                          stream: Optional[int], workspace: Optional[int] = None,
                          workspace_bytes: int = 0) -> int:
    return C.lib().fa_flex_attention_fwd(
        dtype, B, H, H_kv, q_len, kv_len, D,
        q, C.Stride3(*q_stride), k, C.Stride3(*k_stride),
        v, C.Stride3(*v_stride), scale, ctypes.byref(bm),
        ctypes.byref(score) if score is not None else None, workspace,
        workspace_bytes, o, lse, stream)


def fa_flex_attention_fwd_split(dtype: int, B: int, H: int, H_kv: int,
                                q_len: int, kv_len: int, D: int, q: int,
                                q_stride, k: int, k_stride, v: int, v_stride,
                                scale: float, bm: C.fa_block_mask,
                                score: Optional[C.fa_score_mod],
                                num_splits: int, workspace: Optional[int],
                                workspace_bytes: int, o: int,
                                lse: Optional[int],
                                stream: Optional[int]) -> int:
    return C.lib().fa_flex_attention_fwd_split(
        dtype, B, H, H_kv, q_len, kv_len, D,
        q, C.Stride3(*q_stride), k, C.Stride3(*k_stride),
        v, C.Stride3(*v_stride), scale, ctypes.byref(bm),
        ctypes.byref(score) if score is not None else None, num_splits,
        workspace, workspace_bytes, o, lse, stream)


def fa_flex_attention_fwd_split_noalloc(dtype: int, B: int, H: int,
                                        H_kv: int, q_len: int, kv_len: int,
                                        D: int, q: int, q_stride, k: int,
                                        k_stride, v: int, v_stride,
                                        scale: float, bm: C.fa_block_mask,
                                        score: Optional[C.fa_score_mod],
                                        num_splits: int, o: int,
                                        lse: Optional[int],
                                        stream: Optional[int]) -> int:
    return C.lib().fa_flex_attention_fwd_split_noalloc(
        dtype, B, H, H_kv, q_len, kv_len, D,
        q, C.Stride3(*q_stride), k, C.Stride3(*k_stride),
        v, C.Stride3(*v_stride), scale, ctypes.byref(bm),
        ctypes.byref(score) if score is not None else None, num_splits,
        o, lse, stream)


def fa_split_workspace_bytes(B: int, H: int, q_len: int, D: int,
                             num_splits: int) -> int:
    n = ctypes.c_uint64()
    C.check(C.lib().fa_split_workspace_bytes(B, H, q_len, D, num_splits,
                                             ctypes.byref(n)),
            "fa_split_workspace_bytes")
    return n.value


def fa_flex_attention_bwd(dtype: int, B: int, H: int, H_kv: int, q_len: int,
                          kv_len: int, D: int, q: int, q_stride, k: int,
                          k_stride, v: int, v_stride, scale: float,
                          bm: C.fa_block_mask, score: Optional[C.fa_score_mod],
                          dq_kv_order: int, num_splits: int, o: int,
                          lse: int, dout: int, workspace: Optional[int],
                          workspace_bytes: int, dq: int, dk: int, dv: int,
                          stream: Optional[int]) -> int:
    return C.lib().fa_flex_attention_bwd(
        dtype, B, H, H_kv, q_len, kv_len, D,
        q, C.Stride3(*q_stride), k, C.Stride3(*k_stride),
        v, C.Stride3(*v_stride), scale, ctypes.byref(bm),
        ctypes.byref(score) if score is not None else None, dq_kv_order,
        num_splits, o, lse, dout, workspace, workspace_bytes, dq, dk, dv,
        stream)


def fa_bwd_workspace_bytes(B: int, H: int, H_kv: int, q_len: int,
                           kv_len: int, D: int, bm: C.fa_block_mask,
                           num_splits: int = 1) -> int:
    n = ctypes.c_uint64()
    C.check(C.lib().fa_bwd_workspace_bytes(B, H, H_kv, q_len, kv_len, D,
                                           ctypes.byref(bm), num_splits,
                                           ctypes.byref(n)),
            "fa_bwd_workspace_bytes")
    return n.value


def fa_flex_attention_decode_paged(B: int, H: int, H_kv: int, D: int, q: int,
                                   q_stride, k_pages: int, k_stride,
                                   v_pages: int, v_stride, num_pages: int,
                                   page_size: int, page_table: int,
                                   max_pages: int, seq_lens: int,
                                   scale: float, mask: C.fa_mask_mod,
                                   score: Optional[C.fa_score_mod],
                                   num_splits: int, workspace: Optional[int],
                                   workspace_bytes: int, o: int,
                                   lse: Optional[int],
                                   stream: Optional[int]) -> int:
    return C.lib().fa_flex_attention_decode_paged(
        B, H, H_kv, D, q, C.Stride2(*q_stride), k_pages, C.Stride3(*k_stride),
        v_pages, C.Stride3(*v_stride), num_pages, page_size, page_table,
        max_pages, seq_lens, scale, ctypes.byref(mask),
        ctypes.byref(score) if score is not None else None, num_splits,
        workspace, workspace_bytes, o, lse, stream)


def fa_masked_softmax(BH: int, q_len: int, kv_len: int, q_offset: int,
                      scores: int, score_stride, mask: C.fa_mask_mod,
                      probs: int, stream: Optional[int]) -> int:
    return C.lib().fa_masked_softmax(BH, q_len, kv_len, q_offset, scores,
                                     C.Stride2(*score_stride),
                                     ctypes.byref(mask), probs, stream)


def auto_decode_splits(B: int, H_kv: int, max_tokens: int,
                       num_cus: int) -> int:
    """Parts per (sequence, key head) for the paged decode: about sixteen
    single-wavefront workgroups per compute unit (a few are resident at a
    time; the rest even out ragged lengths: on the decode workload 32 parts
    ran 1.8% faster than 16, 40 parts 2% slower), at most one part per
    64-key stage of the longest possible sequence, at most 64."""
    wgs = B * H_kv
    if wgs == 0:
        return 1
    stages = max(1, -(-max_tokens // 64))
    return max(1, min(C.FA_MAX_SPLITS, stages, -(-16 * num_cus // wgs)))


def auto_bwd_splits(B: int, H_kv: int, num_kv_blocks: int,
                    num_cus: int) -> int:
    """Parts per gradient row for the backward: 1 when the dK / dV kernel's
    B * H_kv * NKVB workgroups (one resident per compute unit) already
    cover the compute units, else enough parts for about two workgroups per
    unit (the second wave of workgroups evens out rows of unequal length),
    at most 16 and at most NKVB."""
    wgs = B * H_kv * num_kv_blocks
    if wgs == 0 or wgs >= num_cus:
        return 1
    return max(1, min(16, num_kv_blocks, -(-2 * num_cus // wgs)))


def auto_num_splits(dtype: torch.dtype, B: int, H: int, num_q_blocks: int,
                    num_cus: int) -> int:
    """Split-KV parts per query block so that the forward launches about two
    workgroups per compute unit: 1 (no split) when B * H * NQB already gives
    at least one per unit or the dtype is not bf16."""
    wgs = B * H * num_q_blocks
    if dtype != torch.bfloat16 or wgs == 0 or wgs >= num_cus:
        return 1
    return max(1, min(C.FA_MAX_SPLITS, -(-2 * num_cus // wgs)))


# ------------------------------------------------------------- BlockMask
def _check_lists(num, idx, fnum, fidx, nkvb):
    """Host check of caller-supplied lists: in every row the listed
    in-range entries are distinct, and no block is in both lists."""
    def listed(n, i):
        n = n.cpu().numpy().clip(0, nkvb)
        i = i.cpu().numpy()
        keep = np.arange(nkvb)[None, None, None, :] < n[..., None]
        keep &= (i >= 0) & (i < nkvb)
        return i, keep

    def seen(i, keep):
        # per row, how often each block number is listed
        rows = i.reshape(-1, nkvb)
        k = keep.reshape(-1, nkvb)
        cnt = np.zeros((rows.shape[0], nkvb), dtype=np.int64)
        r, c = np.nonzero(k)
        np.add.at(cnt, (r, rows[r, c]), 1)
        return cnt

    cnt = seen(*listed(num, idx))
    if (cnt > 1).any():
        raise ValueError("a row of kv_indices lists a block twice")
    if fnum is not None:
        fcnt = seen(*listed(fnum, fidx))
        if (fcnt > 1).any():
            raise ValueError("a row of full_kv_indices lists a block twice")
        if ((cnt > 0) & (fcnt > 0)).any():
            raise ValueError("a block is listed both as partial and as full")


class BlockMask:
    """Block mask: index tensors (int32, on the device) plus the mask_mod
    they were built from. Built once, reused by any number of
    flex_attention calls (the mask stays valid while its tensors live)."""

    def __init__(self, mask: MaskMod, B: int, H: int, q_len: int,
                 kv_len: int, block_m: int, block_n: int,
                 kv_num_blocks: torch.Tensor, kv_indices: torch.Tensor,
                 full_kv_num_blocks: Optional[torch.Tensor],
                 full_kv_indices: Optional[torch.Tensor]):
        self.mask = mask
        self.B, self.H = B, H
        self.q_len, self.kv_len = q_len, kv_len
        self.block_m, self.block_n = block_m, block_n
        self.kv_num_blocks = kv_num_blocks
        self.kv_indices = kv_indices
        self.full_kv_num_blocks = full_kv_num_blocks
        self.full_kv_indices = full_kv_indices
        self.num_q_blocks = kv_num_blocks.shape[-1]
        self.num_kv_blocks = kv_indices.shape[-1]
        # order of the backward's dQ accumulation over key blocks (tensorplay
        # create_block_mask page, dq_kv_order): True descending, False
        # ascending. Either is deterministic and needs no stored metadata.
        self.dq_kv_order = True

    @property
    def separate_full_blocks(self) -> bool:
        return self.full_kv_num_blocks is not None

    def to_c(self) -> C.fa_block_mask:
        f = self.full_kv_num_blocks
        fi = self.full_kv_indices
        return C.fa_block_mask(
            mask=self.mask.to_c(), B=self.B, H=self.H, q_len=self.q_len,
            kv_len=self.kv_len, block_m=self.block_m, block_n=self.block_n,
            num_q_blocks=self.num_q_blocks, num_kv_blocks=self.num_kv_blocks,
            separate_full_blocks=int(self.separate_full_blocks),
            kv_num_blocks=self.kv_num_blocks.data_ptr(),
            kv_indices=self.kv_indices.data_ptr(),
            full_kv_num_blocks=f.data_ptr() if f is not None else None,
            full_kv_indices=fi.data_ptr() if fi is not None else None)

    @classmethod
    def from_kv_blocks(cls, kv_num_blocks: torch.Tensor,
                       kv_indices: torch.Tensor,
                       full_kv_num_blocks: Optional[torch.Tensor] = None,
                       full_kv_indices: Optional[torch.Tensor] = None, *,
                       mask_mod=None, q_len: int, kv_len: int,
                       BLOCK_SIZE: Union[int, Tuple[int, int]] = 128,
                       window=None, doc_id=None,
                       check_lists: bool = True) -> "BlockMask":
        """Wrap caller-provided index tensors (tensorplay
        create_block_mask page: precomputed metadata is supplied through
        BlockMask.from_kv_blocks). The mask_mod is still applied to the
        listed partial blocks; full blocks are taken as wholly allowed.

        Shapes: ``kv_num_blocks [B, H, NQB]`` and ``kv_indices [B, H, NQB,
        NKVB]`` with NQB = ceil(q_len / block_m), NKVB = ceil(kv_len /
        block_n) (B, H = 1 broadcast), the full pair the same, int32,
        contiguous, on one device. Counts outside [0, NKVB] are clamped and
        listed entries outside [0, NKVB) are skipped by the kernels. The
        listed entries of a row must be distinct and the partial and full
        lists disjoint (the forward would visit a repeated block twice);
        ``check_lists`` verifies that on the host (one device-to-host copy)."""
        bm_, bn_ = ((BLOCK_SIZE, BLOCK_SIZE) if isinstance(BLOCK_SIZE, int)
                    else BLOCK_SIZE)
        if (full_kv_num_blocks is None) != (full_kv_indices is None):
            raise ValueError("give both full block tensors or neither")
        tensors = [t for t in (kv_num_blocks, kv_indices, full_kv_num_blocks,
                               full_kv_indices) if t is not None]
        for t in tensors:
            if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
                raise ValueError("index tensors must be contiguous int32 "
                                 "device tensors")
            if t.device != kv_num_blocks.device:
                raise ValueError("index tensors must be on one device")
        nqb, nkvb = fa_block_mask_dims(q_len, kv_len, bm_, bn_)
        if kv_num_blocks.dim() != 3 or kv_num_blocks.shape[2] != nqb:
            raise ValueError(f"kv_num_blocks must be [B, H, {nqb}] "
                             f"(NQB = ceil(q_len / block_m))")
        want = (*kv_num_blocks.shape, nkvb)
        if tuple(kv_indices.shape) != want:
            raise ValueError(f"kv_indices must be {list(want)} "
                             f"(NKVB = ceil(kv_len / block_n))")
        if full_kv_num_blocks is not None:
            if full_kv_num_blocks.shape != kv_num_blocks.shape or \
                    tuple(full_kv_indices.shape) != want:
                raise ValueError("the full block tensors must have the "
                                 "shapes of the partial ones")
        B, H = kv_num_blocks.shape[0], kv_num_blocks.shape[1]
        mask = _mask_from(mask_mod, window, doc_id)
        if mask.kind == C.FA_MASK_DOCUMENT and mask.per_batch and \
                mask.doc_id.shape[0] != B:
            raise ValueError("per-batch doc_id [B, L] needs B = the index "
                             "tensors' first dimension")
        if mask.doc_id is not None and mask.doc_id.device != kv_num_blocks.device:
            raise ValueError("doc_id must live on the index tensors' device")
        if check_lists:
            _check_lists(kv_num_blocks, kv_indices, full_kv_num_blocks,
                         full_kv_indices, nkvb)
        return cls(mask, B, H, q_len, kv_len, bm_, bn_, kv_num_blocks,
                   kv_indices, full_kv_num_blocks, full_kv_indices)

    def __repr__(self):
        return (f"BlockMask(B={self.B}, H={self.H}, q_len={self.q_len}, "
                f"kv_len={self.kv_len}, block=({self.block_m}, "
                f"{self.block_n}), separate_full_blocks="
                f"{self.separate_full_blocks})")


def create_block_mask(mask_mod, B: Optional[int], H: Optional[int],
                      Q_LEN: int, KV_LEN: int, device="cuda",
                      BLOCK_SIZE: Union[int, Tuple[int, int]] = 128,
                      separate_full_blocks: bool = True,
                      compute_dq_write_order: bool = False,
                      dq_kv_order: bool = True, *, window=None,
                      doc_id=None) -> BlockMask:
    """Build a block mask on the device (one call of fa_create_block_mask).

    ``mask_mod``: a :class:`MaskMod` or one of "causal", "sliding_window" /
    "local_window" (with ``window``), "document" (with ``doc_id``, ``[L]`` or
    per batch entry ``[B, L]``), "none". ``B``/``H`` None broadcast the mask
    over every batch entry / head.

    ``dq_kv_order`` picks the order in which the backward sums each dQ row
    over its key blocks (True: descending block index, False: ascending).
    ``compute_dq_write_order`` is accepted for the page's signature: the
    backward here accumulates every dQ row in one workgroup, so its order
    needs no precomputed metadata and the flag changes nothing."""
    mask = _mask_from(mask_mod, window, doc_id)
    device = torch.device(device)
    if device.type != "cuda":
        raise ValueError("the block mask is built on a HIP device")
    bm_, bn_ = ((BLOCK_SIZE, BLOCK_SIZE) if isinstance(BLOCK_SIZE, int)
                else BLOCK_SIZE)
    Bm = 1 if B is None else int(B)
    Hm = 1 if H is None else int(H)
    if mask.kind == C.FA_MASK_DOCUMENT and mask.per_batch and \
            mask.doc_id.shape[0] != Bm:
        raise ValueError("per-batch doc_id [B, L] needs B = its first "
                         "dimension (the mask depends on the batch entry)")
    nqb, nkvb = fa_block_mask_dims(Q_LEN, KV_LEN, bm_, bn_)
    opts = dict(dtype=torch.int32, device=device)
    num = torch.empty((Bm, Hm, nqb), **opts)
    idx = torch.empty((Bm, Hm, nqb, nkvb), **opts)
    fnum = torch.empty((Bm, Hm, nqb), **opts) if separate_full_blocks else None
    fidx = (torch.empty((Bm, Hm, nqb, nkvb), **opts)
            if separate_full_blocks else None)
    if mask.doc_id is not None and mask.doc_id.device != device:
        raise ValueError("doc_id must live on the mask's device")
    cbm = C.fa_block_mask(
        kv_num_blocks=num.data_ptr(), kv_indices=idx.data_ptr(),
        full_kv_num_blocks=fnum.data_ptr() if fnum is not None else None,
        full_kv_indices=fidx.data_ptr() if fidx is not None else None)
    with torch.cuda.device(device):
        C.check(fa_create_block_mask(mask.to_c(), Bm, Hm, Q_LEN, KV_LEN, bm_,
                                     bn_, int(separate_full_blocks), cbm,
                                     _stream_handle(device)),
                "fa_create_block_mask")
    out = BlockMask(mask, Bm, Hm, Q_LEN, KV_LEN, bm_, bn_, num, idx, fnum,
                    fidx)
    out.dq_kv_order = bool(dq_kv_order)
    return out


_DTYPES = {torch.bfloat16: C.FA_BF16, torch.float32: C.FA_FP32}

# One zeroed scheduler workspace per (device, stream): calls on one stream
# run in order and each leaves the counters zero again; calls on different
# streams must not share one.
_SCHED_WS = {}


def fwd_workspace(device: torch.device) -> torch.Tensor:
    """The forward's scheduler workspace for the current stream of
    ``device`` (allocated zeroed on first use)."""
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _SCHED_WS.get(key)
    if ws is None:
        ws = torch.zeros(C.FA_FWD_WORKSPACE_BYTES, dtype=torch.uint8,
                         device=device)
        _SCHED_WS[key] = ws
    return ws


def _check_doc_rows(block_mask: BlockMask, B: int) -> None:
    """A per-batch doc_id is read at row b for every batch entry b < B (the
    C ABI has no row count to check it against)."""
    m = block_mask.mask
    if m.kind == C.FA_MASK_DOCUMENT and m.per_batch and m.doc_id.shape[0] != B:
        raise ValueError(f"per-batch doc_id has {m.doc_id.shape[0]} rows "
                         f"for a batch of {B}")


def flex_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                   block_mask: BlockMask, score_mod=None,
                   scale: Optional[float] = None, return_lse: bool = True,
                   out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None,
                   num_splits: Optional[int] = None,
                   persistent: bool = False):
    """Fused block-sparse attention forward.

    q: (B, H, Q_LEN, D); k, v: (B, H_kv, KV_LEN, D), bf16 or fp32, on the
    same HIP device, last dimension contiguous. ``score_mod``: None,
    "alibi", ("softcap", cap) or a :class:`ScoreMod`. ``scale`` defaults to
    1/sqrt(D). Returns ``(O, LSE)`` (``LSE`` fp32 (B, H, Q_LEN), natural
    log; ``None`` when ``return_lse`` is False).

    ``num_splits``: split-KV parts per query block (bf16 only). None picks
    :func:`auto_num_splits` for the device; 1 is one fa_flex_attention_fwd
    call, more is fa_flex_attention_fwd_split with a workspace allocated
    here. ``persistent`` (num_splits 1): pass the stream's scheduler
    workspace, so resident workgroups take query blocks from counters
    (measured no faster on MI355X, whose clock drops as idle gaps close);
    False (default) launches one workgroup per query block."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D (B, H, S, D)")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPES:
        raise ValueError("q, k, v must share a dtype in {bf16, fp32}")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be HIP device tensors")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    B, H, q_len, D = q.shape
    Bk, H_kv, kv_len, Dk = k.shape
    if k.shape != v.shape or Bk != B or Dk != D:
        raise ValueError("k and v must be (B, H_kv, KV_LEN, D)")
    for t in (q, k, v):
        if t.numel() and t.stride(-1) != 1:
            raise ValueError("the head dimension must be contiguous")
    _check_doc_rows(block_mask, B)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    score = _score_from(score_mod)
    if out is None:
        out = torch.empty((B, H, q_len, D), dtype=q.dtype, device=q.device)
    elif (out.shape != (B, H, q_len, D) or out.dtype != q.dtype
          or out.device != q.device or not out.is_contiguous()):
        raise ValueError("out must be a contiguous (B, H, Q_LEN, D) tensor "
                         "of q's dtype on q's device")
    if not return_lse:
        lse = None
    elif lse is None:
        lse = torch.empty((B, H, q_len), dtype=torch.float32, device=q.device)
    elif (lse.shape != (B, H, q_len) or lse.dtype != torch.float32
          or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous fp32 (B, H, Q_LEN) tensor "
                         "on q's device")
    if num_splits is None:
        num_splits = auto_num_splits(
            q.dtype, B, H, block_mask.num_q_blocks,
            torch.cuda.get_device_properties(q.device).multi_processor_count)
    with torch.cuda.device(q.device):
        if num_splits == 1:
            ws = fwd_workspace(q.device) if persistent else None
            st = fa_flex_attention_fwd(
                _DTYPES[q.dtype], B, H, H_kv, q_len, kv_len, D,
                q.data_ptr(), q.stride()[:3], k.data_ptr(), k.stride()[:3],
                v.data_ptr(), v.stride()[:3], float(scale),
                block_mask.to_c(), score.to_c(), out.data_ptr(),
                lse.data_ptr() if lse is not None else None,
                _stream_handle(q.device),
                ws.data_ptr() if ws is not None else None,
                ws.numel() if ws is not None else 0)
            C.check(st, "fa_flex_attention_fwd")
            return out, lse
        nbytes = fa_split_workspace_bytes(B, H, q_len, D, num_splits)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
        st = fa_flex_attention_fwd_split(
            _DTYPES[q.dtype], B, H, H_kv, q_len, kv_len, D,
            q.data_ptr(), q.stride()[:3], k.data_ptr(), k.stride()[:3],
            v.data_ptr(), v.stride()[:3], float(scale), block_mask.to_c(),
            score.to_c(), num_splits, ws.data_ptr(), nbytes, out.data_ptr(),
            lse.data_ptr() if lse is not None else None,
            _stream_handle(q.device))
    C.check(st, "fa_flex_attention_fwd_split")
    return out, lse


def flex_attention_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                            o: torch.Tensor, lse: torch.Tensor,
                            dout: torch.Tensor, block_mask: BlockMask,
                            score_mod=None, scale: Optional[float] = None,
                            dq_kv_order: Optional[bool] = None,
                            num_splits: Optional[int] = None):
    """Gradients ``(dQ, dK, dV)`` of ``O = flex_attention(q, k, v,
    block_mask, score_mod, scale)`` for the upstream gradient ``dout``.

    bf16 only; ``o`` and ``lse`` are what the forward returned for the same
    arguments; ``block_mask`` block sizes in {64, 128} (an int or a pair).
    One fa_flex_attention_bwd call with a workspace allocated here;
    the results are deterministic. ``dq_kv_order`` (default: the block
    mask's) is the order of dQ's sum over key blocks, True descending.
    ``num_splits``: parts per gradient row (1 ... 64), added by one more
    kernel; None picks :func:`auto_bwd_splits` for the device."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D (B, H, S, D)")
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype
            == torch.bfloat16):
        raise ValueError("the backward takes bf16 q, k, v, o and dout")
    for t in (q, k, v, o, lse, dout):
        if not t.is_cuda or t.device != q.device:
            raise ValueError("all tensors must be on q's HIP device")
    B, H, q_len, D = q.shape
    Bk, H_kv, kv_len, Dk = k.shape
    if k.shape != v.shape or Bk != B or Dk != D:
        raise ValueError("k and v must be (B, H_kv, KV_LEN, D)")
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must have q's shape")
    if lse.shape != (B, H, q_len) or lse.dtype != torch.float32:
        raise ValueError("lse must be fp32 (B, H, Q_LEN)")
    for t in (q, k, v):
        if t.numel() and t.stride(-1) != 1:
            raise ValueError("the head dimension must be contiguous")
    _check_doc_rows(block_mask, B)
    o = o.contiguous()
    dout = dout.contiguous()
    lse = lse.contiguous()
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    score = _score_from(score_mod)
    dq = torch.empty((B, H, q_len, D), dtype=q.dtype, device=q.device)
    dk = torch.empty((B, H_kv, kv_len, D), dtype=q.dtype, device=q.device)
    dv = torch.empty_like(dk)
    if dq_kv_order is None:
        dq_kv_order = getattr(block_mask, "dq_kv_order", True)
    bm = block_mask.to_c()
    if num_splits is None:
        num_splits = auto_bwd_splits(
            B, H_kv, block_mask.num_kv_blocks,
            torch.cuda.get_device_properties(q.device).multi_processor_count)
    nbytes = fa_bwd_workspace_bytes(B, H, H_kv, q_len, kv_len, D, bm,
                                    num_splits)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        st = fa_flex_attention_bwd(
            C.FA_BF16, B, H, H_kv, q_len, kv_len, D,
            q.data_ptr(), q.stride()[:3], k.data_ptr(), k.stride()[:3],
            v.data_ptr(), v.stride()[:3], float(scale), bm, score.to_c(),
            int(bool(dq_kv_order)), int(num_splits), o.data_ptr(),
            lse.data_ptr(),
            dout.data_ptr(), ws.data_ptr(),
            nbytes, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
            _stream_handle(q.device))
    C.check(st, "fa_flex_attention_bwd")
    return dq, dk, dv


def flex_attention_decode_paged(q: torch.Tensor, k_pages: torch.Tensor,
                                v_pages: torch.Tensor,
                                page_table: torch.Tensor,
                                seq_lens: torch.Tensor, mask_mod="causal",
                                score_mod=None, scale: Optional[float] = None,
                                num_splits: Optional[int] = None, *,
                                window=None, doc_id=None,
                                return_lse: bool = True):
    """One decode step per sequence over a paged key/value cache.

    ``q``: bf16 ``(B, H, D)``, each sequence's newest token (already in the
    cache). ``k_pages`` / ``v_pages``: bf16 ``(num_pages, page_size, H_kv,
    D)`` pools (any strides with D contiguous). ``page_table``: int32
    ``(B, max_pages)``; ``seq_lens``: int32 ``(B,)`` cached tokens per
    sequence. ``mask_mod``: "causal", "none", "sliding_window" /
    "local_window" (``window``), "document" (``doc_id`` by token position)
    or a :class:`MaskMod`. Returns ``(O (B, H, D), LSE (B, H))``.
    ``num_splits`` None picks :func:`auto_decode_splits`."""
    if q.dim() != 3 or k_pages.dim() != 4 or v_pages.dim() != 4:
        raise ValueError("q must be (B, H, D) and the pools (P, page, H_kv, D)")
    if not (q.dtype == k_pages.dtype == v_pages.dtype == torch.bfloat16):
        raise ValueError("the paged decode takes bf16 q and pools")
    if page_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("page_table and seq_lens must be int32")
    for t in (q, k_pages, v_pages, page_table, seq_lens):
        if not t.is_cuda or t.device != q.device:
            raise ValueError("all tensors must be on q's HIP device")
    B, H, D = q.shape
    P, page_size, H_kv, Dk = k_pages.shape
    if v_pages.shape != k_pages.shape or Dk != D:
        raise ValueError("k_pages and v_pages must be (P, page_size, H_kv, D)")
    if page_table.dim() != 2 or page_table.shape[0] != B or \
            not page_table.is_contiguous():
        raise ValueError("page_table must be a contiguous (B, max_pages) tensor")
    if seq_lens.shape != (B,) or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous (B,) tensor")
    for t in (q, k_pages, v_pages):
        if t.numel() and t.stride(-1) != 1:
            raise ValueError("the head dimension must be contiguous")
    max_pages = page_table.shape[1]
    mask = _mask_from(mask_mod, window, doc_id)
    if mask.kind == C.FA_MASK_DOCUMENT and mask.per_batch and \
            mask.doc_id.shape[0] != B:
        raise ValueError("per-sequence doc_id must be (B, L)")
    score = _score_from(score_mod)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if num_splits is None:
        num_splits = auto_decode_splits(
            B, H_kv, max_pages * page_size,
            torch.cuda.get_device_properties(q.device).multi_processor_count)
    out = torch.empty((B, H, D), dtype=q.dtype, device=q.device)
    lse = (torch.empty((B, H), dtype=torch.float32, device=q.device)
           if return_lse else None)
    nbytes = fa_split_workspace_bytes(B, H, 1, D, num_splits)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        st = fa_flex_attention_decode_paged(
            B, H, H_kv, D, q.data_ptr(), q.stride()[:2], k_pages.data_ptr(),
            k_pages.stride()[:3], v_pages.data_ptr(), v_pages.stride()[:3], P,
            page_size, page_table.data_ptr(), max_pages, seq_lens.data_ptr(),
            float(scale), mask.to_c(), score.to_c(), num_splits,
            ws.data_ptr(), nbytes, out.data_ptr(),
            lse.data_ptr() if lse is not None else None,
            _stream_handle(q.device))
    C.check(st, "fa_flex_attention_decode_paged")
    return out, lse


def masked_softmax(scores: torch.Tensor, mask_mod="causal", q_offset: int = 0,
                   *, window=None, doc_id=None,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Softmax over the last axis of bf16 scores ``(..., Q, K)`` with a
    built-in mask_mod folded in (row i is query position ``i + q_offset``):
    masked entries are exactly 0, a row with no allowed key is all zeros.
    One fa_masked_softmax call; returns bf16 probabilities of the same
    shape (contiguous)."""
    if scores.dtype != torch.bfloat16 or not scores.is_cuda:
        raise ValueError("scores must be a bf16 HIP device tensor")
    if scores.dim() < 2:
        raise ValueError("scores must be (..., Q, K)")
    Q, K = scores.shape[-2], scores.shape[-1]
    x = scores.reshape(-1, Q, K) if scores.dim() != 3 else scores
    if x.numel() and x.stride(-1) != 1:
        x = x.contiguous()
    BH = x.shape[0]
    mask = _mask_from(mask_mod, window, doc_id)
    if mask.kind == C.FA_MASK_DOCUMENT and mask.per_batch:
        raise ValueError("the masked softmax takes one shared doc_id array")
    if out is None:
        out = torch.empty(scores.shape, dtype=torch.bfloat16, device=scores.device)
    with torch.cuda.device(scores.device):
        st = fa_masked_softmax(BH, Q, K, int(q_offset), x.data_ptr(),
                               (x.stride(0), x.stride(1)), mask.to_c(),
                               out.data_ptr(), _stream_handle(scores.device))
    C.check(st, "fa_masked_softmax")
    return out

