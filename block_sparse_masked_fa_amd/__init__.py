"""block_sparse_masked_fa_amd: FlexAttention-style block-sparse masked
attention (forward and backward) for MI355X (gfx950).

The work runs in ``libflexattn.so`` (hand-written HIP kernels behind a C ABI,
``include/flexattn.h``); this package is its Python binding. Importing it
does not load the library; the first call does, and fails loudly if the
library has not been built (``python -m block_sparse_masked_fa_amd.build``).
"""
from .api import (  # noqa: F401
    BlockMask, FlexAttnError, MaskMod, ScoreMod, alibi, auto_num_splits,
    causal, create_block_mask, document, fa_block_mask_dims,
    fa_bwd_workspace_bytes, fa_create_block_mask, fa_flex_attention_bwd,
    fa_flex_attention_fwd, fa_flex_attention_fwd_split,
    fa_split_workspace_bytes, flex_attention, flex_attention_backward,
    auto_bwd_splits, auto_decode_splits, fa_flex_attention_decode_paged,
    flex_attention_decode_paged, local_window, no_mask, masked_softmax,
    fa_masked_softmax, fwd_workspace, fa_flex_attention_fwd_split_noalloc,
    sliding_window,
    softcap,
)
from ._capi import LIB_PATH, lib  # noqa: F401
