"""The no-allocation split-KV forward (fa_flex_attention_fwd_split_noalloc)
against the workspace one (fa_flex_attention_fwd_split): both run the same
kernels, so the outputs must be identical, on two calls in a row with the
second one smaller; sampled rows also against the fp64 oracle. A request
larger than the fixed scratch is refused before anything is launched."""
import numpy as np
import pytest
import torch

import block_sparse_masked_fa_amd as fa
from block_sparse_masked_fa_amd import _capi as C
import workloads as WL
from tests.helpers import TOL, assert_close, oracle_case, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _noalloc(q, k, v, bm, score, scale, num_splits):
    B, H, q_len, D = q.shape
    H_kv, kv_len = k.shape[1], k.shape[2]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, q_len), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        st = fa.fa_flex_attention_fwd_split_noalloc(
            C.FA_BF16, B, H, H_kv, q_len, kv_len, D, q.data_ptr(),
            q.stride()[:3], k.data_ptr(), k.stride()[:3], v.data_ptr(),
            v.stride()[:3], scale, bm.to_c(), score, num_splits, o.data_ptr(),
            lse.data_ptr(), torch.cuda.current_stream(q.device).cuda_stream)
    return st, o, lse


def _case(w, seed, num_splits, mask_kind, score_c, score_arg):
    rng = np.random.default_rng(seed)
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16) for x in WL.draw_qkv(rng, w))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    bm = fa.create_block_mask(mask_kind, None, None, w.q_len, w.kv_len,
                              device=DEV, BLOCK_SIZE=w.block_m, window=w.window)
    st, o_n, l_n = _noalloc(qd, kd, vd, bm, score_c, w.scale, num_splits)
    C.check(st, "fa_flex_attention_fwd_split_noalloc")
    o_w, l_w = fa.flex_attention(qd, kd, vd, bm, score_mod=score_arg,
                                 scale=w.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    assert torch.equal(o_n, o_w) and torch.equal(l_n, l_w), \
        "no-allocation split differs from the workspace split"
    rows = sample_rows(w.q_len, w.block_m, None, n_random=24, seed=seed)
    o_ref, l_ref = oracle_case(q, k, v, w, None, rows=rows)
    r = torch.from_numpy(rows).to(DEV)
    assert_close(o_n[:, :, r], l_n[:, :, r], o_ref, l_ref, TOL["bf16"],
                 f"no-allocation split {num_splits}")


def test_noalloc_split_matches_workspace_split_twice():
    # first call: c2's shape and part count (dense causal 8K, 8 parts);
    # second call, smaller: 3 heads of a ragged 1500-token sliding window
    # with ALiBi in 5 parts, on the same scratch
    w1 = WL.get("c2")
    print("[noalloc] call 1: c2 shape, 8 parts", flush=True)
    _case(w1, 1, 8, "causal", C.fa_score_mod(kind=C.FA_SCORE_NONE), None)
    w2 = WL.Workload("small", "bf16", 1, 3, 3, 1500, 1500, 128,
                     "sliding_window", 128, 128, seed=0, window=300,
                     score="alibi")
    print("[noalloc] call 2: smaller, 5 parts", flush=True)
    _case(w2, 2, 5, "sliding_window", C.fa_score_mod(kind=C.FA_SCORE_ALIBI),
          "alibi")


def test_noalloc_refuses_more_than_its_scratch():
    # 64 parts of a 32-head 8K-row problem need ~1.1 GB of partial results
    B, H, q_len, D = 1, 32, 8192, 128
    need = fa.fa_split_workspace_bytes(B, H, q_len, D, 64)
    assert need > C.FA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, q_len, D), dtype=torch.bfloat16, device=DEV)
    bm = fa.create_block_mask("causal", None, None, q_len, q_len, device=DEV)
    st, _, _ = _noalloc(q, q, q, bm, None, 0.088, 64)
    assert st == C.FA_ERR_INVALID_VALUE
    assert b"scratch" in C.lib().fa_last_error()


def test_noalloc_one_part_is_the_plain_forward():
    # num_splits = 1 uses no scratch: the forward itself (D = 64, document
    # mask with soft-cap), bitwise equal to flex_attention unsplit
    w = WL.Workload("small", "bf16", 2, 4, 2, 700, 700, 64, "document", 128,
                    128, seed=0, score="softcap", softcap=20.0)
    rng = np.random.default_rng(5)
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(DEV) for x in WL.draw_qkv(rng, w))
    doc = torch.from_numpy(np.sort(rng.integers(0, 3, 700)).astype(np.int32)).to(DEV)
    bm = fa.create_block_mask("document", None, None, 700, 700, device=DEV, doc_id=doc)
    print("[noalloc] one part", flush=True)
    st, o_n, l_n = _noalloc(q, k, v, bm,
                            C.fa_score_mod(kind=C.FA_SCORE_SOFTCAP, softcap=20.0),
                            w.scale, 1)
    C.check(st, "fa_flex_attention_fwd_split_noalloc")
    o_w, l_w = fa.flex_attention(q, k, v, bm, score_mod=("softcap", 20.0), scale=w.scale,
                                 num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(o_n, o_w) and torch.equal(l_n, l_w)
