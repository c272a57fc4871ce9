"""The longest rows: causal attention with ALiBi over Q = KV = 131072 tokens
(1024 key blocks of 128 in the last query block's list, 524,800 live blocks
in all), D = 128, one head. The forward (unsplit and in 4 parts) on sampled
rows, and the backward: dQ on sampled rows, dK and dV of the last 64 keys
(under the causal mask only the last 64 rows see them), all against the fp64
oracle, which evaluates those rows only."""
import numpy as np
import pytest
import torch

import block_sparse_masked_fa_amd as fa
import workloads as WL
from oracle import oracle as O
from tests.helpers import TOL, assert_close, sample_rows
from tests.test_gpu_backward import assert_grad_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
L = 131072


def test_longest_rows_forward_and_backward():
    w = WL.Workload("long", "bf16", 1, 1, 1, L, L, 128, "causal", 128, 128, seed=0,
                    score="alibi")
    rng = np.random.default_rng(21)
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16) for x in WL.draw_qkv(rng, w))
    do = torch.from_numpy(rng.standard_normal(q.shape, dtype=np.float32)).to(torch.bfloat16)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    bm = fa.create_block_mask("causal", None, None, L, L, device=DEV)
    assert int(bm.kv_num_blocks[0, 0, -1]) + int(bm.full_kv_num_blocks[0, 0, -1]) == L // 128
    tail = np.arange(L - 64, L)
    rows = np.union1d(sample_rows(L, 128, None, n_random=12, seed=3), tail)
    o_ref, l_ref = O.attention(q, k, v, mask="causal", score="alibi", scale=w.scale, rows=rows)
    r = torch.from_numpy(rows).to(DEV)
    for ns in (1, 4):
        print(f"[long] forward splits={ns}", flush=True)
        o, lse = fa.flex_attention(qd, kd, vd, bm, score_mod="alibi", scale=w.scale,
                                   num_splits=ns)
        torch.cuda.synchronize()
        assert_close(o[:, :, r], lse[:, :, r], o_ref, l_ref, TOL["bf16"], f"long splits={ns}")
    print("[long] backward", flush=True)
    o, lse = fa.flex_attention(qd, kd, vd, bm, score_mod="alibi", scale=w.scale, num_splits=1)
    dq, dk, dv = fa.flex_attention_backward(qd, kd, vd, o, lse, dod, bm, score_mod="alibi",
                                            scale=w.scale, num_splits=1)
    torch.cuda.synchronize()
    dq_ref, dk_ref, dv_ref = O.attention_backward(q, k, v, do, mask="causal", score="alibi",
                                                  scale=w.scale, rows=rows)
    assert_grad_close(dq[:, :, r], dq_ref, "dQ long")
    cols = torch.from_numpy(tail).to(DEV)
    assert_grad_close(dk[:, :, cols], dk_ref[:, :, tail], "dK long")
    assert_grad_close(dv[:, :, cols], dv_ref[:, :, tail], "dV long")
