"""Element offsets past 2^31: Q, K and V as views whose batch stride is
2^31 + 4096 elements (the second batch entry lies more than 4 GiB into its
buffer), and a paged key/value pool whose pages in use sit past element
2^31 of the pool. The shapes are small, so every row is compared with the
fp64 oracle: the forward (unsplit and in parts), the backward, and the
paged decode step. Each buffer is about 4.3 GB of device memory."""
import numpy as np
import pytest
import torch

import block_sparse_masked_fa_amd as fa
import workloads as WL
from oracle import oracle as O
from tests.helpers import TOL, assert_close
from tests.test_gpu_backward import assert_grad_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BIG_STRIDE = 2 ** 31 + 4096  # elements between batch entries


def _big_view(x: torch.Tensor) -> torch.Tensor:
    """``x`` (B, H, S, D) copied into a device view with batch stride
    BIG_STRIDE (the memory between the entries is never written)."""
    B, H, S, D = x.shape
    buf = torch.empty(BIG_STRIDE * (B - 1) + H * S * D, dtype=x.dtype, device=DEV)
    v = buf.as_strided((B, H, S, D), (BIG_STRIDE, S * D, D, 1))
    v.copy_(x.to(DEV))
    return v


def _inputs(w, seed):
    rng = np.random.default_rng(seed)
    q, k, v = WL.draw_qkv(rng, w)
    do = rng.standard_normal(q.shape, dtype=np.float32)
    return tuple(torch.from_numpy(a).to(torch.bfloat16) for a in (q, k, v, do))


@pytest.mark.parametrize("mask,score", [("causal", "alibi"), ("sliding_window", "softcap")])
def test_forward_and_backward_past_2_31(mask, score):
    w = WL.Workload("big", "bf16", 2, 4, 2, 520, 520, 128, mask, 128, 128, seed=0,
                    window=300 if mask == "sliding_window" else None, score=score,
                    softcap=20.0 if score == "softcap" else None)
    q, k, v, do = _inputs(w, 3)
    print(f"[large offsets] {mask} {score}", flush=True)
    qv, kv, vv = _big_view(q), _big_view(k), _big_view(v)
    assert qv.storage_offset() == 0 and qv.stride(0) * (qv.shape[0] - 1) > 2 ** 31
    bm = fa.create_block_mask(mask, None, None, w.q_len, w.kv_len, device=DEV,
                              window=w.window)
    sm = {"alibi": "alibi", "softcap": ("softcap", 20.0)}[score]
    o_ref, l_ref = O.attention(q, k, v, mask=mask, score=score, scale=w.scale,
                               window=w.window, softcap=w.softcap)
    for ns in (1, 3):
        o, lse = fa.flex_attention(qv, kv, vv, bm, score_mod=sm, scale=w.scale,
                                   num_splits=ns)
        torch.cuda.synchronize()
        assert_close(o, lse, o_ref, l_ref, TOL["bf16"], f"{mask} {score} splits={ns}")
    o, lse = fa.flex_attention(qv, kv, vv, bm, score_mod=sm, scale=w.scale, num_splits=1)
    dq, dk, dvg = fa.flex_attention_backward(qv, kv, vv, o, lse, do.to(DEV), bm,
                                             score_mod=sm, scale=w.scale, num_splits=1)
    torch.cuda.synchronize()
    g_ref = O.attention_backward(q, k, v, do, mask=mask, score=score, scale=w.scale,
                                 window=w.window, softcap=w.softcap)
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dvg), g_ref):
        assert_grad_close(g, r, f"{name} {mask} {score}")
    del qv, kv, vv
    torch.cuda.empty_cache()


def test_decode_pages_past_2_31():
    # pool of (P, 128, 1, 128) pages: page 131072 starts at element 2^31
    page, H_kv, D, H = 128, 1, 128, 4
    P = 2 ** 31 // (page * H_kv * D) + 24
    lens = np.array([300, 1000, 129], dtype=np.int32)
    B = len(lens)
    max_pages = int(-(-lens.max() // page))
    rng = np.random.default_rng(9)
    # pages in use: straddling element 2^31 of the pool and past it
    first = 2 ** 31 // (page * H_kv * D) - 3
    table = np.full((B, max_pages), -1, dtype=np.int32)
    used = rng.permutation(np.arange(first, P))[: int(sum(-(-n // page) for n in lens))]
    u = 0
    for b, n in enumerate(lens):
        for t in range(-(-int(n) // page)):
            table[b, t] = used[u]
            u += 1
    q = torch.from_numpy(rng.standard_normal((B, H, D), dtype=np.float32)).to(torch.bfloat16)
    print("[large offsets] decode", flush=True)
    kp = torch.empty((P, page, H_kv, D), dtype=torch.bfloat16, device=DEV)
    vp = torch.empty_like(kp)
    # the oracle's pool: the used pages only, the table remapped onto it
    small_k = torch.from_numpy(
        rng.standard_normal((len(used), page, H_kv, D), dtype=np.float32)).to(torch.bfloat16)
    small_v = torch.from_numpy(
        rng.standard_normal((len(used), page, H_kv, D), dtype=np.float32)).to(torch.bfloat16)
    idx = torch.from_numpy(used.astype(np.int64)).to(DEV)
    kp[idx] = small_k.to(DEV)
    vp[idx] = small_v.to(DEV)
    remap = {int(pg): i for i, pg in enumerate(used)}
    small_table = np.vectorize(lambda x: remap.get(int(x), -1))(table).astype(np.int32)
    o_ref, l_ref = O.decode_paged(q, small_k, small_v, small_table, lens, mask="causal",
                                  score="alibi", scale=D ** -0.5)
    for ns in (1, 4):
        o, lse = fa.flex_attention_decode_paged(
            q.to(DEV), kp, vp, torch.from_numpy(table).to(DEV),
            torch.from_numpy(lens).to(DEV), mask_mod="causal", score_mod="alibi",
            scale=D ** -0.5, num_splits=ns)
        torch.cuda.synchronize()
        og = o.float().cpu().double().numpy()
        lg = lse.cpu().double().numpy()
        assert np.abs(og - o_ref).max() <= TOL["bf16"], f"decode splits={ns}"
        assert np.abs(lg - l_ref).max() <= TOL["bf16"], f"decode LSE splits={ns}"
    del kp, vp
    torch.cuda.empty_cache()
