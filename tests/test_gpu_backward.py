"""GPU parity of fa_flex_attention_bwd (dQ, dK, dV) against the fp64 oracle.

The forward's O and LSE come from the GPU (the backward consumes them); the
oracle's gradients are computed from the same bf16 inputs by the chain rule.
Small cases compare every element of the three gradients; the workloads at
full size compare dQ on a deterministic row sample and dK / dV of the last
keys (whose rows the oracle evaluates), plus identities over all keys."""
import zlib

import numpy as np
import pytest
import torch

import block_sparse_masked_fa_amd as fa
import workloads as WL
from oracle import oracle as O
from tests.helpers import caller_lists, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# Bar: max |grad - oracle| <= TOL_BWD * max(1, max |oracle grad|), per tensor.
# The kernels round P and dT = dS * score_mod' to bf16 before the MFMA
# products (relative 2^-9 each) and the gradients to bf16 on output (another
# 2^-9 of the value); delta uses the forward's bf16 O. Summed over the
# contraction with random signs these stay well below 1% of the largest
# gradient; 2e-2 leaves room for the heavy-tailed rows of small cases.
TOL_BWD = 2e-2


def _score_arg(score, cap):
    if score == "softcap":
        return ("softcap", cap)
    return None if score == "none" else score


def _doc_t(doc):
    return torch.from_numpy(np.ascontiguousarray(doc)).to(DEV) if doc is not None else None


def gpu_fwd_bwd(w, q, k, v, do, doc=None, sep=True, bm=None, order=None,
                splits=1):
    if bm is None:
        bm = fa.create_block_mask(w.mask, None, None, w.q_len, w.kv_len,
                                  device=DEV, BLOCK_SIZE=w.block_m,
                                  separate_full_blocks=sep, window=w.window,
                                  doc_id=_doc_t(doc))
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    sm = _score_arg(w.score, w.softcap)
    o, lse = fa.flex_attention(qd, kd, vd, bm, score_mod=sm, scale=w.scale,
                               num_splits=1)
    dq, dk, dv = fa.flex_attention_backward(qd, kd, vd, o, lse, dod, bm,
                                            score_mod=sm, scale=w.scale,
                                            dq_kv_order=order, num_splits=splits)
    torch.cuda.synchronize()
    return dq, dk, dv


def oracle_bwd(w, q, k, v, do, doc=None, rows=None):
    return O.attention_backward(q, k, v, do, mask=w.mask, score=w.score,
                                scale=w.scale, window=w.window, doc_id=doc,
                                softcap=w.softcap, rows=rows)


def assert_grad_close(g_gpu, g_ref, what):
    g = g_gpu.detach().float().cpu().double().numpy()
    assert g.shape == g_ref.shape, (what, g.shape, g_ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite gradient"
    if g.size == 0:
        return 0.0
    ref_max = max(1.0, float(np.abs(g_ref).max()))
    err = float(np.abs(g - g_ref).max())
    assert err <= TOL_BWD * ref_max, \
        f"{what}: max |err| = {err:.3g} > {TOL_BWD} * {ref_max:.3g}"
    return err / ref_max


def _inputs(w, seed):
    rng = np.random.default_rng(seed)
    q, k, v = WL.draw_qkv(rng, w)
    do = rng.standard_normal(q.shape, dtype=np.float32)
    return tuple(torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v, do))


SMALL = []
for D, blk in ((128, 128), (64, 128), (128, 64), (64, 64)):
    for mask in ("causal", "sliding_window", "document", "none", "local_window"):
        for score in ("none", "softcap", "alibi"):
            SMALL.append((D, blk, mask, score))


@pytest.mark.parametrize("D,blk,mask,score", SMALL)
def test_small_backward(D, blk, mask, score):
    # several tiles and ragged tails on both axes, q_len != kv_len, grouped
    # heads (dK / dV sum over two query heads), both list layouts (with the
    # descending and the ascending dQ order), unsplit and split into parts
    # (the automatic count: here one part per key block, so some parts of
    # short rows are empty)
    ql, kl = 3 * blk + 37, 2 * blk + 101
    w = WL.Workload("small", "bf16", 2, 4, 2, ql, kl, D, mask, blk, blk,
                    seed=0, window=blk + 13 if "window" in mask else None,
                    score=score, softcap=3.0 if score == "softcap" else None)
    rng = np.random.default_rng(zlib.crc32(f"bwd{D}{blk}{mask}{score}".encode()))
    doc = (np.sort(rng.integers(0, 4, max(ql, kl))).astype(np.int32)
           if mask == "document" else None)
    q, k, v, do = _inputs(w, 23)
    ref = oracle_bwd(w, q, k, v, do, doc)
    for sep, ns in ((True, 1), (False, 1), (False, None)):
        print(f"[bwd small] D={D} blk={blk} {mask} {score} sep={sep} splits={ns}",
              flush=True)
        got = gpu_fwd_bwd(w, q, k, v, do, doc, sep=sep, order=sep, splits=ns)
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            assert_grad_close(g, r, f"{name} D={D} blk={blk} {mask} {score} sep={sep} "
                                    f"splits={ns}")


@pytest.mark.parametrize("D,blk", [(128, 128), (64, 64)])
def test_backward_per_batch_documents_and_per_head_masks(D, blk):
    # doc_id [B, L] (a block mask per batch entry), then a block mask built
    # for explicit B and H (no broadcast of the lists)
    B, H, T = 3, 2, 3 * blk + 45
    w = WL.Workload("small", "bf16", B, H, H, T, T, D, "document", blk, blk,
                    seed=0)
    rng = np.random.default_rng(D + blk + 1)
    doc = np.stack([np.sort(rng.integers(0, n, T)) for n in (3, 6, 1)]
                   ).astype(np.int32)
    q, k, v, do = _inputs(w, 43)
    ref = oracle_bwd(w, q, k, v, do, doc)
    bm = fa.create_block_mask("document", B, None, T, T, device=DEV,
                              BLOCK_SIZE=blk, doc_id=_doc_t(doc))
    for ns in (1, 3):
        print(f"[bwd per-batch docs] D={D} blk={blk} splits={ns}", flush=True)
        got = gpu_fwd_bwd(w, q, k, v, do, doc, bm=bm, splits=ns)
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            assert_grad_close(g, r, f"{name} per-batch docs D={D} splits={ns}")
    w2 = w.replace(mask="causal")
    ref2 = oracle_bwd(w2, q, k, v, do)
    bm2 = fa.create_block_mask("causal", B, H, T, T, device=DEV, BLOCK_SIZE=blk)
    for ns in (1, 3):
        print(f"[bwd per-head lists] D={D} blk={blk} splits={ns}", flush=True)
        got2 = gpu_fwd_bwd(w2, q, k, v, do, bm=bm2, splits=ns)
        for name, g, r in zip(("dQ", "dK", "dV"), got2, ref2):
            assert_grad_close(g, r, f"{name} per-head lists D={D} splits={ns}")


def test_backward_rows_without_keys():
    # rows i >= kv_len + W - 1 see no key: their dQ is 0 and they add
    # nothing to dK / dV
    w = WL.Workload("empty", "bf16", 1, 2, 1, 400, 150, 64, "sliding_window",
                    64, 64, seed=0, window=60)
    q, k, v, do = _inputs(w, 6)
    ref = oracle_bwd(w, q, k, v, do)
    for ns in (1, 4):
        print(f"[bwd rows without keys] splits={ns}", flush=True)
        got = gpu_fwd_bwd(w, q, k, v, do, splits=ns)
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            assert_grad_close(g, r, f"{name} rows without keys splits={ns}")
        assert (got[0][:, :, 209:] == 0).all()


def test_backward_zero_lengths():
    # no keys: dQ = 0; no queries: dK = dV = 0 (outputs pre-filled with NaN
    # must be overwritten)
    blk = 128
    q = torch.randn(1, 2, 130, 128, device=DEV).to(torch.bfloat16)
    k0 = torch.zeros(1, 1, 0, 128, device=DEV, dtype=torch.bfloat16)
    bm = fa.create_block_mask("causal", None, None, 130, 0, device=DEV,
                              BLOCK_SIZE=blk)
    o, lse = fa.flex_attention(q, k0, k0, bm, num_splits=1)
    print("[bwd zero-length keys]", flush=True)
    dq, dk, dv = fa.flex_attention_backward(q, k0, k0, o, lse, torch.randn_like(q),
                                            bm)
    torch.cuda.synchronize()
    assert (dq == 0).all() and dk.numel() == 0 and dv.numel() == 0

    q0 = torch.zeros(1, 2, 0, 128, device=DEV, dtype=torch.bfloat16)
    k = torch.randn(1, 1, 200, 128, device=DEV).to(torch.bfloat16)
    bm = fa.create_block_mask("causal", None, None, 0, 200, device=DEV,
                              BLOCK_SIZE=blk)
    lse0 = torch.zeros(1, 2, 0, device=DEV)
    dk = torch.full((1, 1, 200, 128), float("nan"), device=DEV, dtype=torch.bfloat16)
    dv = dk.clone()
    nbytes = fa.fa_bwd_workspace_bytes(1, 2, 1, 0, 200, 128, bm.to_c())
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
    print("[bwd zero-length queries]", flush=True)
    st = fa.fa_flex_attention_bwd(
        0, 1, 2, 1, 0, 200, 128, q0.data_ptr(), q0.stride()[:3], k.data_ptr(),
        k.stride()[:3], k.data_ptr(), k.stride()[:3], 128 ** -0.5, bm.to_c(),
        None, 1, 1, q0.data_ptr(), lse0.data_ptr(), q0.data_ptr(), ws.data_ptr(),
        nbytes, q0.data_ptr(), dk.data_ptr(), dv.data_ptr(), None)
    torch.cuda.synchronize()
    assert st == 0
    assert (dk == 0).all() and (dv == 0).all()


def test_backward_strided_views_and_nan_tails():
    # q, k, v as (B, S, H, D) memory viewed as (B, H, S, D); the sequences
    # end inside larger buffers whose rows past the end hold NaN: the
    # gradient must read neither query rows past Q_LEN nor keys past KV_LEN
    ql, kl, D = 300, 230, 64
    w = WL.Workload("view", "bf16", 2, 4, 2, ql, kl, D, "local_window", 64, 64,
                    seed=0, window=50, score="alibi")
    q, k, v, do = _inputs(w, 9)
    ref = oracle_bwd(w, q, k, v, do)
    qb = torch.full((2, ql + 64, 4, D), float("nan"), dtype=torch.bfloat16)
    kb = torch.full((2, 2, kl + 64, 2, D), float("nan"), dtype=torch.bfloat16)
    qb[:, :ql] = q.transpose(1, 2)
    kb[0, :, :kl] = k.transpose(1, 2)
    kb[1, :, :kl] = v.transpose(1, 2)
    qb, kb = qb.to(DEV), kb.to(DEV)
    qv = qb[:, :ql].transpose(1, 2)
    kv_, vv = kb[0, :, :kl].transpose(1, 2), kb[1, :, :kl].transpose(1, 2)
    bm = fa.create_block_mask("local_window", None, None, ql, kl, device=DEV,
                              BLOCK_SIZE=64, window=50)
    o, lse = fa.flex_attention(qv, kv_, vv, bm, score_mod="alibi", num_splits=1)
    for ns in (1, 2):
        print(f"[bwd strided views, NaN tails] splits={ns}", flush=True)
        got = fa.flex_attention_backward(qv, kv_, vv, o, lse, do.to(DEV), bm,
                                         score_mod="alibi", num_splits=ns)
        torch.cuda.synchronize()
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            assert_grad_close(g, r, f"{name} strided views splits={ns}")


def test_backward_deterministic():
    w = WL.Workload("det", "bf16", 2, 4, 2, 700, 700, 128, "document", 128,
                    128, seed=0, score="softcap", softcap=20.0)
    doc = WL.doc_ids([250, 300, 150])
    q, k, v, do = _inputs(w, 3)
    print("[bwd deterministic]", flush=True)
    first = gpu_fwd_bwd(w, q, k, v, do, doc)
    for _ in range(3):
        again = gpu_fwd_bwd(w, q, k, v, do, doc)
        for a, b in zip(first, again):
            assert torch.equal(a, b)


@pytest.mark.parametrize("mask", ["causal", "document", "none"])
def test_backward_dq_order(mask):
    # dq_kv_order: ascending and descending key-block order give dQ within
    # the bar of the oracle and of each other, each bit-reproducible; dK and
    # dV do not depend on it
    blk = 64
    w = WL.Workload("order", "bf16", 1, 2, 2, 5 * blk + 11, 5 * blk + 11, 128,
                    mask, blk, blk, seed=0, score="softcap", softcap=5.0)
    doc = WL.doc_ids([100, 150, 81]) if mask == "document" else None
    q, k, v, do = _inputs(w, 77)
    ref = oracle_bwd(w, q, k, v, do, doc)
    res = {}
    for order in (False, True):
        print(f"[bwd dq order] {mask} descending={order}", flush=True)
        a = gpu_fwd_bwd(w, q, k, v, do, doc, order=order)
        b = gpu_fwd_bwd(w, q, k, v, do, doc, order=order)
        for x, y in zip(a, b):
            assert torch.equal(x, y)
        for name, g, r in zip(("dQ", "dK", "dV"), a, ref):
            assert_grad_close(g, r, f"{name} {mask} descending={order}")
        res[order] = a
    assert torch.equal(res[False][1], res[True][1])
    assert torch.equal(res[False][2], res[True][2])
    assert (res[False][0].float() - res[True][0].float()).abs().max().item() <= \
        TOL_BWD * max(1.0, float(np.abs(ref[0]).max()))


PAIRS = []
for D in (128, 64):
    for bq, bk in ((128, 64), (64, 128)):
        for mask in ("causal", "sliding_window", "document", "none", "local_window"):
            for score in ("none", "softcap", "alibi"):
                PAIRS.append((D, bq, bk, mask, score))


@pytest.mark.parametrize("D,bq,bk,mask,score", PAIRS)
def test_backward_block_size_pairs(D, bq, bk, mask, score):
    # BLOCK_SIZE as a (q, kv) pair: query and key blocks of different sizes,
    # ragged tails on both axes, grouped heads
    ql, kl = 3 * bq + 29, 3 * bk + 77
    w = WL.Workload("pair", "bf16", 2, 4, 2, ql, kl, D, mask, bq, bk, seed=0,
                    window=bk + 21 if "window" in mask else None, score=score,
                    softcap=3.0 if score == "softcap" else None)
    rng = np.random.default_rng(zlib.crc32(f"bwdpair{D}{bq}{bk}{mask}{score}".encode()))
    doc = (np.sort(rng.integers(0, 3, max(ql, kl))).astype(np.int32)
           if mask == "document" else None)
    q, k, v, do = _inputs(w, 37)
    ref = oracle_bwd(w, q, k, v, do, doc)
    bm = fa.create_block_mask(mask, None, None, ql, kl, device=DEV,
                              BLOCK_SIZE=(bq, bk), window=w.window, doc_id=_doc_t(doc))
    for ns in (1, 2):
        print(f"[bwd block pair] D={D} ({bq},{bk}) {mask} {score} splits={ns}",
              flush=True)
        got = gpu_fwd_bwd(w, q, k, v, do, doc, bm=bm, splits=ns)
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            assert_grad_close(g, r, f"{name} pair ({bq},{bk}) D={D} {mask} {score} "
                                    f"splits={ns}")


@pytest.mark.parametrize("mask,blk", [("causal", 64), ("document", 128),
                                      ("sliding_window", 64)])
def test_backward_split_parts(mask, blk):
    # num_splits from 2 up to 64 (more parts than any row has blocks: the
    # surplus parts are empty and write zero sums), grouped heads (the parts
    # of a dK / dV row cut across its query heads), both dQ orders: within
    # the bar of the oracle and of the unsplit result, each bit-reproducible
    T = 9 * blk + 23
    w = WL.Workload("parts", "bf16", 1, 6, 2, T, T, 128, mask, blk, blk, seed=0,
                    window=2 * blk + 5 if "window" in mask else None,
                    score="alibi")
    doc = WL.doc_ids([T // 3, T // 2, T - T // 3 - T // 2]) if mask == "document" else None
    q, k, v, do = _inputs(w, 61)
    ref = oracle_bwd(w, q, k, v, do, doc)
    base = gpu_fwd_bwd(w, q, k, v, do, doc, splits=1)
    scale = [max(1.0, float(np.abs(x).max())) for x in ref]
    for ns in (2, 5, 16, 64):
        for order in (True, False):
            print(f"[bwd split parts] {mask} blk={blk} splits={ns} descending={order}",
                  flush=True)
            a = gpu_fwd_bwd(w, q, k, v, do, doc, splits=ns, order=order)
            b = gpu_fwd_bwd(w, q, k, v, do, doc, splits=ns, order=order)
            for x, y in zip(a, b):
                assert torch.equal(x, y)
            for name, g, r, g0, sc in zip(("dQ", "dK", "dV"), a, ref, base, scale):
                assert_grad_close(g, r, f"{name} {mask} splits={ns}")
                assert (g.float() - g0.float()).abs().max().item() <= TOL_BWD * sc


def test_backward_errors():
    bm = fa.create_block_mask("causal", None, None, 256, 256, device=DEV,
                              BLOCK_SIZE=(128, 32))
    q = torch.randn(1, 1, 256, 128, device=DEV).to(torch.bfloat16)
    lse = torch.zeros(1, 1, 256, device=DEV)
    with pytest.raises(fa.FlexAttnError, match="UNSUPPORTED"):
        fa.flex_attention_backward(q, q, q, q, lse, q, bm)
    bm = fa.create_block_mask("causal", None, None, 256, 256, device=DEV,
                              BLOCK_SIZE=128)
    with pytest.raises(ValueError):
        fa.flex_attention_backward(q.float(), q.float(), q.float(), q.float(),
                                   lse, q.float(), bm)


@pytest.fixture(scope="module")
def workload_inputs():
    cache = {}

    def get(name):
        if name not in cache:
            cache.clear()
            w = WL.get(name)
            q, k, v, doc = WL.make_inputs(w)
            rng = np.random.default_rng(w.seed + 100)
            do = torch.from_numpy(
                rng.standard_normal(q.shape, dtype=np.float32)).to(torch.bfloat16)
            cache[name] = (w, q, k, v, do, doc)
        return cache[name]
    return get


@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c5"])
def test_workload_backward(name, workload_inputs):
    # full size: dQ on sampled rows and dK / dV of the last 64 keys (every
    # row allowed to see them is among the last 64 rows under causal,
    # window and document masks) against the oracle, which evaluates only
    # those rows; then identities of the exact gradient over all keys, per
    # key head (summed over its query heads):
    #   sum_j dV_j = sum over rows with keys of dO_i  (rows of P sum to 1)
    #   sum_j dK_j = 0 for score_mods with derivative 1 (none, ALiBi),
    #   since every row of dS sums to 0
    w, q, k, v, do, doc = workload_inputs(name)
    assert w.q_len == w.kv_len
    ns = None if name == "c2" else 1     # c2: the automatic split count
    print(f"[bwd workload] {name} splits={ns}", flush=True)
    dq, dk, dv = gpu_fwd_bwd(w, q, k, v, do, doc, splits=ns)
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and \
        torch.isfinite(dv).all()
    L = w.q_len
    tail = np.arange(L - 64, L)
    rows = np.union1d(sample_rows(L, w.block_m, doc, n_random=16, seed=w.seed),
                      tail)
    dq_ref, dk_ref, dv_ref = oracle_bwd(w, q, k, v, do, doc, rows=rows)
    idx = torch.from_numpy(rows).to(DEV)
    e = assert_grad_close(dq.index_select(2, idx), dq_ref, f"dQ {name}")
    cols = torch.from_numpy(tail).to(DEV)
    ek = assert_grad_close(dk.index_select(2, cols), dk_ref[:, :, tail], f"dK {name}")
    ev = assert_grad_close(dv.index_select(2, cols), dv_ref[:, :, tail], f"dV {name}")
    print(f"[bwd workload] {name}: max err / scale dQ {e:.3g} dK {ek:.3g} "
          f"dV {ev:.3g}", flush=True)

    group = w.H // w.H_kv
    # every row of these workloads has at least one key (causal, window and
    # document masks all allow the diagonal)
    dsum = do.to(DEV).double().sum(dim=2)                      # [B, H, D]
    dsum = dsum.view(w.B, w.H_kv, group, w.D).sum(dim=2)       # [B, H_kv, D]
    dv_sum = dv.double().sum(dim=2)
    # relative to the sums' own magnitude: bf16 P and output rounding add
    # random errors of about 2^-9 / sqrt(L) of it; 1e-3 also holds a
    # missing or doubled key block (128 of L terms) in view
    mag = dv.double().abs().sum(dim=2) + do.to(DEV).double().abs().sum(dim=2).view(
        w.B, w.H_kv, group, w.D).sum(dim=2)
    rel = ((dv_sum - dsum).abs() / mag).max().item()
    print(f"[bwd workload] {name}: |sum dV - sum dO| / magnitude = {rel:.3g}",
          flush=True)
    assert rel <= 1e-3
    if w.score in ("none", "alibi"):
        krel = (dk.double().sum(dim=2).abs() / dk.double().abs().sum(dim=2)).max().item()
        print(f"[bwd workload] {name}: |sum dK| / sum |dK| = {krel:.3g}", flush=True)
        assert krel <= 1e-2


def test_workload_backward_middle_key_block(workload_inputs):
    # c3 at full size (sliding window W): the keys of one key block in the
    # middle of the sequence are seen by rows [j0, j0 + 128 + W - 1) only, so
    # the oracle over those rows gives their dK and dV exactly. Unlike the
    # last keys, this block is reached after many stages of the dK / dV
    # kernel's visit sequence and through both of its LDS buffers.
    w, q, k, v, do, doc = workload_inputs("c3")
    assert w.mask == "sliding_window" and w.block_n == 128
    print("[bwd workload] c3 middle key block", flush=True)
    dq, dk, dv = gpu_fwd_bwd(w, q, k, v, do, doc, splits=1)
    j0 = 32 * w.block_n
    keys = np.arange(j0, j0 + w.block_n)
    rows = np.arange(j0, min(j0 + w.block_n + w.window - 1, w.q_len))
    _, dk_ref, dv_ref = oracle_bwd(w, q, k, v, do, doc, rows=rows)
    cols = torch.from_numpy(keys).to(DEV)
    ek = assert_grad_close(dk.index_select(2, cols), dk_ref[:, :, keys], "dK c3 middle block")
    ev = assert_grad_close(dv.index_select(2, cols), dv_ref[:, :, keys], "dV c3 middle block")
    print(f"[bwd workload] c3 middle key block: max err / scale dK {ek:.3g} dV {ev:.3g}",
          flush=True)


@pytest.mark.parametrize("mask,score", [("causal", "none"), ("sliding_window", "alibi"),
                                        ("document", "softcap")])
def test_backward_caller_lists(mask, score):
    # BlockMask.from_kv_blocks lists (oracle-built, all-partial no-skip,
    # out-of-range entries with counts above NKVB): the backward's transposed
    # lists are built from them and the gradients match the oracle, unsplit
    # and in parts
    blk = 128
    ql = kl = 3 * blk + 45
    w = WL.Workload("small", "bf16", 2, 4, 2, ql, kl, 128, mask, blk, blk,
                    seed=0, window=blk + 9 if mask == "sliding_window" else None,
                    score=score, softcap=5.0 if score == "softcap" else None)
    rng = np.random.default_rng(zlib.crc32(f"bwdlists{mask}{score}".encode()))
    doc = (np.sort(rng.integers(0, 4, ql)).astype(np.int32)
           if mask == "document" else None)
    q, k, v, do = _inputs(w, 73)
    ref = oracle_bwd(w, q, k, v, do, doc)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV) if a is not None else None
    for kind in ("oracle", "no_skip", "clamped"):
        num, idx, fnum, fidx = caller_lists(kind, mask, ql, kl, blk, blk,
                                            window=w.window, doc_id=doc)
        bm = fa.BlockMask.from_kv_blocks(t(num), t(idx), t(fnum), t(fidx),
                                         mask_mod=mask, q_len=ql, kv_len=kl,
                                         BLOCK_SIZE=blk, window=w.window,
                                         doc_id=_doc_t(doc))
        for ns in (1, 3):
            print(f"[bwd caller lists] {mask} {score} {kind} splits={ns}", flush=True)
            got = gpu_fwd_bwd(w, q, k, v, do, doc, bm=bm, splits=ns)
            for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
                assert_grad_close(g, r, f"{name} caller lists {kind} {mask} {score} "
                                        f"splits={ns}")
