"""GPU parity of fa_flex_attention_fwd against the fp64 oracle, plus the
special cases with exact answers.

Small cases are compared on every row; the five workloads at full size are
compared on a deterministic row sample (every row is computed on the GPU,
the oracle evaluates the sampled rows one by one)."""
import zlib

import numpy as np
import pytest
import torch

import block_sparse_masked_fa_amd as fa
import workloads as WL
from oracle import oracle as O
from tests.helpers import TOL, assert_close, caller_lists, oracle_case, \
    sample_rows, torch_dtype

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _score_arg(score, cap):
    if score == "softcap":
        return ("softcap", cap)
    return None if score == "none" else score


def run_gpu(w: WL.Workload, q, k, v, doc=None, sep=True, score=None,
            cap=None, bm=None, num_splits=1):
    score = w.score if score is None else score
    cap = w.softcap if cap is None else cap
    doc_t = torch.from_numpy(doc).to(DEV) if doc is not None else None
    if bm is None:
        bm = fa.create_block_mask(w.mask, None, None, w.q_len, w.kv_len,
                                  device=DEV, BLOCK_SIZE=w.block_m,
                                  separate_full_blocks=sep, window=w.window,
                                  doc_id=doc_t)
    o, lse = fa.flex_attention(q.to(DEV), k.to(DEV), v.to(DEV), bm,
                               score_mod=_score_arg(score, cap),
                               scale=w.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return o, lse


def _inputs(w, seed):
    rng = np.random.default_rng(seed)
    q, k, v = WL.draw_qkv(rng, w)
    dt = torch_dtype(w.dtype)
    return tuple(torch.from_numpy(x).to(dt) for x in (q, k, v))


SMALL = []
for dtype, D, blk in (("bf16", 128, 128), ("bf16", 64, 128),
                      ("bf16", 128, 64), ("bf16", 64, 64), ("fp32", 64, 64),
                      ("fp32", 128, 128)):
    for mask in ("causal", "sliding_window", "document", "none", "local_window"):
        for score in ("none", "softcap", "alibi"):
            SMALL.append((dtype, D, blk, mask, score))


@pytest.mark.parametrize("dtype,D,blk,mask,score", SMALL)
def test_small_full_rows(dtype, D, blk, mask, score):
    # several tiles plus a ragged tail on both sequence axes, q_len != kv_len,
    # grouped heads
    ql, kl = 3 * blk + 37, 2 * blk + 101
    w = WL.Workload("small", dtype, 2, 4, 2, ql, kl, D, mask, blk, blk,
                    seed=0, window=blk + 13 if "window" in mask else None,
                    score=score, softcap=3.0 if score == "softcap" else None)
    rng = np.random.default_rng(zlib.crc32(f"{dtype}{D}{blk}{mask}{score}".encode()))
    doc = (np.sort(rng.integers(0, 4, max(ql, kl))).astype(np.int32)
           if mask == "document" else None)
    q, k, v = _inputs(w, 17)
    print(f"[fwd small] {dtype} D={D} blk={blk} {mask} {score}", flush=True)
    for sep in (True, False):
        o, lse = run_gpu(w, q, k, v, doc, sep=sep)
        o_ref, l_ref = oracle_case(q, k, v, w, doc)
        assert_close(o, lse, o_ref, l_ref, TOL[dtype],
                     f"{dtype} D={D} blk={blk} {mask} {score} sep={sep}")


SERIES = []
for D, blk in ((128, 128), (64, 128), (128, 64)):
    for mask in ("causal", "document", "none", "sliding_window"):
        SERIES.append((D, blk, mask))


@pytest.mark.parametrize("D,blk,mask", SERIES)
def test_softcap_large_cap(D, blk, mask):
    # soft-cap 50 (the document workload's cap) at a small size: capped
    # scores close to the raw ones on N(0, 1) data, and on the rows of the
    # second query block, scaled by 3, well into the cap's curve; every row
    # against the oracle
    ql, kl = 3 * blk + 37, 3 * blk + 11
    w = WL.Workload("small", "bf16", 2, 4, 2, ql, kl, D, mask, blk, blk,
                    seed=0, window=2 * blk + 13 if "window" in mask else None,
                    score="softcap", softcap=50.0)
    rng = np.random.default_rng(zlib.crc32(f"series{D}{blk}{mask}".encode()))
    doc = (np.sort(rng.integers(0, 3, max(ql, kl))).astype(np.int32)
           if mask == "document" else None)
    q, k, v = _inputs(w, 41)
    q[:, :, blk:2 * blk] = (q[:, :, blk:2 * blk].float() * 3.0).to(q.dtype)
    print(f"[fwd softcap 50] D={D} blk={blk} {mask}", flush=True)
    o_ref, l_ref = oracle_case(q, k, v, w, doc)
    for sep in (True, False):
        o, lse = run_gpu(w, q, k, v, doc, sep=sep)
        assert_close(o, lse, o_ref, l_ref, TOL["bf16"],
                     f"softcap 50 D={D} blk={blk} {mask} sep={sep}")


PAIRS = []
for D in (128, 64):
    for bq, bk in ((128, 64), (64, 128)):
        for mask in ("causal", "sliding_window", "document", "none", "local_window"):
            for score in ("none", "alibi"):
                PAIRS.append((D, bq, bk, mask, score))


@pytest.mark.parametrize("D,bq,bk,mask,score", PAIRS)
def test_small_block_size_pairs(D, bq, bk, mask, score):
    # BLOCK_SIZE as a (q, kv) pair: query blocks and key blocks of different
    # sizes, ragged tails on both axes; every row against the oracle, whole
    # and through split-KV
    ql, kl = 3 * bq + 29, 3 * bk + 77
    w = WL.Workload("small", "bf16", 2, 2, 2, ql, kl, D, mask, bq, bk, seed=0,
                    window=bk + 21 if "window" in mask else None,
                    score=score)
    rng = np.random.default_rng(zlib.crc32(f"pair{D}{bq}{bk}{mask}{score}".encode()))
    doc = (np.sort(rng.integers(0, 3, max(ql, kl))).astype(np.int32)
           if mask == "document" else None)
    q, k, v = _inputs(w, 31)
    o_ref, l_ref = oracle_case(q, k, v, w, doc)
    for ns in (1, 3):
        print(f"[fwd block pair] D={D} ({bq},{bk}) {mask} {score} splits={ns}",
              flush=True)
        doc_t = torch.from_numpy(doc).to(DEV) if doc is not None else None
        bm = fa.create_block_mask(mask, None, None, ql, kl, device=DEV,
                                  BLOCK_SIZE=(bq, bk), window=w.window,
                                  doc_id=doc_t)
        o, lse = run_gpu(w, q, k, v, doc, bm=bm, num_splits=ns)
        assert_close(o, lse, o_ref, l_ref, TOL["bf16"],
                     f"pair ({bq},{bk}) D={D} {mask} {score} split {ns}")


SPLIT_SMALL = []
for D, blk in ((128, 128), (64, 128), (128, 64), (64, 64)):
    for mask in ("causal", "sliding_window", "document", "none", "local_window"):
        for score in ("none", "softcap", "alibi"):
            SPLIT_SMALL.append((D, blk, mask, score))


@pytest.mark.parametrize("D,blk,mask,score", SPLIT_SMALL)
def test_small_split_rows(D, blk, mask, score):
    # split-KV: each row's visit list in several parts (some empty: more
    # parts than key blocks), merged; every row against the oracle
    ql, kl = 3 * blk + 37, 4 * blk + 101
    w = WL.Workload("small", "bf16", 2, 4, 2, ql, kl, D, mask, blk, blk,
                    seed=0, window=blk + 13 if "window" in mask else None,
                    score=score, softcap=3.0 if score == "softcap" else None)
    rng = np.random.default_rng(zlib.crc32(f"split{D}{blk}{mask}{score}".encode()))
    doc = (np.sort(rng.integers(0, 4, max(ql, kl))).astype(np.int32)
           if mask == "document" else None)
    q, k, v = _inputs(w, 23)
    o_ref, l_ref = oracle_case(q, k, v, w, doc)
    for ns in (2, 3, 7):
        print(f"[fwd split small] D={D} blk={blk} {mask} {score} splits={ns}",
              flush=True)
        o, lse = run_gpu(w, q, k, v, doc, sep=ns != 3, num_splits=ns)
        assert_close(o, lse, o_ref, l_ref, TOL["bf16"],
                     f"split {ns} D={D} blk={blk} {mask} {score}")


@pytest.mark.parametrize("dtype,D,blk", [("bf16", 128, 128), ("bf16", 64, 64),
                                         ("fp32", 64, 64)])
def test_per_batch_document_ids(dtype, D, blk):
    # a batch of packed sequences with a different packing per entry
    # (doc_id [B, L]); every row against the oracle, whole and split
    B, H, T = 3, 2, 3 * blk + 45
    w = WL.Workload("small", dtype, B, H, H, T, T, D, "document", blk, blk,
                    seed=0)
    rng = np.random.default_rng(D + blk)
    doc = np.stack([np.sort(rng.integers(0, n, T)) for n in (3, 6, 1)]
                   ).astype(np.int32)
    q, k, v = _inputs(w, 41)
    o_ref, l_ref = oracle_case(q, k, v, w, doc)
    bm = fa.create_block_mask("document", B, None, T, T, device=DEV,
                              BLOCK_SIZE=blk,
                              doc_id=torch.from_numpy(doc).to(DEV))
    for ns in ((1, 4) if dtype == "bf16" else (1,)):
        print(f"[fwd per-batch docs] {dtype} D={D} blk={blk} splits={ns}",
              flush=True)
        o, lse = run_gpu(w, q, k, v, doc, bm=bm, num_splits=ns)
        assert_close(o, lse, o_ref, l_ref, TOL[dtype],
                     f"per-batch docs {dtype} D={D} split {ns}")


@pytest.mark.parametrize("D,bq,bk", [(128, 128, 128), (64, 128, 64),
                                     (128, 64, 128), (64, 64, 64)])
@pytest.mark.parametrize("mask", ["causal", "none", "local_window"])
def test_keys_past_the_sequence_end_are_never_used(D, bq, bk, mask):
    # K and V are views into buffers whose rows after KV_LEN hold NaN: any
    # read of a key past the end (the last key block is ragged, and its
    # later stage lies wholly past the end) would poison the output
    ql, kl = 300, 300 if bk == 128 else 290
    w = WL.Workload("tail", "bf16", 1, 2, 2, ql, kl, D, mask, bq, bk, seed=0,
                    window=70 if mask == "local_window" else None)
    q, k, v = _inputs(w, 53)
    o_ref, l_ref = oracle_case(q, k, v, w, None)
    pad = 512
    kp = torch.full((1, 2, pad, D), float("nan"), dtype=torch.bfloat16)
    vp = torch.full((1, 2, pad, D), float("nan"), dtype=torch.bfloat16)
    kp[:, :, :kl] = k
    vp[:, :, :kl] = v
    kd, vd = kp.to(DEV)[:, :, :kl], vp.to(DEV)[:, :, :kl]
    bm = fa.create_block_mask(mask, None, None, ql, kl, device=DEV,
                              BLOCK_SIZE=(bq, bk), window=w.window)
    for ns in (1, 3):
        print(f"[fwd tail] D={D} ({bq},{bk}) {mask} splits={ns}", flush=True)
        o, lse = fa.flex_attention(q.to(DEV), kd, vd, bm, scale=w.scale,
                                   num_splits=ns)
        torch.cuda.synchronize()
        assert_close(o, lse, o_ref, l_ref, TOL["bf16"],
                     f"tail D={D} ({bq},{bk}) {mask} split {ns}")


def test_split_extremes():
    # the largest part count, and a single key block per row
    w = WL.Workload("small", "bf16", 1, 2, 2, 300, 300, 64, "causal", 128,
                    128, seed=0)
    q, k, v = _inputs(w, 5)
    o_ref, l_ref = oracle_case(q, k, v, w, None)
    for ns in (1, 64):
        print(f"[fwd split extremes] splits={ns}", flush=True)
        o, lse = run_gpu(w, q, k, v, num_splits=ns)
        assert_close(o, lse, o_ref, l_ref, TOL["bf16"], f"split {ns}")
    w = WL.Workload("small", "bf16", 1, 2, 2, 128, 128, 128, "none", 128,
                    128, seed=0)
    q, k, v = _inputs(w, 6)
    o_ref, l_ref = oracle_case(q, k, v, w, None)
    o, lse = run_gpu(w, q, k, v, num_splits=4)
    assert_close(o, lse, o_ref, l_ref, TOL["bf16"], "one block, 4 parts")


@pytest.fixture(scope="module")
def workload_inputs():
    cache = {}

    def get(name):
        if name not in cache:
            cache.clear()
            w = WL.get(name)
            q, k, v, doc = WL.make_inputs(w)
            cache[name] = (w, q, k, v, doc)
        return cache[name]
    return get


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_workload_parity(name, workload_inputs):
    w, q, k, v, doc = workload_inputs(name)
    print(f"[fwd workload] {name}", flush=True)
    o, lse = run_gpu(w, q, k, v, doc)
    if name == "c1":
        rows = None
        o_s, l_s = o, lse
    else:
        rows = sample_rows(w.q_len, w.block_m, doc,
                           n_random=64 if name in ("c2", "c3") else 24,
                           seed=w.seed)
        idx = torch.from_numpy(rows).to(DEV)
        o_s, l_s = o.index_select(2, idx), lse.index_select(2, idx)
    o_ref, l_ref = oracle_case(q, k, v, w, doc, rows=rows)
    e_o, e_l = assert_close(o_s, l_s, o_ref, l_ref, TOL[w.dtype], name)
    print(f"[fwd workload] {name}: max|dO|={e_o:.3g} max|dLSE|={e_l:.3g}",
          flush=True)
    # every row, not only the sampled ones, is finite
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("name,ns", [("c2", None), ("c3", 2), ("c5", 3)])
def test_workload_parity_split(name, ns, workload_inputs):
    # split-KV at full size (None: the binding's automatic choice, 8 parts
    # for c2 on 256 compute units), on the sampled rows
    w, q, k, v, doc = workload_inputs(name)
    if ns is None:
        ns = fa.auto_num_splits(torch.bfloat16, w.B, w.H, w.q_len // w.block_m,
                                torch.cuda.get_device_properties(0)
                                .multi_processor_count)
        assert ns > 1
    print(f"[fwd workload split] {name} splits={ns}", flush=True)
    o, lse = run_gpu(w, q, k, v, doc, num_splits=ns)
    rows = sample_rows(w.q_len, w.block_m, doc, n_random=24, seed=w.seed)
    idx = torch.from_numpy(rows).to(DEV)
    o_ref, l_ref = oracle_case(q, k, v, w, doc, rows=rows)
    assert_close(o.index_select(2, idx), lse.index_select(2, idx), o_ref,
                 l_ref, TOL[w.dtype], f"{name} split {ns}")
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    # and every row agrees with the unsplit kernel
    o1, l1 = run_gpu(w, q, k, v, doc, num_splits=1)
    assert (o.float() - o1.float()).abs().max().item() <= TOL["bf16"]
    assert (lse - l1).abs().max().item() <= TOL["bf16"]


def test_separate_full_blocks_agree_at_full_size(workload_inputs):
    w, q, k, v, doc = workload_inputs("c3")
    o1, l1 = run_gpu(w, q, k, v, doc, sep=True)
    o2, l2 = run_gpu(w, q, k, v, doc, sep=False)
    assert (o1.float() - o2.float()).abs().max().item() <= TOL["bf16"]
    assert (l1 - l2).abs().max().item() <= TOL["bf16"]


@pytest.mark.parametrize("dtype,D,blk", [("bf16", 128, 128), ("bf16", 64, 64),
                                         ("fp32", 64, 64)])
@pytest.mark.parametrize("score", ["none", "softcap", "alibi"])
def test_window_one_copies_values(dtype, D, blk, score):
    # W = 1: every query sees only itself, so O_i = v_i exactly and
    # LSE_i = score_mod(scale * q_i . k_i)
    w = WL.Workload("w1", dtype, 1, 2, 2, 2 * blk + 5, 2 * blk + 5, D,
                    "sliding_window", blk, blk, seed=0, window=1, score=score,
                    softcap=2.0)
    q, k, v = _inputs(w, 3)
    o, lse = run_gpu(w, q, k, v)
    assert torch.equal(o.cpu(), v), "O must equal V bit for bit"
    _, l_ref = oracle_case(q, k, v, w)
    assert np.abs(lse.cpu().double().numpy() - l_ref).max() <= TOL[dtype]


@pytest.mark.parametrize("mask", ["causal", "sliding_window", "document",
                                  "local_window"])
def test_uniform_keys_give_log_counts(mask):
    # K = 0, no score_mod: LSE_i = ln(number of allowed keys)
    w = WL.Workload("k0", "bf16", 1, 2, 2, 600, 600, 128, mask, 128, 128,
                    seed=0, window=150 if "window" in mask else None)
    q, k, v = _inputs(w, 4)
    k = torch.zeros_like(k)
    doc = np.repeat(np.arange(3, dtype=np.int32), [100, 333, 167]) \
        if mask == "document" else None
    o, lse = run_gpu(w, q, k, v, doc)
    allowed = O.dense_mask(mask, 600, 600, window=w.window, doc_id=doc)
    n = allowed.sum(axis=1)
    got = lse.cpu().double().numpy()
    assert np.abs(got - np.log(n)[None, None]).max() < 1e-5
    vo = torch.ones_like(v)
    o1, _ = run_gpu(w, q, k, vo, doc)
    assert (o1.float() - 1).abs().max().item() <= 2 ** -7


def test_masked_positions_do_not_change_outputs():
    # changing keys/values a query may not see leaves its output bit-identical
    w = WL.Workload("inv", "bf16", 1, 2, 2, 512, 512, 128, "sliding_window",
                    128, 128, seed=0, window=100)
    q, k, v = _inputs(w, 5)
    o, lse = run_gpu(w, q, k, v)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, :50] += 7.0
    v2[:, :, :50] -= 3.0
    o2, l2 = run_gpu(w, q, k2, v2)
    # rows >= 149 cannot see keys 0..49
    assert torch.equal(o[:, :, 149:], o2[:, :, 149:])
    assert torch.equal(lse[:, :, 149:], l2[:, :, 149:])
    assert not torch.equal(o[:, :, :149], o2[:, :, :149])


def test_rows_without_keys():
    # q_len > kv_len with a sliding window: rows i >= kv_len + W - 1 have no
    # allowed key, giving O = 0 and LSE = -inf
    for dtype, blk in (("bf16", 128), ("fp32", 64)):
        w = WL.Workload("empty", dtype, 1, 1, 1, 400, 150, 64,
                        "sliding_window", blk, blk, seed=0, window=60)
        q, k, v = _inputs(w, 6)
        o, lse = run_gpu(w, q, k, v)
        o_ref, l_ref = oracle_case(q, k, v, w)
        assert np.isneginf(l_ref[0, 0, 209:]).all()
        assert_close(o, lse, o_ref, l_ref, TOL[dtype], f"empty rows {dtype}")
        assert (o[0, 0, 209:] == 0).all()


def test_zero_length_keys():
    w = WL.Workload("nokeys", "bf16", 1, 2, 2, 130, 0, 128, "causal", 128,
                    128, seed=0)
    q = torch.randn(1, 2, 130, 128).to(torch.bfloat16)
    k = torch.zeros(1, 2, 0, 128, dtype=torch.bfloat16)
    o, lse = run_gpu(w, q, k, k)
    assert (o == 0).all() and torch.isneginf(lse).all()


def test_repeated_runs_bit_identical(workload_inputs):
    w, q, k, v, doc = workload_inputs("c3")
    o1, l1 = run_gpu(w, q, k, v, doc)
    for _ in range(3):
        o2, l2 = run_gpu(w, q, k, v, doc)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_noncontiguous_views():
    # q/k/v as (B, S, H, D) memory viewed as (B, H, S, D): strides are honoured
    w = WL.Workload("view", "bf16", 2, 4, 4, 300, 300, 64, "causal", 64, 64,
                    seed=0, score="alibi")
    base = torch.randn(3, 2, 300, 4, 64).to(torch.bfloat16)
    q, k, v = (base[i].transpose(1, 2) for i in range(3))
    bm = fa.create_block_mask("causal", None, None, 300, 300, device=DEV,
                              BLOCK_SIZE=64)
    o, lse = fa.flex_attention(q.contiguous().to(DEV), k.contiguous().to(DEV),
                               v.contiguous().to(DEV), bm, score_mod="alibi")
    dq = base.to(DEV)
    o2, l2 = fa.flex_attention(*(dq[i].transpose(1, 2) for i in range(3)), bm,
                               score_mod="alibi")
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_case(q, k, v, w)
    assert_close(o, lse, o_ref, l_ref, TOL["bf16"], "contiguous copy")
    assert_close(o2, l2, o_ref, l_ref, TOL["bf16"], "strided view")


def test_errors_surface_as_exceptions():
    bm = fa.create_block_mask("causal", None, None, 256, 256, device=DEV,
                              BLOCK_SIZE=128)
    q = torch.randn(1, 1, 128, 128, device=DEV).to(torch.bfloat16)
    with pytest.raises(fa.FlexAttnError, match="SHAPE_MISMATCH"):
        fa.flex_attention(q, q, q, bm)
    q = torch.randn(1, 1, 256, 96, device=DEV).to(torch.bfloat16)
    with pytest.raises(fa.FlexAttnError, match="UNSUPPORTED"):
        fa.flex_attention(q, q, q, bm)


@pytest.mark.parametrize("blk", [128, 64])
@pytest.mark.parametrize("mask,score", [("causal", "alibi"),
                                        ("sliding_window", "none"),
                                        ("document", "softcap")])
def test_caller_lists(blk, mask, score):
    # BlockMask.from_kv_blocks (the tensorplay create_block_mask page's route
    # for precomputed metadata), unsplit and split: lists from the oracle's
    # create_block_mask, every block listed as partial (the no-skip mode
    # bench.py times), and lists with out-of-range entries and counts above
    # NKVB (skipped and clamped). Each gives the plain attention.
    ql = kl = 3 * blk + 45
    w = WL.Workload("small", "bf16", 2, 4, 2, ql, kl, 128, mask, blk, blk,
                    seed=0, window=blk + 9 if mask == "sliding_window" else None,
                    score=score, softcap=5.0 if score == "softcap" else None)
    rng = np.random.default_rng(zlib.crc32(f"lists{blk}{mask}{score}".encode()))
    doc = (np.sort(rng.integers(0, 4, ql)).astype(np.int32)
           if mask == "document" else None)
    q, k, v = _inputs(w, 71)
    o_ref, l_ref = oracle_case(q, k, v, w, doc)
    doc_t = torch.from_numpy(doc).to(DEV) if doc is not None else None
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV) if a is not None else None
    for kind in ("oracle", "no_skip", "clamped"):
        num, idx, fnum, fidx = caller_lists(kind, mask, ql, kl, blk, blk,
                                            window=w.window, doc_id=doc)
        bm = fa.BlockMask.from_kv_blocks(t(num), t(idx), t(fnum), t(fidx),
                                         mask_mod=mask, q_len=ql, kv_len=kl,
                                         BLOCK_SIZE=blk, window=w.window,
                                         doc_id=doc_t)
        for ns in (1, 3):
            print(f"[fwd caller lists] blk={blk} {mask} {score} {kind} splits={ns}",
                  flush=True)
            o, lse = run_gpu(w, q, k, v, doc, bm=bm, num_splits=ns)
            assert_close(o, lse, o_ref, l_ref, TOL["bf16"],
                         f"caller lists {kind} blk={blk} {mask} {score} split {ns}")


def test_caller_lists_are_checked():
    # shapes, dtype, and the uniqueness / disjointness rule are refused on
    # the host before any launch
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)
    num, idx, fnum, fidx = caller_lists("oracle", "causal", 300, 300, 128, 128)
    kw = dict(mask_mod="causal", q_len=300, kv_len=300, BLOCK_SIZE=128)
    fa.BlockMask.from_kv_blocks(t(num), t(idx), t(fnum), t(fidx), **kw)
    with pytest.raises(ValueError):
        fa.BlockMask.from_kv_blocks(t(num[0]), t(idx[0]), **kw)
    with pytest.raises(ValueError):
        fa.BlockMask.from_kv_blocks(t(num), t(idx[..., :2]), **kw)
    with pytest.raises(ValueError):
        fa.BlockMask.from_kv_blocks(t(num), t(idx), t(fnum), None, **kw)
    dup = idx.copy()
    dup[0, 0, 2, 1] = dup[0, 0, 2, 0]
    n2 = num.copy()
    n2[0, 0, 2] = 2
    with pytest.raises(ValueError):
        fa.BlockMask.from_kv_blocks(t(n2), t(dup), **kw)
    both = fidx.copy()  # row 1: partial {1}, full {0} -> full {1}
    both[0, 0, 1, 0] = idx[0, 0, 1, 0]
    with pytest.raises(ValueError):
        fa.BlockMask.from_kv_blocks(t(num), t(idx), t(fnum), t(both), **kw)
    # out = / lse = of the wrong shape or dtype
    w = WL.Workload("small", "bf16", 1, 2, 2, 300, 300, 64, "causal", 128, 128, seed=0)
    q, k, v = (x.to(DEV) for x in _inputs(w, 1))
    bm = fa.create_block_mask("causal", None, None, 300, 300, device=DEV)
    with pytest.raises(ValueError):
        fa.flex_attention(q, k, v, bm, out=torch.empty(1, 2, 299, 64, dtype=torch.bfloat16,
                                                       device=DEV))
    with pytest.raises(ValueError):
        fa.flex_attention(q, k, v, bm, lse=torch.empty(1, 2, 300, device=DEV,
                                                       dtype=torch.float64))


@pytest.mark.parametrize("cap", [3.0, 50.0, 55.0, 56.0, 300.0])
@pytest.mark.parametrize("mask", ["causal", "document"])
def test_softcap_reference_range(cap, mask):
    # Caps up to 55.45 (cap log2 e <= 80) run the stages against a constant
    # reference set from the cap; larger caps track the row maximum. Both
    # sides of that limit, with the scores pushed to both ends of the cap:
    # every key gets a shared component u, the second query block points
    # along +u (scores near +cap) and the third along -u (every score of
    # those rows near -cap, the smallest weights the constant reference
    # produces); whole and through split-KV, every row against the oracle.
    blk = 128
    ql = kl = 4 * blk + 19
    w = WL.Workload("small", "bf16", 1, 4, 2, ql, kl, 128, mask, blk, blk,
                    seed=0, score="softcap", softcap=cap)
    rng = np.random.default_rng(zlib.crc32(f"capref{cap}{mask}".encode()))
    doc = (np.sort(rng.integers(0, 2, kl)).astype(np.int32)
           if mask == "document" else None)
    q, k, v = WL.draw_qkv(rng, w)
    u = rng.standard_normal(128).astype(np.float32)
    k = k + 2.0 * u
    big = 4.0 * cap / 50.0
    q[:, :, blk:2 * blk] = q[:, :, blk:2 * blk] * 0.25 + big * u
    q[:, :, 2 * blk:3 * blk] = q[:, :, 2 * blk:3 * blk] * 0.25 - big * u
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v))
    o_ref, l_ref = oracle_case(q, k, v, w, doc)
    for ns in (1, 3):
        print(f"[fwd softcap reference] cap={cap} {mask} splits={ns}", flush=True)
        o, lse = run_gpu(w, q, k, v, doc, num_splits=ns)
        assert_close(o, lse, o_ref, l_ref, TOL["bf16"],
                     f"softcap {cap} {mask} splits={ns}")


@pytest.mark.parametrize("jump", [12.0, 40.0, 100.0, 400.0])
@pytest.mark.parametrize("score", ["none", "alibi"])
def test_reference_jumps(score, jump):
    # Without a soft-cap, a row's stages after its first are formed against
    # the reference the row already has and only their sums are checked:
    # here the keys of the first key block (visited last by every later
    # query block) score about `jump` log2 units above all other keys, so
    # that last stage's weights come out near 2^jump against the reference:
    # kept as they are (12), rescaled after the product (40), formed again
    # against the row max (100: sums past 2^64; 400: past the fp32 range).
    # Causal and no mask, whole and through split-KV, every row against the
    # oracle.
    blk = 128
    ql = kl = 4 * blk + 19
    for mask in ("causal", "none"):
        w = WL.Workload("small", "bf16", 1, 4, 2, ql, kl, 128, mask, blk, blk,
                        seed=0, score=score)
        rng = np.random.default_rng(zlib.crc32(f"jump{score}{jump}{mask}".encode()))
        q, k, v = WL.draw_qkv(rng, w)
        u = rng.standard_normal(128).astype(np.float32)
        u /= np.linalg.norm(u)
        a = 4.0
        b = jump / (a * w.scale * np.log2(np.e))
        q = q + a * u
        k[:, :, :blk] += b * u
        q, k, v = (torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v))
        o_ref, l_ref = oracle_case(q, k, v, w, None)
        for ns in (1, 3):
            print(f"[fwd reference jump] {score} jump={jump} {mask} splits={ns}",
                  flush=True)
            o, lse = run_gpu(w, q, k, v, None, num_splits=ns)
            assert_close(o, lse, o_ref, l_ref, TOL["bf16"],
                         f"{score} jump={jump} {mask} splits={ns}")


@pytest.mark.parametrize("edge", ["series3", "series", "exact"])
@pytest.mark.parametrize("cap", [50.0, 5.0])
@pytest.mark.parametrize("mask", ["causal", "document"])
def test_softcap_series_edge(mask, cap, edge):
    # Full soft-cap stages whose every |q.k scale / cap| is at most 0.15 take
    # tanh's odd series to y^3, up to 0.25 to y^5; the others the exact form.
    # Here every query points along one direction u and every key along +-u
    # with a length spread of +-20%, so the |y| of a row lie in [0.10, 0.14]
    # (series to y^3), [0.16, 0.24] (to y^5; its cubic term then moves the
    # scores of one row by up to 0.1 of the cap against each other) or
    # [0.26, 0.40] (the exact form). Whole and in 3 parts, every row against
    # the oracle.
    blk = 128
    ql = kl = 3 * blk + 40
    w = WL.Workload("small", "bf16", 1, 2, 2, ql, kl, 128, mask, blk, blk,
                    seed=0, score="softcap", softcap=cap)
    rng = np.random.default_rng(zlib.crc32(f"series{mask}{cap}{edge}".encode()))
    doc = (np.sort(rng.integers(0, 2, kl)).astype(np.int32)
           if mask == "document" else None)
    u = rng.standard_normal(128).astype(np.float32)
    u /= np.linalg.norm(u)
    y0 = {"series3": 0.12, "series": 0.2, "exact": 0.33}[edge]
    alpha = y0 * cap / w.scale
    sign = np.where(rng.random((1, 2, kl, 1)) < 0.5, -1.0, 1.0).astype(np.float32)
    z = rng.uniform(-0.19, 0.19, (1, 2, kl, 1)).astype(np.float32)
    k = sign * (1.0 + z) * u + 0.01 * rng.standard_normal((1, 2, kl, 128)).astype(np.float32)
    q = alpha * u + 0.01 * rng.standard_normal((1, 2, ql, 128)).astype(np.float32)
    v = rng.standard_normal((1, 2, kl, 128)).astype(np.float32)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16) for x in (q, k, v))
    # where the scores lie, from the rounded inputs
    ys = (q.double() @ k.double().transpose(-1, -2)).numpy() * w.scale / cap
    ymax = np.abs(ys).max()
    lim = {"series3": (0.0, 0.15), "series": (0.15, 0.25), "exact": (0.25, 1.0)}[edge]
    assert lim[0] < np.abs(ys).min() and ymax < lim[1], (np.abs(ys).min(), ymax)
    o_ref, l_ref = oracle_case(q, k, v, w, doc)
    for ns in (1, 3):
        print(f"[fwd softcap series] {mask} cap={cap} {edge} |y|max={ymax:.3f} splits={ns}",
              flush=True)
        o, lse = run_gpu(w, q, k, v, doc, num_splits=ns)
        assert_close(o, lse, o_ref, l_ref, TOL["bf16"], f"softcap series {mask} {cap} {edge} ns={ns}")
