"""GPU parity of the persistent forward schedule (fa_flex_attention_fwd with
a scheduler workspace): resident workgroups take query blocks from counters
instead of one workgroup per block. Each row's arithmetic is the same either
way, so the two launches must agree bit for bit on every row; sampled rows
are also compared with the fp64 oracle. The grids here have more query
blocks than two per compute unit, so the persistent path is the one that
runs."""
import zlib

import numpy as np
import pytest
import torch

import block_sparse_masked_fa_amd as fa
import workloads as WL
from oracle import oracle as O
from tests.helpers import TOL, assert_close, oracle_case, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _cus():
    return torch.cuda.get_device_properties(DEV).multi_processor_count


def _inputs(w, seed):
    rng = np.random.default_rng(seed)
    q, k, v = WL.draw_qkv(rng, w)
    return tuple(torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v))


def _score_arg(w):
    return {"none": None, "alibi": "alibi",
            "softcap": ("softcap", w.softcap)}[w.score]


def _both(w, qd, kd, vd, bm):
    """(O, LSE) from the persistent launch and from one workgroup per query
    block."""
    outs = []
    for persistent in (True, False):
        o, lse = fa.flex_attention(qd, kd, vd, bm, score_mod=_score_arg(w),
                                   scale=w.scale, num_splits=1,
                                   persistent=persistent)
        outs.append((o, lse))
    torch.cuda.synchronize()
    return outs


def _check(w, q, k, v, doc, bm, what):
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    (o_p, l_p), (o_1, l_1) = _both(w, qd, kd, vd, bm)
    assert torch.equal(o_p, o_1), f"{what}: O differs from one workgroup per block"
    assert torch.equal(l_p, l_1), f"{what}: LSE differs from one workgroup per block"
    # every head (ALiBi's slopes depend on the head count), sampled rows
    rows = sample_rows(w.q_len, w.block_m, doc, n_random=24, seed=7)
    o_ref, l_ref = oracle_case(q, k, v, w, doc, rows=rows)
    r = torch.from_numpy(rows).to(DEV)
    assert_close(o_p[:, :, r], l_p[:, :, r], o_ref, l_ref, TOL["bf16"], what)


CASES = []
for mask in ("causal", "sliding_window", "document", "none", "local_window"):
    for score in ("none", "softcap", "alibi"):
        CASES.append((128, 128, 128, mask, score))
for D, bq, bk in ((64, 64, 64), (128, 128, 64), (64, 64, 128), (64, 128, 128)):
    for mask in ("causal", "document", "sliding_window"):
        CASES.append((D, bq, bk, mask, "none"))


@pytest.mark.parametrize("D,bq,bk,mask,score", CASES)
def test_persistent_matches_per_block_launch(D, bq, bk, mask, score):
    # enough query blocks for the persistent grid (more than two per
    # compute unit), ragged tails on both axes, grouped heads
    nqb = -(-2 * _cus() // 32) + 3
    ql = nqb * bq - 37
    kl = ql + 19
    w = WL.Workload("persist", "bf16", 2, 16, 8, ql, kl, D, mask, bq, bk,
                    seed=0, window=3 * bk + 5 if "window" in mask else None,
                    score=score, softcap=4.0 if score == "softcap" else None)
    assert w.B * w.H * -(-ql // bq) > 2 * _cus()
    rng = np.random.default_rng(zlib.crc32(f"persist{D}{bq}{bk}{mask}{score}".encode()))
    doc = (np.sort(rng.integers(0, 5, max(ql, kl))).astype(np.int32)
           if mask == "document" else None)
    q, k, v = _inputs(w, 61)
    print(f"[fwd persistent] D={D} ({bq},{bk}) {mask} {score} q={ql} kv={kl}",
          flush=True)
    bm = fa.create_block_mask(mask, None, None, ql, kl, device=DEV,
                              BLOCK_SIZE=(bq, bk), window=w.window,
                              doc_id=torch.from_numpy(doc).to(DEV) if doc is not None else None)
    _check(w, q, k, v, doc, bm, f"persistent D={D} ({bq},{bk}) {mask} {score}")


def test_workspace_is_zero_again_and_reused():
    # the counters are left zero by every launch: repeated calls on one
    # workspace give identical bits, a smaller launch after a larger one is
    # still complete, and the workspace reads zero after each
    w = WL.Workload("persist", "bf16", 2, 16, 16, 4096, 4096, 128, "causal",
                    128, 128, seed=0, score="alibi")
    q, k, v = _inputs(w, 3)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    bm = fa.create_block_mask("causal", None, None, 4096, 4096, device=DEV)
    ws = fa.fwd_workspace(torch.device(DEV))
    first = None
    for rep in range(5):
        print(f"[fwd persistent reuse] call {rep}", flush=True)
        o, lse = fa.flex_attention(qd, kd, vd, bm, score_mod="alibi", persistent=True)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero().item()) == 0, "counters not cleared"
        if first is None:
            first = (o.clone(), lse.clone())
        else:
            assert torch.equal(o, first[0]) and torch.equal(lse, first[1])
    # a smaller grid (still persistent) on the same workspace
    q2, k2, v2 = qd[:1, :, :3000], kd[:1, :, :3000], vd[:1, :, :3000]
    bm2 = fa.create_block_mask("causal", None, None, 3000, 3000, device=DEV)
    w2 = w.replace(B=1, q_len=3000, kv_len=3000)
    o2, l2 = fa.flex_attention(q2, k2, v2, bm2, score_mod="alibi", persistent=True)
    o2b, l2b = fa.flex_attention(q2, k2, v2, bm2, score_mod="alibi", persistent=False)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero().item()) == 0
    assert torch.equal(o2, o2b) and torch.equal(l2, l2b)
    rows = sample_rows(3000, 128, None, n_random=16, seed=2)
    o_ref, l_ref = oracle_case(q[:1, :, :3000], k[:1, :, :3000], v[:1, :, :3000],
                               w2, None, rows=rows)
    r = torch.from_numpy(rows).to(DEV)
    assert_close(o2[:, :, r], l2[:, :, r], o_ref, l_ref, TOL["bf16"],
                 "smaller grid after a larger one")


def test_rows_without_keys_and_caller_lists():
    # caller lists (BlockMask.from_kv_blocks): rows with no block at all (no
    # stage: O = 0, LSE = -inf), rows whose list holds entries outside
    # [0, NKVB) (skipped) and counts above NKVB (clamped)
    B, H, T, blk = 2, 16, 24 * 128 + 50, 128
    nqb = -(-T // blk)
    assert B * H * nqb > 2 * _cus()
    w = WL.Workload("persist", "bf16", B, H, H, T, T, 128, "causal", blk, blk, seed=0)
    q, k, v = _inputs(w, 9)
    ref = O.create_block_mask("causal", 1, 1, T, T, blk, blk)
    num = ref["kv_num_blocks"].copy()
    idx = ref["kv_indices"].copy()
    fnum = ref["full_kv_num_blocks"].copy()
    fidx = ref["full_kv_indices"].copy()
    # every third query block: no block listed at all
    dead = np.arange(0, nqb, 3)
    num[0, 0, dead] = 0
    fnum[0, 0, dead] = 0
    # every fourth (live) block row: out-of-range entries after its partial
    # blocks and a count above NKVB (the clamped count reads them)
    for m in range(1, nqb, 4):
        if m in dead:
            continue
        c = num[0, 0, m]
        bad = np.array([-1, nqb + 3, 2 ** 30, -(2 ** 31)], dtype=np.int32)
        tail = np.resize(bad, nqb - c)
        idx[0, 0, m, c:] = tail
        num[0, 0, m] = nqb + 5
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    bm = fa.BlockMask.from_kv_blocks(t(num), t(idx), t(fnum), t(fidx),
                                     mask_mod="causal", q_len=T, kv_len=T,
                                     BLOCK_SIZE=blk)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    print("[fwd persistent caller lists]", flush=True)
    (o_p, l_p), (o_1, l_1) = _both(w, qd, kd, vd, bm)
    assert torch.equal(o_p, o_1) and torch.equal(l_p, l_1)
    # the oracle: causal attention, with the rows of dead blocks empty
    rows = np.arange(T)
    o_ref, l_ref = oracle_case(q[:, :1], k[:, :1], v[:, :1], w.replace(B=B, H=1, H_kv=1),
                               None, rows=rows)
    dead_rows = np.concatenate([np.arange(m * blk, min(T, (m + 1) * blk)) for m in dead])
    o_ref[:, :, dead_rows] = 0.0
    l_ref[:, :, dead_rows] = -np.inf
    assert_close(o_p[:, :1], l_p[:, :1], o_ref, l_ref, TOL["bf16"],
                 "caller lists, persistent")
