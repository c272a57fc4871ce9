"""GPU parity of fa_flex_attention_decode_paged against the fp64 oracle's
paged decode step: ragged context lengths (empty, one token, page and
stage boundaries), every mask and score_mod, grouped heads up to 32 per key
head, pages scattered over a pool whose unused rows hold NaN, split into
parts or not, and the decode workload at full size."""
import numpy as np
import pytest
import torch

import block_sparse_masked_fa_amd as fa
import workloads as WL
from oracle import oracle as O
from tests.helpers import TOL

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _score_arg(score, cap):
    if score == "softcap":
        return ("softcap", cap)
    return None if score == "none" else score


def run_decode(w, inputs, num_splits, doc=None):
    q, kp, vp, table, lens = (t.to(DEV) for t in inputs)
    o, lse = fa.flex_attention_decode_paged(
        q, kp, vp, table, lens, mask_mod=w.mask,
        score_mod=_score_arg(w.score, w.softcap), scale=w.scale,
        num_splits=num_splits, window=w.window,
        doc_id=torch.from_numpy(doc).to(DEV) if doc is not None else None)
    torch.cuda.synchronize()
    return o, lse


def oracle_decode(w, inputs, doc=None, seqs=None):
    q, kp, vp, table, lens = inputs
    if seqs is not None:
        idx = torch.from_numpy(np.asarray(seqs))
        q, table, lens = q[idx], table[idx], lens[idx]
        if doc is not None and doc.ndim == 2:
            doc = doc[np.asarray(seqs)]
    return O.decode_paged(q, kp, vp, table.numpy(), lens.numpy(), mask=w.mask,
                          score=w.score, scale=w.scale, window=w.window,
                          doc_id=doc, softcap=w.softcap)


def assert_decode_close(o, lse, o_ref, l_ref, what, seqs=None):
    og = o.float().cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    if seqs is not None:
        og, lg = og[seqs], lg[seqs]
    assert og.shape == o_ref.shape
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(lg), fin), f"{what}: -inf rows differ"
    assert np.isfinite(og).all(), f"{what}: non-finite output"
    err_o = np.abs(og - o_ref).max() if og.size else 0.0
    err_l = np.abs(lg[fin] - l_ref[fin]).max() if fin.any() else 0.0
    assert err_o <= TOL["bf16"], f"{what}: max |O - oracle| = {err_o:.3g}"
    assert err_l <= TOL["bf16"], f"{what}: max |LSE - oracle| = {err_l:.3g}"
    assert (og[~fin] == 0).all()
    return err_o, err_l


# lengths: empty, one token, stage and page edges, several pages
LENS = [0, 1, 63, 64, 65, 127, 128, 129, 300, 1000]

CASES = []
for D in (128, 64):
    for mask in ("causal", "sliding_window", "document", "none", "local_window"):
        for score in ("none", "softcap", "alibi"):
            CASES.append((D, mask, score))


@pytest.mark.parametrize("D,mask,score", CASES)
def test_small_decode(D, mask, score):
    page = 64 if mask in ("causal", "document") else 128
    H, H_kv = (8, 2) if D == 128 else (12, 3)
    w = WL.DecodeWorkload("small", len(LENS), H, H_kv, D, page, 1, 1, seed=11,
                          mask=mask, window=100 if "window" in mask else None,
                          score=score, softcap=4.0 if score == "softcap" else None)
    inputs = WL.make_paged_inputs(w, lens=LENS)
    doc = None
    if mask == "document":
        rng = np.random.default_rng(D)
        doc = np.sort(rng.integers(0, 4, (len(LENS), page * inputs[3].shape[1])),
                      axis=1).astype(np.int32)
    o_ref, l_ref = oracle_decode(w, inputs, doc)
    for ns in (1, 3, None):
        print(f"[decode small] D={D} {mask} {score} splits={ns}", flush=True)
        o, lse = run_decode(w, inputs, ns, doc)
        assert_decode_close(o, lse, o_ref, l_ref, f"D={D} {mask} {score} splits={ns}")


@pytest.mark.parametrize("H,H_kv", [(32, 1), (4, 4), (6, 2)])
def test_decode_head_groups(H, H_kv):
    # 32 query heads on one key head (the MFMA column limit), one query head
    # per key head, and a group of 3
    w = WL.DecodeWorkload("groups", 4, H, H_kv, 128, 128, 1, 1, seed=12,
                          score="alibi")
    inputs = WL.make_paged_inputs(w, lens=[700, 1, 256, 2049])
    o_ref, l_ref = oracle_decode(w, inputs)
    for ns in (1, 5):
        print(f"[decode groups] H={H} H_kv={H_kv} splits={ns}", flush=True)
        o, lse = run_decode(w, inputs, ns)
        assert_decode_close(o, lse, o_ref, l_ref, f"H={H} H_kv={H_kv} splits={ns}")


def test_decode_invalid_page_entries_are_left_out():
    # a page-table entry outside [0, num_pages) drops its tokens: the same
    # as the oracle over the remaining keys (checked against a cache whose
    # dropped rows are masked by a document id)
    w = WL.DecodeWorkload("holes", 2, 4, 2, 128, 64, 1, 1, seed=13)
    q, kp, vp, table, lens = WL.make_paged_inputs(w, lens=[300, 200])
    table = table.clone()
    table[0, 1] = 10 ** 6          # tokens 64..127 of sequence 0
    table[1, 0] = -5               # tokens 0..63 of sequence 1
    o, lse = run_decode(w, (q, kp, vp, table, lens), 1)
    doc = np.zeros((2, 64 * table.shape[1]), dtype=np.int32)
    doc[0, 64:128] = 1
    doc[1, :64] = 1
    wd = WL.DecodeWorkload("holes", 2, 4, 2, 128, 64, 1, 1, seed=13,
                           mask="document")
    good = table.clone()
    good[0, 1] = good[0, 0]        # any readable page: its keys are masked
    good[1, 0] = good[1, 1]
    o_ref, l_ref = oracle_decode(wd, (q, kp, vp, good, lens), doc)
    assert_decode_close(o, lse, o_ref, l_ref, "invalid page entries")


def test_decode_repeatable_and_split_agrees():
    w = WL.DecodeWorkload("rep", 6, 16, 4, 128, 128, 1, 4000, seed=14,
                          score="softcap", softcap=30.0)
    inputs = WL.make_paged_inputs(w)
    o1, l1 = run_decode(w, inputs, 1)
    for _ in range(2):
        o2, l2 = run_decode(w, inputs, 1)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o8, l8 = run_decode(w, inputs, 8)
    assert (o8.float() - o1.float()).abs().max().item() <= TOL["bf16"]
    assert (l8 - l1).abs().max().item() <= TOL["bf16"]


def test_decode_workload_full_size():
    w = WL.DECODE
    inputs = WL.make_paged_inputs(w)
    print(f"[decode workload] B={w.B} H={w.H} H_kv={w.H_kv} total tokens "
          f"{int(inputs[4].sum())}", flush=True)
    o_ref, l_ref = oracle_decode(w, inputs)
    for ns in (None, 1):
        o, lse = run_decode(w, inputs, ns)
        e_o, e_l = assert_decode_close(o, lse, o_ref, l_ref, f"decode_paged splits={ns}")
        print(f"[decode workload] splits={ns}: max|dO|={e_o:.3g} max|dLSE|={e_l:.3g}",
              flush=True)
