"""GPU parity of fa_create_block_mask: bit-exact against the oracle on every
array, tails included, for the five workloads and random small cases."""
import numpy as np
import pytest
import torch

import block_sparse_masked_fa_amd as fa
import workloads as WL
from oracle import oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def gpu_mask(kind, B, H, ql, kl, bm_, bn_, window=None, doc=None, sep=True):
    doc_t = (torch.from_numpy(np.ascontiguousarray(doc, np.int32)).to(DEV)
             if doc is not None else None)
    m = fa.create_block_mask(kind, B, H, ql, kl, device=DEV,
                             BLOCK_SIZE=(bm_, bn_), separate_full_blocks=sep,
                             window=window, doc_id=doc_t)
    torch.cuda.synchronize()
    out = {"kv_num_blocks": m.kv_num_blocks.cpu().numpy(),
           "kv_indices": m.kv_indices.cpu().numpy()}
    if sep:
        out["full_kv_num_blocks"] = m.full_kv_num_blocks.cpu().numpy()
        out["full_kv_indices"] = m.full_kv_indices.cpu().numpy()
    return out


def assert_same(got, want, label):
    for key, arr in got.items():
        ref = want[key]
        assert arr.dtype == np.int32 and arr.shape == ref.shape, (label, key)
        if not np.array_equal(arr, ref):
            bad = np.argwhere(arr != ref)[:5]
            raise AssertionError(f"{label} {key} differs at {bad.tolist()}")


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_block_mask_workloads_bit_exact(name):
    w = WL.get(name)
    doc = None
    if w.mask == "document":
        rng = np.random.default_rng(w.seed)
        doc = WL.doc_ids(WL.doc_lengths(rng, w.kv_len, w.n_docs,
                                        w.min_doc_len))
    print(f"[block mask] {name}", flush=True)
    got = gpu_mask(w.mask, 1, 1, w.q_len, w.kv_len, w.block_m, w.block_n,
                   w.window, doc)
    want = O.create_block_mask(w.mask, 1, 1, w.q_len, w.kv_len, w.block_m,
                               w.block_n, window=w.window, doc_id=doc)
    assert_same(got, want, name)


def test_block_mask_known_counts():
    # the hand counts of the oracle pins, now from the GPU builder
    got = gpu_mask("sliding_window", 1, 1, 8192, 8192, 128, 128, window=1024)
    assert got["kv_num_blocks"].sum() == 120
    assert got["full_kv_num_blocks"].sum() == 420
    got = gpu_mask("causal", 1, 1, 16384, 16384, 128, 128)
    assert got["kv_num_blocks"].sum() == 128
    assert got["full_kv_num_blocks"].sum() == 8128


@pytest.mark.parametrize("seed", range(6))
def test_block_mask_random_small(seed):
    rng = np.random.default_rng(1000 + seed)
    for _ in range(8):
        ql = int(rng.integers(1, 700))
        kl = int(rng.integers(1, 700))
        bm_ = int(rng.choice([1, 3, 16, 32, 64, 100, 128]))
        bn_ = int(rng.choice([1, 5, 16, 32, 64, 128, 200]))
        if -(-kl // bn_) > 4096:
            continue
        kind = str(rng.choice(O.MASK_KINDS))
        W = int(rng.integers(1, 300))
        L = max(ql, kl)
        doc = np.sort(rng.integers(0, 6, size=L)).astype(np.int32)
        sep = bool(rng.integers(0, 2))
        B, H = (int(x) for x in rng.choice([1, 2, 3], size=2))
        label = f"{kind} ql={ql} kl={kl} bm={bm_} bn={bn_} W={W} sep={sep}"
        print(f"[block mask] {label}", flush=True)
        got = gpu_mask(kind, B, H, ql, kl, bm_, bn_, W, doc, sep)
        want = O.create_block_mask(kind, B, H, ql, kl, bm_, bn_, window=W,
                                   doc_id=doc, separate_full_blocks=sep)
        assert_same(got, want, label)


def test_block_mask_unsorted_document_ids():
    # document ids need not be sorted or contiguous: ids drawn per key, runs
    # of ids in shuffled order (several distinct ids per key block, ids that
    # recur after others), and blocks wider than 128 keys, ragged tails
    rng = np.random.default_rng(7)
    doc = rng.integers(0, 3, size=500).astype(np.int32)
    got = gpu_mask("document", 1, 1, 500, 500, 32, 32, doc=doc)
    want = O.create_block_mask("document", 1, 1, 500, 500, 32, 32,
                               doc_id=doc)
    assert_same(got, want, "unsorted docs")
    for t in range(12):
        ql, kl = int(rng.integers(100, 1500)), int(rng.integers(100, 1500))
        bm_ = int(rng.choice([32, 64, 128, 256]))
        bn_ = int(rng.choice([8, 64, 128, 256]))
        L = max(ql, kl)
        run = int(rng.choice([1, 7, 40, 130]))
        doc = np.repeat(rng.integers(0, 5, -(-L // run)), run)[:L].astype(np.int32)
        label = f"unsorted docs ql={ql} kl={kl} bm={bm_} bn={bn_} run={run}"
        got = gpu_mask("document", 1, 1, ql, kl, bm_, bn_, doc=doc)
        want = O.create_block_mask("document", 1, 1, ql, kl, bm_, bn_, doc_id=doc)
        assert_same(got, want, label)


def test_block_mask_empty_lengths():
    got = gpu_mask("causal", 1, 1, 0, 256, 128, 128)
    assert got["kv_num_blocks"].shape == (1, 1, 0)
    got = gpu_mask("causal", 1, 2, 256, 0, 128, 128)
    assert got["kv_num_blocks"].shape == (1, 2, 2)
    assert (got["kv_num_blocks"] == 0).all()
    assert (got["full_kv_num_blocks"] == 0).all()
    assert got["kv_indices"].shape == (1, 2, 2, 0)


def test_block_mask_reuse_and_stream_order():
    # building twice into fresh buffers on a side stream gives the same bits
    a = gpu_mask("sliding_window", 2, 3, 1000, 1000, 64, 64, window=200)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = gpu_mask("sliding_window", 2, 3, 1000, 1000, 64, 64, window=200)
    for k in a:
        assert np.array_equal(a[k], b[k])


@pytest.mark.parametrize("kind", ["causal", "sliding_window", "document",
                                  "none", "local_window"])
def test_block_mask_maximum_sizes(kind):
    # the largest key-block count a row may have (32768: one key per block)
    # and the largest block size (1024), with ragged tails
    rng = np.random.default_rng(11)
    for ql, kl, bm_, bn_ in ((200, 32768, 128, 1), (3000, 9000, 1024, 1024),
                             (1024, 32768, 1024, 1)):
        doc = (np.sort(rng.integers(0, 5, size=max(ql, kl))).astype(np.int32)
               if kind == "document" else None)
        W = 700 if "window" in kind else None
        label = f"{kind} ql={ql} kl={kl} bm={bm_} bn={bn_}"
        print(f"[block mask max] {label}", flush=True)
        got = gpu_mask(kind, 1, 1, ql, kl, bm_, bn_, W, doc)
        want = O.create_block_mask(kind, 1, 1, ql, kl, bm_, bn_, window=W,
                                   doc_id=doc)
        assert_same(got, want, label)


def test_block_mask_limits_refused():
    # one key block too many, and a block size above 1024, are refused on
    # the host before any launch
    with pytest.raises(fa.FlexAttnError):
        fa.create_block_mask("causal", 1, 1, 64, 32769, device=DEV,
                             BLOCK_SIZE=(64, 1))
    with pytest.raises(fa.FlexAttnError):
        fa.create_block_mask("causal", 1, 1, 2048, 2048, device=DEV,
                             BLOCK_SIZE=2048)


def test_block_mask_per_batch_document_ids():
    # a batch of packed sequences: each entry's own ids, one set of rows per
    # entry, bit-exact against the oracle
    rng = np.random.default_rng(19)
    for ql, kl, bm_, bn_ in ((700, 700, 64, 64), (1000, 600, 128, 32)):
        B, H = 3, 2
        L = max(ql, kl)
        doc = np.stack([np.sort(rng.integers(0, n, L)) for n in (2, 5, 1)]
                       ).astype(np.int32)
        label = f"per-batch docs ql={ql} kl={kl} bm={bm_} bn={bn_}"
        print(f"[block mask] {label}", flush=True)
        got = gpu_mask("document", B, H, ql, kl, bm_, bn_, doc=doc)
        want = O.create_block_mask("document", B, H, ql, kl, bm_, bn_,
                                   doc_id=doc)
        assert_same(got, want, label)
    with pytest.raises(ValueError):
        gpu_mask("document", 1, 1, 700, 700, 64, 64, doc=doc)
