"""GPU parity of fa_masked_softmax against the fp64 oracle: every mask kind,
query offsets (including rows with no allowed key), strided score rows, long
rows and the fallback workload at full size on sampled rows. Masked entries
must be exact zeros; allowed ones within bf16 rounding of the oracle."""
import numpy as np
import pytest
import torch

import block_sparse_masked_fa_amd as fa
import workloads as WL
from oracle import oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def check(p_gpu, scores, mask, q_offset, what, window=None, doc=None):
    got = p_gpu.float().cpu().double().numpy()
    ref = np.stack([O.masked_softmax(scores[b], mask, q_offset=q_offset,
                                     window=window, doc_id=doc)
                    for b in range(scores.shape[0])])
    assert np.isfinite(got).all(), what
    masked = ref == 0
    assert (got[masked] == 0).all(), f"{what}: masked entries not exactly 0"
    # bf16 rounding of the result (2^-9 relative) plus fp32 arithmetic
    err = np.abs(got - ref) - 2.0 ** -8 * ref
    assert err.max() <= 1e-6, f"{what}: max excess error {err.max():.3g}"
    return np.abs(got - ref).max()


CASES = [(m, off) for m in ("causal", "sliding_window", "local_window",
                            "document", "none")
         for off in (0, 5, 300)]


@pytest.mark.parametrize("mask,off", CASES)
def test_small_masked_softmax(mask, off):
    rng = np.random.default_rng(len(mask) * 1000 + off)
    BH, Q, K = 3, 37, 264
    s = torch.from_numpy(rng.standard_normal((BH, Q, K), dtype=np.float32) * 3).to(
        torch.bfloat16)
    window = 50 if "window" in mask else None
    doc = None
    if mask == "document":
        doc = np.sort(rng.integers(0, 5, max(K, Q + off))).astype(np.int32)
    print(f"[masked softmax] {mask} offset={off}", flush=True)
    p = fa.masked_softmax(s.to(DEV), mask, q_offset=off, window=window,
                          doc_id=torch.from_numpy(doc).to(DEV) if doc is not None else None)
    torch.cuda.synchronize()
    check(p, s, mask, off, f"{mask} offset={off}", window, doc)


def test_masked_softmax_strided_rows_and_long_rows():
    # rows padded in memory (a view), and rows long enough to loop
    rng = np.random.default_rng(1)
    base = torch.from_numpy(rng.standard_normal((2, 5, 20000), dtype=np.float32)).to(
        torch.bfloat16)
    s = base[:, :, :16384]
    print("[masked softmax] strided, K=16384", flush=True)
    p = fa.masked_softmax(s.to(DEV)[:, :, :], "sliding_window", q_offset=9000,
                          window=7000)
    sv = base.to(DEV)[:, :, :16384]            # non-contiguous view
    p2 = fa.masked_softmax(sv, "sliding_window", q_offset=9000, window=7000)
    torch.cuda.synchronize()
    check(p, s, "sliding_window", 9000, "K=16384", window=7000)
    assert torch.equal(p, p2)


def test_masked_softmax_fallback_workload_sampled_rows():
    w = WL.SOFTMAX
    s = WL.make_scores(w)
    print(f"[masked softmax] {w.name} {w.q_len}x{w.kv_len} offset {w.q_offset}",
          flush=True)
    p = fa.masked_softmax(s.to(DEV), w.mask, q_offset=w.q_offset)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, w.q_len - 1],
                                     np.random.default_rng(0).integers(0, w.q_len, 24)]))
    for r in rows:
        got = p[0, r:r + 1].unsqueeze(0)
        check(got, s[:, r:r + 1], w.mask, w.q_offset + int(r), f"row {r}")
    # every row sums to one within bf16 rounding
    sums = p.float().sum(dim=-1)
    assert (sums - 1).abs().max().item() < 1e-2


@pytest.mark.parametrize("mask", ["causal", "document", "local_window"])
def test_masked_softmax_rows_longer_than_32k(mask):
    # rows past 32768 keys take the two-pass path
    rng = np.random.default_rng(2)
    K, off = 32768 + 64, 30000
    s = torch.from_numpy(rng.standard_normal((1, 3, K), dtype=np.float32) * 2).to(
        torch.bfloat16)
    doc = (np.sort(rng.integers(0, 3, K)).astype(np.int32)
           if mask == "document" else None)
    window = 3000 if mask == "local_window" else None
    print(f"[masked softmax] K={K} {mask}", flush=True)
    p = fa.masked_softmax(s.to(DEV), mask, q_offset=off, window=window,
                          doc_id=torch.from_numpy(doc).to(DEV) if doc is not None else None)
    torch.cuda.synchronize()
    check(p, s, mask, off, f"K={K} {mask}", window, doc)

