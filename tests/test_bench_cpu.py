"""Host-side pieces of bench.py: the JSON contract's refusal of several GPUs,
and the exact-work diagnostic's pair count against the oracle's dense mask."""
import subprocess
import sys
import os

import numpy as np
import pytest

import bench
import workloads as WL
from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("mask,window", [("none", None), ("causal", None),
                                         ("sliding_window", 5),
                                         ("sliding_window", 1),
                                         ("sliding_window", 400),
                                         ("local_window", 1),
                                         ("local_window", 6),
                                         ("local_window", 300),
                                         ("document", None)])
@pytest.mark.parametrize("ql,kl", [(37, 37), (50, 23), (23, 50)])
def test_allowed_pairs_matches_dense_mask(mask, window, ql, kl):
    w = WL.Workload("t", "bf16", 1, 1, 1, ql, kl, 64, mask, 64, 64, seed=0,
                    window=window)
    doc = None
    if mask == "document":
        rng = np.random.default_rng(ql * 100 + kl)
        doc = np.sort(rng.integers(0, 4, max(ql, kl))).astype(np.int32)
    dense = O.dense_mask(mask, ql, kl, window=window, doc_id=doc)
    assert bench.allowed_pairs(w, doc) == int(dense.sum())


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True,
                       cwd=ROOT, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
