"""Benchmark of the block-sparse masked attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
build the block mask from the mask_mod (fa_create_block_mask) and run the
fused forward (fa_flex_attention_fwd). Inputs are resident in HBM before the
timed region starts. The JSON line reports live-block TFLOP/s:

    sum over (b, h) of live blocks x 4 * BM * BN * D  /  time per step

(partial blocks count their full area) on the headline workload (default
c4: document-packed 32K with tanh soft-cap, the largest single-GPU
configuration), its fraction of the bf16 MFMA peak, the speedup of the same
kernel over a dense causal block mask at the same shape, the other bf16
workloads (c2, c3, c5) as sub-objects, the oracle timed on the host cores as
a baseline, and (outside the step) the backward's time and algorithmic rate,
and the HBM rates of the paged decode workload and of the masked-softmax
fallback workload, and, as context only, the rate of a plain bf16 GEMM
through torch on the same chip.

Timing protocol: every workload is first run back to back for at least
--warm-ms of GPU time (the clock settles: MI355X lowers it under sustained
load), then K steps are timed with HIP events on the launch stream (one
event pair around the loop for the step rate, one per step for the in-step
forward), then the forward alone R times back to back between two events:
the roofline's `achieved` uses that back-to-back forward time, the figure
rocprofv3's kernel trace averages.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c4]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as WL  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 (published)
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E (published)
FWD_KERNEL = "fwd_bf16_kernel"
KERNEL_SOURCES = ["fwd_common.hpp", "fwd_asm.hpp", "fwd_bf16.hpp", "fwd_bf16_d64.hip",
                  "fwd_bf16_d128.hip", "fwd_fp32.hpp", "fwd_fp32.hip"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "block_sparse_masked_fa_amd", "csrc",
                               name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def live_blocks(bm) -> int:
    n = int(bm.kv_num_blocks.sum().item())
    if bm.full_kv_num_blocks is not None:
        n += int(bm.full_kv_num_blocks.sum().item())
    return n


def allowed_pairs(w: WL.Workload, doc) -> int:
    """Allowed (query, key) pairs of one (b, h), counted from the built-in
    masks' definitions (exact-work diagnostic: 4 D flops per pair)."""
    i = np.arange(w.q_len, dtype=np.int64)
    hi = np.minimum(i + 1, w.kv_len)                  # keys j <= i, j < KV
    if w.mask == "none":
        return int(w.q_len) * int(w.kv_len)
    if w.mask == "causal":
        return int(hi.sum())
    if w.mask == "sliding_window":
        lo = np.maximum(i - w.window + 1, 0)
        return int(np.maximum(hi - lo, 0).sum())
    if w.mask == "local_window":
        lo = np.maximum(i - w.window + 1, 0)
        return int(np.maximum(np.minimum(i + w.window, w.kv_len) - lo, 0).sum())
    # document: keys j <= i with doc[j] == doc[i]
    d = np.asarray(doc)
    total = 0
    for v in np.unique(d[:w.q_len]):
        keys = np.flatnonzero(d[:w.kv_len] == v)
        rows = np.flatnonzero(d[:w.q_len] == v)
        total += int(np.searchsorted(keys, rows, side="right").sum())
    return total


def describe(w: WL.Workload) -> str:
    s = (f"{w.name}: {w.dtype} B={w.B} H={w.H} Q=KV={w.q_len} D={w.D} "
         f"{w.mask}")
    if w.window:
        s += f" W={w.window}"
    if w.n_docs:
        s += f" docs={w.n_docs}"
    if w.score != "none":
        s += f" score_mod={w.score}" + (f"({w.softcap:g})" if w.softcap
                                         else "")
    return s + f" BLOCK={w.block_m}"


def traffic_for(workload: str):
    """HBM bytes per forward launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"fwd_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(w, q, k, v, doc, live_flops, budget_s):
    """Time the fp64 oracle on a bounded sample of query rows of the first
    head and scale to the whole workload."""
    from oracle import oracle as O
    host_cpus = len(os.sched_getaffinity(0))
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        blas = max([i.get("num_threads", 1) for i in info
                    if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        blas = int(os.environ.get("OMP_NUM_THREADS", host_cpus))
    cores = min(blas, host_cpus)  # threads the oracle's matrix products run on
    kw = dict(mask=w.mask, score=w.score, scale=w.scale, window=w.window,
              doc_id=doc, softcap=w.softcap)
    rng = np.random.default_rng(123)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    O.attention(q[:1, :1], k[:1, :1], v[:1, :1], rows=np.arange(8), **kw)
    done, t, used = 0, 0.0, 0
    for b, h in heads:
        if t >= budget_s:
            break
        hk = h // (w.H // w.H_kv)
        q1, k1, v1 = q[b:b + 1, h:h + 1], k[b:b + 1, hk:hk + 1], v[b:b + 1, hk:hk + 1]
        order = rng.permutation(w.q_len)
        used += 1
        for c0 in range(0, w.q_len, 512):
            rows = np.sort(order[c0:c0 + 512])
            t0 = time.perf_counter()
            O.attention(q1, k1, v1, rows=rows, **kw)
            t += time.perf_counter() - t0
            done += len(rows)
            if t >= budget_s:
                break
    n = done
    total_rows = w.B * w.H * w.q_len
    t_full = t / n * total_rows
    return {"value": live_flops / t_full / 1e12, "unit": "TFLOP/s",
            "cores": int(cores), "host_cpus": int(host_cpus),
            "blas_threads": int(blas), "kind": "oracle",
            "sample": (f"{n} query rows over the first {used} head(s), dense fp64 "
                       f"numpy, {t:.1f} s measured, scaled by "
                       f"{total_rows}/{n} rows to {t_full:.0f} s")}


SUB_WORKLOADS = ("c2", "c3", "c5")


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_back_to_back(torch, stream, fn, reps):
    """Average time of fn over reps launches enqueued back to back (ms)."""
    e0, e1 = _events(torch)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def warm_up(torch, stream, fn, min_calls, min_ms):
    """Run fn back to back for at least min_calls calls and min_ms of GPU
    time, so that the clock has settled before anything is timed."""
    done, spent = 0, 0.0
    while done < min_calls or spent < min_ms:
        n = max(1, min_calls if done == 0 else 4)
        spent += time_back_to_back(torch, stream, fn, n) * n
        done += n
    return done


class Case:
    """One workload on the device: inputs, its block mask and the forward."""

    def __init__(self, torch, fa, w, dev, num_splits=None):
        self.w = w
        q, k, v, doc = WL.make_inputs(w)
        self.q_cpu, self.k_cpu, self.v_cpu, self.doc = q, k, v, doc
        self.q, self.k, self.v = (t.to(dev) for t in (q, k, v))
        self.doc_t = torch.from_numpy(doc).to(dev) if doc is not None else None
        self.score = {"none": None, "alibi": "alibi",
                      "softcap": ("softcap", w.softcap)}[w.score]
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:3], dtype=torch.float32, device=dev)
        self.fa, self.torch, self.dev = fa, torch, dev
        if num_splits is None:
            num_splits = fa.auto_num_splits(
                self.q.dtype, w.B, w.H, -(-w.q_len // w.block_m),
                torch.cuda.get_device_properties(dev).multi_processor_count)
        self.num_splits = num_splits
        self.bm = self.build()
        torch.cuda.synchronize()
        self.live_bh = live_blocks(self.bm)
        self.flops_per_block = 4 * w.block_m * w.block_n * w.D
        self.live_flops = self.live_bh * w.B * w.H * self.flops_per_block

    def build(self, mask_kind=None):
        w = self.w
        return self.fa.create_block_mask(mask_kind or w.mask, None, None, w.q_len,
                                         w.kv_len, device=self.dev,
                                         BLOCK_SIZE=w.block_m, window=w.window,
                                         doc_id=self.doc_t)

    def fwd(self, bm=None):
        self.fa.flex_attention(self.q, self.k, self.v, bm or self.bm,
                               score_mod=self.score, scale=self.w.scale,
                               out=self.o, lse=self.lse,
                               num_splits=self.num_splits)

    def step(self):
        self.fwd(self.build())

    def free(self):
        del self.q, self.k, self.v, self.o, self.lse, self.bm
        self.torch.cuda.empty_cache()


def measure(torch, stream, case, steps, warmup, warm_ms, fwd_reps):
    """Step rate (mask build + forward), the in-step forward and the
    back-to-back forward of one workload."""
    warm_up(torch, stream, case.step, warmup, warm_ms)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record(stream)
        bm_s = case.build()
        ev[s][1].record(stream)
        case.fwd(bm_s)
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mask_ms = [e[0].elapsed_time(e[1]) for e in ev]
    fwd_in_step = [e[1].elapsed_time(e[2]) for e in ev]
    step_ms = ev[0][0].elapsed_time(ev[-1][2]) / steps
    fwd_ms = time_back_to_back(torch, stream, case.fwd, fwd_reps)
    return {"step_ms": step_ms, "wall_ms": wall / steps * 1e3,
            "mask_ms": float(np.mean(mask_ms)),
            "fwd_in_step_ms": float(np.mean(fwd_in_step)),
            "fwd_in_step_min_ms": float(np.min(fwd_in_step)),
            "fwd_ms": fwd_ms}


def reference_masks(torch, stream, fa, case, warm_ms, no_skip=True):
    """The same kernel on the dense causal block mask (same shape and
    score_mod) and, optionally, with every block listed as partial."""
    w = case.w
    out = {}
    if w.mask != "causal":
        bm_c = case.build("causal")
        torch.cuda.synchronize()
        live_c = live_blocks(bm_c)
        f = lambda: case.fwd(bm_c)  # noqa: E731
        warm_up(torch, stream, f, 3, warm_ms / 2)
        t_c = time_back_to_back(torch, stream, f, 10)
        t_x = time_back_to_back(torch, stream, case.fwd, 10)
        fl_c = live_c * w.B * w.H * case.flops_per_block
        out.update({
            "fwd_ms_dense_causal": round(t_c, 5),
            "fwd_ms_config": round(t_x, 5),
            "speedup_vs_dense_causal": round(t_c / t_x, 3),
            "ideal_speedup_vs_dense_causal": round(live_c / case.live_bh, 3),
            "dense_causal_tflops": round(fl_c / (t_c * 1e-3) / 1e12, 1)})
    else:
        out.update({"speedup_vs_dense_causal": 1.0,
                    "ideal_speedup_vs_dense_causal": 1.0})
    if no_skip:
        # every key block listed as partial, mask_mod applied
        nqb, nkvb = case.bm.num_q_blocks, case.bm.num_kv_blocks
        allnum = torch.full((1, 1, nqb), nkvb, dtype=torch.int32, device=case.dev)
        allidx = torch.arange(nkvb, dtype=torch.int32, device=case.dev).repeat(
            1, 1, nqb, 1).contiguous()
        bm_ns = fa.BlockMask.from_kv_blocks(
            allnum, allidx, mask_mod=case.bm.mask, q_len=w.q_len,
            kv_len=w.kv_len, BLOCK_SIZE=w.block_m)
        f = lambda: case.fwd(bm_ns)  # noqa: E731
        f()
        t_ns = time_back_to_back(torch, stream, f, 3)
        t_x = out.get("fwd_ms_config") or time_back_to_back(torch, stream, case.fwd, 5)
        out.update({"fwd_ms_no_skip": round(t_ns, 5),
                    "speedup_vs_no_skip": round(t_ns / t_x, 3)})
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warm-ms", type=float, default=400.0,
                    help="GPU time each workload runs before it is timed")
    ap.add_argument("--config", default="c4", choices=sorted(WL.CONFIGS))
    ap.add_argument("--sub", default=",".join(SUB_WORKLOADS),
                    help="comma-separated workloads reported as sub-objects "
                         "('' for none)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--num-splits", type=int, default=None,
                    help="split-KV parts per query block (default: the "
                         "binding's automatic choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-reference-masks", action="store_true",
                    help="skip the dense-causal and no-skip timings")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the timing of the backward (dQ, dK, dV)")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the timing of the paged decode workload")
    ap.add_argument("--no-softmax", action="store_true",
                    help="skip the timing of the masked softmax workload")
    ap.add_argument("--no-gemm-reference", action="store_true",
                    help="skip the timing of a plain bf16 GEMM (context only)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB copy kernel (for counter "
                         "calibration under rocprofv3 --pmc)")
    a = ap.parse_args(argv)

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        log("bench.py measures one GPU: libflexattn has no multi-GPU path; "
            "run with --gpus 1.")
        return 2

    import torch
    import block_sparse_masked_fa_amd as fa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    w = WL.get(a.config)
    log(f"[bench] generating inputs for {describe(w)}")
    case = Case(torch, fa, w, dev, a.num_splits)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    log(f"[bench] timing {a.steps} steps after >= {a.warm_ms:.0f} ms of warm-up")
    m = measure(torch, stream, case, a.steps, a.warmup, a.warm_ms,
                fwd_reps=max(10, a.steps))
    step_ms, fwd_ms = m["step_ms"], m["fwd_ms"]
    value = case.live_flops / (step_ms * 1e-3) / 1e12
    achieved = case.live_flops / (fwd_ms * 1e-3) / 1e12
    log(f"[bench] step {step_ms:.4f} ms (wall {m['wall_ms']:.4f}), forward "
        f"{fwd_ms:.4f} ms back to back, {m['fwd_in_step_ms']:.4f} ms in step, "
        f"mask {m['mask_ms']:.4f} ms")

    extra = {}
    if not a.no_reference_masks:
        extra = reference_masks(torch, stream, fa, case, a.warm_ms)
        log(f"[bench] reference masks: {extra}")

    # backward of the same attention (not part of the step): one
    # fa_flex_attention_bwd call per repetition, O and LSE from an unsplit
    # forward, a seeded upstream gradient
    bwd = None
    if not a.no_backward and w.dtype == "bf16":
        gen = torch.Generator(device=dev).manual_seed(w.seed)
        dout = torch.randn(case.q.shape, generator=gen, device=dev).to(case.q.dtype)
        o1, l1 = fa.flex_attention(case.q, case.k, case.v, case.bm,
                                   score_mod=case.score, scale=w.scale,
                                   num_splits=1)
        bwd_splits = fa.auto_bwd_splits(
            w.B, w.H_kv, case.bm.num_kv_blocks,
            torch.cuda.get_device_properties(dev).multi_processor_count)

        def bwd_call():
            return fa.flex_attention_backward(case.q, case.k, case.v, o1, l1,
                                              dout, case.bm,
                                              score_mod=case.score,
                                              scale=w.scale,
                                              num_splits=bwd_splits)
        warm_up(torch, stream, bwd_call, 2, a.warm_ms / 2)
        reps = max(3, min(a.steps, 20))
        bwd_ms = time_back_to_back(torch, stream, bwd_call, reps)
        # algorithmic work: five products per live tile (S recomputed, dP,
        # dV, dK, dQ) = 2.5 x the forward's two
        bwd_flops = 2.5 * case.live_flops
        bwd = {"ms": round(bwd_ms, 5), "reps": reps, "num_splits": bwd_splits,
               "flops_per_call": bwd_flops,
               "tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2),
               "frac_of_peak": round(bwd_flops / (bwd_ms * 1e-3) / 1e12 / peak, 4),
               "ratio_to_fwd": round(bwd_ms / fwd_ms, 3)}
        log(f"[bench] backward {bwd_ms:.4f} ms ({bwd['tflops']} TFLOP/s "
            f"algorithmic)")
        del o1, l1, dout

    if a.copy_calibration:
        # an elementwise kernel that reads 256 MiB and writes 256 MiB
        x = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            torch.mul(x, 1.0, out=y)
        torch.cuda.synchronize()
        del x, y

    exact = allowed_pairs(w, case.doc) * w.B * w.H * 4 * w.D
    headline = {"live_flops": case.live_flops, "exact_flops": exact}
    q_cpu, k_cpu, v_cpu, doc_np = case.q_cpu, case.k_cpu, case.v_cpu, case.doc
    live_bh = case.live_bh
    blocks_bh = case.bm.num_q_blocks * case.bm.num_kv_blocks
    num_splits = case.num_splits
    case.free()
    del case

    # the other bf16 workloads, each timed with the same protocol
    subs = {}
    for name in [x for x in a.sub.split(",") if x and x != a.config]:
        ws = WL.get(name)
        log(f"[bench] sub-workload {describe(ws)}")
        c = Case(torch, fa, ws, dev)
        ms = measure(torch, stream, c, a.steps, a.warmup, a.warm_ms / 2,
                     fwd_reps=max(10, a.steps))
        sub = {"workload": describe(ws), "num_splits": c.num_splits,
               "live_blocks_per_head": c.live_bh,
               "step_ms": round(ms["step_ms"], 5),
               "step_tflops": round(c.live_flops / (ms["step_ms"] * 1e-3) / 1e12, 2),
               "fwd_ms": round(ms["fwd_ms"], 5),
               "fwd_in_step_ms": round(ms["fwd_in_step_ms"], 5),
               "fwd_tflops": round(c.live_flops / (ms["fwd_ms"] * 1e-3) / 1e12, 2),
               "frac": round(c.live_flops / (ms["fwd_ms"] * 1e-3) / 1e12 / peak, 4),
               "mask_build_ms": round(ms["mask_ms"], 5)}
        if not a.no_reference_masks:
            sub.update(reference_masks(torch, stream, fa, c, a.warm_ms / 2,
                                       no_skip=False))
        log(f"[bench] {name}: {sub}")
        subs[name] = sub
        c.free()
        del c

    # paged decode workload (not part of the step): one
    # fa_flex_attention_decode_paged call per repetition over a seeded
    # paged cache; HBM-bound, rated on the key/value bytes it must read
    dec = None
    if not a.no_decode:
        dw = WL.DECODE
        log(f"[bench] generating the paged decode inputs ({dw.name})")
        dq_, dkp, dvp, dtab, dlens = (t.to(dev) for t in WL.make_paged_inputs(dw))
        dsplits = fa.auto_decode_splits(
            dw.B, dw.H_kv, dtab.shape[1] * dw.page_size,
            torch.cuda.get_device_properties(dev).multi_processor_count)

        def dec_call():
            return fa.flex_attention_decode_paged(dq_, dkp, dvp, dtab, dlens,
                                                  scale=dw.scale,
                                                  num_splits=dsplits)
        warm_up(torch, stream, dec_call, 3, a.warm_ms / 4)
        reps = 50
        dec_ms = time_back_to_back(torch, stream, dec_call, reps)
        tokens = int(dlens.sum().item())
        kv_bytes = tokens * dw.H_kv * dw.D * 2 * 2
        io_bytes = kv_bytes + 2 * dw.B * dw.H * dw.D * 2 + dw.B * dw.H * 4
        dec = {"workload": f"{dw.name}: bf16 B={dw.B} H={dw.H} H_kv={dw.H_kv} "
                           f"D={dw.D} page={dw.page_size} lens {dw.min_len}-"
                           f"{dw.max_len} (total {tokens} tokens), causal",
               "us": round(dec_ms * 1e3, 2), "reps": reps,
               "num_splits": dsplits, "algorithmic_bytes": io_bytes,
               "achieved_GBps": round(io_bytes / (dec_ms * 1e-3) / 1e9, 1),
               "peak_GBps": PEAK_HBM_GBPS,
               "frac": round(io_bytes / (dec_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
        log(f"[bench] decode {dec_ms * 1e3:.1f} us, {dec['achieved_GBps']} GB/s")
        del dq_, dkp, dvp, dtab, dlens

    # masked softmax over materialised scores (the fallback workload; not
    # part of the step), HBM-bound: allowed scores read once, every
    # probability written once
    smx = None
    if not a.no_softmax:
        sw = WL.SOFTMAX
        log(f"[bench] generating the masked-softmax scores ({sw.name})")
        sc = WL.make_scores(sw).to(dev)
        sp = torch.empty_like(sc)

        def sm_call():
            fa.masked_softmax(sc, sw.mask, q_offset=sw.q_offset, out=sp)
        warm_up(torch, stream, sm_call, 3, a.warm_ms / 4)
        reps = 20
        sm_ms = time_back_to_back(torch, stream, sm_call, reps)
        allowed = sum(min(sw.kv_len, sw.q_offset + r + 1) for r in range(sw.q_len))
        sm_bytes = sw.BH * (allowed * 2 + sw.q_len * sw.kv_len * 2)
        smx = {"workload": f"{sw.name}: bf16 scores {sw.BH}x{sw.q_len}x{sw.kv_len}, "
                           f"causal, query offset {sw.q_offset}",
               "us": round(sm_ms * 1e3, 2), "reps": reps,
               "algorithmic_bytes": sm_bytes,
               "achieved_GBps": round(sm_bytes / (sm_ms * 1e-3) / 1e9, 1),
               "peak_GBps": PEAK_HBM_GBPS,
               "frac": round(sm_bytes / (sm_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
        log(f"[bench] masked softmax {sm_ms * 1e3:.1f} us, {smx['achieved_GBps']} GB/s")
        del sc, sp

    # context, not part of the path: a plain bf16 product of two 8192 x 8192
    # matrices through torch (the vendor GEMM library) on the same chip and
    # under the same power limit, the rate an MFMA-bound kernel can expect
    gemm = None
    if not a.no_gemm_reference:
        ga = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
        gb = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
        gf = lambda: torch.matmul(ga, gb)  # noqa: E731
        warm_up(torch, stream, gf, 5, a.warm_ms)
        g_ms = time_back_to_back(torch, stream, gf, 20)
        g_tf = 2 * 8192 ** 3 / (g_ms * 1e-3) / 1e12
        gemm = {"what": "torch.matmul bf16 8192x8192x8192 (vendor library), context only",
                "ms": round(g_ms, 4), "tflops": round(g_tf, 1),
                "frac_of_peak": round(g_tf / PEAK_BF16_TFLOPS, 4),
                "forward_over_gemm": round(achieved / g_tf, 3)}
        log(f"[bench] bf16 GEMM reference {g_tf:.0f} TFLOP/s; forward at "
            f"{achieved / g_tf:.2f} of it")
        del ga, gb

    cpu = None
    if not a.no_cpu_baseline:
        log("[bench] timing the oracle on the host")
        cpu = cpu_baseline(w, q_cpu, k_cpu, v_cpu, doc_np, headline["live_flops"],
                           a.cpu_budget)
        log(f"[bench] oracle {cpu['value']:.3g} TFLOP/s ({cpu['sample']})")

    traffic = traffic_for(w.name)
    line = {
        "metric": "live-block TFLOP/s (fraction of bf16 MFMA peak; speedup "
                  "vs dense causal)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": describe(w), "global_batch": w.B,
                   "seq_len": w.q_len, "heads": w.H, "head_dim": w.D,
                   "block": w.block_m,
                   "live_blocks_per_head": live_bh,
                   "blocks_per_head": blocks_bh,
                   "num_splits": num_splits,
                   "parallelism": "single GPU"},
        "frac_of_peak": round(value / peak, 4),
        "fwd_ms": round(fwd_ms, 5),
        "fwd_in_step_ms": round(m["fwd_in_step_ms"], 5),
        "fwd_in_step_min_ms": round(m["fwd_in_step_min_ms"], 5),
        "exact_work_tflops": round(headline["exact_flops"] / (fwd_ms * 1e-3) / 1e12, 2),
        "mask_build_ms": round(m["mask_ms"], 5),
        "warm_ms": a.warm_ms,
        **extra,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": traffic,
                     "kernel": FWD_KERNEL,
                     "per_launch_flops": headline["live_flops"],
                     "timing": "forward launches back to back, HIP events "
                               "on the launch stream"},
        "workloads": subs,
        "cpu_baseline": cpu,
        "backward": bwd,
        "decode": dec,
        "masked_softmax": smx,
        "gemm_reference": gemm,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
