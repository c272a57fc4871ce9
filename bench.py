"""Benchmark of the block-sparse masked attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
build the block mask from the mask_mod (fa_create_block_mask) and run the
fused forward (fa_flex_attention_fwd). Inputs are resident in HBM before the
timed region starts. The JSON line reports live-block TFLOP/s:

    sum over (b, h) of live blocks x 4 * BM * BN * D  /  time per step

(partial blocks count their full area), its fraction of the bf16 MFMA peak,
the speedup of the same kernel over a dense causal block mask at the same
shape, the oracle timed on the host cores as a baseline, and (outside the
step) the backward's time and algorithmic rate, and the HBM rates of the
paged decode workload and of the masked-softmax fallback workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c3]
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
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 1) for i in info
                     if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
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
            "cores": int(cores), "kind": "oracle",
            "sample": (f"{n} query rows over the first {used} head(s), dense fp64 "
                       f"numpy, {t:.1f} s measured, scaled by "
                       f"{total_rows}/{n} rows to {t_full:.0f} s")}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c3", choices=sorted(WL.CONFIGS))
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
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB copy kernel (for counter "
                         "calibration under rocprofv3 --pmc)")
    a = ap.parse_args(argv)

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        log("bench.py measures one GPU: the library has no multi-GPU path "
            "(run with --gpus 1).")
        return 2

    import torch
    import block_sparse_masked_fa_amd as fa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WL.get(a.config)
    log(f"[bench] generating inputs for {describe(w)}")
    q, k, v, doc = WL.make_inputs(w)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    doc_t = torch.from_numpy(doc).to(dev) if doc is not None else None
    score = {"none": None, "alibi": "alibi",
             "softcap": ("softcap", w.softcap)}[w.score]
    o = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)

    def build(mask_kind=w.mask):
        return fa.create_block_mask(mask_kind, None, None, w.q_len, w.kv_len,
                                    device=dev, BLOCK_SIZE=w.block_m,
                                    window=w.window, doc_id=doc_t)

    num_splits = a.num_splits
    if num_splits is None:
        num_splits = fa.auto_num_splits(
            qd.dtype, w.B, w.H, -(-w.q_len // w.block_m),
            torch.cuda.get_device_properties(dev).multi_processor_count)

    def fwd(bm):
        fa.flex_attention(qd, kd, vd, bm, score_mod=score, scale=w.scale,
                          out=o, lse=lse, num_splits=num_splits)

    bm = build()
    torch.cuda.synchronize()
    live_bh = live_blocks(bm)                      # per (b, h): broadcast
    flops_per_block = 4 * w.block_m * w.block_n * w.D
    live_flops = live_bh * w.B * w.H * flops_per_block

    for _ in range(a.warmup):
        build()
        fwd(bm)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
          for _ in range(a.steps)]
    log(f"[bench] timing {a.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(a.steps):
        ev[s][0].record(stream)
        bm_s = build()
        ev[s][1].record(stream)
        fwd(bm_s)
        ev[s][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mask_ms = [e[0].elapsed_time(e[1]) for e in ev]
    fwd_ms = [e[1].elapsed_time(e[2]) for e in ev]
    step_ms = ev[0][0].elapsed_time(ev[-1][2]) / a.steps
    fwd_avg = float(np.mean(fwd_ms))
    log(f"[bench] step {step_ms:.4f} ms (wall {wall / a.steps * 1e3:.4f}), "
        f"fwd avg {fwd_avg:.4f} ms min {min(fwd_ms):.4f}, mask avg "
        f"{np.mean(mask_ms):.4f} ms")

    value = live_flops / (step_ms * 1e-3) / 1e12
    achieved = live_flops / (fwd_avg * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS

    # backward of the same attention (not part of the step): one
    # fa_flex_attention_bwd call per repetition, O and LSE from an unsplit
    # forward, a seeded upstream gradient
    bwd = None
    if not a.no_backward and w.dtype == "bf16":
        gen = torch.Generator(device=dev).manual_seed(w.seed)
        dout = torch.randn(qd.shape, generator=gen, device=dev).to(qd.dtype)
        o1, l1 = fa.flex_attention(qd, kd, vd, bm, score_mod=score,
                                   scale=w.scale, num_splits=1)

        bwd_splits = fa.auto_bwd_splits(
            w.B, w.H_kv, bm.num_kv_blocks,
            torch.cuda.get_device_properties(dev).multi_processor_count)

        def bwd_call():
            return fa.flex_attention_backward(qd, kd, vd, o1, l1, dout, bm,
                                              score_mod=score, scale=w.scale,
                                              num_splits=bwd_splits)
        for _ in range(2):
            bwd_call()
        reps = max(3, min(a.steps, 20))
        b0 = torch.cuda.Event(enable_timing=True)
        b1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        b0.record(stream)
        for _ in range(reps):
            bwd_call()
        b1.record(stream)
        torch.cuda.synchronize()
        bwd_ms = b0.elapsed_time(b1) / reps
        # algorithmic work: five products per live tile (S recomputed, dP,
        # dV, dK, dQ) = 2.5 x the forward's two
        bwd_flops = 2.5 * live_flops
        bwd = {"ms": round(bwd_ms, 5), "reps": reps, "num_splits": bwd_splits,
               "flops_per_call": bwd_flops,
               "tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2),
               "frac_of_peak": round(bwd_flops / (bwd_ms * 1e-3) / 1e12 / peak, 4),
               "ratio_to_fwd": round(bwd_ms / fwd_avg, 3)}
        log(f"[bench] backward {bwd_ms:.4f} ms ({bwd['tflops']} TFLOP/s "
            f"algorithmic)")
        del o1, l1, dout

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
        for _ in range(3):
            dec_call()
        reps = 50
        d0 = torch.cuda.Event(enable_timing=True)
        d1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        d0.record(stream)
        for _ in range(reps):
            dec_call()
        d1.record(stream)
        torch.cuda.synchronize()
        dec_ms = d0.elapsed_time(d1) / reps
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
        for _ in range(3):
            sm_call()
        reps = 20
        t0e = torch.cuda.Event(enable_timing=True)
        t1e = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0e.record(stream)
        for _ in range(reps):
            sm_call()
        t1e.record(stream)
        torch.cuda.synchronize()
        sm_ms = t0e.elapsed_time(t1e) / reps
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

    extra = {}
    if not a.no_reference_masks:
        def time_fwd(bm_x, reps=20):
            for _ in range(3):
                fwd(bm_x)
            s0 = torch.cuda.Event(enable_timing=True)
            s1 = torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            for _ in range(reps):
                fwd(bm_x)
            s1.record(stream)
            torch.cuda.synchronize()
            return s0.elapsed_time(s1) / reps

        bm_c = build("causal")
        torch.cuda.synchronize()
        live_c = live_blocks(bm_c)
        t_c = time_fwd(bm_c)
        t_x = time_fwd(bm)
        # no-skip: every key block listed as partial, mask_mod applied
        nqb, nkvb = bm.num_q_blocks, bm.num_kv_blocks
        allnum = torch.full((1, 1, nqb), nkvb, dtype=torch.int32, device=dev)
        allidx = torch.arange(nkvb, dtype=torch.int32, device=dev).repeat(
            1, 1, nqb, 1).contiguous()
        bm_ns = fa.BlockMask.from_kv_blocks(
            allnum, allidx, mask_mod=bm.mask, q_len=w.q_len, kv_len=w.kv_len,
            BLOCK_SIZE=w.block_m)
        t_ns = time_fwd(bm_ns, reps=5)
        fl_c = live_c * w.B * w.H * flops_per_block
        extra = {
            "fwd_ms_config": round(t_x, 5),
            "fwd_ms_dense_causal": round(t_c, 5),
            "speedup_vs_dense_causal": round(t_c / t_x, 3),
            "ideal_speedup_vs_dense_causal": round(live_c / live_bh, 3),
            "dense_causal_tflops": round(fl_c / (t_c * 1e-3) / 1e12, 1),
            "fwd_ms_no_skip": round(t_ns, 5),
            "speedup_vs_no_skip": round(t_ns / t_x, 3),
        }
        log(f"[bench] causal {t_c:.4f} ms, config {t_x:.4f} ms, no-skip "
            f"{t_ns:.4f} ms")

    if a.copy_calibration:
        # an elementwise kernel that reads 256 MiB and writes 256 MiB
        x = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            torch.mul(x, 1.0, out=y)
        torch.cuda.synchronize()

    cpu = None
    if not a.no_cpu_baseline:
        log("[bench] timing the oracle on the host")
        cpu = cpu_baseline(w, q, k, v, doc, live_flops, a.cpu_budget)
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
                   "blocks_per_head": bm.num_q_blocks * bm.num_kv_blocks,
                   "num_splits": num_splits,
                   "parallelism": "single GPU"},
        "frac_of_peak": round(value / peak, 4),
        "fwd_ms": round(fwd_avg, 5),
        "fwd_ms_median": round(float(np.median(fwd_ms)), 5),
        "fwd_ms_min": round(float(np.min(fwd_ms)), 5),
        "exact_work_tflops": round(
            allowed_pairs(w, doc) * w.B * w.H * 4 * w.D / (fwd_avg * 1e-3) / 1e12, 2),
        "mask_build_ms": round(float(np.mean(mask_ms)), 5),
        **extra,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": traffic,
                     "kernel": FWD_KERNEL,
                     "per_launch_flops": live_flops},
        "cpu_baseline": cpu,
        "backward": bwd,
        "decode": dec,
        "masked_softmax": smx,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
