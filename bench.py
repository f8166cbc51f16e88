#!/usr/bin/env python3
"""Benchmark of the fused attention path on one MI355X.

One step = one forward (attn_forward) plus one backward over the workload's
synthetic batch, inputs resident in device memory.  The backward is the one
attn_backward runs, in every dtype: the dQ kernel (which recomputes S and dP
from lse and also forms D = rowsum(dO*O)), then the dK/dV kernel (which
recomputes P from lse and reads D); its only scratch is D, B*NH*T floats.
The fp32 dS block store order (the D pre-pass, a dK/dV kernel that also
stores dS, a dQ kernel that reads it; O(T^2) caller-owned memory) is timed
beside it as fp32_ds_store_order.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload 3] [--dtype f32|bf16|f16|f32_rc|f32_ds]

value = useful fwd+bwd TFLOP/s = (4 + 10) * hs * pairs * B * NH / step time,
pairs = T(T+1)/2 for causal (masked pairs are not counted; the backward's
recomputation of the scores is counted, as one of its five contractions).
The step time is that of K steps of the C-ABI calls launched one by one,
each kernel between HIP events recorded on the stream it runs on (torch's
current stream, which the binding hands to libattn).  The same step captured
once in a HIP graph (the stage calls allocate nothing) and replayed K times
is reported beside it (graph_ms_per_step).

Also reported: per-step median and minimum, forward and backward apart
(step_stats), the same with a 512 MB buffer written before every step so
that no input sits in the last-level cache (step_stats.flushed), the
compulsory HBM bytes and their rate (hbm), the flop rate under the
12 * hs * pairs count that leaves out the backward's score recompute,
the peaks recomputed from rocminfo (device_peaks), a plain copy's HBM rate
(hbm_copy), the LayerNorm over the workload's activation rows in GB/s
(layernorm), and the CPU oracle with its forward and backward timed apart,
also on the two small workloads with one thread.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd+bwd causal TFLOP/s and % MFMA peak, B8 T1024 C768 NH12"
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6, "f16": 2516.6, "fp8": 5033.2}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "transformer_causal_head_attn_amd", "csrc")
KERNEL_SOURCE = {"f32": "flash_f32.hip", "f32_ds": "flash_f32.hip", "f32_rc": "flash_f32.hip",
                 "bf16": "flash_half.hip", "f16": "flash_half.hip"}


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5,
                   help="untimed steps per dtype (at least; see --warmup-ms)")
    p.add_argument("--warmup-ms", type=float, default=150.0,
                   help="after the --warmup steps, keep running untimed steps until this much "
                        "time has passed since the first one: the kernels reach their steady "
                        "speed only after ~30 ms (fp32) to ~70 ms (bf16) of work, whatever "
                        "the step count")
    p.add_argument("--workload", type=int, default=3,
                   help="workload key in workloads.py (3: the GPT-2 layer, the headline)")
    p.add_argument("--dtype", choices=["f32", "f32_rc", "f32_ds", "bf16", "f16"], default=None,
                   help="the step's dtype (default: the workload's); f32_rc and f32_ds time the "
                        "fp32 step through the recompute-order or the dS block store stage calls "
                        "instead of attn_backward's")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-budget-s", type=float, default=15.0,
                   help="CPU seconds the oracle baseline may spend on its sample")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the secondary measurements (other dtypes, the other workloads, "
                        "materialised mode, decode)")
    p.add_argument("--no-others", action="store_true",
                   help="skip the other workloads (keep only the chosen workload's shape)")
    p.add_argument("--flush-mb", type=int, default=512,
                   help="size of the buffer written between the steps of the cache-flushed "
                        "timing (0: skip it); the MI355X last-level cache holds 256 MB")
    p.add_argument("--layernorm-only", action="store_true",
                   help="only time the LayerNorm forward and backward over the workload's "
                        "activation rows (fp32 and bf16) and print them as one JSON line")
    p.add_argument("--fp8-only", action="store_true",
                   help="only time the fp8 forward (and the bf16 forward on the same values) on "
                        "the GPT-2, ViT and long-context inputs and print them as one JSON line")
    p.add_argument("--projections-only", action="store_true",
                   help="only time the QKV and output projections over the workload's "
                        "activation rows (fp32 and bf16) and print them as one JSON line")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                   help="only run a plain device-to-device copy of MB megabytes (3 times), "
                        "to calibrate the HBM byte counters of a profiler run")
    return p.parse_args()


def calibrate_copy(torch, mb):
    n = mb * (1 << 20) // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": n * 4, "copy_bytes_written_per_launch": n * 4,
                      "launches": 3}), flush=True)


def device_peaks():
    """Peaks recomputed from the device: compute units x maximum engine
    clock (rocminfo) x matrix-core flops per clock per CU (four SIMDs; a
    v_mfma_f32_16x16x4_f32 is 2048 flops in 32 cycles, a
    v_mfma_f32_16x16x32_bf16 16384 flops in 16 cycles).  Called before the
    process touches the GPU; None if rocminfo is not there."""
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    for blk in txt.split("Agent "):
        if "gfx950" not in blk:
            continue
        cu = re.search(r"Compute Unit:\s+(\d+)", blk)
        mhz = re.search(r"Max Clock Freq\. \(MHz\):\s+(\d+)", blk)
        if not (cu and mhz):
            return None
        cus, clk = int(cu.group(1)), int(mhz.group(1))
        return {"cus": cus, "max_clock_mhz": clk,
                "fp32_mfma_tflops": round(cus * clk * 1e6 * 4 * 64 / 1e12, 1),
                "bf16_mfma_tflops": round(cus * clk * 1e6 * 4 * 1024 / 1e12, 1),
                "fp8_mfma_tflops": round(cus * clk * 1e6 * 4 * 2048 / 1e12, 1),
                "source": "rocminfo: compute units x max engine clock x matrix-core flops "
                          "per clock (fp32 256, bf16/fp16 4096, fp8 8192 per CU)"}
    return None


def hbm_copy(torch, mb=1024, reps=10):
    """Achievable HBM rate: a plain device-to-device copy of mb megabytes
    (read once, written once), averaged over reps copies."""
    n = mb * (1 << 20) // 4
    src = torch.empty(n, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = 2 * n * 4 / (ms * 1e-3) / 1e9
    del src, dst
    return {"bytes_moved_per_copy": 2 * n * 4, "gbs": round(gbs, 1),
            "frac_of_8000_gbs": round(gbs / PEAK_HBM_GBS, 4)}


def compulsory_bytes(w, dtype):
    """Compulsory HBM bytes of one forward and one backward: the forward
    reads qkv once and writes out and lse; the backward reads qkv, out, dout
    and lse, writes and reads D, and writes dqkv."""
    esz = 4 if dtype.startswith("f32") else 2
    io = w.B * w.T * w.C * esz
    rows = 4 * w.B * w.NH * w.T
    return 3 * io + io + rows, 3 * io + 2 * io + rows + 2 * rows + 3 * io


def hbm_report(w, dtype, fwd_ms, bwd_ms):
    fb, bb = compulsory_bytes(w, dtype)
    return {"compulsory_bytes_fwd": fb, "compulsory_bytes_bwd": bb,
            "gbs_fwd": round(fb / (fwd_ms * 1e-3) / 1e9, 1),
            "gbs_bwd": round(bb / (bwd_ms * 1e-3) / 1e9, 1),
            "frac_hbm_peak_step": round((fb + bb) / ((fwd_ms + bwd_ms) * 1e-3) / 1e9
                                        / PEAK_HBM_GBS, 4)}


def kernel_flops(w, dtype):
    """Algorithmic flops of each kernel for one launch: 2*hs per unmasked
    (query, key) pair per contraction it performs."""
    u = 2 * w.hs * w.pairs * w.B * w.NH
    if dtype == "f32":              # attn_backward: pre-pass, then dK, dV and dQ in one kernel
        return {"fwd": 2 * u,       # S = Q K^T, O = P V
                "prepass": 0,       # D = dO.O per row, dQ cleared (HBM-bound)
                "dkdvdq": 5 * u}    # S, dV, dP, dK, dQ = dS K (added with atomics)
    if dtype == "f32_ds":           # the fp32 dS block store order
        return {"fwd": 2 * u,
                "prepass": 0,       # D = dO.O per row (HBM-bound)
                "dkdv": 4 * u,      # S, dV = P^T dO, dP = dO V^T, dK = dS^T Q (+ dS stored)
                "dq": u}            # dQ = dS K from the stored dS
    # the recompute order: the 16-bit attn_backward_* and the fp32 stages
    # attn_backward_dq + attn_backward_dkdv ("f32_rc")
    return {"fwd": 2 * u,
            "dkdv": 4 * u,          # S, dV = P^T dO, dP = dO V^T, dK = dS^T Q
            "dq": 3 * u,            # S, dP, dQ = dS K (plus the D = dO.O row sums)
            "bwd_short": 5 * u}     # one kernel: S, dP, dV, dK, dQ (dS kept in LDS)


def short_backward(w, dtype):
    """Whether the library's fused 16-bit backward runs its one-workgroup-
    per-head kernel for this shape (the rule of tiles::bwd_short_applies in
    csrc/tiles.hpp, checked against this one by tests/test_tiles.py); the
    step then times attn_backward_* as one stage."""
    return dtype in ("bf16", "f16") and w.hs <= 64 and w.T <= 256 and (w.T > 128 or w.hs == 16)


def source_sha(dtype):
    with open(os.path.join(CSRC, KERNEL_SOURCE[dtype]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel, dtype, workload_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this kernel, if its kernel source is unchanged since it was taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{kernel}_{dtype}_workload{workload_key}.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    sha = re.search(r"source_sha256_16:\s*([0-9a-f]+)", txt)
    fetch = re.search(r"fetch_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    write = re.search(r"write_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not (sha and fetch and write) or sha.group(1) != source_sha(dtype):
        return None
    return float(fetch.group(1)) + float(write.group(1))


def warm_up(torch, stages, warmup, warmup_ms):
    """`warmup` untimed steps, then more until `warmup_ms` have passed since
    the first (the clocks and caches settle after tens of milliseconds of
    work, not after a fixed step count).  Returns (steps run, ms)."""
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(max(1, warmup) if n == 0 else 10):
            for _, fn in stages:
                fn()
            n += 1
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3
        if n >= warmup and ms >= warmup_ms:
            return n, ms


def run_gpu(la, torch, w, dtype, steps, warmup, flush_mb=0, warmup_ms=150.0):
    from workloads import workload_inputs
    qkv_c, dout_c = workload_inputs(w, "f32" if dtype.startswith("f32") else dtype)
    qkv, dout = qkv_c.cuda(), dout_c.cuda()
    B, T, C, NH = w.B, w.T, w.C, w.NH
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}.get(dtype, torch.float32)
    out = torch.empty((B, T, C), dtype=tdt, device="cuda")
    lse = torch.empty((B, NH, T), dtype=torch.float32, device="cuda")
    dqkv = torch.empty_like(qkv)
    D = torch.empty((B, NH, T), dtype=torch.float32, device="cuda")
    sfx = "" if dtype.startswith("f32") else "_" + dtype
    fwd = getattr(la, "attn_forward" + sfx)
    dkdv = getattr(la, "attn_backward_dkdv" + sfx)
    dq = getattr(la, "attn_backward_dq" + sfx)
    c = int(w.causal)
    if dtype == "f32_ds":
        # caller-owned dS block store (O(T^2) floats)
        dS = torch.empty((la.attn_backward_ds_bytes(B, T, C, NH, c) // 4,), device="cuda")
        stages = [("fwd", lambda: fwd(out, lse, qkv, B, T, C, NH, c)),
                  ("prepass", lambda: la.attn_backward_preprocess(D, dout, out, B, T, C, NH)),
                  ("dkdv", lambda: la.attn_backward_dkdv_ds(dqkv, dS, dout, qkv, lse, D,
                                                            B, T, C, NH, c)),
                  ("dq", lambda: la.attn_backward_dq_ds(dqkv, dS, qkv, B, T, C, NH, c))]
    elif dtype == "f32":
        # attn_backward's two stages: D and a cleared dQ, then dK, dV, dQ
        stages = [("fwd", lambda: fwd(out, lse, qkv, B, T, C, NH, c)),
                  ("prepass", lambda: la.attn_backward_prepare(dqkv, D, dout, out, B, T, C, NH)),
                  ("dkdvdq", lambda: la.attn_backward_dkdvdq(dqkv, dout, qkv, lse, D,
                                                             B, T, C, NH, c))]
    elif short_backward(w, dtype):
        bwd = getattr(la, "attn_backward" + sfx)
        stages = [("fwd", lambda: fwd(out, lse, qkv, B, T, C, NH, c)),
                  ("bwd_short", lambda: bwd(dqkv, dout, qkv, out, lse, B, T, C, NH, c))]
    else:
        stages = [("fwd", lambda: fwd(out, lse, qkv, B, T, C, NH, c)),
                  ("dq", lambda: dq(dqkv, D, dout, qkv, out, lse, B, T, C, NH, c)),
                  ("dkdv", lambda: dkdv(dqkv, dout, qkv, lse, D, B, T, C, NH, c))]

    warm_steps, warm_ms = warm_up(torch, stages, warmup, warmup_ms)

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(steps)]
    t0 = time.perf_counter()
    for k in range(steps):
        ev[k][0].record()
        for i, (_, fn) in enumerate(stages):
            fn()
            ev[k][i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_kernel = {}
    for i, (name, _) in enumerate(stages):
        per_kernel[name] = sum(ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(steps)) / steps
    eager_ms = ev[0][0].elapsed_time(ev[-1][-1]) / steps
    step_t = [ev[k][0].elapsed_time(ev[k][-1]) for k in range(steps)]
    fwd_t = [ev[k][0].elapsed_time(ev[k][1]) for k in range(steps)]
    bwd_t = [ev[k][1].elapsed_time(ev[k][-1]) for k in range(steps)]
    stats = {"step_ms_median": round(statistics.median(step_t), 5),
             "step_ms_min": round(min(step_t), 5),
             "fwd_ms_median": round(statistics.median(fwd_t), 5),
             "fwd_ms_min": round(min(fwd_t), 5),
             "bwd_ms_median": round(statistics.median(bwd_t), 5),
             "bwd_ms_min": round(min(bwd_t), 5)}

    if flush_mb:
        # Each step preceded by a write of flush_mb megabytes (a fill kernel
        # on the same stream), so no input is left in the last-level cache
        # (256 MB) when the step starts; only the step is between the events.
        buf = torch.empty(flush_mb << 20, dtype=torch.uint8, device="cuda")
        fe = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for k in range(steps):
            buf.fill_(k & 0x7F)
            fe[k][0].record()
            for i, (_, fn) in enumerate(stages):
                fn()
                if i == 0:
                    fe[k][1].record()
            fe[k][2].record()
        torch.cuda.synchronize()
        del buf
        stats["flushed"] = {
            "flush_mb": flush_mb,
            "step_ms_median": round(statistics.median(
                [fe[k][0].elapsed_time(fe[k][2]) for k in range(steps)]), 5),
            "fwd_ms_median": round(statistics.median(
                [fe[k][0].elapsed_time(fe[k][1]) for k in range(steps)]), 5),
            "bwd_ms_median": round(statistics.median(
                [fe[k][1].elapsed_time(fe[k][2]) for k in range(steps)]), 5)}

    # The same step captured once in a HIP graph (the stage calls allocate
    # nothing) and replayed K times: the kernels then follow each other
    # without host launch gaps.  The per-kernel times above stay eager.
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _, fn in stages:
            fn()
    for _ in range(20):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1) / steps
    stats["warmup_steps_run"] = warm_steps
    stats["warmup_ms"] = round(warm_ms, 1)
    return eager_ms, graph_ms, wall * 1e3 / steps, per_kernel, stats


def run_materialized(la, torch, w, steps, warmup):
    """Time the materialised fp32 forward and backward (whole calls) and
    report them against their compulsory traffic: every T x T matrix the
    mode produces is written once and every one it consumes is read once."""
    from workloads import workload_inputs
    qkv_c, dout_c = workload_inputs(w, "f32")
    qkv, dout = qkv_c.cuda(), dout_c.cuda()
    B, T, C, NH, c = w.B, w.T, w.C, w.NH, int(w.causal)
    out = torch.empty((B, T, C), device="cuda")
    pre = torch.empty((B, NH, T, T), device="cuda")
    att = torch.empty_like(pre)
    datt = torch.empty_like(pre)
    dpre = torch.empty_like(pre)
    dqkv = torch.empty_like(qkv)
    fwd = lambda: la.attn_forward_materialized(out, pre, att, qkv, B, T, C, NH, c)
    bwd = lambda: la.attn_backward_materialized(dqkv, dpre, datt, dout, qkv, att, B, T, C, NH, c)
    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    tf = tb = 0.0
    for _ in range(steps):
        e[0].record()
        fwd()
        e[1].record()
        bwd()
        e[2].record()
        torch.cuda.synchronize()
        tf += e[0].elapsed_time(e[1])
        tb += e[1].elapsed_time(e[2])
    tf, tb = tf / steps, tb / steps
    M = B * NH * T * T * 4
    io = B * T * C * 4
    fwd_bytes = 3 * io + 2 * M + io          # qkv in; preatt, att, out out
    bwd_bytes = io + 3 * io + M + 2 * M + 3 * io   # dout, qkv, att in; datt, dpreatt, dqkv out
    return {"workload": f"{w.name} {w.label()}", "fwd_ms": round(tf, 4), "bwd_ms": round(tb, 4),
            "fwd_gbs": round(fwd_bytes / (tf * 1e-3) / 1e9, 1),
            "bwd_gbs": round(bwd_bytes / (tb * 1e-3) / 1e9, 1),
            "bytes_note": "compulsory bytes: each T x T matrix written or read once, "
                          "packed tensors once"}


def run_decode(la, torch, w, dtype, steps, warmup):
    """Time attn_decode (last query row against all T keys, key ranges
    merged) on the workload's inputs.  It is HBM-bound: the compulsory bytes
    are every key and value row of every head read once, plus the query row
    and the output."""
    from workloads import workload_inputs
    qkv_c, _ = workload_inputs(w, dtype)
    qkv = qkv_c.cuda()
    B, T, C, NH = w.B, w.T, w.C, w.NH
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}.get(dtype, torch.float32)
    out = torch.empty((B, C), dtype=tdt, device="cuda")
    lse = torch.empty((B, NH), device="cuda")
    fn = {"bf16": la.attn_decode_bf16, "f16": la.attn_decode_f16}.get(dtype, la.attn_decode)
    call = lambda: fn(out, lse, qkv, B, T, C, NH)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    esz = 4 if dtype == "f32" else 2
    nbytes = (2 * B * T * C + 2 * B * C) * esz + B * NH * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"decode over {w.name} {w.label()}", "dtype": dtype,
            "us": round(ms * 1e3, 2), "gbs": round(gbs, 1),
            "frac_hbm_peak": round(gbs / 8000.0, 4),
            "bytes_note": "compulsory bytes: K and V of every head once, q row and out"}


def _time_call(torch, fn, steps, warmup_ms):
    """Average ms of `fn` over `steps` calls between HIP events on the current
    stream, after untimed calls for `warmup_ms`."""
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < warmup_ms:
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def run_splitkv(la, torch, steps=20, warmup_ms=100.0):
    """The split-KV forward and the split backward against the plain ones
    (bf16) on one GPU's share of the long-context workload under an 8-way
    head split (2 heads of T = 8192, hs = 128: 128 query tiles for the plain
    forward grid) and on the whole workload (16 heads).  Useful flops: 4 (fwd)
    and 10 (bwd) * hs * pairs * B * NH."""
    from workloads import WORKLOADS, workload_inputs
    w = WORKLOADS[5]
    qkv_full, dout_full = workload_inputs(w, "bf16")
    res = []
    for nh in (2, w.NH):
        C = nh * w.hs
        qkv = torch.cat([qkv_full[:, :, p * w.C:p * w.C + C] for p in range(3)], dim=2).contiguous().cuda()
        dout = dout_full[:, :, :C].contiguous().cuda()
        out = torch.empty((w.B, w.T, C), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((w.B, nh, w.T), device="cuda")
        dqkv = torch.empty_like(qkv)
        ffl = 4 * w.hs * w.pairs * w.B * nh
        bfl = 10 * w.hs * w.pairs * w.B * nh
        auto = la.attn_forward_splitkv_chunk(w.B, w.T, C, nh, 1)
        rec = {"workload": f"long-context B{w.B} T{w.T} NH{nh} hs{w.hs} causal bf16",
               "auto_chunk": auto}

        def put(name, f_ms, b_ms):
            rec[name] = {"fwd_us": round(f_ms * 1e3, 2), "bwd_us": round(b_ms * 1e3, 2),
                         "fwd_frac_mfma_peak": round(ffl / (f_ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], 4),
                         "bwd_frac_mfma_peak": round(bfl / (b_ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], 4),
                         "step_tflops": round((ffl + bfl) / ((f_ms + b_ms) * 1e-3) / 1e12, 1)}

        la.attn_forward_bf16(out, lse, qkv, w.B, w.T, C, nh, 1)
        f_ms = _time_call(torch, lambda: la.attn_forward_bf16(out, lse, qkv, w.B, w.T, C, nh, 1),
                          steps, warmup_ms)
        b_ms = _time_call(torch, lambda: la.attn_backward_bf16(dqkv, dout, qkv, out, lse, w.B, w.T,
                                                                C, nh, 1), steps, warmup_ms)
        put("plain", f_ms, b_ms)
        for chunk in sorted({auto, 1024, 2048, 4096}):
            if chunk >= w.T:
                continue
            nf = la.attn_forward_splitkv_bytes(w.B, w.T, C, nh, 1, chunk) // 4
            nb = la.attn_backward_splitkv_bytes(w.B, w.T, C, nh, 1, chunk) // 4
            wf = torch.empty((max(nf, 4),), device="cuda")
            wb = torch.empty((max(nb, 4),), device="cuda")
            f_ms = _time_call(torch, lambda: la.attn_forward_splitkv_bf16(
                out, lse, qkv, wf, w.B, w.T, C, nh, 1, chunk), steps, warmup_ms)
            b_ms = _time_call(torch, lambda: la.attn_backward_splitkv_bf16(
                dqkv, dout, qkv, out, lse, wb, w.B, w.T, C, nh, 1, chunk), steps, warmup_ms)
            put(f"chunk{chunk}", f_ms, b_ms)
            del wf, wb
        res.append(rec)
    return res


def run_fp8_forward(la, torch, keys=(3, 4, 5), steps=20, warmup_ms=100.0):
    """The fp8 forward (E4M3 q, k, v; bf16 out) on the inputs of workloads
    `keys` rounded to E4M3, in TFLOP/s of the forward's useful 4*hs*P*B*NH
    flops against the fp8 matrix-core peak, beside the bf16 forward on the
    same (E4M3-valued) inputs."""
    from workloads import WORKLOADS, workload_inputs
    res = []
    for key in keys:
        w = WORKLOADS[key]
        q8 = workload_inputs(w, "fp8")[0].cuda()
        qb = q8.to(torch.bfloat16)
        B, T, C, NH, c = w.B, w.T, w.C, w.NH, int(w.causal)
        out = torch.empty((B, T, C), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, NH, T), dtype=torch.float32, device="cuda")
        ms8 = _time_call(torch, lambda: la.attn_forward_fp8(out, lse, q8, B, T, C, NH, c), steps, warmup_ms)
        msb = _time_call(torch, lambda: la.attn_forward_bf16(out, lse, qb, B, T, C, NH, c), steps, warmup_ms)
        tf8 = w.flops_fwd / (ms8 * 1e-3) / 1e12
        res.append({"workload": f"{w.name} {w.label().rsplit(' ', 1)[0]} fp8", "fp8_us": round(ms8 * 1e3, 2),
                    "tflops": round(tf8, 1), "frac_fp8_mfma_peak": round(tf8 / PEAK_TFLOPS["fp8"], 4),
                    "bf16_forward_us": round(msb * 1e3, 2)})
    return res


def run_projections(la, torch, M, C, steps=20, warmup_ms=100.0):
    """The QKV projection (M x C times C x 3C, + bias) and the output
    projection (M x C times C x C, + bias + residual) at the workload's
    activation rows, fp32 and bf16, in TFLOP/s of 2*M*K*N flops against the
    matrix-core peak of the dtype."""
    from workloads import randn
    res = []
    for dtype in ("f32", "bf16"):
        tdt = torch.float32 if dtype == "f32" else torch.bfloat16
        for name, N, resid in (("qkv_projection", 3 * C, False), ("out_projection", C, True)):
            x = randn((M, C), 41, 1.0, dtype).cuda()
            w = randn((N, C), 42, 0.02, dtype).cuda()
            b = randn((N,), 43, 0.02, "f32").cuda()
            y = torch.empty((M, N), dtype=tdt, device="cuda")
            if resid:
                r = randn((M, N), 44, 1.0, dtype).cuda()
                fn = {"f32": la.attn_out_projection, "bf16": la.attn_out_projection_bf16}[dtype]
                call = lambda fn=fn, x=x, w=w, b=b, r=r, y=y, N=N: fn(y, x, w, b, r, M, C, N)
            else:
                fn = {"f32": la.attn_qkv_projection, "bf16": la.attn_qkv_projection_bf16}[dtype]
                call = lambda fn=fn, x=x, w=w, b=b, y=y, N=N: fn(y, x, w, b, M, C, N)
            ms = _time_call(torch, call, steps, warmup_ms)
            tf = 2.0 * M * C * N / (ms * 1e-3) / 1e12
            res.append({"op": name, "dtype": dtype, "M": M, "K": C, "N": N, "us": round(ms * 1e3, 2),
                        "tflops": round(tf, 1), "frac_mfma_peak": round(tf / PEAK_TFLOPS[dtype], 4)})
    return res


def run_layernorm(la, torch, N, C, dtype, steps=50, warmup=100):
    """Time the LayerNorm forward and backward over N rows of C (the GPT-2
    layer's activations when N = B*T = 8192, C = 768).  Both are HBM-bound:
    the compulsory bytes are the rows read and written once (forward: inp
    in, out out; backward: dout and inp in, dinp out), plus the per-row
    mean and rstd and the per-column weight, bias and their gradients."""
    from workloads import randn
    esz = 4 if dtype == "f32" else 2
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    x = randn((N, C), 31).to(tdt).cuda()
    dy = randn((N, C), 32).to(tdt).cuda()
    wt = (1.0 + 0.5 * randn((C,), 33)).cuda()
    bs = randn((C,), 34).cuda()
    out, mean, rstd = la.layernorm(x, wt, bs)
    dx = torch.empty_like(x)
    dw = torch.empty(C, device="cuda")
    db = torch.empty(C, device="cuda")
    ffn = la.layernorm_forward if dtype == "f32" else la.layernorm_forward_bf16
    bfn = la.layernorm_backward if dtype == "f32" else la.layernorm_backward_bf16
    fwd = lambda: ffn(out, mean, rstd, x, wt, bs, N, C)
    bwd = lambda: bfn(dx, dw, db, dy, x, wt, mean, rstd, N, C)
    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    for _ in range(steps):
        fwd()
    ev[1].record()
    for _ in range(steps):
        bwd()
    ev[2].record()
    torch.cuda.synchronize()
    tf = ev[0].elapsed_time(ev[1]) / steps
    tb = ev[1].elapsed_time(ev[2]) / steps
    fb = 2 * N * C * esz + 2 * C * 4 + 8 * N
    bb = 3 * N * C * esz + 3 * C * 4 + 8 * N
    return {"workload": f"layernorm N{N} C{C}", "dtype": dtype,
            "fwd_us": round(tf * 1e3, 2), "bwd_us": round(tb * 1e3, 2),
            "fwd_gbs": round(fb / (tf * 1e-3) / 1e9, 1), "bwd_gbs": round(bb / (tb * 1e-3) / 1e9, 1),
            "bytes_note": "compulsory bytes: rows read and written once, per-row mean and rstd, "
                          "per-column weight, bias and gradients"}


def cpu_baseline(w, dtype, budget_s):
    """The fp64 oracle, as it stands, on the first heads of the same
    workload in (b, h) order until the CPU budget is spent.  The inputs are
    widened to float64 and the heads cut out before the clock starts; value
    is the useful flop count of the heads done over the oracle's own
    forward + backward time."""
    import numpy as np
    import oracle
    from workloads import workload_inputs
    qkv, dout = workload_inputs(w, dtype)
    q64 = np.ascontiguousarray(qkv.double().numpy())
    d64 = np.ascontiguousarray(dout.double().numpy())
    heads = [(b, h) for b in range(w.B) for h in range(w.NH)]
    done = 0
    tf = tb = 0.0
    for b, h in heads:
        qs = oracle.head_slice(q64, b, h, w.NH, packed=True)
        ds = oracle.head_slice(d64, b, h, w.NH, packed=False)
        t1 = time.perf_counter()
        oracle.forward(qs, 1, w.causal)
        t2 = time.perf_counter()
        oracle.backward(qs, ds, 1, w.causal)
        tf += t2 - t1
        tb += time.perf_counter() - t2
        done += 1
        if tf + tb >= budget_s:
            break
    flops = 14 * w.hs * w.pairs * done
    return {"value": flops / (tf + tb) / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"{done} of {len(heads)} heads (first in (b,h) order) of the same workload, "
                      f"fp64 forward+backward, {tf + tb:.2f} s of oracle time",
            "fwd_s": round(tf, 3), "bwd_s": round(tb, 3),
            "host": host_description(),
            "small_configs": oracle_small_configs()}


def host_description():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)),
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


def oracle_small_configs():
    """The oracle on the whole of the two small workloads (tiny B1 T64 C64
    NH4 and small B4 T256 C256 NH4, fp32 inputs), forward and backward timed
    apart, with all threads and with one."""
    import oracle
    from workloads import WORKLOADS, workload_inputs
    nmax = oracle.max_threads()
    res = []
    try:
        for key in (1, 2):
            wo = WORKLOADS[key]
            qkv, dout = workload_inputs(wo, "f32")
            for n in (nmax, 1):
                oracle.set_threads(n)
                t0 = time.perf_counter()
                oracle.forward(qkv, wo.NH, wo.causal)
                t1 = time.perf_counter()
                oracle.backward(qkv, dout, wo.NH, wo.causal)
                t2 = time.perf_counter()
                res.append({"workload": f"{wo.name} {wo.label()}", "threads": n,
                            "fwd_ms": round((t1 - t0) * 1e3, 3),
                            "bwd_ms": round((t2 - t1) * 1e3, 3)})
    finally:
        oracle.set_threads(nmax)
    return res


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU mode).", file=sys.stderr)
        sys.exit(2)
    peaks = (device_peaks() if not (args.calibrate_copy or args.layernorm_only or args.fp8_only
                                    or args.projections_only) else None)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(torch, args.calibrate_copy)
        return
    import transformer_causal_head_attn_amd as la
    from workloads import WORKLOADS

    la.load()
    w = WORKLOADS[args.workload]
    if args.layernorm_only:
        print(json.dumps({"layernorm": [run_layernorm(la, torch, w.B * w.T, w.C, "f32"),
                                        run_layernorm(la, torch, w.B * w.T, w.C, "bf16")]}),
              flush=True)
        return
    if args.fp8_only:
        print(json.dumps({"fp8_forward": run_fp8_forward(la, torch, steps=args.steps)}), flush=True)
        return
    if args.projections_only:
        print(json.dumps({"projections": run_projections(la, torch, w.B * w.T, w.C, steps=args.steps)}),
              flush=True)
        return
    dtype = args.dtype or w.dtype
    total_ms, graph_ms, wall_ms, per_kernel, stats = run_gpu(la, torch, w, dtype, args.steps,
                                                             args.warmup, args.flush_mb,
                                                             args.warmup_ms)
    flops = w.flops_fwd + w.flops_bwd
    value = flops / (total_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dtype.split("_")[0]]

    kf = kernel_flops(w, dtype)
    kernels = {}
    for name, ms in per_kernel.items():
        rec = {"ms": round(ms, 5)}
        if kf[name]:
            rec["tflops"] = round(kf[name] / (ms * 1e-3) / 1e12, 2)
            rec["frac_peak"] = round(rec["tflops"] / peak, 4)
        else:   # the D pre-pass: reads out and dout, writes D (and clears dQ in fp32)
            nb = (2 * w.B * w.T * w.C * (4 if dtype.startswith("f32") else 2)
                  + 4 * w.B * w.NH * w.T + (4 * w.B * w.T * w.C if dtype == "f32" else 0))
            rec["gbs"] = round(nb / (ms * 1e-3) / 1e9, 1)
            rec["frac_hbm_peak"] = round(rec["gbs"] / PEAK_HBM_GBS, 4)
        kernels[name] = rec
    dom = max(per_kernel, key=per_kernel.get)
    achieved = kf[dom] / (per_kernel[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": measured_traffic(dom, dtype, w.key),
                "algorithmic_flops_per_launch": kf[dom]}

    metric = METRIC if args.workload == 3 else \
        f"attention fwd+bwd TFLOP/s and % MFMA peak, {w.label()}"
    line = {
        "metric": metric, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "warmup_note": f"{stats['warmup_steps_run']} untimed steps were run: the --warmup "
                       f"count, then more until {args.warmup_ms:g} ms had passed",
        "ms_per_step": round(total_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic (seeded N(0,1) qkv and dout, no dataset)",
        "config": {"workload": f"{w.name} {w.label()}", "B": w.B, "T": w.T, "C": w.C,
                   "NH": w.NH, "hs": w.hs, "causal": w.causal},
        "frac_mfma_peak": round(value / peak, 4),
        "timing": "ms_per_step and kernels: the C-ABI calls launched one by one, each kernel "
                  "between HIP events; graph_ms_per_step: K replays of the step captured in "
                  "one HIP graph",
        "backward": ("attn_backward: pre-pass (D = dO.O, dQ cleared), then one kernel per "
                     "key tile forming dV, dK and adding dQ = scale dS K with float atomics; "
                     "scratch B*NH*T floats" if dtype == "f32" else
                     "dS block store stages: pre-pass D, dK/dV also storing dS, dQ = scale dS K "
                     "from the store; O(T^2) caller-owned floats" if dtype == "f32_ds" else
                     "the recompute order: dQ (recomputes S and dP from lse, forms D), "
                     "then dK/dV (recomputes P, reads D); scratch B*NH*T floats"),
        "graph_ms_per_step": round(graph_ms, 5),
        "graph_tflops": round(flops / (graph_ms * 1e-3) / 1e12, 3),
        "wall_ms_per_step": round(wall_ms, 5),
        "step_stats": stats,
        "tflops_no_recompute_count": round(12 * w.hs * w.pairs * w.B * w.NH
                                           / (total_ms * 1e-3) / 1e12, 3),
        "hbm": hbm_report(w, dtype, stats["fwd_ms_median"], stats["bwd_ms_median"]),
        "kernels": kernels,
        "roofline": roofline,
        "device_peaks": peaks,
    }

    if not args.no_extra and dtype == "f32":
        # the atomic-free recompute order through its stage calls (dQ kernel
        # recomputing S and dP, then dK/dV): bitwise reproducible dq
        r_total, r_graph, _, r_kernels, r_stats = run_gpu(la, torch, w, "f32_rc", args.steps,
                                                          args.warmup, 0, args.warmup_ms)
        r_val = flops / (r_total * 1e-3) / 1e12
        rkf = kernel_flops(w, "f32_rc")
        line["fp32_recompute_order"] = {
            "order": "dQ (recomputes S and dP, forms D), then dK/dV; no atomics",
            "ms_per_step": round(r_total, 5), "tflops": round(r_val, 3),
            "frac_mfma_peak": round(r_val / PEAK_TFLOPS["f32"], 4),
            "graph_ms_per_step": round(r_graph, 5), "step_stats": r_stats,
            "kernels": {k: {"ms": round(v, 5),
                            "frac_peak": round(rkf[k] / (v * 1e-3) / 1e12 / PEAK_TFLOPS["f32"], 4)}
                        for k, v in r_kernels.items()}}
    if not args.no_extra and dtype == "f32":
        # the fp32 dS block store order through the stage calls, with a
        # caller-owned store of O(T^2) floats
        d_total, d_graph, _, d_kernels, d_stats = run_gpu(la, torch, w, "f32_ds", args.steps,
                                                          args.warmup, 0, args.warmup_ms)
        d_val = flops / (d_total * 1e-3) / 1e12
        dkf = kernel_flops(w, "f32_ds")
        line["fp32_ds_store_order"] = {
            "order": "pre-pass D, dK/dV also storing dS, dQ = scale dS K from the store",
            "ds_store_bytes": la.attn_backward_ds_bytes(w.B, w.T, w.C, w.NH, int(w.causal)),
            "ms_per_step": round(d_total, 5), "tflops": round(d_val, 3),
            "frac_mfma_peak": round(d_val / PEAK_TFLOPS["f32"], 4),
            "graph_ms_per_step": round(d_graph, 5), "step_stats": d_stats,
            "kernels": {k: ({"ms": round(v, 5),
                             "frac_peak": round(dkf[k] / (v * 1e-3) / 1e12 / PEAK_TFLOPS["f32"], 4)}
                            if dkf[k] else {"ms": round(v, 5)})
                        for k, v in d_kernels.items()}}

    if not args.no_extra:
        for other in ("f32", "bf16", "f16"):
            if other == dtype:
                continue
            o_total, o_graph, _, o_kernels, o_stats = run_gpu(la, torch, w, other, args.steps,
                                                              args.warmup, 0, args.warmup_ms)
            o_val = flops / (o_total * 1e-3) / 1e12
            line["same_workload_" + other] = {
                "ms_per_step": round(o_total, 5), "tflops": round(o_val, 3),
                "step_stats": o_stats,
                "hbm": hbm_report(w, other, o_stats["fwd_ms_median"], o_stats["bwd_ms_median"]),
                "graph_ms_per_step": round(o_graph, 5),
                "graph_tflops": round(flops / (o_graph * 1e-3) / 1e12, 3),
                "frac_mfma_peak": round(o_val / PEAK_TFLOPS[other], 4),
                "kernels_ms": {k: round(v, 5) for k, v in o_kernels.items()}}

    if not args.no_extra and not args.no_others:
        # the other workloads of the parity suite, each in its own dtype (fewer
        # warm-up steps: they only place the headline among its neighbours)
        others = []
        for key in sorted(WORKLOADS):
            if key == args.workload:
                continue
            wo = WORKLOADS[key]
            o_total, o_graph, _, o_kernels, o_stats = run_gpu(la, torch, wo, wo.dtype,
                                                              args.steps, args.warmup, 0,
                                                              args.warmup_ms)
            o_flops = wo.flops_fwd + wo.flops_bwd
            o_val = o_flops / (o_total * 1e-3) / 1e12
            others.append({"workload": f"{wo.name} {wo.label()}", "dtype": wo.dtype,
                           "ms_per_step": round(o_total, 5), "tflops": round(o_val, 3),
                           "graph_ms_per_step": round(o_graph, 5),
                           "graph_tflops": round(o_flops / (o_graph * 1e-3) / 1e12, 3),
                           "frac_mfma_peak": round(o_val / PEAK_TFLOPS[wo.dtype], 4),
                           "step_stats": o_stats,
                           "hbm": hbm_report(wo, wo.dtype, o_stats["fwd_ms_median"],
                                             o_stats["bwd_ms_median"]),
                           "kernels_ms": {k: round(v, 5) for k, v in o_kernels.items()}})
        line["other_workloads"] = others

    if not args.no_extra and dtype == "f32":
        line["materialized_f32"] = run_materialized(la, torch, w, min(args.steps, 10), 2)

    if not args.no_extra:
        line["hbm_copy"] = hbm_copy(torch)
        line["layernorm"] = [run_layernorm(la, torch, w.B * w.T, w.C, "f32"),
                             run_layernorm(la, torch, w.B * w.T, w.C, "bf16")]

    if not args.no_extra:
        line["splitkv"] = run_splitkv(la, torch)
        line["projections"] = run_projections(la, torch, w.B * w.T, w.C)
        line["fp8_forward"] = run_fp8_forward(la, torch)

    if not args.no_extra:
        line["decode"] = [run_decode(la, torch, w, dtype, 50, 200),
                          run_decode(la, torch, WORKLOADS[5], "bf16", 50, 200)]

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, dtype, args.cpu_budget_s)

    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
