"""Benchmark of the PSA attention hot path on one MI355X.

One step = one fused PSA forward (psa_attention_fwd: PsaPackQkv + FA2 over
V_lo and V_hi + PsaMergeAttn in one kernel, writing the NCHW output, the NCHW
V residual and the LSE) over the 80x80 workload map (B=4, heads=8,
KEY_DIM=64, N=6400, bf16, synthetic N(0,1) input). ``value`` is its
throughput in TFLOP/s, counting the algorithmic 6*BH*N^2*KEY_DIM flops
(Q K^T once, P [V_lo | V_hi]).

Also measured and reported in the same JSON line: the unfused chain (pack,
FA2 x2, merge, extract), the layout kernels' GB/s against HBM peak (input and
output buffers rotated over 8 sets, far larger than the 256 MB Infinity Cache), the
40x40 forward, the FA2 backward workload, the PSA backward on the 40x40 map, and
detect-decode and the CIoU loss forward/backward on a batch of 64 images of 640x640 (GB/s against
HBM peak). The CPU oracle is timed on a bounded sample of the same workload as a reported baseline.

Before any timed region, the launch is repeated (untimed) until its duration stops falling:
an idle GPU raises its clocks over the first tens of milliseconds of load, and the figures
reported are those of the GPU under sustained load. The number of such launches and the first
and settled launch times are reported in the JSON line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "PSA attention fwd TFLOP/s + % bf16 MFMA peak; pack/merge GB/s % HBM"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E peak
WORKLOAD = "psa_fwd_bf16_80x80"
ATTN_KERNEL_SRC = os.path.join(ROOT, "vision_transformer_attention_psapackqkv_amd", "csrc", "attn_fwd.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_psa_fused_fwd_80x80.json")
LAYOUT_SETS = 8             # rotated buffer sets of the layout measurements


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-step", action="store_true",
                    help="time only the fused step (for profiler runs)")
    ap.add_argument("--layout-only", action="store_true",
                    help="only run pack, merge and extract a few times (for profiler runs)")
    ap.add_argument("--fa2-bwd-only", action="store_true",
                    help="time only the FA2 backward on the 40x40 workload (for profiling)")
    ap.add_argument("--psa-bwd-only", action="store_true",
                    help="time only the PSA backward on the 40x40 map (for profiling)")
    ap.add_argument("--yolo-only", action="store_true",
                    help="time only detect-decode and the CIoU loss kernels (for profiling)")
    ap.add_argument("--small-only", action="store_true",
                    help="time only the 8x8 and 20x20 maps, eager and as HIP-graph replays")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 512 MiB device copy 3 times (HBM counter calibration)")
    return ap.parse_args()


def fwd_flops(BH, N, KD):
    return 6.0 * BH * N * N * KD


def settle(fn, torch, max_s=3.0, tol=0.01):
    """Repeat `fn` until its launch time stops falling; returns (launches, first, last) in ms.

    An idle MI355X raises its clocks over the first tens of milliseconds of sustained load:
    back to back, the fused 80x80 forward takes ~600 us per launch at first and ~490 us once
    the clocks have settled (about 40 launches). Launches are timed in chunks of at least
    10 launches and 5 ms of GPU time; the loop ends when a chunk's mean launch time is within
    `tol` of the previous chunk's (after at least 3 chunks), or after `max_s` seconds.
    None of these launches is part of any timed region."""
    def chunk(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn(0)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n
    t0 = time.perf_counter()
    first = chunk(1)
    n = max(10, int(5.0 / max(first, 1e-3)) + 1)
    launches, prev, cur, chunks = 1, None, first, 0
    while time.perf_counter() - t0 < max_s:
        cur = chunk(n)
        launches += n
        chunks += 1
        if prev is not None and chunks >= 3 and abs(cur - prev) <= tol * prev:
            break
        prev = cur
    return launches, first, cur


def time_events(fn, steps, warmup, torch):
    """Average and total duration (ms) of `fn` launches, HIP events on the current stream
    (after the clocks have settled under this launch's load and `warmup` untimed launches)."""
    settle(fn, torch, max_s=1.0)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        fn(warmup + i)
        ends[i].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return sum(per) / len(per), min(per), wall


def time_batched(fn, steps, torch):
    """Average duration (ms) of `fn` launched `steps` times back to back on the current
    stream between one pair of HIP events (no event between the launches)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(steps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def back_to_back(fn, steps, torch):
    """Average launch time (ms) of `fn` over `steps` launches back to back between one event
    pair, best of three such runs (the kernel-trace duration of the launch; an event pair around
    every launch adds the dispatch and drain of each launch to it)."""
    return min(time_batched(fn, steps, torch) for _ in range(3))


def with_back_to_back(entry, fn, steps, torch, flops):
    """Adds the back-to-back launch time and the rate it gives to a component entry."""
    bb = back_to_back(fn, steps, torch)
    t = flops / (bb * 1e-3) / 1e12
    entry.update({"back_to_back_ms": round(bb, 5), "TFLOP/s_back_to_back": round(t, 3),
                  "pct_bf16_mfma_peak_back_to_back": round(100 * t / PEAK_BF16_TFLOPS, 2)})
    return entry


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def load_traffic(per_launch_flops):
    """HBM bytes per launch of the fused kernel from committed PMC counters, if still current."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("source_sha256") != source_sha(ATTN_KERNEL_SRC):
        return None
    return t.get("hbm_bytes_per_launch")


def host_cpu():
    """The host CPU's model name, the cores this process may run on and the cores the OS sees."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return model, usable, os.cpu_count() or 1


def cpu_baseline(qkv_cpu, w):
    """The float64 oracle on a bounded sample of the workload (whole batch-heads, each timed)."""
    import numpy as np
    from oracle import psa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    model, usable, total = host_cpu()
    x = qkv_cpu.to(dtype=__import__("torch").float64).numpy()
    packed = O.pack_qkv(x, w.B, w.heads, w.key_dim, w.H, w.W)
    s = O.default_scale(w.key_dim)
    per_bh, t0 = [], time.perf_counter()
    while len(per_bh) < w.BH and time.perf_counter() - t0 < 10.0:
        sl = slice(len(per_bh), len(per_bh) + 1)
        t1 = time.perf_counter()
        O.attention(packed[0][sl], packed[1][sl], packed[2][sl], s)
        O.attention(packed[0][sl], packed[1][sl], packed[3][sl], s)
        per_bh.append(time.perf_counter() - t1)
    el = time.perf_counter() - t0
    done = len(per_bh)
    flops = fwd_flops(done, w.N, w.key_dim)
    bh_flops = fwd_flops(1, w.N, w.key_dim)
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"float64 oracle attention (both V halves) on {done} of {w.BH} batch-heads "
                      f"of the {w.name} map, {el:.1f} s wall; pack timed once outside",
            "per_batch_head_s": {"median": round(float(np.median(per_bh)), 4),
                                 "min": round(min(per_bh), 4), "mean": round(el / done, 4)},
            "value_at_median": round(bh_flops / float(np.median(per_bh)) / 1e12, 6),
            "host": {"cpu_model": model, "cores_usable": usable, "cores_os": total,
                     "blas_threads": int(threads)}}


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: runs on one GPU only; --gpus must be 1. (Every batch-head is an "
              "independent problem, so several GPUs would each run this same kernel on their "
              "share of the batch with no exchange; that mode is not implemented.)", file=sys.stderr)
        sys.exit(2)

    import torch

    import psa_inputs as I
    import vision_transformer_attention_psapackqkv_amd as psa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        # A copy kernel of known size: reads and writes exactly 512 MiB per launch.
        src = torch.ones(256 * 1024 * 1024, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes_read": src.numel() * 2,
                          "calibration_copy_bytes_written": dst.numel() * 2}))
        return
    if args.fa2_bwd_only:
        print(json.dumps({"fa2_bwd_40x40": fa2_bwd_component(torch, psa, I, dev, args.steps, args.warmup)}))
        return
    if args.psa_bwd_only:
        print(json.dumps({"psa_bwd_40x40": psa_bwd_component(torch, psa, I, dev, args.steps, args.warmup)}))
        return
    if args.yolo_only:
        print(json.dumps(yolo_components(torch, psa, dev, args.steps, args.warmup)))
        return
    if args.small_only:
        print(json.dumps(small_map_components(torch, psa, I, dev, args.steps, args.warmup)))
        return
    w = I.WORKLOADS[WORKLOAD]
    qkv_cpu = I.make_workload_qkv(w)
    qkv = qkv_cpu.to(dev)
    # The timed step cycles over this many input/output sets (each 105 MB of qkv, 2 x 52 MB of
    # output and the LSE; 630 MB in all, beyond the 256 MB Infinity Cache), so every launch reads
    # its qkv from HBM rather than from the cache a previous launch left it in.
    step_sets = 3
    if args.layout_only:
        # Each layout op `steps` times back to back over the rotated buffer sets, as timed
        # in the components (for kernel traces and counters).
        for name, (fn, *_rest) in layout_fns(torch, psa, w, qkv).items():
            if name.startswith("device_copy"):
                continue
            for i in range(args.steps):
                fn(i)
            torch.cuda.synchronize()
        print(json.dumps({"layout_only": True, "workload": w.name, "launches_per_op": args.steps}))
        return
    qkvs = [qkv] + [qkv.clone() for _ in range(step_sets - 1)]
    outs = [torch.empty((w.B, w.out_channels, w.H, w.W), dtype=torch.bfloat16, device=dev)
            for _ in range(step_sets)]
    vress = [torch.empty_like(o) for o in outs]
    lses = [torch.empty((w.BH, w.N), dtype=torch.float32, device=dev) for _ in range(step_sets)]

    # The tail-split workspace is allocated once, outside the timed region.
    ws = torch.empty(psa.psa_attention_fwd_workspace_bytes(w.B, w.heads, w.key_dim, w.H, w.W),
                     dtype=torch.uint8, device=dev)

    def step(i):
        j = i % step_sets
        psa.psa_attention_fwd(qkvs[j], w.heads, w.key_dim, out=outs[j], v_out=vress[j], lse=lses[j],
                              workspace=ws)

    # Untimed: run the step until the GPU's clocks have settled under its load, then the
    # `warmup` steps; then the timed region: exactly `steps` fused forward steps.
    settle_n, settle_first, settle_last = settle(step, torch)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    per_launch = []
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        marks[i][0].record()
        step(i)
        marks[i][1].record()
    ev1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    per_launch = [a.elapsed_time(b) for a, b in marks]
    srt = sorted(per_launch)
    med_ms = srt[len(srt) // 2] if len(srt) % 2 else 0.5 * (srt[len(srt) // 2 - 1] + srt[len(srt) // 2])
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    kernel_ms = sum(per_launch) / len(per_launch)
    flops = fwd_flops(w.BH, w.N, w.key_dim)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    traffic = load_traffic(flops)

    result = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "heads": w.heads, "key_dim": w.key_dim,
                   "H": w.H, "W": w.W, "N": w.N, "path": "psa_attention_fwd (fused)",
                   "parallelism": "single GPU"},
        "pct_bf16_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "kernel": "attn_fwd_bf16<64,128,NCHW> + attn_fwd_merge (one psa_attention_fwd)",
                     "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "avg_kernel_ms": round(kernel_ms, 5), "median_kernel_ms": round(med_ms, 5),
                     "min_kernel_ms": round(srt[0], 5), "flops_per_launch": flops,
                     "inputs": f"{step_sets} rotated qkv/out/v/lse sets (630 MB, beyond the 256 MB "
                               "Infinity Cache)"},
        "wall_ms_timed_region": round(wall_ms, 3),
        "settle": {"launches_before_warmup": settle_n, "first_launch_ms": round(settle_first, 5),
                   "settled_launch_ms": round(settle_last, 5),
                   "note": "untimed launches until the launch time stopped falling (clock ramp of an idle GPU)"},
    }

    if not args.only_step:
        result["components"] = components(torch, psa, I, w, qkv, args)
        # The same step on one buffer set (its 210 MB of inputs and outputs may stay in the
        # Infinity Cache between launches): shows the headline does not depend on that cache.
        one, _, _ = time_events(lambda _i: step(0), args.steps, args.warmup, torch)
        result["components"]["fused_fwd_80x80_one_buffer_set"] = {
            "avg_ms": round(one, 5), "TFLOP/s": round(flops / (one * 1e-3) / 1e12, 3)}
    if not args.no_cpu_baseline and not args.only_step:
        result["cpu_baseline"] = cpu_baseline(qkv_cpu, w)
    print(json.dumps(result), flush=True)


def layout_fns(torch, psa, w, qkv):
    """Pack, merge, extract and a plain device copy of pack's size, each cycling over 8
    buffer sets, so that the bytes one op touches over a cycle (>= 840 MB: merge and extract
    read half of each packed buffer) far exceed the 256 MB Infinity Cache and every launch
    reads and writes HBM.
    name -> (fn(i), algorithmic bytes per launch, packed buffers, NCHW output buffers)."""
    dev = qkv.device
    B, h, KD, H, W = w.B, w.heads, w.key_dim, w.H, w.W
    sets = LAYOUT_SETS
    qkvs = [qkv] + [qkv.clone() for _ in range(sets - 1)]
    packs = [torch.empty((4, w.BH, w.N, KD), dtype=qkv.dtype, device=dev) for _ in range(sets)]
    outs = [torch.empty((B, w.out_channels, H, W), dtype=qkv.dtype, device=dev) for _ in range(sets)]
    elt = 2
    e_qkv = B * w.qkv_channels * w.N
    e_out = B * w.out_channels * w.N
    copies = [torch.empty_like(qkv) for _ in range(sets)]
    return {
        "pack": (lambda i: psa.psa_pack_qkv(qkvs[i % sets], h, KD, out=packs[i % sets]), 2 * e_qkv * elt,
                 packs, outs),
        "merge": (lambda i: psa.psa_merge_attn(packs[i % sets][:2], B, h, KD, H, W, out=outs[i % sets]),
                  2 * e_out * elt),
        "extract": (lambda i: psa.psa_extract_v(packs[i % sets], B, h, KD, H, W, out=outs[i % sets]),
                    2 * e_out * elt),
        "device_copy_same_size_as_pack": (lambda i: copies[i % sets].copy_(qkvs[i % sets]), 2 * e_qkv * elt),
    }


def components(torch, psa, I, w, qkv, args):
    """Side measurements: unfused chain, layout GB/s, other workloads."""
    dev = qkv.device
    steps, warm = max(args.steps, 10), max(args.warmup, 3)
    comp = {}
    B, h, KD, H, W = w.B, w.heads, w.key_dim, w.H, w.W
    layout = layout_fns(torch, psa, w, qkv)
    packs, outs = layout["pack"][2], layout["pack"][3]
    # Each op is timed two ways after its clocks settle: an event pair around every launch,
    # and `steps` launches back to back between one event pair. The second matches the
    # kernel durations of a rocprofv3 kernel trace of the same launches (an event pair adds
    # ~1-3 us around each of these 20-40 us kernels, a HIP graph replay ~1 us per node, and
    # the host's launches keep ahead of the GPU), so it gives the GB/s.
    for name, (fn, nbytes, *_bufs) in layout.items():
        avg, best, _ = time_events(fn, steps, warm, torch)
        bat = time_batched(fn, max(steps, 4 * LAYOUT_SETS), torch)
        gbps = nbytes / (bat * 1e-3) / 1e9
        comp[name] = {"avg_ms": round(bat, 5), "avg_ms_event_pair_per_launch": round(avg, 5),
                      "min_ms_event_pair_per_launch": round(best, 5), "bytes": nbytes,
                      "GB/s": round(gbps, 1), "pct_hbm_peak": round(100 * gbps / PEAK_HBM_GBPS, 2),
                      "GB/s_event_pair_per_launch": round(nbytes / (avg * 1e-3) / 1e9, 1),
                      "timing": "launches back to back over %d rotated buffer sets" % LAYOUT_SETS}
    # Unfused chain on the same map: pack, FA2(V_lo), FA2(V_hi), merge, extract.
    o2 = torch.empty((2, w.BH, w.N, KD), dtype=qkv.dtype, device=dev)
    lse = torch.empty((w.BH, w.N), dtype=torch.float32, device=dev)
    pk, out = packs[0], outs[0]
    ws_fa = torch.empty(psa.fa2_fwd_workspace_bytes(w.BH, w.N, w.N, KD), dtype=torch.uint8, device=dev)

    def unfused(_i):
        psa.psa_pack_qkv(qkv, h, KD, out=pk)
        psa.fa2_fwd(pk[0], pk[1], pk[2], out=o2[0], lse=lse, workspace=ws_fa)
        psa.fa2_fwd(pk[0], pk[1], pk[3], out=o2[1], want_lse=False, workspace=ws_fa)
        psa.psa_merge_attn(o2, B, h, KD, H, W, out=out)
        psa.psa_extract_v(pk, B, h, KD, H, W, out=outs[1])

    avg, best, _ = time_events(unfused, steps, warm, torch)
    comp["unfused_chain"] = {"avg_ms": round(avg, 5), "TFLOP/s": round(fwd_flops(w.BH, w.N, KD) / (avg * 1e-3) / 1e12, 3)}
    fa_fn = lambda i: psa.fa2_fwd(pk[0], pk[1], pk[2], out=o2[0], lse=lse, workspace=ws_fa)
    fa_avg, _, _ = time_events(fa_fn, steps, warm, torch)
    fa_flops = 4.0 * w.BH * w.N ** 2 * KD
    comp["fa2_fwd_one_half"] = with_back_to_back(
        {"avg_ms": round(fa_avg, 5), "TFLOP/s": round(fa_flops / (fa_avg * 1e-3) / 1e12, 3)},
        fa_fn, steps, torch, fa_flops)
    # The 40x40 forward workload (fused).
    w2 = I.WORKLOADS["psa_fwd_bf16_40x40_peaked"]
    q2 = I.make_workload_qkv(w2).to(dev)
    o_2 = torch.empty((w2.B, w2.out_channels, w2.H, w2.W), dtype=q2.dtype, device=dev)
    v_2 = torch.empty_like(o_2)
    l_2 = torch.empty((w2.BH, w2.N), dtype=torch.float32, device=dev)
    ws_2 = torch.empty(psa.psa_attention_fwd_workspace_bytes(w2.B, w2.heads, w2.key_dim, w2.H, w2.W),
                       dtype=torch.uint8, device=dev)
    f2 = lambda i: psa.psa_attention_fwd(q2, w2.heads, w2.key_dim, out=o_2, v_out=v_2, lse=l_2, workspace=ws_2)
    avg, _, _ = time_events(f2, steps, warm, torch)
    flops2 = fwd_flops(w2.BH, w2.N, w2.key_dim)
    t2 = flops2 / (avg * 1e-3) / 1e12
    comp["fused_fwd_40x40"] = with_back_to_back(
        {"avg_ms": round(avg, 5), "TFLOP/s": round(t2, 3), "pct_bf16_mfma_peak": round(100 * t2 / PEAK_BF16_TFLOPS, 2)},
        f2, steps, torch, flops2)
    del q2, o_2, v_2, l_2
    comp.update(small_map_components(torch, psa, I, dev, steps, warm))
    comp["fa2_bwd_40x40"] = fa2_bwd_component(torch, psa, I, dev, steps, warm)
    comp["psa_bwd_40x40"] = psa_bwd_component(torch, psa, I, dev, steps, warm)
    comp.update(yolo_components(torch, psa, dev, steps, warm))
    comp["reference_torch_bf16_gemm_8192"] = reference_gemm(torch, dev, steps)
    return comp


def reference_gemm(torch, dev, steps):
    """torch's bf16 GEMM (the vendor BLAS) on 8192^3, back to back on the same box: what a
    library contraction reaches here, as context for the attention rates (boxes differ in the
    clock they hold under MFMA load by up to ~10 %)."""
    n = 8192
    g = torch.Generator(device=dev).manual_seed(3)
    a = torch.randn((n, n), generator=g, device=dev).to(torch.bfloat16)
    b = torch.randn((n, n), generator=g, device=dev).to(torch.bfloat16)
    c = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
    fn = lambda _i: torch.mm(a, b, out=c)
    settle(fn, torch, max_s=1.0)
    t = back_to_back(fn, max(10, steps // 4), torch)
    tf = 2.0 * n ** 3 / (t * 1e-3) / 1e12
    del a, b, c
    return {"avg_ms": round(t, 5), "TFLOP/s": round(tf, 3), "pct_bf16_mfma_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
            "note": "torch.mm bf16 8192x8192x8192, launches back to back; not part of the PSA path"}


def time_graph(fns, steps, warm, torch):
    """Average duration (ms) of one of `fns`, all captured back to back in one HIP graph
    (so that host launch cost does not pace the GPU), over `steps` replays."""
    for f in fns:
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    settle(lambda _i: g.replay(), torch, max_s=1.0)
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / (steps * len(fns))


def yolo_components(torch, psa, dev, steps, warm):
    """Detect-decode and the CIoU loss forward/backward on a batch of 64 images of 640x640
    (8400 anchors each), HBM-bound: GB/s of algorithmic bytes against the HBM peak. Each
    kernel cycles over enough buffer sets (> 256 MB in all) that its data come from HBM."""
    import yolo_inputs as yi
    B, A = 64, 8400
    N = B * A
    res = {}
    ax, ay, st = (t.to(dev) for t in yi.anchor_grid())
    for name, dtype, elt in (("detect_decode_f32_b64", torch.float32, 4),
                             ("detect_decode_bf16_b64", torch.bfloat16, 2)):
        per = 2 * B * 4 * A * elt
        sets = -(-300_000_000 // per)
        ins = [yi.ltrb_boxes(B, A, dtype=dtype, seed=i).to(dev) for i in range(sets)]
        outs = [torch.empty_like(x) for x in ins]
        fns = [lambda x=x, o=o: psa.detect_decode(x, ax, ay, st, out=o) for x, o in zip(ins, outs)]
        avg = time_graph(fns, steps, warm, torch)
        nbytes = per + 3 * A * 4
        res[name] = {"avg_ms": round(avg, 6), "bytes": nbytes, "GB/s": round(nbytes / (avg * 1e-3) / 1e9, 1),
                     "pct_hbm_peak": round(100 * nbytes / (avg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
                     "B": B, "A": A, "sets": sets}
        del ins, outs, fns
    sets = -(-300_000_000 // (48 * N))
    data = [tuple(t.to(dev) for t in yi.ciou_boxes(N, seed=i)) for i in range(sets)]
    saved = [psa.ciou_loss_fwd(p, g) for p, g, _ in data]
    fwd_out = [tuple(torch.empty(N, device=dev) for _ in range(4)) for _ in range(sets)]

    avg = time_graph([lambda i=i: psa.ciou_loss_fwd(data[i][0], data[i][1], out=fwd_out[i])
                      for i in range(sets)], steps, warm, torch)
    res["ciou_fwd_n537600"] = {"avg_ms": round(avg, 6), "bytes": 48 * N,
                               "GB/s": round(48 * N / (avg * 1e-3) / 1e9, 1),
                               "pct_hbm_peak": round(100 * 48 * N / (avg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
                               "N": N, "sets": sets}
    dps = [torch.empty((4, N), device=dev) for _ in range(sets)]
    fns = [lambda i=i: psa.ciou_loss_bwd(data[i][0], data[i][1], saved[i][1], saved[i][2], saved[i][3],
                                         data[i][2], dpred=dps[i]) for i in range(sets)]
    avg = time_graph(fns, steps, warm, torch)
    res["ciou_bwd_n537600"] = {"avg_ms": round(avg, 6), "bytes": 64 * N,
                               "GB/s": round(64 * N / (avg * 1e-3) / 1e9, 1),
                               "pct_hbm_peak": round(100 * 64 * N / (avg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
                               "N": N, "sets": sets}
    return res


def fa2_bwd_component(torch, psa, I, dev, steps, warm):
    """The FA2 backward workload (Delta + dK/dV + dQ launches), O and LSE from fa2_fwd."""
    wb = I.WORKLOADS["fa2_bwd_bf16_40x40"]
    q, k, v, do = (t.to(dev) for t in I.make_workload_bwd(wb))
    o, lse_b = psa.fa2_fwd(q, k, v)
    ws = torch.empty((psa.load_library().fa2_bwd_workspace_bytes(wb.BH, wb.N) // 4,), dtype=torch.float32,
                     device=dev)
    fn = lambda i: psa.fa2_bwd(q, k, v, o, do, lse_b, workspace=ws)
    avg, _, _ = time_events(fn, steps, warm, torch)
    flops = 10.0 * wb.BH * wb.N ** 2 * wb.key_dim
    tb = flops / (avg * 1e-3) / 1e12
    return with_back_to_back(
        {"avg_ms": round(avg, 5), "TFLOP/s": round(tb, 3), "pct_bf16_mfma_peak": round(100 * tb / PEAK_BF16_TFLOPS, 2),
         "flops": "10*BH*N^2*D"}, fn, steps, torch, flops)


def small_map_components(torch, psa, I, dev, steps, warm):
    """The two small maps (8x8 in float32, 20x20 in bf16), fused forward and forward + backward,
    which are bound by launch cost, not by the GPU's arithmetic: an event pair around each step,
    steps back to back, and 32 steps captured in one HIP graph and replayed (the GPU-side time
    of a step without the host's launches pacing it)."""
    res = {}
    for name, tag in (("psa_fwd_f32_tiny_8x8", "8x8_f32"), ("psa_fwd_bf16_20x20", "20x20")):
        w = I.WORKLOADS[name]
        x = I.make_workload_qkv(w).to(dev)
        shape = (w.B, w.out_channels, w.H, w.W)
        out, v, dout = (torch.empty(shape, dtype=x.dtype, device=dev) for _ in range(3))
        dout.copy_(torch.randn(shape, generator=torch.Generator(device=dev).manual_seed(9), device=dev))
        lse = torch.empty((w.BH, w.N), dtype=torch.float32, device=dev)
        dqkv = torch.empty_like(x)
        nb = psa.psa_attention_fwd_workspace_bytes(w.B, w.heads, w.key_dim, w.H, w.W, dtype=x.dtype)
        ws_f = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev) if nb else None
        ws_b = torch.empty((max(psa.load_library().psa_attention_bwd_workspace_bytes(w.B, w.heads, w.H, w.W), 4) // 4,),
                           dtype=torch.float32, device=dev)
        fwd = lambda _i=0: psa.psa_attention_fwd(x, w.heads, w.key_dim, out=out, v_out=v, lse=lse, workspace=ws_f)

        def fwd_bwd(_i=0):
            fwd()
            psa.psa_attention_bwd(x, out, lse, dout, w.heads, w.key_dim, dv=dout, dqkv=dqkv, workspace=ws_b)

        for label, fn, flops in (("fused_fwd", fwd, fwd_flops(w.BH, w.N, w.key_dim)),
                                 ("fused_fwd_bwd", fwd_bwd, (6.0 + 14.0) * w.BH * w.N ** 2 * w.key_dim)):
            avg, _, _ = time_events(fn, steps, warm, torch)
            bb = back_to_back(fn, steps, torch)
            gr = time_graph([fn] * 32, steps, warm, torch)
            res[f"{label}_{tag}"] = {
                "avg_us_event_pair": round(1e3 * avg, 2), "back_to_back_us": round(1e3 * bb, 2),
                "graph_replay_us": round(1e3 * gr, 2),
                "TFLOP/s_graph_replay": round(flops / (gr * 1e-3) / 1e12, 3),
                "note": "launch-bound map; %s flops per step" % ("6*BH*N^2*KD" if label == "fused_fwd" else "(6+14)*BH*N^2*KD")}
        del x, out, v, dout, lse, dqkv, ws_f, ws_b
    return res


def psa_bwd_component(torch, psa, I, dev, steps, warm):
    """The PSA backward (psa_attention_bwd: d(qkv) from dOut and the V-residual gradient) on
    the 40x40 forward map, O and LSE from the fused forward."""
    w = I.WORKLOADS["psa_fwd_bf16_40x40_peaked"]
    x = I.make_workload_qkv(w).to(dev)
    out, _, lse = psa.psa_attention_fwd(x, w.heads, w.key_dim, want_v=False)
    g = torch.randn(out.shape, generator=torch.Generator(device=dev).manual_seed(7), device=dev).to(out.dtype)
    gv = torch.randn(out.shape, generator=torch.Generator(device=dev).manual_seed(8), device=dev).to(out.dtype)
    dqkv = torch.empty_like(x)
    ws = torch.empty((psa.load_library().psa_attention_bwd_workspace_bytes(w.B, w.heads, w.H, w.W) // 4,),
                     dtype=torch.float32, device=dev)
    fn = lambda i: psa.psa_attention_bwd(x, out, lse, g, w.heads, w.key_dim, dv=gv, dqkv=dqkv, workspace=ws)
    avg, _, _ = time_events(fn, steps, warm, torch)
    flops = 14.0 * w.BH * w.N ** 2 * w.key_dim
    t = flops / (avg * 1e-3) / 1e12
    return with_back_to_back(
        {"avg_ms": round(avg, 5), "TFLOP/s": round(t, 3), "pct_bf16_mfma_peak": round(100 * t / PEAK_BF16_TFLOPS, 2),
         "flops": "14*BH*N^2*KD (QK^T, dO V^T over 2KD, P^T dO over 2KD, dS^T Q, dS K)"}, fn, steps, torch, flops)


if __name__ == "__main__":
    main()
