#!/usr/bin/env python3
"""Benchmark of the RoPE apply path on one MI355X: achieved HBM GB/s (and fraction of the
8 TB/s peak) and tokens/s.

One step is one pass of the in-place partial interleave op over one batch of the headline
workload: bf16 x [8,4096,1,576], slice [512,576), fp32 cos/sin [8,4096,1,64] (32768 tokens).
The cos/sin-cache kernel is timed the same way on its three workloads (rope NeoX bf16, rope
GPT-J fp16 with a pass-through half, mrope bf16) and reported in `kernels`.

Timing: inputs are resident in HBM; launches cycle over enough copies of the inputs that
every pass touches >= 2 GiB before a buffer is reused, so that MI355X's 256 MB Infinity
Cache holds none of a buffer set's lines when it comes round again; the host queues the timed launches behind a short GPU spin so
that they run back to back, and two HIP events on the launch stream bracket exactly `steps`
launches.  Rank 0 prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
# Bytes touched between reuses of one buffer set.  At 512 MiB, lines of a set were still in
# the Infinity Cache at its next use (the in-place kernel measured 2-3% faster, a
# write-through variant of it 7-10%); from 1 GiB to 2 GiB the times are equal, and much
# larger rotations start to add TLB misses of their own.
MALL_DEFEAT_BYTES = 2 << 30
KERNEL_SRC = os.path.join(ROOT, "rope_partial_inplace_amd", "csrc", "rope_kernels.hip")


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_code_hash() -> str:
    """sha256[:16] of rope_kernels.hip with its // comments, trailing blanks and blank lines
    removed: it changes when the kernels' code does, not when a comment is edited, so a
    traffic figure stays attached to the code it was measured on."""
    with open(KERNEL_SRC, encoding="utf-8") as f:
        lines = [re.sub(r"//.*$", "", line).rstrip() for line in f.read().splitlines()]
    return hashlib.sha256("\n".join(x for x in lines if x).encode()).hexdigest()[:16]


# ------------------------------------------------------------------------------------------
# GPU timing
# ------------------------------------------------------------------------------------------

def spin_cycles_per_ms(torch) -> float:
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    torch.cuda._sleep(2_000_000)
    b.record()
    torch.cuda.synchronize()
    return 2_000_000 / max(a.elapsed_time(b), 1e-3)


def time_launches(torch, calls, steps: int, warmup: int, cyc_per_ms: float):
    """Mean GPU time per launch (ms) over `steps` back-to-back launches cycling over calls."""
    n = len(calls)
    for i in range(warmup):
        calls[i % n]()
    torch.cuda.synchronize()
    # host enqueue cost per launch, to size the spin that hides it
    t0 = time.perf_counter()
    for i in range(min(steps, 20)):
        calls[i % n]()
    host_ms = (time.perf_counter() - t0) * 1e3 / min(steps, 20)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for attempt in range(3):
        spin_ms = 1.0 + 1.5 * host_ms * steps * (1 + attempt)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(spin_ms * cyc_per_ms))
        t0 = time.perf_counter()
        start.record()
        for i in range(steps):
            calls[i % n]()
        end.record()
        enqueue_ms = (time.perf_counter() - t0) * 1e3
        torch.cuda.synchronize()
        if enqueue_ms < spin_ms:  # the GPU never waited for the host
            break
        log(f"host enqueue {enqueue_ms:.2f} ms exceeded the {spin_ms:.2f} ms spin; retrying")
    return start.elapsed_time(end) / steps


def graph_replay_us(torch, ra, case, n_sets: int, reps: int = 3) -> float:
    """Per-launch time of the in-place op when its launches over the n_sets buffer sets are
    captured in one HIP graph and the graph is replayed back to back (inputs rotated as in
    the stream timing).  Reported beside the stream-launch figure: a serving loop that
    replays a captured graph pays this per-launch cost instead."""
    xs = [case.x] + [case.x.clone() for _ in range(n_sets - 1)]
    cs = [case.cos] + [case.cos.clone() for _ in range(n_sets - 1)]
    ss = [case.sin] + [case.sin.clone() for _ in range(n_sets - 1)]
    fn = ra.rope_partial_inplace_backward if case.backward else ra.rope_partial_inplace

    def launches():
        for x, c, sn in zip(xs, cs, ss):
            fn(x, c, sn, case.rotary_mode, case.partial_slice)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture, as capture requires
        launches()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launches()
    g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / (reps * n_sets)
    del g, xs, cs, ss
    torch.cuda.empty_cache()
    return ms * 1e3


def launch_floor_us(torch, ra, W, dev, cyc) -> float:
    """Per-launch time of the smallest in-place launch (one row of 64 fp32 elements, one
    workgroup) issued back to back: the cost of a launch itself on this GPU and runtime."""
    case = W.inplace_case("floor", 1, 1, 1, 64, torch.float32, torch.float32, [0, 64], seed=7,
                          device=dev)
    calls = inplace_calls(ra, case, 1)
    return time_launches(torch, calls, 200, 20, cyc) * 1e3


def copy_ceiling_gbs(torch, nbytes=1 << 30) -> float:
    """Device-to-device copy bandwidth (read + write bytes) at a footprint well above the
    Infinity Cache: the attainable-bandwidth context for the kernels."""
    a = torch.empty(nbytes // 2, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(10):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / 10
    return 2 * a.numel() / (ms * 1e-3) / 1e9


def copy_same_bytes(torch, moved: int, cyc: float, steps: int = 100) -> dict:
    """A device-to-device copy (torch's copy_) that reads and writes `moved` bytes in all,
    timed like the kernels (buffer pairs rotated over MALL_DEFEAT_BYTES, launches back to
    back): what a plain copy of the headline's bytes achieves at the same footprint."""
    half = moved // 2
    n_sets = max(1, math.ceil(MALL_DEFEAT_BYTES / moved))
    pairs = [(torch.empty(half, dtype=torch.uint8, device="cuda"),
              torch.empty(half, dtype=torch.uint8, device="cuda")) for _ in range(n_sets)]
    calls = [(lambda a=a, b=b: b.copy_(a)) for a, b in pairs]
    ms = time_launches(torch, calls, steps, 10, cyc)
    del calls, pairs
    torch.cuda.empty_cache()
    return {"bytes": 2 * half, "us": round(ms * 1e3, 3),
            "gbs": round(2 * half / (ms * 1e-3) / 1e9, 1), "buffer_sets": n_sets}


# ------------------------------------------------------------------------------------------
# workloads
# ------------------------------------------------------------------------------------------

# Workloads reported beside the configurations, with what they show.
EXTRA = {"inplace_f32_1x524288x2x64":
         "scaled variant of the fp32 [1,16,2,64] workload (same dtype, slice and BS1D layout, "
         "S = 524288): the kernel's streaming rate at 768 MiB per launch"}


def n_sets_for(algo_bytes: int) -> int:
    return max(1, math.ceil(MALL_DEFEAT_BYTES / algo_bytes))


def inplace_calls(ra, case, n_sets):
    calls = []
    for i in range(n_sets):
        x = case.x if i == 0 else case.x.clone()
        c = case.cos if i == 0 else case.cos.clone()
        s = case.sin if i == 0 else case.sin.clone()
        calls.append(ra.prepare_partial_inplace(x, c, s, case.rotary_mode, case.partial_slice,
                                                backward=case.backward))
    return calls


def cache_calls(ra, torch, case, n_sets):
    calls = []
    for i in range(n_sets):
        q = case.query if i == 0 else case.query.clone()
        k = case.key if i == 0 else case.key.clone()
        p = case.positions if i == 0 else case.positions.clone()
        qo, ko = torch.empty_like(q), torch.empty_like(k)
        calls.append(ra.prepare_with_cos_sin_cache(p, q, k, case.cache, case.mrope_section,
                                                   case.head_size, case.is_neox, qo, ko,
                                                   cache_mode=case.cache_mode))
    return calls


def describe_case(name, case):
    if hasattr(case, "x"):
        what = "InplacePartialRotaryMul backward (gradient)" if case.backward else \
            "InplacePartialRotaryMul"
        mode = "interleave" if case.rotary_mode == 1 else "half mode"
        return (f"{what} {mode} x {str(case.x.dtype)[6:]} "
                f"{list(case.x.shape)} slice {case.partial_slice} cos/sin "
                f"{str(case.cos.dtype)[6:]} {list(case.cos.shape)}")
    mode = f"mrope {case.mrope_section}" if case.mrope_section else "rope"
    if case.mrope_section and case.cache_mode == 1:
        mode += " interleaved (cacheMode 1)"
    style = "NeoX" if case.is_neox else "GPT-J"
    return (f"RopeWithSinCosCache {mode} {style} {str(case.query.dtype)[6:]} T={case.tokens} "
            f"q {list(case.query.shape)} k {list(case.key.shape)} headSize {case.head_size} "
            f"rotaryDim {case.cache.shape[1]}")


def kernel_name(case) -> str:
    """The kernel a workload's launches run.  The cache op takes its wavefront kernel when q/k
    and the cache rows allow 16-byte access, a head holds at most 64 units (NeoX: two
    16-byte vectors each, GPT-J: one) and the positions are 8-byte aligned; the profile
    summaries under profiles/ record the symbol each workload's dispatches actually had."""
    if hasattr(case, "x"):
        return "inplace_rope_kernel"
    es = case.query.element_size()
    units = case.head_size * es // (32 if case.is_neox else 16)
    aligned = all(t.data_ptr() % 16 == 0 and (t.stride(0) * es) % 16 == 0
                  for t in (case.query, case.key, case.cache))
    wave = aligned and units <= 64 and case.positions.data_ptr() % 8 == 0
    return "cos_sin_cache_wave_kernel" if wave else "cos_sin_cache_kernel"


def traffic_for(workload: str):
    """Measured HBM bytes per launch from the committed PMC summary, when it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_code_sha256_16") != kernel_code_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def size_sweep(torch, ra, W, dev, cyc):
    """Per-launch time of the same kernels at growing token counts, and the least-squares fit
    time = fixed + bytes / marginal_rate: the fixed part is what bounds a short launch."""
    import numpy as np
    shapes = {
        "inplace_rope_kernel": [
            (f"bf16 x [{8 * m},4096,1,576] slice [512,576) f32 cos/sin", m,
             lambda m=m: W.inplace_case("sweep", 8 * m, 4096, 1, 576, torch.bfloat16,
                                        torch.float32, [512, 576], seed=1100 + m, device=dev))
            for m in (1, 2, 4, 8, 16)],
        "cos_sin_cache_wave_kernel": [
            (f"rope NeoX bf16 T={8192 * m} q 32x128 k 8x128", m,
             lambda m=m: W.cache_case("sweep", 8192 * m, 32, 8, 128, 128, torch.bfloat16, True,
                                      32768, seed=1200 + m, device=dev))
            for m in (1, 2, 4, 8)],
    }
    out = {}
    for kern, rows in shapes.items():
        pts = []
        for what, m, make in rows:
            case = make()
            n_sets = n_sets_for(case.algo_bytes)
            calls = (inplace_calls(ra, case, n_sets) if hasattr(case, "x")
                     else cache_calls(ra, torch, case, n_sets))
            us = time_launches(torch, calls, 100, 10, cyc) * 1e3
            pts.append({"workload": what, "tokens": case.tokens, "bytes": case.algo_bytes,
                        "us": round(us, 3), "gbs": round(case.algo_bytes / us / 1e3, 1)})
            log(f"sweep {kern} {what}: {us:.3f} us, {case.algo_bytes / us / 1e3:.0f} GB/s")
            del calls, case
            torch.cuda.empty_cache()
        b = np.array([p["bytes"] for p in pts], dtype=np.float64)
        t = np.array([p["us"] for p in pts], dtype=np.float64)
        slope, fixed = np.polyfit(b, t, 1)
        out[kern] = {"points": pts, "fit_fixed_us": round(float(fixed), 3),
                     "fit_marginal_gbs": round(float(1e-3 / slope), 1)}
    return {"sweep": out, "kernel_code_sha256_16": kernel_code_hash()}


# ------------------------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands, on the host
# ------------------------------------------------------------------------------------------

def _oracle_rate(case, threads: int, budget_s: float):
    """Run the oracle (unchanged, single-threaded C) over the headline batch for ~budget_s
    from `threads` host threads at once, each on its own block of rows: the batch is viewed
    as [B*S, 1, N, D] rows (cos/sin alike, which keeps each row's cos/sin row), and thread k
    rotates rows [k*R/threads, (k+1)*R/threads) again and again.  ctypes releases the GIL
    during each call.  Returns (bytes/s, tokens/s, passes over the whole batch)."""
    import threading
    import oracle
    B, S, N, D = case.x.shape
    x = case.x.cpu().reshape(B * S, 1, N, D).contiguous()
    c = case.cos.cpu().reshape(B * S, 1, case.cos.shape[2], case.cos.shape[3]).contiguous()
    sn = case.sin.cpu().reshape(B * S, 1, case.sin.shape[2], case.sin.shape[3]).contiguous()
    assert case.cos.shape[:2] == (B, S), "the CPU baseline needs per-(b, s) cos/sin rows"
    rows = B * S
    edges = [rows * k // threads for k in range(threads + 1)]
    done = [0.0] * threads
    stop = threading.Event()

    def work(k):
        lo, hi = edges[k], edges[k + 1]
        xs, cs, ss = x[lo:hi], c[lo:hi], sn[lo:hi]
        while not stop.is_set():
            st, _ = oracle.rope_partial_inplace(xs, cs, ss, case.rotary_mode, case.partial_slice)
            assert st == 0, oracle.last_error()
            done[k] += (hi - lo) / rows

    pool = [threading.Thread(target=work, args=(k,)) for k in range(threads)]
    t0 = time.perf_counter()
    for t in pool:
        t.start()
    time.sleep(budget_s)
    stop.set()
    for t in pool:
        t.join()
    el = time.perf_counter() - t0
    passes = sum(done)
    return case.algo_bytes * passes / el, case.tokens * passes / el, passes, el


def cpu_baseline(case, budget_s: float):
    """The oracle as it stands on the host: on all the cores this process may use (up to 16,
    the host share of one GPU), plus the single-thread figure."""
    cores = min(16, len(os.sched_getaffinity(0)))
    bps, tps, passes, el = _oracle_rate(case, cores, budget_s)
    bps1, tps1, passes1, el1 = _oracle_rate(case, 1, max(2.0, budget_s / 3))
    return {
        "value": round(bps / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"the full headline batch ({case.tokens} tokens) rotated {passes:.1f} times in "
                   f"{el:.1f} s by the single-threaded C oracle run from {cores} host threads at "
                   f"once, each on its own block of rows"),
        "tokens_per_s": round(tps, 1),
        "single_thread": {"value": round(bps1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                          "tokens_per_s": round(tps1, 1),
                          "sample": f"{passes1:.1f} passes over the batch in {el1:.1f} s"},
        "host_cpu": platform.processor() or platform.machine(),
        "host_cores_visible": len(os.sched_getaffinity(0)),
    }


# ------------------------------------------------------------------------------------------

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workloads", default=",".join(
                        ["inplace_bf16_8x4096x1x576_s512", "inplace_f32_1x16x2x64",
                         "cache_rope_neox_bf16_t8192", "cache_rope_gptj_f16_t32768_rd64",
                         "cache_mrope_neox_bf16_t16384",
                         "inplace_backward_bf16_8x4096x1x576_s512",
                         "cache_mrope_interleaved_neox_bf16_t16384",
                         "inplace_half_bf16_8x4096x1x576_s512",
                         "inplace_heads_bf16_4x2048x32x192_s128_bs1d",
                         "inplace_f32_1x524288x2x64"]),
                    help="first is the headline; the rest are reported under `kernels`")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=10.0)
    ap.add_argument("--resident", action="store_true",
                    help="also time without buffer rotation (Infinity-Cache-resident)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the benchmark line, time the headline in-place shape and "
                         "the rope NeoX cache shape at 1..16x their tokens and fit fixed cost "
                         "+ bytes / marginal bandwidth (one JSON line)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the RoPE path has no cross-GPU step; see the sharding notes)", file=sys.stderr)
        return 2

    import torch
    sys.path.insert(0, ROOT)
    import rope_partial_inplace_amd as ra
    import rope_workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} ({getattr(props, 'gcnArchName', '?')}), "
        f"{props.multi_processor_count} CUs")
    cyc = spin_cycles_per_ms(torch)
    if args.sweep:
        print(json.dumps(size_sweep(torch, ra, W, dev, cyc)), flush=True)
        return 0
    names = [w.strip() for w in args.workloads.split(",") if w.strip()]
    results = {}
    cases = {}
    for wi, name in enumerate(names):
        case = W.CONFIGS[name](dev)
        cases[name] = case
        n_sets = 1 if name == "inplace_f32_1x16x2x64" else n_sets_for(case.algo_bytes)
        calls = (inplace_calls(ra, case, n_sets) if hasattr(case, "x")
                 else cache_calls(ra, torch, case, n_sets))
        steps = args.steps if wi == 0 else max(20, min(args.steps, 100))
        ms = time_launches(torch, calls, steps, args.warmup, cyc)
        gbs = case.algo_bytes / (ms * 1e-3) / 1e9
        r = {"workload": describe_case(name, case), "kernel": kernel_name(case),
             "us_per_launch": round(ms * 1e3, 3), "gbs": round(gbs, 1),
             "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
             "tokens_per_s": round(case.tokens / (ms * 1e-3), 1),
             "algo_bytes_per_launch": case.algo_bytes, "buffer_sets": n_sets, "steps": steps,
             "traffic": traffic_for(name)}
        if name in EXTRA:
            r["extra"] = EXTRA[name]
        if args.resident:
            ms_r = time_launches(torch, calls[:1], steps, args.warmup, cyc)
            r["resident_us_per_launch"] = round(ms_r * 1e3, 3)
            r["resident_gbs"] = round(case.algo_bytes / (ms_r * 1e-3) / 1e9, 1)
        results[name] = r
        log(f"{name}: {r['us_per_launch']} us/launch, {r['gbs']} GB/s "
            f"({100 * r['frac_of_hbm_peak']:.1f}% of peak), {n_sets} buffer sets")
        del calls
        if wi > 0:
            del cases[name]
        torch.cuda.empty_cache()

    head = names[0]
    hr = results[head]
    if hasattr(cases[head], "x") and head != "inplace_f32_1x16x2x64":
        gus = graph_replay_us(torch, ra, cases[head], hr["buffer_sets"])
        hr["graph_replay"] = {"us_per_launch": round(gus, 3),
                              "gbs": round(cases[head].algo_bytes / gus / 1e3, 1)}
        log(f"{head} replayed from one HIP graph: {gus:.3f} us/launch")
    floor_us = launch_floor_us(torch, ra, W, dev, cyc)
    ideal_us = hr["algo_bytes_per_launch"] / (HBM_PEAK_GBS * 1e3)
    log(f"launch floor {floor_us:.3f} us: the headline could reach at most "
        f"{100 * ideal_us / (floor_us + ideal_us):.1f}% of peak per launch")
    ceiling = copy_ceiling_gbs(torch)
    same = copy_same_bytes(torch, hr["algo_bytes_per_launch"], cyc)
    log(f"copy of the headline's bytes: {same['us']} us, {same['gbs']} GB/s")
    log(f"device-to-device copy: {ceiling:.0f} GB/s")
    out = {
        "metric": "achieved HBM GB/s (and % of peak) + tokens/sec for RoPE apply on one MI355X",
        "value": hr["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": hr["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(hr["us_per_launch"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) activations, RoPE angle tables theta=10000)",
        "config": {"workload": hr["workload"], "tokens": cases[head].tokens,
                   "algo_bytes_per_step": hr["algo_bytes_per_launch"],
                   "buffer_sets": hr["buffer_sets"], "name": head},
        "tokens_per_s": hr["tokens_per_s"],
        "roofline": {"bound": "hbm", "achieved": hr["gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": hr["frac_of_hbm_peak"],
                     "traffic": traffic_for(head), "kernel": hr["kernel"]},
        "graph_replay": hr.get("graph_replay"),
        # the cost of one launch (a one-row launch back to back) and what it leaves of the peak
        # for the headline's bytes: floor + bytes at the full 8 TB/s
        "launch_floor": {"us": round(floor_us, 3),
                         "headline_frac_ceiling": round(ideal_us / (floor_us + ideal_us), 4)},
        "kernels": {k: v for k, v in results.items() if k != head},
        "copy_ceiling_gbs": round(ceiling, 1),
        "copy_same_bytes": same,
        "kernel_code_sha256_16": kernel_code_hash(),
    }
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle for ~{args.cpu_budget_s:.0f} s")
        out["cpu_baseline"] = cpu_baseline(cases[head], args.cpu_budget_s)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
