#!/usr/bin/env python3
"""Benchmark of the RoPE apply path on one MI355X: achieved HBM GB/s (and fraction of the
8 TB/s peak) and tokens/s.

One step is one launch of the headline workload, the largest single-GPU configuration: the
cos/sin-cache op in GPT-J style, fp16, 32768 tokens, q and k [32768, 32*128], rotaryDim 64 of
headSize 128 (the other 64 dims copied through), cache [65536, 64] (1078 MB per launch).  The
other configurations (the in-place op on fp32 [1,16,2,64] and on bf16 [8,4096,1,576] with a
[512,576) slice; the cache op in rope NeoX bf16 and mrope [16,24,24] bf16) and extra workloads
(the in-place gradient, half mode, the multi-head in-place shape, interleaved mrope stitching,
a 768 MiB fp32 in-place launch) are timed the same way and reported under `kernels`.

Timing: inputs are resident in HBM; launches cycle over enough copies of the inputs that
every pass touches >= 2 GiB before a buffer is reused, so that MI355X's 256 MB Infinity Cache
holds none of a buffer set's lines when it comes round again; the host queues the timed
launches behind a short GPU spin so that they run back to back, and two HIP events on the
launch stream bracket exactly `steps` launches.

Beside each kernel: per-launch percentiles (each launch between its own pair of events, in a
separate pass), the per-launch time of the same launches replayed from one captured HIP graph
(in-place workloads), a measured ceiling that does the same memory traffic with no arithmetic
(bench_ceiling.hip: the in-place access pattern, or a dense copy of the cache op's bytes), and
the CPU oracle's rate on the same workload at 1 thread and on all usable host cores.  One
JSON line on stdout; progress goes to stderr.

Other modes (each one JSON line instead of the benchmark line): --sweep (the same kernels at
growing sizes, fixed cost + marginal rate), --latency (decode-size launches of both ops),
--patterns (the strided-slice and NeoX pair-unit access patterns against dense ones),
--calibrate (copies of known size for scaling the HBM byte counters of a profiled run).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import platform
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
# Bytes touched between reuses of one buffer set.  At 512 MiB, lines of a set were still in
# the Infinity Cache at its next use (the in-place kernel measured 2-3% faster, a
# write-through variant of it 7-10%); from 1 GiB to 2 GiB the times are equal, and much
# larger rotations start to add TLB misses of their own.
MALL_DEFEAT_BYTES = 2 << 30
# The sources that decide what a launch does: the kernels and the launch plans (which kernel,
# grid and layout a workload gets).
KERNEL_SOURCES = [os.path.join(ROOT, "rope_partial_inplace_amd", "csrc", f)
                  for f in ("rope_kernels.hip", "rope_plan.h", "rope_plan.cpp")]
CEILING_SRC = os.path.join(ROOT, "bench_ceiling.hip")
CEILING_LIB = os.path.join(ROOT, "libbench_ceiling.so")
HEADLINE = "cache_rope_gptj_f16_t32768_rd64"
WORKLOADS = [HEADLINE, "inplace_bf16_8x4096x1x576_s512", "inplace_f32_1x16x2x64",
             "cache_rope_neox_bf16_t8192", "cache_mrope_neox_bf16_t16384",
             "inplace_backward_bf16_8x4096x1x576_s512", "cache_mrope_interleaved_neox_bf16_t16384",
             "inplace_half_bf16_8x4096x1x576_s512", "inplace_heads_bf16_4x2048x32x192_s128_bs1d",
             "inplace_f32_1x524288x2x64"]


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_code_hash() -> str:
    """sha256[:16] of the kernel and launch-plan sources with their // comments, trailing
    blanks and blank lines removed: it changes when their code does, not when a comment is
    edited, so a traffic figure stays attached to the code it was measured on."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, encoding="utf-8") as f:
            lines = [re.sub(r"//.*$", "", line).rstrip() for line in f.read().splitlines()]
        h.update(os.path.basename(path).encode() + b"\0")
        h.update("\n".join(x for x in lines if x).encode() + b"\0")
    return h.hexdigest()[:16]


def build_ceiling(verbose: bool = False) -> str:
    """Compile bench_ceiling.hip (gfx950) into libbench_ceiling.so beside this file."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = [os.path.join(rocm, "bin", "hipcc"), "--offload-arch=gfx950", "-mcode-object-version=5",
           "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
           CEILING_SRC, "-o", CEILING_LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(CEILING_LIB + ".tmp", CEILING_LIB)
    return CEILING_LIB


def load_ceiling():
    if not os.path.exists(CEILING_LIB):
        raise SystemExit(f"{CEILING_LIB} is missing: build it first (python __graft_entry__.py)")
    lib = ctypes.CDLL(CEILING_LIB)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.ceiling_copy.argtypes = [vp, vp, i64, vp]
    lib.ceiling_copy.restype = ctypes.c_int
    lib.ceiling_rows.argtypes = [vp, i64, i64, i64, i64, i64, i64, vp, vp, i64, i64, ctypes.c_int,
                                 vp]
    lib.ceiling_rows.restype = ctypes.c_int
    lib.ceiling_pairs.argtypes = [vp, vp, i64, i64, i64, vp]
    lib.ceiling_pairs.restype = ctypes.c_int
    return lib


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


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


def _host_ms_per_launch(torch, calls, n):
    t0 = time.perf_counter()
    for i in range(n):
        calls[i % len(calls)]()
    ms = (time.perf_counter() - t0) * 1e3 / n
    torch.cuda.synchronize()
    return ms


def time_launches(torch, calls, steps: int, warmup: int, cyc_per_ms: float):
    """Mean GPU time per launch (ms) over `steps` back-to-back launches cycling over calls."""
    n = len(calls)
    for i in range(warmup):
        calls[i % n]()
    torch.cuda.synchronize()
    host_ms = _host_ms_per_launch(torch, calls, min(steps, 20))  # sizes the spin
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


def launch_percentiles(torch, calls, steps: int, cyc_per_ms: float) -> dict:
    """p10 / median / p90 of single launches, each between its own pair of events (queued
    behind a spin so they run back to back; the events add a little to short launches)."""
    n = len(calls)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    host_ms = _host_ms_per_launch(torch, calls, min(steps, 20))
    torch.cuda._sleep(int((1.0 + 2.0 * host_ms * steps) * cyc_per_ms))
    ev[0].record()
    for i in range(steps):
        calls[i % n]()
        ev[i + 1].record()
    torch.cuda.synchronize()
    d = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps))

    def q(p):
        return round(d[min(len(d) - 1, int(p * (len(d) - 1) + 0.5))], 3)
    return {"p10_us": q(0.1), "median_us": q(0.5), "p90_us": q(0.9), "launches": steps}


def graph_replay_us(torch, ra, case, sets, reps: int = 3) -> float:
    """Per-launch time of the in-place op when its launches over the buffer sets (at least 32
    launches, cycling over the sets) are captured in one HIP graph and the graph is replayed
    back to back.  A serving loop that replays a captured graph pays this per-launch cost
    instead of the stream-launch one."""
    fn = ra.rope_partial_inplace_backward if case.backward else ra.rope_partial_inplace
    order = [sets[i % len(sets)] for i in range(max(len(sets), 32))]  # >= 32 launches a graph

    def launches():
        for x, c, sn in order:
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
    ms = start.elapsed_time(end) / (reps * len(order))
    del g
    torch.cuda.empty_cache()
    return ms * 1e3


def launch_floor_us(torch, ra, W, dev, cyc) -> float:
    """Per-launch time of the smallest in-place launch (one row of 64 fp32 elements, one
    workgroup) issued back to back: the cost of a launch itself on this GPU and runtime."""
    case = W.inplace_case("floor", 1, 1, 1, 64, torch.float32, torch.float32, [0, 64], seed=7,
                          device=dev)
    calls = inplace_calls(ra, case, 1)
    return time_launches(torch, calls, 200, 20, cyc) * 1e3


def copy_calls(torch, lib, moved: int, max_sets: int = 1 << 16):
    """Dense copies (bench_ceiling's copy kernel) that read and write `moved` bytes in all,
    over enough buffer pairs to rotate through MALL_DEFEAT_BYTES (at most max_sets pairs)."""
    half = max(16, (moved // 2) // 16 * 16)
    n_sets = min(max_sets, max(1, math.ceil(MALL_DEFEAT_BYTES / (2 * half))))
    pairs = [(torch.empty(half, dtype=torch.uint8, device="cuda"),
              torch.empty(half, dtype=torch.uint8, device="cuda")) for _ in range(n_sets)]
    stream = torch.cuda.current_stream().cuda_stream

    def one(a, b):
        st = lib.ceiling_copy(b.data_ptr(), a.data_ptr(), half, stream)
        if st != 0:
            raise RuntimeError(f"ceiling_copy failed ({st})")
    return [(lambda a=a, b=b: one(a, b)) for a, b in pairs], pairs, 2 * half


def copy_ceiling(torch, lib, moved: int, cyc: float, steps: int = 50,
                 max_sets: int = 1 << 16) -> dict:
    calls, pairs, nbytes = copy_calls(torch, lib, moved, max_sets)
    ms = time_launches(torch, calls, steps, 5, cyc)
    out = {"bytes": nbytes, "us": round(ms * 1e3, 3), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "buffer_sets": len(pairs)}
    del calls, pairs
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------------------------------
# workloads
# ------------------------------------------------------------------------------------------

# Workloads reported beside the configurations, with what they show.
EXTRA = {"inplace_f32_1x524288x2x64":
         "scaled variant of the fp32 [1,16,2,64] workload (same dtype, slice and BS1D layout, "
         "S = 524288): the kernel's streaming rate at 768 MiB per launch"}


def n_sets_for(algo_bytes: int) -> int:
    return max(1, math.ceil(MALL_DEFEAT_BYTES / algo_bytes))


def inplace_sets(case, n_sets):
    """(x, cos, sin) per buffer set; set 0 is the case's own tensors."""
    sets = []
    for i in range(n_sets):
        if i == 0:
            sets.append((case.x, case.cos, case.sin))
        else:
            sets.append((case.x.clone(), case.cos.clone(), case.sin.clone()))
    return sets


def inplace_calls(ra, case, n_sets, sets=None):
    sets = sets or inplace_sets(case, n_sets)
    return [ra.prepare_partial_inplace(x, c, s, case.rotary_mode, case.partial_slice,
                                       backward=case.backward) for x, c, s in sets]


def cache_calls(ra, torch, case, n_sets):
    """Launches over n_sets copies of every input, the cos/sin table included: a table shared
    by the sets would stay in the Infinity Cache between launches (4% faster on the rope NeoX
    workload), which a model's per-layer calls, with weights streaming in between, do not see."""
    calls = []
    for i in range(n_sets):
        q = case.query if i == 0 else case.query.clone()
        k = case.key if i == 0 else case.key.clone()
        p = case.positions if i == 0 else case.positions.clone()
        c = case.cache if i == 0 else case.cache.clone()
        qo, ko = torch.empty_like(q), torch.empty_like(k)
        calls.append(ra.prepare_with_cos_sin_cache(p, q, k, c, case.mrope_section,
                                                   case.head_size, case.is_neox, qo, ko,
                                                   cache_mode=case.cache_mode))
    return calls


def inplace_pattern(case) -> dict:
    """The in-place kernel's memory traffic as bench_ceiling's row pattern: the slice of each
    x row in lanes of the kernel's x width (16 bytes for the wider of x and cos/sin, so 8 bytes
    of bf16/f16 x beside float32 cos/sin); with cos/sin shared by the heads of a (b, s), a lane
    takes its chunk in 4 or 2 consecutive heads (the larger that divides N and keeps a lane's
    x bytes at 32 or less, the in-place kernel's rule) and loads the cos/sin chunk once; one cos
    and one sin row per (b, s) (BS1D) or per row (BSND)."""
    B, S, N, D = case.x.shape
    xs, cs = case.x.element_size(), case.cos.element_size()
    start, end = case.partial_slice if case.partial_slice else (0, D)
    L = end - start
    assert tuple(case.cos.shape[:2]) == (B, S) and case.cos.shape[2] in (1, N)
    per_head = case.cos.shape[2] == N
    lane = (16 // max(xs, cs)) * xs
    rpl = 1
    if not per_head and N > 1:
        rpl = next((c for c in (4, 2) if N % c == 0 and c * lane <= 32), 1)
    return {"rows": B * S * N, "row_bytes": D * xs, "off": start * xs, "len": L * xs,
            "lane_bytes": lane, "rows_per_lane": rpl, "side_bytes": L * cs,
            "rows_per_side": 1 if per_head else N, "side_stream": int(per_head or N == rpl)}


def pattern_calls(torch, lib, case, sets):
    pat = inplace_pattern(case)
    stream = torch.cuda.current_stream().cuda_stream

    def one(x, c, s):
        st = lib.ceiling_rows(x.data_ptr(), pat["rows"], pat["row_bytes"], pat["off"], pat["len"],
                              pat["lane_bytes"], pat["rows_per_lane"], c.data_ptr(), s.data_ptr(),
                              pat["side_bytes"], pat["rows_per_side"], pat["side_stream"], stream)
        if st != 0:
            raise RuntimeError(f"ceiling_rows rejected {pat} ({st})")
    return [(lambda x=x, c=c, s=s: one(x, c, s)) for x, c, s in sets]


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
    """Measured HBM bytes per launch from the committed PMC summary, when it was taken on
    the current kernel and launch-plan sources (kernel_code_hash); else None."""
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

def _host_copies(case):
    """Host copies of a workload's inputs (outside any timed region) and the function that
    runs the oracle, unchanged, over token block [lo, hi) of them."""
    import torch
    import oracle
    if hasattr(case, "x"):
        B, S, N, D = case.x.shape
        assert tuple(case.cos.shape[:2]) == (B, S), "the CPU baseline needs per-(b, s) cos/sin"
        x = case.x.cpu().reshape(B * S, 1, N, D).contiguous()
        c = case.cos.cpu().reshape(B * S, 1, case.cos.shape[2], case.cos.shape[3]).contiguous()
        s = case.sin.cpu().reshape(B * S, 1, case.sin.shape[2], case.sin.shape[3]).contiguous()
        fn = oracle.rope_partial_inplace_backward if case.backward else \
            oracle.rope_partial_inplace

        def run(lo, hi):
            st, _ = fn(x[lo:hi], c[lo:hi], s[lo:hi], case.rotary_mode, case.partial_slice)
            assert st == 0, oracle.last_error()
        return B * S, run
    pos = case.positions.cpu()
    q, k, cache = case.query.cpu(), case.key.cpu(), case.cache.cpu()
    qo, ko = torch.empty_like(q), torch.empty_like(k)

    def run(lo, hi):
        p = pos[lo:hi] if pos.dim() == 1 else pos[:, lo:hi]
        st, _, _ = oracle.rope_with_cos_sin_cache(p, q[lo:hi], k[lo:hi], cache,
                                                  case.mrope_section, case.head_size,
                                                  case.is_neox, qo[lo:hi], ko[lo:hi],
                                                  cache_mode=case.cache_mode)
        assert st == 0, oracle.last_error()
    return case.tokens, run


def _oracle_rate(tokens, run, algo_bytes, threads: int, budget_s: float):
    """Run the oracle (single-threaded C) over the whole batch again and again for about
    budget_s from `threads` host threads at once, each on its own block of tokens; ctypes
    releases the GIL during each call.  Returns (bytes/s, tokens/s, passes, seconds)."""
    import threading
    edges = [tokens * k // threads for k in range(threads + 1)]
    done = [0.0] * threads
    stop = threading.Event()

    def work(k):
        lo, hi = edges[k], edges[k + 1]
        while not stop.is_set() and hi > lo:
            run(lo, hi)
            done[k] += (hi - lo) / tokens

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
    return algo_bytes * passes / el, tokens * passes / el, passes, el


def cpu_baseline(case, budget_s: float, budget1_s: float) -> dict:
    """The oracle as it stands on the host: on all the cores this process may use (up to 16,
    the host share of one GPU; at most one thread per 512 tokens, since a thread with a handful
    of tokens per call measures the call overhead), and on one thread."""
    tokens, run = _host_copies(case)
    cores = max(1, min(16, len(os.sched_getaffinity(0)), tokens // 512))
    bps, tps, passes, el = _oracle_rate(tokens, run, case.algo_bytes, cores, budget_s)
    bps1, tps1, passes1, el1 = _oracle_rate(tokens, run, case.algo_bytes, 1, budget1_s)
    return {
        "value": round(bps / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"the whole batch ({tokens} tokens) passed {passes:.2f} times in {el:.1f} s "
                   f"through the single-threaded C oracle, run from {cores} host threads at "
                   f"once, each on its own block of tokens"),
        "tokens_per_s": round(tps, 1),
        "single_thread": {"value": round(bps1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                          "tokens_per_s": round(tps1, 1),
                          "sample": f"{passes1:.2f} passes over the batch in {el1:.1f} s"},
    }


# ------------------------------------------------------------------------------------------

def read_write_bytes(case) -> tuple[int, int]:
    """Algorithmic bytes a launch reads and writes: the in-place op writes its slice back,
    the cache op writes whole q/k rows; everything else is read."""
    if hasattr(case, "x"):
        B, S, N, D = case.x.shape
        start, end = case.partial_slice if case.partial_slice else (0, D)
        written = B * S * N * (end - start) * case.x.element_size()
    else:
        written = (case.query.numel() + case.key.numel()) * case.query.element_size()
    return case.algo_bytes - written, written


def calibrate(torch, lib, W, dev, cyc, names):
    """For each workload, a dense copy (bench_ceiling's copy kernel) that reads as many bytes
    as the workload's launch does (and writes as many), 20 launches each, in workload order:
    what FETCH_SIZE and WRITE_SIZE read for a copy of known size at that size scales the
    workload's own readings.  Prints one JSON line."""
    out = []
    for name in names:
        case = W.CONFIGS[name](dev)
        rd, wr = read_write_bytes(case)
        del case
        torch.cuda.empty_cache()
        r = copy_ceiling(torch, lib, 2 * rd, cyc, steps=20, max_sets=256)
        r.update(workload=name, read_bytes=r["bytes"] // 2, workload_read_bytes=rd,
                 workload_write_bytes=wr)
        out.append(r)
        log(f"copy for {name}: {r['read_bytes']} B read, {r['us']} us")
    print(json.dumps({"calibration_copies": out}), flush=True)


def single_launch_us(torch, call, reps: int = 50) -> dict:
    """Latency of one launch issued to an idle GPU: events around each launch, the GPU
    synchronized between launches (median and p90 over `reps`)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d = []
    for _ in range(reps + 5):
        torch.cuda.synchronize()
        a.record()
        call()
        b.record()
        torch.cuda.synchronize()
        d.append(a.elapsed_time(b) * 1e3)
    d = sorted(d[5:])
    return {"median_us": round(d[len(d) // 2], 3), "p90_us": round(d[int(0.9 * (len(d) - 1))], 3)}


def graph_calls_us(torch, make_call, n_sets: int, reps: int = 5) -> float:
    """Per-launch time of `max(n_sets, 32)` launches captured in one HIP graph and replayed
    back to back; make_call(i) issues launch i on the current stream (called during capture)."""
    order = list(range(max(n_sets, 32)))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in order:
            make_call(i % n_sets)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in order:
            make_call(i % n_sets)
    g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    del g
    return s.elapsed_time(e) * 1e3 / (reps * len(order))


def latency(torch, ra, W, dev, cyc) -> dict:
    """Decode-size launches: the in-place op on bf16 x [B,1,32,128] with f32 BS1D tables and the
    cache op in rope NeoX bf16 (32 + 8 heads of 128, cache [32768,128]) at 1-1024 tokens: the
    per-launch time of launches run back to back (stream and graph replay) and the latency of
    one launch on an idle GPU."""
    out = {"inplace_rope_kernel": [], "cos_sin_cache_wave_kernel": []}
    for t in (1, 8, 64, 256, 1024):
        case = W.inplace_case("lat", t, 1, 32, 128, torch.bfloat16, torch.float32, [0, 128],
                              seed=1300 + t, device=dev)
        n = n_sets_for(case.algo_bytes)
        sets = inplace_sets(case, min(n, 256))
        calls = inplace_calls(ra, case, len(sets), sets)
        b2b = time_launches(torch, calls, 200, 20, cyc) * 1e3
        one = single_launch_us(torch, calls[0])
        gus = graph_calls_us(torch, lambda i: ra.rope_partial_inplace(
            sets[i][0], sets[i][1], sets[i][2], 1, [0, 128]), len(sets))
        out["inplace_rope_kernel"].append({"tokens": t, "bytes": case.algo_bytes,
                                           "back_to_back_us": round(b2b, 3),
                                           "graph_replay_us": round(gus, 3), "single": one})
        log(f"latency in-place {t} tokens: {b2b:.3f} us back to back, {one['median_us']} us alone")
        del calls, sets, case
        cc = W.cache_case("lat", t, 32, 8, 128, 128, torch.bfloat16, True, 32768,
                          seed=1400 + t, device=dev)
        n = min(n_sets_for(cc.algo_bytes), 256)
        calls = cache_calls(ra, torch, cc, n)
        b2b = time_launches(torch, calls, 200, 20, cyc) * 1e3
        one = single_launch_us(torch, calls[0])
        qs = [cc.query.clone() for _ in range(n)]
        ks = [cc.key.clone() for _ in range(n)]
        outs = [(torch.empty_like(q), torch.empty_like(k)) for q, k in zip(qs, ks)]
        gus = graph_calls_us(torch, lambda i: ra.rope_with_cos_sin_cache(
            cc.positions, qs[i], ks[i], cc.cache, None, 128, True, outs[i][0], outs[i][1]), n)
        out["cos_sin_cache_wave_kernel"].append({"tokens": t, "bytes": cc.algo_bytes,
                                                 "back_to_back_us": round(b2b, 3),
                                                 "graph_replay_us": round(gus, 3),
                                                 "single": one})
        log(f"latency cache {t} tokens: {b2b:.3f} us back to back, {one['median_us']} us alone")
        del calls, qs, ks, outs, cc
        torch.cuda.empty_cache()
    floor = launch_floor_us(torch, ra, W, dev, cyc)
    fcase = W.inplace_case("floor", 1, 1, 1, 64, torch.float32, torch.float32, [0, 64], seed=7,
                           device=dev)
    floor_one = single_launch_us(torch, inplace_calls(ra, fcase, 1)[0])
    return {"latency": out, "launch_floor_us": round(floor, 3),
            # the same single-launch measurement for the one-row launch: what the events, an
            # idle GPU's wake-up and a minimal kernel cost before any of the work above
            "launch_floor_single": floor_one,
            "kernel_code_sha256_16": kernel_code_hash()}


def patterns(torch, ra, W, lib, dev, cyc) -> dict:
    """The memory-side costs the design notes attribute to two layouts, measured with the
    no-arithmetic kernels of bench_ceiling.hip beside the RoPE kernels on the same shapes:
      - the strided slice: bf16 x [128,4096,1,576] with slice [512,576) (128 B of every 1152)
        against dense rows with the same bytes, x [128,4096,1,64] (403 MB each, f32 BS1D
        tables): the in-place kernel and its access pattern on each;
      - the NeoX pair units: a copy of the rope NeoX workload's q and k rows (8192 tokens x 40
        heads of 256 B) in the pair-unit layout (two 16-byte vectors half a head apart per
        lane; one head row per lane, as the kernel takes it, and two), against a dense copy of
        the same bytes, beside the cache kernel on that workload."""
    out = {}
    rows = {}
    for tag, D, sl in (("strided_1152B_rows", 576, [512, 576]), ("dense_128B_rows", 64, [0, 64])):
        case = W.inplace_case(tag, 128, 4096, 1, D, torch.bfloat16, torch.float32, sl,
                              seed=1500 + D, device=dev)
        sets = inplace_sets(case, n_sets_for(case.algo_bytes))
        k_ms = time_launches(torch, inplace_calls(ra, case, len(sets), sets), 50, 5, cyc)
        p_ms = time_launches(torch, pattern_calls(torch, lib, case, sets), 50, 5, cyc)
        rows[tag] = {"workload": describe_case(tag, case), "bytes": case.algo_bytes,
                     "kernel_us": round(k_ms * 1e3, 3),
                     "kernel_gbs": round(case.algo_bytes / (k_ms * 1e-3) / 1e9, 1),
                     "pattern_us": round(p_ms * 1e3, 3),
                     "pattern_gbs": round(case.algo_bytes / (p_ms * 1e-3) / 1e9, 1)}
        log(f"{tag}: kernel {k_ms * 1e3:.2f} us, pattern {p_ms * 1e3:.2f} us")
        del sets, case
        torch.cuda.empty_cache()
    out["strided_slice"] = rows
    case = W.CONFIGS["cache_rope_neox_bf16_t8192"](dev)
    k_ms = time_launches(torch, cache_calls(ra, torch, case, n_sets_for(case.algo_bytes)), 50, 5,
                         cyc)
    heads = case.tokens * (case.query.shape[1] + case.key.shape[1]) // case.head_size
    head_bytes = case.head_size * case.query.element_size()
    nbytes = heads * head_bytes
    n_sets = max(1, math.ceil(MALL_DEFEAT_BYTES / (2 * nbytes)))
    bufs = [(torch.empty(nbytes, dtype=torch.uint8, device=dev),
             torch.empty(nbytes, dtype=torch.uint8, device=dev)) for _ in range(n_sets)]
    stream = torch.cuda.current_stream().cuda_stream

    def pair_call(a, b, k):
        st = lib.ceiling_pairs(b.data_ptr(), a.data_ptr(), heads, head_bytes, k, stream)
        if st != 0:
            raise RuntimeError(f"ceiling_pairs failed ({st})")
    res = {"workload": describe_case("cache_rope_neox_bf16_t8192", case),
           "bytes_moved": 2 * nbytes, "kernel_us": round(k_ms * 1e3, 3)}
    for k in (2, 1):
        ms = time_launches(torch, [(lambda a=a, b=b, k=k: pair_call(a, b, k)) for a, b in bufs],
                           50, 5, cyc)
        res[f"pair_copy_{k}_rows_per_lane_us"] = round(ms * 1e3, 3)
    del bufs
    torch.cuda.empty_cache()
    res["dense_copy_us"] = copy_ceiling(torch, lib, 2 * nbytes, cyc)["us"]
    log(f"neox pairs: kernel {res['kernel_us']} us, pair copy {res['pair_copy_2_rows_per_lane_us']}"
        f" us, dense copy {res['dense_copy_us']} us")
    out["neox_pairs"] = res
    out["kernel_code_sha256_16"] = kernel_code_hash()
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workloads", default=",".join(WORKLOADS),
                    help="first is the headline; the rest are reported under `kernels`")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=10.0,
                    help="oracle time on all cores for the headline (others: a third of it)")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the launches only (no percentiles, graph replay or ceilings)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the benchmark line, time the [8,4096,1,576] in-place shape "
                         "and the rope NeoX cache shape at 1..16x their tokens and fit fixed cost "
                         "+ bytes / marginal bandwidth (one JSON line)")
    ap.add_argument("--latency", action="store_true",
                    help="instead of the benchmark line, time decode-size launches of both "
                         "operations (1-1024 tokens): back to back, graph replay, and one "
                         "launch on an idle GPU (one JSON line)")
    ap.add_argument("--patterns", action="store_true",
                    help="instead of the benchmark line, measure the strided-slice and NeoX "
                         "pair-unit access patterns against dense ones (one JSON line)")
    ap.add_argument("--calibrate", action="store_true",
                    help="instead of the benchmark line, run one dense copy per workload that "
                         "reads as many bytes as the workload (for scaling the HBM byte "
                         "counters of a profiled run)")
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
    lib = load_ceiling()
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} ({getattr(props, 'gcnArchName', '?')}), "
        f"{props.multi_processor_count} CUs")
    cyc = spin_cycles_per_ms(torch)
    if args.sweep:
        print(json.dumps(size_sweep(torch, ra, W, dev, cyc)), flush=True)
        return 0
    if args.latency:
        print(json.dumps(latency(torch, ra, W, dev, cyc)), flush=True)
        return 0
    if args.patterns:
        print(json.dumps(patterns(torch, ra, W, lib, dev, cyc)), flush=True)
        return 0
    names = [w.strip() for w in args.workloads.split(",") if w.strip()]
    if args.calibrate:
        calibrate(torch, lib, W, dev, cyc, names)
        return 0
    results, head_case = {}, None
    for wi, name in enumerate(names):
        case = W.CONFIGS[name](dev)
        inplace = hasattr(case, "x")
        n_sets = 1 if name == "inplace_f32_1x16x2x64" else n_sets_for(case.algo_bytes)
        sets = inplace_sets(case, n_sets) if inplace else None
        calls = inplace_calls(ra, case, n_sets, sets) if inplace else \
            cache_calls(ra, torch, case, n_sets)
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
        if not args.no_extras:
            r["per_launch"] = launch_percentiles(torch, calls, steps, cyc)
            if inplace:
                gus = graph_replay_us(torch, ra, case, sets)
                r["graph_replay"] = {"us_per_launch": round(gus, 3),
                                     "gbs": round(case.algo_bytes / gus / 1e3, 1)}
                pms = time_launches(torch, pattern_calls(torch, lib, case, sets), steps,
                                    args.warmup, cyc)
                r["ceiling"] = {"what": "the same x slice and cos/sin traffic with no "
                                        "arithmetic (bench_ceiling.hip ceiling_rows)",
                                "us_per_launch": round(pms * 1e3, 3),
                                "gbs": round(case.algo_bytes / (pms * 1e-3) / 1e9, 1)}
            else:
                cc = copy_ceiling(torch, lib, case.algo_bytes, cyc, steps=min(steps, 50))
                r["ceiling"] = {"what": "a dense copy of the same number of bytes "
                                        "(bench_ceiling.hip ceiling_copy)",
                                "us_per_launch": cc["us"], "gbs": cc["gbs"]}
            r["ceiling"]["kernel_over_ceiling"] = round(r["ceiling"]["us_per_launch"] /
                                                        r["us_per_launch"], 4)
        results[name] = r
        log(f"{name}: {r['us_per_launch']} us/launch, {r['gbs']} GB/s "
            f"({100 * r['frac_of_hbm_peak']:.1f}% of peak), {n_sets} buffer sets"
            + (f"; ceiling {r['ceiling']['us_per_launch']} us" if "ceiling" in r else ""))
        del calls, sets
        torch.cuda.empty_cache()
        if not args.no_cpu_baseline:
            budget = args.cpu_budget_s if wi == 0 else args.cpu_budget_s / 3
            log(f"{name}: timing the CPU oracle for ~{budget + max(2.0, budget / 3):.0f} s")
            r["cpu_baseline"] = cpu_baseline(case, budget, max(2.0, budget / 3))
        if wi == 0:
            head_case = case
        else:
            del case
        torch.cuda.empty_cache()

    head = names[0]
    hr = results[head]
    floor_us = launch_floor_us(torch, ra, W, dev, cyc)
    ideal_us = hr["algo_bytes_per_launch"] / (HBM_PEAK_GBS * 1e3)
    log(f"launch floor {floor_us:.3f} us: the headline could reach at most "
        f"{100 * ideal_us / (floor_us + ideal_us):.1f}% of peak per launch")
    ceiling = copy_ceiling(torch, lib, 1 << 30, cyc, steps=20)
    log(f"dense copy of 1 GiB: {ceiling['gbs']} GB/s")
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
        "config": {"workload": hr["workload"], "name": head, "tokens": head_case.tokens,
                   "algo_bytes_per_step": hr["algo_bytes_per_launch"],
                   "buffer_sets": hr["buffer_sets"]},
        "tokens_per_s": hr["tokens_per_s"],
        "roofline": {"bound": "hbm", "achieved": hr["gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": hr["frac_of_hbm_peak"],
                     "traffic": hr["traffic"], "kernel": hr["kernel"]},
        "per_launch": hr.get("per_launch"),
        "ceiling": hr.get("ceiling"),
        # the cost of one launch (a one-row launch back to back) and what it leaves of the peak
        # for the headline's bytes: floor + bytes at the full 8 TB/s
        "launch_floor": {"us": round(floor_us, 3),
                         "headline_frac_ceiling": round(ideal_us / (floor_us + ideal_us), 4)},
        "kernels": {k: v for k, v in results.items() if k != head},
        "copy_ceiling_1gib": ceiling,
        "kernel_code_sha256_16": kernel_code_hash(),
        "cpu_baseline": None,
    }
    if "cpu_baseline" in hr:
        cb = dict(hr["cpu_baseline"])
        cb["host_cpu"] = host_cpu_model()
        cb["host_cores_visible"] = len(os.sched_getaffinity(0))
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
