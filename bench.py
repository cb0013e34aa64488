#!/usr/bin/env python3
"""Benchmark of the capacity-padded, permute-free MoE FFN forward on one MI355X.

One step = the whole forward (top-K routing + capacity selection + align in
one call, gather-in-GEMM FC1+SwiGLU, FC2, gather-combine) over one batch of seeded
synthetic inputs already resident in HBM, replayed from one captured
hipGraph.  Prints ONE JSON line on stdout; progress goes to stderr.

Timed regions (all on the stream the library launches on):
  1. K graph replays between two HIP events -> ms_per_step, value.
  2. K eager forwards queued back to back, a HIP event between consecutive
     C-ABI calls ->
     average duration of each call's kernels (route+capacity+align, FC1,
     FC2, combine) -> TFLOP/s, GB/s and the roofline of the dominant kernel
     (FC1): HBM-bound at this shape (arithmetic intensity below the ridge).
  3. cpu_baseline: the CPU oracle on the same inputs (median of a few full
     forwards), rank 0 only.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--variant capacity|dropless|backward]

--variant dropless measures the dropless form instead (every route kept,
block-padded segments, the extent a device scalar): its own JSON line, with
the algorithmic work taken at the real padded extent.  --variant backward
measures the layer's training step (forward keeping the pre-activation, then
the backward for a seeded dy), with the roofline of the slowest backward
kernel; with --main-grad the weight gradients are added into float32 main
gradients instead of written as bf16.  --variant serving measures variable-N serving of the dropless form
from a ladder of captured bucket graphs against one graph at the worst-case
shape and against eager launches (a seeded stream of item sizes).
--variant ep-local measures the grouped FFN on one expert-parallel rank's
share (--ep, default 8): E/ep experts with C*ep received rows each.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed tokens/s + grouped-GEMM TFLOP/s (% bf16 MFMA peak), MoE FFN fwd, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_fc1_swiglu_qwen3_30b_a3b.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the FFN kernel's sources (the kernel file and the headers it
    includes): counter summaries taken on other code are void."""
    h = hashlib.sha256()
    for f in ("grouped_ffn.hip", "slot_gemm.h", "gemm_common.h", "moe_common.h"):
        h.update(open(os.path.join(ROOT, "mixture_experts_expert_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def provenance(torch) -> dict:
    """What produced the numbers: a hash of every library source, the commit
    when the tree is a git checkout, and the ROCm / torch / device it ran on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_expert_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    h.update(open(os.path.join(ROOT, "include", "moe_native.h"), "rb").read())
    git = None
    if os.path.isdir(os.path.join(ROOT, ".git")):
        try:
            git = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                                 text=True, timeout=10).stdout.strip() or None
        except (OSError, subprocess.SubprocessError):
            git = None
    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        rocm = None
    props = torch.cuda.get_device_properties(0)
    return {"source_sha": h.hexdigest()[:16], "git_sha": git, "rocm": rocm, "hip": torch.version.hip,
            "torch": torch.__version__, "device": props.name,
            "arch": getattr(props, "gcnArchName", None)}


def algorithmic_bytes(w, C, Cp, kept):
    """Bytes each call must move at least once (read + write), per forward."""
    N, H, I, E, K = w.N, w.H, w.I, w.E, w.K
    R = E * Cp
    return {
        # logits in; top-K ids/probs out and back in; route_slot, counts, the
        # route list, its inverse and the per-token counts out
        "route_capacity_align": N * E * 4 + N * K * (4 + 4) * 2 + N * K * 4 + E * 4
                                + R * 8 + (R // 32) * 4 + E * 4 + N * K * 4 + N * 4 + 4,
        "fc1": E * 2 * I * H * 2 + N * H * 2 + R * 8 + R * I * 2,
        "fc2": E * H * I * 2 + R * I * 2 + R * H * 2,
        "combine": kept * H * 2 + N * K * 4 + N * H * 2,
    }


def algorithmic_bytes_dropless(w, X, Rd, BM):
    """The same for the dropless form, whose FFN rows are the real padded
    extent X (every route kept); Rd is the static bound of the route list."""
    N, H, I, E, K = w.N, w.H, w.I, w.E, w.K
    return {
        # logits in; top-K ids/probs out and back in; per-route rank and
        # per-expert counts; the route list to the extent, the block tags,
        # block starts, the inverse, the per-token counts and the extent out
        "route_dropless": N * E * 4 + N * K * (4 + 4) * 2 + N * K * 4 * 2 + E * 4 * 2
                          + X * 8 + (Rd // BM) * 4 + E * 4 + N * K * 4 + N * 4 + 4,
        "fc1": E * 2 * I * H * 2 + N * H * 2 + X * 8 + X * I * 2,
        "fc2": E * H * I * 2 + X * I * 2 + X * H * 2,
        "combine": N * K * H * 2 + N * K * 4 + N * H * 2,
    }


def pmc_traffic(workload):
    """FC1's HBM traffic per launch from the committed rocprofv3 counter summary,
    scaled by the copy-kernel calibration; None if absent, taken on other code
    or on another workload."""
    try:
        d = json.load(open(PMC_SUMMARY))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha") != kernel_source_hash() or d.get("workload") != workload:
        return None
    return int(d["fetch_bytes_per_launch"] * d["fetch_scale"] + d["write_bytes_per_launch"] * d["write_scale"])


def vendor_reference(torch, moe, w, args):
    """torch's bf16 batched matmul (hipBLASLt) on the layer's per-expert
    products, E x (Cp x 2I x H) and E x (Cp x H x I), without the gather and
    the epilogue: one JSON line of microseconds and TFLOP/s."""
    Cp = int(moe.moe_padded_capacity(moe.moe_source_capacity(w.N, w.K, w.E, w.F)))
    out = {"workload": w.name, "kind": "torch bf16 bmm (hipBLASLt), per-expert products"}
    stream = torch.cuda.Stream()
    for name, (M, N, K) in (("fc1", (Cp, 2 * w.I, w.H)), ("fc2", (Cp, w.H, w.I))):
        g = torch.Generator(device="cuda").manual_seed(7)
        a = torch.randn(w.E, M, K, generator=g, device="cuda").to(torch.bfloat16)
        b = torch.randn(w.E, K, N, generator=g, device="cuda").to(torch.bfloat16).contiguous()
        with torch.cuda.stream(stream):
            warm(lambda: torch.bmm(a, b), args.warmup, args.warmup_seconds, stream)
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(args.steps):
                torch.bmm(a, b)
            ev1.record(stream)
            stream.synchronize()
        us = ev0.elapsed_time(ev1) / args.steps * 1e3
        out[name] = {"shape": [w.E, M, N, K], "us": us, "tflops": 2.0 * w.E * M * N * K / us / 1e6}
        log(f"[bench] vendor bmm {name} {w.E}x({M}x{N}x{K}): {us:.1f} us, {out[name]['tflops']:.0f} TFLOP/s")
        del a, b
    # a large square product: what a bf16 GEMM with no gather reaches on this device
    g = torch.Generator(device="cuda").manual_seed(8)
    a = torch.randn(8192, 8192, generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randn(8192, 8192, generator=g, device="cuda").to(torch.bfloat16)
    with torch.cuda.stream(stream):
        warm(lambda: torch.mm(a, b), args.warmup, args.warmup_seconds, stream)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(args.steps):
            torch.mm(a, b)
        ev1.record(stream)
        stream.synchronize()
    us = ev0.elapsed_time(ev1) / args.steps * 1e3
    out["square_8192"] = {"shape": [1, 8192, 8192, 8192], "us": us, "tflops": 2.0 * 8192 ** 3 / us / 1e6}
    log(f"[bench] vendor mm 8192^3: {us:.1f} us, {out['square_8192']['tflops']:.0f} TFLOP/s")
    print(json.dumps(out))


def copy_rate(torch, stream, nbytes=1 << 30, reps=10):
    """GB/s of a plain device-to-device copy (read + write bytes), the HBM
    headroom the kernels are compared against."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        for _ in range(3):
            dst.copy_(src)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(reps):
            dst.copy_(src)
        ev1.record(stream)
        stream.synchronize()
    gbs = 2 * nbytes * reps / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    del src, dst
    log(f"[bench] device copy: {gbs:.0f} GB/s")
    return gbs


def hbm_probes(torch, moe, stream, nbytes=2 << 30, reps=10):
    """GB/s this device's HBM reaches for a plain streaming read, streaming
    write and copy (the library's probe kernels, 2 GiB buffers; bytes moved:
    read and write count once, the copy twice).  These are the measured
    ceilings the layer's kernels are set against; the published 8 TB/s is
    nominal."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    calls = {"read": (lambda: moe.moe_probe_read(src, sink, stream), nbytes),
             "write": (lambda: moe.moe_probe_write(dst, stream), nbytes),
             "copy": (lambda: moe.moe_probe_copy(src, dst, stream), 2 * nbytes)}
    out = {}
    with torch.cuda.stream(stream):
        moe.moe_probe_write(src, stream)
        for name, (fn, moved) in calls.items():
            for _ in range(3):
                fn()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(reps):
                fn()
            ev1.record(stream)
            stream.synchronize()
            out[name] = moved * reps / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    del src, dst, sink
    log("[bench] HBM probes GB/s: " + ", ".join(f"{k} {v:.0f}" for k, v in out.items()))
    return out


def compute_probes(torch, moe, stream, reps=5):
    """What a compute unit's matrix cores and LDS reach with nothing else in
    the way (the library's matrix-core and LDS-read probes, one workgroup per
    compute unit): the bf16 MFMA rate and the engine clock it runs at, and
    the LDS read bytes per engine clock per compute unit.  The matrix-core
    rate is the attainable one on this device: under full MFMA load the
    engine clock drops below the 2.4 GHz the published peak assumes."""
    groups = torch.cuda.get_device_properties(0).multi_processor_count
    clocks = torch.zeros(2 * groups, dtype=torch.int64, device="cuda")
    out = {}
    with torch.cuda.stream(stream):
        for name, fn, iters in (("mfma", moe.moe_probe_mfma_rate, 10000), ("lds", moe.moe_probe_lds_read, 10000)):
            for _ in range(2):
                fn(groups, iters, clocks, stream)
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(reps):
                fn(groups, iters, clocks, stream)
            ev1.record(stream)
            stream.synchronize()
            sec = ev0.elapsed_time(ev1) * 1e-3 / reps
            c = clocks.view(groups, 2).double().cpu()
            ghz = float((c[:, 0] / c[:, 1]).median()) * 0.1
            if name == "mfma":
                flops = groups * 8 * 4 * iters * 32768.0
                out["mfma_tflops"] = flops / sec / 1e12
                out["mfma_frac_bf16_peak"] = out["mfma_tflops"] / PEAK_BF16_TFLOPS
                out["mfma_clock_ghz"] = ghz
            else:
                per_wg = 8 * 8 * 1024.0 * iters
                out["lds_read_bytes_per_clock_per_cu"] = per_wg / float(c[:, 0].median())
                out["lds_read_tbs"] = groups * per_wg / sec / 1e12
                out["lds_clock_ghz"] = ghz
    log("[bench] compute probes: " + ", ".join(f"{k} {v:.3f}" for k, v in out.items()))
    return out


def access_order_probes(torch, moe, w, reps=10):
    """GB/s of the library's access-order probes over a buffer the size of
    the workload's W1 ([E, 2I, H] bf16, as panels of 256 rows of H*2 bytes):
    reads and writes in the order a GEMM tile walks a weight panel (pieces of
    128, 256 or 512 bytes of every row in turn) against front to back, writes
    in the order the weight-gradient GEMM's output tiles reach memory (tiles
    of 256 rows x 512 or 1024 bytes, neighbouring tiles on one XCD), and the
    GEMMs' LDS-DMA ring alone at 2-5 stages.  Prints one JSON line."""
    row = w.H * 2
    panel = 256 * row
    nbytes = (w.E * 2 * w.I * w.H * 2) // panel * panel
    nbytes -= nbytes % (1 << 20)
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    pieces = [p for p in (128, 256, 512) if row % p == 0] + [row]

    def rate(fn):
        with torch.cuda.stream(stream):
            for _ in range(3):
                fn()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(reps):
                fn()
            ev1.record(stream)
            stream.synchronize()
        return nbytes * reps / (ev0.elapsed_time(ev1) * 1e-3) / 1e9

    out = {"probe": "access_order", "workload": w.name, "buffer_bytes": nbytes, "row_bytes": row,
           "rows_per_panel": 256, "reps": reps,
           "read_gbs": {}, "write_gbs": {"nontemporal": {}, "default": {}},
           "write_tiles_gbs": {"nontemporal": {}, "default": {}}, "lds_ring_gbs": {}}
    moe.moe_probe_write(buf, stream)
    for p in pieces:
        key = "front_to_back" if p == row else str(p)
        out["read_gbs"][key] = rate(lambda: moe.moe_probe_read_pieces(buf, row, 256, p, sink, stream))
        for nt in (True, False):
            out["write_gbs"]["nontemporal" if nt else "default"][key] = rate(
                lambda: moe.moe_probe_write_pieces(buf, row, 256, p, nt, stream))
    for p in (512, 1024):
        if row % p:
            continue
        for nt in (True, False):
            out["write_tiles_gbs"]["nontemporal" if nt else "default"][str(p)] = rate(
                lambda: moe.moe_probe_write_tiles(buf, row, 256, p, nt, stream))
    for st in (2, 3, 4, 5):
        out["lds_ring_gbs"][str(st)] = rate(lambda: moe.moe_probe_lds_ring(buf, st, sink, stream))
    log("[bench] access-order probes GB/s: " + json.dumps(
        {k: out[k] for k in ("read_gbs", "write_gbs", "write_tiles_gbs", "lds_ring_gbs")}))
    print(json.dumps(out))


def gemm_loop_probe(torch, moe, w, reps=10):
    """The grouped GEMMs' K loop alone (the library's GEMM-loop probe: same
    tiles, rings and MFMA, no gather, no epilogue) at the workload's FC1 and
    FC2 shapes, with seeded random bf16 operands, beside the layer's own FC1
    and FC2 timed the same way in the same process.  Prints one JSON line."""
    Cp = moe.moe_padded_capacity(moe.moe_source_capacity(w.N, w.K, w.E, w.F))
    Cp = (Cp + 255) // 256 * 256                          # whole 256-row tiles
    shapes = {"fc1": (2 * w.I, w.H), "fc2": (w.H, w.I)}   # (N, K) of each product
    out = {"probe": "gemm_loop", "workload": w.name, "E": w.E, "Cp": Cp, "reps": reps, "shapes": {}}
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    g = torch.Generator(device="cuda").manual_seed(5)
    for name, (Nn, Kd) in shapes.items():
        a = torch.randn(w.E * Cp, Kd, generator=g, device="cuda").to(torch.bfloat16)
        b = (torch.randn(w.E, Nn, Kd, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        flops = 2.0 * w.E * Cp * Nn * Kd
        with torch.cuda.stream(stream):
            warm(lambda: moe.moe_probe_gemm_loop(a, b, w.E, Cp, sink, stream), 3, 0.5, stream)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            for _ in range(reps):
                moe.moe_probe_gemm_loop(a, b, w.E, Cp, sink, stream)
            ev[1].record(stream)
            stream.synchronize()
        us = ev[0].elapsed_time(ev[1]) * 1e3 / reps
        out["shapes"][name] = {"N": Nn, "K": Kd, "gflop": flops / 1e9, "loop_us": us,
                               "loop_tflops": flops / (us * 1e-6) / 1e12}
        del a, b
    # the layer's own FC1 and FC2 on the workload's inputs, in the same process
    import moe_inputs
    T = moe_inputs.make_tensors(w, "cuda")
    buf = moe.MoEBuffers(w.N, w.H, w.I, w.E, w.K, w.F, "cuda")
    buf.route_capacity_align(T["logits"])
    for name, fn in (("fc1", lambda: buf.fc1_swiglu(T["x"], T["w1"], stream)),
                     ("fc2", lambda: buf.fc2(T["w2"], stream))):
        with torch.cuda.stream(stream):
            warm(fn, 3, 0.5, stream)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            for _ in range(reps):
                fn()
            ev[1].record(stream)
            stream.synchronize()
        us = ev[0].elapsed_time(ev[1]) * 1e3 / reps
        rec = out["shapes"][name]
        rec["kernel_us"] = us
        rec["kernel_tflops"] = rec["gflop"] * 1e9 / (us * 1e-6) / 1e12
    log("[bench] gemm-loop probe: " + json.dumps(out["shapes"]))
    print(json.dumps(out))


def copy_calibration(torch, nbytes=1 << 30, reps=5):
    """A plain device copy of known size, for scaling the FETCH/WRITE counters."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}))


def warm(fn, steps, seconds, stream):
    """Untimed warm-up: at least `steps` calls and at least `seconds` of
    back-to-back work, so clocks and power state settle before timing (a few
    milliseconds of work leaves the first timed steps ~10% slow)."""
    t0 = time.perf_counter()
    n = 0
    while n < steps or time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        n += 10
        stream.synchronize()


def cpu_baseline(T, w, forwards, min_seconds=12.0, dropless=False):
    import numpy as np
    import moe_inputs
    import oracle
    threads, blas = blas_threads()
    lg = T["logits"].cpu().numpy()
    x = moe_inputs.bf16_bits(T["x"])
    w1 = moe_inputs.bf16_bits(T["w1"])
    w2 = moe_inputs.bf16_bits(T["w2"])
    times = []
    while len(times) < forwards or (sum(times) < min_seconds and len(times) < 20):
        t0 = time.perf_counter()
        if dropless:
            oracle.dropless_forward(lg, x, w1, w2, w.K)
        else:
            oracle.forward(lg, x, w1, w2, w.K, w.F)
        times.append(time.perf_counter() - t0)
        log(f"  oracle forward {len(times)}: {times[-1]:.2f} s")
    med = statistics.median(times)
    return {"value": w.N / med, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(times)} full {'dropless ' if dropless else ''}forwards of the {w.name} workload "
                      f"({sum(times):.1f} s in all, median {med:.2f} s), numpy float64 with {blas} BLAS"}


def time_graph(torch, step, stream, args, stats=None):
    """Capture one step as a hipGraph and time K replays between two HIP
    events on the launch stream; returns ms per step.  With `stats` (a dict),
    K more replays are timed one by one (an event pair around each) and their
    median and 90th percentile go into it, in microseconds."""
    with torch.cuda.stream(stream):
        for _ in range(3):
            step()
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        warm(graph.replay, args.warmup, args.warmup_seconds, stream)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        ev1.record(stream)
        stream.synchronize()
        wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    log(f"[bench] graph replay: {ms * 1e3:.1f} us/step (wall {wall / args.steps * 1e6:.1f} us)")
    if stats is not None:
        # Single replays, each between its own pair of events.  The timed
        # replays are queued behind untimed ones, so the host is ahead of the
        # GPU throughout and each interval holds one replay's kernels and the
        # graph's launch gap on the device, not the host's enqueue latency.
        with torch.cuda.stream(stream):
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
            for _ in range(8):
                graph.replay()
            evs[0].record(stream)
            for i in range(args.steps):
                graph.replay()
                evs[i + 1].record(stream)
            stream.synchronize()
        each = [evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(args.steps)]
        srt = sorted(each)
        q = lambda f: srt[min(len(srt) - 1, int(f * len(srt)))]     # noqa: E731
        stats.update({"interval": "device time of one replay, replays queued back to back",
                      "median": statistics.median(srt), "p90": q(0.9), "p99": q(0.99), "max": srt[-1],
                      "all": [round(v, 1) for v in each]})
        # host-inclusive latency: launch one replay and wait for it
        host = []
        with torch.cuda.stream(stream):
            for _ in range(min(args.steps, 50)):
                t0 = time.perf_counter()
                graph.replay()
                stream.synchronize()
                host.append((time.perf_counter() - t0) * 1e6)
        host.sort()
        stats["host_launch_to_done_us"] = {"median": statistics.median(host),
                                           "p90": host[min(len(host) - 1, int(0.9 * len(host)))]}
        log(f"[bench] single replays: median {stats['median']:.1f} us, p90 {stats['p90']:.1f}, "
            f"p99 {stats['p99']:.1f}, max {stats['max']:.1f}; launch-to-done on the host "
            f"{stats['host_launch_to_done_us']['median']:.1f} us")
    return ms


def time_calls(torch, names, calls, stream, args):
    """Average duration of each call's kernels: K eager steps queued back to
    back with a HIP event between consecutive calls and no host wait between
    steps, so the host runs ahead and each interval holds the call's kernels,
    not the host's launch latency."""
    def step():
        for c in calls:
            c()
    tot = {n: 0.0 for n in names}
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
           for _ in range(args.steps)]
    with torch.cuda.stream(stream):
        warm(step, args.warmup, args.warmup_seconds, stream)
        for s in range(args.steps):
            evs[s][0].record(stream)
            for i, c in enumerate(calls):
                c()
                evs[s][i + 1].record(stream)
        stream.synchronize()
    for s in range(args.steps):
        for i, n in enumerate(names):
            tot[n] += evs[s][i].elapsed_time(evs[s][i + 1])
    us = {n: tot[n] / args.steps * 1e3 for n in names}
    log("[bench] eager per-call us: " + ", ".join(f"{n} {us[n]:.1f}" for n in names))
    return us


def roofline(name, flops, nbytes, us, traffic=None, probes=None):
    """Roofline of one kernel: its bound is whichever resource needs the
    longer time at peak; `achieved` is the algorithmic work per launch over
    the launch time, against that resource's peak."""
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    gbs = nbytes / (us * 1e-6) / 1e9
    tflops = flops / (us * 1e-6) / 1e12
    common = {"kernel": name, "traffic": traffic, "algorithmic_bytes": nbytes, "flops": flops,
              "launch_us": us, "arithmetic_intensity": flops / nbytes,
              "attainable_frac": max(t_hbm, t_mfma) / (us * 1e-6)}
    if probes:
        # against what this device's HBM sustains (the probes), not the nominal peak
        common["measured_ceiling_gbs"] = {"read": probes["read"], "copy": probes["copy"]}
        common["frac_of_measured_read"] = gbs / probes["read"]
    if t_hbm >= t_mfma:
        return {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": gbs / PEAK_HBM_GBS, "mfma_tflops": tflops,
                "mfma_frac": tflops / PEAK_BF16_TFLOPS, **common}
    return {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": tflops / PEAK_BF16_TFLOPS, "hbm_gbs": gbs, "hbm_frac": gbs / PEAK_HBM_GBS, **common}


def backward_work(w, Cp, kept, main_grad=False):
    """Algorithmic work of each call of the training step (forward keeping
    the pre-activation, then the backward): (flops, bytes) per call.
    main_grad: the weight gradients are added into float32 main gradients
    (each read and written once, 8 bytes per element instead of 2)."""
    N, H, I, E, K = w.N, w.H, w.I, w.E, w.K
    R = E * Cp
    dwb = 8 if main_grad else 2
    route = N * E * 4 + N * K * (4 + 4) * 2 + N * K * 4 + E * 4 \
        + R * 8 + (R // 32) * 4 + E * 4 + N * K * 4 + N * 4 + 4
    return {
        "route_capacity_align": (0.0, route),
        # FC1 + SwiGLU, also writing the 2I pre-activation
        "fc1_save": (2.0 * R * 2 * I * H, E * 2 * I * H * 2 + N * H * 2 + R * 8 + R * I * 2 + R * 2 * I * 2),
        "fc2": (2.0 * R * H * I, E * H * I * 2 + R * I * 2 + R * H * 2),
        "combine": (0.0, kept * H * 2 + N * K * 4 + N * H * 2),
        # dy gathered (each token row once), W2 streamed, d_act written
        "fc2_dgrad": (2.0 * R * H * I, E * H * I * 2 + N * H * 2 + R * 4 + R * I * 2),
        # pre-activation and d_act in; act, d_preact, d_prob out
        "swiglu_bwd": (0.0, R * 2 * I * 2 + R * I * 2 + R * 4 + R * I * 2 + R * 2 * I * 2 + R * 4),
        "fc1_dgrad": (2.0 * R * 2 * I * H, E * 2 * I * H * 2 + R * 2 * I * 2 + R * H * 2),
        "dx_combine": (0.0, kept * H * 2 + N * K * 4 + N * H * 2),
        # dy rows once, act in, dW2 out
        "fc2_wgrad": (2.0 * R * H * I, N * H * 2 + R * 4 + R * I * 2 + E * H * I * dwb),
        "fc1_wgrad": (2.0 * R * 2 * I * H, R * 2 * I * 2 + N * H * 2 + R * 4 + E * 2 * I * H * dwb),
        "route_bwd": (0.0, N * K * (4 + 4 + 4 + 4) + N * E * 4),
    }


def bench_backward(args, w, T, torch, moe):
    """One step = the layer's training step: routing, FC1 keeping the
    pre-activation, FC2, combine, then the whole backward for a seeded dy."""
    import moe_inputs
    buf = moe.MoEBuffers(w.N, w.H, w.I, w.E, w.K, w.F, "cuda")
    bw = moe.MoEBackwardBuffers(buf, main_grad=args.main_grad)
    dy = moe_inputs.make_dy(w, "cuda")
    x, w1, w2 = T["x"], T["w1"], T["w2"]
    names = ["route_capacity_align", "fc1_save", "fc2", "combine", "fc2_dgrad", "swiglu_bwd",
             "fc1_dgrad", "dx_combine", "fc2_wgrad", "fc1_wgrad", "route_bwd"]
    calls = [lambda: buf.route_capacity_align(T["logits"]), lambda: bw.fc1_swiglu_save(x, w1),
             lambda: buf.fc2(w2), buf.combine, lambda: bw.fc2_dgrad(dy, w2), bw.swiglu_bwd,
             lambda: bw.fc1_dgrad(w1), bw.dx_combine, lambda: bw.fc2_wgrad(dy),
             lambda: bw.fc1_wgrad(x), bw.route_bwd]
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()

    def step():
        for c in calls:
            c()

    ms_per_step = time_graph(torch, step, stream, args)
    us = time_calls(torch, names, calls, stream, args)
    kept = int((buf.token_routes >= 0).sum().item())
    work = backward_work(w, buf.Cp, kept, args.main_grad)
    bwd_names = names[4:]
    dom = max(bwd_names, key=lambda n: us[n])
    gemms = ["fc1_save", "fc2", "fc2_dgrad", "fc1_dgrad", "fc2_wgrad", "fc1_wgrad"]
    gflops = sum(work[n][0] for n in gemms)
    gus = sum(us[n] for n in gemms)
    rec = {
        "metric": METRIC.replace("MoE FFN fwd", "MoE FFN fwd+bwd (training step)"),
        "value": w.N / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "env": provenance(torch),
        "config": {"workload": w.name + ("/fwd+bwd+main_grad" if args.main_grad else "/fwd+bwd"),
                   "N": w.N, "H": w.H, "E": w.E, "K": w.K,
                   "I": w.I, "F": w.F, "C": buf.C, "Cp": buf.Cp,
                   "weight_gradients": ("added into float32 main gradients" if args.main_grad
                                        else "written as bf16"),
                   "timed": "hipGraph replay of forward (pre-activation kept) + backward"},
        "gemm_tflops": gflops / (gus * 1e-6) / 1e12,
        "gemm_frac_bf16_peak": gflops / (gus * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
        "kernel_us": us,
        "kernel_tflops": {n: work[n][0] / (us[n] * 1e-6) / 1e12 for n in names},
        "kernel_gbs": {n: work[n][1] / (us[n] * 1e-6) / 1e9 for n in names},
        "kernel_frac_hbm_peak": {n: work[n][1] / (us[n] * 1e-6) / 1e9 / PEAK_HBM_GBS for n in names},
        "kept_routes": kept,
        "roofline": roofline(dom, work[dom][0], work[dom][1], us[dom]),
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu_baseline: timing the oracle (forward + backward)")
        rec["cpu_baseline"] = cpu_baseline_backward(T, dy, w)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec))


def bench_ep_local(args, w, torch, moe):
    """One step = the grouped FFN (FC1 + SwiGLU, FC2) on one expert-parallel
    rank's share of the layer: E/ep local experts with C*ep received rows
    each, already grouped by expert (the route list is the identity).  The
    exchange itself needs more than one GPU and is not timed."""
    import moe_inputs
    ep = args.ep
    C = int(moe.moe_source_capacity(w.N, w.K, w.E, w.F)) * ep
    d = moe_inputs.make_ep_local(w, ep, C, "cuda")
    E = d["E"]
    N = E * C
    H, I = w.H, w.I
    ssi = torch.arange(N, dtype=torch.int32, device="cuda")
    act = torch.empty(N, I, dtype=torch.bfloat16, device="cuda")
    ro = torch.empty(N, H, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    names = ["fc1", "fc2"]
    calls = [lambda: moe.moe_grouped_fc1_swiglu(d["x"], d["w1"], ssi, d["probs"], C, act, stream),
             lambda: moe.moe_grouped_fc2(act, d["w2"], N, C, ro, stream)]

    def step():
        for c in calls:
            c()

    ms_per_step = time_graph(torch, step, stream, args)
    us = time_calls(torch, names, calls, stream, args)
    # the receive buffer as an all-to-all leaves it (source-major): FC1 reads
    # it in expert order through a fixed route list
    perm = torch.as_tensor(moe_inputs.ep_receive_order(E, ep, C // ep), device="cuda")
    x_recv = torch.empty_like(d["x"])
    x_recv[perm.long()] = d["x"]
    act_sm = torch.empty_like(act)
    torch.cuda.synchronize()
    us_sm = time_calls(torch, ["fc1_source_major"],
                       [lambda: moe.moe_grouped_fc1_swiglu(x_recv, d["w1"], perm, d["probs"], C, act_sm,
                                                           stream)], stream, args)["fc1_source_major"]
    inv = torch.empty_like(perm)
    inv[perm.long()] = torch.arange(N, dtype=torch.int32, device="cuda")
    back = torch.empty_like(ro)
    torch.cuda.synchronize()
    us_back = time_calls(torch, ["return_reorder"],
                         [lambda: moe.moe_dispatch_rows(ro, inv, back, stream)], stream, args)["return_reorder"]
    # or FC2 writes its rows there directly through the row map
    ro_map = torch.empty_like(ro)
    us_map = time_calls(torch, ["fc2_rows"],
                        [lambda: moe.moe_grouped_fc2_rows(act, d["w2"], perm, N, C, ro_map, stream)],
                        stream, args)["fc2_rows"]
    flops = {"fc1": 2.0 * N * 2 * I * H, "fc2": 2.0 * N * H * I}
    nbytes = {"fc1": E * 2 * I * H * 2 + N * H * 2 + N * 8 + N * I * 2,
              "fc2": E * H * I * 2 + N * I * 2 + N * H * 2}
    gemm_tflops = (flops["fc1"] + flops["fc2"]) / ((us["fc1"] + us["fc2"]) * 1e-6) / 1e12
    # the dispatch side on a source rank: route the whole layer's tokens, then
    # pack the send buffer (each slot's token row in route order)
    T = moe_inputs.make_tensors(w, "cuda", weights=False)
    src = moe.MoEBuffers(w.N, H, I, w.E, w.K, w.F, "cuda")
    src.route_capacity_align(T["logits"])
    R = src.sorted_slot_ids.shape[0]
    send = torch.empty(R, H, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    kept = int((src.token_routes >= 0).sum().item())
    pack_us = time_calls(torch, ["dispatch_rows"],
                         [lambda: moe.moe_dispatch_rows(T["x"], src.sorted_slot_ids, send, stream)],
                         stream, args)["dispatch_rows"]
    pack_bytes = kept * H * 2 + R * 4 + R * H * 2
    log(f"[bench] dispatch rows (source rank, {R} slot rows): {pack_us:.1f} us, "
        f"{pack_bytes / (pack_us * 1e-6) / 1e9:.0f} GB/s")
    rec = {
        "metric": f"expert-parallel rank's grouped FFN (EP={ep} share): rows/s + grouped-GEMM TFLOP/s "
                  "(% bf16 MFMA peak), 1 GPU",
        "value": N / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "env": provenance(torch),
        "config": {"workload": f"{w.name}/ep{ep}-local", "E_local": E, "rows_per_expert": C,
                   "rows": N, "H": H, "I": I,
                   "timed": "hipGraph replay of FC1 + FC2 on the rank's received rows"},
        "gemm_tflops": gemm_tflops,
        "gemm_frac_bf16_peak": gemm_tflops / PEAK_BF16_TFLOPS,
        "kernel_us": us,
        "kernel_tflops": {n: flops[n] / (us[n] * 1e-6) / 1e12 for n in names},
        "kernel_gbs": {n: nbytes[n] / (us[n] * 1e-6) / 1e9 for n in names},
        "roofline": roofline("fc1_swiglu (FC1 + SwiGLU*prob on the received rows)", flops["fc1"],
                             nbytes["fc1"], us["fc1"]),
        # FC1 on the source-major receive buffer through its route list
        "fc1_source_major_us": us_sm,
        # route_out back into source-major chunks for the return exchange
        "return_reorder_us": us_back,
        # FC2 writing route_out straight into the source-major chunks
        "fc2_rows_us": us_map,
        # not part of the timed step: the source rank's send-buffer pack
        # before the exchange (moe_dispatch_rows), eager, HIP events
        "dispatch_rows": {"us": pack_us, "slot_rows": R, "algorithmic_bytes": pack_bytes,
                          "gbs": pack_bytes / (pack_us * 1e-6) / 1e9,
                          "frac_hbm_peak": pack_bytes / (pack_us * 1e-6) / 1e9 / PEAK_HBM_GBS},
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu_baseline: timing the oracle on one local expert")
        rec["cpu_baseline"] = cpu_baseline_ep_local(d, E, C)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec))


def cpu_baseline_ep_local(d, E, C, min_seconds=10.0):
    """The oracle's expert FFN on the rows of one local expert (repeated for
    at least ``min_seconds``), scaled to the rank's E experts."""
    import moe_inputs
    import oracle
    threads, blas = blas_threads()
    x = moe_inputs.bf16_bits(d["x"][:C])
    w1 = moe_inputs.bf16_bits(d["w1"][0])
    w2 = moe_inputs.bf16_bits(d["w2"][0])
    p = d["probs"][:C].cpu().numpy()
    times = []
    while len(times) < 2 or sum(times) < min_seconds:
        t0 = time.perf_counter()
        oracle.expert_ffn(x, w1, w2, p)
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    return {"value": C / med, "unit": "rows/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(times)} runs of oracle.expert_ffn on one local expert's {C} rows "
                      f"({sum(times):.1f} s in all, median {med:.2f} s; the rank's step is {E} such experts), "
                      f"numpy float64 with {blas} BLAS"}


def cpu_baseline_backward(T, dy, w, min_seconds=10.0):
    import oracle
    import moe_inputs
    lg = T["logits"].cpu().numpy()
    x, w1, w2 = (moe_inputs.bf16_bits(T[k]) for k in ("x", "w1", "w2"))
    dyb = moe_inputs.bf16_bits(dy)
    times = []
    while not times or (sum(times) < min_seconds and len(times) < 5):
        t0 = time.perf_counter()
        f = oracle.forward(lg, x, w1, w2, w.K, w.F)
        oracle.backward(f, x, w1, w2, dyb)
        times.append(time.perf_counter() - t0)
        log(f"  oracle forward+backward {len(times)}: {times[-1]:.2f} s")
    med = statistics.median(times)
    threads, blas = blas_threads()
    return {"value": w.N / med, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(times)} full forward+backward passes of the {w.name} workload "
                      f"({sum(times):.1f} s in all, median {med:.2f} s), numpy float64 with {blas} BLAS"}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        return (max([p.get("num_threads", 1) for p in info] or [1]),
                ",".join(sorted({p.get("internal_api", "?") for p in info})))
    except Exception:  # threadpoolctl missing: report the affinity set
        return len(os.sched_getaffinity(0)), "unknown"


def bench_serving(args, w, torch, moe):
    """Variable-N serving of the dropless forward: a seeded stream of items
    whose token counts cluster just above 0.5x and 1.0x of the expected size
    (where routing scatter puts them), run three ways on one stream with the
    inputs resident in HBM: the bucket ladder of captured graphs, one graph
    at the worst-case shape, and eager launches at each item's exact size."""
    import numpy as np
    import moe_inputs
    expected, top = w.N, 2 * w.N
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, 7]))
    items = args.serving_items
    centers = np.where(rng.random(items) < 0.5, 0.5, 1.0)
    sizes = np.clip((centers * (1.0 + rng.uniform(0.0, 0.08, items)) * expected).astype(int), 1, top)
    T = moe_inputs.make_tensors(w, "cuda")
    lg = torch.from_numpy(moe_inputs.make_logits(top, w.E, w.seed + 100)).to("cuda")
    g = torch.Generator(device="cuda").manual_seed(w.seed * 1000 + 9)
    xs = torch.randn(top, w.H, generator=g, device="cuda").to(torch.bfloat16)
    modes = {
        "bucketed": moe.ServingLadder(T["w1"], T["w2"], w.K, expected, top, reserve_bytes=8 << 30),
        "one_graph_at_worst_case": moe.ServingLadder(T["w1"], T["w2"], w.K, expected, top,
                                                     factors=(2.0,), max_padding_ratio=1e9,
                                                     reserve_bytes=8 << 30),
        "eager": moe.ServingLadder(T["w1"], T["w2"], w.K, expected, top, reserve_bytes=1 << 60),
    }
    res = {}
    for name, lad in modes.items():
        caps = lad.capture()
        log(f"[bench] serving/{name}: captured buckets {caps}")

        def stream_all():
            for n in sizes:
                lad.run(lg[:n], xs[:n])
        warm(stream_all, 1, args.warmup_seconds, lad.stream)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(lad.stream)
        for _ in range(args.serving_passes):
            stream_all()
        ev1.record(lad.stream)
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / args.serving_passes
        res[name] = {"ms_per_pass": ms, "tokens_per_s": float(sizes.sum()) / (ms * 1e-3),
                     "replays": {str(k): v for k, v in lad.counts.items() if v}}
        log(f"[bench] serving/{name}: {ms:.2f} ms per pass of {items} items "
            f"({res[name]['tokens_per_s'] / 1e6:.2f} M tokens/s)")
        del lad
        modes[name] = None
    b = res["bucketed"]
    rec = {
        "metric": "routed tokens/s, MoE FFN fwd (dropless), variable-N serving from bucketed hipGraphs, 1 GPU",
        "value": b["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.serving_passes,
        "warmup": args.warmup,
        "ms_per_step": b["ms_per_pass"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "env": provenance(torch),
        "config": {"workload": w.name + "/serving", "H": w.H, "E": w.E, "K": w.K, "I": w.I,
                   "expected_tokens": expected, "max_tokens": top, "items_per_pass": items,
                   "item_tokens": {"min": int(sizes.min()), "max": int(sizes.max()),
                                   "mean": float(sizes.mean())},
                   "timed": "one pass = every item once, inputs resident in HBM"},
        "modes": res,
        "bucketed_vs_worst_case_graph": res["one_graph_at_worst_case"]["ms_per_pass"] / b["ms_per_pass"],
        "bucketed_vs_eager": res["eager"]["ms_per_pass"] / b["ms_per_pass"],
        "roofline": None,
        "cpu_baseline": None,
    }
    print(json.dumps(rec))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-seconds", type=float, default=0.5,
                    help="minimum wall time of untimed warm-up before each timed region")
    ap.add_argument("--workload", default=None, help="workload name (default: the Qwen3-30B-A3B-shaped layer)")
    ap.add_argument("--cpu-forwards", type=int, default=3,
                    help="minimum oracle forwards timed for cpu_baseline (more, up to 20, until 12 s of work)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--serving-items", type=int, default=32, help="items per pass (--variant serving)")
    ap.add_argument("--serving-passes", type=int, default=5, help="timed passes (--variant serving)")
    ap.add_argument("--ep", type=int, default=8, help="expert-parallel degree (--variant ep-local)")
    ap.add_argument("--variant", choices=["capacity", "dropless", "backward", "serving", "ep-local"],
                    default="capacity",
                    help="fixed-capacity forward (the headline), the dropless form, or the "
                         "training step (forward keeping the pre-activation + backward)")
    ap.add_argument("--main-grad", action="store_true",
                    help="with --variant backward: add the weight gradients into float32 main "
                         "gradients (gradient accumulation) instead of writing them as bf16")
    ap.add_argument("--vendor-reference", action="store_true",
                    help="only time torch's bf16 batched GEMM (hipBLASLt) at the layer's per-expert "
                         "FC1 and FC2 shapes, as context for the grouped kernels, and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--access-order-probes", action="store_true",
                    help="only time the library's access-order and LDS-ring probes over a buffer "
                         "the size of the workload's W1, print one JSON line and exit")
    ap.add_argument("--gemm-loop-probe", action="store_true",
                    help="only time the library's GEMM-loop probe (the grouped GEMMs' K loop with no "
                         "gather and no epilogue) at the workload's FC1 and FC2 shapes, print one JSON "
                         "line and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the MoE FFN forward on one GPU only: it has no multi-GPU path, "
              "since one GPU holds the whole layer's weights and tokens", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_inputs
    import mixture_experts_expert_amd as moe

    if args.copy_calibration:
        copy_calibration(torch)
        return

    w = moe_inputs.WORKLOADS[args.workload or moe_inputs.HEADLINE]
    if args.access_order_probes:
        access_order_probes(torch, moe, w)
        return
    if args.gemm_loop_probe:
        gemm_loop_probe(torch, moe, w)
        return
    if args.vendor_reference:
        vendor_reference(torch, moe, w, args)
        return
    if w.skew:
        raise SystemExit("skewed workloads are parity cases, not bench lines")
    log(f"[bench] {w.name}: N={w.N} H={w.H} E={w.E} K={w.K} F={w.F} I={w.I}")
    if args.variant == "serving":
        bench_serving(args, w, torch, moe)
        return
    if args.variant == "ep-local":
        bench_ep_local(args, w, torch, moe)
        return
    T = moe_inputs.make_tensors(w, "cuda")
    if args.variant == "backward":
        bench_backward(args, w, T, torch, moe)
        return
    dropless = args.variant == "dropless"
    if dropless:
        buf = moe.DroplessBuffers(w.N, w.H, w.I, w.E, w.K, "cuda")
        route = lambda: buf.route(T["logits"])                     # noqa: E731
        route_name = "route_dropless"
    else:
        buf = moe.MoEBuffers(w.N, w.H, w.I, w.E, w.K, w.F, "cuda")
        route = lambda: buf.route_capacity_align(T["logits"])      # noqa: E731
        route_name = "route_capacity_align"
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()

    names = [route_name, "fc1", "fc2", "combine"]
    calls = [route, lambda: buf.fc1_swiglu(T["x"], T["w1"]), lambda: buf.fc2(T["w2"]), buf.combine]

    def fwd():
        for c in calls:
            c()

    # timed region 1: graph replays; timed region 2: per-call kernel times
    replay = {}
    ms_per_step = time_graph(torch, fwd, stream, args, replay)
    us = time_calls(torch, names, calls, stream, args)
    probes = hbm_probes(torch, moe, stream)
    cprobes = compute_probes(torch, moe, stream)

    kept = int((buf.token_routes >= 0).sum().item())
    if dropless:
        rows = int(buf.num_tokens_post_padded.item())
        nbytes = algorithmic_bytes_dropless(w, rows, buf.R, buf.BM)
        traffic = None      # the committed counters were taken on the capacity form
        shape = {"R_bound": buf.R, "extent": rows, "timed": "hipGraph replay of the whole dropless forward"}
    else:
        rows = w.E * buf.Cp
        nbytes = algorithmic_bytes(w, buf.C, buf.Cp, kept)
        traffic = pmc_traffic(w.name)
        shape = {"C": buf.C, "Cp": buf.Cp, "timed": "hipGraph replay of the whole forward"}
    fc1_flops = 2.0 * rows * (2 * w.I) * w.H
    fc2_flops = 2.0 * rows * w.H * w.I
    gemm_tflops = (fc1_flops + fc2_flops) / ((us["fc1"] + us["fc2"]) * 1e-6) / 1e12
    gbs = {n: nbytes[n] / (us[n] * 1e-6) / 1e9 for n in names}

    rec = {
        "metric": METRIC,
        "value": w.N / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "env": provenance(torch),
        "config": {"workload": w.name + ("/dropless" if dropless else ""), "N": w.N, "H": w.H,
                   "E": w.E, "K": w.K, "I": w.I, **({} if dropless else {"F": w.F}), **shape},
        "routes_per_s": w.N * w.K / (ms_per_step * 1e-3),
        "replay_us": replay,
        "gemm_tflops": gemm_tflops,
        "gemm_frac_bf16_peak": gemm_tflops / PEAK_BF16_TFLOPS,
        # the same GEMM time credited only with the kept routes' work
        "useful_tflops": 6.0 * w.H * w.I * kept / ((us["fc1"] + us["fc2"]) * 1e-6) / 1e12,
        # the matrix cores' attainable rate on this device (a probe issuing
        # nothing but MFMAs) and the LDS read rate, with their engine clocks
        "compute_probe": cprobes,
        "gemm_frac_mfma_probe": gemm_tflops / cprobes["mfma_tflops"],
        "kernel_us": us,
        "kernel_gbs": gbs,
        "kernel_frac_hbm_peak": {n: gbs[n] / PEAK_HBM_GBS for n in names},
        # the scan / scatter / gather steps together (routing call + combine)
        "route_combine_frac_hbm_peak": (nbytes[route_name] + nbytes["combine"])
                                       / ((us[route_name] + us["combine"]) * 1e-6) / 1e9 / PEAK_HBM_GBS,
        # torch's own device copy: a reference point for HBM rates
        "torch_copy_gbs": copy_rate(torch, stream),
        # the measured ceilings (the library's HBM probes), and each call's
        # rate of algorithmic bytes against the probe read and copy rates
        "hbm_probe_gbs": probes,
        "kernel_frac_probe": {n: {"read": gbs[n] / probes["read"], "copy": gbs[n] / probes["copy"]}
                              for n in names},
        # the combine reads route_out right after FC2 wrote it; most of those
        # 134 MB come from the 256 MB last-level cache, so its rate is an
        # effective, cache-assisted one, not an HBM-efficiency figure
        "combine_rate_note": "effective (cache-assisted): route_out is read from the last-level cache FC2 just filled",
        "kept_routes": kept,
        "roofline": roofline("fc1_swiglu (gather-in-GEMM FC1 + SwiGLU*prob)", fc1_flops,
                             nbytes["fc1"], us["fc1"], traffic, probes),
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu_baseline: timing the oracle")
        rec["cpu_baseline"] = cpu_baseline(T, w, args.cpu_forwards, dropless=dropless)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
