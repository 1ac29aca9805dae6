#!/usr/bin/env python3
"""Benchmark of the MSDA core (forward + backward) on one MI355X.

One step = one forward call and one backward call of the C ABI on the
resident, seeded synthetic inputs of a workload (default: the decoder-shaped
bf16 workload, B=4 Q=300 M=8 D=32 L=4 K=4, levels of an 800x1333 image). The
backward runs with the library's default accumulation (AUTO) and includes
every kernel it launches.

Timed region: the step is captured once in a HIP graph and replayed K times
between two events (host dispatch removed, as with the pages' CUDA-graph
cross-check); an eager run of the same steps is reported beside it. Per-kernel
device times come from an instrumented eager pass: the library records a HIP
event right before and right after each of its launches on the call's stream.

Prints one JSON line:
  value / ms_per_step   microseconds per forward+backward step (lower is better)
  kernels               per-kernel average device time and algorithmic GB/s
  roofline              the dominant kernel against the 8 TB/s HBM roofline:
                        algorithmic bytes per launch / average launch duration
  phases                the forward and the backward call as wholes: their
                        kernels' algorithmic bytes / summed launch times
  cold_us_per_step      context: one step timed alone after 1 GiB is written
                        (L2 and the 256 MB MALL evicted)
  device_copy_GBps      context: a 1 GiB device copy, bytes read + written / time
  cpu_baseline          the CPU oracle (fp64 loops, OpenMP) on the same workload

Algorithmic bytes per launch (e = element size of value / grad rows, pe = of
locations / weights (fp32 beside 16-bit values in mixed workloads),
P = B*Q*M*L*K points,
U = distinct (b, row, m) value rows with at least one in-bounds corner,
C = in-bounds corners, N = B*S*M*D grad_value elements):
  forward          3*P*pe (locations + weights) + B*Q*M*D*e (output) + U*D*e
  backward kernel  (msda_bwd_kernel; msda_grad_kernel without the atomics term
                   when some level is binned)
                   3*P*pe (params) + B*Q*M*D*e (grad_output) + U*D*e (value)
                   + 3*P*pe (grad locations + grad weights)
                   + atomics: 2*U'*D*e_acc (read-modify-write of the touched rows
                     of levels not binned; e_acc = 4 for fp32 rows)
  scatter          3*(P-P')*pe + B*Q*M*D*e + 2*U'*D*e_acc (atomics of the unbinned levels)
  binned levels only (P', C', N' = their points, corners, grad_value elements):
  bin count        2*P'*pe;  bin place  3*P'*pe + 8*C' (records written)
  bin scan         3*nbins*4 (one workgroup), or tile sums nbins*4, tile offsets
                   3*ntiles*4, tile scans 3*nbins*4 (large bin counts)
  bin local sort   3*P'*pe + 8*C' + 8*nbins (count and place in one launch,
                   bin ranges written) + N*e when it also zero-fills grad_value
  bin accumulate   8*C' + B*Q*M*D*e + N'*e
  scatter + accumulate in one launch: the sum of the two; likewise gradients +
  local sort (+ zero fill) in one launch
  zero fill        bytes written;  scratch add  rows * D * (4 + 2e)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MSDA fwd+bwd µs/call + achieved HBM GB/s (% of peak), decoder & encoder shapes"
HBM_PEAK_GBPS = 8000.0
# Pages' own decoder-preset figure for this workload and metric, on another
# machine (H100, Triton, bf16: forward 8 us + backward 56 us; msda-triton
# README, section "Benchmarks"). Context for vs_baseline, not a target.
PAGES_DECODER_BF16_US = 8.0 + 56.0
# Device-scope atomic adds on MI355X are request-bound: about 21 G requests/s
# measured for requests of 1 to 16 dwords inside one 64-byte segment.
ATOMIC_CEILING_GREQ = 21.0
ATOMIC_KERNELS = ("msda_bwd_kernel", "msda_scatter_kernel", "scatter_accum_kernel")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def touched_rows(inp, only_levels=None):
    """(U, C): distinct (b, row, m) value rows that at least one in-bounds
    corner lands on, and the number of in-bounds corners. Host-side
    accounting of compulsory bytes (single-rounding pixel mapping as in the
    kernels; products of an fp32 location and an integer width are exact in
    fp64)."""
    value = inp["value"]
    B, S, M, D = value.shape
    loc = inp["sampling_locations"].to(torch.float64).numpy()
    shapes = inp["spatial_shapes"].tolist()
    mark = np.zeros(B * S * M, dtype=bool)
    corners = 0
    b_idx = np.arange(B).reshape(B, 1, 1, 1)
    m_idx = np.arange(M).reshape(1, 1, M, 1)
    start = 0
    for l, (H, W) in enumerate(shapes):
        if only_levels is not None and l not in only_levels:
            start += H * W
            continue
        x = (loc[:, :, :, l, :, 0] * W - 0.5).astype(np.float32)
        y = (loc[:, :, :, l, :, 1] * H - 0.5).astype(np.float32)
        x0 = np.floor(x).astype(np.int64)
        y0 = np.floor(y).astype(np.int64)
        for dy in (0, 1):
            for dx in (0, 1):
                xx, yy = x0 + dx, y0 + dy
                ok = (xx >= 0) & (xx < W) & (yy >= 0) & (yy < H)
                row = start + yy * W + xx
                key = (b_idx * S + row) * M + m_idx
                mark[key[ok]] = True
                corners += int(ok.sum())
        start += H * W
    return int(mark.sum()), corners


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in ("scale_deformable_attention_amd/csrc/msda_kernels.hip",
                "scale_deformable_attention_amd/csrc/msda_api.cpp",
                "scale_deformable_attention_amd/csrc/msda_launch.h",
                "scale_deformable_attention_amd/csrc/msda_device.h"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, kernel: str, src_hash: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("#") or "=" not in line:
            continue
        k, v = line.split("=", 1)
        fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha") != src_hash:
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_graph(fn, reps: int, inner: int) -> float:
    """Average device time of `fn` per call: `inner` calls captured in one HIP
    graph, replayed `reps` times between events on the capture stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(inner):
            fn()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * inner)  # us


def cpu_baseline(inp, min_seconds: float = 10.0, max_reps: int = 2000):
    import oracle  # the CPU-baseline leg is the only product-side user of the oracle
    args = (inp["value"], inp["spatial_shapes"], None, inp["sampling_locations"],
            inp["attention_weights"])
    oracle.forward(*args)  # warm (page-in, thread pool)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(*args)
        oracle.backward(*args, inp["grad_output"])
        reps += 1
        el = time.perf_counter() - t0
        if (el >= min_seconds and reps >= 3) or reps >= max_reps:
            break
    return el / reps * 1e6, reps, oracle.max_threads()


def time_foil(g, call, fwd_bytes: int, reps: int = 20) -> dict:
    """The point-parallel forward foil against the forward kernel, each timed
    with the library's per-launch event pairs (same bias for both)."""
    from scale_deformable_attention_amd._binding import (msda_forward_point_parallel,
                                                         set_launch_events)
    args = (g["value"], g["spatial_shapes"], None, g["sampling_locations"], g["attention_weights"])
    fout = msda_forward_point_parallel(*args)
    out = call.forward()
    torch.cuda.synchronize()
    diff = float((fout.float() - out.float()).abs().max())

    def kernel_us(fn):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for pair in evs:
            for e in pair:
                e.record()
        torch.cuda.synchronize()
        for pair in evs:
            set_launch_events(pair)
            fn()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3

    foil_us = kernel_us(lambda: msda_forward_point_parallel(*args, output=fout))
    fwd_us = kernel_us(call.forward)
    log(f"point-parallel foil {foil_us:.2f} us vs forward kernel {fwd_us:.2f} us "
        f"(max |difference| {diff:.3g})")
    gbps = lambda us: fwd_bytes / (us * 1e-6) / 1e9
    return {"kernel": "msda_foil_kernel", "us": round(foil_us, 3), "GBps": round(gbps(foil_us), 1),
            "frac": round(gbps(foil_us) / HBM_PEAK_GBPS, 4), "forward_us": round(fwd_us, 3),
            "forward_GBps": round(gbps(fwd_us), 1),
            "forward_frac": round(gbps(fwd_us) / HBM_PEAK_GBPS, 4),
            "max_abs_diff_vs_forward": diff}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decoder_bf16")
    ap.add_argument("--accum", default="auto",
                    choices=["auto", "native", "fp32_scratch", "per_level", "binned", "mixed"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--profile-only", action="store_true",
                    help="run warmup + timed steps only (for rocprofv3 runs)")
    ap.add_argument("--foil", action="store_true",
                    help="also time the point-parallel forward foil against the forward kernel")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="with --profile-only: also run 5 plain device copies of this many MiB "
                         "(reference dispatches for scaling FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)

    from scale_deformable_attention_amd import PreparedCall, load_library
    from scale_deformable_attention_amd.workloads import make_inputs, workload

    load_library()  # raises if the HIP library is missing
    wl = workload(args.workload)
    dev = torch.device("cuda:0")
    log(f"workload {wl.name}: B={wl.B} Q={wl.num_queries} S={wl.S} M={wl.M} D={wl.D} "
        f"L={wl.L} K={wl.K} {wl.dtype}")
    inp = make_inputs(wl)
    g = {k: (v.to(dev) if k != "spatial_shapes" else v) for k, v in inp.items()}
    call = PreparedCall(g["value"], g["spatial_shapes"], None, g["sampling_locations"],
                        g["attention_weights"], g["grad_output"], accum=args.accum)
    log(f"backward accumulation: {args.accum} -> {call.resolved_accum}")

    def step():
        call.forward()
        call.backward()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")
    if args.profile_only:
        K = args.steps
        for _ in range(K):
            step()
        torch.cuda.synchronize()
        log(f"ran {K} eager steps")
        if args.foil:
            from scale_deformable_attention_amd._binding import msda_forward_point_parallel
            for _ in range(K):
                msda_forward_point_parallel(g["value"], g["spatial_shapes"], None,
                                            g["sampling_locations"], g["attention_weights"])
            torch.cuda.synchronize()
            log(f"ran {K} point-parallel foil forwards")
        if args.calib_copy_mb:
            n = args.calib_copy_mb * (1 << 20) // 4
            src = torch.ones(n, dtype=torch.float32, device=dev)
            dst = torch.empty_like(src)
            for _ in range(5):
                dst.copy_(src)
            torch.cuda.synchronize()
            log(f"calibration: 5 copies of {args.calib_copy_mb} MiB (read {args.calib_copy_mb} MiB, "
                f"write {args.calib_copy_mb} MiB each)")
        return

    K = args.steps
    # Timed region: K replays of one captured step.
    graph_ok = True
    try:
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_cap):
            step()
        torch.cuda.current_stream().wait_stream(s_cap)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
    except Exception as exc:  # fall back to eager stepping
        graph_ok = False
        log(f"graph capture failed ({exc}); timing eager steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(K):
        if graph_ok:
            graph.replay()
        else:
            step()
    e1.record()
    torch.cuda.synchronize()
    us_step = e0.elapsed_time(e1) * 1e3 / K
    # Eager steps, for context.
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    e0.record()
    for _ in range(K):
        step()
    e1.record()
    h1 = time.perf_counter()
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1e3 / K
    host_us = (h1 - h0) * 1e6 / K
    log(f"timed {K} steps: {us_step:.2f} us/step ({'graph replay' if graph_ok else 'eager'}); "
        f"eager {eager_us:.2f} us/step, host enqueue {host_us:.2f} us/step")

    # Cold caches, for context: a 1 GiB write between steps evicts L2 and the
    # 256 MB MALL; each step is timed alone (one launch of the captured step).
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    n_cold = min(K, 50)
    c_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n_cold)]
    for c0, c1 in c_evs:
        flush.fill_(1.0)
        c0.record()
        if graph_ok:
            graph.replay()
        else:
            step()
        c1.record()
    torch.cuda.synchronize()
    cold_us = float(np.mean([c0.elapsed_time(c1) for c0, c1 in c_evs])) * 1e3
    # Device copy bandwidth, for context: 10 copies of 1 GiB (read + write).
    cp_src = flush
    cp_dst = torch.empty_like(cp_src)
    cp_dst.copy_(cp_src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        cp_dst.copy_(cp_src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 10 * 2 * cp_src.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del flush, cp_src, cp_dst
    log(f"cold-cache step {cold_us:.2f} us (1 GiB written between steps); "
        f"device copy {copy_gbps:.0f} GB/s")

    # Per-kernel device times: events right before / after each launch.
    from scale_deformable_attention_amd._binding import (launch_event_names, launch_events_recorded,
                                                         set_launch_events)
    n_inst = min(K, 50)
    nev = 16
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 + nev)] for _ in range(n_inst)]
    for row in evs:
        for ev in row:
            ev.record()
    torch.cuda.synchronize()
    n_bwd = None
    for i in range(n_inst):
        set_launch_events(evs[i][:2])
        call.forward()
        set_launch_events(evs[i][2:])
        call.backward()
        n_bwd = launch_events_recorded() // 2
    bwd_names = launch_event_names()  # the library names each instrumented launch
    torch.cuda.synchronize()
    assert n_bwd == len(bwd_names), (n_bwd, bwd_names)
    ktimes = {"msda_fwd_kernel": float(np.mean([evs[i][0].elapsed_time(evs[i][1])
                                                 for i in range(n_inst)])) * 1e3}
    for j, nm in enumerate(bwd_names):
        ktimes[nm] = float(np.mean([evs[i][2 + 2 * j].elapsed_time(evs[i][3 + 2 * j])
                                    for i in range(n_inst)])) * 1e3
    log("kernels (us): " + ", ".join(f"{k} {v:.2f}" for k, v in ktimes.items()))

    # Algorithmic bytes per launch.
    e = torch.finfo(wl.dtype).bits // 8
    pe = torch.finfo(wl.param_dtype or wl.dtype).bits // 8  # locations / weights
    B, S, M, D, L, Kp, Q = wl.B, wl.S, wl.M, wl.D, wl.L, wl.K, wl.num_queries
    P = B * Q * M * L * Kp
    N = B * S * M * D
    U, C = touched_rows(inp)
    level_modes, nb = call.plan()
    scr_levels = [l for l, m in enumerate(level_modes) if m == "fp32_scratch"]
    bin_levels = [l for l, m in enumerate(level_modes) if m == "binned"]
    U_scr = touched_rows(inp, only_levels=scr_levels)[0] if scr_levels else 0
    U_bin, C_bin = touched_rows(inp, only_levels=bin_levels) if bin_levels else (0, 0)
    scratch_rows = sum(B * h * w * M for l, (h, w) in enumerate(wl.levels) if l in scr_levels)
    bin_rows = sum(B * h * w * M for l, (h, w) in enumerate(wl.levels) if l in bin_levels)
    P_bin = B * Q * M * Kp * len(bin_levels)
    common = 3 * P * pe + B * Q * M * D * e + U * D * e + 3 * P * pe
    e_acc = 4 if wl.dtype == torch.float32 else e
    # a zero fill that did not get its own launch ran inside the sort's launch
    zero_fused = int("zero_fill" not in ktimes and any(m != "binned" for m in level_modes))
    kbytes = {"msda_fwd_kernel": 3 * P * pe + B * Q * M * D * e + U * D * e,
              "zero_fill": N * e, "scratch_zero": scratch_rows * D * 4,
              "scratch_add_kernel": scratch_rows * D * (4 + 2 * e),
              # atomics: read-modify-write of the touched rows of unbinned levels
              "msda_bwd_kernel": common + 2 * ((U - U_scr - U_bin) * D * e_acc + U_scr * D * 4),
              "msda_grad_kernel": common,
              "msda_scatter_kernel": 3 * (P - P_bin) * pe + B * Q * M * D * e
              + 2 * (U - U_bin) * D * e_acc,
              "bin_zero": (nb + 1) * 4, "bin_count": 2 * P_bin * pe, "bin_scan": 3 * nb * 4,
              "bin_place": 3 * P_bin * pe + 8 * C_bin,
              "bin_local_sort": 3 * P_bin * pe + 8 * C_bin + 8 * nb + zero_fused * N * e,
              "bin_tile_sum": nb * 4, "bin_tile_offsets": 3 * (-(-nb // 4096)) * 4,
              "bin_tile_scan": 3 * nb * 4,
              "bin_accum_kernel": 8 * C_bin + B * Q * M * D * e + bin_rows * D * e}
    kbytes["scatter_accum_kernel"] = kbytes["msda_scatter_kernel"] + kbytes["bin_accum_kernel"]
    kbytes["grad_sort_kernel"] = kbytes["msda_grad_kernel"] + kbytes["bin_local_sort"]
    kernels = {k: {"us": round(v, 3), "bytes": int(kbytes[k]),
                   "GBps": round(kbytes[k] / (v * 1e-6) / 1e9, 1)} for k, v in ktimes.items()}
    # The forward call and the backward call as wholes: algorithmic bytes of
    # their kernels over the sum of their launch times (event pairs), against
    # the 8 TB/s peak.
    phases = {}
    for ph, names in (("forward", ["msda_fwd_kernel"]),
                      ("backward", [k for k in ktimes if k != "msda_fwd_kernel"])):
        t = sum(ktimes[k] for k in names)
        by = sum(kbytes[k] for k in names)
        phases[ph] = {"us": round(t, 3), "bytes": int(by),
                      "GBps": round(by / (t * 1e-6) / 1e9, 1),
                      "frac": round(by / (t * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    kname = max(ktimes, key=ktimes.get)
    kus = ktimes[kname]
    achieved = kbytes[kname] / (kus * 1e-6) / 1e9
    src_hash = kernel_source_hash()
    traffic = load_traffic(wl.name, kname, src_hash)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic, "kernel": kname, "kernel_us": round(kus, 3),
                "algorithmic_bytes_per_launch": int(kbytes[kname]), "kernel_source_sha": src_hash}

    # Context for a kernel bound by atomics rather than HBM: its requests (one
    # per in-bounds corner per 64-byte segment of the target row: packed
    # 16-bit rows of D*e bytes, fp32 rows of D*4) per second of launch time,
    # against the measured request ceiling.
    atomic_rate = None
    if kname in ATOMIC_KERNELS:
        seg = {"native": -(-D * (4 if wl.dtype == torch.float32 else e) // 64),
               "fp32_scratch": -(-D * 4 // 64)}
        reqs = sum(touched_rows(inp, only_levels=[l])[1] * seg[m]
                   for l, m in enumerate(level_modes) if m in seg)
        rate = reqs / (kus * 1e-6) / 1e9
        atomic_rate = {"kernel": kname, "requests": int(reqs), "achieved": round(rate, 2),
                       "ceiling": ATOMIC_CEILING_GREQ, "unit": "G requests/s",
                       "frac": round(rate / ATOMIC_CEILING_GREQ, 4)}

    result = {
        "metric": METRIC, "value": round(us_step, 3), "unit": "us/call (fwd+bwd)",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(us_step / 1e3, 6),
        "higher_is_better": False, "scaling": "weak",
        "vs_baseline": round(us_step / PAGES_DECODER_BF16_US, 4)
        if wl.name == "decoder_bf16" else None,
        "dtype": {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[wl.dtype],
        "data": "synthetic (seeded; stands in for Deformable-DETR COCO inputs)",
        "config": {"workload": wl.name, "B": B, "Q": Q, "S": S, "M": M, "D": D, "L": L, "K": Kp,
                   "levels": [list(x) for x in wl.levels], "accum": call.resolved_accum,
                   "param_dtype": str(wl.param_dtype or wl.dtype).replace("torch.", ""),
                   "parallelism": "single GPU"},
        "timing": "graph replay" if graph_ok else "eager",
        "eager_us_per_step": round(eager_us, 3), "host_enqueue_us": round(host_us, 3),
        "cold_us_per_step": round(cold_us, 3), "cold_flush_bytes": 1 << 30,
        "device_copy_GBps": round(copy_gbps, 1),
        "fwd_us": round(ktimes["msda_fwd_kernel"], 3),
        "bwd_us": round(sum(v for k, v in ktimes.items() if k != "msda_fwd_kernel"), 3),
        "kernels": kernels, "phases": phases, "touched_rows_U": U, "corners_C": C, "points_P": P,
        "roofline": roofline, "atomic_rate": atomic_rate,
    }
    if args.foil:
        result["foil"] = time_foil(g, call, kbytes["msda_fwd_kernel"])
    if not args.no_cpu_baseline:
        log("timing the CPU oracle (cpu_baseline)")
        cpu_us, reps_done, threads = cpu_baseline(inp, args.cpu_seconds)
        result["cpu_baseline"] = {
            "value": round(cpu_us, 1), "unit": "us/call (fwd+bwd)", "cores": threads,
            "kind": "oracle",
            "sample": f"full {wl.name} workload, {reps_done} forward+backward calls, "
                      f"{platform.processor() or platform.machine()}"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
