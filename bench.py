#!/usr/bin/env python3
"""Benchmark of the MSDA core (forward + backward) on one MI355X.

One step = one forward call and one backward call of the C ABI on the
resident, seeded synthetic inputs of a workload (default: the decoder-shaped
bf16 workload, B=4 Q=300 M=8 D=32 L=4 K=4, levels of an 800x1333 image). The
backward runs with the library's default accumulation (AUTO) and includes
every stage: zero-fill, the scatter kernel and the fp32->dtype pass when the
scratch path is taken.

Prints one JSON line:
  value / ms_per_step   microseconds per forward+backward step (lower is better)
  fwd_us, bwd_us        per-call device time from HIP events in the timed region
  roofline              the dominant kernel against the 8 TB/s HBM roofline:
                        algorithmic bytes per launch / average launch duration
  cpu_baseline          the CPU oracle (fp64 loops, OpenMP) on the same workload

Algorithmic bytes per launch (e = element size, P = B*Q*M*L*K points,
U = distinct (b, row, m) value rows with at least one in-bounds corner):
  forward       3*P*e (locations + weights) + B*Q*M*D*e (output) + U*D*e
  scatter       3*P*e (params) + B*Q*M*D*e (grad_output) + U*D*e (value)
                + 2*U*D*e_acc (read-modify-write of touched grad rows; e_acc = 4
                  for rows of levels accumulated in fp32 scratch)
                + 3*P*e (grad locations + grad weights)
  zero fill     B*S*M*D*e (+ scratch rows * 4);  scratch add  rows * D * (4 + 2e)
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


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def touched_rows(inp, only_levels=None) -> int:
    """U: distinct (b, row, m) value rows that at least one in-bounds corner
    lands on. Host-side accounting of compulsory bytes (single-rounding
    pixel mapping as in the kernels; products of an fp32 location and an
    integer width are exact in fp64)."""
    value = inp["value"]
    B, S, M, D = value.shape
    loc = inp["sampling_locations"].to(torch.float64).numpy()
    shapes = inp["spatial_shapes"].tolist()
    mark = np.zeros(B * S * M, dtype=bool)
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
        start += H * W
    return int(mark.sum())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in ("scale_deformable_attention_amd/csrc/msda_kernels.hip",
                "scale_deformable_attention_amd/csrc/msda_api.cpp",
                "scale_deformable_attention_amd/csrc/msda_launch.h"):
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


def cpu_baseline(inp, min_seconds: float = 10.0, max_reps: int = 200):
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decoder_bf16")
    ap.add_argument("--accum", default="auto", choices=["auto", "native", "fp32_scratch"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--profile-only", action="store_true",
                    help="run warmup + timed steps only (for rocprofv3 runs)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="with --profile-only: also run 5 plain device copies of this many MiB "
                         "(reference dispatches for scaling FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
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

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    e_start.record()
    for i in range(K):
        ev[i][0].record()
        call.forward()
        ev[i][1].record()
        call.backward()
        ev[i][2].record()
    e_end.record()
    h1 = time.perf_counter()
    torch.cuda.synchronize()
    total_ms = e_start.elapsed_time(e_end)
    us_step = total_ms * 1e3 / K
    fwd_us = float(np.mean([ev[i][0].elapsed_time(ev[i][1]) for i in range(K)])) * 1e3
    bwd_us = float(np.mean([ev[i][1].elapsed_time(ev[i][2]) for i in range(K)])) * 1e3
    host_us = (h1 - h0) * 1e6 / K
    log(f"timed {K} steps: {us_step:.2f} us/step (fwd {fwd_us:.2f}, bwd {bwd_us:.2f}, "
        f"host enqueue {host_us:.2f} us/step)")
    if args.profile_only:
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

    # Per-kernel device time, host overhead removed by graph replay.
    reps, inner = 20, 20
    fwd_kernel_us = time_graph(call.forward, reps, inner)
    # the scatter kernel alone, as the default accumulation runs it: add into
    # grad_value and keep adding into the scratch levels (no fill, no final add)
    from scale_deformable_attention_amd._binding import FLAG_CONTINUE_SCRATCH, FLAG_DEFER_SCRATCH
    call.backward()
    scatter_us = time_graph(lambda: call.backward(
        accumulate=True, flags=FLAG_CONTINUE_SCRATCH | FLAG_DEFER_SCRATCH), reps, inner)
    scatter_native_us = time_graph(lambda: call.backward(accumulate=True, accum="native"), reps,
                                   inner)
    graph_step_us = time_graph(step, reps, 5)
    log(f"graph replay: forward kernel {fwd_kernel_us:.2f} us, scatter kernel ({call.resolved_accum}) "
        f"{scatter_us:.2f} us, all-native scatter kernel {scatter_native_us:.2f} us, "
        f"full step {graph_step_us:.2f} us")

    # Algorithmic bytes.
    e = torch.finfo(wl.dtype).bits // 8
    B, S, M, D, L, Kp, Q = wl.B, wl.S, wl.M, wl.D, wl.L, wl.K, wl.num_queries
    P = B * Q * M * L * Kp
    U = touched_rows(inp)
    U_scr = touched_rows(inp, only_levels=call.scratch_levels()) if call.scratch_levels() else 0
    fwd_bytes = 3 * P * e + B * Q * M * D * e + U * D * e
    # grad rows: read + write once each, 2 bytes per element in bf16/fp16 levels
    # and 4 in fp32 ones (fp32 data, or the scratch levels of 16-bit data)
    grad_rows = 2 * ((U - U_scr) * D * e + U_scr * D * 4)
    scatter_bytes = 3 * P * e + B * Q * M * D * e + U * D * e + grad_rows + 3 * P * e
    fwd_gbps = fwd_bytes / (fwd_kernel_us * 1e-6) / 1e9
    scatter_gbps = scatter_bytes / (scatter_us * 1e-6) / 1e9
    # Dominant kernel: the longer of the two hot kernels.
    src_hash = kernel_source_hash()
    if scatter_us >= fwd_kernel_us:
        kname, kus, kbytes = "msda_bwd_kernel", scatter_us, scatter_bytes
    else:
        kname, kus, kbytes = "msda_fwd_kernel", fwd_kernel_us, fwd_bytes
    achieved = kbytes / (kus * 1e-6) / 1e9
    traffic = load_traffic(wl.name, kname, src_hash)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic, "kernel": kname, "kernel_us": round(kus, 3),
                "algorithmic_bytes_per_launch": int(kbytes), "kernel_source_sha": src_hash}

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
                   "parallelism": "single GPU"},
        "fwd_us": round(fwd_us, 3), "bwd_us": round(bwd_us, 3), "host_enqueue_us": round(host_us, 3),
        "graph_step_us": round(graph_step_us, 3),
        "fwd_kernel_us": round(fwd_kernel_us, 3), "fwd_kernel_GBps": round(fwd_gbps, 1),
        "scatter_kernel_us": round(scatter_us, 3), "scatter_kernel_GBps": round(scatter_gbps, 1),
        "scatter_all_native_kernel_us": round(scatter_native_us, 3),
        "touched_rows_U": U, "points_P": P,
        "roofline": roofline,
    }
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
