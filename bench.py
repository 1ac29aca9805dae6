#!/usr/bin/env python3
"""Benchmark of the MSDA core (forward + backward) on one MI355X.

One step = one forward call and one backward call of the C ABI on the
resident, seeded synthetic inputs of a workload. The headline workload is the
decoder-shaped bf16 one (B=4 Q=300 M=8 D=32 L=4 K=4, levels of an 800x1333
image); the encoder-shaped workloads (fp16 encoder, odd-head fp32, large bf16
encoder) are measured the same way in the line's `configs` object. The
backward runs with the library's default accumulation (AUTO) and includes
every kernel it launches.

Timing. The step is captured once in a HIP graph and replayed K times between
two events (host dispatch removed, as with the pages' CUDA-graph cross-check);
per-kernel device times and the phases' device spans come from an
instrumented eager pass: the library launches each kernel with a pair of HIP
events that the launch itself stamps at the kernel's start and end
(hipExtLaunchKernel), the same interval rocprofv3's kernel trace reports.

Algorithmic bytes (the method's own traffic; e = element size of value /
output / grad rows, pe = of locations / weights, P = B*Q*M*L*K points,
U = distinct (b, row, m) value rows with at least one in-bounds corner,
N = B*S*M*D grad_value elements; U is computed exactly on the host):
  forward    3*P*pe + B*Q*M*D*e + U*D*e
  backward   3*P*pe + B*Q*M*D*e + U*D*e + 3*P*pe + N*e
             (parameters, upstream gradient and touched value rows read;
             grad_loc / grad_attn written; grad_value written once in full)
Each term belongs to exactly one kernel, so the kernels' shares add up to the
phase: parameters, upstream gradient, value rows and the per-point gradients
to the kernel that writes grad_loc / grad_attn; of grad_value, the rows of
levels summed with atomics that some corner touches to the kernel issuing
those atomics, their untouched rows to the zero fill, the rows of binned
levels to the accumulation, the rows of fp32-scratch levels to the scratch
add (fp32-scratch and pre-reduced levels). Everything else a kernel moves is
reported apart as `overhead_bytes`
(modelled, not measured): the zero fill's rows that atomics or bins later
overwrite, the read of each atomically updated row (U_a*D*e_acc, e_acc = 4
for fp32 rows), the scatter kernel's second read of parameters and upstream
gradient, bin records (8 bytes per in-bounds corner of a binned level, or
per distinct (query, pixel) where the library merges a query's corners on
one pixel, for pixel queries with K = 2 or 4; written by the place / sort
step and read by the accumulation), the count
and sort steps' parameter reads, the accumulation's reads of upstream
gradient rows, the pre-reduction's reads of its levels' parameters (the
locations three times: window placement, count, place; the weights once) and
of the upstream gradient, and its read-modify-write of touched fp32 rows
(counted once per row: a lower bound, as chunks and overlapping windows add
more), and the fp32 scratch's fill, read-modify-writes and read.

Prints one JSON line:
  value / ms_per_step   microseconds per forward+backward step of the headline
                        workload (lower is better): exactly `--steps` steps
                        replayed from HIP graphs of 10 steps each (one-step
                        graphs for a remainder), so each replay's own launch
                        cost is spread over 10 steps
  phases                forward and backward as wholes: algorithmic bytes / device
                        span (first kernel's start to last kernel's end, from
                        the launch-stamped events) against the 8 TB/s peak;
                        each phase alone as a graph replay beside it (a
                        replay adds ROCm's graph launch cost, ~10 us)
  kernels               per kernel: time, algorithmic share, overhead bytes
  roofline              the kernel with the largest time, its algorithmic share
                        per launch / its average launch time
  configs               the same figures for the encoder-shaped workloads
  cpu_baseline          the CPU oracle (fp64 loops, OpenMP) on a bounded sample
                        of the same workload, scaled to one call
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
HEADLINE = "decoder_bf16"
DEFAULT_CONFIGS = ("encoder_fp16", "oddhead_fp32", "large_encoder_bf16")
GRADIENT_KERNELS = ("msda_grad_kernel", "grad_sort_kernel", "msda_bwd_kernel")
# Device-scope no-return atomic adds: about 21.3 G requests/s, one request
# covering up to 16 dwords of one 64-byte segment (atomic_probe_kernel,
# `bench.py --atomic-probe`; profiles/atomic_probe_kernel_request_ceiling.md).
ATOMIC_CEILING_GREQ = 21.3
ATOMIC_KERNELS = ("msda_bwd_kernel", "msda_scatter_kernel", "scatter_accum_kernel")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------- byte accounting

def touched_rows_per_level(inp):
    """Per level l: (U_l, C_l), the distinct (b, row, m) value rows of level l
    that at least one in-bounds corner lands on, and the number of in-bounds
    corners. Host-side accounting of compulsory bytes with the single-rounding
    pixel mapping of the kernels (the product of an fp32 location and an
    integer size is exact in fp64). Levels here never overlap (default level
    starts), so counts over several levels are sums of these."""
    value = inp["value"]
    B, S, M, D = value.shape
    loc_t = inp["sampling_locations"]
    out = []
    m_idx = np.arange(M, dtype=np.int64).reshape(1, M, 1)
    for l, (H, W) in enumerate(inp["spatial_shapes"].tolist()):
        mark = np.zeros(B * H * W * M, dtype=bool)
        corners = 0
        for b in range(B):  # one batch at a time bounds host memory
            lxy = loc_t[b, :, :, l].to(torch.float64).numpy()  # (Q, M, K, 2)
            x0 = np.floor((lxy[..., 0] * W - 0.5).astype(np.float32)).astype(np.int64)
            y0 = np.floor((lxy[..., 1] * H - 0.5).astype(np.float32)).astype(np.int64)
            del lxy
            for dy in (0, 1):
                for dx in (0, 1):
                    xx, yy = x0 + dx, y0 + dy
                    ok = (xx >= 0) & (xx < W) & (yy >= 0) & (yy < H)
                    mark[((b * H * W + yy * W + xx) * M + m_idx)[ok]] = True
                    corners += int(ok.sum())
        out.append((int(mark.sum()), corners))
    return out


def merged_records_per_level(inp):
    """Per level: the bin records when the corners of one query's points
    that fall on one pixel share a record, i.e. the distinct (b, q, m, pixel)
    among the in-bounds corners. A corner (cx, cy) of point k is at
    (x0_k + cx, y0_k + cy); it repeats a corner of an earlier point k' of the
    same (b, q, m) exactly when cx + x0_k - x0_k' and cy + y0_k - y0_k' are
    both 0 or 1."""
    loc_t = inp["sampling_locations"]
    B, Q, M, L, K, _ = loc_t.shape
    out = []
    for l, (H, W) in enumerate(inp["spatial_shapes"].tolist()):
        n = 0
        for b in range(B):
            lxy = loc_t[b, :, :, l].to(torch.float64).numpy()  # (Q, M, K, 2)
            x0 = np.floor((lxy[..., 0] * W - 0.5).astype(np.float32)).astype(np.int64)
            y0 = np.floor((lxy[..., 1] * H - 0.5).astype(np.float32)).astype(np.int64)
            del lxy
            for k in range(K):
                for cy in (0, 1):
                    for cx in (0, 1):
                        xx, yy = x0[..., k] + cx, y0[..., k] + cy
                        keep = (xx >= 0) & (xx < W) & (yy >= 0) & (yy < H)
                        for k2 in range(k):
                            px = cx + x0[..., k] - x0[..., k2]
                            py = cy + y0[..., k] - y0[..., k2]
                            keep &= ~((px >= 0) & (px <= 1) & (py >= 0) & (py <= 1))
                        n += int(keep.sum())
        out.append(n)
    return out


class ByteModel:
    """Algorithmic bytes of one forward and one backward call, their split
    over the kernels, and the modelled overhead traffic (module docstring)."""

    def __init__(self, wl, inp, level_modes, nbins):
        e = torch.finfo(wl.dtype).bits // 8
        pe = torch.finfo(wl.param_dtype or wl.dtype).bits // 8
        B, S, M, D, L, K, Q = wl.B, wl.S, wl.M, wl.D, wl.L, wl.K, wl.num_queries
        self.P = P = B * Q * M * L * K
        self.N = N = B * S * M * D
        t0 = time.perf_counter()
        per = touched_rows_per_level(inp)
        atomic = [l for l, m in enumerate(level_modes) if m == "native"]
        scratch = [l for l, m in enumerate(level_modes) if m == "fp32_scratch"]
        binned = [l for l, m in enumerate(level_modes) if m == "binned"]
        prered = [l for l, m in enumerate(level_modes) if m == "prereduce"]
        self.U, self.C = sum(u for u, _ in per), sum(c for _, c in per)
        U_a = sum(per[l][0] for l in atomic)
        U_s = sum(per[l][0] for l in scratch)
        C_b = sum(per[l][1] for l in binned)
        # records of the binned levels: one per in-bounds corner, or one per
        # distinct (query, pixel) where the library merges (pixel queries,
        # K = 2 or 4, sorted by the count / place chain: above 2048 points
        # per (b, m, level); the one-launch local sort below that keeps all)
        if wl.Q is None and K in (2, 4) and Q * K > 2048 and binned:
            merged = merged_records_per_level(inp)
            C_b = sum(merged[l] for l in binned)
        self.records = C_b
        log(f"byte model: U={self.U} rows, C={self.C} corners, {C_b} binned records, "
            f"{time.perf_counter() - t0:.1f} s")
        U_p = sum(per[l][0] for l in prered)
        rows = lambda lv: sum(B * wl.levels[l][0] * wl.levels[l][1] * M for l in lv)
        N_a, N_s, N_b = rows(atomic) * D, rows(scratch + prered) * D, rows(binned) * D
        P_p = B * Q * M * K * len(prered)
        e_acc = 4 if wl.dtype == torch.float32 else e
        P_a, P_b = B * Q * M * K * len(atomic), B * Q * M * K * len(binned)
        go = B * Q * M * D * e
        self.fwd = 3 * P * pe + go + self.U * D * e
        self.bwd = 3 * P * pe + go + self.U * D * e + 3 * P * pe + N * e
        grad = 3 * P * pe + go + self.U * D * e + 3 * P * pe
        sh = {  # algorithmic share of each kernel
            "msda_fwd_kernel": self.fwd,
            "msda_grad_kernel": grad,
            # (rows of fp32-scratch levels: their grad_value write is the
            # scratch add's; the atomics into the scratch are overhead)
            "msda_bwd_kernel": grad + U_a * D * e,
            "msda_scatter_kernel": U_a * D * e,
            "zero_fill": (N_a - U_a * D) * e,
            "bin_accum_kernel": N_b * e,
            "scratch_add_kernel": N_s * e,
        }
        sh["scatter_accum_kernel"] = sh["msda_scatter_kernel"] + sh["bin_accum_kernel"]
        sh["grad_sort_kernel"] = grad + sh["zero_fill"]
        rec = 8 * C_b
        nt = -(-nbins // 4096)  # scan tiles of 4096 counts
        ov = {  # modelled traffic beyond the share
            "zero_fill": N * e - sh["zero_fill"],
            "msda_bwd_kernel": U_a * D * e_acc + 2 * U_s * D * 4,
            "msda_scatter_kernel": 3 * P_a * pe + go + U_a * D * e_acc + 2 * U_s * D * 4,
            "scratch_zero": N_s * 4, "scratch_add_kernel": N_s * 4,
            "bin_zero": (nbins + 1) * 4, "bin_count": 2 * P_b * pe,
            "bin_scan": 3 * nbins * 4, "bin_tile_sum": nbins * 4,
            "bin_tile_scan": 3 * nbins * 4 + 2 * nt * (nt - 1),  # + the earlier tiles' totals
            "bin_place": 3 * P_b * pe + rec,
            "bin_local_sort": 3 * P_b * pe + rec + 8 * nbins,
            "bin_accum_kernel": rec + go,
            # pre-reduction: its levels' locations read three times and weights
            # once, the upstream gradient, one read-modify-write of every
            # touched fp32 row
            "prereduce_kernel": 7 * P_p * pe + go + 2 * U_p * D * 4,
        }
        ov["scatter_accum_kernel"] = ov["msda_scatter_kernel"] + ov["bin_accum_kernel"]
        # the gradient launch that also sorts and fills
        ov["grad_sort_kernel"] = ov["bin_local_sort"] + ov["zero_fill"]
        self.share, self.overhead = sh, ov
        # atomic requests: one per in-bounds corner per 64-byte segment of
        # its target row (16-bit rows of D*e bytes, fp32 rows of D*4)
        seg16, seg32 = -(-D * e_acc // 64), -(-D * 4 // 64)
        self.atomic_requests = (sum(per[l][1] for l in atomic) * seg16
                                + sum(per[l][1] for l in scratch) * seg32)

    def kernel(self, name):
        return self.share.get(name, 0), self.overhead.get(name, 0)


# ------------------------------------------------------------------- timing

STEPS_PER_GRAPH = 10  # calls captured in one graph: amortises the replay's own launch cost


def capture(fn, calls=1):
    """A HIP graph of `calls` calls of `fn` (after two warm calls on the capture stream)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    return g


def time_replays(g, reps, g_many=None, many=STEPS_PER_GRAPH):
    """Microseconds per call over exactly `reps` calls: replays of `g_many`
    (a graph of `many` calls) while at least `many` calls remain, then of `g`
    (one call)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    left = reps
    while g_many is not None and left >= many:
        g_many.replay()
        left -= many
    for _ in range(left):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps  # us


def kernel_times(call, n_inst):
    """Average device time of every kernel of the forward and of the backward,
    from the library's per-launch events (stamped at kernel start and end),
    and each call's device span: from its first kernel's start to its last
    kernel's end, whichever streams they ran on (averages over n_inst calls).
    Returns (per-kernel us, forward span us, backward span us)."""
    from scale_deformable_attention_amd._binding import (launch_event_names,
                                                         launch_events_recorded,
                                                         set_launch_events)
    nev = 32
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 + nev)] for _ in range(n_inst)]
    for row in evs:
        for ev in row:
            ev.record()  # torch creates the HIP event on first record
    torch.cuda.synchronize()
    names = None
    for i in range(n_inst):
        set_launch_events(evs[i][:2])
        call.forward()
        set_launch_events(evs[i][2:])
        call.backward()
        n_bwd = launch_events_recorded() // 2
        names = launch_event_names()
        assert n_bwd == len(names), (n_bwd, names)
    torch.cuda.synchronize()
    kt = {"msda_fwd_kernel": float(np.mean([r[0].elapsed_time(r[1]) for r in evs])) * 1e3}
    for j, nm in enumerate(names):
        key = nm if nm not in kt else f"{nm}#{j}"
        kt[key] = float(np.mean([r[2 + 2 * j].elapsed_time(r[3 + 2 * j]) for r in evs])) * 1e3
    n = len(names)

    def span(r):  # relative to the first launch's start event
        starts = [r[2].elapsed_time(r[2 + 2 * j]) for j in range(n)]
        stops = [r[2].elapsed_time(r[3 + 2 * j]) for j in range(n)]
        return max(stops) - min(0.0, min(starts))
    bwd_span = float(np.mean([span(r) for r in evs])) * 1e3
    return kt, kt["msda_fwd_kernel"], bwd_span


def kernel_source_hash() -> str:
    """Hash of every source the library is built from (csrc/), by name order."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "scale_deformable_attention_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".cpp", ".h")):
            h.update(name.encode())
            with open(os.path.join(csrc, name), "rb") as f:
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


def frac(nbytes, us):
    gbps = nbytes / (us * 1e-6) / 1e9 if us > 0 else 0.0
    return round(gbps, 1), round(gbps / HBM_PEAK_GBPS, 4)


# --------------------------------------------------------------- cpu oracle

def cpu_baseline(inp, seconds: float):
    """The oracle's forward + backward on a bounded sample of the workload,
    scaled to one call. The sample is the first Q' queries of every batch
    (all of them when a whole call fits the time budget); the per-call fixed
    cost (fp64 conversion of value, the grad_value fill) is timed with zero
    queries and counted once, the rest scaled by Q / Q'."""
    import oracle  # the CPU-baseline leg is the only product-side user of the oracle
    Q = inp["sampling_locations"].shape[1]

    def sub(qn):
        return {k: (v[:, :qn].contiguous() if k in ("sampling_locations", "attention_weights",
                                                    "grad_output") else v)
                for k, v in inp.items()}

    def call(d):
        args = (d["value"], d["spatial_shapes"], None, d["sampling_locations"],
                d["attention_weights"])
        t0 = time.perf_counter()
        oracle.forward(*args)
        oracle.backward(*args, d["grad_output"])
        return time.perf_counter() - t0

    fixed = min(call(sub(0)) for _ in range(2))
    q_probe = min(Q, 64)
    per_q = max(call(sub(q_probe)) - fixed, 1e-9) / q_probe
    q_s = int(min(Q, max(q_probe, (seconds / 2) / per_q)))
    d = sub(q_s)
    times, t_start = [], time.perf_counter()
    while True:
        times.append(call(d))
        if len(times) >= 3 or time.perf_counter() - t_start >= seconds / 2:
            break
    t = float(np.median(times))
    est = t if q_s == Q else fixed + max(t - fixed, 0.0) * Q / q_s
    sample = (f"all {Q} queries" if q_s == Q else f"queries [0, {q_s}) of {Q} per batch, "
              f"scaled by Q/Q' (fixed per-call cost {fixed * 1e3:.0f} ms counted once)")
    return est * 1e6, len(times), oracle.max_threads(), sample


# ------------------------------------------------------------- measurement

def measure(name, accum, steps, warmup, n_inst, headline=False):
    from scale_deformable_attention_amd import PreparedCall
    from scale_deformable_attention_amd.workloads import make_inputs, workload

    wl = workload(name)
    dev = torch.device("cuda:0")
    log(f"workload {wl.name}: B={wl.B} Q={wl.num_queries} S={wl.S} M={wl.M} D={wl.D} "
        f"L={wl.L} K={wl.K} {wl.dtype}")
    inp = make_inputs(wl)
    g = {k: (v.to(dev) if k != "spatial_shapes" else v) for k, v in inp.items()}
    call = PreparedCall(g["value"], g["spatial_shapes"], None, g["sampling_locations"],
                        g["attention_weights"], g["grad_output"], accum=accum)
    log(f"backward accumulation: {accum} -> {call.resolved_accum}")

    def step():
        call.forward()
        call.backward()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    g_step, g_fwd, g_bwd = capture(step), capture(call.forward), capture(call.backward)
    g_steps = capture(step, STEPS_PER_GRAPH)
    us_step = time_replays(g_step, steps, g_steps)
    del g_steps
    fwd_graph_us = time_replays(g_fwd, steps)
    bwd_graph_us = time_replays(g_bwd, steps)
    kt, fwd_us, bwd_us = kernel_times(call, n_inst)
    log(f"{name}: {us_step:.2f} us/step ({steps} steps, graphs of {STEPS_PER_GRAPH}); forward {fwd_us:.2f} us, "
        f"backward {bwd_us:.2f} us (device spans; alone as graph replays {fwd_graph_us:.2f} / "
        f"{bwd_graph_us:.2f} us)")
    log("kernels (us): " + ", ".join(f"{k} {v:.2f}" for k, v in kt.items()))
    modes, nbins = call.plan()
    bm = ByteModel(wl, inp, modes, nbins)
    kernels = {}
    for k, us in kt.items():
        share, over = bm.kernel(k.split("#")[0])
        gbps, fr = frac(share, us)
        kernels[k] = {"us": round(us, 3), "bytes": int(share), "overhead_bytes": int(over),
                      "GBps": gbps, "frac": fr}
    fg, ff = frac(bm.fwd, fwd_us)
    bg, bf = frac(bm.bwd, bwd_us)
    phases = {"forward": {"us": round(fwd_us, 3), "bytes": int(bm.fwd), "GBps": fg, "frac": ff,
                          "graph_replay_us": round(fwd_graph_us, 3)},
              "backward": {"us": round(bwd_us, 3), "bytes": int(bm.bwd), "GBps": bg, "frac": bf,
                           "graph_replay_us": round(bwd_graph_us, 3),
                           "overhead_bytes": int(sum(kernels[k]["overhead_bytes"]
                                                     for k in kernels
                                                     if k != "msda_fwd_kernel")),
                           "kernel_sum_us": round(sum(v for k, v in kt.items()
                                                      if k != "msda_fwd_kernel"), 3)}}
    kname = max(kt, key=kt.get)
    src_hash = kernel_source_hash()
    kshare = kernels[kname]["bytes"]
    roofline = {"bound": "hbm", "achieved": kernels[kname]["GBps"], "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": kernels[kname]["frac"],
                "traffic": load_traffic(wl.name, kname.split("#")[0], src_hash),
                "kernel": kname, "kernel_us": kernels[kname]["us"],
                "algorithmic_bytes_per_launch": int(kshare),
                "kernel_source_sha": src_hash}
    atomic_rate = None
    if kname.split("#")[0] in ATOMIC_KERNELS and bm.atomic_requests:
        rate = bm.atomic_requests / (kt[kname] * 1e-6) / 1e9
        atomic_rate = {"kernel": kname, "requests": int(bm.atomic_requests),
                       "achieved": round(rate, 2), "ceiling": ATOMIC_CEILING_GREQ,
                       "unit": "G requests/s", "frac": round(rate / ATOMIC_CEILING_GREQ, 4)}
    res = {"workload": wl.name, "dtype": str(wl.dtype).replace("torch.", ""),
           "param_dtype": str(wl.param_dtype or wl.dtype).replace("torch.", ""),
           "B": wl.B, "Q": wl.num_queries, "S": wl.S, "M": wl.M, "D": wl.D, "L": wl.L,
           "K": wl.K, "levels": [list(x) for x in wl.levels], "accum": call.resolved_accum,
           "level_modes": modes, "us_per_step": round(us_step, 3), "steps": steps,
           "phases": phases, "kernels": kernels, "roofline": roofline, "atomic_rate": atomic_rate,
           "touched_rows_U": bm.U, "corners_C": bm.C, "points_P": bm.P}
    extra = {"inp": inp, "g": g, "call": call, "step": step, "g_step": g_step, "wl": wl}
    return res, extra


def atomic_probe(reps=20):
    """Request rate of no-return atomic adds (fp32 and packed bf16) for runs of
    1, 4 and 16 dwords per 64-byte segment, on an L2-sized and an HBM-sized
    target; kernel times from the launch-stamped events."""
    from scale_deformable_attention_amd._binding import probe_atomic_requests, set_launch_events
    out = []
    for mib in (4, 64):
        buf = torch.zeros(mib << 18, dtype=torch.float32, device="cuda:0")
        for bf16 in (False, True):
            for run in (1, 4, 16):
                wgs, iters = 4096, 64 if run == 1 else 256
                evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                       for _ in range(reps)]
                for pair in evs:
                    for e in pair:
                        e.record()
                probe_atomic_requests(buf, bf16, run, wgs, iters)  # warm
                torch.cuda.synchronize()
                req = 0
                for pair in evs:
                    set_launch_events(pair)
                    req = probe_atomic_requests(buf, bf16, run, wgs, iters)
                torch.cuda.synchronize()
                us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
                rate = req / (us * 1e-6) / 1e9
                out.append({"target_MiB": mib, "type": "pk_bf16" if bf16 else "f32",
                            "dwords_per_request": run, "requests": req, "us": round(us, 2),
                            "G_requests_per_s": round(rate, 2),
                            "G_dwords_per_s": round(rate * run, 1)})
                log(f"atomic probe {mib} MiB {'pk_bf16' if bf16 else 'f32'} run={run}: "
                    f"{req} requests in {us:.1f} us = {rate:.2f} G requests/s")
        del buf
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--accum", default="auto",
                    choices=["auto", "native", "fp32_scratch", "per_level", "binned", "mixed",
                             "prereduce"])
    ap.add_argument("--configs", default=",".join(DEFAULT_CONFIGS),
                    help="comma-separated workloads measured besides the headline ('none': skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU budget of the headline's oracle sample (each config gets half)")
    ap.add_argument("--profile-only", action="store_true",
                    help="run warmup + timed steps of --workload only (for rocprofv3 runs)")
    ap.add_argument("--foil", action="store_true",
                    help="with --profile-only: also run the point-parallel forward foil")
    ap.add_argument("--atomic-probe", action="store_true",
                    help="measure the atomic request rate instead (measurement kernel)")
    ap.add_argument("--single-stream", action="store_true",
                    help="with --profile-only: backward on the caller's stream only "
                         "(MSDA_FLAG_SINGLE_STREAM), so per-kernel times have no overlap")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="with --profile-only: also run 5 plain device copies of this many MiB "
                         "(reference dispatches for scaling FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; every box here has one, so "
                                   "--gpus must be 1", "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)

    from scale_deformable_attention_amd import PreparedCall, load_library
    from scale_deformable_attention_amd.workloads import make_inputs, workload

    load_library()  # raises if the HIP library is missing
    dev = torch.device("cuda:0")

    if args.atomic_probe:
        rows = atomic_probe()
        print(json.dumps({"atomic_probe": rows}), flush=True)
        return

    if args.profile_only:
        wl = workload(args.workload)
        inp = make_inputs(wl)
        g = {k: (v.to(dev) if k != "spatial_shapes" else v) for k, v in inp.items()}
        call = PreparedCall(g["value"], g["spatial_shapes"], None, g["sampling_locations"],
                            g["attention_weights"], g["grad_output"], accum=args.accum)
        log(f"workload {wl.name}, backward accumulation {args.accum} -> {call.resolved_accum}")
        if args.single_stream:
            from scale_deformable_attention_amd._binding import msda_backward
            bargs = (g["value"], g["spatial_shapes"], None, g["sampling_locations"],
                     g["attention_weights"], g["grad_output"])
        for _ in range(args.warmup + args.steps):
            call.forward()
            if args.single_stream:
                msda_backward(*bargs, accum=args.accum, single_stream=True)
            else:
                call.backward()
        torch.cuda.synchronize()
        log(f"ran {args.warmup} + {args.steps} eager steps")
        if args.foil:
            from scale_deformable_attention_amd._binding import msda_forward_point_parallel
            for _ in range(args.steps):
                msda_forward_point_parallel(g["value"], g["spatial_shapes"], None,
                                            g["sampling_locations"], g["attention_weights"])
            torch.cuda.synchronize()
            log(f"ran {args.steps} point-parallel foil forwards")
        if args.calib_copy_mb:
            n = args.calib_copy_mb * (1 << 20) // 4
            src = torch.ones(n, dtype=torch.float32, device=dev)
            dst = torch.empty_like(src)
            for _ in range(5):
                dst.copy_(src)
            torch.cuda.synchronize()
            log(f"calibration: 5 copies of {args.calib_copy_mb} MiB (read {args.calib_copy_mb} "
                f"MiB, write {args.calib_copy_mb} MiB each)")
        return

    K = args.steps
    head, ex = measure(args.workload, args.accum, K, args.warmup, n_inst=min(K, 50),
                       headline=True)
    wl, call, step, g_step = ex["wl"], ex["call"], ex["step"], ex["g_step"]

    # Context for the headline: eager steps, host enqueue, cold caches, copy bandwidth.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
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
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    n_cold = min(K, 50)
    c_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n_cold)]
    for c0, c1 in c_evs:
        flush.fill_(1.0)  # 1 GiB written: L2 and the 256 MB MALL evicted
        c0.record()
        g_step.replay()
        c1.record()
    torch.cuda.synchronize()
    cold_us = float(np.mean([c0.elapsed_time(c1) for c0, c1 in c_evs])) * 1e3
    cp_dst = torch.empty_like(flush)
    cp_dst.copy_(flush)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        cp_dst.copy_(flush)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 10 * 2 * flush.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del flush, cp_dst
    log(f"eager {eager_us:.2f} us/step, host enqueue {host_us:.2f} us/step, cold {cold_us:.2f} "
        f"us, device copy {copy_gbps:.0f} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle on {wl.name}")
        cpu_us, reps, threads, sample = cpu_baseline(ex["inp"], args.cpu_seconds)
        cpu = {"value": round(cpu_us, 1), "unit": "us/call (fwd+bwd)", "cores": threads,
               "kind": "oracle",
               "sample": f"{wl.name}: {sample}; {reps} timed calls; "
                         f"{platform.processor() or platform.machine()}"}
    del ex

    configs = {}
    names = [] if args.configs in ("", "none") else args.configs.split(",")
    for name in names:
        if name == args.workload:
            continue
        res, cex = measure(name, args.accum, max(10, min(K, 50)), min(args.warmup, 5),
                           n_inst=10)
        if not args.no_cpu_baseline:
            log(f"timing the CPU oracle on {name}")
            cpu_us, reps, threads, sample = cpu_baseline(cex["inp"], args.cpu_seconds / 2)
            res["cpu_baseline"] = {"value": round(cpu_us, 1), "unit": "us/call (fwd+bwd)",
                                   "cores": threads, "kind": "oracle",
                                   "sample": f"{name}: {sample}; {reps} timed calls"}
        del cex
        torch.cuda.empty_cache()
        configs[name] = res

    result = {
        "metric": METRIC, "value": head["us_per_step"], "unit": "us/call (fwd+bwd)",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(head["us_per_step"] / 1e3, 6),
        "higher_is_better": False, "scaling": "weak",
        "vs_baseline": round(head["us_per_step"] / PAGES_DECODER_BF16_US, 4)
        if wl.name == HEADLINE else None,
        "dtype": {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[wl.dtype],
        "data": "synthetic (seeded; stands in for Deformable-DETR COCO inputs)",
        "config": {k: head[k] for k in ("workload", "B", "Q", "S", "M", "D", "L", "K", "levels",
                                        "accum", "param_dtype")} | {"parallelism": "single GPU"},
        "timing": f"graph replay, {STEPS_PER_GRAPH} steps per graph; kernels: launch-stamped events",
        "fwd_us": head["phases"]["forward"]["us"], "bwd_us": head["phases"]["backward"]["us"],
        "phases": head["phases"], "kernels": head["kernels"], "roofline": head["roofline"],
        "atomic_rate": head["atomic_rate"],
        "level_modes": head["level_modes"],
        "touched_rows_U": head["touched_rows_U"], "corners_C": head["corners_C"],
        "points_P": head["points_P"],
        "eager_us_per_step": round(eager_us, 3), "host_enqueue_us": round(host_us, 3),
        "cold_us_per_step": round(cold_us, 3), "cold_flush_bytes": 1 << 30,
        "device_copy_GBps": round(copy_gbps, 1),
        "configs": configs,
    }
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
