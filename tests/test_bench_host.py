"""Host-side logic of bench.py (no GPU): the touched-row and corner counts
of the byte model against brute force, the split of the algorithmic
bytes (per unit of work: 3e of parameters per point, D·e of output per
(b, q, m), D·e per touched value row; the backward adds the per-point
gradients and the whole grad_value) over the kernels each plan launches, the
counter-file lookup keyed by the library source hash, and the refusal of
more than one GPU."""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from scale_deformable_attention_amd.workloads import Workload, make_inputs  # noqa: E402


def brute_counts(inp):
    """(U_l, C_l) per level by explicit loops over every point and corner."""
    loc = inp["sampling_locations"].to(torch.float64).numpy()
    B, Q, M, L, K, _ = loc.shape
    out = []
    for l, (H, W) in enumerate(inp["spatial_shapes"].tolist()):
        rows, corners = set(), 0
        for b in range(B):
            for q in range(Q):
                for m in range(M):
                    for k in range(K):
                        x = np.floor(np.float32(loc[b, q, m, l, k, 0] * W - 0.5))
                        y = np.floor(np.float32(loc[b, q, m, l, k, 1] * H - 0.5))
                        for dy in (0, 1):
                            for dx in (0, 1):
                                xx, yy = int(x) + dx, int(y) + dy
                                if 0 <= xx < W and 0 <= yy < H:
                                    rows.add((b, yy * W + xx, m))
                                    corners += 1
        out.append((len(rows), corners))
    return out


def small(seed=5, lo=-0.2, hi=1.2, dtype=torch.bfloat16):
    wl = Workload(name="host", dtype=dtype, B=2, Q=23, M=3, D=8, K=3,
                  levels=((5, 7), (3, 4)), loc_kind="uniform", loc_lo=lo, loc_hi=hi, seed=seed)
    return wl, make_inputs(wl)


def test_touched_rows_match_brute_force():
    for seed in (5, 6):
        _, inp = small(seed)
        assert bench.touched_rows_per_level(inp) == brute_counts(inp)


def test_touched_rows_hand_example():
    # one point on the centre of pixel (x=1, y=0) of a 2 x 3 level: x0 = 1,
    # y0 = 0, all four corners (1,0) (2,0) (1,1) (2,1) in bounds: 4 rows and
    # 4 corners; a point left of the level (x0 = -1) keeps its right column
    # only: 2 rows, 2 corners
    shapes = torch.tensor([[2, 3]])
    for (x, y), want in (((1.5 / 3, 0.5 / 2), (4, 4)), ((0.1 / 3, 0.5 / 2), (2, 2))):
        loc = torch.tensor([x, y], dtype=torch.float32).view(1, 1, 1, 1, 1, 2)
        inp = {"value": torch.zeros(1, 6, 1, 4), "spatial_shapes": shapes,
               "sampling_locations": loc}
        assert bench.touched_rows_per_level(inp) == [want]


@pytest.mark.parametrize("modes,kernels", [
    (["native", "native"], ["msda_bwd_kernel", "zero_fill"]),
    (["fp32_scratch", "fp32_scratch"], ["msda_bwd_kernel", "zero_fill", "scratch_add_kernel"]),
    (["binned", "binned"], ["msda_grad_kernel", "bin_accum_kernel"]),
    (["native", "binned"], ["grad_sort_kernel", "scatter_accum_kernel"]),
    (["native", "binned"], ["msda_grad_kernel", "msda_scatter_kernel", "zero_fill",
                            "bin_accum_kernel"]),
    (["native", "prereduce"], ["msda_bwd_kernel", "zero_fill", "scratch_add_kernel"]),
])
def test_kernel_shares_add_up_to_the_backward(modes, kernels):
    """Every plan's kernels together carry exactly the backward's algorithmic
    bytes: each term of the definition goes to one kernel."""
    wl, inp = small()
    bm = bench.ByteModel(wl, inp, modes, nbins=10)
    e, pe = 2, 2
    B, S, M, D, L, K, Q = wl.B, wl.S, wl.M, wl.D, wl.L, wl.K, wl.num_queries
    P = B * Q * M * L * K
    U = sum(u for u, _ in brute_counts(inp))
    assert bm.fwd == 3 * P * pe + B * Q * M * D * e + U * D * e
    assert bm.bwd == 3 * P * pe + B * Q * M * D * e + U * D * e + 3 * P * pe + B * S * M * D * e
    assert sum(bm.kernel(k)[0] for k in kernels) == bm.bwd
    assert bm.kernel("msda_fwd_kernel")[0] == bm.fwd


def test_atomic_requests_count_native_corners():
    """One atomic request per in-bounds corner and 64-byte segment of its
    row: bf16 rows of D = 8 are one segment; fp32 scratch rows of D = 8 too."""
    wl, inp = small()
    counts = brute_counts(inp)
    bm = bench.ByteModel(wl, inp, ["native", "binned"], nbins=10)
    assert bm.atomic_requests == counts[0][1]
    bm = bench.ByteModel(wl, inp, ["fp32_scratch", "native"], nbins=0)
    assert bm.atomic_requests == counts[0][1] + counts[1][1]


def test_counter_files_are_keyed_by_source_hash():
    sha = bench.kernel_source_hash()
    assert len(sha) == 16 and sha == bench.kernel_source_hash()
    files = [f for f in os.listdir(os.path.join(ROOT, "profiles")) if f.endswith("_counters.txt")]
    assert files
    for f in files:
        kernel, workload = None, None
        fields = dict(line.split("=", 1) for line in open(os.path.join(ROOT, "profiles", f))
                      if "=" in line and not line.startswith("#"))
        kernel, workload = fields["kernel "].strip(), fields["workload "].strip()
        assert f == f"{kernel}_{workload}_counters.txt"
        got = bench.load_traffic(workload, kernel, fields["kernel_source_sha "].strip())
        assert got == float(fields["hbm_bytes_per_launch "])
        assert bench.load_traffic(workload, kernel, "0" * 16) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "--gpus must be 1" in r.stdout


def brute_records(inp):
    """Distinct (b, q, m, pixel) among the in-bounds corners, per level."""
    loc = inp["sampling_locations"].to(torch.float64).numpy()
    B, Q, M, L, K, _ = loc.shape
    out = []
    for l, (H, W) in enumerate(inp["spatial_shapes"].tolist()):
        seen = set()
        for b in range(B):
            for q in range(Q):
                for m in range(M):
                    for k in range(K):
                        x = int(np.floor(np.float32(loc[b, q, m, l, k, 0] * W - 0.5)))
                        y = int(np.floor(np.float32(loc[b, q, m, l, k, 1] * H - 0.5)))
                        for dy in (0, 1):
                            for dx in (0, 1):
                                if 0 <= x + dx < W and 0 <= y + dy < H:
                                    seen.add((b, q, m, (y + dy) * W + x + dx))
        out.append(len(seen))
    return out


def test_merged_records_match_brute_force():
    """Pixel queries sampling within a pixel of their own position: many
    points of one query share pixels (and some lie outside the level)."""
    wl = Workload(name="host_px", dtype=torch.float32, B=2, Q=None, M=2, D=8, K=4,
                  levels=((6, 9), (3, 4)), loc_kind="reference", loc_sigma=0.08, seed=3)
    inp = make_inputs(wl)
    got = bench.merged_records_per_level(inp)
    assert got == brute_records(inp)
    counts = brute_counts(inp)
    assert all(r < c for r, (_, c) in zip(got, counts))  # merging happened on every level
