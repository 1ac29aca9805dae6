"""Parity rule between the HIP path and the CPU oracle.

A slice passes when every element satisfies
    |gpu - oracle| <= tol * (|oracle| + rms(oracle slice)) [+ rounding term],
with slices = the whole tensor for output and grad_attention_weights, and one
slice per level for grad_value (rows of that level) and
grad_sampling_locations (entries of that level), because magnitudes scale
with W_l, H_l and with how many points share a pixel.

Tolerances (relative): fp32 1e-5 everywhere; fp16 / bf16 2e-2 on output,
grad_sampling_locations and grad_attention_weights, 5e-2 on grad_value.

Exact parts: a grad_value row no in-bounds corner lands on, and an output
row none of whose points has an in-bounds corner, must be exactly zero.

Rounding term (grad_value levels summed with packed 16-bit atomics only).
Such a sum rounds every term to the 16-bit type and every add to it, in an
order that changes from run to run (course page "5. The backward kernel",
section "Atomics make gradients nondeterministic"). For n terms c_i added one
by one with unit roundoff u, in any order, the standard bound on recursive
summation gives |fl(sum) - sum| <= gamma(n) * sum |c_i|, gamma(n) =
n*u / (1 - n*u): each of the n term roundings errs by at most u|c_i| and each
of the n-1 add roundings by at most u times a partial sum, itself at most
sum |c_i|. The oracle exports, per element, sum |c_i| and n
(oracle.scatter_stats); u = 2^-8 for bf16 (8 significant bits), 2^-11 for
fp16 (11), and each rounding may also err by half the spacing of the
type's subnormals (2^-25 for fp16, 2^-134 for bf16), so an element's
rounding term is gamma(n) * sum|c_i| + 2 n * that. It is added to the bar
above on those levels only; every level summed in fp32 (fp32 data, fp32
scratch, binned, pre-reduced) is held to the bar alone. Which levels a call accumulates
with 16-bit atomics is derived here from the documented policy
(expected_level_modes) and the library's own report must equal it, so a
wrong plan fails the test instead of loosening it.
"""

from __future__ import annotations

import numpy as np
import torch

TOL = {
    torch.float32: {"output": 1e-5, "grad_value": 1e-5, "grad_sampling_locations": 1e-5,
                    "grad_attention_weights": 1e-5},
    torch.float16: {"output": 2e-2, "grad_value": 5e-2, "grad_sampling_locations": 2e-2,
                    "grad_attention_weights": 2e-2},
    torch.bfloat16: {"output": 2e-2, "grad_value": 5e-2, "grad_sampling_locations": 2e-2,
                     "grad_attention_weights": 2e-2},
}

# unit roundoff and half the subnormal spacing of the 16-bit types
UNIT_ROUNDOFF = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}
SUBNORMAL_HALF_SPACING = {torch.bfloat16: 2.0 ** -134, torch.float16: 2.0 ** -25}

# Contributions per pixel (Q * K * 4 / (H * W)) above which a level counts as
# contended, and above which PREREDUCE sums it in LDS (include/msda.h,
# msda_accum_t).
CONTENDED = 4.0
PREREDUCED = 256.0

# The per-level plan of every named workload under each accumulation mode, as
# include/msda.h's policy gives it (contributions per pixel in comments).
WORKLOAD_PLANS = {
    # 1.6, 6.4
    "tiny_fp32": {"auto": ["native", "binned"], "mixed": ["native", "binned"],
                  "binned": ["binned", "binned"], "native": ["native", "native"],
                  "fp32_scratch": ["native", "native"], "per_level": ["native", "native"],
                  "prereduce": ["native", "binned"]},
    # 0.29, 1.14, 4.57, 17.6
    "decoder_bf16": {"auto": ["native", "native", "binned", "binned"],
                     "mixed": ["native", "native", "binned", "binned"],
                     "binned": ["binned"] * 4, "native": ["native"] * 4,
                     "fp32_scratch": ["fp32_scratch"] * 4,
                     "per_level": ["native", "native", "fp32_scratch", "fp32_scratch"],
                     "prereduce": ["native", "native", "binned", "binned"]},
    # 21.3, 84.7, 339, 1302
    "encoder_fp16": {"auto": ["binned"] * 4, "mixed": ["binned"] * 4, "binned": ["binned"] * 4,
                     "native": ["native"] * 4, "fp32_scratch": ["fp32_scratch"] * 4,
                     "per_level": ["fp32_scratch"] * 4,
                     "prereduce": ["binned", "binned", "prereduce", "prereduce"]},
    # 0.43, 1.72, 6.86, 27.4
    "oddhead_fp32": {"auto": ["native", "native", "binned", "binned"],
                     "mixed": ["native", "native", "binned", "binned"],
                     "binned": ["binned"] * 4, "native": ["native"] * 4,
                     "fp32_scratch": ["native"] * 4, "per_level": ["native"] * 4,
                     "prereduce": ["native", "native", "binned", "binned"]},
    # 21.2, 85.0, 340, 1360
    "large_encoder_bf16": {"auto": ["binned"] * 4, "mixed": ["binned"] * 4,
                           "binned": ["binned"] * 4, "native": ["native"] * 4,
                           "fp32_scratch": ["fp32_scratch"] * 4,
                           "per_level": ["fp32_scratch"] * 4,
                           "prereduce": ["binned", "binned", "prereduce", "prereduce"]},
}
WORKLOAD_PLANS["decoder_mixed"] = WORKLOAD_PLANS["decoder_bf16"]
WORKLOAD_PLANS["encoder_mixed"] = WORKLOAD_PLANS["encoder_fp16"]


def to_np(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def accum_name(accum) -> str:
    """The pages' fp32_grad_accum tri-state or a mode name, as a mode name."""
    return {None: "auto", False: "native", True: "fp32_scratch"}.get(accum, accum)


def level_row_ranges(spatial_shapes, level_start_index=None):
    shp = [tuple(map(int, r)) for r in torch.as_tensor(spatial_shapes).tolist()]
    out, acc = [], 0
    for i, (h, w) in enumerate(shp):
        s = acc if level_start_index is None else int(level_start_index[i])
        out.append((s, s + h * w))
        acc += h * w
    return out


def contended_levels(spatial_shapes, Q, K, threshold=CONTENDED) -> tuple:
    """Levels whose pixels receive more than `threshold` contributions on
    average: Q * K * 4 / (H * W)."""
    shp = torch.as_tensor(spatial_shapes).tolist()
    return tuple(l for l, (h, w) in enumerate(shp) if Q * K * 4 / (h * w) > threshold)


def binning_applies(dtype, B, S, M, D, Q, K, L, spatial_shapes, level_start_index=None) -> bool:
    """The conditions include/msda.h states for BINNED / MIXED: levels that do
    not overlap and batch slices of value and grad_output below 2 GiB (plus
    the record-index limits, far above every tested size)."""
    e = torch.finfo(dtype).bits // 8
    rng = level_row_ranges(spatial_shapes, level_start_index)
    overlap = any(a0 < b1 and b0 < a1 for i, (a0, a1) in enumerate(rng)
                  for (b0, b1) in rng[i + 1:])
    lim = 2 ** 31 - 64
    return (not overlap and S * M * D * e <= lim and Q * M * D * e <= lim and Q < 2 ** 28
            and 4 * B * Q * M * L * K < 2 ** 32)


def expected_level_modes(dtype, accum, spatial_shapes, B, S, M, D, Q, K,
                         level_start_index=None, flat=False) -> list:
    """Per-level accumulation ("native", "fp32_scratch", "binned" or
    "prereduce") that include/msda.h's policy gives for this call."""
    accum = accum_name(accum)
    L = len(torch.as_tensor(spatial_shapes).tolist())
    hot = set(contended_levels(spatial_shapes, Q, K))
    # flat: the plain-load path is forced (msda_debug_force_flat_gathers), which
    # plans as for a value slice of 2 GiB or more: no binning
    bins = not flat and binning_applies(dtype, B, S, M, D, Q, K, L, spatial_shapes,
                                        level_start_index)
    half = dtype != torch.float32
    if accum == "prereduce":
        assert bins and D <= 256, "PREREDUCE does not apply to this problem"
        very = set(contended_levels(spatial_shapes, Q, K, PREREDUCED))
        return ["prereduce" if l in very else "binned" if l in hot else "native"
                for l in range(L)]
    if accum in ("auto", "mixed") and bins:
        return ["binned" if l in hot else "native" for l in range(L)]
    if accum == "binned":
        assert bins, "BINNED does not apply to this problem"
        return ["binned"] * L
    assert accum != "mixed", "MIXED does not apply to this problem"
    if accum == "auto":
        accum = "per_level" if dtype == torch.bfloat16 else "native"
    if accum == "fp32_scratch" and half:
        return ["fp32_scratch"] * L
    if accum == "per_level" and half:
        return ["fp32_scratch" if l in hot else "native" for l in range(L)]
    return ["native"] * L


def plan_for(dtype, accum, inp, level_start_index=None, workload_name=None, flat=False) -> list:
    """The expected per-level plan of a call on `inp`; for a named workload
    also the hard-coded table entry, which must agree."""
    v, loc = inp["value"], inp["sampling_locations"]
    B, S, M, D = v.shape
    Q, K = loc.shape[1], loc.shape[4]
    modes = expected_level_modes(dtype, accum, inp["spatial_shapes"], B, S, M, D, Q, K,
                                 level_start_index, flat)
    if workload_name is not None:
        table = WORKLOAD_PLANS[workload_name][accum_name(accum)]
        assert modes == table, (workload_name, accum, modes, table)
    return modes


def assert_library_plan(modes, inp, accum, level_start_index=None):
    """The library's own report of its plan must equal the expected one."""
    from scale_deformable_attention_amd._binding import msda_backward_level_modes
    got = msda_backward_level_modes(inp["value"], inp["spatial_shapes"], level_start_index,
                                    inp["sampling_locations"], inp["attention_weights"],
                                    accum_name(accum))
    assert list(got) == list(modes), f"library plan {got} != expected {modes}"


def needs_rounding_stats(dtype, modes) -> bool:
    return dtype in UNIT_ROUNDOFF and "native" in modes


def rounding_stats(inp, level_start_index=None, grad_output=None):
    """oracle.scatter_stats on the call's inputs: (abs_sum, count)."""
    import oracle
    v = inp["value"]
    return oracle.scatter_stats(inp["spatial_shapes"], level_start_index,
                                inp["sampling_locations"], inp["attention_weights"],
                                inp["grad_output"] if grad_output is None else grad_output,
                                v.shape[1], v.shape[3])


def rounding_term(dtype, abs_sum, count, passes: int = 1) -> np.ndarray:
    """Bound on the error of a sum made with packed 16-bit atomics, per
    element (module docstring). `passes` calls that each add the same terms
    into one buffer (the accumulate flag) count as passes * n terms whose
    absolute values sum to passes * abs_sum."""
    u = UNIT_ROUNDOFF[dtype]
    n = passes * np.asarray(count, dtype=np.float64)
    nu = n * u
    gamma = np.where(nu < 1.0, nu / np.maximum(1.0 - nu, 1e-300), np.inf)
    return (gamma[..., None] * passes * abs_sum
            + 2.0 * n[..., None] * SUBNORMAL_HALF_SPACING[dtype])


def check_slice(name: str, got: np.ndarray, ref: np.ndarray, tol: float,
                extra: np.ndarray = None) -> dict:
    got = got.astype(np.float64).ravel()
    ref = ref.astype(np.float64).ravel()
    if ref.size == 0:
        return {"name": name, "n": 0}
    rms = float(np.sqrt(np.mean(ref * ref)))
    diff = np.abs(got - ref)
    bound = tol * (np.abs(ref) + rms)
    if extra is not None:
        bound = bound + np.asarray(extra, dtype=np.float64).ravel()
    bad = ~(diff <= bound)  # NaN counts as bad
    scaled = diff / np.maximum(np.abs(ref) + rms, 1e-300)
    denom = float(np.linalg.norm(ref))
    stats = {
        "name": name, "n": int(ref.size), "max_abs": float(np.nanmax(diff)),
        "max_scaled": float(np.nanmax(scaled)), "rms_ref": rms,
        "normwise": float(np.linalg.norm(got - ref) / denom) if denom > 0 else 0.0,
        "cos": float(np.dot(got, ref) / (np.linalg.norm(got) * denom))
        if denom > 0 and np.linalg.norm(got) > 0 else 1.0,
    }
    if extra is not None:
        stats["name"] = name + " (+16-bit rounding term)"
        stats["past_plain_bar"] = int((~(diff <= tol * (np.abs(ref) + rms))).sum())
    if bad.any():
        i = int(np.argmax(np.where(np.isnan(scaled), np.inf, diff - bound)))
        raise AssertionError(
            f"{name}: {int(bad.sum())}/{ref.size} elements outside the bound (tol {tol:g}"
            f"{', + rounding term' if extra is not None else ''}); worst #{i}: "
            f"gpu={got[i]!r} oracle={ref[i]!r} bound={bound[i]!r} (max abs "
            f"{stats['max_abs']:.3e}, max scaled {stats['max_scaled']:.3e}, normwise "
            f"{stats['normwise']:.3e}, cos {stats['cos']:.6f})")
    return stats


def check_forward(dtype, out_gpu, out_ref, touched=None) -> list:
    got, ref = to_np(out_gpu), np.asarray(out_ref)
    stats = [check_slice("output", got, ref, TOL[dtype]["output"])]
    if touched is not None:
        B, Q, M = touched.shape
        g = got.reshape(B, Q, M, -1)
        untouched = ~touched
        assert np.all(g[untouched] == 0), "output of a query with no in-bounds corner is not exactly 0"
    return stats


def check_grad_value(dtype, gv, rgv, spatial_shapes, level_start_index=None, modes=None,
                     stats=None, passes: int = 1, tol=None) -> list:
    """grad_value level by level; levels whose mode is "native" in a 16-bit
    dtype also get the rounding term (stats = oracle.scatter_stats)."""
    tol = TOL[dtype]["grad_value"] if tol is None else tol
    out = []
    for l, (r0, r1) in enumerate(level_row_ranges(spatial_shapes, level_start_index)):
        extra = None
        if modes is not None and modes[l] == "native" and dtype in UNIT_ROUNDOFF:
            assert stats is not None, "16-bit atomic level needs oracle.scatter_stats"
            abs_sum, count = stats
            extra = rounding_term(dtype, abs_sum[:, r0:r1], count[:, r0:r1], passes)
        out.append(check_slice(f"grad_value[level {l}]", gv[:, r0:r1], rgv[:, r0:r1], tol,
                               extra))
    return out


def check_backward(dtype, gpu, ref, spatial_shapes, level_start_index=None,
                   touched_rows=None, param_dtype=None, modes=None, stats=None) -> list:
    """`param_dtype`: dtype of the locations / weights and their gradients
    when it differs from the value dtype (mixed calls); their tolerances follow
    it, since those gradients are fp32 sums rounded once to it.
    `modes`: the call's expected per-level plan (expected_level_modes);
    `stats`: oracle.scatter_stats of the call, needed when a 16-bit level is
    accumulated with atomics."""
    gv, gl, ga = (to_np(t) for t in gpu)
    rgv, rgl, rga = ref
    tol = dict(TOL[dtype])
    if param_dtype is not None:
        for k in ("grad_attention_weights", "grad_sampling_locations"):
            tol[k] = TOL[param_dtype][k]
    out = [check_slice("grad_attention_weights", ga, rga, tol["grad_attention_weights"])]
    out += check_grad_value(dtype, gv, rgv, spatial_shapes, level_start_index, modes, stats)
    for l, _ in enumerate(level_row_ranges(spatial_shapes, level_start_index)):
        out.append(check_slice(f"grad_sampling_locations[level {l}]", gl[:, :, :, l],
                               rgl[:, :, :, l], tol["grad_sampling_locations"]))
    if touched_rows is not None:
        assert np.all(gv[~touched_rows] == 0), \
            "grad_value row with no in-bounds corner is not exactly 0"
    return out


def parity_kwargs(dtype, accum, inp, level_start_index=None, workload_name=None,
                  check_library=True, grad_output=None, flat=False) -> dict:
    """check_backward's `modes` and `stats` for a call on `inp`: the expected
    plan (checked against the library's report) and, when some level is
    accumulated with 16-bit atomics, the oracle's rounding statistics."""
    modes = plan_for(dtype, accum, inp, level_start_index, workload_name, flat)
    if check_library:
        assert_library_plan(modes, inp, accum, level_start_index)
    stats = rounding_stats(inp, level_start_index, grad_output) \
        if needs_rounding_stats(dtype, modes) else None
    return {"modes": modes, "stats": stats}
