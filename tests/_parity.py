"""Parity rule between the HIP path and the CPU oracle.

A slice passes when every element satisfies
    |gpu - oracle| <= tol * (|oracle| + rms(oracle slice)),
with slices = the whole tensor for output and grad_attention_weights, and one
slice per level for grad_value (rows of that level) and
grad_sampling_locations (entries of that level), because magnitudes scale
with W_l, H_l and with how many points share a pixel.

Tolerances (relative): fp32 1e-5 everywhere; fp16 / bf16 2e-2 on output,
grad_sampling_locations and grad_attention_weights, 5e-2 on grad_value.

Exact parts: a grad_value row no in-bounds corner lands on, and an output
row none of whose points has an in-bounds corner, must be exactly zero.

Packed 16-bit atomics round the running sum to the value dtype on every add
(8 significant bits for bf16, 11 for fp16). Where contributions of one
element nearly cancel, the rounding of the large partial sums leaves an
absolute error of up to about one 16-bit ulp of the largest partial sum,
which for such an element can exceed the elementwise bar whatever the order
of the adds (seen: one element in 4.3 M on the decoder's level 1, bf16, at
1.1 contributions per pixel). So on levels accumulated with 16-bit atomics
grad_value may have a few such elements (at most 1e-5 of the level, and at
least one allowed) provided the level's normwise error stays within the same
bar and the cosine above 0.998; on bf16 levels above 4 contributions per
pixel (Q*K*4 / (H*W)), which only forced NATIVE accumulation sends to bf16
atomics, the level is held normwise only. Every level summed in fp32 (fp32
data, fp32 scratch, binned) is held element by element.
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


def to_np(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def check_slice(name: str, got: np.ndarray, ref: np.ndarray, tol: float) -> dict:
    got = got.astype(np.float64).ravel()
    ref = ref.astype(np.float64).ravel()
    if ref.size == 0:
        return {"name": name, "n": 0}
    rms = float(np.sqrt(np.mean(ref * ref)))
    diff = np.abs(got - ref)
    bound = tol * (np.abs(ref) + rms)
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
    if bad.any():
        i = int(np.argmax(np.where(np.isnan(scaled), np.inf, scaled)))
        raise AssertionError(
            f"{name}: {int(bad.sum())}/{ref.size} elements outside tol {tol:g}; worst #{i}: "
            f"gpu={got[i]!r} oracle={ref[i]!r} (max abs {stats['max_abs']:.3e}, "
            f"max scaled {stats['max_scaled']:.3e}, normwise {stats['normwise']:.3e}, "
            f"cos {stats['cos']:.6f})")
    return stats


def level_row_ranges(spatial_shapes, level_start_index=None):
    shp = [tuple(map(int, r)) for r in torch.as_tensor(spatial_shapes).tolist()]
    out, acc = [], 0
    for i, (h, w) in enumerate(shp):
        s = acc if level_start_index is None else int(level_start_index[i])
        out.append((s, s + h * w))
        acc += h * w
    return out


def check_forward(dtype, out_gpu, out_ref, touched=None) -> list:
    got, ref = to_np(out_gpu), np.asarray(out_ref)
    stats = [check_slice("output", got, ref, TOL[dtype]["output"])]
    if touched is not None:
        B, Q, M = touched.shape
        g = got.reshape(B, Q, M, -1)
        untouched = ~touched
        assert np.all(g[untouched] == 0), "output of a query with no in-bounds corner is not exactly 0"
    return stats


def contended_levels(spatial_shapes, Q, K, threshold=4.0) -> tuple:
    """Levels whose pixels receive more than `threshold` contributions on
    average: Q * K * 4 / (H * W)."""
    shp = torch.as_tensor(spatial_shapes).tolist()
    return tuple(l for l, (h, w) in enumerate(shp) if Q * K * 4 / (h * w) > threshold)


def atomic_level_rules(dtype, accum, inp, level_start_index=None) -> dict:
    """check_backward's keyword arguments for the levels that the library
    accumulates with 16-bit atomics on this problem (see the module
    docstring): normwise_levels (bf16, contended) and outlier_levels."""
    if dtype not in (torch.float16, torch.bfloat16):
        return {}
    from scale_deformable_attention_amd._binding import msda_backward_level_modes
    accum = {None: "auto", False: "native", True: "fp32_scratch"}.get(accum, accum)
    modes = msda_backward_level_modes(inp["value"], inp["spatial_shapes"], level_start_index,
                                      inp["sampling_locations"], inp["attention_weights"], accum)
    loc = inp["sampling_locations"]
    hot = contended_levels(inp["spatial_shapes"], loc.shape[1], loc.shape[4])
    native = [l for l, m in enumerate(modes) if m == "native"]
    normwise = tuple(l for l in native if dtype == torch.bfloat16 and l in hot)
    return {"normwise_levels": normwise,
            "outlier_levels": tuple(l for l in native if l not in normwise)}


def _normwise(name, got, want, tol):
    nw = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    cos = float(np.dot(got, want) / max(np.linalg.norm(got) * np.linalg.norm(want), 1e-300))
    assert nw <= tol and cos > 0.998, f"{name} (16-bit atomics): normwise {nw:.3e}, cos {cos:.6f}"
    return nw


def check_grad_value_level(name, got, want, tol, normwise=False, outliers=False) -> dict:
    """One level's grad_value rows: elementwise within `tol`; for a level
    accumulated with 16-bit atomics, normwise only (`normwise`: bf16 on a
    contended level), or at most max(1, 1e-5 n) rounding outliers with the
    normwise bound (`outliers`)."""
    got, want = np.asarray(got).ravel(), np.asarray(want).ravel()
    if normwise:
        nw = _normwise(name, got, want, tol)
        return {"name": name + " normwise", "n": got.size, "max_scaled": float("nan"),
                "normwise": nw}
    if outliers and want.size:
        rms = float(np.sqrt(np.mean(want * want)))
        bad = ~(np.abs(got - want) <= tol * (np.abs(want) + rms))
        if bad.any():
            assert bad.sum() <= max(1, int(1e-5 * want.size)), \
                f"{name}: {int(bad.sum())}/{want.size} elements outside tol (16-bit atomics)"
            nw = _normwise(name, got, want, tol)
            return {"name": name + f" ({int(bad.sum())} rounding outliers)", "n": got.size,
                    "max_scaled": float("nan"), "normwise": nw}
    return check_slice(name, got, want, tol)


def check_backward(dtype, gpu, ref, spatial_shapes, level_start_index=None,
                   touched_rows=None, param_dtype=None, normwise_levels=(),
                   outlier_levels=()) -> list:
    """`param_dtype`: dtype of the locations / weights and their gradients
    when it differs from the value dtype (mixed calls); their tolerances follow
    it, since those gradients are fp32 sums rounded once to it.
    `normwise_levels` / `outlier_levels`: levels accumulated with 16-bit
    atomics (see the module docstring; atomic_level_rules gives both)."""
    gv, gl, ga = (to_np(t) for t in gpu)
    rgv, rgl, rga = ref
    tol = dict(TOL[dtype])
    if param_dtype is not None:
        for k in ("grad_attention_weights", "grad_sampling_locations"):
            tol[k] = TOL[param_dtype][k]
    stats = [check_slice("grad_attention_weights", ga, rga, tol["grad_attention_weights"])]
    for l, (r0, r1) in enumerate(level_row_ranges(spatial_shapes, level_start_index)):
        stats.append(check_grad_value_level(f"grad_value[level {l}]", gv[:, r0:r1],
                                            rgv[:, r0:r1], tol["grad_value"],
                                            normwise=l in normwise_levels,
                                            outliers=l in outlier_levels))
        stats.append(check_slice(f"grad_sampling_locations[level {l}]", gl[:, :, :, l],
                                 rgl[:, :, :, l], tol["grad_sampling_locations"]))
    if touched_rows is not None:
        assert np.all(gv[~touched_rows] == 0), \
            "grad_value row with no in-bounds corner is not exactly 0"
    return stats
