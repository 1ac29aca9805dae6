"""CPU oracle for the MSDA sampling/aggregation core (forward and backward).

TEST INFRASTRUCTURE ONLY. Only `tests/`, `__graft_entry__.smoke()` and the
CPU-baseline leg of `bench.py` may import this package. The product path (the
HIP library and its Python binding) never calls it and shares no code with it.

The arithmetic lives in `msda_oracle.c` (plain fp64 loops; see its header for
the sources on the web pages and the readings taken). This module only
marshals arrays: every float input is converted exactly to fp64 (all of
fp32/fp16/bf16 embed exactly in fp64), every output comes back as fp64.

Modes:
    "pinned_f32"  pixel mapping x = fmaf(loc_x, W, -0.5f) in fp32, as the pages'
                  kernel computes it; used for all parity against the GPU.
    "exact_f64"   pixel mapping in fp64; used for finite differences and the
                  grid_sample cross-check.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmsda_oracle.so")

MODES = {"pinned_f32": 0, "exact_f64": 1}
_ERRORS = {1: "bad size argument", 2: "bad level table (shape < 1 or level outside S)",
           3: "non-finite sampling location", 4: "out of memory"}

_lib = None


def build(verbose: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (plain C99 + OpenMP, no fp contraction)."""
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", "-o", out + ".tmp",
           src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # MSDA_ORACLE_LIB lets the mutation test point the pins at a planted-mistake copy.
    path = os.environ.get("MSDA_ORACLE_LIB", _LIB_PATH)
    if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(path)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    common = [i64, i64, i64, i64, i64, vp, vp, i64, i64]
    lib.msda_oracle_forward.argtypes = common + [vp, vp, vp, vp, vp, i32, i32]
    lib.msda_oracle_forward.restype = i32
    lib.msda_oracle_backward.argtypes = common + [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32]
    lib.msda_oracle_backward.restype = i32
    lib.msda_oracle_scatter_stats.argtypes = common + [vp, vp, vp, vp, vp, i32, i32]
    lib.msda_oracle_scatter_stats.restype = i32
    lib.msda_oracle_max_threads.argtypes = []
    lib.msda_oracle_max_threads.restype = i32
    _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor: exact upcast on the CPU
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dims(value, spatial_shapes, loc):
    B, S, M, D = value.shape
    L = spatial_shapes.shape[0]
    if loc.ndim != 6 or loc.shape[0] != B or loc.shape[2] != M or loc.shape[3] != L \
            or loc.shape[5] != 2:
        raise ValueError(f"sampling_locations shape {loc.shape} does not match value "
                         f"{value.shape} and {L} levels")
    Q, K = loc.shape[1], loc.shape[4]
    return B, S, M, D, L, Q, K


def max_threads() -> int:
    return int(_load().msda_oracle_max_threads())


def forward(value, spatial_shapes, level_start_index, sampling_locations,
            attention_weights, mode: str = "pinned_f32", num_threads: int = 0,
            return_touched: bool = False):
    """out (B, Q, M*D) fp64 [, touched (B, Q, M) bool]."""
    lib = _load()
    v, loc, a = _f64(value), _f64(sampling_locations), _f64(attention_weights)
    shp = _i64(spatial_shapes).reshape(-1, 2)
    st = None if level_start_index is None else _i64(level_start_index)
    B, S, M, D, L, Q, K = _dims(v, shp, loc)
    out = np.zeros((B, Q, M, D), dtype=np.float64)
    touched = np.zeros((B, Q, M), dtype=np.uint8) if return_touched else None
    rc = lib.msda_oracle_forward(B, S, M, D, L, _ptr(shp), _ptr(st), Q, K, _ptr(v),
                                 _ptr(loc), _ptr(a), _ptr(out), _ptr(touched),
                                 MODES[mode], num_threads)
    if rc:
        raise ValueError(f"oracle forward: {_ERRORS.get(rc, rc)}")
    out = out.reshape(B, Q, M * D)
    return (out, touched.astype(bool)) if return_touched else out


def backward(value, spatial_shapes, level_start_index, sampling_locations,
             attention_weights, grad_output, mode: str = "pinned_f32",
             num_threads: int = 0, return_touched: bool = False):
    """(grad_value, grad_sampling_locations, grad_attention_weights) in fp64
    [, touched_rows (B, S, M) bool]."""
    lib = _load()
    v, loc, a = _f64(value), _f64(sampling_locations), _f64(attention_weights)
    g = _f64(grad_output)
    shp = _i64(spatial_shapes).reshape(-1, 2)
    st = None if level_start_index is None else _i64(level_start_index)
    B, S, M, D, L, Q, K = _dims(v, shp, loc)
    if g.size != B * Q * M * D:
        raise ValueError(f"grad_output has {g.size} elements, expected {B * Q * M * D}")
    gv = np.empty_like(v)
    gl = np.zeros_like(loc)
    ga = np.zeros(loc.shape[:-1], dtype=np.float64)
    touched = np.zeros((B, S, M), dtype=np.uint8) if return_touched else None
    rc = lib.msda_oracle_backward(B, S, M, D, L, _ptr(shp), _ptr(st), Q, K, _ptr(v),
                                  _ptr(loc), _ptr(a), _ptr(g), _ptr(gv), _ptr(gl),
                                  _ptr(ga), _ptr(touched), MODES[mode], num_threads)
    if rc:
        raise ValueError(f"oracle backward: {_ERRORS.get(rc, rc)}")
    res = (gv, gl, ga)
    return res + (touched.astype(bool),) if return_touched else res


def scatter_stats(spatial_shapes, level_start_index, sampling_locations, attention_weights,
                  grad_output, num_keys: int, head_dim: int, mode: str = "pinned_f32",
                  num_threads: int = 0):
    """Per grad_value element, the sum of the absolute values of the terms
    A * w_ij * g[d] that the scatter adds into it, and per (b, row, m) row the
    number of those terms (in-bounds corners landing on the row).

    Returns (abs_sum (B, S, M, D) fp64, count (B, S, M) int64). With them a
    sum of `count` terms, each rounded once to a type with unit roundoff u and
    added with one rounding per add in any order, is within
    gamma(count) * abs_sum of the exact sum, gamma(n) = n*u / (1 - n*u)
    (course page "5. The backward kernel", section "Atomics make gradients
    nondeterministic", for why half-precision atomics round on each add)."""
    lib = _load()
    loc, a, g = _f64(sampling_locations), _f64(attention_weights), _f64(grad_output)
    shp = _i64(spatial_shapes).reshape(-1, 2)
    st = None if level_start_index is None else _i64(level_start_index)
    if loc.ndim != 6 or loc.shape[3] != shp.shape[0] or loc.shape[5] != 2:
        raise ValueError(f"sampling_locations shape {loc.shape} does not match "
                         f"{shp.shape[0]} levels")
    B, Q, M, L, K, _ = loc.shape
    S, D = int(num_keys), int(head_dim)
    if g.size != B * Q * M * D:
        raise ValueError(f"grad_output has {g.size} elements, expected {B * Q * M * D}")
    abs_sum = np.empty((B, S, M, D), dtype=np.float64)
    count = np.empty((B, S, M), dtype=np.int64)
    rc = lib.msda_oracle_scatter_stats(B, S, M, D, L, _ptr(shp), _ptr(st), Q, K, _ptr(loc),
                                       _ptr(a), _ptr(g), _ptr(abs_sum), _ptr(count),
                                       MODES[mode], num_threads)
    if rc:
        raise ValueError(f"oracle scatter_stats: {_ERRORS.get(rc, rc)}")
    return abs_sum, count
