"""Python binding of the C ABI in include/msda.h: argument marshalling only.

Every step of the computation runs in the HIP library (libmsda_amd.so). This
module checks tensor shapes, dtypes and devices, makes inputs contiguous
(course page "4. The forward kernel", section "The wrapper": the wrapper owns
the layout contract), allocates outputs and the optional fp32 workspace with
the PyTorch caching allocator, and passes raw pointers plus the current HIP
stream. There is no CPU fallback: if the library is missing, every call
raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple, Union

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmsda_amd.so")

MSDA_F32, MSDA_F16, MSDA_BF16 = 0, 1, 2
ACCUM_AUTO, ACCUM_NATIVE, ACCUM_FP32_SCRATCH, ACCUM_PER_LEVEL, ACCUM_BINNED, ACCUM_MIXED, \
    ACCUM_PREREDUCE = -1, 0, 1, 2, 3, 4, 5
_RESOLVED = {ACCUM_NATIVE: "native", ACCUM_FP32_SCRATCH: "fp32_scratch", ACCUM_PER_LEVEL: "per_level",
             ACCUM_BINNED: "binned", ACCUM_MIXED: "mixed", ACCUM_PREREDUCE: "prereduce"}
LEVEL_MODES = {0: "native", 1: "fp32_scratch", 2: "binned", 3: "prereduce"}
FLAG_ACCUMULATE_GRAD_VALUE = 1
FLAG_CONTINUE_SCRATCH = 2
FLAG_DEFER_SCRATCH = 4
FLAG_SINGLE_STREAM = 8
MAX_LEVELS = 16

_DTYPE_CODES = {torch.float32: MSDA_F32, torch.float16: MSDA_F16, torch.bfloat16: MSDA_BF16}
_ACCUM_CODES = {"auto": ACCUM_AUTO, None: ACCUM_AUTO, "native": ACCUM_NATIVE, False: ACCUM_NATIVE,
                "fp32_scratch": ACCUM_FP32_SCRATCH, True: ACCUM_FP32_SCRATCH,
                "per_level": ACCUM_PER_LEVEL, "binned": ACCUM_BINNED, "mixed": ACCUM_MIXED,
                "prereduce": ACCUM_PREREDUCE}

# every symbol include/msda.h declares
EXPORTED_SYMBOLS = ("msda_forward", "msda_forward_ex", "msda_forward_point_parallel",
                    "msda_backward", "msda_backward_ex",
                    "msda_backward_workspace_size",
                    "msda_backward_resolve_accum", "msda_backward_plan", "msda_status_string",
                    "msda_last_error",
                    "msda_abi_version", "msda_set_launch_events", "msda_launch_events_recorded",
                    "msda_launch_events_name", "msda_sampling_prep",
                    "msda_sampling_prep_backward", "msda_release_thread_resources",
                    "msda_backward_noalloc", "msda_probe_atomic_requests",
                    "msda_debug_force_flat_gathers")

_lib = None


class MSDAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library {path} is not built; run `python -m scale_deformable_attention_amd.build`"
            " or __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    i64, vp, i32, u32, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t
    prob = [i32, i64, i64, i64, i64, i64, vp, vp, i64, i64]
    lib.msda_forward.argtypes = prob + [vp, vp, vp, vp, vp]
    lib.msda_forward.restype = i32
    lib.msda_forward_ex.argtypes = [i32] + prob + [vp, vp, vp, vp, vp]
    lib.msda_forward_ex.restype = i32
    lib.msda_backward_ex.argtypes = [i32] + prob + [vp, vp, vp, vp, vp, vp, vp, i32, u32, vp, sz, vp]
    lib.msda_backward_ex.restype = i32
    lib.msda_forward_point_parallel.argtypes = prob + [vp, vp, vp, vp, vp]
    lib.msda_forward_point_parallel.restype = i32
    lib.msda_backward.argtypes = prob + [vp, vp, vp, vp, vp, vp, vp, i32, u32, vp, sz, vp]
    lib.msda_backward.restype = i32
    lib.msda_backward_workspace_size.argtypes = prob + [i32]
    lib.msda_backward_workspace_size.restype = sz
    lib.msda_backward_resolve_accum.argtypes = prob + [i32]
    lib.msda_backward_resolve_accum.restype = i32
    lib.msda_backward_plan.argtypes = prob + [i32, ctypes.POINTER(ctypes.c_int)]
    lib.msda_backward_plan.restype = i64
    prep = [i32, i64, i64, i64, i64, i64, vp, i32]
    lib.msda_sampling_prep.argtypes = prep + [vp, vp, vp, vp, vp, vp]
    lib.msda_sampling_prep.restype = i32
    lib.msda_sampling_prep_backward.argtypes = prep + [vp, vp, vp, vp, vp, vp, vp]
    lib.msda_sampling_prep_backward.restype = i32
    lib.msda_status_string.argtypes = [i32]
    lib.msda_status_string.restype = ctypes.c_char_p
    lib.msda_last_error.argtypes = []
    lib.msda_last_error.restype = ctypes.c_char_p
    lib.msda_abi_version.argtypes = []
    lib.msda_abi_version.restype = i32
    lib.msda_set_launch_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), i32]
    lib.msda_set_launch_events.restype = i32
    lib.msda_launch_events_recorded.argtypes = []
    lib.msda_launch_events_recorded.restype = i32
    lib.msda_launch_events_name.argtypes = [i32]
    lib.msda_launch_events_name.restype = ctypes.c_char_p
    lib.msda_backward_noalloc.argtypes = prob + [vp, vp, vp, vp, vp, vp, vp, i32, u32, vp]
    lib.msda_backward_noalloc.restype = i32
    lib.msda_probe_atomic_requests.argtypes = [vp, sz, i32, i32, i64, i32,
                                               ctypes.POINTER(ctypes.c_int64), vp]
    lib.msda_probe_atomic_requests.restype = i32
    lib.msda_release_thread_resources.argtypes = []
    lib.msda_release_thread_resources.restype = i32
    lib.msda_debug_force_flat_gathers.argtypes = [i32]
    lib.msda_debug_force_flat_gathers.restype = i32
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        lib = load_library()
        msg = lib.msda_last_error().decode() or lib.msda_status_string(status).decode()
        raise MSDAError(status, msg)


class _Levels:
    """Host copies of spatial_shapes / level_start_index (the ABI takes host arrays)."""

    def __init__(self, spatial_shapes, level_start_index):
        shp = torch.as_tensor(spatial_shapes).detach().to("cpu", torch.int64).contiguous()
        if shp.dim() != 2 or shp.shape[1] != 2:
            raise ValueError(f"spatial_shapes must be (L, 2), got {tuple(shp.shape)}")
        self.shapes = shp
        self.L = shp.shape[0]
        if level_start_index is None:
            self.starts = None
        else:
            st = torch.as_tensor(level_start_index).detach().to("cpu", torch.int64).contiguous()
            if st.shape != (self.L,):
                raise ValueError(f"level_start_index must be ({self.L},), got {tuple(st.shape)}")
            self.starts = st

    def ptrs(self):
        return (ctypes.c_void_p(self.shapes.data_ptr()),
                None if self.starts is None else ctypes.c_void_p(self.starts.data_ptr()))


def _dims(value: torch.Tensor, levels: _Levels, loc: torch.Tensor, attn: torch.Tensor):
    if value.dim() != 4:
        raise ValueError(f"value must be (B, S, M, D), got {tuple(value.shape)}")
    B, S, M, D = value.shape
    if loc.dim() != 6 or loc.shape[0] != B or loc.shape[2] != M or loc.shape[3] != levels.L \
            or loc.shape[5] != 2:
        raise ValueError(f"sampling_locations must be (B, Q, M, L, K, 2) = ({B}, Q, {M}, "
                         f"{levels.L}, K, 2), got {tuple(loc.shape)}")
    Q, K = loc.shape[1], loc.shape[4]
    if tuple(attn.shape) != (B, Q, M, levels.L, K):
        raise ValueError(f"attention_weights must be {(B, Q, M, levels.L, K)}, got {tuple(attn.shape)}")
    return B, S, M, D, Q, K


def _dtype_code(*tensors: torch.Tensor) -> int:
    dt = tensors[0].dtype
    if dt not in _DTYPE_CODES:
        raise TypeError(f"unsupported dtype {dt}; use float32, float16 or bfloat16")
    dev = tensors[0].device
    for t in tensors:
        if t.dtype != dt:
            raise TypeError(f"all floating tensors must share one dtype, got {dt} and {t.dtype}")
        if t.device != dev:
            raise ValueError(f"all tensors must be on one device, got {dev} and {t.device}")
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a GPU (cuda/hip device), got {dev}")
    return _DTYPE_CODES[dt]


def _dtype_codes(value: torch.Tensor, loc: torch.Tensor, attn: torch.Tensor,
                 *value_typed: torch.Tensor) -> Tuple[int, int]:
    """(value dtype, parameter dtype) codes. Locations and weights share one
    dtype: the value dtype, or float32 beside float16 / bfloat16 values."""
    for t in (value, loc, attn) + value_typed:
        if t.dtype not in _DTYPE_CODES:
            raise TypeError(f"unsupported dtype {t.dtype}; use float32, float16 or bfloat16")
    for t in value_typed:
        if t.dtype != value.dtype:
            raise TypeError(f"grad_output must be {value.dtype}, got {t.dtype}")
    if attn.dtype != loc.dtype:
        raise TypeError(f"sampling_locations and attention_weights must share one dtype, "
                        f"got {loc.dtype} and {attn.dtype}")
    vcode, pcode = _DTYPE_CODES[value.dtype], _DTYPE_CODES[loc.dtype]
    if pcode != vcode and not (pcode == MSDA_F32 and vcode != MSDA_F32):
        raise TypeError(f"sampling_locations / attention_weights must be {value.dtype} or "
                        f"float32 beside 16-bit values, got {loc.dtype}")
    _dtype_code(value, *value_typed)  # device checks
    _dtype_code(loc, attn)
    if loc.device != value.device:
        raise ValueError(f"all tensors must be on one device, got {value.device} and {loc.device}")
    return vcode, pcode


def _stream(device: torch.device, stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return ctypes.c_void_p(handle)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _problem(code, B, S, M, D, levels, Q, K):
    shp, st = levels.ptrs()
    return (code, B, S, M, D, levels.L, shp, st, Q, K)


def msda_forward(value: torch.Tensor, spatial_shapes, level_start_index,
                 sampling_locations: torch.Tensor, attention_weights: torch.Tensor,
                 output: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Forward of the MSDA core; returns (B, Q, M*D) in the value dtype.
    Locations and weights may be float32 beside float16 / bfloat16 values."""
    lib = load_library()
    levels = _Levels(spatial_shapes, level_start_index)
    code, pcode = _dtype_codes(value, sampling_locations, attention_weights)
    value = value.contiguous()
    loc = sampling_locations.contiguous()
    attn = attention_weights.contiguous()
    B, S, M, D, Q, K = _dims(value, levels, loc, attn)
    if output is None:
        output = torch.empty((B, Q, M * D), dtype=value.dtype, device=value.device)
    elif output.shape != (B, Q, M * D) or output.dtype != value.dtype or not output.is_contiguous():
        raise ValueError("output must be a contiguous (B, Q, M*D) tensor of the input dtype")
    _check(lib.msda_forward_ex(code, pcode, *_problem(code, B, S, M, D, levels, Q, K)[1:],
                               _ptr(value), _ptr(loc), _ptr(attn), _ptr(output),
                               _stream(value.device, stream)))
    return output


def msda_forward_point_parallel(value: torch.Tensor, spatial_shapes, level_start_index,
                                sampling_locations: torch.Tensor, attention_weights: torch.Tensor,
                                output: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The point-parallel measurement foil (same result as msda_forward)."""
    lib = load_library()
    levels = _Levels(spatial_shapes, level_start_index)
    code = _dtype_code(value, sampling_locations, attention_weights)
    value = value.contiguous()
    loc = sampling_locations.contiguous()
    attn = attention_weights.contiguous()
    B, S, M, D, Q, K = _dims(value, levels, loc, attn)
    if output is None:
        output = torch.empty((B, Q, M * D), dtype=value.dtype, device=value.device)
    _check(lib.msda_forward_point_parallel(*_problem(code, B, S, M, D, levels, Q, K), _ptr(value),
                                           _ptr(loc), _ptr(attn), _ptr(output),
                                           _stream(value.device, stream)))
    return output


def msda_backward_workspace_size(value: torch.Tensor, spatial_shapes, level_start_index,
                                 sampling_locations: torch.Tensor,
                                 attention_weights: torch.Tensor, accum="auto") -> int:
    lib = load_library()
    levels = _Levels(spatial_shapes, level_start_index)
    code = _DTYPE_CODES[value.dtype]
    B, S, M, D, Q, K = _dims(value, levels, sampling_locations, attention_weights)
    return int(lib.msda_backward_workspace_size(*_problem(code, B, S, M, D, levels, Q, K),
                                                _ACCUM_CODES[accum]))


def msda_backward_resolve_accum(value: torch.Tensor, spatial_shapes, level_start_index,
                                sampling_locations: torch.Tensor,
                                attention_weights: torch.Tensor, accum="auto") -> str:
    lib = load_library()
    levels = _Levels(spatial_shapes, level_start_index)
    code = _DTYPE_CODES[value.dtype]
    B, S, M, D, Q, K = _dims(value, levels, sampling_locations, attention_weights)
    r = int(lib.msda_backward_resolve_accum(*_problem(code, B, S, M, D, levels, Q, K),
                                            _ACCUM_CODES[accum]))
    if r < 0:
        _check(int(MSDAErrorCodes.DTYPE))
    return _RESOLVED[r]


def msda_backward_level_modes(value: torch.Tensor, spatial_shapes, level_start_index,
                              sampling_locations: torch.Tensor, attention_weights: torch.Tensor,
                              accum="auto"):
    """How msda_backward would accumulate each level's grad_value for this
    problem: a list of "native" (atomics of the value dtype), "fp32_scratch"
    or "binned". Host-only (msda_backward_plan)."""
    lib = load_library()
    levels = _Levels(spatial_shapes, level_start_index)
    if value.dtype not in _DTYPE_CODES:
        raise TypeError(f"unsupported dtype {value.dtype}; use float32, float16 or bfloat16")
    code = _DTYPE_CODES[value.dtype]  # the plan depends on the value dtype only
    B, S, M, D, Q, K = _dims(value, levels, sampling_locations, attention_weights)
    if accum not in _ACCUM_CODES:
        raise ValueError(f"unknown accumulation mode {accum!r}")
    modes = (ctypes.c_int * levels.L)()
    nb = int(lib.msda_backward_plan(*_problem(code, B, S, M, D, levels, Q, K),
                                    _ACCUM_CODES[accum], modes))
    if nb < 0:
        raise MSDAError(8, lib.msda_last_error().decode())
    return [LEVEL_MODES[int(m)] for m in modes]


def probe_atomic_requests(buffer: torch.Tensor, bf16: bool, dwords_per_request: int,
                          workgroups: int, iters: int, stream=None) -> int:
    """Launch the atomic request-rate probe (msda_probe_atomic_requests) on
    `buffer` (a device tensor, overwritten); returns the requests it makes."""
    lib = load_library()
    if buffer.device.type != "cuda" or not buffer.is_contiguous():
        raise ValueError("buffer must be a contiguous device tensor")
    req = ctypes.c_int64(0)
    _check(lib.msda_probe_atomic_requests(_ptr(buffer), buffer.numel() * buffer.element_size(),
                                          1 if bf16 else 0, dwords_per_request, workgroups,
                                          iters, ctypes.byref(req),
                                          _stream(buffer.device, stream)))
    return int(req.value)


def release_thread_resources() -> None:
    """Destroy this thread's side streams and events (msda_release_thread_resources)."""
    _check(load_library().msda_release_thread_resources())


class force_flat_gathers:
    """Context manager (tests only): within it, calls address the value slice
    with plain loads, as for batch slices of 2 GiB or more
    (msda_debug_force_flat_gathers); the previous setting comes back on exit."""

    def __enter__(self):
        self._prev = load_library().msda_debug_force_flat_gathers(1)
        return self

    def __exit__(self, *exc):
        load_library().msda_debug_force_flat_gathers(self._prev)
        return False


def set_launch_events(events) -> None:
    """Instrument the next msda_forward / msda_backward call of this thread:
    events[i] (torch.cuda.Event, already created) is recorded on the call's
    stream right after its i-th kernel launch."""
    lib = load_library()
    handles = (ctypes.c_void_p * max(1, len(events)))(*[ctypes.c_void_p(e.cuda_event) for e in events])
    _check(lib.msda_set_launch_events(handles, len(events)))


def launch_events_recorded() -> int:
    return int(load_library().msda_launch_events_recorded())


def launch_event_names():
    """Kernel names of the last instrumented call's launches, in order."""
    lib = load_library()
    n = int(lib.msda_launch_events_recorded()) // 2
    return [lib.msda_launch_events_name(i).decode() for i in range(n)]


class MSDAErrorCodes:
    NULL_ARG, SHAPE, LEVELS, DTYPE, ALIGN, WORKSPACE, HIP, UNSUPPORTED = range(1, 9)


def msda_backward(value: torch.Tensor, spatial_shapes, level_start_index,
                  sampling_locations: torch.Tensor, attention_weights: torch.Tensor,
                  grad_output: torch.Tensor, grad_value: Optional[torch.Tensor] = None,
                  grad_sampling_locations: Optional[torch.Tensor] = None,
                  grad_attention_weights: Optional[torch.Tensor] = None,
                  accum: Union[str, bool, None] = "auto", accumulate: bool = False,
                  workspace: Optional[torch.Tensor] = None, stream=None,
                  continue_scratch: bool = False, defer_scratch: bool = False,
                  single_stream: bool = False
                  ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Backward of the MSDA core: (grad_value, grad_sampling_locations,
    grad_attention_weights). `accum` is "auto", "native", "fp32_scratch",
    "per_level", "binned" or "mixed" (True/False/None are accepted as in the
    pages' fp32_grad_accum switch).
    With `accumulate`, grad_value (given) is added into instead of overwritten.
    `continue_scratch` / `defer_scratch` map to MSDA_FLAG_CONTINUE_SCRATCH /
    MSDA_FLAG_DEFER_SCRATCH (fp32 accumulation across calls in `workspace`);
    `single_stream` to MSDA_FLAG_SINGLE_STREAM (no side stream)."""
    lib = load_library()
    levels = _Levels(spatial_shapes, level_start_index)
    code, pcode = _dtype_codes(value, sampling_locations, attention_weights, grad_output)
    value = value.contiguous()
    loc = sampling_locations.contiguous()
    attn = attention_weights.contiguous()
    gout = grad_output.contiguous()
    B, S, M, D, Q, K = _dims(value, levels, loc, attn)
    if gout.numel() != B * Q * M * D:
        raise ValueError(f"grad_output must hold B*Q*M*D = {B * Q * M * D} elements, got {gout.numel()}")
    if accum not in _ACCUM_CODES:
        raise ValueError(f"accum must be one of {list(_ACCUM_CODES)}, got {accum!r}")

    def out_like(t, ref, name):
        if t is None:
            return torch.empty_like(ref)
        if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor like {tuple(ref.shape)} {ref.dtype}")
        return t

    if accumulate and grad_value is None:
        raise ValueError("accumulate=True needs the grad_value to add into")
    grad_value = out_like(grad_value, value, "grad_value")
    grad_loc = out_like(grad_sampling_locations, loc, "grad_sampling_locations")
    grad_attn = out_like(grad_attention_weights, attn, "grad_attention_weights")
    prob = _problem(code, B, S, M, D, levels, Q, K)
    acode = _ACCUM_CODES[accum]
    need = int(lib.msda_backward_workspace_size(*prob, acode))
    if need and workspace is None:
        if continue_scratch or defer_scratch:
            raise ValueError("continue_scratch / defer_scratch need the caller's workspace")
        workspace = torch.empty(need, dtype=torch.uint8, device=value.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    flags = (FLAG_ACCUMULATE_GRAD_VALUE if accumulate else 0) | \
        (FLAG_CONTINUE_SCRATCH if continue_scratch else 0) | \
        (FLAG_DEFER_SCRATCH if defer_scratch else 0) | (FLAG_SINGLE_STREAM if single_stream else 0)
    _check(lib.msda_backward_ex(code, pcode, *prob[1:], _ptr(value), _ptr(loc), _ptr(attn), _ptr(gout),
                             _ptr(grad_value), _ptr(grad_loc), _ptr(grad_attn), acode, flags,
                             _ptr(workspace), ws_bytes, _stream(value.device, stream)))
    return grad_value, grad_loc, grad_attn


def msda_backward_noalloc(value: torch.Tensor, spatial_shapes, level_start_index,
                          sampling_locations: torch.Tensor, attention_weights: torch.Tensor,
                          grad_output: torch.Tensor, grad_value: torch.Tensor,
                          grad_sampling_locations: torch.Tensor,
                          grad_attention_weights: torch.Tensor, accum="auto",
                          accumulate: bool = False, stream=None) -> None:
    """msda_backward into caller-given outputs with the library's static
    scratch as workspace (msda_backward_noalloc): allocates nothing, so the
    inputs must already be contiguous and in one dtype."""
    lib = load_library()
    levels = _Levels(spatial_shapes, level_start_index)
    code = _dtype_code(value, sampling_locations, attention_weights, grad_output, grad_value,
                       grad_sampling_locations, grad_attention_weights)
    for t in (value, sampling_locations, attention_weights, grad_output, grad_value,
              grad_sampling_locations, grad_attention_weights):
        if not t.is_contiguous():
            raise ValueError("msda_backward_noalloc needs contiguous tensors")
    B, S, M, D, Q, K = _dims(value, levels, sampling_locations, attention_weights)
    if grad_output.numel() != B * Q * M * D or grad_value.shape != value.shape or \
            grad_sampling_locations.shape != sampling_locations.shape or \
            grad_attention_weights.shape != attention_weights.shape:
        raise ValueError("gradient tensors must match their inputs' shapes")
    _check(lib.msda_backward_noalloc(*_problem(code, B, S, M, D, levels, Q, K), _ptr(value),
                                     _ptr(sampling_locations), _ptr(attention_weights),
                                     _ptr(grad_output), _ptr(grad_value),
                                     _ptr(grad_sampling_locations), _ptr(grad_attention_weights),
                                     _ACCUM_CODES[accum],
                                     FLAG_ACCUMULATE_GRAD_VALUE if accumulate else 0,
                                     _stream(value.device, stream)))


class PreparedCall:
    """Pre-marshalled forward/backward calls on fixed tensors.

    Holds the ctypes argument tuples for one problem so that repeated calls
    (training loops, benchmarks, graph capture) cost one foreign call each.
    The tensors must stay alive and keep their storage while this object is
    used; outputs are written in place.
    """

    def __init__(self, value, spatial_shapes, level_start_index, sampling_locations,
                 attention_weights, grad_output=None, accum="auto", stream=None):
        self.lib = load_library()
        levels = _Levels(spatial_shapes, level_start_index)
        code, pcode = _dtype_codes(value, sampling_locations, attention_weights)
        for t in (value, sampling_locations, attention_weights):
            if not t.is_contiguous():
                raise ValueError("PreparedCall needs contiguous tensors")
        B, S, M, D, Q, K = _dims(value, levels, sampling_locations, attention_weights)
        self.levels = levels  # keeps the host arrays alive
        self.value, self.loc, self.attn = value, sampling_locations, attention_weights
        self.output = torch.empty((B, Q, M * D), dtype=value.dtype, device=value.device)
        self.prob = _problem(code, B, S, M, D, levels, Q, K)
        self.device = value.device
        self._stream_arg = stream  # None: torch's current stream at each call (graph capture)
        ex = (code, pcode) + self.prob[1:]  # the _ex entry points' leading arguments
        self._fwd_args = ex + (_ptr(value), _ptr(sampling_locations),
                               _ptr(attention_weights), _ptr(self.output))
        self.accum_code = _ACCUM_CODES[accum]
        self.grad_output = grad_output
        if grad_output is not None:
            if grad_output.numel() != B * Q * M * D or not grad_output.is_contiguous() \
                    or grad_output.dtype != value.dtype:
                raise ValueError("grad_output must be a contiguous (B, Q, M*D) tensor of the input dtype")
            self.grad_value = torch.empty_like(value)
            self.grad_loc = torch.empty_like(sampling_locations)
            self.grad_attn = torch.empty_like(attention_weights)
            need = int(self.lib.msda_backward_workspace_size(*self.prob, self.accum_code))
            self.workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=value.device) \
                if need else None
            self._bwd_head = ex + (_ptr(value), _ptr(sampling_locations),
                                          _ptr(attention_weights), _ptr(grad_output),
                                          _ptr(self.grad_value), _ptr(self.grad_loc),
                                          _ptr(self.grad_attn))
            self._ws = (_ptr(self.workspace), need)
        self.resolved_accum = _RESOLVED.get(
            int(self.lib.msda_backward_resolve_accum(*self.prob, self.accum_code)))

    def plan(self):
        """(per-level accumulation names, number of grad_value bins) of this
        call's backward, as the library plans it."""
        modes = (ctypes.c_int * self.levels.L)()
        nb = int(self.lib.msda_backward_plan(*self.prob, self.accum_code, modes))
        if nb < 0:
            raise MSDAError(8, self.lib.msda_last_error().decode())
        return [LEVEL_MODES[int(m)] for m in modes], nb

    def bin_count(self) -> int:
        """Number of grad_value bins of the binned levels (0 if none)."""
        return self.plan()[1]

    def scratch_levels(self):
        """Levels whose grad_value rows the backward accumulates in fp32 scratch."""
        return [l for l, m in enumerate(self.plan()[0]) if m == "fp32_scratch"]

    def binned_levels(self):
        """Levels whose grad_value rows the backward sums through bins."""
        return [l for l, m in enumerate(self.plan()[0]) if m == "binned"]

    def forward(self) -> torch.Tensor:
        _check(self.lib.msda_forward_ex(*self._fwd_args, _stream(self.device, self._stream_arg)))
        return self.output

    def backward(self, accumulate: bool = False, accum=None, flags: int = 0):
        """One backward call; `flags` adds MSDA_FLAG_* bits (CONTINUE / DEFER scratch)."""
        code = self.accum_code if accum is None else _ACCUM_CODES[accum]
        ws = self._ws if accum is None else (self._ws if code == self.accum_code else (None, 0))
        fl = (FLAG_ACCUMULATE_GRAD_VALUE if accumulate else 0) | flags
        _check(self.lib.msda_backward_ex(*self._bwd_head, code, fl, ws[0], ws[1],
                                      _stream(self.device, self._stream_arg)))
        return self.grad_value, self.grad_loc, self.grad_attn


# ------------------------------------------------ sampling-parameter prep

def _prep_dims(reference_points: torch.Tensor, sampling_offsets: torch.Tensor, L: int):
    if sampling_offsets.dim() != 6 or sampling_offsets.shape[3] != L or \
            sampling_offsets.shape[5] != 2:
        raise ValueError(f"sampling_offsets must be (B, Q, M, {L}, K, 2), "
                         f"got {tuple(sampling_offsets.shape)}")
    B, Q, M, _, K, _ = sampling_offsets.shape
    if tuple(reference_points.shape) == (B, Q, 2):
        per_level = 0
    elif tuple(reference_points.shape) == (B, Q, L, 2):
        per_level = 1
    else:
        raise ValueError(f"reference_points must be ({B}, {Q}, 2) or ({B}, {Q}, {L}, 2), "
                         f"got {tuple(reference_points.shape)}")
    return B, Q, M, K, per_level


def msda_sampling_prep(reference_points: torch.Tensor, sampling_offsets: torch.Tensor,
                       attention_logits: torch.Tensor, spatial_shapes, stream=None):
    """(sampling_locations (B,Q,M,L,K,2), attention_weights (B,Q,M,L,K)) from
    normalised reference points (B,Q,2) or (B,Q,L,2), offsets in pixels of
    each level (B,Q,M,L,K,2) and logits (B,Q,M,L*K) or (B,Q,M,L,K): location =
    reference + offset / (W_l, H_l), weights = softmax over the L*K points."""
    lib = load_library()
    levels = _Levels(spatial_shapes, None)
    B, Q, M, K, per_level = _prep_dims(reference_points, sampling_offsets, levels.L)
    L = levels.L
    if attention_logits.numel() != B * Q * M * L * K or attention_logits.shape[:3] != (B, Q, M):
        raise ValueError(f"attention_logits must be ({B}, {Q}, {M}, {L * K}), "
                         f"got {tuple(attention_logits.shape)}")
    code = _dtype_code(reference_points, sampling_offsets, attention_logits)
    ref = reference_points.contiguous()
    off = sampling_offsets.contiguous()
    logits = attention_logits.contiguous()
    loc = torch.empty_like(off)
    attn = torch.empty((B, Q, M, L, K), dtype=off.dtype, device=off.device)
    _check(lib.msda_sampling_prep(code, B, Q, M, L, K, levels.ptrs()[0], per_level, _ptr(ref),
                                  _ptr(off), _ptr(logits), _ptr(loc), _ptr(attn),
                                  _stream(off.device, stream)))
    return loc, attn


def msda_sampling_prep_backward(attention_weights: torch.Tensor,
                                grad_sampling_locations: torch.Tensor,
                                grad_attention_weights: torch.Tensor, spatial_shapes,
                                ref_per_level: bool = False, need_reference_grad: bool = True,
                                stream=None):
    """(grad_reference_points or None, grad_sampling_offsets (B,Q,M,L,K,2),
    grad_attention_logits (B,Q,M,L*K)) of msda_sampling_prep."""
    lib = load_library()
    levels = _Levels(spatial_shapes, None)
    L = levels.L
    code = _dtype_code(attention_weights, grad_sampling_locations, grad_attention_weights)
    gl = grad_sampling_locations.contiguous()
    if gl.dim() != 6 or gl.shape[3] != L or gl.shape[5] != 2:
        raise ValueError(f"grad_sampling_locations must be (B, Q, M, {L}, K, 2), "
                         f"got {tuple(gl.shape)}")
    B, Q, M, _, K, _ = gl.shape
    a = attention_weights.contiguous()
    ga = grad_attention_weights.contiguous()
    for name, t in (("attention_weights", a), ("grad_attention_weights", ga)):
        if tuple(t.shape) != (B, Q, M, L, K):
            raise ValueError(f"{name} must be {(B, Q, M, L, K)}, got {tuple(t.shape)}")
    g_off = torch.empty_like(gl)
    g_logits = torch.empty((B, Q, M, L * K), dtype=gl.dtype, device=gl.device)
    g_ref = None
    if need_reference_grad:
        shape = (B, Q, L, 2) if ref_per_level else (B, Q, 2)
        g_ref = torch.empty(shape, dtype=gl.dtype, device=gl.device)
    _check(lib.msda_sampling_prep_backward(code, B, Q, M, L, K, levels.ptrs()[0],
                                           1 if ref_per_level else 0, _ptr(a), _ptr(gl), _ptr(ga),
                                           _ptr(g_ref), _ptr(g_off), _ptr(g_logits),
                                           _stream(gl.device, stream)))
    return g_ref, g_off, g_logits
