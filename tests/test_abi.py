"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/msda.h declares, and
reject every bad argument with its status code before any HIP call. No call
here reaches a kernel launch: each one either fails validation or has an
empty batch / query set.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msda.h")

from scale_deformable_attention_amd import _binding as bind  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bind.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return bind.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msda_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_match_binding_list():
    assert _declared_functions() == sorted(bind.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), f"{name} not exported"
    assert lib.msda_abi_version() == 1


def test_status_strings(lib):
    for code in range(9):
        assert lib.msda_status_string(code).decode()
    assert lib.msda_status_string(99).decode() == "unknown status"


# A valid small problem: two levels (8,10), (4,5) -> S = 100.
SHAPES = (ctypes.c_int64 * 4)(8, 10, 4, 5)
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below stops before a launch


def fwd(lib, dtype=0, B=1, S=100, M=2, D=8, L=2, shapes=SHAPES, starts=None, Q=16, K=2,
        value=FAKE, loc=FAKE, attn=FAKE, out=FAKE):
    return lib.msda_forward(dtype, B, S, M, D, L, shapes, starts, Q, K, value, loc, attn, out, None)


def bwd(lib, dtype=0, B=1, S=100, M=2, D=8, L=2, shapes=SHAPES, starts=None, Q=16, K=2,
        accum=-1, flags=0, ws=None, ws_bytes=0, gv=FAKE, gout=FAKE):
    return lib.msda_backward(dtype, B, S, M, D, L, shapes, starts, Q, K, FAKE, FAKE, FAKE, gout,
                             gv, FAKE, FAKE, accum, flags, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), 4),
    (dict(B=-1), 2),
    (dict(Q=-1), 2),
    (dict(M=0), 2),
    (dict(D=0), 2),
    (dict(K=0), 2),
    (dict(L=0), 2),
    (dict(L=17), 8),
    (dict(shapes=None), 1),
    (dict(S=99), 3),  # levels need 100 rows
    (dict(shapes=(ctypes.c_int64 * 4)(8, 10, 0, 5)), 3),
    (dict(shapes=(ctypes.c_int64 * 4)(1 << 24, 1, 4, 5), S=(1 << 24) + 20), 8),
    (dict(starts=(ctypes.c_int64 * 2)(0, 90)), 3),
    (dict(starts=(ctypes.c_int64 * 2)(-1, 80)), 3),
    (dict(value=None), 1),
    (dict(loc=None), 1),
    (dict(attn=None), 1),
    (dict(out=None), 1),
    (dict(value=ctypes.c_void_p(0x10002)), 5),
    (dict(dtype=2, out=ctypes.c_void_p(0x10001)), 5),
    (dict(D=(1 << 20)), 8),  # more than 64 lanes at every vector width
])
def test_forward_rejects(lib, kw, status):
    assert fwd(lib, **kw) == status
    assert lib.msda_last_error().decode() != ""


def test_mixed_dtype_pairs(lib):
    # (value, param): (bf16, fp32) and (fp16, fp32) are accepted; any other
    # differing pair is a dtype error, checked before any launch
    for v, pdt, status in [(2, 0, 0), (1, 0, 0), (0, 2, 4), (2, 1, 4), (1, 2, 4), (0, 1, 4)]:
        got = lib.msda_forward_ex(v, pdt, 1, 100, 2, 8, 2, SHAPES, None, 0, 2, FAKE, FAKE, FAKE,
                                  FAKE, None)
        assert got == status, (v, pdt, got)
        got = lib.msda_backward_ex(v, pdt, 0, 100, 2, 8, 2, SHAPES, None, 16, 2, FAKE, FAKE, FAKE,
                                   FAKE, FAKE, FAKE, FAKE, 0, 0, None, 0, None)
        assert got == status, (v, pdt, got)
    # fp32 parameters are checked at fp32 alignment
    assert lib.msda_forward_ex(2, 0, 1, 100, 2, 8, 2, SHAPES, None, 16, 2, FAKE,
                               ctypes.c_void_p(0x10002), FAKE, FAKE, None) == 5


def test_point_parallel_foil_limits(lib):
    args = (0, 1, 100, 2, 8, 2, SHAPES, None, 16, 2, FAKE, FAKE, FAKE, FAKE, None)
    assert lib.msda_forward_point_parallel(*args[:5], 2, SHAPES, None, 0, 2, *args[10:]) == 0
    # L*K = 2*3 does not divide 256; D = 65 is above 64
    assert lib.msda_forward_point_parallel(0, 1, 100, 2, 8, 2, SHAPES, None, 16, 3, *args[10:]) == 8
    assert lib.msda_forward_point_parallel(0, 1, 100, 2, 65, 2, SHAPES, None, 16, 2, *args[10:]) == 8
    assert lib.msda_forward_point_parallel(0, 1, 100, 2, 8, 2, SHAPES, None, 16, 2, None,
                                           *args[11:]) == 1


def test_forward_empty_batch_or_queries_is_ok_without_launch(lib):
    assert fwd(lib, B=0) == 0
    assert fwd(lib, Q=0) == 0
    assert lib.msda_last_error().decode() == ""


def test_forward_given_start_index_may_differ_from_prefix(lib):
    # valid but non-prefix start index with an empty query set: accepted
    assert fwd(lib, Q=0, starts=(ctypes.c_int64 * 2)(20, 0)) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(accum=6), 4),
    (dict(accum=-2), 4),
    (dict(accum=5, D=300), 8),  # PREREDUCE: head_dim above 256
    (dict(flags=16), 2),
    (dict(flags=2), 2),  # scratch flags need an explicit scratch-capable mode
    (dict(gv=None, accum=0), 1),
    (dict(gout=None, accum=0), 1),
    (dict(accum=3), 6),  # binned: workspace needed
    (dict(dtype=2, accum=-1), 6),  # bf16 AUTO: per-level scratch needs a workspace
    (dict(dtype=2, accum=1), 6),  # scratch needed, no workspace
    (dict(dtype=2, accum=1, ws=ctypes.c_void_p(0x10000), ws_bytes=100), 6),
    (dict(dtype=2, accum=1, ws=ctypes.c_void_p(0x10008), ws_bytes=1 << 20), 5),
])
def test_backward_rejects(lib, kw, status):
    assert bwd(lib, **kw) == status


def test_backward_empty_batch_is_ok(lib):
    assert bwd(lib, B=0) == 0


def test_workspace_size_and_accum_resolution(lib):
    prob = (1, 100, 2, 8, 2, SHAPES, None, 16, 2)
    # fp32 never needs scratch; bf16 fp32-scratch needs B*S*M*D*4 bytes
    assert lib.msda_backward_workspace_size(0, *prob, 1) == 0
    assert lib.msda_backward_workspace_size(2, *prob, 1) == 1 * 100 * 2 * 8 * 4
    assert lib.msda_backward_workspace_size(2, *prob, 0) == 0
    assert lib.msda_backward_workspace_size(1, *prob, 1) == 1 * 100 * 2 * 8 * 4
    assert lib.msda_backward_resolve_accum(2, *prob, 0) == 0
    assert lib.msda_backward_resolve_accum(2, *prob, 1) == 1
    # PER_LEVEL: contributions per pixel Q*K*4/(H*W): (8,10): 1.6 -> packed
    # atomics; (4,5): 6.4 -> fp32 scratch of 20 rows
    assert lib.msda_backward_resolve_accum(2, *prob, 2) == 2
    assert lib.msda_backward_workspace_size(2, *prob, 2) == 1 * 20 * 2 * 8 * 4
    assert lib.msda_backward_resolve_accum(1, *prob, 2) == 2
    assert lib.msda_backward_resolve_accum(0, *prob, 2) == 0  # fp32: nothing to switch
    # AUTO = MIXED: level (4,5) at 6.4 contributions per pixel is binned, level
    # (8,10) at 1.6 keeps native atomics. Two 16-row bins per (b, m) for the
    # binned level: 4 bins; starts (5 x 4 B), cursors (4 x 4 B) and the scan's
    # tile offsets (2 x 2 x 4 B for one tile) padded to 256 B each; records:
    # 4 corners x (16 queries x 2 heads x 2 points) x 8 B.
    for dtype in (0, 1, 2):
        assert lib.msda_backward_resolve_accum(dtype, *prob, -1) == 4
        assert lib.msda_backward_resolve_accum(dtype, *prob, 4) == 4
        assert lib.msda_backward_workspace_size(dtype, *prob, -1) == 3 * 256 + 4 * 64 * 8
    # BINNED: bins of 16 rows (the cap) at both levels -> 5 + 2 bins per
    # (b, m): 14 bins; starts (15 x 4 B), cursors (14 x 4 B) and tile offsets
    # each padded to 256 B; records: 4 corners x 128 points x 8 B.
    for dtype in (0, 1, 2):
        assert lib.msda_backward_resolve_accum(dtype, *prob, 3) == 3
        assert lib.msda_backward_workspace_size(dtype, *prob, 3) == 3 * 256 + 4 * 128 * 8
    # BINNED / MIXED do not apply to overlapping levels; AUTO falls back to
    # PER_LEVEL for bf16 and NATIVE otherwise
    over = (1, 100, 2, 8, 2, SHAPES, (ctypes.c_int64 * 2)(0, 70), 16, 2)
    assert lib.msda_backward_resolve_accum(2, *over, 3) == -1 and lib.msda_last_error()
    assert lib.msda_backward_resolve_accum(2, *over, 4) == -1
    assert lib.msda_backward_workspace_size(2, *over, 3) == 0
    assert lib.msda_backward_resolve_accum(2, *over, -1) == 2
    assert lib.msda_backward_resolve_accum(1, *over, -1) == 0
    # no query: nothing is contended, MIXED resolves to NATIVE
    empty = (1, 100, 2, 8, 2, SHAPES, None, 0, 2)
    assert lib.msda_backward_resolve_accum(2, *empty, 4) == 0
    assert lib.msda_backward_resolve_accum(2, *prob, 7) == -1
    assert lib.msda_backward_workspace_size(9, *prob, 1) == 0 and lib.msda_last_error()


def test_backward_plan_per_level(lib):
    prob = (1, 100, 2, 8, 2, SHAPES, None, 16, 2)
    modes = (ctypes.c_int * 2)()

    def plan(dtype, accum, p=prob):
        nb = lib.msda_backward_plan(dtype, *p, accum, modes)
        return list(modes), nb

    assert plan(2, -1) == ([0, 2], 4)   # MIXED: native, binned
    assert plan(2, 3) == ([2, 2], 14)   # BINNED
    assert plan(2, 2) == ([0, 1], 0)    # PER_LEVEL: native, fp32 scratch
    assert plan(2, 1) == ([1, 1], 0)    # FP32_SCRATCH
    assert plan(0, 1) == ([0, 0], 0)    # fp32 data never uses scratch
    assert plan(1, 0) == ([0, 0], 0)    # NATIVE
    over = (1, 100, 2, 8, 2, SHAPES, (ctypes.c_int64 * 2)(0, 70), 16, 2)
    assert plan(2, -1, over) == ([0, 1], 0)
    assert lib.msda_backward_plan(2, *over, 3, modes) == -1
    assert lib.msda_backward_plan(2, *prob, 9, None) == -1
    assert lib.msda_backward_plan(2, *prob, -1, None) == 4


def test_launch_event_instrumentation_validation(lib):
    assert lib.msda_launch_events_name(-1) is None
    assert lib.msda_launch_events_name(10 ** 6) is None
    assert lib.msda_set_launch_events(None, 0) == 0
    assert lib.msda_set_launch_events(None, 1) == 1
    assert lib.msda_set_launch_events(None, 65) == 2
    nulls = (ctypes.c_void_p * 2)(None, None)
    assert lib.msda_set_launch_events(nulls, 2) == 1


def test_python_binding_rejects_bad_tensors_on_cpu():
    import torch
    from scale_deformable_attention_amd import msda_forward
    v = torch.zeros(1, 100, 2, 8)
    loc = torch.zeros(1, 16, 2, 2, 2, 2)
    a = torch.zeros(1, 16, 2, 2, 2)
    with pytest.raises(ValueError, match="GPU"):
        msda_forward(v, [[8, 10], [4, 5]], None, loc, a)
    with pytest.raises(TypeError):
        msda_forward(v, [[8, 10], [4, 5]], None, loc.double(), a)
    with pytest.raises(ValueError):
        msda_forward(v, [[8, 10], [4, 5], [2, 2]], None, loc, a)


def prep(lib, dtype=0, B=1, Q=16, M=2, L=2, K=2, shapes=SHAPES, per_level=0, ref=FAKE, off=FAKE,
         logits=FAKE, loc=FAKE, attn=FAKE):
    return lib.msda_sampling_prep(dtype, B, Q, M, L, K, shapes, per_level, ref, off, logits, loc,
                                  attn, None)


def prep_bwd(lib, dtype=0, B=1, Q=16, M=2, L=2, K=2, shapes=SHAPES, per_level=0, attn=FAKE,
             gl=FAKE, ga=FAKE, gref=FAKE, goff=FAKE, glog=FAKE):
    return lib.msda_sampling_prep_backward(dtype, B, Q, M, L, K, shapes, per_level, attn, gl, ga,
                                           gref, goff, glog, None)


@pytest.mark.parametrize("kw,status", [
    ({"dtype": 3}, 4), ({"B": -1}, 2), ({"M": 0}, 2), ({"L": 0}, 2), ({"K": 0}, 2),
    ({"L": 17}, 8), ({"per_level": 2}, 2), ({"shapes": None}, 1),
    ({"shapes": (ctypes.c_int64 * 4)(8, 0, 4, 5)}, 3),
    ({"shapes": (ctypes.c_int64 * 4)(8, 1 << 24, 4, 5)}, 8),
    ({"ref": None}, 1), ({"logits": None}, 1), ({"attn": None}, 1),
    ({"off": ctypes.c_void_p(0x10002)}, 5), ({"dtype": 1, "loc": ctypes.c_void_p(0x10001)}, 5),
    ({"B": 1 << 40, "Q": 1 << 30}, 2), ({"B": 1 << 20, "Q": 1 << 12, "M": 2048}, 8),
])
def test_sampling_prep_rejects(lib, kw, status):
    assert prep(lib, **kw) == status, lib.msda_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    ({"dtype": 7}, 4), ({"Q": -2}, 2), ({"attn": None}, 1), ({"gl": None}, 1), ({"ga": None}, 1),
    ({"goff": None}, 1), ({"glog": None}, 1), ({"gref": ctypes.c_void_p(0x10002)}, 5),
    ({"per_level": -1}, 2),
])
def test_sampling_prep_backward_rejects(lib, kw, status):
    assert prep_bwd(lib, **kw) == status, lib.msda_last_error().decode()


def test_sampling_prep_empty_is_ok_without_launch(lib):
    assert prep(lib, B=0) == 0
    assert prep(lib, Q=0, ref=None, off=None, logits=None, loc=None, attn=None) == 0
    assert prep_bwd(lib, B=0, gref=None) == 0


def test_python_prep_binding_rejects_bad_tensors_on_cpu():
    import torch
    from scale_deformable_attention_amd import msda_sampling_prep
    ref = torch.zeros(1, 16, 2)
    off = torch.zeros(1, 16, 2, 2, 2, 2)
    logits = torch.zeros(1, 16, 2, 4)
    with pytest.raises(ValueError, match="GPU"):
        msda_sampling_prep(ref, off, logits, [[8, 10], [4, 5]])
    with pytest.raises(ValueError, match="reference_points"):
        msda_sampling_prep(torch.zeros(1, 16, 3), off, logits, [[8, 10], [4, 5]])
    with pytest.raises(ValueError, match="sampling_offsets"):
        msda_sampling_prep(ref, off, logits, [[8, 10], [4, 5], [2, 2]])
    with pytest.raises(ValueError, match="attention_logits"):
        msda_sampling_prep(ref, off, torch.zeros(1, 16, 2, 5), [[8, 10], [4, 5]])
    with pytest.raises(TypeError):
        msda_sampling_prep(ref.double(), off, logits, [[8, 10], [4, 5]])


def test_workload_plans_match_the_documented_policy(lib):
    """For every named workload and accumulation mode, the library's per-level
    plan (msda_backward_plan, host-only) equals the table the GPU parity
    tests hard-code, and the test-side reading of include/msda.h's policy."""
    import sys
    import torch
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from _parity import WORKLOAD_PLANS, expected_level_modes
    from scale_deformable_attention_amd.workloads import workload
    for name, plans in WORKLOAD_PLANS.items():
        wl = workload(name)
        L = len(wl.levels)
        v = torch.empty((wl.B, wl.S, wl.M, wl.D), dtype=wl.dtype, device="meta")
        pdt = wl.param_dtype or wl.dtype
        loc = torch.empty((wl.B, wl.num_queries, wl.M, L, wl.K, 2), dtype=pdt, device="meta")
        attn = torch.empty((wl.B, wl.num_queries, wl.M, L, wl.K), dtype=pdt, device="meta")
        for accum, table in plans.items():
            got = bind.msda_backward_level_modes(v, torch.tensor(wl.levels), None, loc, attn,
                                                 accum)
            want = expected_level_modes(wl.dtype, accum, torch.tensor(wl.levels), wl.B, wl.S,
                                        wl.M, wl.D, wl.num_queries, wl.K)
            assert got == table == want, (name, accum, got, table, want)


def test_release_thread_resources_without_any_is_ok(lib):
    """No binned backward ran on this thread: nothing to release, no HIP call,
    MSDA_OK (twice in a row too)."""
    assert lib.msda_release_thread_resources() == 0
    assert lib.msda_release_thread_resources() == 0
    bind.release_thread_resources()


def test_single_stream_flag_is_known(lib):
    """MSDA_FLAG_SINGLE_STREAM (8) passes flag validation; an unknown bit does
    not (both stop before any launch: B = 0 returns after validation)."""
    assert bwd(lib, B=0, flags=8) == 0
    assert bwd(lib, B=0, flags=16) == 2


def test_noalloc_backward_rejects_before_any_hip_call(lib):
    """msda_backward_noalloc: a problem whose workspace exceeds the 32 MiB
    static scratch is refused with MSDA_ERR_WORKSPACE, the scratch-continuing
    flags with MSDA_ERR_SHAPE, invalid sizes with their own status; an empty
    batch is OK. None of these reaches a HIP call."""
    def nb(dtype=2, B=1, S=100, M=2, D=8, Q=16, K=2, accum=-1, flags=0, shapes=SHAPES):
        return lib.msda_backward_noalloc(dtype, B, S, M, D, 2, shapes, None, Q, K, FAKE, FAKE,
                                         FAKE, FAKE, FAKE, FAKE, FAKE, accum, flags, None)
    # fp32 scratch of B*S*M*D fp32 = 16384 * 100 * 2 * 8 * 4 bytes = 100 MiB > 32 MiB
    assert nb(B=16384, accum=1) == 6
    assert "static scratch" in lib.msda_last_error().decode()
    assert nb(flags=2) == 2 and nb(flags=4) == 2
    assert nb(M=0) == 2
    assert nb(B=0) == 0


def test_flat_gathers_hook_plans_as_for_large_slices(lib):
    """msda_debug_force_flat_gathers (a testing hook): returns the previous
    setting; while set, binned accumulation no longer applies (as for a batch
    value slice of 2 GiB or more), AUTO falls back to PER_LEVEL for bf16, and
    mixed dtypes are refused; all host-only."""
    import sys
    import torch
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from _parity import WORKLOAD_PLANS
    from scale_deformable_attention_amd.workloads import workload
    wl = workload("decoder_bf16")
    L = len(wl.levels)
    v = torch.empty((wl.B, wl.S, wl.M, wl.D), dtype=wl.dtype, device="meta")
    loc = torch.empty((wl.B, wl.num_queries, wl.M, L, wl.K, 2), dtype=wl.dtype, device="meta")
    attn = torch.empty((wl.B, wl.num_queries, wl.M, L, wl.K), dtype=wl.dtype, device="meta")
    shapes = torch.tensor(wl.levels)
    assert lib.msda_debug_force_flat_gathers(0) == 0
    try:
        assert lib.msda_debug_force_flat_gathers(1) == 0
        assert bind.msda_backward_level_modes(v, shapes, None, loc, attn, "auto") == \
            WORKLOAD_PLANS["decoder_bf16"]["per_level"]
        for accum in ("binned", "mixed", "prereduce"):
            with pytest.raises(bind.MSDAError) as err:
                bind.msda_backward_level_modes(v, shapes, None, loc, attn, accum)
            assert err.value.status == 8
        # mixed dtypes (fp32 parameters beside bf16 values) need the buffer path
        st = lib.msda_forward_ex(2, 0, 1, 100, 2, 8, 2, SHAPES, None, 16, 2, FAKE, FAKE, FAKE,
                                 FAKE, None)
        assert st == 8, lib.msda_last_error()
        assert lib.msda_debug_force_flat_gathers(0) == 1
    finally:
        lib.msda_debug_force_flat_gathers(0)
    assert bind.msda_backward_level_modes(v, shapes, None, loc, attn, "auto") == \
        WORKLOAD_PLANS["decoder_bf16"]["auto"]
