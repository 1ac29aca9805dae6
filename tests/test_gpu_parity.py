"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Every workload runs forward + backward on the GPU and is compared element by
element with the oracle on the same seeded inputs (tests/_parity.py holds the
tolerance rule), at the workloads' full sizes. Edge cases cover ragged query blocks,
channel widths that need masking, misaligned pointers, custom level tables,
empty inputs, out-of-bounds points, integer-aligned points, accumulation,
determinism and 64-bit indexing.
"""

import numpy as np
import pytest
import torch

import oracle
from scale_deformable_attention_amd import MSDAError, PreparedCall, msda_backward, msda_forward
from scale_deformable_attention_amd.workloads import Workload, make_inputs, workload

from _parity import (check_backward, check_forward, check_grad_value, level_row_ranges,
                     parity_kwargs, plan_for, to_np)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _library():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from scale_deformable_attention_amd import _binding
    import os
    if not os.path.exists(_binding.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    _binding.load_library()


def say(msg):
    print(msg, flush=True)


def to_dev(inp):
    return {k: (v.to(DEV) if k != "spatial_shapes" else v) for k, v in inp.items()}


def gpu_run(inp, accum="auto", starts=None):
    g = to_dev(inp)
    out = msda_forward(g["value"], g["spatial_shapes"], starts, g["sampling_locations"],
                       g["attention_weights"])
    grads = msda_backward(g["value"], g["spatial_shapes"], starts, g["sampling_locations"],
                          g["attention_weights"], g["grad_output"], accum=accum)
    torch.cuda.synchronize()
    return out.cpu(), tuple(t.cpu() for t in grads)


def oracle_run(inp, starts=None):
    args = (inp["value"], inp["spatial_shapes"], starts, inp["sampling_locations"],
            inp["attention_weights"])
    out, touched = oracle.forward(*args, return_touched=True)
    gv, gl, ga, trows = oracle.backward(*args, inp["grad_output"], return_touched=True)
    return out, touched, (gv, gl, ga), trows


def report(stats):
    for s in stats:
        if s.get("n"):
            extra = f" past_plain_bar={s['past_plain_bar']}" if "past_plain_bar" in s else ""
            say(f"  {s['name']:50s} max_scaled={s['max_scaled']:.2e} "
                f"normwise={s['normwise']:.2e}{extra}")


def full_check(inp, dtype, accum="auto", starts=None, ref=None, workload_name=None, flat=False):
    kw = parity_kwargs(dtype, accum, inp, starts, workload_name, flat=flat)
    out, grads = gpu_run(inp, accum, starts)
    ref_out, touched, ref_grads, trows = ref if ref is not None else oracle_run(inp, starts)
    stats = check_forward(dtype, out, ref_out, touched)
    stats += check_backward(dtype, grads, ref_grads, inp["spatial_shapes"], starts, trows, **kw)
    report(stats)
    return out, grads


# ------------------------------------------------------------- workloads

_REF_CACHE = {}


def _cached(name):
    if name not in _REF_CACHE:
        inp = make_inputs(workload(name))
        _REF_CACHE[name] = (inp, oracle_run(inp))
    return _REF_CACHE[name]


@pytest.mark.parametrize("name,accum", [
    ("tiny_fp32", "auto"), ("tiny_fp32", "binned"),
    ("decoder_bf16", "auto"), ("decoder_bf16", "native"), ("decoder_bf16", "fp32_scratch"),
    ("decoder_bf16", "binned"), ("decoder_bf16", "per_level"), ("oddhead_fp32", "mixed"),
    ("encoder_fp16", "auto"), ("encoder_fp16", "fp32_scratch"), ("encoder_fp16", "native"),
    ("oddhead_fp32", "auto"), ("oddhead_fp32", "binned"), ("encoder_fp16", "prereduce"),
])
def test_workload_parity(name, accum):
    wl = workload(name)
    say(f"case {name} accum={accum}: B={wl.B} Q={wl.num_queries} M={wl.M} D={wl.D} "
        f"L={wl.L} K={wl.K} {wl.dtype}")
    inp, ref = _cached(name)
    full_check(inp, wl.dtype, accum, ref=ref, workload_name=name)


@pytest.mark.parametrize("accum", ["auto", "fp32_scratch", "prereduce"])
def test_large_encoder_parity(accum):
    name = "large_encoder_bf16"
    wl = workload(name)
    say(f"case {name} accum={accum}: B={wl.B} Q={wl.num_queries} M={wl.M} D={wl.D} "
        f"L={wl.L} K={wl.K} {wl.dtype}")
    inp, ref = _cached(name)
    full_check(inp, wl.dtype, accum, ref=ref, workload_name=name)


def test_native_bf16_atomics_on_contended_levels():
    """Forced NATIVE on the large encoder: packed bf16 atomics round every
    add to 8 significant bits (course page "5. The backward kernel", section
    "Atomics make gradients nondeterministic") on levels of 21 to 1360
    contributions per pixel. Every element must stay within the derived
    rounding bound; the counts of elements past the plain 5e-2 bar (printed)
    are why AUTO sums these levels in fp32 through bins instead."""
    name = "large_encoder_bf16"
    wl = workload(name)
    say(f"case {name} accum=native (16-bit rounding bound)")
    inp, (ref_out, touched, ref_grads, trows) = _cached(name)
    kw = parity_kwargs(wl.dtype, "native", inp, workload_name=name)
    _, grads = gpu_run(inp, "native")
    report(check_backward(wl.dtype, grads, ref_grads, inp["spatial_shapes"], None, trows, **kw))


# ------------------------------------------------------------ edge cases

def _small(dtype, D=8, Q=37, M=3, K=3, levels=((6, 9), (3, 5), (2, 2)), B=2, lo=-0.15, hi=1.15,
           seed=77):
    wl = Workload(name="edge", dtype=dtype, B=B, Q=Q, M=M, D=D, K=K, levels=levels,
                  loc_kind="uniform", loc_lo=lo, loc_hi=hi, seed=seed)
    return wl, make_inputs(wl)


DTYPES = [torch.float32, torch.float16, torch.bfloat16]


@pytest.mark.parametrize("dtype", DTYPES, ids=str)
@pytest.mark.parametrize("D", [1, 3, 8, 16, 24, 32, 48, 64, 128, 256])
def test_head_dims_and_ragged_queries(dtype, D):
    wl, inp = _small(dtype, D=D)
    say(f"case head_dim D={D} {dtype} Q={wl.Q}")
    full_check(inp, dtype, "native")
    full_check(inp, dtype, "binned")
    if dtype != torch.float32:
        full_check(inp, dtype, "fp32_scratch")


@pytest.mark.parametrize("dtype", DTYPES, ids=str)
def test_widest_head_dim(dtype):
    D = 512 if dtype != torch.float32 else 256  # 64 lanes x widest vector
    wl, inp = _small(dtype, D=D, Q=9, M=2)
    say(f"case widest head_dim D={D} {dtype}")
    full_check(inp, dtype, "native")
    full_check(inp, dtype, "binned")


@pytest.mark.parametrize("dtype", DTYPES, ids=str)
@pytest.mark.parametrize("K,L", [(1, 1), (8, 2), (5, 3), (2, 16)])
def test_points_and_levels(dtype, K, L):
    levels = tuple((3 + (i % 4), 2 + (i % 5)) for i in range(L))
    wl, inp = _small(dtype, K=K, levels=levels, Q=300, B=1, M=2, D=16)
    say(f"case K={K} L={L} {dtype}")
    # tiny levels: up to 1600 contributions per pixel, so bf16 goes through
    # the default (fp32 scratch) accumulation
    full_check(inp, dtype, "auto")


@pytest.mark.parametrize("dtype", DTYPES, ids=str)
@pytest.mark.parametrize("accum", ["native", "fp32_scratch", "binned"])
def test_degenerate_level_shapes(dtype, accum):
    """Levels of one pixel, one row and one column beside a small 2-D level:
    a corner off the single row or column is out of bounds, and every
    in-bounds corner of a 1 x 1 level is that one pixel. Points spread past
    the map on all sides."""
    if dtype == torch.float32 and accum == "fp32_scratch":
        pytest.skip("identical to native for fp32")
    levels = ((1, 1), (1, 7), (7, 1), (2, 3))
    wl, inp = _small(dtype, D=32, K=4, levels=levels, Q=50, M=4, lo=-0.3, hi=1.3, seed=97)
    say(f"case degenerate level shapes {dtype} {accum}")
    full_check(inp, dtype, accum)


@pytest.mark.parametrize("dtype", DTYPES, ids=str)
def test_custom_level_start_and_padding_rows(dtype):
    levels = ((6, 9), (3, 5), (2, 2))
    wl, inp = _small(dtype, levels=levels)
    # levels stored in another order along S, with 11 unused rows (19..29)
    starts = torch.tensor([30, 4, 0])
    S = 30 + 54
    g = torch.Generator().manual_seed(3)
    B, _, M, D = inp["value"].shape
    inp["value"] = torch.randn(B, S, M, D, generator=g).to(dtype)
    say(f"case custom level_start_index {starts.tolist()} S={S} {dtype}")
    full_check(inp, dtype, "native", starts=starts)
    # binned: the padding rows belong to no bin and must come out zero
    full_check(inp, dtype, "binned", starts=starts)


@pytest.mark.parametrize("dtype", DTYPES, ids=str)
def test_misaligned_pointers_fall_back_to_narrow_access(dtype):
    wl, inp = _small(dtype, D=32, Q=20)
    g = to_dev(inp)
    say(f"case misaligned value/output pointers {dtype}")
    ref_out, touched, ref_grads, trows = oracle_run(inp)
    # views starting one element into a larger buffer: element-aligned only
    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        return v
    v, loc, a, go = (shifted(g[k]) for k in ("value", "sampling_locations", "attention_weights",
                                              "grad_output"))
    out = shifted(torch.empty(wl.B, wl.Q, wl.M * wl.D, dtype=dtype, device=DEV))
    msda_forward(v, g["spatial_shapes"], None, loc, a, output=out)
    gv = shifted(torch.empty_like(g["value"]))
    gl = shifted(torch.empty_like(g["sampling_locations"]))
    ga = shifted(torch.empty_like(g["attention_weights"]))
    kw = dict(grad_value=gv, grad_sampling_locations=gl, grad_attention_weights=ga)
    if dtype != torch.float32:
        # packed atomics would straddle the tensor's edge: refused, scratch works
        with pytest.raises(MSDAError, match="4-byte aligned"):
            msda_backward(v, g["spatial_shapes"], None, loc, a, go, accum="native", **kw)
    msda_backward(v, g["spatial_shapes"], None, loc, a, go,
                  accum="native" if dtype == torch.float32 else "fp32_scratch", **kw)
    torch.cuda.synchronize()
    check_forward(dtype, out.cpu(), ref_out, touched)
    check_backward(dtype, (gv.cpu(), gl.cpu(), ga.cpu()), ref_grads, inp["spatial_shapes"], None,
                   trows)
    msda_backward(v, g["spatial_shapes"], None, loc, a, go, accum="binned", **kw)
    torch.cuda.synchronize()
    check_backward(dtype, (gv.cpu(), gl.cpu(), ga.cpu()), ref_grads, inp["spatial_shapes"], None,
                   trows)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=str)
@pytest.mark.parametrize("accum", ["auto", "mixed", "binned"])
def test_grad_output_off_16_byte_alignment(dtype, accum):
    """grad_output two elements into a buffer (4-byte aligned, not 16): the
    accumulation reads it 4 bytes per lane instead of 16 (64-byte rows), in
    the launch shared with the atomic scatter and in the standalone one."""
    wl, inp = _small(dtype, D=32, Q=150, M=2, K=4, levels=((20, 30), (6, 9), (3, 4)))
    say(f"case grad_output 4-byte aligned {dtype} {accum}")
    _, _, ref_grads, trows = oracle_run(inp)
    g = to_dev(inp)
    buf = torch.empty(g["grad_output"].numel() + 2, dtype=dtype, device=DEV)
    go = buf[2:].view(g["grad_output"].shape)
    go.copy_(g["grad_output"])
    assert go.data_ptr() % 16 != 0 and go.data_ptr() % 4 == 0
    grads = msda_backward(g["value"], g["spatial_shapes"], None, g["sampling_locations"],
                          g["attention_weights"], go, accum=accum)
    torch.cuda.synchronize()
    check_backward(dtype, tuple(t.cpu() for t in grads), ref_grads, inp["spatial_shapes"], None,
                   trows, **parity_kwargs(dtype, accum, inp))


@pytest.mark.parametrize("dtype", DTYPES, ids=str)
@pytest.mark.parametrize("accum", ["auto", "native", "binned"])
def test_non_contiguous_inputs(dtype, accum):
    """Strided views of every input (the binding makes dense copies before
    the call): forward and backward match the oracle on the same values."""
    wl, inp = _small(dtype, D=16)
    g = to_dev(inp)
    say(f"case non-contiguous inputs {dtype} {accum}")
    # same values, non-contiguous storage
    v = g["value"].transpose(1, 2).contiguous().transpose(1, 2)
    loc = g["sampling_locations"].permute(5, 0, 1, 2, 3, 4).contiguous().permute(1, 2, 3, 4, 5, 0)
    a = g["attention_weights"].transpose(0, 4).contiguous().transpose(0, 4)
    go = g["grad_output"].transpose(1, 2).contiguous().transpose(1, 2)
    assert not any(t.is_contiguous() for t in (v, loc, a, go))
    out = msda_forward(v, g["spatial_shapes"], None, loc, a)
    grads = msda_backward(v, g["spatial_shapes"], None, loc, a, go, accum=accum)
    torch.cuda.synchronize()
    ref_out, touched, ref_grads, trows = oracle_run(inp)
    report(check_forward(dtype, out.cpu(), ref_out, touched))
    report(check_backward(dtype, tuple(t.cpu() for t in grads), ref_grads, inp["spatial_shapes"],
                          None, trows, **parity_kwargs(dtype, accum, inp)))


@pytest.mark.parametrize("dtype", DTYPES, ids=str)
def test_empty_batch_and_queries(dtype):
    say(f"case empty B/Q {dtype}")
    wl, inp = _small(dtype, Q=0)
    g = to_dev(inp)
    out = msda_forward(g["value"], g["spatial_shapes"], None, g["sampling_locations"],
                       g["attention_weights"])
    assert out.shape == (wl.B, 0, wl.M * wl.D)
    for accum in ("native", "fp32_scratch", "auto", "binned"):
        gv = torch.full_like(g["value"], 7.0)
        gv, gl, ga = msda_backward(g["value"], g["spatial_shapes"], None, g["sampling_locations"],
                                   g["attention_weights"], g["grad_output"], grad_value=gv,
                                   accum=accum)
        torch.cuda.synchronize()
        assert torch.all(gv == 0) and gl.numel() == 0 and ga.numel() == 0
    wl, inp = _small(dtype, B=0)
    g = to_dev(inp)
    out = msda_forward(g["value"], g["spatial_shapes"], None, g["sampling_locations"],
                       g["attention_weights"])
    assert out.shape[0] == 0


ALL_MODES = ["native", "fp32_scratch", "binned", "mixed", "auto", "prereduce"]


@pytest.mark.parametrize("dtype", DTYPES, ids=str)
@pytest.mark.parametrize("accum", ALL_MODES)
def test_all_points_out_of_bounds(dtype, accum):
    """Every point outside its level: the output and all three gradients are
    exactly zero, whatever the accumulation (course page "5. The backward
    kernel", section "Scatter needs atomics")."""
    wl, inp = _small(dtype)
    loc = inp["sampling_locations"].float()
    sel = torch.rand(loc.shape[:-1], generator=torch.Generator().manual_seed(1)) < 0.5
    loc[..., 0] = torch.where(sel, torch.tensor(1.6), torch.tensor(-0.8))
    inp["sampling_locations"] = loc.to(dtype)
    say(f"case all points out of bounds {dtype} {accum}")
    out, (gv, gl, ga) = gpu_run(inp, accum)
    assert torch.all(out == 0) and torch.all(gv == 0) and torch.all(gl == 0) and torch.all(ga == 0)


@pytest.mark.parametrize("dtype", DTYPES, ids=str)
@pytest.mark.parametrize("accum", ALL_MODES)
def test_integer_aligned_points_reproduce_rows_exactly(dtype, accum):
    """Points on pixel centres with one-hot weights: each output row is one
    value row, bit for bit, in every dtype; the backward matches the oracle,
    and grad_value rows that only zero-weight corners land on are exactly 0."""
    levels = ((8, 16), (4, 8))
    B, Q, M, D, K, L = 2, 50, 2, 16, 2, 2
    g = torch.Generator().manual_seed(12)
    S = sum(h * w for h, w in levels)
    value = torch.randn(B, S, M, D, generator=g).to(dtype)
    loc = torch.empty(B, Q, M, L, K, 2)
    for l, (H, W) in enumerate(levels):
        ix = torch.randint(W, (B, Q, M, K), generator=g)
        iy = torch.randint(H, (B, Q, M, K), generator=g)
        loc[:, :, :, l, :, 0] = (ix + 0.5) / W
        loc[:, :, :, l, :, 1] = (iy + 0.5) / H
    hot = torch.randint(L * K, (B, Q, M), generator=g)
    attn = torch.nn.functional.one_hot(hot, L * K).float().reshape(B, Q, M, L, K)
    inp = {"value": value, "spatial_shapes": torch.tensor(levels),
           "sampling_locations": loc.to(dtype), "attention_weights": attn.to(dtype),
           "grad_output": torch.randn(B, Q, M * D, generator=g).to(dtype)}
    say(f"case integer-aligned one-hot points {dtype} {accum}")
    out, grads = gpu_run(inp, accum)
    ref_out, touched, ref_grads, trows = oracle_run(inp)
    # each output row is exactly one value row: bit-exact in every dtype
    assert torch.equal(out.double(), torch.from_numpy(ref_out).to(dtype).double())
    assert np.array_equal(to_np(out), ref_out)
    report(check_backward(dtype, grads, ref_grads, inp["spatial_shapes"], None, trows,
                          **parity_kwargs(dtype, accum, inp)))
    # rows reached only by corners of zero weight receive exactly nothing
    zero_rows = np.all(ref_grads[0] == 0, axis=-1) & trows
    assert zero_rows.any()
    assert np.all(to_np(grads[0])[zero_rows] == 0)


@pytest.mark.parametrize("dtype", DTYPES, ids=str)
@pytest.mark.parametrize("accum", ["native", "fp32_scratch", "binned"])
@pytest.mark.parametrize("D", [16, 32])
def test_accumulate_flag_doubles_grad_value(dtype, accum, D):
    """A second backward with `accumulate` adds to the first one's grad_value.
    D = 32 gives 16-bit dtypes 64-byte rows (the binned accumulation's wide
    mode) and fp32 two 64-byte slot groups per row."""
    if dtype == torch.float32 and accum == "fp32_scratch":
        pytest.skip("identical to native for fp32")
    wl, inp = _small(dtype, D=D)
    g = to_dev(inp)
    say(f"case accumulate twice {dtype} {accum} D={D}")
    args = (g["value"], g["spatial_shapes"], None, g["sampling_locations"], g["attention_weights"],
            g["grad_output"])
    gv1, _, _ = msda_backward(*args, accum=accum)
    once = gv1.clone()
    msda_backward(*args, grad_value=gv1, accum=accum, accumulate=True)
    torch.cuda.synchronize()
    ref = oracle.backward(inp["value"], inp["spatial_shapes"], None, inp["sampling_locations"],
                          inp["attention_weights"], inp["grad_output"])[0]
    # levels accumulated with 16-bit atomics: the rounding bound of check_backward,
    # for the second result with the terms of both calls (passes=2)
    kw = parity_kwargs(dtype, accum, inp)
    report(check_grad_value(dtype, to_np(once), ref, inp["spatial_shapes"], **kw))
    report(check_grad_value(dtype, to_np(gv1), 2 * ref, inp["spatial_shapes"], passes=2, **kw))


@pytest.mark.parametrize("dtype", DTYPES, ids=str)
def test_deterministic_outputs(dtype):
    wl, inp = _small(dtype, D=32, Q=200)
    say(f"case determinism {dtype}")
    for accum in ("fp32_scratch" if dtype != torch.float32 else "native", "binned"):
        out1, (gv1, gl1, ga1) = gpu_run(inp, accum)
        out2, (gv2, gl2, ga2) = gpu_run(inp, accum)
        assert torch.equal(out1, out2) and torch.equal(gl1, gl2) and torch.equal(ga1, ga2)
        # grad_value: accumulation order may differ; fp32 sums keep runs within rounding
        d = (gv1.double() - gv2.double()).abs().max().item()
        scale = gv1.double().abs().max().item()
        assert d <= 1e-6 * scale + (2.0 ** -8 if dtype != torch.float32 else 0.0) * scale


def test_int64_indexing_beyond_2_pow_31_elements():
    """B*S*M*D above 2^31 elements: the last batch's value rows sit past
    element 2^31; every other batch holds a constant sentinel."""
    levels = ((512, 896), (256, 448), (128, 224), (64, 112))
    S = sum(h * w for h, w in levels)
    B, M, D, K, Q = 16, 8, 32, 4, 512
    assert B * S * M * D > 2 ** 31
    dtype = torch.bfloat16
    say(f"case int64 indexing: B={B} S={S} M={M} D={D} bf16 ({B * S * M * D / 2**30:.2f} Gi elements)")
    wl = Workload(name="int64", dtype=dtype, B=1, Q=Q, M=M, D=D, K=K, levels=levels,
                  loc_kind="uniform", seed=99)
    last = make_inputs(wl)  # batch B-1's inputs
    value = torch.full((B, S, M, D), 1000.0, dtype=dtype, device=DEV)
    value[B - 1].copy_(last["value"][0].to(DEV))
    def rep(t):
        return t.to(DEV).expand(B, *t.shape[1:]).contiguous()
    loc, attn, gout = rep(last["sampling_locations"]), rep(last["attention_weights"]), \
        rep(last["grad_output"])
    shapes = last["spatial_shapes"]
    out = msda_forward(value, shapes, None, loc, attn)
    torch.cuda.synchronize()
    out_last = out[B - 1:].cpu()
    del out
    ref_out, touched, ref_grads, trows = oracle_run(last)
    check_forward(dtype, out_last, ref_out, touched)
    for accum in ("native", "binned"):
        say(f"  backward accum={accum}")
        gv, gl, ga = msda_backward(value, shapes, None, loc, attn, gout, accum=accum)
        torch.cuda.synchronize()
        gv_last = gv[B - 1:].cpu()
        gl_last, ga_last = gl[B - 1:].cpu(), ga[B - 1:].cpu()
        del gv, gl, ga
        torch.cuda.empty_cache()
        check_backward(dtype, (gv_last, gl_last, ga_last), ref_grads, shapes, None, trows,
                       **parity_kwargs(dtype, accum, last))


def test_accumulation_resolution_on_the_decoder_workload():
    from scale_deformable_attention_amd import msda_backward_resolve_accum
    inp = make_inputs(workload("decoder_bf16"), with_grad=False)
    g = to_dev(inp)
    say("case decoder_bf16 accumulation resolution")
    args = (g["value"], g["spatial_shapes"], None, g["sampling_locations"], g["attention_weights"])
    # contributions per pixel 300*4*4/(H*W): 0.29, 1.1 (native atomics), 4.6, 17.6 (binned)
    assert msda_backward_resolve_accum(*args) == "mixed"
    assert msda_backward_resolve_accum(*args, accum="per_level") == "per_level"
    assert msda_backward_resolve_accum(*args, accum="binned") == "binned"
    call = PreparedCall(g["value"], g["spatial_shapes"], None, g["sampling_locations"],
                        g["attention_weights"])
    modes, nb = call.plan()
    assert modes == ["native", "native", "binned", "binned"] and nb > 0
    # the encoder workload is contended at every level: all binned
    enc = make_inputs(workload("encoder_fp16"), with_grad=False)
    ge = to_dev(enc)
    assert msda_backward_resolve_accum(ge["value"], ge["spatial_shapes"], None,
                                       ge["sampling_locations"], ge["attention_weights"]) == "binned"


@pytest.mark.parametrize("dtype", DTYPES, ids=str)
@pytest.mark.parametrize("accum", ["per_level", "fp32_scratch"])
def test_micro_batches_accumulate_in_deferred_scratch(dtype, accum):
    """Two backward calls with different upstream gradients: the first leaves
    its fp32 sums in the workspace, the second continues them and adds once.
    grad_value is linear in grad_output, so the result is the oracle's
    gradient for the sum of the two upstream gradients."""
    if dtype == torch.float32 and accum == "fp32_scratch":
        pytest.skip("fp32 data has no scratch")
    from scale_deformable_attention_amd import msda_backward_workspace_size
    wl, inp = _small(dtype, D=32, Q=200, K=4, levels=((12, 15), (6, 8), (3, 4)))
    g = to_dev(inp)
    g2 = torch.randn(inp["grad_output"].shape, generator=torch.Generator().manual_seed(5)).to(dtype)
    say(f"case micro-batch accumulation {dtype} {accum}")
    args = (g["value"], g["spatial_shapes"], None, g["sampling_locations"], g["attention_weights"])
    need = msda_backward_workspace_size(*args, accum=accum)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    gv, _, _ = msda_backward(*args, g["grad_output"], accum=accum, workspace=ws, defer_scratch=True)
    msda_backward(*args, g2.to(DEV), grad_value=gv, accum=accum, workspace=ws, accumulate=True,
                  continue_scratch=True)
    torch.cuda.synchronize()
    gsum = inp["grad_output"].double() + g2.double()
    ref = oracle.backward(inp["value"], inp["spatial_shapes"], None, inp["sampling_locations"],
                          inp["attention_weights"], gsum)[0]
    tol = 1e-5 if dtype == torch.float32 else 5e-2
    from _parity import check_slice
    for l, (r0, r1) in enumerate(level_row_ranges(inp["spatial_shapes"])):
        check_slice(f"grad_value[level {l}]", to_np(gv)[:, r0:r1], ref[:, r0:r1], tol)


@pytest.mark.parametrize("dtype", DTYPES, ids=str)
@pytest.mark.parametrize("accum", ["auto", "native", "fp32_scratch"])
def test_overlapping_levels(dtype, accum):
    """A caller-given level_start_index may make levels share rows; every
    level's contributions must land in the shared rows."""
    levels = ((12, 16), (8, 10), (6, 6))
    # rows: level 0 [0,192), level 1 [100,180), level 2 [150,186): all three share [150,180)
    starts = torch.tensor([0, 100, 150])
    wl, inp = _small(dtype, levels=levels, Q=50, D=16, K=2)
    S = 192
    inp["value"] = torch.randn(wl.B, S, wl.M, wl.D,
                               generator=torch.Generator().manual_seed(4)).to(dtype)
    say(f"case overlapping levels {starts.tolist()} {dtype} {accum}")
    full_check(inp, dtype, accum, starts=starts)


@pytest.mark.parametrize("name", ["tiny_fp32", "decoder_bf16", "oddhead_fp32"])
def test_point_parallel_foil_parity(name):
    """The point-parallel foil (a measurement study) computes the same forward."""
    from scale_deformable_attention_amd._binding import msda_forward_point_parallel
    wl = workload(name)
    say(f"case {name} point-parallel foil")
    inp, (ref_out, touched, _, _) = _cached(name)
    g = to_dev(inp)
    out = msda_forward_point_parallel(g["value"], g["spatial_shapes"], None,
                                      g["sampling_locations"], g["attention_weights"])
    torch.cuda.synchronize()
    check_forward(wl.dtype, out.cpu(), ref_out, touched)


@pytest.mark.parametrize("name,accum", [("decoder_mixed", "auto"), ("decoder_mixed", "native"),
                                        ("decoder_mixed", "per_level"), ("encoder_mixed", "auto")])
def test_mixed_dtype_parity(name, accum):
    """16-bit values with fp32 locations and weights: output and grad_value in
    the value dtype, grad_loc / grad_attn in fp32 at the fp32 tolerance."""
    wl = workload(name)
    say(f"case {name} accum={accum}: value {wl.dtype}, parameters {wl.param_dtype}")
    inp, ref = _cached(name)
    assert inp["sampling_locations"].dtype == torch.float32 and inp["value"].dtype == wl.dtype
    out, grads = gpu_run(inp, accum)
    assert out.dtype == wl.dtype and grads[0].dtype == wl.dtype
    assert grads[1].dtype == torch.float32 and grads[2].dtype == torch.float32
    ref_out, touched, ref_grads, trows = ref
    check_forward(wl.dtype, out, ref_out, touched)
    check_backward(wl.dtype, grads, ref_grads, inp["spatial_shapes"], None, trows,
                   param_dtype=torch.float32,
                   **parity_kwargs(wl.dtype, accum, inp, workload_name=name))


def test_mixed_dtype_rejections():
    wl = workload("decoder_mixed")
    inp = make_inputs(wl.replace(Q=8))
    g = to_dev(inp)
    v16 = g["value"].to(torch.float16)  # fp16 value with bf16 parameters: not a valid pair
    with pytest.raises(TypeError):
        msda_forward(g["value"], g["spatial_shapes"], None, g["sampling_locations"].bfloat16(),
                     g["attention_weights"])
    with pytest.raises(TypeError):
        msda_forward(v16, g["spatial_shapes"], None, g["sampling_locations"].bfloat16(),
                     g["attention_weights"].bfloat16())


# ------------------------------------------- launch paths at their size limits

def _backward_launch_names(inp, accum):
    """Run the backward with per-launch instrumentation; return the launch
    names and the gradients."""
    from scale_deformable_attention_amd._binding import launch_event_names, set_launch_events
    g = to_dev(inp)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(40)]
    for e in evs:
        e.record()  # torch creates the HIP event on first record
    torch.cuda.synchronize()
    set_launch_events(evs)
    grads = msda_backward(g["value"], g["spatial_shapes"], None, g["sampling_locations"],
                          g["attention_weights"], g["grad_output"], accum=accum)
    torch.cuda.synchronize()
    return launch_event_names(), tuple(t.cpu() for t in grads)


# name, dtype, Q, K, M, D, levels, accum, a launch the path must make, launches it must not
PATH_CASES = [
    # Q*K = 2048: gradients, one-launch sort and fill share a launch
    ("fused_sort_at_2048_points", torch.bfloat16, 512, 4, 2, 32, ((64, 64), (32, 32)), "auto",
     "grad_sort_kernel", ("bin_count", "bin_local_sort")),
    # Q*K = 2052: count / scan / place
    ("sort_chain_past_2048_points", torch.bfloat16, 513, 4, 2, 32, ((64, 64), (32, 32)), "auto",
     "bin_count", ("grad_sort_kernel", "bin_local_sort")),
    # every level binned; 5625 bins on level 0: the one-launch sort without the
    # gradients (above 4096 bins)
    ("local_sort_above_4096_bins", torch.float16, 64, 2, 1, 16, ((300, 300), (8, 8)), "binned",
     "bin_local_sort", ("grad_sort_kernel", "bin_count")),
    # 40000 bins on level 0: the chain, with the scan over tiles of 4096
    ("sort_chain_above_32000_bins", torch.float32, 64, 2, 1, 16, ((800, 800), (8, 8)), "binned",
     "bin_tile_sum", ("bin_local_sort",)),
]


@pytest.mark.parametrize("case", PATH_CASES, ids=lambda c: c[0])
def test_sort_paths_at_their_limits(case):
    name, dtype, Q, K, M, D, levels, accum, must, must_not = case
    wl = Workload(name=name, dtype=dtype, B=2, Q=Q, M=M, D=D, K=K, levels=levels,
                  loc_kind="uniform", loc_lo=-0.05, loc_hi=1.05, seed=91)
    inp = make_inputs(wl)
    say(f"case {name}: Q={Q} K={K} levels={levels} accum={accum} {dtype}")
    names, grads = _backward_launch_names(inp, accum)
    assert must in names and not set(must_not) & set(names), names
    _, _, ref_grads, trows = oracle_run(inp)
    check_backward(dtype, grads, ref_grads, inp["spatial_shapes"], None, trows,
                   **parity_kwargs(dtype, accum, inp))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=str)
@pytest.mark.parametrize("accum", ["auto", "binned", "native"])
def test_non_finite_upstream_gradient_stays_local(dtype, accum):
    """An infinite upstream gradient at one (batch, query, head) makes
    non-finite exactly the grad_value entries that the oracle makes
    non-finite (the rows that query's in-bounds corners of that head land
    on) and that query's own location and weight gradients; every other
    entry is finite and matches the oracle. Guards the lanes of the binned
    accumulation that hold no record: they must read no upstream-gradient
    row, whatever it holds. Q*K = 2400 takes the count / scan / place chain."""
    wl = workload("decoder_bf16").replace(name="decoder_q600", dtype=dtype, B=1, Q=600, seed=23)
    inp = make_inputs(wl)
    D, m_bad, q_bad = wl.D, 3, 7
    go = inp["grad_output"].clone()
    go[0, q_bad, m_bad * D:(m_bad + 1) * D] = float("inf")
    inp["grad_output"] = go
    say(f"case non-finite grad_output {dtype} accum={accum}")
    _, _, (gv_ref, gl_ref, ga_ref), _ = oracle_run(inp)
    g = to_dev(inp)
    got = msda_backward(g["value"], g["spatial_shapes"], None, g["sampling_locations"],
                        g["attention_weights"], g["grad_output"], accum=accum)
    torch.cuda.synchronize()
    tol = 1e-5 if dtype == torch.float32 else 2e-2
    for name, t, ref in zip(("grad_value", "grad_sampling_locations",
                             "grad_attention_weights"), got, (gv_ref, gl_ref, ga_ref)):
        a = t.detach().float().cpu().numpy().astype(np.float64)
        ref = np.asarray(ref, dtype=np.float64).reshape(a.shape)
        fin, fin_ref = np.isfinite(a), np.isfinite(ref)
        assert (~fin_ref).any(), f"{name}: the oracle has no non-finite entry"
        assert np.array_equal(fin, fin_ref), \
            f"{name}: {int((fin != fin_ref).sum())} entries differ in finiteness"
        if name == "grad_value":  # only head m_bad is touched (B = 1)
            assert not np.delete(~fin, m_bad, axis=2).any()
        else:  # only query q_bad, head m_bad
            bad = ~fin.reshape(1, wl.num_queries, wl.M, -1)
            assert bad[0, q_bad, m_bad].any()
            bad[0, q_bad, m_bad] = False
            assert not bad.any()
        err = np.linalg.norm(a[fin] - ref[fin]) / max(np.linalg.norm(ref[fin]), 1e-300)
        assert err <= tol, f"{name}: normwise error {err:.3e} on the finite entries"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("accum", ["auto", "binned", "native"])
def test_non_finite_locations_are_out_of_bounds(dtype, accum):
    """A NaN, infinite or huge sampling coordinate puts its point outside the level:
    every result equals the oracle's with that coordinate moved far out of
    bounds (-10), i.e. the point adds exactly 0 to the output and to
    grad_value, and its own location and weight gradients are 0. (The oracle
    itself refuses non-finite locations; the substitution pins the reading
    that they count as out of bounds.)"""
    wl, inp = _small(dtype, D=32, Q=40, M=2, K=4, levels=((12, 16), (6, 8), (3, 4)))
    nan, inf = float("nan"), float("inf")
    bad = [((0, 3, 1, 0, 2, 0), nan), ((0, 5, 0, 1, 1, 1), inf), ((1, 7, 1, 2, 3, 0), -inf),
           ((1, 9, 0, 0, 0, 0), nan), ((1, 9, 0, 0, 0, 1), nan), ((0, 11, 1, 2, 0, 1), -inf),
           ((0, 13, 0, 1, 2, 0), 1e38)]  # finite, but its product with W overflows fp32
    loc, sub = inp["sampling_locations"].clone(), inp["sampling_locations"].clone()
    for idx, v in bad:
        loc[idx] = v
        sub[idx] = -10.0
    ref_inp = dict(inp, sampling_locations=sub)
    say(f"case non-finite locations {dtype} accum={accum}")
    ref_out, touched, ref_grads, trows = oracle_run(ref_inp)
    g = to_dev(dict(inp, sampling_locations=loc))
    out = msda_forward(g["value"], g["spatial_shapes"], None, g["sampling_locations"],
                       g["attention_weights"])
    grads = msda_backward(g["value"], g["spatial_shapes"], None, g["sampling_locations"],
                          g["attention_weights"], g["grad_output"], accum=accum)
    torch.cuda.synchronize()
    check_forward(dtype, out.cpu(), ref_out, touched)
    grads = tuple(t.cpu() for t in grads)
    check_backward(dtype, grads, ref_grads, inp["spatial_shapes"], None, trows,
                   **parity_kwargs(dtype, accum, ref_inp))
    for idx, _ in bad:
        assert float(grads[1][idx[:5]].abs().max()) == 0.0 and float(grads[2][idx[:5]]) == 0.0


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
def test_non_finite_locations_under_the_quad_setup(dtype):
    """The same reading as above on shapes that take the quad setup (4-lane
    groups holding a whole head row, one lane group per query) in the
    forward and the gradients-only kernel, and the binned chain with merged
    records (pixel queries, K = 4): NaN, infinite and overflowing coordinates,
    among them all four points of one (query, level) and a point whose x
    alone is NaN, count as out of bounds."""
    D = 16 if dtype == torch.float32 else 32
    wl = Workload(name="quad_nonfinite", dtype=dtype, B=2, Q=None, M=8, D=D, K=4,
                  levels=((40, 56), (20, 28), (10, 14), (5, 7)), loc_kind="reference",
                  loc_sigma=0.03, seed=81)
    inp = make_inputs(wl)
    nan, inf = float("nan"), float("inf")
    bad = [((0, 100, 3, 0, 2, 0), nan), ((1, 2300, 5, 1, 1, 1), inf),
           ((1, 2900, 7, 3, 3, 0), -inf), ((0, 17, 0, 2, 0, 1), 1e38)]
    bad += [((1, 2950, 2, 3, k, c), nan) for k in range(4) for c in range(2)]  # a whole quad
    loc, sub = inp["sampling_locations"].clone(), inp["sampling_locations"].clone()
    for idx, v in bad:
        loc[idx] = v
        sub[idx] = -10.0
    ref_inp = dict(inp, sampling_locations=sub)
    say(f"case non-finite locations, quad setup {dtype}")
    ref_out, touched, ref_grads, trows = oracle_run(ref_inp)
    g = to_dev(dict(inp, sampling_locations=loc))
    out = msda_forward(g["value"], g["spatial_shapes"], None, g["sampling_locations"],
                       g["attention_weights"])
    grads = msda_backward(g["value"], g["spatial_shapes"], None, g["sampling_locations"],
                          g["attention_weights"], g["grad_output"], accum="binned")
    torch.cuda.synchronize()
    check_forward(dtype, out.cpu(), ref_out, touched)
    grads = tuple(t.cpu() for t in grads)
    check_backward(dtype, grads, ref_grads, inp["spatial_shapes"], None, trows,
                   **parity_kwargs(dtype, "binned", ref_inp))
    for idx, _ in bad:
        assert float(grads[1][idx[:5]].abs().max()) == 0.0 and float(grads[2][idx[:5]]) == 0.0


def test_single_stream_flag_and_side_stream_release():
    """The odd-head workload bins about 9 * 10^5 records, so by default its
    binned chain runs on the thread's side stream. With single_stream the
    whole backward stays on the caller's stream. Both must match the oracle;
    after msda_release_thread_resources the next call creates the side stream
    again and still matches."""
    from scale_deformable_attention_amd._binding import release_thread_resources
    name = "oddhead_fp32"
    wl = workload(name)
    inp, (ref_out, touched, ref_grads, trows) = _cached(name)
    kw = parity_kwargs(wl.dtype, "auto", inp, workload_name=name)
    g = to_dev(inp)
    args = (g["value"], g["spatial_shapes"], None, g["sampling_locations"], g["attention_weights"],
            g["grad_output"])
    for single, release in ((True, False), (False, True), (False, False)):
        say(f"case {name} single_stream={single} release_after={release}")
        grads = msda_backward(*args, accum="auto", single_stream=single)
        torch.cuda.synchronize()
        report(check_backward(wl.dtype, tuple(t.cpu() for t in grads), ref_grads,
                              inp["spatial_shapes"], None, trows, **kw))
        if release:
            release_thread_resources()


def _reorder_levels(inp, levels, order):
    """Store the levels along S in `order` (value rows and, for pixel queries,
    the queries move together); returns the level_start_index that still
    tiles [0, S)."""
    sizes = [h * w for h, w in levels]
    st, acc = [0] * len(levels), 0
    for l in order:
        st[l] = acc
        acc += sizes[l]
    dflt = np.cumsum([0] + sizes[:-1])
    perm = np.concatenate([np.arange(dflt[l], dflt[l] + sizes[l]) for l in order])
    inp["value"] = inp["value"][:, perm].contiguous()
    for k in ("sampling_locations", "attention_weights", "grad_output"):
        inp[k] = inp[k][:, perm].contiguous()
    return torch.tensor(st)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("reordered", [False, True])
def test_pixel_queries_in_column_groups(dtype, reordered):
    """Encoder-style queries (every pyramid pixel, sampling near its own
    pixel) with fewer (batch, head group) pairs than XCDs: the forward and
    gradient kernels visit the queries in column groups of every level.
    Odd level widths give ragged tiles at every group edge; `reordered`
    stores the levels in another order along S (a given level_start_index
    that still tiles [0, S)). Results must match the oracle as in any order."""
    levels = ((24, 37), (12, 19), (6, 10), (3, 5))
    wl = Workload(name="pixels", dtype=dtype, B=1, Q=None, M=4, D=32, K=4, levels=levels,
                  loc_kind="reference", loc_sigma=0.05, seed=31)
    inp = make_inputs(wl)
    starts = _reorder_levels(inp, levels, [2, 0, 3, 1]) if reordered else None
    say(f"case pixel queries in column groups {dtype} reordered={reordered}")
    for accum in ("auto", "native"):
        full_check(inp, dtype, accum, starts=starts)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=str)
@pytest.mark.parametrize("K", [2, 4])
def test_pixel_query_points_sharing_pixels(dtype, K):
    """Pixel queries whose K points lie within a fraction of a pixel of one
    another on the coarse levels, so two, three or all K of one query's points
    put a corner on the same pixel; the binned chain's count and place merge
    such corners into one record. A tenth of the points is pushed outside
    its level (some corners or all of them out of bounds). grad_value must
    match the oracle exactly as without merging."""
    levels = ((30, 44), (15, 22), (8, 11), (4, 6))
    wl = Workload(name="shared", dtype=dtype, B=2, Q=None, M=2, D=16, K=K, levels=levels,
                  loc_kind="reference", loc_sigma=0.01, seed=41)
    inp = make_inputs(wl)
    loc = inp["sampling_locations"]
    far = torch.rand(loc.shape[:-1], generator=torch.Generator().manual_seed(7)) < 0.1
    loc[far] = (loc[far].float() * 1.6 - 0.3).to(loc.dtype)
    say(f"case pixel queries sharing pixels K={K} {dtype}")
    names, grads = _backward_launch_names(inp, "binned")
    assert "bin_count" in names and "bin_place" in names, names  # the chain that merges
    _, _, ref_grads, trows = oracle_run(inp)
    check_backward(dtype, grads, ref_grads, inp["spatial_shapes"], None, trows,
                   **parity_kwargs(dtype, "binned", inp))


@pytest.mark.parametrize("dtype", DTYPES, ids=str)
@pytest.mark.parametrize("case", ["pixels", "uniform_k8"])
def test_quad_setup_matches_plain_forward(dtype, case):
    """Four-lane groups holding exactly D channels (D = 32 in 16-bit types,
    D = 16 in fp32), one lane group per query and chunks inside one level:
    the forward and the gradients-only kernel work out each point's cell,
    weights and offsets once per quad and broadcast them. The forced
    plain-load path works every point out in every lane; the two forwards
    must agree bit for bit (the same arithmetic), and the forward and the
    binned backward (whose gradients come from the gradients-only kernel)
    must match the oracle. 'pixels': encoder-style queries with a tenth of
    the points pushed outside their level; 'uniform_k8': 2048 queries with
    uniform locations (some out of bounds), K = 8 on 2 levels."""
    from scale_deformable_attention_amd._binding import force_flat_gathers
    D = 16 if dtype == torch.float32 else 32
    if case == "pixels":
        wl = Workload(name="quad", dtype=dtype, B=2, Q=None, M=8, D=D, K=4,
                      levels=((40, 56), (20, 28), (10, 14), (5, 7)), loc_kind="reference",
                      loc_sigma=0.05, seed=61)
    else:
        wl = Workload(name="quad", dtype=dtype, B=2, Q=2048, M=8, D=D, K=8,
                      levels=((30, 41), (15, 21)), loc_kind="uniform", loc_lo=-0.1, loc_hi=1.1,
                      seed=62)
    inp = make_inputs(wl)
    if case == "pixels":
        loc = inp["sampling_locations"]
        far = torch.rand(loc.shape[:-1], generator=torch.Generator().manual_seed(9)) < 0.1
        loc[far] = (loc[far].float() * 1.6 - 0.3).to(loc.dtype)
    say(f"case quad setup {dtype} {case}")
    g = to_dev(inp)
    args = (g["value"], g["spatial_shapes"], None, g["sampling_locations"],
            g["attention_weights"])
    out = msda_forward(*args).cpu()
    with force_flat_gathers():
        out_plain = msda_forward(*args).cpu()
    assert torch.equal(out, out_plain), (out.float() - out_plain.float()).abs().max()
    names, _ = _backward_launch_names(inp, "binned")
    assert "msda_grad_kernel" in names, names
    full_check(inp, dtype, "binned")


@pytest.mark.parametrize("dtype", DTYPES, ids=str)
def test_quad_setup_with_element_aligned_parameters(dtype):
    """The quad setup when the locations and weights (and their gradients)
    start one element into their buffers: value rows stay 16-byte aligned, so
    the forward and the gradients-only kernel keep the quad setup, but each
    lane loads its chunk's parameters element by element instead of with
    vector loads. Forward bit for bit against the plain-load path; forward and
    binned backward against the oracle."""
    from scale_deformable_attention_amd._binding import force_flat_gathers
    D = 16 if dtype == torch.float32 else 32
    wl = Workload(name="quad_align", dtype=dtype, B=2, Q=None, M=8, D=D, K=4,
                  levels=((40, 56), (20, 28), (10, 14), (5, 7)), loc_kind="reference",
                  loc_sigma=0.04, seed=91)
    inp = make_inputs(wl)
    g = to_dev(inp)
    say(f"case quad setup, element-aligned parameters {dtype}")

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        return v
    loc, a = shifted(g["sampling_locations"]), shifted(g["attention_weights"])
    args = (g["value"], g["spatial_shapes"], None, loc, a)
    out = msda_forward(*args).cpu()
    with force_flat_gathers():
        out_plain = msda_forward(*args).cpu()
    assert torch.equal(out, out_plain), (out.float() - out_plain.float()).abs().max()
    ref_out, touched, ref_grads, trows = oracle_run(inp)
    check_forward(dtype, out, ref_out, touched)
    gl = shifted(torch.empty_like(g["sampling_locations"]))
    ga = shifted(torch.empty_like(g["attention_weights"]))
    grads = msda_backward(*args, g["grad_output"], grad_sampling_locations=gl,
                          grad_attention_weights=ga, accum="binned")
    torch.cuda.synchronize()
    check_backward(dtype, tuple(t.cpu() for t in grads), ref_grads, inp["spatial_shapes"], None,
                   trows, **parity_kwargs(dtype, "binned", inp))


# Levels above 256 contributions per pixel, summed by PREREDUCE's in-LDS sort:
# pixel queries (merged tiles; levels stored out of order; a wide head whose
# tiles shrink to fit LDS), consecutive-query blocks, a level larger than the
# window (corners outside it add straight into the scratch) and a wide head
# with 8 points whose blocks shrink.
PRE_CASES = {
    "pixels": dict(B=2, Q=None, M=4, D=32, K=4, levels=((24, 37), (12, 19), (6, 10), (3, 5)),
                   loc_kind="reference", loc_sigma=0.05, seed=41),
    "pixels_reordered": dict(B=2, Q=None, M=4, D=32, K=4,
                             levels=((24, 37), (12, 19), (6, 10), (3, 5)),
                             loc_kind="reference", loc_sigma=0.05, seed=42),
    "pixels_wide_head": dict(B=1, Q=None, M=1, D=128, K=4,
                             levels=((24, 37), (12, 19), (6, 10), (3, 5)),
                             loc_kind="reference", loc_sigma=0.05, seed=43),
    "linear": dict(B=2, Q=600, M=2, D=16, K=4, levels=((9, 11), (4, 5), (2, 3)),
                   loc_kind="uniform", loc_lo=-0.1, loc_hi=1.1, seed=44),
    "beyond_window": dict(B=1, Q=30000, M=1, D=8, K=4, levels=((40, 40),),
                          loc_kind="uniform", loc_lo=-0.1, loc_hi=1.1, seed=45),
    "linear_wide_head": dict(B=1, Q=700, M=2, D=256, K=8, levels=((6, 7), (3, 4)),
                             loc_kind="uniform", loc_lo=-0.1, loc_hi=1.1, seed=46),
}


@pytest.mark.parametrize("dtype", DTYPES, ids=str)
@pytest.mark.parametrize("case", list(PRE_CASES))
def test_prereduce_cases(dtype, case):
    """PREREDUCE against the oracle; the plan (which levels are pre-reduced)
    is checked against the documented policy inside parity_kwargs."""
    wl = Workload(name=case, dtype=dtype, **PRE_CASES[case])
    inp = make_inputs(wl)
    starts = _reorder_levels(inp, wl.levels, [2, 0, 3, 1]) if case == "pixels_reordered" else None
    modes = plan_for(dtype, "prereduce", inp, starts)
    assert "prereduce" in modes, modes
    say(f"case prereduce {case} {dtype}: Q={wl.num_queries} D={wl.D} K={wl.K} plan={modes}")
    full_check(inp, dtype, "prereduce", starts=starts)


@pytest.mark.parametrize("dtype", DTYPES, ids=str)
@pytest.mark.parametrize("accum", ["binned", "prereduce"])
def test_degenerate_levels_with_pixel_queries(dtype, accum):
    """Pixel queries over levels of one pixel, one row and one column, points
    spread well past the map: binned with merged records (K = 4), and with
    the 1 x 1 level pre-reduced (every in-bounds corner of all its points is
    the one pixel)."""
    wl = Workload(name="pixels_degenerate", dtype=dtype, B=2, Q=None, M=4, D=32, K=4,
                  levels=((1, 1), (1, 7), (7, 1), (2, 3)), loc_kind="reference",
                  loc_sigma=0.3, seed=47)
    inp = make_inputs(wl)
    modes = plan_for(dtype, accum, inp)
    assert accum in modes, modes
    say(f"case degenerate levels, pixel queries {dtype} {accum}: plan={modes}")
    full_check(inp, dtype, accum)


@pytest.mark.parametrize("dtype", DTYPES, ids=str)
def test_prereduce_accumulates_and_ignores_out_of_bounds_points(dtype):
    """PREREDUCE with MSDA_FLAG_ACCUMULATE_GRAD_VALUE adds the pre-reduced sums
    into the existing grad_value; with every point outside its level the
    gradients are exactly zero."""
    wl = Workload(name="linear", dtype=dtype, **PRE_CASES["linear"])
    inp = make_inputs(wl)
    g = to_dev(inp)
    say(f"case prereduce accumulate twice {dtype}")
    args = (g["value"], g["spatial_shapes"], None, g["sampling_locations"], g["attention_weights"],
            g["grad_output"])
    gv1, _, _ = msda_backward(*args, accum="prereduce")
    once = gv1.clone()
    msda_backward(*args, grad_value=gv1, accum="prereduce", accumulate=True)
    torch.cuda.synchronize()
    ref = oracle.backward(inp["value"], inp["spatial_shapes"], None, inp["sampling_locations"],
                          inp["attention_weights"], inp["grad_output"])[0]
    kw = parity_kwargs(dtype, "prereduce", inp)
    report(check_grad_value(dtype, to_np(once), ref, inp["spatial_shapes"], **kw))
    report(check_grad_value(dtype, to_np(gv1), 2 * ref, inp["spatial_shapes"], passes=2, **kw))

    loc = inp["sampling_locations"].float()
    sel = torch.rand(loc.shape[:-1], generator=torch.Generator().manual_seed(2)) < 0.5
    loc[..., 1] = torch.where(sel, torch.tensor(1.7), torch.tensor(-0.9))
    inp["sampling_locations"] = loc.to(dtype)
    say(f"case prereduce all points out of bounds {dtype}")
    out, (gv, gl, ga) = gpu_run(inp, "prereduce")
    assert torch.all(out == 0) and torch.all(gv == 0) and torch.all(gl == 0) and torch.all(ga == 0)


@pytest.mark.parametrize("dtype", DTYPES, ids=str)
@pytest.mark.parametrize("accum", ["auto", "native", "fp32_scratch"])
def test_plain_load_path_for_large_slices(dtype, accum):
    """The gathers' fallback for batch value slices of 2 GiB or more (plain
    loads from clamped addresses instead of a buffer resource), forced on a
    small problem with out-of-bounds corners on every side: forward and
    backward against the oracle, planned as for such slices (no binning)."""
    from scale_deformable_attention_amd._binding import force_flat_gathers
    wl, inp = _small(dtype, D=16, Q=97, K=4, levels=((6, 9), (3, 5), (2, 2)), lo=-0.2, hi=1.2,
                     seed=81)
    say(f"case plain-load gathers {dtype} {accum}")
    with force_flat_gathers():
        modes = plan_for(dtype, accum, inp, flat=True)
        assert "binned" not in modes and "prereduce" not in modes, modes
        full_check(inp, dtype, accum, flat=True)
