"""The steps around the core on the GPU against their oracle (oracle/module.py).

msda_sampling_prep / msda_sampling_prep_backward are compared element by
element with the oracle's reference scaling and softmax over L*K (msda-triton
README, sections "The operator" and "Quickstart"), over lane layouts with
L*K a power of two, not a power of two, and above 64 (several points per
lane), with one reference point per query and one per level, in fp32 and in
bf16. The MSDeformAttn module (projections + prep + core) is compared with
the oracle-composed module: output and every gradient.

Tolerance (|gpu - oracle| <= tol * (|oracle| + rms)): fp32 1e-5 for the prep
steps (one fp32 division / a softmax with one exp per point); fp32 module
2e-5, because each value passes through up to three fp32 GEMMs with
reductions over d_model or B*S rows, each adding a relative error of order
sqrt(n) * 2^-24 on top of the core's; bf16 2e-2 (outputs, prep) and 5e-2
(gradients), the core's bf16 bars.

Locations are piecewise-differentiable: a point whose pixel coordinate is
within rounding of an integer takes its slope from either cell. The GPU's
locations come from GEMMs and divisions in fp32, the oracle's in fp64, so the
module cases use seeds whose oracle pixel coordinates keep a margin from
every integer (asserted); the bf16 module case keeps its sampling parameters
in fp32 (param_dtype), as 16-bit offsets would move the locations by a few
hundredths of a pixel. An all-bf16 module is checked normwise.
"""

import numpy as np
import pytest
import torch

from oracle import module as om

from _parity import check_slice, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _library():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import os
    from scale_deformable_attention_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    _binding.load_library()


def say(msg):
    print(msg, flush=True)


def _prep_inputs(seed, B, Q, M, levels, K, per_level, dtype):
    g = torch.Generator().manual_seed(seed)
    L = len(levels)
    ref = torch.rand((B, Q, L, 2) if per_level else (B, Q, 2), generator=g)
    off = torch.randn(B, Q, M, L, K, 2, generator=g) * 3.0
    logits = torch.randn(B, Q, M, L * K, generator=g) * 2.0
    grad_loc = torch.randn(B, Q, M, L, K, 2, generator=g)
    grad_attn = torch.randn(B, Q, M, L, K, generator=g)
    attn = torch.softmax(torch.randn(B, Q, M, L * K, generator=g), -1).view(B, Q, M, L, K)
    return [t.to(dtype) for t in (ref, off, logits, grad_loc, grad_attn, attn)]


PREP_CASES = [
    # name, B, Q, M, levels, K
    ("lk16", 2, 37, 8, ((100, 167), (50, 84), (25, 42), (13, 21)), 4),
    ("lk9_padded_lanes", 1, 50, 3, ((7, 9), (5, 4), (2, 3)), 3),
    ("lk80_two_per_lane", 1, 20, 2, ((16, 16), (8, 8), (4, 4), (2, 2)), 20),
    ("lk1", 3, 5, 1, ((6, 6),), 1),
]


@pytest.mark.parametrize("per_level", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("case", PREP_CASES, ids=lambda c: c[0])
def test_sampling_prep_matches_oracle(case, dtype, per_level):
    from scale_deformable_attention_amd import msda_sampling_prep, msda_sampling_prep_backward
    name, B, Q, M, levels, K = case
    say(f"case prep {name} {dtype} per_level={per_level}")
    ref, off, logits, grad_loc, grad_attn, attn = _prep_inputs(17, B, Q, M, levels, K, per_level,
                                                               dtype)
    shapes = torch.tensor(levels)
    loc_g, attn_g = msda_sampling_prep(ref.to(DEV), off.to(DEV), logits.to(DEV), shapes)
    g_ref, g_off, g_logits = msda_sampling_prep_backward(
        attn.to(DEV), grad_loc.to(DEV), grad_attn.to(DEV), shapes, ref_per_level=per_level)
    torch.cuda.synchronize()
    loc_o, attn_o = om.sampling_prep(ref, off, logits, shapes)
    r_ref, r_off, r_logits = om.sampling_prep_backward(attn, grad_loc, grad_attn, shapes,
                                                       ref_per_level=per_level)
    tol = 1e-5 if dtype == torch.float32 else 2e-2
    check_slice("sampling_locations", to_np(loc_g), loc_o, tol)
    check_slice("attention_weights", to_np(attn_g), attn_o, tol)
    check_slice("grad_sampling_offsets", to_np(g_off), r_off, tol)
    check_slice("grad_attention_logits", to_np(g_logits), r_logits, tol)
    check_slice("grad_reference_points", to_np(g_ref), r_ref, tol)
    assert loc_g.dtype == dtype and g_logits.shape == logits.shape


def test_sampling_prep_empty_and_no_reference_grad():
    from scale_deformable_attention_amd import msda_sampling_prep, msda_sampling_prep_backward
    shapes = [[4, 4], [2, 2]]
    loc, attn = msda_sampling_prep(torch.zeros(2, 0, 2, device=DEV),
                                   torch.zeros(2, 0, 3, 2, 2, 2, device=DEV),
                                   torch.zeros(2, 0, 3, 4, device=DEV), shapes)
    assert loc.shape == (2, 0, 3, 2, 2, 2) and attn.shape == (2, 0, 3, 2, 2)
    ref, off, logits, gl, ga, a = _prep_inputs(3, 1, 4, 2, ((4, 4), (2, 2)), 2, False,
                                               torch.float32)
    g_ref, g_off, g_logits = msda_sampling_prep_backward(a.to(DEV), gl.to(DEV), ga.to(DEV), shapes,
                                                         need_reference_grad=False)
    assert g_ref is None
    torch.cuda.synchronize()
    r_ref, r_off, r_logits = om.sampling_prep_backward(a, gl, ga, shapes)
    check_slice("grad_sampling_offsets", to_np(g_off), r_off, 1e-5)


# ------------------------------------------------------------------ module

MODULE_LEVELS = ((12, 20), (6, 10), (3, 5))


def _module_case(dtype, per_level, seed):
    from scale_deformable_attention_amd import MSDeformAttn
    B, Q, C, M, K = 2, 24, 32, 4, 2
    L = len(MODULE_LEVELS)
    torch.manual_seed(seed)
    mod = MSDeformAttn(d_model=C, n_levels=L, n_heads=M, n_points=K)
    with torch.no_grad():  # offsets of a few pixels
        mod.sampling_offsets.weight.mul_(4.0)
        mod.sampling_offsets.bias.normal_(0.0, 2.0)
    g = torch.Generator().manual_seed(seed + 1)
    S = sum(h * w for h, w in MODULE_LEVELS)
    x = torch.randn(B, Q, C, generator=g)
    ref = 0.1 + 0.8 * torch.rand((B, Q, L, 2) if per_level else (B, Q, 2), generator=g)
    inp = torch.randn(B, S, C, generator=g)
    gout = torch.randn(B, Q, C, generator=g)
    params = {k: v.detach().clone() for k, v in mod.state_dict().items()}
    # the oracle computes from the weights and inputs as stored in `dtype`
    if dtype != torch.float32:
        params = {k: v.to(dtype) for k, v in params.items()}
        x, ref, inp, gout = (t.to(dtype) for t in (x, ref, inp, gout))
    return mod, params, x, ref, inp, gout, M, K


def _kink_margin(params, x, ref, inp, M, K):
    _, it = om.module_forward(params, x, ref, inp, MODULE_LEVELS, heads=M, points=K,
                              return_intermediates=True)
    loc = it["loc"]
    m = np.inf
    for l, (H, W) in enumerate(MODULE_LEVELS):
        for c, size in ((0, W), (1, H)):
            pix = loc[:, :, :, l, :, c] * size - 0.5
            m = min(m, float(np.min(np.abs(pix - np.round(pix)))))
    return m


def _first_seed_with_margin(dtype, per_level, margin):
    for seed in range(100, 140):
        _, params, x, ref, inp, _, M, K = _module_case(dtype, per_level, seed)
        if _kink_margin(params, x, ref, inp, M, K) > margin:
            return seed
    raise AssertionError("no seed keeps the pixel coordinates away from integers")


@pytest.mark.parametrize("per_level", [False, True])
@pytest.mark.parametrize("dtype,param_dtype", [(torch.float32, None),
                                               (torch.bfloat16, torch.float32)])
def test_module_forward_backward_matches_oracle(dtype, param_dtype, per_level):
    say(f"case module {dtype} params {param_dtype} per_level={per_level}")
    seed = _first_seed_with_margin(dtype, per_level, 2e-4)
    mod, params, x, ref, inp, gout, M, K = _module_case(dtype, per_level, seed)
    mod.param_dtype = param_dtype
    mod = mod.to(device=DEV, dtype=dtype)
    xg = x.to(DEV).requires_grad_(True)
    refg = ref.to(DEV).requires_grad_(True)
    inpg = inp.to(DEV).requires_grad_(True)
    out = mod(xg, refg, inpg, torch.tensor(MODULE_LEVELS))
    out.backward(gout.to(DEV))
    torch.cuda.synchronize()
    ref_out = om.module_forward(params, x, ref, inp, MODULE_LEVELS, heads=M, points=K)
    grads = om.module_backward(params, x, ref, inp, MODULE_LEVELS, gout, heads=M, points=K)
    tol_out, tol_grad = (2e-5, 2e-5) if dtype == torch.float32 else (2e-2, 5e-2)
    check_slice("output", to_np(out), ref_out, tol_out)
    got = {"query": xg.grad, "reference_points": refg.grad, "input_flatten": inpg.grad}
    got.update({n: p.grad for n, p in mod.named_parameters()})
    for name, want in grads.items():
        g = to_np(got[name])
        assert g.shape == want.shape, name
        check_slice(name, g, want, tol_grad)


def test_module_all_bf16_normwise():
    """Offsets, locations and weights in bf16 too: the locations carry bf16
    rounding (a few hundredths of a pixel), so the output is held normwise to
    the bf16 forward bar and every gradient must be finite."""
    say("case module all bf16")
    mod, params, x, ref, inp, gout, M, K = _module_case(torch.bfloat16, False, 100)
    mod = mod.to(device=DEV, dtype=torch.bfloat16)
    xg = x.to(DEV).requires_grad_(True)
    inpg = inp.to(DEV).requires_grad_(True)
    out = mod(xg, ref.to(DEV), inpg, MODULE_LEVELS)
    out.backward(gout.to(DEV))
    torch.cuda.synchronize()
    want = om.module_forward(params, x, ref, inp, MODULE_LEVELS, heads=M, points=K)
    got = to_np(out)
    assert np.linalg.norm(got - want) / np.linalg.norm(want) <= 2e-2
    for t in [xg.grad, inpg.grad] + [p.grad for p in mod.parameters()]:
        assert torch.isfinite(t).all()


def test_module_mixed_param_dtype_runs_fp32_locations():
    """bf16 module with fp32 offsets, logits, locations and weights: the
    sampling parameters stay fp32 into the core (mixed-dtype entry points)."""
    from scale_deformable_attention_amd import MSDeformAttn
    say("case module bf16 with fp32 sampling parameters")
    torch.manual_seed(5)
    mod = MSDeformAttn(d_model=32, n_levels=3, n_heads=4, n_points=2,
                       param_dtype=torch.float32).to(device=DEV, dtype=torch.bfloat16)
    seen = {}
    import scale_deformable_attention_amd.module as mm
    orig = mm.multi_scale_deformable_attention

    def spy(value, shapes, starts, loc, attn, switch):
        seen["dtypes"] = (value.dtype, loc.dtype, attn.dtype)
        return orig(value, shapes, starts, loc, attn, switch)
    mm.multi_scale_deformable_attention = spy
    try:
        S = sum(h * w for h, w in MODULE_LEVELS)
        x = torch.randn(2, 10, 32, device=DEV, dtype=torch.bfloat16, requires_grad=True)
        inp = torch.randn(2, S, 32, device=DEV, dtype=torch.bfloat16, requires_grad=True)
        ref = torch.rand(2, 10, 2, device=DEV)
        out = mod(x, ref, inp, MODULE_LEVELS)
        out.float().sum().backward()
        torch.cuda.synchronize()
    finally:
        mm.multi_scale_deformable_attention = orig
    assert seen["dtypes"] == (torch.bfloat16, torch.float32, torch.float32)
    assert out.dtype == torch.bfloat16 and torch.isfinite(out).all()
    assert torch.isfinite(x.grad).all() and torch.isfinite(inp.grad).all()
    assert mod.sampling_offsets.weight.grad is not None


def test_module_padding_mask_zeroes_value_rows():
    """input_padding_mask zeroes the value rows of padded input positions: the
    output does not change when those inputs change, and their input
    gradients are zero."""
    from scale_deformable_attention_amd import MSDeformAttn
    say("case module padding mask")
    torch.manual_seed(9)
    mod = MSDeformAttn(d_model=32, n_levels=3, n_heads=4, n_points=2).to(DEV)
    S = sum(h * w for h, w in MODULE_LEVELS)
    g = torch.Generator().manual_seed(10)
    x = torch.randn(2, 12, 32, generator=g).to(DEV)
    ref = (0.1 + 0.8 * torch.rand(2, 12, 2, generator=g)).to(DEV)
    inp = torch.randn(2, S, 32, generator=g).to(DEV)
    mask = torch.rand(2, S, generator=g).to(DEV) < 0.3
    other = inp.clone()
    other[mask] = torch.randn(int(mask.sum()), 32, device=DEV) * 5.0
    a = mod(x, ref, inp, MODULE_LEVELS, input_padding_mask=mask)
    inp_b = other.clone().requires_grad_(True)
    b = mod(x, ref, inp_b, MODULE_LEVELS, input_padding_mask=mask)
    b.sum().backward()
    torch.cuda.synchronize()
    assert torch.allclose(a, b, rtol=0, atol=0), "padded inputs changed the output"
    assert not inp_b.grad[mask].any(), "padded inputs received gradient"
    assert inp_b.grad[~mask].abs().sum() > 0


def test_module_graph_capture_replays_match_eager():
    """MSDeformAttn forward + backward captured in one HIP graph (the
    projections, the prep kernels and the core): every replay with new inputs
    copied into the captured buffers matches an eager run on those inputs."""
    from scale_deformable_attention_amd import MSDeformAttn
    say("case module graph capture")
    torch.manual_seed(12)
    mod = MSDeformAttn(d_model=32, n_levels=3, n_heads=4, n_points=2).to(DEV)
    shapes = torch.tensor(MODULE_LEVELS)  # host table: nothing to copy under capture
    S = sum(h * w for h, w in MODULE_LEVELS)
    x = torch.zeros(2, 16, 32, device=DEV, requires_grad=True)
    ref = torch.zeros(2, 16, 2, device=DEV)
    inp = torch.zeros(2, S, 32, device=DEV, requires_grad=True)
    gout = torch.zeros(2, 16, 32, device=DEV)

    def fill(seed):
        g = torch.Generator().manual_seed(seed)
        with torch.no_grad():
            x.copy_(torch.randn(2, 16, 32, generator=g))
            ref.copy_(0.1 + 0.8 * torch.rand(2, 16, 2, generator=g))
            inp.copy_(torch.randn(2, S, 32, generator=g))
            gout.copy_(torch.randn(2, 16, 32, generator=g))

    fill(1)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            out = mod(x, ref, inp, shapes)
            out.backward(gout)
            del out
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    mod.zero_grad(set_to_none=False)
    x.grad.zero_()
    inp.grad.zero_()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        static_out = mod(x, ref, inp, shapes)
        static_out.backward(gout)
    torch.cuda.synchronize()
    params = dict(mod.named_parameters())
    static_grads = {n: p.grad for n, p in params.items()}  # the tensors the graph adds into
    for trial in range(3):
        fill(100 + trial)
        for p in params.values():
            p.grad.zero_()
        x.grad.zero_()
        inp.grad.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {"out": static_out.detach().clone(), "x": x.grad.clone(), "inp": inp.grad.clone()}
        got.update({n: p.grad.clone() for n, p in params.items()})
        # eager on the same inputs
        xe = x.detach().clone().requires_grad_(True)
        ie = inp.detach().clone().requires_grad_(True)
        for p in params.values():
            p.grad = None
        oe = mod(xe, ref, ie, shapes)
        oe.backward(gout)
        torch.cuda.synchronize()
        want = {"out": oe.detach(), "x": xe.grad, "inp": ie.grad}
        want.update({n: p.grad for n, p in params.items()})
        for k in want:
            # grad_value atomics (and so the input and value-projection
            # gradients) may sum in another order: fp32 rounding only
            assert torch.allclose(got[k], want[k], rtol=1e-5, atol=1e-6), (trial, k)
        for n, p in params.items():
            p.grad = static_grads[n]


def test_sampling_prep_encoder_size_and_strided_inputs():
    """The prep kernels at the encoder workload's size (711 K rows of L*K = 16
    points, per-level reference points) against the oracle, with
    non-contiguous inputs (the binding copies them to dense tensors)."""
    from scale_deformable_attention_amd import msda_sampling_prep, msda_sampling_prep_backward
    say("case prep encoder size, strided inputs")
    levels = ((100, 167), (50, 84), (25, 42), (13, 21))
    B, Q, M, K, L = 4, 22223, 8, 4, 4
    g = torch.Generator().manual_seed(23)
    ref = torch.rand(B, Q, L, 2, generator=g)
    off = torch.randn(B, Q, M, L, K, 2, generator=g) * 2.0
    logits = torch.randn(B, Q, M, L * K, generator=g)
    gl = torch.randn(B, Q, M, L, K, 2, generator=g)
    ga = torch.randn(B, Q, M, L, K, generator=g)
    a = torch.softmax(torch.randn(B, Q, M, L * K, generator=g), -1).view(B, Q, M, L, K)
    shapes = torch.tensor(levels)
    # offsets as a transposed view: same values, non-contiguous on the device
    off_t = off.to(DEV).transpose(0, 1).contiguous().transpose(0, 1)
    assert not off_t.is_contiguous()
    loc_g, attn_g = msda_sampling_prep(ref.to(DEV), off_t, logits.to(DEV), shapes)
    g_ref, g_off, g_log = msda_sampling_prep_backward(a.to(DEV), gl.to(DEV), ga.to(DEV), shapes,
                                                      ref_per_level=True)
    torch.cuda.synchronize()
    loc_o, attn_o = om.sampling_prep(ref, off, logits, shapes)
    r_ref, r_off, r_log = om.sampling_prep_backward(a, gl, ga, shapes, ref_per_level=True)
    check_slice("sampling_locations", to_np(loc_g), loc_o, 1e-5)
    check_slice("attention_weights", to_np(attn_g), attn_o, 1e-5)
    check_slice("grad_sampling_offsets", to_np(g_off), r_off, 1e-5)
    check_slice("grad_attention_logits", to_np(g_log), r_log, 1e-5)
    check_slice("grad_reference_points", to_np(g_ref), r_ref, 1e-5)
