"""Pins for the CPU oracle, against things other than the oracle itself.

Each test fixes the oracle to something the pages or mathematics determine:
hand-worked examples (tests/golden), a library routine that computes the same
special case (PyTorch grid_sample in fp64), brute-force finite differences,
closed forms (integer-aligned points, affine and constant fields, all points
out of bounds) and invariants (adjoint identity, per-level conservation,
no wrap-around, thread-count independence).

Sources: msda-triton README ("The operator", "Kernel design": grid_sample
with align_corners=False and zero padding); course page "4. The forward
kernel, line by line" ("Bilinear sampling", "The corner gathers",
"Accumulate and store"); course page "5. The backward kernel" ("What the
backward pass must produce", "Scatter needs atomics").
"""

import glob
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from scale_deformable_attention_amd.workloads import make_inputs, workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(seed, B=2, Q=7, M=3, D=5, K=3, levels=((5, 7), (3, 4), (2, 2)),
               lo=-0.2, hi=1.2, starts=None):
    g = torch.Generator().manual_seed(seed)
    S = sum(h * w for h, w in levels) if starts is None else \
        max(s + h * w for s, (h, w) in zip(starts, levels))
    L = len(levels)
    value = torch.randn(B, S, M, D, generator=g, dtype=torch.float64)
    loc = torch.rand(B, Q, M, L, K, 2, generator=g, dtype=torch.float64) * (hi - lo) + lo
    attn = torch.rand(B, Q, M, L, K, generator=g, dtype=torch.float64)
    gout = torch.randn(B, Q, M * D, generator=g, dtype=torch.float64)
    shapes = torch.tensor(levels, dtype=torch.int64)
    st = None if starts is None else torch.tensor(starts, dtype=torch.int64)
    return value, shapes, st, loc, attn, gout


def _starts(shapes, st):
    if st is not None:
        return [int(s) for s in st]
    out, acc = [], 0
    for h, w in shapes.tolist():
        out.append(acc)
        acc += h * w
    return out


def _grid_sample_msda(value, shapes, st, loc, attn):
    """The core written with torch's grid_sample (align_corners=False, zero
    padding), grid = 2*loc - 1, one call per level, in fp64."""
    B, S, M, D = value.shape
    Q, K = loc.shape[1], loc.shape[4]
    out = torch.zeros(B, Q, M, D, dtype=torch.float64)
    for l, ((H, W), s0) in enumerate(zip(shapes.tolist(), _starts(shapes, st))):
        v = value[:, s0:s0 + H * W].permute(0, 2, 3, 1).reshape(B * M, D, H, W)
        grid = (2 * loc[:, :, :, l] - 1).permute(0, 2, 1, 3, 4).reshape(B * M, Q, K, 2)
        smp = F.grid_sample(v, grid, mode="bilinear", padding_mode="zeros",
                            align_corners=False)  # (B*M, D, Q, K)
        smp = smp.reshape(B, M, D, Q, K).permute(0, 3, 1, 4, 2)  # (B, Q, M, K, D)
        out = out + (attn[:, :, :, l, :, None] * smp).sum(3)
    return out.reshape(B, Q, M * D)


def _close(a, b, rtol):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    scale = np.abs(b) + np.sqrt(np.mean(b * b)) + 1e-300
    err = np.abs(a - b) / scale
    assert err.max() <= rtol, f"max rel err {err.max():.3e} (max abs {np.abs(a - b).max():.3e})"


# ---------------------------------------------------------------- golden

@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(GOLDEN, "*.json"))),
                         ids=lambda p: os.path.basename(p)[:-5])
@pytest.mark.parametrize("mode", ["pinned_f32", "exact_f64"])
def test_golden_worked_examples(path, mode):
    d = json.load(open(path))
    value = np.array(d["value"], np.float64)
    shapes = np.array(d["spatial_shapes"], np.int64)
    st = None if d["level_start_index"] is None else np.array(d["level_start_index"], np.int64)
    loc = np.array(d["sampling_locations"], np.float64)
    attn = np.array(d["attention_weights"], np.float64)
    g = np.array(d["grad_output"], np.float64)
    ex = d["expected"]
    out = oracle.forward(value, shapes, st, loc, attn, mode=mode)
    np.testing.assert_array_equal(out, np.array(ex["output"]))
    gv, gl, ga, touched = oracle.backward(value, shapes, st, loc, attn, g, mode=mode,
                                          return_touched=True)
    np.testing.assert_array_equal(ga, np.array(ex["grad_attention_weights"]))
    np.testing.assert_array_equal(gl, np.array(ex["grad_sampling_locations"]))
    np.testing.assert_array_equal(gv, np.array(ex["grad_value"]))
    np.testing.assert_array_equal(touched, np.array(ex["touched_rows"], bool))


# ---------------------------------------------------------- grid_sample

@pytest.mark.parametrize("seed,starts", [(0, None), (1, None), (2, (30, 0, 13))])
def test_matches_grid_sample_fp64(seed, starts):
    value, shapes, st, loc, attn, gout = _rand_case(seed, starts=starts)
    v, l, a = (t.clone().requires_grad_(True) for t in (value, loc, attn))
    ref = _grid_sample_msda(v, shapes, st, l, a)
    (ref * gout).sum().backward()
    out = oracle.forward(value, shapes, st, loc, attn, mode="exact_f64")
    _close(out, ref.detach().numpy(), 1e-12)
    gv, gl, ga = oracle.backward(value, shapes, st, loc, attn, gout, mode="exact_f64")
    _close(gv, v.grad.numpy(), 1e-12)
    _close(ga, a.grad.numpy(), 1e-12)
    _close(gl, l.grad.numpy(), 1e-11)


def test_matches_grid_sample_on_tiny_workload():
    inp = make_inputs(workload("tiny_fp32"))
    value, loc, attn, gout = (inp[k].double() for k in
                              ("value", "sampling_locations", "attention_weights", "grad_output"))
    shapes = inp["spatial_shapes"]
    v, l, a = (t.clone().requires_grad_(True) for t in (value, loc, attn))
    ref = _grid_sample_msda(v, shapes, None, l, a)
    (ref * gout).sum().backward()
    out = oracle.forward(value, shapes, None, loc, attn, mode="exact_f64")
    _close(out, ref.detach().numpy(), 1e-12)
    gv, gl, ga = oracle.backward(value, shapes, None, loc, attn, gout, mode="exact_f64")
    _close(gv, v.grad.numpy(), 1e-12)
    _close(ga, a.grad.numpy(), 1e-12)
    _close(gl, l.grad.numpy(), 1e-11)


# ---------------------------------------------------- finite differences

def _loss(value, shapes, loc, attn, g):
    return float((oracle.forward(value, shapes, None, loc, attn, mode="exact_f64") * g).sum())


def test_finite_differences_tiny():
    value, shapes, _, loc, attn, gout = _rand_case(7, B=1, Q=4, M=2, D=3, K=2,
                                                   levels=((4, 5), (2, 3)))
    value, loc, attn, g = (t.numpy().copy() for t in (value, loc, attn, gout))
    gv, gl, ga = oracle.backward(value, shapes, None, loc, attn, g, mode="exact_f64")

    # Linear in value and in the attention weights: central differences are exact.
    fd_v = np.zeros_like(value)
    for idx in np.ndindex(*value.shape):
        vp, vm = value.copy(), value.copy()
        vp[idx] += 1.0
        vm[idx] -= 1.0
        fd_v[idx] = (_loss(vp, shapes, loc, attn, g) - _loss(vm, shapes, loc, attn, g)) / 2
    _close(gv, fd_v, 1e-12)
    fd_a = np.zeros_like(attn)
    for idx in np.ndindex(*attn.shape):
        ap, am = attn.copy(), attn.copy()
        ap[idx] += 1.0
        am[idx] -= 1.0
        fd_a[idx] = (_loss(value, shapes, loc, ap, g) - _loss(value, shapes, loc, am, g)) / 2
    _close(ga, fd_a, 1e-12)

    # Piecewise linear in each coordinate: exact within a cell; skip entries
    # whose pixel coordinate is within reach of an integer (a kink).
    h = 1e-7
    checked = 0
    for idx in np.ndindex(*loc.shape):
        l_ = idx[3]
        H, W = shapes[l_].tolist()
        size = W if idx[5] == 0 else H
        pix = loc[idx] * size - 0.5
        frac = pix - np.floor(pix)
        if min(frac, 1 - frac) < 4 * h * size:
            continue
        lp, lm = loc.copy(), loc.copy()
        lp[idx] += h
        lm[idx] -= h
        fd = (_loss(value, shapes, lp, attn, g) - _loss(value, shapes, lm, attn, g)) / (2 * h)
        assert abs(fd - gl[idx]) <= 1e-7 * (abs(gl[idx]) + 1.0), (idx, fd, gl[idx])
        checked += 1
    assert checked > 0.9 * loc.size


# ---------------------------------------------------------- closed forms

def test_integer_aligned_points_reproduce_rows_exactly():
    levels = ((8, 16), (4, 8))  # powers of two: (i + 0.5) / W is exact
    B, Q, M, D, K = 2, 6, 2, 4, 3
    L = len(levels)
    g = torch.Generator().manual_seed(11)
    shapes = torch.tensor(levels)
    S = sum(h * w for h, w in levels)
    value = torch.randn(B, S, M, D, generator=g).double()  # fp32 draws, exact in fp64
    loc = torch.zeros(B, Q, M, L, K, 2, dtype=torch.float64)
    pix = {}
    for idx in np.ndindex(B, Q, M, L, K):
        H, W = levels[idx[3]]
        ix = int(torch.randint(W, (1,), generator=g))
        iy = int(torch.randint(H, (1,), generator=g))
        loc[idx] = torch.tensor([(ix + 0.5) / W, (iy + 0.5) / H], dtype=torch.float64)
        pix[idx] = (ix, iy)
    hot = torch.randint(L * K, (B, Q, M), generator=g)
    attn = F.one_hot(hot, L * K).double().reshape(B, Q, M, L, K)
    gout = torch.randn(B, Q, M * D, generator=g).double()
    starts = _starts(shapes, None)
    out = oracle.forward(value, shapes, None, loc, attn, mode="pinned_f32").reshape(B, Q, M, D)
    gv, gl, ga = oracle.backward(value, shapes, None, loc, attn, gout, mode="pinned_f32")
    gq = gout.reshape(B, Q, M, D).numpy()
    expect_gv = np.zeros_like(gv)
    for b, q, m in np.ndindex(B, Q, M):
        l_, k = divmod(int(hot[b, q, m]), K)
        ix, iy = pix[(b, q, m, l_, k)]
        H, W = levels[l_]
        row = starts[l_] + iy * W + ix
        np.testing.assert_array_equal(out[b, q, m], value[b, row, m].numpy())
        expect_gv[b, row, m] += gq[b, q, m]
        # Right-sided slopes at an integer point: next column / next row minus this one.
        v = value[b, :, m].numpy()
        right = v[row + 1] if ix + 1 < W else 0.0
        down = v[row + W] if iy + 1 < H else 0.0
        np.testing.assert_allclose(gl[b, q, m, l_, k, 0], W * np.dot(gq[b, q, m], right - v[row]),
                                   rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(gl[b, q, m, l_, k, 1], H * np.dot(gq[b, q, m], down - v[row]),
                                   rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(gv, expect_gv)
    # Zero attention weight: no location gradient at all.
    mask0 = (attn.numpy() == 0)
    assert np.all(gl[mask0] == 0)
    # grad_attn of an aligned point is g . value[row].
    for idx in np.ndindex(B, Q, M, L, K):
        ix, iy = pix[idx]
        H, W = levels[idx[3]]
        row = starts[idx[3]] + iy * W + ix
        np.testing.assert_allclose(ga[idx], np.dot(gq[idx[:3]], value[idx[0], row, idx[2]].numpy()),
                                   rtol=1e-13, atol=1e-13)


def _interior_locations(g, shape, levels):
    """Locations whose four corners are all in bounds: x_im in [0, W-1)."""
    loc = torch.empty(*shape, dtype=torch.float64)
    for l_, (H, W) in enumerate(levels):
        u = torch.rand(*shape[:3], shape[4], 2, generator=g, dtype=torch.float64)
        loc[:, :, :, l_, :, 0] = (0.5 + u[..., 0] * (W - 1) * 0.999) / W
        loc[:, :, :, l_, :, 1] = (0.5 + u[..., 1] * (H - 1) * 0.999) / H
    return loc


def test_affine_field_closed_form():
    levels = ((6, 9), (3, 5))
    B, Q, M, D, K = 1, 5, 2, 3, 2
    L = len(levels)
    g = torch.Generator().manual_seed(5)
    shapes = torch.tensor(levels)
    starts = _starts(shapes, None)
    S = sum(h * w for h, w in levels)
    a = torch.randn(M, D, generator=g, dtype=torch.float64)
    bcoef = torch.randn(M, D, generator=g, dtype=torch.float64)
    c = torch.randn(M, D, generator=g, dtype=torch.float64)
    value = torch.zeros(B, S, M, D, dtype=torch.float64)
    for l_, (H, W) in enumerate(levels):
        for y in range(H):
            for x in range(W):
                value[:, starts[l_] + y * W + x] = a * x + bcoef * y + c
    loc = _interior_locations(g, (B, Q, M, L, K, 2), levels)
    attn = torch.rand(B, Q, M, L, K, generator=g, dtype=torch.float64)
    gout = torch.randn(B, Q, M * D, generator=g, dtype=torch.float64)
    out = oracle.forward(value, shapes, None, loc, attn, mode="exact_f64").reshape(B, Q, M, D)
    gv, gl, ga = oracle.backward(value, shapes, None, loc, attn, gout, mode="exact_f64")
    gq = gout.reshape(B, Q, M, D)
    expect = torch.zeros(B, Q, M, D, dtype=torch.float64)
    for l_, (H, W) in enumerate(levels):
        x = loc[:, :, :, l_, :, 0] * W - 0.5  # (B, Q, M, K), page convention
        y = loc[:, :, :, l_, :, 1] * H - 0.5
        field = a[None, None, :, None] * x[..., None] + bcoef[None, None, :, None] * y[..., None] \
            + c[None, None, :, None]  # (B, Q, M, K, D)
        expect += (attn[:, :, :, l_, :, None] * field).sum(3)
        gx = W * attn[:, :, :, l_] * (gq * a).sum(-1)[..., None]
        gy = H * attn[:, :, :, l_] * (gq * bcoef).sum(-1)[..., None]
        _close(gl[:, :, :, l_, :, 0], gx.numpy(), 1e-12)
        _close(gl[:, :, :, l_, :, 1], gy.numpy(), 1e-12)
    _close(out, expect.numpy(), 1e-12)


def test_constant_field_with_normalised_weights():
    levels = ((6, 9), (3, 5))
    B, Q, M, D, K = 2, 5, 2, 3, 2
    L = len(levels)
    g = torch.Generator().manual_seed(6)
    shapes = torch.tensor(levels)
    S = sum(h * w for h, w in levels)
    c = torch.randn(M, D, generator=g, dtype=torch.float64)
    value = c.expand(B, S, M, D).contiguous()
    loc = _interior_locations(g, (B, Q, M, L, K, 2), levels)
    attn = torch.softmax(torch.randn(B, Q, M, L * K, generator=g, dtype=torch.float64), -1)
    attn = attn.reshape(B, Q, M, L, K)
    gout = torch.randn(B, Q, M * D, generator=g, dtype=torch.float64)
    out = oracle.forward(value, shapes, None, loc, attn, mode="pinned_f32").reshape(B, Q, M, D)
    _close(out, c.expand(B, Q, M, D).numpy(), 1e-14)
    _, gl, _ = oracle.backward(value, shapes, None, loc, attn, gout, mode="pinned_f32")
    assert np.all(gl == 0)


def test_all_points_out_of_bounds_give_exact_zeros():
    value, shapes, _, loc, attn, gout = _rand_case(3)
    W = shapes[:, 1].double()
    # x_im >= W: both columns past the right edge, or <= -2: both before the left.
    loc[..., 0] = torch.where(torch.rand(loc.shape[:-1]) < 0.5, 1.0 + 1.0 / W.max() + 0.3, -1.5)
    for mode in ("pinned_f32", "exact_f64"):
        out, touched = oracle.forward(value, shapes, None, loc, attn, mode=mode, return_touched=True)
        assert np.all(out == 0) and not touched.any()
        gv, gl, ga, trows = oracle.backward(value, shapes, None, loc, attn, gout, mode=mode,
                                            return_touched=True)
        assert np.all(gv == 0) and np.all(gl == 0) and np.all(ga == 0) and not trows.any()


# ------------------------------------------------------------ invariants

@pytest.mark.parametrize("mode", ["pinned_f32", "exact_f64"])
def test_adjoint_identity(mode):
    value, shapes, st, loc, attn, gout = _rand_case(21, starts=(20, 0, 40))
    out = oracle.forward(value, shapes, st, loc, attn, mode=mode)
    gv, gl, ga = oracle.backward(value, shapes, st, loc, attn, gout, mode=mode)
    lhs = float((out * gout.numpy()).sum())
    assert abs(lhs - float((gv * value.numpy()).sum())) <= 1e-12 * abs(lhs)
    assert abs(lhs - float((ga * attn.numpy()).sum())) <= 1e-12 * abs(lhs)


def test_per_level_conservation_of_grad_value():
    levels = ((6, 9), (3, 5), (2, 2))
    B, Q, M, D, K = 2, 9, 3, 4, 3
    L = len(levels)
    g = torch.Generator().manual_seed(8)
    shapes = torch.tensor(levels)
    starts = _starts(shapes, None)
    S = sum(h * w for h, w in levels)
    value = torch.randn(B, S, M, D, generator=g, dtype=torch.float64)
    loc = _interior_locations(g, (B, Q, M, L, K, 2), levels)  # all weights sum to 1
    attn = torch.rand(B, Q, M, L, K, generator=g, dtype=torch.float64)
    gout = torch.randn(B, Q, M, D, generator=g, dtype=torch.float64)
    gv, _, _ = oracle.backward(value, shapes, None, loc, attn, gout.reshape(B, Q, M * D))
    for l_, (H, W) in enumerate(levels):
        got = gv[:, starts[l_]:starts[l_] + H * W].sum(1)  # (B, M, D)
        want = (attn[:, :, :, l_].sum(-1)[..., None] * gout).sum(1)  # (B, M, D)
        _close(got, want.numpy(), 1e-12)


def test_no_wraparound_across_rows_or_levels():
    """Samples on the left edge (x0 = -1) and the bottom edge (y1 = H) of a
    level must not read the previous row's last pixel or the next level."""
    levels = ((3, 4), (2, 3))
    shapes = torch.tensor(levels)
    starts = _starts(shapes, None)
    S = sum(h * w for h, w in levels)
    B, M, D, K, L = 1, 1, 2, 2, 2
    value = torch.ones(B, S, M, D, dtype=torch.float64)
    H0, W0 = levels[0]
    for y in range(H0):
        value[0, starts[0] + y * W0 + (W0 - 1)] = 1e30  # last column of level 0
    value[0, starts[1]:] = 1e30  # all of level 1
    Q = 8
    g = torch.Generator().manual_seed(9)
    loc = torch.full((B, Q, M, L, K, 2), 5.0, dtype=torch.float64)  # level 1 unused: OOB
    u = torch.rand(B, Q, M, K, generator=g, dtype=torch.float64)
    # Left edge: x_im in (-1, 0) -> x0 = -1; rows 1..H0-1 so that row y0 has a row above.
    loc[:, :4, :, 0, :, 0] = (u[:, :4] * 0.9 + 0.05 - 0.5 + 0.5) / W0 * 0.999
    loc[:, :4, :, 0, :, 1] = (1.0 + u[:, :4] * 0.9 + 0.5) / H0
    # Bottom edge: y_im in (H0-1, H0) -> y1 = H0, just past the last row of level 0.
    loc[:, 4:, :, 0, :, 0] = (u[:, 4:] * (W0 - 2) + 0.5) / W0
    loc[:, 4:, :, 0, :, 1] = (H0 - 1 + 0.05 + u[:, 4:] * 0.9 + 0.5) / H0
    attn = torch.ones(B, Q, M, L, K, dtype=torch.float64)
    for mode in ("pinned_f32", "exact_f64"):
        out = oracle.forward(value, shapes, None, loc, attn, mode=mode)
        assert np.all(np.abs(out) < 10), np.abs(out).max()


def test_thread_count_does_not_change_results():
    inp = make_inputs(workload("tiny_fp32").replace(B=2, Q=40))
    args = (inp["value"], inp["spatial_shapes"], None, inp["sampling_locations"],
            inp["attention_weights"])
    o1 = oracle.forward(*args, num_threads=1)
    o8 = oracle.forward(*args, num_threads=8)
    np.testing.assert_array_equal(o1, o8)
    b1 = oracle.backward(*args, inp["grad_output"], num_threads=1)
    b8 = oracle.backward(*args, inp["grad_output"], num_threads=8)
    for x, y in zip(b1, b8):
        np.testing.assert_array_equal(x, y)


def test_linearity_in_value():
    value, shapes, _, loc, attn, _ = _rand_case(31)
    v2 = torch.randn(value.shape, generator=torch.Generator().manual_seed(32), dtype=torch.float64)
    o1 = oracle.forward(value, shapes, None, loc, attn)
    o2 = oracle.forward(v2, shapes, None, loc, attn)
    o12 = oracle.forward(2.0 * value - 3.0 * v2, shapes, None, loc, attn)
    _close(o12, 2.0 * o1 - 3.0 * o2, 1e-13)


def test_pinned_mapping_uses_one_rounding():
    """The pinned mode maps x_im = fma(loc_x, W, -0.5) rounded once to fp32.
    Find fp32 locations where rounding loc*W first would land on the other
    side of an integer, and check which corner the oracle picks."""
    # Search widths W and target integers n for fp32 locations a few ulps from
    # (n + 0.5) / W; exact products of a 24-bit loc and a small W fit in fp64.
    found = []
    for W in range(3, 400):
        n = np.arange(1, W, dtype=np.float64)
        base = ((n + 0.5) / W).astype(np.float32)
        for step in range(-6, 7):
            loc32 = base.copy()
            for _ in range(abs(step)):
                loc32 = np.nextafter(loc32, np.float32(np.sign(step) * np.inf))
            exact = loc32.astype(np.float64) * W - 0.5
            fma32 = exact.astype(np.float32)  # one rounding
            two32 = (loc32 * np.float32(W)).astype(np.float32) - np.float32(0.5)
            for i in np.nonzero(np.floor(fma32) != np.floor(two32))[0]:
                found.append((W, loc32[i], fma32[i]))
        if len(found) >= 8:
            break
    assert found, "no distinguishing location found"
    for W, l32, f32 in found[:8]:
        x0 = int(np.floor(f32))
        # one level 1 x W, one point; the touched columns tell which cell was used
        value = np.arange(1, W + 1, dtype=np.float64).reshape(1, W, 1, 1)
        loc = np.array([l32, 0.5], np.float64).reshape(1, 1, 1, 1, 1, 2)
        attn = np.ones((1, 1, 1, 1, 1))
        g = np.ones((1, 1, 1))
        _, _, _, touched = oracle.backward(value, np.array([[1, W]]), None, loc, attn, g,
                                           mode="pinned_f32", return_touched=True)
        cols = set(np.nonzero(touched[0, :, 0])[0].tolist())
        assert cols == {c for c in (x0, x0 + 1) if 0 <= c < W}, (W, l32, x0, cols)


def test_bad_levels_are_rejected():
    value, shapes, _, loc, attn, gout = _rand_case(1)
    with pytest.raises(ValueError):
        oracle.forward(value, shapes, torch.tensor([0, 35, 60]), loc, attn)
    bad = shapes.clone()
    bad[0, 0] = 0
    with pytest.raises(ValueError):
        oracle.forward(value, bad, None, loc, attn)
    loc2 = loc.clone()
    loc2[0, 0, 0, 0, 0, 0] = float("nan")
    with pytest.raises(ValueError):
        oracle.forward(value, shapes, None, loc2, attn)


# ------------------------------------------- grad_value rounding statistics
#
# oracle.scatter_stats gives, per grad_value element, the sum of the absolute
# values of its terms A * w_ij * g[d] and, per row, their number; the GPU
# parity rule for sums made with 16-bit atomics is built on them (backward
# course page, section "Atomics make gradients nondeterministic").

def test_scatter_stats_golden():
    d = json.load(open(os.path.join(GOLDEN, "rounding", "scatter_rounding_stats.json")))
    shapes = np.array(d["spatial_shapes"], np.int64)
    loc = np.array(d["sampling_locations"], np.float64)
    attn = np.array(d["attention_weights"], np.float64)
    g = np.array(d["grad_output"], np.float64)
    S, D = d["num_keys"], d["head_dim"]
    ex = d["expected"]
    for mode in ("pinned_f32", "exact_f64"):
        abs_sum, count = oracle.scatter_stats(shapes, None, loc, attn, g, S, D, mode=mode)
        np.testing.assert_array_equal(abs_sum, np.array(ex["abs_sum"]))
        np.testing.assert_array_equal(count, np.array(ex["count"]))
        value = np.zeros((1, S, 1, D))
        gv = oracle.backward(value, shapes, None, loc, attn, g, mode=mode)[0]
        np.testing.assert_array_equal(gv, np.array(ex["grad_value"]))


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_scatter_stats_equal_signed_sum_when_terms_share_a_sign(sign):
    """With non-negative weights A and an upstream gradient of one sign, every
    term A * w_ij * g[d] has that sign, so the sum of absolute values equals
    the absolute value of the sum: abs_sum == |grad_value| exactly (the same
    terms added in the same order)."""
    value, shapes, st, loc, attn, gout = _rand_case(21, starts=(30, 0, 13))
    gpos = sign * gout.abs()
    gv = oracle.backward(value, shapes, st, loc, attn, gpos)[0]
    abs_sum, count = oracle.scatter_stats(shapes, st, loc, attn, gpos, value.shape[1],
                                          value.shape[3])
    np.testing.assert_array_equal(abs_sum, np.abs(gv))
    assert (count > 0).sum() > 0


def test_scatter_stats_bound_the_signed_sum_and_count_corners():
    """Mixed signs: |grad_value| <= abs_sum elementwise (triangle inequality),
    equality on rows that receive one term; the upstream gradient's sign does
    not change abs_sum; doubling it doubles abs_sum exactly; count > 0
    exactly on the rows the backward reports as touched, and the counts add
    up to the in-bounds corners counted point by point in numpy."""
    value, shapes, st, loc, attn, gout = _rand_case(22, Q=11, starts=(30, 0, 13))
    attn = attn - 0.5  # weights of both signs
    S, D = value.shape[1], value.shape[3]
    gv, _, _, touched = oracle.backward(value, shapes, st, loc, attn, gout, return_touched=True)
    abs_sum, count = oracle.scatter_stats(shapes, st, loc, attn, gout, S, D)
    assert np.all(np.abs(gv) <= abs_sum * (1 + 1e-15))
    one = count == 1
    np.testing.assert_allclose(np.abs(gv)[one], abs_sum[one], rtol=1e-15, atol=0)
    assert np.all(abs_sum[count >= 2] >= np.abs(gv)[count >= 2])
    assert (np.abs(gv)[count >= 2] < abs_sum[count >= 2] * (1 - 1e-12)).any()
    np.testing.assert_array_equal(oracle.scatter_stats(shapes, st, loc, attn, -gout, S, D)[0],
                                  abs_sum)
    np.testing.assert_array_equal(oracle.scatter_stats(shapes, st, loc, attn, 2 * gout, S, D)[0],
                                  2 * abs_sum)
    np.testing.assert_array_equal(count > 0, touched)
    # in-bounds corners point by point (single-rounding fp32 mapping)
    corners = 0
    for l, (H, W) in enumerate(shapes.tolist()):
        lx = loc[:, :, :, l, :, 0].numpy().astype(np.float32)
        ly = loc[:, :, :, l, :, 1].numpy().astype(np.float32)
        x0 = np.floor((lx.astype(np.float64) * W - 0.5).astype(np.float32)).astype(np.int64)
        y0 = np.floor((ly.astype(np.float64) * H - 0.5).astype(np.float32)).astype(np.int64)
        for dy in (0, 1):
            for dx in (0, 1):
                corners += int((((x0 + dx) >= 0) & ((x0 + dx) < W) &
                                ((y0 + dy) >= 0) & ((y0 + dy) < H)).sum())
    assert int(count.sum()) == corners
