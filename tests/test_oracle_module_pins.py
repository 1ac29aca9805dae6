"""Pins for the oracle of the steps around the core (oracle/module.py).

Each check fixes the oracle to what the pages or mathematics determine, not to
itself: closed forms of the softmax (uniform weights, the two-point logistic
form, shift invariance), exact reference scaling (a one-pixel offset moves a
location by exactly 1/W_l or 1/H_l; a reference point on a pixel centre plus
an integer offset reproduces that pixel through the core), a whole module with
identity projections and per-head integer offsets reproducing shifted pixels,
and central finite differences of every gradient.

Sources: msda-triton README, section "The operator" (the module equation with
reference points, offsets, softmax-normalised weights and the projections
around the core) and section "Quickstart" (softmax over the flattened L*K
axis).

The checks take the module under test as an argument so that
tests/test_oracle_mutations.py can run them against copies with planted
mistakes.
"""

import numpy as np
import pytest

import oracle
from oracle import module as oracle_module

LEVELS = ((4, 5), (2, 3))


def _close(a, b, rtol, atol=0.0):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    err = np.abs(a - b)
    bound = rtol * (np.abs(b) + np.sqrt(np.mean(b * b))) + atol
    assert (err <= bound).all(), f"max abs err {err.max():.3e}"


def _params(rng, C, M, D, L, K, scale=0.3):
    def lin(n_out, n_in):
        return rng.standard_normal((n_out, n_in)) * scale, rng.standard_normal(n_out) * scale
    p = {}
    for name, (n_out, n_in) in {"value_proj": (M * D, C), "sampling_offsets": (M * L * K * 2, C),
                                "attention_weights": (M * L * K, C),
                                "output_proj": (C, M * D)}.items():
        p[name + ".weight"], p[name + ".bias"] = lin(n_out, n_in)
    return p


# ----------------------------------------------------------------- checks

def check_softmax_closed_forms(om):
    rng = np.random.default_rng(1)
    z = rng.standard_normal((2, 3, 2, 8))
    a = om.sampling_prep(np.zeros((2, 3, 2)), np.zeros((2, 3, 2, 2, 4, 2)), z, ((3, 3), (2, 2)))[1]
    a = a.reshape(2, 3, 2, 8)
    _close(a.sum(-1), np.ones((2, 3, 2)), 1e-14)
    # shift invariance per (b, q, m)
    a2 = om.sampling_prep(np.zeros((2, 3, 2)), np.zeros((2, 3, 2, 2, 4, 2)),
                          z + rng.standard_normal((2, 3, 2, 1)) * 5, ((3, 3), (2, 2)))[1]
    _close(a2.reshape(a.shape), a, 1e-12)
    # equal logits: uniform over all L*K points (not per level)
    u = om.sampling_prep(np.zeros((1, 1, 2)), np.zeros((1, 1, 1, 2, 4, 2)),
                         np.full((1, 1, 1, 8), 0.7), ((3, 3), (2, 2)))[1]
    _close(u, np.full(u.shape, 1.0 / 8), 1e-15)
    # two points: the logistic function of the logit difference, in the
    # flattened order (level-major, then point)
    z2 = np.array([0.3, -1.1]).reshape(1, 1, 1, 2)
    a2 = om.sampling_prep(np.zeros((1, 1, 2)), np.zeros((1, 1, 1, 2, 1, 2)), z2,
                          ((3, 3), (2, 2)))[1].reshape(2)
    _close(a2, [1 / (1 + np.exp(-1.4)), 1 / (1 + np.exp(1.4))], 1e-15)


def check_reference_scaling_exact(om):
    shapes = ((4, 6), (3, 5))
    rng = np.random.default_rng(2)
    ref = rng.random((2, 3, 2))
    zero = np.zeros((2, 3, 2, 2, 3, 2))
    loc = om.sampling_prep(ref, zero, np.zeros((2, 3, 2, 6)), shapes)[0]
    for l in range(2):
        for c in range(2):
            assert np.array_equal(loc[:, :, :, l, :, c],
                                  np.broadcast_to(ref[:, :, None, None, c], loc.shape[:3] + (3,)))
    # one pixel along x moves by 1/W_l, along y by 1/H_l (exact in fp64)
    one_x = zero.copy()
    one_x[..., 0] = 1.0
    one_y = zero.copy()
    one_y[..., 1] = 1.0
    lx = om.sampling_prep(ref, one_x, np.zeros((2, 3, 2, 6)), shapes)[0]
    ly = om.sampling_prep(ref, one_y, np.zeros((2, 3, 2, 6)), shapes)[0]
    for l, (H, W) in enumerate(shapes):
        _close(lx[:, :, :, l, :, 0] - loc[:, :, :, l, :, 0], np.full(lx.shape[:3] + (3,), 1 / W),
               1e-12)
        _close(ly[:, :, :, l, :, 1] - loc[:, :, :, l, :, 1], np.full(ly.shape[:3] + (3,), 1 / H),
               1e-12)
        assert np.array_equal(lx[:, :, :, l, :, 1], loc[:, :, :, l, :, 1])
        assert np.array_equal(ly[:, :, :, l, :, 0], loc[:, :, :, l, :, 0])
    # per-level reference points: level l uses its own point
    ref4 = rng.random((2, 3, 2, 2))
    loc4 = om.sampling_prep(ref4, zero, np.zeros((2, 3, 2, 6)), shapes)[0]
    for l in range(2):
        assert np.array_equal(loc4[:, :, 0, l, 0, :], ref4[:, :, l, :])


def check_pixel_centre_plus_integer_offset(om):
    """A reference on the centre of pixel (i, j) of level l plus an integer
    offset (dj, di) samples exactly pixel (i+di, j+dj) of that level (power-
    of-two level sizes keep every coordinate exact in fp32)."""
    shapes = np.array([(4, 8), (2, 4)])
    rng = np.random.default_rng(3)
    M, D, K = 2, 3, 1
    S = int((shapes[:, 0] * shapes[:, 1]).sum())
    value = rng.standard_normal((1, S, M, D))
    starts = [0, 32]
    cases = [(0, 1, 2, 3, -1), (0, 3, 7, -2, 0), (1, 1, 3, -3, -1), (1, 0, 0, 2, 1)]
    for l, i, j, dj, di in cases:
        H, W = shapes[l]
        ref = np.array([[[(j + 0.5) / W, (i + 0.5) / H]]])
        off = np.zeros((1, 1, M, 2, K, 2))
        off[0, 0, :, l, 0] = (dj, di)
        logits = np.full((1, 1, M, 2 * K), -np.inf)
        logits[0, 0, :, l * K] = 0.0  # all weight on level l
        loc, attn = om.sampling_prep(ref, off, np.where(np.isinf(logits), -1e300, logits), shapes)
        out = oracle.forward(value, shapes, None, loc, attn).reshape(M, D)
        row = starts[l] + (i + di) * W + (j + dj)
        assert np.array_equal(out, value[0, row]), (l, i, j, dj, di)


def check_identity_module_closed_form(om):
    """Identity projections, zero query weights, per-head integer offsets in
    the offset bias and equal logits: head m of the output is the mean over
    levels of the input pixel at (i, j + m) of each level, per-level reference
    points on pixel centres (power-of-two level sizes: exact in fp32)."""
    shapes = np.array([(4, 8), (2, 4)])
    M, D, K, L = 2, 3, 2, 2
    C = M * D
    rng = np.random.default_rng(4)
    S = int((shapes[:, 0] * shapes[:, 1]).sum())
    inp = rng.standard_normal((1, S, C))
    p = {"value_proj.weight": np.eye(C), "value_proj.bias": np.zeros(C),
         "output_proj.weight": np.eye(C), "output_proj.bias": np.zeros(C),
         "sampling_offsets.weight": np.zeros((M * L * K * 2, C)),
         "attention_weights.weight": np.zeros((M * L * K, C)),
         "attention_weights.bias": np.zeros(M * L * K)}
    bias = np.zeros((M, L, K, 2))
    for m in range(M):
        bias[m, :, :, 0] = m  # head m looks m pixels to the right
    p["sampling_offsets.bias"] = bias.reshape(-1)
    i, j = 1, 2
    ref = np.zeros((1, 1, L, 2))
    for l, (H, W) in enumerate(shapes):
        ref[0, 0, l] = ((j + 0.5) / W, (i + 0.5) / H)
    query = rng.standard_normal((1, 1, C))
    out = om.module_forward(p, query, ref, inp, shapes, heads=M, points=K).reshape(M, D)
    starts = [0, 32]
    want = np.zeros((M, D))
    for m in range(M):
        for l, (H, W) in enumerate(shapes):
            want[m] += inp[0, starts[l] + i * W + j + m, m * D:(m + 1) * D] / L
    _close(out, want, 1e-14)


def _module_case(seed):
    rng = np.random.default_rng(seed)
    B, Q, C, M, D, K = 1, 3, 4, 2, 2, 2
    shapes = np.array(LEVELS)
    L = len(LEVELS)
    S = int((shapes[:, 0] * shapes[:, 1]).sum())
    p = _params(rng, C, M, D, L, K)
    x = rng.standard_normal((B, Q, C))
    ref = 0.2 + 0.6 * rng.random((B, Q, 2))
    inp = rng.standard_normal((B, S, C))
    g = rng.standard_normal((B, Q, C))
    return p, x, ref, inp, shapes, g, M, K


def _module_loss(om, p, x, ref, inp, shapes, g, M, K):
    out = om.module_forward(p, x, ref, inp, shapes, heads=M, points=K, mode="exact_f64")
    return float((out * g).sum())


def _min_kink_margin(om, p, x, ref, inp, shapes, M, K):
    _, it = om.module_forward(p, x, ref, inp, shapes, heads=M, points=K, mode="exact_f64",
                              return_intermediates=True)
    loc = it["loc"]
    m = np.inf
    for l, (H, W) in enumerate(shapes):
        for c, size in ((0, W), (1, H)):
            pix = loc[:, :, :, l, :, c] * size - 0.5
            m = min(m, float(np.min(np.abs(pix - np.round(pix)))))
    return m


def check_module_finite_differences(om):
    p, x, ref, inp, shapes, g, M, K = _module_case(11)
    assert _min_kink_margin(om, p, x, ref, inp, shapes, M, K) > 1e-3
    grads = om.module_backward(p, x, ref, inp, shapes, g, heads=M, points=K, mode="exact_f64")
    h = 1e-6
    rng = np.random.default_rng(12)

    def fd(get, set_):
        base = get().copy()
        n = base.size
        for idx in rng.choice(n, size=min(n, 6), replace=False):
            plus, minus = base.copy().ravel(), base.copy().ravel()
            plus[idx] += h
            minus[idx] -= h
            set_(plus.reshape(base.shape))
            lp = _module_loss(om, p, x, ref, inp, shapes, g, M, K)
            set_(minus.reshape(base.shape))
            lm = _module_loss(om, p, x, ref, inp, shapes, g, M, K)
            set_(base)
            yield idx, (lp - lm) / (2 * h)

    holders = {"query": x, "reference_points": ref, "input_flatten": inp}
    for name in list(p) + list(holders):
        def get(name=name):
            return p[name] if name in p else holders[name]

        def set_(v, name=name):
            if name in p:
                p[name] = v
            else:
                holders[name][...] = v
        want = grads[name].ravel()
        for idx, val in fd(get, set_):
            assert abs(val - want[idx]) <= 1e-6 * (abs(want[idx]) + 1.0), (name, idx, val,
                                                                          want[idx])


def check_prep_backward_finite_differences(om):
    rng = np.random.default_rng(13)
    shapes = ((4, 6), (3, 5))
    B, Q, M, L, K = 2, 2, 2, 2, 3
    for ref_levels in (False, True):
        ref = rng.random((B, Q, L, 2) if ref_levels else (B, Q, 2))
        off = rng.standard_normal((B, Q, M, L, K, 2))
        z = rng.standard_normal((B, Q, M, L * K))
        wl = rng.standard_normal((B, Q, M, L, K, 2))
        wa = rng.standard_normal((B, Q, M, L, K))

        def loss(ref, off, z):
            loc, a = om.sampling_prep(ref, off, z, shapes)
            return float((loc * wl).sum() + (a * wa).sum())
        a = om.sampling_prep(ref, off, z, shapes)[1]
        g_ref, g_off, g_z = om.sampling_prep_backward(a, wl, wa, shapes, ref_per_level=ref_levels)
        h = 1e-6
        for arr, grad in ((ref, g_ref), (off, g_off), (z, g_z)):
            assert grad.shape == arr.shape
            flat = arr.reshape(-1)
            for idx in range(flat.size):
                keep = flat[idx]
                flat[idx] = keep + h
                lp = loss(ref, off, z)
                flat[idx] = keep - h
                lm = loss(ref, off, z)
                flat[idx] = keep
                fdv = (lp - lm) / (2 * h)
                assert abs(fdv - grad.reshape(-1)[idx]) <= 1e-7 * (abs(fdv) + 1.0)


CHECKS = [check_softmax_closed_forms, check_reference_scaling_exact,
          check_pixel_centre_plus_integer_offset, check_identity_module_closed_form,
          check_module_finite_differences, check_prep_backward_finite_differences]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_module_oracle_pin(check):
    check(oracle_module)
