"""CPU oracle for the steps around the MSDA core: the sampling-parameter
preparation (reference scaling and the softmax over levels x points) and the
whole deformable-attention module (projections around the core).

TEST INFRASTRUCTURE ONLY. Only `tests/`, `__graft_entry__.smoke()` and the
CPU-baseline leg of `bench.py` may import this module. The product path never
calls it and shares no code with it. Plain numpy in fp64, loops over levels in
the order of the definition; the core itself is the C oracle of this package.

Sources (web pages):
  [README] msda-triton README, section "The operator": the module is
      out(q) = sum_m W_m [ sum_l sum_k A_mlqk * x_l(phi_l(p_q) + dp_mlqk) ],
      the bracketed core computed by the C oracle, with learned offsets dp,
      softmax-normalised weights A, and the linear projections around the
      core being ordinary matrix products.
  [README] section "Quickstart": the weights are a softmax over the flattened
      L*K axis of each (b, q, m), attention_weights.flatten(3).softmax(-1).

Readings taken where the pages leave a step open:
  - reference points p_q are normalised to [0, 1]^2 as (x, y), like the
    sampling locations the core takes; shape (B, Q, 2), or (B, Q, L, 2) for
    one point per level;
  - phi_l maps p_q to level l; in normalised coordinates that map is the
    identity, and the offsets dp are in pixels of level l, so the normalised
    sampling location is p_q + (dp_x / W_l, dp_y / H_l);
  - the value fed to the core is a linear projection of the flattened
    multi-level input, split into M heads of D channels (W'_m of the original
    formulation; the pages' x_l is that projected map); W_m is one linear
    output projection over the concatenated heads;
  - every linear map is y = x @ weight.T + bias (PyTorch's convention).
"""

from __future__ import annotations

import numpy as np

from . import backward as core_backward
from . import forward as core_forward


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _shapes(spatial_shapes) -> list:
    s = spatial_shapes
    if hasattr(s, "detach"):
        s = s.detach().cpu().numpy()
    return [(int(h), int(w)) for h, w in np.asarray(s, dtype=np.int64).reshape(-1, 2)]


def _ref_at_level(ref: np.ndarray, l: int) -> np.ndarray:
    """(B, Q, 2) reference points used at level l."""
    return ref if ref.ndim == 3 else ref[:, :, l, :]


def softmax_lk(logits: np.ndarray) -> np.ndarray:
    """Softmax over the last axis (the flattened L*K points of one (b, q, m)).
    Shifting by the row maximum changes nothing mathematically and keeps
    exp() finite."""
    z = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def sampling_prep(reference_points, sampling_offsets, attention_logits, spatial_shapes):
    """(sampling_locations (B,Q,M,L,K,2), attention_weights (B,Q,M,L,K)) in fp64.

    reference_points (B,Q,2) or (B,Q,L,2); sampling_offsets (B,Q,M,L,K,2) in
    pixels of each level; attention_logits (B,Q,M,L*K) or (B,Q,M,L,K)."""
    ref, off = _f64(reference_points), _f64(sampling_offsets)
    shapes = _shapes(spatial_shapes)
    B, Q, M, L, K, _ = off.shape
    logits = _f64(attention_logits).reshape(B, Q, M, L * K)
    loc = np.empty_like(off)
    for l, (H, W) in enumerate(shapes):
        r = _ref_at_level(ref, l)
        loc[:, :, :, l, :, 0] = r[:, :, None, None, 0] + off[:, :, :, l, :, 0] / W
        loc[:, :, :, l, :, 1] = r[:, :, None, None, 1] + off[:, :, :, l, :, 1] / H
    attn = softmax_lk(logits).reshape(B, Q, M, L, K)
    return loc, attn


def sampling_prep_backward(attention_weights, grad_sampling_locations, grad_attention_weights,
                           spatial_shapes, ref_per_level: bool = False):
    """(grad_reference_points, grad_sampling_offsets, grad_attention_logits).

    Chain rule through sampling_prep: d loc_x / d dp_x = 1 / W_l,
    d loc_y / d dp_y = 1 / H_l, d loc / d p_q = 1 (summed over every m, k and,
    for one point per query, every l); the softmax Jacobian gives
    g_logit_j = A_j * (g_j - sum_i A_i g_i) over the L*K points."""
    a, gl, ga = (_f64(t) for t in (attention_weights, grad_sampling_locations,
                                   grad_attention_weights))
    shapes = _shapes(spatial_shapes)
    B, Q, M, L, K, _ = gl.shape
    g_off = np.empty_like(gl)
    for l, (H, W) in enumerate(shapes):
        g_off[:, :, :, l, :, 0] = gl[:, :, :, l, :, 0] / W
        g_off[:, :, :, l, :, 1] = gl[:, :, :, l, :, 1] / H
    per_level = gl.sum(axis=(2, 4))  # (B, Q, L, 2)
    g_ref = per_level if ref_per_level else per_level.sum(axis=2)
    af = a.reshape(B, Q, M, L * K)
    gf = ga.reshape(B, Q, M, L * K)
    inner = (af * gf).sum(axis=-1, keepdims=True)
    g_logits = af * (gf - inner)
    return g_ref, g_off, g_logits


# ------------------------------------------------------------------ module

def _linear(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    return x @ w.T + b


def module_forward(params: dict, query, reference_points, input_flatten, spatial_shapes,
                   level_start_index=None, heads: int = 8, points: int = 4,
                   return_intermediates: bool = False, mode: str = "pinned_f32"):
    """The deformable-attention module in fp64.

    params: value_proj.{weight,bias}, sampling_offsets.{weight,bias},
    attention_weights.{weight,bias}, output_proj.{weight,bias} (PyTorch
    Linear layouts). query (B,Q,C), input_flatten (B,S,C). Returns (B,Q,C).
    `mode` is the core oracle's pixel-mapping mode."""
    p = {k: _f64(v) for k, v in params.items()}
    x, inp, ref = _f64(query), _f64(input_flatten), _f64(reference_points)
    shapes = _shapes(spatial_shapes)
    B, Q, _ = x.shape
    S = inp.shape[1]
    L, M, K = len(shapes), heads, points
    value = _linear(inp, p["value_proj.weight"], p["value_proj.bias"])
    D = value.shape[-1] // M
    value = value.reshape(B, S, M, D)
    off = _linear(x, p["sampling_offsets.weight"], p["sampling_offsets.bias"])
    off = off.reshape(B, Q, M, L, K, 2)
    logits = _linear(x, p["attention_weights.weight"], p["attention_weights.bias"])
    logits = logits.reshape(B, Q, M, L * K)
    loc, attn = sampling_prep(ref, off, logits, shapes)
    core = core_forward(value, np.asarray(shapes, dtype=np.int64), level_start_index, loc, attn,
                        mode=mode)
    out = _linear(core, p["output_proj.weight"], p["output_proj.bias"])
    if return_intermediates:
        return out, {"value": value, "loc": loc, "attn": attn, "core": core}
    return out


def module_backward(params: dict, query, reference_points, input_flatten, spatial_shapes,
                    grad_output, level_start_index=None, heads: int = 8, points: int = 4,
                    mode: str = "pinned_f32"):
    """Gradients of sum(out * grad_output) in fp64: a dict with 'query',
    'reference_points', 'input_flatten' and every parameter name."""
    p = {k: _f64(v) for k, v in params.items()}
    x, inp, ref = _f64(query), _f64(input_flatten), _f64(reference_points)
    g = _f64(grad_output)
    shapes = _shapes(spatial_shapes)
    _, it = module_forward(p, x, ref, inp, shapes, level_start_index, heads, points,
                           return_intermediates=True, mode=mode)
    B, Q, C = x.shape
    S = inp.shape[1]
    value, loc, attn, core = it["value"], it["loc"], it["attn"], it["core"]
    grads = {}
    # out = core @ Wo.T + bo
    g2 = g.reshape(-1, g.shape[-1])
    grads["output_proj.weight"] = g2.T @ core.reshape(-1, core.shape[-1])
    grads["output_proj.bias"] = g2.sum(axis=0)
    g_core = g @ p["output_proj.weight"]
    # the core
    gv, gl, ga = core_backward(value, np.asarray(shapes, dtype=np.int64), level_start_index,
                               loc, attn, g_core, mode=mode)
    # sampling preparation
    g_ref, g_off, g_logits = sampling_prep_backward(attn, gl, ga, shapes,
                                                    ref_per_level=ref.ndim == 4)
    grads["reference_points"] = g_ref
    g_off2 = g_off.reshape(B * Q, -1)
    g_log2 = g_logits.reshape(B * Q, -1)
    x2 = x.reshape(B * Q, C)
    grads["sampling_offsets.weight"] = g_off2.T @ x2
    grads["sampling_offsets.bias"] = g_off2.sum(axis=0)
    grads["attention_weights.weight"] = g_log2.T @ x2
    grads["attention_weights.bias"] = g_log2.sum(axis=0)
    grads["query"] = (g_off2 @ p["sampling_offsets.weight"] +
                      g_log2 @ p["attention_weights.weight"]).reshape(B, Q, C)
    # value = input_flatten @ Wv.T + bv
    gv2 = gv.reshape(B * S, -1)
    grads["value_proj.weight"] = gv2.T @ inp.reshape(B * S, -1)
    grads["value_proj.bias"] = gv2.sum(axis=0)
    grads["input_flatten"] = (gv2 @ p["value_proj.weight"]).reshape(B, S, -1)
    return grads
