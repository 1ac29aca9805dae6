"""The deformable-attention module around the MSDA core.

msda-triton README, section "The operator": for query features z_q with
reference points p_q,

    MSDA(q) = sum_m W_m [ sum_l sum_k A_mlqk * x_l(phi_l(p_q) + dp_mlqk) ]

with learned offsets dp and softmax-normalised weights A; the linear
projections around the bracketed core are ordinary matrix products. Here:

    value     = value_proj(input_flatten)            -> (B, S, M, D)
    offsets   = sampling_offsets(query)              -> (B, Q, M, L, K, 2), pixels of level l
    logits    = attention_weights(query)             -> (B, Q, M, L*K)
    locations = p_q + offsets / (W_l, H_l),  A = softmax over L*K   (HIP: msda_sampling_prep)
    core      = MSDA core(value, locations, A)       -> (B, Q, M*D)   (HIP: msda_forward/backward)
    output    = output_proj(core)                    -> (B, Q, d_model)

Reference points are normalised (x, y) in [0, 1], one per query (B, Q, 2) or
one per query and level (B, Q, L, 2). The projections are torch.nn.Linear
layers (library GEMMs); the sampling-parameter preparation and the core run in
the HIP library, forward and backward. `param_dtype=torch.float32` computes
the offset and weight projections, the locations and the weights in fp32
beside 16-bit values (the library's mixed-dtype entry points): a 16-bit
offset carries about 2^-9 of its own size in error, a few hundredths of a
pixel for offsets of several pixels, which the bilinear sample passes on in
full.
"""

from __future__ import annotations

from typing import Optional

import torch
from torch import nn
from torch.nn import functional as F
from torch.autograd.function import once_differentiable

from . import _binding
from .autograd import multi_scale_deformable_attention


class SamplingPrepFunction(torch.autograd.Function):
    """(reference_points, sampling_offsets, attention_logits) ->
    (sampling_locations, attention_weights) through msda_sampling_prep."""

    @staticmethod
    def forward(ctx, reference_points, sampling_offsets, attention_logits, spatial_shapes):
        loc, attn = _binding.msda_sampling_prep(reference_points, sampling_offsets,
                                                attention_logits, spatial_shapes)
        ctx.save_for_backward(attn)
        ctx.shapes = spatial_shapes
        ctx.ref_per_level = reference_points.dim() == 4
        ctx.logits_shape = attention_logits.shape
        return loc, attn

    @staticmethod
    @once_differentiable
    def backward(ctx, grad_loc, grad_attn):
        (attn,) = ctx.saved_tensors
        if grad_loc is None:
            B, Q, M, L, K = attn.shape
            grad_loc = attn.new_zeros((B, Q, M, L, K, 2))
        if grad_attn is None:
            grad_attn = torch.zeros_like(attn)
        g_ref, g_off, g_logits = _binding.msda_sampling_prep_backward(
            attn, grad_loc, grad_attn, ctx.shapes, ref_per_level=ctx.ref_per_level,
            need_reference_grad=ctx.needs_input_grad[0])
        return g_ref, g_off, g_logits.view(ctx.logits_shape), None


def sampling_prep(reference_points: torch.Tensor, sampling_offsets: torch.Tensor,
                  attention_logits: torch.Tensor, spatial_shapes):
    """Differentiable msda_sampling_prep; spatial_shapes is read on the host."""
    return SamplingPrepFunction.apply(reference_points, sampling_offsets, attention_logits,
                                      spatial_shapes)


class MSDeformAttn(nn.Module):
    """Multi-scale deformable attention (see the module docstring).

    d_model: query / input feature size C; n_heads M; n_levels L; n_points K;
    head_dim D (default d_model // n_heads). fp32_grad_accum: the core's
    grad_value accumulation switch (None, True, False or a mode name)."""

    def __init__(self, d_model: int = 256, n_levels: int = 4, n_heads: int = 8,
                 n_points: int = 4, head_dim: Optional[int] = None, fp32_grad_accum=None,
                 param_dtype: Optional[torch.dtype] = None, device=None, dtype=None):
        super().__init__()
        if head_dim is None:
            if d_model % n_heads:
                raise ValueError(f"d_model {d_model} is not divisible by n_heads {n_heads}")
            head_dim = d_model // n_heads
        self.d_model, self.n_levels, self.n_heads, self.n_points = d_model, n_levels, n_heads, n_points
        self.head_dim = head_dim
        self.fp32_grad_accum = fp32_grad_accum
        self.param_dtype = param_dtype
        kw = {"device": device, "dtype": dtype}
        self.value_proj = nn.Linear(d_model, n_heads * head_dim, **kw)
        self.sampling_offsets = nn.Linear(d_model, n_heads * n_levels * n_points * 2, **kw)
        self.attention_weights = nn.Linear(d_model, n_heads * n_levels * n_points, **kw)
        self.output_proj = nn.Linear(n_heads * head_dim, d_model, **kw)

    def forward(self, query: torch.Tensor, reference_points: torch.Tensor,
                input_flatten: torch.Tensor, spatial_shapes, level_start_index=None,
                input_padding_mask: Optional[torch.Tensor] = None) -> torch.Tensor:
        """query (B, Q, C), reference_points (B, Q, 2) or (B, Q, L, 2),
        input_flatten (B, S, C), spatial_shapes (L, 2) rows (H_l, W_l);
        input_padding_mask (B, S) bool, True where the input is padding (its
        value rows are zeroed). Returns (B, Q, C)."""
        B, Q, _ = query.shape
        S = input_flatten.shape[1]
        M, L, K, D = self.n_heads, self.n_levels, self.n_points, self.head_dim
        shapes = torch.as_tensor(spatial_shapes).detach().to("cpu", torch.int64)  # one host copy
        if shapes.shape != (L, 2):
            raise ValueError(f"spatial_shapes must be ({L}, 2), got {tuple(shapes.shape)}")
        starts = None if level_start_index is None else \
            torch.as_tensor(level_start_index).detach().to("cpu", torch.int64)
        value = self.value_proj(input_flatten)
        if input_padding_mask is not None:
            value = value.masked_fill(input_padding_mask[..., None], 0.0)
        value = value.view(B, S, M, D)
        pd = self.param_dtype
        if pd is not None and pd != query.dtype:
            q = query.to(pd)
            off = F.linear(q, self.sampling_offsets.weight.to(pd), self.sampling_offsets.bias.to(pd))
            logits = F.linear(q, self.attention_weights.weight.to(pd),
                              self.attention_weights.bias.to(pd))
        else:
            off = self.sampling_offsets(query)
            logits = self.attention_weights(query)
        off = off.view(B, Q, M, L, K, 2)
        logits = logits.view(B, Q, M, L * K)
        ref = reference_points.to(off.dtype)
        loc, attn = sampling_prep(ref, off, logits, shapes)
        core = multi_scale_deformable_attention(value, shapes, starts, loc, attn,
                                                self.fp32_grad_accum)
        return self.output_proj(core)
