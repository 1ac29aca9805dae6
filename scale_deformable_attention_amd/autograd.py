"""PyTorch autograd integration of the MSDA core.

`multi_scale_deformable_attention(value, spatial_shapes, level_start_index,
sampling_locations, attention_weights, fp32_grad_accum=None)` returns the
(B, Q, M*D) output with the operator signature of the msda-triton README
(section "Quickstart"); both passes run the HIP kernels through the C ABI.
The backward returns gradients for value, sampling_locations and
attention_weights and None for the level tables and the switch, and is
once-differentiable (course page "5. The backward kernel: gradients,
atomics, and a precision switch", section "The autograd wrapper").

`fp32_grad_accum` keeps the pages' tri-state meaning: None lets the library
choose (AUTO), True forces fp32 accumulation of grad_value (FP32_SCRATCH),
False forces atomics of the value dtype (NATIVE). The library's other modes
("per_level", "binned", "mixed") are accepted by name.

Graph capture: the level tables are read on the host. Pass them as CPU
tensors or Python lists when the call is captured in a HIP graph (a device
tensor would need a device-to-host copy, which capture forbids); they are
copied once in the forward and reused by the backward.
"""

from __future__ import annotations

from typing import Union

import torch
from torch.autograd.function import once_differentiable

from . import _binding

_ACCUM_BY_SWITCH = {None: "auto", True: "fp32_scratch", False: "native"}


def _accum_name(fp32_grad_accum: Union[bool, str, None]) -> str:
    if isinstance(fp32_grad_accum, str):
        if fp32_grad_accum not in _binding._ACCUM_CODES:
            raise ValueError(f"unknown accumulation mode {fp32_grad_accum!r}")
        return fp32_grad_accum
    if fp32_grad_accum not in _ACCUM_BY_SWITCH:
        raise ValueError(f"fp32_grad_accum must be None, True, False or a mode name, "
                         f"got {fp32_grad_accum!r}")
    return _ACCUM_BY_SWITCH[fp32_grad_accum]


class MultiScaleDeformableAttnFunction(torch.autograd.Function):
    """The MSDA core as an autograd node (see the module docstring)."""

    @staticmethod
    def forward(ctx, value, spatial_shapes, level_start_index, sampling_locations,
                attention_weights, fp32_grad_accum=None):
        levels = _binding._Levels(spatial_shapes, level_start_index)  # host copies, once
        value = value.contiguous()
        sampling_locations = sampling_locations.contiguous()
        attention_weights = attention_weights.contiguous()
        out = _binding.msda_forward(value, levels.shapes, levels.starts, sampling_locations,
                                    attention_weights)
        ctx.save_for_backward(value, sampling_locations, attention_weights)
        ctx.levels = (levels.shapes, levels.starts)
        ctx.accum = _accum_name(fp32_grad_accum)
        return out

    @staticmethod
    @once_differentiable
    def backward(ctx, grad_output):
        value, loc, attn = ctx.saved_tensors
        shapes, starts = ctx.levels
        grad_value, grad_loc, grad_attn = _binding.msda_backward(
            value, shapes, starts, loc, attn, grad_output.contiguous(), accum=ctx.accum)
        need = ctx.needs_input_grad
        return (grad_value if need[0] else None, None, None,
                grad_loc if need[3] else None, grad_attn if need[4] else None, None)


def multi_scale_deformable_attention(value: torch.Tensor, spatial_shapes, level_start_index,
                                     sampling_locations: torch.Tensor,
                                     attention_weights: torch.Tensor,
                                     fp32_grad_accum: Union[bool, str, None] = None) -> torch.Tensor:
    """Differentiable MSDA core: value (B, S, M, D), sampling_locations
    (B, Q, M, L, K, 2), attention_weights (B, Q, M, L, K) -> (B, Q, M*D)."""
    _accum_name(fp32_grad_accum)  # reject a bad switch before any launch
    return MultiScaleDeformableAttnFunction.apply(value, spatial_shapes, level_start_index,
                                                  sampling_locations, attention_weights,
                                                  fp32_grad_accum)
