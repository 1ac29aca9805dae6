"""Seeded synthetic inputs for the multi-scale deformable attention (MSDA) core.

This module only draws random tensors of the right shapes, value distributions
and structure. It holds none of the operator's arithmetic: no coordinate
mapping, no bilinear weights, no sums. Both the HIP path and the CPU oracle are
fed from here, so neither depends on the other.

Shapes follow the operator's layout (msda-triton README, section "Quickstart"):
    value               (B, S, M, D)
    spatial_shapes      (L, 2) int64, rows (H_l, W_l)
    sampling_locations  (B, Q, M, L, K, 2), normalised, last axis (x, y)
    attention_weights   (B, Q, M, L, K)
    grad_output         (B, Q, M*D)

Recipe for every workload (draws are fp32 from one seeded CPU generator, in
the fixed order value, logits, locations, grad_output; then one cast to the
workload dtype):
    value        N(0, 1)
    weights      softmax over the L*K axis of N(0, 1) logits, in fp32 (the
                 caller's job according to the README's quickstart, so it is
                 input preparation, not part of the operator)
    locations    "uniform": U(lo, hi) per coordinate
                 "reference": encoder style, every pyramid pixel is one query
                 whose reference point is the centre of its own pixel,
                 ((x + 0.5) / W, (y + 0.5) / H) at its own level, plus a
                 N(0, sigma) offset per (m, l, k, coordinate), optionally
                 clamped
    grad_output  N(0, 1)

The decoder/encoder level shapes are those of an 800x1333 image at strides
8..64 (README, section "Benchmarks"); the large encoder pyramid is 4096x7168
at the same strides. These synthetic draws stand in for the trained offsets and
attention weights of a Deformable-DETR model on COCO, which are not used.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence, Tuple

import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "workload"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: torch.dtype
    B: int
    Q: Optional[int]  # None: every pyramid pixel is a query (Q = S)
    M: int
    D: int
    K: int
    levels: Tuple[Tuple[int, int], ...]
    loc_kind: str  # "uniform" or "reference"
    loc_lo: float = 0.0
    loc_hi: float = 1.0
    loc_sigma: float = 0.0
    loc_clamp: Optional[Tuple[float, float]] = None
    seed: int = 0
    param_dtype: Optional[torch.dtype] = None  # locations / weights; None: dtype

    @property
    def L(self) -> int:
        return len(self.levels)

    @property
    def S(self) -> int:
        return sum(h * w for h, w in self.levels)

    @property
    def num_queries(self) -> int:
        return self.S if self.Q is None else self.Q

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_DECODER_LEVELS = ((100, 167), (50, 84), (25, 42), (13, 21))

WORKLOADS = {
    "tiny_fp32": Workload(
        name="tiny_fp32", dtype=torch.float32, B=1, Q=16, M=2, D=8, K=2,
        levels=((8, 10), (4, 5)), loc_kind="uniform", loc_lo=-0.1, loc_hi=1.1,
        seed=1001),
    "decoder_bf16": Workload(
        name="decoder_bf16", dtype=torch.bfloat16, B=4, Q=300, M=8, D=32, K=4,
        levels=_DECODER_LEVELS, loc_kind="uniform", seed=1002),
    "encoder_fp16": Workload(
        name="encoder_fp16", dtype=torch.float16, B=4, Q=None, M=8, D=32, K=4,
        levels=_DECODER_LEVELS, loc_kind="reference", loc_sigma=0.02,
        loc_clamp=(-0.05, 1.05), seed=1003),
    "oddhead_fp32": Workload(
        name="oddhead_fp32", dtype=torch.float32, B=2, Q=900, M=8, D=48, K=8,
        levels=((200, 334), (100, 167), (50, 84), (25, 42)),
        loc_kind="uniform", seed=1004),
    "large_encoder_bf16": Workload(
        name="large_encoder_bf16", dtype=torch.bfloat16, B=1, Q=None, M=8,
        D=32, K=4, levels=((512, 896), (256, 448), (128, 224), (64, 112)),
        loc_kind="reference", loc_sigma=0.01, seed=1005),
    # mixed dtypes: bf16 / fp16 values, fp32 locations and weights
    "decoder_mixed": Workload(
        name="decoder_mixed", dtype=torch.bfloat16, B=4, Q=300, M=8, D=32, K=4,
        levels=_DECODER_LEVELS, loc_kind="uniform", seed=1006, param_dtype=torch.float32),
    "encoder_mixed": Workload(
        name="encoder_mixed", dtype=torch.float16, B=4, Q=None, M=8, D=32, K=4,
        levels=_DECODER_LEVELS, loc_kind="reference", loc_sigma=0.02,
        loc_clamp=(-0.05, 1.05), seed=1007, param_dtype=torch.float32),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _reference_points(levels: Sequence[Tuple[int, int]]) -> torch.Tensor:
    """(S, 2) fp32 pixel-centre points, pixels enumerated level by level, row-major."""
    pts = []
    for h, w in levels:
        ys, xs = torch.meshgrid(torch.arange(h, dtype=torch.float64),
                                torch.arange(w, dtype=torch.float64), indexing="ij")
        pts.append(torch.stack(((xs + 0.5) / w, (ys + 0.5) / h), dim=-1).reshape(-1, 2))
    return torch.cat(pts, 0).to(torch.float32)


def make_inputs(wl: Workload, seed: Optional[int] = None, device="cpu",
                with_grad: bool = True) -> dict:
    """Draw one seeded input set for workload `wl`.

    Returns a dict of CPU (or `device`) tensors in the workload dtype:
    value, spatial_shapes (int64), sampling_locations, attention_weights and,
    if `with_grad`, grad_output. Locations and weights take
    `wl.param_dtype` when it is set.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(wl.seed if seed is None else seed)
    B, M, D, L, K = wl.B, wl.M, wl.D, wl.L, wl.K
    S, Q = wl.S, wl.num_queries

    value = torch.randn((B, S, M, D), generator=g, dtype=torch.float32)
    logits = torch.randn((B, Q, M, L * K), generator=g, dtype=torch.float32)
    attn = torch.softmax(logits, dim=-1).reshape(B, Q, M, L, K)
    del logits
    if wl.loc_kind == "uniform":
        loc = torch.rand((B, Q, M, L, K, 2), generator=g, dtype=torch.float32)
        loc = loc * (wl.loc_hi - wl.loc_lo) + wl.loc_lo
    elif wl.loc_kind == "reference":
        if wl.Q is not None and wl.Q != S:
            raise ValueError("reference-point locations need Q == S")
        ref = _reference_points(wl.levels)  # (Q, 2)
        loc = torch.randn((B, Q, M, L, K, 2), generator=g, dtype=torch.float32)
        loc.mul_(wl.loc_sigma).add_(ref.view(1, Q, 1, 1, 1, 2))
        if wl.loc_clamp is not None:
            loc.clamp_(wl.loc_clamp[0], wl.loc_clamp[1])
    else:
        raise ValueError(f"unknown location kind {wl.loc_kind!r}")
    out = {
        "value": value.to(wl.dtype),
        "spatial_shapes": torch.tensor(wl.levels, dtype=torch.int64).reshape(L, 2),
        "sampling_locations": loc.to(wl.param_dtype or wl.dtype),
        "attention_weights": attn.to(wl.param_dtype or wl.dtype),
    }
    del value, loc, attn
    if with_grad:
        out["grad_output"] = torch.randn((B, Q, M * D), generator=g,
                                         dtype=torch.float32).to(wl.dtype)
    if device != "cpu":
        out = {k: (v.to(device) if k != "spatial_shapes" else v) for k, v in out.items()}
    return out
