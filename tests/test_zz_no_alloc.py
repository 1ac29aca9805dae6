"""The allocation-free backward (msda_backward_noalloc) against msda_backward.

msda_backward_noalloc takes its workspace from a static scratch array inside
the library. Two calls in a row, the second on a smaller problem, must give
what msda_backward gives on the same inputs: grad_sampling_locations and
grad_attention_weights bit for bit (no atomics behind them), grad_value
within the oracle parity rule (its summation order may differ between runs).
Each mode that needs a workspace runs: AUTO (bins for two levels), BINNED
(bins for all levels), PER_LEVEL (fp32 sums for two levels), and on pixel
queries PREREDUCE (two levels pre-reduced in LDS, two binned).
"""

import os

import pytest
import torch

from scale_deformable_attention_amd.workloads import make_inputs, workload

from _parity import check_backward, parity_kwargs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _library():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from scale_deformable_attention_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    _binding.load_library()


@pytest.mark.parametrize("accum", ["auto", "binned", "per_level"])
def test_noalloc_matches_backward_on_two_calls(accum):
    import oracle
    from scale_deformable_attention_amd._binding import (msda_backward,
                                                         msda_backward_noalloc,
                                                         msda_backward_workspace_size)
    for B, Q, seed in ((4, 300, 1002), (2, 120, 7)):  # the second call is smaller
        wl = workload("decoder_bf16").replace(name=f"decoder_B{B}_Q{Q}", B=B, Q=Q, seed=seed)
        inp = make_inputs(wl)
        g = {k: (v.to(DEV) if k != "spatial_shapes" else v) for k, v in inp.items()}
        args = (g["value"], g["spatial_shapes"], None, g["sampling_locations"],
                g["attention_weights"], g["grad_output"])
        need = msda_backward_workspace_size(*args[:5], accum=accum)
        print(f"case noalloc {accum} B={B} Q={Q}: workspace {need} bytes", flush=True)
        assert 0 < need <= 32 << 20
        gv = torch.empty_like(g["value"])
        gl = torch.empty_like(g["sampling_locations"])
        ga = torch.empty_like(g["attention_weights"])
        msda_backward_noalloc(*args, gv, gl, ga, accum=accum)
        ref_gv, ref_gl, ref_ga = msda_backward(*args, accum=accum)
        torch.cuda.synchronize()
        assert torch.equal(gl, ref_gl) and torch.equal(ga, ref_ga)
        o_args = (inp["value"], inp["spatial_shapes"], None, inp["sampling_locations"],
                  inp["attention_weights"])
        ref_grads = oracle.backward(*o_args, inp["grad_output"], return_touched=True)
        kw = parity_kwargs(wl.dtype, accum, inp)
        for got in ((gv, gl, ga), (ref_gv, ref_gl, ref_ga)):
            check_backward(wl.dtype, tuple(t.cpu() for t in got), ref_grads[:3],
                           inp["spatial_shapes"], None, ref_grads[3], **kw)


@pytest.mark.parametrize("accum", ["auto", "binned", "prereduce"])
def test_noalloc_pixel_queries_on_two_calls(accum):
    """Pixel queries (every pyramid pixel a query, K = 4) take the count /
    scan / place chain, whose records merge a query's corners that share a
    pixel; two calls in a row, the second smaller, against msda_backward."""
    import oracle
    from scale_deformable_attention_amd._binding import (msda_backward,
                                                         msda_backward_noalloc,
                                                         msda_backward_workspace_size)
    from scale_deformable_attention_amd.workloads import Workload
    for B, levels, seed in ((2, ((30, 44), (15, 22), (8, 11), (4, 6)), 51),
                            (1, ((20, 28), (10, 14), (5, 7), (3, 4)), 52)):
        wl = Workload(name=f"pixels_B{B}", dtype=torch.bfloat16, B=B, Q=None, M=2, D=32, K=4,
                      levels=levels, loc_kind="reference", loc_sigma=0.02, seed=seed)
        inp = make_inputs(wl)
        g = {k: (v.to(DEV) if k != "spatial_shapes" else v) for k, v in inp.items()}
        args = (g["value"], g["spatial_shapes"], None, g["sampling_locations"],
                g["attention_weights"], g["grad_output"])
        need = msda_backward_workspace_size(*args[:5], accum=accum)
        print(f"case noalloc pixel queries {accum} B={B} S={wl.S}: workspace {need} bytes",
              flush=True)
        assert 0 < need <= 32 << 20 and wl.S * wl.K > 2048
        gv = torch.empty_like(g["value"])
        gl = torch.empty_like(g["sampling_locations"])
        ga = torch.empty_like(g["attention_weights"])
        msda_backward_noalloc(*args, gv, gl, ga, accum=accum)
        ref_gv, ref_gl, ref_ga = msda_backward(*args, accum=accum)
        torch.cuda.synchronize()
        assert torch.equal(gl, ref_gl) and torch.equal(ga, ref_ga)
        o_args = (inp["value"], inp["spatial_shapes"], None, inp["sampling_locations"],
                  inp["attention_weights"])
        ref_grads = oracle.backward(*o_args, inp["grad_output"], return_touched=True)
        kw = parity_kwargs(wl.dtype, accum, inp)
        for got in ((gv, gl, ga), (ref_gv, ref_gl, ref_ga)):
            check_backward(wl.dtype, tuple(t.cpu() for t in got), ref_grads[:3],
                           inp["spatial_shapes"], None, ref_grads[3], **kw)
