"""Autograd wrapper and HIP-graph capture of the HIP path.

The autograd node must give the oracle's gradients for value, locations and
weights and None for the level tables (course page "5. The backward kernel",
section "The autograd wrapper"), honour the fp32_grad_accum tri-state, and a
whole forward + backward must be capturable in a HIP graph: each replay,
with new inputs copied into the captured buffers before it (eager work and
synchronisations in between), must match an eager run on the same inputs
bit for bit where no atomics are involved, and the oracle in full.
"""

import os

import pytest
import torch

import oracle
from scale_deformable_attention_amd import (msda_backward, msda_backward_resolve_accum,
                                            msda_forward, multi_scale_deformable_attention)
from scale_deformable_attention_amd.workloads import Workload, make_inputs, workload

from _parity import check_backward, check_forward, check_slice, parity_kwargs, to_np

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


def say(msg):
    print(msg, flush=True)


def _leaves(inp, grads=(True, True, True)):
    v = inp["value"].to(DEV).requires_grad_(grads[0])
    loc = inp["sampling_locations"].to(DEV).requires_grad_(grads[1])
    a = inp["attention_weights"].to(DEV).requires_grad_(grads[2])
    return v, loc, a


def _oracle(inp):
    args = (inp["value"], inp["spatial_shapes"], None, inp["sampling_locations"],
            inp["attention_weights"])
    out, touched = oracle.forward(*args, return_touched=True)
    gv, gl, ga, trows = oracle.backward(*args, inp["grad_output"], return_touched=True)
    return out, touched, (gv, gl, ga), trows


_REF = {}


def _case(name):
    if name not in _REF:
        inp = make_inputs(workload(name))
        _REF[name] = (inp, _oracle(inp))
    return _REF[name]


def _autograd_check(name, switch, device_shapes=False):
    inp, (ref_out, touched, ref_grads, trows) = _case(name)
    dtype = inp["value"].dtype
    v, loc, a = _leaves(inp)
    shapes = inp["spatial_shapes"].to(DEV) if device_shapes else inp["spatial_shapes"]
    out = multi_scale_deformable_attention(v, shapes, None, loc, a, fp32_grad_accum=switch)
    B, Q, M, L, K, _ = loc.shape
    assert out.shape == (B, Q, M * v.shape[3]) and out.dtype == dtype
    out.backward(inp["grad_output"].to(DEV).reshape(out.shape))
    torch.cuda.synchronize()
    check_forward(dtype, out.detach().cpu(), ref_out, touched)
    check_backward(dtype, (v.grad.cpu(), loc.grad.cpu(), a.grad.cpu()), ref_grads,
                   inp["spatial_shapes"], None, trows,
                   **parity_kwargs(dtype, switch, inp, workload_name=name))


def test_autograd_matches_oracle_tiny():
    say("case tiny_fp32 autograd, device level table")
    _autograd_check("tiny_fp32", None, device_shapes=True)


@pytest.mark.parametrize("switch", [None, True, False, "per_level", "binned", "mixed"])
def test_autograd_accumulation_switch_decoder(switch):
    say(f"case decoder_bf16 autograd fp32_grad_accum={switch!r}")
    _autograd_check("decoder_bf16", switch)


def test_autograd_switch_maps_to_library_modes():
    inp, _ = _case("tiny_fp32")
    g = {k: (t.to(DEV) if k != "spatial_shapes" else t) for k, t in inp.items()}
    args = (g["value"], g["spatial_shapes"], None, g["sampling_locations"], g["attention_weights"])
    # fp32 data: True asks for fp32 scratch, which fp32 data never needs
    assert msda_backward_resolve_accum(*args, accum=True) == "native"
    assert msda_backward_resolve_accum(*args, accum=False) == "native"
    assert msda_backward_resolve_accum(*args, accum=None) == msda_backward_resolve_accum(*args)
    with pytest.raises(ValueError):
        multi_scale_deformable_attention(*args, fp32_grad_accum="sometimes")


def test_autograd_only_requested_inputs_get_gradients():
    say("case tiny_fp32 autograd, only value requires grad")
    inp, (_, _, ref_grads, trows) = _case("tiny_fp32")
    v, loc, a = _leaves(inp, grads=(True, False, False))
    out = multi_scale_deformable_attention(v, inp["spatial_shapes"], None, loc, a)
    out.backward(inp["grad_output"].to(DEV).reshape(out.shape))
    assert loc.grad is None and a.grad is None
    got = to_np(v.grad.cpu())
    check_slice("grad_value", got, to_np(ref_grads[0]), 1e-5)


def test_autograd_is_once_differentiable():
    inp, _ = _case("tiny_fp32")
    v, loc, a = _leaves(inp)
    out = multi_scale_deformable_attention(v, inp["spatial_shapes"], None, loc, a)
    (gv,) = torch.autograd.grad(out.sum(), v, create_graph=True)
    with pytest.raises(RuntimeError):
        gv.sum().backward()


def test_autograd_empty_query_set():
    wl = Workload(name="empty_q", dtype=torch.float32, B=2, Q=0, M=2, D=8, K=2,
                  levels=((8, 10), (4, 5)), loc_kind="uniform", seed=7)
    inp = make_inputs(wl)
    v, loc, a = _leaves(inp)
    out = multi_scale_deformable_attention(v, inp["spatial_shapes"], None, loc, a)
    assert out.shape == (2, 0, 16)
    out.sum().backward()
    torch.cuda.synchronize()
    assert v.grad is not None and not v.grad.any()
    assert loc.grad.shape == loc.shape and a.grad.shape == a.shape


# ------------------------------------------------------------- HIP graphs

@pytest.mark.parametrize("name,switch", [("decoder_bf16", None), ("decoder_bf16", "binned"),
                                         ("decoder_bf16", "per_level"), ("decoder_bf16", False),
                                         ("oddhead_fp32", None), ("encoder_fp16", None)])
def test_graph_capture_replays_match_eager(name, switch):
    """Capture forward + backward once, replay with three fresh input sets.
    The odd-head and encoder cases bin enough records to run the binned chain
    on the side stream, captured as a fork and a join."""
    wl = workload(name)
    say(f"case {name} graph capture, fp32_grad_accum={switch!r}")
    inp = make_inputs(wl)
    shapes = inp["spatial_shapes"].tolist()  # host level table: no copy under capture
    v, loc, a = _leaves(inp)
    gout = inp["grad_output"].to(DEV).reshape(wl.B, wl.num_queries, wl.M * wl.D).contiguous()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            out = multi_scale_deformable_attention(v, shapes, None, loc, a, switch)
            out.backward(gout)
            v.grad = loc.grad = a.grad = None
            del out  # no autograd graph of the warm-up may outlive it
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        static_out = multi_scale_deformable_attention(v, shapes, None, loc, a, switch)
        static_out.backward(gout)
    torch.cuda.synchronize()

    accum = {None: "auto", False: "native"}.get(switch, switch)
    for trial in range(3):
        fresh = make_inputs(wl, seed=5000 + trial)
        with torch.no_grad():
            v.copy_(fresh["value"].to(DEV))
            loc.copy_(fresh["sampling_locations"].to(DEV))
            a.copy_(fresh["attention_weights"].to(DEV))
            gout.copy_(fresh["grad_output"].to(DEV).reshape(gout.shape))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        with torch.no_grad():
            e_out = msda_forward(v.detach(), shapes, None, loc.detach(), a.detach())
            e_gv, e_gl, e_ga = msda_backward(v.detach(), shapes, None, loc.detach(), a.detach(),
                                             gout, accum=accum)
        torch.cuda.synchronize()
        # no atomics behind these three: bit-identical
        assert torch.equal(static_out, e_out), f"replay {trial}: output differs"
        assert torch.equal(loc.grad, e_gl), f"replay {trial}: grad_sampling_locations differs"
        assert torch.equal(a.grad, e_ga), f"replay {trial}: grad_attention_weights differs"
        # grad_value: the summation order may differ between runs (atomics,
        # records within a bin), so each replay is held to the oracle instead
        ref_out, touched, ref_grads, trows = _oracle(fresh)
        check_forward(wl.dtype, static_out.cpu(), ref_out, touched)
        check_backward(wl.dtype, (v.grad.cpu(), loc.grad.cpu(), a.grad.cpu()), ref_grads,
                       fresh["spatial_shapes"], None, trows,
                       **parity_kwargs(wl.dtype, switch, fresh, workload_name=name))


def test_capture_on_a_thread_without_side_stream():
    """A binned backward captured by a thread that never made one before runs
    on the caller's stream alone (no side stream is created under capture);
    its replays must still match the oracle. The odd-head workload bins
    enough records to use a side stream otherwise."""
    import threading
    from scale_deformable_attention_amd import PreparedCall
    wl = workload("oddhead_fp32")
    inp = make_inputs(wl)
    g = {k: (t.to(DEV) if k != "spatial_shapes" else t) for k, t in inp.items()}
    errors = []

    def body():
        try:
            torch.cuda.set_device(0)
            call = PreparedCall(g["value"], g["spatial_shapes"], None, g["sampling_locations"],
                                g["attention_weights"], g["grad_output"], accum="mixed")
            stream = torch.cuda.Stream()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                call.forward()
                call.backward()
            for _ in range(2):
                graph.replay()
                torch.cuda.synchronize()
                ref_out, touched, ref_grads, trows = _oracle(inp)
                check_forward(wl.dtype, call.output.cpu(), ref_out, touched)
                check_backward(wl.dtype, (call.grad_value.cpu(), call.grad_loc.cpu(),
                                          call.grad_attn.cpu()), ref_grads,
                               inp["spatial_shapes"], None, trows)
        except Exception as e:  # reported in the main thread
            errors.append(e)

    say("case oddhead_fp32 capture in a fresh thread (mixed)")
    th = threading.Thread(target=body)
    th.start()
    th.join()
    if errors:
        raise errors[0]


def test_instrumented_launch_names():
    from scale_deformable_attention_amd import PreparedCall
    from scale_deformable_attention_amd._binding import (launch_event_names,
                                                         set_launch_events)
    inp = make_inputs(workload("decoder_bf16"))
    g = {k: (t.to(DEV) if k != "spatial_shapes" else t) for k, t in inp.items()}
    call = PreparedCall(g["value"], g["spatial_shapes"], None, g["sampling_locations"],
                        g["attention_weights"], g["grad_output"], accum="mixed")
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(20)]
    for e in evs:
        e.record()  # torch creates the HIP event on first record
    torch.cuda.synchronize()
    set_launch_events(evs[:2])
    call.forward()
    assert launch_event_names() == ["msda_fwd_kernel"]
    set_launch_events(evs)
    call.backward()
    torch.cuda.synchronize()
    assert launch_event_names() == ["grad_sort_kernel", "scatter_accum_kernel"]
    for i in range(2):
        assert evs[2 * i].elapsed_time(evs[2 * i + 1]) >= 0.0
