"""MI355X-native multi-scale deformable attention (MSDA) core.

The computation runs in hand-written gfx950 HIP kernels behind a C ABI
(include/msda.h, libmsda_amd.so); this package is the thin Python layer:

    msda_forward, msda_backward          the C entry points, with torch tensors
    PreparedCall                         the same calls pre-marshalled for loops
    multi_scale_deformable_attention     autograd wrapper (autograd.py)
    msda_sampling_prep(_backward)        reference scaling + softmax over L*K (C entry points)
    MSDeformAttn, sampling_prep          the module around the core (module.py)
    workloads                            seeded synthetic inputs

The library is loaded on first use, so importing the package (for example for
the input generators) needs neither a GPU nor a built library.
"""

from ._binding import (ACCUM_AUTO, ACCUM_FP32_SCRATCH, ACCUM_NATIVE, EXPORTED_SYMBOLS,  # noqa: F401
                       MSDAError, PreparedCall, load_library, msda_backward,
                       msda_backward_resolve_accum, msda_backward_workspace_size, msda_forward,
                       msda_sampling_prep, msda_sampling_prep_backward)
from .autograd import MultiScaleDeformableAttnFunction, multi_scale_deformable_attention
from .module import MSDeformAttn, SamplingPrepFunction, sampling_prep

__all__ = ["msda_forward", "msda_backward", "msda_backward_workspace_size",
           "msda_backward_resolve_accum", "MSDAError", "PreparedCall", "load_library",
           "multi_scale_deformable_attention", "MultiScaleDeformableAttnFunction",
           "msda_sampling_prep", "msda_sampling_prep_backward", "MSDeformAttn",
           "SamplingPrepFunction", "sampling_prep"]
