// Internal interface between the host-side C ABI (msda_api.cpp) and the
// gfx950 kernels (msda_kernels.hip). Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msda.h"

namespace msda {

// Level table passed by value in the kernel arguments (no device copy, no
// host synchronisation). H, W < 2^24 so that they are exact in fp32.
struct LevelTable {
    int32_t H[MSDA_MAX_LEVELS];
    int32_t W[MSDA_MAX_LEVELS];
    int64_t start[MSDA_MAX_LEVELS];
};

// Everything a launch needs, validated by the host layer.
struct Problem {
    int dtype;          // msda_dtype_t
    int64_t B, S, M, D, L, Q, K;
    LevelTable levels;
};

// Lane mapping chosen on the host: each query's channels are spread over
// G = 2^log2_group lanes holding `vec` consecutive channels each; 2^log2_split
// lane groups share one query and split its L*K points between them.
struct Mapping {
    int vec;
    int log2_group;
    int log2_split;
};

hipError_t launch_forward(const Problem &p, const Mapping &mp, const void *value,
                          const void *loc, const void *attn, void *out,
                          hipStream_t stream);

// accum_fp32: atomics go to `acc_target` as fp32 (the scratch buffer, or
// grad_value itself for fp32 data); otherwise packed atomics of the value
// dtype go straight into grad_value.
hipError_t launch_backward(const Problem &p, const Mapping &mp, const void *value,
                           const void *loc, const void *attn, const void *grad_out,
                           void *acc_target, bool accum_fp32, void *grad_loc,
                           void *grad_attn, hipStream_t stream);

// Fill `bytes` bytes (a multiple of 2) at `dst` with zeros.
hipError_t launch_zero(void *dst, size_t bytes, hipStream_t stream);

// grad_value[i] = (dtype) scratch[i], or += with `accumulate`, for n elements.
hipError_t launch_downcast(int dtype, const float *scratch, void *grad_value, int64_t n,
                           bool accumulate, hipStream_t stream);

}  // namespace msda
