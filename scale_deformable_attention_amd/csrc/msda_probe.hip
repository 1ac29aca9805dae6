// Measurement kernel, not part of the MSDA computation: the request rate of
// device-scope no-return atomic adds on gfx950, which bounds the backward's
// grad_value scatter on levels accumulated with atomics (course page "5. The
// backward kernel", section "Scatter needs atomics").
//
// Every lane issues `iters` adds. Lanes are grouped in runs of 2^log2run
// consecutive lanes (1 to 16); a run targets one 64-byte segment, lane i of
// the run its dword i, so one instruction of a wave makes 64 / run requests
// of run dwords each. Runs visit segments in a stride that keeps the runs in
// flight on distinct segments (no same-address serialisation): segment =
// (run + it * runs) mod nseg, nseg a power of two.

#include "msda_device.h"
#include "msda_launch.h"

namespace msda {
namespace {

typedef __bf16 probe_bf16x2_t __attribute__((ext_vector_type(2)));

template <bool BF16>
__global__ __launch_bounds__(kBlock) void atomic_probe_kernel(uint32_t *__restrict__ buf,
                                                              uint32_t seg_mask, int iters,
                                                              int log2run) {
    const uint32_t gtid = blockIdx.x * (uint32_t)kBlock + threadIdx.x;
    const uint32_t run = gtid >> log2run;
    const uint32_t lane = gtid & ((1u << log2run) - 1u);
    const uint32_t runs = (gridDim.x * (uint32_t)kBlock) >> log2run;
    for (int it = 0; it < iters; ++it) {
        const uint32_t seg = (run + (uint32_t)it * runs) & seg_mask;
        uint32_t *p = buf + (size_t)seg * 16u + lane;
        if constexpr (BF16) {
            probe_bf16x2_t v;
            v.x = (__bf16)1.0f;
            v.y = (__bf16)1.0f;
            __builtin_amdgcn_global_atomic_fadd_v2bf16(reinterpret_cast<probe_bf16x2_t *>(p), v);
        } else {
            __hip_atomic_fetch_add(reinterpret_cast<float *>(p), 1.0f, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace

hipError_t launch_atomic_probe(void *buf, int64_t nseg, int bf16, int log2run, int64_t workgroups,
                               int iters, hipStream_t stream) {
    if (bf16)
        MSDA_LAUNCH(atomic_probe_kernel<true>, dim3((unsigned)workgroups), dim3(kBlock), 0, stream,
                    static_cast<uint32_t *>(buf), (uint32_t)(nseg - 1), iters, log2run);
    else
        MSDA_LAUNCH(atomic_probe_kernel<false>, dim3((unsigned)workgroups), dim3(kBlock), 0,
                    stream, static_cast<uint32_t *>(buf), (uint32_t)(nseg - 1), iters, log2run);
    return hipGetLastError();
}

}  // namespace msda
