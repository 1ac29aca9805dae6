// gfx950 kernels of the steps that turn a deformable-attention module's
// linear outputs into the core's inputs, and their backward (msda-triton
// README, section "The operator": offsets added to the reference point
// mapped to each level, weights normalised by a softmax; section
// "Quickstart": the softmax runs over the flattened L*K points of each
// (b, q, m)).
//
//   sampling_locations[b,q,m,l,k] = ref[b,q(,l)] + (dx / W_l, dy / H_l)
//   attention_weights[b,q,m,:]    = softmax(logits[b,q,m,:])  over L*K
//
// Lane layout: each (b, q, m) row of L*K points is owned by P lanes, P the
// power of two >= L*K capped at 64; lane j of a row handles points j, j + P,
// ... A row's max and sums are butterfly reductions over its P lanes (rows
// are aligned to P within a wave, so every shuffle stays inside the row), and
// consecutive lanes touch consecutive points, so every access is coalesced.
// All arithmetic is fp32, rounded once to the storage type at the store.

#include "msda_device.h"
#include "msda_launch.h"

namespace msda {
namespace {

template <class T>
__device__ __forceinline__ float ld(const typename T::S *p, int64_t i) {
    return to_f32(T{}, p[i]);
}

__device__ __forceinline__ float row_max(float v, int P) {
    for (int o = 1; o < P; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float row_sum(float v, int P) {
    for (int o = 1; o < P; o <<= 1) v += __shfl_xor(v, o);
    return v;
}

template <class T>
__global__ __launch_bounds__(kBlock) void sampling_prep_kernel(
    const typename T::S *__restrict__ ref, const typename T::S *__restrict__ off,
    const typename T::S *__restrict__ logits, typename T::S *__restrict__ loc,
    typename T::S *__restrict__ attn, const PrepProblem p, const int64_t rows, const int log2p) {
    const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int64_t row = t >> log2p;  // (b, q, m)
    if (row >= rows) return;         // a row's P lanes leave together
    const int P = 1 << log2p;
    const int jl = (int)(t & (P - 1));
    const int K = (int)p.K, LK = (int)(p.L * p.K);
    const int64_t base = row * LK;
    float mx = -INFINITY;
    for (int j = jl; j < LK; j += P) mx = fmaxf(mx, ld<T>(logits, base + j));
    mx = row_max(mx, P);
    float sum = 0.0f;
    for (int j = jl; j < LK; j += P) sum += expf(ld<T>(logits, base + j) - mx);
    sum = row_sum(sum, P);
    const int64_t bq = row / p.M;
    for (int j = jl; j < LK; j += P) {
        attn[base + j] = from_f32(T{}, expf(ld<T>(logits, base + j) - mx) / sum);
        const int l = j / K;
        const int64_t ri = (p.ref_levels == 1 ? bq : bq * p.L + l) * 2;
        const int64_t pi = (base + j) * 2;
        loc[pi] = from_f32(T{}, ld<T>(ref, ri) + ld<T>(off, pi) / p.W[l]);
        loc[pi + 1] = from_f32(T{}, ld<T>(ref, ri + 1) + ld<T>(off, pi + 1) / p.H[l]);
    }
}

// d logit_j = A_j (g_j - sum_i A_i g_i); d offset = d location / (W_l, H_l).
template <class T>
__global__ __launch_bounds__(kBlock) void sampling_prep_bwd_kernel(
    const typename T::S *__restrict__ attn, const typename T::S *__restrict__ grad_loc,
    const typename T::S *__restrict__ grad_attn, typename T::S *__restrict__ grad_off,
    typename T::S *__restrict__ grad_logits, const PrepProblem p, const int64_t rows,
    const int log2p) {
    const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int64_t row = t >> log2p;
    if (row >= rows) return;
    const int P = 1 << log2p;
    const int jl = (int)(t & (P - 1));
    const int K = (int)p.K, LK = (int)(p.L * p.K);
    const int64_t base = row * LK;
    float dot = 0.0f;
    for (int j = jl; j < LK; j += P) dot = fmaf(ld<T>(attn, base + j), ld<T>(grad_attn, base + j), dot);
    dot = row_sum(dot, P);
    for (int j = jl; j < LK; j += P) {
        const float a = ld<T>(attn, base + j), g = ld<T>(grad_attn, base + j);
        grad_logits[base + j] = from_f32(T{}, a * (g - dot));
        const int l = j / K;
        const int64_t pi = (base + j) * 2;
        grad_off[pi] = from_f32(T{}, ld<T>(grad_loc, pi) / p.W[l]);
        grad_off[pi + 1] = from_f32(T{}, ld<T>(grad_loc, pi + 1) / p.H[l]);
    }
}

// One wave per (b, q): the reference gradient is the sum of the location
// gradients over heads and points (and levels, for one point per query).
// Lanes stride over the (m, k) pairs of one level at a time; wave butterfly.
template <class T>
__global__ __launch_bounds__(kBlock) void reference_grad_kernel(
    const typename T::S *__restrict__ grad_loc, typename T::S *__restrict__ grad_ref,
    const PrepProblem p, const int64_t nbq) {
    const int lane = threadIdx.x & 63;
    const int64_t bq = (int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
    if (bq >= nbq) return;  // whole waves
    const int M = (int)p.M, L = (int)p.L, K = (int)p.K, MK = M * K;
    float sx = 0.0f, sy = 0.0f;
    for (int l = 0; l < L; ++l) {
        for (int i = lane; i < MK; i += 64) {
            const int m = i / K, k = i - m * K;
            const int64_t pi = (((bq * M + m) * L + l) * K + k) * 2;
            sx += ld<T>(grad_loc, pi);
            sy += ld<T>(grad_loc, pi + 1);
        }
        if (p.ref_levels != 1 || l == L - 1) {
            const float x = row_sum(sx, 64), y = row_sum(sy, 64);
            if (lane == 0) {
                const int64_t ri = (p.ref_levels == 1 ? bq : bq * L + l) * 2;
                grad_ref[ri] = from_f32(T{}, x);
                grad_ref[ri + 1] = from_f32(T{}, y);
            }
            sx = sy = 0.0f;
        }
    }
}

int lanes_log2(int64_t lk) {
    int s = 0;
    while ((1 << s) < lk && s < 6) ++s;
    return s;
}

template <class T>
hipError_t prep_launch(const PrepProblem &p, const void *ref, const void *off, const void *logits,
                       void *loc, void *attn, hipStream_t stream) {
    using S = typename T::S;
    const int64_t rows = p.B * p.Q * p.M;
    const int lg = lanes_log2(p.L * p.K);
    const int64_t grid = ((rows << lg) + kBlock - 1) / kBlock;
    MSDA_LAUNCH(sampling_prep_kernel<T>, dim3((unsigned)grid), dim3(kBlock), 0, stream,
                       static_cast<const S *>(ref), static_cast<const S *>(off),
                       static_cast<const S *>(logits), static_cast<S *>(loc),
                       static_cast<S *>(attn), p, rows, lg);
    return hipGetLastError();
}

template <class T>
hipError_t prep_bwd_launch(const PrepProblem &p, const void *attn, const void *grad_loc,
                           const void *grad_attn, void *grad_off, void *grad_logits,
                           hipStream_t stream) {
    using S = typename T::S;
    const int64_t rows = p.B * p.Q * p.M;
    const int lg = lanes_log2(p.L * p.K);
    const int64_t grid = ((rows << lg) + kBlock - 1) / kBlock;
    MSDA_LAUNCH(sampling_prep_bwd_kernel<T>, dim3((unsigned)grid), dim3(kBlock), 0, stream,
                       static_cast<const S *>(attn), static_cast<const S *>(grad_loc),
                       static_cast<const S *>(grad_attn), static_cast<S *>(grad_off),
                       static_cast<S *>(grad_logits), p, rows, lg);
    return hipGetLastError();
}

template <class T>
hipError_t ref_grad_launch(const PrepProblem &p, const void *grad_loc, void *grad_ref,
                           hipStream_t stream) {
    using S = typename T::S;
    const int64_t nbq = p.B * p.Q;
    const int64_t grid = (nbq + kBlock / 64 - 1) / (kBlock / 64);
    MSDA_LAUNCH(reference_grad_kernel<T>, dim3((unsigned)grid), dim3(kBlock), 0, stream,
                       static_cast<const S *>(grad_loc), static_cast<S *>(grad_ref), p, nbq);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sampling_prep(const PrepProblem &p, const void *ref, const void *offsets,
                                const void *logits, void *loc, void *attn, hipStream_t stream) {
    switch (p.dtype) {
        case MSDA_F32: return prep_launch<F32T>(p, ref, offsets, logits, loc, attn, stream);
        case MSDA_F16: return prep_launch<F16T>(p, ref, offsets, logits, loc, attn, stream);
        case MSDA_BF16: return prep_launch<BF16T>(p, ref, offsets, logits, loc, attn, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_sampling_prep_backward(const PrepProblem &p, const void *attn,
                                         const void *grad_loc, const void *grad_attn,
                                         void *grad_offsets, void *grad_logits,
                                         hipStream_t stream) {
    switch (p.dtype) {
        case MSDA_F32:
            return prep_bwd_launch<F32T>(p, attn, grad_loc, grad_attn, grad_offsets, grad_logits,
                                         stream);
        case MSDA_F16:
            return prep_bwd_launch<F16T>(p, attn, grad_loc, grad_attn, grad_offsets, grad_logits,
                                         stream);
        case MSDA_BF16:
            return prep_bwd_launch<BF16T>(p, attn, grad_loc, grad_attn, grad_offsets, grad_logits,
                                          stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_reference_grad(const PrepProblem &p, const void *grad_loc, void *grad_ref,
                                 hipStream_t stream) {
    switch (p.dtype) {
        case MSDA_F32: return ref_grad_launch<F32T>(p, grad_loc, grad_ref, stream);
        case MSDA_F16: return ref_grad_launch<F16T>(p, grad_loc, grad_ref, stream);
        case MSDA_BF16: return ref_grad_launch<BF16T>(p, grad_loc, grad_ref, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace msda
