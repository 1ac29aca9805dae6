// gfx950 (MI355X, CDNA4) kernels of the multi-scale deformable attention
// sampling/aggregation core.
//
// Work decomposition (course page "4. The forward kernel, line by line",
// section "The design question: what does one program own?"): one workgroup
// owns a block of consecutive queries of one (batch, head) pair and computes
// their whole output privately, with no inter-workgroup reduction. On wave64
// hardware the query's D channels are spread over a lane group of G lanes,
// each holding `VEC` consecutive channels (16-byte accesses where the pointers
// allow), so a corner row of value is fetched as one contiguous run by
// neighbouring lanes; 2^log2_split lane groups may share one query and split
// its L*K points to put more waves in flight when there are few queries.
//
// The bilinear setup (section "Bilinear sampling") is computed in fp32 with
// one fused multiply-add for the pixel mapping and per-dimension validity
// masks; masked corners issue no load and no atomic. Accumulation is fp32 in
// registers and the output is rounded once at the store (section "Accumulate
// and store").
//
// The backward (course page "5. The backward kernel") recomputes the setup
// from the saved inputs, reduces the three per-point dot products across the
// lane group with DPP moves (no LDS traffic), writes grad_attention_weights /
// grad_sampling_locations with plain stores, and scatters grad_value with
// relaxed, agent-scope, no-return atomics: fp32 adds, or packed two-wide
// fp16 / bf16 adds straight into a half-precision grad_value.
//
// Workgroup order is XCD-aware: MI355X dispatches consecutive workgroups
// round-robin over its 8 XCDs, each with its own L2; the block index is
// remapped so that each XCD receives a contiguous range of (batch, head,
// query-block) tiles, keeping one (b, m) slice of value in one L2.

#include "msda_launch.h"

namespace msda {
namespace {

constexpr int kBlock = 256;
constexpr int kXcds = 8;

// ------------------------------------------------------------ element types

struct F32T {
    using S = float;
};
struct F16T {
    using S = uint16_t;
};
struct BF16T {
    using S = uint16_t;
};

__device__ __forceinline__ float to_f32(F32T, float v) { return v; }
__device__ __forceinline__ float to_f32(F16T, uint16_t v) {
    return (float)__builtin_bit_cast(_Float16, v);
}
__device__ __forceinline__ float to_f32(BF16T, uint16_t v) {
    return __uint_as_float((uint32_t)v << 16);
}
__device__ __forceinline__ float from_f32(F32T, float v) { return v; }
__device__ __forceinline__ uint16_t from_f32(F16T, float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}
__device__ __forceinline__ uint16_t from_f32(BF16T, float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}

struct alignas(4) U32x3 {
    uint32_t x, y, z;
};
template <int BYTES>
struct RawVec;
template <>
struct RawVec<2> {
    using type = uint16_t;
};
template <>
struct RawVec<4> {
    using type = uint32_t;
};
template <>
struct RawVec<8> {
    using type = uint2;
};
template <>
struct RawVec<12> {
    using type = U32x3;
};
template <>
struct RawVec<16> {
    using type = uint4;
};

template <class DT, int VEC>
__device__ __forceinline__ void load_vec(const typename DT::S *p, float (&out)[VEC]) {
    using E = typename DT::S;
    using R = typename RawVec<VEC * (int)sizeof(E)>::type;
    const R r = *reinterpret_cast<const R *>(p);
    E e[VEC];
    __builtin_memcpy(e, &r, sizeof(R));
#pragma unroll
    for (int i = 0; i < VEC; ++i) out[i] = to_f32(DT{}, e[i]);
}

template <class DT, int VEC>
__device__ __forceinline__ void store_vec(typename DT::S *p, const float (&v)[VEC]) {
    using E = typename DT::S;
    using R = typename RawVec<VEC * (int)sizeof(E)>::type;
    E e[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) e[i] = from_f32(DT{}, v[i]);
    R r;
    __builtin_memcpy(&r, e, sizeof(R));
    *reinterpret_cast<R *>(p) = r;
}

// Two consecutive elements (x, y) of a sampling location; only element
// alignment is guaranteed, so two scalar loads.
template <class DT>
__device__ __forceinline__ void load_xy(const typename DT::S *p, float &x, float &y) {
    x = to_f32(DT{}, p[0]);
    y = to_f32(DT{}, p[1]);
}

// ------------------------------------------------------- cross-lane sums

template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over an aligned group of 2^log2g lanes, result in every lane of the
// group. All 64 lanes must be active. quad_perm [1,0,3,2] and [2,3,0,1] pair
// lanes inside a quad; after them every lane holds its quad sum, so the
// half-row mirror (lane i <-> 7-i) and the row mirror (i <-> 15-i) each add
// the sum of the other half.
__device__ __forceinline__ float group_sum(float v, int log2g) {
    if (log2g >= 1) v += dpp_move<0xB1>(v);
    if (log2g >= 2) v += dpp_move<0x4E>(v);
    if (log2g >= 3) v += dpp_move<0x141>(v);
    if (log2g >= 4) v += dpp_move<0x140>(v);
    if (log2g >= 5) v += __shfl_xor(v, 16);
    if (log2g >= 6) v += __shfl_xor(v, 32);
    return v;
}

// -------------------------------------------------------------- atomics

__device__ __forceinline__ void atomic_add_f32(float *p, float v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void atomic_add_pk(F16T, uint16_t *p, float a, float b) {
    f16x2_t v;
    v.x = (_Float16)a;
    v.y = (_Float16)b;
    __builtin_amdgcn_global_atomic_fadd_v2f16(reinterpret_cast<f16x2_t *>(p), v);
}
__device__ __forceinline__ void atomic_add_pk(BF16T, uint16_t *p, float a, float b) {
    bf16x2_t v;
    v.x = (__bf16)a;
    v.y = (__bf16)b;
    __builtin_amdgcn_global_atomic_fadd_v2bf16(reinterpret_cast<bf16x2_t *>(p), v);
}

// Add coef * g[0:VEC] into VEC consecutive elements at `t`.
template <class DT, int VEC, bool FP32ACC>
struct Scatter;

template <class DT, int VEC>
struct Scatter<DT, VEC, true> {  // fp32 target
    __device__ __forceinline__ static void add(void *t, int64_t off, float coef,
                                               const float (&g)[VEC]) {
        float *p = static_cast<float *>(t) + off;
#pragma unroll
        for (int i = 0; i < VEC; ++i) atomic_add_f32(p + i, coef * g[i]);
    }
};

template <class DT, int VEC>
struct Scatter<DT, VEC, false> {  // packed half-precision target
    __device__ __forceinline__ static void add(void *t, int64_t off, float coef,
                                               const float (&g)[VEC]) {
        uint16_t *p = static_cast<uint16_t *>(t) + off;
        if constexpr (VEC % 2 == 0) {
            // the host guarantees 4-byte alignment of every pair
#pragma unroll
            for (int i = 0; i < VEC; i += 2) atomic_add_pk(DT{}, p + i, coef * g[i], coef * g[i + 1]);
        } else {
            // single element: packed add on the enclosing aligned word with
            // +0 for the neighbouring element (x + 0 == x)
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                uint16_t *e = p + i;
                const bool hi = (reinterpret_cast<uintptr_t>(e) & 2) != 0;
                uint16_t *w = reinterpret_cast<uint16_t *>(reinterpret_cast<uintptr_t>(e) & ~uintptr_t(3));
                const float v = coef * g[i];
                atomic_add_pk(DT{}, w, hi ? 0.0f : v, hi ? v : 0.0f);
            }
        }
    }
};

// ------------------------------------------------------------ utilities

// Logical tile for this workgroup; the grid has kXcds * per_xcd workgroups and
// XCD x = blockIdx % 8 takes logical tiles [x * per_xcd, (x + 1) * per_xcd).
__device__ __forceinline__ int64_t logical_block() {
    const uint32_t per_xcd = gridDim.x / kXcds;
    return (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
}

// Everything that depends only on the point's location: cell, weights (times
// the attention weight for the forward), masks and corner row offsets.
struct Cell {
    float fx, fy;          // fractional position inside the cell
    bool v00, v01, v10, v11;
    int64_t row00;         // start_l + y0 * W + x0 (meaningful when a corner is valid)
};

__device__ __forceinline__ Cell map_cell(float loc_x, float loc_y, float Hf, float Wf, int W,
                                         int64_t start) {
    Cell c;
    // x = loc_x * W - 0.5 with a single rounding (README "Kernel design").
    const float xf = __builtin_fmaf(loc_x, Wf, -0.5f);
    const float yf = __builtin_fmaf(loc_y, Hf, -0.5f);
    const float x0f = __builtin_floorf(xf);
    const float y0f = __builtin_floorf(yf);
    c.fx = xf - x0f;
    c.fy = yf - y0f;
    const bool vx0 = (x0f >= 0.0f) & (x0f < Wf);
    const bool vx1 = (x0f >= -1.0f) & (x0f < Wf - 1.0f);
    const bool vy0 = (y0f >= 0.0f) & (y0f < Hf);
    const bool vy1 = (y0f >= -1.0f) & (y0f < Hf - 1.0f);
    c.v00 = vy0 & vx0;
    c.v01 = vy0 & vx1;
    c.v10 = vy1 & vx0;
    c.v11 = vy1 & vx1;
    // Clamp before the integer conversion; any valid corner has x0 in [-1, W-1].
    const int x0 = (int)__builtin_fminf(__builtin_fmaxf(x0f, -1.0f), Wf);
    const int y0 = (int)__builtin_fminf(__builtin_fmaxf(y0f, -1.0f), Hf);
    c.row00 = start + (int64_t)y0 * W + x0;
    return c;
}

// ------------------------------------------------------------- forward

template <class DT, int VEC>
__global__ __launch_bounds__(kBlock) void msda_fwd_kernel(
    const typename DT::S *__restrict__ value, const typename DT::S *__restrict__ loc,
    const typename DT::S *__restrict__ attn, typename DT::S *__restrict__ out,
    const LevelTable lt, const int64_t S, const int64_t Q, const int M, const int D,
    const int L, const int K, const int qblocks, const int64_t ntiles, const int log2g,
    const int log2s) {
    using E = typename DT::S;
    const int64_t tile = logical_block();
    if (tile >= ntiles) return;  // whole workgroup leaves together
    const int64_t bm = tile / qblocks;
    const int qb = (int)(tile - bm * qblocks);
    const int64_t b = bm / M;
    const int m = (int)(bm - b * M);

    const int tid = threadIdx.x;
    const int c = tid & ((1 << log2g) - 1);
    const int s = (tid >> log2g) & ((1 << log2s) - 1);
    const int qpb = kBlock >> (log2g + log2s);
    const int64_t q = (int64_t)qb * qpb + (tid >> (log2g + log2s));
    const bool q_ok = q < Q;
    const int c0 = c * VEC;
    const bool live = q_ok && (c0 < D);
    const int split = 1 << log2s;
    const int LK = L * K;

    const int64_t pq = (b * Q + (q_ok ? q : 0)) * M + m;
    const E *loc_q = loc + pq * LK * 2;
    const E *attn_q = attn + pq * LK;
    const int64_t MD = (int64_t)M * D;
    const E *val = value + b * S * MD + (int64_t)m * D + (c0 < D ? c0 : 0);

    float acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.0f;

    for (int l = 0; l < L; ++l) {
        const int H = lt.H[l], W = lt.W[l];
        const int64_t start = lt.start[l];
        const float Hf = (float)H, Wf = (float)W;
#pragma unroll 4
        for (int k = s; k < K; k += split) {
            const int p = l * K + k;
            float lx = 0.0f, ly = 0.0f, a = 0.0f;
            if (q_ok) {
                load_xy<DT>(loc_q + 2 * p, lx, ly);
                a = to_f32(DT{}, attn_q[p]);
            }
            const Cell cl = map_cell(lx, ly, Hf, Wf, W, start);
            const E *p00 = val + cl.row00 * MD;
            const E *p10 = p00 + (int64_t)W * MD;
            float v00[VEC], v01[VEC], v10[VEC], v11[VEC];
#pragma unroll
            for (int i = 0; i < VEC; ++i) v00[i] = v01[i] = v10[i] = v11[i] = 0.0f;
            if (live && cl.v00) load_vec<DT, VEC>(p00, v00);
            if (live && cl.v01) load_vec<DT, VEC>(p00 + MD, v01);
            if (live && cl.v10) load_vec<DT, VEC>(p10, v10);
            if (live && cl.v11) load_vec<DT, VEC>(p10 + MD, v11);
            const float gx = 1.0f - cl.fx, gy = 1.0f - cl.fy;
            const float w00 = a * (gx * gy), w01 = a * (cl.fx * gy);
            const float w10 = a * (gx * cl.fy), w11 = a * (cl.fx * cl.fy);
#pragma unroll
            for (int i = 0; i < VEC; ++i)
                acc[i] += w00 * v00[i] + w01 * v01[i] + w10 * v10[i] + w11 * v11[i];
        }
    }
    // Sum the split lane groups of one query (all lanes active here).
    for (int off = 1 << log2g; off < (1 << (log2g + log2s)); off <<= 1) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[i] += __shfl_xor(acc[i], off);
    }
    if (live && s == 0) store_vec<DT, VEC>(out + pq * D + c0, acc);
}

// ------------------------------------------------------------ backward

template <class DT, int VEC, bool FP32ACC>
__global__ __launch_bounds__(kBlock) void msda_bwd_kernel(
    const typename DT::S *__restrict__ value, const typename DT::S *__restrict__ loc,
    const typename DT::S *__restrict__ attn, const typename DT::S *__restrict__ grad_out,
    void *__restrict__ acc_target, typename DT::S *__restrict__ grad_loc,
    typename DT::S *__restrict__ grad_attn, const LevelTable lt, const int64_t S,
    const int64_t Q, const int M, const int D, const int L, const int K, const int qblocks,
    const int64_t ntiles, const int log2g, const int log2s) {
    using E = typename DT::S;
    const int64_t tile = logical_block();
    if (tile >= ntiles) return;
    const int64_t bm = tile / qblocks;
    const int qb = (int)(tile - bm * qblocks);
    const int64_t b = bm / M;
    const int m = (int)(bm - b * M);

    const int tid = threadIdx.x;
    const int c = tid & ((1 << log2g) - 1);
    const int s = (tid >> log2g) & ((1 << log2s) - 1);
    const int qpb = kBlock >> (log2g + log2s);
    const int64_t q = (int64_t)qb * qpb + (tid >> (log2g + log2s));
    const bool q_ok = q < Q;
    const int c0 = c * VEC;
    const bool live = q_ok && (c0 < D);
    const int split = 1 << log2s;
    const int LK = L * K;

    const int64_t pq = (b * Q + (q_ok ? q : 0)) * M + m;
    const E *loc_q = loc + pq * LK * 2;
    const E *attn_q = attn + pq * LK;
    const int64_t MD = (int64_t)M * D;
    const int64_t col = (int64_t)m * D + (c0 < D ? c0 : 0);
    const E *val = value + b * S * MD + col;
    const int64_t tgt_base = b * S * MD + col;  // element offset into grad_value / scratch

    float g[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) g[i] = 0.0f;
    if (live) load_vec<DT, VEC>(grad_out + pq * D + c0, g);

    for (int l = 0; l < L; ++l) {
        const int H = lt.H[l], W = lt.W[l];
        const int64_t start = lt.start[l];
        const float Hf = (float)H, Wf = (float)W;
#pragma unroll 2
        for (int k = s; k < K; k += split) {
            const int p = l * K + k;
            float lx = 0.0f, ly = 0.0f, a = 0.0f;
            if (q_ok) {
                load_xy<DT>(loc_q + 2 * p, lx, ly);
                a = to_f32(DT{}, attn_q[p]);
            }
            const Cell cl = map_cell(lx, ly, Hf, Wf, W, start);
            const int64_t r00 = cl.row00 * MD;
            const int64_t r10 = r00 + (int64_t)W * MD;
            float v00[VEC], v01[VEC], v10[VEC], v11[VEC];
#pragma unroll
            for (int i = 0; i < VEC; ++i) v00[i] = v01[i] = v10[i] = v11[i] = 0.0f;
            if (live && cl.v00) load_vec<DT, VEC>(val + r00, v00);
            if (live && cl.v01) load_vec<DT, VEC>(val + r00 + MD, v01);
            if (live && cl.v10) load_vec<DT, VEC>(val + r10, v10);
            if (live && cl.v11) load_vec<DT, VEC>(val + r10 + MD, v11);
            const float gx = 1.0f - cl.fx, gy = 1.0f - cl.fy;
            const float w00 = gx * gy, w01 = cl.fx * gy, w10 = gx * cl.fy, w11 = cl.fx * cl.fy;
            float ds = 0.0f, dx = 0.0f, dy = 0.0f;
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                const float smp = w00 * v00[i] + w01 * v01[i] + w10 * v10[i] + w11 * v11[i];
                const float sx = gy * (v01[i] - v00[i]) + cl.fy * (v11[i] - v10[i]);
                const float sy = gx * (v10[i] - v00[i]) + cl.fx * (v11[i] - v01[i]);
                ds += g[i] * smp;
                dx += g[i] * sx;
                dy += g[i] * sy;
            }
            ds = group_sum(ds, log2g);
            dx = group_sum(dx, log2g);
            dy = group_sum(dy, log2g);
            if (q_ok && c == 0) {
                const int64_t pp = pq * LK + p;
                grad_attn[pp] = from_f32(DT{}, ds);
                grad_loc[2 * pp] = from_f32(DT{}, Wf * a * dx);
                grad_loc[2 * pp + 1] = from_f32(DT{}, Hf * a * dy);
            }
            if (live) {
                if (cl.v00) Scatter<DT, VEC, FP32ACC>::add(acc_target, tgt_base + r00, a * w00, g);
                if (cl.v01) Scatter<DT, VEC, FP32ACC>::add(acc_target, tgt_base + r00 + MD, a * w01, g);
                if (cl.v10) Scatter<DT, VEC, FP32ACC>::add(acc_target, tgt_base + r10, a * w10, g);
                if (cl.v11) Scatter<DT, VEC, FP32ACC>::add(acc_target, tgt_base + r10 + MD, a * w11, g);
            }
        }
    }
}

// ------------------------------------------------ zero fill and downcast

__global__ __launch_bounds__(kBlock) void zero_kernel_16(uint4 *__restrict__ dst, int64_t n16) {
    const uint4 z = {0u, 0u, 0u, 0u};
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n16;
         i += (int64_t)gridDim.x * kBlock)
        dst[i] = z;
}

__global__ __launch_bounds__(kBlock) void zero_kernel_2(uint16_t *__restrict__ dst, int64_t n2) {
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n2;
         i += (int64_t)gridDim.x * kBlock)
        dst[i] = 0;
}

template <class DT>
__global__ __launch_bounds__(kBlock) void downcast_kernel(const float *__restrict__ src,
                                                          typename DT::S *__restrict__ dst,
                                                          int64_t n, int accumulate) {
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kBlock) {
        float v = src[i];
        if (accumulate) v += to_f32(DT{}, dst[i]);
        dst[i] = from_f32(DT{}, v);
    }
}

template <class DT>
__global__ __launch_bounds__(kBlock) void downcast_kernel_x4(const float4 *__restrict__ src,
                                                             uint2 *__restrict__ dst, int64_t n4,
                                                             int accumulate) {
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * kBlock) {
        const float4 v = src[i];
        float f[4] = {v.x, v.y, v.z, v.w};
        if (accumulate) {
            float o[4];
            load_vec<DT, 4>(reinterpret_cast<const typename DT::S *>(dst + i), o);
#pragma unroll
            for (int j = 0; j < 4; ++j) f[j] += o[j];
        }
        store_vec<DT, 4>(reinterpret_cast<typename DT::S *>(dst + i), f);
    }
}

int grid_for(int64_t work_items) {
    const int64_t blocks = (work_items + kBlock - 1) / kBlock;
    const int64_t cap = 256 * 16;  // enough to fill 256 CUs several times over
    return (int)(blocks < 1 ? 1 : (blocks > cap ? cap : blocks));
}

// ------------------------------------------------------------ dispatch

template <class DT, int VEC>
hipError_t fwd_launch(const Problem &p, const Mapping &mp, const void *value, const void *loc,
                      const void *attn, void *out, hipStream_t stream) {
    using E = typename DT::S;
    const int qpb = kBlock >> (mp.log2_group + mp.log2_split);
    const int qblocks = (int)((p.Q + qpb - 1) / qpb);
    const int64_t ntiles = p.B * p.M * qblocks;
    const int64_t per_xcd = (ntiles + kXcds - 1) / kXcds;
    hipLaunchKernelGGL((msda_fwd_kernel<DT, VEC>), dim3((unsigned)(per_xcd * kXcds)),
                       dim3(kBlock), 0, stream, static_cast<const E *>(value),
                       static_cast<const E *>(loc), static_cast<const E *>(attn),
                       static_cast<E *>(out), p.levels, p.S, p.Q, (int)p.M, (int)p.D, (int)p.L,
                       (int)p.K, qblocks, ntiles, mp.log2_group, mp.log2_split);
    return hipGetLastError();
}

template <class DT, int VEC, bool FP32ACC>
hipError_t bwd_launch(const Problem &p, const Mapping &mp, const void *value, const void *loc,
                      const void *attn, const void *grad_out, void *acc_target, void *grad_loc,
                      void *grad_attn, hipStream_t stream) {
    using E = typename DT::S;
    const int qpb = kBlock >> (mp.log2_group + mp.log2_split);
    const int qblocks = (int)((p.Q + qpb - 1) / qpb);
    const int64_t ntiles = p.B * p.M * qblocks;
    const int64_t per_xcd = (ntiles + kXcds - 1) / kXcds;
    hipLaunchKernelGGL((msda_bwd_kernel<DT, VEC, FP32ACC>), dim3((unsigned)(per_xcd * kXcds)),
                       dim3(kBlock), 0, stream, static_cast<const E *>(value),
                       static_cast<const E *>(loc), static_cast<const E *>(attn),
                       static_cast<const E *>(grad_out), acc_target, static_cast<E *>(grad_loc),
                       static_cast<E *>(grad_attn), p.levels, p.S, p.Q, (int)p.M, (int)p.D,
                       (int)p.L, (int)p.K, qblocks, ntiles, mp.log2_group, mp.log2_split);
    return hipGetLastError();
}

template <class DT>
hipError_t fwd_by_vec(const Problem &p, const Mapping &mp, const void *v, const void *l,
                      const void *a, void *o, hipStream_t st) {
    switch (mp.vec) {
        case 1: return fwd_launch<DT, 1>(p, mp, v, l, a, o, st);
        case 2: return fwd_launch<DT, 2>(p, mp, v, l, a, o, st);
        case 4: return fwd_launch<DT, 4>(p, mp, v, l, a, o, st);
        default: break;
    }
    if constexpr (sizeof(typename DT::S) == 4) {
        if (mp.vec == 3) return fwd_launch<DT, 3>(p, mp, v, l, a, o, st);
    } else {
        if (mp.vec == 8) return fwd_launch<DT, 8>(p, mp, v, l, a, o, st);
    }
    return hipErrorInvalidValue;
}

template <class DT, bool FP32ACC>
hipError_t bwd_by_vec(const Problem &p, const Mapping &mp, const void *v, const void *l,
                      const void *a, const void *go, void *t, void *gl, void *ga,
                      hipStream_t st) {
    switch (mp.vec) {
        case 1: return bwd_launch<DT, 1, FP32ACC>(p, mp, v, l, a, go, t, gl, ga, st);
        case 2: return bwd_launch<DT, 2, FP32ACC>(p, mp, v, l, a, go, t, gl, ga, st);
        case 4: return bwd_launch<DT, 4, FP32ACC>(p, mp, v, l, a, go, t, gl, ga, st);
        default: break;
    }
    if constexpr (sizeof(typename DT::S) == 4) {
        if (mp.vec == 3) return bwd_launch<DT, 3, FP32ACC>(p, mp, v, l, a, go, t, gl, ga, st);
    } else {
        if (mp.vec == 8) return bwd_launch<DT, 8, FP32ACC>(p, mp, v, l, a, go, t, gl, ga, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_forward(const Problem &p, const Mapping &mp, const void *value,
                          const void *loc, const void *attn, void *out, hipStream_t stream) {
    switch (p.dtype) {
        case MSDA_F32: return fwd_by_vec<F32T>(p, mp, value, loc, attn, out, stream);
        case MSDA_F16: return fwd_by_vec<F16T>(p, mp, value, loc, attn, out, stream);
        case MSDA_BF16: return fwd_by_vec<BF16T>(p, mp, value, loc, attn, out, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_backward(const Problem &p, const Mapping &mp, const void *value,
                           const void *loc, const void *attn, const void *grad_out,
                           void *acc_target, bool accum_fp32, void *grad_loc, void *grad_attn,
                           hipStream_t stream) {
    switch (p.dtype) {
        case MSDA_F32:
            return bwd_by_vec<F32T, true>(p, mp, value, loc, attn, grad_out, acc_target, grad_loc,
                                          grad_attn, stream);
        case MSDA_F16:
            return accum_fp32 ? bwd_by_vec<F16T, true>(p, mp, value, loc, attn, grad_out,
                                                       acc_target, grad_loc, grad_attn, stream)
                              : bwd_by_vec<F16T, false>(p, mp, value, loc, attn, grad_out,
                                                        acc_target, grad_loc, grad_attn, stream);
        case MSDA_BF16:
            return accum_fp32 ? bwd_by_vec<BF16T, true>(p, mp, value, loc, attn, grad_out,
                                                        acc_target, grad_loc, grad_attn, stream)
                              : bwd_by_vec<BF16T, false>(p, mp, value, loc, attn, grad_out,
                                                         acc_target, grad_loc, grad_attn, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_zero(void *dst, size_t bytes, hipStream_t stream) {
    if (bytes == 0) return hipSuccess;
    if ((reinterpret_cast<uintptr_t>(dst) % 16 == 0) && (bytes % 16 == 0)) {
        const int64_t n16 = (int64_t)(bytes / 16);
        hipLaunchKernelGGL(zero_kernel_16, dim3(grid_for(n16)), dim3(kBlock), 0, stream,
                           static_cast<uint4 *>(dst), n16);
    } else {
        const int64_t n2 = (int64_t)(bytes / 2);
        hipLaunchKernelGGL(zero_kernel_2, dim3(grid_for(n2)), dim3(kBlock), 0, stream,
                           static_cast<uint16_t *>(dst), n2);
    }
    return hipGetLastError();
}

hipError_t launch_downcast(int dtype, const float *scratch, void *grad_value, int64_t n,
                           bool accumulate, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const bool x4 = (n % 4 == 0) && (reinterpret_cast<uintptr_t>(scratch) % 16 == 0) &&
                    (reinterpret_cast<uintptr_t>(grad_value) % 8 == 0);
    if (dtype == MSDA_F16) {
        if (x4)
            hipLaunchKernelGGL(downcast_kernel_x4<F16T>, dim3(grid_for(n / 4)), dim3(kBlock), 0,
                               stream, reinterpret_cast<const float4 *>(scratch),
                               static_cast<uint2 *>(grad_value), n / 4, (int)accumulate);
        else
            hipLaunchKernelGGL(downcast_kernel<F16T>, dim3(grid_for(n)), dim3(kBlock), 0, stream,
                               scratch, static_cast<uint16_t *>(grad_value), n, (int)accumulate);
    } else if (dtype == MSDA_BF16) {
        if (x4)
            hipLaunchKernelGGL(downcast_kernel_x4<BF16T>, dim3(grid_for(n / 4)), dim3(kBlock), 0,
                               stream, reinterpret_cast<const float4 *>(scratch),
                               static_cast<uint2 *>(grad_value), n / 4, (int)accumulate);
        else
            hipLaunchKernelGGL(downcast_kernel<BF16T>, dim3(grid_for(n)), dim3(kBlock), 0, stream,
                               scratch, static_cast<uint16_t *>(grad_value), n, (int)accumulate);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace msda
