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

#include <algorithm>
#include <type_traits>

#include "msda_device.h"
#include "msda_launch.h"

namespace msda {
namespace {

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

// Pin a value in a register at this point of the program: every load it
// depends on must be issued before here. Used after a chunk's parameter
// loads so that the compiler cannot sink them next to their first use,
// which would put one memory round trip per point on the critical path.
__device__ __forceinline__ void pin(uint32_t &v) { asm volatile("" : "+v"(v)::"memory"); }

// ------------------------------------------------------------- gathers
//
// Corner rows are read through a raw buffer resource covering one batch's
// value slice: an offset outside the slice reads as zero and moves no data,
// so an out-of-bounds corner needs no branch (a branch around a load makes
// the compiler wait for that load before the branch joins, which would
// serialise the gathers). Slices above 2 GiB use plain loads from a clamped
// address followed by a select.

constexpr uint32_t kOutOfRange = 0x80000000u;  // >= every buffer size used
constexpr int kRawBufferConfig = 0x00020000;  // gfx9-family raw buffer descriptor word 3

template <int BYTES>
__device__ __forceinline__ typename RawVec<BYTES>::type buffer_load_raw(__amdgpu_buffer_rsrc_t r,
                                                                         uint32_t off);
template <>
__device__ __forceinline__ uint16_t buffer_load_raw<2>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
template <>
__device__ __forceinline__ uint32_t buffer_load_raw<4>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
template <>
__device__ __forceinline__ uint2 buffer_load_raw<8>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
template <>
__device__ __forceinline__ U32x3 buffer_load_raw<12>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0);
    return U32x3{v[0], v[1], v[2]};
}
template <>
__device__ __forceinline__ uint4 buffer_load_raw<16>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <class R>
__device__ __forceinline__ R zero_raw() {
    R r;
    __builtin_memset(&r, 0, sizeof(R));
    return r;
}

// One batch's value slice: `base` in bytes and, for BUF, its buffer resource.
template <bool BUF>
struct Slice {
    const char *base;
    __amdgpu_buffer_rsrc_t rsrc;

    __device__ __forceinline__ Slice(const void *p, int64_t bytes) : base((const char *)p) {
        if constexpr (BUF)
            rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes,
                                                     kRawBufferConfig);
    }

    // sizeof(R) bytes at byte offset `off`; zero when !ok.
    template <class R>
    __device__ __forceinline__ R gather(int64_t off, bool ok) const {
        if constexpr (BUF) {
            return buffer_load_raw<(int)sizeof(R)>(rsrc, ok ? (uint32_t)off : kOutOfRange);
        } else {
            const R v = *reinterpret_cast<const R *>(base + (ok ? off : 0));
            return ok ? v : zero_raw<R>();
        }
    }
};

template <class DT, int N, class R>
__device__ __forceinline__ void raw_to_f32(const R &r, float (&out)[N]) {
    typename DT::S e[N];
    __builtin_memcpy(e, &r, sizeof(R));
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = to_f32(DT{}, e[i]);
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// acc + sum over the N channels a lane holds of g[i] * v[i], with `graw` /
// `vraw` the raw channels and `g` the upstream gradient in fp32. 16-bit data
// with whole channel pairs uses the two-channel dot-product instructions
// (v_dot2c_f32_f16 / _bf16: no conversions, products exact in fp32); other
// data converts and multiply-adds.
template <class DT, int N, class R>
__device__ __forceinline__ float lane_dot(const R &graw, const float (&g)[N], const R &vraw,
                                          float acc) {
    if constexpr (sizeof(typename DT::S) == 2 && N % 2 == 0) {
        uint32_t gw[N / 2], vw[N / 2];
        __builtin_memcpy(gw, &graw, sizeof(R));
        __builtin_memcpy(vw, &vraw, sizeof(R));
#pragma unroll
        for (int p = 0; p < N / 2; ++p) {
            if constexpr (std::is_same<DT, F16T>::value)
                acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, gw[p]),
                                             __builtin_bit_cast(f16x2_t, vw[p]), acc, false);
            else
                acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, gw[p]),
                                                      __builtin_bit_cast(bf16x2_t, vw[p]), acc,
                                                      false);
        }
    } else {
        float v[N];
        raw_to_f32<DT, N>(vraw, v);
#pragma unroll
        for (int i = 0; i < N; ++i) acc = __builtin_fmaf(g[i], v[i], acc);
    }
    return acc;
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

// Lane t's value in every lane of its quad (DPP quad_perm [t, t, t, t]).
template <int T>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, T * 0x55, 0xF, 0xF, true);
}
template <int T>
__device__ __forceinline__ float quad_bcast(float v) {
    return __uint_as_float(quad_bcast<T>(__float_as_uint(v)));
}

// -------------------------------------------------------------- atomics

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

// ------------------------------------------------------------ utilities

// A point's contributions to grad_attn (before A) and to grad_loc (before
// A * W, A * H) from the dot products d[cn] of its corner rows 00, 01, 10, 11
// with the upstream gradient: the bilinear sample and the sample's slopes
// along x and y (course page "5. The backward kernel", section "What the
// backward pass must produce", items 1 and 2).
__device__ __forceinline__ void point_sums(const float (&d)[4], float fx, float fy, float &ds,
                                           float &dx, float &dy) {
    const float gx = 1.0f - fx, gy = 1.0f - fy;
    ds = gx * gy * d[0] + fx * gy * d[1] + gx * fy * d[2] + fx * fy * d[3];
    dx = gy * (d[1] - d[0]) + fy * (d[3] - d[2]);
    dy = gx * (d[2] - d[0]) + fx * (d[3] - d[1]);
}


// Order of the query tiles of the forward and gradient kernels.
//
// Linear (nc == 0): tile = (b, head group, block of qs consecutive queries),
// query block fastest; XCD x takes a contiguous range of tiles, i.e. whole
// (b, head group) pairs when there are at least 8 of them.
//
// Column groups (nc > 1), for pixel queries when there are fewer (b, head
// group) pairs than XCDs: when the queries are the pyramid's own pixels in S
// order (Q == S and the levels tile [0, S) without overlap, as in a
// deformable-attention encoder), every query samples near its own pixel, and
// a linear range of queries is a few full-width rows whose sampled
// neighbourhoods, for 4 heads of 64-byte rows, exceed one XCD's 4 MB L2. The
// pixels of every level are then cut into nc column groups, and region
// (b, head group, column group) takes per_region consecutive logical tiles
// (one region per XCD): its column group of level 0 row by row, then level
// 1's, and so on, each row's part cut into tiles of qs = 2^log2qs queries
// (the last one ragged; the tail of a smaller region is empty). Any order
// gives the same results: only the assignment of queries to workgroups
// changes. All tile arithmetic is 32-bit (the host checks the ranges).
struct TileOrder {
    int32_t nc;          // column groups (0: linear order)
    int32_t per_region;  // logical tiles per region
};

struct TileQueries {
    int64_t b;   // batch
    int hg;      // head group
    int64_t q0;  // first query of the tile
    int qn;      // queries in the tile (<= qs)
};

// Columns [x0, x1) of column group c of a level of width W, and its tiles per row.
__host__ __device__ __forceinline__ uint32_t group_columns(uint32_t W, uint32_t c, uint32_t nc,
                                                          int log2qs, uint32_t *x0,
                                                          uint32_t *x1) {
    *x0 = (c * W) / nc;
    *x1 = ((c + 1) * W) / nc;
    return (*x1 - *x0 + (1u << log2qs) - 1) >> log2qs;
}

// The queries of logical tile `tile`; false for an empty tile (the padded
// tail of a region). Uniform over the workgroup.
__device__ __forceinline__ bool tile_queries(int64_t tile, const TileOrder &to,
                                             const LevelTable &lt, int L, int64_t Q, int log2qs,
                                             int ngroups, int qblocks, TileQueries &tq) {
    const int qs = 1 << log2qs;
    if (to.nc == 0) {
        const int64_t bg = tile / qblocks;
        const int qb = (int)(tile - bg * qblocks);
        tq.b = bg / ngroups;
        tq.hg = (int)(bg - tq.b * ngroups);
        tq.q0 = (int64_t)qb * qs;
        tq.qn = (int)(Q - tq.q0 < qs ? Q - tq.q0 : qs);
        return true;
    }
    const uint32_t t32 = (uint32_t)tile, per = (uint32_t)to.per_region, nc = (uint32_t)to.nc;
    const uint32_t region = t32 / per;
    uint32_t idx = t32 - region * per;
    const uint32_t c = region % nc, bg = region / nc;
    tq.b = bg / (uint32_t)ngroups;
    tq.hg = (int)(bg - (uint32_t)tq.b * (uint32_t)ngroups);
    for (int l = 0; l < L; ++l) {
        uint32_t x0, x1;
        const uint32_t tpr = group_columns((uint32_t)lt.W[l], c, nc, log2qs, &x0, &x1);
        const uint32_t n = (uint32_t)lt.H[l] * tpr;
        if (idx < n) {
            const uint32_t row = idx / tpr;
            const uint32_t xs = x0 + ((idx - row * tpr) << log2qs);
            tq.q0 = lt.start[l] + (int64_t)row * lt.W[l] + xs;
            tq.qn = (int)(x1 - xs < (uint32_t)qs ? x1 - xs : (uint32_t)qs);
            return true;
        }
        idx -= n;
    }
    return false;  // the padded tail of the region
}

// ------------------------------------------------------------- forward
//
// A lane group handles the points p = i * split + s (i = 0, 1, ...) of its
// query; split divides K, so the level of the i-th point, (i * split) / K, is
// the same for every lane of the wave and the level table is read with
// scalar loads. Points are taken CH at a time: the locations and weights of
// the chunk are loaded first, then all 4 * CH corner gathers are issued, and
// only then consumed, so a wave waits for two memory round trips per chunk
// instead of two per point.

// Heads per workgroup of the forward and gradients-only kernels: the query
// slots of a workgroup hold HG heads of each of its queries, head fastest,
// so that one store instruction writes a query's results for HG neighbouring
// heads, which share memory lines (one head per workgroup would leave each
// line to be filled by workgroups on different XCDs, written back in parts),
// and heads that sample near the same pixels share L1 / L2 lines. The
// largest of 4, 2, 1 that divides M and is at most the slots per workgroup.
__host__ __device__ inline int grad_heads(int M, int slots) {
    return (M % 4 == 0 && slots >= 4) ? 4 : (M % 2 == 0 && slots >= 2) ? 2 : 1;
}

// The forward groups heads only for rows of at most 64 bytes (measured: the
// encoder workloads' forward 204 -> 177 us and 2147 -> 1794 us with 64-byte
// rows, the odd-head workload's 192-byte fp32 rows 52 -> 57 us).
__host__ __device__ inline int fwd_heads(int M, int slots, int row_bytes) {
    return row_bytes <= 64 ? grad_heads(M, slots) : 1;
}

template <class DT, class PT, int VEC, int CH, bool BUF, bool QUAD>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 4))) void msda_fwd_kernel(
    const typename DT::S *__restrict__ value, const typename PT::S *__restrict__ loc,
    const typename PT::S *__restrict__ attn, typename DT::S *__restrict__ out,
    const LevelTable lt, const int64_t S, const int64_t Q, const int M, const int D,
    const int L, const int K, const int qblocks, const int64_t ntiles, const int log2g,
    const int log2s, const TileOrder to, const bool pvec) {
    using E = typename DT::S;
    using R = typename RawVec<VEC * (int)sizeof(E)>::type;
    const int64_t tile = logical_block();
    if (tile >= ntiles) return;  // whole workgroup leaves together
    const int tid = threadIdx.x;
    const int c = tid & ((1 << log2g) - 1);
    const int s = (tid >> log2g) & ((1 << log2s) - 1);
    const int qpb = kBlock >> (log2g + log2s);  // query slots
    const int HG = fwd_heads(M, qpb, D * (int)sizeof(E));
    const int slot = tid >> (log2g + log2s);
    TileQueries tq;
    const int log2qs = 8 - log2g - log2s - (HG == 4 ? 2 : HG == 2 ? 1 : 0);  // queries per tile
    if (!tile_queries(tile, to, lt, L, Q, log2qs, M / HG, qblocks, tq)) return;
    const int64_t b = tq.b;
    const int m = tq.hg * HG + slot % HG;
    const int64_t q = tq.q0 + slot / HG;
    const bool q_ok = slot / HG < tq.qn;
    const int c0 = c * VEC;
    const bool live = q_ok && (c0 < D);
    const int split = 1 << log2s;
    const int LK = L * K;
    const int per_lane = LK >> log2s;

    const int64_t pq = (b * Q + (q_ok ? q : 0)) * M + m;  // clamped: always a valid query
    const typename PT::S *loc_q = loc + pq * LK * 2;
    const typename PT::S *attn_q = attn + pq * LK;
    const int64_t MD = (int64_t)M * D;
    const int64_t row_bytes = MD * (int64_t)sizeof(E);
    const Slice<BUF> slice(value + b * S * MD, S * row_bytes);
    const int64_t lane_bytes = ((int64_t)m * D + (c0 < D ? c0 : 0)) * (int64_t)sizeof(E);

    float acc[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc[i] = 0.0f;

    // chunk k's parameters live in lane k of the group (at most G chunks)
    const bool owned = per_lane <= (CH << log2g);
    ChunkParams<PT, CH> own;
    if (owned) own_chunk_params<PT, CH>(loc_q, attn_q, c, per_lane, split, s, pvec, own);
    const int group_base = (tid & 63) & ~((1 << log2g) - 1);

    // QUAD (4-lane groups that hold exactly D channels, chunks inside one
    // level, parameters owned, buffer gathers; chosen on the host): lane k of
    // a group works out point k of the chunk (cell, weights, corner offsets,
    // out-of-range for out-of-bounds corners) and the quad broadcasts each
    // point's 8 values, instead of every lane working out all CH points (the
    // same arithmetic, so the same results).
    static_assert(!QUAD || (BUF && CH == 4), "quad setup: buffer gathers, 4-point chunks");
    // QUAD: 32-bit offsets, kOutOfRange for out-of-bounds corners (ok unused)
    using Off = typename std::conditional<QUAD, uint32_t, int64_t>::type;
    for (int i0 = 0; i0 < per_lane; i0 += CH) {
        Off off[CH][4];
        bool ok[CH][4];
        float w[CH][4];
        if constexpr (QUAD) {
            float px, py, pa;
            point_params<PT, CH>(own, group_base + i0 / CH, c, px, py, pa);
            const bool p_live = live && (i0 + c < per_lane);
            const float a = (q_ok && i0 + c < per_lane) ? pa : 0.0f;
            int l = (i0 * split) / K;  // the chunk's level
            l = l < L ? l : L - 1;
            const int H = lt.H[l], W = lt.W[l];
            const Cell cl = map_cell(px, py, (float)H, (float)W, W, lt.start[l]);
            // 32-bit offsets without the lane's channels (the slice is buffer-addressable)
            const uint32_t rb = (uint32_t)row_bytes;
            const uint32_t o00 = (uint32_t)cl.row00 * rb, o10 = o00 + (uint32_t)W * rb;
            uint32_t po[4] = {p_live && cl.v00 ? o00 : kOutOfRange,
                              p_live && cl.v01 ? o00 + rb : kOutOfRange,
                              p_live && cl.v10 ? o10 : kOutOfRange,
                              p_live && cl.v11 ? o10 + rb : kOutOfRange};
            const float gx = 1.0f - cl.fx, gy = 1.0f - cl.fy;
            float pw[4] = {a * (gx * gy), a * (cl.fx * gy), a * (gx * cl.fy), a * (cl.fx * cl.fy)};
            auto take = [&](auto tc) {
                constexpr int T = decltype(tc)::value;
#pragma unroll
                for (int cn = 0; cn < 4; ++cn) {
                    // kOutOfRange plus the lane's bytes is still past the slice
                    off[T][cn] = quad_bcast<T>(po[cn]) + (uint32_t)lane_bytes;
                    w[T][cn] = quad_bcast<T>(pw[cn]);
                }
            };
            take(std::integral_constant<int, 0>{});
            take(std::integral_constant<int, 1>{});
            take(std::integral_constant<int, 2>{});
            take(std::integral_constant<int, 3>{});
        } else {
        float lx[CH], ly[CH], aw[CH];
        if (owned) {
            chunk_params<PT, CH>(own, group_base + i0 / CH, lx, ly, aw);
        } else {
            uint32_t bx[CH], by[CH], ba[CH];
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                const int p = (i0 + t < per_lane ? i0 + t : 0) * split + s;
                bx[t] = load_bits<PT>(loc_q + 2 * p);
                by[t] = load_bits<PT>(loc_q + 2 * p + 1);
                ba[t] = load_bits<PT>(attn_q + p);
            }
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                pin(bx[t]);
                pin(by[t]);
                pin(ba[t]);
            }
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                lx[t] = bits_to_f32<PT>(bx[t]);
                ly[t] = bits_to_f32<PT>(by[t]);
                aw[t] = bits_to_f32<PT>(ba[t]);
            }
        }
#pragma unroll
        for (int t = 0; t < CH; ++t) aw[t] = (q_ok && i0 + t < per_lane) ? aw[t] : 0.0f;
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            const bool t_live = live && (i0 + t < per_lane);
            int l = ((i0 + t) * split) / K;
            l = l < L ? l : L - 1;
            const int H = lt.H[l], W = lt.W[l];
            const Cell cl = map_cell(lx[t], ly[t], (float)H, (float)W, W, lt.start[l]);
            off[t][0] = cl.row00 * row_bytes + lane_bytes;
            off[t][1] = off[t][0] + row_bytes;
            off[t][2] = off[t][0] + (int64_t)W * row_bytes;
            off[t][3] = off[t][2] + row_bytes;
            ok[t][0] = t_live && cl.v00;
            ok[t][1] = t_live && cl.v01;
            ok[t][2] = t_live && cl.v10;
            ok[t][3] = t_live && cl.v11;
            const float gx = 1.0f - cl.fx, gy = 1.0f - cl.fy;
            w[t][0] = aw[t] * (gx * gy);
            w[t][1] = aw[t] * (cl.fx * gy);
            w[t][2] = aw[t] * (gx * cl.fy);
            w[t][3] = aw[t] * (cl.fx * cl.fy);
        }
        }
        __builtin_amdgcn_sched_barrier(0);
        R raw[CH][4];
#pragma unroll
        for (int t = 0; t < CH; ++t)
#pragma unroll
            for (int cn = 0; cn < 4; ++cn) {
                if constexpr (QUAD)
                    raw[t][cn] = buffer_load_raw<(int)sizeof(R)>(slice.rsrc, off[t][cn]);
                else
                    raw[t][cn] = slice.template gather<R>(off[t][cn], ok[t][cn]);
            }
        __builtin_amdgcn_sched_barrier(0);  // all 4 * CH gathers in flight before any use
#pragma unroll
        for (int t = 0; t < CH; ++t) {
#pragma unroll
            for (int cn = 0; cn < 4; ++cn) {
                float v[VEC];
                raw_to_f32<DT, VEC>(raw[t][cn], v);
#pragma unroll
                for (int i = 0; i < VEC; ++i) acc[i] += w[t][cn] * v[i];
            }
        }
    }
    // Sum the split lane groups of one query (all lanes active here).
    for (int off = 1 << log2g; off < (1 << (log2g + log2s)); off <<= 1) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[i] += __shfl_xor(acc[i], off);
    }
    if (live && s == 0) store_vec<DT, VEC>(out + pq * D + c0, acc);
}

// ------------------------------------------------ point-parallel foil
//
// The decomposition the forward page sets against its own (course page "4.
// The forward kernel, line by line", section "The design question: what does
// one program own?"): one thread per sampling point (b, q, m, l, k), points
// in their memory order, so neighbouring lanes sample unrelated locations and
// each lane reads its four corner rows alone (VEC channels per load, no
// coalescing across lanes). A workgroup holds the points of kBlock / (L*K)
// whole queries; each thread's D partial sums go through LDS and are added
// per query and channel. Kept for measurement only (occupancy versus
// bandwidth); the product forward is msda_fwd_kernel.
template <class DT, int VEC, int MAXD>
__global__ __launch_bounds__(kBlock) void msda_foil_kernel(
    const typename DT::S *__restrict__ value, const typename DT::S *__restrict__ loc,
    const typename DT::S *__restrict__ attn, typename DT::S *__restrict__ out,
    const LevelTable lt, const int64_t S, const int64_t Q, const int M, const int D,
    const int L, const int K, const int64_t P) {
    using E = typename DT::S;
    extern __shared__ float part[];  // kBlock x D
    const int tid = threadIdx.x;
    const int LK = L * K;
    const int64_t pt = (int64_t)blockIdx.x * kBlock + tid;
    const bool ok = pt < P;
    const int64_t pc = ok ? pt : 0;
    const int64_t bqm = pc / LK;
    const int pp = (int)(pc - bqm * LK);
    const int l = pp / K;
    const int64_t b = bqm / (Q * M);
    const int m = (int)(bqm % M);
    const int W = lt.W[l];
    const Cell cl = map_cell(to_f32(DT{}, loc[2 * pc]), to_f32(DT{}, loc[2 * pc + 1]),
                             (float)lt.H[l], (float)W, W, lt.start[l]);
    const float a = ok ? to_f32(DT{}, attn[pc]) : 0.0f;
    const float gx = 1.0f - cl.fx, gy = 1.0f - cl.fy;
    const float w[4] = {a * gx * gy, a * cl.fx * gy, a * gx * cl.fy, a * cl.fx * cl.fy};
    const bool vc[4] = {ok && cl.v00, ok && cl.v01, ok && cl.v10, ok && cl.v11};
    const int64_t MD = (int64_t)M * D;
    const E *rows[4];
    const int64_t r00 = cl.row00;
    const int64_t drow[4] = {0, 1, W, (int64_t)W + 1};
#pragma unroll
    for (int cn = 0; cn < 4; ++cn)
        rows[cn] = value + ((b * S + (vc[cn] ? r00 + drow[cn] : 0)) * MD + (int64_t)m * D);
    float acc[MAXD];
#pragma unroll
    for (int d = 0; d < MAXD; ++d) acc[d] = 0.0f;
#pragma unroll
    for (int d0 = 0; d0 < MAXD; d0 += VEC) {
        if (d0 < D) {
#pragma unroll
            for (int cn = 0; cn < 4; ++cn) {
                if (!vc[cn]) continue;
                float v[VEC];
                load_vec<DT, VEC>(rows[cn] + d0, v);
#pragma unroll
                for (int i = 0; i < VEC; ++i) acc[d0 + i] += w[cn] * v[i];
            }
        }
    }
#pragma unroll
    for (int d = 0; d < MAXD; ++d)
        if (d < D) part[tid * D + d] = acc[d];
    __syncthreads();
    const int qpw = kBlock / LK;
    const int64_t bqm0 = (int64_t)blockIdx.x * qpw;
    const int64_t nq = P / LK;
    for (int i = tid; i < qpw * D; i += kBlock) {
        const int j = i / D, d = i - j * D;
        if (bqm0 + j >= nq) continue;
        float sum = 0.0f;
        for (int t = 0; t < LK; ++t) sum += part[(j * LK + t) * D + d];
        out[(bqm0 + j) * D + d] = from_f32(DT{}, sum);
    }
}

// ------------------------------------------------- backward, gradients only
//
// grad_attention_weights and grad_sampling_locations when no level's
// grad_value needs atomics (every level binned): the forward's lane layout
// (VEC consecutive channels per lane, 16-byte gathers) with the query's
// upstream gradient held in the same layout. Per point the lane forms its
// share of g . s, g . ds/dx and g . ds/dy (course page "5. The backward
// kernel", section "What the backward pass must produce"); the group's
// shares are summed with DPP moves and lane c stores point t0 + c of the
// chunk, so a group writes consecutive points with one instruction.
#define MSDA_GRAD_PARAMS                                                                      \
    const typename DT::S *__restrict__ value, const typename PT::S *__restrict__ loc,         \
        const typename PT::S *__restrict__ attn, const typename DT::S *__restrict__ grad_out, \
        typename PT::S *__restrict__ grad_loc, typename PT::S *__restrict__ grad_attn,        \
        const LevelTable &lt, const int64_t S, const int64_t Q, const int M, const int D,     \
        const int L, const int K, const int qblocks, const int log2g, const int log2s,        \
        const TileOrder &to, const bool pvec
#define MSDA_GRAD_ARGS value, loc, attn, grad_out, grad_loc, grad_attn, lt, S, Q, M, D, L, K, \
                       qblocks, log2g, log2s, to, pvec

template <class DT, class PT, int VEC, int CH, bool BUF, bool QUAD = false>
__device__ __forceinline__ void grad_tile(MSDA_GRAD_PARAMS, const int64_t tile) {
    using E = typename DT::S;
    using R = typename RawVec<VEC * (int)sizeof(E)>::type;
    const int tid = threadIdx.x;
    const int G = 1 << log2g;
    const int c = tid & (G - 1);
    const int s = (tid >> log2g) & ((1 << log2s) - 1);
    const int qpb = kBlock >> (log2g + log2s);  // query slots
    const int HG = grad_heads(M, qpb);
    const int slot = tid >> (log2g + log2s);
    TileQueries tq;
    const int log2qs = 8 - log2g - log2s - (HG == 4 ? 2 : HG == 2 ? 1 : 0);  // queries per tile
    if (!tile_queries(tile, to, lt, L, Q, log2qs, M / HG, qblocks, tq)) return;
    const int64_t b = tq.b;
    const int m = tq.hg * HG + slot % HG;
    const int64_t q = tq.q0 + slot / HG;
    const bool q_ok = slot / HG < tq.qn;
    const int c0 = c * VEC;
    const bool live = q_ok && (c0 < D);
    const int split = 1 << log2s;
    const int LK = L * K;
    const int per_lane = LK >> log2s;

    const int64_t pq = (b * Q + (q_ok ? q : 0)) * M + m;  // clamped: always a valid query
    const typename PT::S *loc_q = loc + pq * LK * 2;
    const typename PT::S *attn_q = attn + pq * LK;
    const int64_t MD = (int64_t)M * D;
    const int64_t row_bytes = MD * (int64_t)sizeof(E);
    const Slice<BUF> slice(value + b * S * MD, S * row_bytes);
    const int64_t lane_bytes = ((int64_t)m * D + (c0 < D ? c0 : 0)) * (int64_t)sizeof(E);
    float g[VEC];
    R graw;
    {
        const R r = *reinterpret_cast<const R *>(grad_out + pq * D + (c0 < D ? c0 : 0));
        graw = live ? r : zero_raw<R>();
        raw_to_f32<DT, VEC>(graw, g);
    }

    // chunk k's parameters live in lane k of the group (at most G chunks)
    const bool owned = per_lane <= (CH << log2g);
    ChunkParams<PT, CH> own;
    if (owned) own_chunk_params<PT, CH>(loc_q, attn_q, c, per_lane, split, s, pvec, own);
    const int group_base = (tid & 63) & ~(G - 1);

    // QUAD: as in the forward, lane k of a 4-lane group works out point k of
    // the chunk and the quad broadcasts its corner offsets; its fractions and
    // slope scales stay in lane k, which sums and stores point k
    static_assert(!QUAD || (BUF && CH == 4), "quad setup: buffer gathers, 4-point chunks");
    using Off = typename std::conditional<QUAD, uint32_t, int64_t>::type;
    for (int i0 = 0; i0 < per_lane; i0 += CH) {
        Off off[CH][4];
        bool ok[CH][4];
        float fx[CH], fy[CH], sw[CH], sh[CH];
        float fx_own = 0.0f, fy_own = 0.0f;  // QUAD: lane k's own point's fractions
        if constexpr (QUAD) {
            float px, py, pa;
            point_params<PT, CH>(own, group_base + i0 / CH, c, px, py, pa);
            const bool p_live = live && (i0 + c < per_lane);
            const float aw = (q_ok && i0 + c < per_lane) ? pa : 0.0f;
            int l = (i0 * split) / K;  // the chunk's level
            l = l < L ? l : L - 1;
            const int H = lt.H[l], W = lt.W[l];
            sw[0] = (float)W * aw;  // lane k's own point's scales
            sh[0] = (float)H * aw;
            const Cell cl = map_cell(px, py, (float)H, (float)W, W, lt.start[l]);
            fx_own = cl.fx;
            fy_own = cl.fy;
            const uint32_t rb = (uint32_t)row_bytes;
            const uint32_t o00 = (uint32_t)cl.row00 * rb, o10 = o00 + (uint32_t)W * rb;
            const uint32_t po[4] = {p_live && cl.v00 ? o00 : kOutOfRange,
                                    p_live && cl.v01 ? o00 + rb : kOutOfRange,
                                    p_live && cl.v10 ? o10 : kOutOfRange,
                                    p_live && cl.v11 ? o10 + rb : kOutOfRange};
            auto take = [&](auto tc) {
                constexpr int T = decltype(tc)::value;
#pragma unroll
                for (int cn = 0; cn < 4; ++cn)
                    off[T][cn] = quad_bcast<T>(po[cn]) + (uint32_t)lane_bytes;
            };
            take(std::integral_constant<int, 0>{});
            take(std::integral_constant<int, 1>{});
            take(std::integral_constant<int, 2>{});
            take(std::integral_constant<int, 3>{});
        } else {
        float lx[CH], ly[CH], la[CH];
        if (owned) {
            chunk_params<PT, CH>(own, group_base + i0 / CH, lx, ly, la);
        } else {
            uint32_t bx[CH], by[CH], ba[CH];
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                const int p = (i0 + t < per_lane ? i0 + t : 0) * split + s;
                bx[t] = load_bits<PT>(loc_q + 2 * p);
                by[t] = load_bits<PT>(loc_q + 2 * p + 1);
                ba[t] = load_bits<PT>(attn_q + p);
            }
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                pin(bx[t]);
                pin(by[t]);
                pin(ba[t]);
            }
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                lx[t] = bits_to_f32<PT>(bx[t]);
                ly[t] = bits_to_f32<PT>(by[t]);
                la[t] = bits_to_f32<PT>(ba[t]);
            }
        }
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            const bool t_live = live && (i0 + t < per_lane);
            int l = ((i0 + t) * split) / K;
            l = l < L ? l : L - 1;
            const int H = lt.H[l], W = lt.W[l];
            const float aw = (q_ok && i0 + t < per_lane) ? la[t] : 0.0f;
            sw[t] = (float)W * aw;
            sh[t] = (float)H * aw;
            const Cell cl = map_cell(lx[t], ly[t], (float)H, (float)W, W, lt.start[l]);
            fx[t] = cl.fx;
            fy[t] = cl.fy;
            off[t][0] = cl.row00 * row_bytes + lane_bytes;
            off[t][1] = off[t][0] + row_bytes;
            off[t][2] = off[t][0] + (int64_t)W * row_bytes;
            off[t][3] = off[t][2] + row_bytes;
            ok[t][0] = t_live && cl.v00;
            ok[t][1] = t_live && cl.v01;
            ok[t][2] = t_live && cl.v10;
            ok[t][3] = t_live && cl.v11;
        }
        }
        __builtin_amdgcn_sched_barrier(0);
        R raw[CH][4];
#pragma unroll
        for (int t = 0; t < CH; ++t)
#pragma unroll
            for (int cn = 0; cn < 4; ++cn) {
                if constexpr (QUAD)
                    raw[t][cn] = buffer_load_raw<(int)sizeof(R)>(slice.rsrc, off[t][cn]);
                else
                    raw[t][cn] = slice.template gather<R>(off[t][cn], ok[t][cn]);
            }
        __builtin_amdgcn_sched_barrier(0);  // all 4 * CH gathers in flight before any use
        // The sample and its two slopes are linear in the corner rows, so
        // their dot products with the upstream gradient follow from the four
        // rows' own dot products.
        if constexpr (QUAD) {
            // Reduce-scatter of the lanes' 16 partial dot products over the
            // quad: lanes k and k ^ 2 swap the halves of the chunk the other
            // keeps (points with bit 1 of t equal to its own), then lanes k
            // and k ^ 1 do so for one point, so lane k ends with point k's
            // four sums and combines them once, for the point it stores.
            float d[CH][4];
#pragma unroll
            for (int t = 0; t < CH; ++t)
#pragma unroll
                for (int cn = 0; cn < 4; ++cn) d[t][cn] = lane_dot<DT, VEC>(graw, g, raw[t][cn], 0.0f);
            const bool hi2 = (c & 2) != 0, hi1 = (c & 1) != 0;
            float e[2][4], f[4];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int cn = 0; cn < 4; ++cn) {
                    const float keep = hi2 ? d[j + 2][cn] : d[j][cn];
                    const float give = hi2 ? d[j][cn] : d[j + 2][cn];
                    e[j][cn] = keep + dpp_move<0x4E>(give);  // quad_perm [2, 3, 0, 1]
                }
#pragma unroll
            for (int cn = 0; cn < 4; ++cn) {
                const float keep = hi1 ? e[1][cn] : e[0][cn];
                const float give = hi1 ? e[0][cn] : e[1][cn];
                f[cn] = keep + dpp_move<0xB1>(give);  // quad_perm [1, 0, 3, 2]
            }
            float vs, vx, vy;
            point_sums(f, fx_own, fy_own, vs, vx, vy);
            vx *= sw[0];  // lane k's scales are point k's
            vy *= sh[0];
            if (q_ok && i0 + c < per_lane) {
                const int64_t pp = pq * LK + (i0 + c) * split + s;
                grad_attn[pp] = from_f32(PT{}, vs);
                grad_loc[2 * pp] = from_f32(PT{}, vx);
                grad_loc[2 * pp + 1] = from_f32(PT{}, vy);
            }
            continue;
        }
        float ds[CH], dx[CH], dy[CH];
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            float d[4];
#pragma unroll
            for (int cn = 0; cn < 4; ++cn) d[cn] = lane_dot<DT, VEC>(graw, g, raw[t][cn], 0.0f);
            point_sums(d, fx[t], fy[t], ds[t], dx[t], dy[t]);
        }
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            ds[t] = group_sum(ds[t], log2g);
            dx[t] = group_sum(dx[t], log2g) * sw[t];
            dy[t] = group_sum(dy[t], log2g) * sh[t];
        }
        for (int t0 = 0; t0 < CH; t0 += G) {
            const int t = t0 + c;
            float vs = ds[0], vx = dx[0], vy = dy[0];
#pragma unroll
            for (int k = 1; k < CH; ++k) {
                vs = t == k ? ds[k] : vs;
                vx = t == k ? dx[k] : vx;
                vy = t == k ? dy[k] : vy;
            }
            if (q_ok && t < CH && i0 + t < per_lane) {
                const int64_t pp = pq * LK + (i0 + t) * split + s;
                grad_attn[pp] = from_f32(PT{}, vs);
                grad_loc[2 * pp] = from_f32(PT{}, vx);
                grad_loc[2 * pp + 1] = from_f32(PT{}, vy);
            }
        }
    }
}

template <class DT, class PT, int VEC, int CH, bool BUF, bool QUAD>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 4))) void msda_grad_kernel(
    const typename DT::S *__restrict__ value, const typename PT::S *__restrict__ loc,
    const typename PT::S *__restrict__ attn, const typename DT::S *__restrict__ grad_out,
    typename PT::S *__restrict__ grad_loc, typename PT::S *__restrict__ grad_attn,
    const LevelTable lt, const int64_t S, const int64_t Q, const int M, const int D,
    const int L, const int K, const int qblocks, const int64_t ntiles, const int log2g,
    const int log2s, const TileOrder to, const bool pvec) {
    const int64_t tile = logical_block();
    if (tile >= ntiles) return;  // whole workgroup leaves together
    grad_tile<DT, PT, VEC, CH, BUF, QUAD>(MSDA_GRAD_ARGS, tile);
}

// ------------------------------------------------------------ backward
//
// Lane layout. MI355X's L2 executes atomics per request, one request covering
// up to 16 dwords of one 64-byte segment; a request carrying one dword costs
// about as much as one carrying sixteen. So the backward gives each query a
// group of G <= 16 lanes and lane c owns the slots c, c + G, ... of a corner
// row: one instruction of the group touches G consecutive slots, i.e. one
// contiguous segment, for the gathers and for the atomics alike. A slot is a
// dword of 16-bit data (two channels, packed atomics) or one fp32 channel.
// For fp32 targets (fp32 data, or the fp32 scratch of 16-bit data) the
// upstream gradient is also held in channel layout (channel c + iG) so that
// every fp32 atomic instruction covers G consecutive dwords.

// grad_value += A * w_ij * g on the in-bounds corners of one point of level l
// (course page "5. The backward kernel", section "Scatter needs atomics"):
// fp32 atomics in channel layout (channel c + iG) for fp32 targets (fp32 data,
// or the level's fp32 scratch), packed 16-bit atomics in slot layout (slot
// c + jG) otherwise. Levels that are binned are skipped by the callers.
template <class DT, int SLOT, int J>
__device__ __forceinline__ void scatter_point(const Cell &cl, float aw, const LevelTable &lt,
                                              int l, void *grad_value, float *workspace,
                                              int64_t b, int64_t bS, int m, int M, int D,
                                              int64_t MD, int c, int G, const bool (&slot_ok)[J],
                                              const float (&g)[J][SLOT],
                                              const float (&gc)[J * SLOT]) {
    constexpr bool kF32 = sizeof(typename DT::S) == 4;
    constexpr int JC = J * SLOT;
    const float fx = cl.fx, fy = cl.fy, gx = 1.0f - fx, gy = 1.0f - fy;
    const int W = lt.W[l];
    const int64_t start = lt.start[l];
    const int64_t soff = lt.scratch_off[l];
    const int64_t HW = (int64_t)lt.H[l] * W;
    const bool vc[4] = {cl.v00, cl.v01, cl.v10, cl.v11};
    const float coef[4] = {aw * gx * gy, aw * fx * gy, aw * gx * fy, aw * fx * fy};
    const int64_t drow[4] = {0, 1, W, (int64_t)W + 1};  // pixel rows from row00
#pragma unroll
    for (int cn = 0; cn < 4; ++cn) {
        if (!vc[cn]) continue;
        const int64_t row = cl.row00 + drow[cn];
        if (kF32 || soff >= 0) {
            float *tp = kF32 ? static_cast<float *>(grad_value) + (bS + row) * MD + (int64_t)m * D
                             : workspace + soff + ((b * HW + (row - start)) * M + m) * (int64_t)D;
#pragma unroll
            for (int i = 0; i < JC; ++i) {
                const int ch = c + i * G;
                if (ch < D) atomic_add_f32(tp + ch, coef[cn] * gc[i]);
            }
        } else if constexpr (!kF32) {
            uint16_t *tp = static_cast<uint16_t *>(grad_value) + (bS + row) * MD + (int64_t)m * D;
#pragma unroll
            for (int j = 0; j < J; ++j) {
                if (!slot_ok[j]) continue;
                uint16_t *e = tp + (int64_t)(c + j * G) * SLOT;
                if constexpr (SLOT == 2) {
                    // one dword, 4-byte aligned (host-checked)
                    atomic_add_pk(DT{}, e, coef[cn] * g[j][0], coef[cn] * g[j][1]);
                } else {
                    // single element: packed add on the enclosing aligned word
                    // with +0 for the neighbour (x + 0 == x); the host
                    // guarantees that word lies inside grad_value
                    const bool hi = (reinterpret_cast<uintptr_t>(e) & 2) != 0;
                    uint16_t *wd = reinterpret_cast<uint16_t *>(reinterpret_cast<uintptr_t>(e) &
                                                                ~uintptr_t(3));
                    const float v = coef[cn] * g[j][0];
                    atomic_add_pk(DT{}, wd, hi ? 0.0f : v, hi ? v : 0.0f);
                }
            }
        }
    }
}

// The query's upstream gradient in slot layout (g, slot c + jG) and, for fp32
// targets, in channel layout (gc, channel c + iG).
template <class DT, int SLOT, int J>
__device__ __forceinline__ void load_upstream(
    const typename DT::S *grad_out, int64_t pq, int D, int c, int G, bool q_ok, bool (&slot_ok)[J],
    float (&g)[J][SLOT], float (&gc)[J * SLOT],
    typename RawVec<SLOT * (int)sizeof(typename DT::S)>::type (&graw)[J]) {
    using R = typename RawVec<SLOT * (int)sizeof(typename DT::S)>::type;
    const int nslots = D / SLOT;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int sl = c + j * G;
        slot_ok[j] = q_ok && sl < nslots;
        const R r = *reinterpret_cast<const R *>(grad_out + pq * D + (sl < nslots ? sl : 0) * SLOT);
        graw[j] = slot_ok[j] ? r : zero_raw<R>();
        raw_to_f32<DT, SLOT>(graw[j], g[j]);
    }
    if constexpr (SLOT == 1) {
#pragma unroll
        for (int j = 0; j < J; ++j) gc[j] = g[j][0];
    } else {
#pragma unroll
        for (int i = 0; i < J * SLOT; ++i) {
            const int ch = c + i * G;
            const float v = to_f32(DT{}, grad_out[pq * D + (ch < D ? ch : 0)]);
            gc[i] = (q_ok && ch < D) ? v : 0.0f;
        }
    }
}

// Points per chunk for the backward: about 8 slots of corner data per lane.
template <int J>
struct BwdChunk {
    static constexpr int value = J >= 8 ? 1 : (J >= 3 ? 2 : 8 / J);
};

template <class DT, class PT, int SLOT, int J, bool BUF>
__global__ __launch_bounds__(kBlock) void msda_bwd_kernel(
    const typename DT::S *__restrict__ value, const typename PT::S *__restrict__ loc,
    const typename PT::S *__restrict__ attn, const typename DT::S *__restrict__ grad_out,
    void *__restrict__ grad_value, float *__restrict__ workspace,
    typename PT::S *__restrict__ grad_loc, typename PT::S *__restrict__ grad_attn,
    const LevelTable lt, const int64_t S, const int64_t Q, const int M, const int D,
    const int L, const int K, const int qblocks, const int64_t ntiles, const int log2g,
    const int log2s) {
    using E = typename DT::S;
    using R = typename RawVec<SLOT * (int)sizeof(E)>::type;  // one slot
    constexpr int JC = J * SLOT;  // fp32-channel-layout registers per lane
    constexpr int CH = BwdChunk<J>::value;
    const int64_t tile = logical_block();
    if (tile >= ntiles) return;
    const int64_t bm = tile / qblocks;
    const int qb = (int)(tile - bm * qblocks);
    const int64_t b = bm / M;
    const int m = (int)(bm - b * M);

    const int tid = threadIdx.x;
    const int G = 1 << log2g;
    const int c = tid & (G - 1);
    const int s = (tid >> log2g) & ((1 << log2s) - 1);
    const int qpb = kBlock >> (log2g + log2s);
    const int64_t q = (int64_t)qb * qpb + (tid >> (log2g + log2s));
    const bool q_ok = q < Q;
    const int split = 1 << log2s;
    const int LK = L * K;
    const int per_lane = LK >> log2s;

    const int64_t pq = (b * Q + (q_ok ? q : 0)) * M + m;  // clamped: always a valid query
    const typename PT::S *loc_q = loc + pq * LK * 2;
    const typename PT::S *attn_q = attn + pq * LK;
    const int64_t MD = (int64_t)M * D;
    const int64_t row_bytes = MD * (int64_t)sizeof(E);
    const int64_t bS = b * S;
    const Slice<BUF> slice(value + bS * MD, S * row_bytes);
    const int64_t head_bytes = (int64_t)m * D * (int64_t)sizeof(E);

    bool slot_ok[J];
    float g[J][SLOT], gc[JC];
    R graw[J];
    load_upstream<DT, SLOT, J>(grad_out, pq, D, c, G, q_ok, slot_ok, g, gc, graw);

    for (int i0 = 0; i0 < per_lane; i0 += CH) {
        float lx[CH], ly[CH], aw[CH];
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            const bool t_ok = i0 + t < per_lane;  // uniform
            const int p = (t_ok ? i0 + t : 0) * split + s;
            load_xy<PT>(loc_q + 2 * p, lx[t], ly[t]);
            const float a = to_f32(PT{}, attn_q[p]);
            aw[t] = (q_ok && t_ok) ? a : 0.0f;
        }
        Cell cl[CH];
        int lvl[CH];
        R raw[CH][4][J];
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            const bool t_ok = i0 + t < per_lane;
            int l = ((i0 + t) * split) / K;
            l = l < L ? l : L - 1;
            lvl[t] = l;
            const int W = lt.W[l];
            cl[t] = map_cell(lx[t], ly[t], (float)lt.H[l], (float)W, W, lt.start[l]);
            if (!t_ok) cl[t].v00 = cl[t].v01 = cl[t].v10 = cl[t].v11 = false;  // uniform
            const int64_t o00 = cl[t].row00 * row_bytes + head_bytes;
            const int64_t o10 = o00 + (int64_t)W * row_bytes;
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int64_t so = (int64_t)(c + j * G) * SLOT * (int64_t)sizeof(E);
                raw[t][0][j] = slice.template gather<R>(o00 + so, slot_ok[j] && cl[t].v00);
                raw[t][1][j] = slice.template gather<R>(o00 + row_bytes + so, slot_ok[j] && cl[t].v01);
                raw[t][2][j] = slice.template gather<R>(o10 + so, slot_ok[j] && cl[t].v10);
                raw[t][3][j] = slice.template gather<R>(o10 + row_bytes + so, slot_ok[j] && cl[t].v11);
            }
        }
        float ds[CH], dx[CH], dy[CH];
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            // the four corner rows' dot products with the upstream gradient
            float d[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < J; ++j)
#pragma unroll
                for (int cn = 0; cn < 4; ++cn) d[cn] = lane_dot<DT, SLOT>(graw[j], g[j], raw[t][cn][j], d[cn]);
            point_sums(d, cl[t].fx, cl[t].fy, ds[t], dx[t], dy[t]);
        }
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            ds[t] = group_sum(ds[t], log2g);
            dx[t] = group_sum(dx[t], log2g);
            dy[t] = group_sum(dy[t], log2g);
        }
        // Every lane of the group holds the chunk's sums: lane c stores those
        // of point t0 + c, so one instruction of the group writes up to G
        // points' grad_attn (and grad_loc x, y) instead of one point each.
        float gsx[CH], gsy[CH];
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            gsx[t] = (float)lt.W[lvl[t]] * aw[t] * dx[t];
            gsy[t] = (float)lt.H[lvl[t]] * aw[t] * dy[t];
        }
        for (int t0 = 0; t0 < CH; t0 += G) {
            const int t = t0 + c;
            float vs = ds[0], vx = gsx[0], vy = gsy[0];
#pragma unroll
            for (int k = 1; k < CH; ++k) {
                vs = t == k ? ds[k] : vs;
                vx = t == k ? gsx[k] : vx;
                vy = t == k ? gsy[k] : vy;
            }
            if (q_ok && t < CH && i0 + t < per_lane) {
                const int64_t pp = pq * LK + (i0 + t) * split + s;
                grad_attn[pp] = from_f32(PT{}, vs);
                grad_loc[2 * pp] = from_f32(PT{}, vx);
                grad_loc[2 * pp + 1] = from_f32(PT{}, vy);
            }
        }
#pragma unroll
        for (int t = 0; t < CH; ++t) {
            if (!(q_ok && i0 + t < per_lane)) continue;
            // binned or pre-reduced levels are summed by their own kernels
            if (lt.bin_shift[lvl[t]] >= 0 || ((lt.prered >> lvl[t]) & 1u)) continue;
            scatter_point<DT, SLOT, J>(cl[t], aw[t], lt, lvl[t], grad_value, workspace, b, bS, m,
                                       M, D, MD, c, G, slot_ok, g, gc);
        }
    }
}

// Atomic scatter only (course page "5. The backward kernel", section
// "Scatter needs atomics"), for the levels that are not binned when
// grad_loc / grad_attn come from msda_grad_kernel: no value gathers, no dot
// products. Same lane mapping as msda_bwd_kernel; a group walks the points of
// each unbinned level, CH at a time with their parameter loads issued first.
#define MSDA_SCATTER_PARAMS                                                                   \
    const typename PT::S *__restrict__ loc, const typename PT::S *__restrict__ attn,          \
        const typename DT::S *__restrict__ grad_out, void *__restrict__ grad_value,           \
        float *__restrict__ workspace, const LevelTable &lt, const int64_t S, const int64_t Q, \
        const int M, const int D, const int L, const int K, const int qblocks,                \
        const int log2g, const int log2s
#define MSDA_SCATTER_ARGS loc, attn, grad_out, grad_value, workspace, lt, S, Q, M, D, L, K, qblocks, \
                          log2g, log2s

template <class DT, class PT, int SLOT, int J>
__device__ __forceinline__ void scatter_tile(MSDA_SCATTER_PARAMS, const int64_t tile) {
    constexpr int JC = J * SLOT;
    constexpr int CH = 8;
    const int64_t bm = tile / qblocks;
    const int qb = (int)(tile - bm * qblocks);
    const int64_t b = bm / M;
    const int m = (int)(bm - b * M);
    const int tid = threadIdx.x;
    const int G = 1 << log2g;
    const int c = tid & (G - 1);
    const int s = (tid >> log2g) & ((1 << log2s) - 1);
    const int qpb = kBlock >> (log2g + log2s);
    const int64_t q = (int64_t)qb * qpb + (tid >> (log2g + log2s));
    const bool q_ok = q < Q;
    const int split = 1 << log2s;
    const int LK = L * K;
    const int64_t pq = (b * Q + (q_ok ? q : 0)) * M + m;  // clamped: always a valid query
    const typename PT::S *loc_q = loc + pq * LK * 2;
    const typename PT::S *attn_q = attn + pq * LK;
    const int64_t MD = (int64_t)M * D;
    const int64_t bS = b * S;
    bool slot_ok[J];
    float g[J][SLOT], gc[JC];
    typename RawVec<SLOT * (int)sizeof(typename DT::S)>::type graw[J];  // unused here
    load_upstream<DT, SLOT, J>(grad_out, pq, D, c, G, q_ok, slot_ok, g, gc, graw);
    for (int l = 0; l < L; ++l) {
        // binned or pre-reduced: summed by their own kernels
        if (lt.bin_shift[l] >= 0 || ((lt.prered >> l) & 1u)) continue;
        const int W = lt.W[l];
        const float Hf = (float)lt.H[l], Wf = (float)W;
        for (int k0 = 0; k0 < K; k0 += split * CH) {
            uint32_t bx[CH], by[CH], ba[CH];
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                const int k = k0 + t * split;  // + s: the group's own point of this stride
                const int p = l * K + (k < K ? k + s : s);
                bx[t] = load_bits<PT>(loc_q + 2 * p);
                by[t] = load_bits<PT>(loc_q + 2 * p + 1);
                ba[t] = load_bits<PT>(attn_q + p);
            }
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                pin(bx[t]);
                pin(by[t]);
                pin(ba[t]);
            }
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                if (!(q_ok && k0 + t * split < K)) continue;
                const Cell cl = map_cell(bits_to_f32<PT>(bx[t]), bits_to_f32<PT>(by[t]), Hf, Wf, W,
                                         lt.start[l]);
                scatter_point<DT, SLOT, J>(cl, bits_to_f32<PT>(ba[t]), lt, l, grad_value, workspace,
                                           b, bS, m, M, D, MD, c, G, slot_ok, g, gc);
            }
        }
    }
}

template <class DT, class PT, int SLOT, int J>
__global__ __launch_bounds__(kBlock) void msda_scatter_kernel(
    const typename PT::S *__restrict__ loc, const typename PT::S *__restrict__ attn,
    const typename DT::S *__restrict__ grad_out, void *__restrict__ grad_value,
    float *__restrict__ workspace, const LevelTable lt, const int64_t S, const int64_t Q,
    const int M, const int D, const int L, const int K, const int qblocks, const int64_t ntiles,
    const int log2g, const int log2s) {
    const int64_t tile = logical_block();
    if (tile >= ntiles) return;
    scatter_tile<DT, PT, SLOT, J>(MSDA_SCATTER_ARGS, tile);
}

// ------------------------------------------------------ binned grad_value
//
// grad_value without float atomics on global memory. Every in-bounds corner
// of every point contributes A * w_ij * g[b, q, m, :] to one destination row.
// The rows of level l of one (b, m) are cut into bins of 2^bin_shift[l] pixel
// rows. A counting sort (count, scan, place) groups the contributions by bin
// as 8-byte records; then one workgroup per bin sums its records into an fp32
// tile in LDS and writes each row of the bin once, rounded once.
//
// Count and place aggregate a workgroup's corners per bin in an LDS hash
// table before touching the global counters, so a counter receives one
// atomic per (workgroup, bin) rather than one per corner. Consecutive points
// of one (b, m) fall into few bins, so counters of heavily shared coarse
// levels see little contention.

constexpr int kBinBlock = 512;  // threads (one point each) of the count / place workgroups
constexpr int kHashBits = 12;
constexpr int kHashSlots = 1 << kHashBits;   // > 4 corners x kBinBlock points: never full
constexpr uint32_t kEmptyKey = 0xFFFFFFFFu;  // bin ids stay below 2^31
constexpr int kRankedKeys = 256;             // bins per workgroup visited in key order

// One thread per point of a binned level of one (b, m): workgroup w of pair bm
// takes the (query, binned point) indices [w * kBinBlock, (w + 1) * kBinBlock)
// of that pair (512 points: more corners share each (workgroup, bin) atomic,
// at the 32 waves per CU that the 37.5 KB of LDS leaves). Count
// (PLACE = false) adds the workgroup's per-bin totals to counter[bin]. Place
// (PLACE = true) reserves a range of each bin with one returning atomic on
// counter[bin] (the bin's cursor, initialised to its start by the scan) and
// writes the records: x = query << 4 | row within the bin (bins have at most
// 16 rows), y = fp32 bits of A * w_ij (summed over the query's points that
// share the pixel, when merging; count counts every in-bounds corner, so a
// bin's count bounds its records from above). Both derive cells with the
// same map_cell as the backward, so they agree on every in-bounds corner.
template <class DT, bool PLACE>
__global__ __launch_bounds__(kBinBlock) void bin_sort_kernel(
    const typename DT::S *__restrict__ loc, const typename DT::S *__restrict__ attn,
    const LevelTable lt, uint32_t *__restrict__ counter, uint2 *__restrict__ records,
    const int64_t Q, const int M, const int L, const int K, const int64_t nbbm,
    const int64_t wpb, const int64_t ntiles, const bool merge) {
    __shared__ uint32_t keys[kHashSlots];
    __shared__ uint32_t cnt[kHashSlots];
    __shared__ uint16_t used[4 * kBinBlock];
    __shared__ uint32_t nused;
    __shared__ uint32_t ukey[kRankedKeys];
    __shared__ uint16_t order[kRankedKeys];
    const int64_t wg = logical_block();
    if (wg >= ntiles) return;
    const int tid = threadIdx.x;
    for (int i = tid; i < kHashSlots; i += kBinBlock) {
        keys[i] = kEmptyKey;
        cnt[i] = 0u;
    }
    if (tid == 0) nused = 0u;
    __syncthreads();

    const int64_t bm = wg / wpb;
    const int64_t w = wg - bm * wpb;
    const int64_t b = bm / M;
    const int m = (int)(bm - b * M);
    const int LK = L * K;
    const int LKb = lt.nblev * K;  // points of the binned levels per query
    // 32-bit index arithmetic: the host keeps 4 * B * Q * M * L * K below
    // 2^32; shifts for power-of-two divisors (the choice is uniform)
    const uint32_t i = (uint32_t)(w * kBinBlock) + (uint32_t)tid;
    const bool ok = i < (uint32_t)(Q * LKb);
    const uint32_t q = !ok ? 0u
                           : ((LKb & (LKb - 1)) == 0 ? i >> __builtin_ctz((unsigned)LKb)
                                                     : i / (uint32_t)LKb);
    const int r = ok ? (int)(i - q * (uint32_t)LKb) : 0;
    const int rk = (K & (K - 1)) == 0 ? r >> __builtin_ctz((unsigned)K) : r / K;
    const int l = lt.blevel[rk];
    const int pp = l * K + (r - rk * K);
    const int64_t pt = ((b * Q + q) * M + m) * LK + pp;
    float x, y;
    load_xy<DT>(loc + 2 * pt, x, y);
    const int W = lt.W[l];
    const int64_t start = lt.start[l];
    const Cell cl = map_cell(x, y, (float)lt.H[l], (float)W, W, start);
    const int shl = lt.bin_shift[l];
    const bool binned = ok && shl >= 0;  // levels left to atomics make no records
    const int sh = shl >= 0 ? shl : 0;
    const uint32_t kbase = (uint32_t)(bm * nbbm + lt.bin_off[l]);
    bool vc[4] = {binned && cl.v00, binned && cl.v01, binned && cl.v10, binned && cl.v11};
    uint32_t slot[4], rank[4], rib[4], key[4];
    int id[4];  // pixel of the corner in the level; a value of its own when out of bounds
#pragma unroll
    for (int cn = 0; cn < 4; ++cn) {
        slot[cn] = rank[cn] = rib[cn] = key[cn] = 0u;
        const int64_t rel = cl.row00 + ((cn & 2) ? W : 0) + (cn & 1) - start;
        id[cn] = vc[cn] ? (int)rel : -1 - (tid * 4 + cn);
        if (!vc[cn]) continue;
        rib[cn] = (uint32_t)(rel & ((1 << sh) - 1));
        key[cn] = kbase + (uint32_t)(rel >> sh);
    }
    float coef[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (PLACE) {
        const float a = ok ? to_f32(DT{}, attn[pt]) : 0.0f;
#pragma unroll
        for (int cn = 0; cn < 4; ++cn) {
            const float wx = (cn & 1) ? cl.fx : 1.0f - cl.fx;
            const float wy = (cn & 2) ? cl.fy : 1.0f - cl.fy;
            coef[cn] = a * wx * wy;
        }
    }
    // With `merge` (K = 2 or 4), the K points of one (query, level) are the
    // lanes of one aligned quad (pair). Their corners that fall on one pixel
    // add to the same grad_value row with the same upstream gradient, so they
    // make one record: the lowest point k holding the pixel keeps its corner
    // and adds the other points' own coefficients, the others drop theirs.
    // Only place merges (count counts every in-bounds corner, an upper
    // bound). The quad's values rotate by DPP quad permutes (no LDS traffic).
    float sum[4];  // coefficient of this point's record per corner
#pragma unroll
    for (int cn = 0; cn < 4; ++cn) sum[cn] = coef[cn];
    if (merge) {
        const int k = tid & (K - 1);
        bool drop[4] = {false, false, false, false};
        // lane k against lane (k + j) mod K, whose values arrive by quad permute CTRL
        auto visit = [&](auto ctrl, const int j) {
            constexpr int CTRL = decltype(ctrl)::value;
            const bool earlier = k + j >= K;  // the other lane holds an earlier point
            int oid[4];
            float oc[4];  // the other point's own coefficients, not its sums so far
#pragma unroll
            for (int cn = 0; cn < 4; ++cn) {
                oid[cn] = __builtin_amdgcn_update_dpp(0, id[cn], CTRL, 0xF, 0xF, true);
                oc[cn] = PLACE ? dpp_move<CTRL>(coef[cn]) : 0.0f;
            }
#pragma unroll
            for (int cn = 0; cn < 4; ++cn)
#pragma unroll
                for (int c2 = 0; c2 < 4; ++c2) {
                    const bool e = id[cn] == oid[c2];
                    drop[cn] = drop[cn] || (e && earlier);
                    if constexpr (PLACE) sum[cn] += (e && !earlier) ? oc[c2] : 0.0f;
                }
        };
        if (K == 2) {
            visit(std::integral_constant<int, 0xB1>{}, 1);  // [1, 0, 3, 2]
        } else {
            visit(std::integral_constant<int, 0x39>{}, 1);  // [1, 2, 3, 0]
            visit(std::integral_constant<int, 0x4E>{}, 2);  // [2, 3, 0, 1]
            visit(std::integral_constant<int, 0x93>{}, 3);  // [3, 0, 1, 2]
        }
#pragma unroll
        for (int cn = 0; cn < 4; ++cn) vc[cn] = vc[cn] && !drop[cn];
    }
    // The two corners of a pair (00-01, 10-11: neighbouring rows) mostly
    // share a bin; then one hash access and one counter add of 2 serve both,
    // and the second corner takes the rank after the first's.
#pragma unroll
    for (int cn = 0; cn < 4; ++cn) {
        if (!vc[cn]) continue;
        if ((cn & 1) && vc[cn - 1] && key[cn] == key[cn - 1]) {
            slot[cn] = slot[cn - 1];
            rank[cn] = rank[cn - 1] + 1u;
            continue;
        }
        const uint32_t n = (!(cn & 1) && vc[cn + 1] && key[cn + 1] == key[cn]) ? 2u : 1u;
        uint32_t h = (key[cn] * 2654435761u) >> (32 - kHashBits);
        // linear probing; at most 4 * kBinBlock keys per workgroup, so an empty
        // slot always exists and the loop ends
        while (true) {
            const uint32_t prev = atomicCAS(&keys[h], kEmptyKey, key[cn]);
            if (prev == kEmptyKey) {
                used[atomicAdd(&nused, 1u)] = (uint16_t)h;
                break;
            }
            if (prev == key[cn]) break;
            h = (h + 1) & (kHashSlots - 1);
        }
        slot[cn] = h;
        if constexpr (PLACE) rank[cn] = atomicAdd(&cnt[h], n);
        else atomicAdd(&cnt[h], n);
    }
    __syncthreads();
    const uint32_t nu = nused;
    // One atomic request covers every lane of an instruction that falls in
    // the same 64-byte segment, i.e. 16 neighbouring bin counters. Visiting
    // the workgroup's bins in key order lets lanes with neighbouring bins
    // share requests; keys are ranked by counting when there are at most
    // kRankedKeys of them (local sampling patterns give a few dozen),
    // otherwise the insertion order stands.
    const bool ranked = nu <= (uint32_t)kRankedKeys;  // uniform over the workgroup
    if (ranked) {
        if (tid < nu) ukey[tid] = keys[used[tid]];
        __syncthreads();
        if (tid < nu) {
            const uint32_t k = ukey[tid];
            uint32_t rk = 0u;
            for (uint32_t j = 0; j < nu; ++j) rk += ukey[j] < k ? 1u : 0u;
            order[rk] = used[tid];  // keys are distinct: ranks are a permutation
        }
        __syncthreads();
    }
    for (uint32_t u = tid; u < nu; u += kBinBlock) {
        const uint32_t h = ranked ? order[u] : used[u];
        if constexpr (PLACE)
            cnt[h] = __hip_atomic_fetch_add(counter + keys[h], cnt[h], __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
        else
            __hip_atomic_fetch_add(counter + keys[h], cnt[h], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
    if constexpr (PLACE) {
        __syncthreads();
        const uint32_t qx = (uint32_t)q << 4;
#pragma unroll
        for (int cn = 0; cn < 4; ++cn) {
            if (!vc[cn]) continue;
            records[cnt[slot[cn]] + rank[cn]] = make_uint2(qx | rib[cn], __float_as_uint(sum[cn]));
        }
    }
}

// One workgroup per (b, m, binned level) does count, scan and place in one
// launch when the pair has at most kSortBlock * kSortPts points on the level:
// each thread keeps its points' corners in registers, the level's per-bin
// counts live in LDS as two 16-bit halves of a word (an LDS integer atomic
// per corner), a block scan turns them into offsets, the bin's record range
// [starts, ends) is written, and the cached corners are placed at their
// bin's LDS cursor. Records of the segment go to its own fixed region of
// 4 * Q * K records, so no global counter, scan or zero fill is needed.
// Workgroups past the segments zero-fill grad_value (n16 16-byte stores),
// which the same launch can do since nothing here reads it.
constexpr int kSortBlock = 1024;
constexpr int kSortPts = 2;  // points per thread

#define MSDA_SORT_PARAMS                                                                      \
    const typename DT::S *__restrict__ loc, const typename DT::S *__restrict__ attn,          \
        const LevelTable &lt, uint32_t *__restrict__ starts, uint32_t *__restrict__ ends,     \
        uint2 *__restrict__ records, const int64_t Q, const int M, const int L, const int K,  \
        const int64_t nbbm
#define MSDA_SORT_ARGS loc, attn, lt, starts, ends, records, Q, M, L, K, nbbm

// Workgroups of BLOCK threads, PTS points per thread (Q * K <= BLOCK * PTS);
// `hist`: the dynamic LDS counters.
template <class DT, int BLOCK, int PTS>
__device__ __forceinline__ void local_sort_segment(uint32_t *hist, MSDA_SORT_PARAMS,
                                                   const int64_t seg) {
    constexpr int kSortBlock = BLOCK;
    constexpr int kSortPts = PTS;
    constexpr int kWaves = kSortBlock / 64;
    __shared__ uint32_t wsum[kWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t bm = seg / lt.nblev;
    const int l = lt.blevel[seg - bm * lt.nblev];
    const int64_t b = bm / M;
    const int m = (int)(bm - b * M);
    const int sh = lt.bin_shift[l];
    const int W = lt.W[l];
    const int64_t start = lt.start[l];
    const int64_t HW = (int64_t)lt.H[l] * W;
    const int nb = (int)((HW + (1 << sh) - 1) >> sh);
    const int nw = (nb + 1) >> 1;
    const int npts = (int)Q * K;
    const int LK = L * K;
    const uint32_t rbase = (uint32_t)seg * (uint32_t)(4 * npts);
    const int64_t gbin0 = bm * nbbm + lt.bin_off[l];
    for (int w = tid; w < nw; w += kSortBlock) hist[w] = 0u;

    // this thread's points: corner bins (-1: no record), rows in the bin, coefficients
    int bin[kSortPts][4];
    uint32_t key[kSortPts][4];
    float coef[kSortPts][4];
#pragma unroll
    for (int r = 0; r < kSortPts; ++r) {
        const int i = tid + r * kSortBlock;
        const bool ok = i < npts;
        const int q = ok ? i / K : 0;
        const int64_t pt = ((b * Q + q) * M + m) * LK + l * K + (ok ? i - q * K : 0);
        float x, y;
        load_xy<DT>(loc + 2 * pt, x, y);
        const float a = to_f32(DT{}, attn[pt]);
        const Cell cl = map_cell(x, y, (float)lt.H[l], (float)W, W, start);
        const bool vc[4] = {ok && cl.v00, ok && cl.v01, ok && cl.v10, ok && cl.v11};
#pragma unroll
        for (int cn = 0; cn < 4; ++cn) {
            const int64_t rel = cl.row00 + ((cn & 2) ? W : 0) + (cn & 1) - start;
            bin[r][cn] = vc[cn] ? (int)(rel >> sh) : -1;
            key[r][cn] = ((uint32_t)q << 4) | (uint32_t)(rel & ((1 << sh) - 1));
            const float wx = (cn & 1) ? cl.fx : 1.0f - cl.fx;
            const float wy = (cn & 2) ? cl.fy : 1.0f - cl.fy;
            coef[r][cn] = a * wx * wy;
        }
    }
    __syncthreads();  // hist cleared
#pragma unroll
    for (int r = 0; r < kSortPts; ++r)
#pragma unroll
        for (int cn = 0; cn < 4; ++cn)
            if (bin[r][cn] >= 0) atomicAdd(&hist[bin[r][cn] >> 1], 1u << ((bin[r][cn] & 1) << 4));
    __syncthreads();

    // exclusive scan: thread t owns words [t * per, (t + 1) * per)
    const int per = (nw + kSortBlock - 1) / kSortBlock;
    const int w0 = tid * per, w1 = min(nw, w0 + per);
    uint32_t tot = 0;
    for (int w = w0; w < w1; ++w) tot += (hist[w] & 0xffffu) + (hist[w] >> 16);
    uint32_t inc = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(inc, off);
        if (lane >= off) inc += y;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        uint32_t v = lane < kWaves ? wsum[lane] : 0u;
#pragma unroll
        for (int off = 1; off < kWaves; off <<= 1) {
            const uint32_t y = __shfl_up(v, off);
            if (lane >= off) v += y;
        }
        if (lane < kWaves) wsum[lane] = v;
    }
    __syncthreads();
    uint32_t run = inc - tot + (wave > 0 ? wsum[wave - 1] : 0u);
    for (int w = w0; w < w1; ++w) {
        const uint32_t v = hist[w];
        const uint32_t c0 = v & 0xffffu, c1 = v >> 16;
        const uint32_t o0 = run, o1 = run + c0;
        run = o1 + c1;
        hist[w] = o0 | (o1 << 16);  // both <= 4 * Q * K <= 4 * kSortBlock * kSortPts
        const int64_t g = gbin0 + 2 * w;
        starts[g] = rbase + o0;
        ends[g] = rbase + o1;
        if (2 * w + 1 < nb) {
            starts[g + 1] = rbase + o1;
            ends[g + 1] = rbase + o1 + c1;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kSortPts; ++r)
#pragma unroll
        for (int cn = 0; cn < 4; ++cn) {
            if (bin[r][cn] < 0) continue;
            const int hs = (bin[r][cn] & 1) << 4;
            const uint32_t slot = (atomicAdd(&hist[bin[r][cn] >> 1], 1u << hs) >> hs) & 0xffffu;
            records[rbase + slot] = make_uint2(key[r][cn], __float_as_uint(coef[r][cn]));
        }
}

// n16 16-byte zero stores by the workgroups [0, nblocks) of a role
// Non-temporal stores: the fill shares its launch with the gradients and
// the sort, and the rows are next touched by another launch's atomics
// (decoder workload step 45.8 -> 44.7 us; the stand-alone zero_kernel_16 of
// a 272 MB grad_value got slower with them, 42 -> 69 us, and keeps plain
// stores).
typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void zero_part(uint4 *__restrict__ dst, const int64_t n16,
                                          const int64_t block, const int64_t nblocks) {
    const u32x4_nt z = {0u, 0u, 0u, 0u};
    const int64_t stride = nblocks * blockDim.x;
    for (int64_t i = block * blockDim.x + threadIdx.x; i < n16; i += stride)
        __builtin_nontemporal_store(z, reinterpret_cast<u32x4_nt *>(dst + i));
}

template <class DT>
__global__ __launch_bounds__(kSortBlock) void bin_local_sort_kernel(
    const typename DT::S *__restrict__ loc, const typename DT::S *__restrict__ attn,
    const LevelTable lt, uint32_t *__restrict__ starts, uint32_t *__restrict__ ends,
    uint2 *__restrict__ records, const int64_t Q, const int M, const int L, const int K,
    const int64_t nbbm, const int64_t nseg, uint4 *__restrict__ zero_dst, const int64_t zero_n16) {
    extern __shared__ uint32_t hist[];  // bin i: half (i & 1) of word i >> 1
    const int64_t seg = blockIdx.x;
    if (seg >= nseg) zero_part(zero_dst, zero_n16, seg - nseg, (int64_t)gridDim.x - nseg);
    else local_sort_segment<DT, kSortBlock, kSortPts>(hist, MSDA_SORT_ARGS, seg);
}

// The gradients (msda_grad_kernel), the local bin sort and the grad_value zero
// fill in one launch: none reads what another writes, so the sort's and the
// fill's workgroups run beside the gradient tiles. The fill and the sort come
// first, so that their streams of stores and their latency chains start with
// the gathers of the gradient tiles rather than after them: workgroups
// [0, nzero) zero-fill, [nzero, nzero + nsegp) sort segments (nsegp = nseg
// rounded up to a multiple of 8), the rest take gradient tiles in XCD-aware
// order (nzero, nsegp and ngrad are multiples of 8).
constexpr int kFusedSortPts = 8;  // 256 threads x 8 points: the local sort's 2048 points

template <class DT, class PT, int VEC>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 4))) void grad_sort_kernel(
    const typename DT::S *__restrict__ value, const typename PT::S *__restrict__ loc,
    const typename PT::S *__restrict__ attn, const typename DT::S *__restrict__ grad_out,
    typename PT::S *__restrict__ grad_loc, typename PT::S *__restrict__ grad_attn,
    const LevelTable lt, const int64_t S, const int64_t Q, const int M, const int D,
    const int L, const int K, const int qblocks, const int64_t ntiles, const int log2g,
    const int log2s, const bool pvec, const uint32_t ngrad, uint32_t *__restrict__ starts,
    uint32_t *__restrict__ ends, uint2 *__restrict__ records, const int64_t nbbm,
    const uint32_t nseg, const uint32_t nsegp, const uint32_t nzero, uint4 *__restrict__ zero_dst,
    const int64_t zero_n16) {
    extern __shared__ uint32_t hist[];
    const uint32_t bx = blockIdx.x;
    if (bx < nzero) {
        zero_part(zero_dst, zero_n16, bx, nzero);
    } else if (bx < nzero + nsegp) {
        const uint32_t seg = bx - nzero;
        if (seg < nseg)
            local_sort_segment<PT, kBlock, kFusedSortPts>(hist, loc, attn, lt, starts, ends, records,
                                                          Q, M, L, K, nbbm, (int64_t)seg);
    } else {
        const uint32_t g = bx - nzero - nsegp;
        const int64_t tile = (int64_t)(g % kXcds) * (ngrad / kXcds) + g / kXcds;
        const TileOrder to = {0, 0};  // linear
        if (tile < ntiles) grad_tile<DT, PT, VEC, 4, true>(MSDA_GRAD_ARGS, tile);
    }
}

// One workgroup: counts[0:nb] -> exclusive starts[0:nb+1], cursor = starts.
// Tiles of 4 * kScanBlock counts, each thread owning 4 consecutive ones; the
// next tile's loads are issued before the current tile is scanned (wave
// shuffles, then the 16 wave totals), and a running carry joins the tiles.
constexpr int kScanBlock = 1024;
__global__ __launch_bounds__(kScanBlock) void bin_scan_kernel(uint32_t *__restrict__ starts,
                                                             uint32_t *__restrict__ cursor,
                                                             const int64_t nb) {
    constexpr int kWaves = kScanBlock / 64;
    constexpr int64_t kTile = 4 * kScanBlock;
    __shared__ uint32_t wsum[kWaves];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t ntiles = (nb + kTile - 1) / kTile;
    uint32_t cur[4], nxt[4] = {0u, 0u, 0u, 0u};
    auto load4 = [&](int64_t t, uint32_t(&v)[4]) {
        const int64_t i0 = t * kTile + 4 * (int64_t)tid;
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = i0 + k < nb ? starts[i0 + k] : 0u;
    };
    load4(0, cur);
    uint32_t carry = 0;
    for (int64_t t = 0; t < ntiles; ++t) {
        if (t + 1 < ntiles) load4(t + 1, nxt);
        const uint32_t s0 = cur[0], s1 = s0 + cur[1], s2 = s1 + cur[2], s3 = s2 + cur[3];
        uint32_t x = s3;  // inclusive scan over the wave
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) wsum[wv] = x;
        __syncthreads();
        if (wv == 0) {
            uint32_t w = lane < kWaves ? wsum[lane] : 0u;
#pragma unroll
            for (int off = 1; off < kWaves; off <<= 1) {
                const uint32_t y = __shfl_up(w, off);
                if (lane >= off) w += y;
            }
            if (lane < kWaves) wsum[lane] = w;
        }
        __syncthreads();
        const uint32_t excl = carry + (wv > 0 ? wsum[wv - 1] : 0u) + x - s3;
        const uint32_t out[4] = {excl, excl + s0, excl + s1, excl + s2};
        const int64_t i0 = t * kTile + 4 * (int64_t)tid;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (i0 + k < nb) {
                starts[i0 + k] = out[k];
                cursor[i0 + k] = out[k];
            }
        carry += wsum[kWaves - 1];
        __syncthreads();  // wsum is rewritten by the next tile
#pragma unroll
        for (int k = 0; k < 4; ++k) cur[k] = nxt[k];
    }
    if (tid == 0) starts[nb] = carry;
}

// Parallel scan of large count arrays, in tiles of kScanTile counts (each
// thread of a kScanBlock workgroup owns 4 consecutive ones): tile totals
// (bin_tile_sum_kernel), an exclusive scan of the totals by bin_scan_kernel
// over the short totals array, then every tile's exclusive scan plus its
// offset (bin_tile_scan_kernel), in place over the counts. The single-
// workgroup scan alone serialises on its barriers (each waits for the
// tile's loads and stores); these three launches run every tile at once.
constexpr int64_t kScanTile = 4 * kScanBlock;

__device__ __forceinline__ uint32_t block_sum_1024(uint32_t v, uint32_t *wsum) {
    constexpr int kWaves = kScanBlock / 64;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) wsum[wv] = v;
    __syncthreads();
    uint32_t t = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) t += wsum[i];
    return t;
}

__global__ __launch_bounds__(kScanBlock) void bin_tile_sum_kernel(const uint32_t *__restrict__ counts,
                                                                 uint32_t *__restrict__ tsum,
                                                                 const int64_t nb) {
    __shared__ uint32_t wsum[kScanBlock / 64];
    const int64_t i0 = (int64_t)blockIdx.x * kScanTile + 4 * (int64_t)threadIdx.x;
    uint32_t v = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) v += i0 + k < nb ? counts[i0 + k] : 0u;
    const uint32_t t = block_sum_1024(v, wsum);
    if (threadIdx.x == 0) tsum[blockIdx.x] = t;
}

// starts[0:nb] (counts) -> exclusive starts, cursor = starts; toff = the
// exclusive scan of the tile totals (toff[ntiles] = total -> starts[nb]).
// Every tile's exclusive scan plus its offset, the sum of the earlier tiles'
// totals (`tsum`, from bin_tile_sum_kernel), which wave 0 adds up itself:
// there are few tiles (4096 counts each), so no separate scan of the totals
// is launched. The last tile also writes starts[nb], the total.
__global__ __launch_bounds__(kScanBlock) void bin_tile_scan_kernel(uint32_t *__restrict__ starts,
                                                                  uint32_t *__restrict__ cursor,
                                                                  const uint32_t *__restrict__ tsum,
                                                                  const int64_t nb) {
    constexpr int kWaves = kScanBlock / 64;
    __shared__ uint32_t wsum[kWaves];
    __shared__ uint32_t tile_before;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t i0 = (int64_t)blockIdx.x * kScanTile + 4 * (int64_t)tid;
    uint32_t c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = i0 + k < nb ? starts[i0 + k] : 0u;
    if (wv == 0) {
        uint32_t t = 0;
        for (uint32_t j = lane; j < blockIdx.x; j += 64) t += tsum[j];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off);
        if (lane == 0) tile_before = t;
    }
    const uint32_t s3 = c[0] + c[1] + c[2] + c[3];
    uint32_t x = s3;  // inclusive scan over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    uint32_t before = tile_before;
    for (int i = 0; i < wv; ++i) before += wsum[i];
    uint32_t o = before + x - s3;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (i0 + k < nb) {
            starts[i0 + k] = o;
            cursor[i0 + k] = o;
        }
        o += c[k];
    }
    if (blockIdx.x == gridDim.x - 1 && tid == kScanBlock - 1) starts[nb] = o;
}

// One workgroup per bin, no atomics. The workgroup has kAccGroups lane
// groups of 16 lanes (slot layout as in the backward) and a bin has at most
// kAccGroups rows; with rep = kAccGroups / rows replicas of each row there
// are exactly kAccGroups (row, replica) slots, slot s = row * rep + replica
// belonging to lane group s, which sums its records in registers.
//
// Records come in rounds of kAccRPT * kBlock, kAccRPT per thread (the next
// round's loads are issued before the current round is processed), and each
// round is counting-sorted by slot in LDS: a returning add on the wave's own
// counter of the slot gives every record its rank among the wave's records of
// the same slot, one wave scans the 64 counters (and clears them for the
// next round), and the records are written in slot order. Two
// records per thread halve the rounds, and with them the barriers and the
// scan, per record; the sums per slot grow to twice the length. A group then reads its slot's records
// contiguously, U at a time, with all their upstream-gradient loads (32-bit
// offsets into a buffer over the batch's grad_output) issued before use. At
// the end every group stores its sums to an LDS tile, the replicas of each
// row are added, and the row is written (or added, with `accumulate`) to
// grad_value, V channels per access.
constexpr int kAccGroups = kBlock / 16;
constexpr int kAccRPT = 2;  // records per thread in one counting-sort round

#define MSDA_ACCUM_PARAMS                                                                     \
    const typename DT::S *__restrict__ grad_out, typename DT::S *__restrict__ grad_value,     \
        const uint32_t *__restrict__ starts, const uint32_t *__restrict__ ends,               \
        const uint2 *__restrict__ records, const LevelTable &lt, const int64_t S,             \
        const int64_t Q, const int M, const int D, const int L, const int64_t nbbm,           \
        const int accumulate
#define MSDA_ACCUM_ARGS grad_out, grad_value, starts, ends, records, lt, S, Q, M, D, L, nbbm, accumulate

// With WIDE (rows of exactly 64 bytes, J == 1) a group reads four records at
// a time instead of one: its lanes form four sub-groups of 4, sub-group r
// takes records r, r + 4, ... of the slot and each lane gathers 16 bytes of
// the row, as the forward does, so one load instruction of a wave covers 16
// records rather than 4; the sub-groups' sums are added with two cross-lane
// steps once per bin.
//
// `tile`: kAccGroups x D floats of LDS (the kernel's dynamic LDS).
template <class DT, int SLOT, int J, int V, bool WIDE>
__device__ __forceinline__ void accum_bin(float *tile, MSDA_ACCUM_PARAMS, const int64_t bin) {
    using E = typename DT::S;
    using R = typename RawVec<SLOT * (int)sizeof(E)>::type;
    static_assert(!WIDE || (J == 1 && SLOT * sizeof(E) == 4), "wide mode: 64-byte rows");
    constexpr int G = 16;
    constexpr int U = J == 1 ? 16 : (J == 2 ? 8 : 4);
    constexpr int VW = 16 / (int)sizeof(E);  // elements per 16-byte gather (wide mode)
    constexpr int UW = 4;                    // records per sub-group in flight (wide mode)
    constexpr int kWaves = kBlock / 64;
    __shared__ uint2 sorted[kAccRPT * kBlock];
    __shared__ uint32_t wcount[kAccGroups * kWaves];   // [slot][wave]
    __shared__ uint32_t woff[kAccGroups * kWaves + 1];  // exclusive prefix, slot-major
    const int64_t bm = bin / nbbm;
    const int lb = (int)(bin - bm * nbbm);
    const int64_t b = bm / M;
    const int m = (int)(bm - b * M);
    int l = 0;
    for (int i = 1; i < L; ++i)
        if (lb >= lt.bin_off[i]) l = i;
    const int sh = lt.bin_shift[l];  // 0..4
    const int log2rep = 4 - sh;
    const int64_t HW = (int64_t)lt.H[l] * lt.W[l];
    const int64_t r0 = (int64_t)(lb - lt.bin_off[l]) << sh;
    const int rows = (int)(((int64_t)1 << sh) < HW - r0 ? ((int64_t)1 << sh) : HW - r0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = tid & (G - 1);
    const int gid = tid >> 4;
    const int nslots = D / SLOT;
    const int64_t MD = (int64_t)M * D;
    // grad_output rows of batch b, head m: row q at byte q * MD * e
    const E *gq = grad_out + (b * Q * M + m) * (int64_t)D;
    const Slice<true> gslice(gq, (Q - 1) * MD * (int64_t)sizeof(E) + D * (int64_t)sizeof(E));
    const uint32_t row_bytes = (uint32_t)(MD * (int64_t)sizeof(E));
    uint32_t soff[J];
    bool slot_ok[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        slot_ok[j] = c + j * G < nslots;
        soff[j] = (uint32_t)((c + j * G) * SLOT * (int)sizeof(E));
    }
    float acc[J][SLOT];
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int v = 0; v < SLOT; ++v) acc[j][v] = 0.0f;
    float accw[VW];
#pragma unroll
    for (int v = 0; v < VW; ++v) accw[v] = 0.0f;
    const int sub = c >> 2;                     // wide mode: record of four
    const uint32_t lbytes = (uint32_t)(c & 3) * 16u;  // wide mode: 16-byte chunk of the row

    const uint32_t rb = starts[bin], re = ends[bin];
    // kAccRPT records per thread per round; record k of a round is
    // base + k * kBlock + tid (the next round's are loaded before this one is
    // processed; an empty bin reads nothing)
    uint2 next[kAccRPT];
#pragma unroll
    for (int k = 0; k < kAccRPT; ++k) {
        const uint32_t i = rb + k * kBlock + tid;
        next[k] = rb < re ? records[i < re ? i : re - 1] : make_uint2(0u, 0u);
    }
    static_assert(kAccGroups * kWaves == 64, "one counter per lane of wave 0");
    if (tid < 64) wcount[tid] = 0u;
    __syncthreads();
    for (uint32_t base = rb; base < re; base += kAccRPT * kBlock) {
        uint2 rec[kAccRPT];
        bool valid[kAccRPT];
        uint32_t slot[kAccRPT];
#pragma unroll
        for (int k = 0; k < kAccRPT; ++k) {
            rec[k] = next[k];
            const uint32_t i = base + k * kBlock + tid;
            valid[k] = i < re;
            const uint32_t ni = i + kAccRPT * kBlock;
            if (base + kAccRPT * kBlock < re) next[k] = records[ni < re ? ni : re - 1];
            uint32_t rr = rec[k].x & 15u;
            rr = rr < (uint32_t)rows ? rr : 0u;  // keeps every access in range
            slot[k] = (rr << log2rep) | (i & ((1u << log2rep) - 1u));
        }
        // each record's rank among this wave's records of its slot: a
        // returning add on the wave's own counter of the slot (record index
        // k = 0 first, so records k' < k of a slot come first in its run)
        uint32_t rank[kAccRPT];
#pragma unroll
        for (int k = 0; k < kAccRPT; ++k)
            rank[k] = valid[k] ? atomicAdd(&wcount[slot[k] * kWaves + wave], 1u) : 0u;
        __syncthreads();  // every wave's counts in; the previous round's records and offsets consumed
        if (wave == 0) {  // exclusive scan of the 64 counts, slot-major; counts cleared for the next round
            const uint32_t x = wcount[lane];
            wcount[lane] = 0u;
            uint32_t inc = x;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t y = __shfl_up(inc, off);
                if (lane >= off) inc += y;
            }
            woff[lane] = inc - x;
            if (lane == 63) woff[64] = inc;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kAccRPT; ++k)
            if (valid[k]) sorted[woff[slot[k] * kWaves + wave] + rank[k]] = rec[k];
        __syncthreads();
        const uint32_t first = woff[gid * kWaves], n = woff[gid * kWaves + kWaves] - first;
        // a record past the slot's end reads neither LDS past the round nor
        // its row: coefficient 0 and a zero row, whatever grad_output holds
        if constexpr (WIDE) {
            static_assert(UW == 4, "one record per lane of a sub-group");
            for (uint32_t i0 = 0; __ballot(i0 < n); i0 += 4 * UW) {
                // lane k of the sub-group (an aligned quad) decodes its record
                // u = k, out-of-range offset past the slot's end, and the quad
                // broadcasts each record's coefficient and row offset
                const uint32_t idx = i0 + 4 * (c & 3) + sub;
                const bool okk = idx < n;
                const uint2 rc = sorted[okk ? first + idx : 0u];
                const float ck = __uint_as_float(rc.y & (0u - (uint32_t)okk));
                const uint32_t rq = rc.x >> 4;
                const uint32_t ok_off = okk ? (rq < (uint64_t)Q ? rq : 0u) * row_bytes : kOutOfRange;
                const float coef[UW] = {quad_bcast<0>(ck), quad_bcast<1>(ck), quad_bcast<2>(ck),
                                        quad_bcast<3>(ck)};
                // kOutOfRange plus the chunk's bytes is still past the slice
                const uint32_t qo[UW] = {quad_bcast<0>(ok_off) + lbytes, quad_bcast<1>(ok_off) + lbytes,
                                         quad_bcast<2>(ok_off) + lbytes, quad_bcast<3>(ok_off) + lbytes};
                uint4 gr[UW];
#pragma unroll
                for (int u = 0; u < UW; ++u) gr[u] = buffer_load_raw<16>(gslice.rsrc, qo[u]);
                __builtin_amdgcn_sched_barrier(0);  // every gather issued before any use
#pragma unroll
                for (int u = 0; u < UW; ++u) {
                    float gv[VW];
                    if constexpr (std::is_same<DT, BF16T>::value) {
                        const uint32_t w4[4] = {gr[u].x, gr[u].y, gr[u].z, gr[u].w};
#pragma unroll
                        for (int h = 0; h < 4; ++h) {  // bf16 pair -> two floats
                            gv[2 * h] = __uint_as_float(w4[h] << 16);
                            gv[2 * h + 1] = __uint_as_float(w4[h] & 0xFFFF0000u);
                        }
                    } else {
                        raw_to_f32<DT, VW>(gr[u], gv);
                    }
#pragma unroll
                    for (int v = 0; v < VW; ++v) accw[v] = __builtin_fmaf(coef[u], gv[v], accw[v]);
                }
            }
            continue;
        }
        for (uint32_t i0 = 0; __ballot(i0 < n); i0 += U) {
            float coef[U];
            uint32_t qo[U];
            bool okr[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                okr[u] = i0 + u < n;
                const uint2 rc = sorted[okr[u] ? first + i0 + u : 0u];
                coef[u] = okr[u] ? __uint_as_float(rc.y) : 0.0f;
                const uint32_t rq = rc.x >> 4;
                qo[u] = (rq < (uint64_t)Q ? rq : 0u) * row_bytes;
            }
            R gr[U][J];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int j = 0; j < J; ++j)
                    gr[u][j] = gslice.template gather<R>(qo[u] + soff[j], slot_ok[j] && okr[u]);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    float gv[SLOT];
                    raw_to_f32<DT, SLOT>(gr[u][j], gv);
#pragma unroll
                    for (int v = 0; v < SLOT; ++v) acc[j][v] = __builtin_fmaf(coef[u], gv[v], acc[j][v]);
                }
        }
    }
    // every group's sums (zeros for a group without records) -> tile row gid
    if constexpr (WIDE) {
#pragma unroll
        for (int v = 0; v < VW; ++v) {
            accw[v] += __shfl_xor(accw[v], 4);
            accw[v] += __shfl_xor(accw[v], 8);
        }
        if (sub == 0)
#pragma unroll
            for (int v = 0; v < VW; ++v) tile[gid * D + (c & 3) * VW + v] = accw[v];
    } else {
#pragma unroll
        for (int j = 0; j < J; ++j)
            if (slot_ok[j])
#pragma unroll
                for (int v = 0; v < SLOT; ++v) tile[gid * D + (c + j * G) * SLOT + v] = acc[j][v];
    }
    __syncthreads();
    E *dst = grad_value + ((b * S + lt.start[l] + r0) * M + m) * (int64_t)D;
    const int vpr = D / V;
    const int nrep = 1 << log2rep;
    for (int i = tid; i < rows * vpr; i += kBlock) {
        const int rr = i / vpr, cv = i - rr * vpr;
        E *d = dst + (int64_t)rr * MD + cv * V;
        float v[V];
#pragma unroll
        for (int k = 0; k < V; ++k) v[k] = 0.0f;
        for (int r = 0; r < nrep; ++r) {
            const float *t = tile + ((rr << log2rep) + r) * D + cv * V;
#pragma unroll
            for (int k = 0; k < V; ++k) v[k] += t[k];
        }
        if (accumulate) {
            float o[V];
            load_vec<DT, V>(d, o);
#pragma unroll
            for (int k = 0; k < V; ++k) v[k] += o[k];
        }
        store_vec<DT, V>(d, v);
    }
}

template <class DT, int SLOT, int J, int V, bool WIDE>
__global__ __launch_bounds__(kBlock) void bin_accum_kernel(
    const typename DT::S *__restrict__ grad_out, typename DT::S *__restrict__ grad_value,
    const uint32_t *__restrict__ starts, const uint32_t *__restrict__ ends,
    const uint2 *__restrict__ records, const LevelTable lt, const int64_t S, const int64_t Q,
    const int M, const int D, const int L, const int64_t nbbm, const int64_t nbins,
    const int accumulate) {
    extern __shared__ float dyn_tile[];  // kAccGroups x D
    const int64_t bin = logical_block();  // neighbouring bins share upstream-gradient rows
    if (bin >= nbins) return;
    accum_bin<DT, SLOT, J, V, WIDE>(dyn_tile, MSDA_ACCUM_ARGS, bin);
}

// The unbinned levels' atomic scatter and the binned levels' accumulation in
// one launch: they touch disjoint grad_value rows and depend only on work
// already finished (zero fill, bin sort), so their workgroups share the chip;
// the accumulation's latency-bound rounds fill the gaps of the scatter's
// atomic-bound stream. Workgroups come in rows of 8 (one per XCD); of the
// R = gridDim / 8 rows, Rs = nsc / 8 scatter and the others accumulate,
// spread evenly over the grid so both run from the start. The accumulation
// keeps its own kernel's XCD-aware order (neighbouring bins on one XCD);
// scatter tiles are dealt to the XCDs in turn, so every XCD's atomics cover
// all heads and batches rather than a block of 4 heads of one batch, whose
// rows would fill only half of each pixel's 8 heads' rows (measured:
// scatter launch 21.7-22.3 -> 21.4-21.8 us on the decoder; nsc is a multiple
// of 8).
template <class DT, class PT, int SLOT, int J, int V, bool WIDE>
__global__ __launch_bounds__(kBlock) void scatter_accum_kernel(
    const typename PT::S *__restrict__ loc, const typename PT::S *__restrict__ attn,
    const typename DT::S *__restrict__ grad_out, void *__restrict__ grad_value,
    const LevelTable lt, const int64_t S, const int64_t Q, const int M, const int D, const int L,
    const int K, const int qblocks, const int64_t ntiles, const int log2g, const int log2s,
    const uint32_t nsc, const uint32_t *__restrict__ starts, const uint32_t *__restrict__ ends,
    const uint2 *__restrict__ records, const int64_t nbbm, const int64_t nbins,
    const int accumulate) {
    extern __shared__ float dyn_tile[];
    const uint32_t bx = blockIdx.x, xcd = bx % kXcds;
    const int64_t r = bx / kXcds, R = gridDim.x / kXcds, Rs = nsc / kXcds;
    const int64_t k = r * Rs / R;  // scatter rows before row r
    if ((r + 1) * Rs / R > k) {    // row r is scatter row k
        const int64_t tile = k * kXcds + xcd;
        if (tile < ntiles) {
            float *workspace = nullptr;
            scatter_tile<DT, PT, SLOT, J>(MSDA_SCATTER_ARGS, tile);
        }
    } else {
        const int64_t bin = (int64_t)xcd * (R - Rs) + (r - k);
        if (bin < nbins) {
            typename DT::S *gv = static_cast<typename DT::S *>(grad_value);
            accum_bin<DT, SLOT, J, V, WIDE>(dyn_tile, grad_out, gv, starts, ends, records, lt, S, Q, M,
                                      D, L, nbbm, accumulate, bin);
        }
    }
}

// ------------------------------------------------ zero fill and scratch add

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

// blockIdx.y = scratch level index (into lvl); the level's fp32 block
// (B, H*W, M, D) is added into grad_value rows [start, start + H*W) of every
// batch, 4 elements at a time (host-checked alignment and divisibility) or 1.
struct ScratchLevels {
    int32_t level[MSDA_MAX_LEVELS];
    int32_t count;
};

template <class DT, int V>
__global__ __launch_bounds__(kBlock) void scratch_add_kernel(const float *__restrict__ ws,
                                                             typename DT::S *__restrict__ gv,
                                                             const LevelTable lt,
                                                             const ScratchLevels sl,
                                                             const int64_t B, const int64_t S,
                                                             const int64_t MD) {
    using E = typename DT::S;
    const int l = sl.level[blockIdx.y];
    const int64_t n = (int64_t)lt.H[l] * lt.W[l] * MD;  // elements per batch
    const int64_t total = B * n;
    const float *src = ws + lt.scratch_off[l];
    const int64_t start = lt.start[l];
    for (int64_t i = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * V; i < total;
         i += (int64_t)gridDim.x * kBlock * V) {
        const int64_t bb = i / n, off = i - bb * n;
        E *dst = gv + (bb * S + start) * MD + off;
        float acc[V], old[V];
        load_vec<F32T, V>(src + i, acc);
        load_vec<DT, V>(dst, old);
#pragma unroll
        for (int u = 0; u < V; ++u) acc[u] += old[u];
        store_vec<DT, V>(dst, acc);
    }
}

int grid_for(int64_t work_items) {
    const int64_t blocks = (work_items + kBlock - 1) / kBlock;
    const int64_t cap = 256 * 16;  // enough to fill 256 CUs several times over
    return (int)(blocks < 1 ? 1 : (blocks > cap ? cap : blocks));
}

// ------------------------------------------------------------ dispatch

// The queries are the pyramid's own pixels in S order: Q == S and the levels
// tile [0, S) without overlap.
bool pixel_queries(const Problem &p) {
    if (p.Q != p.S) return false;
    int64_t covered = 0;
    for (int i = 0; i < (int)p.L; ++i) {
        const int64_t a0 = p.levels.start[i], a1 = a0 + (int64_t)p.levels.H[i] * p.levels.W[i];
        covered += a1 - a0;
        for (int k = i + 1; k < (int)p.L; ++k) {
            const int64_t b0 = p.levels.start[k], b1 = b0 + (int64_t)p.levels.H[k] * p.levels.W[k];
            if (a0 < b1 && b0 < a1) return false;
        }
    }
    return covered == p.S;
}

// Tile order and tile count of the forward / gradient kernels (TileOrder):
// column groups for pixel queries with fewer (b, head group) pairs than XCDs
// (as many groups as give every XCD one region), else linear.
TileOrder tile_order(const Problem &p, int log2qs, int ngroups, int64_t *ntiles) {
    TileOrder to = {0, 0};
    const int qs = 1 << log2qs;
    const int64_t qblocks = (p.Q + qs - 1) / qs;
    *ntiles = p.B * ngroups * qblocks;
    const int64_t bg = p.B * ngroups;
    if (!pixel_queries(p) || bg >= kXcds || kXcds % bg != 0)
        return to;
    const int nc = (int)(kXcds / bg);
    int64_t per_region = 0;
    for (int c = 0; c < nc; ++c) {
        int64_t n = 0;
        for (int l = 0; l < (int)p.L; ++l) {
            uint32_t x0, x1;
            n += (int64_t)p.levels.H[l] *
                 group_columns((uint32_t)p.levels.W[l], (uint32_t)c, (uint32_t)nc, log2qs, &x0, &x1);
        }
        per_region = std::max(per_region, n);
    }
    if (bg * nc * per_region >= ((int64_t)1 << 31)) return to;  // 32-bit tile arithmetic
    to = {nc, (int32_t)per_region};
    *ntiles = bg * nc * per_region;
    return to;
}

// Chunk-owner parameter loads may use vector loads: no point split, whole
// chunks of `ch` points, and the chunk's locations / weights aligned for 16-
// and 8- (16-bit) or 16-byte (fp32) loads.
bool params_vectorizable(const Problem &p, int log2s, int ch, const void *loc, const void *attn) {
    const uintptr_t e = p.pdtype == MSDA_F32 ? 4 : 2;
    return log2s == 0 && (p.L * p.K) % ch == 0 && reinterpret_cast<uintptr_t>(loc) % 16 == 0 &&
           reinterpret_cast<uintptr_t>(attn) % (e == 2 ? 8 : 16) == 0;
}

}  // namespace

// Buffer gathers address one batch slice with 32-bit offsets (unless a test
// forces the plain-load path, msda_debug_force_flat_gathers).
bool slice_fits_buffer(const Problem &p) {
    const int64_t e = p.dtype == MSDA_F32 ? 4 : 2;
    return p.S * p.M * p.D * e <= (int64_t)kOutOfRange - 64 && !flat_gathers_forced();
}

namespace {

template <class DT, class PT, int VEC>
hipError_t fwd_launch(const Problem &p, const Mapping &mp, const void *value, const void *loc,
                      const void *attn, void *out, hipStream_t stream) {
    // 4 points per chunk; 16-byte gathers keep 16 x 4 VGPRs of raw data in flight
    constexpr int CH = 4;
    using E = typename DT::S;
    using P = typename PT::S;
    const int qpb = kBlock >> (mp.log2_group + mp.log2_split);
    const int hg = fwd_heads((int)p.M, qpb, (int)(p.D * (int64_t)sizeof(typename DT::S)));
    const int qblocks = (int)((p.Q + qpb / hg - 1) / (qpb / hg));
    int64_t ntiles;
    const int log2qs = 8 - mp.log2_group - mp.log2_split - (hg == 4 ? 2 : hg == 2 ? 1 : 0);
    const TileOrder to = tile_order(p, log2qs, (int)(p.M / hg), &ntiles);
    const int64_t per_xcd = (ntiles + kXcds - 1) / kXcds;
    // the quad setup (see msda_fwd_kernel)
    const int64_t per_lane = (p.L * p.K) >> mp.log2_split;
    const bool quad = mp.log2_group == 2 && p.D == 4 * VEC && per_lane <= (CH << 2) &&
                      p.K % ((int64_t)CH << mp.log2_split) == 0;
    if constexpr (VEC * sizeof(E) == 16) {  // 16-byte lane vectors: 64-byte fp16 / bf16 or fp32 rows
        if (slice_fits_buffer(p) && quad) {
            MSDA_LAUNCH((msda_fwd_kernel<DT, PT, VEC, CH, true, true>),
                        dim3((unsigned)(per_xcd * kXcds)), dim3(kBlock), 0, stream,
                        static_cast<const E *>(value), static_cast<const P *>(loc),
                        static_cast<const P *>(attn), static_cast<E *>(out), p.levels, p.S, p.Q,
                        (int)p.M, (int)p.D, (int)p.L, (int)p.K, qblocks, ntiles, mp.log2_group,
                        mp.log2_split, to, params_vectorizable(p, mp.log2_split, CH, loc, attn));
            return hipGetLastError();
        }
    }
    if (slice_fits_buffer(p))
        MSDA_LAUNCH((msda_fwd_kernel<DT, PT, VEC, CH, true, false>), dim3((unsigned)(per_xcd * kXcds)),
                           dim3(kBlock), 0, stream, static_cast<const E *>(value),
                           static_cast<const P *>(loc), static_cast<const P *>(attn),
                           static_cast<E *>(out), p.levels, p.S, p.Q, (int)p.M, (int)p.D,
                           (int)p.L, (int)p.K, qblocks, ntiles, mp.log2_group, mp.log2_split, to,
                           params_vectorizable(p, mp.log2_split, CH, loc, attn));
    else if constexpr (std::is_same<DT, PT>::value)
        MSDA_LAUNCH((msda_fwd_kernel<DT, PT, VEC, CH, false, false>), dim3((unsigned)(per_xcd * kXcds)),
                           dim3(kBlock), 0, stream, static_cast<const E *>(value),
                           static_cast<const P *>(loc), static_cast<const P *>(attn),
                           static_cast<E *>(out), p.levels, p.S, p.Q, (int)p.M, (int)p.D,
                           (int)p.L, (int)p.K, qblocks, ntiles, mp.log2_group, mp.log2_split, to,
                           params_vectorizable(p, mp.log2_split, CH, loc, attn));
    else
        return hipErrorInvalidValue;  // mixed dtypes need a buffer-addressable slice
    return hipGetLastError();
}

template <class DT, class PT, int VEC>
hipError_t grad_launch(const Problem &p, const Mapping &mp, const void *value, const void *loc,
                       const void *attn, const void *grad_out, void *grad_loc, void *grad_attn,
                       hipStream_t stream) {
    constexpr int CH = 4;
    using E = typename DT::S;
    using P = typename PT::S;
    const int qpb = kBlock >> (mp.log2_group + mp.log2_split);
    const int hg = grad_heads((int)p.M, qpb);
    const int qblocks = (int)((p.Q + qpb / hg - 1) / (qpb / hg));
    int64_t ntiles;
    const int log2qs = 8 - mp.log2_group - mp.log2_split - (hg == 4 ? 2 : hg == 2 ? 1 : 0);
    const TileOrder to = tile_order(p, log2qs, (int)(p.M / hg), &ntiles);
    const int64_t per_xcd = (ntiles + kXcds - 1) / kXcds;
    if (!slice_fits_buffer(p)) return hipErrorInvalidValue;  // binning requires it
    if constexpr (VEC * sizeof(E) == 16) {  // the quad setup (see grad_tile)
        const int64_t per_lane = (p.L * p.K) >> mp.log2_split;
        if (mp.log2_group == 2 && p.D == 4 * VEC && per_lane <= (CH << 2) &&
            p.K % ((int64_t)CH << mp.log2_split) == 0) {
            MSDA_LAUNCH((msda_grad_kernel<DT, PT, VEC, CH, true, true>),
                        dim3((unsigned)(per_xcd * kXcds)), dim3(kBlock), 0, stream,
                        static_cast<const E *>(value), static_cast<const P *>(loc),
                        static_cast<const P *>(attn), static_cast<const E *>(grad_out),
                        static_cast<P *>(grad_loc), static_cast<P *>(grad_attn), p.levels, p.S,
                        p.Q, (int)p.M, (int)p.D, (int)p.L, (int)p.K, qblocks, ntiles,
                        mp.log2_group, mp.log2_split, to,
                        params_vectorizable(p, mp.log2_split, CH, loc, attn));
            return hipGetLastError();
        }
    }
    MSDA_LAUNCH((msda_grad_kernel<DT, PT, VEC, CH, true, false>), dim3((unsigned)(per_xcd * kXcds)),
                       dim3(kBlock), 0, stream, static_cast<const E *>(value),
                       static_cast<const P *>(loc), static_cast<const P *>(attn),
                       static_cast<const E *>(grad_out), static_cast<P *>(grad_loc),
                       static_cast<P *>(grad_attn), p.levels, p.S, p.Q, (int)p.M, (int)p.D,
                       (int)p.L, (int)p.K, qblocks, ntiles, mp.log2_group, mp.log2_split, to,
                       params_vectorizable(p, mp.log2_split, CH, loc, attn));
    return hipGetLastError();
}

template <class DT, class PT, int SLOT, int J>
hipError_t bwd_launch(const Problem &p, const BwdMapping &mp, const void *value, const void *loc,
                      const void *attn, const void *grad_out, void *grad_value, float *workspace,
                      void *grad_loc, void *grad_attn, hipStream_t stream) {
    using E = typename DT::S;
    using P = typename PT::S;
    const int qpb = kBlock >> (mp.log2_group + mp.log2_split);
    const int qblocks = (int)((p.Q + qpb - 1) / qpb);
    const int64_t ntiles = p.B * p.M * qblocks;
    const int64_t per_xcd = (ntiles + kXcds - 1) / kXcds;
    if (slice_fits_buffer(p))
        MSDA_LAUNCH((msda_bwd_kernel<DT, PT, SLOT, J, true>),
                           dim3((unsigned)(per_xcd * kXcds)), dim3(kBlock), 0, stream,
                           static_cast<const E *>(value), static_cast<const P *>(loc),
                           static_cast<const P *>(attn), static_cast<const E *>(grad_out),
                           grad_value, workspace, static_cast<P *>(grad_loc),
                           static_cast<P *>(grad_attn), p.levels, p.S, p.Q, (int)p.M, (int)p.D,
                           (int)p.L, (int)p.K, qblocks, ntiles, mp.log2_group, mp.log2_split);
    else if constexpr (std::is_same<DT, PT>::value)
        MSDA_LAUNCH((msda_bwd_kernel<DT, PT, SLOT, J, false>),
                           dim3((unsigned)(per_xcd * kXcds)), dim3(kBlock), 0, stream,
                           static_cast<const E *>(value), static_cast<const P *>(loc),
                           static_cast<const P *>(attn), static_cast<const E *>(grad_out),
                           grad_value, workspace, static_cast<P *>(grad_loc),
                           static_cast<P *>(grad_attn), p.levels, p.S, p.Q, (int)p.M, (int)p.D,
                           (int)p.L, (int)p.K, qblocks, ntiles, mp.log2_group, mp.log2_split);
    else
        return hipErrorInvalidValue;  // mixed dtypes need a buffer-addressable slice
    return hipGetLastError();
}

// The accumulation reads 16 bytes per lane when a row is exactly 64 bytes
// (J == 1) and grad_output is 16-byte aligned.
template <class DT, int SLOT, int J>
bool accum_wide(const Problem &p, const void *grad_out) {
    constexpr int e = (int)sizeof(typename DT::S);
    return J == 1 && SLOT * e == 4 && p.D * e == 64 &&
           reinterpret_cast<uintptr_t>(grad_out) % 16 == 0;
}

template <class DT, int SLOT, int J, int V, bool WIDE>
hipError_t accum_launch_w(const Problem &p, const BwdMapping &mp, const void *grad_out,
                          void *grad_value, const BinnedBuffers &bins, bool accumulate,
                          hipStream_t stream) {
    using E = typename DT::S;
    const size_t lds = (size_t)kAccGroups * (size_t)p.D * sizeof(float);
    const int64_t per_xcd = (bins.nbins + kXcds - 1) / kXcds;
    MSDA_LAUNCH((bin_accum_kernel<DT, SLOT, J, V, WIDE>), dim3((unsigned)(per_xcd * kXcds)),
                       dim3(kBlock), lds, stream, static_cast<const E *>(grad_out),
                       static_cast<E *>(grad_value), bins.starts, bins.ends, bins.records, p.levels, p.S,
                       p.Q, (int)p.M, (int)p.D, (int)p.L, p.nbbm, bins.nbins, (int)accumulate);
    return hipGetLastError();
}

template <class DT, int SLOT, int J, int V>
hipError_t accum_launch_v(const Problem &p, const BwdMapping &mp, const void *grad_out,
                          void *grad_value, const BinnedBuffers &bins, bool accumulate,
                          hipStream_t stream) {
    if constexpr (J == 1 && SLOT * sizeof(typename DT::S) == 4)
        if (accum_wide<DT, SLOT, J>(p, grad_out))
            return accum_launch_w<DT, SLOT, J, V, true>(p, mp, grad_out, grad_value, bins,
                                                        accumulate, stream);
    return accum_launch_w<DT, SLOT, J, V, false>(p, mp, grad_out, grad_value, bins, accumulate,
                                                 stream);
}

// Write-back width: the widest of 16, 8, 4 bytes (or one element) that
// divides a row and to which grad_value is aligned.
template <class DT, int SLOT, int J>
hipError_t accum_launch(const Problem &p, const BwdMapping &mp, const void *grad_out,
                        void *grad_value, const BinnedBuffers &bins, bool accumulate,
                        hipStream_t stream) {
    constexpr int e = (int)sizeof(typename DT::S);
    const uintptr_t a = reinterpret_cast<uintptr_t>(grad_value);
    auto fits = [&](int v) { return p.D % v == 0 && a % (uintptr_t)(v * e) == 0; };
    if (fits(16 / e)) return accum_launch_v<DT, SLOT, J, 16 / e>(p, mp, grad_out, grad_value, bins, accumulate, stream);
    if (fits(8 / e)) return accum_launch_v<DT, SLOT, J, 8 / e>(p, mp, grad_out, grad_value, bins, accumulate, stream);
    if constexpr (e == 2)
        if (fits(2)) return accum_launch_v<DT, SLOT, J, 2>(p, mp, grad_out, grad_value, bins, accumulate, stream);
    return accum_launch_v<DT, SLOT, J, 1>(p, mp, grad_out, grad_value, bins, accumulate, stream);
}

template <class DT, class PT>
hipError_t fwd_by_vec(const Problem &p, const Mapping &mp, const void *v, const void *l,
                      const void *a, void *o, hipStream_t st) {
    switch (mp.vec) {
        case 1: return fwd_launch<DT, PT, 1>(p, mp, v, l, a, o, st);
        case 2: return fwd_launch<DT, PT, 2>(p, mp, v, l, a, o, st);
        case 4: return fwd_launch<DT, PT, 4>(p, mp, v, l, a, o, st);
        default: break;
    }
    if constexpr (sizeof(typename DT::S) == 4) {
        if (mp.vec == 3) return fwd_launch<DT, PT, 3>(p, mp, v, l, a, o, st);
    } else {
        if (mp.vec == 8) return fwd_launch<DT, PT, 8>(p, mp, v, l, a, o, st);
    }
    return hipErrorInvalidValue;
}

template <class DT, class PT, int SLOT, int J>
hipError_t scatter_launch(const Problem &p, const BwdMapping &mp, const void *loc, const void *attn,
                          const void *grad_out, void *grad_value, float *workspace,
                          hipStream_t stream) {
    using E = typename DT::S;
    using P = typename PT::S;
    const int qpb = kBlock >> (mp.log2_group + mp.log2_split);
    const int qblocks = (int)((p.Q + qpb - 1) / qpb);
    const int64_t ntiles = p.B * p.M * qblocks;
    const int64_t per_xcd = (ntiles + kXcds - 1) / kXcds;
    MSDA_LAUNCH((msda_scatter_kernel<DT, PT, SLOT, J>), dim3((unsigned)(per_xcd * kXcds)),
                       dim3(kBlock), 0, stream, static_cast<const P *>(loc),
                       static_cast<const P *>(attn), static_cast<const E *>(grad_out), grad_value,
                       workspace, p.levels, p.S, p.Q, (int)p.M, (int)p.D, (int)p.L, (int)p.K,
                       qblocks, ntiles, mp.log2_group, mp.log2_split);
    return hipGetLastError();
}

template <class DT, class PT, int SLOT>
hipError_t scatter_by_j(const Problem &p, const BwdMapping &mp, const void *l, const void *a,
                        const void *go, void *gv, float *ws, hipStream_t st) {
    switch (mp.j) {
        case 1: return scatter_launch<DT, PT, SLOT, 1>(p, mp, l, a, go, gv, ws, st);
        case 2: return scatter_launch<DT, PT, SLOT, 2>(p, mp, l, a, go, gv, ws, st);
        case 3: return scatter_launch<DT, PT, SLOT, 3>(p, mp, l, a, go, gv, ws, st);
        case 4: return scatter_launch<DT, PT, SLOT, 4>(p, mp, l, a, go, gv, ws, st);
        case 8: return scatter_launch<DT, PT, SLOT, 8>(p, mp, l, a, go, gv, ws, st);
        case 16: return scatter_launch<DT, PT, SLOT, 16>(p, mp, l, a, go, gv, ws, st);
        default: break;
    }
    if constexpr (SLOT == 1) {
        if (mp.j == 32) return scatter_launch<DT, PT, SLOT, 32>(p, mp, l, a, go, gv, ws, st);
    }
    return hipErrorInvalidValue;
}

template <class DT, class PT, int SLOT>
hipError_t bwd_by_j(const Problem &p, const BwdMapping &mp, const void *v, const void *l,
                    const void *a, const void *go, void *gv, float *ws, void *gl, void *ga,
                    hipStream_t st) {
    switch (mp.j) {
        case 1: return bwd_launch<DT, PT, SLOT, 1>(p, mp, v, l, a, go, gv, ws, gl, ga, st);
        case 2: return bwd_launch<DT, PT, SLOT, 2>(p, mp, v, l, a, go, gv, ws, gl, ga, st);
        case 3: return bwd_launch<DT, PT, SLOT, 3>(p, mp, v, l, a, go, gv, ws, gl, ga, st);
        case 4: return bwd_launch<DT, PT, SLOT, 4>(p, mp, v, l, a, go, gv, ws, gl, ga, st);
        case 8: return bwd_launch<DT, PT, SLOT, 8>(p, mp, v, l, a, go, gv, ws, gl, ga, st);
        case 16: return bwd_launch<DT, PT, SLOT, 16>(p, mp, v, l, a, go, gv, ws, gl, ga, st);
        default: break;
    }
    if constexpr (SLOT == 1) {
        if (mp.j == 32) return bwd_launch<DT, PT, SLOT, 32>(p, mp, v, l, a, go, gv, ws, gl, ga, st);
    }
    return hipErrorInvalidValue;
}

template <class DT, class PT>
hipError_t grad_by_vec(const Problem &p, const Mapping &mp, const void *v, const void *l,
                       const void *a, const void *go, void *gl, void *ga, hipStream_t st) {
    switch (mp.vec) {
        case 1: return grad_launch<DT, PT, 1>(p, mp, v, l, a, go, gl, ga, st);
        case 2: return grad_launch<DT, PT, 2>(p, mp, v, l, a, go, gl, ga, st);
        case 4: return grad_launch<DT, PT, 4>(p, mp, v, l, a, go, gl, ga, st);
        default: break;
    }
    if constexpr (sizeof(typename DT::S) == 4) {
        if (mp.vec == 3) return grad_launch<DT, PT, 3>(p, mp, v, l, a, go, gl, ga, st);
    } else {
        if (mp.vec == 8) return grad_launch<DT, PT, 8>(p, mp, v, l, a, go, gl, ga, st);
    }
    return hipErrorInvalidValue;
}

template <class DT, int SLOT>
hipError_t accum_by_j(const Problem &p, const BwdMapping &mp, const void *go, void *gv,
                      const BinnedBuffers &bn, bool acc, hipStream_t st) {
    switch (mp.j) {
        case 1: return accum_launch<DT, SLOT, 1>(p, mp, go, gv, bn, acc, st);
        case 2: return accum_launch<DT, SLOT, 2>(p, mp, go, gv, bn, acc, st);
        case 3: return accum_launch<DT, SLOT, 3>(p, mp, go, gv, bn, acc, st);
        case 4: return accum_launch<DT, SLOT, 4>(p, mp, go, gv, bn, acc, st);
        case 8: return accum_launch<DT, SLOT, 8>(p, mp, go, gv, bn, acc, st);
        case 16: return accum_launch<DT, SLOT, 16>(p, mp, go, gv, bn, acc, st);
        default: break;
    }
    if constexpr (SLOT == 1) {
        if (mp.j == 32) return accum_launch<DT, SLOT, 32>(p, mp, go, gv, bn, acc, st);
    }
    return hipErrorInvalidValue;
}

template <class DT>
hipError_t scratch_add(const Problem &p, const float *ws, void *gv, hipStream_t stream) {
    using E = typename DT::S;
    ScratchLevels sl;
    sl.count = 0;
    int64_t largest = 0;
    for (int l = 0; l < (int)p.L; ++l) {
        if (p.levels.scratch_off[l] < 0) continue;
        sl.level[sl.count++] = l;
        const int64_t n = p.B * (int64_t)p.levels.H[l] * p.levels.W[l] * p.M * p.D;
        if (n > largest) largest = n;
    }
    if (sl.count == 0) return hipSuccess;
    // Levels whose row ranges overlap (a caller-given level_start_index) would
    // read-modify-write the same grad_value rows from concurrent workgroups:
    // then add one level per launch, in stream order.
    bool overlap = false;
    for (int i = 0; i < sl.count && !overlap; ++i)
        for (int k = i + 1; k < sl.count && !overlap; ++k) {
            const int a = sl.level[i], b = sl.level[k];
            const int64_t a0 = p.levels.start[a], a1 = a0 + (int64_t)p.levels.H[a] * p.levels.W[a];
            const int64_t b0 = p.levels.start[b], b1 = b0 + (int64_t)p.levels.H[b] * p.levels.W[b];
            overlap = a0 < b1 && b0 < a1;
        }
    if (overlap && sl.count > 1) {
        for (int i = 0; i < sl.count; ++i) {
            Problem one = p;
            for (int l = 0; l < (int)p.L; ++l)
                if (l != sl.level[i]) one.levels.scratch_off[l] = -1;
            const hipError_t err = scratch_add<DT>(one, ws, gv, stream);
            if (err != hipSuccess) return err;
        }
        return hipSuccess;
    }
    const int64_t MD = p.M * p.D;
    // 4-wide when a batch block never splits a group of 4 and both sides are aligned
    const bool v4 = MD % 4 == 0 && reinterpret_cast<uintptr_t>(gv) % 8 == 0 &&
                    reinterpret_cast<uintptr_t>(ws) % 16 == 0;
    if (v4) {
        MSDA_LAUNCH((scratch_add_kernel<DT, 4>), dim3(grid_for(largest / 4), sl.count),
                           dim3(kBlock), 0, stream, ws, static_cast<E *>(gv), p.levels, sl, p.B,
                           p.S, MD);
    } else {
        MSDA_LAUNCH((scratch_add_kernel<DT, 1>), dim3(grid_for(largest), sl.count),
                           dim3(kBlock), 0, stream, ws, static_cast<E *>(gv), p.levels, sl, p.B,
                           p.S, MD);
    }
    return hipGetLastError();
}

}  // namespace

// Parameter type: the value type, or fp32 beside 16-bit values.
#define MSDA_BY_PT(DTT, CALL)                                        \
    (p.pdtype == MSDA_F32 ? CALL(DTT, F32T) : CALL(DTT, DTT))

hipError_t launch_forward(const Problem &p, const Mapping &mp, const void *value,
                          const void *loc, const void *attn, void *out, hipStream_t stream) {
#define MSDA_FWD(T, P) fwd_by_vec<T, P>(p, mp, value, loc, attn, out, stream)
    switch (p.dtype) {
        case MSDA_F32: return MSDA_FWD(F32T, F32T);
        case MSDA_F16: return MSDA_BY_PT(F16T, MSDA_FWD);
        case MSDA_BF16: return MSDA_BY_PT(BF16T, MSDA_FWD);
        default: return hipErrorInvalidValue;
    }
#undef MSDA_FWD
}

hipError_t launch_backward(const Problem &p, const BwdMapping &mp, const void *value,
                           const void *loc, const void *attn, const void *grad_out,
                           void *grad_value, float *workspace, void *grad_loc, void *grad_attn,
                           hipStream_t stream) {
#define MSDA_BWD1(T, P) bwd_by_j<T, P, 1>(p, mp, value, loc, attn, grad_out, grad_value, workspace, grad_loc, grad_attn, stream)
#define MSDA_BWD2(T, P) bwd_by_j<T, P, 2>(p, mp, value, loc, attn, grad_out, grad_value, workspace, grad_loc, grad_attn, stream)
    switch (p.dtype) {
        case MSDA_F32: return MSDA_BWD1(F32T, F32T);
        case MSDA_F16: return mp.slot == 2 ? MSDA_BY_PT(F16T, MSDA_BWD2) : MSDA_BY_PT(F16T, MSDA_BWD1);
        case MSDA_BF16: return mp.slot == 2 ? MSDA_BY_PT(BF16T, MSDA_BWD2) : MSDA_BY_PT(BF16T, MSDA_BWD1);
        default: return hipErrorInvalidValue;
    }
#undef MSDA_BWD1
#undef MSDA_BWD2
}

hipError_t launch_scatter(const Problem &p, const BwdMapping &mp, const void *loc,
                          const void *attn, const void *grad_out, void *grad_value,
                          float *workspace, hipStream_t stream) {
#define MSDA_SC1(T, P) scatter_by_j<T, P, 1>(p, mp, loc, attn, grad_out, grad_value, workspace, stream)
#define MSDA_SC2(T, P) scatter_by_j<T, P, 2>(p, mp, loc, attn, grad_out, grad_value, workspace, stream)
    switch (p.dtype) {
        case MSDA_F32: return MSDA_SC1(F32T, F32T);
        case MSDA_F16: return mp.slot == 2 ? MSDA_BY_PT(F16T, MSDA_SC2) : MSDA_BY_PT(F16T, MSDA_SC1);
        case MSDA_BF16: return mp.slot == 2 ? MSDA_BY_PT(BF16T, MSDA_SC2) : MSDA_BY_PT(BF16T, MSDA_SC1);
        default: return hipErrorInvalidValue;
    }
#undef MSDA_SC1
#undef MSDA_SC2
}

hipError_t launch_gradients(const Problem &p, const Mapping &mp, const void *value,
                            const void *loc, const void *attn, const void *grad_out,
                            void *grad_loc, void *grad_attn, hipStream_t stream) {
#define MSDA_GR(T, P) grad_by_vec<T, P>(p, mp, value, loc, attn, grad_out, grad_loc, grad_attn, stream)
    switch (p.dtype) {
        case MSDA_F32: return MSDA_GR(F32T, F32T);
        case MSDA_F16: return MSDA_BY_PT(F16T, MSDA_GR);
        case MSDA_BF16: return MSDA_BY_PT(BF16T, MSDA_GR);
        default: return hipErrorInvalidValue;
    }
#undef MSDA_GR
}

hipError_t launch_bin_sort(const Problem &p, const void *loc, const void *attn,
                           const BinnedBuffers &bins, bool place, hipStream_t stream) {
    const int64_t wpb = (p.Q * p.levels.nblev * p.K + kBinBlock - 1) / kBinBlock;
    const int64_t ntiles = p.B * p.M * wpb;
    if (ntiles == 0) return hipSuccess;
    const int64_t grid = (ntiles + kXcds - 1) / kXcds * kXcds;
    uint32_t *counter = place ? bins.cursor : bins.starts;
    // Merged records where a query's points cluster: pixel queries sample
    // near their own pixel, so on coarse levels several points of one query
    // share pixels (encoder workload: 32% fewer records, accumulation 298 ->
    // 231 us); elsewhere the comparisons would cost without merging anything.
    // Only place merges: count's totals then bound each bin's records from
    // above, the bin's range keeps an unused tail, and the accumulation ends
    // each bin at its cursor after place.
    const bool merge = place && (p.K == 2 || p.K == 4) && pixel_queries(p);
#define MSDA_SORT(T, PL)                                                                        \
    MSDA_LAUNCH((bin_sort_kernel<T, PL>), dim3((unsigned)grid), dim3(kBinBlock), 0, stream, \
                       static_cast<const typename T::S *>(loc),                                 \
                       static_cast<const typename T::S *>(attn), p.levels, counter,             \
                       bins.records, p.Q, (int)p.M, (int)p.L, (int)p.K, p.nbbm, wpb, ntiles, merge)
    switch (p.pdtype) {  // the kernels read only the parameters
        case MSDA_F32: if (place) MSDA_SORT(F32T, true); else MSDA_SORT(F32T, false); break;
        case MSDA_F16: if (place) MSDA_SORT(F16T, true); else MSDA_SORT(F16T, false); break;
        case MSDA_BF16: if (place) MSDA_SORT(BF16T, true); else MSDA_SORT(BF16T, false); break;
        default: return hipErrorInvalidValue;
    }
#undef MSDA_SORT
    return hipGetLastError();
}

int local_sort_max_points() { return kSortBlock * kSortPts; }

hipError_t launch_bin_local_sort(const Problem &p, const void *loc, const void *attn,
                                 const BinnedBuffers &bins, int max_level_bins, void *zero_dst,
                                 size_t zero_bytes, hipStream_t stream) {
    const int64_t nseg = p.B * p.M * p.levels.nblev;
    if (nseg == 0 || p.Q * p.K > kSortBlock * kSortPts) return hipErrorInvalidValue;
    const size_t lds = (size_t)((max_level_bins + 1) / 2) * 4;
    const int64_t n16 = (int64_t)(zero_bytes / 16);
    const int64_t nzero = n16 > 0 ? std::min<int64_t>((n16 + kSortBlock - 1) / kSortBlock, 1024) : 0;
    if (nseg + nzero >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
#define MSDA_LSORT(T)                                                                          \
    MSDA_LAUNCH((bin_local_sort_kernel<T>), dim3((unsigned)(nseg + nzero)),             \
                       dim3(kSortBlock), lds, stream, static_cast<const typename T::S *>(loc),  \
                       static_cast<const typename T::S *>(attn), p.levels, bins.starts,         \
                       bins.cursor, bins.records, p.Q, (int)p.M, (int)p.L, (int)p.K, p.nbbm,    \
                       nseg, static_cast<uint4 *>(zero_dst), n16)
    switch (p.pdtype) {
        case MSDA_F32: MSDA_LSORT(F32T); break;
        case MSDA_F16: MSDA_LSORT(F16T); break;
        case MSDA_BF16: MSDA_LSORT(BF16T); break;
        default: return hipErrorInvalidValue;
    }
#undef MSDA_LSORT
    return hipGetLastError();
}

template <class DT, class PT, int J, bool WIDE>
hipError_t scatter_accum_launch(const Problem &p, const BwdMapping &mp, const void *loc,
                                const void *attn, const void *grad_out, void *grad_value,
                                const BinnedBuffers &bins, bool accumulate, hipStream_t stream) {
    using E = typename DT::S;
    using P = typename PT::S;
    constexpr int V = 8;  // 16-byte grad_value writes
    const int qpb = kBlock >> (mp.log2_group + mp.log2_split);
    const int qblocks = (int)((p.Q + qpb - 1) / qpb);
    const int64_t ntiles = p.B * p.M * qblocks;
    const int64_t nsc = (ntiles + kXcds - 1) / kXcds * kXcds;
    const int64_t nacc = (bins.nbins + kXcds - 1) / kXcds * kXcds;
    if (nsc + nacc >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const size_t lds = (size_t)kAccGroups * (size_t)p.D * sizeof(float);
    MSDA_LAUNCH((scatter_accum_kernel<DT, PT, 2, J, V, WIDE>), dim3((unsigned)(nsc + nacc)),
                       dim3(kBlock), lds, stream, static_cast<const P *>(loc),
                       static_cast<const P *>(attn), static_cast<const E *>(grad_out), grad_value,
                       p.levels, p.S, p.Q, (int)p.M, (int)p.D, (int)p.L, (int)p.K, qblocks, ntiles,
                       mp.log2_group, mp.log2_split, (uint32_t)nsc, bins.starts, bins.ends,
                       bins.records, p.nbbm, bins.nbins, (int)accumulate);
    return hipGetLastError();
}

template <class DT, class PT>
hipError_t scatter_accum_by_j(const Problem &p, const BwdMapping &mp, const void *loc,
                              const void *attn, const void *grad_out, void *grad_value,
                              const BinnedBuffers &bins, bool accumulate, hipStream_t stream) {
    switch (mp.j) {
        case 1:
            if (accum_wide<DT, 2, 1>(p, grad_out))
                return scatter_accum_launch<DT, PT, 1, true>(p, mp, loc, attn, grad_out, grad_value, bins, accumulate, stream);
            return scatter_accum_launch<DT, PT, 1, false>(p, mp, loc, attn, grad_out, grad_value, bins, accumulate, stream);
        case 2: return scatter_accum_launch<DT, PT, 2, false>(p, mp, loc, attn, grad_out, grad_value, bins, accumulate, stream);
        case 4: return scatter_accum_launch<DT, PT, 4, false>(p, mp, loc, attn, grad_out, grad_value, bins, accumulate, stream);
        default: return hipErrorInvalidValue;
    }
}

bool scatter_accumulate_fits(const Problem &p, const BwdMapping &mp, const void *grad_value) {
    return p.dtype != MSDA_F32 && mp.slot == 2 && (mp.j == 1 || mp.j == 2 || mp.j == 4) &&
           p.D % 8 == 0 && reinterpret_cast<uintptr_t>(grad_value) % 16 == 0;
}

hipError_t launch_scatter_accumulate(const Problem &p, const BwdMapping &mp, const void *loc,
                                     const void *attn, const void *grad_out, void *grad_value,
                                     const BinnedBuffers &bins, bool accumulate,
                                     hipStream_t stream) {
    if (!scatter_accumulate_fits(p, mp, grad_value)) return hipErrorInvalidValue;
    const bool f32p = p.pdtype == MSDA_F32;
    if (p.dtype == MSDA_F16)
        return f32p ? scatter_accum_by_j<F16T, F32T>(p, mp, loc, attn, grad_out, grad_value, bins, accumulate, stream)
                    : scatter_accum_by_j<F16T, F16T>(p, mp, loc, attn, grad_out, grad_value, bins, accumulate, stream);
    return f32p ? scatter_accum_by_j<BF16T, F32T>(p, mp, loc, attn, grad_out, grad_value, bins, accumulate, stream)
                : scatter_accum_by_j<BF16T, BF16T>(p, mp, loc, attn, grad_out, grad_value, bins, accumulate, stream);
}

template <class DT, class PT, int VEC>
hipError_t grad_sort_launch(const Problem &p, const Mapping &mp, const void *value, const void *loc,
                            const void *attn, const void *grad_out, void *grad_loc, void *grad_attn,
                            const BinnedBuffers &bins, int max_level_bins, void *zero_dst,
                            size_t zero_bytes, hipStream_t stream) {
    using E = typename DT::S;
    using P = typename PT::S;
    const int qpb = kBlock >> (mp.log2_group + mp.log2_split);
    const int hg = grad_heads((int)p.M, qpb);
    const int qblocks = (int)((p.Q + qpb / hg - 1) / (qpb / hg));
    const int64_t ntiles = p.B * (p.M / hg) * qblocks;
    const int64_t ngrad = (ntiles + kXcds - 1) / kXcds * kXcds;
    const int64_t nseg = p.B * p.M * p.levels.nblev;
    const int64_t nsegp = (nseg + kXcds - 1) / kXcds * kXcds;
    const int64_t n16 = (int64_t)(zero_bytes / 16);
    // 128 long-running fill workgroups (measured on the decoder: 64 and 256
    // are slower), or fewer for a small fill
    const int64_t nzero =
        n16 > 0 ? std::min<int64_t>((n16 + kBlock - 1) / kBlock + kXcds - 1, 128) / kXcds * kXcds : 0;
    if (ngrad + nsegp + nzero >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const size_t lds = (size_t)((max_level_bins + 1) / 2) * 4;
    MSDA_LAUNCH((grad_sort_kernel<DT, PT, VEC>), dim3((unsigned)(nzero + nsegp + ngrad)),
                       dim3(kBlock), lds, stream, static_cast<const E *>(value),
                       static_cast<const P *>(loc), static_cast<const P *>(attn),
                       static_cast<const E *>(grad_out), static_cast<P *>(grad_loc),
                       static_cast<P *>(grad_attn), p.levels, p.S, p.Q, (int)p.M, (int)p.D,
                       (int)p.L, (int)p.K, qblocks, ntiles, mp.log2_group, mp.log2_split,
                       params_vectorizable(p, mp.log2_split, 4, loc, attn), (uint32_t)ngrad,
                       bins.starts, bins.cursor, bins.records, p.nbbm,
                       (uint32_t)nseg, (uint32_t)nsegp, (uint32_t)nzero,
                       static_cast<uint4 *>(zero_dst), n16);
    return hipGetLastError();
}

template <class DT, class PT>
hipError_t grad_sort_by_vec(const Problem &p, const Mapping &mp, const void *v, const void *l,
                            const void *a, const void *go, void *gl, void *ga,
                            const BinnedBuffers &bins, int mlb, void *zd, size_t zb,
                            hipStream_t st) {
    switch (mp.vec) {
        case 1: return grad_sort_launch<DT, PT, 1>(p, mp, v, l, a, go, gl, ga, bins, mlb, zd, zb, st);
        case 2: return grad_sort_launch<DT, PT, 2>(p, mp, v, l, a, go, gl, ga, bins, mlb, zd, zb, st);
        case 4: return grad_sort_launch<DT, PT, 4>(p, mp, v, l, a, go, gl, ga, bins, mlb, zd, zb, st);
        case 8: return grad_sort_launch<DT, PT, 8>(p, mp, v, l, a, go, gl, ga, bins, mlb, zd, zb, st);
        default: return hipErrorInvalidValue;
    }
}

bool grad_sort_fits(const Problem &p, const Mapping &mp, int max_level_bins) {
    return p.dtype != MSDA_F32 && p.Q * p.K <= kBlock * kFusedSortPts &&
           max_level_bins <= kMaxFusedSortBins && slice_fits_buffer(p) &&
           (mp.vec == 1 || mp.vec == 2 || mp.vec == 4 || mp.vec == 8);
}

hipError_t launch_gradients_and_sort(const Problem &p, const Mapping &mp, const void *value,
                                     const void *loc, const void *attn, const void *grad_out,
                                     void *grad_loc, void *grad_attn, const BinnedBuffers &bins,
                                     int max_level_bins, void *zero_dst, size_t zero_bytes,
                                     hipStream_t stream) {
    if (!grad_sort_fits(p, mp, max_level_bins)) return hipErrorInvalidValue;
    const bool f32p = p.pdtype == MSDA_F32;
#define MSDA_GS(T, P) grad_sort_by_vec<T, P>(p, mp, value, loc, attn, grad_out, grad_loc, grad_attn, \
                                             bins, max_level_bins, zero_dst, zero_bytes, stream)
    if (p.dtype == MSDA_F16) return f32p ? MSDA_GS(F16T, F32T) : MSDA_GS(F16T, F16T);
    return f32p ? MSDA_GS(BF16T, F32T) : MSDA_GS(BF16T, BF16T);
#undef MSDA_GS
}

int64_t scan_tiles(int64_t nbins) { return (nbins + kScanTile - 1) / kScanTile; }

hipError_t launch_bin_scan(const BinnedBuffers &bins, hipStream_t stream) {
    MSDA_LAUNCH(bin_scan_kernel, dim3(1), dim3(kScanBlock), 0, stream, bins.starts,
                       bins.cursor, bins.nbins);
    return hipGetLastError();
}

hipError_t launch_bin_tile_sums(const BinnedBuffers &bins, hipStream_t stream) {
    const int64_t nt = scan_tiles(bins.nbins);
    if (nt < 1 || nt >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    MSDA_LAUNCH(bin_tile_sum_kernel, dim3((unsigned)nt), dim3(kScanBlock), 0, stream,
                       bins.starts, bins.tile_offsets, bins.nbins);
    return hipGetLastError();
}

hipError_t launch_bin_tile_scan(const BinnedBuffers &bins, hipStream_t stream) {
    const int64_t nt = scan_tiles(bins.nbins);
    MSDA_LAUNCH(bin_tile_scan_kernel, dim3((unsigned)nt), dim3(kScanBlock), 0, stream,
                       bins.starts, bins.cursor, bins.tile_offsets, bins.nbins);
    return hipGetLastError();
}

hipError_t launch_bin_accumulate(const Problem &p, const BwdMapping &mp, const void *grad_out,
                                 void *grad_value, const BinnedBuffers &bins, bool accumulate,
                                 hipStream_t stream) {
    switch (p.dtype) {
        case MSDA_F32: return accum_by_j<F32T, 1>(p, mp, grad_out, grad_value, bins, accumulate, stream);
        case MSDA_F16:
            return mp.slot == 2 ? accum_by_j<F16T, 2>(p, mp, grad_out, grad_value, bins, accumulate, stream)
                                : accum_by_j<F16T, 1>(p, mp, grad_out, grad_value, bins, accumulate, stream);
        case MSDA_BF16:
            return mp.slot == 2 ? accum_by_j<BF16T, 2>(p, mp, grad_out, grad_value, bins, accumulate, stream)
                                : accum_by_j<BF16T, 1>(p, mp, grad_out, grad_value, bins, accumulate, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_forward_foil(const Problem &p, int vec, const void *value, const void *loc,
                               const void *attn, void *out, hipStream_t stream) {
    const int64_t P = p.B * p.Q * p.M * p.L * p.K;
    const int64_t grid = (P + kBlock - 1) / kBlock;
    const size_t lds = (size_t)kBlock * (size_t)p.D * sizeof(float);
#define MSDA_FOIL(T, V)                                                                         \
    MSDA_LAUNCH((msda_foil_kernel<T, V, 64>), dim3((unsigned)grid), dim3(kBlock), lds,    \
                       stream, static_cast<const typename T::S *>(value),                       \
                       static_cast<const typename T::S *>(loc),                                 \
                       static_cast<const typename T::S *>(attn),                                \
                       static_cast<typename T::S *>(out), p.levels, p.S, p.Q, (int)p.M,         \
                       (int)p.D, (int)p.L, (int)p.K, P)
    switch (p.dtype) {
        case MSDA_F32:
            if (vec == 4) MSDA_FOIL(F32T, 4); else MSDA_FOIL(F32T, 1);
            break;
        case MSDA_F16:
            if (vec == 8) MSDA_FOIL(F16T, 8); else MSDA_FOIL(F16T, 1);
            break;
        case MSDA_BF16:
            if (vec == 8) MSDA_FOIL(BF16T, 8); else MSDA_FOIL(BF16T, 1);
            break;
        default: return hipErrorInvalidValue;
    }
#undef MSDA_FOIL
    return hipGetLastError();
}

hipError_t launch_zero(void *dst, size_t bytes, hipStream_t stream) {
    if (bytes == 0) return hipSuccess;
    if ((reinterpret_cast<uintptr_t>(dst) % 16 == 0) && (bytes % 16 == 0)) {
        const int64_t n16 = (int64_t)(bytes / 16);
        MSDA_LAUNCH(zero_kernel_16, dim3(grid_for(n16)), dim3(kBlock), 0, stream,
                           static_cast<uint4 *>(dst), n16);
    } else {
        const int64_t n2 = (int64_t)(bytes / 2);
        MSDA_LAUNCH(zero_kernel_2, dim3(grid_for(n2)), dim3(kBlock), 0, stream,
                           static_cast<uint16_t *>(dst), n2);
    }
    return hipGetLastError();
}

hipError_t launch_scratch_add(const Problem &p, const float *workspace, void *grad_value,
                              hipStream_t stream) {
    switch (p.dtype) {
        case MSDA_F16: return scratch_add<F16T>(p, workspace, grad_value, stream);
        case MSDA_BF16: return scratch_add<BF16T>(p, workspace, grad_value, stream);
        default: return scratch_add<F32T>(p, workspace, grad_value, stream);  // pre-reduced levels
    }
}

}  // namespace msda
