// Device-side helpers shared by the kernel sources of the library: the
// storage type of each dtype and its exact conversions to and from fp32
// (rounding to nearest even on the way down), the XCD-aware workgroup order,
// fp32 atomics, and the bilinear cell of a sampling point. Included by .hip
// files only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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


// Raw bits of one element, widened to a register.
template <class DT>
__device__ __forceinline__ uint32_t load_bits(const typename DT::S *p) {
    if constexpr (sizeof(typename DT::S) == 4) return __float_as_uint(*p);
    else return (uint32_t)*p;
}
template <class DT>
__device__ __forceinline__ float bits_to_f32(uint32_t v) {
    if constexpr (sizeof(typename DT::S) == 4) return __uint_as_float(v);
    else return to_f32(DT{}, (uint16_t)v);
}


// Logical tile for this workgroup; the grid has kXcds * per_xcd workgroups and
// XCD x = blockIdx % 8 takes logical tiles [x * per_xcd, (x + 1) * per_xcd).
__device__ __forceinline__ int64_t logical_block() {
    const uint32_t per_xcd = gridDim.x / kXcds;
    return (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
}


__device__ __forceinline__ void atomic_add_f32(float *p, float v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// Everything that depends only on the point's location: cell, weights (times
// the attention weight for the forward), masks and corner row offsets.
struct Cell {
    float fx, fy;          // fractional position inside the cell
    bool v00, v01, v10, v11;
    int x0, y0;            // the cell's corner 00, clamped to [-1, W] x [-1, H]
    int64_t row00;         // start_l + y0 * W + x0 (meaningful when a corner is valid)
};

__device__ __forceinline__ Cell map_cell(float loc_x, float loc_y, float Hf, float Wf, int W,
                                         int64_t start) {
    Cell c;
    // A non-finite coordinate, or one beyond 1e30 in magnitude (whose product
    // with the level size could overflow), becomes -4 (normalised), outside
    // the level in that dimension like the coordinate it replaces: the point
    // then has no in-bounds corner and finite weights, so it adds exactly 0
    // to every result (left as it is, its NaN weights would make NaN of the
    // zero corners they multiply). Other coordinates pass unchanged.
    loc_x = __builtin_fabsf(loc_x) <= 1.0e30f ? loc_x : -4.0f;
    loc_y = __builtin_fabsf(loc_y) <= 1.0e30f ? loc_y : -4.0f;
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
    c.x0 = x0;
    c.y0 = y0;
    c.row00 = start + (int64_t)y0 * W + x0;
    return c;
}

// -------------------------------------------------- sampling parameters
//
// The G lanes of a group share every point (they hold different channels), so
// loading a point's location and weight in every lane would cost G load
// instructions per parameter, each as expensive for the vector memory path as
// a corner gather. Instead lane k of the group loads the parameters of chunk
// k (points kCH .. kCH + CH - 1 of the group's list) once, before the chunk
// loop, and chunk k's parameters are shuffled from lane k when its turn comes
// (needs at most G chunks). Parameters are kept as raw dwords: 16-bit types
// hold a point's (x, y) in one dword and two points' weights in another;
// fp32 types one value per dword.
template <class PT, int CH>
struct ChunkParams {
    static constexpr int kE = (int)sizeof(typename PT::S);
    static constexpr int kLocW = CH * 2 * kE / 4;    // 16-bit: CH; fp32: 2 CH
    static constexpr int kAttW = (CH * kE + 3) / 4;  // 16-bit: CH / 2; fp32: CH
    uint32_t loc[kLocW];
    uint32_t att[kAttW];
};

// Lane k's own chunk: points i = k * CH + t (t < CH) of the group's list,
// i < per_lane, point index i * split + s. `vec`: the chunk is whole and its
// dwords are aligned for 16-byte (locations) and 8- or 16-byte (weights)
// loads (split == 1, checked on the host), else element loads.
template <class PT, int CH>
__device__ __forceinline__ void own_chunk_params(const typename PT::S *loc_q,
                                                 const typename PT::S *attn_q, int k,
                                                 int per_lane, int split, int s, bool vec,
                                                 ChunkParams<PT, CH> &cp) {
    using C = ChunkParams<PT, CH>;
    static_assert(C::kLocW % 4 == 0 && (C::kAttW == 2 || C::kAttW % 4 == 0), "chunk layout");
#pragma unroll
    for (int w = 0; w < C::kLocW; ++w) cp.loc[w] = 0;
#pragma unroll
    for (int w = 0; w < C::kAttW; ++w) cp.att[w] = 0;
    const int i0 = k * CH;
    if (i0 >= per_lane) return;
    if (vec) {
        const uint4 *lp = reinterpret_cast<const uint4 *>(loc_q + 2 * i0);
#pragma unroll
        for (int w = 0; w < C::kLocW / 4; ++w) {
            const uint4 v = lp[w];
            cp.loc[4 * w] = v.x;
            cp.loc[4 * w + 1] = v.y;
            cp.loc[4 * w + 2] = v.z;
            cp.loc[4 * w + 3] = v.w;
        }
        if constexpr (C::kAttW == 2) {
            const uint2 v = *reinterpret_cast<const uint2 *>(attn_q + i0);
            cp.att[0] = v.x;
            cp.att[1] = v.y;
        } else {
            const uint4 *ap = reinterpret_cast<const uint4 *>(attn_q + i0);
#pragma unroll
            for (int w = 0; w < C::kAttW / 4; ++w) {
                const uint4 v = ap[w];
                cp.att[4 * w] = v.x;
                cp.att[4 * w + 1] = v.y;
                cp.att[4 * w + 2] = v.z;
                cp.att[4 * w + 3] = v.w;
            }
        }
        return;
    }
#pragma unroll
    for (int t = 0; t < CH; ++t) {
        const int i = i0 + t;
        const int p = (i < per_lane ? i : i0) * split + s;  // in-bounds address
        const uint32_t x = load_bits<PT>(loc_q + 2 * p), y = load_bits<PT>(loc_q + 2 * p + 1);
        const uint32_t a = i < per_lane ? load_bits<PT>(attn_q + p) : 0u;
        if constexpr (C::kE == 2) {
            cp.loc[t] = (x & 0xFFFFu) | (y << 16);
            cp.att[t / 2] |= (a & 0xFFFFu) << (16 * (t & 1));
        } else {
            cp.loc[2 * t] = x;
            cp.loc[2 * t + 1] = y;
            cp.att[t] = a;
        }
    }
}

// Chunk parameters from lane `src` (absolute lane of the wave), unpacked.
template <class PT, int CH>
__device__ __forceinline__ void chunk_params(const ChunkParams<PT, CH> &own, int src,
                                             float (&lx)[CH], float (&ly)[CH], float (&aw)[CH]) {
    using C = ChunkParams<PT, CH>;
    uint32_t lw[C::kLocW], aw_[C::kAttW];
#pragma unroll
    for (int w = 0; w < C::kLocW; ++w) lw[w] = (uint32_t)__shfl((int)own.loc[w], src, 64);
#pragma unroll
    for (int w = 0; w < C::kAttW; ++w) aw_[w] = (uint32_t)__shfl((int)own.att[w], src, 64);
#pragma unroll
    for (int t = 0; t < CH; ++t) {
        if constexpr (C::kE == 2) {
            lx[t] = bits_to_f32<PT>(lw[t] & 0xFFFFu);
            ly[t] = bits_to_f32<PT>(lw[t] >> 16);
            aw[t] = bits_to_f32<PT>((aw_[t / 2] >> (16 * (t & 1))) & 0xFFFFu);
        } else {
            lx[t] = __uint_as_float(lw[2 * t]);
            ly[t] = __uint_as_float(lw[2 * t + 1]);
            aw[t] = __uint_as_float(aw_[t]);
        }
    }
}

// Point k (< CH) of the chunk owned by lane `src`, unpacked: the chunk's
// dwords are shuffled as in chunk_params and point k's are kept.
template <class PT, int CH>
__device__ __forceinline__ void point_params(const ChunkParams<PT, CH> &own, int src, int k,
                                             float &x, float &y, float &a) {
    using C = ChunkParams<PT, CH>;
    uint32_t lw[C::kLocW], aw_[C::kAttW];
#pragma unroll
    for (int w = 0; w < C::kLocW; ++w) lw[w] = (uint32_t)__shfl((int)own.loc[w], src, 64);
#pragma unroll
    for (int w = 0; w < C::kAttW; ++w) aw_[w] = (uint32_t)__shfl((int)own.att[w], src, 64);
    if constexpr (C::kE == 2) {
        uint32_t l = lw[0], at = aw_[0];
#pragma unroll
        for (int t = 1; t < CH; ++t) l = k == t ? lw[t] : l;
#pragma unroll
        for (int w = 1; w < C::kAttW; ++w) at = (k >> 1) == w ? aw_[w] : at;
        x = bits_to_f32<PT>(l & 0xFFFFu);
        y = bits_to_f32<PT>(l >> 16);
        a = bits_to_f32<PT>((at >> (16 * (k & 1))) & 0xFFFFu);
    } else {
        uint32_t lx = lw[0], ly = lw[1], at = aw_[0];
#pragma unroll
        for (int t = 1; t < CH; ++t) {
            lx = k == t ? lw[2 * t] : lx;
            ly = k == t ? lw[2 * t + 1] : ly;
            at = k == t ? aw_[t] : at;
        }
        x = __uint_as_float(lx);
        y = __uint_as_float(ly);
        a = __uint_as_float(at);
    }
}

}  // namespace
}  // namespace msda
