// Pre-reduced grad_value for contended levels (msda-triton README, section
// "Benchmarks": a shared-memory pre-reduction ahead of the global atomics).
//
// A level whose pixels receive many contributions (the coarse levels of an
// encoder, where every pyramid pixel is a query sampling near its own
// position) spends most of a plain scatter on atomics that serialise on the
// same few rows, and most of a global counting sort on records and on
// re-gathering one upstream-gradient row per record. Here one workgroup owns
// one head and a block of queries, whose upstream-gradient rows it stages in
// LDS once. For each such level it counting-sorts the corners of its points
// by pixel of a window placed at the mean of the block's samples on the level
// (integer LDS atomics, one per corner), then one lane per (pixel, channel)
// sums up to kPreChunk records' contributions A * w_ij * g (course page "5.
// The backward kernel", section "What the backward pass must produce") in a
// register and adds the sum into the pixel's fp32 scratch row. A corner
// outside the window adds straight into the scratch, so any input gives the
// plain scatter's sum; spatially coherent blocks make that rare. The scratch
// is rounded into grad_value afterwards (scratch_add_kernel).
//
// Float atomics in LDS are not used: on gfx950 a wave's ds_add_f32 kept the
// LDS busy for about 185 cycles in measurement, which made any variant built
// on them slower than the sort.
//
// Blocks: for pixel queries (the queries are the pyramid's pixels in S order)
// a block is a tile of pixels of the largest level together with the pixels
// of every other level in the same normalised area, so all its samples on a
// coarse level fall in one small neighbourhood; otherwise a block is a fixed
// number of consecutive queries.

#include "msda_device.h"
#include "msda_launch.h"

namespace msda {
namespace {


// Block `r` of one (b, m): its query count, and its queries' indexes into
// qidx (LDS). Pixel blocks: tile (ty, tx) of the reference level and the
// matching rows and columns of every level (pre_tile_span), level by level,
// row-major within each. Linear blocks: pt.lin_queries consecutive queries.
__device__ __forceinline__ int block_queries(const PreTiles &pt, const LevelTable &lt, int L,
                                             int64_t Q, int64_t r, int32_t *qidx) {
    const int tid = threadIdx.x;
    if (!pt.pixel) {
        const int64_t q0 = r * pt.lin_queries, rem = Q - q0;
        const int n = (int)(rem < pt.lin_queries ? rem : pt.lin_queries);
        for (int j = tid; j < n; j += kPreBlock) qidx[j] = (int32_t)(q0 + j);
        return n;
    }
    return merged_tile_queries(lt, L, pt.ref, pt.tile, r, qidx, tid, kPreBlock);
}

template <class DT, class PT>
__global__ __launch_bounds__(kPreBlock) void prereduce_kernel(
    const typename PT::S *__restrict__ loc, const typename PT::S *__restrict__ attn,
    const typename DT::S *__restrict__ grad_out, float *__restrict__ ws, const LevelTable lt,
    const PreTiles pt, const int64_t Q, const int M, const int D, const int L, const int K,
    const int64_t blocks_per_bm, const int64_t ntiles) {
    using E = typename DT::S;
    // dynamic LDS (pre_lds_bytes): record weights and record queries
    // (max_records each), the window's row starts (max_px + 1), cursors
    // (max_px) and chunk starts (max_px + 1), each chunk's pixel (max_chunks),
    // the block's query indexes (max_queries), then its upstream-gradient rows
    // (max_queries rows of D + 1 elements)
    extern __shared__ float lds[];
    const int64_t tile = logical_block();
    if (tile >= ntiles) return;  // whole workgroup
    const int64_t bm = tile / blocks_per_bm;
    const int64_t b = bm / M;
    const int m = (int)(bm - b * M);
    const int tid = threadIdx.x;
    const int LK = L * K;
    const int64_t MD = (int64_t)M * D;
    const int pitch = D + 1;  // upstream-gradient row pitch: rows start in different banks
    float *rec_w = lds;
    int32_t *rec_j = reinterpret_cast<int32_t *>(rec_w + pt.max_records);
    int32_t *rstart = rec_j + pt.max_records;
    int32_t *cursor = rstart + pt.max_px + 1;
    int32_t *cstart = cursor + pt.max_px;              // max_px + 1
    int32_t *chunk_px = cstart + pt.max_px + 1;        // max_chunks
    int32_t *qidx = chunk_px + pt.max_chunks;
    E *gst = reinterpret_cast<E *>(qidx + pt.max_queries);
    __shared__ float msum[MSDA_MAX_LEVELS][3];
    __shared__ int32_t origin[MSDA_MAX_LEVELS][2];

    if (tid < 3 * pt.nlev) msum[tid / 3][tid % 3] = 0.0f;
    const int n = block_queries(pt, lt, L, Q, tile - bm * blocks_per_bm, qidx);
    __syncthreads();
    for (int i = tid; i < n * D; i += kPreBlock) {  // rows of D consecutive channels
        const int j = i / D, c = i - j * D;
        gst[j * pitch + c] = grad_out[((b * Q + qidx[j]) * M + m) * D + c];
    }

    // 1. Window origins: the mean sample position of the block on each level
    //    (fp32 sums; a window only speeds things up, so its place needs no
    //    exactness). Each thread sums its points, the wave adds its lanes with
    //    shuffles, one lane per wave adds into LDS.
    const int nk = n * K;  // the block's points on one level
    for (int li = 0; li < pt.nlev; ++li) {
        const int l = pt.lev[li];
        float sx = 0.0f, sy = 0.0f, sn = 0.0f;
        for (int t = tid; t < nk; t += kPreBlock) {
            const int j = t / K;
            const int64_t p = ((b * Q + qidx[j]) * M + m) * LK + l * K + (t - j * K);
            const float x = bits_to_f32<PT>(load_bits<PT>(loc + 2 * p));
            const float y = bits_to_f32<PT>(load_bits<PT>(loc + 2 * p + 1));
            if (__builtin_fabsf(x) <= 4.0f && __builtin_fabsf(y) <= 4.0f) {  // skip wild samples
                sx += x;
                sy += y;
                sn += 1.0f;
            }
        }
        for (int o = 32; o > 0; o >>= 1) {
            sx += __shfl_xor(sx, o);
            sy += __shfl_xor(sy, o);
            sn += __shfl_xor(sn, o);
        }
        if ((tid & 63) == 0) {
            atomicAdd(&msum[li][0], sx);
            atomicAdd(&msum[li][1], sy);
            atomicAdd(&msum[li][2], sn);
        }
    }
    __syncthreads();
    if (tid < pt.nlev) {
        const int l = pt.lev[tid];
        const float cnt = msum[tid][2];
        const float mx = cnt > 0.0f ? msum[tid][0] / cnt : 0.5f;
        const float my = cnt > 0.0f ? msum[tid][1] / cnt : 0.5f;
        const int wx = pt.wx[tid], wy = pt.wy[tid];
        int ox = (int)__builtin_floorf(mx * (float)lt.W[l] - 0.5f) - (wx - 1) / 2;
        int oy = (int)__builtin_floorf(my * (float)lt.H[l] - 0.5f) - (wy - 1) / 2;
        ox = ox > lt.W[l] - wx ? lt.W[l] - wx : ox;  // windows never exceed their level
        oy = oy > lt.H[l] - wy ? lt.H[l] - wy : oy;
        origin[tid][0] = ox < 0 ? 0 : ox;
        origin[tid][1] = oy < 0 ? 0 : oy;
    }

    // 2. Per level: a counting sort of the block's corner records by window
    //    pixel (integer LDS atomics: one per corner, not one per channel),
    //    then one lane per (pixel, channel) sums its records' A * w_ij * g
    //    in a register and adds the sum into the pixel's scratch row. Corners
    //    outside the window go straight to the scratch with global atomics.
    const int lanes = D < 64 ? D : 64;
    const int per = kPreBlock / lanes;  // pixels summed side by side
    const int ch0 = tid % lanes, rsl = tid / lanes;
    const int wave = tid >> 6, lane = tid & 63;
    for (int li = 0; li < pt.nlev; ++li) {
        const int l = pt.lev[li];
        const int W = lt.W[l], H = lt.H[l];
        const float Wf = (float)W, Hf = (float)H;
        const int64_t start = lt.start[l];
        const int wx = pt.wx[li], wy = pt.wy[li], npx = wx * wy;
        float *scr = ws + lt.scratch_off[l] + (b * (int64_t)H * W * M + m) * D;
        __syncthreads();  // the origins; the previous level's records are summed
        const int ox = origin[li][0], oy = origin[li][1];
        for (int i = tid; i < npx; i += kPreBlock) cursor[i] = 0;
        __syncthreads();
        for (int t = tid; t < nk; t += kPreBlock) {  // count
            const int j = t / K;
            const int64_t p = ((b * Q + qidx[j]) * M + m) * LK + l * K + (t - j * K);
            const Cell cl = map_cell(bits_to_f32<PT>(load_bits<PT>(loc + 2 * p)),
                                     bits_to_f32<PT>(load_bits<PT>(loc + 2 * p + 1)), Hf, Wf, W,
                                     start);
            const bool vc[4] = {cl.v00, cl.v01, cl.v10, cl.v11};
#pragma unroll
            for (int cn = 0; cn < 4; ++cn) {
                const int dx = cl.x0 + (cn & 1) - ox, dy = cl.y0 + (cn >> 1) - oy;
                if (vc[cn] && dx >= 0 && dx < wx && dy >= 0 && dy < wy)
                    atomicAdd(cursor + dy * wx + dx, 1);
            }
        }
        __syncthreads();
        if (wave == 0) {  // exclusive scans of the counts (row starts, and the
                          // cursors) and of the pixels' chunk counts
            int carry = 0, ccarry = 0;
            for (int base = 0; base < npx; base += 64) {
                const int i = base + lane;
                const int v = i < npx ? cursor[i] : 0;
                const int cv = (v + kPreChunk - 1) / kPreChunk;
                int incl = v, cincl = cv;
                for (int o = 1; o < 64; o <<= 1) {
                    const int u = __shfl_up(incl, o), cu = __shfl_up(cincl, o);
                    incl += lane >= o ? u : 0;
                    cincl += lane >= o ? cu : 0;
                }
                if (i < npx) {
                    rstart[i] = carry + incl - v;
                    cursor[i] = carry + incl - v;
                    cstart[i] = ccarry + cincl - cv;
                }
                carry += __shfl(incl, 63);
                ccarry += __shfl(cincl, 63);
            }
            if (lane == 0) {
                rstart[npx] = carry;
                cstart[npx] = ccarry;
            }
        }
        __syncthreads();
        for (int i = tid; i < npx; i += kPreBlock)  // each chunk names its pixel
            for (int c = cstart[i]; c < cstart[i + 1]; ++c) chunk_px[c] = i;
        for (int t = tid; t < nk; t += kPreBlock) {  // place
            const int j = t / K;
            const int64_t p = ((b * Q + qidx[j]) * M + m) * LK + l * K + (t - j * K);
            const float a = bits_to_f32<PT>(load_bits<PT>(attn + p));
            const Cell cl = map_cell(bits_to_f32<PT>(load_bits<PT>(loc + 2 * p)),
                                     bits_to_f32<PT>(load_bits<PT>(loc + 2 * p + 1)), Hf, Wf, W,
                                     start);
            const float fx = cl.fx, fy = cl.fy;
            const float wts[4] = {a * (1.0f - fx) * (1.0f - fy), a * fx * (1.0f - fy),
                                  a * (1.0f - fx) * fy, a * fx * fy};
            const bool vc[4] = {cl.v00, cl.v01, cl.v10, cl.v11};
#pragma unroll
            for (int cn = 0; cn < 4; ++cn) {
                if (!vc[cn]) continue;
                const int dx = cl.x0 + (cn & 1) - ox, dy = cl.y0 + (cn >> 1) - oy;
                if (dx >= 0 && dx < wx && dy >= 0 && dy < wy) {
                    const int slot = atomicAdd(cursor + dy * wx + dx, 1);
                    rec_w[slot] = wts[cn];
                    rec_j[slot] = j * pitch;
                } else {
                    float *dst = scr + ((int64_t)(cl.y0 + (cn >> 1)) * W + cl.x0 + (cn & 1)) * MD;
                    const E *g = gst + j * pitch;
                    for (int c = 0; c < D; ++c) atomic_add_f32(dst + c, wts[cn] * to_f32(DT{}, g[c]));
                }
            }
        }
        __syncthreads();
        const int nchunks = cstart[npx];
        for (int c = rsl; c < nchunks && rsl < per; c += per) {  // sum and flush
            const int px = chunk_px[c];
            const int r0 = rstart[px] + (c - cstart[px]) * kPreChunk;
            const int r1 = min(r0 + kPreChunk, rstart[px + 1]);
            const int64_t row = (int64_t)(oy + px / wx) * W + (ox + px % wx);
            for (int ch = ch0; ch < D; ch += lanes) {
                float acc0 = 0.0f, acc1 = 0.0f;
                int r = r0;
                for (; r + 1 < r1; r += 2) {
                    acc0 += rec_w[r] * to_f32(DT{}, gst[rec_j[r] + ch]);
                    acc1 += rec_w[r + 1] * to_f32(DT{}, gst[rec_j[r + 1] + ch]);
                }
                if (r < r1) acc0 += rec_w[r] * to_f32(DT{}, gst[rec_j[r] + ch]);
                atomic_add_f32(scr + row * MD + ch, acc0 + acc1);
            }
        }
    }
}

}  // namespace

hipError_t launch_prereduce(const Problem &p, const PreTiles &pt, const void *loc, const void *attn,
                            const void *grad_out, float *workspace, hipStream_t stream) {
    if (pt.nlev == 0 || p.B == 0 || p.Q == 0) return hipSuccess;
    int64_t blocks = 0;
    if (pt.pixel) {
        blocks = (int64_t)((p.levels.H[pt.ref] + pt.tile - 1) / pt.tile) *
                 ((p.levels.W[pt.ref] + pt.tile - 1) / pt.tile);
    } else {
        blocks = (p.Q + pt.lin_queries - 1) / pt.lin_queries;
    }
    const int64_t ntiles = p.B * p.M * blocks;
    const int64_t per_xcd = (ntiles + kXcds - 1) / kXcds;
    const size_t lds = pre_lds_bytes(pt, p.D, p.dtype == MSDA_F32 ? 4 : 2);
#define MSDA_PRE_LAUNCH(T, P)                                                                   \
    MSDA_LAUNCH((prereduce_kernel<T, P>), dim3((unsigned)(per_xcd * kXcds)), dim3(kPreBlock), lds, \
                stream, static_cast<const typename P::S *>(loc),                                \
                static_cast<const typename P::S *>(attn),                                       \
                static_cast<const typename T::S *>(grad_out), workspace, p.levels, pt, p.Q,     \
                (int)p.M, (int)p.D, (int)p.L, (int)p.K, blocks, ntiles)
    if (p.dtype == MSDA_F32) MSDA_PRE_LAUNCH(F32T, F32T);
    else if (p.dtype == MSDA_F16 && p.pdtype == MSDA_F32) MSDA_PRE_LAUNCH(F16T, F32T);
    else if (p.dtype == MSDA_F16) MSDA_PRE_LAUNCH(F16T, F16T);
    else if (p.pdtype == MSDA_F32) MSDA_PRE_LAUNCH(BF16T, F32T);
    else MSDA_PRE_LAUNCH(BF16T, BF16T);
#undef MSDA_PRE_LAUNCH
    return hipGetLastError();
}

}  // namespace msda
