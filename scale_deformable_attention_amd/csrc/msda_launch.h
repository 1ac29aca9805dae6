// Internal interface between the host-side C ABI (msda_api.cpp) and the
// gfx950 kernels (msda_kernels.hip). Not installed, not part of the ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msda.h"

namespace msda {

// Launch instrumentation (msda_set_launch_events): when `stop` is set, the next
// kernel launch of this thread records `start` when that kernel starts and
// `stop` when it ends (the launch packet's own timestamps); a helper that
// launches several kernels records `start` at its first and `stop` at its last.
struct TimedLaunch {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
TimedLaunch &timed_launch();  // this thread's pending events (msda_api.cpp)

// Every kernel launch of the library goes through this macro.
#define MSDA_LAUNCH(kernel, grid, block, lds, stream, ...)                                     \
    do {                                                                                        \
        ::msda::TimedLaunch &tl_ = ::msda::timed_launch();                                     \
        if (tl_.stop) {                                                                         \
            hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, tl_.start, tl_.stop, 0,     \
                                  __VA_ARGS__);                                                 \
            tl_.start = nullptr;                                                                \
        } else {                                                                                \
            hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);                  \
        }                                                                                       \
    } while (0)

// Level table passed by value in the kernel arguments (no device copy, no
// host synchronisation). H, W < 2^24 so that they are exact in fp32.
// scratch_off[l] >= 0: the backward accumulates level l's grad_value rows in
// fp32 at workspace + scratch_off[l] (elements), laid out (B, H*W, M, D);
// -1: atomics of the value dtype go straight into grad_value.
//
// Binned grad_value: the rows of level l of one (b, m) are cut into bins of
// 2^bin_shift[l] pixel rows (bin_shift[l] = -1: level not binned); bin_off[l]
// is the index of level l's first bin among the nbbm bins of one (b, m).
struct LevelTable {
    int32_t H[MSDA_MAX_LEVELS];
    int32_t W[MSDA_MAX_LEVELS];
    int64_t start[MSDA_MAX_LEVELS];
    int64_t scratch_off[MSDA_MAX_LEVELS];
    int32_t bin_shift[MSDA_MAX_LEVELS];
    int32_t bin_off[MSDA_MAX_LEVELS];
    int32_t blevel[MSDA_MAX_LEVELS];  // the binned levels, in order
    int32_t nblev;
    uint32_t prered;  // bit l: level l is pre-reduced in LDS (launch_prereduce)
};

// Pre-reduced levels (launch_prereduce): their fp32 scratch rows receive the
// per-window sums of one workgroup. One workgroup per (b, m, block of
// queries): for pixel queries a tile of `tile` x `tile` pixels of the largest
// level (ref) together with the rows and columns of every other level in the
// same normalised area (pre_tile_span), else lin_queries consecutive queries.
// Window li (of level lev[li]) is wx[li] x wy[li] pixels.
struct PreTiles {
    int32_t pixel;
    int32_t ref;          // pixel tiles: the level with the most pixels
    int32_t tile;         // pixel tiles: side, in pixels of the reference level
    int32_t lin_queries;  // linear blocks: queries per block
    int32_t nlev;
    int32_t lev[MSDA_MAX_LEVELS];
    int32_t wx[MSDA_MAX_LEVELS];
    int32_t wy[MSDA_MAX_LEVELS];
    int32_t max_px;       // pixels of the largest window
    int32_t max_queries;  // queries of the largest block
    int32_t max_records;  // 4 corners of every point of the largest block on one level
    int32_t max_chunks;   // record chunks of one level: max_records / kPreChunk + max_px
};

constexpr int kPreBlock = 256;  // threads of a pre-reduction workgroup
constexpr int kPreChunk = 32;   // records a lane sums before it adds into the scratch

// First row (column) on a level of n rows (columns) of tile i of `tiles`
// tiles of `side` rows over the reference level's n0 rows: the rows whose
// normalised position falls in the tile's, rounded to the nearest row
// boundary; the last tile ends at n.
__host__ __device__ inline int32_t pre_tile_span(int64_t i, int32_t side, int32_t n, int32_t n0,
                                                 int64_t tiles) {
    return i >= tiles ? n : (int32_t)((i * side * n + n0 / 2) / n0);
}

// The queries of merged tile r of pixel queries (those of the pyramid's own
// pixels in S order): tile (ty, tx) of `side` x `side` pixels of level ref,
// and on every level l the rows and columns pre_tile_span assigns it, level
// by level, row-major within each. Writes their indexes to qidx (threads
// tid, tid + nthreads, ... of the workgroup share the work) and returns
// their count; every thread walks the same levels.
__device__ inline int merged_tile_queries(const LevelTable &lt, int L, int ref, int side,
                                          int64_t r, int32_t *qidx, int tid, int nthreads) {
    const int32_t H0 = lt.H[ref], W0 = lt.W[ref];
    const int64_t ny = (H0 + side - 1) / side, nx = (W0 + side - 1) / side;
    const int64_t ty = r / nx, tx = r - ty * nx;
    int n = 0;
    for (int l = 0; l < L; ++l) {
        const int32_t y0 = pre_tile_span(ty, side, lt.H[l], H0, ny);
        const int32_t y1 = pre_tile_span(ty + 1, side, lt.H[l], H0, ny);
        const int32_t x0 = pre_tile_span(tx, side, lt.W[l], W0, nx);
        const int32_t w = pre_tile_span(tx + 1, side, lt.W[l], W0, nx) - x0;
        const int cnt = (y1 - y0) * w;
        for (int i = tid; i < cnt; i += nthreads) {
            const int dy = i / w;
            qidx[n + i] = (int32_t)(lt.start[l] + (int64_t)(y0 + dy) * lt.W[l] + x0 + (i - dy * w));
        }
        n += cnt;
    }
    return n;
}

// Dynamic LDS bytes of one pre-reduction workgroup: record weights and
// record queries, window row starts, cursors and chunk starts, chunk pixels,
// query indexes (4 bytes each), then the upstream-gradient rows (D + 1
// elements of `esize` bytes).
inline size_t pre_lds_bytes(const PreTiles &pt, int64_t D, int esize) {
    return (2 * (size_t)pt.max_records + 3 * (size_t)pt.max_px + 2 + (size_t)pt.max_chunks +
            (size_t)pt.max_queries) * 4 +
           (size_t)pt.max_queries * (size_t)(D + 1) * (size_t)esize;
}

// Everything a launch needs, validated by the host layer.
struct Problem {
    int dtype;   // msda_dtype_t of value, output, grad_output, grad_value
    int pdtype;  // of sampling_locations, attention_weights and their gradients:
                 // dtype, or MSDA_F32 beside 16-bit values
    int64_t B, S, M, D, L, Q, K;
    LevelTable levels;
    int64_t nbbm;  // bins per (b, m) of the binned grad_value (0: not planned)
};

// Workspace of the binned grad_value: starts[nbins + 1] (counts before the
// scan), cursor[nbins], and one 8-byte record per in-bounds corner of a
// binned level: x = query << 4 | row within the bin, y = fp32 bits of A * w_ij.
struct BinnedBuffers {
    uint32_t *starts;
    uint32_t *cursor;
    const uint32_t *ends;  // bin i's records are [starts[i], ends[i]): the cursors after place
    uint32_t *tile_offsets;  // scan_tiles(nbins) tile totals of the scan (2 * (scan_tiles + 1) reserved)
    uint2 *records;
    int64_t nbins;
};

// Forward lane mapping: each query's channels are spread over
// G = 2^log2_group lanes holding `vec` consecutive channels each (16-byte
// gathers where the pointers allow); 2^log2_split lane groups share one
// query and split its L*K points.
struct Mapping {
    int vec;
    int log2_group;
    int log2_split;
};

// Backward lane mapping: G = 2^log2_group lanes per query (at most 16, so one
// instruction of the group covers one 64-byte segment); lane c owns the
// "slots" c, c + G, ..., c + (J-1) G of the corner row, a slot being `slot`
// channels (2 = one dword of 16-bit data, else 1).
struct BwdMapping {
    int slot;
    int j;
    int log2_group;
    int log2_split;
};

// The value slice of one batch can be addressed by a buffer resource (32-bit
// offsets), and no test forces plain loads (msda_debug_force_flat_gathers).
bool slice_fits_buffer(const Problem &p);
bool flat_gathers_forced();

hipError_t launch_forward(const Problem &p, const Mapping &mp, const void *value,
                          const void *loc, const void *attn, void *out,
                          hipStream_t stream);


// Scatter kernel: writes grad_loc / grad_attn, adds into grad_value (levels
// with scratch_off < 0; fp32 adds for fp32 data, packed adds for 16-bit data)
// and into the fp32 workspace (levels with scratch_off >= 0); binned levels
// (bin_shift >= 0) are left to the binned kernels.
hipError_t launch_backward(const Problem &p, const BwdMapping &mp, const void *value,
                           const void *loc, const void *attn, const void *grad_out,
                           void *grad_value, float *workspace, void *grad_loc, void *grad_attn,
                           hipStream_t stream);

// Binned grad_value, in stream order: zero starts[0:nbins] (launch_zero);
// launch_bin_sort(place = false) counts the in-bounds corners per bin into
// starts; launch_bin_scan turns the counts into starts and cursors;
// launch_bin_sort(place = true) writes the records, each bin's from its start
// up to its cursor (fewer than counted where place merges records, so a bin
// ends at its cursor, not at the next start); launch_gradients writes
// grad_loc / grad_attn, launch_scatter the unbinned levels' atomics (if any);
// launch_bin_accumulate writes the binned levels' grad_value rows.
hipError_t launch_bin_sort(const Problem &p, const void *loc, const void *attn,
                           const BinnedBuffers &bins, bool place, hipStream_t stream);
hipError_t launch_bin_scan(const BinnedBuffers &bins, hipStream_t stream);
// The same scan in two launches over tiles of 4096 counts (tile totals;
// every tile's scan plus the sum of the earlier totals), for large bin counts.
int64_t scan_tiles(int64_t nbins);
hipError_t launch_bin_tile_sums(const BinnedBuffers &bins, hipStream_t stream);
hipError_t launch_bin_tile_scan(const BinnedBuffers &bins, hipStream_t stream);
// launch_gradients, launch_bin_local_sort and the zero fill as one launch
// (16-bit data, Q * K <= 2048, every binned level at most kMaxFusedSortBins
// bins, value slices buffer-addressable).
constexpr int kMaxFusedSortBins = 4096;  // 8 KB of LDS counters
bool grad_sort_fits(const Problem &p, const Mapping &mp, int max_level_bins);
hipError_t launch_gradients_and_sort(const Problem &p, const Mapping &mp, const void *value,
                                     const void *loc, const void *attn, const void *grad_out,
                                     void *grad_loc, void *grad_attn, const BinnedBuffers &bins,
                                     int max_level_bins, void *zero_dst, size_t zero_bytes,
                                     hipStream_t stream);
// launch_scatter and launch_bin_accumulate as one launch (16-bit data, two
// channels per lane slot, D a multiple of 8, grad_value 16-byte aligned).
bool scatter_accumulate_fits(const Problem &p, const BwdMapping &mp, const void *grad_value);
hipError_t launch_scatter_accumulate(const Problem &p, const BwdMapping &mp, const void *loc,
                                     const void *attn, const void *grad_out, void *grad_value,
                                     const BinnedBuffers &bins, bool accumulate,
                                     hipStream_t stream);
// Count, scan and place in one launch, one workgroup per (b, m, binned level),
// when Q * K <= local_sort_max_points() and every binned level has at most
// kMaxLocalSortBins bins: records of segment s at [s * 4QK, (s + 1) * 4QK),
// bin ranges in [starts[i], cursor[i]) (so bins.ends = bins.cursor). Extra
// workgroups of the same launch zero-fill zero_bytes (a multiple of 16, at a
// 16-byte aligned zero_dst) when zero_bytes > 0.
constexpr int kMaxLocalSortBins = 32000;  // 64000 bytes of LDS counters
int local_sort_max_points();
hipError_t launch_bin_local_sort(const Problem &p, const void *loc, const void *attn,
                                 const BinnedBuffers &bins, int max_level_bins, void *zero_dst,
                                 size_t zero_bytes, hipStream_t stream);
// grad_value atomics only, for the levels that are not binned (no value
// gathers); used with launch_gradients when some levels are binned.
hipError_t launch_scatter(const Problem &p, const BwdMapping &mp, const void *loc,
                          const void *attn, const void *grad_out, void *grad_value,
                          float *workspace, hipStream_t stream);

// grad_loc / grad_attn only, in the forward's lane mapping.
hipError_t launch_gradients(const Problem &p, const Mapping &mp, const void *value,
                            const void *loc, const void *attn, const void *grad_out,
                            void *grad_loc, void *grad_attn, hipStream_t stream);
hipError_t launch_bin_accumulate(const Problem &p, const BwdMapping &mp, const void *grad_out,
                                 void *grad_value, const BinnedBuffers &bins, bool accumulate,
                                 hipStream_t stream);

// Point-parallel forward foil (measurement only); vec = channels per load
// (16 bytes when D and the pointers allow, else 1). Needs L*K dividing 256 and
// D <= 64 (host-checked).
hipError_t launch_forward_foil(const Problem &p, int vec, const void *value, const void *loc,
                               const void *attn, void *out, hipStream_t stream);

// Fill `bytes` bytes (a multiple of 2) at `dst` with zeros.
// Sampling-parameter preparation around the core (msda_prep_kernels.hip):
// locations = reference + offset / (W_l, H_l), weights = softmax over the
// L*K points of each (b, q, m), and the matching backward. `dtype` is the
// storage type of every tensor of these calls; `ref_levels` is 1 for one
// reference point per query, L for one per (query, level).
struct PrepProblem {
    int dtype;
    int64_t B, Q, M, L, K;
    int ref_levels;
    float H[MSDA_MAX_LEVELS];
    float W[MSDA_MAX_LEVELS];
};

hipError_t launch_sampling_prep(const PrepProblem &p, const void *ref, const void *offsets,
                                const void *logits, void *loc, void *attn, hipStream_t stream);
hipError_t launch_sampling_prep_backward(const PrepProblem &p, const void *attn,
                                         const void *grad_loc, const void *grad_attn,
                                         void *grad_offsets, void *grad_logits,
                                         hipStream_t stream);
hipError_t launch_reference_grad(const PrepProblem &p, const void *grad_loc, void *grad_ref,
                                 hipStream_t stream);

hipError_t launch_zero(void *dst, size_t bytes, hipStream_t stream);

// The pre-reduced levels' contributions into their fp32 scratch rows (the
// scratch must be zero-filled first; scratch_add rounds it into grad_value).
hipError_t launch_prereduce(const Problem &p, const PreTiles &pt, const void *loc, const void *attn,
                            const void *grad_out, float *workspace, hipStream_t stream);

// Atomic request-rate probe (msda_probe.hip, measurement only): workgroups of
// 256 threads, each lane `iters` no-return adds (fp32, or packed bf16 pairs)
// in runs of 2^log2run lanes per 64-byte segment of `buf` (nseg segments).
hipError_t launch_atomic_probe(void *buf, int64_t nseg, int bf16, int log2run, int64_t workgroups,
                               int iters, hipStream_t stream);

// For every level with scratch_off >= 0 and every batch:
// grad_value rows of that level += (dtype) workspace block.
hipError_t launch_scratch_add(const Problem &p, const float *workspace, void *grad_value,
                              hipStream_t stream);

}  // namespace msda
