// Host side of the C ABI declared in include/msda.h: argument validation, the
// level table, the lane mapping, the accumulation policy and the launches.
//
// Every check runs before the first HIP call, so a rejected call has no side
// effect and works on a host without a GPU. The default level_start_index is
// the exclusive prefix sum of H_l * W_l (msda-triton README, section
// "Quickstart"; course page "4. The forward kernel", section "The wrapper").

#include <stdarg.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <string>

#include "msda_launch.h"

namespace {

thread_local std::string g_last_error;

// Launch events of msda_set_launch_events (this thread's next call only).
constexpr int kMaxLaunchEvents = 64;
thread_local hipEvent_t g_launch_events[kMaxLaunchEvents];
thread_local int g_launch_events_n = 0;
thread_local int g_launch_events_next = 0;

thread_local msda::TimedLaunch g_timed_launch;

// Arm the next launch's event pair (called as an argument of marked(), so it
// runs right before the launch call itself): the launch records them at its
// kernel's start and end.
hipStream_t before(hipStream_t s) {
    if (g_launch_events_next + 1 < g_launch_events_n)
        g_timed_launch = {g_launch_events[g_launch_events_next],
                          g_launch_events[g_launch_events_next + 1]};
    return s;
}

thread_local const char *g_launch_names[kMaxLaunchEvents / 2];
thread_local const char *g_recorded_names[kMaxLaunchEvents / 2];

// After a launch: disarm the pair and keep its name (the pair is consumed
// only when both fit in the caller's array). A helper that launched nothing
// (an empty fill) gets both events recorded here, back to back.
hipError_t marked(hipError_t err, hipStream_t s, const char *name) {
    if (g_launch_events_next + 1 < g_launch_events_n) {
        if (err == hipSuccess && g_timed_launch.start) {
            err = hipEventRecord(g_timed_launch.start, s);
            if (err == hipSuccess) err = hipEventRecord(g_timed_launch.stop, s);
        }
        g_timed_launch = {};
        g_launch_names[g_launch_events_next / 2] = name;
        g_launch_events_next += 2;
    }
    return err;
}

thread_local int g_launch_events_recorded = 0;

struct LaunchEventsScope {  // clears the instrumentation when a call returns
    ~LaunchEventsScope() {
        if (g_launch_events_n) {
            g_launch_events_recorded = g_launch_events_next;
            for (int i = 0; i < g_launch_events_next / 2; ++i) g_recorded_names[i] = g_launch_names[i];
        }
        g_launch_events_n = g_launch_events_next = 0;
        g_timed_launch = {};
    }
};

// Side stream of the binned backward: per thread and device, created on the
// first binned call (default priority, non-blocking), never destroyed. The
// binned chain (count, scan, place, accumulate) runs on it while the caller's
// stream runs the zero fill and the gradient / scatter kernels; two event
// waits fork it from the caller's stream and one joins it back, so the call
// stays stream-ordered and capturable in a HIP graph.
constexpr int kMaxDevices = 64;
struct SideStream {
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, zeroed = nullptr, join = nullptr;
};
thread_local SideStream g_side[kMaxDevices];

// The side stream for the device of `s`, or nullptr to run the chain on `s`
// itself (no usable device, or `s` is being captured and the side stream
// does not exist yet: creating one is not done under capture).
SideStream *side_stream(hipStream_t s) {
    int dev = -1;
    if (s ? hipStreamGetDevice(s, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
        return nullptr;
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    SideStream &ss = g_side[dev];
    if (ss.stream) return &ss;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
        return nullptr;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    SideStream made;
    bool good = hipStreamCreateWithFlags(&made.stream, hipStreamNonBlocking) == hipSuccess &&
                hipEventCreateWithFlags(&made.fork, hipEventDisableTiming) == hipSuccess &&
                hipEventCreateWithFlags(&made.zeroed, hipEventDisableTiming) == hipSuccess &&
                hipEventCreateWithFlags(&made.join, hipEventDisableTiming) == hipSuccess;
    if (cur != dev) (void)hipSetDevice(cur);
    if (!good) return nullptr;  // (partially created handles are kept out of use)
    ss = made;
    return &ss;
}

// Destroy this thread's side streams and events on every device.
hipError_t release_side_streams() {
    hipError_t first = hipSuccess;
    int cur = -1;
    bool have_cur = false;
    for (int dev = 0; dev < kMaxDevices; ++dev) {
        SideStream &ss = g_side[dev];
        if (!ss.stream) continue;
        if (!have_cur) have_cur = hipGetDevice(&cur) == hipSuccess;
        hipError_t e = hipSetDevice(dev);
        // (destroying a stream with work still queued lets that work finish first)
        if (e == hipSuccess) e = hipStreamDestroy(ss.stream);
        for (hipEvent_t ev : {ss.fork, ss.zeroed, ss.join}) {
            const hipError_t ee = hipEventDestroy(ev);
            if (e == hipSuccess) e = ee;
        }
        if (first == hipSuccess) first = e;
        ss = SideStream();
    }
    if (have_cur) (void)hipSetDevice(cur);
    return first;
}

int fail(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return MSDA_OK;
}

size_t elem_size(int dtype) { return dtype == MSDA_F32 ? 4 : 2; }

bool mul_ok(int64_t a, int64_t b, int64_t *out) {
    __int128 r = (__int128)a * (__int128)b;
    if (r > (__int128)INT64_MAX) return false;
    *out = (int64_t)r;
    return true;
}

// Validate sizes and build the level table.
int make_problem(int dtype, int64_t B, int64_t S, int64_t M, int64_t D, int64_t L,
                 const int64_t *shapes, const int64_t *starts, int64_t Q, int64_t K,
                 msda::Problem *p) {
    if (dtype != MSDA_F32 && dtype != MSDA_F16 && dtype != MSDA_BF16)
        return fail(MSDA_ERR_DTYPE, "unknown dtype %d (0=f32, 1=f16, 2=bf16)", dtype);
    if (B < 0 || Q < 0) return fail(MSDA_ERR_SHAPE, "batch (%lld) and num_queries (%lld) must be >= 0",
                                    (long long)B, (long long)Q);
    if (S < 1 || M < 1 || D < 1 || K < 1)
        return fail(MSDA_ERR_SHAPE,
                    "num_keys (%lld), num_heads (%lld), head_dim (%lld) and num_points (%lld) "
                    "must be >= 1",
                    (long long)S, (long long)M, (long long)D, (long long)K);
    if (L < 1) return fail(MSDA_ERR_SHAPE, "num_levels must be >= 1, got %lld", (long long)L);
    if (L > MSDA_MAX_LEVELS)
        return fail(MSDA_ERR_UNSUPPORTED, "num_levels %lld exceeds the limit of %d", (long long)L,
                    MSDA_MAX_LEVELS);
    if (!shapes) return fail(MSDA_ERR_NULL_ARG, "spatial_shapes is NULL");
    // Products used for indexing must fit comfortably in int64 / int32.
    int64_t t, bsmd, bqmlk;
    if (!mul_ok(B, S, &t) || !mul_ok(t, M, &t) || !mul_ok(t, D, &bsmd) ||
        bsmd > ((int64_t)1 << 62))
        return fail(MSDA_ERR_SHAPE, "value tensor B*S*M*D overflows");
    if (!mul_ok(B, Q, &t) || !mul_ok(t, M, &t) || !mul_ok(t, L, &t) || !mul_ok(t, K, &bqmlk) ||
        bqmlk > ((int64_t)1 << 61))
        return fail(MSDA_ERR_SHAPE, "sampling tensor B*Q*M*L*K overflows");
    if (M > INT32_MAX || D > INT32_MAX || L * K > (1 << 20) || Q > INT32_MAX)
        return fail(MSDA_ERR_UNSUPPORTED,
                    "num_heads, head_dim, num_queries or num_levels*num_points too large");
    p->dtype = dtype;
    p->pdtype = dtype;
    p->B = B;
    p->S = S;
    p->M = M;
    p->D = D;
    p->L = L;
    p->Q = Q;
    p->K = K;
    memset(&p->levels, 0, sizeof(p->levels));
    for (int l = 0; l < MSDA_MAX_LEVELS; ++l) {
        p->levels.scratch_off[l] = -1;
        p->levels.bin_shift[l] = -1;
    }
    p->nbbm = 0;
    int64_t acc = 0;
    for (int64_t l = 0; l < L; ++l) {
        const int64_t H = shapes[2 * l], W = shapes[2 * l + 1];
        if (H < 1 || W < 1)
            return fail(MSDA_ERR_LEVELS, "level %lld has shape (%lld, %lld); both must be >= 1",
                        (long long)l, (long long)H, (long long)W);
        if (H >= (1 << 24) || W >= (1 << 24))
            return fail(MSDA_ERR_UNSUPPORTED, "level %lld shape (%lld, %lld) exceeds 2^24",
                        (long long)l, (long long)H, (long long)W);
        const int64_t st = starts ? starts[l] : acc;
        acc += H * W;
        if (st < 0 || st > S || H * W > S - st)
            return fail(MSDA_ERR_LEVELS,
                        "level %lld (start %lld, %lld x %lld) does not fit in num_keys = %lld",
                        (long long)l, (long long)st, (long long)H, (long long)W, (long long)S);
        p->levels.H[l] = (int32_t)H;
        p->levels.W[l] = (int32_t)W;
        p->levels.start[l] = st;
    }
    return MSDA_OK;
}

bool aligned(const void *ptr, size_t a) { return reinterpret_cast<uintptr_t>(ptr) % a == 0; }

// msda_debug_force_flat_gathers: process-wide, read at planning and launch.
std::atomic<int> g_flat_gathers{0};

int log2_ceil(int64_t x) {
    int r = 0;
    while (((int64_t)1 << r) < x) ++r;
    return r;
}

// Pick the channel vector width and the lane mapping. `vec_ptrs` are the
// pointers accessed VEC channels at a time (value, output, grad_output,
// grad_value); `need4` asks for 4-byte aligned channel pairs (packed atomics).
int choose_mapping(const msda::Problem &p, const void *const *vec_ptrs, int nptrs,
                   msda::Mapping *mp) {
    const size_t e = elem_size(p.dtype);
    static const int cand32[] = {4, 3, 2, 1};
    static const int cand16[] = {8, 4, 2, 1};
    const int *cand = e == 4 ? cand32 : cand16;
    int best = 0;
    double best_eff = -1.0;
    for (int i = 0; i < 4; ++i) {
        const int v = cand[i];
        if (p.D % v) continue;
        const size_t need = (v == 3) ? e : (size_t)v * e;
        bool ok_align = true;
        for (int j = 0; j < nptrs; ++j) ok_align = ok_align && aligned(vec_ptrs[j], need);
        if (!ok_align) continue;
        const int64_t lanes = p.D / v;
        const int lg = log2_ceil(lanes);
        if (lg > 6) continue;
        const double eff = (double)lanes / (double)((int64_t)1 << lg);
        if (eff > best_eff + 1e-9) {
            best_eff = eff;
            best = v;
        }
    }
    if (!best)
        return fail(MSDA_ERR_UNSUPPORTED,
                    "head_dim %lld needs more than 64 lanes at every supported vector width",
                    (long long)p.D);
    mp->vec = best;
    mp->log2_group = log2_ceil(p.D / best);
    // Few queries: let up to 4 lane groups split one query's points so that
    // enough waves are in flight (about 8 per CU on 256 CUs).
    const int64_t target_lanes = (int64_t)256 * 8 * 64;
    const int64_t lanes = p.B * p.M * p.Q * ((int64_t)1 << mp->log2_group);
    int ls = 0;
    // The lanes of one query (group x split) must stay inside one 64-lane wave.
    while (ls < 2 && p.K % ((int64_t)2 << ls) == 0 && lanes * ((int64_t)1 << ls) < target_lanes &&
           mp->log2_group + ls + 1 <= 6)
        ++ls;
    mp->log2_split = ls;
    // Workgroups: 2^(8 - group - split) queries each, B*M*ceil(Q/that) of them.
    const int64_t qpb = (int64_t)256 >> (mp->log2_group + mp->log2_split);
    const int64_t qblocks = (p.Q + qpb - 1) / qpb;
    if (qblocks > INT32_MAX || p.B * p.M * qblocks > (int64_t)INT32_MAX - 8)
        return fail(MSDA_ERR_UNSUPPORTED, "too many workgroups for one launch");
    return MSDA_OK;
}

int check_ptr(const void *ptr, const char *name, int dtype) {
    if (!ptr) return fail(MSDA_ERR_NULL_ARG, "%s is NULL", name);
    if (!aligned(ptr, elem_size(dtype)))
        return fail(MSDA_ERR_ALIGN, "%s is not aligned to its element size", name);
    return MSDA_OK;
}

int hip_fail(hipError_t err, const char *what) {
    return fail(MSDA_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

// Average number of contributions a pixel of level l receives: every query
// samples K points per level, each touching 4 corners.
double contributions_per_pixel(const msda::Problem &p, int l) {
    return (double)p.Q * (double)p.K * 4.0 /
           ((double)p.levels.H[l] * (double)p.levels.W[l]);
}

int binned_levels(const msda::Problem &p) {
    int n = 0;
    for (int l = 0; l < (int)p.L; ++l) n += p.levels.bin_shift[l] >= 0;
    return n;
}

int resolved_mode(const msda::Problem &p) {
    if (p.levels.prered) return MSDA_ACCUM_PREREDUCE;
    const int nb = binned_levels(p);
    if (nb > 0) return nb == (int)p.L ? MSDA_ACCUM_BINNED : MSDA_ACCUM_MIXED;
    int n = 0;
    for (int l = 0; l < (int)p.L; ++l) n += p.levels.scratch_off[l] >= 0;
    if (n == 0) return MSDA_ACCUM_NATIVE;
    return n == (int)p.L ? MSDA_ACCUM_FP32_SCRATCH : MSDA_ACCUM_PER_LEVEL;
}

bool valid_accum(int accum) { return accum >= MSDA_ACCUM_AUTO && accum <= MSDA_ACCUM_PREREDUCE; }

// A level is "contended" above this many contributions per pixel.
constexpr double kContended = 4.0;

// Decide, per level, whether the backward accumulates in fp32 scratch, and
// lay the scratch blocks out back to back. Returns the workspace bytes.
// FP32_SCRATCH: every level of 16-bit data; PER_LEVEL: 16-bit levels above 4
// contributions per pixel (bf16 keeps 8 significant bits: long chains of
// rounded packed adds drift beyond the 5e-2 parity bar in the tails, while
// fp16's 11 bits held parity on every tested shape); NATIVE: none.
size_t plan_scratch(msda::Problem *p, int mode) {
    size_t total = 0;
    for (int l = 0; l < (int)p->L; ++l) {
        bool scratch = false;
        if (p->dtype != MSDA_F32) {
            if (mode == MSDA_ACCUM_FP32_SCRATCH) scratch = true;
            else if (mode == MSDA_ACCUM_PER_LEVEL) scratch = contributions_per_pixel(*p, l) > kContended;
        }
        if (scratch) {
            p->levels.scratch_off[l] = (int64_t)(total / sizeof(float));
            total += (size_t)(p->B * (int64_t)p->levels.H[l] * p->levels.W[l] * p->M * p->D) *
                     sizeof(float);
        } else {
            p->levels.scratch_off[l] = -1;
        }
    }
    return total;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool levels_overlap(const msda::Problem &p) {
    for (int i = 0; i < (int)p.L; ++i)
        for (int k = i + 1; k < (int)p.L; ++k) {
            const int64_t a0 = p.levels.start[i], a1 = a0 + (int64_t)p.levels.H[i] * p.levels.W[i];
            const int64_t b0 = p.levels.start[k], b1 = b0 + (int64_t)p.levels.H[k] * p.levels.W[k];
            if (a0 < b1 && b0 < a1) return true;
        }
    return false;
}

// Rows of [0, S) outside every level (padding rows) are written by no bin.
bool levels_leave_gaps(const msda::Problem &p) {
    int64_t covered = 0;
    for (int l = 0; l < (int)p.L; ++l) covered += (int64_t)p.levels.H[l] * p.levels.W[l];
    return covered != p.S;  // levels do not overlap here, so equality covers [0, S)
}

// Binned grad_value plan: per level a bin height of 2^bin_shift pixel rows,
// at most 16, so that a bin holds about kBinRecords records if the level's
// points spread evenly (contributions per pixel Q*K*4 / (H*W)). Returns false
// where the path cannot apply; on success fills the level table and the
// workspace layout. Measured on MI355X (encoder workload step): 256 records
// per bin 1439 us, 1024 1275 us, 4096 1239 us, 16384 1303 us.
constexpr double kBinRecords = 4096.0;
// Up to this many tiles of 4096 bin counts one workgroup scans them (one
// launch); beyond, the scan runs as three launches over all tiles at once.
constexpr int64_t kSingleScanTiles = 2;

struct BinPlan {
    int64_t nbins = 0, records = 0;
    size_t starts_off = 0, cursor_off = 0, tiles_off = 0, records_off = 0, bytes = 0;
    int max_level_bins = 0;    // bins of the binned level with the most
    bool local_sort = false;   // one-launch count / scan / place applies
};

// Bins the levels selected by `contended_only` (all levels, or those above
// kContended contributions per pixel); the other levels keep bin_shift = -1.
bool plan_bins(msda::Problem *p, BinPlan *bp, bool contended_only,
               double max_contributions = 1e300) {
    const int64_t e = p->dtype == MSDA_F32 ? 4 : 2;
    const int64_t P = p->B * p->Q * p->M * p->L * p->K;
    // 28-bit query field; 32-bit record indices; buffer-addressed value and
    // grad_output slices of one batch
    if (levels_overlap(*p) || p->Q >= ((int64_t)1 << 28) || 4 * P >= ((int64_t)1 << 32) ||
        !msda::slice_fits_buffer(*p) ||
        p->Q * p->M * p->D * e > ((int64_t)1 << 31) - 64 || p->B * p->Q * p->M >= ((int64_t)1 << 31))
        return false;
    // rows per bin: a power of two, at most the 16 lane groups of the
    // accumulating workgroup (each sums one row, or one replica of a row)
    const int tp_max = 16;
    int64_t nbbm = 0;
    int nlev = 0;
    for (int l = 0; l < (int)p->L; ++l) {
        const double c = contributions_per_pixel(*p, l);
        p->levels.bin_off[l] = (int32_t)nbbm;  // a level without bins shares the next level's offset
        p->levels.bin_shift[l] = -1;
        if (contended_only && !(c > kContended)) continue;
        if (!(c <= max_contributions)) continue;  // pre-reduced instead
        const double want = c > 0 ? kBinRecords / c : (double)tp_max;
        const int64_t HW = (int64_t)p->levels.H[l] * p->levels.W[l];
        int sh = 0;  // no taller than the level itself rounded up to a power of two
        while ((1 << (sh + 1)) <= tp_max && (double)(1 << (sh + 1)) <= want &&
               ((int64_t)1 << sh) < HW)
            ++sh;
        p->levels.bin_shift[l] = sh;
        const int64_t nbl = (HW + (1 << sh) - 1) >> sh;
        nbbm += nbl;
        if (nbl > bp->max_level_bins) bp->max_level_bins = (int)std::min<int64_t>(nbl, INT32_MAX);
        p->levels.blevel[nlev++] = l;
        p->levels.nblev = nlev;
        if (nbbm >= ((int64_t)1 << 31)) return false;
    }
    const int64_t nbins = p->B * p->M * nbbm;
    if (nbins >= ((int64_t)1 << 31) - 1) return false;
    p->nbbm = nbbm;
    bp->nbins = nbins;
    bp->records = 4 * p->B * p->Q * p->M * p->K * nlev;
    // one workgroup per (b, m, binned level) can sort the level's records in
    // LDS with 16-bit counters
    bp->local_sort = p->Q * p->K <= msda::local_sort_max_points() &&
                     bp->max_level_bins <= msda::kMaxLocalSortBins;
    bp->starts_off = 0;
    bp->cursor_off = align_up((size_t)(nbins + 1) * 4, 256);
    bp->tiles_off = bp->cursor_off + align_up((size_t)nbins * 4, 256);
    bp->records_off = bp->tiles_off + align_up((size_t)(msda::scan_tiles(nbins) + 1) * 8, 256);
    bp->bytes = bp->records_off + (size_t)bp->records * 8;
    return true;
}

// Pre-reduced levels (PREREDUCE): those above kPreReduce contributions per
// pixel. Their fp32 scratch follows the bins in the workspace (256-byte
// aligned at `offset`); returns its bytes and fills the launch layout.
constexpr double kPreReduce = 256.0;
constexpr int64_t kPreWindowPixels = 1024;       // per level, shaped like the level
constexpr int64_t kPreMaxLdsBytes = 152 * 1024;  // at most, beside the static LDS

bool pixel_queries(const msda::Problem &p) {
    if (p.Q != p.S || levels_overlap(p)) return false;
    int64_t covered = 0;
    for (int l = 0; l < (int)p.L; ++l) covered += (int64_t)p.levels.H[l] * p.levels.W[l];
    return covered == p.S;
}

// Returns false when the LDS a workgroup needs does not fit.
bool plan_prereduce(msda::Problem *p, size_t offset, msda::PreTiles *pt, size_t *bytes) {
    memset(pt, 0, sizeof(*pt));
    *bytes = 0;
    p->levels.prered = 0;
    size_t total = 0;
    for (int l = 0; l < (int)p->L; ++l) {
        if (!(contributions_per_pixel(*p, l) > kPreReduce)) continue;
        p->levels.prered |= 1u << l;
        p->levels.scratch_off[l] = (int64_t)((offset + total) / sizeof(float));
        total += (size_t)(p->B * (int64_t)p->levels.H[l] * p->levels.W[l] * p->M * p->D) *
                 sizeof(float);
        pt->lev[pt->nlev++] = l;
    }
    *bytes = total;
    if (!pt->nlev) return true;
    pt->pixel = pixel_queries(*p) ? 1 : 0;
    // windows of about kPreWindowPixels, shaped like their level
    for (int li = 0; li < pt->nlev; ++li) {
        const int l = pt->lev[li];
        const double H = p->levels.H[l], W = p->levels.W[l];
        int64_t wy = std::max<int64_t>(1, (int64_t)std::sqrt((double)kPreWindowPixels * H / W));
        wy = std::min<int64_t>(wy, p->levels.H[l]);
        const int64_t wx =
            std::min<int64_t>(std::max<int64_t>(1, kPreWindowPixels / wy), p->levels.W[l]);
        pt->wx[li] = (int32_t)wx;
        pt->wy[li] = (int32_t)wy;
        pt->max_px = std::max<int32_t>(pt->max_px, (int32_t)(wx * wy));
    }
    const msda::LevelTable &lt = p->levels;
    if (pt->pixel)
        for (int l = 1; l < (int)p->L; ++l)
            if ((int64_t)lt.H[l] * lt.W[l] > (int64_t)lt.H[pt->ref] * lt.W[pt->ref]) pt->ref = l;
    // blocks: the largest whose working set fits in LDS (pixel tiles of 16 x
    // 16 pixels of the reference level, or 256 consecutive queries, halved
    // until it fits)
    for (int side = pt->pixel ? 16 : 256; side >= 1; side /= 2) {
        int64_t maxq = side;
        if (pt->pixel) {  // the largest merged tile
            pt->tile = side;
            const int32_t H0 = lt.H[pt->ref], W0 = lt.W[pt->ref];
            const int64_t ny = (H0 + side - 1) / side, nx = (W0 + side - 1) / side;
            maxq = 0;
            for (int64_t ty = 0; ty < ny; ++ty)
                for (int64_t tx = 0; tx < nx; ++tx) {
                    int64_t n = 0;
                    for (int l = 0; l < (int)p->L; ++l)
                        n += (int64_t)(msda::pre_tile_span(ty + 1, side, lt.H[l], H0, ny) -
                                       msda::pre_tile_span(ty, side, lt.H[l], H0, ny)) *
                             (msda::pre_tile_span(tx + 1, side, lt.W[l], W0, nx) -
                              msda::pre_tile_span(tx, side, lt.W[l], W0, nx));
                    maxq = std::max(maxq, n);
                }
        } else {
            pt->lin_queries = side;
        }
        if (4 * maxq * p->K >= INT32_MAX) continue;
        pt->max_queries = (int32_t)maxq;
        pt->max_records = (int32_t)(4 * maxq * p->K);
        pt->max_chunks = pt->max_records / msda::kPreChunk + pt->max_px;
        if (msda::pre_lds_bytes(*pt, p->D, p->dtype == MSDA_F32 ? 4 : 2) <= kPreMaxLdsBytes)
            return true;
    }
    return false;
}

// Why an explicit BINNED / MIXED / PREREDUCE request was refused.
const char *inapplicable_mode(int accum) {
    return accum == MSDA_ACCUM_PREREDUCE
               ? "pre-reduced accumulation does not apply to this problem (it needs the binned "
                 "conditions, head_dim <= 256 and room in LDS)"
               : "binned accumulation does not apply to this problem";
}

void clear_bins(msda::Problem *p) {
    for (int l = 0; l < MSDA_MAX_LEVELS; ++l) {
        p->levels.bin_shift[l] = -1;
        p->levels.bin_off[l] = 0;
        p->levels.blevel[l] = 0;
    }
    p->levels.nblev = 0;
    p->nbbm = 0;
}

// Resolve `accum` and plan the buffers. Returns the resolved mode, or -1 if
// an explicit BINNED / MIXED cannot apply. *bytes = workspace bytes needed.
// AUTO is MIXED where binning applies (BINNED when every level is contended,
// NATIVE when none is), else PER_LEVEL for bf16 and NATIVE otherwise.
// Measured on MI355X: native atomics are fastest on levels whose pixels
// receive a few contributions; on contended levels they serialise on the same
// addresses (and bf16 adds lose precision), where the binned sum wins.
int plan_accum(msda::Problem *p, int accum, size_t *bytes, BinPlan *bp,
               msda::PreTiles *pt = nullptr) {
    clear_bins(p);
    plan_scratch(p, MSDA_ACCUM_NATIVE);
    p->levels.prered = 0;
    *bytes = 0;
    if (accum == MSDA_ACCUM_PREREDUCE) {
        msda::PreTiles tmp;
        if (!pt) pt = &tmp;
        // (D <= 256: a block's upstream-gradient rows leave room for windows
        // in LDS)
        if (p->D > 256 || !plan_bins(p, bp, true, kPreReduce)) {
            clear_bins(p);
            return -1;
        }
        if (bp->nbins == 0) clear_bins(p);
        const size_t off = bp->nbins > 0 ? align_up(bp->bytes, 256) : 0;
        size_t scr = 0;
        if (!plan_prereduce(p, off, pt, &scr)) {
            clear_bins(p);
            plan_scratch(p, MSDA_ACCUM_NATIVE);
            p->levels.prered = 0;
            return -1;
        }
        *bytes = scr ? off + scr : (bp->nbins > 0 ? bp->bytes : 0);
        return resolved_mode(*p);
    }
    if (accum == MSDA_ACCUM_BINNED || accum == MSDA_ACCUM_MIXED || accum == MSDA_ACCUM_AUTO) {
        if (plan_bins(p, bp, accum != MSDA_ACCUM_BINNED)) {
            if (bp->nbins > 0) *bytes = bp->bytes;
            else clear_bins(p);
            return resolved_mode(*p);
        }
        clear_bins(p);
        if (accum != MSDA_ACCUM_AUTO) return -1;
    }
    int mode = accum;
    if (accum == MSDA_ACCUM_AUTO)
        mode = p->dtype == MSDA_BF16 ? MSDA_ACCUM_PER_LEVEL : MSDA_ACCUM_NATIVE;
    *bytes = plan_scratch(p, mode);
    return resolved_mode(*p);
}

// Backward lane mapping: slots of one dword for 16-bit data with even D and
// 4-byte aligned pointers, else one channel; G = min(16, slots) lanes per
// query so that one instruction of a group covers one 64-byte segment.
int choose_bwd_mapping(const msda::Problem &p, bool pairs_aligned, msda::BwdMapping *mp) {
    const size_t e = elem_size(p.dtype);
    mp->slot = (e == 2 && p.D % 2 == 0 && pairs_aligned) ? 2 : 1;
    const int64_t nslots = p.D / mp->slot;
    const int lg = log2_ceil(nslots) < 4 ? log2_ceil(nslots) : 4;
    mp->log2_group = lg;
    const int64_t per_lane = (nslots + (1 << lg) - 1) >> lg;
    static const int js[] = {1, 2, 3, 4, 8, 16, 32};
    mp->j = 0;
    for (int j : js)
        if (j >= per_lane) {
            mp->j = j;
            break;
        }
    if (!mp->j || (mp->slot == 2 && mp->j > 16))
        return fail(MSDA_ERR_UNSUPPORTED, "head_dim %lld too large for the backward (max 512)",
                    (long long)p.D);
    const int64_t target_lanes = (int64_t)256 * 8 * 64;
    const int64_t lanes = p.B * p.M * p.Q * ((int64_t)1 << lg);
    int ls = 0;
    while (ls < 2 && p.K % ((int64_t)2 << ls) == 0 && lanes * ((int64_t)1 << ls) < target_lanes &&
           lg + ls + 1 <= 6)
        ++ls;
    mp->log2_split = ls;
    const int64_t qpb = (int64_t)256 >> (lg + ls);
    const int64_t qblocks = (p.Q + qpb - 1) / qpb;
    if (qblocks > INT32_MAX || p.B * p.M * qblocks > (int64_t)INT32_MAX - 8)
        return fail(MSDA_ERR_UNSUPPORTED, "too many workgroups for one launch");
    return MSDA_OK;
}

// Parameter dtype of a call (sampling locations, attention weights and their
// gradients): the value dtype, or fp32 beside 16-bit values (msda-triton
// README, section "Caveats": 16-bit locations quantise coordinates at large
// resolutions). The mixed kernels address the batch's value slice through a
// buffer resource, so that slice must stay below 2 GiB.
int set_param_dtype(msda::Problem *p, int pdtype) {
    if (pdtype != p->dtype && !(pdtype == MSDA_F32 && p->dtype != MSDA_F32))
        return fail(MSDA_ERR_DTYPE,
                    "param_dtype %d must equal value_dtype %d or be MSDA_F32 beside 16-bit values",
                    pdtype, p->dtype);
    if (pdtype != p->dtype && !msda::slice_fits_buffer(*p))
        return fail(MSDA_ERR_UNSUPPORTED,
                    "mixed dtypes need a value slice of one batch below 2 GiB");
    p->pdtype = pdtype;
    return MSDA_OK;
}

}  // namespace

namespace msda {
TimedLaunch &timed_launch() { return g_timed_launch; }
bool flat_gathers_forced() { return g_flat_gathers.load(std::memory_order_relaxed) != 0; }
}  // namespace msda

extern "C" {

int msda_abi_version(void) { return MSDA_ABI_VERSION; }

int msda_launch_events_recorded(void) { return g_launch_events_recorded; }

const char *msda_launch_events_name(int i) {
    if (i < 0 || i >= g_launch_events_recorded / 2) return nullptr;
    return g_recorded_names[i];
}

int msda_set_launch_events(void *const *events, int count) {
    if (count < 0 || count > kMaxLaunchEvents)
        return fail(MSDA_ERR_SHAPE, "launch event count %d outside [0, %d]", count, kMaxLaunchEvents);
    if (count > 0 && !events) return fail(MSDA_ERR_NULL_ARG, "events is NULL");
    for (int i = 0; i < count; ++i) {
        if (!events[i]) return fail(MSDA_ERR_NULL_ARG, "event %d is NULL", i);
        g_launch_events[i] = static_cast<hipEvent_t>(events[i]);
    }
    g_launch_events_n = count;
    g_launch_events_next = 0;
    return ok();
}

const char *msda_last_error(void) { return g_last_error.c_str(); }

int msda_probe_atomic_requests(void *buffer, size_t buffer_bytes, int bf16,
                               int dwords_per_request, int64_t workgroups, int iters,
                               int64_t *requests, void *stream) {
    LaunchEventsScope events_scope;
    if (!buffer || !requests) return fail(MSDA_ERR_NULL_ARG, "buffer or requests is NULL");
    if (!aligned(buffer, 64)) return fail(MSDA_ERR_ALIGN, "buffer must be 64-byte aligned");
    int log2run = -1;
    for (int r = 0; r <= 4; ++r)
        if (dwords_per_request == (1 << r)) log2run = r;
    if (log2run < 0)
        return fail(MSDA_ERR_SHAPE, "dwords_per_request must be 1, 2, 4, 8 or 16, got %d",
                    dwords_per_request);
    // the largest power of two of whole 64-byte segments that fits
    int64_t nseg = 1;
    while (nseg * 2 <= (int64_t)(buffer_bytes / 64) && nseg < ((int64_t)1 << 30)) nseg *= 2;
    if ((int64_t)(buffer_bytes / 64) < 1)
        return fail(MSDA_ERR_SHAPE, "buffer must hold at least one 64-byte segment");
    if (workgroups < 1 || workgroups > ((int64_t)1 << 24) || iters < 1)
        return fail(MSDA_ERR_SHAPE, "workgroups must be in [1, 2^24] and iters >= 1");
    *requests = (workgroups * 256 >> log2run) * (int64_t)iters;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t err =
        marked(msda::launch_atomic_probe(buffer, nseg, bf16 ? 1 : 0, log2run, workgroups, iters,
                                         before(s)),
               s, "atomic_probe_kernel");
    if (err != hipSuccess) return hip_fail(err, "probe launch");
    return ok();
}

int msda_release_thread_resources(void) {
    const hipError_t err = release_side_streams();
    if (err != hipSuccess) return hip_fail(err, "releasing the side stream");
    return ok();
}

int msda_debug_force_flat_gathers(int enable) {
    return g_flat_gathers.exchange(enable ? 1 : 0) ? 1 : 0;
}

const char *msda_status_string(int status) {
    switch (status) {
        case MSDA_OK: return "ok";
        case MSDA_ERR_NULL_ARG: return "null argument";
        case MSDA_ERR_SHAPE: return "bad shape";
        case MSDA_ERR_LEVELS: return "bad level table";
        case MSDA_ERR_DTYPE: return "bad dtype or accumulation mode";
        case MSDA_ERR_ALIGN: return "misaligned pointer";
        case MSDA_ERR_WORKSPACE: return "workspace missing or too small";
        case MSDA_ERR_HIP: return "HIP error";
        case MSDA_ERR_UNSUPPORTED: return "unsupported size";
        default: return "unknown status";
    }
}

static int forward_impl(int dtype, int pdtype, int64_t batch, int64_t num_keys,
                        int64_t num_heads, int64_t head_dim, int64_t num_levels,
                        const int64_t *spatial_shapes, const int64_t *level_start_index,
                        int64_t num_queries, int64_t num_points, const void *value,
                        const void *sampling_locations, const void *attention_weights,
                        void *output, void *stream) {
    LaunchEventsScope events_scope;
    msda::Problem p;
    int st = make_problem(dtype, batch, num_keys, num_heads, head_dim, num_levels, spatial_shapes,
                          level_start_index, num_queries, num_points, &p);
    if (st) return st;
    if ((st = set_param_dtype(&p, pdtype))) return st;
    if (p.B == 0 || p.Q == 0) return ok();  // empty tensors may carry NULL pointers
    if ((st = check_ptr(value, "value", dtype))) return st;
    if ((st = check_ptr(sampling_locations, "sampling_locations", pdtype))) return st;
    if ((st = check_ptr(attention_weights, "attention_weights", pdtype))) return st;
    if ((st = check_ptr(output, "output", dtype))) return st;
    const void *vec_ptrs[] = {value, output};
    msda::Mapping mp;
    if ((st = choose_mapping(p, vec_ptrs, 2, &mp))) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err = marked(msda::launch_forward(p, mp, value, sampling_locations,
                                                 attention_weights, output, before(s)),
                            s, "msda_fwd_kernel");
    if (err != hipSuccess) return hip_fail(err, "forward launch");
    return ok();
}

int msda_forward(int dtype, int64_t batch, int64_t num_keys, int64_t num_heads, int64_t head_dim,
                 int64_t num_levels, const int64_t *spatial_shapes,
                 const int64_t *level_start_index, int64_t num_queries, int64_t num_points,
                 const void *value, const void *sampling_locations, const void *attention_weights,
                 void *output, void *stream) {
    return forward_impl(dtype, dtype, batch, num_keys, num_heads, head_dim, num_levels,
                        spatial_shapes, level_start_index, num_queries, num_points, value,
                        sampling_locations, attention_weights, output, stream);
}

int msda_forward_ex(int value_dtype, int param_dtype, int64_t batch, int64_t num_keys,
                    int64_t num_heads, int64_t head_dim, int64_t num_levels,
                    const int64_t *spatial_shapes, const int64_t *level_start_index,
                    int64_t num_queries, int64_t num_points, const void *value,
                    const void *sampling_locations, const void *attention_weights, void *output,
                    void *stream) {
    return forward_impl(value_dtype, param_dtype, batch, num_keys, num_heads, head_dim,
                        num_levels, spatial_shapes, level_start_index, num_queries, num_points,
                        value, sampling_locations, attention_weights, output, stream);
}

int msda_forward_point_parallel(int dtype, int64_t batch, int64_t num_keys, int64_t num_heads,
                                int64_t head_dim, int64_t num_levels,
                                const int64_t *spatial_shapes, const int64_t *level_start_index,
                                int64_t num_queries, int64_t num_points, const void *value,
                                const void *sampling_locations, const void *attention_weights,
                                void *output, void *stream) {
    LaunchEventsScope events_scope;
    msda::Problem p;
    int st = make_problem(dtype, batch, num_keys, num_heads, head_dim, num_levels, spatial_shapes,
                          level_start_index, num_queries, num_points, &p);
    if (st) return st;
    const int64_t LK = p.L * p.K;
    if (LK > 256 || 256 % LK != 0 || p.D > 64)
        return fail(MSDA_ERR_UNSUPPORTED,
                    "the point-parallel foil needs num_levels*num_points dividing 256 and "
                    "head_dim <= 64 (got %lld, %lld)", (long long)LK, (long long)p.D);
    if (p.B == 0 || p.Q == 0) return ok();
    if ((st = check_ptr(value, "value", dtype))) return st;
    if ((st = check_ptr(sampling_locations, "sampling_locations", dtype))) return st;
    if ((st = check_ptr(attention_weights, "attention_weights", dtype))) return st;
    if ((st = check_ptr(output, "output", dtype))) return st;
    const size_t e = elem_size(dtype);
    const int wide = e == 4 ? 4 : 8;
    const int vec = (p.D % wide == 0 && aligned(value, (size_t)wide * e)) ? wide : 1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t err = marked(msda::launch_forward_foil(p, vec, value, sampling_locations,
                                                            attention_weights, output, before(s)),
                                  s, "msda_foil_kernel");
    if (err != hipSuccess) return hip_fail(err, "foil launch");
    return ok();
}

int msda_backward_resolve_accum(int dtype, int64_t batch, int64_t num_keys, int64_t num_heads,
                                int64_t head_dim, int64_t num_levels,
                                const int64_t *spatial_shapes, const int64_t *level_start_index,
                                int64_t num_queries, int64_t num_points, int accum) {
    msda::Problem p;
    if (make_problem(dtype, batch, num_keys, num_heads, head_dim, num_levels, spatial_shapes,
                     level_start_index, num_queries, num_points, &p))
        return -1;
    if (!valid_accum(accum)) {
        fail(MSDA_ERR_DTYPE, "unknown accumulation mode %d", accum);
        return -1;
    }
    size_t bytes;
    BinPlan bp;
    const int mode = plan_accum(&p, accum, &bytes, &bp);
    if (mode < 0) fail(MSDA_ERR_UNSUPPORTED, "%s", inapplicable_mode(accum));
    return mode;
}

int64_t msda_backward_plan(int dtype, int64_t batch, int64_t num_keys, int64_t num_heads,
                           int64_t head_dim, int64_t num_levels, const int64_t *spatial_shapes,
                           const int64_t *level_start_index, int64_t num_queries,
                           int64_t num_points, int accum, int *level_modes) {
    msda::Problem p;
    if (make_problem(dtype, batch, num_keys, num_heads, head_dim, num_levels, spatial_shapes,
                     level_start_index, num_queries, num_points, &p))
        return -1;
    if (!valid_accum(accum)) {
        fail(MSDA_ERR_DTYPE, "unknown accumulation mode %d", accum);
        return -1;
    }
    size_t bytes;
    BinPlan bp;
    if (plan_accum(&p, accum, &bytes, &bp) < 0) {
        fail(MSDA_ERR_UNSUPPORTED, "%s", inapplicable_mode(accum));
        return -1;
    }
    if (level_modes)
        for (int l = 0; l < (int)p.L; ++l)
            level_modes[l] = (p.levels.prered >> l) & 1u   ? MSDA_LEVEL_PREREDUCE
                             : p.levels.bin_shift[l] >= 0    ? MSDA_LEVEL_BINNED
                             : p.levels.scratch_off[l] >= 0 ? MSDA_LEVEL_FP32_SCRATCH
                                                            : MSDA_LEVEL_NATIVE;
    return binned_levels(p) > 0 ? bp.nbins : 0;
}

size_t msda_backward_workspace_size(int dtype, int64_t batch, int64_t num_keys, int64_t num_heads,
                                    int64_t head_dim, int64_t num_levels,
                                    const int64_t *spatial_shapes,
                                    const int64_t *level_start_index, int64_t num_queries,
                                    int64_t num_points, int accum) {
    msda::Problem p;
    if (make_problem(dtype, batch, num_keys, num_heads, head_dim, num_levels, spatial_shapes,
                     level_start_index, num_queries, num_points, &p))
        return 0;
    if (!valid_accum(accum)) {
        fail(MSDA_ERR_DTYPE, "unknown accumulation mode %d", accum);
        return 0;
    }
    size_t bytes = 0;
    BinPlan bp;
    if (plan_accum(&p, accum, &bytes, &bp) < 0) {
        fail(MSDA_ERR_UNSUPPORTED, "%s", inapplicable_mode(accum));
        return 0;
    }
    return bytes;
}

static int backward_impl(int dtype, int pdtype, int64_t batch, int64_t num_keys,
                         int64_t num_heads, int64_t head_dim, int64_t num_levels,
                         const int64_t *spatial_shapes, const int64_t *level_start_index,
                         int64_t num_queries, int64_t num_points, const void *value,
                         const void *sampling_locations, const void *attention_weights,
                         const void *grad_output, void *grad_value, void *grad_sampling_locations,
                         void *grad_attention_weights, int accum, unsigned flags,
                         void *workspace, size_t workspace_bytes, void *stream) {
    LaunchEventsScope events_scope;
    msda::Problem p;
    int st = make_problem(dtype, batch, num_keys, num_heads, head_dim, num_levels, spatial_shapes,
                          level_start_index, num_queries, num_points, &p);
    if (st) return st;
    if ((st = set_param_dtype(&p, pdtype))) return st;
    if (!valid_accum(accum)) return fail(MSDA_ERR_DTYPE, "unknown accumulation mode %d", accum);
    const unsigned known = MSDA_FLAG_ACCUMULATE_GRAD_VALUE | MSDA_FLAG_CONTINUE_SCRATCH |
                           MSDA_FLAG_DEFER_SCRATCH | MSDA_FLAG_SINGLE_STREAM;
    if (flags & ~known) return fail(MSDA_ERR_SHAPE, "unknown flag bits 0x%x", flags & ~known);
    if (p.B == 0) return ok();
    const bool accumulate = (flags & MSDA_FLAG_ACCUMULATE_GRAD_VALUE) != 0;
    const bool keep_sums = (flags & MSDA_FLAG_CONTINUE_SCRATCH) != 0;
    const bool defer = (flags & MSDA_FLAG_DEFER_SCRATCH) != 0;
    if ((keep_sums || defer) && accum != MSDA_ACCUM_FP32_SCRATCH && accum != MSDA_ACCUM_PER_LEVEL &&
        accum != MSDA_ACCUM_NATIVE)
        return fail(MSDA_ERR_SHAPE,
                    "CONTINUE_SCRATCH / DEFER_SCRATCH need an explicit NATIVE, FP32_SCRATCH or "
                    "PER_LEVEL accumulation");
    size_t need = 0;
    BinPlan bp;
    msda::PreTiles pt;
    const int mode = plan_accum(&p, accum, &need, &bp, &pt);
    if (mode < 0)
        return fail(MSDA_ERR_UNSUPPORTED, "%s", inapplicable_mode(accum));
    const bool binned = mode == MSDA_ACCUM_BINNED || mode == MSDA_ACCUM_MIXED ||
                        (p.levels.prered && bp.nbins > 0);
    const bool all_binned = mode == MSDA_ACCUM_BINNED;
    if ((st = check_ptr(value, "value", dtype))) return st;
    if ((st = check_ptr(grad_value, "grad_value", dtype))) return st;
    if (need) {
        if (!workspace) return fail(MSDA_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", need);
        if (workspace_bytes < need)
            return fail(MSDA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
        if (!aligned(workspace, 16)) return fail(MSDA_ERR_ALIGN, "workspace is not 16-byte aligned");
    }
    // Native half-precision atomics update aligned 4-byte pairs; every pair
    // must lie inside grad_value.
    if (!all_binned && mode != MSDA_ACCUM_FP32_SCRATCH && dtype != MSDA_F32 &&
        (!aligned(grad_value, 4) || (p.B * p.S * p.M * p.D) % 2 != 0))
        return fail(MSDA_ERR_ALIGN,
                    "native half-precision atomics need a 4-byte aligned grad_value with an even "
                    "element count; use MSDA_ACCUM_FP32_SCRATCH");
    msda::BwdMapping mp = {1, 1, 0, 0};
    msda::Mapping gmp = {1, 0, 0};  // gradients-only kernel (binned modes)
    if (p.Q > 0) {
        if ((st = check_ptr(sampling_locations, "sampling_locations", pdtype))) return st;
        if ((st = check_ptr(attention_weights, "attention_weights", pdtype))) return st;
        if ((st = check_ptr(grad_output, "grad_output", dtype))) return st;
        if ((st = check_ptr(grad_sampling_locations, "grad_sampling_locations", pdtype))) return st;
        if ((st = check_ptr(grad_attention_weights, "grad_attention_weights", pdtype))) return st;
        const bool pairs = aligned(value, 4) && aligned(grad_output, 4) && aligned(grad_value, 4);
        if ((st = choose_bwd_mapping(p, pairs, &mp))) return st;
        const void *vec_ptrs[2] = {value, grad_output};
        if (binned && (st = choose_mapping(p, vec_ptrs, 2, &gmp))) return st;
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t gv_bytes = (size_t)(p.B * p.S * p.M * p.D) * elem_size(dtype);
    hipError_t err;
    if (binned) {
        // Rows outside every binned level are written by no bin: zero all of
        // grad_value first when there are such rows (padding rows, levels
        // left to atomics, or no queries at all).
        const bool zero_gv = !accumulate && (p.Q == 0 || !all_binned || levels_leave_gaps(p));
        if (p.Q == 0) {
            if (zero_gv && (err = marked(msda::launch_zero(grad_value, gv_bytes, before(s)), s,
                                         "zero_fill")) != hipSuccess)
                return hip_fail(err, "grad_value zero fill");
            return ok();
        }
        char *ws = static_cast<char *>(workspace);
        msda::BinnedBuffers bins;
        bins.starts = reinterpret_cast<uint32_t *>(ws + bp.starts_off);
        bins.cursor = reinterpret_cast<uint32_t *>(ws + bp.cursor_off);
        bins.tile_offsets = reinterpret_cast<uint32_t *>(ws + bp.tiles_off);
        bins.records = reinterpret_cast<uint2 *>(ws + bp.records_off);
        bins.nbins = bp.nbins;
        // a bin's records end at its cursor after place (count's totals are
        // upper bounds where place merges records)
        bins.ends = bins.cursor;
        // The binned chain (t) overlaps the zero fill and the gradient /
        // scatter kernels (s); it forks after the caller's earlier work on s
        // and is joined back on every path below. The fork and join cost
        // about 20 us per call on MI355X (measured with graph replays), more
        // than the overlap gains below ~2^19 records (the decoder workload's
        // 3 * 10^5 lose 20 us; the odd-head workload's 9 * 10^5 gain 24 us).
        // (the one-launch local sort serves small problems and runs on s)
        SideStream *side = !bp.local_sort && bp.records >= ((int64_t)1 << 19) &&
                                   !(flags & MSDA_FLAG_SINGLE_STREAM)
                               ? side_stream(s)
                               : nullptr;
        // the local sort's launch also zero-fills grad_value when it can
        const bool fused_zero = bp.local_sort && zero_gv && aligned(grad_value, 16) &&
                                gv_bytes % 16 == 0;
        const hipStream_t t = side ? side->stream : s;
        if (side && ((err = hipEventRecord(side->fork, s)) != hipSuccess ||
                     (err = hipStreamWaitEvent(t, side->fork, 0)) != hipSuccess))
            return hip_fail(err, "side stream fork");
        // grad_loc / grad_attn come from msda_grad_kernel (forward lane
        // mapping) except for fp32 data with unbinned levels: fp32 rows span
        // several 64-byte atomic segments, and there the fused msda_bwd_kernel,
        // which overlaps those atomics with its gathers, measures faster.
        const bool grad_path = all_binned || dtype != MSDA_F32;
        // Small problems on one stream: the gradients, the local sort and the
        // zero fill share a launch, then the unbinned levels' scatter and the
        // accumulation share another (each pair touches disjoint data).
        const bool fuse_gs = bp.local_sort && !side && grad_path &&
                             msda::grad_sort_fits(p, gmp, bp.max_level_bins);
        const bool fuse_sa = !side && !all_binned && dtype != MSDA_F32 &&
                             msda::scatter_accumulate_fits(p, mp, grad_value);
        const char *what = nullptr;
        do {
            if (fuse_gs) {
                if ((err = marked(msda::launch_gradients_and_sort(
                                      p, gmp, value, sampling_locations, attention_weights,
                                      grad_output, grad_sampling_locations, grad_attention_weights,
                                      bins, bp.max_level_bins, fused_zero ? grad_value : nullptr,
                                      fused_zero ? gv_bytes : 0, before(s)),
                                  s, "grad_sort_kernel")) != hipSuccess) {
                    what = "gradient / sort launch";
                    break;
                }
            } else if (bp.local_sort) {
                if ((err = marked(msda::launch_bin_local_sort(
                                      p, sampling_locations, attention_weights, bins,
                                      bp.max_level_bins, fused_zero ? grad_value : nullptr,
                                      fused_zero ? gv_bytes : 0, before(t)),
                                  t, "bin_local_sort")) != hipSuccess) {
                    what = "bin local sort launch";
                    break;
                }
            } else if ((err = marked(msda::launch_zero(bins.starts, align_up((size_t)(bp.nbins + 1) * 4, 16),
                                                before(t)),
                              t, "bin_zero")) != hipSuccess) {
                // (the counts start at zero; the fill works in 2-byte units,
                // so the byte count is rounded up to an even number of them)
                what = "bin count zero fill";
                break;
            } else if ((err = marked(msda::launch_bin_sort(p, sampling_locations,
                                                           attention_weights, bins, false,
                                                           before(t)),
                                     t, "bin_count")) != hipSuccess) {
                what = "bin count launch";
                break;
            } else if (msda::scan_tiles(bp.nbins) <= kSingleScanTiles
                           ? (err = marked(msda::launch_bin_scan(bins, before(t)), t, "bin_scan")) !=
                                 hipSuccess
                           : ((err = marked(msda::launch_bin_tile_sums(bins, before(t)), t,
                                            "bin_tile_sum")) != hipSuccess ||
                              (err = marked(msda::launch_bin_tile_scan(bins, before(t)), t,
                                            "bin_tile_scan")) != hipSuccess)) {
                what = "bin scan launch";
                break;
            } else if ((err = marked(msda::launch_bin_sort(p, sampling_locations,
                                                           attention_weights, bins, true,
                                                           before(t)),
                                     t, "bin_place")) != hipSuccess) {
                what = "bin place launch";
                break;
            }
            if (zero_gv && !fused_zero &&
                (err = marked(msda::launch_zero(grad_value, gv_bytes, before(s)), s,
                              "zero_fill")) != hipSuccess) {
                what = "grad_value zero fill";
                break;
            }
            if (side && (err = hipEventRecord(side->zeroed, s)) != hipSuccess) {
                what = "side stream event";
                break;
            }
            // the unbinned levels' grad_value (if any) by a gather-free
            // atomic scatter
            if (grad_path) {
                if (!fuse_gs &&
                    (err = marked(msda::launch_gradients(p, gmp, value, sampling_locations,
                                                         attention_weights, grad_output,
                                                         grad_sampling_locations,
                                                         grad_attention_weights, before(s)),
                                  s, "msda_grad_kernel")) != hipSuccess) {
                    what = "gradient launch";
                    break;
                }
                if (fuse_sa) {
                    if ((err = marked(msda::launch_scatter_accumulate(
                                          p, mp, sampling_locations, attention_weights, grad_output,
                                          grad_value, bins, accumulate, before(s)),
                                      s, "scatter_accum_kernel")) != hipSuccess)
                        what = "scatter / accumulate launch";
                    break;  // done (the accumulation ran too)
                }
                if (!all_binned &&
                    (err = marked(msda::launch_scatter(p, mp, sampling_locations, attention_weights,
                                                       grad_output, grad_value, nullptr, before(s)),
                                  s, "msda_scatter_kernel")) != hipSuccess) {
                    what = "scatter launch";
                    break;
                }
            } else if ((err = marked(msda::launch_backward(p, mp, value, sampling_locations,
                                                           attention_weights, grad_output,
                                                           grad_value, nullptr,
                                                           grad_sampling_locations,
                                                           grad_attention_weights, before(s)),
                                     s, "msda_bwd_kernel")) != hipSuccess) {
                what = "backward launch";
                break;
            }
            // the accumulation writes whole rows: after the zero fill
            if (side && (err = hipStreamWaitEvent(t, side->zeroed, 0)) != hipSuccess) {
                what = "side stream wait";
                break;
            }
            if ((err = marked(msda::launch_bin_accumulate(p, mp, grad_output, grad_value, bins,
                                                          accumulate, before(t)),
                              t, "bin_accum_kernel")) != hipSuccess) {
                what = "bin accumulate launch";
                break;
            }
        } while (false);
        // pre-reduced levels: their fp32 rows (after the bins in the
        // workspace) summed in LDS windows, then rounded into grad_value
        // after the zero fill; disjoint from the binned rows
        if (err == hipSuccess && p.levels.prered) {
            char *scr0 = ws + align_up(bp.bytes, 256);
            const size_t scr_bytes = need - align_up(bp.bytes, 256);
            if ((err = marked(msda::launch_zero(scr0, scr_bytes, before(s)), s, "scratch_zero")) !=
                hipSuccess)
                what = "scratch zero fill";
            else if ((err = marked(msda::launch_prereduce(p, pt, sampling_locations,
                                                          attention_weights, grad_output,
                                                          reinterpret_cast<float *>(ws),
                                                          before(s)),
                                   s, "prereduce_kernel")) != hipSuccess)
                what = "pre-reduce launch";
            else if ((err = marked(msda::launch_scratch_add(p, reinterpret_cast<float *>(ws),
                                                            grad_value, before(s)),
                                   s, "scratch_add_kernel")) != hipSuccess)
                what = "scratch add launch";
        }
        if (side) {
            hipError_t je = hipEventRecord(side->join, t);
            if (je == hipSuccess) je = hipStreamWaitEvent(s, side->join, 0);
            if (err == hipSuccess && je != hipSuccess) {
                err = je;
                what = "side stream join";
            }
        }
        if (err != hipSuccess) return hip_fail(err, what);
        return ok();
    }
    if (!accumulate && (err = marked(msda::launch_zero(grad_value, gv_bytes, before(s)), s,
                                     "zero_fill")) != hipSuccess)
        return hip_fail(err, "grad_value zero fill");
    if (need && !keep_sums && (err = marked(msda::launch_zero(workspace, need, before(s)), s,
                                            "scratch_zero")) != hipSuccess)
        return hip_fail(err, "scratch zero fill");
    if (p.Q > 0 &&
        (err = marked(msda::launch_backward(p, mp, value, sampling_locations, attention_weights,
                                            grad_output, grad_value,
                                            static_cast<float *>(workspace),
                                            grad_sampling_locations, grad_attention_weights,
                                            before(s)),
                      s, "msda_bwd_kernel")) != hipSuccess)
        return hip_fail(err, "backward launch");
    if (p.Q > 0 && p.levels.prered &&
        (err = marked(msda::launch_prereduce(p, pt, sampling_locations, attention_weights,
                                             grad_output, static_cast<float *>(workspace),
                                             before(s)),
                      s, "prereduce_kernel")) != hipSuccess)
        return hip_fail(err, "pre-reduce launch");
    if (need && !defer &&
        (err = marked(msda::launch_scratch_add(p, static_cast<const float *>(workspace),
                                               grad_value, before(s)),
                      s, "scratch_add_kernel")) != hipSuccess)
        return hip_fail(err, "scratch add launch");
    return ok();
}

int msda_backward(int dtype, int64_t batch, int64_t num_keys, int64_t num_heads, int64_t head_dim,
                  int64_t num_levels, const int64_t *spatial_shapes,
                  const int64_t *level_start_index, int64_t num_queries, int64_t num_points,
                  const void *value, const void *sampling_locations, const void *attention_weights,
                  const void *grad_output, void *grad_value, void *grad_sampling_locations,
                  void *grad_attention_weights, int accum, unsigned flags, void *workspace,
                  size_t workspace_bytes, void *stream) {
    return backward_impl(dtype, dtype, batch, num_keys, num_heads, head_dim, num_levels,
                         spatial_shapes, level_start_index, num_queries, num_points, value,
                         sampling_locations, attention_weights, grad_output, grad_value,
                         grad_sampling_locations, grad_attention_weights, accum, flags, workspace,
                         workspace_bytes, stream);
}

}  // extern "C"

// ------------------------------------------------ allocation-free backward
//
// msda_backward_noalloc runs msda_backward with a workspace taken from this
// file-scope device array instead of the caller's memory, for callers that
// cannot allocate. Each GPU the library runs on holds its own copy until the
// process ends; in host code the array's name only stands for it, so its
// device address is looked up once per device (with that device current) and
// only that address is handed to kernels. Every call on one GPU shares the
// array: the backward clears what must start at zero (bin counters, fp32
// sums) itself, and calls that overlap on one GPU race.
namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on device `dev` (looked up on first use).
int scratch_address(int dev, void **out) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        hipError_t err = hipGetDevice(&cur);
        if (err == hipSuccess && cur != dev) err = hipSetDevice(dev);
        void *ptr = nullptr;
        if (err == hipSuccess) err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur >= 0 && cur != dev) (void)hipSetDevice(cur);
        if (err != hipSuccess) return hip_fail(err, "looking up the static scratch address");
        if (!ptr) return fail(MSDA_ERR_HIP, "the static scratch has no device address");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MSDA_OK;
}

}  // namespace

extern "C" {

int msda_backward_noalloc(int dtype, int64_t batch, int64_t num_keys, int64_t num_heads,
                          int64_t head_dim, int64_t num_levels, const int64_t *spatial_shapes,
                          const int64_t *level_start_index, int64_t num_queries,
                          int64_t num_points, const void *value, const void *sampling_locations,
                          const void *attention_weights, const void *grad_output,
                          void *grad_value, void *grad_sampling_locations,
                          void *grad_attention_weights, int accum, unsigned flags,
                          void *stream) {
    if (flags & (MSDA_FLAG_CONTINUE_SCRATCH | MSDA_FLAG_DEFER_SCRATCH))
        return fail(MSDA_ERR_SHAPE,
                    "msda_backward_noalloc takes no CONTINUE_SCRATCH / DEFER_SCRATCH: its "
                    "scratch is shared by every call on the GPU");
    // Size the workspace first (host only), so an oversized problem is
    // rejected before any HIP call.
    const size_t need = msda_backward_workspace_size(dtype, batch, num_keys, num_heads, head_dim,
                                                     num_levels, spatial_shapes,
                                                     level_start_index, num_queries, num_points,
                                                     accum);
    // (need == 0 for invalid arguments too: msda_backward's own validation
    // below then returns their status)
    if (need > kNoAllocScratchBytes)
        return fail(MSDA_ERR_WORKSPACE,
                    "this backward needs %zu bytes of workspace, above the %zu bytes of "
                    "msda_backward_noalloc's static scratch; call msda_backward with a "
                    "workspace instead",
                    need, kNoAllocScratchBytes);
    void *ws = nullptr;
    if (need && batch > 0) {
        const hipStream_t s = static_cast<hipStream_t>(stream);
        int dev = -1;
        const hipError_t err = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
        if (err != hipSuccess) return hip_fail(err, "finding the stream's device");
        if (dev < 0 || dev >= kMaxDevices)
            return fail(MSDA_ERR_UNSUPPORTED, "device %d outside [0, %d)", dev, kMaxDevices);
        const int st = scratch_address(dev, &ws);
        if (st) return st;
    }
    return backward_impl(dtype, dtype, batch, num_keys, num_heads, head_dim, num_levels,
                         spatial_shapes, level_start_index, num_queries, num_points, value,
                         sampling_locations, attention_weights, grad_output, grad_value,
                         grad_sampling_locations, grad_attention_weights, accum,
                         flags | MSDA_FLAG_SINGLE_STREAM, ws, ws ? kNoAllocScratchBytes : 0,
                         stream);
}

int msda_backward_ex(int value_dtype, int param_dtype, int64_t batch, int64_t num_keys,
                     int64_t num_heads, int64_t head_dim, int64_t num_levels,
                     const int64_t *spatial_shapes, const int64_t *level_start_index,
                     int64_t num_queries, int64_t num_points, const void *value,
                     const void *sampling_locations, const void *attention_weights,
                     const void *grad_output, void *grad_value, void *grad_sampling_locations,
                     void *grad_attention_weights, int accum, unsigned flags, void *workspace,
                     size_t workspace_bytes, void *stream) {
    return backward_impl(value_dtype, param_dtype, batch, num_keys, num_heads, head_dim,
                         num_levels, spatial_shapes, level_start_index, num_queries, num_points,
                         value, sampling_locations, attention_weights, grad_output, grad_value,
                         grad_sampling_locations, grad_attention_weights, accum, flags, workspace,
                         workspace_bytes, stream);
}

// ------------------------------------------------ sampling-parameter prep

static int make_prep(int dtype, int64_t B, int64_t Q, int64_t M, int64_t L, int64_t K,
                     const int64_t *shapes, int ref_per_level, msda::PrepProblem *p) {
    if (dtype != MSDA_F32 && dtype != MSDA_F16 && dtype != MSDA_BF16)
        return fail(MSDA_ERR_DTYPE, "unknown dtype %d (0=f32, 1=f16, 2=bf16)", dtype);
    if (B < 0 || Q < 0) return fail(MSDA_ERR_SHAPE, "batch (%lld) and num_queries (%lld) must be >= 0",
                                    (long long)B, (long long)Q);
    if (M < 1 || K < 1 || L < 1)
        return fail(MSDA_ERR_SHAPE, "num_heads (%lld), num_levels (%lld), num_points (%lld) must be >= 1",
                    (long long)M, (long long)L, (long long)K);
    if (L > MSDA_MAX_LEVELS)
        return fail(MSDA_ERR_UNSUPPORTED, "num_levels %lld exceeds the limit of %d", (long long)L,
                    MSDA_MAX_LEVELS);
    if (K >= ((int64_t)1 << 26)) return fail(MSDA_ERR_UNSUPPORTED, "num_points %lld too large", (long long)K);
    if (ref_per_level != 0 && ref_per_level != 1)
        return fail(MSDA_ERR_SHAPE, "ref_per_level must be 0 or 1, got %d", ref_per_level);
    if (!shapes) return fail(MSDA_ERR_NULL_ARG, "spatial_shapes is NULL");
    int64_t rows = 0, pts = 0;
    // 2 * rows * L * K elements must fit int64 indexing, and rows * 64 lanes
    // one launch (at most 2^31 - 1 workgroups of 256 threads)
    if (!mul_ok(B, Q, &rows) || !mul_ok(rows, M, &rows) || !mul_ok(rows, L * K * 2, &pts))
        return fail(MSDA_ERR_SHAPE, "sampling tensor B*Q*M*L*K overflows");
    if (rows >= ((int64_t)1 << 33))
        return fail(MSDA_ERR_UNSUPPORTED, "B*Q*M = %lld rows exceed one launch", (long long)rows);
    p->dtype = dtype;
    p->B = B;
    p->Q = Q;
    p->M = M;
    p->L = L;
    p->K = K;
    p->ref_levels = ref_per_level ? (int)L : 1;
    for (int l = 0; l < MSDA_MAX_LEVELS; ++l) p->H[l] = p->W[l] = 1.0f;
    for (int64_t l = 0; l < L; ++l) {
        const int64_t H = shapes[2 * l], W = shapes[2 * l + 1];
        if (H < 1 || W < 1)
            return fail(MSDA_ERR_LEVELS, "level %lld has shape (%lld, %lld); both must be >= 1",
                        (long long)l, (long long)H, (long long)W);
        if (H >= ((int64_t)1 << 24) || W >= ((int64_t)1 << 24))
            return fail(MSDA_ERR_UNSUPPORTED, "level %lld shape (%lld, %lld) exceeds 2^24",
                        (long long)l, (long long)H, (long long)W);
        p->H[l] = (float)H;
        p->W[l] = (float)W;
    }
    return ok();
}

int msda_sampling_prep(int dtype, int64_t batch, int64_t num_queries, int64_t num_heads,
                       int64_t num_levels, int64_t num_points, const int64_t *spatial_shapes,
                       int ref_per_level, const void *reference_points,
                       const void *sampling_offsets, const void *attention_logits,
                       void *sampling_locations, void *attention_weights, void *stream) {
    LaunchEventsScope events_scope;
    msda::PrepProblem p;
    int st = make_prep(dtype, batch, num_queries, num_heads, num_levels, num_points, spatial_shapes,
                       ref_per_level, &p);
    if (st) return st;
    if (p.B == 0 || p.Q == 0) return ok();
    if ((st = check_ptr(reference_points, "reference_points", dtype))) return st;
    if ((st = check_ptr(sampling_offsets, "sampling_offsets", dtype))) return st;
    if ((st = check_ptr(attention_logits, "attention_logits", dtype))) return st;
    if ((st = check_ptr(sampling_locations, "sampling_locations", dtype))) return st;
    if ((st = check_ptr(attention_weights, "attention_weights", dtype))) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t err = marked(msda::launch_sampling_prep(p, reference_points, sampling_offsets,
                                                             attention_logits, sampling_locations,
                                                             attention_weights, before(s)),
                                  s, "sampling_prep_kernel");
    if (err != hipSuccess) return hip_fail(err, "sampling prep launch");
    return ok();
}

int msda_sampling_prep_backward(int dtype, int64_t batch, int64_t num_queries, int64_t num_heads,
                                int64_t num_levels, int64_t num_points,
                                const int64_t *spatial_shapes, int ref_per_level,
                                const void *attention_weights, const void *grad_sampling_locations,
                                const void *grad_attention_weights, void *grad_reference_points,
                                void *grad_sampling_offsets, void *grad_attention_logits,
                                void *stream) {
    LaunchEventsScope events_scope;
    msda::PrepProblem p;
    int st = make_prep(dtype, batch, num_queries, num_heads, num_levels, num_points, spatial_shapes,
                       ref_per_level, &p);
    if (st) return st;
    if (p.B == 0 || p.Q == 0) return ok();
    if ((st = check_ptr(attention_weights, "attention_weights", dtype))) return st;
    if ((st = check_ptr(grad_sampling_locations, "grad_sampling_locations", dtype))) return st;
    if ((st = check_ptr(grad_attention_weights, "grad_attention_weights", dtype))) return st;
    if ((st = check_ptr(grad_sampling_offsets, "grad_sampling_offsets", dtype))) return st;
    if ((st = check_ptr(grad_attention_logits, "grad_attention_logits", dtype))) return st;
    if (grad_reference_points &&
        (st = check_ptr(grad_reference_points, "grad_reference_points", dtype)))
        return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err = marked(msda::launch_sampling_prep_backward(
                                p, attention_weights, grad_sampling_locations,
                                grad_attention_weights, grad_sampling_offsets,
                                grad_attention_logits, before(s)),
                            s, "sampling_prep_bwd_kernel");
    if (err == hipSuccess && grad_reference_points)
        err = marked(msda::launch_reference_grad(p, grad_sampling_locations, grad_reference_points,
                                                 before(s)),
                     s, "reference_grad_kernel");
    if (err != hipSuccess) return hip_fail(err, "sampling prep backward launch");
    return ok();
}

}  // extern "C"
