/*
 * msda.h - C ABI of the multi-scale deformable attention (MSDA) sampling and
 * aggregation core for AMD Instinct MI355X (gfx950).
 *
 * The operation is the bracketed core of the MSDA operator (msda-triton
 * README, section "The operator"): for every batch b, query q and head m,
 *
 *   out[b,q,m,:] = sum_l sum_k A[b,q,m,l,k] * bilinear_l(value[b,:,m,:], loc[b,q,m,l,k])
 *
 * where bilinear_l samples level l of the multi-level value map at the pixel
 * x = loc_x * W_l - 0.5, y = loc_y * H_l - 0.5 with zero padding outside the
 * level (README, section "Kernel design"; course page "4. The forward kernel,
 * line by line", sections "Bilinear sampling" and "Accumulate and store").
 * The x mapping is computed as one fused multiply-add rounded once to fp32,
 * then floor; every in/out-of-bounds decision is taken per dimension on the
 * integer cell coordinates, so a column past an edge never aliases a
 * neighbouring row or level.
 *
 * The backward gives the three gradients of course page "5. The backward
 * kernel: gradients, atomics, and a precision switch", section "What the
 * backward pass must produce": grad_attention_weights (g . sample),
 * grad_sampling_locations (corner slopes x A x W_l, and x H_l for y) and
 * grad_value (A * w_ij * g scattered onto every in-bounds corner with relaxed
 * atomics; out-of-bounds corners receive nothing, section "Scatter needs
 * atomics").
 *
 * Tensor layouts (all dense, row-major, on the device; one dtype for every
 * floating tensor of a call, except in the _ex entry points, where the
 * locations, weights and their gradients may be fp32 beside 16-bit values):
 *   value                    (B, S, M, D)       S = rows of all levels
 *   sampling_locations       (B, Q, M, L, K, 2) normalised (x, y), not clamped
 *   attention_weights        (B, Q, M, L, K)    used as given (no softmax)
 *   output / grad_output     (B, Q, M, D)       == (B, Q, M*D)
 *   grad_value               (B, S, M, D)
 *   grad_sampling_locations  (B, Q, M, L, K, 2)
 *   grad_attention_weights   (B, Q, M, L, K)
 * Level tables are HOST arrays:
 *   spatial_shapes     L x 2 int64, rows (H_l, W_l), each >= 1
 *   level_start_index  L int64, or NULL for the exclusive prefix sum of
 *                      H_l * W_l (README, section "Quickstart"); a given index
 *                      is used as given and only checked for memory safety:
 *                      0 <= start_l and start_l + H_l * W_l <= S.
 *
 * Ownership and threading: the caller owns every buffer. The library
 * allocates no device memory and never synchronises. Its only state is
 * thread-local: an error string and, for backward calls that bin some level,
 * one side stream (default priority) and three events per device, created by
 * the first such call of a thread that is not under graph capture and kept
 * until msda_release_thread_resources() (or the thread's end); a call with
 * MSDA_FLAG_SINGLE_STREAM neither uses nor creates them. Work is enqueued on
 * the caller's stream (a hipStream_t passed as void*; NULL is the default
 * stream); the binned part of a backward forks onto the side stream after the
 * caller's earlier work and is joined back before the call returns, so each
 * call is ordered on the caller's stream as a whole and can be captured in a
 * HIP graph (a call captured before its thread has a side stream runs
 * entirely on the caller's stream). Calls are reentrant. Device pointers must
 * be aligned to their element size; wider vector accesses are used
 * automatically when every pointer allows them.
 *
 * Errors: every entry point returns an msda_status_t. All argument checks run
 * before any HIP call, so a rejected call has no side effect and needs no GPU.
 * A failed kernel launch returns MSDA_ERR_HIP; faults during execution
 * surface at the caller's next synchronisation. msda_last_error() gives a
 * thread-local message for the last non-OK status.
 */
#ifndef MSDA_H
#define MSDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSDA_ABI_VERSION 1
#define MSDA_MAX_LEVELS 16

typedef enum msda_dtype {
    MSDA_F32 = 0,
    MSDA_F16 = 1,
    MSDA_BF16 = 2
} msda_dtype_t;

/* How the backward accumulates grad_value (course page "5. The backward
 * kernel", sections "Scatter needs atomics" and "The fix: accumulate in FP32,
 * downcast at the end").
 *   NATIVE        atomics of the value dtype straight into grad_value
 *                 (fp32 atomics, or packed two-wide fp16 / bf16 atomics);
 *   FP32_SCRATCH  fp32 atomics into the caller's workspace, then one pass
 *                 adding it into grad_value (identical to NATIVE for fp32);
 *   PER_LEVEL     16-bit data: fp32 scratch for the levels whose pixels
 *                 receive more than 4 contributions on average
 *                 (Q*K*4 / (H_l*W_l) > 4), packed atomics for the others;
 *   BINNED        no float atomics: every in-bounds corner becomes an 8-byte
 *                 record in the bin of its destination rows (count, scan,
 *                 place), and one workgroup per bin sums its records in fp32
 *                 and writes the bin's grad_value rows once, rounded once.
 *                 Needs non-overlapping levels and batch slices of value and
 *                 grad_output below 2 GiB; the workspace holds 8 bytes per
 *                 corner of every binned level's points;
 *   MIXED         BINNED for the levels above 4 contributions per pixel,
 *                 native atomics for the others (same conditions as BINNED);
 *   PREREDUCE     the levels above 256 contributions per pixel are summed
 *                 in LDS first (msda-triton README, section "Benchmarks": a
 *                 shared-memory pre-reduction): one workgroup per head and
 *                 block of queries (a 2-D tile of pixels and the matching
 *                 pixels of the other levels when the queries are the
 *                 pyramid's pixels in S order, else consecutive queries)
 *                 counting-sorts its corners on such a level by pixel of a
 *                 window placed at the mean of its samples there, sums each
 *                 pixel's records in fp32 and adds the sums into the level's
 *                 fp32 workspace rows (corners outside the window add there
 *                 directly); the workspace is rounded once into grad_value.
 *                 The levels above 4 are BINNED, the others native (same
 *                 conditions as BINNED, and D up to 256). Measured slower
 *                 than MIXED on the encoder shapes; AUTO does not pick it;
 *   AUTO          MIXED where binning applies (which is BINNED when every
 *                 level is above the threshold, NATIVE when none is), else
 *                 PER_LEVEL for bf16 and NATIVE for fp16 / fp32.
 * A scratch level is laid out (B, H_l*W_l, M, D) in fp32. grad_value is the
 * fp32 sum rounded once to the value dtype except for levels accumulated with
 * packed 16-bit atomics, which round every add. */
typedef enum msda_accum {
    MSDA_ACCUM_AUTO = -1,
    MSDA_ACCUM_NATIVE = 0,
    MSDA_ACCUM_FP32_SCRATCH = 1,
    MSDA_ACCUM_PER_LEVEL = 2,
    MSDA_ACCUM_BINNED = 3,
    MSDA_ACCUM_MIXED = 4,
    MSDA_ACCUM_PREREDUCE = 5
} msda_accum_t;

/* How msda_backward accumulates one level's grad_value rows. */
typedef enum msda_level_mode {
    MSDA_LEVEL_NATIVE = 0,        /* atomics of the value dtype       */
    MSDA_LEVEL_FP32_SCRATCH = 1,  /* fp32 atomics into the workspace  */
    MSDA_LEVEL_BINNED = 2,        /* records, summed per bin          */
    MSDA_LEVEL_PREREDUCE = 3      /* LDS sums, then fp32 scratch      */
} msda_level_mode_t;

typedef enum msda_status {
    MSDA_OK = 0,
    MSDA_ERR_NULL_ARG = 1,    /* a required pointer is NULL              */
    MSDA_ERR_SHAPE = 2,       /* a size is negative, zero or too large   */
    MSDA_ERR_LEVELS = 3,      /* bad spatial_shapes / level_start_index  */
    MSDA_ERR_DTYPE = 4,       /* unknown dtype or accumulation mode      */
    MSDA_ERR_ALIGN = 5,       /* pointer not aligned to its element size */
    MSDA_ERR_WORKSPACE = 6,   /* workspace missing or too small          */
    MSDA_ERR_HIP = 7,         /* a HIP launch failed                     */
    MSDA_ERR_UNSUPPORTED = 8  /* valid but outside the library's limits  */
} msda_status_t;

/* Add into grad_value instead of overwriting it (training-style gradient
 * accumulation); without it the library zero-fills grad_value first. */
#define MSDA_FLAG_ACCUMULATE_GRAD_VALUE 1u
/* The workspace already holds this problem's fp32 partial sums from an earlier
 * call made with MSDA_FLAG_DEFER_SCRATCH: keep adding to them instead of
 * zero-filling the workspace first. CONTINUE_SCRATCH and DEFER_SCRATCH need
 * an explicit FP32_SCRATCH or PER_LEVEL mode. */
#define MSDA_FLAG_CONTINUE_SCRATCH 2u
/* Leave the fp32 sums of the scratch levels in the workspace instead of
 * adding them into grad_value at the end. With CONTINUE_SCRATCH this lets
 * several backward calls (micro-batches) accumulate in fp32 and round into
 * grad_value once, by a last call without DEFER_SCRATCH. */
#define MSDA_FLAG_DEFER_SCRATCH 4u
/* Run the whole backward on the caller's stream: no side stream is used or
 * created (by default a backward binning at least 2^19 records runs its
 * binned chain on this thread's side stream, see "Ownership and threading"). */
#define MSDA_FLAG_SINGLE_STREAM 8u

/*
 * Forward. Writes every element of `output` (B, Q, M, D).
 * B == 0 or Q == 0: returns MSDA_OK without touching the device.
 * Limits (MSDA_ERR_UNSUPPORTED): L <= MSDA_MAX_LEVELS, H_l and W_l < 2^24,
 * D <= 64 * v where v is the widest channel vector that divides D.
 */
int msda_forward(int dtype, int64_t batch, int64_t num_keys, int64_t num_heads,
                 int64_t head_dim, int64_t num_levels,
                 const int64_t *spatial_shapes, const int64_t *level_start_index,
                 int64_t num_queries, int64_t num_points,
                 const void *value, const void *sampling_locations,
                 const void *attention_weights, void *output, void *stream);

/*
 * Mixed dtypes: msda_forward with a separate dtype for sampling_locations and
 * attention_weights (param_dtype). param_dtype is value_dtype, or MSDA_F32
 * beside fp16 / bf16 values (fp32 locations keep sub-pixel precision at large
 * resolutions, msda-triton README, section "Caveats"); value and output take
 * value_dtype. MSDA_ERR_DTYPE for any other pair; MSDA_ERR_UNSUPPORTED for a
 * mixed pair whose per-batch value slice is 2 GiB or more.
 */
int msda_forward_ex(int value_dtype, int param_dtype, int64_t batch, int64_t num_keys,
                    int64_t num_heads, int64_t head_dim, int64_t num_levels,
                    const int64_t *spatial_shapes, const int64_t *level_start_index,
                    int64_t num_queries, int64_t num_points, const void *value,
                    const void *sampling_locations, const void *attention_weights, void *output,
                    void *stream);

/*
 * Measurement foil, not a forward to use: the point-parallel decomposition
 * that the forward page contrasts with its own (course page "4. The forward
 * kernel, line by line", section "The design question: what does one
 * program own?"), one thread per sampling point reading its corner rows
 * alone, partial outputs added per query through LDS. Same arguments and
 * result as msda_forward (summation order aside). MSDA_ERR_UNSUPPORTED unless
 * num_levels * num_points divides 256 and head_dim <= 64.
 */
int msda_forward_point_parallel(int dtype, int64_t batch, int64_t num_keys, int64_t num_heads,
                                int64_t head_dim, int64_t num_levels,
                                const int64_t *spatial_shapes, const int64_t *level_start_index,
                                int64_t num_queries, int64_t num_points,
                                const void *value, const void *sampling_locations,
                                const void *attention_weights, void *output, void *stream);

/*
 * Measurement kernel, not part of the MSDA computation: the request rate of
 * device-scope no-return atomic adds, which bounds the backward's grad_value
 * scatter on atomically accumulated levels (course page "5. The backward
 * kernel", section "Scatter needs atomics"). Launches `workgroups` x 256
 * threads; every thread makes `iters` adds of 1 (fp32, or packed bf16 pairs
 * when bf16 != 0) into `buffer` (device, 64-byte aligned; the largest power
 * of two of whole 64-byte segments in buffer_bytes is used, up to 2^30;
 * contents overwritten), in runs of dwords_per_request
 * (1, 2, 4, 8 or 16) consecutive lanes that each address one 64-byte
 * segment, lane i of a run its dword i, and no two runs in flight the same
 * segment. *requests receives the number of atomic requests the launch makes
 * (threads / dwords_per_request * iters); time the launch with
 * msda_set_launch_events. workgroups in [1, 2^24], iters >= 1.
 */
int msda_probe_atomic_requests(void *buffer, size_t buffer_bytes, int bf16,
                               int dwords_per_request, int64_t workgroups, int iters,
                               int64_t *requests, void *stream);

/*
 * Bytes of device workspace msda_backward needs for `accum` on this problem
 * (0 for NATIVE, and for fp32 data). Returns 0 and sets the last error for
 * invalid arguments; host-only, needs no GPU.
 */
size_t msda_backward_workspace_size(int dtype, int64_t batch, int64_t num_keys,
                                    int64_t num_heads, int64_t head_dim,
                                    int64_t num_levels, const int64_t *spatial_shapes,
                                    const int64_t *level_start_index,
                                    int64_t num_queries, int64_t num_points,
                                    int accum);

/*
 * The accumulation msda_backward will use for `accum` on this problem:
 * BINNED (every level binned), MIXED (some levels), NATIVE (no level uses
 * scratch or bins; always the case for fp32 data without bins), FP32_SCRATCH
 * (every level uses scratch), PER_LEVEL (some levels do), or -1 on invalid
 * arguments (and for BINNED / MIXED where binning cannot apply).
 */
int msda_backward_resolve_accum(int dtype, int64_t batch, int64_t num_keys,
                                int64_t num_heads, int64_t head_dim,
                                int64_t num_levels, const int64_t *spatial_shapes,
                                const int64_t *level_start_index,
                                int64_t num_queries, int64_t num_points, int accum);

/*
 * The per-level plan behind msda_backward_resolve_accum: writes
 * msda_level_mode_t values to level_modes[0:L] (a host array, or NULL) and
 * returns the number of grad_value bins (0 when no level is binned), or -1 on
 * invalid arguments. Host-only, needs no GPU.
 */
int64_t msda_backward_plan(int dtype, int64_t batch, int64_t num_keys, int64_t num_heads,
                           int64_t head_dim, int64_t num_levels, const int64_t *spatial_shapes,
                           const int64_t *level_start_index, int64_t num_queries,
                           int64_t num_points, int accum, int *level_modes);

/*
 * Backward, given grad_output (B, Q, M, D). Writes every element of
 * grad_sampling_locations and grad_attention_weights; grad_value is
 * zero-filled and then accumulated into (or only accumulated into, with
 * MSDA_FLAG_ACCUMULATE_GRAD_VALUE). `workspace` must hold at least
 * msda_backward_workspace_size(...) bytes, 16-byte aligned (NULL if 0).
 * grad_value is bitwise nondeterministic run to run (the order of atomics,
 * or of records within a bin); the two other gradients are deterministic.
 * B == 0: returns MSDA_OK. Q == 0: only the grad_value zero-fill runs.
 */
int msda_backward(int dtype, int64_t batch, int64_t num_keys, int64_t num_heads,
                  int64_t head_dim, int64_t num_levels,
                  const int64_t *spatial_shapes, const int64_t *level_start_index,
                  int64_t num_queries, int64_t num_points,
                  const void *value, const void *sampling_locations,
                  const void *attention_weights, const void *grad_output,
                  void *grad_value, void *grad_sampling_locations,
                  void *grad_attention_weights, int accum, unsigned flags,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * msda_backward for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments and results without the workspace, which comes from a static
 * scratch array of 32 MiB inside the library instead (device memory each
 * GPU the library runs on holds until the process ends). No device memory is
 * allocated or freed, and the whole backward runs on the caller's stream (as
 * with MSDA_FLAG_SINGLE_STREAM). Every call on one GPU shares that GPU's
 * scratch: each call clears what must start at zero itself, and calls that
 * overlap in time on one GPU race (order them on one stream, or use
 * msda_backward with separate workspaces). MSDA_ERR_WORKSPACE when the
 * problem needs more than 32 MiB of workspace for `accum`
 * (msda_backward_workspace_size), before any HIP call; MSDA_ERR_SHAPE for the
 * CONTINUE_SCRATCH / DEFER_SCRATCH flags, which would rely on the shared
 * scratch's earlier contents.
 */
int msda_backward_noalloc(int dtype, int64_t batch, int64_t num_keys, int64_t num_heads,
                          int64_t head_dim, int64_t num_levels, const int64_t *spatial_shapes,
                          const int64_t *level_start_index, int64_t num_queries,
                          int64_t num_points, const void *value, const void *sampling_locations,
                          const void *attention_weights, const void *grad_output,
                          void *grad_value, void *grad_sampling_locations,
                          void *grad_attention_weights, int accum, unsigned flags,
                          void *stream);

/*
 * Mixed dtypes for the backward, as msda_forward_ex: sampling_locations,
 * attention_weights, grad_sampling_locations and grad_attention_weights take
 * param_dtype; value, grad_output and grad_value take value_dtype. Workspace
 * sizes and accumulation plans depend on value_dtype only
 * (msda_backward_workspace_size and friends take it as their dtype).
 */
int msda_backward_ex(int value_dtype, int param_dtype, int64_t batch, int64_t num_keys,
                     int64_t num_heads, int64_t head_dim, int64_t num_levels,
                     const int64_t *spatial_shapes, const int64_t *level_start_index,
                     int64_t num_queries, int64_t num_points, const void *value,
                     const void *sampling_locations, const void *attention_weights,
                     const void *grad_output, void *grad_value, void *grad_sampling_locations,
                     void *grad_attention_weights, int accum, unsigned flags, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * Sampling-parameter preparation: the steps between a deformable-attention
 * module's linear layers and the core (msda-triton README, section "The
 * operator": sampling points are the query's reference point mapped to each
 * level plus learned offsets, weights are softmax-normalised; section
 * "Quickstart": the softmax runs over the flattened L*K points of each
 * (b, q, m)). With normalised (x, y) reference points and offsets in pixels of
 * each level:
 *   sampling_locations[b,q,m,l,k,:] = ref + (off_x / W_l, off_y / H_l)
 *   attention_weights[b,q,m,:]      = softmax(attention_logits[b,q,m,:])
 * Layouts (dense, row-major, device, all in `dtype`):
 *   reference_points  (B, Q, 2), or (B, Q, L, 2) with ref_per_level = 1
 *   sampling_offsets  (B, Q, M, L, K, 2)    pixels of level l
 *   attention_logits  (B, Q, M, L*K)
 *   outputs as msda_forward's sampling_locations / attention_weights.
 * Computed in fp32, rounded once at the store. spatial_shapes is the host
 * (L, 2) table of msda_forward; only the shapes matter here. B == 0 or Q == 0:
 * MSDA_OK, nothing launched. Rows whose logits are all -inf give NaN weights,
 * as a softmax does.
 */
int msda_sampling_prep(int dtype, int64_t batch, int64_t num_queries, int64_t num_heads,
                       int64_t num_levels, int64_t num_points, const int64_t *spatial_shapes,
                       int ref_per_level, const void *reference_points,
                       const void *sampling_offsets, const void *attention_logits,
                       void *sampling_locations, void *attention_weights, void *stream);

/*
 * Backward of msda_sampling_prep, given the core's gradients with respect to
 * its locations and weights and the weights msda_sampling_prep produced:
 *   grad_sampling_offsets = grad_sampling_locations / (W_l, H_l)
 *   grad_attention_logits[j] = A_j * (g_j - sum_i A_i g_i) over the L*K points
 *   grad_reference_points = sum over heads and points (and levels, unless
 *                           ref_per_level) of grad_sampling_locations
 * grad_reference_points may be NULL (not computed). Every element of the
 * non-NULL outputs is written; deterministic (fixed summation order).
 */
int msda_sampling_prep_backward(int dtype, int64_t batch, int64_t num_queries, int64_t num_heads,
                                int64_t num_levels, int64_t num_points,
                                const int64_t *spatial_shapes, int ref_per_level,
                                const void *attention_weights, const void *grad_sampling_locations,
                                const void *grad_attention_weights, void *grad_reference_points,
                                void *grad_sampling_offsets, void *grad_attention_logits,
                                void *stream);

/*
 * Instrumentation for profilers and benchmarks: the next msda_forward or
 * msda_backward call made by this thread records events[2i] (hipEvent_t
 * passed as void*) when its i-th kernel starts on the device and events[2i+1]
 * when it ends (hipExtLaunchKernel's launch-packet timestamps), while
 * 2i+1 < count (count <= 64); the setting then clears itself. Kernel i's
 * device time is the time between the two events (a launch step that ran no
 * kernel records both back to back). The events are the caller's.
 */
int msda_set_launch_events(void *const *events, int count);

/* How many events the last instrumented call of this thread recorded
 * (twice the number of kernels it launched, up to its count). */
int msda_launch_events_recorded(void);

/* Kernel name of the i-th instrumented launch of that call (the one between
 * events 2i and 2i+1), e.g. "msda_fwd_kernel" or "bin_accum_kernel"; NULL when
 * i is out of range. Static storage. */
const char *msda_launch_events_name(int i);

/* Static text for a status code. */
const char *msda_status_string(int status);

/* Thread-local detail for the last non-OK status of this thread ("" if none). */
const char *msda_last_error(void);

/*
 * Destroys this thread's side streams and their events on every device (the
 * only resources the library keeps, see "Ownership and threading"). Work
 * already queued on them still completes, and HIP graphs captured earlier keep
 * working (they hold nodes, not the streams). A later binned backward on this
 * thread creates them again. Returns MSDA_OK when there is nothing to release
 * (no HIP call is made then), MSDA_ERR_HIP if a destroy fails.
 */
int msda_release_thread_resources(void);

/*
 * Testing hook, for tests only: with enable != 0, every later call addresses
 * the value slice with plain loads from clamped addresses, the path the
 * library otherwise takes only for batch slices of 2 GiB or more, and plans
 * as it does for such slices (no binned or pre-reduced accumulation, no
 * mixed dtypes). Results are the same up to fp32 summation order. The
 * setting is process-wide and not synchronised with calls in flight on other
 * threads. Returns the previous setting (0 or 1); host-only, no HIP call.
 */
int msda_debug_force_flat_gathers(int enable);

/* MSDA_ABI_VERSION of the built library. */
int msda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSDA_H */
