/*
 * CPU oracle for the multi-scale deformable attention (MSDA) sampling and
 * aggregation core, forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code,
 * header, table or helper with the HIP library; nothing in the product path
 * may call it.
 *
 * It is deliberately plain and slow: nested loops in the order of the
 * definition, fp64 arithmetic, no blocking, no fusion. Where a step is fixed
 * in fp32 by the pages (the pixel mapping, see below) the oracle takes that
 * step in fp32 too, so that both sides take every integer decision (which
 * corner, in or out of bounds) on the same fp32 number.
 *
 * Sources (web pages):
 *  [FWD] "4. The forward kernel, line by line" (msda-triton course):
 *        section "Bilinear sampling: the same math as the naive loop" for the
 *        pixel mapping, the cell and the fractions; section "The corner
 *        gathers" for row addressing and per-dimension zero padding; section
 *        "Accumulate and store" for the four corner weights and the
 *        attention-weighted sum.
 *  [BWD] "5. The backward kernel: gradients, atomics, and a precision switch"
 *        (msda-triton course): section "What the backward pass must produce"
 *        for the three gradients; section "Scatter needs atomics" for the
 *        rule that an out-of-bounds corner receives no gradient.
 *  [README] msda-triton README: section "The operator" for the bracketed core
 *        that is computed here; section "Kernel design" for the convention
 *        x_im = x * W_l - 0.5 with zero padding (grid_sample with
 *        align_corners=False); section "Quickstart" for level_start_index
 *        being optional.
 *
 * Readings taken where the pages are silent or garbled (the display equations
 * of the backward page were lost):
 *  - corner v_ij: i is the y offset (row y0 + i), j the x offset (x0 + j);
 *  - sample s = sum_ij w_ij v_ij with w00=(1-lx)(1-ly), w01=lx(1-ly),
 *    w10=(1-lx)ly, w11=lx*ly;
 *  - d s / d x_im = (1-ly)(v01-v00) + ly(v11-v10), d s / d y_im =
 *    (1-lx)(v10-v00) + lx(v11-v01), with out-of-bounds corners taken as 0;
 *    chain rule through x_im = loc_x*W - 0.5 gives the factor W (H for y);
 *    at an integer coordinate this is the right-sided derivative;
 *  - PINNED_F32 mode computes x_im = fmaf(loc_x, W, -0.5f) with one rounding,
 *    floor and fraction in fp32 (exact), then everything else in fp64;
 *  - EXACT_F64 mode does the mapping in fp64 (for finite-difference and
 *    library cross-checks that need sub-fp32 perturbations);
 *  - level_start_index, when given, is used as given; NULL means the exclusive
 *    prefix sum of H_l*W_l;
 *  - locations must be finite (non-finite input returns an error).
 *
 * Layouts (all dense, row-major):
 *   value  (B, S, M, D)        loc (B, Q, M, L, K, 2)   attn (B, Q, M, L, K)
 *   out / grad_out (B, Q, M, D) grad_value like value, grad_loc like loc,
 *   grad_attn like attn; spatial_shapes (L, 2) rows (H_l, W_l).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_PINNED_F32 0
#define ORACLE_EXACT_F64 1

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_LEVELS 2
#define ORACLE_ERR_NONFINITE 3
#define ORACLE_ERR_NOMEM 4

/* One sampling point mapped to its cell: top-left corner (x0, y0) and the
 * fractional offsets (lx, ly) inside the cell. [FWD] "Bilinear sampling". */
typedef struct {
    int64_t x0, y0;
    double lx, ly;
} cell_t;

static int map_point(double loc_x, double loc_y, int64_t H, int64_t W, int mode,
                     cell_t *c)
{
    double fx, fy; /* floor(x_im), floor(y_im) */
    if (!isfinite(loc_x) || !isfinite(loc_y))
        return ORACLE_ERR_NONFINITE;
    if (mode == ORACLE_PINNED_F32) {
        float xf = fmaf((float)loc_x, (float)W, -0.5f);
        float yf = fmaf((float)loc_y, (float)H, -0.5f);
        float x0f = floorf(xf), y0f = floorf(yf);
        c->lx = (double)(xf - x0f);
        c->ly = (double)(yf - y0f);
        fx = (double)x0f;
        fy = (double)y0f;
    } else {
        double x = loc_x * (double)W - 0.5;
        double y = loc_y * (double)H - 0.5;
        fx = floor(x);
        fy = floor(y);
        c->lx = x - fx;
        c->ly = y - fy;
    }
    /* Clamp far-away cells before the integer conversion. Any x0 <= -2 has
     * both columns out of bounds, as has any x0 >= W, so the clamp keeps
     * every in/out decision and only avoids an overflowing conversion. */
    if (fx < -2.0) fx = -2.0;
    if (fx > (double)W) fx = (double)W;
    if (fy < -2.0) fy = -2.0;
    if (fy > (double)H) fy = (double)H;
    c->x0 = (int64_t)fx;
    c->y0 = (int64_t)fy;
    return ORACLE_OK;
}

/* Corner (i, j) = row y0+i, column x0+j. Zero padding is decided per
 * dimension on the integer coordinates, never on the flat row index.
 * [FWD] "Bilinear sampling" (the four masks) and "The corner gathers". */
static int corner_valid(const cell_t *c, int i, int j, int64_t H, int64_t W)
{
    int64_t yy = c->y0 + i, xx = c->x0 + j;
    return yy >= 0 && yy < H && xx >= 0 && xx < W;
}

static double corner_weight(const cell_t *c, int i, int j)
{
    double wy = i ? c->ly : 1.0 - c->ly;
    double wx = j ? c->lx : 1.0 - c->lx;
    return wy * wx;
}

/* Pointer to value[b, start + (y0+i)*W + (x0+j), m, 0:D], or NULL if the
 * corner is out of bounds (it then reads as zero). */
static const double *corner_row(const double *value, int64_t S, int64_t M,
                                int64_t D, int64_t b, int64_t m, int64_t start,
                                const cell_t *c, int i, int j, int64_t H,
                                int64_t W)
{
    if (!corner_valid(c, i, j, H, W))
        return NULL;
    int64_t row = start + (c->y0 + i) * W + (c->x0 + j);
    return value + ((b * S + row) * M + m) * D;
}

/* Level table: starts from the caller or the exclusive prefix sum of H*W;
 * every level must fit inside the S rows. */
static int level_table(int64_t S, int64_t L, const int64_t *shapes,
                       const int64_t *level_start, int64_t *starts)
{
    int64_t acc = 0;
    for (int64_t l = 0; l < L; ++l) {
        int64_t H = shapes[2 * l], W = shapes[2 * l + 1];
        if (H < 1 || W < 1)
            return ORACLE_ERR_LEVELS;
        starts[l] = level_start ? level_start[l] : acc;
        acc += H * W;
        if (starts[l] < 0 || starts[l] + H * W > S)
            return ORACLE_ERR_LEVELS;
    }
    return ORACLE_OK;
}

static int check_sizes(int64_t B, int64_t S, int64_t M, int64_t D, int64_t L,
                       int64_t Q, int64_t K)
{
    if (B < 0 || S < 0 || M < 1 || D < 1 || L < 1 || Q < 0 || K < 1)
        return ORACLE_ERR_ARG;
    return ORACLE_OK;
}

static void set_threads(int num_threads)
{
#ifdef _OPENMP
    omp_set_num_threads(num_threads > 0 ? num_threads : omp_get_num_procs());
#else
    (void)num_threads;
#endif
}

int msda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Forward: out[b,q,m,:] = sum_l sum_k A[b,q,m,l,k] * sample_l(loc[b,q,m,l,k]),
 * where sample_l is the zero-padded bilinear sample of level l of
 * value[b,:,m,:]. [README] "The operator"; [FWD] "Accumulate and store".
 *
 * touched (optional, B*Q*M bytes): 1 where at least one corner of one point
 * of (b,q,m) is in bounds, else 0 (such an output is exactly zero).
 * Parallel over (b, q); each output row is summed in the fixed order
 * (l, k, corner 00, 01, 10, 11), so the result does not depend on threads.
 */
int msda_oracle_forward(int64_t B, int64_t S, int64_t M, int64_t D, int64_t L,
                        const int64_t *spatial_shapes,
                        const int64_t *level_start_index, int64_t Q, int64_t K,
                        const double *value, const double *loc,
                        const double *attn, double *out, unsigned char *touched,
                        int mode, int num_threads)
{
    int status = check_sizes(B, S, M, D, L, Q, K);
    if (status)
        return status;
    int64_t *starts = (int64_t *)malloc(sizeof(int64_t) * (size_t)L);
    if (!starts)
        return ORACLE_ERR_NOMEM;
    status = level_table(S, L, spatial_shapes, level_start_index, starts);
    if (status) {
        free(starts);
        return status;
    }
    set_threads(num_threads);
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 16) reduction(| : bad)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t q = 0; q < Q; ++q) {
            double *sample = (double *)malloc(sizeof(double) * (size_t)D);
            if (!sample) {
                bad |= 1;
                continue;
            }
            for (int64_t m = 0; m < M; ++m) {
                double *o = out + ((b * Q + q) * M + m) * D;
                int any = 0;
                for (int64_t d = 0; d < D; ++d)
                    o[d] = 0.0;
                for (int64_t l = 0; l < L; ++l) {
                    int64_t H = spatial_shapes[2 * l], W = spatial_shapes[2 * l + 1];
                    for (int64_t k = 0; k < K; ++k) {
                        int64_t p = ((b * Q + q) * M + m) * L * K + l * K + k;
                        cell_t c;
                        if (map_point(loc[2 * p], loc[2 * p + 1], H, W, mode, &c)) {
                            bad |= 2;
                            continue;
                        }
                        for (int64_t d = 0; d < D; ++d)
                            sample[d] = 0.0;
                        for (int i = 0; i < 2; ++i) {
                            for (int j = 0; j < 2; ++j) {
                                const double *v = corner_row(value, S, M, D, b, m, starts[l],
                                                             &c, i, j, H, W);
                                if (!v)
                                    continue;
                                any = 1;
                                double w = corner_weight(&c, i, j);
                                for (int64_t d = 0; d < D; ++d)
                                    sample[d] += w * v[d];
                            }
                        }
                        double a = attn[p];
                        for (int64_t d = 0; d < D; ++d)
                            o[d] += a * sample[d];
                    }
                }
                if (touched)
                    touched[(b * Q + q) * M + m] = (unsigned char)any;
            }
            free(sample);
        }
    }
    free(starts);
    if (bad & 1)
        return ORACLE_ERR_NOMEM;
    if (bad & 2)
        return ORACLE_ERR_NONFINITE;
    return ORACLE_OK;
}

/*
 * Backward, given g = dLoss/dout (B, Q, M, D). [BWD] "What the backward pass
 * must produce":
 *   grad_attn[p]    = sum_d g[d] * s[d]                       (s: the sample)
 *   grad_loc[p].x   = W * A * sum_d g[d] * ((1-ly)(v01-v00) + ly(v11-v10))
 *   grad_loc[p].y   = H * A * sum_d g[d] * ((1-lx)(v10-v00) + lx(v11-v01))
 *   grad_value[row_ij, m, d] += A * w_ij * g[d] for every in-bounds corner.
 * Out-of-bounds corners read as zero and receive nothing ([BWD] "Scatter
 * needs atomics").
 *
 * grad_value is overwritten (zeroed first). The per-point gradients are
 * parallel over (b, q). The grad_value sum is parallel over (b, m): each such
 * task owns head m of batch b, a set of rows no other task writes, and adds
 * its contributions in the fixed order (q, l, k, corner), so the result does
 * not depend on the thread count and needs no atomics.
 *
 * touched_rows (optional, B*S*M bytes): 1 where at least one in-bounds corner
 * landed on (b, row, m), else 0 (such a grad_value row is exactly zero).
 */
int msda_oracle_backward(int64_t B, int64_t S, int64_t M, int64_t D, int64_t L,
                         const int64_t *spatial_shapes,
                         const int64_t *level_start_index, int64_t Q, int64_t K,
                         const double *value, const double *loc,
                         const double *attn, const double *grad_out,
                         double *grad_value, double *grad_loc, double *grad_attn,
                         unsigned char *touched_rows, int mode, int num_threads)
{
    int status = check_sizes(B, S, M, D, L, Q, K);
    if (status)
        return status;
    int64_t *starts = (int64_t *)malloc(sizeof(int64_t) * (size_t)L);
    if (!starts)
        return ORACLE_ERR_NOMEM;
    status = level_table(S, L, spatial_shapes, level_start_index, starts);
    if (status) {
        free(starts);
        return status;
    }
    set_threads(num_threads);
    int bad = 0;

    /* Gradients of the attention weights and of the sampling locations. */
#pragma omp parallel for collapse(2) schedule(dynamic, 16) reduction(| : bad)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t q = 0; q < Q; ++q) {
            for (int64_t m = 0; m < M; ++m) {
                const double *g = grad_out + ((b * Q + q) * M + m) * D;
                for (int64_t l = 0; l < L; ++l) {
                    int64_t H = spatial_shapes[2 * l], W = spatial_shapes[2 * l + 1];
                    for (int64_t k = 0; k < K; ++k) {
                        int64_t p = ((b * Q + q) * M + m) * L * K + l * K + k;
                        cell_t c;
                        if (map_point(loc[2 * p], loc[2 * p + 1], H, W, mode, &c)) {
                            bad |= 2;
                            continue;
                        }
                        const double *v00 = corner_row(value, S, M, D, b, m, starts[l], &c, 0, 0, H, W);
                        const double *v01 = corner_row(value, S, M, D, b, m, starts[l], &c, 0, 1, H, W);
                        const double *v10 = corner_row(value, S, M, D, b, m, starts[l], &c, 1, 0, H, W);
                        const double *v11 = corner_row(value, S, M, D, b, m, starts[l], &c, 1, 1, H, W);
                        double w00 = corner_weight(&c, 0, 0), w01 = corner_weight(&c, 0, 1);
                        double w10 = corner_weight(&c, 1, 0), w11 = corner_weight(&c, 1, 1);
                        double dot_s = 0.0, dot_x = 0.0, dot_y = 0.0;
                        for (int64_t d = 0; d < D; ++d) {
                            double a00 = v00 ? v00[d] : 0.0, a01 = v01 ? v01[d] : 0.0;
                            double a10 = v10 ? v10[d] : 0.0, a11 = v11 ? v11[d] : 0.0;
                            double s = w00 * a00 + w01 * a01 + w10 * a10 + w11 * a11;
                            double sx = (1.0 - c.ly) * (a01 - a00) + c.ly * (a11 - a10);
                            double sy = (1.0 - c.lx) * (a10 - a00) + c.lx * (a11 - a01);
                            dot_s += g[d] * s;
                            dot_x += g[d] * sx;
                            dot_y += g[d] * sy;
                        }
                        double a = attn[p];
                        grad_attn[p] = dot_s;
                        grad_loc[2 * p] = (double)W * a * dot_x;
                        grad_loc[2 * p + 1] = (double)H * a * dot_y;
                    }
                }
            }
        }
    }

    /* Gradient of the value map: the scatter, done as an owner-computes sum. */
#pragma omp parallel for collapse(2) schedule(dynamic, 1) reduction(| : bad)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t m = 0; m < M; ++m) {
            for (int64_t s = 0; s < S; ++s) {
                double *gv = grad_value + ((b * S + s) * M + m) * D;
                for (int64_t d = 0; d < D; ++d)
                    gv[d] = 0.0;
                if (touched_rows)
                    touched_rows[(b * S + s) * M + m] = 0;
            }
            for (int64_t q = 0; q < Q; ++q) {
                const double *g = grad_out + ((b * Q + q) * M + m) * D;
                for (int64_t l = 0; l < L; ++l) {
                    int64_t H = spatial_shapes[2 * l], W = spatial_shapes[2 * l + 1];
                    for (int64_t k = 0; k < K; ++k) {
                        int64_t p = ((b * Q + q) * M + m) * L * K + l * K + k;
                        cell_t c;
                        if (map_point(loc[2 * p], loc[2 * p + 1], H, W, mode, &c)) {
                            bad |= 2;
                            continue;
                        }
                        double a = attn[p];
                        for (int i = 0; i < 2; ++i) {
                            for (int j = 0; j < 2; ++j) {
                                if (!corner_valid(&c, i, j, H, W))
                                    continue;
                                int64_t row = starts[l] + (c.y0 + i) * W + (c.x0 + j);
                                double *gv = grad_value + ((b * S + row) * M + m) * D;
                                double coef = a * corner_weight(&c, i, j);
                                for (int64_t d = 0; d < D; ++d)
                                    gv[d] += coef * g[d];
                                if (touched_rows)
                                    touched_rows[(b * S + row) * M + m] = 1;
                            }
                        }
                    }
                }
            }
        }
    }
    free(starts);
    if (bad & 2)
        return ORACLE_ERR_NONFINITE;
    return ORACLE_OK;
}

/*
 * Rounding statistics of the grad_value scatter, for judging a sum whose
 * every add is rounded to a 16-bit type (course page "5. The backward
 * kernel", section "Atomics make gradients nondeterministic": native
 * half-precision atomics round on each add, so the result depends on the
 * order and carries the rounding of every partial sum).
 *
 * For each grad_value element (b, row, m, d) this returns
 *   abs_sum[b,row,m,d] = sum over the in-bounds corners that land on row of
 *                        |A * w_ij * g[d]|  (the same terms whose signed sum
 *                        msda_oracle_backward returns as grad_value)
 *   count[b,row,m]     = the number of those corners (the same for every d).
 * With these, the recursive-summation bound of numerical analysis gives
 * |fl(sum) - sum| <= gamma_n * abs_sum, gamma_n = n*u / (1 - n*u), for n
 * terms each rounded once to the 16-bit type and added one by one with
 * rounding, in any order; the test suite applies that bound.
 *
 * Same loops, same order and same ownership as the grad_value part of
 * msda_oracle_backward (parallel over (b, m)); value is not needed.
 */
int msda_oracle_scatter_stats(int64_t B, int64_t S, int64_t M, int64_t D, int64_t L,
                              const int64_t *spatial_shapes,
                              const int64_t *level_start_index, int64_t Q, int64_t K,
                              const double *loc, const double *attn,
                              const double *grad_out, double *abs_sum, int64_t *count,
                              int mode, int num_threads)
{
    int status = check_sizes(B, S, M, D, L, Q, K);
    if (status)
        return status;
    int64_t *starts = (int64_t *)malloc(sizeof(int64_t) * (size_t)L);
    if (!starts)
        return ORACLE_ERR_NOMEM;
    status = level_table(S, L, spatial_shapes, level_start_index, starts);
    if (status) {
        free(starts);
        return status;
    }
    set_threads(num_threads);
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1) reduction(| : bad)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t m = 0; m < M; ++m) {
            for (int64_t s = 0; s < S; ++s) {
                double *as = abs_sum + ((b * S + s) * M + m) * D;
                for (int64_t d = 0; d < D; ++d)
                    as[d] = 0.0;
                count[(b * S + s) * M + m] = 0;
            }
            for (int64_t q = 0; q < Q; ++q) {
                const double *g = grad_out + ((b * Q + q) * M + m) * D;
                for (int64_t l = 0; l < L; ++l) {
                    int64_t H = spatial_shapes[2 * l], W = spatial_shapes[2 * l + 1];
                    for (int64_t k = 0; k < K; ++k) {
                        int64_t p = ((b * Q + q) * M + m) * L * K + l * K + k;
                        cell_t c;
                        if (map_point(loc[2 * p], loc[2 * p + 1], H, W, mode, &c)) {
                            bad |= 2;
                            continue;
                        }
                        double a = attn[p];
                        for (int i = 0; i < 2; ++i) {
                            for (int j = 0; j < 2; ++j) {
                                if (!corner_valid(&c, i, j, H, W))
                                    continue;
                                int64_t row = starts[l] + (c.y0 + i) * W + (c.x0 + j);
                                double *as = abs_sum + ((b * S + row) * M + m) * D;
                                double term = a * corner_weight(&c, i, j);
                                for (int64_t d = 0; d < D; ++d)
                                    as[d] += fabs(term * g[d]);
                                count[(b * S + row) * M + m] += 1;
                            }
                        }
                    }
                }
            }
        }
    }
    free(starts);
    if (bad & 2)
        return ORACLE_ERR_NONFINITE;
    return ORACLE_OK;
}
