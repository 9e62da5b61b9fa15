/*
 * q4ref.c -- CPU oracle for the affine-Q4 row-batched matrix-vector product.
 *
 * TEST INFRASTRUCTURE. Only the tests, the package smoke check and the benchmark's CPU
 * baseline may load this library. Nothing on the product path links, loads or calls it,
 * and it shares no source, header or helper with the device library.
 *
 * Definition (evaluated in double precision, in the order written):
 *
 *   y[m][r][o] = sum over groups g of
 *                  S[m][o][g] * sum_{j<64} q[m][o][64g+j] * x[m][r][64g+j]
 *                + B[m][o][g] * sum_{j<64} x[m][r][64g+j]
 *
 * which is y = W x for the dequantised weight W[o][i] = S[o][i/64] * q[o][i] + B[o][i/64].
 * Passages followed:
 *   - Constant BATCH_MSL page, quantized_rows section, fn_q4_rows_h: each chunk of codes is
 *     folded as  acc = s * sum(q*x) + b * sum(x)  with the scale and bias of its 64-group;
 *   - same page, prefill helpers, fn_qmv_small_b: the direct per-word form
 *     acc = fma(s[grp], sum q*x, fma(b[grp], sum x, acc)), group index = column / 64,
 *     scale row stride = in_dim / 64.
 * Codes are read UNPACKED here (one byte per code, 0..15), so that an error in the device
 * side's packing can never cancel against the same error in the oracle.
 *
 * bf16 decode: the 16 stored bits are the high half of an IEEE-754 binary32 (memra-engine
 * qwen4exp_gpu.rs page, NgramTable bf16 row read). The decode is exact.
 *
 * bound[m][r][o] = sum_i ( |S q x| + |B x| ) over the in_dim columns of that output, the
 * magnitude against which the per-element error of a faster evaluation is checked.
 *
 * Layouts (all row-major, contiguous):
 *   q  u8  [n_mat][out_dim][in_dim]         x  f32 [n_mat][nb][in_dim]
 *   S,B u16 [n_mat][out_dim][in_dim/64]      y, bound f64 [n_mat][nb][out_dim]
 * Returns 0 on success, -1 on a bad argument.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GROUP 64

static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* One output row (matrix m, row o) for all nb activation rows. */
static void row_all_nb(const uint8_t *q, const uint16_t *S, const uint16_t *B, const float *x,
                       int64_t out_dim, int64_t in_dim, int64_t nb, int64_t m, int64_t o,
                       double *y_out, double *bound_out, int64_t y_stride)
{
    const int64_t groups = in_dim / GROUP;
    const uint8_t *qrow = q + (m * out_dim + o) * in_dim;
    const uint16_t *srow = S + (m * out_dim + o) * groups;
    const uint16_t *brow = B + (m * out_dim + o) * groups;
    for (int64_t r = 0; r < nb; r++) {
        const float *xr = x + (m * nb + r) * in_dim;
        double acc = 0.0, bnd = 0.0;
        for (int64_t g = 0; g < groups; g++) {
            const double s = bf16_value(srow[g]);
            const double b = bf16_value(brow[g]);
            double qx = 0.0, xs = 0.0, qax = 0.0, ax = 0.0;
            for (int64_t j = 0; j < GROUP; j++) {
                const double xv = (double)xr[g * GROUP + j];
                const double qv = (double)qrow[g * GROUP + j];
                qx += qv * xv;
                xs += xv;
                qax += qv * fabs(xv);
                ax += fabs(xv);
            }
            acc += s * qx + b * xs;
            bnd += fabs(s) * qax + fabs(b) * ax;
        }
        y_out[r * y_stride] = acc;
        if (bound_out) bound_out[r * y_stride] = bnd;
    }
}

typedef struct {
    const uint8_t *q;
    const uint16_t *S, *B;
    const float *x;
    int64_t n_mat, out_dim, in_dim, nb;
    /* full mode: rows [lo, hi) of the flattened (m, o) range */
    int64_t lo, hi;
    /* sampled mode: selections [lo, hi) of sel_mat/sel_row */
    const int64_t *sel_mat, *sel_row;
    double *y, *bound;
} job_t;

static void *full_worker(void *arg)
{
    job_t *j = (job_t *)arg;
    for (int64_t t = j->lo; t < j->hi; t++) {
        const int64_t m = t / j->out_dim, o = t % j->out_dim;
        double *yp = j->y + m * j->nb * j->out_dim + o;
        double *bp = j->bound ? j->bound + m * j->nb * j->out_dim + o : NULL;
        row_all_nb(j->q, j->S, j->B, j->x, j->out_dim, j->in_dim, j->nb, m, o, yp, bp,
                   j->out_dim);
    }
    return NULL;
}

static void *sel_worker(void *arg)
{
    job_t *j = (job_t *)arg;
    for (int64_t t = j->lo; t < j->hi; t++) {
        double *yp = j->y + t * j->nb;
        double *bp = j->bound ? j->bound + t * j->nb : NULL;
        row_all_nb(j->q, j->S, j->B, j->x, j->out_dim, j->in_dim, j->nb, j->sel_mat[t],
                   j->sel_row[t], yp, bp, 1);
    }
    return NULL;
}

static int run_threads(job_t *base, int64_t total, int nthreads, void *(*fn)(void *))
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (total < nthreads) nthreads = total > 0 ? (int)total : 1;
    pthread_t th[256];
    int running[256];
    job_t jobs[256];
    for (int t = 0; t < nthreads; t++) {
        jobs[t] = *base;
        jobs[t].lo = total * t / nthreads;
        jobs[t].hi = total * (t + 1) / nthreads;
        running[t] = 0;
        if (t < nthreads - 1 && pthread_create(&th[t], NULL, fn, &jobs[t]) == 0)
            running[t] = 1;
        else
            fn(&jobs[t]); /* last block, or a thread could not start: do it here */
    }
    for (int t = 0; t < nthreads; t++)
        if (running[t]) pthread_join(th[t], NULL);
    return 0;
}

static int check_shape(const void *q, const void *S, const void *B, const void *x,
                       const void *y, int64_t n_mat, int64_t out_dim, int64_t in_dim,
                       int64_t nb)
{
    if (!q || !S || !B || !x || !y) return -1;
    if (n_mat < 1 || out_dim < 1 || nb < 1 || in_dim < GROUP || in_dim % GROUP) return -1;
    return 0;
}

/* Every output: y, bound f64 [n_mat][nb][out_dim] (bound may be NULL). */
int q4ref_gemv(const uint8_t *q, const uint16_t *S, const uint16_t *B, const float *x,
               int64_t n_mat, int64_t out_dim, int64_t in_dim, int64_t nb, double *y,
               double *bound, int nthreads)
{
    if (check_shape(q, S, B, x, y, n_mat, out_dim, in_dim, nb)) return -1;
    job_t j = {q, S, B, x, n_mat, out_dim, in_dim, nb, 0, 0, NULL, NULL, y, bound};
    return run_threads(&j, n_mat * out_dim, nthreads, full_worker);
}

/* Selected outputs only: for t < n_sel, matrix sel_mat[t], output row sel_row[t], all nb
   activation rows -> y, bound f64 [n_sel][nb] (bound may be NULL). */
int q4ref_gemv_rows(const uint8_t *q, const uint16_t *S, const uint16_t *B, const float *x,
                    int64_t n_mat, int64_t out_dim, int64_t in_dim, int64_t nb,
                    const int64_t *sel_mat, const int64_t *sel_row, int64_t n_sel, double *y,
                    double *bound, int nthreads)
{
    if (check_shape(q, S, B, x, y, n_mat, out_dim, in_dim, nb)) return -1;
    if (!sel_mat || !sel_row || n_sel < 1) return -1;
    for (int64_t t = 0; t < n_sel; t++)
        if (sel_mat[t] < 0 || sel_mat[t] >= n_mat || sel_row[t] < 0 || sel_row[t] >= out_dim)
            return -1;
    job_t j = {q, S, B, x, n_mat, out_dim, in_dim, nb, 0, 0, sel_mat, sel_row, y, bound};
    return run_threads(&j, n_sel, nthreads, sel_worker);
}
