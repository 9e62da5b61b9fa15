/* Driver for an AddressSanitizer / UndefinedBehaviorSanitizer build of the C oracle
 * (oracle/q4ref.c). Every buffer is allocated at exactly the size the oracle's layout
 * documents, so a read or write past any of them is reported. Inputs come from a 64-bit
 * linear congruential generator; the checks are closed forms of the definition (codes all 8
 * with bias = -8 * scale gives 0; scale 1, bias 0, x 1 gives the row sums of the codes) and
 * the status of invalid calls. Exit status 0 when every check passes. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int q4ref_gemv(const uint8_t *q, const uint16_t *S, const uint16_t *B, const float *x,
               int64_t n_mat, int64_t out_dim, int64_t in_dim, int64_t nb, double *y,
               double *bound, int nthreads);
int q4ref_gemv_rows(const uint8_t *q, const uint16_t *S, const uint16_t *B, const float *x,
                    int64_t n_mat, int64_t out_dim, int64_t in_dim, int64_t nb,
                    const int64_t *sel_mat, const int64_t *sel_row, int64_t n_sel, double *y,
                    double *bound, int nthreads);

static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint32_t next(void)
{
    st = st * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(st >> 33);
}

static int fails = 0;
#define CHECK(c, ...) do { if (!(c)) { fprintf(stderr, __VA_ARGS__); fputc('\n', stderr); fails++; } } while (0)

static void run_case(int64_t n_mat, int64_t out_dim, int64_t in_dim, int64_t nb, int threads)
{
    const int64_t nq = n_mat * out_dim * in_dim, ng = n_mat * out_dim * (in_dim / 64);
    const int64_t nx = n_mat * nb * in_dim, ny = n_mat * nb * out_dim;
    uint8_t *q = malloc(nq);
    uint16_t *S = malloc(ng * 2), *B = malloc(ng * 2);
    float *x = malloc(nx * 4);
    double *y = malloc(ny * 8), *bound = malloc(ny * 8);
    /* random values: only memory safety and the status are checked */
    for (int64_t i = 0; i < nq; i++) q[i] = next() & 15;
    for (int64_t i = 0; i < ng; i++) { S[i] = 0x3C00 | (next() & 0x3FF); B[i] = next() & 0xBFFF; }
    for (int64_t i = 0; i < nx; i++) x[i] = (float)((int)(next() % 2001) - 1000) / 256.0f;
    CHECK(q4ref_gemv(q, S, B, x, n_mat, out_dim, in_dim, nb, y, bound, threads) == 0,
          "gemv %lldx%lldx%lld nb %lld failed", (long long)n_mat, (long long)out_dim,
          (long long)in_dim, (long long)nb);
    CHECK(q4ref_gemv(q, S, B, x, n_mat, out_dim, in_dim, nb, y, NULL, threads) == 0,
          "gemv without bound failed");
    /* codes 8, bias = -8 * scale (bf16 exponent + 3): every output is exactly 0 */
    for (int64_t i = 0; i < nq; i++) q[i] = 8;
    for (int64_t i = 0; i < ng; i++) { S[i] = 0x3F80 | (next() & 0x7F); B[i] = (uint16_t)((S[i] + (3 << 7)) | 0x8000); }
    q4ref_gemv(q, S, B, x, n_mat, out_dim, in_dim, nb, y, bound, threads);
    for (int64_t i = 0; i < ny; i++) CHECK(y[i] == 0.0, "mid-code output %lld = %g", (long long)i, y[i]);
    /* scale 1, bias 0, x 1: the row sum of the codes */
    for (int64_t i = 0; i < nq; i++) q[i] = next() & 15;
    for (int64_t i = 0; i < ng; i++) { S[i] = 0x3F80; B[i] = 0; }
    for (int64_t i = 0; i < nx; i++) x[i] = 1.0f;
    q4ref_gemv(q, S, B, x, n_mat, out_dim, in_dim, nb, y, bound, threads);
    for (int64_t m = 0; m < n_mat; m++)
        for (int64_t o = 0; o < out_dim; o++) {
            double want = 0;
            for (int64_t i = 0; i < in_dim; i++) want += q[(m * out_dim + o) * in_dim + i];
            for (int64_t r = 0; r < nb; r++)
                CHECK(y[(m * nb + r) * out_dim + o] == want, "row sum m %lld o %lld", (long long)m, (long long)o);
        }
    /* selected rows: the first and last output of every matrix */
    const int64_t n_sel = 2 * n_mat;
    int64_t *sm = malloc(n_sel * 8), *sr = malloc(n_sel * 8);
    double *ys = malloc(n_sel * nb * 8), *bs = malloc(n_sel * nb * 8);
    for (int64_t m = 0; m < n_mat; m++) { sm[2 * m] = sm[2 * m + 1] = m; sr[2 * m] = 0; sr[2 * m + 1] = out_dim - 1; }
    CHECK(q4ref_gemv_rows(q, S, B, x, n_mat, out_dim, in_dim, nb, sm, sr, n_sel, ys, bs, threads) == 0,
          "gemv_rows failed");
    for (int64_t t = 0; t < n_sel; t++)
        for (int64_t r = 0; r < nb; r++)
            CHECK(ys[t * nb + r] == y[(sm[t] * nb + r) * out_dim + sr[t]], "gemv_rows t %lld", (long long)t);
    /* invalid calls are refused */
    sr[0] = out_dim;
    CHECK(q4ref_gemv_rows(q, S, B, x, n_mat, out_dim, in_dim, nb, sm, sr, n_sel, ys, bs, threads) == -1,
          "row past out_dim accepted");
    CHECK(q4ref_gemv(q, S, B, x, n_mat, out_dim, in_dim + 32, nb, y, bound, threads) == -1,
          "in_dim % 64 != 0 accepted");
    CHECK(q4ref_gemv(NULL, S, B, x, n_mat, out_dim, in_dim, nb, y, bound, threads) == -1,
          "NULL codes accepted");
    free(q); free(S); free(B); free(x); free(y); free(bound); free(sm); free(sr); free(ys); free(bs);
}

int main(void)
{
    run_case(1, 1, 64, 1, 1);
    run_case(2, 3, 128, 2, 4);
    run_case(3, 17, 192, 5, 16);   /* more threads than rows */
    run_case(1, 40, 640, 16, 3);
    run_case(2, 9, 2560, 3, 8);
    if (fails) fprintf(stderr, "%d checks failed\n", fails);
    else printf("sanitized oracle: all checks passed\n");
    return fails != 0;
}
