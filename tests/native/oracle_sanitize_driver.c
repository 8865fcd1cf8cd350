/* Drives the oracle's C entry points under AddressSanitizer and UndefinedBehavior-
 * Sanitizer: every dtype, ragged key ranges, selected and repeated rows, causal masks,
 * grouped K/V heads, and every argument the oracle must reject.  It checks return codes
 * and that outputs are finite; the values themselves are pinned by the Python tests. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int ra_oracle_rows_masked(int dtype, const void *Q, int64_t l_q, const void *K,
                          const void *V, int64_t L, int B, int H, int H_kv, int d,
                          double scale, const int64_t *rows, int64_t n_rows,
                          const int64_t *key_lo, const int64_t *key_hi, int n_ranges,
                          const int64_t *qpos, const int64_t *kpos, double *O, double *M,
                          double *Z, int nthreads);
int ra_oracle_rows(int dtype, const void *Q, int64_t l_q, const void *K, const void *V,
                   int64_t L, int B, int H, int H_kv, int d, double scale,
                   const int64_t *rows, int64_t n_rows, const int64_t *key_lo,
                   const int64_t *key_hi, int n_ranges, double *O, double *M, double *Z,
                   int nthreads);

static int failures = 0;
#define CHECK(cond, what)                                   \
    do {                                                    \
        if (!(cond)) {                                      \
            fprintf(stderr, "FAIL: %s (line %d)\n", what, __LINE__); \
            failures++;                                     \
        }                                                   \
    } while (0)

static uint32_t rng = 12345u;
static float frand(void)
{
    rng = rng * 1664525u + 1013904223u;
    return ((float)(rng >> 8) / 16777216.0f) * 2.0f - 1.0f;
}

/* Exactly-sized heap buffers, so any out-of-bounds access is caught. */
static void *fill(int dtype, int64_t n)
{
    if (dtype == 0) {
        float *p = malloc(sizeof(float) * (size_t)n);
        for (int64_t i = 0; i < n; i++) p[i] = frand();
        return p;
    }
    if (dtype == 1) {
        uint16_t *p = malloc(sizeof(uint16_t) * (size_t)n);
        for (int64_t i = 0; i < n; i++) {
            float f = frand();
            uint32_t u;
            memcpy(&u, &f, 4);
            p[i] = (uint16_t)(u >> 16);
        }
        return p;
    }
    double *p = malloc(sizeof(double) * (size_t)n);
    for (int64_t i = 0; i < n; i++) p[i] = frand();
    return p;
}

static int all_finite(const double *x, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        if (!isfinite(x[i])) return 0;
    return 1;
}

static void run_case(int dtype, int B, int H, int H_kv, int d, int64_t l_q, int64_t L,
                     int masked, int nthreads)
{
    void *Q = fill(dtype, (int64_t)B * H * l_q * d);
    void *K = fill(dtype, (int64_t)B * H_kv * L * d);
    void *V = fill(dtype, (int64_t)B * H_kv * L * d);
    const int64_t n_all = (int64_t)B * H * l_q;
    /* every row, then the last row twice and the first once */
    const int64_t n_rows = n_all + 3;
    int64_t *rows = malloc(sizeof(int64_t) * (size_t)n_rows);
    for (int64_t i = 0; i < n_all; i++) rows[i] = i;
    rows[n_all] = n_all - 1;
    rows[n_all + 1] = n_all - 1;
    rows[n_all + 2] = 0;
    /* ragged key ranges covering [0, L) out of order */
    int64_t lo[3], hi[3];
    int n_ranges = 1;
    lo[0] = 0;
    hi[0] = L;
    if (L >= 3) {
        n_ranges = 3;
        lo[0] = L / 2; hi[0] = L;
        lo[1] = 0;     hi[1] = 1;
        lo[2] = 1;     hi[2] = L / 2;
    }
    int64_t *qpos = NULL, *kpos = NULL;
    if (masked) { /* query r sees keys with position <= r + 1 (key 0 always) */
        qpos = malloc(sizeof(int64_t) * (size_t)n_rows);
        kpos = malloc(sizeof(int64_t) * (size_t)L);
        for (int64_t i = 0; i < n_rows; i++) qpos[i] = rows[i] % l_q + 1;
        for (int64_t k = 0; k < L; k++) kpos[k] = k;
    }
    double *O = malloc(sizeof(double) * (size_t)(n_rows * d));
    double *M = malloc(sizeof(double) * (size_t)n_rows);
    double *Z = malloc(sizeof(double) * (size_t)n_rows);
    int rc = masked
        ? ra_oracle_rows_masked(dtype, Q, l_q, K, V, L, B, H, H_kv, d, 0.125, rows, n_rows, lo,
                                hi, n_ranges, qpos, kpos, O, M, Z, nthreads)
        : ra_oracle_rows(dtype, Q, l_q, K, V, L, B, H, H_kv, d, 0.125, rows, n_rows, lo, hi,
                         n_ranges, O, M, Z, nthreads);
    CHECK(rc == 0, "valid call succeeds");
    if (rc == 0) {
        CHECK(all_finite(O, n_rows * d) && all_finite(M, n_rows) && all_finite(Z, n_rows),
              "finite outputs");
        for (int c = 0; c < d; c++)  /* repeated rows give identical results */
            CHECK(O[(n_all - 1) * d + c] == O[n_all * d + c], "repeat row equal");
    }
    free(Q); free(K); free(V); free(rows); free(qpos); free(kpos); free(O); free(M); free(Z);
}

static void invalid_args(void)
{
    float q[8 * 4], k[8 * 4], v[8 * 4];
    memset(q, 0, sizeof q); memset(k, 0, sizeof k); memset(v, 0, sizeof v);
    int64_t rows[2] = {0, 1}, lo[1] = {0}, hi[1] = {8}, bad_hi[1] = {9}, empty_hi[1] = {0};
    int64_t bad_rows[1] = {8}, neg_rows[1] = {-1}, pos[8] = {0};
    double O[2 * 4], M[2], Z[2];
    /* Q [1,1,8,4], K/V [1,1,8,4] */
#define CALL(dt, QQ, lq, LL, B, H, Hkv, d, r, nr, l, h, nrg, qp, kp, o)                        \
    ra_oracle_rows_masked(dt, QQ, lq, k, v, LL, B, H, Hkv, d, 0.5, r, nr, l, h, nrg, qp, kp,   \
                          o, M, Z, 1)
    CHECK(CALL(0, q, 8, 8, 1, 1, 1, 4, rows, 2, lo, hi, 1, NULL, NULL, O) == 0, "baseline ok");
    CHECK(CALL(7, q, 8, 8, 1, 1, 1, 4, rows, 2, lo, hi, 1, NULL, NULL, O) == 1, "dtype");
    CHECK(CALL(0, NULL, 8, 8, 1, 1, 1, 4, rows, 2, lo, hi, 1, NULL, NULL, O) == 1, "null Q");
    CHECK(CALL(0, q, 0, 8, 1, 1, 1, 4, rows, 2, lo, hi, 1, NULL, NULL, O) == 1, "l_q 0");
    CHECK(CALL(0, q, 8, 8, 1, 2, 3, 4, rows, 2, lo, hi, 1, NULL, NULL, O) == 1, "H % H_kv");
    CHECK(CALL(0, q, 8, 8, 1, 1, 1, 0, rows, 2, lo, hi, 1, NULL, NULL, O) == 1, "d 0");
    CHECK(CALL(0, q, 8, 8, 1, 1, 1, 4, rows, 2, lo, bad_hi, 1, NULL, NULL, O) == 1, "range > L");
    CHECK(CALL(0, q, 8, 8, 1, 1, 1, 4, rows, 2, lo, empty_hi, 1, NULL, NULL, O) == 1, "no keys");
    CHECK(CALL(0, q, 8, 8, 1, 1, 1, 4, bad_rows, 1, lo, hi, 1, NULL, NULL, O) == 1, "row >= n");
    CHECK(CALL(0, q, 8, 8, 1, 1, 1, 4, neg_rows, 1, lo, hi, 1, NULL, NULL, O) == 1, "row < 0");
    CHECK(CALL(0, q, 8, 8, 1, 1, 1, 4, rows, 2, lo, hi, 1, pos, NULL, O) == 1, "one mask side");
    CHECK(CALL(0, q, 8, 8, 1, 1, 1, 4, rows, 2, lo, hi, 0, NULL, NULL, O) == 1, "no ranges");
    CHECK(CALL(0, q, 8, 8, 1, 1, 1, 4, rows, 2, lo, hi, 1, NULL, NULL, NULL) == 1, "null O");
    {   /* a row that sees no key under the mask is reported, not computed */
        int64_t qp[2] = {-1, 0}, kp[8] = {0, 1, 2, 3, 4, 5, 6, 7};
        CHECK(CALL(0, q, 8, 8, 1, 1, 1, 4, rows, 2, lo, hi, 1, qp, kp, O) == 3, "empty row");
    }
#undef CALL
}

int main(void)
{
    for (int dtype = 0; dtype < 3; dtype++) {
        run_case(dtype, 1, 2, 2, 4, 5, 7, 0, 1);   /* tiny, odd sizes */
        run_case(dtype, 2, 4, 2, 8, 3, 11, 0, 3);  /* batch, grouped K/V, threads */
        run_case(dtype, 1, 3, 1, 16, 4, 9, 1, 2);  /* causal mask, MQA */
        run_case(dtype, 1, 1, 1, 64, 2, 1, 0, 1);  /* one key */
        run_case(dtype, 1, 2, 2, 128, 6, 33, 1, 4);
    }
    invalid_args();
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("oracle sanitize driver: ok\n");
    return 0;
}
