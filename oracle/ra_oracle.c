/*
 * ra_oracle.c -- plain fp64 CPU reference for one ring member's attention share.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no source with the GPU library.
 *
 * What it computes (the plain definition, no tiling, no online softmax):
 *   Ring Attention (slowleelab "Ring Attention" page, L4 section 4.2 and the
 *   closing remark of 4.3) states that after the N ring steps, rank i holds the
 *   complete attention of its resident query block Q_i over the whole sequence;
 *   the FlashAttention explainer (aliyun page, section 2) states that blockwise
 *   FlashAttention is mathematically the same as standard attention.  Standard
 *   scaled dot-product attention is S = Q K^T / sqrt(d), A = softmax(S), O = A V
 *   (lnwmold page, section 2.1), with the softmax taken over keys and made safe by
 *   subtracting the row maximum (slowleelab page, 4.3).  Grouped-query attention
 *   lets a group of query heads share one K/V head (lnwmold page, section 2.2);
 *   groups are contiguous, kv head g = h / (H / H_kv).
 *
 * For every selected query row (b, h, r) and a list of key ranges [lo, hi)
 * (a union of ring blocks; all L keys for a whole share, the blocks visited so
 * far for a partial share):
 *     s_k = scale * sum_c Q[b,h,r,c] * K[b,g,k,c]       for every listed key k
 *     M   = max_k s_k
 *     p_k = exp(s_k - M)
 *     Z   = sum_k p_k
 *     O   = (sum_k p_k * V[b,g,k,:]) / Z
 * All arithmetic is fp64 and every score of the row is materialised.  Inputs are
 * read as their stored bits (fp32 or bf16, both widened to fp64 exactly, or fp64
 * values such as dequantized fp8 inputs, which fp32 cannot hold exactly).
 *
 * Layouts (row-major): Q is [B, H, l_q, d]; K and V are [B, H_kv, L, d].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORA_F32 0
#define ORA_BF16 1
#define ORA_F64 2

static double widen(const void *base, int dtype, int64_t idx)
{
    if (dtype == ORA_F32)
        return (double)((const float *)base)[idx];
    if (dtype == ORA_F64)
        return ((const double *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * Causal masking (optional).  With qpos and kpos given, key k takes part in row i's
 * softmax only if kpos[k] <= qpos[i]: a query attends to itself and to earlier
 * tokens only (slowleelab page, 4.5 limitation 2: under causal attention the query
 * block Q_i attends only to K blocks at or before it).  qpos[i] is the global
 * sequence position of selected row i, kpos[k] that of key row k; the caller derives
 * both from how tokens are assigned to ring members.  With both NULL every listed
 * key is used.  A row left with no key is reported as an error (code 3).
 *
 * Returns 0 on success, 1 on a bad argument, 2 on allocation failure, 3 if a row has
 * no admissible key.
 */
int ra_oracle_rows_masked(int dtype, const void *Q, int64_t l_q, const void *K,
                          const void *V, int64_t L, int B, int H, int H_kv, int d,
                          double scale, const int64_t *rows, int64_t n_rows,
                          const int64_t *key_lo, const int64_t *key_hi, int n_ranges,
                          const int64_t *qpos, const int64_t *kpos, double *O, double *M,
                          double *Z, int nthreads)
{
    if ((dtype != ORA_F32 && dtype != ORA_BF16 && dtype != ORA_F64) || !Q || !K || !V || !rows || !O || !M ||
        !Z || l_q < 1 || L < 1 || B < 1 || H < 1 || H_kv < 1 || d < 1 || H % H_kv != 0 ||
        n_rows < 0 || n_ranges < 1 || !key_lo || !key_hi || (!qpos) != (!kpos))
        return 1;
    int64_t n_keys = 0;
    for (int i = 0; i < n_ranges; i++) {
        if (key_lo[i] < 0 || key_hi[i] > L || key_lo[i] > key_hi[i])
            return 1;
        n_keys += key_hi[i] - key_lo[i];
    }
    if (n_keys < 1)
        return 1;
    for (int64_t i = 0; i < n_rows; i++)
        if (rows[i] < 0 || rows[i] >= (int64_t)B * H * l_q)
            return 1;
    const int group = H / H_kv;
    int failed = 0;
    if (nthreads < 1)
        nthreads = 1;

#pragma omp parallel num_threads(nthreads)
    {
        double *q = (double *)malloc(sizeof(double) * (size_t)d);
        double *s = (double *)malloc(sizeof(double) * (size_t)n_keys);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        if (!q || !s || !acc) {
#pragma omp atomic write
            failed = 2;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_rows; i++) {
            if (!q || !s || !acc)
                continue;
            const int64_t flat = rows[i];
            const int64_t r = flat % l_q;
            const int64_t bh = flat / l_q;
            const int h = (int)(bh % H);
            const int b = (int)(bh / H);
            const int g = h / group;
            const int64_t q_base = flat * d;
            const int64_t kv_base = ((int64_t)b * H_kv + g) * L * d;
            (void)r;
            for (int c = 0; c < d; c++)
                q[c] = widen(Q, dtype, q_base + c);

            /* scores of every listed, admissible key */
            int64_t n = 0;
            for (int rg = 0; rg < n_ranges; rg++)
                for (int64_t k = key_lo[rg]; k < key_hi[rg]; k++) {
                    if (qpos && kpos[k] > qpos[i])
                        continue;
                    double dot = 0.0;
                    for (int c = 0; c < d; c++)
                        dot += q[c] * widen(K, dtype, kv_base + k * d + c);
                    s[n++] = scale * dot;
                }
            if (n == 0) {
#pragma omp atomic write
                failed = 3;
                continue;
            }
            /* safe softmax: maximum, shifted exponentials, their sum */
            double mx = s[0];
            for (int64_t k = 1; k < n; k++)
                if (s[k] > mx)
                    mx = s[k];
            double z = 0.0;
            for (int64_t k = 0; k < n; k++) {
                s[k] = exp(s[k] - mx);
                z += s[k];
            }
            /* weighted sum of V, normalised once */
            for (int c = 0; c < d; c++)
                acc[c] = 0.0;
            n = 0;
            for (int rg = 0; rg < n_ranges; rg++)
                for (int64_t k = key_lo[rg]; k < key_hi[rg]; k++) {
                    if (qpos && kpos[k] > qpos[i])
                        continue;
                    const double p = s[n++];
                    for (int c = 0; c < d; c++)
                        acc[c] += p * widen(V, dtype, kv_base + k * d + c);
                }
            for (int c = 0; c < d; c++)
                O[i * d + c] = acc[c] / z;
            M[i] = mx;
            Z[i] = z;
        }
        free(q);
        free(s);
        free(acc);
    }
    return failed;
}

/* Unmasked form: every listed key of every selected row. */
int ra_oracle_rows(int dtype, const void *Q, int64_t l_q, const void *K, const void *V,
                   int64_t L, int B, int H, int H_kv, int d, double scale,
                   const int64_t *rows, int64_t n_rows, const int64_t *key_lo,
                   const int64_t *key_hi, int n_ranges, double *O, double *M, double *Z,
                   int nthreads)
{
    return ra_oracle_rows_masked(dtype, Q, l_q, K, V, L, B, H, H_kv, d, scale, rows, n_rows,
                                 key_lo, key_hi, n_ranges, NULL, NULL, O, M, Z, nthreads);
}

/* Thread count the OpenMP runtime would use by default (for reporting). */
int ra_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
