/*
 * Oracle core: softmax attention over a visible key prefix, in fp64.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.
 *
 * What it computes is the plain definition of the attention that the
 * context-parallel method reproduces blockwise ("Megatron-LM 篇", §3.1 and
 * §3.3: the blockwise results are corrected so that they equal the
 * unblocked result; §3.2: each rank's O equals its slice of the non-CP O).
 * For every batch n, query head h and listed query row i:
 *
 *     g     = h / (hq / hkv)           contiguous GQA grouping ("Megatron
 *                                      面试题（一）", M014: one KV group serves
 *                                      a contiguous block of query heads)
 *     z_j   = scale * sum_t q[n,i,h,t] * k[n,j,g,t]     for j < kend[i]
 *     m     = max_j z_j
 *     S     = sum_j exp(z_j - m)
 *     L     = m + ln S                  natural-log log-sum-exp
 *     O[t]  = sum_j (exp(z_j - m) / S) * v[n,j,g,t]
 *
 * A causal row at position p sees keys 0..p, i.e. kend = p + 1 (lower-
 * triangular mask, diagonal included). A "no mask" row sees every key it is
 * given. kend = 0 means no visible key: L = -inf and O = 0 (the empty sum).
 *
 * No tiling, no online rescaling, no reordering: one row at a time, keys in
 * ascending order, dimensions in ascending order. Rows are independent, so
 * OpenMP spreads them over host threads without changing any result.
 *
 * Layouts (C order, element strides implied):
 *   q   [b, nq, hq, d]      k, v [b, nk, hkv, d]      kend [nq]
 *   o   [b, nq, hq, d]      lse  [b, hq, nq]
 *
 * Returns 0 on success, -1 on a bad argument (nothing written).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int oracle_attention(const double *q, const double *k, const double *v,
                     int64_t b, int64_t nq, int64_t nk, int64_t hq, int64_t hkv,
                     int64_t d, double scale, const int64_t *kend,
                     double *o, double *lse, int nthreads) {
    if (!q || !k || !v || !kend || !o || !lse) return -1;
    if (b < 0 || nq < 0 || nk < 0 || hq <= 0 || hkv <= 0 || d <= 0) return -1;
    if (hq % hkv != 0) return -1;
    for (int64_t i = 0; i < nq; ++i)
        if (kend[i] < 0 || kend[i] > nk) return -1;
    const int64_t group = hq / hkv;
    const int64_t total = b * hq * nq;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int failed = 0;
#pragma omp parallel
    {
        double *z = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
        if (!z) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 8)
        for (int64_t item = 0; item < total; ++item) {
            if (!z) continue;
            const int64_t i = item % nq;
            const int64_t h = (item / nq) % hq;
            const int64_t n = item / (nq * hq);
            const int64_t g = h / group;
            const int64_t kn = kend[i];
            const double *qi = q + ((n * nq + i) * hq + h) * d;
            double *oi = o + ((n * nq + i) * hq + h) * d;
            double *li = lse + (n * hq + h) * nq + i;
            if (kn == 0) {
                for (int64_t t = 0; t < d; ++t) oi[t] = 0.0;
                *li = -INFINITY;
                continue;
            }
            /* scores */
            for (int64_t j = 0; j < kn; ++j) {
                const double *kj = k + ((n * nk + j) * hkv + g) * d;
                double dot = 0.0;
                for (int64_t t = 0; t < d; ++t) dot += qi[t] * kj[t];
                z[j] = scale * dot;
            }
            /* log-sum-exp */
            double m = z[0];
            for (int64_t j = 1; j < kn; ++j)
                if (z[j] > m) m = z[j];
            double s = 0.0;
            for (int64_t j = 0; j < kn; ++j) s += exp(z[j] - m);
            *li = m + log(s);
            /* softmax-weighted sum of values */
            for (int64_t t = 0; t < d; ++t) oi[t] = 0.0;
            for (int64_t j = 0; j < kn; ++j) {
                const double w = exp(z[j] - m) / s;
                const double *vj = v + ((n * nk + j) * hkv + g) * d;
                for (int64_t t = 0; t < d; ++t) oi[t] += w * vj[t];
            }
        }
        free(z);
    }
    return failed ? -1 : 0;
}

/*
 * Backward of the same attention, in fp64: the gradients of a scalar loss
 * whose gradient with respect to O is dO.  The pages name the backward only
 * through the communication it adds under context parallelism ("超大规模集群…",
 * "CP 与其他技术结合": an all-gather of K/V and a reduce-scatter of their
 * gradients); the arithmetic is the derivative of the definition above,
 * written out.  For every batch n, query head h and query row i:
 *
 *     P_j   = exp(z_j - L)                         (the softmax weights)
 *     O[t]  = sum_j P_j v_j[t]                     (recomputed, as above)
 *     D     = sum_t dO[t] O[t]
 *     dP_j  = sum_t dO[t] v_j[t]
 *     dS_j  = P_j (dP_j - D)                       (softmax derivative)
 *     dq[t] = scale * sum_j dS_j k_j[t]
 *     dk_j[t] += scale * dS_j q[t]                 (summed over every row i
 *     dv_j[t] += P_j dO[t]                          and every head h of the
 *                                                   group g of head h)
 *
 * Work is split over (batch, KV head) so every dk/dv row has one writer;
 * inside a group, heads ascend, then rows, then keys.
 *
 * Layouts: q, dq, dout [b, nq, hq, d]; k, v, dk, dv [b, nk, hkv, d];
 * kend [nq].  dq, dk and dv are overwritten.
 */
int oracle_attention_bwd(const double *q, const double *k, const double *v,
                         const double *dout, int64_t b, int64_t nq, int64_t nk,
                         int64_t hq, int64_t hkv, int64_t d, double scale,
                         const int64_t *kend, double *dq, double *dk, double *dv,
                         int nthreads) {
    if (!q || !k || !v || !dout || !kend || !dq || !dk || !dv) return -1;
    if (b < 0 || nq < 0 || nk < 0 || hq <= 0 || hkv <= 0 || d <= 0) return -1;
    if (hq % hkv != 0) return -1;
    for (int64_t i = 0; i < nq; ++i)
        if (kend[i] < 0 || kend[i] > nk) return -1;
    const int64_t group = hq / hkv;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int failed = 0;
#pragma omp parallel
    {
        const size_t nkz = (size_t)(nk > 0 ? nk : 1);
        double *z = (double *)malloc(sizeof(double) * nkz);
        double *o = (double *)malloc(sizeof(double) * (size_t)d);
        if (!z || !o) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t item = 0; item < b * hkv; ++item) {
            if (!z || !o) continue;
            const int64_t n = item / hkv, g = item % hkv;
            for (int64_t j = 0; j < nk; ++j)
                for (int64_t t = 0; t < d; ++t) {
                    dk[((n * nk + j) * hkv + g) * d + t] = 0.0;
                    dv[((n * nk + j) * hkv + g) * d + t] = 0.0;
                }
            for (int64_t h = g * group; h < (g + 1) * group; ++h)
                for (int64_t i = 0; i < nq; ++i) {
                    const int64_t kn = kend[i];
                    const double *qi = q + ((n * nq + i) * hq + h) * d;
                    const double *doi = dout + ((n * nq + i) * hq + h) * d;
                    double *dqi = dq + ((n * nq + i) * hq + h) * d;
                    for (int64_t t = 0; t < d; ++t) dqi[t] = 0.0;
                    if (kn == 0) continue;
                    for (int64_t j = 0; j < kn; ++j) {
                        const double *kj = k + ((n * nk + j) * hkv + g) * d;
                        double dot = 0.0;
                        for (int64_t t = 0; t < d; ++t) dot += qi[t] * kj[t];
                        z[j] = scale * dot;
                    }
                    double m = z[0];
                    for (int64_t j = 1; j < kn; ++j)
                        if (z[j] > m) m = z[j];
                    double s = 0.0;
                    for (int64_t j = 0; j < kn; ++j) s += exp(z[j] - m);
                    const double lse = m + log(s);
                    for (int64_t t = 0; t < d; ++t) o[t] = 0.0;
                    for (int64_t j = 0; j < kn; ++j) {
                        const double p = exp(z[j] - lse);
                        const double *vj = v + ((n * nk + j) * hkv + g) * d;
                        for (int64_t t = 0; t < d; ++t) o[t] += p * vj[t];
                    }
                    double dd = 0.0;
                    for (int64_t t = 0; t < d; ++t) dd += doi[t] * o[t];
                    for (int64_t j = 0; j < kn; ++j) {
                        const double p = exp(z[j] - lse);
                        const double *kj = k + ((n * nk + j) * hkv + g) * d;
                        const double *vj = v + ((n * nk + j) * hkv + g) * d;
                        double *dkj = dk + ((n * nk + j) * hkv + g) * d;
                        double *dvj = dv + ((n * nk + j) * hkv + g) * d;
                        double dp = 0.0;
                        for (int64_t t = 0; t < d; ++t) dp += doi[t] * vj[t];
                        const double ds = p * (dp - dd);
                        for (int64_t t = 0; t < d; ++t) {
                            dqi[t] += scale * ds * kj[t];
                            dkj[t] += scale * ds * qi[t];
                            dvj[t] += p * doi[t];
                        }
                    }
                }
        }
        free(z);
        free(o);
    }
    return failed ? -1 : 0;
}
