/*
 * Host driver for the sanitizer build of the oracle core (attention.c):
 * runs the forward and backward definitions on small seeded inputs with
 * every kind of visible-key count (none, some, all), so AddressSanitizer
 * sees every index the core computes and UndefinedBehaviorSanitizer every
 * integer and pointer operation.  Also checks the facts that hold for any
 * input: a row that sees no key gets L = -inf and O = 0; otherwise O is
 * finite and, with V == 1, exactly 1 up to rounding; and the sum of dK and
 * dV contributions is finite.  Exit status 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_attention(const double *q, const double *k, const double *v, int64_t b, int64_t nq,
                     int64_t nk, int64_t hq, int64_t hkv, int64_t d, double scale,
                     const int64_t *kend, double *o, double *lse, int nthreads);
int oracle_attention_bwd(const double *q, const double *k, const double *v, const double *dout,
                         int64_t b, int64_t nq, int64_t nk, int64_t hq, int64_t hkv, int64_t d,
                         double scale, const int64_t *kend, double *dq, double *dk, double *dv,
                         int nthreads);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double uniform(void) {   /* xorshift64*, then [-1, 1) */
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (double)((state * 0x2545F4914F6CDD1Dull) >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static double *fill(size_t n, int ones) {
    double *x = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) x[i] = ones ? 1.0 : uniform();
    return x;
}

static int run(int64_t b, int64_t nq, int64_t nk, int64_t hq, int64_t hkv, int64_t d) {
    const size_t nqe = (size_t)(b * nq * hq * d), nke = (size_t)(b * nk * hkv * d);
    double *q = fill(nqe, 0), *k = fill(nke, 0), *v = fill(nke, 1), *dout = fill(nqe, 0);
    double *o = malloc(nqe * sizeof(double)), *lse = malloc((size_t)(b * hq * nq) * sizeof(double));
    double *dq = malloc(nqe * sizeof(double)), *dk = malloc(nke * sizeof(double));
    double *dv = malloc(nke * sizeof(double));
    int64_t *kend = malloc((size_t)nq * sizeof(int64_t));
    for (int64_t i = 0; i < nq; ++i) kend[i] = (i * 7) % (nk + 1);   /* 0 .. nk */
    kend[nq - 1] = nk;
    int bad = 0;
    if (oracle_attention(q, k, v, b, nq, nk, hq, hkv, d, 1.0 / sqrt((double)d), kend, o, lse, 2))
        bad = 1;
    for (int64_t n = 0; n < b && !bad; ++n)
        for (int64_t i = 0; i < nq; ++i)
            for (int64_t h = 0; h < hq; ++h) {
                const double l = lse[(n * hq + h) * nq + i];
                for (int64_t t = 0; t < d; ++t) {
                    const double x = o[((n * nq + i) * hq + h) * d + t];
                    if (kend[i] == 0 ? (x != 0.0 || !isinf(l) || l > 0)
                                     : (!isfinite(x) || fabs(x - 1.0) > 1e-12))
                        bad = 1;
                }
            }
    if (!bad && oracle_attention_bwd(q, k, v, dout, b, nq, nk, hq, hkv, d, 0.3, kend, dq, dk, dv,
                                     2))
        bad = 1;
    for (size_t i = 0; i < nke && !bad; ++i)
        if (!isfinite(dk[i]) || !isfinite(dv[i])) bad = 1;
    /* invalid arguments are refused, nothing written */
    kend[0] = nk + 1;
    if (oracle_attention(q, k, v, b, nq, nk, hq, hkv, d, 1.0, kend, o, lse, 1) != -1) bad = 1;
    kend[0] = 0;
    if (oracle_attention(q, k, v, b, nq, nk, hq, hq + 1, d, 1.0, kend, o, lse, 1) != -1) bad = 1;
    free(q); free(k); free(v); free(dout); free(o); free(lse);
    free(dq); free(dk); free(dv); free(kend);
    return bad;
}

int main(void) {
    static const int64_t shapes[][6] = {{1, 1, 1, 1, 1, 8}, {2, 13, 17, 4, 2, 16},
                                        {1, 40, 40, 6, 3, 32}, {3, 9, 30, 2, 1, 4}};
    for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i) {
        const int64_t *s = shapes[i];
        if (run(s[0], s[1], s[2], s[3], s[4], s[5])) {
            fprintf(stderr, "oracle sanitizer driver: shape %zu failed\n", i);
            return 1;
        }
    }
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
