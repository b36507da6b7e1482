/* oracle_driver.c -- runs every function of the fp64 oracle (oracle/gdn_oracle.c) on small
 * seeded inputs under AddressSanitizer and UndefinedBehaviorSanitizer: varlen prep with and
 * without conv caches (an empty and a one-token sequence among them), the recurrence in both
 * orders with a head subset, a decode step and the gated RMSNorm.  Checks that every output
 * is finite and that the decode step of a one-token sequence equals the prefill of it.  Test
 * infrastructure: built with gcc together with the oracle source. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_prep(const double *x, const double *w, const int32_t *cu, int N, const double *cs_in, double *cs_out,
                 double *q, double *k, double *v, int T, int Hk, int Hv, int dk, int dv, double eps);
void oracle_recurrence(const double *q, const double *k, const double *v, const float *g, const float *beta,
                       const int32_t *cu, int N, const float *s0, double *s_final, double *o, double scale, int T,
                       int Hk, int Hv, int dk, int dv, const int32_t *heads, int n_heads, int order);
void oracle_decode(const double *x, const double *w, const double *cs_in, double *cs_out, const float *g,
                   const float *beta, const float *state_in, double *state_out, double *o, double scale,
                   double eps, int B, int Hk, int Hv, int dk, int dv, int order);
void oracle_gated_rmsnorm(const double *y, const double *z, const double *gamma, double *out, long rows, int dv,
                          double eps);

static uint64_t rng = 88172645463325252ull;
static double uni(void) {   /* xorshift64 in [-1, 1) */
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}
static double *dalloc(size_t n) { double *p = malloc(n * sizeof(double)); for (size_t i = 0; i < n; ++i) p[i] = uni(); return p; }
static float *falloc(size_t n, double lo, double hi) {
    float *p = malloc(n * sizeof(float));
    for (size_t i = 0; i < n; ++i) p[i] = (float)(lo + (hi - lo) * 0.5 * (uni() + 1.0));
    return p;
}
static int finite_all(const double *p, size_t n) {
    for (size_t i = 0; i < n; ++i) if (!isfinite(p[i])) return 0;
    return 1;
}

int main(void) {
    const int Hk = 1, Hv = 2, dk = 8, dv = 4, C = 2 * Hk * dk + Hv * dv;
    const int32_t cu[5] = {0, 5, 5, 6, 20};   /* lengths 5, 0, 1, 14 */
    const int N = 4, T = 20;
    double *x = dalloc((size_t)T * C), *w = dalloc((size_t)C * 4), *cs = dalloc((size_t)N * 3 * C);
    double *cso = calloc((size_t)N * 3 * C, sizeof(double));
    double *q = calloc((size_t)T * Hk * dk, sizeof(double)), *k = calloc((size_t)T * Hk * dk, sizeof(double));
    double *v = calloc((size_t)T * Hv * dv, sizeof(double)), *o = calloc((size_t)T * Hv * dv, sizeof(double));
    double *fin = calloc((size_t)N * Hv * dk * dv, sizeof(double));
    float *g = falloc((size_t)T * Hv, -1.0, 0.0), *b = falloc((size_t)T * Hv, 0.0, 1.0);
    float *s0 = falloc((size_t)N * Hv * dk * dv, -0.2, 0.2);
    int ok = 1;
    oracle_prep(x, w, cu, N, cs, cso, q, k, v, T, Hk, Hv, dk, dv, 1e-6);
    oracle_prep(x, w, cu, N, NULL, NULL, q, k, v, T, Hk, Hv, dk, dv, 1e-6);
    oracle_prep(x, w, cu, N, cs, cso, q, k, v, T, Hk, Hv, dk, dv, 1e-6);
    ok &= finite_all(q, (size_t)T * Hk * dk) && finite_all(v, (size_t)T * Hv * dv) && finite_all(cso, (size_t)N * 3 * C);
    const int32_t heads[1] = {1};
    for (int order = 0; order < 2; ++order) {
        oracle_recurrence(q, k, v, g, b, cu, N, s0, fin, o, 0.5, T, Hk, Hv, dk, dv, NULL, 0, order);
        ok &= finite_all(o, (size_t)T * Hv * dv) && finite_all(fin, (size_t)N * Hv * dk * dv);
        oracle_recurrence(q, k, v, g, b, cu, N, NULL, NULL, o, 1.0, T, Hk, Hv, dk, dv, heads, 1, order);
    }
    /* decode of sequence 2 (one token, cache = its incoming conv cache) equals its prefill */
    double *od = calloc((size_t)Hv * dv, sizeof(double)), *sd = calloc((size_t)Hv * dk * dv, sizeof(double));
    double *csd = calloc((size_t)3 * C, sizeof(double));
    oracle_prep(x, w, cu, N, cs, cso, q, k, v, T, Hk, Hv, dk, dv, 1e-6);
    oracle_recurrence(q, k, v, g, b, cu, N, s0, fin, o, 1.0, T, Hk, Hv, dk, dv, NULL, 0, 0);
    oracle_decode(x + (size_t)5 * C, w, cs + (size_t)2 * 3 * C, csd, g + 5 * Hv, b + 5 * Hv,
                  s0 + (size_t)2 * Hv * dk * dv, sd, od, 1.0, 1e-6, 1, Hk, Hv, dk, dv, 0);
    for (int i = 0; i < Hv * dv; ++i) ok &= fabs(od[i] - o[(size_t)5 * Hv * dv + i]) < 1e-12;
    for (int i = 0; i < Hv * dk * dv; ++i) ok &= fabs(sd[i] - fin[(size_t)2 * Hv * dk * dv + i]) < 1e-12;
    for (int i = 0; i < 3 * C; ++i) ok &= csd[i] == cso[(size_t)2 * 3 * C + i];
    double *z = dalloc((size_t)T * Hv * dv), *gm = dalloc(dv), *out = calloc((size_t)T * Hv * dv, sizeof(double));
    oracle_gated_rmsnorm(o, z, gm, out, (long)T * Hv, dv, 1e-6);
    ok &= finite_all(out, (size_t)T * Hv * dv);
    free(x); free(w); free(cs); free(cso); free(q); free(k); free(v); free(o); free(fin); free(g); free(b); free(s0);
    free(od); free(sd); free(csd); free(z); free(gm); free(out);
    if (!ok) { fprintf(stderr, "oracle driver: a check failed\n"); return 1; }
    printf("oracle driver ok\n");
    return 0;
}
