/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the Gated DeltaNet token mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP library under hybrid_linear_attention_gated_amd/) never calls it
 * and shares no code, header or table with it.
 *
 * Sources (cited by page title and section):
 *   [HF-MoE]  "Hugging Face Transformers: Qwen3.5-MoE series explained"
 *             (devpress.csdn.net), section 4.3 (GatedDeltaNet recurrent-mode
 *             formula), section 4.4 (linear vs full attention table), section
 *             8.2 (cache update flow of a linear_attention layer).
 *   [Book]    "7.6 Qwen3.5: the linear-attention hybrid" (LLM full-stack book,
 *             paper.xwysyy.cn), section 7.6.2 (recurrence, depthwise causal
 *             conv1d with kernel 4, L2 normalisation of q and k).
 *
 * Everything here is computed in double precision.  Inputs are passed as double
 * arrays (the pre-conv x, conv weights, conv caches, the gate z) or as float32 arrays
 * (g, beta, the recurrent states, which the library stores in fp32); the bf16 and
 * fp32 values of stored inputs are exact in either, so the oracle sees the exact
 * stored values, and inputs that are themselves exact products (the layer's
 * projections) reach it unrounded.
 *
 * Layouts (row-major, contiguous):
 *   x        [T][conv_dim]        conv_dim = 2*Hk*dk + Hv*dv, channel order q | k | v
 *   conv_w   [conv_dim][4]        tap 3 multiplies the current token
 *   conv_st  [N][3][conv_dim]     slot 0 is the oldest of the last three inputs
 *   q, k     [T][Hk][dk]          v [T][Hv][dv]
 *   g, beta  [T][Hv]              g is the log of the decay gate a (a = exp(g))
 *   state    [N][Hv][dk][dv]      k-major: S[i][j] with i over dk, j over dv
 *   o        [T][Hv][dv]
 *   cu       [N+1] int32          sequence t0 = cu[s], length = cu[s+1]-cu[s]
 *
 * Parity status: every function below is pinned by the CPU test suite against
 * closed forms, invariants, a library convolution, an exact-rational brute
 * force and a hand-worked example (see tests/test_oracle_pins.py).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define CONV_K 4            /* conv kernel width, [Book] 7.6.2 */
#define CONV_HIST (CONV_K - 1)

/* Number of OpenMP threads the oracle would use for `units` independent jobs. */
int oracle_threads(int units)
{
#ifdef _OPENMP
    int n = omp_get_max_threads();
    return units < n ? units : n;
#else
    (void)units;
    return 1;
#endif
}

/* SiLU(y) = y * sigmoid(y).  Applied to every conv channel after the conv. */
static double silu(double y) { return y / (1.0 + exp(-y)); }

/*
 * Depthwise causal conv1d (kernel 4, no bias) + SiLU + split into q|k|v +
 * per-head L2 normalisation of q and k.  [Book] 7.6.2 gives the conv (one
 * filter per channel, left context only) and the L2 step; [HF-MoE] 8.2 gives
 * the conv cache (the last inputs of the sequence are kept for decoding).
 *
 * y[p][c] = sum_{j=0..3} w[c][j] * xe[p-3+j][c], where xe[-3..-1] is the
 * sequence's conv_state_in (or zeros) and xe[p] = x[cu[s]+p][c].
 * q_hat = q / sqrt(|q|^2 + eps), same for k, per k-head.
 * conv_state_out[s] = xe[L-3], xe[L-2], xe[L-1].
 *
 * cs_in may be NULL (zero history).  cs_out may be NULL.
 */
void oracle_prep(const double *x, const double *w, const int32_t *cu, int N,
                 const double *cs_in, double *cs_out,
                 double *q, double *k, double *v,
                 int T, int Hk, int Hv, int dk, int dv, double eps)
{
    const int conv_dim = 2 * Hk * dk + Hv * dv;
    const int qk_dim = Hk * dk;
    (void)T;
    for (int s = 0; s < N; ++s) {
        const int t0 = cu[s];
        const int L = cu[s + 1] - cu[s];
#pragma omp parallel for schedule(static)
        for (int p = 0; p < L; ++p) {
            double *y = (double *)malloc(sizeof(double) * (size_t)conv_dim);
            for (int c = 0; c < conv_dim; ++c) {
                double acc = 0.0;
                for (int j = 0; j < CONV_K; ++j) {
                    int pos = p - CONV_HIST + j;     /* position within the sequence */
                    double xv;
                    if (pos >= 0)
                        xv = (double)x[(size_t)(t0 + pos) * conv_dim + c];
                    else if (cs_in)
                        xv = (double)cs_in[((size_t)s * CONV_HIST + (CONV_HIST + pos)) * conv_dim + c];
                    else
                        xv = 0.0;
                    acc += (double)w[(size_t)c * CONV_K + j] * xv;
                }
                y[c] = silu(acc);
            }
            const size_t t = (size_t)(t0 + p);
            for (int h = 0; h < Hk; ++h) {
                const double *yq = y + h * dk;
                const double *yk = y + qk_dim + h * dk;
                double nq = 0.0, nk = 0.0;
                for (int i = 0; i < dk; ++i) { nq += yq[i] * yq[i]; nk += yk[i] * yk[i]; }
                nq = 1.0 / sqrt(nq + eps);
                nk = 1.0 / sqrt(nk + eps);
                for (int i = 0; i < dk; ++i) {
                    q[(t * Hk + h) * dk + i] = yq[i] * nq;
                    k[(t * Hk + h) * dk + i] = yk[i] * nk;
                }
            }
            for (int c = 0; c < Hv * dv; ++c)
                v[t * (size_t)(Hv * dv) + c] = y[2 * qk_dim + c];
            free(y);
        }
        if (cs_out) {
            /* The last three inputs of the sequence, reaching into the
             * incoming history when the sequence is shorter than three. */
            for (int slot = 0; slot < CONV_HIST; ++slot) {
                int pos = L - CONV_HIST + slot;
                for (int c = 0; c < conv_dim; ++c) {
                    double xv;
                    if (pos >= 0)
                        xv = (double)x[(size_t)(t0 + pos) * conv_dim + c];
                    else if (cs_in)
                        xv = (double)cs_in[((size_t)s * CONV_HIST + (CONV_HIST + pos)) * conv_dim + c];
                    else
                        xv = 0.0;
                    cs_out[((size_t)s * CONV_HIST + slot) * conv_dim + c] = xv;
                }
            }
        }
    }
}

/*
 * One token of the gated delta rule on a k-major state S[dk][dv], in the
 * order of the recurrent-mode formula of [HF-MoE] 4.3:
 *   S <- a*S                         (decay)
 *   m_j = sum_i S[i][j] * k_i        (retrieve)
 *   delta_j = b * (v_j - m_j)        (correction)
 *   S[i][j] += k_i * delta_j         (write)
 *   o_j = sum_i S[i][j] * q_i        (read)
 * m and delta are caller-provided scratch of length dv.
 *
 * order = 1 is the order of [Book] 7.6.2, S_t = a S_{t-1} + k [b (v - S_{t-1}^T k)]^T:
 * the retrieval reads the state before the decay (retrieve, then decay, correct,
 * write, read).  The two orders agree when a = 1.
 */
static void delta_rule_token(double *S, const double *q, const double *k, const double *v,
                             double a, double b, int dk, int dv, double *m, double *delta, double *o,
                             int order)
{
    if (order == 0)
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] *= a;
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * k[i];
        m[j] = acc;
    }
    if (order != 0)
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] *= a;
    for (int j = 0; j < dv; ++j) delta[j] = b * (v[j] - m[j]);
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] += k[i] * delta[j];
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * q[i];
        o[j] = acc;
    }
}

/*
 * Token-by-token gated delta rule over packed varlen sequences.
 * v-head h reads k-head h / (Hv/Hk) (contiguous groups).  The query is
 * multiplied by `scale` (1.0 reproduces the pages' o = S q).
 * s0 may be NULL (zero initial state); s_final may be NULL.
 * heads[0..n_heads) selects the v-heads to compute (NULL = all); outputs of
 * unselected heads are left untouched.
 */
void oracle_recurrence(const double *q, const double *k, const double *v,
                       const float *g, const float *beta,
                       const int32_t *cu, int N,
                       const float *s0, double *s_final, double *o,
                       double scale, int T, int Hk, int Hv, int dk, int dv,
                       const int32_t *heads, int n_heads, int order)
{
    (void)T;
    const int group = Hv / Hk;
    const int nh = heads ? n_heads : Hv;
    const int units = N * nh;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < units; ++u) {
        const int s = u / nh;
        const int h = heads ? heads[u % nh] : (u % nh);
        const int kh = h / group;
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        double *qs = (double *)malloc(sizeof(double) * (size_t)dk);
        double *m = (double *)malloc(sizeof(double) * (size_t)dv);
        double *delta = (double *)malloc(sizeof(double) * (size_t)dv);
        const size_t st_off = ((size_t)s * Hv + h) * (size_t)dk * dv;
        for (size_t e = 0; e < (size_t)dk * dv; ++e) S[e] = s0 ? (double)s0[st_off + e] : 0.0;
        for (int t = cu[s]; t < cu[s + 1]; ++t) {
            const double *kt = k + ((size_t)t * Hk + kh) * dk;
            const double *qt = q + ((size_t)t * Hk + kh) * dk;
            for (int i = 0; i < dk; ++i) qs[i] = scale * qt[i];
            const double a = exp((double)g[(size_t)t * Hv + h]);
            const double b = (double)beta[(size_t)t * Hv + h];
            delta_rule_token(S, qs, kt, v + ((size_t)t * Hv + h) * dv, a, b, dk, dv, m, delta,
                             o + ((size_t)t * Hv + h) * dv, order);
        }
        if (s_final)
            for (size_t e = 0; e < (size_t)dk * dv; ++e) s_final[st_off + e] = S[e];
        free(S); free(qs); free(m); free(delta);
    }
}

/*
 * One decode step for B sequences ([HF-MoE] 8.2: the conv cache is advanced by
 * one input and the recurrent rule is applied once).
 *   window = [cs[b][0], cs[b][1], cs[b][2], x[b]] -> conv -> SiLU -> split -> L2
 *   one token of the delta rule on state[b][h]
 *   cs[b] <- [cs[b][1], cs[b][2], x[b]]
 * Inputs are never modified; updated caches go to cs_out / state_out.
 */
void oracle_decode(const double *x, const double *w, const double *cs_in, double *cs_out,
                   const float *g, const float *beta, const float *state_in, double *state_out,
                   double *o, double scale, double eps,
                   int B, int Hk, int Hv, int dk, int dv, int order)
{
    const int conv_dim = 2 * Hk * dk + Hv * dv;
    const int qk_dim = Hk * dk;
    const int group = Hv / Hk;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        double *y = (double *)malloc(sizeof(double) * (size_t)conv_dim);
        double *qs = (double *)malloc(sizeof(double) * (size_t)dk);
        double *kn = (double *)malloc(sizeof(double) * (size_t)dk);
        double *m = (double *)malloc(sizeof(double) * (size_t)dv);
        double *delta = (double *)malloc(sizeof(double) * (size_t)dv);
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        for (int c = 0; c < conv_dim; ++c) {
            double win[CONV_K];
            for (int j = 0; j < CONV_HIST; ++j)
                win[j] = (double)cs_in[((size_t)b * CONV_HIST + j) * conv_dim + c];
            win[CONV_HIST] = (double)x[(size_t)b * conv_dim + c];
            double acc = 0.0;
            for (int j = 0; j < CONV_K; ++j) acc += (double)w[(size_t)c * CONV_K + j] * win[j];
            y[c] = silu(acc);
            for (int j = 0; j < CONV_HIST; ++j)
                cs_out[((size_t)b * CONV_HIST + j) * conv_dim + c] = win[j + 1];
        }
        for (int h = 0; h < Hv; ++h) {
            const int kh = h / group;
            const double *yq = y + kh * dk;
            const double *yk = y + qk_dim + kh * dk;
            double nq = 0.0, nk = 0.0;
            for (int i = 0; i < dk; ++i) { nq += yq[i] * yq[i]; nk += yk[i] * yk[i]; }
            nq = 1.0 / sqrt(nq + eps);
            nk = 1.0 / sqrt(nk + eps);
            for (int i = 0; i < dk; ++i) { qs[i] = scale * yq[i] * nq; kn[i] = yk[i] * nk; }
            const size_t st_off = ((size_t)b * Hv + h) * (size_t)dk * dv;
            for (size_t e = 0; e < (size_t)dk * dv; ++e) S[e] = (double)state_in[st_off + e];
            const double a = exp((double)g[(size_t)b * Hv + h]);
            const double bb = (double)beta[(size_t)b * Hv + h];
            delta_rule_token(S, qs, kn, y + 2 * qk_dim + h * dv, a, bb, dk, dv, m, delta,
                             o + ((size_t)b * Hv + h) * dv, order);
            for (size_t e = 0; e < (size_t)dk * dv; ++e) state_out[st_off + e] = S[e];
        }
        free(y); free(qs); free(kn); free(m); free(delta); free(S);
    }
}

/*
 * Gated RMSNorm epilogue of the layer output, [Book] 7.6.2 ("gated RMSNorm
 * output": o = RMSNorm(y) (.) SiLU(z), z a separate projection of the layer
 * input) with the RMSNorm of [Book] 7.6.3 (x * rsqrt(mean(x^2) + eps), then a
 * per-channel gain, computed in full precision).  Readings: the norm runs over
 * each head's dv outputs (the recurrence's y_t = S_t q_t is per head); the
 * per-channel gain `gamma` [dv] is passed as it is applied (the zero-centred
 * parameterisation of 7.6.3 passes 1 + w).
 *
 *   y   [rows][dv]  the recurrence output, one row per (token, value head)
 *   z   [rows][dv]  the gate
 *   out [rows][dv]  out[r][j] = y[r][j] / sqrt(mean_j y[r][j]^2 + eps) * gamma[j] * SiLU(z[r][j])
 */
void oracle_gated_rmsnorm(const double *y, const double *z, const double *gamma, double *out,
                          long rows, int dv, double eps)
{
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) {
        const double *yr = y + (size_t)r * dv;
        double ss = 0.0;
        for (int j = 0; j < dv; ++j) ss += yr[j] * yr[j];
        const double inv = 1.0 / sqrt(ss / (double)dv + eps);
        for (int j = 0; j < dv; ++j)
            out[(size_t)r * dv + j] = yr[j] * inv * (double)gamma[j] * silu((double)z[(size_t)r * dv + j]);
    }
}
