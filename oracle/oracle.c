/*
 * oracle.c -- plain, slow CPU oracle for the temperature-T BCJR soft quantizer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg load
 * this library.  It shares no code, header, table or helper with the GPU path, and neither includes the
 * other.
 *
 * Source: "BCJR-QAT: A Differentiable Relaxation of Trellis-Coded Weight Quantization" (arXiv 2605.10655).
 *   - Abstract (searcharxiv.org page): the Viterbi argmax of trellis-coded quantization is replaced by the BCJR
 *     forward-backward sum-product pass at temperature T; the soft codeword is the Boltzmann expectation
 *     over trellis paths; T -> 0 gives back the hard code; the pass equals a 1-D Ising transfer-matrix product.
 *   - gist.science Technical Summary, "Core Mechanism": paths carry a Boltzmann weight; the soft codeword at
 *     step t is sum_s c(s) p_T(s_t = s | w); it is exactly differentiable in the weight pre-image w.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *   - trellis: bitshift, L state bits, k new bits per step entering at the low end:
 *       Succ_b(s) = ((s << k) & (2^L - 1)) | b,   Pred_a(s') = (s' >> k) | (a << (L - k)).
 *   - path energy E = sum_t (w_t - c(s_t))^2, path weight exp(-E / T); transitions carry no cost.
 *   - free mode: s_1 is any state, s_n any state.  sigma mode: a non-emitting start s_0 = sigma, the first
 *     emitting state is a successor of sigma, and the last emitting state s_n = sigma (sigma masked to L bits).
 *   - log_z = ln Z over the emitting states only (no factor for the non-emitting start).
 *
 * Every soft quantity is computed in float64 with IEEE libm exp/log; the Viterbi pass is IEEE float32 with
 * the operation order fixed below (built without FMA contraction and without fast-math).
 *
 * Each routine works on one sequence at a time with plain per-state loops (no grouping of states, no
 * blocking); sequences are independent and are spread over OpenMP threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_NOMEM (-2)

/* ------------------------------------------------------------------------------------------------ */
/* trellis                                                                                           */

static inline uint32_t succ(uint32_t s, uint32_t b, int L, int k) {
    return ((s << k) & ((1u << L) - 1u)) | b;
}

static inline uint32_t pred(uint32_t s, uint32_t a, int L, int k) {
    return (s >> k) | (a << (L - k));
}

/* log(sum_i exp(x_i)); returns -inf when every x_i is -inf. */
static double log_sum_exp(const double* x, int m) {
    double mx = -INFINITY;
    for (int i = 0; i < m; ++i)
        if (x[i] > mx) mx = x[i];
    if (mx == -INFINITY) return -INFINITY;
    double s = 0.0;
    for (int i = 0; i < m; ++i) s += exp(x[i] - mx);
    return mx + log(s);
}

/* theta_t(s) = -(w_t - c(s))^2 / T : the log Boltzmann weight of emitting c(s) at step t. */
static inline double log_weight(double wt, double cs, double T) {
    double d = wt - cs;
    return -(d * d) / T;
}

static int check_args(int64_t B, int64_t n, int L, int k) {
    if (B < 0 || n < 1 || k < 1 || L <= k || L > 24) return ORACLE_ERR_ARG;
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------------------------------ */
/* forward pass: alpha_t(s) = theta_t(s) + logsumexp_a alpha_{t-1}(Pred_a(s)), stored for every t.     */

static void forward(const float* w, const float* c, int64_t n, int L, int k, double T, int has_sigma,
                    uint32_t sigma, double* alpha /* [n][S] */) {
    const uint32_t S = 1u << L, P = 1u << k, gmask = (1u << (L - k)) - 1u;
    double x[64];
    for (uint32_t s = 0; s < S; ++s) {
        double th = log_weight(w[0], c[s], T);
        /* sigma mode: s_1 must be a successor of sigma, i.e. share its top L-k bits with sigma's low ones */
        alpha[s] = (!has_sigma || (s >> k) == (sigma & gmask)) ? th : -INFINITY;
    }
    for (int64_t t = 1; t < n; ++t) {
        const double* ap = alpha + (size_t)(t - 1) * S;
        double* at = alpha + (size_t)t * S;
        for (uint32_t s = 0; s < S; ++s) {
            for (uint32_t a = 0; a < P; ++a) x[a] = ap[pred(s, a, L, k)];
            at[s] = log_weight(w[t], c[s], T) + log_sum_exp(x, (int)P);
        }
    }
}

/* beta_t(s) from beta_{t+1}: logsumexp_b [theta_{t+1}(Succ_b(s)) + beta_{t+1}(Succ_b(s))]. */
static void backward_step(const float* w, const float* c, int64_t t, int L, int k, double T,
                          const double* bnext, double* bcur) {
    const uint32_t S = 1u << L, P = 1u << k;
    double x[64];
    for (uint32_t s = 0; s < S; ++s) {
        for (uint32_t b = 0; b < P; ++b) {
            uint32_t u = succ(s, b, L, k);
            x[b] = log_weight(w[t + 1], c[u], T) + bnext[u];
        }
        bcur[s] = log_sum_exp(x, (int)P);
    }
}

static void backward_init(int L, int has_sigma, uint32_t sigma, double* b) {
    const uint32_t S = 1u << L;
    for (uint32_t s = 0; s < S; ++s) b[s] = (!has_sigma || s == sigma) ? 0.0 : -INFINITY;
}

/* ------------------------------------------------------------------------------------------------ */
/* soft codeword                                                                                     */

/*
 * For one sequence: alpha by the forward pass, beta by the backward pass, ln Z = logsumexp_s(alpha_t + beta_t)
 * (the same for every t), p_t(s) = exp(alpha_t(s) + beta_t(s) - ln Z), w_soft_t = sum_s c(s) p_t(s).
 * lnz_dev receives max_t |logsumexp_s(alpha_t + beta_t) - ln Z|, a self-check of the two passes.
 */
static void soft_one(const float* w, const float* c, int64_t n, int L, int k, double T, int has_sigma,
                     uint32_t sigma, double* w_soft, double* log_z, double* lnz_dev, double* alpha,
                     double* b0, double* b1, double* tmp) {
    const uint32_t S = 1u << L;
    forward(w, c, n, L, k, T, has_sigma, sigma, alpha);
    double* bcur = b0;
    double* bnext = b1;
    backward_init(L, has_sigma, sigma, bcur);
    const double* an = alpha + (size_t)(n - 1) * S;
    for (uint32_t s = 0; s < S; ++s) tmp[s] = an[s] + bcur[s];
    const double lnz = log_sum_exp(tmp, (int)S);
    double dev = 0.0;
    for (int64_t t = n - 1; t >= 0; --t) {
        if (t < n - 1) {
            double* sw = bcur; bcur = bnext; bnext = sw;   /* bnext now holds beta_{t+1} */
            backward_step(w, c, t, L, k, T, bnext, bcur);
        }
        const double* at = alpha + (size_t)t * S;
        for (uint32_t s = 0; s < S; ++s) tmp[s] = at[s] + bcur[s];
        double lz_t = log_sum_exp(tmp, (int)S);
        if (isfinite(lz_t) && isfinite(lnz)) {
            double e = fabs(lz_t - lnz);
            if (e > dev) dev = e;
        }
        double acc = 0.0;
        for (uint32_t s = 0; s < S; ++s) {
            if (tmp[s] == -INFINITY) continue;
            acc += (double)c[s] * exp(tmp[s] - lnz);
        }
        w_soft[t] = isfinite(lnz) ? acc : NAN;
    }
    if (log_z) *log_z = lnz;
    if (lnz_dev) *lnz_dev = dev;
}

int oracle_soft(const float* w, const float* c, int64_t B, int64_t n, int L, int k, double T,
                const int32_t* sigma, double* w_soft, double* log_z, double* lnz_dev) {
    if (check_args(B, n, L, k) != ORACLE_OK || k > 6 || !(T > 0.0) || !w || !c || !w_soft) return ORACLE_ERR_ARG;
    const size_t S = (size_t)1 << L;
    int err = ORACLE_OK;
#pragma omp parallel
    {
        double* alpha = (double*)malloc(sizeof(double) * S * (size_t)n);
        double* b0 = (double*)malloc(sizeof(double) * S);
        double* b1 = (double*)malloc(sizeof(double) * S);
        double* tmp = (double*)malloc(sizeof(double) * S);
        if (!alpha || !b0 || !b1 || !tmp) {
#pragma omp atomic write
            err = ORACLE_ERR_NOMEM;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t b = 0; b < B; ++b) {
                uint32_t sg = sigma ? ((uint32_t)sigma[b] & (uint32_t)(S - 1)) : 0u;
                soft_one(w + b * n, c, n, L, k, T, sigma != NULL, sg, w_soft + b * n,
                         log_z ? log_z + b : NULL, lnz_dev ? lnz_dev + b : NULL, alpha, b0, b1, tmp);
            }
        }
        free(alpha); free(b0); free(b1); free(tmp);
    }
    return err;
}

/* ------------------------------------------------------------------------------------------------ */
/* gradient of the soft codeword                                                                     */

/*
 * d w_soft_t / d w_u = (2/T) Cov_p(c(s_t), c(s_u)), since d(-E/T)/d w_u = -(2/T)(w_u - c(s_u)).
 * So for an upstream gradient g, grad_u = sum_t g_t dw_soft_t/dw_u = (2/T) Cov_p(c(s_u), F) with
 * F = sum_t g_t c(s_t).  Cov_p(c(s_u), F) = sum_s p_u(s) (c(s) - w_soft_u)(E[F | s_u = s] - E[F]).
 *
 * E[F | s_u = s] splits at u because the posterior is a Markov chain:
 *   ra_u(s) = E[sum_{t<=u} g_t c(s_t) | s_u = s]
 *           = g_u c(s) + sum_a P(s_{u-1} = Pred_a(s) | s_u = s) ra_{u-1}(Pred_a(s)),
 *     where P(s_{u-1} = Pred_a(s) | s_u = s) = softmax_a alpha_{u-1}(Pred_a(s));
 *   rb_u(s) = E[sum_{t>u} g_t c(s_t) | s_u = s]
 *           = sum_b P(s_{u+1} = Succ_b(s) | s_u = s) [g_{u+1} c(Succ_b(s)) + rb_{u+1}(Succ_b(s))],
 *     where P(s_{u+1} = Succ_b(s) | s_u = s) = softmax_b [theta_{u+1}(Succ_b(s)) + beta_{u+1}(Succ_b(s))].
 * States of zero posterior weight contribute nothing.
 *
 * Codebook gradient (the soft codeword is differentiable in the trellis parameters as well, gist.science Technical
 * Summary, "Core Mechanism"; the parameters of a bitshift trellis with a table codebook are the values c(s)).
 * d(-E/T)/d c(v) = (2/T) sum_u (w_u - c(v)) [s_u = v], and w_soft_t depends on c(v) directly through c(s_t) as well
 * as through the path measure, so
 *   dL/dc(v) = sum_t g_t P(s_t = v) + Cov_p(F, (2/T) sum_u (w_u - c(v)) [s_u = v])
 *            = sum_u P(s_u = v) [ g_u + (2/T) (w_u - c(v)) (E[F | s_u = v] - E[F]) ],
 * summed here per sequence (the caller adds sequences up).
 */
static void softmax_weights(const double* x, int m, double* pw) {
    double mx = -INFINITY;
    for (int i = 0; i < m; ++i)
        if (x[i] > mx) mx = x[i];
    if (mx == -INFINITY) {
        for (int i = 0; i < m; ++i) pw[i] = 0.0;
        return;
    }
    double s = 0.0;
    for (int i = 0; i < m; ++i) { pw[i] = exp(x[i] - mx); s += pw[i]; }
    for (int i = 0; i < m; ++i) pw[i] /= s;
}

static void grad_one(const float* w, const float* c, const float* g, int64_t n, int L, int k, double T,
                     int has_sigma, uint32_t sigma, double* grad, double* w_soft, double* gc, double* alpha,
                     double* ra, double* b0, double* b1, double* rb0, double* rb1, double* tmp) {
    const uint32_t S = 1u << L, P = 1u << k;
    double x[64], pw[64];
    if (gc)
        for (uint32_t s = 0; s < S; ++s) gc[s] = 0.0;
    forward(w, c, n, L, k, T, has_sigma, sigma, alpha);
    /* ra: forward expectation pass */
    for (uint32_t s = 0; s < S; ++s) ra[s] = (double)g[0] * (double)c[s];
    for (int64_t t = 1; t < n; ++t) {
        const double* ap = alpha + (size_t)(t - 1) * S;
        const double* rp = ra + (size_t)(t - 1) * S;
        double* rt = ra + (size_t)t * S;
        for (uint32_t s = 0; s < S; ++s) {
            for (uint32_t a = 0; a < P; ++a) x[a] = ap[pred(s, a, L, k)];
            softmax_weights(x, (int)P, pw);
            double acc = 0.0;
            for (uint32_t a = 0; a < P; ++a)
                if (pw[a] != 0.0) acc += pw[a] * rp[pred(s, a, L, k)];
            rt[s] = (double)g[t] * (double)c[s] + acc;
        }
    }
    /* ln Z */
    double *bcur = b0, *bnext = b1, *rbcur = rb0, *rbnext = rb1;
    backward_init(L, has_sigma, sigma, bcur);
    for (uint32_t s = 0; s < S; ++s) rbcur[s] = 0.0;
    const double* an = alpha + (size_t)(n - 1) * S;
    for (uint32_t s = 0; s < S; ++s) tmp[s] = an[s] + bcur[s];
    const double lnz = log_sum_exp(tmp, (int)S);
    for (int64_t t = n - 1; t >= 0; --t) {
        if (t < n - 1) {
            double* sw = bcur; bcur = bnext; bnext = sw;
            sw = rbcur; rbcur = rbnext; rbnext = sw;
            backward_step(w, c, t, L, k, T, bnext, bcur);
            for (uint32_t s = 0; s < S; ++s) {
                for (uint32_t b = 0; b < P; ++b) {
                    uint32_t u = succ(s, b, L, k);
                    x[b] = log_weight(w[t + 1], c[u], T) + bnext[u];
                }
                softmax_weights(x, (int)P, pw);
                double acc = 0.0;
                for (uint32_t b = 0; b < P; ++b) {
                    if (pw[b] == 0.0) continue;
                    uint32_t u = succ(s, b, L, k);
                    acc += pw[b] * ((double)g[t + 1] * (double)c[u] + rbnext[u]);
                }
                rbcur[s] = acc;
            }
        }
        /* posterior at step t, mean codeword and mean of E[F | s_t] */
        const double* at = alpha + (size_t)t * S;
        const double* rt = ra + (size_t)t * S;
        double m0 = 0.0, mr = 0.0;
        for (uint32_t s = 0; s < S; ++s) {
            double lp = at[s] + bcur[s];
            tmp[s] = (lp == -INFINITY) ? 0.0 : exp(lp - lnz);
            if (tmp[s] != 0.0) {
                m0 += tmp[s] * (double)c[s];
                mr += tmp[s] * (rt[s] + rbcur[s]);
            }
        }
        /* centred two-pass covariance */
        double cov = 0.0;
        for (uint32_t s = 0; s < S; ++s)
            if (tmp[s] != 0.0) cov += tmp[s] * ((double)c[s] - m0) * (rt[s] + rbcur[s] - mr);
        if (gc && isfinite(lnz))
            for (uint32_t s = 0; s < S; ++s)
                if (tmp[s] != 0.0)
                    gc[s] += tmp[s] * ((double)g[t] + (2.0 / T) * ((double)w[t] - (double)c[s]) * (rt[s] + rbcur[s] - mr));
        if (isfinite(lnz)) {
            grad[t] = (2.0 / T) * cov;
            if (w_soft) w_soft[t] = m0;
        } else {
            grad[t] = NAN;
            if (w_soft) w_soft[t] = NAN;
        }
    }
    if (gc && !isfinite(lnz))   /* no path satisfies the boundary: the loss, hence its gradient, is undefined */
        for (uint32_t s = 0; s < S; ++s) gc[s] = NAN;
}

static int grad_all(const float* w, const float* c, const float* g, int64_t B, int64_t n, int L, int k, double T,
                    const int32_t* sigma, double* grad, double* w_soft, double* gc) {
    if (check_args(B, n, L, k) != ORACLE_OK || k > 6 || !(T > 0.0) || !w || !c || !g || !grad)
        return ORACLE_ERR_ARG;
    const size_t S = (size_t)1 << L;
    int err = ORACLE_OK;
#pragma omp parallel
    {
        double* alpha = (double*)malloc(sizeof(double) * S * (size_t)n);
        double* ra = (double*)malloc(sizeof(double) * S * (size_t)n);
        double* b0 = (double*)malloc(sizeof(double) * S);
        double* b1 = (double*)malloc(sizeof(double) * S);
        double* rb0 = (double*)malloc(sizeof(double) * S);
        double* rb1 = (double*)malloc(sizeof(double) * S);
        double* tmp = (double*)malloc(sizeof(double) * S);
        if (!alpha || !ra || !b0 || !b1 || !rb0 || !rb1 || !tmp) {
#pragma omp atomic write
            err = ORACLE_ERR_NOMEM;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t b = 0; b < B; ++b) {
                uint32_t sg = sigma ? ((uint32_t)sigma[b] & (uint32_t)(S - 1)) : 0u;
                grad_one(w + b * n, c, g + b * n, n, L, k, T, sigma != NULL, sg, grad + b * n,
                         w_soft ? w_soft + b * n : NULL, gc ? gc + (size_t)b * S : NULL, alpha, ra, b0, b1, rb0,
                         rb1, tmp);
            }
        }
        free(alpha); free(ra); free(b0); free(b1); free(rb0); free(rb1); free(tmp);
    }
    return err;
}

/* grad [B, n]: dL/dw for upstream g = dL/dw_soft; w_soft [B, n] optional. */
int oracle_grad(const float* w, const float* c, const float* g, int64_t B, int64_t n, int L, int k, double T,
                const int32_t* sigma, double* grad, double* w_soft) {
    return grad_all(w, c, g, B, n, L, k, T, sigma, grad, w_soft, NULL);
}

/* The same, plus gc [B, 2^L]: dL/dc of each sequence on its own (NaN for a sequence with no admissible path). */
int oracle_grad_codebook(const float* w, const float* c, const float* g, int64_t B, int64_t n, int L, int k,
                         double T, const int32_t* sigma, double* grad, double* w_soft, double* gc) {
    if (!gc) return ORACLE_ERR_ARG;
    return grad_all(w, c, g, B, n, L, k, T, sigma, grad, w_soft, gc);
}

/* ------------------------------------------------------------------------------------------------ */
/* Viterbi hard code (the T -> 0 limit), IEEE float32 with a fixed operation order                  */

/*
 * M_1(s) = fl(d*d) with d = fl(w_1 - c(s));   M_t(s) = fl(fl(d*d) + min_a M_{t-1}(Pred_a(s))).
 * The back pointer of s at step t is the smallest a attaining the min (scan a = 0, 1, ... with a strict <),
 * the end state is the smallest s attaining min_s M_n(s) (sigma mode: s_n = sigma), and the path is traced
 * back through the back pointers.  cost = M_n(s_n).  No normalisation and no fused multiply-add.
 */
static void viterbi_one(const float* w, const float* c, int64_t n, int L, int k, int has_sigma, uint32_t sigma,
                        int32_t* states, float* w_hard, float* cost, float* m0, float* m1, uint8_t* bp) {
    const uint32_t S = 1u << L, P = 1u << k, gmask = (1u << (L - k)) - 1u;
    float* mcur = m0;
    float* mprev = m1;
    for (uint32_t s = 0; s < S; ++s) {
        float d = w[0] - c[s];
        float e = d * d;
        mcur[s] = (!has_sigma || (s >> k) == (sigma & gmask)) ? e : INFINITY;
    }
    for (int64_t t = 1; t < n; ++t) {
        float* sw = mcur; mcur = mprev; mprev = sw;
        uint8_t* bpt = bp + (size_t)t * S;
        for (uint32_t s = 0; s < S; ++s) {
            float best = mprev[pred(s, 0, L, k)];
            uint32_t arg = 0;
            for (uint32_t a = 1; a < P; ++a) {
                float v = mprev[pred(s, a, L, k)];
                if (v < best) { best = v; arg = a; }
            }
            float d = w[t] - c[s];
            float e = d * d;
            mcur[s] = e + best;
            bpt[s] = (uint8_t)arg;
        }
    }
    uint32_t s_end;
    if (has_sigma) {
        s_end = sigma;
    } else {
        s_end = 0;
        for (uint32_t s = 1; s < S; ++s)
            if (mcur[s] < mcur[s_end]) s_end = s;
    }
    if (cost) *cost = mcur[s_end];
    uint32_t s = s_end;
    for (int64_t t = n - 1; t >= 0; --t) {
        states[t] = (int32_t)s;
        if (w_hard) w_hard[t] = c[s];
        if (t > 0) s = pred(s, bp[(size_t)t * S + s], L, k);
    }
}

int oracle_viterbi(const float* w, const float* c, int64_t B, int64_t n, int L, int k, const int32_t* sigma,
                   int32_t* states, float* w_hard, float* cost) {
    if (check_args(B, n, L, k) != ORACLE_OK || k > 8 || !w || !c || !states) return ORACLE_ERR_ARG;
    const size_t S = (size_t)1 << L;
    int err = ORACLE_OK;
#pragma omp parallel
    {
        float* m0 = (float*)malloc(sizeof(float) * S);
        float* m1 = (float*)malloc(sizeof(float) * S);
        uint8_t* bp = (uint8_t*)malloc(S * (size_t)n);
        if (!m0 || !m1 || !bp) {
#pragma omp atomic write
            err = ORACLE_ERR_NOMEM;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t b = 0; b < B; ++b) {
                uint32_t sg = sigma ? ((uint32_t)sigma[b] & (uint32_t)(S - 1)) : 0u;
                viterbi_one(w + b * n, c, n, L, k, sigma != NULL, sg, states + b * n,
                            w_hard ? w_hard + b * n : NULL, cost ? cost + b : NULL, m0, m1, bp);
            }
        }
        free(m0); free(m1); free(bp);
    }
    return err;
}

/* Number of OpenMP threads a parallel region of this library uses (reported next to oracle timings). */
int oracle_num_threads(void) {
    int nt = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            nt = omp_get_num_threads();
#endif
        }
    }
    return nt;
}
