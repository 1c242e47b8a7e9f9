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
 *   - V weights per step: each state emits a V-vector c(s) = (c(s, 0), .., c(s, V-1)), a sequence of n steps holds
 *     n V weights (step t owns w[t V .. t V + V - 1]), and c is stored [2^L][V].  V = 1 is the scalar trellis.
 *   - path energy E = sum_t |w_t - c(s_t)|^2 (squared Euclidean distance over the V components), path weight
 *     exp(-E / T); transitions carry no cost.
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

/* theta_t(s) = -|w_t - c(s)|^2 / T : the log Boltzmann weight of emitting c(s) at step t (V components). */
static inline double log_weight(const float* wt, const float* cs, int V, double T) {
    double e = 0.0;
    for (int v = 0; v < V; ++v) {
        double d = (double)wt[v] - (double)cs[v];
        e += d * d;
    }
    return -e / T;
}

/* <g_t, c(s)> over the V components */
static inline double dot_v(const float* gt, const float* cs, int V) {
    double e = 0.0;
    for (int v = 0; v < V; ++v) e += (double)gt[v] * (double)cs[v];
    return e;
}

static int check_args(int64_t B, int64_t n, int L, int k, int V) {
    if (B < 0 || n < 1 || k < 1 || L <= k || L > 24 || V < 1 || V > 16) return ORACLE_ERR_ARG;
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------------------------------ */
/* forward pass: alpha_t(s) = theta_t(s) + logsumexp_a alpha_{t-1}(Pred_a(s)), stored for every t.     */

static void forward(const float* w, const float* c, int64_t n, int L, int k, int V, double T, int has_sigma,
                    uint32_t sigma, double* alpha /* [n][S] */) {
    const uint32_t S = 1u << L, P = 1u << k, gmask = (1u << (L - k)) - 1u;
    double x[64];
    for (uint32_t s = 0; s < S; ++s) {
        double th = log_weight(w, c + (size_t)s * V, V, T);
        /* sigma mode: s_1 must be a successor of sigma, i.e. share its top L-k bits with sigma's low ones */
        alpha[s] = (!has_sigma || (s >> k) == (sigma & gmask)) ? th : -INFINITY;
    }
    for (int64_t t = 1; t < n; ++t) {
        const double* ap = alpha + (size_t)(t - 1) * S;
        double* at = alpha + (size_t)t * S;
        for (uint32_t s = 0; s < S; ++s) {
            for (uint32_t a = 0; a < P; ++a) x[a] = ap[pred(s, a, L, k)];
            at[s] = log_weight(w + t * V, c + (size_t)s * V, V, T) + log_sum_exp(x, (int)P);
        }
    }
}

/* beta_t(s) from beta_{t+1}: logsumexp_b [theta_{t+1}(Succ_b(s)) + beta_{t+1}(Succ_b(s))]. */
static void backward_step(const float* w, const float* c, int64_t t, int L, int k, int V, double T,
                          const double* bnext, double* bcur) {
    const uint32_t S = 1u << L, P = 1u << k;
    double x[64];
    for (uint32_t s = 0; s < S; ++s) {
        for (uint32_t b = 0; b < P; ++b) {
            uint32_t u = succ(s, b, L, k);
            x[b] = log_weight(w + (t + 1) * V, c + (size_t)u * V, V, T) + bnext[u];
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
 * (the same for every t), p_t(s) = exp(alpha_t(s) + beta_t(s) - ln Z), w_soft_t = sum_s c(s) p_t(s) (per component).
 * lnz_dev receives max_t |logsumexp_s(alpha_t + beta_t) - ln Z|, a self-check of the two passes.
 */
static void soft_one(const float* w, const float* c, int64_t n, int L, int k, int V, double T, int has_sigma,
                     uint32_t sigma, double* w_soft, double* log_z, double* lnz_dev, double* alpha,
                     double* b0, double* b1, double* tmp) {
    const uint32_t S = 1u << L;
    forward(w, c, n, L, k, V, T, has_sigma, sigma, alpha);
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
            backward_step(w, c, t, L, k, V, T, bnext, bcur);
        }
        const double* at = alpha + (size_t)t * S;
        for (uint32_t s = 0; s < S; ++s) tmp[s] = at[s] + bcur[s];
        double lz_t = log_sum_exp(tmp, (int)S);
        if (isfinite(lz_t) && isfinite(lnz)) {
            double e = fabs(lz_t - lnz);
            if (e > dev) dev = e;
        }
        for (int v = 0; v < V; ++v) {
            double acc = 0.0;
            for (uint32_t s = 0; s < S; ++s) {
                if (tmp[s] == -INFINITY) continue;
                acc += (double)c[(size_t)s * V + v] * exp(tmp[s] - lnz);
            }
            w_soft[t * V + v] = isfinite(lnz) ? acc : NAN;
        }
    }
    if (log_z) *log_z = lnz;
    if (lnz_dev) *lnz_dev = dev;
}

/* w [B, n V], c [2^L, V], w_soft [B, n V], log_z [B] and lnz_dev [B] optional; n counts trellis steps. */
int oracle_soft(const float* w, const float* c, int64_t B, int64_t n, int L, int k, int V, double T,
                const int32_t* sigma, double* w_soft, double* log_z, double* lnz_dev) {
    if (check_args(B, n, L, k, V) != ORACLE_OK || k > 6 || !(T > 0.0) || !w || !c || !w_soft) return ORACLE_ERR_ARG;
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
                soft_one(w + b * n * V, c, n, L, k, V, T, sigma != NULL, sg, w_soft + b * n * V,
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
 * With V components per step the same holds per component: d w_soft_{t,v} / d w_{u,v'} =
 * (2/T) Cov_p(c(s_t, v), c(s_u, v')), F = sum_t <g_t, c(s_t)>, and grad_{u,v} = (2/T) Cov_p(c(s_u, v), F).
 *
 * E[F | s_u = s] splits at u because the posterior is a Markov chain:
 *   ra_u(s) = E[sum_{t<=u} <g_t, c(s_t)> | s_u = s]
 *           = <g_u, c(s)> + sum_a P(s_{u-1} = Pred_a(s) | s_u = s) ra_{u-1}(Pred_a(s)),
 *     where P(s_{u-1} = Pred_a(s) | s_u = s) = softmax_a alpha_{u-1}(Pred_a(s));
 *   rb_u(s) = E[sum_{t>u} <g_t, c(s_t)> | s_u = s]
 *           = sum_b P(s_{u+1} = Succ_b(s) | s_u = s) [<g_{u+1}, c(Succ_b(s))> + rb_{u+1}(Succ_b(s))],
 *     where P(s_{u+1} = Succ_b(s) | s_u = s) = softmax_b [theta_{u+1}(Succ_b(s)) + beta_{u+1}(Succ_b(s))].
 * States of zero posterior weight contribute nothing.
 *
 * Codebook gradient (the soft codeword is differentiable in the trellis parameters as well, gist.science Technical
 * Summary, "Core Mechanism"; the parameters of a bitshift trellis with a table codebook are the values c(s)).
 * d(-E/T)/d c(v) = (2/T) sum_u (w_u - c(v)) [s_u = v], and w_soft_t depends on c(v) directly through c(s_t) as well
 * as through the path measure, so
 *   dL/dc(v) = sum_t g_t P(s_t = v) + Cov_p(F, (2/T) sum_u (w_u - c(v)) [s_u = v])
 *            = sum_u P(s_u = v) [ g_u + (2/T) (w_u - c(v)) (E[F | s_u = v] - E[F]) ],
 * summed here per sequence (the caller adds sequences up); with V components, per component of c(v), g_u and w_u.
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

static void grad_one(const float* w, const float* c, const float* g, int64_t n, int L, int k, int V, double T,
                     int has_sigma, uint32_t sigma, double* grad, double* w_soft, double* gc, double* alpha,
                     double* ra, double* b0, double* b1, double* rb0, double* rb1, double* tmp) {
    const uint32_t S = 1u << L, P = 1u << k;
    double x[64], pw[64], m0[16], cov[16];
    if (gc)
        for (size_t i = 0; i < (size_t)S * V; ++i) gc[i] = 0.0;
    forward(w, c, n, L, k, V, T, has_sigma, sigma, alpha);
    /* ra: forward expectation pass */
    for (uint32_t s = 0; s < S; ++s) ra[s] = dot_v(g, c + (size_t)s * V, V);
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
            rt[s] = dot_v(g + t * V, c + (size_t)s * V, V) + acc;
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
            backward_step(w, c, t, L, k, V, T, bnext, bcur);
            for (uint32_t s = 0; s < S; ++s) {
                for (uint32_t b = 0; b < P; ++b) {
                    uint32_t u = succ(s, b, L, k);
                    x[b] = log_weight(w + (t + 1) * V, c + (size_t)u * V, V, T) + bnext[u];
                }
                softmax_weights(x, (int)P, pw);
                double acc = 0.0;
                for (uint32_t b = 0; b < P; ++b) {
                    if (pw[b] == 0.0) continue;
                    uint32_t u = succ(s, b, L, k);
                    acc += pw[b] * (dot_v(g + (t + 1) * V, c + (size_t)u * V, V) + rbnext[u]);
                }
                rbcur[s] = acc;
            }
        }
        /* posterior at step t, mean codeword and mean of E[F | s_t] */
        const double* at = alpha + (size_t)t * S;
        const double* rt = ra + (size_t)t * S;
        double mr = 0.0;
        for (int v = 0; v < V; ++v) m0[v] = 0.0;
        for (uint32_t s = 0; s < S; ++s) {
            double lp = at[s] + bcur[s];
            tmp[s] = (lp == -INFINITY) ? 0.0 : exp(lp - lnz);
            if (tmp[s] != 0.0) {
                for (int v = 0; v < V; ++v) m0[v] += tmp[s] * (double)c[(size_t)s * V + v];
                mr += tmp[s] * (rt[s] + rbcur[s]);
            }
        }
        /* centred two-pass covariance, per component */
        for (int v = 0; v < V; ++v) {
            cov[v] = 0.0;
            for (uint32_t s = 0; s < S; ++s)
                if (tmp[s] != 0.0) cov[v] += tmp[s] * ((double)c[(size_t)s * V + v] - m0[v]) * (rt[s] + rbcur[s] - mr);
        }
        if (gc && isfinite(lnz))
            for (uint32_t s = 0; s < S; ++s)
                if (tmp[s] != 0.0)
                    for (int v = 0; v < V; ++v) {
                        const double wv = (double)w[t * V + v], cv = (double)c[(size_t)s * V + v];
                        gc[(size_t)s * V + v] += tmp[s] * ((double)g[t * V + v] + (2.0 / T) * (wv - cv) * (rt[s] + rbcur[s] - mr));
                    }
        for (int v = 0; v < V; ++v) {
            if (isfinite(lnz)) {
                grad[t * V + v] = (2.0 / T) * cov[v];
                if (w_soft) w_soft[t * V + v] = m0[v];
            } else {
                grad[t * V + v] = NAN;
                if (w_soft) w_soft[t * V + v] = NAN;
            }
        }
    }
    if (gc && !isfinite(lnz))   /* no path satisfies the boundary: the loss, hence its gradient, is undefined */
        for (size_t i = 0; i < (size_t)S * V; ++i) gc[i] = NAN;
}

static int grad_all(const float* w, const float* c, const float* g, int64_t B, int64_t n, int L, int k, int V,
                    double T, const int32_t* sigma, double* grad, double* w_soft, double* gc) {
    if (check_args(B, n, L, k, V) != ORACLE_OK || k > 6 || !(T > 0.0) || !w || !c || !g || !grad)
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
                grad_one(w + b * n * V, c, g + b * n * V, n, L, k, V, T, sigma != NULL, sg, grad + b * n * V,
                         w_soft ? w_soft + b * n * V : NULL, gc ? gc + (size_t)b * S * V : NULL, alpha, ra, b0, b1,
                         rb0, rb1, tmp);
            }
        }
        free(alpha); free(ra); free(b0); free(b1); free(rb0); free(rb1); free(tmp);
    }
    return err;
}

/* grad [B, n V]: dL/dw for upstream g = dL/dw_soft [B, n V]; w_soft [B, n V] optional. */
int oracle_grad(const float* w, const float* c, const float* g, int64_t B, int64_t n, int L, int k, int V, double T,
                const int32_t* sigma, double* grad, double* w_soft) {
    return grad_all(w, c, g, B, n, L, k, V, T, sigma, grad, w_soft, NULL);
}

/* The same, plus gc [B, 2^L, V]: dL/dc of each sequence on its own (NaN for a sequence with no admissible path). */
int oracle_grad_codebook(const float* w, const float* c, const float* g, int64_t B, int64_t n, int L, int k, int V,
                         double T, const int32_t* sigma, double* grad, double* w_soft, double* gc) {
    if (!gc) return ORACLE_ERR_ARG;
    return grad_all(w, c, g, B, n, L, k, V, T, sigma, grad, w_soft, gc);
}

/* ------------------------------------------------------------------------------------------------ */
/* Viterbi hard code (the T -> 0 limit), IEEE float32 with a fixed operation order                  */

/*
 * M_1(s) = e_1(s);   M_t(s) = fl(e_t(s) + min_a M_{t-1}(Pred_a(s))),  where e_t(s) = fl(d_0 * d_0) with
 * d_v = fl(w_{t,v} - c(s, v)), and for V > 1 the components are added in order, e = fl(e + fl(d_v * d_v)).
 * The back pointer of s at step t is the smallest a attaining the min (scan a = 0, 1, ... with a strict <),
 * the end state is the smallest s attaining min_s M_n(s) (sigma mode: s_n = sigma), and the path is traced
 * back through the back pointers.  cost = M_n(s_n).  No normalisation and no fused multiply-add.
 */
/* fl32 squared distance |w_t - c(s)|^2, components added in index order */
static inline float sq_dist32(const float* wt, const float* cs, int V) {
    float d = wt[0] - cs[0];
    float e = d * d;
    for (int v = 1; v < V; ++v) {
        float dv = wt[v] - cs[v];
        float ev = dv * dv;
        e = e + ev;
    }
    return e;
}

static void viterbi_one(const float* w, const float* c, int64_t n, int L, int k, int V, int has_sigma,
                        uint32_t sigma, int32_t* states, float* w_hard, float* cost, float* m0, float* m1,
                        uint8_t* bp) {
    const uint32_t S = 1u << L, P = 1u << k, gmask = (1u << (L - k)) - 1u;
    float* mcur = m0;
    float* mprev = m1;
    for (uint32_t s = 0; s < S; ++s) {
        float e = sq_dist32(w, c + (size_t)s * V, V);
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
            float e = sq_dist32(w + t * V, c + (size_t)s * V, V);
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
        if (w_hard)
            for (int v = 0; v < V; ++v) w_hard[t * V + v] = c[(size_t)s * V + v];
        if (t > 0) s = pred(s, bp[(size_t)t * S + s], L, k);
    }
}

/* states [B, n] (one per step), w_hard [B, n V] optional, cost [B] optional. */
int oracle_viterbi(const float* w, const float* c, int64_t B, int64_t n, int L, int k, int V, const int32_t* sigma,
                   int32_t* states, float* w_hard, float* cost) {
    if (check_args(B, n, L, k, V) != ORACLE_OK || k > 8 || !w || !c || !states) return ORACLE_ERR_ARG;
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
                viterbi_one(w + b * n * V, c, n, L, k, V, sigma != NULL, sg, states + b * n,
                            w_hard ? w_hard + b * n * V : NULL, cost ? cost + b : NULL, m0, m1, bp);
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
