/*
 * gn_oracle.c -- plain fp64 CPU reference of GroupNorm forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no code, header, table or
 * helper with the HIP path.
 *
 * What it computes (the plain definition, written out with no blocking,
 * fusion or reordering):
 *
 *   A tensor of N samples, C channels and HW spatial positions is split into
 *   G groups of D = C/G consecutive channels.  A "slice" is one (n, g) pair;
 *   it holds M = D*HW elements.
 *
 *   Forward, per slice (POPCORNBENCH GroupNorm trace, page 2: mean and the
 *   biased variance -- denominator (C/G)*H*W -- over the group's channels and
 *   spatial positions, then (x - mean)/sqrt(var + eps), then the per-channel
 *   weight and bias):
 *       mu   = (1/M) * sum x
 *       var  = (1/M) * sum (x - mu)^2          (two passes over the slice)
 *       r    = 1 / sqrt(var + eps)
 *       xhat = (x - mu) * r
 *       y    = gamma_c * xhat + beta_c
 *   The saved statistics are mu and r per slice, stored at index n*G + g
 *   (baracuda-kernels group_norm_backward.rs, GroupNormBackwardArgs: saved
 *   per-(N, group) mean and inv_std).
 *
 *   Backward (the three stages of the baracuda-kernels GroupNorm backward
 *   plan, module header: a per-group reduction, the per-cell dx, the
 *   per-channel dgamma/dbeta), with mu and r recomputed here in fp64 from x,
 *   as the fp64 autograd reference of the apex PR #2018 reproducer does:
 *       dbeta_c  = sum over n, p of dy
 *       dgamma_c = sum over n, p of dy * xhat
 *       per slice:  A = sum gamma_c * dy,   B = sum gamma_c * dy * xhat
 *       dx = r * (gamma_c * dy - A/M - xhat * B/M)
 *   The dx formula is the derivative of sum(y * dy) with respect to x for the
 *   forward above; it is pinned by central finite differences in the tests.
 *
 *   With no affine parameters (gamma == NULL) gamma is 1 and beta is 0.
 *
 * Layouts (element (n, c, p) with p the flattened spatial index):
 *   NCHW (layout 0): offset ((n*C + c)*HW + p)
 *   NHWC (layout 1): offset ((n*HW + p)*C + c)   -- channels_last
 *
 * All arithmetic is fp64; the inputs are the fp64 images of the exact
 * (already quantised) values the device receives.  OpenMP splits the work
 * over independent slices or channels only, so every sum is taken in the
 * order written here whatever the thread count.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define GNO_NCHW 0
#define GNO_NHWC 1

#ifdef GNO_MUTANTS
/* Planted-mistake switch, compiled only into the separate mutant build that
 * the oracle's own tests use to show that the pins catch such mistakes. */
int gno_mutation = 0;
#define MUT(k) (gno_mutation == (k))
#else
#define MUT(k) 0
#endif

static inline size_t off(int layout, int64_t N, int64_t C, int64_t HW,
                         int64_t n, int64_t c, int64_t p) {
    (void)N;
    if (layout == GNO_NCHW) return (size_t)((n * C + c) * HW + p);
    return (size_t)((n * HW + p) * C + c);
}

/* mean and 1/sqrt(var + eps) of one slice, two passes (definition). */
static void slice_stats(int layout, int64_t N, int64_t C, int64_t HW, int64_t G,
                        const double* x, int64_t n, int64_t g, double eps,
                        double* mu_out, double* r_out) {
    const int64_t D = C / G;
    const double M = (double)(D * HW);
    double s = 0.0;
    for (int64_t c = g * D; c < (g + 1) * D; ++c)
        for (int64_t p = 0; p < HW; ++p) s += x[off(layout, N, C, HW, n, c, p)];
    const double mu = s / M;
    double ss = 0.0;
    for (int64_t c = g * D; c < (g + 1) * D; ++c)
        for (int64_t p = 0; p < HW; ++p) {
            const double d = x[off(layout, N, C, HW, n, c, p)] - mu;
            ss += d * d;
        }
    double var = MUT(1) ? ss / (M - 1.0) : ss / M; /* mutant 1: unbiased */
    if (MUT(2)) var = ss / M - mu * mu;             /* mutant 2: wrong moment */
    *mu_out = mu;
    *r_out = MUT(3) ? 1.0 / sqrt(var) + 0.0 * eps : 1.0 / sqrt(var + eps); /* mutant 3: eps dropped */
}

static int check_args(int64_t N, int64_t C, int64_t HW, int64_t G, int layout) {
    if (N < 0 || C < 0 || HW < 0 || G <= 0) return 1;
    if (C % G != 0) return 1;
    if (layout != GNO_NCHW && layout != GNO_NHWC) return 1;
    return 0;
}

/*
 * Forward.  x: [N*C*HW] in `layout`.  gamma, beta: [C] or both NULL.
 * y: same shape as x, or NULL to skip the output.  mean, rstd: [N*G].
 * Returns 0 on success, 1 on an invalid argument.
 */
int gno_forward(int64_t N, int64_t C, int64_t HW, int64_t G, int layout,
                const double* x, const double* gamma, const double* beta,
                double eps, double* y, double* mean, double* rstd) {
    if (check_args(N, C, HW, G, layout)) return 1;
    if ((gamma == NULL) != (beta == NULL)) return 1;
    const int64_t D = C / G;
    const int64_t S = N * G;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t s = 0; s < S; ++s) {
        const int64_t n = s / G, g = s % G;
        double mu, r;
        slice_stats(layout, N, C, HW, G, x, n, g, eps, &mu, &r);
        mean[s] = mu;
        rstd[s] = r;
        if (y == NULL) continue;
        for (int64_t c = g * D; c < (g + 1) * D; ++c) {
            const double ga = gamma ? gamma[c] : 1.0;
            const double be = beta ? beta[c] : 0.0;
            for (int64_t p = 0; p < HW; ++p) {
                const size_t o = off(layout, N, C, HW, n, c, p);
                const double xhat = (x[o] - mu) * r;
                y[o] = MUT(4) ? ga * xhat : ga * xhat + be; /* mutant 4: beta dropped */
            }
        }
    }
    return 0;
}

/*
 * Backward.  dy, x: [N*C*HW] in `layout`.  gamma: [C] or NULL (= 1).
 * dx (same shape), dgamma [C], dbeta [C]: each may be NULL to skip it.
 * mean, rstd: optional [N*G] outputs of the fp64 statistics used (may be NULL).
 * Scratch of 2*N*G doubles is taken from `work` (caller-owned, may be NULL
 * only if dx is NULL).
 */
int gno_backward(int64_t N, int64_t C, int64_t HW, int64_t G, int layout,
                 const double* dy, const double* x, const double* gamma,
                 double eps, double* dx, double* dgamma, double* dbeta,
                 double* mean, double* rstd, double* work) {
    if (check_args(N, C, HW, G, layout)) return 1;
    if (dx != NULL && work == NULL) return 1;
    const int64_t D = C / G;
    const int64_t S = N * G;
    const double M = (double)(D * HW);
    double* mu_all = work;            /* [S] */
    double* r_all = work ? work + S : NULL;

    /* statistics and the per-slice reductions A, B, then dx */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t s = 0; s < S; ++s) {
        const int64_t n = s / G, g = s % G;
        double mu, r;
        slice_stats(layout, N, C, HW, G, x, n, g, eps, &mu, &r);
        if (mean) mean[s] = mu;
        if (rstd) rstd[s] = r;
        if (mu_all) { mu_all[s] = mu; r_all[s] = r; }
        if (dx == NULL) continue;
        double A = 0.0, B = 0.0;
        for (int64_t c = g * D; c < (g + 1) * D; ++c) {
            const double ga = gamma ? gamma[c] : 1.0;
            for (int64_t p = 0; p < HW; ++p) {
                const size_t o = off(layout, N, C, HW, n, c, p);
                const double xhat = (x[o] - mu) * r;
                A += ga * dy[o];
                B += ga * dy[o] * xhat;
            }
        }
        for (int64_t c = g * D; c < (g + 1) * D; ++c) {
            const double ga = gamma ? gamma[c] : 1.0;
            for (int64_t p = 0; p < HW; ++p) {
                const size_t o = off(layout, N, C, HW, n, c, p);
                const double xhat = (x[o] - mu) * r;
                double v;
                if (MUT(5)) v = r * (ga * dy[o] - A / M);                /* mutant 5: B term dropped */
                else if (MUT(6)) v = r * (ga * dy[o] - A / M + xhat * B / M); /* mutant 6: sign */
                else v = r * (ga * dy[o] - A / M - xhat * B / M);
                dx[o] = v;
            }
        }
    }

    /* per-channel parameter gradients: sum over n, then p */
    if (dgamma != NULL || dbeta != NULL) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t c = 0; c < C; ++c) {
            const int64_t g = c / D;
            double sb = 0.0, sg = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double mu, r;
                if (mu_all) { mu = mu_all[n * G + g]; r = r_all[n * G + g]; }
                else slice_stats(layout, N, C, HW, G, x, n, g, eps, &mu, &r);
                for (int64_t p = 0; p < HW; ++p) {
                    const size_t o = off(layout, N, C, HW, n, c, p);
                    const double xhat = (x[o] - mu) * r;
                    sb += dy[o];
                    sg += MUT(7) ? dy[o] * x[o] : dy[o] * xhat; /* mutant 7: raw x */
                }
            }
            if (dbeta) dbeta[c] = sb;
            if (dgamma) dgamma[c] = sg;
        }
    }
    return 0;
}

/*
 * RMSNorm over rows.  ROCm/pytorch PR #3564 benchmarks an rms_norm operator
 * next to layer_norm (its summary table) and checks its gamma backward and
 * autograd against a CPU reference (its test list), but prints no formula.
 * Reading: PyTorch's rms_norm -- the root mean square over the normalised
 * (last) dimension, no mean subtracted, a weight and no bias.  Rows are the
 * D = C/G consecutive channels (n, g) of an [N, C] tensor (G = 1: one row per
 * sample, as in that table):
 *     r    = 1 / sqrt((1/D) * sum x^2 + eps)
 *     xhat = x * r
 *     y    = gamma_c * xhat
 * backward (the derivative of sum(y * dy) with respect to x and gamma):
 *     per row: B = sum gamma_c * dy * xhat
 *     dx = r * (gamma_c * dy - xhat * B/D)
 *     dgamma_c = sum over n of dy * xhat
 * rstd holds r per row at index n*G + g.  gamma may be NULL (= 1).
 */
static double rms_row_r(int64_t C, int64_t G, const double* x, int64_t n, int64_t g, double eps) {
    const int64_t D = C / G;
    double ss = 0.0;
    if (MUT(8)) { /* mutant 8: mean subtracted (a LayerNorm variance) */
        double s = 0.0;
        for (int64_t c = g * D; c < (g + 1) * D; ++c) s += x[n * C + c];
        const double mu = s / (double)D;
        for (int64_t c = g * D; c < (g + 1) * D; ++c) ss += (x[n * C + c] - mu) * (x[n * C + c] - mu);
    } else {
        for (int64_t c = g * D; c < (g + 1) * D; ++c) ss += x[n * C + c] * x[n * C + c];
    }
    const double ms = ss / (double)D;
    return MUT(9) ? 1.0 / sqrt(ms) + 0.0 * eps : 1.0 / sqrt(ms + eps); /* mutant 9: eps dropped */
}

int gno_rms_forward(int64_t N, int64_t C, int64_t G, const double* x, const double* gamma, double eps,
                    double* y, double* rstd) {
    if (N < 0 || C < 0 || G <= 0 || C % G != 0) return 1;
    const int64_t D = C / G;
    const int64_t S = N * G;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t s = 0; s < S; ++s) {
        const int64_t n = s / G, g = s % G;
        const double r = rms_row_r(C, G, x, n, g, eps);
        rstd[s] = r;
        if (y == NULL) continue;
        for (int64_t c = g * D; c < (g + 1) * D; ++c)
            y[n * C + c] = (gamma ? gamma[c] : 1.0) * (x[n * C + c] * r);
    }
    return 0;
}

/* rstd: [N*G], required (the per-row r, computed once and reused by the
 * dgamma sums). */
int gno_rms_backward(int64_t N, int64_t C, int64_t G, const double* dy, const double* x, const double* gamma,
                     double eps, double* dx, double* dgamma, double* rstd) {
    if (N < 0 || C < 0 || G <= 0 || C % G != 0 || rstd == NULL) return 1;
    const int64_t D = C / G;
    const int64_t S = N * G;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t s = 0; s < S; ++s) {
        const int64_t n = s / G, g = s % G;
        const double r = rms_row_r(C, G, x, n, g, eps);
        rstd[s] = r;
        if (dx == NULL) continue;
        double B = 0.0;
        for (int64_t c = g * D; c < (g + 1) * D; ++c)
            B += (gamma ? gamma[c] : 1.0) * dy[n * C + c] * (x[n * C + c] * r);
        for (int64_t c = g * D; c < (g + 1) * D; ++c) {
            const double ga = gamma ? gamma[c] : 1.0;
            const double xhat = x[n * C + c] * r;
            dx[n * C + c] = MUT(10) ? r * ga * dy[n * C + c]                       /* mutant 10: B term dropped */
                                    : r * (ga * dy[n * C + c] - xhat * B / (double)D);
        }
    }
    if (dgamma != NULL) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t c = 0; c < C; ++c) {
            const int64_t g = c / D;
            double sg = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const double r = rstd[n * G + g];
                sg += MUT(11) ? dy[n * C + c] * x[n * C + c] : dy[n * C + c] * (x[n * C + c] * r); /* mutant 11: raw x */
            }
            dgamma[c] = sg;
        }
    }
    return 0;
}

/* Threads OpenMP will use for the parallel loops above (1 without OpenMP). */
int gno_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void gno_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
