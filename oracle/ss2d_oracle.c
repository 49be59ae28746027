/*
 * CPU oracle for the SS2D forward operator and its bidirectional 1D variant.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU
 * baseline load this library.  It shares no code, header or constant with the GPU path:
 * it is a plain sequential loop in float64, written from the pages' definitions.
 *
 * What it computes, per (b, d) channel:
 *
 *   for each route k = 0 .. K-1 (in this order), from a zero state h = 0:
 *     for t = 0 .. L-1:
 *       l     = pi_k(t)                       image position visited at step t of route k
 *       u     = x[b, d, l]
 *       delta = softplus(dt_raw[b, k, d, t] + dt_bias[k, d])
 *       h_n   = exp(delta * A[k, d, n]) * h_n + delta * Bs[b, k, n, t] * u   (n = 0..N-1)
 *       y[b, d, l] += sum_n Cs[b, k, n, t] * h_n + Ds[k, d] * u
 *   with A[k, d, n] = -exp(A_log[k, d, n]).
 *
 * Sources (page titles as printed in the reference pages):
 *   - Recurrence, zero initial state, output taken after the update, skip term D * x:
 *     "Vision Mamba" explainer (dileepadev), SelectiveSSM._selective_scan listing; the
 *     discrete system h_t = Abar h_{t-1} + Bbar x_t, y_t = C h_t in the Vim summary
 *     (aipaper.cc), section 4.1.
 *   - Discretisation Abar = exp(delta * A) and Bbar x = delta * B * x (exponential for A, first
 *     order for B): the explainer's listing (dA, dB) and the VMamba review (nubint.ai),
 *     "Proposed method".
 *   - delta = softplus(dt_proj(.)) with the projection's bias inside the softplus, and
 *     A = -exp(A_log) real and diagonal: the explainer's SelectiveSSM.__init__ / forward.
 *   - Four routes and their inverses: the explainer's CrossScanModule listing (row-major,
 *     its flip, column-major, its flip; inverse flips and (W,H) -> (H,W) transposes) and
 *     the Chinese VMamba article, section 1 (cross_scan); the outputs are summed (the
 *     explainer's prose on the Cross-Scan Module).  The sum is taken in route order
 *     k = 0, 1, 2, 3 for every position.
 *   - K = 2: the Vim block's forward path and a backward path over a reversed copy of the
 *     sequence, added together (Vim summary, section 4.3).
 *
 * Two options (the _ex entry points):
 *   - Gate z (B, D, H, W), optional: every route's output is multiplied by SiLU(z) at its
 *     image position before the routes are added, SiLU(z) = z / (1 + exp(-z)) (Vim
 *     summary, section 4.3, "Gating and Merging"; the explainer's MambaBlock.forward, which
 *     multiplies the scan output by silu(z)).
 *   - ORACLE_ZOH: zero-order hold for B as well, Bbar = (exp(delta A) - 1) / A * B in
 *     place of delta * B (the Vim summary, section 4.1, defines Abar = exp(delta A) and
 *     Bbar = (delta A)^-1 (exp(delta A) - I) delta B).  Written with expm1 so that small
 *     |delta A| keeps its digits; A = 0 takes the limit delta * B.
 *
 * A per-route front end (oracle_project: causal depthwise conv + SiLU, x_proj, dt_proj for
 * each route; oracle_project_lr: the same without dt_proj) and the operator over its
 * per-route inputs (oracle_forward_routes_ex; oracle_forward_routes_lr_ex with dt_proj
 * applied per step) are described where they are defined, below.
 *
 * Layouts (all contiguous, row-major):
 *   x, y      (B, D, H, W)    y written in full
 *   dt_raw    (B, K, D, L)    scan order of route k (position t is step t of that route)
 *   Bs, Cs    (B, K, N, L)    scan order of route k
 *   A_log     (K, D, N)       Ds, dt_bias (K, D)
 * Inputs arrive as float (the exact values the GPU path receives, bfloat16 widened where
 * applicable); every operation is done in double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_ZOH 1

/* log(1 + e^z), written to stay finite for large |z| */
static double softplus(double z) {
    const double m = z > 0.0 ? z : 0.0;
    return m + log1p(exp(-fabs(z)));
}

/* Raster index (h * W + w) of the image position visited at step t of route k.
 * K = 4: 0 row-major, 1 row-major reversed, 2 column-major, 3 column-major reversed.
 * K = 2: 0 forward, 1 reversed (H = 1, W = L). */
static int64_t route_position(int K, int k, int64_t t, int64_t H, int64_t W) {
    const int64_t L = H * W;
    int64_t s;
    if (K == 2)
        return k == 0 ? t : L - 1 - t;
    switch (k) {
    case 0:
        return t;
    case 1:
        return L - 1 - t;
    case 2:
        return (t % H) * W + t / H;
    default:
        s = L - 1 - t;
        return (s % H) * W + s / H;
    }
}

/* z * sigmoid(z), the gate nonlinearity */
static double silu(double z) {
    return z / (1.0 + exp(-z));
}

/* All K routes of one (b, d) channel, summed into out[0 .. L-1] (image order).  The input
 * of step t of route k is x[b, d, pi_k(t)], or, when u_routes is given, u_routes[b, k, d, t]
 * (each route's own input sequence, already in its scan order). */
static void channel_forward(int K, const float *x, const float *u_routes, const float *dt_raw,
                            const float *dt_lr, const float *dt_w, int64_t R,
                            const float *A_log, const float *Bs, const float *Cs,
                            const float *Ds, const float *dt_bias, const float *z, int flags,
                            int64_t D, int64_t H, int64_t W, int64_t N, int64_t b, int64_t d,
                            double *out, double *h, double *A) {
    const int64_t L = H * W;
    const float *xc = u_routes ? NULL : x + (b * D + d) * L;
    const float *zc = z ? z + (b * D + d) * L : NULL;
    const int zoh = (flags & ORACLE_ZOH) != 0;
    for (int64_t l = 0; l < L; ++l)
        out[l] = 0.0;
    for (int k = 0; k < K; ++k) {
        const double bias = dt_bias[k * D + d];
        const double Dk = Ds[k * D + d];
        const float *dt = dt_lr ? NULL : dt_raw + ((b * K + k) * D + d) * L;
        const float *lr = dt_lr ? dt_lr + (b * K + k) * R * L : NULL;
        const float *wr = dt_lr ? dt_w + (k * D + d) * R : NULL;
        const float *Bk = Bs + (b * K + k) * N * L;
        const float *Ck = Cs + (b * K + k) * N * L;
        for (int64_t n = 0; n < N; ++n) {
            A[n] = -exp((double)A_log[(k * D + d) * N + n]);
            h[n] = 0.0;
        }
        const float *uk = u_routes ? u_routes + ((b * K + k) * D + d) * L : NULL;
        for (int64_t t = 0; t < L; ++t) {
            const int64_t l = route_position(K, k, t, H, W);
            const double u = uk ? uk[t] : xc[l];
            double dtv = 0.0;
            if (lr) {
                for (int64_t r = 0; r < R; ++r)
                    dtv += (double)wr[r] * (double)lr[r * L + t];
            } else {
                dtv = dt[t];
            }
            const double delta = softplus(dtv + bias);
            double yk = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const double a = exp(delta * A[n]);
                double bbar = delta;
                if (zoh && A[n] != 0.0)
                    bbar = expm1(delta * A[n]) / A[n];
                h[n] = a * h[n] + bbar * (double)Bk[n * L + t] * u;
                yk += (double)Ck[n * L + t] * h[n];
            }
            const double gate = zc ? silu((double)zc[l]) : 1.0;
            out[l] += (yk + Dk * u) * gate;
        }
    }
}

static int pick_threads(int nthreads) {
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* Full output y (B, D, H, W) in double.  K is 4 (SS2D) or 2 (bidirectional 1D, H = 1).
 * z (B, D, H, W) is the optional gate (NULL: none); flags is 0 or ORACLE_ZOH.
 * Returns the number of threads used, or -1 on bad arguments / allocation failure. */
static int forward_all(int K, const float *x, const float *u_routes, const float *dt_raw,
                       const float *dt_lr, const float *dt_w, int64_t R,
                       const float *A_log, const float *Bs, const float *Cs, const float *Ds,
                       const float *dt_bias, const float *z, int flags, double *y, int64_t B,
                       int64_t D, int64_t H, int64_t W, int64_t N, int nthreads) {
    if ((K != 2 && K != 4) || B < 0 || D < 0 || H < 0 || W < 0 || N <= 0)
        return -1;
    if (flags & ~ORACLE_ZOH)
        return -1;
    if (K == 2 && H != 1)
        return -1;
    const int threads = pick_threads(nthreads);
    const int64_t L = H * W;
    const int64_t total = B * D;
    int failed = 0;
#ifdef _OPENMP
#pragma omp parallel num_threads(threads) reduction(| : failed)
#endif
    {
        double *h = (double *)malloc(sizeof(double) * (size_t)(2 * N));
        if (!h) {
            failed = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (int64_t i = 0; i < total; ++i) {
                const int64_t b = i / D, d = i % D;
                channel_forward(K, x, u_routes, dt_raw, dt_lr, dt_w, R, A_log, Bs, Cs, Ds,
                                dt_bias, z, flags, D, H, W, N, b, d, y + i * L, h, h + N);
            }
            free(h);
        }
    }
    return failed ? -1 : threads;
}

int oracle_forward_ex(int K, const float *x, const float *dt_raw, const float *A_log,
                      const float *Bs, const float *Cs, const float *Ds, const float *dt_bias,
                      const float *z, int flags, double *y, int64_t B, int64_t D, int64_t H,
                      int64_t W, int64_t N, int nthreads) {
    return forward_all(K, x, NULL, dt_raw, NULL, NULL, 0, A_log, Bs, Cs, Ds, dt_bias, z, flags,
                       y, B, D, H, W, N, nthreads);
}

/* The same operator when every route brings its own input sequence: u (B, K, D, L), step t
 * of route k reading u[b, k, d, t] (the per-route conv + SiLU output of oracle_project) in
 * place of x at the position visited.  Outputs are still added at the visited positions, in
 * route order, with the optional gate z (B, D, H, W) at those positions. */
int oracle_forward_routes_ex(int K, const float *u, const float *dt_raw, const float *A_log,
                             const float *Bs, const float *Cs, const float *Ds,
                             const float *dt_bias, const float *z, int flags, double *y,
                             int64_t B, int64_t D, int64_t H, int64_t W, int64_t N,
                             int nthreads) {
    return forward_all(K, NULL, u, dt_raw, NULL, NULL, 0, A_log, Bs, Cs, Ds, dt_bias, z, flags,
                       y, B, D, H, W, N, nthreads);
}

/* The same with dt_proj folded in: step t of route k takes
 *   dt_raw = sum_{r < R} dt_w[k, d, r] * dt_lr[b, k, r, t]
 * from the R-row x_proj output dt_lr (B, K, R, L) and the dt_proj weight dt_w (K, D, R)
 * (the [Explainer]'s dt_proj(dt) before the softplus; its bias is dt_bias). */
int oracle_forward_routes_lr_ex(int K, const float *u, const float *dt_lr, const float *dt_w,
                                int64_t R, const float *A_log, const float *Bs,
                                const float *Cs, const float *Ds, const float *dt_bias,
                                const float *z, int flags, double *y, int64_t B, int64_t D,
                                int64_t H, int64_t W, int64_t N, int nthreads) {
    if (R <= 0)
        return -1;
    return forward_all(K, NULL, u, NULL, dt_lr, dt_w, R, A_log, Bs, Cs, Ds, dt_bias, z, flags,
                       y, B, D, H, W, N, nthreads);
}

/* Output planes y[b_idx[i], d_idx[i], :, :] for i < nsel, written to y_sel (nsel, H, W).
 * Same arithmetic as oracle_forward_ex; used to check large outputs on sampled channels. */
int oracle_forward_channels_ex(int K, const float *x, const float *dt_raw, const float *A_log,
                               const float *Bs, const float *Cs, const float *Ds,
                               const float *dt_bias, const float *z, int flags, int64_t B,
                               int64_t D, int64_t H, int64_t W, int64_t N,
                               const int64_t *b_idx, const int64_t *d_idx, int64_t nsel,
                               double *y_sel, int nthreads) {
    if ((K != 2 && K != 4) || N <= 0 || (K == 2 && H != 1))
        return -1;
    if (flags & ~ORACLE_ZOH)
        return -1;
    for (int64_t i = 0; i < nsel; ++i)
        if (b_idx[i] < 0 || b_idx[i] >= B || d_idx[i] < 0 || d_idx[i] >= D)
            return -1;
    const int threads = pick_threads(nthreads);
    const int64_t L = H * W;
    int failed = 0;
#ifdef _OPENMP
#pragma omp parallel num_threads(threads) reduction(| : failed)
#endif
    {
        double *h = (double *)malloc(sizeof(double) * (size_t)(2 * N));
        if (!h) {
            failed = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (int64_t i = 0; i < nsel; ++i)
                channel_forward(K, x, NULL, dt_raw, NULL, NULL, 0, A_log, Bs, Cs, Ds, dt_bias,
                                z, flags, D, H, W, N, b_idx[i], d_idx[i], y_sel + i * L, h,
                                h + N);
            free(h);
        }
    }
    return failed ? -1 : threads;
}

/* The plain operator: no gate, delta * B for B. */
int oracle_forward(int K, const float *x, const float *dt_raw, const float *A_log,
                   const float *Bs, const float *Cs, const float *Ds, const float *dt_bias,
                   double *y, int64_t B, int64_t D, int64_t H, int64_t W, int64_t N,
                   int nthreads) {
    return oracle_forward_ex(K, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, NULL, 0, y, B, D, H, W,
                             N, nthreads);
}

int oracle_forward_channels(int K, const float *x, const float *dt_raw, const float *A_log,
                            const float *Bs, const float *Cs, const float *Ds,
                            const float *dt_bias, int64_t B, int64_t D, int64_t H, int64_t W,
                            int64_t N, const int64_t *b_idx, const int64_t *d_idx,
                            int64_t nsel, double *y_sel, int nthreads) {
    return oracle_forward_channels_ex(K, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, NULL, 0, B, D,
                                      H, W, N, b_idx, d_idx, nsel, y_sel, nthreads);
}

/* ---- per-route front end -----------------------------------------------------------------
 * What feeds each route's scan when every direction carries its own input layers, as in the
 * explainer's CrossScanModule (four independent SelectiveSSM modules, one per scan direction)
 * and in the Vim block (section 4.3: inside the forward and the backward path, a Conv1d, a
 * SiLU, and Delta, B, C generated from the activated output).  For route k of image b, with
 * s_t = x[b, d, pi_k(t)] the route's input sequence and s_t = 0 for t < 0:
 *   c[d, t]      = conv_b[k, d] + sum_{j < KW} conv_w[k, d, j] * s_{t - (KW - 1) + j}
 *                  (the explainer's depthwise Conv1d with padding d_conv - 1, of which the first
 *                  L outputs are kept: causal, cross-correlation order of the taps)
 *   u[d, t]      = SiLU(c[d, t])
 *   xd[m, t]     = sum_d x_proj_w[k, m, d] * u[d, t]          m < R + 2N (x_proj, no bias)
 *   dt_raw[d, t] = sum_{r < R} dt_proj_w[k, d, r] * xd[r, t]   (dt_proj without its bias:
 *                  the bias is dt_bias, added inside the softplus by the scan)
 *   Bs[n, t]     = xd[R + n, t],   Cs[n, t] = xd[R + N + n, t]
 * (the explainer splits x_proj's output as [dt, B, C] = [1, N, N]; R is that first width).
 * Layouts: x (B, D, H, W); conv_w (K, D, KW); conv_b (K, D); x_proj_w (K, R + 2N, D);
 * dt_proj_w (K, D, R); outputs u, dt_raw (B, K, D, L) and Bs, Cs (B, K, N, L) in scan order.
 * Returns the number of threads used, or -1 on bad arguments / allocation failure. */
static int project_all(int K, const float *x, const float *conv_w, const float *conv_b,
                       const float *x_proj_w, const float *dt_proj_w, double *u, double *dt_raw,
                       double *dt_lr, double *Bs, double *Cs, int64_t B, int64_t D, int64_t H,
                       int64_t W, int64_t N, int64_t R, int64_t KW, int nthreads) {
    if ((K != 2 && K != 4) || B < 0 || D < 0 || H < 0 || W < 0 || N <= 0 || R <= 0 || KW <= 0)
        return -1;
    if (K == 2 && H != 1)
        return -1;
    const int threads = pick_threads(nthreads);
    const int64_t L = H * W;
    const int64_t M = R + 2 * N;
    int failed = 0;
#ifdef _OPENMP
#pragma omp parallel num_threads(threads) reduction(| : failed)
#endif
    {
        double *xd = (double *)malloc(sizeof(double) * (size_t)M);
        if (!xd) {
            failed = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (int64_t i = 0; i < B * K; ++i) {
                const int64_t b = i / K;
                const int k = (int)(i % K);
                double *uk = u + i * D * L;
                /* causal depthwise conv along the route, then SiLU */
                for (int64_t d = 0; d < D; ++d) {
                    const float *xc = x + (b * D + d) * L;
                    const float *w = conv_w + ((int64_t)k * D + d) * KW;
                    for (int64_t t = 0; t < L; ++t) {
                        double c = conv_b[(int64_t)k * D + d];
                        for (int64_t j = 0; j < KW; ++j) {
                            const int64_t tau = t - (KW - 1) + j;
                            if (tau >= 0)
                                c += (double)w[j] * (double)xc[route_position(K, k, tau, H, W)];
                        }
                        uk[d * L + t] = silu(c);
                    }
                }
                /* x_proj, then dt_proj, one step at a time */
                for (int64_t t = 0; t < L; ++t) {
                    for (int64_t m = 0; m < M; ++m) {
                        double acc = 0.0;
                        for (int64_t d = 0; d < D; ++d)
                            acc += (double)x_proj_w[((int64_t)k * M + m) * D + d] * uk[d * L + t];
                        xd[m] = acc;
                    }
                    for (int64_t d = 0; dt_raw && d < D; ++d) {
                        double acc = 0.0;
                        for (int64_t r = 0; r < R; ++r)
                            acc += (double)dt_proj_w[((int64_t)k * D + d) * R + r] * xd[r];
                        dt_raw[(i * D + d) * L + t] = acc;
                    }
                    for (int64_t r = 0; dt_lr && r < R; ++r)
                        dt_lr[(i * R + r) * L + t] = xd[r];
                    for (int64_t n = 0; n < N; ++n) {
                        Bs[(i * N + n) * L + t] = xd[R + n];
                        Cs[(i * N + n) * L + t] = xd[R + N + n];
                    }
                }
            }
            free(xd);
        }
    }
    return failed ? -1 : threads;
}

int oracle_project(int K, const float *x, const float *conv_w, const float *conv_b,
                   const float *x_proj_w, const float *dt_proj_w, double *u, double *dt_raw,
                   double *Bs, double *Cs, int64_t B, int64_t D, int64_t H, int64_t W,
                   int64_t N, int64_t R, int64_t KW, int nthreads) {
    return project_all(K, x, conv_w, conv_b, x_proj_w, dt_proj_w, u, dt_raw, NULL, Bs, Cs, B,
                       D, H, W, N, R, KW, nthreads);
}

/* The front end without dt_proj: the first R rows of x_proj's output, dt_lr (B, K, R, L),
 * in place of dt_raw (for the operator with dt_proj folded into the scan). */
int oracle_project_lr(int K, const float *x, const float *conv_w, const float *conv_b,
                      const float *x_proj_w, double *u, double *dt_lr, double *Bs, double *Cs,
                      int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int64_t R,
                      int64_t KW, int nthreads) {
    return project_all(K, x, conv_w, conv_b, x_proj_w, NULL, u, NULL, dt_lr, Bs, Cs, B, D, H,
                       W, N, R, KW, nthreads);
}

/* ---- backward ----------------------------------------------------------------------------
 * Gradients of L = sum over (b, d, l) of dy[b, d, l] * y[b, d, l] for the plain operator (no
 * gate, delta * B), by reverse-mode differentiation of the recurrence above.  Per route, with
 * g_t = dy at the position visited at step t:
 *   lambda_t,n = g_t C_t,n + a_t+1,n lambda_t+1,n          (adjoint of h_t,n; lambda_L = 0)
 *   dC_t,n     = g_t h_t,n              dB_t,n = lambda_t,n delta_t u_t
 *   da_t,n     = lambda_t,n h_t-1,n     (h_-1 = 0)
 *   ddelta_t   = sum_n (da_t,n a_t,n A_n + lambda_t,n B_t,n u_t)
 *   du_t       = g_t D + sum_n lambda_t,n delta_t B_t,n
 *   dA_n      += da_t,n a_t,n delta_t,   dA_log_n = A_n dA_n   (A = -exp(A_log))
 *   dD        += g_t u_t
 *   ddt_raw_t  = ddelta_t sigmoid(dt_raw_t + dt_bias)          (softplus' = sigmoid)
 *   ddt_bias  += ddt_raw_t
 * dx accumulates du_t at the visited position over the routes; dBs, dCs sum over the
 * channels d (Bs and Cs are shared by all channels of a (b, k)).  Everything in double.
 * Work is split over images b (each thread owns whole images, so no sum is shared between
 * threads); the per-image contributions to dA_log, dDs and ddt_bias are added in b order.
 *
 * Gated operator (the Vim block's gate, Vim summary section 4.3: out = y * SiLU(z) with y the
 * route sum above): by the product rule every route sees g = dy SiLU(z) in place of dy, and
 *   dz = dy y SiLU'(z),   SiLU'(z) = sigma(z) (1 + z (1 - sigma(z))),
 * with y the ungated route sum, accumulated here from the same recomputed states.
 *
 * Zero-order hold (ORACLE_ZOH; Vim summary section 4.1): the update is h = a h + bb B u with
 * bb = expm1(delta A) / A, so in the sums above delta u becomes bb u and
 *   dB_t,n = lambda bb u,    du_t = g D + sum_n lambda bb B,
 *   ddelta_t = sum_n lambda a (h_prev A + B u)                  (d bb / d delta = a),
 *   dA_n += lambda (h_prev a delta + B u d bb / dA),            d bb / dA = delta^2 psi(delta A),
 *   psi(x) = (x e^x - expm1(x)) / x^2 = sum_k x^k (k + 1) / (k + 2)!   (psi(0) = 1/2). */

static double sigmoid(double z) {
    return 1.0 / (1.0 + exp(-z));
}

/* d/dz of z sigmoid(z) */
static double silu_grad(double z) {
    const double s = sigmoid(z);
    return s * (1.0 + z * (1.0 - s));
}

/* psi(x) = (x e^x - (e^x - 1)) / x^2: its power series below |x| = 1/64 (terms to x^6,
 * truncation below 1e-16 relative), the closed form above */
static double zoh_psi(double x) {
    if (fabs(x) < 1.0 / 64.0) {
        double p = 0.0, f = 2.0; /* f = (k + 2)! */
        double xk = 1.0;
        for (int k = 0; k <= 6; ++k) {
            p += xk * (double)(k + 1) / f;
            xk *= x;
            f *= (double)(k + 3);
        }
        return p;
    }
    return (x * exp(x) - expm1(x)) / (x * x);
}

/* One image b, all routes and channels.  Accumulates into dx_b (D, L), ddt_b (K, D, L),
 * dB_b, dC_b (K, N, L) and the parameter partials pA (K, D, N), pD (K, D), pbias (K, D);
 * with the gate z (else NULL), writes dz_b (D, L).  ws holds 2 L N + 3 L + 2 N doubles. */
static void image_backward(int K, const float *x, const float *u_routes, const float *dt_raw,
                           const float *A_log, const float *Bs, const float *Cs,
                           const float *Ds, const float *dt_bias, const float *z, int flags,
                           const float *dy, int64_t D, int64_t H, int64_t W, int64_t N,
                           int64_t b, double *dx_b, double *ddt_b, double *dB_b, double *dC_b,
                           double *pA, double *pD, double *pbias, double *dz_b, double *ws) {
    const int64_t L = H * W;
    const int zoh = (flags & ORACLE_ZOH) != 0;
    double *hs = ws;               /* h_t,n, t-major */
    double *as = hs + L * N;       /* a_t,n */
    double *delta = as + L * N;    /* delta_t */
    double *lam = delta + L;       /* lambda_n */
    double *A = lam + N;           /* A_n */
    double *ysum = A + N;          /* ungated route sum y_l (gate only) */
    for (int64_t d = 0; d < D; ++d) {
        const float *xc = u_routes ? NULL : x + (b * D + d) * L;
        const float *gc = dy + (b * D + d) * L;
        const float *zc = z ? z + (b * D + d) * L : NULL;
        for (int64_t l = 0; l < L; ++l)
            ysum[l] = 0.0;
        for (int k = 0; k < K; ++k) {
            const double bias = dt_bias[k * D + d];
            const double Dk = Ds[k * D + d];
            const float *dt = dt_raw + ((b * K + k) * D + d) * L;
            const float *Bk = Bs + (b * K + k) * N * L;
            const float *Ck = Cs + (b * K + k) * N * L;
            const float *uk = u_routes ? u_routes + ((b * K + k) * D + d) * L : NULL;
            for (int64_t n = 0; n < N; ++n)
                A[n] = -exp((double)A_log[(k * D + d) * N + n]);
            /* forward, keeping every state */
            for (int64_t t = 0; t < L; ++t) {
                const int64_t l = route_position(K, k, t, H, W);
                const double u = uk ? (double)uk[t] : (double)xc[l];
                delta[t] = softplus((double)dt[t] + bias);
                double yroute = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double a = exp(delta[t] * A[n]);
                    const double hprev = t > 0 ? hs[(t - 1) * N + n] : 0.0;
                    double bb = delta[t];
                    if (zoh && A[n] != 0.0)
                        bb = expm1(delta[t] * A[n]) / A[n];
                    as[t * N + n] = a;
                    hs[t * N + n] = a * hprev + bb * (double)Bk[n * L + t] * u;
                    yroute += (double)Ck[n * L + t] * hs[t * N + n];
                }
                ysum[l] += yroute + Dk * u;
            }
            /* reverse */
            for (int64_t n = 0; n < N; ++n)
                lam[n] = 0.0;
            for (int64_t t = L - 1; t >= 0; --t) {
                const int64_t l = route_position(K, k, t, H, W);
                const double u = uk ? (double)uk[t] : (double)xc[l];
                const double g = zc ? (double)gc[l] * silu((double)zc[l]) : (double)gc[l];
                double ddelta = 0.0, du = g * Dk;
                pD[k * D + d] += g * u;
                for (int64_t n = 0; n < N; ++n) {
                    const double anext = t + 1 < L ? as[(t + 1) * N + n] : 0.0;
                    lam[n] = g * (double)Ck[n * L + t] + anext * lam[n];
                    const double hprev = t > 0 ? hs[(t - 1) * N + n] : 0.0;
                    const double a = as[t * N + n];
                    const double da = lam[n] * hprev;
                    const double Bv = (double)Bk[n * L + t];
                    /* bb and its derivatives in delta and A */
                    double bb = delta[t], bb_delta = 1.0, bb_A = 0.0;
                    if (zoh) {
                        bb_delta = a;
                        bb_A = delta[t] * delta[t] * zoh_psi(delta[t] * A[n]);
                        if (A[n] != 0.0)
                            bb = expm1(delta[t] * A[n]) / A[n];
                    }
                    dC_b[(k * N + n) * L + t] += g * hs[t * N + n];
                    dB_b[(k * N + n) * L + t] += lam[n] * bb * u;
                    ddelta += da * a * A[n] + lam[n] * bb_delta * Bv * u;
                    pA[(k * D + d) * N + n] +=
                        (da * a * delta[t] + lam[n] * Bv * u * bb_A) * A[n];
                    du += lam[n] * bb * Bv;
                }
                const double dr = ddelta * sigmoid((double)dt[t] + bias);
                ddt_b[(k * D + d) * L + t] = dr;
                pbias[k * D + d] += dr;
                if (uk)
                    dx_b[(k * D + d) * L + t] = du; /* du per route, in scan order */
                else
                    dx_b[d * L + l] += du;
            }
        }
        if (zc)
            for (int64_t l = 0; l < L; ++l)
                dz_b[d * L + l] = (double)gc[l] * ysum[l] * silu_grad((double)zc[l]);
    }
}

/* Gradients of sum(dy * y) with respect to every input (outputs in double, caller-owned):
 *   dx (B, D, H, W), ddt_raw (B, K, D, L), dA_log (K, D, N), dBs, dCs (B, K, N, L),
 *   dDs, ddt_bias (K, D); with the gate z (B, D, H, W) (else NULL), y is the gated output
 *   and dz (B, D, H, W) receives its gradient with respect to z; flags is 0 or ORACLE_ZOH
 *   (the zero-order-hold operator).
 * Returns the number of threads used, or -1 on bad arguments / allocation failure. */
static int backward_all(int K, const float *x, const float *u_routes, const float *dt_raw,
                        const float *A_log, const float *Bs, const float *Cs, const float *Ds,
                        const float *dt_bias, const float *z, int flags, const float *dy,
                        double *dx, double *ddt_raw, double *dA_log, double *dBs, double *dCs,
                        double *dDs, double *ddt_bias, double *dz, int64_t B, int64_t D,
                        int64_t H, int64_t W, int64_t N, int nthreads) {
    if ((K != 2 && K != 4) || B < 0 || D < 0 || H < 0 || W < 0 || N <= 0)
        return -1;
    if (flags & ~ORACLE_ZOH)
        return -1;
    if (K == 2 && H != 1)
        return -1;
    if (z && !dz)
        return -1;
    const int threads = pick_threads(nthreads);
    const int64_t L = H * W;
    const int64_t np = K * D * N + 2 * K * D; /* per-image parameter partials */
    double *part = (double *)calloc((size_t)(B > 0 ? B : 1) * (size_t)np, sizeof(double));
    if (!part)
        return -1;
    for (int64_t i = 0; i < (u_routes ? K : 1) * B * D * L; ++i)
        dx[i] = 0.0;
    for (int64_t i = 0; i < B * K * N * L; ++i) {
        dBs[i] = 0.0;
        dCs[i] = 0.0;
    }
    int failed = 0;
#ifdef _OPENMP
#pragma omp parallel num_threads(threads) reduction(| : failed)
#endif
    {
        double *ws = (double *)malloc(sizeof(double) * (size_t)(2 * L * N + 3 * L + 2 * N));
        if (!ws) {
            failed = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (int64_t b = 0; b < B; ++b) {
                double *p = part + b * np;
                image_backward(K, x, u_routes, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, flags,
                               dy, D, H, W, N, b,
                               dx + b * (u_routes ? K : 1) * D * L, ddt_raw + b * K * D * L,
                               dBs + b * K * N * L, dCs + b * K * N * L, p, p + K * D * N,
                               p + K * D * N + K * D, z ? dz + b * D * L : NULL, ws);
            }
            free(ws);
        }
    }
    for (int64_t i = 0; i < K * D * N; ++i)
        dA_log[i] = 0.0;
    for (int64_t i = 0; i < K * D; ++i) {
        dDs[i] = 0.0;
        ddt_bias[i] = 0.0;
    }
    for (int64_t b = 0; b < B; ++b) {
        const double *p = part + b * np;
        for (int64_t i = 0; i < K * D * N; ++i)
            dA_log[i] += p[i];
        for (int64_t i = 0; i < K * D; ++i) {
            dDs[i] += p[K * D * N + i];
            ddt_bias[i] += p[K * D * N + K * D + i];
        }
    }
    free(part);
    return failed ? -1 : threads;
}

int oracle_backward_ex(int K, const float *x, const float *dt_raw, const float *A_log,
                       const float *Bs, const float *Cs, const float *Ds,
                       const float *dt_bias, const float *z, int flags, const float *dy,
                       double *dx, double *ddt_raw, double *dA_log, double *dBs, double *dCs,
                       double *dDs, double *ddt_bias, double *dz, int64_t B, int64_t D,
                       int64_t H, int64_t W, int64_t N, int nthreads) {
    return backward_all(K, x, NULL, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, flags, dy, dx,
                        ddt_raw, dA_log, dBs, dCs, dDs, ddt_bias, dz, B, D, H, W, N,
                        nthreads);
}

/* The same for the operator over per-route inputs (oracle_forward_routes_ex): u (B, K, D, L)
 * in each route's scan order in place of x, and du (B, K, D, L), the gradient of each
 * route's own input at each step, in place of dx (the routes do not share their input, so
 * nothing is summed across routes). */
int oracle_backward_routes_ex(int K, const float *u, const float *dt_raw, const float *A_log,
                              const float *Bs, const float *Cs, const float *Ds,
                              const float *dt_bias, const float *z, int flags,
                              const float *dy, double *du, double *ddt_raw, double *dA_log,
                              double *dBs, double *dCs, double *dDs, double *ddt_bias,
                              double *dz, int64_t B, int64_t D, int64_t H, int64_t W,
                              int64_t N, int nthreads) {
    if (!u)
        return -1;
    return backward_all(K, NULL, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, flags, dy, du,
                        ddt_raw, dA_log, dBs, dCs, dDs, ddt_bias, dz, B, D, H, W, N,
                        nthreads);
}

/* The plain operator's gradients (no gate). */
int oracle_backward(int K, const float *x, const float *dt_raw, const float *A_log,
                    const float *Bs, const float *Cs, const float *Ds, const float *dt_bias,
                    const float *dy, double *dx, double *ddt_raw, double *dA_log, double *dBs,
                    double *dCs, double *dDs, double *ddt_bias, int64_t B, int64_t D,
                    int64_t H, int64_t W, int64_t N, int nthreads) {
    return oracle_backward_ex(K, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, NULL, 0, dy, dx,
                              ddt_raw, dA_log, dBs, dCs, dDs, ddt_bias, NULL, B, D, H, W, N,
                              nthreads);
}
