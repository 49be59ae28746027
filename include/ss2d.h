/*
 * ss2d.h -- C ABI of libss2d.so, the MI355X (gfx950) SS2D forward operator.
 *
 * The operator (VMamba's 2D selective scan, "SS2D"):
 *   1. Cross-scan: a (B, D, H, W) feature map is read along four routes, each a sequence of
 *      length L = H * W over every channel d:
 *        route 0  row-major              pi_0(t) = t
 *        route 1  row-major, reversed    pi_1(t) = L - 1 - t
 *        route 2  column-major           pi_2(t) = (t mod H) * W + floor(t / H)
 *        route 3  column-major, reversed pi_3(t) = pi_2(L - 1 - t)
 *      (pi_k(t) is the raster index h * W + w visited at step t.)  Sources: the "Vision
 *      Mamba" explainer (dileepadev), CrossScanModule listing and its prose; the Chinese
 *      VMamba article (mhpn.cn), section 1, cross_scan; the VMamba review (nubint.ai),
 *      "Proposed method" (Cross-Scan Module with four routes).
 *   2. Selective scan on every route k and channel d, from a zero state h (N values):
 *        delta_t = softplus(dt_raw[b,k,d,t] + dt_bias[k,d])
 *        A_n     = -exp(A_log[k,d,n])
 *        h_n     = exp(delta_t * A_n) * h_n + delta_t * Bs[b,k,n,t] * x[b,d,pi_k(t)]
 *        y_k,t   = sum_n Cs[b,k,n,t] * h_n + Ds[k,d] * x[b,d,pi_k(t)]
 *      Sources: the explainer's SelectiveSSM listing (softplus of the dt projection with
 *      its bias, A = -exp(A_log), the exp discretisation of A and delta * B for B, zero
 *      initial state, output after the update, D skip term); the Vim summary (aipaper.cc),
 *      section 4.1 (discrete recurrence); one independent parameter set per route (the
 *      explainer's four SSMs).
 *   3. Cross-merge: y[b,d,pi_k(t)] = sum over k of y_k,t, each route's permutation undone
 *      and the routes summed (the explainer's CrossScanModule: inverse flips and
 *      transposes, outputs summed).
 *   ss1d_bidir_forward is the K = 2 case over a 1D sequence: route 0 forward, route 1 over
 *   the reversed sequence, summed after undoing the reversal (Vim summary, section 4.3).
 *
 * Precision: x, dt_raw, Bs, Cs and y share one data type (fp32 or bfloat16); A_log, Ds and
 * dt_bias are always fp32.  delta, the state h and every sum are fp32; y is rounded once
 * (round to nearest even for bfloat16).  The state never leaves the chip.
 *
 * Layouts (contiguous, row-major, device pointers, caller-owned):
 *   x, y      (B, D, H, W)          [ss1d_bidir_forward: (B, D, L)]
 *   dt_raw    (B, K, D, L)          in the scan order of route k (index t = step t)
 *   Bs, Cs    (B, K, N, L)          in the scan order of route k
 *   A_log     (K, D, N)  fp32
 *   Ds        (K, D)     fp32
 *   dt_bias   (K, D)     fp32
 * with K = 4 for ss2d_forward and K = 2 for ss1d_bidir_forward.
 *
 * Conventions shared by every entry point:
 *   - Inputs are read only.  y is written in full (no pre-zeroing needed) and must not
 *     overlap any input (z included, for the entry points that take it).
 *   - All arguments are validated before anything is enqueued; on an error nothing is
 *     launched and y is untouched.  Nothing is printed and no exception crosses the ABI.
 *   - The call is asynchronous on `stream` (a hipStream_t; NULL is the default stream).
 *     Faults inside the kernels surface at the caller's next synchronisation.
 *   - Calls keep no data between them (the training pair below hands its state over in a
 *     caller-owned buffer).  Internal scratch (a transposed copy of x, per-route
 *     fp32 partial outputs, chunk carries) is allocated on `stream` from a stream-ordered
 *     memory pool of the library's own (one per device, created at the first call on that
 *     device, held until the process ends) and released on `stream` in the same call.  The
 *     pool keeps freed blocks for later calls (its release threshold is unlimited), so the
 *     device memory of the largest scratch used so far stays reserved by the library until
 *     ss2d_scratch_trim hands it back; the device's default pool and its attributes are not
 *     touched.  Under stream capture the
 *     scratch becomes an allocation node of the graph (no synchronisation, copy or memset
 *     is enqueued, so every entry point can be captured).
 *   - Results are deterministic: identical inputs, shapes and device give bitwise identical
 *     y (no atomics; the routes are summed in the fixed order 0, 1, 2, 3).
 *   - B == 0 or D == 0 is a valid empty call: it returns SS2D_OK, launches nothing and reads
 *     no pointer.
 *   - Thread safety: calls from several host threads are safe; calls on different streams
 *     run independently.
 */
#ifndef SS2D_H
#define SS2D_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SS2D_ABI_VERSION 12

/* Status codes returned by every entry point. */
#define SS2D_OK 0
#define SS2D_ERR_NULL 1        /* a required pointer is NULL                                */
#define SS2D_ERR_SHAPE 2       /* a negative dimension, H/W/L/N < 1, or a size beyond the
                                  kernels' index range (L >= 2^30, or any tensor with
                                  2^62 elements or more)                                   */
#define SS2D_ERR_UNSUPPORTED 3 /* N not in {1, 2, 4, 8, 16, 32}, an unknown dtype or flag, or
                                  a size an entry point documents as unsupported          */
#define SS2D_ERR_ALIGN 4       /* a pointer not aligned to its element size                 */
#define SS2D_ERR_HIP 5         /* a HIP runtime call failed (see ss2d_last_hip_error)       */
#define SS2D_ERR_ALIAS 6       /* an output overlaps an input (or another output)            */
#define SS2D_ERR_SCRATCH 7     /* ss2d_forward_noalloc: the call needs more scratch than
                                  SS2D_NOALLOC_SCRATCH_BYTES                               */

/* Data types of x, dt_raw, Bs, Cs and y. */
#define SS2D_F32 0
#define SS2D_BF16 1

/* Four-route SS2D forward.  x, y: (B, D, H, W); dt_raw: (B, 4, D, L); Bs, Cs: (B, 4, N, L);
 * A_log: (4, D, N); Ds, dt_bias: (4, D); L = H * W.  dtype is SS2D_F32 or SS2D_BF16.
 * Returns SS2D_OK or one of the SS2D_ERR_* codes above. */
int ss2d_forward(const void *x, const void *dt_raw, const float *A_log, const void *Bs,
                 const void *Cs, const float *Ds, const float *dt_bias, void *y, int64_t B,
                 int64_t D, int64_t H, int64_t W, int64_t N, int dtype, void *stream);

/* Bidirectional 1D selective scan forward (Vim block: forward route plus reversed route,
 * summed).  x, y: (B, D, L); dt_raw: (B, 2, D, L); Bs, Cs: (B, 2, N, L); A_log: (2, D, N);
 * Ds, dt_bias: (2, D).  Same dtypes, errors and conventions as ss2d_forward. */
int ss1d_bidir_forward(const void *x, const void *dt_raw, const float *A_log, const void *Bs,
                       const void *Cs, const float *Ds, const float *dt_bias, void *y,
                       int64_t B, int64_t D, int64_t L, int64_t N, int dtype, void *stream);

/* ---- options: gate and zero-order hold --------------------------------------------------
 * ss2d_forward_ex and ss1d_bidir_forward_ex take two more arguments than the plain entry
 * points (which equal them with z = NULL, flags = 0):
 *
 *   z      optional gate, NULL for none.  Same shape, layout and data type as x and y.
 *          Each route's output is multiplied by SiLU(z) = z / (1 + exp(-z)) at its image
 *          position before the routes are added (the Vim summary, section 4.3, "Gating and
 *          Merging": forward and backward outputs each gated by SiLU(z), then added; the
 *          explainer's MambaBlock multiplies the scan output by silu(z)).  As z is shared by
 *          the routes, the library applies SiLU(z) once to the fp32 sum, before the single
 *          rounding.  z must be aligned to its element size and must not overlap y.
 *   flags  0 or SS2D_FLAG_ZOH.  SS2D_FLAG_ZOH discretises B by zero-order hold as well:
 *          Bbar = (exp(delta A) - 1) / A * B in place of delta * B (the Vim summary,
 *          section 4.1: Bbar = (delta A)^-1 (exp(delta A) - I) delta B); A = 0 takes the
 *          limit delta * B.  Unknown bits give SS2D_ERR_UNSUPPORTED.
 *
 * Every other argument, error and convention is that of the plain entry point. */
#define SS2D_FLAG_ZOH 1

int ss2d_forward_ex(const void *x, const void *dt_raw, const float *A_log, const void *Bs,
                    const void *Cs, const float *Ds, const float *dt_bias, const void *z,
                    void *y, int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype,
                    int flags, void *stream);

int ss1d_bidir_forward_ex(const void *x, const void *dt_raw, const float *A_log,
                          const void *Bs, const void *Cs, const float *Ds,
                          const float *dt_bias, const void *z, void *y, int64_t B, int64_t D,
                          int64_t L, int64_t N, int dtype, int flags, void *stream);

/* ---- the forward without allocation ----------------------------------------------------------
 * For callers that cannot allocate device memory during the call: code under HIP graph
 * capture that must not record allocation nodes, tight serving loops, harnesses that forbid
 * hipMalloc.  ss2d_forward_noalloc is ss2d_forward_ex (same arguments, same kernels, same
 * result bit for bit) except for its scratch (the transposed copy of x, the per-route fp32
 * outputs, chunk carries): instead of the stream-ordered pool it uses a fixed device array
 * of SS2D_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs on until the
 * process ends.  The call allocates and frees nothing (no hipMalloc, hipFree or stream-
 * ordered allocation; the array's address is looked up once per device at its first call).
 *
 * Size limit: the scratch a call needs is about 2 bytes per element of x for the
 * transposed copy (4 for fp32 data) plus 16 bytes per element of x for the four routes'
 * fp32 outputs, plus chunk carries when the plan cuts long sequences (e.g. the fp32
 * VMamba-T stage-1 shape with B = 8, D = 192, 56 x 56, N = 16 needs ~103 MB); a call needing
 * more returns SS2D_ERR_SCRATCH before anything is enqueued.  Use ss2d_forward_ex for
 * larger calls.
 *
 * Every call on one device shares that device's array, which keeps the last call's
 * contents (nothing in it needs to start at zero): two calls that overlap in time on one
 * device (on different streams, or from different host threads) race on it and give
 * undefined results.  Calls on one stream are ordered and safe. */
#define SS2D_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int ss2d_forward_noalloc(const void *x, const void *dt_raw, const float *A_log, const void *Bs,
                         const void *Cs, const float *Ds, const float *dt_bias, const void *z,
                         void *y, int64_t B, int64_t D, int64_t H, int64_t W, int64_t N,
                         int dtype, int flags, void *stream);

/* ---- backward ---------------------------------------------------------------------------
 * Gradients of the scalar sum over (b, d, l) of dy[b, d, l] * y[b, d, l], y being the output
 * of ss2d_forward (ss1d_bidir_forward) on the same inputs, with respect to every input:
 *   dx (shape of x), ddt_raw (shape of dt_raw), dBs, dCs (shape of Bs, Cs): the data type
 *     of x (dtype), each rounded once from an fp32 sum;
 *   dA_log (K, D, N), dDs (K, D), ddt_bias (K, D): fp32.
 * dy has the shape and data type of x.  Every output is written in full (not accumulated
 * into) and must overlap neither an input nor another output.
 *
 * The gradients follow reverse-mode differentiation of the forward recurrence (the Vim
 * summary, section 4.4: the backward pass recomputes the intermediate states instead of
 * storing them): per route, the adjoint lambda_t = dy_t C_t + Abar_t+1 lambda_t+1 runs
 * backwards from the end of the sequence; dC_t += dy_t h_t and dB_t += lambda_t delta_t u_t
 * are summed over the channels that share Bs and Cs; delta's gradient passes softplus'
 * derivative sigmoid(dt_raw + dt_bias).  States are recomputed from checkpoints taken every
 * 32 steps (scratch, 4 B * B * K * D * ceil(L / 32) * N); sums over channels and images are
 * taken in a fixed order, so results are deterministic.
 *
 * Supported: the plain operator (no gate, delta * B; ss2d_backward_ex below takes the gate
 * and the zero-order hold) with N in {1, 2, 4, 8, 16, 32}, as the forward; other N give
 * SS2D_ERR_UNSUPPORTED.  The kernels split each channel's states over four lanes: N = 1
 * and 2 run as four states, the extra ones with zero B and C rows, which keep them exactly
 * zero (scratch: padded copies of Bs, Cs and A_log and of their gradients); N = 32 runs at
 * two waves per SIMD.  Otherwise the conventions of ss2d_forward apply. */
int ss2d_backward(const void *x, const void *dt_raw, const float *A_log, const void *Bs,
                  const void *Cs, const float *Ds, const float *dt_bias, const void *dy,
                  void *dx, void *ddt_raw, float *dA_log, void *dBs, void *dCs, float *dDs,
                  float *ddt_bias, int64_t B, int64_t D, int64_t H, int64_t W, int64_t N,
                  int dtype, void *stream);

int ss1d_bidir_backward(const void *x, const void *dt_raw, const float *A_log,
                        const void *Bs, const void *Cs, const float *Ds,
                        const float *dt_bias, const void *dy, void *dx, void *ddt_raw,
                        float *dA_log, void *dBs, void *dCs, float *dDs, float *ddt_bias,
                        int64_t B, int64_t D, int64_t L, int64_t N, int dtype, void *stream);

/* ---- backward of the gated and the zero-order-hold operator --------------------------------
 * Gradients of the scalar sum over (b, d, l) of dy[b, d, l] * y[b, d, l], y being the output
 * of ss2d_forward_ex (ss1d_bidir_forward_ex) with the same gate z and flags.  With z = NULL
 * and flags = 0 this is ss2d_backward (ss1d_bidir_backward).
 *
 * Gate (z not NULL): y = (sum over the routes of y_k) * SiLU(z) (the gate of the Vim block,
 * Vim summary section 4.3; the explainer's SelectiveSSM output multiplied by the activated
 * z branch).  By the product rule every route's output receives g = dy * SiLU(z), and
 *   dz = dy * ys * SiLU'(z),   SiLU'(z) = sigmoid(z) * (1 + z * (1 - sigmoid(z))),
 * with ys the ungated route sum; dz (the shape and data type of x) must then be given, is
 * written in full and must overlap neither an input nor another output (with z = NULL, dz
 * is not used).  The checkpoint pass also writes the per-route outputs (scratch, fp32, as
 * in the forward), and the merge kernel forms g and dz from them; g stays in fp32 (scratch,
 * 4 B * B * D * L, twice that for the four routes' transposed copy) whatever the data type,
 * so that bfloat16 data lose nothing to a rounding of the gated gradient.
 *
 * SS2D_FLAG_ZOH: the zero-order-hold operator (Vim summary section 4.1), whose update is
 * h = a h + bb B u with a = exp(delta A) and bb = (a - 1) / A.  The adjoint recurrence is
 * unchanged; with bb in place of delta, dBs sums lambda * bb * u and dx sums
 * lambda * bb * B; d bb / d delta = a, so ddelta takes sum_n lambda * a * B * u in place of
 * sum_n lambda * B * u; and dA_log gains A * lambda * B * u * d bb / dA with
 * d bb / dA = delta^2 * psi(delta A), psi(v) = (v e^v - (e^v - 1)) / v^2 (its power series
 * for |v| < 1/4).
 *
 * Everything else, supported shapes and errors included, is as in ss2d_backward; flags
 * other than SS2D_FLAG_ZOH give SS2D_ERR_UNSUPPORTED. */
int ss2d_backward_ex(const void *x, const void *dt_raw, const float *A_log, const void *Bs,
                     const void *Cs, const float *Ds, const float *dt_bias, const void *z,
                     const void *dy, void *dx, void *ddt_raw, float *dA_log, void *dBs,
                     void *dCs, float *dDs, float *ddt_bias, void *dz, int64_t B, int64_t D,
                     int64_t H, int64_t W, int64_t N, int dtype, int flags, void *stream);

int ss1d_bidir_backward_ex(const void *x, const void *dt_raw, const float *A_log,
                           const void *Bs, const void *Cs, const float *Ds,
                           const float *dt_bias, const void *z, const void *dy, void *dx,
                           void *ddt_raw, float *dA_log, void *dBs, void *dCs, float *dDs,
                           float *ddt_bias, void *dz, int64_t B, int64_t D, int64_t L,
                           int64_t N, int dtype, int flags, void *stream);

/* ---- training: a forward that keeps the backward's checkpoints ---------------------------
 * In training the forward and the backward run on the same inputs.  The backward restarts
 * every 8-step quarter of the scan from the state before it, which ss2d_backward_ex obtains
 * by running the forward scan once more (the Vim summary, section 4.4: states are
 * recomputed, not kept in HBM per step); ss2d_forward_save keeps those states while it
 * computes y, and ss2d_backward_saved starts from them, so that the pair does the scan's
 * forward work once.
 *
 * saved: caller-owned device memory of ss2d_saved_state_bytes(K, B, D, L, N, gated) bytes
 * (K = 4 with L = H * W for the image operators, K = 2 for the bidirectional one; gated:
 * whether z is given), 16-byte aligned.  Layout: the state before every 8-step quarter,
 * (B, K, D, ceil(L / 8), N) fp32 (the first quarter's, zero, is not written; 16 bytes per
 * element of x for N = 16), then with the
 * gate the ungated route sum ((y_0 + y_1) + y_2) + y_3, (B, D, L) fp32, from which the
 * gate's backward forms g and dz.  ss2d_saved_state_bytes returns -1 for sizes the
 * operator rejects and for N not a multiple of 4.
 *
 * ss2d_forward_save: y as ss2d_forward_ex with the same arguments (bit for bit when that
 * call runs in one pass, i.e. without the chunked plan it takes for batches too small to
 * fill the chip; the training forward always runs one pass), and `saved` filled.
 * ss2d_backward_saved: every gradient as ss2d_backward_ex, bit for bit, reading `saved`
 * instead of recomputing it.  The backward's inputs, z, flags and shapes must be those of
 * the forward that filled `saved`, and `saved` unchanged since; the library cannot check
 * this (the state lives on the device), and other contents give undefined gradients.
 * `saved` overlaps no other argument.  N must be a multiple of 4 (SS2D_ERR_UNSUPPORTED
 * otherwise); everything else is as in ss2d_forward_ex and ss2d_backward_ex. */
int64_t ss2d_saved_state_bytes(int K, int64_t B, int64_t D, int64_t L, int64_t N, int gated);

int ss2d_forward_save(const void *x, const void *dt_raw, const float *A_log, const void *Bs,
                      const void *Cs, const float *Ds, const float *dt_bias, const void *z,
                      void *y, float *saved, int64_t B, int64_t D, int64_t H, int64_t W,
                      int64_t N, int dtype, int flags, void *stream);

int ss1d_bidir_forward_save(const void *x, const void *dt_raw, const float *A_log,
                            const void *Bs, const void *Cs, const float *Ds,
                            const float *dt_bias, const void *z, void *y, float *saved,
                            int64_t B, int64_t D, int64_t L, int64_t N, int dtype, int flags,
                            void *stream);

int ss2d_backward_saved(const void *x, const void *dt_raw, const float *A_log, const void *Bs,
                        const void *Cs, const float *Ds, const float *dt_bias, const void *z,
                        const float *saved, const void *dy, void *dx, void *ddt_raw,
                        float *dA_log, void *dBs, void *dCs, float *dDs, float *ddt_bias,
                        void *dz, int64_t B, int64_t D, int64_t H, int64_t W, int64_t N,
                        int dtype, int flags, void *stream);

int ss1d_bidir_backward_saved(const void *x, const void *dt_raw, const float *A_log,
                              const void *Bs, const void *Cs, const float *Ds,
                              const float *dt_bias, const void *z, const float *saved,
                              const void *dy, void *dx, void *ddt_raw, float *dA_log, void *dBs,
                              void *dCs, float *dDs, float *ddt_bias, void *dz, int64_t B,
                              int64_t D, int64_t L, int64_t N, int dtype, int flags,
                              void *stream);

/* The same pair for the operator over per-route inputs (ss2d_forward_routes,
 * ss2d_backward_routes): u (B, K, D, L) in place of x, du in place of dx; the saved state's
 * size and layout are those above. */
int ss2d_forward_routes_save(const void *u, const void *dt_raw, const float *A_log,
                             const void *Bs, const void *Cs, const float *Ds,
                             const float *dt_bias, const void *z, void *y, float *saved,
                             int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype,
                             int flags, void *stream);

int ss1d_bidir_forward_routes_save(const void *u, const void *dt_raw, const float *A_log,
                                   const void *Bs, const void *Cs, const float *Ds,
                                   const float *dt_bias, const void *z, void *y, float *saved,
                                   int64_t B, int64_t D, int64_t L, int64_t N, int dtype,
                                   int flags, void *stream);

int ss2d_backward_routes_saved(const void *u, const void *dt_raw, const float *A_log,
                               const void *Bs, const void *Cs, const float *Ds,
                               const float *dt_bias, const void *z, const float *saved,
                               const void *dy, void *du, void *ddt_raw, float *dA_log, void *dBs,
                               void *dCs, float *dDs, float *ddt_bias, void *dz, int64_t B,
                               int64_t D, int64_t H, int64_t W, int64_t N, int dtype, int flags,
                               void *stream);

int ss1d_bidir_backward_routes_saved(const void *u, const void *dt_raw, const float *A_log,
                                     const void *Bs, const void *Cs, const float *Ds,
                                     const float *dt_bias, const void *z, const float *saved,
                                     const void *dy, void *du, void *ddt_raw, float *dA_log,
                                     void *dBs, void *dCs, float *dDs, float *ddt_bias, void *dz,
                                     int64_t B, int64_t D, int64_t L, int64_t N, int dtype,
                                     int flags, void *stream);

/* ---- backward of the operator over per-route inputs ---------------------------------------
 * Gradients of the scalar sum over (b, d, l) of dy[b, d, l] * y[b, d, l], y being the output
 * of ss2d_forward_routes (ss1d_bidir_forward_routes) on the same inputs, gate z and flags:
 * the gradients of ss2d_backward_ex, but with each route's own input u (B, K, D, L, in scan
 * order, the data type) in place of x, and du of that shape (the gradient of route k's
 * input at step t; the routes share no input, so nothing is summed across them) in place of
 * dx.  This is the gradient that the per-route front end (ss2d_project) continues with.
 * Every other argument, error and convention is that of ss2d_backward_ex. */
int ss2d_backward_routes(const void *u, const void *dt_raw, const float *A_log, const void *Bs,
                         const void *Cs, const float *Ds, const float *dt_bias, const void *z,
                         const void *dy, void *du, void *ddt_raw, float *dA_log, void *dBs,
                         void *dCs, float *dDs, float *ddt_bias, void *dz, int64_t B,
                         int64_t D, int64_t H, int64_t W, int64_t N, int dtype, int flags,
                         void *stream);

int ss1d_bidir_backward_routes(const void *u, const void *dt_raw, const float *A_log,
                               const void *Bs, const void *Cs, const float *Ds,
                               const float *dt_bias, const void *z, const void *dy, void *du,
                               void *ddt_raw, float *dA_log, void *dBs, void *dCs, float *dDs,
                               float *ddt_bias, void *dz, int64_t B, int64_t D, int64_t L,
                               int64_t N, int dtype, int flags, void *stream);

/* ---- per-route front end and the operator over per-route inputs ---------------------------
 * In the pages' per-direction modules every scan direction carries its own input layers: the
 * explainer's CrossScanModule holds one SelectiveSSM per direction (a depthwise Conv1d with
 * kernel d_conv and padding d_conv - 1 cut to the first L outputs, a SiLU, x_proj to
 * [dt, B, C] and dt_proj), and in the Vim block (Vim summary, section 4.3) each path runs a
 * Conv1d and a SiLU on its own copy of the sequence and generates delta, B and C from the
 * activated output, which is also the input of that path's scan.
 *
 * ss2d_project computes, for every route k and image b, from the shared input x (B, D, H, W)
 * [ss1d_bidir_project: (B, D, L), routes forward and reversed], with s_t = x[b, d, pi_k(t)]
 * and s_t = 0 for t < 0:
 *   u[b,k,d,t]      = SiLU(conv_b[k,d] + sum_{j<KW} conv_w[k,d,j] * s_{t-KW+1+j})
 *   xd[m,t]         = sum_d x_proj_w[k,m,d] * u[b,k,d,t]        m < R + 2N (no bias)
 *   dt_raw[b,k,d,t] = sum_{r<R} dt_proj_w[k,d,r] * xd[r,t]      (dt_proj's bias is dt_bias,
 *                                                               added inside the softplus)
 *   Bs[b,k,n,t]     = xd[R+n,t],   Cs[b,k,n,t] = xd[R+N+n,t]
 * i.e. a causal conv along each route (route 1 is causal in reversed raster order, routes 2
 * and 3 along columns), x_proj's output split [dt (R) | B (N) | C (N)].  Outputs, in the
 * scan order of each route, are exactly the inputs of ss2d_forward_routes:
 *   u, dt_raw (B, K, D, L) and Bs, Cs (B, K, N, L) in dtype;
 *   weights conv_w (K, D, KW), conv_b (K, D), x_proj_w (K, R + 2N, D), dt_proj_w (K, D, R):
 *   fp32, read only.
 * Supported: 1 <= KW <= 8, R >= 1, R + 2N <= 96 (else SS2D_ERR_UNSUPPORTED).  Every output is
 * written in full and must overlap neither an input nor another output (SS2D_ERR_ALIAS).
 * The conv and dt_proj are computed in fp32; x_proj accumulates in fp32 on the matrix cores
 * from u as stored (for bf16, the stored bf16 u, with each fp32 weight split into two bf16
 * parts whose sum carries 16 significant bits).  Scratch: a transposed copy of x for the
 * column routes (stream-ordered, as in ss2d_forward).
 *
 * ss2d_forward_routes is ss2d_forward_ex with each route's own input u (B, K, D, L), in scan
 * order, in place of the gathered x: step t of route k reads u[b,k,d,t] for both the update
 * (delta * B * u) and the skip term (Ds * u); outputs are added at the visited positions in
 * route order, optionally gated by z (B, D, H, W), with flags as in ss2d_forward_ex.
 * Every other argument, error and convention is that of ss2d_forward_ex. */
int ss2d_project(const void *x, const float *conv_w, const float *conv_b,
                 const float *x_proj_w, const float *dt_proj_w, void *u, void *dt_raw, void *Bs,
                 void *Cs, int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int64_t R,
                 int64_t KW, int dtype, void *stream);

int ss1d_bidir_project(const void *x, const float *conv_w, const float *conv_b,
                       const float *x_proj_w, const float *dt_proj_w, void *u, void *dt_raw,
                       void *Bs, void *Cs, int64_t B, int64_t D, int64_t L, int64_t N,
                       int64_t R, int64_t KW, int dtype, void *stream);

int ss2d_forward_routes(const void *u, const void *dt_raw, const float *A_log, const void *Bs,
                        const void *Cs, const float *Ds, const float *dt_bias, const void *z,
                        void *y, int64_t B, int64_t D, int64_t H, int64_t W, int64_t N,
                        int dtype, int flags, void *stream);

int ss1d_bidir_forward_routes(const void *u, const void *dt_raw, const float *A_log,
                              const void *Bs, const void *Cs, const float *Ds,
                              const float *dt_bias, const void *z, void *y, int64_t B,
                              int64_t D, int64_t L, int64_t N, int dtype, int flags,
                              void *stream);

/* ---- the front end and the operator with dt_proj folded into the scan ---------------------
 * dt_proj is linear and has no bias of its own (its bias is dt_bias, added inside the
 * softplus), and the explainer's SelectiveSSM applies it to the R-row dt slice of x_proj's
 * output (dt_rank = ceil(d_model / 16), a low rank): step t's dt_raw[d] is
 * sum_{r<R} dt_proj_w[k,d,r] * xd[r,t].  Forming that sum inside the scan, from the R rows
 * instead of the D rows, leaves the operator unchanged and removes dt_raw (B, K, D, L) from
 * memory: the front end stores the R dt rows and the scan reads them back.
 *
 * ss2d_project_lr / ss1d_bidir_project_lr are ss2d_project / ss1d_bidir_project without
 * dt_proj: in place of dt_raw they write dt_lr[b,k,r,t] = xd[r,t] (B, K, R, L) in dtype, and
 * take no dt_proj_w.  Every other output, argument and error is as there.
 *
 * ss2d_forward_routes_lr / ss1d_bidir_forward_routes_lr are ss2d_forward_routes /
 * ss1d_bidir_forward_routes with dt_raw given as the product
 *   dt_raw[b,k,d,t] = sum_{r<R} dt_w[k,d,r] * dt_lr[b,k,r,t]
 * formed in fp32 at every step (dt_lr (B, K, R, L) in dtype, dt_w (K, D, R) fp32, both read
 * only).  Supported: 1 <= R <= 4 (else SS2D_ERR_UNSUPPORTED); y must overlap neither dt_lr
 * nor dt_w (SS2D_ERR_ALIAS); NULL dt_lr or dt_w gives SS2D_ERR_NULL.  Every other argument,
 * error and convention is that of ss2d_forward_routes. */
int ss2d_project_lr(const void *x, const float *conv_w, const float *conv_b,
                    const float *x_proj_w, void *u, void *dt_lr, void *Bs, void *Cs, int64_t B,
                    int64_t D, int64_t H, int64_t W, int64_t N, int64_t R, int64_t KW,
                    int dtype, void *stream);

int ss1d_bidir_project_lr(const void *x, const float *conv_w, const float *conv_b,
                          const float *x_proj_w, void *u, void *dt_lr, void *Bs, void *Cs,
                          int64_t B, int64_t D, int64_t L, int64_t N, int64_t R, int64_t KW,
                          int dtype, void *stream);

int ss2d_forward_routes_lr(const void *u, const void *dt_lr, const float *dt_w,
                           const float *A_log, const void *Bs, const void *Cs, const float *Ds,
                           const float *dt_bias, const void *z, void *y, int64_t B, int64_t D,
                           int64_t H, int64_t W, int64_t N, int64_t R, int dtype, int flags,
                           void *stream);

int ss1d_bidir_forward_routes_lr(const void *u, const void *dt_lr, const float *dt_w,
                                 const float *A_log, const void *Bs, const void *Cs,
                                 const float *Ds, const float *dt_bias, const void *z, void *y,
                                 int64_t B, int64_t D, int64_t L, int64_t N, int64_t R,
                                 int dtype, int flags, void *stream);

/* ---- launch-plan override (testing and tuning, not part of the operator) ---------------
 * Sets, for calls made later from the calling host thread only, the lanes that share one
 * channel's states in the forward scan (split: 1, 2 or 4; 0 = automatic) and the chunk
 * length of the chunked scan (chunk_len: 0 = one pass, > 0 = chunks of that many steps
 * rounded up to a multiple of 32, -1 = automatic).  The override changes how the work is
 * cut, not what is computed: any setting gives the operator's result (to rounding, which
 * may differ with the cut).  A split that does not divide N, or split 2 with chunks, falls
 * back to what the kernels support.  Returns SS2D_OK, SS2D_ERR_UNSUPPORTED for another
 * split, or SS2D_ERR_SHAPE for chunk_len < -1 or >= 2^30.  The default on every thread is
 * automatic (0, -1); no environment variable is read. */
int ss2d_set_launch_plan(int split, int64_t chunk_len);

/* Static, human-readable text for a status code (never NULL). */
const char *ss2d_status_string(int status);

/* SS2D_ABI_VERSION of the loaded library. */
int ss2d_abi_version(void);

/* hipError_t value of the last failed HIP call made by this library on the calling thread
 * (0 if none). */
int ss2d_last_hip_error(void);

/* ---- scratch pool (memory management, not part of the operator) -----------------------
 * Hands the device memory that the library's scratch pool on the calling thread's current
 * device reserves beyond keep_bytes back to the driver (hipMemPoolTrimTo), for callers that
 * need it for other allocations between calls; later calls allocate it again.  Writes the
 * bytes the pool still reserves afterwards to *reserved (may be NULL).  Only memory that
 * no call uses is released: scratch of a call still running, or whose release is still
 * pending on its stream, stays reserved, so synchronise the streams of earlier calls first.
 * On a device where the library has made no call there is no pool: SS2D_OK with
 * *reserved = 0.  Returns SS2D_OK or SS2D_ERR_HIP. */
int ss2d_scratch_trim(size_t keep_bytes, size_t *reserved);

/* ---- kernel timing (measurement support, not part of the operator) -----------------------
 * While enabled on a host thread, every call from that thread brackets each kernel launch
 * with a pair of HIP events on the call's stream.  ss2d_timing_read waits for the recorded
 * events, adds each kernel's duration to its kind, writes per-kind totals (milliseconds)
 * and launch counts to ms[SS2D_KERNEL_KINDS] and launches[SS2D_KERNEL_KINDS] (either may be
 * NULL), and clears the record.  ss2d_timing_enable returns the previous setting. */
#define SS2D_KERNEL_TRANSPOSE 0 /* per-plane transpose of x for the column routes      */
#define SS2D_KERNEL_SCAN 1      /* selective scan producing per-route outputs          */
#define SS2D_KERNEL_CHUNK_AGG 2 /* chunked scan, first pass (chunk end states)         */
#define SS2D_KERNEL_CARRY 3     /* not launched: chunk start states are composed in the
                                   scan's second pass (the kind keeps its number)        */
#define SS2D_KERNEL_MERGE 4     /* cross-merge into y (backward: route gradients into dx) */
#define SS2D_KERNEL_CHECKPOINT 5 /* backward: forward pass storing states every 8 steps  */
#define SS2D_KERNEL_SCAN_BWD 6  /* backward: adjoint scan                               */
#define SS2D_KERNEL_REDUCE 7    /* backward: sums over channel blocks and images         */
#define SS2D_KERNEL_PROJECT 8   /* per-route front end: conv + SiLU, x_proj, dt_proj      */
#define SS2D_KERNEL_KINDS 9
int ss2d_timing_enable(int enable);
int ss2d_timing_read(double *ms, int64_t *launches);

/* ---- issue-rate probe (measurement support, not part of the operator) ------------------
 * Measures, on the current device and `stream`, the instruction rates that bound the scan
 * kernel (whose state update issues 2 multiplies, 2 fused multiply-adds and one v_exp_f32
 * per state and step): three probe kernels at full occupancy (8 waves per SIMD, 8
 * independent chains per lane), after ~0.1 s of warm-up load, best of 3 runs each.  Writes
 *   out[0]  fp32 fused multiply-adds per second (lane operations),
 *   out[1]  v_exp_f32 per second (lane operations),
 *   out[2]  groups of 4 fused multiply-adds and 1 v_exp_f32 per second (one update's mix:
 *           a multiply issues like a fused multiply-add),
 *   out[3]  the shader clock the chip sustained during the grouped probe (Hz), from the
 *           shader and the 100 MHz reference counters,
 *   out[4]  the device's compute units,
 * to out[SS2D_PROBE_OUTPUTS] (caller-owned host memory).  Synchronises `stream`; takes
 * ~0.2 s.  Returns SS2D_OK, SS2D_ERR_NULL, or SS2D_ERR_HIP. */
#define SS2D_PROBE_OUTPUTS 5
int ss2d_probe_issue_rates(double *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SS2D_H */
