// Device-side helpers and launch interfaces shared by the SS2D kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss2d {

constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kChunkAlign = 32;  // chunk lengths are multiples of this (any tile length divides it)
constexpr int kMaxBlock = 256;   // threads per block of the scan kernel (4 waves)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- element types ---------------------------------------------------------------------
// x, dt_raw, Bs, Cs and y are either fp32 or bfloat16 (raw 16-bit patterns in uint16_t).
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float to_f32(float v) { return v; }
  static __device__ __forceinline__ float from_f32(float v) { return v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float to_f32(uint16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
  }
  static __device__ __forceinline__ float load(const uint16_t* p) { return to_f32(*p); }
  // fp32 -> bfloat16 by the hardware conversion (v_cvt_pk_bf16_f32): round to nearest
  // even; NaN stays a NaN.
  static __device__ __forceinline__ uint16_t from_f32(float v) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
  }
};

// ---- arithmetic ------------------------------------------------------------------------
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// SiLU(v) = v / (1 + e^-v), the gate nonlinearity, with the hardware reciprocal (about
// 1 ulp).  v -> -inf gives -0 (the reciprocal of +inf), v = +inf gives +inf.
__device__ __forceinline__ float silu_f32(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + exp2_hw(-v * kLog2e));
}

// softplus(z) = log(1 + e^z) = max(z, 0) + log1p(e) with e = e^-|z| in (0, 1].  With
// u = 1 + e rounded, c = e - (u - 1) is exactly the rounding error of u, and
// log1p(e) = log(u) + log(1 + c/u) = log(u) + c up to c * (1 - 1/u) <= 2^-24 * log1p(e):
// one log2 and three adds recover the accuracy a plain log(1 + e) loses for small e.
__device__ __forceinline__ float softplus_f32(float z) {
  const float e = exp2_hw(-fabsf(z) * kLog2e);
  const float u = 1.0f + e;
  const float c = e - (u - 1.0f);
  const float l1p = fmaf(__builtin_amdgcn_logf(u), kLn2, c);
  return fmaxf(z, 0.0f) + l1p;
}

// Zero-order hold: B's factor (exp(delta A) - 1) / A = delta * phi(delta A) in one update,
// with phi(v) = (e^v - 1) / v.  For |v| >= 1/16 the update's own exponential
// a = exp(delta A) gives (a - 1) / A to within ~1e-6 relative (a - 1 is exact and a carries
// one rounding); below that, a - 1 would lose digits to cancellation, and phi's Taylor
// polynomial to v^3 (truncation <= v^4 / 120 < 2e-7) is used instead.  Written in
// xa = delta A log2(e), the exponent the update already computes (v = xa ln 2); invA = 1 / A.
constexpr float kZohSmallX = 0.0625f / 0.69314718f;      // |xa| below which the series is used
constexpr float kZohP1 = 0.69314718f / 2.0f;             // ln2 / 2
constexpr float kZohP2 = 0.48045301f / 6.0f;             // ln2^2 / 6
constexpr float kZohP3 = 0.33302465f / 24.0f;            // ln2^3 / 24
__device__ __forceinline__ float zoh_bbar(float dl, float xa, float an, float invA) {
  const float series = dl * fmaf(xa, fmaf(xa, fmaf(xa, kZohP3, kZohP2), kZohP1), 1.0f);
  const float direct = fmaf(an, invA, -invA);  // (a - 1) / A
  return fabsf(xa) < kZohSmallX ? series : direct;
}

// Derivative in A of that factor: d/dA (exp(delta A) - 1) / A = (delta a - bbar) / A
// = delta^2 psi(v), psi(v) = (v e^v - (e^v - 1)) / v^2 = sum_k v^k (k + 1) / (k + 2)!.  The
// difference delta a - bbar ~ delta v / 2 cancels: from a and bbar (each good to about
// 6e-8 / |v| relative) only for |v| >= 1/4 (~2e-6 relative there); below, psi's polynomial
// to v^5 (truncation <= v^6 / 5760 relative to 1/2, < 1e-7), in xa as above.
constexpr float kPsiSmallX = 0.25f / 0.69314718f;        // |xa| below which the series is used
constexpr float kPsiQ1 = 0.69314718f / 3.0f;             // ln2 / 3
constexpr float kPsiQ2 = 0.48045301f / 8.0f;             // ln2^2 / 8
constexpr float kPsiQ3 = 0.33302465f / 30.0f;            // ln2^3 / 30
constexpr float kPsiQ4 = 0.23083510f / 144.0f;           // ln2^4 / 144
constexpr float kPsiQ5 = 0.16000270f / 840.0f;           // ln2^5 / 840
__device__ __forceinline__ float zoh_bbar_dA(float dl, float xa, float an, float bbar,
                                             float invA) {
  const float poly = fmaf(xa, fmaf(xa, fmaf(xa, fmaf(xa, fmaf(xa, kPsiQ5, kPsiQ4), kPsiQ3),
                                                kPsiQ2), kPsiQ1), 0.5f);
  const float direct = fmaf(dl, an, -bbar) * invA;
  return fabsf(xa) < kPsiSmallX ? dl * dl * poly : direct;
}

// Workgroups are handed to the 8 XCDs of the chip round-robin in linear launch order, and
// each XCD has its own L2.  This maps the linear workgroup index to a logical one so that
// logically consecutive workgroups (which share inputs) run on the same XCD: XCD j gets
// the j-th contiguous range of logical indices.
constexpr int kNumXcd = 8;
__device__ __forceinline__ unsigned xcd_local_order(unsigned lin, unsigned total) {
  const unsigned q = total / kNumXcd, r = total % kNumXcd;
  const unsigned j = lin % kNumXcd, i = lin / kNumXcd;
  return j * q + min(j, r) + i;
}

// Issue priority of a wave from its progress through `total` work units: 3 for the first
// half, 2 to three quarters, 1 to nine tenths, 0 for the rest.  Among waves of equal
// priority a SIMD issues from the oldest first, so co-resident blocks that start together
// would otherwise finish far apart, the last one running alone at low utilisation; with
// falling priority a wave that runs ahead yields to those behind it.
__device__ __forceinline__ void progress_priority(int done, int total) {
  const long long d = done, t = total;
  if (2 * d < t) __builtin_amdgcn_s_setprio(3);
  else if (4 * d < 3 * t) __builtin_amdgcn_s_setprio(2);
  else if (10 * d < 9 * t) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// DPP quad_perm helpers (lanes exchange values inside groups of four).  Every lane reads a
// lane of its own quad, so no lane is out of bounds and the old value never shows through:
// bound_ctrl lets the compiler drop the move that would initialise it (or fold the
// permutation into the instruction that consumes it).
template <int P0, int P1, int P2, int P3>
__device__ __forceinline__ float quad_perm(float v) {
  constexpr int ctrl = P0 | (P1 << 2) | (P2 << 4) | (P3 << 6);
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, true));
}

// Value of `v` held by lane q of this lane's channel group (S lanes per channel).
template <int S>
__device__ __forceinline__ float from_owner(float v, int q) {
  if constexpr (S == 1) {
    return v;
  } else if constexpr (S == 2) {
    switch (q) {
      case 0: return quad_perm<0, 0, 2, 2>(v);
      default: return quad_perm<1, 1, 3, 3>(v);
    }
  } else {
    switch (q) {
      case 0: return quad_perm<0, 0, 0, 0>(v);
      case 1: return quad_perm<1, 1, 1, 1>(v);
      case 2: return quad_perm<2, 2, 2, 2>(v);
      default: return quad_perm<3, 3, 3, 3>(v);
    }
  }
}

// Sum of `v` over the S lanes of this lane's channel group, in every one of them.
template <int S>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (S >= 2) v += quad_perm<1, 0, 3, 2>(v);
  if constexpr (S == 4) v += quad_perm<2, 3, 0, 1>(v);
  return v;
}

// ---- launch arguments ------------------------------------------------------------------
struct ScanArgs {
  const void* x_row;      // route source for routes 0 and 1: x, (B, D, L); with x_routes set,
                          // every route's own input u, (B, K, D, L) in scan order
  const void* x_col;      // route source for routes 2 and 3: x transposed per plane, (B, D, L)
  const void* dt_raw;     // (B, K, D, L)
  const void* Bs;         // (B, K, N, L)
  const void* Cs;         // (B, K, N, L)
  const float* A_log;     // (K, D, N)
  const float* Ds;        // (K, D)
  const float* dt_bias;   // (K, D)
  float* y_route;         // (B, K, D, L) fp32 per-route outputs in scan order
  float* h_end;           // (B, K, D, C, N) chunk end states from a zero start
  float* delta_sum;       // (B, K, D, C) sum of delta over each chunk
  float* h_in;            // kModeCkpt(Out): (B, K, D, ck_slots(L), N) states, slot c the
                          // state before step 8 c (slot 0, the zero state, not written)
  int B, K, D, L, N;
  int num_chunks;         // C
  int chunk_len;          // steps per chunk, a multiple of kChunkAlign (>= L when C == 1)
  int chunk_base;         // first chunk index covered by this launch
  int chunks_in_launch;   // chunks covered by this launch per (b, k)
  int zoh;                // nonzero: zero-order hold for B, (exp(delta A) - 1) / A * B
  int x_routes;           // nonzero: x_row holds each route's own input sequence
  const void* dt_lr;      // dt_proj folded in (else NULL): x_proj's dt rows (B, K, R, L) ...
  const float* dt_w;      // ... and the dt_proj weight (K, D, R): dt_raw = dt_w @ dt_lr
  int R;                  // rows of dt_lr, 1 .. kMaxLowRank
};
constexpr int kMaxLowRank = 4;  // dt rows a tile row of the scan's B/C LDS tile can hold

enum ScanMode { kModeOut = 0, kModeAgg = 1, kModeCkpt = 2, kModeCkptOut = 3 };

// Checkpoint slots per sequence of L steps: one per 8-step quarter of a 32-step tile.
__host__ __device__ constexpr int64_t ck_slots(int64_t L) { return (L + 7) / 8; }

// Arguments of the backward scan kernel (gradients of sum(dy * y), plain operator).
struct BwdArgs {
  const void* x_row;      // x, (B, D, L)
  const void* x_col;      // x transposed per plane (routes 2 and 3)
  const void* g_row;      // route gradient g (B, D, L): dy, or dy SiLU(z) for the gate
  const void* g_col;      // g transposed per plane
  const void* dt_raw;     // (B, K, D, L)
  const void* Bs;         // (B, K, N, L)
  const void* Cs;         // (B, K, N, L)
  const float* A_log;     // (K, D, N)
  const float* Ds;        // (K, D)
  const float* dt_bias;   // (K, D)
  const float* h_ck;      // (B, K, D, ck_slots(L), N) state before each 8-step quarter
                          // (slot c: before step 8 c; slot 0, the zero state, is not read)
  float* du_route;        // (B, K, D, L) fp32 dL/du per route, scan order
  void* ddt_raw;          // (B, K, D, L) gradient of dt_raw, element type of the inputs
  float* dbc_part;        // (B, K, n_cb, 2N, L) per channel-block sums of dB (rows < N), dC
  float* dA_part;         // (B, K, D, N) per-image gradient of A_log
  float* dD_part;         // (B, K, D) per-image gradient of Ds
  float* dbias_part;      // (B, K, D) per-image gradient of dt_bias
  int B, K, D, L, N;
  int ck_tiles;           // ceil(L / 32)
  int n_cb;               // channel blocks per (b, k): ceil(D / 64)
  int g_f32;              // nonzero: g is fp32 whatever the data type
  int zoh;                // nonzero: the zero-order-hold operator
  int x_routes;           // nonzero: x_row holds each route's own input (B, K, D, L) in scan
                          // order, and du goes to du_out (same shape, element type) instead
                          // of du_route
  void* du_out;
};

// Arguments of the per-route front end (causal depthwise conv + SiLU, x_proj, dt_proj).
struct ProjArgs {
  const void* x_row;        // x, (B, D, L): the source of routes 0 and 1 (K = 2: both)
  const void* x_col;        // x transposed per plane: the source of routes 2 and 3
  const float* conv_w;      // (K, D, KW)
  const float* conv_b;      // (K, D)
  const float* x_proj_w;    // (K, R + 2N, D)
  const float* dt_proj_w;   // (K, D, R)
  void* u;                  // (B, K, D, L) conv + SiLU output, scan order
  void* dt_raw;             // (B, K, D, L)
  void* Bs;                 // (B, K, N, L)
  void* Cs;                 // (B, K, N, L)
  void* dt_lr;              // not NULL: x_proj's R dt rows (B, K, R, L) are stored here and
                            // dt_proj is not applied (dt_raw and dt_proj_w are unused)
  const void* wprep;        // per (k, 64-channel chunk): x_proj weights and conv taps laid
                            // out as the kernel's LDS image, img_bytes each
  int B, K, D, L, N, R, KW;
  int nchunks;              // ceil(D / 64)
  int img_bytes;
};
constexpr int kProjMaxKW = 8;   // longest conv supported
constexpr int kProjMaxM = 96;   // most x_proj rows (R + 2N) supported

// Host-side launchers (defined in the .hip files).  The _zoh scan launchers run the
// zero-order-hold discretisation of B (a.zoh set), the others delta * B.
int launch_scan_f32(const ScanArgs& a, int split, int mode, hipStream_t st);
int launch_scan_bf16(const ScanArgs& a, int split, int mode, hipStream_t st);
int launch_scan_f32_zoh(const ScanArgs& a, int split, int mode, hipStream_t st);
int launch_scan_bf16_zoh(const ScanArgs& a, int split, int mode, hipStream_t st);
// dt_proj folded in (a.dt_lr set): forward modes only
int launch_scan_f32_lr(const ScanArgs& a, int split, int mode, hipStream_t st);
int launch_scan_bf16_lr(const ScanArgs& a, int split, int mode, hipStream_t st);
int launch_scan_f32_zoh_lr(const ScanArgs& a, int split, int mode, hipStream_t st);
int launch_scan_bf16_zoh_lr(const ScanArgs& a, int split, int mode, hipStream_t st);
int launch_transpose(const void* x, void* xt, int B, int D, int H, int W, int dtype,
                     hipStream_t st);
int launch_scan_bwd_f32(const BwdArgs& a, hipStream_t st);
int launch_scan_bwd_bf16(const BwdArgs& a, hipStream_t st);
int launch_scan_bwd_f32_zoh(const BwdArgs& a, hipStream_t st);
int launch_scan_bwd_bf16_zoh(const BwdArgs& a, hipStream_t st);
// Sums of the backward partials: dBs, dCs over channel blocks; dA_log, dDs, dt_bias over
// images (fixed order).
int launch_bwd_reduce_bc(const float* part, void* dBs, void* dCs, int B, int K, int N, int L,
                         int n_cb, int dtype, hipStream_t st);
// Copies blocks of rows_in rows of len elements (2 or 4 bytes each) into blocks of rows_out
// rows, zero-filling rows past rows_in (or keeping the first rows_out rows).
int launch_copy_rows(const void* src, void* dst, int64_t outer, int rows_in, int rows_out,
                     int64_t len, int elem_bytes, hipStream_t st);
int launch_bwd_reduce_params(const float* dA_part, const float* dD_part,
                             const float* dbias_part, float* dA_log, float* dDs,
                             float* ddt_bias, int B, int K, int D, int N, hipStream_t st);
// z: optional gate (NULL for none), same element type and layout as y.
int launch_merge4(const float* y_route, const void* z, void* y, int B, int D, int H, int W,
                  int dtype, hipStream_t st);
int launch_merge2(const float* y_route, const void* z, void* y, int B, int D, int L,
                  int dtype, hipStream_t st);
// The gate's backward in place of the gated output: from the per-route outputs (the ungated
// route sum v), z and dy (the element type and layout of y), g = dy SiLU(z) in fp32 and
// dz = dy v SiLU'(z) in the element type.
int launch_merge4_gate_bwd(const float* y_route, const void* z, const void* dy, void* g,
                           void* dz, int B, int D, int H, int W, int dtype, hipStream_t st);
int launch_merge2_gate_bwd(const float* y_route, const void* z, const void* dy, void* g,
                           void* dz, int B, int D, int L, int dtype, hipStream_t st);
// Issue-rate probes: kind 0 (fp32 fused multiply-adds), 1 (v_exp_f32), 2 (groups of 4 fused
// multiply-adds and 1 v_exp_f32); `blocks` blocks of probe_block() threads, `iters` loop
// iterations of probe_counts() instructions per lane; sink takes blocks * probe_block()
// floats, clocks 4 per block (shader and reference counters at the start and end).
void probe_counts(int kind, int* fmas, int* exps);
int probe_block();
int launch_probe(int kind, int blocks, int iters, float* sink, unsigned long long* clocks,
                 hipStream_t st);
// Bytes of the prepared weight images of one call (K * ceil(D / 64) images).
size_t project_prep_bytes(int K, int D, int N, int R, int dtype);
// Fills a.wprep (which must hold project_prep_bytes) from the weights, then runs the front
// end; both on `st`.
int launch_project(const ProjArgs& a, int dtype, hipStream_t st);

}  // namespace ss2d
