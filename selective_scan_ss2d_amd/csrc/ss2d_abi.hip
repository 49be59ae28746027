// C ABI of the SS2D forward library: argument validation, the launch plan, stream-ordered
// scratch, and the kernel sequence (transpose -> [chunk aggregates ->] scan -> merge).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <algorithm>
#include <mutex>
#include <vector>

#include "ss2d.h"
#include "ss2d_device.h"
#include "ss2d_gate.h"

namespace {

thread_local int g_last_hip_error = 0;

// Per-thread kernel timing record (see ss2d_timing_enable / ss2d_timing_read).
struct TimedLaunch {
  int kind;
  hipEvent_t start, stop;
};
struct Timing {
  bool enabled = false;
  std::vector<TimedLaunch> launches;
  ~Timing() {
    for (auto& t : launches) {
      (void)hipEventDestroy(t.start);
      (void)hipEventDestroy(t.stop);
    }
  }
};
thread_local Timing g_timing;

// Runs `launch` (which enqueues one kernel on `st` and returns a hipError_t value), between
// two recorded events when timing is enabled on this thread.
template <typename F>
int timed(int kind, hipStream_t st, F&& launch) {
  if (!g_timing.enabled) return launch();
  TimedLaunch t{kind, nullptr, nullptr};
  if (hipEventCreate(&t.start) != hipSuccess) return launch();
  if (hipEventCreate(&t.stop) != hipSuccess) {
    (void)hipEventDestroy(t.start);
    return launch();
  }
  (void)hipEventRecord(t.start, st);
  const int rc = launch();
  (void)hipEventRecord(t.stop, st);
  g_timing.launches.push_back(t);
  return rc;
}

int hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return SS2D_ERR_HIP;
}

// Scratch comes from a stream-ordered memory pool that belongs to this library, one per
// device, created on first use with an unlimited release threshold: freed blocks stay in
// the pool for the next call instead of going back to the driver at every synchronisation,
// so after the first call the per-call allocation is a pool hit.  The device's default pool
// is left as it is.  Under stream capture the allocation becomes a node of the graph.
constexpr int kMaxDevices = 64;
std::mutex g_pool_mu;
hipMemPool_t g_pools[kMaxDevices] = {};

int scratch_pool(int device, hipMemPool_t* out) {
  hipMemPool_t* const pools = g_pools;
  if (device < 0 || device >= kMaxDevices) return hip_fail(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_pool_mu);
  if (!pools[device]) {
    hipMemPoolProps props{};
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = device;
    hipMemPool_t pool = nullptr;
    hipError_t e = hipMemPoolCreate(&pool, &props);
    if (e != hipSuccess) return hip_fail(e);
    uint64_t threshold = UINT64_MAX;
    e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &threshold);
    if (e != hipSuccess) {
      (void)hipMemPoolDestroy(pool);
      return hip_fail(e);
    }
    pools[device] = pool;
  }
  *out = pools[device];
  return SS2D_OK;
}

// Stream-ordered scratch of `bytes` on the current device, released by hipFreeAsync on the
// same stream at the end of the call.
int scratch_alloc(char** ws, size_t bytes, hipStream_t st) {
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return hip_fail(e);
  hipMemPool_t pool = nullptr;
  const int rc = scratch_pool(device, &pool);
  if (rc != SS2D_OK) return rc;
  e = hipMallocFromPoolAsync(reinterpret_cast<void**>(ws), bytes < 256 ? 256 : bytes, pool, st);
  if (e != hipSuccess) return hip_fail(e);
  return SS2D_OK;
}

// ---- scratch of the entry point that allocates nothing ---------------------------------------
// A file-scope device array: every device the library runs on holds its own copy, from the
// time the library's code is loaded on it until the process ends.  In host code the array's
// name is only a handle for hipGetSymbolAddress: its device address is looked up once per
// device (with that device current) and only that address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = SS2D_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

int noalloc_scratch(char** out) {
  static std::mutex mu;
  static char* ptrs[kMaxDevices] = {};
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return hip_fail(e);
  if (device < 0 || device >= kMaxDevices) return hip_fail(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[device]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!ptr) return hip_fail(hipErrorInvalidSymbol);
    ptrs[device] = static_cast<char*>(ptr);
  }
  *out = ptrs[device];
  return SS2D_OK;
}

// Launch-plan override of the calling host thread (ss2d_set_launch_plan): lanes per channel
// (0: automatic) and chunk length (-1: automatic, 0: one pass).
thread_local int g_split_override = 0;
thread_local int64_t g_chunk_override = -1;

constexpr int64_t kMaxL = int64_t(1) << 30;
constexpr int64_t kMaxElems = int64_t(1) << 62;
constexpr int kMaxGridZ = 65535;

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a == 0 || b == 0) { *out = 0; return true; }
  if (a > kMaxElems / b) return false;
  *out = a * b;
  return true;
}

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  const auto pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + static_cast<uintptr_t>(bbytes) && pb < pa + static_cast<uintptr_t>(abytes);
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

struct Plan {
  int split = 1;        // lanes per channel
  int num_chunks = 1;
  int chunk_len = 0;
  bool need_xt = false;
  size_t off_xt = 0, off_yr = 0, off_hend = 0, off_dsum = 0, bytes = 0;
};

// Launch plan.  The scan wants about three resident waves per SIMD (256 CUs x 4 SIMDs)
// to keep the VALU issuing.  Splitting each channel's N states over 4 lanes (partial
// outputs combined with DPP) costs a few extra instructions per step and quadruples the
// waves; it is used whenever N allows.  When even that leaves too few waves, time is cut
// into chunks: a first pass computes each chunk's end state from a zero start, a carry pass
// chains them, and a second pass rescans each chunk from its true start state, so chunking
// roughly doubles the work and is used only for short, long-sequence batches.
Plan make_plan(int K, int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype,
               bool routes) {
  Plan p;
  const int64_t L = H * W;
  const int64_t e = dtype == SS2D_F32 ? 4 : 2;
  int split = (N % 4 == 0) ? 4 : ((N % 2 == 0) ? 2 : 1);
  if (g_split_override != 0) split = g_split_override;
  if (split > N || N % split != 0) split = 1;
  const int64_t waves = B * K * ((D * split + 63) / 64);
  int64_t chunk = 0;
  if (waves < 1536) {
    const int64_t want = (3072 + waves - 1) / waves;  // chunks wanted
    int64_t len = (L + want - 1) / want;
    len = ((len + ss2d::kChunkAlign - 1) / ss2d::kChunkAlign) * ss2d::kChunkAlign;
    if (len < 64) len = 64;
    if (len < L) chunk = len;
  }
  const int64_t forced_chunk = g_chunk_override;
  if (forced_chunk >= 0) {
    int64_t len = ((forced_chunk + ss2d::kChunkAlign - 1) / ss2d::kChunkAlign) * ss2d::kChunkAlign;
    chunk = (len > 0 && len < L) ? len : 0;
  }
  if (chunk > 0 && split == 2) split = 1;  // the chunked passes run 1 or 4 lanes per channel
  p.split = split;
  if (chunk > 0) {
    p.chunk_len = static_cast<int>(chunk);
    p.num_chunks = static_cast<int>((L + chunk - 1) / chunk);
  } else {
    p.num_chunks = 1;
    p.chunk_len = static_cast<int>(((L + ss2d::kChunkAlign - 1) / ss2d::kChunkAlign) *
                                   ss2d::kChunkAlign);
  }
  p.need_xt = !routes && (K == 4) && H > 1 && W > 1;
  size_t off = 0;
  if (p.need_xt) {
    p.off_xt = off;
    off = align256(off + size_t(B * D * L * e));
  }
  p.off_yr = off;
  off = align256(off + size_t(B * K * D * L) * 4);
  if (p.num_chunks > 1) {
    const size_t rows = size_t(B * K * D) * size_t(p.num_chunks);
    p.off_hend = off;
    off = align256(off + rows * size_t(N) * 4);
    p.off_dsum = off;
    off = align256(off + rows * 4);
  }
  p.bytes = off;
  return p;
}

int run_scan(const ss2d::ScanArgs& a, int dtype, int split, int mode, hipStream_t st) {
  if (a.dt_lr) {
    if (a.zoh)
      return dtype == SS2D_F32 ? ss2d::launch_scan_f32_zoh_lr(a, split, mode, st)
                               : ss2d::launch_scan_bf16_zoh_lr(a, split, mode, st);
    return dtype == SS2D_F32 ? ss2d::launch_scan_f32_lr(a, split, mode, st)
                             : ss2d::launch_scan_bf16_lr(a, split, mode, st);
  }
  if (a.zoh)
    return dtype == SS2D_F32 ? ss2d::launch_scan_f32_zoh(a, split, mode, st)
                             : ss2d::launch_scan_bf16_zoh(a, split, mode, st);
  return dtype == SS2D_F32 ? ss2d::launch_scan_f32(a, split, mode, st)
                           : ss2d::launch_scan_bf16(a, split, mode, st);
}

// Launch one scan pass over all images, in batches that keep gridDim.z within range.
int scan_pass(ss2d::ScanArgs a, int dtype, const Plan& p, int mode, int64_t e, hipStream_t st) {
  const int64_t B = a.B;
  const int64_t per = a.chunks_in_launch > 0 ? a.chunks_in_launch : 1;
  const int64_t max_b = kMaxGridZ / per > 0 ? kMaxGridZ / per : 1;
  const int64_t L = a.L, D = a.D, K = a.K, N = a.N;
  const bool ckpt = mode == ss2d::kModeCkpt || mode == ss2d::kModeCkptOut;
  const int64_t C = ckpt ? ss2d::ck_slots(L) : a.num_chunks;
  for (int64_t b0 = 0; b0 < B; b0 += max_b) {
    const int64_t nb = (B - b0 < max_b) ? (B - b0) : max_b;
    ss2d::ScanArgs s = a;
    s.B = static_cast<int>(nb);
    const int64_t x_per_b = (a.x_routes ? K : 1) * D * L * e;  // per-route inputs: (B, K, D, L)
    s.x_row = static_cast<const char*>(a.x_row) + b0 * x_per_b;
    s.x_col = static_cast<const char*>(a.x_col) + b0 * x_per_b;
    if (a.dt_raw) s.dt_raw = static_cast<const char*>(a.dt_raw) + b0 * K * D * L * e;
    if (a.dt_lr) s.dt_lr = static_cast<const char*>(a.dt_lr) + b0 * K * a.R * L * e;
    s.Bs = static_cast<const char*>(a.Bs) + b0 * K * N * L * e;
    s.Cs = static_cast<const char*>(a.Cs) + b0 * K * N * L * e;
    s.y_route = a.y_route ? a.y_route + b0 * K * D * L : nullptr;
    if (a.h_end) s.h_end = a.h_end + b0 * K * D * C * N;
    if (a.delta_sum) s.delta_sum = a.delta_sum + b0 * K * D * C;
    if (a.h_in) s.h_in = a.h_in + b0 * K * D * C * N;
    const int kind = mode == ss2d::kModeAgg ? SS2D_KERNEL_CHUNK_AGG
                     : ckpt                 ? SS2D_KERNEL_CHECKPOINT
                                            : SS2D_KERNEL_SCAN;
    const int rc = timed(kind, st, [&] { return run_scan(s, dtype, p.split, mode, st); });
    if (rc != 0) return hip_fail(static_cast<hipError_t>(rc));
  }
  return SS2D_OK;
}

// The state a training forward keeps for its backward (ss2d_forward_save): the scan's state
// before every 8-step quarter, (B, K, D, ceil(L / 8), N) fp32 (the first quarter's, zero, is
// not written), then with the gate the ungated route sum v, (B, D, L) fp32.  Sizes in bytes;
// -1 for sizes the operator rejects or N not a multiple of 4.
int64_t saved_ck_bytes(int64_t B, int64_t K, int64_t D, int64_t L, int64_t N) {
  return B * K * D * ss2d::ck_slots(L) * N * 4;
}
int64_t saved_bytes(int K, int64_t B, int64_t D, int64_t L, int64_t N, bool gated) {
  if ((K != 2 && K != 4) || B < 0 || D < 0 || L < 1 || L >= kMaxL || N < 4 || N > 32 ||
      (N & (N - 1)) != 0)
    return -1;
  int64_t ck, t, v = 0;
  if (!mul_ok(B * K, D, &t) || !mul_ok(t, ss2d::ck_slots(L) * N * 4, &ck)) return -1;
  if (gated && (!mul_ok(B, D, &t) || !mul_ok(t, L * 4, &v))) return -1;
  return ck + v;
}

// routes: x is every route's own input u (B, K, D, L) in scan order instead of the image x.
// dt_lr (not NULL): dt_proj folded in; dt_raw is then ignored and each step's dt_raw is
// dt_w (K, D, R) times the step's column of dt_lr (B, K, R, L).
int forward(int K, bool routes, const void* x, const void* dt_raw, const float* A_log,
            const void* Bs, const void* Cs, const float* Ds, const float* dt_bias, const void* z,
            void* y, int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype,
            int flags, void* stream, const void* dt_lr = nullptr, const float* dt_w = nullptr,
            int64_t R = 0, bool noalloc = false, float* saved = nullptr, bool save = false) {
  const bool lr = dt_lr != nullptr || dt_w != nullptr || R != 0;
  // ---- validation (nothing is enqueued before all of it passes) -------------------------
  if (dtype != SS2D_F32 && dtype != SS2D_BF16) return SS2D_ERR_UNSUPPORTED;
  if (flags & ~SS2D_FLAG_ZOH) return SS2D_ERR_UNSUPPORTED;
  if (B < 0 || D < 0 || H < 1 || W < 1 || N < 1) return SS2D_ERR_SHAPE;
  if (N != 1 && N != 2 && N != 4 && N != 8 && N != 16 && N != 32) return SS2D_ERR_UNSUPPORTED;
  if (H >= kMaxL || W >= kMaxL || H * W >= kMaxL) return SS2D_ERR_SHAPE;
  const int64_t L = H * W;
  if (D >= (int64_t(1) << 31) / 4 || B >= (int64_t(1) << 31)) return SS2D_ERR_SHAPE;
  int64_t n_x, n_dt, n_bc, tmp;
  if (!mul_ok(B, D, &tmp) || !mul_ok(tmp, L, &n_x)) return SS2D_ERR_SHAPE;
  if (!mul_ok(n_x, K, &n_dt)) return SS2D_ERR_SHAPE;
  if (!mul_ok(B * K, N, &tmp) || !mul_ok(tmp, L, &n_bc)) return SS2D_ERR_SHAPE;
  if (lr && (R < 1 || R > ss2d::kMaxLowRank)) return SS2D_ERR_UNSUPPORTED;
  // save: the training forward (checkpoints need four lanes per channel)
  if (save && N % 4 != 0) return SS2D_ERR_UNSUPPORTED;
  if (B == 0 || D == 0) return SS2D_OK;
  if (!x || !A_log || !Bs || !Cs || !Ds || !dt_bias || !y) return SS2D_ERR_NULL;
  if (save && !saved) return SS2D_ERR_NULL;
  if (save && (reinterpret_cast<uintptr_t>(saved) & 15u)) return SS2D_ERR_ALIGN;
  if (lr ? (!dt_lr || !dt_w) : !dt_raw) return SS2D_ERR_NULL;
  const int64_t e = dtype == SS2D_F32 ? 4 : 2;
  const uintptr_t emask = static_cast<uintptr_t>(e - 1);
  for (const void* ptr : {x, lr ? dt_lr : dt_raw, Bs, Cs, z, static_cast<const void*>(y)})
    if (reinterpret_cast<uintptr_t>(ptr) & emask) return SS2D_ERR_ALIGN;
  if (lr && (reinterpret_cast<uintptr_t>(dt_w) & 3u)) return SS2D_ERR_ALIGN;
  for (const void* ptr : {static_cast<const void*>(A_log), static_cast<const void*>(Ds),
                          static_cast<const void*>(dt_bias)})
    if (reinterpret_cast<uintptr_t>(ptr) & 3u) return SS2D_ERR_ALIGN;
  const int64_t y_bytes = n_x * e;
  if (overlaps(y, y_bytes, x, (routes ? n_dt : n_x) * e) ||
      (lr ? overlaps(y, y_bytes, dt_lr, B * K * R * H * W * e) ||
                overlaps(y, y_bytes, dt_w, int64_t(K) * D * R * 4)
          : overlaps(y, y_bytes, dt_raw, n_dt * e)) ||
      overlaps(y, y_bytes, Bs, n_bc * e) || overlaps(y, y_bytes, Cs, n_bc * e) ||
      overlaps(y, y_bytes, A_log, int64_t(K) * D * N * 4) ||
      overlaps(y, y_bytes, Ds, int64_t(K) * D * 4) ||
      overlaps(y, y_bytes, dt_bias, int64_t(K) * D * 4) ||
      (z && overlaps(y, y_bytes, z, n_x * e)))
    return SS2D_ERR_ALIAS;
  const int64_t tiles = (L + 31) / 32;
  if (save) {
    const int64_t sb = saved_bytes(K, B, D, L, N, z != nullptr);
    if (sb < 0) return SS2D_ERR_SHAPE;
    const void* others[] = {x, dt_raw, Bs, Cs, A_log, Ds, dt_bias, z, y};
    const int64_t other_bytes[] = {(routes ? n_dt : n_x) * e, n_dt * e, n_bc * e, n_bc * e,
                                   int64_t(K) * D * N * 4, int64_t(K) * D * 4,
                                   int64_t(K) * D * 4, n_x * e, y_bytes};
    for (int i = 0; i < 9; ++i)
      if (others[i] && overlaps(saved, sb, others[i], other_bytes[i])) return SS2D_ERR_ALIAS;
  }

  // ---- plan and scratch --------------------------------------------------------------
  hipStream_t st = static_cast<hipStream_t>(stream);
  Plan p = make_plan(K, B, D, H, W, N, dtype, routes);
  if (save) {  // one pass, four lanes per channel, storing the state before every tile
    p.split = 4;
    p.num_chunks = 1;
    p.chunk_len = static_cast<int>(tiles * 32);
  }
  // noalloc: the scratch is the fixed device array (size checked before any HIP call)
  if (noalloc && p.bytes > kNoAllocScratchBytes) return SS2D_ERR_SCRATCH;
  char* ws = nullptr;
  int rc = noalloc ? noalloc_scratch(&ws) : scratch_alloc(&ws, p.bytes, st);
  if (rc != SS2D_OK) return rc;

  ss2d::ScanArgs a{};
  a.x_row = x;
  a.x_col = p.need_xt ? static_cast<const void*>(ws + p.off_xt) : x;
  a.dt_raw = dt_raw;
  a.Bs = Bs;
  a.Cs = Cs;
  a.A_log = A_log;
  a.Ds = Ds;
  a.dt_bias = dt_bias;
  a.y_route = reinterpret_cast<float*>(ws + p.off_yr);
  a.B = static_cast<int>(B);
  a.K = K;
  a.D = static_cast<int>(D);
  a.L = static_cast<int>(L);
  a.N = static_cast<int>(N);
  a.num_chunks = p.num_chunks;
  a.chunk_len = p.chunk_len;
  a.zoh = (flags & SS2D_FLAG_ZOH) ? 1 : 0;
  a.x_routes = routes ? 1 : 0;
  if (lr) {
    a.dt_raw = nullptr;
    a.dt_lr = dt_lr;
    a.dt_w = dt_w;
    a.R = static_cast<int>(R);
  }

  int err = 0;
  if (p.need_xt)
    err = timed(SS2D_KERNEL_TRANSPOSE, st, [&] {
      return ss2d::launch_transpose(x, ws + p.off_xt, a.B, a.D, static_cast<int>(H),
                                    static_cast<int>(W), dtype, st);
    });
  if (!err && save) {
    a.h_in = saved;
    a.chunk_base = 0;
    a.chunks_in_launch = 1;
    rc = scan_pass(a, dtype, p, ss2d::kModeCkptOut, e, st);
  } else if (!err && p.num_chunks > 1) {
    a.h_end = reinterpret_cast<float*>(ws + p.off_hend);
    a.delta_sum = reinterpret_cast<float*>(ws + p.off_dsum);
    ss2d::ScanArgs agg = a;  // aggregates of chunks 0 .. C-2
    agg.chunk_base = 0;
    agg.chunks_in_launch = p.num_chunks - 1;
    rc = scan_pass(agg, dtype, p, ss2d::kModeAgg, e, st);
    if (rc == SS2D_OK) {  // the second pass composes the aggregates into chunk start states
      ss2d::ScanArgs out = a;
      out.h_in = nullptr;
      out.chunk_base = 0;
      out.chunks_in_launch = p.num_chunks;
      rc = scan_pass(out, dtype, p, ss2d::kModeOut, e, st);
    }
  } else if (!err) {
    a.chunk_base = 0;
    a.chunks_in_launch = 1;
    rc = scan_pass(a, dtype, p, ss2d::kModeOut, e, st);
  }
  if (!err && rc == SS2D_OK && save && z) {
    // the gated training forward keeps the ungated route sum (fp32) for the gate's backward,
    // then gates it: the same sum and products as the fused gated merge
    float* v = saved + saved_ck_bytes(B, K, D, L, N) / 4;
    err = timed(SS2D_KERNEL_MERGE, st, [&] {
      return (K == 4) ? ss2d::launch_merge4(a.y_route, nullptr, v, a.B, a.D,
                                            static_cast<int>(H), static_cast<int>(W), SS2D_F32,
                                            st)
                      : ss2d::launch_merge2(a.y_route, nullptr, v, a.B, a.D, a.L, SS2D_F32, st);
    });
    if (!err)
      err = timed(SS2D_KERNEL_MERGE, st,
                  [&] { return ss2d::launch_gate_fwd(v, z, y, n_x, dtype, st); });
  } else if (!err && rc == SS2D_OK) {
    err = timed(SS2D_KERNEL_MERGE, st, [&] {
      return (K == 4) ? ss2d::launch_merge4(a.y_route, z, y, a.B, a.D, static_cast<int>(H),
                                            static_cast<int>(W), dtype, st)
                      : ss2d::launch_merge2(a.y_route, z, y, a.B, a.D, a.L, dtype, st);
    });
  }
  const hipError_t fe = noalloc ? hipSuccess : hipFreeAsync(ws, st);
  if (err) return hip_fail(static_cast<hipError_t>(err));
  if (rc != SS2D_OK) return rc;
  if (fe != hipSuccess) return hip_fail(fe);
  return SS2D_OK;
}

// ---- backward ----------------------------------------------------------------------------
// z (not NULL): gradients of the gated output y SiLU(z); dz receives z's gradient.
// flags: SS2D_FLAG_ZOH for the zero-order-hold operator.
// routes: x is every route's own input u (B, K, D, L) in scan order, and dx receives du of
// that shape (per route and step) instead of the image gradient.
int backward(int K, const void* x, const void* dt_raw, const float* A_log, const void* Bs,
             const void* Cs, const float* Ds, const float* dt_bias, const void* dy, void* dx,
             void* ddt_raw, float* dA_log, void* dBs, void* dCs, float* dDs, float* ddt_bias,
             int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype, void* stream,
             const void* z = nullptr, void* dz = nullptr, int flags = 0, bool routes = false,
             const float* saved = nullptr, bool from_saved = false) {
  const bool gated = z != nullptr;
  if (dtype != SS2D_F32 && dtype != SS2D_BF16) return SS2D_ERR_UNSUPPORTED;
  if (flags & ~SS2D_FLAG_ZOH) return SS2D_ERR_UNSUPPORTED;
  if (B < 0 || D < 0 || H < 1 || W < 1 || N < 1) return SS2D_ERR_SHAPE;
  if (N != 1 && N != 2 && N != 4 && N != 8 && N != 16 && N != 32) return SS2D_ERR_UNSUPPORTED;
  if (H >= kMaxL || W >= kMaxL || H * W >= kMaxL) return SS2D_ERR_SHAPE;
  const int64_t L = H * W;
  if (D >= (int64_t(1) << 31) / 4 || B >= (int64_t(1) << 31)) return SS2D_ERR_SHAPE;
  int64_t n_x, n_dt, n_bc, tmp;
  if (!mul_ok(B, D, &tmp) || !mul_ok(tmp, L, &n_x)) return SS2D_ERR_SHAPE;
  if (!mul_ok(n_x, K, &n_dt)) return SS2D_ERR_SHAPE;
  if (!mul_ok(B * K, N, &tmp) || !mul_ok(tmp, L, &n_bc)) return SS2D_ERR_SHAPE;
  // from_saved: the checkpoints (and with the gate the route sum) a training forward kept
  if (from_saved && N % 4 != 0) return SS2D_ERR_UNSUPPORTED;
  if (B == 0 || D == 0) return SS2D_OK;
  if (from_saved && !saved) return SS2D_ERR_NULL;
  if (from_saved && (reinterpret_cast<uintptr_t>(saved) & 15u)) return SS2D_ERR_ALIGN;
  // z and dz are the last input and output of the gated entry points
  const void* ins[] = {x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, z};
  const void* outs[] = {dx, ddt_raw, dA_log, dBs, dCs, dDs, ddt_bias, dz};
  const int n_in = gated ? 9 : 8, n_out = gated ? 8 : 7;
  for (int i = 0; i < n_in; ++i)
    if (!ins[i]) return SS2D_ERR_NULL;
  for (int i = 0; i < n_out; ++i)
    if (!outs[i]) return SS2D_ERR_NULL;
  const int64_t e = dtype == SS2D_F32 ? 4 : 2;
  const uintptr_t emask = static_cast<uintptr_t>(e - 1);
  for (const void* ptr : {x, dt_raw, Bs, Cs, dy, z, static_cast<const void*>(dx),
                          static_cast<const void*>(ddt_raw), static_cast<const void*>(dBs),
                          static_cast<const void*>(dCs),
                          gated ? static_cast<const void*>(dz) : nullptr})
    if (reinterpret_cast<uintptr_t>(ptr) & emask) return SS2D_ERR_ALIGN;
  for (const void* ptr : {static_cast<const void*>(A_log), static_cast<const void*>(Ds),
                          static_cast<const void*>(dt_bias), static_cast<const void*>(dA_log),
                          static_cast<const void*>(dDs), static_cast<const void*>(ddt_bias)})
    if (reinterpret_cast<uintptr_t>(ptr) & 3u) return SS2D_ERR_ALIGN;
  const int64_t n_in0 = routes ? n_dt : n_x;  // elements of x (u) and of dx (du)
  const int64_t in_bytes[] = {n_in0 * e, n_dt * e, int64_t(K) * D * N * 4, n_bc * e, n_bc * e,
                              int64_t(K) * D * 4, int64_t(K) * D * 4, n_x * e, n_x * e};
  const int64_t out_bytes[] = {n_in0 * e, n_dt * e, int64_t(K) * D * N * 4, n_bc * e, n_bc * e,
                               int64_t(K) * D * 4, int64_t(K) * D * 4, n_x * e};
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j])) return SS2D_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return SS2D_ERR_ALIAS;
  }
  if (from_saved) {
    const int64_t sb = saved_bytes(K, B, D, L, N, gated);
    if (sb < 0) return SS2D_ERR_SHAPE;
    for (int i = 0; i < n_out; ++i)
      if (overlaps(outs[i], out_bytes[i], saved, sb)) return SS2D_ERR_ALIAS;
  }

  hipStream_t st = static_cast<hipStream_t>(stream);
  int rc = SS2D_OK;

  if (N < 4) {
    // N = 1 or 2: the kernels split a channel's states over four lanes, so the call runs
    // with four states, the extra ones with zero B and C rows (and A_log 0).  Their states
    // and adjoints stay exactly zero, so they add exactly nothing to any sum over states:
    // the gradients of the real states are those of the N-state operator.  Padded copies of
    // Bs, Cs and A_log and the padded dBs, dCs and dA_log live in scratch; the first N rows
    // of the latter are copied out.
    constexpr int64_t NP = 4;
    const int64_t n_pad = B * K * NP * L;
    size_t po = 0;
    const size_t o_bs = po;
    po = align256(po + size_t(n_pad * e));
    const size_t o_cs = po;
    po = align256(po + size_t(n_pad * e));
    const size_t o_dbs = po;
    po = align256(po + size_t(n_pad * e));
    const size_t o_dcs = po;
    po = align256(po + size_t(n_pad * e));
    const size_t o_al = po;
    po = align256(po + size_t(K * D * NP) * 4);
    const size_t o_dal = po;
    po = align256(po + size_t(K * D * NP) * 4);
    char* pw = nullptr;
    rc = scratch_alloc(&pw, po, st);
    if (rc != SS2D_OK) return rc;
    const int ni = static_cast<int>(N);
    int err = ss2d::launch_copy_rows(Bs, pw + o_bs, B * K, ni, 4, L, int(e), st);
    if (!err) err = ss2d::launch_copy_rows(Cs, pw + o_cs, B * K, ni, 4, L, int(e), st);
    if (!err) err = ss2d::launch_copy_rows(A_log, pw + o_al, int64_t(K) * D, ni, 4, 1, 4, st);
    if (!err) {
      rc = backward(K, x, dt_raw, reinterpret_cast<const float*>(pw + o_al), pw + o_bs,
                    pw + o_cs, Ds, dt_bias, dy, dx, ddt_raw,
                    reinterpret_cast<float*>(pw + o_dal), pw + o_dbs, pw + o_dcs, dDs, ddt_bias,
                    B, D, H, W, NP, dtype, stream, z, dz, flags, routes);
    }
    if (!err && rc == SS2D_OK) {
      err = ss2d::launch_copy_rows(pw + o_dbs, dBs, B * K, 4, ni, L, int(e), st);
      if (!err) err = ss2d::launch_copy_rows(pw + o_dcs, dCs, B * K, 4, ni, L, int(e), st);
      if (!err)
        err = ss2d::launch_copy_rows(pw + o_dal, dA_log, int64_t(K) * D, 4, ni, 1, 4, st);
    }
    const hipError_t fe = hipFreeAsync(pw, st);
    if (err) return hip_fail(static_cast<hipError_t>(err));
    if (rc != SS2D_OK) return rc;
    if (fe != hipSuccess) return hip_fail(fe);
    return SS2D_OK;
  }

  // Scratch: transposes of x and of the route gradient g, checkpoints, per-route du, dB/dC
  // block partials and the per-image parameter partials; with the gate, g = dy SiLU(z) in
  // fp32 (the gradient every route receives, not rounded to the data type) and, until the
  // adjoint overwrites them with du, the per-route outputs.
  const int64_t tiles = (L + 31) / 32;
  const int64_t n_cb = (D + 63) / 64;
  const bool need_t = (K == 4) && H > 1 && W > 1;
  const bool need_xt = need_t && !routes;  // per-route inputs are read in scan order
  const int64_t ge = gated ? 4 : e;  // bytes per element of g
  size_t off = 0;
  const size_t off_xt = off;
  if (need_xt) off = align256(off + size_t(n_x * e));
  const size_t off_gt = off;
  if (need_t) off = align256(off + size_t(n_x * ge));
  const size_t off_g = off;
  if (gated) off = align256(off + size_t(n_x * 4));
  const size_t off_ck = off;
  if (!from_saved) off = align256(off + size_t(B * K * D) * size_t(ss2d::ck_slots(L) * N) * 4);
  // per-route du in fp32: merged into dx, or (gate) first the route outputs; with per-route
  // inputs and no gate the adjoint writes du straight to the output
  const bool need_du = !routes || gated;
  const size_t off_du = off;
  if (need_du) off = align256(off + size_t(n_dt) * 4);
  const size_t off_bc = off;
  off = align256(off + size_t(B * K * n_cb) * size_t(2 * N * L) * 4);
  const size_t off_pa = off;
  off = align256(off + size_t(B * K * D * N) * 4);
  const size_t off_pd = off;
  off = align256(off + size_t(B * K * D) * 4);
  const size_t off_pb = off;
  off = align256(off + size_t(B * K * D) * 4);
  char* ws = nullptr;
  rc = scratch_alloc(&ws, off, st);
  if (rc != SS2D_OK) return rc;

  int err = 0;
  // g: the gradient every route's output receives (dy, or dy SiLU(z) with the gate)
  const void* g_img = gated ? static_cast<const void*>(ws + off_g) : dy;
  const void* xt = need_xt ? static_cast<const void*>(ws + off_xt) : x;
  const void* gt = need_t ? static_cast<const void*>(ws + off_gt) : g_img;
  if (need_xt)
    err = timed(SS2D_KERNEL_TRANSPOSE, st, [&] {
      return ss2d::launch_transpose(x, ws + off_xt, int(B), int(D), int(H), int(W), dtype, st);
    });
  const float* h_ck = from_saved ? saved : reinterpret_cast<const float*>(ws + off_ck);
  // Checkpoints: the forward scan storing the state before every 8-step quarter (and, with the
  // gate, the per-route outputs, which the merge kernel turns into g and dz), unless a
  // training forward kept them.
  if (!err && !from_saved) {
    ss2d::ScanArgs a{};
    a.x_row = x;
    a.x_col = xt;
    a.dt_raw = dt_raw;
    a.Bs = Bs;
    a.Cs = Cs;
    a.A_log = A_log;
    a.Ds = Ds;
    a.dt_bias = dt_bias;
    a.h_in = reinterpret_cast<float*>(ws + off_ck);
    a.B = int(B);
    a.K = K;
    a.D = int(D);
    a.L = int(L);
    a.N = int(N);
    a.num_chunks = 1;
    a.chunk_len = int(tiles * 32);
    a.chunk_base = 0;
    a.chunks_in_launch = 1;
    a.zoh = (flags & SS2D_FLAG_ZOH) ? 1 : 0;
    a.x_routes = routes ? 1 : 0;
    if (gated) a.y_route = reinterpret_cast<float*>(ws + off_du);
    Plan p;
    p.split = 4;
    rc = scan_pass(a, dtype, p, gated ? ss2d::kModeCkptOut : ss2d::kModeCkpt, e, st);
  }
  if (gated && from_saved && !err)  // g and dz from the route sum the forward kept
    err = timed(SS2D_KERNEL_MERGE, st, [&] {
      const float* v = saved + saved_ck_bytes(B, K, D, L, N) / 4;
      return ss2d::launch_gate_bwd(v, z, dy, reinterpret_cast<float*>(ws + off_g), dz, n_x,
                                   dtype, st);
    });
  else if (gated && !err && rc == SS2D_OK)
    err = timed(SS2D_KERNEL_MERGE, st, [&] {
      const float* yr = reinterpret_cast<const float*>(ws + off_du);
      return (K == 4) ? ss2d::launch_merge4_gate_bwd(yr, z, dy, ws + off_g, dz, int(B), int(D),
                                                     int(H), int(W), dtype, st)
                      : ss2d::launch_merge2_gate_bwd(yr, z, dy, ws + off_g, dz, int(B), int(D),
                                                     int(L), dtype, st);
    });
  if (need_t && !err && rc == SS2D_OK)
    err = timed(SS2D_KERNEL_TRANSPOSE, st, [&] {
      return ss2d::launch_transpose(g_img, ws + off_gt, int(B), int(D), int(H), int(W),
                                    gated ? SS2D_F32 : dtype, st);
    });
  // Adjoint scan, in batches of images that keep gridDim.z in range.
  for (int64_t b0 = 0; !err && rc == SS2D_OK && b0 < B; b0 += kMaxGridZ) {
    const int64_t nb = (B - b0 < kMaxGridZ) ? (B - b0) : kMaxGridZ;
    ss2d::BwdArgs g{};
    const int64_t x_per_b = (routes ? K : 1) * D * L * e;
    g.x_row = static_cast<const char*>(x) + b0 * x_per_b;
    g.x_col = static_cast<const char*>(xt) + b0 * x_per_b;
    g.x_routes = routes ? 1 : 0;
    g.du_out = routes ? static_cast<char*>(dx) + b0 * x_per_b : nullptr;
    g.g_row = static_cast<const char*>(g_img) + b0 * D * L * ge;
    g.g_col = static_cast<const char*>(gt) + b0 * D * L * ge;
    g.g_f32 = gated ? 1 : 0;
    g.zoh = (flags & SS2D_FLAG_ZOH) ? 1 : 0;
    g.dt_raw = static_cast<const char*>(dt_raw) + b0 * K * D * L * e;
    g.Bs = static_cast<const char*>(Bs) + b0 * K * N * L * e;
    g.Cs = static_cast<const char*>(Cs) + b0 * K * N * L * e;
    g.A_log = A_log;
    g.Ds = Ds;
    g.dt_bias = dt_bias;
    g.h_ck = h_ck + b0 * K * D * ss2d::ck_slots(L) * N;
    g.du_route = need_du ? reinterpret_cast<float*>(ws + off_du) + b0 * K * D * L : nullptr;
    g.ddt_raw = static_cast<char*>(ddt_raw) + b0 * K * D * L * e;
    g.dbc_part = reinterpret_cast<float*>(ws + off_bc) + b0 * K * n_cb * 2 * N * L;
    g.dA_part = reinterpret_cast<float*>(ws + off_pa) + b0 * K * D * N;
    g.dD_part = reinterpret_cast<float*>(ws + off_pd) + b0 * K * D;
    g.dbias_part = reinterpret_cast<float*>(ws + off_pb) + b0 * K * D;
    g.B = int(nb);
    g.K = K;
    g.D = int(D);
    g.L = int(L);
    g.N = int(N);
    g.ck_tiles = int(tiles);
    g.n_cb = int(n_cb);
    err = timed(SS2D_KERNEL_SCAN_BWD, st, [&] {
      return dtype == SS2D_F32 ? ss2d::launch_scan_bwd_f32(g, st)
                               : ss2d::launch_scan_bwd_bf16(g, st);
    });
  }
  if (!err && rc == SS2D_OK)
    err = timed(SS2D_KERNEL_REDUCE, st, [&] {
      return ss2d::launch_bwd_reduce_bc(reinterpret_cast<const float*>(ws + off_bc), dBs, dCs,
                                        int(B), K, int(N), int(L), int(n_cb), dtype, st);
    });
  if (!err && rc == SS2D_OK)
    err = timed(SS2D_KERNEL_REDUCE, st, [&] {
      return ss2d::launch_bwd_reduce_params(
          reinterpret_cast<const float*>(ws + off_pa), reinterpret_cast<const float*>(ws + off_pd),
          reinterpret_cast<const float*>(ws + off_pb), dA_log, dDs, ddt_bias, int(B), K, int(D),
          int(N), st);
    });
  if (!err && rc == SS2D_OK && !routes)
    err = timed(SS2D_KERNEL_MERGE, st, [&] {
      const float* du = reinterpret_cast<const float*>(ws + off_du);
      return (K == 4) ? ss2d::launch_merge4(du, nullptr, dx, int(B), int(D), int(H), int(W),
                                            dtype, st)
                      : ss2d::launch_merge2(du, nullptr, dx, int(B), int(D), int(L), dtype, st);
    });
  const hipError_t fe = hipFreeAsync(ws, st);
  if (err) return hip_fail(static_cast<hipError_t>(err));
  if (rc != SS2D_OK) return rc;
  if (fe != hipSuccess) return hip_fail(fe);
  return SS2D_OK;
}

// ---- per-route front end -----------------------------------------------------------------
// dt_lr (not NULL): store x_proj's R dt rows there instead of applying dt_proj (dt_proj_w
// and dt_raw are then unused).
int project(int K, const void* x, const float* conv_w, const float* conv_b,
            const float* x_proj_w, const float* dt_proj_w, void* u, void* dt_raw, void* Bs,
            void* Cs, int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int64_t R,
            int64_t KW, int dtype, void* stream, void* dt_lr = nullptr) {
  const bool lr = dt_lr != nullptr;
  if (dtype != SS2D_F32 && dtype != SS2D_BF16) return SS2D_ERR_UNSUPPORTED;
  if (B < 0 || D < 0 || H < 1 || W < 1 || N < 1 || R < 1 || KW < 1) return SS2D_ERR_SHAPE;
  if (KW > ss2d::kProjMaxKW || R + 2 * N > ss2d::kProjMaxM) return SS2D_ERR_UNSUPPORTED;
  if (H >= kMaxL || W >= kMaxL || H * W >= kMaxL) return SS2D_ERR_SHAPE;
  // the kernel addresses a plane set (D rows of L elements) and the weights with 32-bit
  // byte offsets
  if ((R + 2 * N) * D * 4 >= (int64_t(1) << 31) || D * H * W * 4 >= (int64_t(1) << 31))
    return SS2D_ERR_SHAPE;
  const int64_t L = H * W;
  if (D >= (int64_t(1) << 31) / 4 || B >= (int64_t(1) << 31)) return SS2D_ERR_SHAPE;
  int64_t n_x, n_dt, n_bc, tmp;
  if (!mul_ok(B, D, &tmp) || !mul_ok(tmp, L, &n_x)) return SS2D_ERR_SHAPE;
  if (!mul_ok(n_x, K, &n_dt)) return SS2D_ERR_SHAPE;
  if (!mul_ok(B * K, N, &tmp) || !mul_ok(tmp, L, &n_bc)) return SS2D_ERR_SHAPE;
  if (B == 0 || D == 0) return SS2D_OK;
  // with dt_lr, its place among the outputs is dt_lr's and dt_proj_w's among the inputs
  // is taken by conv_b again (checked twice, harmlessly)
  const void* ins[] = {x, conv_w, conv_b, x_proj_w, lr ? conv_b : dt_proj_w};
  const void* outs[] = {u, lr ? dt_lr : dt_raw, Bs, Cs};
  for (const void* ptr : ins)
    if (!ptr) return SS2D_ERR_NULL;
  for (const void* ptr : outs)
    if (!ptr) return SS2D_ERR_NULL;
  const int64_t e = dtype == SS2D_F32 ? 4 : 2;
  const uintptr_t emask = static_cast<uintptr_t>(e - 1);
  for (const void* ptr : {x, outs[0], outs[1], outs[2], outs[3]})
    if (reinterpret_cast<uintptr_t>(ptr) & emask) return SS2D_ERR_ALIGN;
  for (const void* ptr : {ins[1], ins[2], ins[3], ins[4]})
    if (reinterpret_cast<uintptr_t>(ptr) & 3u) return SS2D_ERR_ALIGN;
  const int64_t in_bytes[] = {n_x * e, int64_t(K) * D * KW * 4, int64_t(K) * D * 4,
                              int64_t(K) * (R + 2 * N) * D * 4,
                              lr ? int64_t(K) * D * 4 : int64_t(K) * D * R * 4};
  const int64_t n_lr = B * K * R * L;
  const int64_t out_bytes[] = {n_dt * e, (lr ? n_lr : n_dt) * e, n_bc * e, n_bc * e};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 5; ++j)
      if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j])) return SS2D_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return SS2D_ERR_ALIAS;
  }

  // Scratch: the transposed copy of x for the column routes, then the prepared weight
  // images (x_proj and conv weights in the kernel's LDS layout, per route and chunk).
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool need_t = (K == 4) && H > 1 && W > 1;
  const size_t off_prep = need_t ? align256(size_t(n_x * e)) : 0;
  const size_t ws_bytes =
      off_prep + ss2d::project_prep_bytes(K, int(D), int(N), int(R), dtype);
  char* ws = nullptr;
  {
    const int rc = scratch_alloc(&ws, ws_bytes, st);
    if (rc != SS2D_OK) return rc;
  }
  int err = 0;
  if (need_t)
    err = timed(SS2D_KERNEL_TRANSPOSE, st, [&] {
      return ss2d::launch_transpose(x, ws, int(B), int(D), int(H), int(W), dtype, st);
    });
  for (int64_t b0 = 0; !err && b0 < B; b0 += kMaxGridZ) {
    const int64_t nb = (B - b0 < kMaxGridZ) ? (B - b0) : kMaxGridZ;
    ss2d::ProjArgs a{};
    a.x_row = static_cast<const char*>(x) + b0 * D * L * e;
    a.x_col = need_t ? static_cast<const void*>(ws + b0 * D * L * e) : a.x_row;
    a.conv_w = conv_w;
    a.conv_b = conv_b;
    a.x_proj_w = x_proj_w;
    a.dt_proj_w = dt_proj_w;
    a.u = static_cast<char*>(u) + b0 * K * D * L * e;
    if (lr)
      a.dt_lr = static_cast<char*>(dt_lr) + b0 * K * R * L * e;
    else
      a.dt_raw = static_cast<char*>(dt_raw) + b0 * K * D * L * e;
    a.Bs = static_cast<char*>(Bs) + b0 * K * N * L * e;
    a.Cs = static_cast<char*>(Cs) + b0 * K * N * L * e;
    a.wprep = ws + off_prep;
    a.B = int(nb);
    a.K = K;
    a.D = int(D);
    a.L = int(L);
    a.N = int(N);
    a.R = int(R);
    a.KW = int(KW);
    err = timed(SS2D_KERNEL_PROJECT, st, [&] { return ss2d::launch_project(a, dtype, st); });
  }
  const hipError_t fe = hipFreeAsync(ws, st);
  if (err) return hip_fail(static_cast<hipError_t>(err));
  if (fe != hipSuccess) return hip_fail(fe);
  return SS2D_OK;
}

}  // namespace

extern "C" {

int ss2d_forward(const void* x, const void* dt_raw, const float* A_log, const void* Bs,
                 const void* Cs, const float* Ds, const float* dt_bias, void* y, int64_t B,
                 int64_t D, int64_t H, int64_t W, int64_t N, int dtype, void* stream) {
  return forward(4, false, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, nullptr, y, B, D, H, W, N, dtype, 0,
                 stream);
}

int ss1d_bidir_forward(const void* x, const void* dt_raw, const float* A_log, const void* Bs,
                       const void* Cs, const float* Ds, const float* dt_bias, void* y,
                       int64_t B, int64_t D, int64_t L, int64_t N, int dtype, void* stream) {
  return forward(2, false, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, nullptr, y, B, D, 1, L, N, dtype, 0,
                 stream);
}

int ss2d_forward_ex(const void* x, const void* dt_raw, const float* A_log, const void* Bs,
                    const void* Cs, const float* Ds, const float* dt_bias, const void* z,
                    void* y, int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype,
                    int flags, void* stream) {
  return forward(4, false, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, y, B, D, H, W, N, dtype, flags,
                 stream);
}

int ss2d_forward_noalloc(const void* x, const void* dt_raw, const float* A_log, const void* Bs,
                         const void* Cs, const float* Ds, const float* dt_bias, const void* z,
                         void* y, int64_t B, int64_t D, int64_t H, int64_t W, int64_t N,
                         int dtype, int flags, void* stream) {
  return forward(4, false, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, y, B, D, H, W, N, dtype, flags,
                 stream, nullptr, nullptr, 0, true);
}

int ss1d_bidir_forward_ex(const void* x, const void* dt_raw, const float* A_log,
                          const void* Bs, const void* Cs, const float* Ds,
                          const float* dt_bias, const void* z, void* y, int64_t B, int64_t D,
                          int64_t L, int64_t N, int dtype, int flags, void* stream) {
  return forward(2, false, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, y, B, D, 1, L, N, dtype, flags,
                 stream);
}

int ss2d_backward(const void* x, const void* dt_raw, const float* A_log, const void* Bs,
                  const void* Cs, const float* Ds, const float* dt_bias, const void* dy,
                  void* dx, void* ddt_raw, float* dA_log, void* dBs, void* dCs, float* dDs,
                  float* ddt_bias, int64_t B, int64_t D, int64_t H, int64_t W, int64_t N,
                  int dtype, void* stream) {
  return backward(4, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, dx, ddt_raw, dA_log, dBs, dCs,
                  dDs, ddt_bias, B, D, H, W, N, dtype, stream);
}

int ss1d_bidir_backward(const void* x, const void* dt_raw, const float* A_log,
                        const void* Bs, const void* Cs, const float* Ds,
                        const float* dt_bias, const void* dy, void* dx, void* ddt_raw,
                        float* dA_log, void* dBs, void* dCs, float* dDs, float* ddt_bias,
                        int64_t B, int64_t D, int64_t L, int64_t N, int dtype, void* stream) {
  return backward(2, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, dx, ddt_raw, dA_log, dBs, dCs,
                  dDs, ddt_bias, B, D, 1, L, N, dtype, stream);
}

int ss2d_backward_ex(const void* x, const void* dt_raw, const float* A_log, const void* Bs,
                     const void* Cs, const float* Ds, const float* dt_bias, const void* z,
                     const void* dy, void* dx, void* ddt_raw, float* dA_log, void* dBs,
                     void* dCs, float* dDs, float* ddt_bias, void* dz, int64_t B, int64_t D,
                     int64_t H, int64_t W, int64_t N, int dtype, int flags, void* stream) {
  return backward(4, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, dx, ddt_raw, dA_log, dBs, dCs,
                  dDs, ddt_bias, B, D, H, W, N, dtype, stream, z, dz, flags);
}

int ss1d_bidir_backward_ex(const void* x, const void* dt_raw, const float* A_log,
                           const void* Bs, const void* Cs, const float* Ds,
                           const float* dt_bias, const void* z, const void* dy, void* dx,
                           void* ddt_raw, float* dA_log, void* dBs, void* dCs, float* dDs,
                           float* ddt_bias, void* dz, int64_t B, int64_t D, int64_t L,
                           int64_t N, int dtype, int flags, void* stream) {
  return backward(2, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, dx, ddt_raw, dA_log, dBs, dCs,
                  dDs, ddt_bias, B, D, 1, L, N, dtype, stream, z, dz, flags);
}

int ss2d_backward_routes(const void* u, const void* dt_raw, const float* A_log, const void* Bs,
                         const void* Cs, const float* Ds, const float* dt_bias, const void* z,
                         const void* dy, void* du, void* ddt_raw, float* dA_log, void* dBs,
                         void* dCs, float* dDs, float* ddt_bias, void* dz, int64_t B,
                         int64_t D, int64_t H, int64_t W, int64_t N, int dtype, int flags,
                         void* stream) {
  return backward(4, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, du, ddt_raw, dA_log, dBs, dCs,
                  dDs, ddt_bias, B, D, H, W, N, dtype, stream, z, dz, flags, true);
}

int ss1d_bidir_backward_routes(const void* u, const void* dt_raw, const float* A_log,
                               const void* Bs, const void* Cs, const float* Ds,
                               const float* dt_bias, const void* z, const void* dy, void* du,
                               void* ddt_raw, float* dA_log, void* dBs, void* dCs, float* dDs,
                               float* ddt_bias, void* dz, int64_t B, int64_t D, int64_t L,
                               int64_t N, int dtype, int flags, void* stream) {
  return backward(2, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, du, ddt_raw, dA_log, dBs, dCs,
                  dDs, ddt_bias, B, D, 1, L, N, dtype, stream, z, dz, flags, true);
}

int64_t ss2d_saved_state_bytes(int K, int64_t B, int64_t D, int64_t L, int64_t N, int gated) {
  return saved_bytes(K, B, D, L, N, gated != 0);
}

int ss2d_forward_save(const void* x, const void* dt_raw, const float* A_log, const void* Bs,
                      const void* Cs, const float* Ds, const float* dt_bias, const void* z,
                      void* y, float* saved, int64_t B, int64_t D, int64_t H, int64_t W,
                      int64_t N, int dtype, int flags, void* stream) {
  return forward(4, false, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, y, B, D, H, W, N, dtype,
                 flags, stream, nullptr, nullptr, 0, false, saved, true);
}

int ss1d_bidir_forward_save(const void* x, const void* dt_raw, const float* A_log,
                            const void* Bs, const void* Cs, const float* Ds,
                            const float* dt_bias, const void* z, void* y, float* saved,
                            int64_t B, int64_t D, int64_t L, int64_t N, int dtype, int flags,
                            void* stream) {
  return forward(2, false, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, y, B, D, 1, L, N, dtype,
                 flags, stream, nullptr, nullptr, 0, false, saved, true);
}

int ss2d_backward_saved(const void* x, const void* dt_raw, const float* A_log, const void* Bs,
                        const void* Cs, const float* Ds, const float* dt_bias, const void* z,
                        const float* saved, const void* dy, void* dx, void* ddt_raw,
                        float* dA_log, void* dBs, void* dCs, float* dDs, float* ddt_bias,
                        void* dz, int64_t B, int64_t D, int64_t H, int64_t W, int64_t N,
                        int dtype, int flags, void* stream) {
  return backward(4, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, dx, ddt_raw, dA_log, dBs, dCs,
                  dDs, ddt_bias, B, D, H, W, N, dtype, stream, z, dz, flags, false, saved,
                  true);
}

int ss1d_bidir_backward_saved(const void* x, const void* dt_raw, const float* A_log,
                              const void* Bs, const void* Cs, const float* Ds,
                              const float* dt_bias, const void* z, const float* saved,
                              const void* dy, void* dx, void* ddt_raw, float* dA_log, void* dBs,
                              void* dCs, float* dDs, float* ddt_bias, void* dz, int64_t B,
                              int64_t D, int64_t L, int64_t N, int dtype, int flags,
                              void* stream) {
  return backward(2, x, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, dx, ddt_raw, dA_log, dBs, dCs,
                  dDs, ddt_bias, B, D, 1, L, N, dtype, stream, z, dz, flags, false, saved, true);
}

int ss2d_forward_routes_save(const void* u, const void* dt_raw, const float* A_log,
                             const void* Bs, const void* Cs, const float* Ds,
                             const float* dt_bias, const void* z, void* y, float* saved,
                             int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int dtype,
                             int flags, void* stream) {
  return forward(4, true, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, y, B, D, H, W, N, dtype,
                 flags, stream, nullptr, nullptr, 0, false, saved, true);
}

int ss1d_bidir_forward_routes_save(const void* u, const void* dt_raw, const float* A_log,
                                   const void* Bs, const void* Cs, const float* Ds,
                                   const float* dt_bias, const void* z, void* y, float* saved,
                                   int64_t B, int64_t D, int64_t L, int64_t N, int dtype,
                                   int flags, void* stream) {
  return forward(2, true, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, y, B, D, 1, L, N, dtype,
                 flags, stream, nullptr, nullptr, 0, false, saved, true);
}

int ss2d_backward_routes_saved(const void* u, const void* dt_raw, const float* A_log,
                               const void* Bs, const void* Cs, const float* Ds,
                               const float* dt_bias, const void* z, const float* saved,
                               const void* dy, void* du, void* ddt_raw, float* dA_log, void* dBs,
                               void* dCs, float* dDs, float* ddt_bias, void* dz, int64_t B,
                               int64_t D, int64_t H, int64_t W, int64_t N, int dtype, int flags,
                               void* stream) {
  return backward(4, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, du, ddt_raw, dA_log, dBs, dCs,
                  dDs, ddt_bias, B, D, H, W, N, dtype, stream, z, dz, flags, true, saved, true);
}

int ss1d_bidir_backward_routes_saved(const void* u, const void* dt_raw, const float* A_log,
                                     const void* Bs, const void* Cs, const float* Ds,
                                     const float* dt_bias, const void* z, const float* saved,
                                     const void* dy, void* du, void* ddt_raw, float* dA_log,
                                     void* dBs, void* dCs, float* dDs, float* ddt_bias, void* dz,
                                     int64_t B, int64_t D, int64_t L, int64_t N, int dtype,
                                     int flags, void* stream) {
  return backward(2, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, dy, du, ddt_raw, dA_log, dBs, dCs,
                  dDs, ddt_bias, B, D, 1, L, N, dtype, stream, z, dz, flags, true, saved, true);
}

int ss2d_project(const void* x, const float* conv_w, const float* conv_b,
                 const float* x_proj_w, const float* dt_proj_w, void* u, void* dt_raw, void* Bs,
                 void* Cs, int64_t B, int64_t D, int64_t H, int64_t W, int64_t N, int64_t R,
                 int64_t KW, int dtype, void* stream) {
  return project(4, x, conv_w, conv_b, x_proj_w, dt_proj_w, u, dt_raw, Bs, Cs, B, D, H, W, N,
                 R, KW, dtype, stream);
}

int ss1d_bidir_project(const void* x, const float* conv_w, const float* conv_b,
                       const float* x_proj_w, const float* dt_proj_w, void* u, void* dt_raw,
                       void* Bs, void* Cs, int64_t B, int64_t D, int64_t L, int64_t N,
                       int64_t R, int64_t KW, int dtype, void* stream) {
  return project(2, x, conv_w, conv_b, x_proj_w, dt_proj_w, u, dt_raw, Bs, Cs, B, D, 1, L, N,
                 R, KW, dtype, stream);
}

int ss2d_project_lr(const void* x, const float* conv_w, const float* conv_b,
                    const float* x_proj_w, void* u, void* dt_lr, void* Bs, void* Cs, int64_t B,
                    int64_t D, int64_t H, int64_t W, int64_t N, int64_t R, int64_t KW,
                    int dtype, void* stream) {
  return project(4, x, conv_w, conv_b, x_proj_w, nullptr, u, nullptr, Bs, Cs, B, D, H, W, N,
                 R, KW, dtype, stream, dt_lr);
}

int ss1d_bidir_project_lr(const void* x, const float* conv_w, const float* conv_b,
                          const float* x_proj_w, void* u, void* dt_lr, void* Bs, void* Cs,
                          int64_t B, int64_t D, int64_t L, int64_t N, int64_t R, int64_t KW,
                          int dtype, void* stream) {
  return project(2, x, conv_w, conv_b, x_proj_w, nullptr, u, nullptr, Bs, Cs, B, D, 1, L, N,
                 R, KW, dtype, stream, dt_lr);
}

int ss2d_forward_routes(const void* u, const void* dt_raw, const float* A_log, const void* Bs,
                        const void* Cs, const float* Ds, const float* dt_bias, const void* z,
                        void* y, int64_t B, int64_t D, int64_t H, int64_t W, int64_t N,
                        int dtype, int flags, void* stream) {
  return forward(4, true, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, y, B, D, H, W, N, dtype,
                 flags, stream);
}

int ss2d_forward_routes_lr(const void* u, const void* dt_lr, const float* dt_w,
                           const float* A_log, const void* Bs, const void* Cs, const float* Ds,
                           const float* dt_bias, const void* z, void* y, int64_t B, int64_t D,
                           int64_t H, int64_t W, int64_t N, int64_t R, int dtype, int flags,
                           void* stream) {
  return forward(4, true, u, nullptr, A_log, Bs, Cs, Ds, dt_bias, z, y, B, D, H, W, N, dtype,
                 flags, stream, dt_lr, dt_w, R);
}

int ss1d_bidir_forward_routes_lr(const void* u, const void* dt_lr, const float* dt_w,
                                 const float* A_log, const void* Bs, const void* Cs,
                                 const float* Ds, const float* dt_bias, const void* z, void* y,
                                 int64_t B, int64_t D, int64_t L, int64_t N, int64_t R,
                                 int dtype, int flags, void* stream) {
  return forward(2, true, u, nullptr, A_log, Bs, Cs, Ds, dt_bias, z, y, B, D, 1, L, N, dtype,
                 flags, stream, dt_lr, dt_w, R);
}

int ss1d_bidir_forward_routes(const void* u, const void* dt_raw, const float* A_log,
                              const void* Bs, const void* Cs, const float* Ds,
                              const float* dt_bias, const void* z, void* y, int64_t B,
                              int64_t D, int64_t L, int64_t N, int dtype, int flags,
                              void* stream) {
  return forward(2, true, u, dt_raw, A_log, Bs, Cs, Ds, dt_bias, z, y, B, D, 1, L, N, dtype,
                 flags, stream);
}

const char* ss2d_status_string(int status) {
  switch (status) {
    case SS2D_OK: return "success";
    case SS2D_ERR_NULL: return "a required pointer is NULL";
    case SS2D_ERR_SHAPE: return "invalid or out-of-range dimensions";
    case SS2D_ERR_UNSUPPORTED: return "unsupported state size N or data type";
    case SS2D_ERR_ALIGN: return "a pointer is not aligned to its element size";
    case SS2D_ERR_HIP: return "a HIP runtime call failed";
    case SS2D_ERR_ALIAS: return "the output overlaps an input";
    case SS2D_ERR_SCRATCH:
      return "the call needs more scratch than the fixed array of ss2d_forward_noalloc holds";
    default: return "unknown status";
  }
}

int ss2d_abi_version(void) { return SS2D_ABI_VERSION; }

int ss2d_set_launch_plan(int split, int64_t chunk_len) {
  if (split != 0 && split != 1 && split != 2 && split != 4) return SS2D_ERR_UNSUPPORTED;
  if (chunk_len < -1 || chunk_len >= kMaxL) return SS2D_ERR_SHAPE;
  g_split_override = split;
  g_chunk_override = chunk_len;
  return SS2D_OK;
}

int ss2d_last_hip_error(void) { return g_last_hip_error; }

int ss2d_scratch_trim(size_t keep_bytes, size_t* reserved) {
  if (reserved) *reserved = 0;
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return hip_fail(e);
  if (device < 0 || device >= kMaxDevices) return hip_fail(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_pool_mu);
  hipMemPool_t pool = g_pools[device];
  if (!pool) return SS2D_OK;  // no call has run on this device: nothing is reserved
  e = hipMemPoolTrimTo(pool, keep_bytes);
  if (e != hipSuccess) return hip_fail(e);
  if (reserved) {
    uint64_t now = 0;
    e = hipMemPoolGetAttribute(pool, hipMemPoolAttrReservedMemCurrent, &now);
    if (e != hipSuccess) return hip_fail(e);
    *reserved = static_cast<size_t>(now);
  }
  return SS2D_OK;
}

int ss2d_probe_issue_rates(double* out, void* stream) {
  if (!out) return SS2D_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int device = 0, cus = 0;
  hipError_t e = hipGetDevice(&device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return hip_fail(e);
  // 8 blocks of 4 waves per CU: 8 waves per SIMD, far more than needed to keep it issuing
  const int blocks = 8 * cus, block = ss2d::probe_block();
  const size_t sink_bytes = align256(size_t(blocks) * block * sizeof(float));
  const size_t clock_bytes = size_t(blocks) * 4 * sizeof(unsigned long long);
  char* ws = nullptr;
  int rc = scratch_alloc(&ws, sink_bytes + clock_bytes, st);
  if (rc != SS2D_OK) return rc;
  float* sink = reinterpret_cast<float*>(ws);
  auto* clocks = reinterpret_cast<unsigned long long*>(ws + sink_bytes);
  std::vector<unsigned long long> host(size_t(blocks) * 4);
  hipEvent_t ev[2] = {nullptr, nullptr};
  e = hipEventCreate(&ev[0]);
  if (e == hipSuccess) e = hipEventCreate(&ev[1]);
  const int iters = 2048;  // a few milliseconds per launch
  double rate[3] = {0.0, 0.0, 0.0}, hz = 0.0;
  // warm-up: ~0.1 s of the fused multiply-add probe brings the clock to its loaded rate
  for (int i = 0; i < 40 && e == hipSuccess; ++i)
    e = static_cast<hipError_t>(ss2d::launch_probe(0, blocks, iters, sink, clocks, st));
  for (int rep = 0; rep < 3 && e == hipSuccess; ++rep) {
    for (int kind = 0; kind < 3 && e == hipSuccess; ++kind) {
      e = hipEventRecord(ev[0], st);
      if (e == hipSuccess)
        e = static_cast<hipError_t>(ss2d::launch_probe(kind, blocks, iters, sink, clocks, st));
      if (e == hipSuccess) e = hipEventRecord(ev[1], st);
      if (e == hipSuccess) e = hipEventSynchronize(ev[1]);
      float ms = 0.0f;
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev[0], ev[1]);
      if (e != hipSuccess || ms <= 0.0f) break;
      int fmas = 0, exps = 0;
      ss2d::probe_counts(kind, &fmas, &exps);
      const double per_lane = double(iters) * (kind == 0 ? fmas : kind == 1 ? exps : exps);
      const double r = double(blocks) * block * per_lane / (double(ms) * 1e-3);
      if (r > rate[kind]) rate[kind] = r;
      if (kind == 2 && e == hipSuccess) {  // the sustained clock, from the last launch
        e = hipMemcpyAsync(host.data(), clocks, clock_bytes, hipMemcpyDeviceToHost, st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
        if (e == hipSuccess) {
          std::vector<double> f;
          for (int b = 0; b < blocks; ++b) {
            const double cyc = double(host[4 * b + 1] - host[4 * b + 0]);
            const double ref = double(host[4 * b + 3] - host[4 * b + 2]);
            if (ref > 0) f.push_back(cyc / ref * 1e8);  // the reference counter runs at 100 MHz
          }
          if (!f.empty()) {
            std::nth_element(f.begin(), f.begin() + f.size() / 2, f.end());
            hz = f[f.size() / 2];
          }
        }
      }
    }
  }
  for (hipEvent_t x : ev)
    if (x) (void)hipEventDestroy(x);
  const hipError_t fe = hipFreeAsync(ws, st);
  if (e != hipSuccess) return hip_fail(e);
  if (fe != hipSuccess) return hip_fail(fe);
  out[0] = rate[0];   // fused multiply-adds per second (lane operations)
  out[1] = rate[1];   // v_exp_f32 per second (lane operations)
  out[2] = rate[2];   // groups of 4 fused multiply-adds + 1 v_exp_f32 per second
  out[3] = hz;        // shader clock during the grouped probe (Hz)
  out[4] = cus;       // compute units
  return SS2D_OK;
}

int ss2d_timing_enable(int enable) {
  const int prev = g_timing.enabled ? 1 : 0;
  g_timing.enabled = enable != 0;
  return prev;
}

int ss2d_timing_read(double* ms, int64_t* launches) {
  double tot[SS2D_KERNEL_KINDS] = {};
  int64_t cnt[SS2D_KERNEL_KINDS] = {};
  int status = SS2D_OK;
  for (auto& t : g_timing.launches) {
    float e = 0.0f;
    hipError_t he = hipEventSynchronize(t.stop);
    if (he == hipSuccess) he = hipEventElapsedTime(&e, t.start, t.stop);
    if (he != hipSuccess) {
      status = hip_fail(he);
    } else if (t.kind >= 0 && t.kind < SS2D_KERNEL_KINDS) {
      tot[t.kind] += e;
      cnt[t.kind] += 1;
    }
    (void)hipEventDestroy(t.start);
    (void)hipEventDestroy(t.stop);
  }
  g_timing.launches.clear();
  for (int i = 0; i < SS2D_KERNEL_KINDS; ++i) {
    if (ms) ms[i] = tot[i];
    if (launches) launches[i] = cnt[i];
  }
  return status;
}

}  // extern "C"
