// Per-route front end: for every route k of every image, the route's input sequence through
// a causal depthwise conv and SiLU (u), x_proj (u -> [dt | B | C]) and dt_proj (dt -> dt_raw),
// written in the route's scan order, ready for the scan.  The structure is that of the
// pages' per-direction modules: the explainer's CrossScanModule holds one SelectiveSSM
// (Conv1d, SiLU, x_proj, dt_proj) per scan direction, and the Vim block (Vim summary,
// section 4.3) runs a Conv1d and a SiLU inside each path before generating delta, B and C.
//
// One workgroup (4 waves) owns 64 consecutive steps of one route of one image, all channels,
// in chunks of 64 channels (16 per wave):
//   1. each wave loads its 16 input rows of the 64 steps, one step per lane, plus the KW - 1
//      steps before them (routes 2 and 3 read the plane-transposed copy of x, the odd routes
//      read backwards, so every row is a run of consecutive addresses); all threads load the
//      chunk's slice of the x_proj weights and the conv taps into LDS;
//   2. conv + SiLU in fp32 in registers: the taps walk down the row by DPP wave shifts (lane
//      l takes lane l - 1's value, lane 0 the step before the tile); u is stored in the I/O
//      precision and its fp32 value goes to LDS, step-major;
//   3. x_proj on the matrix cores: the (R + 2N) x 64-channel weight slice times the
//      64-channel x 64-step slice of u, accumulated over the chunks in fp32 (bf16 I/O:
//      v_mfma_f32_16x16x32_bf16 on operands split into bf16 high and low parts, Whi uhi +
//      Whi ulo + Wlo uhi, which carries both to about 16 significant bits; fp32 I/O:
//      v_mfma_f32_16x16x4_f32).
// After the last chunk the (R + 2N) x 64 outputs go to LDS, the B and C rows are stored, and
// dt_proj (R fused multiply-adds per output, weights from scalar registers) writes dt_raw.
// The kernel is bound by HBM traffic: per step and route it reads D inputs (x, once per
// route) and writes 2D + 2N outputs.
#include "ss2d_device.h"

namespace ss2d {
namespace {

constexpr int kTT = 64;                        // steps per workgroup, one per lane
constexpr int kDC = 64;                        // channels per chunk
constexpr int kMT = kProjMaxM / 16;            // 16-row tiles of x_proj outputs, at most
constexpr int kWaveShr1 = 0x138;               // DPP wave_shr:1

// Weights are read through the constant address space: their loads are uniform across a
// wave and become scalar loads.
typedef const __attribute__((address_space(4))) float cfloat;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Buffer loads: a 128-bit resource (base, size in bytes) in scalar registers and a 32-bit
// byte offset per lane (plus, optionally, a uniform one).  A read at or past the size
// returns 0.
constexpr uint32_t kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, kRsrcWord3);
}
template <typename T> __device__ __forceinline__ float buf_load(__amdgpu_buffer_rsrc_t r,
                                                                uint32_t index);
template <> __device__ __forceinline__ float buf_load<uint16_t>(__amdgpu_buffer_rsrc_t r,
                                                                uint32_t index) {
  return Elem<uint16_t>::to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, index * 2u, 0, 0));
}
template <> __device__ __forceinline__ float buf_load<float>(__amdgpu_buffer_rsrc_t r,
                                                             uint32_t index) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, index * 4u, 0, 0));
}
// fp32 -> bf16 bits, round to nearest even, by the hardware conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
// The output element type from fp32 (bf16: rounded to nearest even).
template <typename T> __device__ __forceinline__ T out_elem(float x);
template <> __device__ __forceinline__ uint16_t out_elem<uint16_t>(float x) { return bf16_bits(x); }
template <> __device__ __forceinline__ float out_elem<float>(float x) { return x; }

// Store of element `index` (per lane) of a resource; at or past its size the store is
// dropped, which discards the lanes past the last step and whole absent rows.
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, uint32_t index, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, index * 2u, 0, 0);
}
__device__ __forceinline__ void buf_store(__amdgpu_buffer_rsrc_t r, uint32_t index, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, index * 4u, 0, 0);
}

// Element at byte offset voff (per lane) + soff (uniform) of the resource.
template <typename T> __device__ __forceinline__ float buf_load_at(__amdgpu_buffer_rsrc_t r,
                                                                   uint32_t voff,
                                                                   uint32_t soff);
template <> __device__ __forceinline__ float buf_load_at<uint16_t>(__amdgpu_buffer_rsrc_t r,
                                                                   uint32_t voff,
                                                                   uint32_t soff) {
  return Elem<uint16_t>::to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
}
template <> __device__ __forceinline__ float buf_load_at<float>(__amdgpu_buffer_rsrc_t r,
                                                                uint32_t voff, uint32_t soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// Matrix-core operands in LDS, per I/O type.  An operand array holds `rows` rows of kRowE
// elements (a row is a step of u or an output row of the weights; the columns are the 64
// channels of the chunk).  Each product covers one k-step of a 16 x 16 output tile: lane l
// supplies the k-step's channels CJ (l / 16) .. + CJ - 1 of weight row l % 16 and of u step
// l % 16; the same channel goes to the same operand slot on both sides.
template <typename T> struct ProjOps;

// bf16 I/O: both operands split into bf16 high and low parts (v = hi + lo to about 16
// significant bits), three products Whi uhi + Whi ulo + Wlo uhi per k-step on
// v_mfma_f32_16x16x32_bf16, so x_proj sees u and the weights at close to fp32 accuracy.
// An array holds the rows of high parts, then the rows of low parts.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
template <> struct ProjOps<uint16_t> {
  using E = uint16_t;
  static constexpr int kK = 32;          // channels per product
  static constexpr int kRowE = kDC + 8;  // 144-byte rows
  static constexpr int elems(int rows) { return 2 * rows * kRowE; }
  static __device__ __forceinline__ void put4(E* base, int rows, int row, int col,
                                              const float (&v)[4]) {
    uint32_t hi[2], lo[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t h2 = 0, l2 = 0;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float x = v[2 * j + q];
        const uint16_t h = bf16_bits(x);
        const uint16_t l = bf16_bits(x - Elem<uint16_t>::to_f32(h));
        h2 |= uint32_t(h) << (16 * q);
        l2 |= uint32_t(l) << (16 * q);
      }
      hi[j] = h2;
      lo[j] = l2;
    }
    *reinterpret_cast<uint2*>(&base[row * kRowE + col]) = make_uint2(hi[0], hi[1]);
    *reinterpret_cast<uint2*>(&base[(rows + row) * kRowE + col]) = make_uint2(lo[0], lo[1]);
  }
  static __device__ __forceinline__ v4f product(const E* w, int wrows, const E* u, int urows,
                                                v4f acc) {
    const v8bf wh = *reinterpret_cast<const v8bf*>(w);
    const v8bf wl = *reinterpret_cast<const v8bf*>(w + wrows * kRowE);
    const v8bf uh = *reinterpret_cast<const v8bf*>(u);
    const v8bf ul = *reinterpret_cast<const v8bf*>(u + urows * kRowE);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wh, uh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wh, ul, acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(wl, uh, acc, 0, 0, 0);
  }
};

// fp32 I/O: v_mfma_f32_16x16x4_f32 on the fp32 values (exact products, fp32 sums).
template <> struct ProjOps<float> {
  using E = float;
  static constexpr int kK = 4;
  static constexpr int kRowE = kDC + 4;  // 272-byte rows
  static constexpr int elems(int rows) { return rows * kRowE; }
  static __device__ __forceinline__ void put4(E* base, int, int row, int col,
                                              const float (&v)[4]) {
    *reinterpret_cast<float4*>(&base[row * kRowE + col]) = make_float4(v[0], v[1], v[2], v[3]);
  }
  static __device__ __forceinline__ v4f product(const E* w, int, const E* u, int, v4f acc) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(w[0], u[0], acc, 0, 0, 0);
  }
};

// Dynamic LDS: the u operand (kTT rows), the weight operand (MP rows, MP = R + 2N rounded
// up to 16), then the conv taps of the chunk's channels, sCW [kDC][kCW] fp32: entry sh < 8
// is the tap applied to the value sh steps back (w[KW - 1 - sh], 0 from sh = KW on), entry
// 8 the bias.  After the chunk loop the x_proj outputs, sXd [MP][kTT] fp32, take the space
// of the operands (MP * 64 * 4 bytes <= (64 + MP) * kRowE * 4 for both element types).
constexpr int kCW = 12;  // 48-byte rows: two 16-byte reads fetch the eight taps
template <typename T> __host__ __device__ constexpr size_t proj_lds_bytes(int MP) {
  return sizeof(typename ProjOps<T>::E) * size_t(ProjOps<T>::elems(kTT + MP)) +
         sizeof(float) * kDC * kCW;
}

// Everything a chunk of 64 channels loads from memory.
struct ProjStage {
  float v[16];       // the wave's 16 input rows at this lane's step
  float h[2];        // halos, packed: element e = i (KW - 1) + m is row i's value m + 1 steps
                     // before the tile, in lane e % 64 of h[e / 64]
  float cw[3];       // taps and biases (kDC x kCW entries over 256 threads)
  float wv[kMT][4];  // x_proj weight slice: row idx / 16, channels 4 (idx % 16) .. + 3
};

// KWC > 0 fixes the conv length at compile time (the common d_conv = 4); KWC = 0 reads it
// from the arguments.
template <typename T, int KWC>
__global__ __launch_bounds__(256) void k_project(ProjArgs a) {
  using Ops = ProjOps<T>;
  using E = typename Ops::E;
  constexpr int KS = Ops::kK;                 // channels per product
  constexpr int CJ = KS / 4;                  // channels per lane per product
  extern __shared__ __align__(16) float smem[];

  // wave is uniform across a wave: saying so keeps row addresses in scalar registers
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k = blockIdx.y, b = blockIdx.z;
  const int L = a.L, D = a.D, N = a.N, R = a.R;
  const int KW = KWC > 0 ? KWC : a.KW;
  const int M = R + 2 * N;
  const int MT = (M + 15) / 16, MP = 16 * MT;
  E* sU = reinterpret_cast<E*>(smem);
  E* sW = sU + Ops::elems(kTT);
  float (*sCW)[kCW] = reinterpret_cast<float (*)[kCW]>(sW + Ops::elems(MP));
  float (*sXd)[kTT] = reinterpret_cast<float (*)[kTT]>(smem);

  const int t0 = blockIdx.x * kTT;
  const int t = t0 + lane;
  const bool col = (a.K == 4) && (k >= 2);
  const bool rev = (k & 1) != 0;
  const T* xplanes = static_cast<const T*>(col ? a.x_col : a.x_row) + int64_t(b) * D * L;
  const int64_t bk = int64_t(b) * a.K + k;
  T* u_out = static_cast<T*>(a.u) + bk * D * L;
  const float* wx = a.x_proj_w + int64_t(k) * M * D;
  const float* wc = a.conv_w + int64_t(k) * D * KW;
  const float* bc = a.conv_b + int64_t(k) * D;
  const int n16 = lane & 15, g = lane >> 4;

  // Step s of a row sits at element (rev ? L - 1 - s : s) of the row.  Row loads go through
  // one buffer resource per row, sized 0 for rows past D: lanes past the last step and
  // absent rows read 0 from the buffer's range check, with no select or branch that would
  // make the compiler wait for each load before issuing the next.
  const uint32_t xo = uint32_t(rev ? L - 1 - t : t);  // past the row when t >= L
  const uint32_t row_bytes = uint32_t(L) * sizeof(T);
  const __amdgpu_buffer_rsrc_t wx_r = make_rsrc(wx, uint32_t(M) * D * 4u);

  auto load_stage = [&](int d0, ProjStage& st) {
    const int nrows = min(kDC, D - d0);
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(xplanes + int64_t(d0) * L, nrows * row_bytes);
    const T* rp = xplanes + int64_t(d0 + wave * 16) * L;  // absent rows: size 0, no access
#pragma unroll
    for (int i = 0; i < 16; ++i, rp += L)
      st.v[i] = buf_load<T>(make_rsrc(rp, wave * 16 + i < nrows ? row_bytes : 0u), xo);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int e = 64 * p + lane;
      const int i = KW > 1 ? e / (KW - 1) : 16, m = KW > 1 ? e % (KW - 1) : 0;
      const int c = wave * 16 + i, s = t0 - 1 - m;
      const bool ok = i < 16 && c < nrows && s >= 0;
      const int sc = ok ? s : 0, cc = ok ? c : 0;
      const uint32_t off = (uint32_t(cc) * uint32_t(L) + uint32_t(rev ? L - 1 - sc : sc)) *
                           sizeof(T);
      const float hv = buf_load_at<T>(xr, off, 0);
      st.h[p] = ok ? hv : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int idx = tid + 256 * i, c = idx / kCW, j = idx % kCW;
      const bool row_ok = idx < kDC * kCW && c < nrows;
      const bool is_tap = row_ok && j < kProjMaxKW && j < KW, is_bias = row_ok && j == 8;
      // one load from a selected address (no branch): the tap, the bias, or a dummy
      const float* src = is_tap ? wc + int64_t(d0 + c) * KW + (KW - 1 - j)
                                : (is_bias ? bc + d0 + c : wc);
      const float val = *src;
      st.cw[i] = (is_tap || is_bias) ? val : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kMT; ++i) {
      const int idx = tid + 256 * i, m = idx / 16, c = d0 + 4 * (idx % 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float w = buf_load<float>(wx_r, uint32_t(m * D + c + j));  // m >= M reads 0
        st.wv[i][j] = c + j < D ? w : 0.0f;
      }
    }
  };

  v4f acc[kMT];
#pragma unroll
  for (int i = 0; i < kMT; ++i) acc[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  for (int d0 = 0; d0 < D; d0 += kDC) {
    // ---- 1. loads; this chunk's weights and taps to LDS, its input rows stay in registers
    ProjStage nx;
    load_stage(d0, nx);
    __syncthreads();  // the previous chunk's products have read sW
#pragma unroll
    for (int i = 0; i < kMT; ++i) {
      const int idx = tid + 256 * i;
      if (i < MT) Ops::put4(sW, MP, idx / 16, 4 * (idx % 16), nx.wv[i]);
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int idx = tid + 256 * i;
      if (idx < kDC * kCW) sCW[idx / kCW][idx % kCW] = nx.cw[i];
    }
    float v[16], h[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = nx.v[i];
    h[0] = nx.h[0];
    h[1] = nx.h[1];
    __syncthreads();

    // ---- 2. conv + SiLU in registers, four rows at a time --------------------------------
    T* up = u_out + int64_t(d0 + wave * 16) * L;  // this row's u; absent rows: size 0
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float uv[4];
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int i = 4 * q + i4;
        const int d = d0 + wave * 16 + i;
        const float4 w03 = *reinterpret_cast<const float4*>(&sCW[wave * 16 + i][0]);
        const float4 w47 = *reinterpret_cast<const float4*>(&sCW[wave * 16 + i][4]);
        const float ws[kProjMaxKW] = {w03.x, w03.y, w03.z, w03.w, w47.x, w47.y, w47.z, w47.w};
        float cur = v[i];
        float cv = fmaf(ws[0], cur, sCW[wave * 16 + i][8]);
#pragma unroll
        for (int sh = 1; sh < kProjMaxKW; ++sh) {
          if (sh < KW) {
            // lane l takes lane l - 1's value; lane 0 takes the value sh steps before the
            // tile (packed halo element i (KW - 1) + sh - 1)
            const int e = i * (KW - 1) + sh - 1;
            const int hb = __builtin_amdgcn_readlane(
                __float_as_int(e < 64 ? h[0] : h[1]), e & 63);
            cur = __int_as_float(__builtin_amdgcn_update_dpp(hb, __float_as_int(cur),
                                                             kWaveShr1, 0xf, 0xf, false));
            cv = fmaf(ws[sh], cur, cv);
          }
        }
        uv[i4] = d < D ? silu_f32(cv) : 0.0f;
        buf_store(make_rsrc(up, d < D ? row_bytes : 0u), uint32_t(t), out_elem<T>(uv[i4]));
        up += L;
      }
      Ops::put4(sU, kTT, lane, wave * 16 + 4 * q, uv);
    }
    __syncthreads();

    // ---- 3. x_proj on the matrix cores: wave w owns steps 16 w .. 16 w + 15 --------------
    const E* urow = sU + (wave * 16 + n16) * Ops::kRowE + CJ * g;
    const E* wrow = sW + n16 * Ops::kRowE + CJ * g;
#pragma unroll 1
    for (int kk = 0; kk < kDC / KS; ++kk) {
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        if (mt < MT)
          acc[mt] = Ops::product(wrow + mt * 16 * Ops::kRowE + kk * KS, MP, urow + kk * KS,
                                 kTT, acc[mt]);
      }
    }
  }
  __syncthreads();  // the last products have read sU and sW

  // ---- 4. x_proj outputs to LDS: lane holds rows 4 (l / 16) + j of column l % 16 -------
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
    if (mt < MT) {
#pragma unroll
      for (int j = 0; j < 4; ++j) sXd[mt * 16 + 4 * g + j][wave * 16 + n16] = acc[mt][j];
    }
  }
  __syncthreads();

  // ---- 5. dt_proj (wave w: channels 16 w .. 16 w + 15 of each chunk of 64), then B, C ---
  T* dt_out = static_cast<T*>(a.dt_raw) + bk * D * L;
  cfloat* wdt = (cfloat*)(a.dt_proj_w + int64_t(k) * D * R);
#pragma unroll 1
  for (int d0 = wave * 16; d0 < D; d0 += kDC) {
    float dv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) dv[i] = 0.0f;
    for (int r = 0; r < R; ++r) {
      const float xr = sXd[r][lane];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        dv[i] = fmaf(wdt[int64_t(min(d0 + i, D - 1)) * R + r], xr, dv[i]);
    }
    T* dp = dt_out + int64_t(d0) * L;
#pragma unroll
    for (int i = 0; i < 16; ++i, dp += L)
      buf_store(make_rsrc(dp, d0 + i < D ? row_bytes : 0u), uint32_t(t), out_elem<T>(dv[i]));
  }
  // B and C: wave w stores rows w, w + 4, ... of the 2N rows (B first), one step per lane
  T* Bo = static_cast<T*>(a.Bs) + bk * N * L;
  T* Co = static_cast<T*>(a.Cs) + bk * N * L;
  for (int row = wave; row < 2 * N; row += 4) {
    T* dst = row < N ? Bo + int64_t(row) * L : Co + int64_t(row - N) * L;
    buf_store(make_rsrc(dst, row_bytes), uint32_t(t), out_elem<T>(sXd[R + row][lane]));
  }
}

}  // namespace

int launch_project(const ProjArgs& a, int dtype, hipStream_t st) {
  if (a.B <= 0 || a.D <= 0 || a.L <= 0) return 0;
  const dim3 grid((a.L + kTT - 1) / kTT, a.K, a.B);
  const int MP = 16 * ((a.R + 2 * a.N + 15) / 16);
  const bool kw4 = a.KW == 4;
  if (dtype == 0) {
    if (kw4)
      k_project<float, 4><<<grid, 256, proj_lds_bytes<float>(MP), st>>>(a);
    else
      k_project<float, 0><<<grid, 256, proj_lds_bytes<float>(MP), st>>>(a);
  } else {
    if (kw4)
      k_project<uint16_t, 4><<<grid, 256, proj_lds_bytes<uint16_t>(MP), st>>>(a);
    else
      k_project<uint16_t, 0><<<grid, 256, proj_lds_bytes<uint16_t>(MP), st>>>(a);
  }
  return static_cast<int>(hipGetLastError());
}

}  // namespace ss2d
