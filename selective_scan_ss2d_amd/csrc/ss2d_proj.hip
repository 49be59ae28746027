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
#include <type_traits>

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
// fp32 -> bf16 bits, round to nearest even, by the hardware conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
// The output element type from fp32 (bf16: rounded to nearest even).
template <typename T> __device__ __forceinline__ T out_elem(float x);
template <> __device__ __forceinline__ uint16_t out_elem<uint16_t>(float x) { return bf16_bits(x); }
template <> __device__ __forceinline__ float out_elem<float>(float x) { return x; }

// Store at byte offset voff (per lane) + soff (uniform) of the resource; dropped by the
// hardware when voff is at or past the resource's size.
__device__ __forceinline__ void buf_store_at(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                             uint32_t soff, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, voff, soff, 0);
}
__device__ __forceinline__ void buf_store_at(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                             uint32_t soff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
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

// Four consecutive elements of a row by one 8-byte (bf16) or 16-byte (fp32) buffer access;
// `rev` reverses their order (the backward routes walk rows downwards).
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
template <typename T> struct Quad;
template <> struct Quad<uint16_t> {
  // Byte selectors of v_perm_b32 that widen element k[j] of the loaded 8 bytes to fp32 (its
  // two bytes on top, zero bytes below) as x[j]: k[j] = j, or 3 - j with rev, for a whole
  // quad; any 0..3 per lane at the end of a row whose length is not a multiple of 4.
  struct Sel {
    uint32_t s[4];
    __device__ __forceinline__ explicit Sel(bool rev) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t k = rev ? 3 - j : j;
        s[j] = ((2 * k + 1) << 24) | ((2 * k) << 16) | 0x0c0cu;
      }
    }
    __device__ __forceinline__ explicit Sel(const int (&k)[4]) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        s[j] = ((2u * k[j] + 1) << 24) | ((2u * k[j]) << 16) | 0x0c0cu;
    }
  };
  static __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t soff, const Sel& sel, float (&x)[4]) {
    const v2u p = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = __uint_as_float(__builtin_amdgcn_perm(p.y, p.x, sel.s[j]));
  }
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff, const float (&u)[4]);
};
template <> struct Quad<float> {
  // x[j] = element j, or 3 - j with rev (whole quads); element k[j] per lane otherwise
  struct Sel {
    bool rev, any;
    int k[4];
    __device__ __forceinline__ explicit Sel(bool r) : rev(r), any(false), k{0, 1, 2, 3} {}
    __device__ __forceinline__ explicit Sel(const int (&kk)[4])
        : rev(false), any(true), k{kk[0], kk[1], kk[2], kk[3]} {}
  };
  static __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t soff, const Sel& sel, float (&x)[4]) {
    const v4u p = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    const float a[4] = {__uint_as_float(p.x), __uint_as_float(p.y), __uint_as_float(p.z),
                        __uint_as_float(p.w)};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (sel.any) {
        const int k = sel.k[j];
        x[j] = k == 0 ? a[0] : k == 1 ? a[1] : k == 2 ? a[2] : a[3];
      } else {
        x[j] = sel.rev ? a[3 - j] : a[j];
      }
    }
  }
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff, const float (&u)[4]) {
    const v4u p = {__float_as_uint(u[0]), __float_as_uint(u[1]), __float_as_uint(u[2]),
                   __float_as_uint(u[3])};
    __builtin_amdgcn_raw_buffer_store_b128(p, r, voff, soff, 0);
  }
};

// Two fp32 values to packed bf16 high parts (returned) and low parts (lo): hi = bf16(x),
// lo = bf16(x - hi), each pair by one v_cvt_pk_bf16_f32.
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t split2(float x0, float x1, uint32_t& lo) {
  const v2f x = {x0, x1};
  const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, v2bf));
  const v2f h = {__uint_as_float(hb << 16), __uint_as_float(hb & 0xffff0000u)};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(x - h, v2bf));
  return hb;
}

__device__ __forceinline__ void Quad<uint16_t>::store(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                      uint32_t soff, const float (&u)[4]) {
  const v2f u01 = {u[0], u[1]}, u23 = {u[2], u[3]};
  const v2u p = {__builtin_bit_cast(uint32_t, __builtin_convertvector(u01, v2bf)),
                 __builtin_bit_cast(uint32_t, __builtin_convertvector(u23, v2bf))};
  __builtin_amdgcn_raw_buffer_store_b64(p, r, voff, soff, 0);
}

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
  // Position of channel col in row `row` of the u operand: its 8-channel (16-byte) group is
  // XORed with bits 2..4 of the row.  The column writes of the four-steps-per-lane kernel
  // touch rows 4 apart, which would otherwise fall on two LDS bank groups (8-way
  // conflicts); the product's 16-byte reads stay whole.
  static __device__ __forceinline__ int ucol(int row, int col) {
    return (((col >> 3) ^ ((row >> 2) & 7)) << 3) | (col & 7);
  }
  static __device__ __forceinline__ const E* u_at(const E* base, int row, int col) {
    return base + row * kRowE + ucol(row, col);
  }
  static __device__ __forceinline__ void put4(E* base, int rows, int row, int col,
                                              const float (&v)[4]) {
    uint32_t hi[2], lo[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) hi[j] = split2(v[2 * j], v[2 * j + 1], lo[j]);
    const int c = ucol(row, col);
    *reinterpret_cast<uint2*>(&base[row * kRowE + c]) = make_uint2(hi[0], hi[1]);
    *reinterpret_cast<uint2*>(&base[(rows + row) * kRowE + c]) = make_uint2(lo[0], lo[1]);
  }
  // v[j] to column col of rows row0 + j (four steps of one channel)
  static __device__ __forceinline__ void put_col4(E* base, int rows, int row0, int col,
                                                  const float (&v)[4]) {
    uint32_t lo01, lo23;
    const uint32_t hi01 = split2(v[0], v[1], lo01), hi23 = split2(v[2], v[3], lo23);
    const uint32_t hs[4] = {hi01 & 0xffffu, hi01 >> 16, hi23 & 0xffffu, hi23 >> 16};
    const uint32_t ls[4] = {lo01 & 0xffffu, lo01 >> 16, lo23 & 0xffffu, lo23 >> 16};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = ucol(row0 + j, col);
      base[(row0 + j) * kRowE + c] = static_cast<E>(hs[j]);
      base[(rows + row0 + j) * kRowE + c] = static_cast<E>(ls[j]);
    }
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
  // Position of channel col in row `row` of the u operand: bits 2..4 of the column XORed
  // with bits 2..4 of the row (the same bank spreading as for bfloat16 operands).
  static __device__ __forceinline__ int ucol(int row, int col) {
    return col ^ (((row >> 2) & 7) << 2);
  }
  static __device__ __forceinline__ const E* u_at(const E* base, int row, int col) {
    return base + row * kRowE + ucol(row, col);
  }
  static __device__ __forceinline__ void put4(E* base, int, int row, int col,
                                              const float (&v)[4]) {
    *reinterpret_cast<float4*>(&base[row * kRowE + ucol(row, col)]) =
        make_float4(v[0], v[1], v[2], v[3]);
  }
  static __device__ __forceinline__ void put_col4(E* base, int, int row0, int col,
                                                  const float (&v)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) base[(row0 + j) * kRowE + ucol(row0 + j, col)] = v[j];
  }
  static __device__ __forceinline__ v4f product(const E* w, int, const E* u, int, v4f acc) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(w[0], u[0], acc, 0, 0, 0);
  }
};

// The per-chunk weight image: the weight operand (MP rows, MP = R + 2N rounded up to 16) in
// the operand layout, then the conv taps of the chunk's channels, [kDC][kCW] fp32 (entry
// sh < 8: the tap applied to the value sh steps back, w[KW - 1 - sh], 0 from sh = KW on;
// entry 8: the bias), padded to a multiple of 1 KB.  k_project_prep writes one image per
// (route, chunk) to memory; k_project copies the chunk's image to LDS with memory-to-LDS
// loads (1 KB per wave instruction).
constexpr int kCW = 12;  // 48-byte rows: two 16-byte reads fetch the eight taps
template <typename T> __host__ __device__ constexpr int proj_img_bytes(int MP) {
  return (int(sizeof(typename ProjOps<T>::E)) * ProjOps<T>::elems(MP) + 4 * kDC * kCW +
          1023) / 1024 * 1024;
}
// Dynamic LDS: the u operand (kTT rows), then the weight image.  After the chunk loop the
// x_proj outputs, sXd [MP][kTT] fp32, take the space of both (MP * 64 * 4 bytes is less).
template <typename T> __host__ __device__ constexpr size_t proj_lds_bytes(int MP) {
  return sizeof(typename ProjOps<T>::E) * size_t(ProjOps<T>::elems(kTT)) +
         size_t(proj_img_bytes<T>(MP));
}

// One block per (chunk, route): the weight image of that chunk.
template <typename T>
__global__ __launch_bounds__(256) void k_project_prep(ProjArgs a) {
  using Ops = ProjOps<T>;
  using E = typename Ops::E;
  const int ch = blockIdx.x, k = blockIdx.y;
  const int D = a.D, N = a.N, R = a.R, KW = a.KW;
  const int M = R + 2 * N, MP = 16 * ((M + 15) / 16);
  const int d0 = ch * kDC;
  char* img = static_cast<char*>(const_cast<void*>(a.wprep)) +
              (int64_t(k) * a.nchunks + ch) * a.img_bytes;
  E* w = reinterpret_cast<E*>(img);
  const float* wx = a.x_proj_w + int64_t(k) * M * D;
  const int plane = MP * Ops::kRowE;  // elements of one operand plane
  for (int e = threadIdx.x; e < plane; e += blockDim.x) {
    const int m = e / Ops::kRowE, c = e % Ops::kRowE;
    const float v = (m < M && c < kDC && d0 + c < D) ? wx[int64_t(m) * D + d0 + c] : 0.0f;
    if constexpr (sizeof(E) == 2) {  // high part, then low part
      const uint16_t h = bf16_bits(v);
      w[e] = h;
      w[plane + e] = bf16_bits(v - Elem<uint16_t>::to_f32(h));
    } else {
      w[e] = v;
    }
  }
  float* taps = reinterpret_cast<float*>(img + sizeof(E) * Ops::elems(MP));
  for (int e = threadIdx.x; e < kDC * kCW; e += blockDim.x) {
    const int c = e / kCW, j = e % kCW, d = d0 + c;
    float v = 0.0f;
    if (d < D && j < kProjMaxKW && j < KW) v = a.conv_w[(int64_t(k) * D + d) * KW + KW - 1 - j];
    if (d < D && j == kProjMaxKW) v = a.conv_b[int64_t(k) * D + d];
    taps[e] = v;
  }
}

// The block's image b, route k and first step t0.  The grid is (tiles, K, B); blocks are
// taken in an order that keeps a block's halo (the KW - 1 steps before its tile, in the
// previous tile's cache lines) in the L2 of its XCD: each XCD runs a contiguous range of
// (image, route pair) groups, tile after tile (the pair's two routes in turn at each tile),
// so the block of the previous tile has just fetched those lines there.  In launch order
// the tiles of a row go round the 8 XCDs and every halo is a miss.  (Mirroring the odd
// route's tiles as well, so that both routes of a pair read the same rows together, halves
// the rows fetched from memory but was measured slower.)
struct ProjBlock {
  int b, k, t0;
};
__device__ __forceinline__ ProjBlock proj_block() {
  const unsigned T = gridDim.x, K = gridDim.y;
  const unsigned lin = blockIdx.x + T * (blockIdx.y + K * blockIdx.z);
  unsigned q = xcd_local_order(lin, T * K * gridDim.z);
  const unsigned r = q % 2;  // route within the pair
  q /= 2;
  const unsigned tile = q % T;
  q /= T;
  const unsigned pair = q % (K / 2);
  return {static_cast<int>(q / (K / 2)), static_cast<int>(2 * pair + r),
          static_cast<int>(tile) * kTT};
}

// Everything a chunk of 64 channels loads into registers.
struct ProjStage {
  float v[16];       // the wave's 16 input rows at this lane's step
  float h[2];        // halos, packed: element e = i (KW - 1) + m is row i's value m + 1 steps
                     // before the tile, in lane e % 64 of h[e / 64]
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
  const ProjBlock blk = proj_block();
  const int k = blk.k, b = blk.b;
  const int L = a.L, D = a.D, N = a.N, R = a.R;
  const int KW = KWC > 0 ? KWC : a.KW;
  const int M = R + 2 * N;
  const int MT = (M + 15) / 16, MP = 16 * MT;
  E* sU = reinterpret_cast<E*>(smem);
  E* sW = sU + Ops::elems(kTT);  // the weight image: operand, then the taps
  float (*sCW)[kCW] = reinterpret_cast<float (*)[kCW]>(sW + Ops::elems(MP));
  const int img_bytes = a.img_bytes;
  float (*sXd)[kTT] = reinterpret_cast<float (*)[kTT]>(smem);

  const int t0 = blk.t0;
  const int t = t0 + lane;
  const bool col = (a.K == 4) && (k >= 2);
  const bool rev = (k & 1) != 0;
  const T* xplanes = static_cast<const T*>(col ? a.x_col : a.x_row) + int64_t(b) * D * L;
  const int64_t bk = int64_t(b) * a.K + k;
  T* u_out = static_cast<T*>(a.u) + bk * D * L;
  const int n16 = lane & 15, g = lane >> 4;

  // Memory goes through buffer resources over whole planes (the host keeps each plane set
  // below 2^31 bytes): a scalar byte offset selects the row, a per-lane one the step.
  // Step s of a row sits at element (rev ? L - 1 - s : s).  Loads read clamped, in-range
  // addresses (the rows past D and steps past L - 1 repeat the last ones, whose values are
  // never stored; the u of rows past D is set to 0 before it reaches the contraction), so
  // no select or branch sits between a load and the next one and all stay in flight.
  // Stores use an offset past the resource for lanes past the last step: the hardware
  // drops them.
  const uint32_t row_bytes = uint32_t(L) * sizeof(T);
  const uint32_t xo = uint32_t(rev ? L - 1 - min(t, L - 1) : min(t, L - 1)) * sizeof(T);
  const uint32_t so_t = t < L ? uint32_t(t) * sizeof(T) : 0x80000000u;
  const __amdgpu_buffer_rsrc_t x_r = make_rsrc(xplanes, uint32_t(D) * row_bytes);
  const __amdgpu_buffer_rsrc_t u_r = make_rsrc(u_out, uint32_t(D) * row_bytes);

  auto load_stage = [&](int d0, ProjStage& st) {
    const int nrows = min(kDC, D - d0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t row = uint32_t(min(d0 + wave * 16 + i, D - 1));
      st.v[i] = buf_load_at<T>(x_r, xo, row * row_bytes);
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int e = 64 * p + lane;
      const int i = KW > 1 ? e / (KW - 1) : 16, m = KW > 1 ? e % (KW - 1) : 0;
      const int c = wave * 16 + i, s = t0 - 1 - m;
      const bool ok = i < 16 && c < nrows && s >= 0;
      const int sc = ok ? s : 0, cc = ok ? c : 0;
      const uint32_t off = (uint32_t(cc) * uint32_t(L) + uint32_t(rev ? L - 1 - sc : sc)) *
                           sizeof(T);
      const float hv = buf_load_at<T>(x_r, off, uint32_t(d0) * row_bytes);
      st.h[p] = ok ? hv : 0.0f;
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
    {
      typedef __attribute__((address_space(3))) void lds_void;
      const char* img = static_cast<const char*>(a.wprep) +
                        (int64_t(k) * a.nchunks + d0 / kDC) * img_bytes;
      for (int j = wave; j < img_bytes / 1024; j += 4)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(img + j * 1024 + lane * 16),
                                         (lds_void*)(reinterpret_cast<char*>(sW) + j * 1024),
                                         16, 0, 0);
      __builtin_amdgcn_s_waitcnt(0);  // the image and this chunk's rows have arrived
    }
    float v[16], h[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = nx.v[i];
    h[0] = nx.h[0];
    h[1] = nx.h[1];
    __syncthreads();

    // ---- 2. conv + SiLU in registers, four rows at a time --------------------------------
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
        if (d < D) buf_store_at(u_r, so_t, uint32_t(d) * row_bytes, out_elem<T>(uv[i4]));
      }
      Ops::put4(sU, kTT, lane, wave * 16 + 4 * q, uv);
    }
    __syncthreads();

    // ---- 3. x_proj on the matrix cores: wave w owns steps 16 w .. 16 w + 15 --------------
    const int urow = wave * 16 + n16;  // this lane's step in the u operand
    const E* wrow = sW + n16 * Ops::kRowE + CJ * g;
#pragma unroll 1
    for (int kk = 0; kk < kDC / KS; ++kk) {
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        if (mt < MT)
          acc[mt] = Ops::product(wrow + mt * 16 * Ops::kRowE + kk * KS, MP,
                                 Ops::u_at(sU, urow, kk * KS + CJ * g), kTT, acc[mt]);
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
  if (a.dt_lr) {  // dt_proj folded into the scan: store x_proj's dt rows instead
    const __amdgpu_buffer_rsrc_t lr_r =
        make_rsrc(static_cast<T*>(a.dt_lr) + bk * R * L, uint32_t(R) * row_bytes);
    for (int row = wave; row < R; row += 4)
      buf_store_at(lr_r, so_t, uint32_t(row) * row_bytes, out_elem<T>(sXd[row][lane]));
  }
  T* dt_out = a.dt_lr ? nullptr : static_cast<T*>(a.dt_raw) + bk * D * L;
  const __amdgpu_buffer_rsrc_t dt_r =
      make_rsrc(dt_out, a.dt_lr ? 0u : uint32_t(D) * row_bytes);
  cfloat* wdt = (cfloat*)(a.dt_lr ? nullptr : a.dt_proj_w + int64_t(k) * D * R);
#pragma unroll 1
  for (int d0 = wave * 16; a.dt_lr == nullptr && d0 < D; d0 += kDC) {
    float dv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) dv[i] = 0.0f;
    if (d0 + 16 <= D) {  // whole group: weights of the 16 rows by stride-R scalar loads
      for (int r = 0; r < R; ++r) {
        const float xr = sXd[r][lane];
        cfloat* w = wdt + int64_t(d0) * R + r;
#pragma unroll
        for (int i = 0; i < 16; ++i) dv[i] = fmaf(w[i * R], xr, dv[i]);
      }
    } else {
      for (int r = 0; r < R; ++r) {
        const float xr = sXd[r][lane];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          dv[i] = fmaf(wdt[int64_t(min(d0 + i, D - 1)) * R + r], xr, dv[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (d0 + i < D) buf_store_at(dt_r, so_t, uint32_t(d0 + i) * row_bytes, out_elem<T>(dv[i]));
  }
  // B and C: wave w stores rows w, w + 4, ... of the 2N rows (B first), one step per lane
  const __amdgpu_buffer_rsrc_t b_r = make_rsrc(static_cast<T*>(a.Bs) + bk * N * L,
                                               uint32_t(N) * row_bytes);
  const __amdgpu_buffer_rsrc_t c_r = make_rsrc(static_cast<T*>(a.Cs) + bk * N * L,
                                               uint32_t(N) * row_bytes);
  for (int row = wave; row < 2 * N; row += 4) {
    const T v = out_elem<T>(sXd[R + row][lane]);
    if (row < N)
      buf_store_at(b_r, so_t, uint32_t(row) * row_bytes, v);
    else
      buf_store_at(c_r, so_t, uint32_t(row - N) * row_bytes, v);
  }
}

// The same front end with four steps per lane, for KW = 4 and L a multiple of 4 (the
// common case): a 16-lane row of a wave covers the 64 steps of one channel, so a wave holds
// four channels per register.  Rows move with 8-byte (bf16) or 16-byte (fp32) accesses, and
// the conv needs the three values before a lane's first step only once per four outputs:
// three DPP row shifts (lane l takes lane l - 1's value within its 16-lane row; lane 0 of a
// row takes the halo), then 16 FMAs for the four outputs.
constexpr int kRowShr1 = 0x111;  // DPP row_shr:1

// MTC: 16-row tiles of x_proj outputs (R + 2N rounded up to 16, over 16), fixed at compile
// time so that the accumulators stay in place.  ANYL: L is not a multiple of 4 (L >= 4),
// so the lane holding a row's last steps has one to three of its four: it loads the last
// four elements of the row (an in-range quad) and picks its own from them per lane, and
// stores element by element.
template <typename T, int MTC, bool ANYL>
__global__ __launch_bounds__(256) void k_project4(ProjArgs a) {
  using Ops = ProjOps<T>;
  using E = typename Ops::E;
  constexpr int KS = Ops::kK;
  constexpr int CJ = KS / 4;
  extern __shared__ __align__(16) float smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const ProjBlock blk = proj_block();
  const int k = blk.k, b = blk.b;
  const int L = a.L, D = a.D, N = a.N, R = a.R;
  const int M = R + 2 * N;
  constexpr int MT = MTC;
  const int MP = 16 * MT;
  (void)M;
  E* sU = reinterpret_cast<E*>(smem);
  E* sW = sU + Ops::elems(kTT);
  float (*sCW)[kCW] = reinterpret_cast<float (*)[kCW]>(sW + Ops::elems(MP));
  const int img_bytes = a.img_bytes;
  float (*sXd)[kTT] = reinterpret_cast<float (*)[kTT]>(smem);

  const int t0 = blk.t0;
  const bool col = (a.K == 4) && (k >= 2);
  const bool rev = (k & 1) != 0;
  const T* xplanes = static_cast<const T*>(col ? a.x_col : a.x_row) + int64_t(b) * D * L;
  const int64_t bk = int64_t(b) * a.K + k;
  const int n16 = lane & 15, g = lane >> 4;
  const int sr = lane >> 4, q4 = lane & 15;  // this lane's channel of the four, step group
  const int ts = t0 + 4 * q4;                // first of this lane's four steps
  const bool ok4 = ts < L;                   // at least one of them exists
  const int nv = ANYL ? min(max(L - ts, 0), 4) : (ok4 ? 4 : 0);  // how many exist

  // Offsets in bytes (the host keeps each plane set below 2^31 bytes).  Loads read clamped,
  // in-range addresses (a quad that would run past the row's end, or start before it on a
  // backward route, is moved inside it and the lane picks its elements out of it); stores
  // of absent steps or channels get an offset past the resource, which the hardware drops.
  const uint32_t row_bytes = uint32_t(L) * sizeof(T);
  const int qs = rev ? max(L - 4 - ts, 0) : min(ts, L - 4);  // first element loaded
  const uint32_t xo4 = uint32_t(qs) * sizeof(T);
  const uint32_t st4 = uint32_t(ts) * sizeof(T);
  constexpr uint32_t kDrop = 0x80000000u;
  const __amdgpu_buffer_rsrc_t x_r = make_rsrc(xplanes, uint32_t(D) * row_bytes);
  const __amdgpu_buffer_rsrc_t u_r =
      make_rsrc(static_cast<T*>(a.u) + bk * D * L, uint32_t(D) * row_bytes);

  v4f acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // four steps of the wave's 16 channels of a chunk (lane group G: channels 4 G .. 4 G + 3),
  // and the three steps before the tile (zero before the first step: t0 is a multiple of
  // 64, so either all three exist or none)
  // Two register sets, used in turn: a chunk is processed from one while the next chunk's
  // rows load into the other.
  float xA[4][4], hA[4][3], xB[4][4], hB[4][3];
  auto make_sel = [&]() {
    if constexpr (ANYL) {
      int kq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)  // element of step ts + j in the loaded quad
        kq[j] = min(max(rev ? L - 1 - ts - j - qs : ts + j - qs, 0), 3);
      return typename Quad<T>::Sel(kq);
    } else {
      return typename Quad<T>::Sel(rev);
    }
  };
  const typename Quad<T>::Sel qsel = make_sel();
  // four values to steps ts .. ts + 3 of a row (voff: the row's byte offset, or kDrop)
  auto store_quad = [&](__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                        const float (&v)[4]) {
    if (!ANYL || nv == 4 || voff == kDrop) {  // kDrop + st4 is past the resource too
      Quad<T>::store(r, voff + st4, soff, v);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        buf_store_at(r, j < nv ? voff + st4 + uint32_t(j) * sizeof(T) : kDrop, soff,
                     out_elem<T>(v[j]));
    }
  };
  auto load_rows = [&](int d0, float (&xv)[4][4], float (&hv)[4][3]) {
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const int rb = min(d0 + wave * 16 + 4 * G, D - 1);
      const uint32_t rel = uint32_t(min(d0 + wave * 16 + 4 * G + sr, D - 1) - rb) * row_bytes;
      const uint32_t so = uint32_t(rb) * row_bytes;
      Quad<T>::load(x_r, rel + xo4, so, qsel, xv[G]);
#pragma unroll
      for (int sh = 1; sh < 4; ++sh) {
        const int s = max(t0 - sh, 0);
        hv[G][sh - 1] = buf_load_at<T>(x_r, rel + uint32_t(rev ? L - 1 - s : s) * sizeof(T), so);
      }
    }
    if (t0 == 0) {
#pragma unroll
      for (int G = 0; G < 4; ++G)
#pragma unroll
        for (int sh = 0; sh < 3; ++sh) hv[G][sh] = 0.0f;
    }
  };
  load_rows(0, xA, hA);

  auto chunk = [&](int d0, const float (&xc)[4][4], const float (&hc)[4][3],
                   float (&xn)[4][4], float (&hn)[4][3]) {
    // ---- 1. this chunk's weight image to LDS (its rows were loaded a chunk ahead) --------
    __syncthreads();  // the previous chunk's products have read sW
    {
      typedef __attribute__((address_space(3))) void lds_void;
      const char* img = static_cast<const char*>(a.wprep) +
                        (int64_t(k) * a.nchunks + d0 / kDC) * img_bytes;
      for (int j = wave; j < img_bytes / 1024; j += 4)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(img + j * 1024 + lane * 16),
                                         (lds_void*)(reinterpret_cast<char*>(sW) + j * 1024),
                                         16, 0, 0);
      __builtin_amdgcn_s_waitcnt(0);  // the image and this chunk's rows have arrived
    }
    __syncthreads();
    if (d0 + kDC < D) load_rows(d0 + kDC, xn, hn);  // before this chunk's stores

    // ---- 2. conv + SiLU, four outputs per lane and group ---------------------------------
#pragma unroll
    for (int G = 0; G < 4; ++G) {
      const int c = wave * 16 + 4 * G + sr, d = d0 + c;
      const float4 w = *reinterpret_cast<const float4*>(&sCW[c][0]);  // taps by shift 0..3
      const float bias = sCW[c][8];
      const float* x = xc[G];
      // the values 1, 2 and 3 steps before this lane's first step
      const float p1 = __int_as_float(__builtin_amdgcn_update_dpp(
          __float_as_int(hc[G][0]), __float_as_int(x[3]), kRowShr1, 0xf, 0xf, false));
      const float p2 = __int_as_float(__builtin_amdgcn_update_dpp(
          __float_as_int(hc[G][1]), __float_as_int(x[2]), kRowShr1, 0xf, 0xf, false));
      const float p3 = __int_as_float(__builtin_amdgcn_update_dpp(
          __float_as_int(hc[G][2]), __float_as_int(x[1]), kRowShr1, 0xf, 0xf, false));
      const float cv[4] = {
          fmaf(w.w, p3, fmaf(w.z, p2, fmaf(w.y, p1, fmaf(w.x, x[0], bias)))),
          fmaf(w.w, p2, fmaf(w.z, p1, fmaf(w.y, x[0], fmaf(w.x, x[1], bias)))),
          fmaf(w.w, p1, fmaf(w.z, x[0], fmaf(w.y, x[1], fmaf(w.x, x[2], bias)))),
          fmaf(w.w, x[0], fmaf(w.z, x[1], fmaf(w.y, x[2], fmaf(w.x, x[3], bias))))};
      float u[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) u[j] = silu_f32(cv[j]);
      if (d0 + kDC > D) {  // a ragged last chunk: channels past D enter x_proj as zeros
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] = d < D ? u[j] : 0.0f;
      }
      const int rb = min(d0 + wave * 16 + 4 * G, D - 1);
      store_quad(u_r, (d < D && ok4) ? uint32_t(sr) * row_bytes : kDrop,
                 uint32_t(rb) * row_bytes, u);
      Ops::put_col4(sU, kTT, 4 * q4, c, u);
    }
    __syncthreads();

    // ---- 3. x_proj on the matrix cores: wave w owns steps 16 w .. 16 w + 15 --------------
    const int urow = wave * 16 + n16;  // this lane's step in the u operand
    const E* wrow = sW + n16 * Ops::kRowE + CJ * g;
#pragma unroll 1
    for (int kk = 0; kk < kDC / KS; ++kk) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[mt] = Ops::product(wrow + mt * 16 * Ops::kRowE + kk * KS, MP,
                               Ops::u_at(sU, urow, kk * KS + CJ * g), kTT, acc[mt]);
      }
    }
  };
  for (int d0 = 0; d0 < D; d0 += 2 * kDC) {
    chunk(d0, xA, hA, xB, hB);
    if (d0 + kDC < D) chunk(d0 + kDC, xB, hB, xA, hA);
  }
  __syncthreads();  // the last products have read sU and sW

  // dt_proj's weights of this route (D x R fp32) go memory -> LDS behind the x_proj outputs
  // when they fit there (no registers held, one wave instruction per 64 floats); otherwise
  // they are read from memory in the loop below.
  const int DR = D * R;
  float* sWdt = &sXd[0][0] + MP * kTT;
  const bool w_lds = a.dt_lr == nullptr &&
                     DR <= (int(Ops::elems(kTT) * sizeof(E)) + img_bytes) / 4 - MP * kTT;
  const float* wdt = a.dt_lr ? nullptr : a.dt_proj_w + int64_t(k) * D * R;
  if (w_lds) {
    typedef __attribute__((address_space(3))) void lds_void;
    for (int e0 = wave * kWave; e0 < DR; e0 += 4 * kWave)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(wdt + min(e0 + lane, DR - 1)),
                                       (lds_void*)(sWdt + e0), 4, 0, 0);
  }

  // ---- 4. x_proj outputs to LDS: lane holds rows 4 (l / 16) + j of column l % 16 -------
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) sXd[mt * 16 + 4 * g + j][wave * 16 + n16] = acc[mt][j];
  }
  if (w_lds) __builtin_amdgcn_s_waitcnt(0);  // this wave's weight copies have landed
  __syncthreads();

  // ---- 5. dt_proj: wave w covers channels 16 w .. 16 w + 15 of each chunk of 64, four
  //         per lane group; then the B and C rows, four rows per wave instruction --------
  if (a.dt_lr) {  // dt_proj folded into the scan: store x_proj's dt rows instead
    const __amdgpu_buffer_rsrc_t lr_r =
        make_rsrc(static_cast<T*>(a.dt_lr) + bk * R * L, uint32_t(R) * row_bytes);
    for (int rg = wave; 4 * rg < R; rg += 4) {
      const int row = 4 * rg + sr;
      const float4 x4 = *reinterpret_cast<const float4*>(&sXd[min(row, R - 1)][4 * q4]);
      const float v[4] = {x4.x, x4.y, x4.z, x4.w};
      store_quad(lr_r, (row < R && ok4) ? uint32_t(row) * row_bytes : kDrop, 0, v);
    }
  }
  const __amdgpu_buffer_rsrc_t dt_r =
      make_rsrc(a.dt_lr ? nullptr : static_cast<T*>(a.dt_raw) + bk * D * L,
                a.dt_lr ? 0u : uint32_t(D) * row_bytes);
  // the weights from LDS or from memory: one copy of the loop for each (w_lds is the same
  // for the whole block), so every load has a known address space
  auto dt_proj = [&](auto wsrc) {
#pragma unroll 1
    for (int dc = wave * 16; dc < D; dc += kDC) {
      float dv[4][4];
#pragma unroll
      for (int G = 0; G < 4; ++G)
#pragma unroll
        for (int j = 0; j < 4; ++j) dv[G][j] = 0.0f;
      for (int r = 0; r < R; ++r) {
        const float4 x4 = *reinterpret_cast<const float4*>(&sXd[r][4 * q4]);
#pragma unroll
        for (int G = 0; G < 4; ++G) {
          const int d = dc + 4 * G + sr;
          const float w = wsrc[min(d, D - 1) * R + r];
          dv[G][0] = fmaf(w, x4.x, dv[G][0]);
          dv[G][1] = fmaf(w, x4.y, dv[G][1]);
          dv[G][2] = fmaf(w, x4.z, dv[G][2]);
          dv[G][3] = fmaf(w, x4.w, dv[G][3]);
        }
      }
#pragma unroll
      for (int G = 0; G < 4; ++G) {
        const int d = dc + 4 * G + sr;
        store_quad(dt_r, (d < D && ok4) ? uint32_t(d) * row_bytes : kDrop, 0, dv[G]);
      }
    }
  };
  if (w_lds) {
    typedef const __attribute__((address_space(3))) float lds_float;
    dt_proj((lds_float*)sWdt);
  } else if (a.dt_lr == nullptr) {
    dt_proj(wdt);
  }
  const __amdgpu_buffer_rsrc_t b_r =
      make_rsrc(static_cast<T*>(a.Bs) + bk * N * L, uint32_t(N) * row_bytes);
  const __amdgpu_buffer_rsrc_t c_r =
      make_rsrc(static_cast<T*>(a.Cs) + bk * N * L, uint32_t(N) * row_bytes);
  for (int rg = wave; 4 * rg < 2 * N; rg += 4) {
    const int row = 4 * rg + sr;  // 0 .. 2N - 1: B rows, then C rows
    const float4 x4 = *reinterpret_cast<const float4*>(&sXd[R + min(row, 2 * N - 1)][4 * q4]);
    const float v[4] = {x4.x, x4.y, x4.z, x4.w};
    if (4 * rg < N)
      store_quad(b_r, (row < N && ok4) ? uint32_t(row) * row_bytes : kDrop, 0, v);
    if (4 * rg + 3 >= N)
      store_quad(c_r, (row >= N && row < 2 * N && ok4) ? uint32_t(row - N) * row_bytes : kDrop,
                 0, v);
  }
}

}  // namespace

size_t project_prep_bytes(int K, int D, int N, int R, int dtype) {
  const int MP = 16 * ((R + 2 * N + 15) / 16);
  const int img = dtype == 0 ? proj_img_bytes<float>(MP) : proj_img_bytes<uint16_t>(MP);
  return size_t(K) * size_t((D + kDC - 1) / kDC) * size_t(img);
}

int launch_project(const ProjArgs& a0, int dtype, hipStream_t st) {
  if (a0.B <= 0 || a0.D <= 0 || a0.L <= 0) return 0;
  ProjArgs a = a0;
  const int MP = 16 * ((a.R + 2 * a.N + 15) / 16);
  a.nchunks = (a.D + kDC - 1) / kDC;
  a.img_bytes = dtype == 0 ? proj_img_bytes<float>(MP) : proj_img_bytes<uint16_t>(MP);
  const dim3 pgrid(a.nchunks, a.K);
  if (dtype == 0)
    k_project_prep<float><<<pgrid, 256, 0, st>>>(a);
  else
    k_project_prep<uint16_t><<<pgrid, 256, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return static_cast<int>(e);
  const dim3 grid((a.L + kTT - 1) / kTT, a.K, a.B);
  const bool kw4 = a.KW == 4;
  if (kw4 && a.L >= 4) {
    const size_t lds = dtype == 0 ? proj_lds_bytes<float>(MP) : proj_lds_bytes<uint16_t>(MP);
    const bool anyl = a.L % 4 != 0;
    auto launch4 = [&](auto mt_tag) {
      constexpr int MTC = decltype(mt_tag)::value;
      if (dtype == 0) {
        if (anyl) k_project4<float, MTC, true><<<grid, 256, lds, st>>>(a);
        else k_project4<float, MTC, false><<<grid, 256, lds, st>>>(a);
      } else {
        if (anyl) k_project4<uint16_t, MTC, true><<<grid, 256, lds, st>>>(a);
        else k_project4<uint16_t, MTC, false><<<grid, 256, lds, st>>>(a);
      }
    };
    switch (MP / 16) {
      case 1: launch4(std::integral_constant<int, 1>{}); break;
      case 2: launch4(std::integral_constant<int, 2>{}); break;
      case 3: launch4(std::integral_constant<int, 3>{}); break;
      case 4: launch4(std::integral_constant<int, 4>{}); break;
      case 5: launch4(std::integral_constant<int, 5>{}); break;
      default: launch4(std::integral_constant<int, kMT>{}); break;
    }
  } else if (dtype == 0) {
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
