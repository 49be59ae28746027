// Support kernels of the SS2D forward operator (gfx950): the per-plane transpose that turns
// the column routes into contiguous walks, and the cross-merge that undoes each route's
// permutation and sums the routes in a fixed order.
#include <type_traits>

#include "ss2d_device.h"
#include "ss2d_gate.h"

namespace ss2d {
namespace {

// What the merge does with the route sum v at a position (GM, a template parameter):
constexpr int kGateNone = 0;  // y = v
constexpr int kGateFwd = 1;   // y = v SiLU(z)
constexpr int kGateBwd = 2;   // gated backward: y = dy SiLU(z) in fp32, dz = dy v SiLU'(z)

// Element type of the merge's output y: the data type, or fp32 for the gated backward's g
// (the gradient every route receives is kept in fp32 for the adjoint scan).
template <typename T, int GM> using MergeOut = std::conditional_t<GM == kGateBwd, float, T>;

// The gate's backward at one position, for out = v SiLU(z): g = dy SiLU(z) is the gradient
// that reaches every route's output, and dz = dy v SiLU'(z), with
// SiLU'(z) = sigma(z) (1 + z (1 - sigma(z))).
__device__ __forceinline__ void gate_bwd(float v, float z, float dy, float& g, float& dz) {
  const float sg = __builtin_amdgcn_rcpf(1.0f + exp2_hw(-z * kLog2e));
  g = dy * (z * sg);
  dz = dy * v * (sg * fmaf(z, 1.0f - sg, 1.0f));
}

constexpr int kTr = 32;        // transpose / merge tile edge
constexpr int kTrRows = 8;     // thread rows per tile (block = 32 x 8)
constexpr int kMaxGridZ = 65535;

// xt[p, w, h] = x[p, h, w] for every plane p of (H, W).
template <typename T>
__global__ void __launch_bounds__(kTr * kTrRows)
k_transpose(const T* __restrict__ x, T* __restrict__ xt, int H, int W, int64_t planes) {
  __shared__ T tile[kTr][kTr + 1];
  const int tx = threadIdx.x, ty = threadIdx.y;
  const int w0 = blockIdx.x * kTr, h0 = blockIdx.y * kTr;
  const int64_t plane_elems = static_cast<int64_t>(H) * W;
  for (int64_t p = blockIdx.z; p < planes; p += gridDim.z) {
    const T* src = x + p * plane_elems;
    T* dst = xt + p * plane_elems;
#pragma unroll
    for (int r = ty; r < kTr; r += kTrRows) {
      const int h = h0 + r, w = w0 + tx;
      if (h < H && w < W) tile[r][tx] = src[static_cast<int64_t>(h) * W + w];
    }
    __syncthreads();
#pragma unroll
    for (int r = ty; r < kTr; r += kTrRows) {
      const int w = w0 + r, h = h0 + tx;
      if (w < W && h < H) dst[static_cast<int64_t>(w) * H + h] = tile[tx][r];
    }
    __syncthreads();
  }
}

// Vectorized transpose for planes whose sides are multiples of 8 (bf16) or 4 (fp32): each
// thread moves one 8x8 (bf16) or 4x4 (fp32) block with 16-byte loads and stores, the
// transposition done in registers.  Consecutive threads take consecutive blocks of a block
// row, so each wave reads whole plane rows and writes whole transposed rows.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

// Moves one 8x8 bf16 block (8 rows of 16 bytes in, 8 columns of 16 bytes out).
__device__ __forceinline__ void load_block8(const uint16_t* src, int W, uint4 (&row)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) row[j] = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(j) * W);
}
__device__ __forceinline__ void store_block8(uint16_t* dst, int H, const uint4 (&row)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t in[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint4 v = row[j];
      in[j] = (c / 2 == 0) ? v.x : (c / 2 == 1) ? v.y : (c / 2 == 2) ? v.z : v.w;
    }
    uint4 o;
    if (c % 2 == 0)
      o = make_uint4(pack_lo(in[0], in[1]), pack_lo(in[2], in[3]), pack_lo(in[4], in[5]),
                     pack_lo(in[6], in[7]));
    else
      o = make_uint4(pack_hi(in[0], in[1]), pack_hi(in[2], in[3]), pack_hi(in[4], in[5]),
                     pack_hi(in[6], in[7]));
    *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(c) * H) = o;
  }
}

// Each thread handles two 8x8 blocks per iteration (both loaded before either is stored).
__global__ void __launch_bounds__(256)
k_transpose_bf16_8x8(const uint16_t* __restrict__ x, uint16_t* __restrict__ xt, int H, int W,
                     int64_t blocks_total) {
  const int hb_n = H / 8, wb_n = W / 8;
  const int64_t per_plane = static_cast<int64_t>(hb_n) * wb_n;
  const int64_t plane_elems = static_cast<int64_t>(H) * W;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  auto src_of = [&](int64_t i) {
    const int64_t p = i / per_plane;
    const int r = static_cast<int>(i % per_plane);
    return x + p * plane_elems + static_cast<int64_t>(r / wb_n * 8) * W + (r % wb_n) * 8;
  };
  auto dst_of = [&](int64_t i) {
    const int64_t p = i / per_plane;
    const int r = static_cast<int>(i % per_plane);
    return xt + p * plane_elems + static_cast<int64_t>(r % wb_n * 8) * H + (r / wb_n) * 8;
  };
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < blocks_total;
       i += 2 * stride) {
    const int64_t i2 = i + stride;
    uint4 a[8], b[8];
    load_block8(src_of(i), W, a);
    if (i2 < blocks_total) load_block8(src_of(i2), W, b);
    store_block8(dst_of(i), H, a);
    if (i2 < blocks_total) store_block8(dst_of(i2), H, b);
  }
}

// Whole-plane bf16 transpose through LDS for planes of up to kPlaneLds elements (sides
// multiples of 8): the plane's rows come in with 16-byte loads and the transposed rows go out
// with 16-byte stores, both contiguous across the threads of a wave.  LDS rows are padded by
// two elements so that the column reads spread over the banks.
constexpr int kPlaneLds = 8192;

__global__ void __launch_bounds__(256)
k_transpose_plane_bf16(const uint16_t* __restrict__ x, uint16_t* __restrict__ xt, int H, int W,
                       int64_t planes) {
  __shared__ uint32_t buf[kPlaneLds / 2];
  uint16_t* tile = reinterpret_cast<uint16_t*>(buf);
  const int rs = W + 2;                       // LDS row stride (elements, even)
  const int chunks = H * W / 8;               // 16-byte chunks per plane
  const int row_chunks = W / 8, col_chunks = H / 8;
  const int64_t plane_elems = static_cast<int64_t>(H) * W;
  for (int64_t p = blockIdx.x; p < planes; p += gridDim.x) {
    const uint16_t* src = x + p * plane_elems;
    uint16_t* dst = xt + p * plane_elems;
#pragma unroll 2
    for (int i = threadIdx.x; i < chunks; i += blockDim.x) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + 8 * i);
      uint32_t* d = reinterpret_cast<uint32_t*>(tile + (i / row_chunks) * rs + (i % row_chunks) * 8);
      d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
    __syncthreads();
#pragma unroll 2
    for (int o = threadIdx.x; o < chunks; o += blockDim.x) {
      const uint16_t* s = tile + (o % col_chunks) * 8 * rs + o / col_chunks;  // column w, rows h0..h0+7
      uint32_t q[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        q[j] = uint32_t(s[2 * j * rs]) | (uint32_t(s[(2 * j + 1) * rs]) << 16);
      *reinterpret_cast<uint4*>(dst + 8 * o) = make_uint4(q[0], q[1], q[2], q[3]);
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(256)
k_transpose_f32_4x4(const float* __restrict__ x, float* __restrict__ xt, int H, int W,
                    int64_t blocks_total) {
  const int hb_n = H / 4, wb_n = W / 4;
  const int64_t per_plane = static_cast<int64_t>(hb_n) * wb_n;
  const int64_t plane_elems = static_cast<int64_t>(H) * W;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < blocks_total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t p = i / per_plane;
    const int r = static_cast<int>(i % per_plane);
    const int hb = r / wb_n, wb = r % wb_n;
    const float* src = x + p * plane_elems + static_cast<int64_t>(hb * 4) * W + wb * 4;
    float* dst = xt + p * plane_elems + static_cast<int64_t>(wb * 4) * H + hb * 4;
    const float4 r0 = *reinterpret_cast<const float4*>(src);
    const float4 r1 = *reinterpret_cast<const float4*>(src + W);
    const float4 r2 = *reinterpret_cast<const float4*>(src + 2 * W);
    const float4 r3 = *reinterpret_cast<const float4*>(src + 3 * W);
    *reinterpret_cast<float4*>(dst) = make_float4(r0.x, r1.x, r2.x, r3.x);
    *reinterpret_cast<float4*>(dst + H) = make_float4(r0.y, r1.y, r2.y, r3.y);
    *reinterpret_cast<float4*>(dst + 2 * H) = make_float4(r0.z, r1.z, r2.z, r3.z);
    *reinterpret_cast<float4*>(dst + 3 * H) = make_float4(r0.w, r1.w, r2.w, r3.w);
  }
}

// Four-route merge.  For image position (h, w), l = h * W + w and s = w * H + h (its step
// on the column-major route):
//   v[l] = ((y0[l] + y1[L-1-l]) + y2[s]) + y3[L-1-s]
// with y_k the per-route outputs in scan order, and y = v, v SiLU(z) or the gate's backward
// (GM).  Column-route values go through an LDS tile so that every global access is a
// contiguous run.  The gate is shared by the routes, so gating the sum once equals summing
// the gated route outputs.
template <typename T, int GM>
__global__ void __launch_bounds__(kTr * kTrRows)
k_merge4(const float* __restrict__ yr, const T* __restrict__ z, const T* __restrict__ dy,
         MergeOut<T, GM>* __restrict__ y, T* __restrict__ dz, int D, int H, int W,
         int64_t planes) {
  __shared__ float t2[kTr][kTr + 1];
  __shared__ float t3[kTr][kTr + 1];
  const int tx = threadIdx.x, ty = threadIdx.y;
  const int w0 = blockIdx.x * kTr, h0 = blockIdx.y * kTr;
  const int64_t L = static_cast<int64_t>(H) * W;
  for (int64_t p = blockIdx.z; p < planes; p += gridDim.z) {
    const int64_t b = p / D, d = p % D;
    const float* y0 = yr + ((b * 4 + 0) * D + d) * L;
    const float* y1 = yr + ((b * 4 + 1) * D + d) * L;
    const float* y2 = yr + ((b * 4 + 2) * D + d) * L;
    const float* y3 = yr + ((b * 4 + 3) * D + d) * L;
#pragma unroll
    for (int r = ty; r < kTr; r += kTrRows) {
      const int w = w0 + r, h = h0 + tx;
      if (w < W && h < H) {
        const int64_t s = static_cast<int64_t>(w) * H + h;
        t2[r][tx] = y2[s];
        t3[r][tx] = y3[L - 1 - s];
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = ty; r < kTr; r += kTrRows) {
      const int h = h0 + r, w = w0 + tx;
      if (h < H && w < W) {
        const int64_t l = static_cast<int64_t>(h) * W + w;
        float v = y0[l] + y1[L - 1 - l];
        v += t2[tx][r];
        v += t3[tx][r];
        if constexpr (GM == kGateBwd) {
          float g, dzv;
          gate_bwd(v, Elem<T>::load(z + p * L + l), Elem<T>::load(dy + p * L + l), g, dzv);
          y[p * L + l] = g;
          dz[p * L + l] = Elem<T>::from_f32(dzv);
        } else {
          if (GM == kGateFwd) v *= silu_f32(Elem<T>::load(z + p * L + l));
          y[p * L + l] = Elem<T>::from_f32(v);
        }
      }
    }
    __syncthreads();
  }
}

// Vectorized four-route merge for maps whose sides are multiples of 4 (fp32 route outputs
// are then 16-byte aligned in every plane).  A block covers a 32 x 32 tile of one plane:
// the column-route values (contiguous along h) are staged in LDS with float4 loads, the
// row-route values are read as float4 runs along w (reversed for route 1), and each thread
// writes 4 consecutive outputs of a row.  Same fixed summation order as k_merge4.
// Four consecutive elements (8- or 16-byte loads), kept raw until used.
template <typename T> struct In4;
template <> struct In4<float> {
  float4 r;
  __device__ __forceinline__ void load(const float* p) { r = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ float4 get() const { return r; }
};
template <> struct In4<uint16_t> {
  uint2 r;
  __device__ __forceinline__ void load(const uint16_t* p) { r = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ float4 get() const {
    return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                       __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
  }
};

template <typename T> struct Out4;
template <> struct Out4<float> {
  static __device__ __forceinline__ void store(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
};
template <> struct Out4<uint16_t> {
  static __device__ __forceinline__ void store(uint16_t* p, float a, float b, float c, float d) {
    const uint32_t lo = Elem<uint16_t>::from_f32(a) | (uint32_t(Elem<uint16_t>::from_f32(b)) << 16);
    const uint32_t hi = Elem<uint16_t>::from_f32(c) | (uint32_t(Elem<uint16_t>::from_f32(d)) << 16);
    *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
  }
};

// The per-route outputs are read exactly once, by the merge: nontemporal loads keep them
// from displacing other data in the caches (measured ~17% faster merge than plain loads on
// the VMamba-T stage-1 shape).
typedef float v4f_stream __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load4_stream(const float* p) {
  const v4f_stream v = __builtin_nontemporal_load(reinterpret_cast<const v4f_stream*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
// The same for a 4-byte aligned address (served at any alignment in the chip's unaligned
// access mode).
typedef float v4f_stream_any __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ float4 load4_stream_any(const float* p) {
  const v4f_stream_any v =
      __builtin_nontemporal_load(reinterpret_cast<const v4f_stream_any*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// Buffer resources over one plane (L elements): 32-bit per-lane offsets instead of 64-bit
// addresses keep the kernel's registers low; loads use the nontemporal policy (the route
// outputs are read exactly once).
constexpr uint32_t kMergeRsrc = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kNt = 2;                       // cache policy: nontemporal
__device__ __forceinline__ __amdgpu_buffer_rsrc_t plane_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, kMergeRsrc);
}
__device__ __forceinline__ float4 rsrc_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNt);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                     __uint_as_float(v.w));
}
// four gate values (the data type) at element offset e of a plane
template <typename T> struct Gate4;
template <> struct Gate4<float> {
  float4 r;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t e) {
    r = rsrc_load4(rs, e * 4);
  }
  __device__ __forceinline__ float4 get() const { return r; }
};
template <> struct Gate4<uint16_t> {
  uint2 r;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t e) {
    typedef unsigned int v2u __attribute__((ext_vector_type(2)));
    const v2u v = __builtin_amdgcn_raw_buffer_load_b64(rs, e * 2, 0, kNt);
    r = make_uint2(v.x, v.y);
  }
  __device__ __forceinline__ float4 get() const {
    return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                       __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
  }
};

template <typename T, int GM>
__global__ void __launch_bounds__(256)
k_merge4_vec(const float* __restrict__ yr, const T* __restrict__ z, const T* __restrict__ dy,
             MergeOut<T, GM>* __restrict__ y, T* __restrict__ dz, int D, int H, int W,
             int64_t planes) {
  constexpr bool GATE = GM != kGateNone;
  // A block covers a 64 x 64 tile (h x w) of one plane; every thread keeps four 16-byte
  // loads of each route (and, with the gate, its four gate loads) in flight before the
  // barrier.
  constexpr int TS = 64;
  __shared__ float t2[TS][TS + 1];
  __shared__ float t3[TS][TS + 1];
  const int tid = threadIdx.x;
  const int w0 = blockIdx.x * TS, h0 = blockIdx.y * TS;
  const int64_t L = static_cast<int64_t>(H) * W;
  const uint32_t pbytes = static_cast<uint32_t>(L * 4);  // L < 2^30
  const int lh = 4 * (tid % 16), lw = tid / 16;     // load phase: (w0 + lw + 16 j, h0 + lh)
  const int ow = 4 * (tid % 16), oh = tid / 16;     // output phase: (h0 + oh + 16 j, w0 + ow)
  for (int64_t p = blockIdx.z; p < planes; p += gridDim.z) {
    const int64_t b = p / D, d = p % D;
    const __amdgpu_buffer_rsrc_t y0 = plane_rsrc(yr + ((b * 4 + 0) * D + d) * L, pbytes);
    const __amdgpu_buffer_rsrc_t y1 = plane_rsrc(yr + ((b * 4 + 1) * D + d) * L, pbytes);
    const __amdgpu_buffer_rsrc_t y2 = plane_rsrc(yr + ((b * 4 + 2) * D + d) * L, pbytes);
    const __amdgpu_buffer_rsrc_t y3 = plane_rsrc(yr + ((b * 4 + 3) * D + d) * L, pbytes);
    float4 c2[4], c3[4], r0[4], r1[4];
    Gate4<T> g[GATE ? 4 : 1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int w = w0 + lw + 16 * j, h = h0 + lh;
      if (w < W && h < H) {
        const uint32_t st = static_cast<uint32_t>(w * H + h);  // steps st .. st+3
        c2[j] = rsrc_load4(y2, st * 4);
        c3[j] = rsrc_load4(y3, static_cast<uint32_t>(L - 4 - st) * 4);
      }
      const int hh = h0 + oh + 16 * j, ww = w0 + ow;
      if (hh < H && ww < W) {
        const uint32_t l = static_cast<uint32_t>(hh * W + ww);  // positions l .. l+3
        r0[j] = rsrc_load4(y0, l * 4);
        r1[j] = rsrc_load4(y1, static_cast<uint32_t>(L - 4 - l) * 4);
        if constexpr (GATE) g[j].load(plane_rsrc(z + p * L, pbytes / 4 * sizeof(T)), l);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int w = w0 + lw + 16 * j, h = h0 + lh;
      if (w < W && h < H) {
        float* a = &t2[lw + 16 * j][lh];
        a[0] = c2[j].x; a[1] = c2[j].y; a[2] = c2[j].z; a[3] = c2[j].w;
        float* c = &t3[lw + 16 * j][lh];
        c[0] = c3[j].w; c[1] = c3[j].z; c[2] = c3[j].y; c[3] = c3[j].x;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int hh = h0 + oh + 16 * j, ww = w0 + ow;
      if (hh < H && ww < W) {
        const int64_t l = static_cast<int64_t>(hh) * W + ww;
        const int ht = oh + 16 * j;
        float v0 = r0[j].x + r1[j].w, v1 = r0[j].y + r1[j].z;
        float v2 = r0[j].z + r1[j].y, v3 = r0[j].w + r1[j].x;
        v0 += t2[ow + 0][ht]; v1 += t2[ow + 1][ht]; v2 += t2[ow + 2][ht]; v3 += t2[ow + 3][ht];
        v0 += t3[ow + 0][ht]; v1 += t3[ow + 1][ht]; v2 += t3[ow + 2][ht]; v3 += t3[ow + 3][ht];
        if constexpr (GM == kGateBwd) {
          // dy is read here, after the barrier, to keep the registers of the loads in flight
          // before it at the gated forward's count
          Gate4<T> gd;
          gd.load(plane_rsrc(dy + p * L, pbytes / 4 * sizeof(T)), static_cast<uint32_t>(l));
          const float4 gz = g[j].get(), gy = gd.get();
          float g0, g1, g2, g3, z0, z1, z2, z3;
          gate_bwd(v0, gz.x, gy.x, g0, z0);
          gate_bwd(v1, gz.y, gy.y, g1, z1);
          gate_bwd(v2, gz.z, gy.z, g2, z2);
          gate_bwd(v3, gz.w, gy.w, g3, z3);
          Out4<float>::store(y + p * L + l, g0, g1, g2, g3);
          Out4<T>::store(dz + p * L + l, z0, z1, z2, z3);
        } else {
          if constexpr (GM == kGateFwd) {
            const float4 gz = g[j].get();
            v0 *= silu_f32(gz.x); v1 *= silu_f32(gz.y); v2 *= silu_f32(gz.z);
            v3 *= silu_f32(gz.w);
          }
          Out4<T>::store(y + p * L + l, v0, v1, v2, v3);
        }
      }
    }
    __syncthreads();
  }
}

// Two-route merge (forward + reversed 1D sequence): v[l] = y0[l] + y1[L-1-l], and y = v,
// v SiLU(z[l]) or the gate's backward (GM).
template <typename T, int GM>
__global__ void __launch_bounds__(256)
k_merge2(const float* __restrict__ yr, const T* __restrict__ z, const T* __restrict__ dy,
         MergeOut<T, GM>* __restrict__ y, T* __restrict__ dz, int D, int L, int64_t planes) {
  const int l = blockIdx.x * blockDim.x + threadIdx.x;
  if (l >= L) return;
  for (int64_t p = blockIdx.y; p < planes; p += gridDim.y) {
    const int64_t b = p / D, d = p % D;
    const float* y0 = yr + ((b * 2 + 0) * D + d) * L;
    const float* y1 = yr + ((b * 2 + 1) * D + d) * L;
    float v = y0[l] + y1[L - 1 - l];
    if constexpr (GM == kGateBwd) {
      float g, dzv;
      gate_bwd(v, Elem<T>::load(z + p * L + l), Elem<T>::load(dy + p * L + l), g, dzv);
      y[p * L + l] = g;
      dz[p * L + l] = Elem<T>::from_f32(dzv);
    } else {
      if (GM == kGateFwd) v *= silu_f32(Elem<T>::load(z + p * L + l));
      y[p * L + l] = Elem<T>::from_f32(v);
    }
  }
}

// Vectorized two-route merge over whole images: with D * L a multiple of 4, the outputs of
// image b form one contiguous run of D * L elements, as do the route-0 outputs (the routes
// are the outer dimension of the per-route buffer).  Each thread takes 4 consecutive
// elements e .. e+3 of the run: route 0 with one 16-byte load, route 1 (reversed within each
// plane of length L) with four 4-byte loads that may straddle a plane boundary.
template <typename T, int GM>
__global__ void __launch_bounds__(256)
k_merge2_vec(const float* __restrict__ yr, const T* __restrict__ z, const T* __restrict__ dy,
             MergeOut<T, GM>* __restrict__ y, T* __restrict__ dz, int D, int L,
             int64_t images) {
  const int64_t run = static_cast<int64_t>(D) * L;
  const int64_t e = 4 * (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x);
  if (e >= run) return;
  // route 1's values of positions e .. e + 3 (reversed within each row): one 16-byte load
  // of any alignment, reversed, when the four lie in one row; else one by one
  const int64_t d0 = e / L;
  const int l0 = static_cast<int>(e - d0 * L);
  const bool one_row = l0 + 3 < L;
  int64_t src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool wrap = l0 + i >= L;
    const int64_t d = wrap ? d0 + 1 : d0;
    const int l = wrap ? l0 + i - L : l0 + i;
    src[i] = d * L + (L - 1 - l);
  }
  for (int64_t b = blockIdx.y; b < images; b += gridDim.y) {
    const float* y0 = yr + b * 2 * run;
    const float* y1 = y0 + run;
    const float4 a = load4_stream(y0 + e);
    float r[4];
    if (one_row) {
      const float4 v = load4_stream_any(y1 + src[3]);
      r[0] = v.w; r[1] = v.z; r[2] = v.y; r[3] = v.x;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = __builtin_nontemporal_load(y1 + src[i]);
    }
    float v0 = a.x + r[0], v1 = a.y + r[1], v2 = a.z + r[2], v3 = a.w + r[3];
    if constexpr (GM == kGateBwd) {
      In4<T> g, gd;
      g.load(z + b * run + e);
      gd.load(dy + b * run + e);
      const float4 gz = g.get(), gy = gd.get();
      float g0, g1, g2, g3, z0, z1, z2, z3;
      gate_bwd(v0, gz.x, gy.x, g0, z0);
      gate_bwd(v1, gz.y, gy.y, g1, z1);
      gate_bwd(v2, gz.z, gy.z, g2, z2);
      gate_bwd(v3, gz.w, gy.w, g3, z3);
      Out4<float>::store(y + b * run + e, g0, g1, g2, g3);
      Out4<T>::store(dz + b * run + e, z0, z1, z2, z3);
    } else {
      if constexpr (GM == kGateFwd) {
        In4<T> g;
        g.load(z + b * run + e);
        const float4 gz = g.get();
        v0 *= silu_f32(gz.x); v1 *= silu_f32(gz.y); v2 *= silu_f32(gz.z); v3 *= silu_f32(gz.w);
      }
      Out4<T>::store(y + b * run + e, v0, v1, v2, v3);
    }
  }
}

// dBs[b, k, n, t] and dCs[b, k, n, t]: sums of the backward kernel's per-channel-block
// partials (B, K, n_cb, 2N, L), over the channel blocks in order, rounded once.
template <typename T>
__global__ void __launch_bounds__(256)
k_bwd_reduce_bc(const float* __restrict__ part, T* __restrict__ dBs, T* __restrict__ dCs,
                int N, int L, int n_cb, int64_t total) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;                      // i = ((bk * 2N) + n2) * L + t
  const int t = static_cast<int>(i % L);
  const int64_t q = i / L;
  const int n2 = static_cast<int>(q % (2 * N));
  const int64_t bk = q / (2 * N);
  const float* p = part + (bk * n_cb * 2 * N + n2) * static_cast<int64_t>(L) + t;
  float v = 0.0f;
  for (int c = 0; c < n_cb; ++c) v += p[static_cast<int64_t>(c) * 2 * N * L];
  T* dst = n2 < N ? dBs : dCs;
  dst[(bk * N + (n2 % N)) * static_cast<int64_t>(L) + t] = Elem<T>::from_f32(v);
}

// The same, four consecutive steps per thread (L a multiple of 4, 16-byte aligned partials
// and 8- (bf16) or 16-byte (fp32) aligned outputs): 16-byte partial loads, the channel
// blocks added in the same order.
template <typename T>
__global__ void __launch_bounds__(256)
k_bwd_reduce_bc4(const float* __restrict__ part, T* __restrict__ dBs, T* __restrict__ dCs,
                 int N, int L, int n_cb, int64_t total4) {
  const int64_t i4 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i4 >= total4) return;
  const int64_t i = 4 * i4;                    // i = ((bk * 2N) + n2) * L + t, t % 4 == 0
  const int64_t q = i / L;
  const int t = static_cast<int>(i - q * L);
  const int n2 = static_cast<int>(q % (2 * N));
  const int64_t bk = q / (2 * N);
  const float* p = part + (bk * n_cb * 2 * N + n2) * static_cast<int64_t>(L) + t;
  float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int c = 0; c < n_cb; ++c) {
    const float4 w = *reinterpret_cast<const float4*>(p + static_cast<int64_t>(c) * 2 * N * L);
    v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
  }
  T* dst = n2 < N ? dBs : dCs;
  Out4<T>::store(dst + (bk * N + (n2 % N)) * static_cast<int64_t>(L) + t, v.x, v.y, v.z, v.w);
}

// dA_log, dDs, ddt_bias: sums over images, in image order, of the per-image partials,
// accumulated in fp64 and rounded once (these sums cancel: over a large batch, an fp32
// running sum would add an error of up to B roundings of the partials' size).
__global__ void __launch_bounds__(256)
k_bwd_reduce_params(const float* __restrict__ dA_part, const float* __restrict__ dD_part,
                    const float* __restrict__ dbias_part, float* __restrict__ dA_log,
                    float* __restrict__ dDs, float* __restrict__ ddt_bias, int B, int KD, int N) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t nA = static_cast<int64_t>(KD) * N;
  if (i >= nA + 2 * KD) return;
  const float* src;
  int64_t stride;
  float* dst;
  if (i < nA) {
    src = dA_part + i; stride = nA; dst = dA_log + i;
  } else if (i < nA + KD) {
    src = dD_part + (i - nA); stride = KD; dst = dDs + (i - nA);
  } else {
    src = dbias_part + (i - nA - KD); stride = KD; dst = ddt_bias + (i - nA - KD);
  }
  // images in order; the loads of 32 images are issued together (a loop of dependent
  // load-then-add steps waits for every load in turn)
  double v = 0.0;
  int b = 0;
  for (; b + 32 <= B; b += 32) {
    float x[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) x[j] = src[static_cast<int64_t>(b + j) * stride];
#pragma unroll
    for (int j = 0; j < 32; ++j) v += static_cast<double>(x[j]);
  }
  for (; b < B; ++b) v += static_cast<double>(src[static_cast<int64_t>(b) * stride]);
  *dst = static_cast<float>(v);
}

// Rows of `len` elements in blocks of rows_in rows to blocks of rows_out rows (outer blocks in
// order): row r of a block is copied when r < rows_in, zero-filled otherwise.  With
// rows_out < rows_in the first rows_out rows of each block are kept.
template <typename E>
__global__ void __launch_bounds__(256)
k_copy_rows(const E* __restrict__ src, E* __restrict__ dst, int64_t outer, int rows_in,
            int rows_out, int64_t len) {
  const int64_t total = outer * rows_out * len;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t t = i % len;
    const int64_t r = (i / len) % rows_out;
    const int64_t o = i / (len * rows_out);
    dst[i] = r < rows_in ? src[(o * rows_in + r) * len + t] : E(0);
  }
}

}  // namespace

int launch_bwd_reduce_bc(const float* part, void* dBs, void* dCs, int B, int K, int N, int L,
                         int n_cb, int dtype, hipStream_t st) {
  const int64_t total = static_cast<int64_t>(B) * K * 2 * N * L;
  const uintptr_t oa = dtype == 0 ? 16 : 8;
  if (L % 4 == 0 && reinterpret_cast<uintptr_t>(part) % 16 == 0 &&
      reinterpret_cast<uintptr_t>(dBs) % oa == 0 && reinterpret_cast<uintptr_t>(dCs) % oa == 0) {
    const int64_t total4 = total / 4;
    const unsigned b4 = static_cast<unsigned>((total4 + 255) / 256);
    if (dtype == 0)
      hipLaunchKernelGGL(k_bwd_reduce_bc4<float>, dim3(b4), dim3(256), 0, st, part,
                         static_cast<float*>(dBs), static_cast<float*>(dCs), N, L, n_cb, total4);
    else
      hipLaunchKernelGGL(k_bwd_reduce_bc4<uint16_t>, dim3(b4), dim3(256), 0, st, part,
                         static_cast<uint16_t*>(dBs), static_cast<uint16_t*>(dCs), N, L, n_cb,
                         total4);
    return static_cast<int>(hipGetLastError());
  }
  const unsigned blocks = static_cast<unsigned>((total + 255) / 256);
  if (dtype == 0)
    hipLaunchKernelGGL(k_bwd_reduce_bc<float>, dim3(blocks), dim3(256), 0, st, part,
                       static_cast<float*>(dBs), static_cast<float*>(dCs), N, L, n_cb, total);
  else
    hipLaunchKernelGGL(k_bwd_reduce_bc<uint16_t>, dim3(blocks), dim3(256), 0, st, part,
                       static_cast<uint16_t*>(dBs), static_cast<uint16_t*>(dCs), N, L, n_cb,
                       total);
  return static_cast<int>(hipGetLastError());
}

int launch_copy_rows(const void* src, void* dst, int64_t outer, int rows_in, int rows_out,
                     int64_t len, int elem_bytes, hipStream_t st) {
  const int64_t total = outer * rows_out * len;
  if (total <= 0) return 0;
  const int64_t want = (total + 255) / 256;
  const unsigned blocks = static_cast<unsigned>(want < 65536 ? want : 65536);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(k_copy_rows<uint16_t>, dim3(blocks), dim3(256), 0, st,
                       static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), outer,
                       rows_in, rows_out, len);
  else
    hipLaunchKernelGGL(k_copy_rows<float>, dim3(blocks), dim3(256), 0, st,
                       static_cast<const float*>(src), static_cast<float*>(dst), outer, rows_in,
                       rows_out, len);
  return static_cast<int>(hipGetLastError());
}

int launch_bwd_reduce_params(const float* dA_part, const float* dD_part,
                             const float* dbias_part, float* dA_log, float* dDs,
                             float* ddt_bias, int B, int K, int D, int N, hipStream_t st) {
  const int KD = K * D;
  const int64_t total = static_cast<int64_t>(KD) * N + 2 * KD;
  hipLaunchKernelGGL(k_bwd_reduce_params, dim3(static_cast<unsigned>((total + 255) / 256)),
                     dim3(256), 0, st, dA_part, dD_part, dbias_part, dA_log, dDs, ddt_bias, B,
                     KD, N);
  return static_cast<int>(hipGetLastError());
}

int launch_transpose(const void* x, void* xt, int B, int D, int H, int W, int dtype,
                     hipStream_t st) {
  const int64_t planes = static_cast<int64_t>(B) * D;
  dim3 grid((W + kTr - 1) / kTr, (H + kTr - 1) / kTr,
            static_cast<unsigned>(planes < kMaxGridZ ? planes : kMaxGridZ));
  dim3 block(kTr, kTrRows);
  const bool aligned = (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(xt) % 16 == 0);
  const int v = dtype == 0 ? 4 : 8;
  if (aligned && dtype == 1 && H % 8 == 0 && W % 8 == 0 && H * (W + 2) <= kPlaneLds) {
    const int64_t nb = planes < (1 << 20) ? planes : (1 << 20);
    hipLaunchKernelGGL(k_transpose_plane_bf16, dim3(static_cast<unsigned>(nb)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(x), static_cast<uint16_t*>(xt), H, W, planes);
    return static_cast<int>(hipGetLastError());
  }
  if (aligned && H % v == 0 && W % v == 0) {
    const int64_t blocks_total = planes * (H / v) * (W / v);
    int64_t nb = (blocks_total + 511) / 512;  // two blocks per thread per iteration
    if (nb > 2048) nb = 2048;                 // grid-stride beyond 8 blocks per CU
    if (dtype == 0)
      hipLaunchKernelGGL(k_transpose_f32_4x4, dim3(static_cast<unsigned>(nb)), dim3(256), 0, st,
                         static_cast<const float*>(x), static_cast<float*>(xt), H, W,
                         blocks_total);
    else
      hipLaunchKernelGGL(k_transpose_bf16_8x8, dim3(static_cast<unsigned>(nb)), dim3(256), 0,
                         st, static_cast<const uint16_t*>(x), static_cast<uint16_t*>(xt), H, W,
                         blocks_total);
    return static_cast<int>(hipGetLastError());
  }
  if (dtype == 0)
    hipLaunchKernelGGL(k_transpose<float>, grid, block, 0, st, static_cast<const float*>(x),
                       static_cast<float*>(xt), H, W, planes);
  else
    hipLaunchKernelGGL(k_transpose<uint16_t>, grid, block, 0, st,
                       static_cast<const uint16_t*>(x), static_cast<uint16_t*>(xt), H, W,
                       planes);
  return static_cast<int>(hipGetLastError());
}

namespace {

// Launches one merge kernel instantiation for the element type and gate mode of the call.
template <template <typename, int> class Launch, typename... Args>
int merge_dispatch(int dtype, int gm, const void* z, const void* dy, void* dz, Args... args) {
  auto run = [&](auto tag) {
    using T = decltype(tag);
    const T* zt = static_cast<const T*>(z);
    const T* dyt = static_cast<const T*>(dy);
    T* dzt = static_cast<T*>(dz);
    if (gm == kGateBwd) return Launch<T, kGateBwd>::run(zt, dyt, dzt, args...);
    if (gm == kGateFwd) return Launch<T, kGateFwd>::run(zt, dyt, dzt, args...);
    return Launch<T, kGateNone>::run(zt, dyt, dzt, args...);
  };
  return dtype == 0 ? run(float{}) : run(uint16_t{});
}

template <typename T, int GM>
struct Merge4Vec {
  static int run(const T* z, const T* dy, T* dz, dim3 g, hipStream_t st, const float* yr,
                 void* y, int D, int H, int W, int64_t planes) {
    hipLaunchKernelGGL((k_merge4_vec<T, GM>), g, dim3(256), 0, st, yr, z, dy,
                       static_cast<MergeOut<T, GM>*>(y), dz, D, H, W, planes);
    return static_cast<int>(hipGetLastError());
  }
};
template <typename T, int GM>
struct Merge4 {
  static int run(const T* z, const T* dy, T* dz, dim3 g, hipStream_t st, const float* yr,
                 void* y, int D, int H, int W, int64_t planes) {
    hipLaunchKernelGGL((k_merge4<T, GM>), g, dim3(kTr, kTrRows), 0, st, yr, z, dy,
                       static_cast<MergeOut<T, GM>*>(y), dz, D, H, W, planes);
    return static_cast<int>(hipGetLastError());
  }
};
template <typename T, int GM>
struct Merge2Vec {
  static int run(const T* z, const T* dy, T* dz, dim3 g, hipStream_t st, const float* yr,
                 void* y, int D, int L, int64_t images) {
    hipLaunchKernelGGL((k_merge2_vec<T, GM>), g, dim3(256), 0, st, yr, z, dy,
                       static_cast<MergeOut<T, GM>*>(y), dz, D, L, images);
    return static_cast<int>(hipGetLastError());
  }
};
template <typename T, int GM>
struct Merge2 {
  static int run(const T* z, const T* dy, T* dz, dim3 g, hipStream_t st, const float* yr,
                 void* y, int D, int L, int64_t planes) {
    hipLaunchKernelGGL((k_merge2<T, GM>), g, dim3(256), 0, st, yr, z, dy,
                       static_cast<MergeOut<T, GM>*>(y), dz, D, L, planes);
    return static_cast<int>(hipGetLastError());
  }
};

bool aligned_to(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

int merge4(const float* y_route, int gm, const void* z, const void* dy, void* y, void* dz,
           int B, int D, int H, int W, int dtype, hipStream_t st) {
  const int64_t planes = static_cast<int64_t>(B) * D;
  const unsigned gz = static_cast<unsigned>(planes < kMaxGridZ ? planes : kMaxGridZ);
  const uintptr_t out_align = dtype == 0 ? 16 : 8;
  const bool aligned = aligned_to(y_route, 16) &&
                       aligned_to(y, gm == kGateBwd ? 16 : out_align) &&
                       aligned_to(z, out_align) && aligned_to(dy, out_align) &&
                       aligned_to(dz, out_align);
  if (aligned && H % 4 == 0 && W % 4 == 0)
    return merge_dispatch<Merge4Vec>(dtype, gm, z, dy, dz,
                                     dim3((W + 63) / 64, (H + 63) / 64, gz), st, y_route, y, D,
                                     H, W, planes);
  return merge_dispatch<Merge4>(dtype, gm, z, dy, dz,
                                dim3((W + kTr - 1) / kTr, (H + kTr - 1) / kTr, gz), st, y_route,
                                y, D, H, W, planes);
}

int merge2(const float* y_route, int gm, const void* z, const void* dy, void* y, void* dz,
           int B, int D, int L, int dtype, hipStream_t st) {
  const int64_t planes = static_cast<int64_t>(B) * D;
  const unsigned gy = static_cast<unsigned>(planes < kMaxGridZ ? planes : kMaxGridZ);
  const uintptr_t out_align = dtype == 0 ? 16 : 8;
  const bool aligned = aligned_to(y_route, 16) &&
                       aligned_to(y, gm == kGateBwd ? 16 : out_align) &&
                       aligned_to(z, out_align) && aligned_to(dy, out_align) &&
                       aligned_to(dz, out_align);
  const int64_t run = static_cast<int64_t>(D) * L;
  if (aligned && run % 4 == 0) {
    const unsigned gb = static_cast<unsigned>(B < kMaxGridZ ? B : kMaxGridZ);
    return merge_dispatch<Merge2Vec>(dtype, gm, z, dy, dz,
                                     dim3(static_cast<unsigned>((run / 4 + 255) / 256), gb), st,
                                     y_route, y, D, L, static_cast<int64_t>(B));
  }
  return merge_dispatch<Merge2>(dtype, gm, z, dy, dz, dim3((L + 255) / 256, gy), st, y_route, y,
                                D, L, planes);
}

}  // namespace

int launch_merge4(const float* y_route, const void* z, void* y, int B, int D, int H, int W,
                  int dtype, hipStream_t st) {
  return merge4(y_route, z ? kGateFwd : kGateNone, z, nullptr, y, nullptr, B, D, H, W, dtype,
                st);
}

int launch_merge2(const float* y_route, const void* z, void* y, int B, int D, int L, int dtype,
                  hipStream_t st) {
  return merge2(y_route, z ? kGateFwd : kGateNone, z, nullptr, y, nullptr, B, D, L, dtype, st);
}

int launch_merge4_gate_bwd(const float* y_route, const void* z, const void* dy, void* g,
                           void* dz, int B, int D, int H, int W, int dtype, hipStream_t st) {
  return merge4(y_route, kGateBwd, z, dy, g, dz, B, D, H, W, dtype, st);
}

int launch_merge2_gate_bwd(const float* y_route, const void* z, const void* dy, void* g,
                           void* dz, int B, int D, int L, int dtype, hipStream_t st) {
  return merge2(y_route, kGateBwd, z, dy, g, dz, B, D, L, dtype, st);
}

namespace {

// The gate over a kept route sum, four positions per thread (16-byte accesses when every
// pointer allows them, element by element otherwise and for the last positions).
template <typename T>
__global__ void __launch_bounds__(256)
k_gate_fwd(const float* __restrict__ v, const T* __restrict__ z, T* __restrict__ y, int64_t n,
           bool vec) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x * 4;
  for (int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4; i < n;
       i += stride) {
    if (vec && i + 4 <= n) {
      const float4 vv = *reinterpret_cast<const float4*>(v + i);
      Out4<T>::store(y + i, vv.x * silu_f32(Elem<T>::load(z + i)),
                     vv.y * silu_f32(Elem<T>::load(z + i + 1)),
                     vv.z * silu_f32(Elem<T>::load(z + i + 2)),
                     vv.w * silu_f32(Elem<T>::load(z + i + 3)));
    } else {
      for (int64_t j = i; j < i + 4 && j < n; ++j)
        y[j] = Elem<T>::from_f32(v[j] * silu_f32(Elem<T>::load(z + j)));
    }
  }
}

template <typename T>
__global__ void __launch_bounds__(256)
k_gate_bwd(const float* __restrict__ v, const T* __restrict__ z, const T* __restrict__ dy,
           float* __restrict__ g, T* __restrict__ dz, int64_t n, bool vec) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x * 4;
  for (int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4; i < n;
       i += stride) {
    if (vec && i + 4 <= n) {
      const float4 vv = *reinterpret_cast<const float4*>(v + i);
      const float vs[4] = {vv.x, vv.y, vv.z, vv.w};
      float gs[4], zs[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        gate_bwd(vs[j], Elem<T>::load(z + i + j), Elem<T>::load(dy + i + j), gs[j], zs[j]);
      Out4<float>::store(g + i, gs[0], gs[1], gs[2], gs[3]);
      Out4<T>::store(dz + i, zs[0], zs[1], zs[2], zs[3]);
    } else {
      for (int64_t j = i; j < i + 4 && j < n; ++j) {
        float gj, zj;
        gate_bwd(v[j], Elem<T>::load(z + j), Elem<T>::load(dy + j), gj, zj);
        g[j] = gj;
        dz[j] = Elem<T>::from_f32(zj);
      }
    }
  }
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

unsigned gate_blocks(int64_t n) {
  const int64_t want = (n + 1023) / 1024;  // four positions per thread
  return static_cast<unsigned>(want < 65536 ? (want > 0 ? want : 1) : 65536);
}

}  // namespace

int launch_gate_fwd(const float* v, const void* z, void* y, int64_t n, int dtype,
                    hipStream_t st) {
  if (n <= 0) return 0;
  const bool vec = aligned16(v) && aligned16(z) && aligned16(y);
  if (dtype == 0)
    hipLaunchKernelGGL(k_gate_fwd<float>, dim3(gate_blocks(n)), dim3(256), 0, st, v,
                       static_cast<const float*>(z), static_cast<float*>(y), n, vec);
  else
    hipLaunchKernelGGL(k_gate_fwd<uint16_t>, dim3(gate_blocks(n)), dim3(256), 0, st, v,
                       static_cast<const uint16_t*>(z), static_cast<uint16_t*>(y), n, vec);
  return static_cast<int>(hipGetLastError());
}

int launch_gate_bwd(const float* v, const void* z, const void* dy, float* g, void* dz,
                    int64_t n, int dtype, hipStream_t st) {
  if (n <= 0) return 0;
  const bool vec = aligned16(v) && aligned16(z) && aligned16(dy) && aligned16(g) && aligned16(dz);
  if (dtype == 0)
    hipLaunchKernelGGL(k_gate_bwd<float>, dim3(gate_blocks(n)), dim3(256), 0, st, v,
                       static_cast<const float*>(z), static_cast<const float*>(dy), g,
                       static_cast<float*>(dz), n, vec);
  else
    hipLaunchKernelGGL(k_gate_bwd<uint16_t>, dim3(gate_blocks(n)), dim3(256), 0, st, v,
                       static_cast<const uint16_t*>(z), static_cast<const uint16_t*>(dy), g,
                       static_cast<uint16_t*>(dz), n, vec);
  return static_cast<int>(hipGetLastError());
}

}  // namespace ss2d
