// Support kernels of the SS2D forward operator (gfx950): the per-plane transpose that turns
// the column routes into contiguous walks, the chunk-carry pass of the chunked scan, and the
// cross-merge that undoes each route's permutation and sums the routes in a fixed order.
#include "ss2d_device.h"

namespace ss2d {
namespace {

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

// Start state of every chunk c >= 1 of every (b, k, d) scan, one thread per state n:
//   h_in[c + 1] = exp(A_n * sum of delta over chunk c) * h_in[c] + h_end[c],  h_in[0] = 0,
// where h_end[c] is chunk c's end state from a zero start.  This is the composition of the
// affine maps h -> a h + b of consecutive chunks, applied in order.
__global__ void __launch_bounds__(256) k_carry(const ScanArgs a) {
  const int64_t total = static_cast<int64_t>(a.B) * a.K * a.D * a.N;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int n = static_cast<int>(i % a.N);
  const int64_t row = i / a.N;                 // (b * K + k) * D + d
  const int d = static_cast<int>(row % a.D);
  const int k = static_cast<int>((row / a.D) % a.K);
  const float Ap = -expf(a.A_log[(static_cast<int64_t>(k) * a.D + d) * a.N + n]) * kLog2e;
  const int C = a.num_chunks;
  float h = 0.0f;
  for (int c = 0; c + 1 < C; ++c) {
    const float decay = exp2_hw(Ap * a.delta_sum[row * C + c]);
    h = fmaf(decay, h, a.h_end[(row * C + c) * a.N + n]);
    a.h_in[(row * C + c + 1) * a.N + n] = h;
  }
}

// Four-route merge.  For image position (h, w), l = h * W + w and s = w * H + h (its step
// on the column-major route):
//   y[l] = ((y0[l] + y1[L-1-l]) + y2[s]) + y3[L-1-s]
// with y_k the per-route outputs in scan order.  Column-route values go through an LDS tile
// so that every global access is a contiguous run.
template <typename T>
__global__ void __launch_bounds__(kTr * kTrRows)
k_merge4(const float* __restrict__ yr, T* __restrict__ y, int D, int H, int W, int64_t planes) {
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
        y[p * L + l] = Elem<T>::from_f32(v);
      }
    }
    __syncthreads();
  }
}

// Two-route merge (forward + reversed 1D sequence): y[l] = y0[l] + y1[L-1-l].
template <typename T>
__global__ void __launch_bounds__(256)
k_merge2(const float* __restrict__ yr, T* __restrict__ y, int D, int L, int64_t planes) {
  const int l = blockIdx.x * blockDim.x + threadIdx.x;
  if (l >= L) return;
  for (int64_t p = blockIdx.y; p < planes; p += gridDim.y) {
    const int64_t b = p / D, d = p % D;
    const float* y0 = yr + ((b * 2 + 0) * D + d) * L;
    const float* y1 = yr + ((b * 2 + 1) * D + d) * L;
    y[p * L + l] = Elem<T>::from_f32(y0[l] + y1[L - 1 - l]);
  }
}

}  // namespace

int launch_transpose(const void* x, void* xt, int B, int D, int H, int W, int dtype,
                     hipStream_t st) {
  const int64_t planes = static_cast<int64_t>(B) * D;
  dim3 grid((W + kTr - 1) / kTr, (H + kTr - 1) / kTr,
            static_cast<unsigned>(planes < kMaxGridZ ? planes : kMaxGridZ));
  dim3 block(kTr, kTrRows);
  if (dtype == 0)
    hipLaunchKernelGGL(k_transpose<float>, grid, block, 0, st, static_cast<const float*>(x),
                       static_cast<float*>(xt), H, W, planes);
  else
    hipLaunchKernelGGL(k_transpose<uint16_t>, grid, block, 0, st,
                       static_cast<const uint16_t*>(x), static_cast<uint16_t*>(xt), H, W,
                       planes);
  return static_cast<int>(hipGetLastError());
}

int launch_carry(const ScanArgs& a, hipStream_t st) {
  const int64_t total = static_cast<int64_t>(a.B) * a.K * a.D * a.N;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(k_carry, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a);
  return static_cast<int>(hipGetLastError());
}

int launch_merge4(const float* y_route, void* y, int B, int D, int H, int W, int dtype,
                  hipStream_t st) {
  const int64_t planes = static_cast<int64_t>(B) * D;
  dim3 grid((W + kTr - 1) / kTr, (H + kTr - 1) / kTr,
            static_cast<unsigned>(planes < kMaxGridZ ? planes : kMaxGridZ));
  dim3 block(kTr, kTrRows);
  if (dtype == 0)
    hipLaunchKernelGGL(k_merge4<float>, grid, block, 0, st, y_route, static_cast<float*>(y), D,
                       H, W, planes);
  else
    hipLaunchKernelGGL(k_merge4<uint16_t>, grid, block, 0, st, y_route,
                       static_cast<uint16_t*>(y), D, H, W, planes);
  return static_cast<int>(hipGetLastError());
}

int launch_merge2(const float* y_route, void* y, int B, int D, int L, int dtype,
                  hipStream_t st) {
  const int64_t planes = static_cast<int64_t>(B) * D;
  dim3 grid((L + 255) / 256, static_cast<unsigned>(planes < kMaxGridZ ? planes : kMaxGridZ));
  if (dtype == 0)
    hipLaunchKernelGGL(k_merge2<float>, grid, dim3(256), 0, st, y_route, static_cast<float*>(y),
                       D, L, planes);
  else
    hipLaunchKernelGGL(k_merge2<uint16_t>, grid, dim3(256), 0, st, y_route,
                       static_cast<uint16_t*>(y), D, L, planes);
  return static_cast<int>(hipGetLastError());
}

}  // namespace ss2d
