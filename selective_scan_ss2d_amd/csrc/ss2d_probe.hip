// Issue-rate probes (measurement support, not part of the operator): the rates that bound the
// scan kernel, measured on the chip instead of taken from its data sheet.  The scan's state
// update issues 2 multiplies, 2 fused multiply-adds and one v_exp_f32 per state and step, so
// three probes run at full occupancy:
//   kind 0: fp32 fused multiply-adds only,
//   kind 1: v_exp_f32 only,
//   kind 2: groups of 4 fused multiply-adds and 1 v_exp_f32 (the update's mix; a multiply
//           issues like a fused multiply-add).
// Each lane runs 8 independent chains, so that no instruction waits for its predecessor's
// result while another wave of its SIMD has work; the chains' values are summed and stored
// at the end so that none of the work can be dropped.  The first lane of each block also
// records the shader clock counter (s_memtime, core cycles) and the 100 MHz reference
// counter (s_memrealtime) at its start and end, from which the host derives the clock the
// chip sustained during the run.
#include "ss2d_device.h"

namespace ss2d {
namespace {

constexpr int kProbeBlock = 256;
constexpr int kProbeRounds = 8;  // unrolled rounds per loop iteration

template <int KIND>
__global__ void __launch_bounds__(kProbeBlock)
k_probe_issue(float* __restrict__ sink, unsigned long long* __restrict__ clocks, float m,
              float c, int iters) {
  unsigned long long t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  float f[8], e[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = m * static_cast<float>(threadIdx.x + i);
#pragma unroll
  for (int i = 0; i < 4; ++i) e[i] = m * static_cast<float>(i + 1);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < kProbeRounds; ++r) {
      if constexpr (KIND == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = fmaf(f[i], m, c);
      } else if constexpr (KIND == 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = exp2_hw(f[i]);
      } else {
        e[r % 4] = exp2_hw(e[r % 4]);
#pragma unroll
        for (int j = 0; j < 4; ++j) f[(4 * r + j) % 8] = fmaf(f[(4 * r + j) % 8], m, c);
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += f[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) s += e[i];
  sink[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    clocks[4 * blockIdx.x + 0] = t0;
    clocks[4 * blockIdx.x + 1] = t1;
    clocks[4 * blockIdx.x + 2] = r0;
    clocks[4 * blockIdx.x + 3] = r1;
  }
}

}  // namespace

// Instructions per lane and loop iteration of each probe kind: (fused multiply-adds, exps).
void probe_counts(int kind, int* fmas, int* exps) {
  *fmas = kind == 0 ? 8 * kProbeRounds : kind == 1 ? 0 : 4 * kProbeRounds;
  *exps = kind == 0 ? 0 : kind == 1 ? 8 * kProbeRounds : kProbeRounds;
}

int probe_block() { return kProbeBlock; }

int launch_probe(int kind, int blocks, int iters, float* sink, unsigned long long* clocks,
                 hipStream_t st) {
  // m and c keep the chains' values from being known at compile time; their magnitude does
  // not matter (an exponential chain runs to +inf, which costs the same)
  const float m = 0.999f, c = 1.0e-3f;
  switch (kind) {
    case 0:
      hipLaunchKernelGGL((k_probe_issue<0>), dim3(blocks), dim3(kProbeBlock), 0, st, sink,
                         clocks, m, c, iters);
      break;
    case 1:
      hipLaunchKernelGGL((k_probe_issue<1>), dim3(blocks), dim3(kProbeBlock), 0, st, sink,
                         clocks, m, c, iters);
      break;
    default:
      hipLaunchKernelGGL((k_probe_issue<2>), dim3(blocks), dim3(kProbeBlock), 0, st, sink,
                         clocks, m, c, iters);
      break;
  }
  return static_cast<int>(hipGetLastError());
}

}  // namespace ss2d
