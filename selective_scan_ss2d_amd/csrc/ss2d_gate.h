// The gate applied to, and differentiated at, a route sum that a forward call kept (the
// training path: ss2d_forward_save / ss2d_backward_saved).  Elementwise over n positions of
// (B, D, L) image-layout tensors; the arithmetic is the merge kernels' own (the same device
// functions, in the same order), so that the results equal the fused merge's bit for bit.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ss2d {

// y = v SiLU(z), rounded once to the data type (dtype 0: fp32, 1: bf16; z and y of that
// type, v fp32).
int launch_gate_fwd(const float* v, const void* z, void* y, int64_t n, int dtype,
                    hipStream_t st);
// g = dy SiLU(z) in fp32 and dz = dy v SiLU'(z) in the data type.
int launch_gate_bwd(const float* v, const void* z, const void* dy, float* g, void* dz,
                    int64_t n, int dtype, hipStream_t st);

}  // namespace ss2d
