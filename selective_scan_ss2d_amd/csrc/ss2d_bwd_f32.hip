// fp32 instantiations of the backward scan kernel.
#include "ss2d_bwd.inc"

namespace ss2d {
int launch_scan_bwd_f32(const BwdArgs& a, hipStream_t st) { return launch_scan_bwd_t<float, float>(a, st); }
}  // namespace ss2d
