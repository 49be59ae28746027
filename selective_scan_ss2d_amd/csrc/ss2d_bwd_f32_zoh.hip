// fp32 instantiations of the backward scan kernel for the zero-order hold.
#include "ss2d_bwd.inc"

namespace ss2d {
int launch_scan_bwd_f32_zoh(const BwdArgs& a, hipStream_t st) {
  return launch_scan_bwd_t<float, float, true>(a, st);
}
}  // namespace ss2d
