// fp32 instantiations of the backward scan kernel, delta * B.
#include "ss2d_bwd.inc"

namespace ss2d {
int launch_scan_bwd_f32(const BwdArgs& a, hipStream_t st) {
  if (a.zoh) return launch_scan_bwd_f32_zoh(a, st);
  return launch_scan_bwd_t<float, float, false>(a, st);
}
}  // namespace ss2d
