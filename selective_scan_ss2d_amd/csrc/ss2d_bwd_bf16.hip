// bfloat16 instantiations of the backward scan kernel (route gradient g in bfloat16, or in
// fp32 for the gated operator), delta * B.
#include "ss2d_bwd.inc"

namespace ss2d {
int launch_scan_bwd_bf16(const BwdArgs& a, hipStream_t st) {
  if (a.zoh) return launch_scan_bwd_bf16_zoh(a, st);
  return a.g_f32 ? launch_scan_bwd_t<uint16_t, float, false>(a, st)
                 : launch_scan_bwd_t<uint16_t, uint16_t, false>(a, st);
}
}  // namespace ss2d
