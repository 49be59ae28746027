// bfloat16 instantiations of the backward scan kernel for the zero-order hold.
#include "ss2d_bwd.inc"

namespace ss2d {
int launch_scan_bwd_bf16_zoh(const BwdArgs& a, hipStream_t st) {
  return a.g_f32 ? launch_scan_bwd_t<uint16_t, float, true>(a, st)
                 : launch_scan_bwd_t<uint16_t, uint16_t, true>(a, st);
}
}  // namespace ss2d
