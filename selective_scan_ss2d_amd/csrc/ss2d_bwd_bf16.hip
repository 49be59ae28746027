// bfloat16 instantiations of the backward scan kernel.
#include "ss2d_bwd.inc"

namespace ss2d {
int launch_scan_bwd_bf16(const BwdArgs& a, hipStream_t st) { return launch_scan_bwd_t<uint16_t>(a, st); }
}  // namespace ss2d
