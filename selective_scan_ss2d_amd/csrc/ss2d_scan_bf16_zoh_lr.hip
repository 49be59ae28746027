// bfloat16 instantiations of the selective-scan kernel, zero-order-hold discretisation of B, dt_proj folded into the scan.
#include "ss2d_scan.inc"

namespace ss2d {
int launch_scan_bf16_zoh_lr(const ScanArgs& a, int split, int mode, hipStream_t st) {
  return launch_scan_t<uint16_t, true, true>(a, split, mode, st);
}
}  // namespace ss2d
