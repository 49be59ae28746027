// bfloat16 instantiations of the selective-scan kernel, delta * B discretisation, dt_proj folded into the scan.
#include "ss2d_scan.inc"

namespace ss2d {
int launch_scan_bf16_lr(const ScanArgs& a, int split, int mode, hipStream_t st) {
  return launch_scan_t<uint16_t, false, true>(a, split, mode, st);
}
}  // namespace ss2d
