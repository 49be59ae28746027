// fp32 instantiations of the selective-scan kernel, zero-order-hold discretisation of B.
#include "ss2d_scan.inc"

namespace ss2d {
int launch_scan_f32_zoh(const ScanArgs& a, int split, int mode, hipStream_t st) {
  return launch_scan_t<float, true, false>(a, split, mode, st);
}
}  // namespace ss2d
