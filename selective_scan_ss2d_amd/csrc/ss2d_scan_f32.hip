// fp32 instantiations of the selective-scan kernel, delta * B discretisation.
#include "ss2d_scan.inc"

namespace ss2d {
int launch_scan_f32(const ScanArgs& a, int split, int mode, hipStream_t st) {
  return launch_scan_t<float, false, false>(a, split, mode, st);
}
}  // namespace ss2d
