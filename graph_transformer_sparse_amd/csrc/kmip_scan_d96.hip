// Score-scan kernels for split-precision rows: 96 bf16 elements standing for
// 32 fp32 elements (three bf16 terms per product).
#include "kmip_scan_kernels.h"

namespace kmip {
hipError_t launch_scan_d96(int kp, const ScanArgs& a, hipStream_t s) {
  return launch_scan_d<96>(kp, a, s);
}
}  // namespace kmip
