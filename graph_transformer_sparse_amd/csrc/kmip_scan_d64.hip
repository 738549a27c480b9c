// Score-scan kernels for rows of 64 bf16 elements.
#include "kmip_scan_kernels.h"

namespace kmip {
hipError_t launch_scan_d64(int kp, const ScanArgs& a, hipStream_t s) {
  return launch_scan_d<64>(kp, a, s);
}
}  // namespace kmip
