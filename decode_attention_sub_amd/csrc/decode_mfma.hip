// MFMA decode path (filled in below); declines every launch until implemented.
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {
hipError_t launch_decode_mfma(const DecodeLaunch& d, hipStream_t st, bool* handled) {
  (void)d; (void)st;
  *handled = false;
  return hipSuccess;
}
}  // namespace kvq
