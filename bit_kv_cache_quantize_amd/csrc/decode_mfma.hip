// Split-K decode attention: placeholder routing to the reference kernel until the
// MFMA kernel lands.
#include "kvq_device.h"

namespace kvq {
hipError_t launch_decode_split(const DecodeArgs& a, const Geometry& g, hipStream_t stream) {
  return launch_decode_split_reference(a, g, stream);
}
}  // namespace kvq
