// Chunkwise KDA prefill (placeholder until the MFMA kernel lands).
#include "internal.h"
#include "kda_device.h"

namespace kda {

hipError_t launch_prefill(const kda_prefill_desc &, const PrefillPlan &, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace kda
