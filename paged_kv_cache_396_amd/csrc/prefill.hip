// Chunked-prefill attention over paged KV (bf16 MFMA).  Not built yet: the
// entry point reports PA_ERR_UNSUPPORTED until the kernel lands.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

bool prefill_supported(int, int, int) { return false; }

hipError_t launch_prefill(const PrefillArgs&, const CacheGeom&, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace pa
