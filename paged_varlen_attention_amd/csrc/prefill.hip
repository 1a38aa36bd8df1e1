// prefill.hip -- tiled bf16-MFMA paged attention for prefill / mixed batches.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

bool prefill_supported(int, int, int) { return false; }

hipError_t launch_prefill(const AttnParams &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pa
