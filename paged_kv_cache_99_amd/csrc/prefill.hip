// prefill.hip -- paged causal attention of prefill chunks (MFMA). Not yet implemented.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

bool prefill_supported(int32_t, int32_t) { return false; }

hipError_t launch_prefill(const PrefillLaunch &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pa
