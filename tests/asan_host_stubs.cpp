// asan_host_stubs.cpp -- TEST INFRASTRUCTURE. Stand-ins for the kernel launchers of the HIP
// library, so that its host code (the C ABI's argument checks in pa_api.cpp, the shape logic in
// pa_shapes.cpp and the block manager) can be built with g++ and the address and undefined-behaviour
// sanitizers into a CPU-only library. Every stand-in reports that no device is present: a call
// whose checks all pass ends with PA_ERR_HIP, and nothing is computed on the CPU.
#include "pa_internal.h"

namespace pa {

hipError_t launch_reshape_and_cache(const CacheDims &, const void *, const void *, void *, void *,
                                    const int32_t *, int32_t, hipStream_t)
{
    return hipErrorNoDevice;
}

hipError_t launch_reshape_and_cache_fp8(const CacheDims &, const void *, const void *, void *,
                                        void *, const int32_t *, int32_t, float, float,
                                        hipStream_t)
{
    return hipErrorNoDevice;
}

hipError_t launch_copy_blocks(const CacheDims &, void *, void *, const int32_t *, int32_t,
                              hipStream_t)
{
    return hipErrorNoDevice;
}

hipError_t launch_decode(const DecodeLaunch &, hipStream_t) { return hipErrorNoDevice; }

hipError_t launch_decode_multi(const DecodeLaunch &, hipStream_t) { return hipErrorNoDevice; }

hipError_t decode_scratch(hipStream_t, void **) { return hipErrorNoDevice; }

hipError_t launch_prefill(const PrefillLaunch &, hipStream_t) { return hipErrorNoDevice; }

}  // namespace pa
