// Stand-ins for the device-side launchers, for the host-only build of the C ABI layer
// (psa_api.cpp) that runs under the address and undefined-behaviour sanitizers on a machine
// without a GPU. Every launcher reports that no device code is present, so a call that
// passes validation returns PSA_ERR_HIP; nothing here touches a device.
#include "psa_launch.h"

namespace psa {
hipError_t launch_pyramid(const PyramidArgs&, hipStream_t) { return hipErrorNoBinaryForGpu; }
hipError_t launch_attention_bwd(const BwdArgs&, hipStream_t) { return hipErrorNoBinaryForGpu; }
hipError_t launch_similarity_cap(const CapArgs&, hipStream_t) { return hipErrorNoBinaryForGpu; }
hipError_t launch_mask(const MaskArgs&, hipStream_t) { return hipErrorNoBinaryForGpu; }
hipError_t launch_attention(const AttnArgs&, hipStream_t) { return hipErrorNoBinaryForGpu; }
hipError_t noalloc_scratch(void**) { return hipErrorNoBinaryForGpu; }
}  // namespace psa
