// SSD chunked forward for gfx950 (placeholder until the kernels land).
#include <hip/hip_runtime.h>

#include "ssm_internal.h"

namespace ssm {
hipError_t launch_ssd_chunk_cumsum(const SSDParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_ssd_chunk_state(const SSDParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_ssd_state_passing(const SSDParams&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_ssd_chunk_scan(const SSDParams&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace ssm
