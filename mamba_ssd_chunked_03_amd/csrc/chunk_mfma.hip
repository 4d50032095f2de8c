// chunk_mfma.hip -- bf16 MFMA kernels for stages 1, 2, 4 and 5 (placeholder: no shape
// is instantiated yet, so every shape takes the fp32 VALU kernels).
#include "ssd_internal.h"

namespace ssd {

bool chunk_state_mfma_supported(const Shape&) { return false; }
hipError_t launch_chunk_state_mfma(const Shape&, const void*, const void*, const float*,
                                   const float*, float*, hipStream_t) {
    return hipErrorInvalidValue;
}
bool chunk_scan_mfma_supported(const Shape&) { return false; }
hipError_t launch_chunk_scan_mfma(const Shape&, const void*, const void*, const void*,
                                  const float*, const float*, const float*, const float*, void*,
                                  hipStream_t) {
    return hipErrorInvalidValue;
}

}  // namespace ssd
