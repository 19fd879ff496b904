// prefill_mfma.hip - matrix-core prefill kernel (placeholder until the banded kernel lands).
#include "swa_device.hpp"
#include "swa_kernels.hpp"

namespace swa {

bool prefill_mfma_supported(const PrefillArgs &) { return false; }

hipError_t launch_prefill_mfma(const PrefillArgs &, const void *, const void *, const void *,
                               void *, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace swa
