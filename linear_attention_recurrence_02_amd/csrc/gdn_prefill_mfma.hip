// Matrix-core (MFMA) prompt-form kernel for bf16 inputs: not yet enabled; the
// ABI routes every prefill call to the vector-ALU kernel until it is.
#include "gdn_internal.hpp"

namespace gdn {

bool prefill_mfma_supports(const PrefillArgs &) { return false; }

hipError_t launch_prefill_mfma(const PrefillArgs &, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace gdn
