// MFMA tree-verify kernel for bf16 q/k/v at d_k = d_v = 128 (in progress).
#include "device_common.hpp"
#include "internal.hpp"

namespace gdn {

bool verify_mfma_supports(const VerifyArgs &) { return false; }

hipError_t launch_verify_mfma(const VerifyArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace gdn
