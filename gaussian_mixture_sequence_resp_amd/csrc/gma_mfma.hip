// MFMA family of the GMA forward (bf16 inputs, fused matrix-core kernels).
#include "gma_internal.h"

namespace gma {

bool mfma_supported(const gma_desc& d, int causal) {
    (void)d;
    (void)causal;
    return false;
}

size_t mfma_workspace(const gma_desc& d, int causal) {
    (void)d;
    (void)causal;
    return 0;
}

hipError_t mfma_forward(const Args& a) {
    (void)a;
    return hipErrorNotSupported;
}

}  // namespace gma
