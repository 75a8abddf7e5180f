// decode_mfma.hip - matrix-core decode kernel (not built yet).
#include "common.hpp"
#include "kernels.hpp"

namespace pkv {

bool decode_mfma_supported(int, int, int, int) { return false; }

hipError_t launch_decode_mfma(int, int, const DecodeParams&, hipStream_t) {
    return hipErrorInvalidValue;
}

}  // namespace pkv
