// Prefill chunk GEMM (placeholder until the kernel lands).
#include "common.h"
#include "launch.h"

namespace qd {

hipError_t launch_chunk_gemm(int, const uint32_t*, const uint16_t*, const uint16_t*,
                             const uint16_t*, float*, int, int, int, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace qd
