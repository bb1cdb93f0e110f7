// Prefill chunk GEMM (placeholder until the MFMA kernels land).
#include "common.h"
#include "launch.h"

namespace qd {

hipError_t launch_chunk_gemm(int, const uint32_t*, const uint16_t*, const uint16_t*,
                             const uint16_t*, float*, int, int, int, hipStream_t) {
    return hipErrorNotSupported;
}

size_t moe_prefill_workspace_bytes(const MoeArgs& m, int T, int k) {
    (void)T;
    return moe_decode_workspace_bytes(m, k);
}

hipError_t launch_moe_prefill(const MoeArgs& m, const int32_t* idx, const float* w, int T, int k,
                              const void* x, int xkind, float* y, void* ws, hipStream_t st) {
    return launch_moe_decode(m, idx, w, T, k, x, xkind, y, ws, st);
}

}  // namespace qd
