// MoE expert block (placeholder until the kernels land).
#include "common.h"
#include "launch.h"

namespace qd {

size_t moe_workspace_bytes(const MoeArgs& m, int T, int k) {
    return (size_t)T * ((size_t)k * m.I + m.Is) * sizeof(float);
}

hipError_t launch_moe_experts(const MoeArgs&, const int32_t*, const float*, int, int, const void*,
                              int, float*, void*, size_t, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace qd
