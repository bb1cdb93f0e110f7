// Host-only stand-ins for everything the C ABI (api.cpp) calls below its
// argument checks: the HIP runtime queries and the kernel launchers. Used
// to build api.cpp with AddressSanitizer and UndefinedBehaviorSanitizer on a
// machine without a GPU; the launchers only count calls and launch nothing.
#include <hip/hip_runtime.h>

#include <cstring>

#include "../../affine_quantized_gemv_qgemv_amd/csrc/launch.h"

int g_launches = 0;

extern "C" {
hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t a, int) {
    *v = a == hipDeviceAttributeMultiprocessorCount ? 256 : 160 * 1024;
    return hipSuccess;
}
hipError_t hipFuncSetAttribute(const void*, hipFuncAttribute, int) { return hipSuccess; }
hipError_t hipFuncGetAttributes(hipFuncAttributes* a, const void*) {
    std::memset(a, 0, sizeof *a);
    return hipSuccess;
}
hipError_t hipOccupancyMaxActiveBlocksPerMultiprocessor(int* n, const void*, int, size_t) {
    *n = 2;
    return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stub error"; }
}

namespace qd {
hipError_t launch_gemv(int, int, const uint32_t*, const uint16_t*, const uint16_t*, const uint32_t*,
                       const void*, int, float*, int, int, int, hipStream_t, const GemvRot*) {
    ++g_launches;
    return hipSuccess;
}
G8Split gemm8_split(int, int K, int) { return {K >= 4096 ? 4 : 1, K / 64}; }
hipError_t launch_gemm8_tokens_split(const uint32_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                                     int, float*, int, int, int, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_route_topk_slices(const float*, int, int, int, int, float*, int32_t*, float*,
                                    hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_route_topk(const float*, int, int, int, int32_t*, float*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
size_t moe_workspace_bytes(const MoeArgs& m, int T, int k) {
    return ((size_t)T * k * m.I + (size_t)T * m.Is) * 8 + 4096;
}
size_t moe_decode_workspace_bytes(const MoeArgs& m, int k) { return ((size_t)k * m.I + m.Is) * 4; }
hipError_t launch_moe_decode_routed(const MoeArgs&, const float*, int, const void*, int, int32_t*,
                                    float*, float*, void*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_moe_decode_routed_noalloc(const MoeArgs&, const float*, int, const void*, int,
                                            int32_t*, float*, float*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_moe_experts(const MoeArgs&, const int32_t*, const float*, int, int, const void*,
                              int, float*, void*, size_t, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
size_t attn_workspace_bytes(int Hq, int, int D, int) { return (size_t)256 * Hq * (D + 2) * 4; }
hipError_t launch_attn_decode(const uint16_t*, const uint16_t*, const uint16_t*, uint16_t*, uint16_t*,
                              int, int, int, int, int, int, float, float*, void*, size_t, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
// K split of shapes with fewer than 128 column x row tiles (N < 8192 at one row tile)
size_t chunk_split_workspace_bytes(int M, int N, int K) {
    const int mt = M <= 32 ? 32 : M <= 64 ? 64 : 128;
    const int tiles = ((N + 63) / 64) * ((M + mt - 1) / mt);
    return tiles < 128 && K >= 2048 ? (size_t)2 * M * N * 4 : 0;
}
hipError_t launch_chunk_gemm(int, const uint32_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                             int, float*, int, int, int, void*, size_t, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
size_t verify_i8_workspace_bytes(int M, int K) { return (size_t)((M + 15) / 16 * 16) * K * 2 + 4096; }
hipError_t launch_verify_i8(const uint32_t*, const uint16_t*, const uint16_t*, const uint16_t*, float*,
                            int, int, int, void*, size_t, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_stream_read(const void*, int64_t, uint32_t*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
}  // namespace qd
