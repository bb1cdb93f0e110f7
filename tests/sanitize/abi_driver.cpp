// Drives every C entry point of libqdecode (include/qdecode.h) through its
// argument checks, for a host build of api.cpp with AddressSanitizer and
// UndefinedBehaviorSanitizer (kernel launchers and HIP runtime replaced by
// abi_stubs.cpp): invalid arguments must return the documented status with a
// message and launch nothing; valid ones must reach the launcher once.
#include <cstdio>
#include <cstring>

#include "../../include/qdecode.h"

extern int g_launches;

alignas(256) static unsigned char mem[4096];
static void* const A = mem;            // an aligned stand-in for device memory (never read)
static void* const MIS = mem + 4;      // misaligned

static int fails = 0;
#define EXPECT(call, want)                                                                    \
    do {                                                                                      \
        const int before = g_launches;                                                        \
        const qd_status got = (call);                                                         \
        const bool launched = g_launches != before;                                           \
        if (got != (want) || launched != ((want) == QD_OK) ||                                 \
            ((want) != QD_OK && std::strlen(qd_last_error()) == 0)) {                         \
            std::fprintf(stderr, "line %d: %s -> %s (want %s), launched %d, msg '%s'\n",       \
                         __LINE__, #call, qd_status_string(got), qd_status_string(want),      \
                         (int)launched, qd_last_error());                                     \
            ++fails;                                                                          \
        }                                                                                     \
    } while (0)

#define U32 (const uint32_t*)
#define U16 (const uint16_t*)

static qd_moe_weights moe(int E = 128, int H = 2816, int I = 704, int Is = 2112, int g = 64,
                          int act = QD_GELU_ERF) {
    qd_moe_weights w;
    w.E = E; w.H = H; w.I = I; w.I_shared = Is; w.group_size = g; w.act = (qd_act)act;
    w.gu_q = w.dn_q = w.sgu_q = w.sdn_q = U32 A;
    w.gu_s = w.gu_b = w.dn_s = w.dn_b = w.sgu_s = w.sgu_b = w.sdn_s = w.sdn_b = U16 A;
    return w;
}

int main() {
    float* y = (float*)A;
    // dense GEMV
    EXPECT(qgemv_affine4(U32 A, U16 A, U16 A, U16 A, QD_F16, y, 16, 128, 1, 64, nullptr), QD_OK);
    EXPECT(qgemv_affine4(U32 A, U16 A, U16 A, U16 A, QD_F16, y, 16, 128, 9, 64, nullptr), QD_ERR_INVALID_ARGUMENT);
    EXPECT(qgemv_affine8(U32 A, U16 A, U16 A, U16 A, QD_BF16, y, 16, 128, 128, 64, nullptr), QD_OK);
    EXPECT(qgemv_affine8(U32 A, U16 A, U16 A, U16 A, QD_F16, y, 16, 128, 129, 64, nullptr), QD_ERR_INVALID_ARGUMENT);
    EXPECT(qgemv_affine4(U32 A, U16 A, U16 A, U16 A, QD_F16, y, 16, 100, 1, 64, nullptr), QD_ERR_INVALID_ARGUMENT);
    EXPECT(qgemv_affine4(U32 A, U16 A, U16 A, U16 A, QD_F16, y, 16, 1 << 23, 1, 64, nullptr), QD_ERR_UNSUPPORTED);
    EXPECT(qgemv_affine4(U32 A, U16 A, U16 A, U16 A, QD_F16, y, 0, 128, 1, 64, nullptr), QD_ERR_INVALID_ARGUMENT);
    EXPECT(qgemv_affine4(U32 A, U16 A, U16 A, U16 A, QD_F16, y, 16, 128, 1, 32, nullptr), QD_ERR_UNSUPPORTED);
    EXPECT(qgemv_affine4(U32 A, U16 A, nullptr, U16 A, QD_F16, y, 16, 128, 1, 64, nullptr), QD_ERR_INVALID_ARGUMENT);
    EXPECT(qgemv_affine4(U32 MIS, U16 A, U16 A, U16 A, QD_F16, y, 16, 128, 1, 64, nullptr), QD_ERR_MISALIGNED);
    EXPECT(qgemv_affine4(U32 A, U16 A, U16 A, U16 A, (qd_dtype)7, y, 16, 128, 1, 64, nullptr), QD_ERR_UNSUPPORTED);
    // Mirai formats and the rotation prologue
    EXPECT(qgemv_mirai_m(U32 A, U16 A, U32 A, U16 A, QD_F16, y, 16, 1088, 8, 64, nullptr), QD_OK);
    EXPECT(qgemv_mirai_m(U32 A, U16 A, nullptr, U16 A, QD_F16, y, 16, 1088, 8, 64, nullptr), QD_ERR_INVALID_ARGUMENT);
    EXPECT(qgemv_mirai_l(U32 A, U16 A, U16 A, QD_BF16, y, 16, 128, 3, 64, nullptr), QD_OK);
    EXPECT(qgemv_mirai_m_rht(U32 A, U16 A, U32 A, U32 A, U16 A, 1e-6f, U16 A, QD_F16, y, 16, 128, 1, 64, nullptr), QD_OK);
    EXPECT(qgemv_mirai_m_rht(U32 A, U16 A, U32 A, nullptr, nullptr, 0.f, U16 A, QD_F16, y, 16, 128, 1, 64, nullptr), QD_OK);
    EXPECT(qgemv_mirai_l_rht(U32 A, U16 A, U32 A, U16 A, -1.f, U16 A, QD_F16, y, 16, 128, 1, 64, nullptr), QD_ERR_INVALID_ARGUMENT);
    EXPECT(qgemv_mirai_l_rht(U32 A, U16 A, U32 MIS, U16 A, 1e-6f, U16 A, QD_F16, y, 16, 128, 1, 64, nullptr), QD_ERR_MISALIGNED);
    // routing
    EXPECT(qmoe_route_topk(y, 4, 128, 8, (int32_t*)A, y, nullptr), QD_OK);
    EXPECT(qmoe_route_topk(y, 4, 1025, 8, (int32_t*)A, y, nullptr), QD_ERR_INVALID_ARGUMENT);
    EXPECT(qmoe_route_topk(y, 4, 8, 9, (int32_t*)A, y, nullptr), QD_ERR_INVALID_ARGUMENT);
    EXPECT(qmoe_route_topk(y, 0, 8, 2, (int32_t*)A, y, nullptr), QD_ERR_INVALID_ARGUMENT);
    // MoE expert block and decode layers
    qd_moe_weights w = moe();
    const size_t ws1 = qmoe_expert_workspace_bytes(&w, 1, 8), ws128 = qmoe_expert_workspace_bytes(&w, 128, 8);
    if (!(ws1 > 0 && ws128 > ws1) || qmoe_expert_workspace_bytes(nullptr, 1, 8) != 0) ++fails;
    EXPECT(qmoe_expert_gemv(&w, (const int32_t*)A, y, 1, 8, A, QD_F16, y, A, ws1, nullptr), QD_OK);
    EXPECT(qmoe_expert_gemv(&w, (const int32_t*)A, y, 128, 8, A, QD_BF16, y, A, ws128, nullptr), QD_OK);
    EXPECT(qmoe_expert_gemv(&w, (const int32_t*)A, y, 128, 8, A, QD_BF16, y, A, ws1, nullptr), QD_ERR_WORKSPACE);
    EXPECT(qmoe_expert_gemv(&w, (const int32_t*)A, y, 129, 8, A, QD_BF16, y, A, ws128, nullptr), QD_ERR_INVALID_ARGUMENT);
    EXPECT(qmoe_expert_gemv(nullptr, (const int32_t*)A, y, 1, 8, A, QD_F16, y, A, ws1, nullptr), QD_ERR_INVALID_ARGUMENT);
    qd_moe_weights bad = moe(128, 100);
    EXPECT(qmoe_expert_gemv(&bad, (const int32_t*)A, y, 1, 8, A, QD_F16, y, A, ws1, nullptr), QD_ERR_INVALID_ARGUMENT);
    bad = moe(128, 2816, 704, 2112, 64, 9);
    EXPECT(qmoe_expert_gemv(&bad, (const int32_t*)A, y, 1, 8, A, QD_F16, y, A, ws1, nullptr), QD_ERR_UNSUPPORTED);
    EXPECT(qmoe_layer_decode(&w, U32 A, U16 A, U16 A, 8, A, QD_F16, y, (int32_t*)A, y, y, A, ws1, nullptr), QD_OK);
    EXPECT(qmoe_layer_decode(&w, U32 A, U16 A, U16 A, 8, A, QD_F16, y, (int32_t*)A, y, y, nullptr, ws1, nullptr), QD_ERR_WORKSPACE);
    EXPECT(qmoe_layer_decode_noalloc(&w, U32 A, U16 A, U16 A, 8, A, QD_F16, y, (int32_t*)A, y, y, nullptr), QD_OK);
    const size_t pws = qmoe_layer_prefill_workspace_bytes(&w, 128, 8);
    if (!(pws > qmoe_expert_workspace_bytes(&w, 128, 8)) || qmoe_layer_prefill_workspace_bytes(&w, 129, 8) != 0) ++fails;
    EXPECT(qmoe_layer_prefill(&w, U32 A, U16 A, U16 A, 8, 128, A, QD_BF16, y, (int32_t*)A, y, y, A, pws, nullptr), QD_OK);
    EXPECT(qmoe_layer_prefill(&w, U32 A, U16 A, U16 A, 8, 128, A, QD_BF16, y, (int32_t*)A, y, y, A, pws - 1, nullptr), QD_ERR_WORKSPACE);
    EXPECT(qmoe_layer_prefill(&w, U32 A, U16 A, U16 A, 8, 129, A, QD_BF16, y, (int32_t*)A, y, y, A, pws, nullptr), QD_ERR_INVALID_ARGUMENT);
    EXPECT(qmoe_layer_prefill(&w, nullptr, U16 A, U16 A, 8, 128, A, QD_BF16, y, (int32_t*)A, y, y, A, pws, nullptr), QD_ERR_INVALID_ARGUMENT);
    bad = moe(64, 2816, 32768, 1024);
    EXPECT(qmoe_layer_decode_noalloc(&bad, U32 A, U16 A, U16 A, 32, A, QD_F16, y, (int32_t*)A, y, y, nullptr), QD_ERR_WORKSPACE);
    bad = moe(257);
    EXPECT(qmoe_layer_decode_noalloc(&bad, U32 A, U16 A, U16 A, 8, A, QD_F16, y, (int32_t*)A, y, y, nullptr), QD_ERR_UNSUPPORTED);
    // chunk and verification GEMMs
    EXPECT(qgemm_affine4_chunk(U32 A, U16 A, U16 A, U16 A, y, 128, 14336, 4096, 64, nullptr, 0, nullptr), QD_OK);
    EXPECT(qgemm_affine4_chunk(U32 A, U16 A, U16 A, U16 A, y, 129, 14336, 4096, 64, nullptr, 0, nullptr), QD_ERR_INVALID_ARGUMENT);
    const size_t cws = qgemm_affine4_chunk_workspace_bytes(128, 4096, 14336);
    if (!(cws > 0) || qgemm_affine4_chunk_workspace_bytes(128, 14336, 4096) != 0) ++fails;
    EXPECT(qgemm_affine4_chunk(U32 A, U16 A, U16 A, U16 A, y, 128, 4096, 14336, 64, A, cws, nullptr), QD_OK);
    EXPECT(qgemm_affine4_chunk(U32 A, U16 A, U16 A, U16 A, y, 128, 4096, 14336, 64, nullptr, cws, nullptr), QD_ERR_WORKSPACE);
    EXPECT(qgemm_affine4_verify(U32 A, U16 A, U16 A, U16 A, QD_F16, y, 32, 14336, 4096, 64, nullptr, 0, nullptr), QD_OK);
    EXPECT(qgemm_affine4_verify(U32 A, U16 A, U16 A, U16 A, (qd_dtype)2, y, 32, 14336, 4096, 64, nullptr, 0, nullptr), QD_ERR_UNSUPPORTED);
    const size_t kws = qgemm_affine4_verify_workspace_bytes(32, 4096, 14336);
    if (!(kws > 0) || qgemm_affine4_verify_workspace_bytes(129, 4096, 14336) != 0) ++fails;
    EXPECT(qgemm_affine4_verify(U32 A, U16 A, U16 A, U16 A, QD_F16, y, 32, 4096, 14336, 64, A, kws, nullptr), QD_OK);
    EXPECT(qgemm_affine4_verify(U32 A, U16 A, U16 A, U16 A, QD_F16, y, 32, 4096, 14336, 64, A, kws - 1, nullptr), QD_ERR_WORKSPACE);
    EXPECT(qgemm_affine4_verify(U32 A, U16 A, U16 A, U16 A, QD_F16, y, 32, 4096, 14336, 64, nullptr, kws, nullptr), QD_ERR_WORKSPACE);
    // decode attention
    const size_t vws = qgemm_affine4_verify_i8_workspace_bytes(32, 4096);
    if (!(vws > 0) || qgemm_affine4_verify_i8_workspace_bytes(33, 4096) != 0) ++fails;
    EXPECT(qgemm_affine4_verify_i8(U32 A, U16 A, U16 A, U16 A, y, 32, 14336, 4096, 64, A, vws, nullptr), QD_OK);
    EXPECT(qgemm_affine4_verify_i8(U32 A, U16 A, U16 A, U16 A, y, 33, 14336, 4096, 64, A, vws, nullptr), QD_ERR_INVALID_ARGUMENT);
    EXPECT(qgemm_affine4_verify_i8(U32 A, U16 A, U16 A, U16 A, y, 32, 14336, 4096, 64, A, vws - 1, nullptr), QD_ERR_WORKSPACE);
    EXPECT(qgemm_affine4_verify_i8(U32 A, U16 A, U16 A, U16 A, y, 32, 14336, 4096, 64, nullptr, vws, nullptr), QD_ERR_WORKSPACE);
    const size_t aws = qattn_decode_workspace_bytes(16, 8, 128, 4096);
    const uint16_t* h = U16 A;
    uint16_t* hc = (uint16_t*)A;
    EXPECT(qattn_decode(h, h, h, hc, hc, 16, 8, 128, 4096, 0, 100, 0.088f, y, A, aws, nullptr), QD_OK);
    EXPECT(qattn_decode(h, h, h, hc, hc, 16, 8, 128, 1024, 1024, 5000, 0.088f, y, A, aws, nullptr), QD_OK);
    EXPECT(qattn_decode(h, h, h, hc, hc, 16, 8, 96, 4096, 0, 100, 0.088f, y, A, aws, nullptr), QD_ERR_UNSUPPORTED);
    EXPECT(qattn_decode(h, h, h, hc, hc, 16, 8, 128, 4096, 0, 4096, 0.088f, y, A, aws, nullptr), QD_ERR_INVALID_ARGUMENT);
    EXPECT(qattn_decode(h, h, h, hc, hc, 16, 8, 128, 4096, 0, 100, 0.088f, y, A, aws - 1, nullptr), QD_ERR_WORKSPACE);
    // the read stream
    EXPECT(qd_stream_read(A, 4096, (uint32_t*)A, nullptr), QD_OK);
    EXPECT(qd_stream_read(A, 0, (uint32_t*)A, nullptr), QD_ERR_INVALID_ARGUMENT);
    EXPECT(qd_stream_read(MIS, 16, (uint32_t*)A, nullptr), QD_ERR_MISALIGNED);
    // status strings
    for (int s = -1; s < 8; ++s)
        if (!qd_status_string((qd_status)s)) ++fails;
    if (fails) {
        std::fprintf(stderr, "%d failures\n", fails);
        return 1;
    }
    std::printf("abi driver ok (%d launches)\n", g_launches);
    return 0;
}
