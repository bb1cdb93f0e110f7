// Internal launch interface between the C ABI (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace qd {

struct DeviceInfo {
    int id = -1;
    int cus = 256;                  // compute units
    size_t max_lds_per_block = 65536;
    size_t lds_per_cu = 65536;
};

// Properties of the calling thread's current device (queried once per device).
const DeviceInfo& device_info();

// Resident workgroups per CU for a kernel at this block size and LDS use.
int occupancy(const void* func, int threads, size_t lds_bytes);

// Rotation prologue of the Mirai formats: x -> H D (RMSNorm(x) * gamma) per
// block of 32 inputs before the contraction.
struct GemvRot {
    const uint32_t* signs;   // [K/32], NULL = no sign flips
    const uint16_t* gamma;   // [K] in x's kind, NULL = no RMSNorm
    float eps;
};

// x kinds: 0 = fp16 bits, 1 = bf16 bits, 2 = fp32.
// fmt: 0 = affine (fp16 s, b); 1 = Mirai-M (bits 4, bf16 s, zero points zp,
// b unused); 2 = Mirai-L (bits 8, signed codes, bf16 s, b and zp unused).
// The Mirai formats take batch <= 8 and optionally the rotation prologue.
hipError_t launch_gemv(int bits, int fmt, const uint32_t* wq, const uint16_t* s,
                       const uint16_t* b, const uint32_t* zp, const void* x, int xkind, float* y,
                       int N, int K, int batch, hipStream_t st, const GemvRot* rot = nullptr);

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                             hipStream_t st);
// Routing from the router's split slices part [splits][T][E]: the logits are
// their sum in split order (also written to `logits`).
hipError_t launch_route_topk_slices(const float* part, int splits, int T, int E, int k,
                                    float* logits, int32_t* idx, float* w, hipStream_t st);

struct MoeArgs {
    int E, H, I, Is, act;
    const uint32_t *gu_q, *dn_q, *sgu_q, *sdn_q;
    const uint16_t *gu_s, *gu_b, *dn_s, *dn_b, *sgu_s, *sgu_b, *sdn_s, *sdn_b;
};

size_t moe_workspace_bytes(const MoeArgs& m, int T, int k);
size_t moe_decode_workspace_bytes(const MoeArgs& m, int k);
size_t moe_prefill_workspace_bytes(const MoeArgs& m, int T, int k);

// One token at a time through the GEMV kernels (workspace: decode bytes).
hipError_t launch_moe_decode(const MoeArgs& m, const int32_t* idx, const float* w, int T, int k,
                             const void* x, int xkind, float* y, void* ws, hipStream_t st);
// Expert-grouped MFMA path for prefill chunks.
hipError_t launch_moe_prefill(const MoeArgs& m, const int32_t* idx, const float* w, int T, int k,
                              const void* x, int xkind, float* y, void* ws, hipStream_t st);

// One decode token from its router logits: top-k ranked inside the gate+up
// kernel (ids and weights written to idx / w), then down + combine.
hipError_t launch_moe_decode_routed(const MoeArgs& m, const float* logits, int k, const void* x,
                                    int xkind, int32_t* idx, float* w, float* y, void* ws,
                                    hipStream_t st);

// The same layer with the gate+up activations in the library's per-device
// scratch (kMoeNoAllocBytes) instead of a caller workspace.
constexpr size_t kMoeNoAllocBytes = size_t(4) << 20;
hipError_t launch_moe_decode_routed_noalloc(const MoeArgs& m, const float* logits, int k,
                                            const void* x, int xkind, int32_t* idx, float* w,
                                            float* y, hipStream_t st);

hipError_t launch_moe_experts(const MoeArgs& m, const int32_t* idx, const float* w, int T, int k,
                              const void* x, int xkind, float* y, void* ws, size_t ws_bytes,
                              hipStream_t st);

// 4-bit affine weights against 2..8 fp16 vectors on the matrix core.
hipError_t launch_gemv_mfma(const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                            const uint16_t* x, float* y, int N, int K, int nb, hipStream_t st);

// Verification GEMM on per-token int8 activations (M <= 32, fp16 X).
size_t verify_i8_workspace_bytes(int M, int K);
hipError_t launch_verify_i8(const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                            const uint16_t* x, float* y, int M, int N, int K, void* ws,
                            size_t ws_bytes, hipStream_t st);

// 8-bit weights over T > 8 tokens (f16 or bf16 activations) on the matrix core.
hipError_t launch_gemm8_tokens(const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                               const uint16_t* x, int xkind, float* y, int N, int K, int T,
                               hipStream_t st);
// The same with K split across workgroups: slices part [splits][T][N], added
// by their reader (launch_route_topk_slices). The split depends on the shape only.
struct G8Split {
    int splits;   // 1 = none
    int gsplit;   // groups per split; the last one takes the rest
};
G8Split gemm8_split(int N, int K, int T);
hipError_t launch_gemm8_tokens_split(const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                                     const uint16_t* x, int xkind, float* part, int N, int K, int T,
                                     hipStream_t st);

// Decode attention of one token over fp16 KV caches (circular when window > 0).
size_t attn_workspace_bytes(int Hq, int Hkv, int D, int cap);
hipError_t launch_attn_decode(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                              uint16_t* kc, uint16_t* vc, int Hq, int Hkv, int D, int cap,
                              int window, int pos, float scale, float* out, void* ws,
                              size_t ws_bytes, hipStream_t st);

// Read-only stream over bytes of device memory (the HBM read ceiling).
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t st);

// x: fp16 or bf16 bits (xkind X_F16 / X_BF16), [M][K]. With a workspace of
// chunk_split_workspace_bytes(M, N, K) bytes, shapes with few tiles split K
// across workgroups (chunk_split) and add the slices in a second pass; with
// ws == nullptr the call runs unsplit.
struct ChunkSplit {
    int splits;   // K splits (1 = none)
    int gsplit;   // groups per split; the last one takes the rest
};
ChunkSplit chunk_split(int M, int N, int K);
size_t chunk_split_workspace_bytes(int M, int N, int K);
hipError_t launch_chunk_gemm(int bits, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                             const uint16_t* x, int xkind, float* y, int M, int N, int K,
                             void* ws, size_t ws_bytes, hipStream_t st);

}  // namespace qd
