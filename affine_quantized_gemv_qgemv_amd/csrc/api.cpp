// C ABI of libqdecode: argument checks, then kernel launches.
//
// Conventions follow the uzu engine as described in
// fiv.co.kr/repos/uzu-deep-dive.html: tensors are checked by shape and dtype
// before use (section 4-3), failures come back as values rather than
// panics (sections 4-2 and 4-4), and an unsupported layout is rejected with
// an error (section 7-1). Every check here runs before any HIP call, so a
// bad argument is reported identically on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>

#include "../../include/qdecode.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

qd_status fail(qd_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

qd_status ok() {
    g_last_error.clear();
    return QD_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

qd_status from_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(QD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define CHECK_PTR(p)                                                               \
    do {                                                                           \
        if (!(p)) return fail(QD_ERR_INVALID_ARGUMENT, "%s is NULL", #p);          \
        if (!aligned16(p)) return fail(QD_ERR_MISALIGNED, "%s is not 16-byte aligned", #p); \
    } while (0)

qd_status check_matrix(const char* fn, int32_t N, int32_t K, int32_t group_size) {
    if (group_size != 64)
        return fail(QD_ERR_UNSUPPORTED, "%s: group_size %d (only 64 is supported)", fn, group_size);
    if (N < 1) return fail(QD_ERR_INVALID_ARGUMENT, "%s: N = %d must be >= 1", fn, N);
    if (K < 64 || K % 64)
        return fail(QD_ERR_INVALID_ARGUMENT, "%s: K = %d must be a positive multiple of 64", fn, K);
    if (K > (1 << 22))
        return fail(QD_ERR_UNSUPPORTED, "%s: K = %d exceeds 4194304", fn, K);
    return QD_OK;
}

// fmt: 0 = affine (biases), 1 = Mirai-M (zeros), 2 = Mirai-L (neither).
qd_status gemv_common(const char* fn, int bits, int fmt, int max_batch, const uint32_t* wq,
                      const uint16_t* scales, const uint16_t* biases, const uint32_t* zeros,
                      const uint16_t* x, qd_dtype x_dtype, float* y, int32_t N, int32_t K,
                      int32_t batch, int32_t group_size, qd_stream stream,
                      const qd::GemvRot* rot = nullptr) {
    qd_status st = check_matrix(fn, N, K, group_size);
    if (st != QD_OK) return st;
    if (batch < 1 || batch > max_batch)
        return fail(QD_ERR_INVALID_ARGUMENT, "%s: batch = %d must be in [1, %d]", fn, batch,
                    max_batch);
    if (x_dtype != QD_F16 && x_dtype != QD_BF16)
        return fail(QD_ERR_UNSUPPORTED, "%s: x_dtype %d", fn, (int)x_dtype);
    CHECK_PTR(wq);
    CHECK_PTR(scales);
    if (fmt == 0) CHECK_PTR(biases);
    if (fmt == 1) CHECK_PTR(zeros);
    CHECK_PTR(x);
    CHECK_PTR(y);
    if (rot) {
        if (rot->signs) CHECK_PTR(rot->signs);
        if (rot->gamma) CHECK_PTR(rot->gamma);
        if (!(rot->eps >= 0.f) || rot->eps > 1e30f)
            return fail(QD_ERR_INVALID_ARGUMENT, "%s: eps = %g must be finite and >= 0", fn,
                        (double)rot->eps);
    }
    const int xkind = x_dtype == QD_F16 ? 0 : 1;
    return from_hip(qd::launch_gemv(bits, fmt, wq, scales, biases, zeros, x, xkind, y, N, K,
                                    batch, (hipStream_t)stream, rot),
                    fn);
}

// The activation field as an int: C callers may store any int in an enum
// field, and reading an out-of-range value through the C++ enum type is
// undefined, so the bytes are copied instead.
int moe_act(const qd_moe_weights* w) {
    int act;
    static_assert(sizeof(act) == sizeof(w->act), "qd_act is int-sized");
    std::memcpy(&act, &w->act, sizeof act);
    return act;
}

qd_status check_moe(const char* fn, const qd_moe_weights* w) {
    if (!w) return fail(QD_ERR_INVALID_ARGUMENT, "%s: weights is NULL", fn);
    if (w->group_size != 64)
        return fail(QD_ERR_UNSUPPORTED, "%s: group_size %d (only 64 is supported)", fn,
                    w->group_size);
    if (w->E < 1) return fail(QD_ERR_INVALID_ARGUMENT, "%s: E = %d must be >= 1", fn, w->E);
    if (w->H < 64 || w->H % 64 || w->I < 64 || w->I % 64 || w->I_shared < 64 ||
        w->I_shared % 64)
        return fail(QD_ERR_INVALID_ARGUMENT,
                    "%s: H = %d, I = %d, I_shared = %d must be positive multiples of 64", fn, w->H,
                    w->I, w->I_shared);
    if (w->H > (1 << 20) || w->I > (1 << 20) || w->I_shared > (1 << 20))
        return fail(QD_ERR_UNSUPPORTED, "%s: H, I and I_shared are limited to 2^20", fn);
    if (moe_act(w) != QD_GELU_ERF && moe_act(w) != QD_GELU_TANH)
        return fail(QD_ERR_UNSUPPORTED, "%s: act %d", fn, moe_act(w));
    CHECK_PTR(w->gu_q);
    CHECK_PTR(w->gu_s);
    CHECK_PTR(w->gu_b);
    CHECK_PTR(w->dn_q);
    CHECK_PTR(w->dn_s);
    CHECK_PTR(w->dn_b);
    CHECK_PTR(w->sgu_q);
    CHECK_PTR(w->sgu_s);
    CHECK_PTR(w->sgu_b);
    CHECK_PTR(w->sdn_q);
    CHECK_PTR(w->sdn_s);
    CHECK_PTR(w->sdn_b);
    return QD_OK;
}

qd::MoeArgs moe_args(const qd_moe_weights* w) {
    qd::MoeArgs m{};
    m.E = w->E;
    m.H = w->H;
    m.I = w->I;
    m.Is = w->I_shared;
    m.act = moe_act(w);
    m.gu_q = w->gu_q;
    m.dn_q = w->dn_q;
    m.sgu_q = w->sgu_q;
    m.sdn_q = w->sdn_q;
    m.gu_s = w->gu_s;
    m.gu_b = w->gu_b;
    m.dn_s = w->dn_s;
    m.dn_b = w->dn_b;
    m.sgu_s = w->sgu_s;
    m.sgu_b = w->sgu_b;
    m.sdn_s = w->sdn_s;
    m.sdn_b = w->sdn_b;
    return m;
}

}  // namespace

namespace qd {

const DeviceInfo& device_info() {
    static DeviceInfo infos[64];
    static std::once_flag flags[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    std::call_once(flags[dev], [dev] {
        DeviceInfo d;
        d.id = dev;
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            v > 0)
            d.cus = v;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) ==
                hipSuccess &&
            v > 0)
            d.max_lds_per_block = (size_t)v;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) ==
                hipSuccess &&
            v > 0)
            d.lds_per_cu = (size_t)v;
        else
            d.lds_per_cu = d.max_lds_per_block;
        infos[dev] = d;
    });
    return infos[dev];
}

int occupancy(const void* func, int threads, size_t lds_bytes) {
    static std::mutex mu;
    static std::map<std::tuple<int, const void*, int, size_t>, int> cache;
    int dev = 0;
    (void)hipGetDevice(&dev);
    const auto key = std::make_tuple(dev, func, threads, lds_bytes);
    {
        std::lock_guard<std::mutex> g(mu);
        auto it = cache.find(key);
        if (it != cache.end()) return it->second;
    }
    // allow launches up to the device's per-workgroup maximum less the
    // kernel's static LDS (a kernel is launched with several dynamic sizes;
    // the attribute must cover the largest)
    if (lds_bytes > 65536) {
        hipFuncAttributes fa{};
        size_t stat = 0;
        if (hipFuncGetAttributes(&fa, func) == hipSuccess) stat = fa.sharedSizeBytes;
        const size_t maxdyn = device_info().max_lds_per_block - std::min(stat, device_info().max_lds_per_block);
        (void)hipFuncSetAttribute(func, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)std::max(maxdyn, lds_bytes));
    }
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, func, threads, lds_bytes) != hipSuccess ||
        n < 1)
        n = 1;
    std::lock_guard<std::mutex> g(mu);
    cache[key] = n;
    return n;
}

}  // namespace qd

extern "C" {

qd_status qgemv_affine4(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                        const uint16_t* x, qd_dtype x_dtype, float* y, int32_t N, int32_t K,
                        int32_t batch, int32_t group_size, qd_stream stream) {
    return gemv_common("qgemv_affine4", 4, 0, 8, wq, scales, biases, nullptr, x, x_dtype, y, N, K,
                       batch, group_size, stream);
}

qd_status qgemv_affine8(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                        const uint16_t* x, qd_dtype x_dtype, float* y, int32_t N, int32_t K,
                        int32_t batch, int32_t group_size, qd_stream stream) {
    return gemv_common("qgemv_affine8", 8, 0, 128, wq, scales, biases, nullptr, x, x_dtype, y, N,
                       K, batch, group_size, stream);
}

qd_status qgemv_mirai_m(const uint32_t* wq, const uint16_t* scales, const uint32_t* zeros,
                        const uint16_t* x, qd_dtype x_dtype, float* y, int32_t N, int32_t K,
                        int32_t batch, int32_t group_size, qd_stream stream) {
    return gemv_common("qgemv_mirai_m", 4, 1, 8, wq, scales, nullptr, zeros, x, x_dtype, y, N, K,
                       batch, group_size, stream);
}

qd_status qgemv_mirai_m_rht(const uint32_t* wq, const uint16_t* scales, const uint32_t* zeros,
                            const uint32_t* signs, const uint16_t* gamma, float eps,
                            const uint16_t* x, qd_dtype x_dtype, float* y, int32_t N, int32_t K,
                            int32_t batch, int32_t group_size, qd_stream stream) {
    const qd::GemvRot rot{signs, gamma, eps};
    return gemv_common("qgemv_mirai_m_rht", 4, 1, 8, wq, scales, nullptr, zeros, x, x_dtype, y, N,
                       K, batch, group_size, stream, &rot);
}

qd_status qgemv_mirai_l_rht(const uint32_t* wq, const uint16_t* scales, const uint32_t* signs,
                            const uint16_t* gamma, float eps, const uint16_t* x, qd_dtype x_dtype,
                            float* y, int32_t N, int32_t K, int32_t batch, int32_t group_size,
                            qd_stream stream) {
    const qd::GemvRot rot{signs, gamma, eps};
    return gemv_common("qgemv_mirai_l_rht", 8, 2, 8, wq, scales, nullptr, nullptr, x, x_dtype, y,
                       N, K, batch, group_size, stream, &rot);
}

qd_status qgemv_mirai_l(const uint32_t* wq, const uint16_t* scales, const uint16_t* x,
                        qd_dtype x_dtype, float* y, int32_t N, int32_t K, int32_t batch,
                        int32_t group_size, qd_stream stream) {
    return gemv_common("qgemv_mirai_l", 8, 2, 8, wq, scales, nullptr, nullptr, x, x_dtype, y, N, K,
                       batch, group_size, stream);
}

qd_status qmoe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* idx,
                          float* weights, qd_stream stream) {
    if (T < 1) return fail(QD_ERR_INVALID_ARGUMENT, "qmoe_route_topk: T = %d must be >= 1", T);
    if (E < 1 || E > 1024)
        return fail(QD_ERR_INVALID_ARGUMENT, "qmoe_route_topk: E = %d must be in [1, 1024]", E);
    if (k < 1 || k > E || k > 32)
        return fail(QD_ERR_INVALID_ARGUMENT, "qmoe_route_topk: k = %d must be in [1, min(E, 32)]",
                    k);
    CHECK_PTR(logits);
    CHECK_PTR(idx);
    CHECK_PTR(weights);
    return from_hip(qd::launch_route_topk(logits, T, E, k, idx, weights, (hipStream_t)stream),
                    "qmoe_route_topk");
}

size_t qmoe_expert_workspace_bytes(const qd_moe_weights* w, int32_t T, int32_t k) {
    if (!w || T < 1 || k < 1 || w->I < 1 || w->I_shared < 1 || w->E < 1) return 0;
    return qd::moe_workspace_bytes(moe_args(w), T, k);
}

qd_status qmoe_expert_gemv(const qd_moe_weights* w, const int32_t* idx, const float* weights,
                           int32_t T, int32_t k, const void* x, qd_dtype x_dtype, float* y,
                           void* workspace, size_t ws_bytes, qd_stream stream) {
    const char* fn = "qmoe_expert_gemv";
    qd_status st = check_moe(fn, w);
    if (st != QD_OK) return st;
    if (T < 1 || T > 128)
        return fail(QD_ERR_INVALID_ARGUMENT, "%s: T = %d must be in [1, 128]", fn, T);
    if (k < 1 || k > w->E || k > 32)
        return fail(QD_ERR_INVALID_ARGUMENT, "%s: k = %d must be in [1, min(E, 32)]", fn, k);
    if (x_dtype != QD_F16 && x_dtype != QD_BF16)
        return fail(QD_ERR_UNSUPPORTED, "%s: x_dtype %d", fn, (int)x_dtype);
    CHECK_PTR(idx);
    CHECK_PTR(weights);
    CHECK_PTR(x);
    CHECK_PTR(y);
    const qd::MoeArgs m = moe_args(w);
    const size_t need = qd::moe_workspace_bytes(m, T, k);
    if (need > 0) {
        if (!workspace)
            return fail(QD_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
        if (!aligned16(workspace))
            return fail(QD_ERR_MISALIGNED, "%s: workspace is not 16-byte aligned", fn);
        if (ws_bytes < need)
            return fail(QD_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, ws_bytes,
                        need);
    }
    return from_hip(qd::launch_moe_experts(m, idx, weights, T, k, x, x_dtype == QD_F16 ? 0 : 1, y,
                                           workspace, ws_bytes, (hipStream_t)stream),
                    fn);
}

}  // extern "C"

namespace {

// Checks shared by the two decode-layer calls (everything but the workspace).
qd_status check_layer_decode(const char* fn, const qd_moe_weights* w, const uint32_t* router_q,
                             const uint16_t* router_s, const uint16_t* router_b, int32_t k,
                             const void* x, qd_dtype x_dtype, const float* logits,
                             const int32_t* idx, const float* weights, const float* y) {
    qd_status st = check_moe(fn, w);
    if (st != QD_OK) return st;
    if (w->E > 256) return fail(QD_ERR_UNSUPPORTED, "%s: E = %d (at most 256)", fn, w->E);
    if (k < 1 || k > w->E || k > 32)
        return fail(QD_ERR_INVALID_ARGUMENT, "%s: k = %d must be in [1, min(E, 32)]", fn, k);
    if (x_dtype != QD_F16 && x_dtype != QD_BF16)
        return fail(QD_ERR_UNSUPPORTED, "%s: x_dtype %d", fn, (int)x_dtype);
    CHECK_PTR(router_q);
    CHECK_PTR(router_s);
    CHECK_PTR(router_b);
    CHECK_PTR(x);
    CHECK_PTR(logits);
    CHECK_PTR(idx);
    CHECK_PTR(weights);
    CHECK_PTR(y);
    return QD_OK;
}

}  // namespace

extern "C" {

qd_status qmoe_layer_decode(const qd_moe_weights* w, const uint32_t* router_q,
                            const uint16_t* router_s, const uint16_t* router_b, int32_t k,
                            const void* x, qd_dtype x_dtype, float* logits, int32_t* idx,
                            float* weights, float* y, void* workspace, size_t ws_bytes,
                            qd_stream stream) {
    const char* fn = "qmoe_layer_decode";
    qd_status st = check_layer_decode(fn, w, router_q, router_s, router_b, k, x, x_dtype, logits,
                                      idx, weights, y);
    if (st != QD_OK) return st;
    const qd::MoeArgs m = moe_args(w);
    const size_t need = qd::moe_workspace_bytes(m, 1, k);
    if (!workspace)
        return fail(QD_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
    if (!aligned16(workspace))
        return fail(QD_ERR_MISALIGNED, "%s: workspace is not 16-byte aligned", fn);
    if (ws_bytes < need)
        return fail(QD_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, ws_bytes, need);
    const int xkind = x_dtype == QD_F16 ? 0 : 1;
    hipError_t e = qd::launch_gemv(8, 0, router_q, router_s, router_b, nullptr, x, xkind, logits,
                                   w->E, w->H, 1, (hipStream_t)stream);
    if (e != hipSuccess) return from_hip(e, fn);
    return from_hip(qd::launch_moe_decode_routed(m, logits, k, x, xkind, idx, weights, y, workspace,
                                                 (hipStream_t)stream),
                    fn);
}

qd_status qmoe_layer_decode_noalloc(const qd_moe_weights* w, const uint32_t* router_q,
                                    const uint16_t* router_s, const uint16_t* router_b, int32_t k,
                                    const void* x, qd_dtype x_dtype, float* logits, int32_t* idx,
                                    float* weights, float* y, qd_stream stream) {
    const char* fn = "qmoe_layer_decode_noalloc";
    qd_status st = check_layer_decode(fn, w, router_q, router_s, router_b, k, x, x_dtype, logits,
                                      idx, weights, y);
    if (st != QD_OK) return st;
    const qd::MoeArgs m = moe_args(w);
    const size_t need = qd::moe_decode_workspace_bytes(m, k);
    if (need > qd::kMoeNoAllocBytes)
        return fail(QD_ERR_WORKSPACE,
                    "%s: k * I + I_shared = %zu activations need %zu bytes of scratch; the "
                    "allocation-free call holds at most %zu (use qmoe_layer_decode)",
                    fn, need / sizeof(float), need, qd::kMoeNoAllocBytes);
    const int xkind = x_dtype == QD_F16 ? 0 : 1;
    hipError_t e = qd::launch_gemv(8, 0, router_q, router_s, router_b, nullptr, x, xkind, logits,
                                   w->E, w->H, 1, (hipStream_t)stream);
    if (e != hipSuccess) return from_hip(e, fn);
    return from_hip(qd::launch_moe_decode_routed_noalloc(m, logits, k, x, xkind, idx, weights, y,
                                                         (hipStream_t)stream),
                    fn);
}

// Prefill layer workspace: the expert block's, then the router's split slices.
static size_t prefill_expert_part(const qd::MoeArgs& m, int T, int k) {
    return (qd::moe_workspace_bytes(m, T, k) + 255) & ~(size_t)255;
}

size_t qmoe_layer_prefill_workspace_bytes(const qd_moe_weights* w, int32_t T, int32_t k) {
    if (!w || T < 1 || T > 128 || k < 1 || w->I < 1 || w->I_shared < 1 || w->E < 1 || w->H < 64 ||
        w->H % 64)
        return 0;
    const qd::G8Split c = qd::gemm8_split(w->E, w->H, T);
    return prefill_expert_part(moe_args(w), T, k) + (size_t)c.splits * T * w->E * sizeof(float);
}

qd_status qmoe_layer_prefill(const qd_moe_weights* w, const uint32_t* router_q,
                             const uint16_t* router_s, const uint16_t* router_b, int32_t k, int32_t T,
                             const void* x, qd_dtype x_dtype, float* logits, int32_t* idx,
                             float* weights, float* y, void* workspace, size_t ws_bytes,
                             qd_stream stream) {
    const char* fn = "qmoe_layer_prefill";
    qd_status st = check_moe(fn, w);
    if (st != QD_OK) return st;
    if (T < 1 || T > 128)
        return fail(QD_ERR_INVALID_ARGUMENT, "%s: T = %d must be in [1, 128]", fn, T);
    if (w->E > 1024) return fail(QD_ERR_UNSUPPORTED, "%s: E = %d (at most 1024)", fn, w->E);
    if (k < 1 || k > w->E || k > 32)
        return fail(QD_ERR_INVALID_ARGUMENT, "%s: k = %d must be in [1, min(E, 32)]", fn, k);
    if (x_dtype != QD_F16 && x_dtype != QD_BF16)
        return fail(QD_ERR_UNSUPPORTED, "%s: x_dtype %d", fn, (int)x_dtype);
    st = check_matrix(fn, w->E, w->H, 64);
    if (st != QD_OK) return st;
    CHECK_PTR(router_q);
    CHECK_PTR(router_s);
    CHECK_PTR(router_b);
    CHECK_PTR(x);
    CHECK_PTR(logits);
    CHECK_PTR(idx);
    CHECK_PTR(weights);
    CHECK_PTR(y);
    const size_t need = qmoe_layer_prefill_workspace_bytes(w, T, k);
    if (!workspace) return fail(QD_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
    if (!aligned16(workspace)) return fail(QD_ERR_MISALIGNED, "%s: workspace is not 16-byte aligned", fn);
    if (ws_bytes < need)
        return fail(QD_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, ws_bytes, need);
    const qd::MoeArgs m = moe_args(w);
    const size_t eb = prefill_expert_part(m, T, k);
    float* part = (float*)((char*)workspace + eb);
    const int xkind = x_dtype == QD_F16 ? 0 : 1;
    const hipStream_t s = (hipStream_t)stream;
    hipError_t e = qd::launch_gemm8_tokens_split(router_q, router_s, router_b, (const uint16_t*)x, xkind,
                                                 part, w->E, w->H, T, s);
    if (e != hipSuccess) return from_hip(e, fn);
    e = qd::launch_route_topk_slices(part, qd::gemm8_split(w->E, w->H, T).splits, T, w->E, k, logits,
                                     idx, weights, s);
    if (e != hipSuccess) return from_hip(e, fn);
    return from_hip(qd::launch_moe_experts(m, idx, weights, T, k, x, xkind, y, workspace, eb, s), fn);
}

// Bytes of the K-split workspace of the chunk kernel (0: the shape runs unsplit).
size_t chunk_workspace_bytes(int32_t M, int32_t N, int32_t K) {
    if (M < 1 || M > 128 || N < 1 || K < 64 || K % 64 || K > (1 << 22)) return 0;
    return qd::chunk_split_workspace_bytes(M, N, K);
}

// The workspace a K-split shape needs: present, aligned and large enough.
qd_status check_split_workspace(const char* fn, size_t need, const void* workspace, size_t ws_bytes) {
    if (need == 0) return QD_OK;
    if (!workspace) return fail(QD_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
    if (!aligned16(workspace)) return fail(QD_ERR_MISALIGNED, "%s: workspace is not 16-byte aligned", fn);
    if (ws_bytes < need)
        return fail(QD_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, ws_bytes, need);
    return QD_OK;
}

size_t qgemm_affine4_chunk_workspace_bytes(int32_t M, int32_t N, int32_t K) {
    return chunk_workspace_bytes(M, N, K);
}

qd_status qgemm_affine4_chunk(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                              const uint16_t* x, float* y, int32_t M, int32_t N, int32_t K,
                              int32_t group_size, void* workspace, size_t ws_bytes,
                              qd_stream stream) {
    const char* fn = "qgemm_affine4_chunk";
    qd_status st = check_matrix(fn, N, K, group_size);
    if (st != QD_OK) return st;
    if (M < 1 || M > 128)
        return fail(QD_ERR_INVALID_ARGUMENT, "%s: M = %d must be in [1, 128]", fn, M);
    CHECK_PTR(wq);
    CHECK_PTR(scales);
    CHECK_PTR(biases);
    CHECK_PTR(x);
    CHECK_PTR(y);
    const size_t need = chunk_workspace_bytes(M, N, K);
    st = check_split_workspace(fn, need, workspace, ws_bytes);
    if (st != QD_OK) return st;
    return from_hip(qd::launch_chunk_gemm(4, wq, scales, biases, x, 1 /* bf16 */, y, M, N, K,
                                          need > 0 ? workspace : nullptr, ws_bytes,
                                          (hipStream_t)stream),
                    fn);
}

size_t qgemm_affine4_verify_workspace_bytes(int32_t M, int32_t N, int32_t K) {
    return chunk_workspace_bytes(M, N, K);
}

qd_status qgemm_affine4_verify(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                               const uint16_t* x, qd_dtype x_dtype, float* y, int32_t M, int32_t N,
                               int32_t K, int32_t group_size, void* workspace, size_t ws_bytes,
                               qd_stream stream) {
    const char* fn = "qgemm_affine4_verify";
    qd_status st = check_matrix(fn, N, K, group_size);
    if (st != QD_OK) return st;
    if (M < 1 || M > 128)
        return fail(QD_ERR_INVALID_ARGUMENT, "%s: M = %d must be in [1, 128]", fn, M);
    if (x_dtype != QD_F16 && x_dtype != QD_BF16)
        return fail(QD_ERR_UNSUPPORTED, "%s: x_dtype %d", fn, (int)x_dtype);
    CHECK_PTR(wq);
    CHECK_PTR(scales);
    CHECK_PTR(biases);
    CHECK_PTR(x);
    CHECK_PTR(y);
    const size_t need = chunk_workspace_bytes(M, N, K);
    st = check_split_workspace(fn, need, workspace, ws_bytes);
    if (st != QD_OK) return st;
    // the staged chunk kernel, whose row tiles follow M (x kinds: 0 fp16, 1 bf16);
    // K split when the shape needs a workspace
    return from_hip(qd::launch_chunk_gemm(4, wq, scales, biases, x, x_dtype == QD_F16 ? 0 : 1, y, M,
                                          N, K, need > 0 ? workspace : nullptr, ws_bytes,
                                          (hipStream_t)stream),
                    fn);
}

size_t qgemm_affine4_verify_i8_workspace_bytes(int32_t M, int32_t K) {
    if (M < 1 || M > 32 || K < 64 || K % 64 || K > (1 << 22)) return 0;
    return qd::verify_i8_workspace_bytes(M, K);
}

qd_status qgemm_affine4_verify_i8(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                                  const uint16_t* x, float* y, int32_t M, int32_t N, int32_t K,
                                  int32_t group_size, void* workspace, size_t ws_bytes,
                                  qd_stream stream) {
    const char* fn = "qgemm_affine4_verify_i8";
    qd_status st = check_matrix(fn, N, K, group_size);
    if (st != QD_OK) return st;
    if (M < 1 || M > 32)
        return fail(QD_ERR_INVALID_ARGUMENT, "%s: M = %d must be in [1, 32]", fn, M);
    CHECK_PTR(wq);
    CHECK_PTR(scales);
    CHECK_PTR(biases);
    CHECK_PTR(x);
    CHECK_PTR(y);
    const size_t need = qd::verify_i8_workspace_bytes(M, K);
    if (!workspace)
        return fail(QD_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
    if (!aligned16(workspace))
        return fail(QD_ERR_MISALIGNED, "%s: workspace is not 16-byte aligned", fn);
    if (ws_bytes < need)
        return fail(QD_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, ws_bytes, need);
    return from_hip(qd::launch_verify_i8(wq, scales, biases, x, y, M, N, K, workspace, ws_bytes,
                                         (hipStream_t)stream),
                    fn);
}

size_t qattn_decode_workspace_bytes(int32_t Hq, int32_t Hkv, int32_t D, int32_t cap) {
    if (Hq < 1 || Hkv < 1 || D < 1 || cap < 1) return 0;
    return qd::attn_workspace_bytes(Hq, Hkv, D, cap);
}

qd_status qattn_decode(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                       uint16_t* k_cache, uint16_t* v_cache, int32_t Hq, int32_t Hkv, int32_t D,
                       int32_t cap, int32_t window, int32_t pos, float scale, float* out,
                       void* workspace, size_t ws_bytes, qd_stream stream) {
    const char* fn = "qattn_decode";
    if (D != 64 && D != 128 && D != 256)
        return fail(QD_ERR_UNSUPPORTED, "%s: head dim %d (64, 128 or 256)", fn, D);
    if (Hkv < 1 || Hq < 1 || Hq % Hkv)
        return fail(QD_ERR_INVALID_ARGUMENT, "%s: Hq = %d must be a positive multiple of Hkv = %d",
                    fn, Hq, Hkv);
    const int g = Hq / Hkv;
    if (g != 1 && g != 2 && g != 4 && g != 8)
        return fail(QD_ERR_UNSUPPORTED, "%s: %d query heads per key/value head (1, 2, 4 or 8)", fn, g);
    if (cap < 1 || cap > (1 << 24))
        return fail(QD_ERR_INVALID_ARGUMENT, "%s: cap = %d must be in [1, 2^24]", fn, cap);
    if (window < 0 || (window > 0 && window != cap))
        return fail(QD_ERR_INVALID_ARGUMENT, "%s: window = %d must be 0 or equal cap = %d", fn,
                    window, cap);
    if (pos < 0 || (window == 0 && pos >= cap))
        return fail(QD_ERR_INVALID_ARGUMENT, "%s: pos = %d out of range for cap = %d", fn, pos, cap);
    if (!(scale == scale) || scale > 3e38f || scale < -3e38f)
        return fail(QD_ERR_INVALID_ARGUMENT, "%s: scale must be finite", fn);
    CHECK_PTR(q);
    CHECK_PTR(k_new);
    CHECK_PTR(v_new);
    CHECK_PTR(k_cache);
    CHECK_PTR(v_cache);
    CHECK_PTR(out);
    const size_t need = qd::attn_workspace_bytes(Hq, Hkv, D, cap);
    if (!workspace)
        return fail(QD_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
    if (!aligned16(workspace))
        return fail(QD_ERR_MISALIGNED, "%s: workspace is not 16-byte aligned", fn);
    if (ws_bytes < need)
        return fail(QD_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, ws_bytes, need);
    return from_hip(qd::launch_attn_decode(q, k_new, v_new, k_cache, v_cache, Hq, Hkv, D, cap,
                                           window, pos, scale, out, workspace, ws_bytes,
                                           (hipStream_t)stream),
                    fn);
}

qd_status qd_stream_read(const void* buf, size_t bytes, uint32_t* sink, qd_stream stream) {
    const char* fn = "qd_stream_read";
    CHECK_PTR(buf);
    CHECK_PTR(sink);
    if (bytes == 0 || bytes > ((size_t)1 << 40))
        return fail(QD_ERR_INVALID_ARGUMENT, "%s: bytes = %zu must be in [1, 2^40]", fn, bytes);
    return from_hip(qd::launch_stream_read(buf, (int64_t)bytes, sink, (hipStream_t)stream), fn);
}

const char* qd_status_string(qd_status s) {
    switch (s) {
        case QD_OK: return "QD_OK";
        case QD_ERR_INVALID_ARGUMENT: return "QD_ERR_INVALID_ARGUMENT";
        case QD_ERR_MISALIGNED: return "QD_ERR_MISALIGNED";
        case QD_ERR_UNSUPPORTED: return "QD_ERR_UNSUPPORTED";
        case QD_ERR_WORKSPACE: return "QD_ERR_WORKSPACE";
        case QD_ERR_HIP: return "QD_ERR_HIP";
    }
    return "QD_UNKNOWN_STATUS";
}

const char* qd_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
