// Top-k expert routing: softmax over E logits, keep the k largest, renormalize.
//
// [TF] jeff.news/article/5193, top section and section "내부 구조가 진짜
// 흥미로운 부분" (internals): the router runs on the GPU and only its top-8
// experts are used per token. Selection compares fp32 logits exactly (equal
// logits go to the lower expert index), so expert ids and their order are
// reproducible bit for bit; the weights are exp(l_j - l_max) over the sum of
// the k kept terms, which equals softmax-then-renormalize.
//
// One wave per token. The logits go to LDS as order-preserving integer keys
// (-0.0 folded into +0.0, so they tie as in the real numbers); every lane
// then ranks its candidates against all E keys, ties going to the lower
// index. (key, index) is a strict total order, so the ranks are a
// permutation and the k lanes holding ranks 0..k-1 write the k slots.
#include "common.h"
#include "launch.h"

namespace qd {

__device__ __forceinline__ uint32_t order_key(float v) {
    const uint32_t u = __float_as_uint(v + 0.0f);  // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int ROUTE_MAX_E = 1024;

template <int PER>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int32_t* __restrict__ idx,
                                                         float* __restrict__ wout) {
    __shared__ __align__(16) uint32_t keys[4][ROUTE_MAX_E];
    __shared__ float sel[4][32];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wv;
    const bool live = t < T;
    const float* l = logits + (int64_t)(live ? t : 0) * E;
    float v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        v[i] = (live && e < E) ? l[e] : 0.f;
        if (e < E) keys[wv][e] = order_key(v[i]);
    }
    __syncthreads();
    int rank[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) rank[i] = 0;
    uint32_t mine[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) mine[i] = order_key(v[i]);
    // 16 keys per iteration, read as four 16-byte broadcasts issued together
    const int E16 = (E + 15) & ~15;
    for (int e2 = E; e2 < E16; ++e2)
        if (lane == 0) keys[wv][e2] = 0u;  // below every real key: never outranks
    __syncthreads();
    for (int e0 = 0; e0 < E16; e0 += 16) {
        uint4 kv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) kv[q] = *(const uint4*)&keys[wv][e0 + 4 * q];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t kk[4] = {kv[q].x, kv[q].y, kv[q].z, kv[q].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int e2 = e0 + 4 * q + c;
#pragma unroll
                for (int i = 0; i < PER; ++i) {
                    const int e = lane + 64 * i;
                    rank[i] += (kk[c] > mine[i]) || (kk[c] == mine[i] && e2 < e);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        if (e < E && rank[i] < k) {
            sel[wv][rank[i]] = v[i];
            if (live) idx[(int64_t)t * k + rank[i]] = e;
        }
    }
    __syncthreads();
    if (live && lane < k) {
        const float lmax = sel[wv][0];
        float tot = 0.f;
        for (int j = 0; j < k; ++j) tot += expf(sel[wv][j] - lmax);
        wout[(int64_t)t * k + lane] = expf(sel[wv][lane] - lmax) / tot;
    }
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                             hipStream_t st) {
    const int threads = 256;
    const int blocks = (T + 3) / 4;
    if (E <= 64)
        hipLaunchKernelGGL(route_topk_kernel<1>, dim3(blocks), dim3(threads), 0, st, logits, T, E, k,
                           idx, w);
    else if (E <= 128)
        hipLaunchKernelGGL(route_topk_kernel<2>, dim3(blocks), dim3(threads), 0, st, logits, T, E, k,
                           idx, w);
    else if (E <= 256)
        hipLaunchKernelGGL(route_topk_kernel<4>, dim3(blocks), dim3(threads), 0, st, logits, T, E, k,
                           idx, w);
    else
        hipLaunchKernelGGL(route_topk_kernel<16>, dim3(blocks), dim3(threads), 0, st, logits, T, E,
                           k, idx, w);
    return hipGetLastError();
}

}  // namespace qd
