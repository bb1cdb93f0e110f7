// Top-k expert routing: softmax over E logits, keep the k largest, renormalize.
//
// [TF] jeff.news/article/5193, top section and section "내부 구조가 진짜
// 흥미로운 부분" (internals): the router runs on the GPU and only its top-8
// experts are used per token. One 256-thread workgroup per token runs the
// ranking of route.h (exact comparison of fp32 logits, ties to the lower
// expert index, weights renormalized over the k kept).
#include "common.h"
#include "launch.h"
#include "route.h"

namespace qd {

template <int PER>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int32_t* __restrict__ idx,
                                                         float* __restrict__ wout) {
    __shared__ __align__(16) uint32_t keys[ROUTE_MAX_E];
    __shared__ int part[4][ROUTE_MAX_E];
    __shared__ float sel[32];
    const int t = blockIdx.x;
    (void)T;
    rank_topk<PER, ROUTE_MAX_E>(logits + (int64_t)t * E, E, k, idx + (int64_t)t * k,
                                wout + (int64_t)t * k, keys, part, sel);
}

// The router's K-split slices part [splits][T][E] added in split order (into
// LDS, and written out as the logits), then ranked as above.
template <int PER>
__global__ __launch_bounds__(256) void route_topk_slices_kernel(const float* __restrict__ part,
                                                                int splits, int T, int E, int k,
                                                                float* __restrict__ logits,
                                                                int32_t* __restrict__ idx,
                                                                float* __restrict__ wout) {
    __shared__ __align__(16) uint32_t keys[ROUTE_MAX_E];
    __shared__ int prt[4][ROUTE_MAX_E];
    __shared__ float sel[32];
    __shared__ float lsum[ROUTE_MAX_E];
    const int t = blockIdx.x;
    const int64_t tn = (int64_t)T * E;
    for (int e = threadIdx.x; e < E; e += 256) {
        const int64_t o = (int64_t)t * E + e;
        float v = part[o];
        for (int sp = 1; sp < splits; ++sp) v += part[sp * tn + o];
        lsum[e] = v;
        logits[o] = v;
    }
    __syncthreads();
    rank_topk<PER, ROUTE_MAX_E>(lsum, E, k, idx + (int64_t)t * k, wout + (int64_t)t * k, keys, prt,
                                sel);
}

hipError_t launch_route_topk_slices(const float* part, int splits, int T, int E, int k,
                                    float* logits, int32_t* idx, float* w, hipStream_t st) {
    const dim3 grid(T), block(256);
    if (E <= 64)
        hipLaunchKernelGGL(route_topk_slices_kernel<1>, grid, block, 0, st, part, splits, T, E, k,
                           logits, idx, w);
    else if (E <= 128)
        hipLaunchKernelGGL(route_topk_slices_kernel<2>, grid, block, 0, st, part, splits, T, E, k,
                           logits, idx, w);
    else if (E <= 256)
        hipLaunchKernelGGL(route_topk_slices_kernel<4>, grid, block, 0, st, part, splits, T, E, k,
                           logits, idx, w);
    else
        hipLaunchKernelGGL(route_topk_slices_kernel<16>, grid, block, 0, st, part, splits, T, E, k,
                           logits, idx, w);
    return hipGetLastError();
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                             hipStream_t st) {
    const int threads = 256;
    const int blocks = T;
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
