// Top-k expert routing: softmax over E logits, keep the k largest, renormalize.
//
// [TF] jeff.news/article/5193, top section and section "내부 구조가 진짜
// 흥미로운 부분" (internals): the router runs on the GPU and only its top-8
// experts are used per token. Selection compares fp32 logits exactly (equal
// logits go to the lower expert index), so expert ids and their order are
// reproducible bit for bit; the weights are exp(l_j - l_max) over the sum of
// the k kept terms, which equals softmax-then-renormalize.
//
// One wave per token: each lane holds E/64 logits; k rounds of a wave-wide
// arg-max (value, then lowest index) pick the experts in order.
#include "common.h"
#include "launch.h"

namespace qd {

struct Cand {
    float v;
    int i;   // expert index, or INT_MAX when the lane has no live candidate
};

__device__ __forceinline__ bool better(const Cand& a, const Cand& b) {
    // a ranks before b: larger logit, then smaller index; a lane without a
    // candidate (i == INT_MAX) never wins
    if (a.i == INT_MAX) return false;
    if (b.i == INT_MAX) return true;
    return a.v > b.v || (a.v == b.v && a.i < b.i);
}

template <int PER>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int32_t* __restrict__ idx,
                                                         float* __restrict__ wout) {
    const int lane = threadIdx.x & 63;
    const int t = (int)((blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6);
    if (t >= T) return;  // uniform per wave
    const float* l = logits + (int64_t)t * E;
    float v[PER];
    bool live[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        live[i] = e < E;
        v[i] = live[i] ? l[e] : 0.f;
    }
    int my_idx = 0;
    float my_val = 0.f;
    for (int j = 0; j < k; ++j) {
        Cand c{0.f, INT_MAX};
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const Cand o{v[i], live[i] ? lane + 64 * i : INT_MAX};
            if (better(o, c)) c = o;
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            Cand o;
            o.v = __shfl_xor(c.v, m, 64);
            o.i = __shfl_xor(c.i, m, 64);
            if (better(o, c)) c = o;
        }
        // c is now the same winner in every lane
        if (c.i != INT_MAX) {
#pragma unroll
            for (int i = 0; i < PER; ++i)
                if (lane + 64 * i == c.i) live[i] = false;
        }
        if (lane == j) {
            my_idx = c.i;
            my_val = c.v;
        }
    }
    const float lmax = __shfl(my_val, 0, 64);
    const float e = lane < k ? expf(my_val - lmax) : 0.f;
    float tot = e;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) tot += __shfl_xor(tot, m, 64);
    if (lane < k) {
        idx[(int64_t)t * k + lane] = my_idx;
        wout[(int64_t)t * k + lane] = e / tot;
    }
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                             hipStream_t st) {
    const int threads = 256;
    const int blocks = (int)(((int64_t)T * 64 + threads - 1) / threads);
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
