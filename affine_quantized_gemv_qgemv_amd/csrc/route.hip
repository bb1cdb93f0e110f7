// Top-k expert routing: softmax over E logits, keep the k largest, renormalize.
//
// [TF] jeff.news/article/5193, top section and section "내부 구조가 진짜
// 흥미로운 부분" (internals): the router runs on the GPU and only its top-8
// experts are used per token. Selection compares fp32 logits exactly (equal
// logits go to the lower expert index), so expert ids and their order are
// reproducible bit for bit; the weights are exp(l_j - l_max) over the sum of
// the k kept terms, which equals softmax-then-renormalize.
//
// One 256-thread workgroup per token. The logits go to LDS as order-preserving
// integer keys (-0.0 folded into +0.0, so they tie as in the real numbers);
// each of the 4 waves ranks every candidate against a quarter of the keys,
// ties going to the lower index, and the partial ranks are summed. (key,
// index) is a strict total order, so the ranks are a permutation and the k
// candidates of rank 0..k-1 fill the k slots.
#include "common.h"
#include "launch.h"

namespace qd {

__device__ __forceinline__ uint32_t order_key(float v) {
    const uint32_t u = __float_as_uint(v + 0.0f);  // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int ROUTE_MAX_E = 1024;

// Top-k of the E logits l[0..E) (global or LDS) of one token into idx[0..k)
// and w[0..k). Threads 0..255 (four waves) rank; every thread of the
// workgroup must call (it holds barriers). keys: ROUTE_MAX_E words of LDS.
template <int PER>
__device__ __forceinline__ void rank_topk(const float* l, int E, int k, int32_t* idx, float* wout,
                                          uint32_t* keys, int (*part)[ROUTE_MAX_E], float* sel) {
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int E64 = (E + 63) & ~63;   // padded: each wave's quarter is a multiple of 16
    for (int e = threadIdx.x; e < E64; e += blockDim.x) keys[e] = e < E ? order_key(l[e]) : 0u;
    __syncthreads();
    if (wv < 4) {
        uint32_t mine[PER];
        int rank[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            mine[i] = keys[lane + 64 * i < E64 ? lane + 64 * i : 0];
            rank[i] = 0;
        }
        const int q = E64 / 4;
        for (int e0 = wv * q; e0 < (wv + 1) * q; e0 += 16) {
            uint4 kv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) kv[j] = *(const uint4*)&keys[e0 + 4 * j];  // broadcast
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t kk[4] = {kv[j].x, kv[j].y, kv[j].z, kv[j].w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int e2 = e0 + 4 * j + c;
#pragma unroll
                    for (int i = 0; i < PER; ++i)
                        rank[i] += (kk[c] > mine[i]) || (kk[c] == mine[i] && e2 < lane + 64 * i);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (lane + 64 * i < E64) part[wv][lane + 64 * i] = rank[i];
    }
    __syncthreads();
    if (wv == 0) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = lane + 64 * i;
            if (e < E) {
                const int r = part[0][e] + part[1][e] + part[2][e] + part[3][e];
                if (r < k) {
                    sel[r] = l[e];
                    idx[r] = e;
                }
            }
        }
    }
    __syncthreads();
    if (wv == 0 && lane < k) {
        const float lmax = sel[0];
        float tot = 0.f;
        for (int j = 0; j < k; ++j) tot += expf(sel[j] - lmax);
        wout[lane] = expf(sel[lane] - lmax) / tot;
    }
}

template <int PER>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int32_t* __restrict__ idx,
                                                         float* __restrict__ wout) {
    __shared__ __align__(16) uint32_t keys[ROUTE_MAX_E];
    __shared__ int part[4][ROUTE_MAX_E];
    __shared__ float sel[32];
    const int t = blockIdx.x;
    (void)T;
    rank_topk<PER>(logits + (int64_t)t * E, E, k, idx + (int64_t)t * k, wout + (int64_t)t * k, keys,
                   part, sel);
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
