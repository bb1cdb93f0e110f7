// Top-k expert selection shared by the routing kernels.
//
// [TF] jeff.news/article/5193, top section and section "내부 구조가 진짜
// 흥미로운 부분" (internals): only the router's top-8 experts are used per
// token. Selection compares fp32 logits exactly (equal logits go to the lower
// expert index), so expert ids and their order are reproducible bit for bit;
// the weights are exp(l_j - l_max) over the sum of the k kept terms, which
// equals softmax-then-renormalize. The logits become order-preserving
// integer keys in LDS (-0.0 folded into +0.0, so they tie as in the real
// numbers); each of four waves ranks every candidate against a quarter of the
// keys, ties going to the lower index, and the partial ranks are summed.
// (key, index) is a strict total order, so the ranks are a permutation and
// the k candidates of rank 0..k-1 fill the k slots.
#pragma once

#include "common.h"

namespace qd {

__device__ __forceinline__ uint32_t order_key(float v) {
    const uint32_t u = __float_as_uint(v + 0.0f);  // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int ROUTE_MAX_E = 1024;

// Top-k of the E logits l[0..E) (global or LDS) of one token into idx[0..k)
// and w[0..k) (global or LDS). Threads 0..255 (four waves) rank; every
// thread of the workgroup must call (it holds barriers). keys: MAXE words of
// LDS, part: 4 x MAXE, sel: 32; E <= MAXE, E <= 64 * PER.
template <int PER, int MAXE>
__device__ __forceinline__ void rank_topk(const float* l, int E, int k, int32_t* idx, float* wout,
                                          uint32_t* keys, int (*part)[MAXE], float* sel) {
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

// Largest / smallest value over a full wave, returned to every lane: rows of
// 16 lanes reduce through DPP (quad swaps, then half-row and row mirrors),
// the four row results through scalar registers. All 64 lanes must be active.
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, int ctrl_sel) {
    switch (ctrl_sel) {
        case 0: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
        case 1: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
        case 2: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);
        default: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);
    }
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int c = 0; c < 4; ++c) v = max(v, dpp_u32(v, c));
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return max(max(r0, r1), max(r2, r3));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
    for (int c = 0; c < 4; ++c) v = min(v, dpp_u32(v, c));
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return min(min(r0, r1), min(r2, r3));
}

// The same top-k by one wave, for callers that rank once per workgroup next
// to other work: k rounds, each taking the largest remaining key by a wave
// reduction and, only when several lanes hold it, the lowest index among
// them by a second one; about 40 instructions a round instead of E * E / 64
// comparisons. l: the E logits (E <= 64 * PER) in LDS; idx, wout: k <= 64
// entries. Only wave 0 of the workgroup may call; the caller synchronizes
// before others read idx and wout. Results equal rank_topk's: the same ids
// in the same order, and the weights from the same expression, summed in
// the same order.
template <int PER>
__device__ __forceinline__ void wave_topk(const float* l, int E, int k, int32_t* idx,
                                          float* wout) {
    const int lane = threadIdx.x & 63;
    uint32_t key[PER];
    bool alive[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        alive[i] = e < E;
        key[i] = alive[i] ? order_key(l[e]) : 0u;
    }
    float mine = 0.f;  // lane j: the j-th selected logit
    for (int j = 0; j < k; ++j) {
        // this lane's best: the largest key, the lowest index among equals
        uint32_t bk = 0u, be = 0xFFFFFFFFu;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (alive[i] && (be == 0xFFFFFFFFu || key[i] > bk)) {
                bk = key[i];
                be = (uint32_t)(lane + 64 * i);
            }
        }
        const uint32_t kmax = wave_max_u32(bk);
        const unsigned long long holders = __ballot(bk == kmax);
        uint32_t win;
        if (__popcll(holders) == 1)
            win = (uint32_t)__builtin_amdgcn_readlane((int)be, __ffsll((long long)holders) - 1);
        else
            win = wave_min_u32(bk == kmax ? be : 0xFFFFFFFFu);
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if ((uint32_t)(lane + 64 * i) == win) alive[i] = false;
        if (lane == j) {
            mine = l[win];
            idx[j] = (int32_t)win;
        }
    }
    const float lmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), 0));
    const float ex = expf(mine - lmax);
    float tot = 0.f;
    for (int j = 0; j < k; ++j)
        tot += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
    if (lane < k) wout[lane] = ex / tot;
}

}  // namespace qd
