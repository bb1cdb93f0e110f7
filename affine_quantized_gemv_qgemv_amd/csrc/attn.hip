// Decode attention for one new token over an fp16 KV cache, split along the
// cached positions and merged exactly.
//
// [TF] jeff.news/article/5193, section "내부 구조가 진짜 흥미로운 부분"
// (internals): sliding-window layers keep keys and values in bounded
// circular storage, full-attention layers in linear storage, and decode
// attention is computed exactly with the key and value paths split. Here:
//  * storage: k/v caches [Hkv][cap][D] fp16; the token at position pos lives
//    at slot pos mod window (circular, cap == window) or at slot pos
//    (linear, window == 0); the occupied slots [0, n), n = min(pos + 1,
//    window) or pos + 1, are exactly the positions inside the window, and
//    attention over a set of positions does not depend on their order;
//  * the step stores the new key and value at its slot (the workgroup whose
//    range holds the slot reads them from the inputs and writes them back,
//    so no other workgroup touches that row);
//  * split pass: workgroup (s, hk) takes slots [s C, (s + 1) C) of key/value
//    head hk for all G = Hq / Hkv query heads that share it, so each cached
//    row is read once. A row spans D / 8 lanes (one 16-byte load each);
//    every lane keeps an online softmax (running max, sum and weighted value
//    sum over its 8 dims) for its rows, and the workgroup merges them into
//    one partial (m, l, o[D]) per query head;
//  * combine pass: per query head, m = max m_s, L = sum_s l_s e^(m_s - m),
//    out = sum_s o_s e^(m_s - m) / L, over the splits in order, so results
//    do not depend on timing.
// Both passes read HBM once per cached byte; the arithmetic is fp32.
#include "common.h"
#include "launch.h"

namespace qd {

constexpr int AT_THREADS = 256;
constexpr int AT_U = 2;   // row steps whose loads are issued together
constexpr int AT_MAXSPLIT = 256;

struct AttnArgs {
    const uint16_t *q, *k_new, *v_new;
    uint16_t *kc, *vc;
    float* part;   // [nsplit][Hq][D + 2]: o[D], m, l
    float* out;    // [Hq][D]
    int Hq, Hkv, D, cap, n, slot, chunk, nsplit;
    float scale;
};

__device__ __forceinline__ void f16x8(const uint4 v, float (&o)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = h2f(w[i] & 0xFFFF);
        o[2 * i + 1] = h2f(w[i] >> 16);
    }
}

template <int D, int G>
__global__ __launch_bounds__(AT_THREADS) void attn_split_kernel(AttnArgs a) {
    constexpr int LPR = D / 8;             // lanes per row
    constexpr int RPW = 64 / LPR;          // rows per wave step
    constexpr int NW = AT_THREADS / 64;
    constexpr int RPS = NW * RPW;          // rows per workgroup step
    __shared__ float red[NW][RPW][G][2];    // per wave and row group: m, l
    __shared__ float ored[NW][G][D];
    const int s = blockIdx.x, hk = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rg = lane / LPR, dl = lane % LPR;   // row group, 8-dim slice
    const int j0 = s * a.chunk, j1 = min(j0 + a.chunk, a.n);
    const int64_t head_off = (int64_t)hk * a.cap * D;

    float qf[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        f16x8(*(const uint4*)(a.q + (int64_t)(hk * G + h) * D + 8 * dl), qf[h]);
#pragma unroll
        for (int i = 0; i < 8; ++i) qf[h][i] *= a.scale;
    }
    float m[G], l[G], o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[h][i] = 0.f;
    }

    for (int jb = j0; jb < j1; jb += RPS * AT_U) {
        uint4 kr[AT_U], vr[AT_U];
#pragma unroll
        for (int u = 0; u < AT_U; ++u) {   // clamped rows; used only if j < j1
            const int j = min(jb + u * RPS + wave * RPW + rg, j1 - 1);
            const uint16_t* kp = j == a.slot ? a.k_new + (int64_t)hk * D : a.kc + head_off + (int64_t)j * D;
            const uint16_t* vp = j == a.slot ? a.v_new + (int64_t)hk * D : a.vc + head_off + (int64_t)j * D;
            kr[u] = *(const uint4*)(kp + 8 * dl);
            vr[u] = *(const uint4*)(vp + 8 * dl);
        }
#pragma unroll
        for (int u = 0; u < AT_U; ++u) {
            const int j = jb + u * RPS + wave * RPW + rg;
            float kf[8], vf[8];
            f16x8(kr[u], kf);
            f16x8(vr[u], vf);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float sc = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) sc = fmaf(qf[h][i], kf[i], sc);
                sc = seg_sum<LPR>(sc);           // the row's score, in all its lanes
                if (j < j1) {                    // uniform across the row's lanes
                    const float mn = fmaxf(m[h], sc);
                    const float c = expf(m[h] - mn);   // 0 on the first row (m = -inf)
                    const float p = expf(sc - mn);
                    l[h] = fmaf(l[h], c, p);
#pragma unroll
                    for (int i = 0; i < 8; ++i) o[h][i] = fmaf(o[h][i], c, p * vf[i]);
                    m[h] = mn;
                }
            }
        }
    }

    // merge the row groups of each wave, then the waves (fixed order)
    if (dl == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            red[wave][rg][h][0] = m[h];
            red[wave][rg][h][1] = l[h];
        }
    }
    __syncthreads();
    float mw[G];   // the workgroup's max per head
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float mm = -INFINITY;
        for (int w = 0; w < NW; ++w)
            for (int r = 0; r < RPW; ++r) mm = fmaxf(mm, red[w][r][h][0]);
        mw[h] = mm;
    }
    // rescale this lane's sums to the workgroup max (rows never seen: m = -inf, weight 0)
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float c = m[h] == -INFINITY ? 0.f : expf(m[h] - mw[h]);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[h][i] *= c;
    }
    // sum over the row groups of the wave (lanes dl, dl + LPR, ...)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if constexpr (LPR <= 8) o[h][i] = xor_add<8>(o[h][i]);
            if constexpr (LPR <= 16) o[h][i] = xor_add<16>(o[h][i]);
            o[h][i] = xor_add<32>(o[h][i]);
        }
    if (rg == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int i = 0; i < 8; ++i) ored[wave][h][8 * dl + i] = o[h][i];
    }
    __syncthreads();
    for (int t = threadIdx.x; t < G * (D + 2); t += AT_THREADS) {
        const int h = t / (D + 2), e = t - h * (D + 2);
        float v;
        if (e < D) {
            v = 0.f;
            for (int w = 0; w < NW; ++w) v += ored[w][h][e];
        } else if (e == D) {
            v = mw[h];
        } else {
            v = 0.f;
            for (int w = 0; w < NW; ++w)
                for (int r = 0; r < RPW; ++r) {
                    const float mr = red[w][r][h][0];
                    if (mr != -INFINITY) v += red[w][r][h][1] * expf(mr - mw[h]);
                }
        }
        a.part[((int64_t)s * a.Hq + hk * G + h) * (D + 2) + e] = v;
    }
    // the new token's row: written by the one workgroup whose range holds it
    if (a.slot >= j0 && a.slot < j1 && threadIdx.x < 2 * LPR) {
        const int which = threadIdx.x / LPR, d8 = threadIdx.x % LPR;
        const uint16_t* src = (which ? a.v_new : a.k_new) + (int64_t)hk * D + 8 * d8;
        uint16_t* dst = (which ? a.vc : a.kc) + head_off + (int64_t)a.slot * D + 8 * d8;
        *(uint4*)dst = *(const uint4*)src;
    }
}

template <int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(AttnArgs a) {
    constexpr int NW = D / 64;
    __shared__ float ms[AT_MAXSPLIT], ls[AT_MAXSPLIT], cs[AT_MAXSPLIT];
    __shared__ float wred[NW], wsum[NW];
    const int h = blockIdx.x, d = threadIdx.x;
    const int lane = d & 63, wave = d >> 6;
    const float* p = a.part + (int64_t)h * (D + 2);
    const int64_t stride = (int64_t)a.Hq * (D + 2);
    // m = max over the splits: strided loads, then a wave reduction and the
    // NW wave maxima
    float lm = -INFINITY;
    for (int s = d; s < a.nsplit; s += D) {
        const float m = p[s * stride + D];
        ms[s] = m;
        ls[s] = p[s * stride + D + 1];
        lm = fmaxf(lm, m);
    }
    lm = wave_max_f(lm);
    if (lane == 0) wred[wave] = lm;
    __syncthreads();
    float M = wred[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, wred[w]);
    // weights e^(m_s - m) and L = sum_s l_s e^(m_s - m), reduced in a fixed
    // tree (each thread its own splits, then the wave, then the waves in order)
    float lp = 0.f;
    for (int s = d; s < a.nsplit; s += D) {
        const float c = ms[s] == -INFINITY ? 0.f : expf(ms[s] - M);
        cs[s] = c;
        lp = fmaf(ls[s], c, lp);
    }
    lp = seg_sum<64>(lp);
    if (lane == 0) wsum[wave] = lp;
    __syncthreads();
    float L = wsum[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) L += wsum[w];
    // o over the splits in order; each batch of 32 loads is issued before
    // any is used (clamped indices, weight 0 past the end), so a combine
    // costs about one memory latency per 32 splits
    float O = 0.f;
    for (int s0 = 0; s0 < a.nsplit; s0 += 32) {
        float v[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = p[min(s0 + i, a.nsplit - 1) * stride + d];
#pragma unroll
        for (int i = 0; i < 32; ++i) O = fmaf(v[i], s0 + i < a.nsplit ? cs[s0 + i] : 0.f, O);
    }
    a.out[(int64_t)h * D + d] = O / L;
}

// Splits for n occupied slots: about two workgroups per CU over all heads,
// each at least one load round of rows (a multiple of 32: two row steps of
// 16), which also keeps a short cache's combine to one batch of 32 splits.
static int attn_split_want(int n, int Hkv) {
    const int cus = device_info().cus;
    const int want = std::max(1, (2 * cus + Hkv - 1) / Hkv);
    return std::max(1, std::min(std::min(want, AT_MAXSPLIT), (n + 31) / 32));
}

static void attn_split(int n, int Hkv, int& nsplit, int& chunk) {
    const int want = attn_split_want(n, Hkv);
    chunk = (n + want - 1) / want;
    chunk = (chunk + 31) & ~31;
    nsplit = (n + chunk - 1) / chunk;
}

// Workspace for every occupancy n <= cap. The split count of n is
// ceil(n / chunk) with chunk >= ceil(n / want(n)), so it never exceeds
// want(n) <= want(cap); it is not monotonic in n (the chunk is rounded up
// to 32 rows), so the size comes from that bound, not from nsplit(cap).
static size_t attn_part_bytes(int nsplit, int Hq, int D) {
    return (size_t)nsplit * Hq * (D + 2) * sizeof(float);
}

size_t attn_workspace_bytes(int Hq, int Hkv, int D, int cap) {
    return attn_part_bytes(attn_split_want(cap, Hkv), Hq, D);
}

template <int D>
static hipError_t attn_launch_d(const AttnArgs& a, int G, hipStream_t st) {
    const dim3 grid(a.nsplit, a.Hkv);
    void (*kern)(AttnArgs);
    switch (G) {
        case 1: kern = attn_split_kernel<D, 1>; break;
        case 2: kern = attn_split_kernel<D, 2>; break;
        case 4: kern = attn_split_kernel<D, 4>; break;
        case 8: kern = attn_split_kernel<D, 8>; break;
        default: return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL(kern, grid, dim3(AT_THREADS), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_combine_kernel<D>, dim3(a.Hq), dim3(D), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_attn_decode(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                              uint16_t* kc, uint16_t* vc, int Hq, int Hkv, int D, int cap,
                              int window, int pos, float scale, float* out, void* ws,
                              size_t ws_bytes, hipStream_t st) {
    AttnArgs a{};
    a.q = q;
    a.k_new = k_new;
    a.v_new = v_new;
    a.kc = kc;
    a.vc = vc;
    a.part = (float*)ws;
    a.out = out;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.D = D;
    a.cap = cap;
    a.n = window > 0 ? std::min(pos + 1, window) : pos + 1;
    a.slot = window > 0 ? pos % window : pos;
    a.scale = scale;
    attn_split(a.n, Hkv, a.nsplit, a.chunk);
    // the split partials must fit the caller's workspace (they always do
    // when it holds attn_workspace_bytes(cap); checked before any launch)
    if (attn_part_bytes(a.nsplit, Hq, D) > ws_bytes) return hipErrorInvalidValue;
    const int G = Hq / Hkv;
    if (D == 64) return attn_launch_d<64>(a, G, st);
    if (D == 128) return attn_launch_d<128>(a, G, st);
    if (D == 256) return attn_launch_d<256>(a, G, st);
    return hipErrorInvalidValue;
}

}  // namespace qd
