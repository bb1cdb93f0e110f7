// MoE experts for a prefill chunk (T > 1 tokens) on MFMA, grouped by expert.
//
// [TF] jeff.news/article/5193, section "내부 구조가 진짜 흥미로운 부분"
// (internals): prefill runs in chunks of at most 128 tokens so that one fetch
// of an expert serves many rows; the shared expert's output is combined with
// the routed output. Same readings as the decode path (moe.hip): routed
// outputs weighted by the renormalized router weights, shared output with
// weight one, GELU gate, fp32 intermediates.
//
// Four launches:
//   1. prep: a counting sort of the T*k (token, slot) pairs by expert
//      (offsets, sorted pair list, each pair's position; pairs with an expert
//      id outside [0, E) are dropped), and the per-group row sums of x;
//   2. gate+up: one workgroup per (expert, 64 columns of I) computes gate and
//      up for the expert's gathered token rows on MFMA (exact codes as the
//      matrix operand, as in chunk.hip), then h' = p * GELU(gate) * up, split
//      into bf16 hi + lo (16 significant bits) for the next MFMA, plus the
//      per-group row sums of hi + lo. The shared expert is one more item with
//      all T tokens and weight one;
//   3. down: one workgroup per (expert, 128 columns of H) runs two MFMA chains
//      (hi and lo activations) against the same codes and writes each pair's
//      output row;
//   4. combine: y[t] = o_shared[t] + sum over the token's slots of its
//      (already weighted) pair rows, in slot order.
// Every expert's weights are read once per chunk; nothing uses atomics on
// the data path, so results are run-to-run deterministic.
#include "common.h"
#include "launch.h"
#include "mfma.h"

namespace qd {

typedef _Float16 halfx8_t __attribute__((ext_vector_type(8)));

struct PrefillWs {
    int* sorted_pair;   // [T*k] pair ids (t*k + j) grouped by expert
    int* pos;           // [T*k] sorted position of each pair, -1 if dropped
    int* offs;          // [E+1] first sorted position of each expert
    float* xsum;        // [T][H/64] row sums of x per group
    uint16_t* hhi;      // [T*k][I] bf16 high part of h' (sorted rows)
    uint16_t* hlo;      // [T*k][I] bf16 low part
    float* hsum;        // [T*k][I/64]
    uint16_t* shhi;     // [T][Is]
    uint16_t* shlo;     // [T][Is]
    float* shsum;       // [T][Is/64]
    float* O;           // [T*k][H] weighted routed outputs (sorted rows)
    float* Os;          // [T][H] shared-expert outputs
};

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static PrefillWs carve(void* base, const MoeArgs& m, int T, int k, size_t* total) {
    PrefillWs w{};
    char* p = (char*)base;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* r = p ? p + off : nullptr;
        off = align256(off + bytes);
        return r;
    };
    const size_t P = (size_t)T * k;
    w.sorted_pair = (int*)take(P * 4);
    w.pos = (int*)take(P * 4);
    w.offs = (int*)take(((size_t)m.E + 1) * 4);
    w.xsum = (float*)take((size_t)T * (m.H / 64) * 4);
    w.hhi = (uint16_t*)take(P * m.I * 2);
    w.hlo = (uint16_t*)take(P * m.I * 2);
    w.hsum = (float*)take(P * (m.I / 64) * 4);
    w.shhi = (uint16_t*)take((size_t)T * m.Is * 2);
    w.shlo = (uint16_t*)take((size_t)T * m.Is * 2);
    w.shsum = (float*)take((size_t)T * (m.Is / 64) * 4);
    w.O = (float*)take(P * m.H * 4);
    w.Os = (float*)take((size_t)T * m.H * 4);
    if (total) *total = off;
    return w;
}

size_t moe_prefill_workspace_bytes(const MoeArgs& m, int T, int k) {
    size_t total = 0;
    carve(nullptr, m, T, k, &total);
    return total;
}

// ---------------------------------------------------------------------------
// 1. prep
// ---------------------------------------------------------------------------
constexpr int PREP_MAX_PAIRS = 128 * 32;
constexpr int PREP_MAX_E = 1024;

__global__ __launch_bounds__(1024) void moe_prep_kernel(const int32_t* __restrict__ idx, int T,
                                                        int k, int E, const void* __restrict__ x,
                                                        int xkind, int H, PrefillWs w) {
    __shared__ int sidx[PREP_MAX_PAIRS];
    __shared__ int cnt[PREP_MAX_E + 1];
    const int P = T * k;
    const int tid = threadIdx.x, bs = blockDim.x;
    for (int i = tid; i < P; i += bs) sidx[i] = idx[i];
    for (int e = tid; e <= E; e += bs) cnt[e] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += bs) {
        const int e = sidx[p];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int e = 0; e < E; ++e) {
            const int c = cnt[e];
            cnt[e] = run;
            run += c;
        }
        cnt[E] = run;
    }
    __syncthreads();
    for (int e = tid; e <= E; e += bs) w.offs[e] = cnt[e];
    __syncthreads();  // offsets are read before the counters advance
    // placement: a slot inside the expert's range from an LDS counter. The
    // order inside an expert's rows does not change any result (every output
    // row is its own dot-product chain), only which row a pair occupies.
    for (int p = tid; p < P; p += bs) {
        const int e = sidx[p];
        if (e >= 0 && e < E) {
            const int ps = atomicAdd(&cnt[e], 1);
            w.pos[p] = ps;
            w.sorted_pair[ps] = p;
        } else {
            w.pos[p] = -1;
        }
    }
    // per-group row sums of x: one (token, group) per thread, 8 x 16-byte loads
    const int G = H / 64;
    for (int item = tid; item < T * G; item += bs) {
        const int t = item / G, g = item - t * G;
        const uint4* src = (const uint4*)((const uint16_t*)x + (int64_t)t * H + g * 64);
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint4 v = src[i];
            const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (xkind == X_F16)
                    s += h2f(wv[j] & 0xFFFF) + h2f(wv[j] >> 16);
                else
                    s += bf2f(wv[j] & 0xFFFF) + bf2f(wv[j] >> 16);
            }
        }
        w.xsum[item] = s;
    }
}

// ---------------------------------------------------------------------------
// Shared MFMA pieces: stage the group slice of up to 128 gathered rows, then
// run one 32-column block per wave over ceil(M/32) row blocks.
// ---------------------------------------------------------------------------
template <bool F16>
__device__ __forceinline__ floatx16 mfma16(const uint4& a, const uint4& b, const floatx16& c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8_t, a),
                                                      __builtin_bit_cast(halfx8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 8 codes of one word -> 16-bit (offset + q), natural k order; magic is the
// offset's bit pattern in both halves (bf16 128.0 or fp16 1024.0).
__device__ __forceinline__ uint4 codes_to_16(uint32_t w, uint32_t magic) {
    const uint32_t t = w & 0x0F0F0F0Fu;
    const uint32_t u = (w >> 4) & 0x0F0F0F0Fu;
    return make_uint4(__builtin_amdgcn_perm(u, t, 0x0C040C00u) | magic,
                      __builtin_amdgcn_perm(u, t, 0x0C050C01u) | magic,
                      __builtin_amdgcn_perm(u, t, 0x0C060C02u) | magic,
                      __builtin_amdgcn_perm(u, t, 0x0C070C03u) | magic);
}

// ---------------------------------------------------------------------------
// 2. gate+up with the GELU gate
// ---------------------------------------------------------------------------
struct GuArgs {
    const uint32_t *gu_q, *sgu_q;
    const uint16_t *gu_s, *gu_b, *sgu_s, *sgu_b;
    const uint16_t* x;   // [T][H] fp16 or bf16 bits
    const float* p;      // [T*k] routing weights in pair order
    int E, H, I, Is, k, T, act;
    PrefillWs w;
};

template <bool F16>
__global__ __launch_bounds__(256) void moe_gu_kernel(GuArgs a) {
    __shared__ __align__(16) uint4 xs_raw[2][128 * XS_STRIDE];
    __shared__ __align__(16) float xsum_raw[2][128];
    __shared__ __align__(16) float zb[128][64];
    __shared__ int tokrow[128];
    __shared__ float prow[128];
    const int ntI = a.I / 64;
    const bool shared = (int)blockIdx.x >= a.E * ntI;
    int e = 0, nt, rb, M, Iw;
    const uint32_t* Wq;
    const uint16_t *Ws, *Wb;
    if (!shared) {
        e = blockIdx.x / ntI;
        nt = blockIdx.x - e * ntI;
        rb = a.w.offs[e];
        M = a.w.offs[e + 1] - rb;
        Iw = a.I;
        const int64_t rows = 2 * (int64_t)a.I;
        Wq = a.gu_q + (int64_t)e * rows * (a.H / 8);
        Ws = a.gu_s + (int64_t)e * rows * (a.H / 64);
        Wb = a.gu_b + (int64_t)e * rows * (a.H / 64);
    } else {
        nt = blockIdx.x - a.E * ntI;
        rb = 0;
        M = a.T;
        Iw = a.Is;
        Wq = a.sgu_q;
        Ws = a.sgu_s;
        Wb = a.sgu_b;
    }
    if (M <= 0) return;  // the whole workgroup leaves together
    const int nmb = (M + 31) / 32;
    const int Mp = nmb * 32;
    const int tid = threadIdx.x;
    if (tid < 128) {
        if (tid < M) {
            const int pr = shared ? -1 : a.w.sorted_pair[rb + tid];
            tokrow[tid] = shared ? tid : pr / a.k;
            prow[tid] = shared ? 1.f : a.p[pr];
        } else {
            tokrow[tid] = 0;
            prow[tid] = 0.f;
        }
    }
    __syncthreads();

    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int G = a.H / 64;
    const int64_t wpr = a.H / 8;
    const int col = ((wave >> 1) ? Iw : 0) + 64 * nt + 32 * (wave & 1) + l32;  // row of W
    const uint32_t* wrow = Wq + (int64_t)col * wpr + 4 * h;
    const uint16_t* srow = Ws + (int64_t)col * G;
    const uint16_t* brow = Wb + (int64_t)col * G;
    const uint32_t magic = F16 ? 0x64006400u : 0x43004300u;
    const float offset = F16 ? 1024.f : 128.f;

    auto load_x = [&](int g, uint4 (&xr)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int item = tid + 256 * i;  // (row, 16-byte chunk) of the 128 x 8 tile
            const int r = item >> 3, c = item & 7;
            if (r < M)
                xr[i] = *(const uint4*)(a.x + (int64_t)tokrow[r] * a.H + (int64_t)g * 64 + 8 * c);
            else
                xr[i] = make_uint4(0, 0, 0, 0);
        }
    };
    auto store_x = [&](int buf, int g, const uint4 (&xr)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int item = tid + 256 * i;
            const int r = item >> 3, c = item & 7;
            if (r < Mp) xs_raw[buf][r * XS_STRIDE + c] = xr[i];
        }
        if (tid < Mp) xsum_raw[buf][tid] = tid < M ? a.w.xsum[(int64_t)tokrow[tid] * G + g] : 0.f;
    };

    floatx16 acc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;

    uint4 xr[4];
    load_x(0, xr);
    uint4 bw = *(const uint4*)wrow;
    uint16_t sv = srow[0], bv = brow[0];
    store_x(0, 0, xr);
    __syncthreads();
    for (int g = 0; g < G; ++g) {
        const int buf = g & 1;
        uint4 bw_next = bw;
        uint16_t sv_next = sv, bv_next = bv;
        if (g + 1 < G) {
            load_x(g + 1, xr);
            bw_next = *(const uint4*)(wrow + (int64_t)(g + 1) * 8);
            sv_next = srow[g + 1];
            bv_next = brow[g + 1];
        }
        floatx16 P[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) P[mb][i] = 0.f;
        const uint32_t wv[4] = {bw.x, bw.y, bw.z, bw.w};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const uint4 bfrag = codes_to_16(wv[st], magic);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                if (mb < nmb) {
                    const uint4 afrag = xs_raw[buf][(32 * mb + l32) * XS_STRIDE + 4 * h + st];
                    P[mb] = mfma16<F16>(afrag, bfrag, P[mb]);
                }
            }
        }
        const float sf = h2f(sv);
        const float bf = h2f(bv) - offset * sf;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            if (mb < nmb) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float4 xb = *(const float4*)(&xsum_raw[buf][32 * mb + 8 * j + 4 * h]);
                    acc[mb][4 * j + 0] = fmaf(bf, xb.x, fmaf(sf, P[mb][4 * j + 0], acc[mb][4 * j + 0]));
                    acc[mb][4 * j + 1] = fmaf(bf, xb.y, fmaf(sf, P[mb][4 * j + 1], acc[mb][4 * j + 1]));
                    acc[mb][4 * j + 2] = fmaf(bf, xb.z, fmaf(sf, P[mb][4 * j + 2], acc[mb][4 * j + 2]));
                    acc[mb][4 * j + 3] = fmaf(bf, xb.w, fmaf(sf, P[mb][4 * j + 3], acc[mb][4 * j + 3]));
                }
            }
        }
        if (g + 1 < G) store_x(buf ^ 1, g + 1, xr);
        __syncthreads();
        bw = bw_next;
        sv = sv_next;
        bv = bv_next;
    }

    // up rows (waves 2, 3) -> LDS; gate rows (waves 0, 1) combine in place
    const int c = 32 * (wave & 1) + l32;
    if (wave >= 2) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
            if (mb < nmb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    zb[32 * mb + 8 * (i / 4) + 4 * h + (i % 4)][c] = acc[mb][i];
    }
    __syncthreads();
    if (wave < 2) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
            if (mb < nmb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = 32 * mb + 8 * (i / 4) + 4 * h + (i % 4);
                    float gl;
                    const float u = acc[mb][i];
                    if (a.act == 1) {
                        const float cc = 0.7978845608028654f;
                        gl = 0.5f * u * (1.f + tanhf(cc * (u + 0.044715f * u * u * u)));
                    } else {
                        gl = 0.5f * u * (1.f + erff(u * 0.7071067811865476f));
                    }
                    zb[r][c] = r < M ? prow[r] * gl * zb[r][c] : 0.f;
                }
    }
    __syncthreads();
    // bf16 hi/lo split and per-group row sums of h'
    uint16_t* dhi = shared ? a.w.shhi : a.w.hhi;
    uint16_t* dlo = shared ? a.w.shlo : a.w.hlo;
    float* dsum = shared ? a.w.shsum : a.w.hsum;
    for (int item = tid; item < M * 16; item += 256) {
        const int r = item >> 4, c4 = (item & 15) * 4;
        uint16_t hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = zb[r][c4 + i];
            hi[i] = f2bf_rne(v);
            lo[i] = f2bf_rne(v - bf2f_bits(hi[i]));
        }
        const int64_t o = (int64_t)(rb + r) * Iw + 64 * nt + c4;
        *(uint2*)(dhi + o) = make_uint2(pack_h2(hi[0], hi[1]), pack_h2(hi[2], hi[3]));
        *(uint2*)(dlo + o) = make_uint2(pack_h2(lo[0], lo[1]), pack_h2(lo[2], lo[3]));
    }
    if (tid < M) {
        float s = 0.f;
        for (int cc = 0; cc < 64; ++cc) {
            const float v = zb[tid][cc];
            const uint16_t hi = f2bf_rne(v);
            const uint16_t lo = f2bf_rne(v - bf2f_bits(hi));
            s += bf2f_bits(hi) + bf2f_bits(lo);
        }
        dsum[(int64_t)(rb + tid) * (Iw / 64) + nt] = s;
    }
}

// ---------------------------------------------------------------------------
// 3. down
// ---------------------------------------------------------------------------
struct DnArgs {
    const uint32_t *dn_q, *sdn_q;
    const uint16_t *dn_s, *dn_b, *sdn_s, *sdn_b;
    int E, H, I, Is, T;
    PrefillWs w;
};

__global__ __launch_bounds__(256) void moe_dn_kernel(DnArgs a) {
    __shared__ __align__(16) uint4 hs_raw[2][2][128 * XS_STRIDE];   // [buf][hi, lo]
    __shared__ __align__(16) float hsum_raw[2][128];
    const int ntH = (a.H + 127) / 128;
    const bool shared = (int)blockIdx.x >= a.E * ntH;
    int e = 0, nt, rb, M, K;
    const uint32_t* Wq;
    const uint16_t *Ws, *Wb;
    const uint16_t *Ahi, *Alo;
    const float* Asum;
    float* Out;
    if (!shared) {
        e = blockIdx.x / ntH;
        nt = blockIdx.x - e * ntH;
        rb = a.w.offs[e];
        M = a.w.offs[e + 1] - rb;
        K = a.I;
        Wq = a.dn_q + (int64_t)e * a.H * (a.I / 8);
        Ws = a.dn_s + (int64_t)e * a.H * (a.I / 64);
        Wb = a.dn_b + (int64_t)e * a.H * (a.I / 64);
        Ahi = a.w.hhi;
        Alo = a.w.hlo;
        Asum = a.w.hsum;
        Out = a.w.O;
    } else {
        nt = blockIdx.x - a.E * ntH;
        rb = 0;
        M = a.T;
        K = a.Is;
        Wq = a.sdn_q;
        Ws = a.sdn_s;
        Wb = a.sdn_b;
        Ahi = a.w.shhi;
        Alo = a.w.shlo;
        Asum = a.w.shsum;
        Out = a.w.Os;
    }
    if (M <= 0) return;
    const int nmb = (M + 31) / 32;
    const int Mp = nmb * 32;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int G = K / 64;
    const int64_t wpr = K / 8;
    const int n = 128 * nt + 32 * wave + l32;
    const int nc = min(n, a.H - 1);
    const uint32_t* wrow = Wq + (int64_t)nc * wpr + 4 * h;
    const uint16_t* srow = Ws + (int64_t)nc * G;
    const uint16_t* brow = Wb + (int64_t)nc * G;

    auto load_a = [&](int g, uint4 (&ar)[2][4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int item = tid + 256 * i;
            const int r = item >> 3, c = item & 7;
            if (r < M) {
                const int64_t o = (int64_t)(rb + r) * K + (int64_t)g * 64 + 8 * c;
                ar[0][i] = *(const uint4*)(Ahi + o);
                ar[1][i] = *(const uint4*)(Alo + o);
            } else {
                ar[0][i] = make_uint4(0, 0, 0, 0);
                ar[1][i] = make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto store_a = [&](int buf, int g, const uint4 (&ar)[2][4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int item = tid + 256 * i;
            const int r = item >> 3, c = item & 7;
            if (r < Mp) {
                hs_raw[buf][0][r * XS_STRIDE + c] = ar[0][i];
                hs_raw[buf][1][r * XS_STRIDE + c] = ar[1][i];
            }
        }
        if (tid < Mp) hsum_raw[buf][tid] = tid < M ? Asum[(int64_t)(rb + tid) * G + g] : 0.f;
    };

    floatx16 acc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;

    uint4 ar[2][4];
    load_a(0, ar);
    uint4 bw = *(const uint4*)wrow;
    uint16_t sv = srow[0], bv = brow[0];
    store_a(0, 0, ar);
    __syncthreads();
    for (int g = 0; g < G; ++g) {
        const int buf = g & 1;
        uint4 bw_next = bw;
        uint16_t sv_next = sv, bv_next = bv;
        if (g + 1 < G) {
            load_a(g + 1, ar);
            bw_next = *(const uint4*)(wrow + (int64_t)(g + 1) * 8);
            sv_next = srow[g + 1];
            bv_next = brow[g + 1];
        }
        floatx16 P[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) P[mb][i] = 0.f;
        const uint32_t wv[4] = {bw.x, bw.y, bw.z, bw.w};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const uint4 bfrag = codes_to_16(wv[st], 0x43004300u);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                if (mb < nmb) {
                    const int ai = (32 * mb + l32) * XS_STRIDE + 4 * h + st;
                    P[mb] = mfma16<false>(hs_raw[buf][0][ai], bfrag, P[mb]);
                    P[mb] = mfma16<false>(hs_raw[buf][1][ai], bfrag, P[mb]);
                }
            }
        }
        const float sf = h2f(sv);
        const float bf = h2f(bv) - 128.f * sf;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            if (mb < nmb) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float4 xb = *(const float4*)(&hsum_raw[buf][32 * mb + 8 * j + 4 * h]);
                    acc[mb][4 * j + 0] = fmaf(bf, xb.x, fmaf(sf, P[mb][4 * j + 0], acc[mb][4 * j + 0]));
                    acc[mb][4 * j + 1] = fmaf(bf, xb.y, fmaf(sf, P[mb][4 * j + 1], acc[mb][4 * j + 1]));
                    acc[mb][4 * j + 2] = fmaf(bf, xb.z, fmaf(sf, P[mb][4 * j + 2], acc[mb][4 * j + 2]));
                    acc[mb][4 * j + 3] = fmaf(bf, xb.w, fmaf(sf, P[mb][4 * j + 3], acc[mb][4 * j + 3]));
                }
            }
        }
        if (g + 1 < G) store_a(buf ^ 1, g + 1, ar);
        __syncthreads();
        bw = bw_next;
        sv = sv_next;
        bv = bv_next;
    }
    if (n < a.H) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
            if (mb < nmb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = 32 * mb + 8 * (i / 4) + 4 * h + (i % 4);
                    if (r < M) Out[(int64_t)(rb + r) * a.H + n] = acc[mb][i];
                }
    }
}

// ---------------------------------------------------------------------------
// 4. combine
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void moe_combine_kernel(const PrefillWs w, int T, int k, int H,
                                                          float* __restrict__ y) {
    const int t = blockIdx.y;
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T || n >= H) return;
    float v = w.Os[(int64_t)t * H + n];
    for (int j = 0; j < k; ++j) {
        const int ps = w.pos[t * k + j];
        if (ps >= 0) v += w.O[(int64_t)ps * H + n];
    }
    y[(int64_t)t * H + n] = v;
}

hipError_t launch_moe_prefill(const MoeArgs& m, const int32_t* idx, const float* wts, int T, int k,
                              const void* x, int xkind, float* y, void* ws, hipStream_t st) {
    if (T * k > PREP_MAX_PAIRS || m.E > PREP_MAX_E || T > 128) return hipErrorInvalidValue;
    const PrefillWs w = carve(ws, m, T, k, nullptr);
    hipLaunchKernelGGL(moe_prep_kernel, dim3(1), dim3(1024), 0, st, idx, T, k, m.E, x, xkind, m.H, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    GuArgs ga{};
    ga.gu_q = m.gu_q;
    ga.sgu_q = m.sgu_q;
    ga.gu_s = m.gu_s;
    ga.gu_b = m.gu_b;
    ga.sgu_s = m.sgu_s;
    ga.sgu_b = m.sgu_b;
    ga.x = (const uint16_t*)x;
    ga.p = wts;
    ga.E = m.E;
    ga.H = m.H;
    ga.I = m.I;
    ga.Is = m.Is;
    ga.k = k;
    ga.T = T;
    ga.act = m.act;
    ga.w = w;
    const int gu_items = m.E * (m.I / 64) + m.Is / 64;
    if (xkind == X_F16)
        hipLaunchKernelGGL(moe_gu_kernel<true>, dim3(gu_items), dim3(256), 0, st, ga);
    else
        hipLaunchKernelGGL(moe_gu_kernel<false>, dim3(gu_items), dim3(256), 0, st, ga);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    DnArgs da{};
    da.dn_q = m.dn_q;
    da.sdn_q = m.sdn_q;
    da.dn_s = m.dn_s;
    da.dn_b = m.dn_b;
    da.sdn_s = m.sdn_s;
    da.sdn_b = m.sdn_b;
    da.E = m.E;
    da.H = m.H;
    da.I = m.I;
    da.Is = m.Is;
    da.T = T;
    da.w = w;
    const int ntH = (m.H + 127) / 128;
    hipLaunchKernelGGL(moe_dn_kernel, dim3(m.E * ntH + ntH), dim3(256), 0, st, da);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    hipLaunchKernelGGL(moe_combine_kernel, dim3((m.H + 255) / 256, T), dim3(256), 0, st, w, T, k,
                       m.H, y);
    return hipGetLastError();
}

}  // namespace qd
