// 4-bit affine GEMM for a few dozen tokens on the matrix core:
//     Y[t][n] = sum_k w[n][k] x[t][k],   w = s[n][g] q[n][k] + b[n][g],
// 4-bit codes q, 8 per uint32 along K (lowest nibble first), group 64.
//
// discuss.pytorch.kr/t/uzu-mac-iphone-llm-apple-silicon-rust/12363 (uzu),
// section "추측 디코딩 구조" (speculative decoding): a draft proposes 16 to 32
// tokens at a time and the target model checks them in one forward pass,
// which turns its projections into small GEMMs over the drafted tokens. This
// is that regime: more tokens than the GEMV kernels serve (at most 8) and far
// fewer than a prefill chunk (128), still bound by the weight stream.
//
// The matrix-core operand is the exact code: a nibble placed in the low
// mantissa of fp16 1024.0 (0x6400) or bf16 128.0 (0x4300) gives 1024 + q or
// 128 + q exactly. Per group, one v_mfma_f32_32x32x16 chain over the four
// K = 16 steps yields P = sum_k x (off + q) and a second chain against an
// all-ones operand yields the group's activation sums X in the accumulator
// layout, so in fp32
//     acc += s P + (b - off s) X,   off = 1024 (fp16) or 128 (bf16).
//
// Tiling: a workgroup owns 32 tokens x 32 NCB outputs and 8 waves that take
// alternate groups of K (wave w: groups w, w + 8, ...), each loading two of
// its groups (activations, codes, scales, biases) before using them. The
// activations come straight from memory (they stay in L2: every workgroup
// reads the same rows); each wave's ones-chain serves its NCB column blocks.
// The 8 partial sums are added in LDS in a fixed order, so results do not
// depend on timing.
#include "common.h"
#include "launch.h"
#include "mfma.h"

namespace qd {

typedef _Float16 f16x8_t4 __attribute__((ext_vector_type(8)));

struct G4Args {
    const uint32_t* wq;   // [N][K/8]
    const uint16_t* s;    // [N][K/64] f16
    const uint16_t* b;    // [N][K/64] f16
    const uint16_t* x;    // [T][K] f16 or bf16
    float* y;             // [T][N]
    int T, N, K;
};

constexpr int G4_WAVES = 8;
constexpr int G4_SLOTS = 2;   // groups loaded together per wave

// 8 codes of one word -> 16-bit (off + q) values in natural k order; hi is
// the operand's high byte (0x64: fp16 1024, 0x43: bf16 128).
__device__ __forceinline__ uint4 codes_to_16(uint32_t w, uint32_t hi2) {
    const uint32_t t = w & 0x0F0F0F0Fu;         // q0 q2 q4 q6 in bytes 0..3
    const uint32_t u = (w >> 4) & 0x0F0F0F0Fu;  // q1 q3 q5 q7
    // v_perm_b32(u, t, sel): selector bytes 0..3 pick t's bytes, 4..7 u's, 0x0C gives 0
    return make_uint4(__builtin_amdgcn_perm(u, t, 0x0C040C00u) | hi2,
                      __builtin_amdgcn_perm(u, t, 0x0C050C01u) | hi2,
                      __builtin_amdgcn_perm(u, t, 0x0C060C02u) | hi2,
                      __builtin_amdgcn_perm(u, t, 0x0C070C03u) | hi2);
}

template <int XF>
__device__ __forceinline__ floatx16 mfma16(uint4 a, uint4 b, floatx16 c) {
    if constexpr (XF == 0)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t4, a),
                                                      __builtin_bit_cast(f16x8_t4, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <int XF, int NCB>   // XF 0: f16 activations, 1: bf16; NCB column blocks of 32
__global__ __launch_bounds__(64 * G4_WAVES) void gemm4_tokens_kernel(G4Args a) {
    __shared__ float red[G4_WAVES - 1][NCB][16][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int t = blockIdx.y * 32 + l32;     // A-operand row (token) of this lane
    const int G = a.K / 64;
    const int tc = min(t, a.T - 1);
    // step st of a group: this lane's k = 32h + 8st + (0..7), i.e. code word 4h + st
    const uint16_t* xrow = a.x + (int64_t)tc * a.K + 32 * h;
    const uint32_t* wrow[NCB];
    const uint16_t *srow[NCB], *brow[NCB];
    int ncol[NCB];
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
        ncol[c] = blockIdx.x * 32 * NCB + 32 * c + l32;   // B-operand column / output column
        const int nc = min(ncol[c], a.N - 1);
        wrow[c] = a.wq + (int64_t)nc * (a.K / 8) + 4 * h;
        srow[c] = a.s + (int64_t)nc * G;
        brow[c] = a.b + (int64_t)nc * G;
    }
    const uint32_t hi2 = in_vgpr(XF == 0 ? 0x64006400u : 0x43004300u);
    const uint32_t one2 = XF == 0 ? 0x3C003C00u : 0x3F803F80u;   // (1.0, 1.0)
    const float off = XF == 0 ? 1024.f : 128.f;

    floatx16 acc[NCB];
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;

    for (int g0 = wave; g0 < G; g0 += G4_WAVES * G4_SLOTS) {
        uint4 xa[G4_SLOTS][4], wb[G4_SLOTS][NCB];
        uint16_t sv[G4_SLOTS][NCB], bv[G4_SLOTS][NCB];
#pragma unroll
        for (int j = 0; j < G4_SLOTS; ++j) {   // clamped loads, used only if g < G
            const int g = min(g0 + G4_WAVES * j, G - 1);
            const uint4* xp = (const uint4*)(xrow + (int64_t)g * 64);
#pragma unroll
            for (int st = 0; st < 4; ++st) xa[j][st] = xp[st];
#pragma unroll
            for (int c = 0; c < NCB; ++c) {
                wb[j][c] = *(const uint4*)(wrow[c] + (int64_t)g * 8);
                sv[j][c] = srow[c][g];
                bv[j][c] = brow[c][g];
            }
        }
#pragma unroll
        for (int j = 0; j < G4_SLOTS; ++j) {
            if (g0 + G4_WAVES * j >= G) break;   // uniform
            floatx16 X1;
#pragma unroll
            for (int i = 0; i < 16; ++i) X1[i] = 0.f;
            const uint4 ones = make_uint4(one2, one2, one2, one2);
#pragma unroll
            for (int st = 0; st < 4; ++st) X1 = mfma16<XF>(xa[j][st], ones, X1);
#pragma unroll
            for (int c = 0; c < NCB; ++c) {
                const uint32_t wv[4] = {wb[j][c].x, wb[j][c].y, wb[j][c].z, wb[j][c].w};
                floatx16 P;
#pragma unroll
                for (int i = 0; i < 16; ++i) P[i] = 0.f;
#pragma unroll
                for (int st = 0; st < 4; ++st) P = mfma16<XF>(xa[j][st], codes_to_16(wv[st], hi2), P);
                const float sf = h2f(sv[j][c]);
                const float bf = h2f(bv[j][c]) - off * sf;
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[c][i] = fmaf(bf, X1[i], fmaf(sf, P[i], acc[c][i]));
                __builtin_amdgcn_sched_barrier(0);   // one column block's chain at a time
            }
        }
    }

    // fixed-order sum of the 8 waves' partial results
    if (wave > 0) {
#pragma unroll
        for (int c = 0; c < NCB; ++c)
#pragma unroll
            for (int i = 0; i < 16; ++i) red[wave - 1][c][i][lane] = acc[c][i];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < G4_WAVES - 1; ++w) {
#pragma unroll
        for (int c = 0; c < NCB; ++c)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[c][i] += red[w][c][i][lane];
        __builtin_amdgcn_sched_barrier(0);   // a bounded number of LDS reads in flight
    }
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
        if (ncol[c] >= a.N) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int tt = blockIdx.y * 32 + 8 * (i / 4) + 4 * h + (i % 4);
            if (tt < a.T) a.y[(int64_t)tt * a.N + ncol[c]] = acc[c][i];
        }
    }
}

#ifdef QD_TUNING
extern "C" int qd_tune_gemm4 = 0;
#endif

hipError_t launch_gemm4_tokens(const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                               const uint16_t* x, int xkind, float* y, int N, int K, int T,
                               hipStream_t st) {
    if (K % 64 != 0 || (xkind != X_F16 && xkind != X_BF16)) return hipErrorInvalidValue;
    G4Args a{wq, s, b, x, y, T, N, K};
    int ncb = 1;
#ifdef QD_TUNING
    if (qd_tune_gemm4) ncb = qd_tune_gemm4;
#endif
    const dim3 grid((N + 32 * ncb - 1) / (32 * ncb), (T + 31) / 32);
    const dim3 block(64 * G4_WAVES);
    void (*kern)(G4Args);
    if (ncb == 2)
        kern = xkind == X_F16 ? gemm4_tokens_kernel<0, 2> : gemm4_tokens_kernel<1, 2>;
    else
        kern = xkind == X_F16 ? gemm4_tokens_kernel<0, 1> : gemm4_tokens_kernel<1, 1>;
    hipLaunchKernelGGL(kern, grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace qd
