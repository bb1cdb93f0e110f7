// 8-bit affine GEMV over a chunk of tokens on the matrix core:
//     Y[t][n] = sum_k w[n][k] x[t][k],   w = s[n][g] q[n][k] + b[n][g],
// 8-bit codes q, 4 per uint32 along K (lowest byte first), group 64.
//
// [TF] jeff.news/article/5193, top section and section "내부 구조가 진짜
// 흥미로운 부분" (internals): the MoE router scores every token against
// every expert; during prefill a whole chunk of up to 128 tokens goes through
// the router at once, so the router product is a small GEMM (tokens x
// experts x hidden) rather than a GEMV. The 8-bit router format is the
// affine format of the decode path with 8-bit codes.
//
// The matrix-core operand is the exact code. For f16 activations a code byte
// placed in the low mantissa of f16 1024.0 (0x6400) gives 1024 + q exactly,
// and one v_mfma_f32_32x32x16_f16 per 16 inputs yields
//     P = sum_k x (1024 + q).
// bf16 has too few mantissa bits for 1024 + q, so for bf16 activations the
// code is split into nibbles, each exact as 128 + nibble (0x4300), and two
// bf16 MFMAs yield P_lo + 16 P_hi = sum_k x q + 2176 Xsum. A third MFMA
// against an all-ones operand gives the row sums Xsum directly in the
// accumulator layout. Per group, in fp32:
//     acc += s P' + (b - off s) Xsum,   off = 1024 (f16) or 2176 (bf16).
//
// Tiling: a workgroup owns 32 tokens x 32 outputs and has 8 waves that take
// alternate groups of K (wave w: groups w, w + 8, ...), each loading up to
// four of its groups at once before using them; the 8 partial sums are added
// in LDS in a fixed order, so results do not depend on timing.
#include "common.h"
#include "launch.h"
#include "mfma.h"

namespace qd {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

struct G8Args {
    const uint32_t* wq;   // [N][K/4]
    const uint16_t* s;    // [N][K/64] f16
    const uint16_t* b;    // [N][K/64] f16
    const uint16_t* x;    // [T][K] f16 or bf16
    float* y;             // [T][N]
    int T, N, K;
};

constexpr int G8_WAVES = 8;
constexpr int G8_SLOTS = 4;   // groups loaded together per wave

// Two code bytes of w (bytes j, j + 1) beside magic bytes m:
// dword = [w.b(j), m, w.b(j+1), m].
__device__ __forceinline__ uint32_t byte_pair(uint32_t w, uint32_t m, uint32_t sel) {
    // v_perm_b32(src0 = m, src1 = w, sel): selector 0..3 picks w's bytes, 4..7 m's
    return __builtin_amdgcn_perm(m, w, sel);
}

template <int XF>   // 0: f16 activations, 1: bf16 activations
__global__ __launch_bounds__(64 * G8_WAVES) void gemm8_tokens_kernel(G8Args a) {
    __shared__ float red[G8_WAVES - 1][16][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int n = blockIdx.x * 32 + l32;   // B-operand column and output column of this lane
    const int t = blockIdx.y * 32 + l32;   // A-operand row of this lane
    const int G = a.K / 64;
    const int nc = min(n, a.N - 1), tc = min(t, a.T - 1);
    const uint32_t* wrow = a.wq + (int64_t)nc * (a.K / 4) + 8 * h;   // words 8h..8h+7 of group 0
    const uint16_t* xrow = a.x + (int64_t)tc * a.K + 32 * h;          // k = 32h.. of group 0
    const uint16_t* srow = a.s + (int64_t)nc * G;
    const uint16_t* brow = a.b + (int64_t)nc * G;
    const uint32_t magic = in_vgpr(XF == 0 ? 0x64646464u : 0x43434343u);
    const uint32_t one2 = XF == 0 ? 0x3C003C00u : 0x3F803F80u;   // (1.0, 1.0)

    floatx16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;

    for (int g0 = wave; g0 < G; g0 += G8_WAVES * G8_SLOTS) {
        uint4 xa[G8_SLOTS][4], wb[G8_SLOTS][2];
        uint16_t sv[G8_SLOTS], bv[G8_SLOTS];
#pragma unroll
        for (int j = 0; j < G8_SLOTS; ++j) {   // clamped loads, used only if g < G
            const int g = min(g0 + G8_WAVES * j, G - 1);
            const uint4* xp = (const uint4*)(xrow + (int64_t)g * 64);
#pragma unroll
            for (int st = 0; st < 4; ++st) xa[j][st] = xp[st];
            const uint4* wp = (const uint4*)(wrow + (int64_t)g * 16);
            wb[j][0] = wp[0];
            wb[j][1] = wp[1];
            sv[j] = srow[g];
            bv[j] = brow[g];
        }
#pragma unroll
        for (int j = 0; j < G8_SLOTS; ++j) {
            if (g0 + G8_WAVES * j >= G) break;   // uniform
            const uint32_t wv[8] = {wb[j][0].x, wb[j][0].y, wb[j][0].z, wb[j][0].w,
                                    wb[j][1].x, wb[j][1].y, wb[j][1].z, wb[j][1].w};
            floatx16 P, Ph, X1;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                P[i] = 0.f;
                Ph[i] = 0.f;
                X1[i] = 0.f;
            }
            // step st: k = 32h + 8st + (0..7) = bytes of words 8h + 2st, 8h + 2st + 1
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const uint32_t w0 = wv[2 * st], w1 = wv[2 * st + 1];
                const uint4 ones = make_uint4(one2, one2, one2, one2);
                if constexpr (XF == 0) {
                    const uint4 bq = make_uint4(byte_pair(w0, magic, 0x04010400u),
                                                byte_pair(w0, magic, 0x04030402u),
                                                byte_pair(w1, magic, 0x04010400u),
                                                byte_pair(w1, magic, 0x04030402u));
                    const f16x8_t av = __builtin_bit_cast(f16x8_t, xa[j][st]);
                    P = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, __builtin_bit_cast(f16x8_t, bq), P,
                                                               0, 0, 0);
                    X1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, __builtin_bit_cast(f16x8_t, ones),
                                                                X1, 0, 0, 0);
                } else {
                    const uint32_t l0 = w0 & 0x0F0F0F0Fu, h0 = (w0 >> 4) & 0x0F0F0F0Fu;
                    const uint32_t l1 = w1 & 0x0F0F0F0Fu, h1 = (w1 >> 4) & 0x0F0F0F0Fu;
                    const uint4 bl = make_uint4(byte_pair(l0, magic, 0x04010400u),
                                                byte_pair(l0, magic, 0x04030402u),
                                                byte_pair(l1, magic, 0x04010400u),
                                                byte_pair(l1, magic, 0x04030402u));
                    const uint4 bh = make_uint4(byte_pair(h0, magic, 0x04010400u),
                                                byte_pair(h0, magic, 0x04030402u),
                                                byte_pair(h1, magic, 0x04010400u),
                                                byte_pair(h1, magic, 0x04030402u));
                    const bf16x8_t av = __builtin_bit_cast(bf16x8_t, xa[j][st]);
                    P = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8_t, bl), P,
                                                                0, 0, 0);
                    Ph = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8_t, bh), Ph,
                                                                 0, 0, 0);
                    X1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8_t, ones),
                                                                 X1, 0, 0, 0);
                }
            }
            const float sf = h2f(sv[j]);
            const float off = XF == 0 ? 1024.f : 2176.f;
            const float bf = h2f(bv[j]) - off * sf;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float pc = XF == 0 ? P[i] : fmaf(16.f, Ph[i], P[i]);
                acc[i] = fmaf(bf, X1[i], fmaf(sf, pc, acc[i]));
            }
        }
    }

    // fixed-order sum of the 8 waves' partial results
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) red[wave - 1][i][lane] = acc[i];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < G8_WAVES - 1; ++w)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] += red[w][i][lane];
    if (n < a.N) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int tt = blockIdx.y * 32 + 8 * (i / 4) + 4 * h + (i % 4);
            if (tt < a.T) a.y[(int64_t)tt * a.N + n] = acc[i];
        }
    }
}

hipError_t launch_gemm8_tokens(const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                               const uint16_t* x, int xkind, float* y, int N, int K, int T,
                               hipStream_t st) {
    if (K % 64 != 0 || (xkind != X_F16 && xkind != X_BF16)) return hipErrorInvalidValue;
    G8Args a{wq, s, b, x, y, T, N, K};
    const dim3 grid((N + 31) / 32, (T + 31) / 32);
    if (xkind == X_F16)
        hipLaunchKernelGGL(gemm8_tokens_kernel<0>, grid, dim3(64 * G8_WAVES), 0, st, a);
    else
        hipLaunchKernelGGL(gemm8_tokens_kernel<1>, grid, dim3(64 * G8_WAVES), 0, st, a);
    return hipGetLastError();
}

}  // namespace qd
