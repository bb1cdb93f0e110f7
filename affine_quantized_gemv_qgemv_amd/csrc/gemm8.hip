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
// The matrix-core operand is the exact centred code q - 128 (w = s (q - 128)
// + (b + 128 s)): for f16 activations a code byte in the low mantissa of f16
// 1024.0 gives 1024 + q, and one v_pk_add_f16 with -1152 leaves q - 128; for
// bf16 activations the code XOR 0x80 is the signed byte q - 128, converted
// exactly (mfma.h). One MFMA per 16 inputs yields P = sum_k x (q - 128), a
// second against an all-ones operand gives the row sums Xsum in the
// accumulator layout, and per group, in fp32,
//     acc += s P + (b + 128 s) Xsum.
// The products carry no offset, so the sums round in proportion to the
// weights' own size.

// Tiling: a workgroup owns 32 tokens x 32 outputs and has 8 waves that take
// alternate groups of K (wave w: groups w, w + 8, ...), each loading six of
// its groups at once before using them (a 2816-input router in one round);
// the 8 partial sums are added in LDS in a fixed order, so results do not
// depend on timing.
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
    float* y;             // [T][N]; with a K split, the [splits][T][N] partial slices
    int T, N, K;
    int gsplit;           // K split: groups per split (blockIdx.z), 0 = whole K
};

constexpr int G8_WAVES = 8;
constexpr int G8_SLOTS = 6;   // groups loaded together per wave

// Two code bytes of w (bytes j, j + 1) beside magic bytes m:
// dword = [w.b(j), m, w.b(j+1), m].
__device__ __forceinline__ uint32_t byte_pair(uint32_t w, uint32_t m, uint32_t sel) {
    // v_perm_b32(src0 = m, src1 = w, sel): selector 0..3 picks w's bytes, 4..7 m's
    return __builtin_amdgcn_perm(m, w, sel);
}

// KS: K split across workgroups: blockIdx.z takes groups [z gsplit,
// min((z + 1) gsplit, K / 64)) and writes slice z of a.y; the slices are added
// in split order by their reader (the routing of a prefill chunk). SLOTS:
// groups a wave loads together; every slot is requested (clamped), so a split
// runs with just enough slots for its groups: each 16-byte activation load
// touches 32 rows' cache lines, and these requests bound the kernel.
template <int XF, bool KS = false, int SLOTS = G8_SLOTS>   // XF 0: f16, 1: bf16 activations
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
    const uint32_t magic = in_vgpr(0x64646464u);   // fp16 1024 in the bytes the codes skip
    const uint32_t one2 = XF == 0 ? 0x3C003C00u : 0x3F803F80u;   // (1.0, 1.0)

    floatx16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;

    int gb = 0, ge = G;   // this workgroup's groups
    if constexpr (KS) {
        gb = (int)blockIdx.z * a.gsplit;
        ge = min(G, gb + a.gsplit);
        a.y += (int64_t)blockIdx.z * a.T * a.N;
    }
    for (int g0 = gb + wave; g0 < ge; g0 += G8_WAVES * SLOTS) {
        uint4 xa[SLOTS][4], wb[SLOTS][2];
        uint16_t sv[SLOTS], bv[SLOTS];
#pragma unroll
        for (int j = 0; j < SLOTS; ++j) {   // clamped loads, used only if g < ge
            const int g = min(g0 + G8_WAVES * j, ge - 1);
            const uint4* xp = (const uint4*)(xrow + (int64_t)g * 64);
#pragma unroll
            for (int st = 0; st < 4; ++st) xa[j][st] = xp[st];
            const uint4* wp = (const uint4*)(wrow + (int64_t)g * 16);
            wb[j][0] = wp[0];
            wb[j][1] = wp[1];
            sv[j] = srow[g];
            bv[j] = brow[g];
        }
        // every slot's loads are in flight before the first is used: slots
        // past G run on their clamped copies with zero factors rather than
        // being skipped (a branch around them would let the compiler sink
        // each slot's loads into it, one memory round trip per group)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < SLOTS; ++j) {
            const bool valid = g0 + G8_WAVES * j < ge;   // uniform
            const uint32_t wv[8] = {wb[j][0].x, wb[j][0].y, wb[j][0].z, wb[j][0].w,
                                    wb[j][1].x, wb[j][1].y, wb[j][1].z, wb[j][1].w};
            floatx16 P, X1;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                P[i] = 0.f;
                X1[i] = 0.f;
            }
            // step st: k = 32h + 8st + (0..7) = bytes of words 8h + 2st, 8h + 2st + 1
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const uint32_t w0 = wv[2 * st], w1 = wv[2 * st + 1];
                const uint4 ones = make_uint4(one2, one2, one2, one2);
                if constexpr (XF == 0) {
                    const uint4 bq = make_uint4(pk_addh(byte_pair(w0, magic, 0x04010400u), kNeg1152),
                                                pk_addh(byte_pair(w0, magic, 0x04030402u), kNeg1152),
                                                pk_addh(byte_pair(w1, magic, 0x04010400u), kNeg1152),
                                                pk_addh(byte_pair(w1, magic, 0x04030402u), kNeg1152));
                    const f16x8_t av = __builtin_bit_cast(f16x8_t, xa[j][st]);
                    P = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, __builtin_bit_cast(f16x8_t, bq), P,
                                                               0, 0, 0);
                    X1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, __builtin_bit_cast(f16x8_t, ones),
                                                                X1, 0, 0, 0);
                } else {
                    const uint2 c0 = bytes_centred_bf16(w0), c1 = bytes_centred_bf16(w1);
                    const uint4 bq = make_uint4(c0.x, c0.y, c1.x, c1.y);
                    const bf16x8_t av = __builtin_bit_cast(bf16x8_t, xa[j][st]);
                    P = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8_t, bq), P,
                                                                0, 0, 0);
                    X1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8_t, ones),
                                                                 X1, 0, 0, 0);
                }
            }
            const float sf = valid ? h2f(sv[j]) : 0.f;
            const float bf = valid ? fmaf(128.f, sf, h2f(bv[j])) : 0.f;   // b + 128 s
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = fmaf(bf, X1[i], fmaf(sf, P[i], acc[i]));
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

// K split of the chunk router: 128 tokens x 128 experts are 16 tiles of 32 x 32,
// each pulling its 32 tokens' activations through one CU. Up to G8_SPLIT
// splits of at least 8 groups each (a 2816-input router: 5 splits of 9
// groups, 80 workgroups), each wave of a split loading G8_SPLIT_SLOTS groups
// at once (measured per c4 MoE layer: 4 splits with 2 slots 187.4 µs, this
// 186.2, unsplit 192.4).
constexpr int G8_SPLIT = 8;
constexpr int G8_SPLIT_SLOTS = 1;

G8Split gemm8_split(int N, int K, int T) {
    const int G = K / 64;
    const int sp = min(G8_SPLIT, G / 8);
    if (N < 1 || T < 1 || G < 1 || sp <= 1) return {1, G};
    const int gs = (G + sp - 1) / sp;
    return {(G + gs - 1) / gs, gs};
}

hipError_t launch_gemm8_tokens_split(const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                                     const uint16_t* x, int xkind, float* part, int N, int K, int T,
                                     hipStream_t st) {
    if (K % 64 != 0 || (xkind != X_F16 && xkind != X_BF16)) return hipErrorInvalidValue;
    const G8Split c = gemm8_split(N, K, T);
    G8Args a{wq, s, b, x, part, T, N, K, c.gsplit};
    const dim3 grid((N + 31) / 32, (T + 31) / 32, c.splits);
    if (xkind == X_F16)
        hipLaunchKernelGGL((gemm8_tokens_kernel<0, true, G8_SPLIT_SLOTS>), grid, dim3(64 * G8_WAVES), 0,
                           st, a);
    else
        hipLaunchKernelGGL((gemm8_tokens_kernel<1, true, G8_SPLIT_SLOTS>), grid, dim3(64 * G8_WAVES), 0,
                           st, a);
    return hipGetLastError();
}

hipError_t launch_gemm8_tokens(const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                               const uint16_t* x, int xkind, float* y, int N, int K, int T,
                               hipStream_t st) {
    if (K % 64 != 0 || (xkind != X_F16 && xkind != X_BF16)) return hipErrorInvalidValue;
    G8Args a{wq, s, b, x, y, T, N, K, 0};
    const dim3 grid((N + 31) / 32, (T + 31) / 32);
    if (xkind == X_F16)
        hipLaunchKernelGGL(gemm8_tokens_kernel<0>, grid, dim3(64 * G8_WAVES), 0, st, a);
    else
        hipLaunchKernelGGL(gemm8_tokens_kernel<1>, grid, dim3(64 * G8_WAVES), 0, st, a);
    return hipGetLastError();
}

}  // namespace qd
