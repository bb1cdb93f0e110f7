// Prefill-chunk GEMM on bf16 MFMA: Y[m][n] = sum_k w[n][k] X[m][k], M <= 128.
//
// [TF] jeff.news/article/5193, section "내부 구조가 진짜 흥미로운 부분"
// (internals): prompts are processed in chunks of at most 128 tokens so that
// one fetch of a weight serves many rows. Weight format as in the decode
// path ("성능과 제약": affine 4-bit, group 64, w = s*q + b).
//
// Rounding w itself to bf16 would lose too much (8 significant bits), so
// the matrix-core operand is the exact code: OR-ing a nibble into the low
// mantissa of bf16 128.0 (0x4300) gives exactly 128 + q. Per group g of 64
// inputs one v_mfma_f32_32x32x16_bf16 chain (4 x K=16) yields
//     P_g[m][n] = sum_{k in g} X[m][k] (128 + q[n][k])        (fp32)
// and the epilogue adds, in fp32,
//     acc[m][n] += s[n][g] * P_g[m][n] + (b[n][g] - 128 s[n][g]) * Xsum_g[m]
// with Xsum_g[m] = sum_{k in g} X[m][k], computed while X is staged.
//
// Tiling: a 256-thread workgroup owns all M (<= 128) rows and 64 output
// columns; wave (wm, wn) computes rows [64 wm, 64 wm + 64) x columns
// [32 wn, 32 wn + 32) as two 32x32 MFMA blocks. The X slice of each group is
// staged in LDS (double buffered, one barrier per group); each lane loads the
// 16 code bytes it feeds to the MFMA (words 4h..4h+3 of its column's group,
// where h is the lane's k-half), and the K order inside a group is permuted
// identically on both operands (step st, half h takes word 4h + st).
#include "common.h"
#include "launch.h"
#include "mfma.h"

namespace qd {

constexpr int CH_NT = 64;    // output columns per workgroup
constexpr int CH_MT = 128;   // rows per workgroup (the whole chunk)


struct ChunkArgs {
    const uint32_t* wq;
    const uint16_t* s;
    const uint16_t* b;
    const uint16_t* x;   // bf16 [M][K]
    float* y;            // [M][N]
    int M, N, K;
    int64_t x_row_stride;   // elements between rows of x
    int64_t y_row_stride;   // elements between rows of y
};

// LDS: xs[2][128][XS_STRIDE] uint4 (64 bf16 per row) then xsum[2][128] fp32.
__device__ __forceinline__ void chunk_load_x(const ChunkArgs& a, int g, uint4 (&xr)[4]) {
    const int t = threadIdx.x;
    const int m = t >> 1, hh = t & 1;
    if (m < a.M) {
        const uint4* src =
            (const uint4*)(a.x + (int64_t)m * a.x_row_stride + (int64_t)g * 64 + 32 * hh);
#pragma unroll
        for (int i = 0; i < 4; ++i) xr[i] = src[i];
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) xr[i] = make_uint4(0, 0, 0, 0);
    }
}

__device__ __forceinline__ void chunk_store_x(uint4* xs, float* xsum, const uint4 (&xr)[4]) {
    const int t = threadIdx.x;
    const int m = t >> 1, hh = t & 1;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        xs[m * XS_STRIDE + 4 * hh + i] = xr[i];
        acc = bf16_pair_sum(xr[i].x, acc);
        acc = bf16_pair_sum(xr[i].y, acc);
        acc = bf16_pair_sum(xr[i].z, acc);
        acc = bf16_pair_sum(xr[i].w, acc);
    }
    acc += __shfl_xor(acc, 1, 64);
    if (hh == 0) xsum[m] = acc;
}

__global__ __launch_bounds__(256) void chunk_gemm_kernel(ChunkArgs a) {
    __shared__ __align__(16) uint4 xs_raw[2][CH_MT * XS_STRIDE];
    __shared__ __align__(16) float xsum_raw[2][CH_MT];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int h = lane >> 5, l32 = lane & 31;
    const int G = a.K / 64;
    const int64_t wpr = a.K / 8;
    const int n = blockIdx.x * CH_NT + wn * 32 + l32;       // this lane's column
    const int nc = min(n, a.N - 1);
    const uint32_t* wrow = a.wq + (int64_t)nc * wpr + 4 * h;  // words 4h..4h+3 of group 0
    const uint16_t* srow = a.s + (int64_t)nc * G;
    const uint16_t* brow = a.b + (int64_t)nc * G;

    floatx16 acc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;

    uint4 xr[4];
    chunk_load_x(a, 0, xr);
    uint4 bw = *(const uint4*)wrow;
    uint16_t sv = srow[0], bv = brow[0];
    chunk_store_x(xs_raw[0], xsum_raw[0], xr);
    __syncthreads();

    for (int g = 0; g < G; ++g) {
        const int buf = g & 1;
        uint4 bw_next = bw;
        uint16_t sv_next = sv, bv_next = bv;
        if (g + 1 < G) {
            chunk_load_x(a, g + 1, xr);
            bw_next = *(const uint4*)(wrow + (int64_t)(g + 1) * 8);
            sv_next = srow[g + 1];
            bv_next = brow[g + 1];
        }
        const uint4* xs = xs_raw[buf];
        const float* xsum = xsum_raw[buf];
        floatx16 P[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) P[mb][i] = 0.f;
        const uint32_t wv[4] = {bw.x, bw.y, bw.z, bw.w};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const bf16x8_t bfrag = codes_to_bf16(wv[st]);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                const int m = 64 * wm + 32 * mb + l32;
                const bf16x8_t afrag = __builtin_bit_cast(bf16x8_t, xs[m * XS_STRIDE + 4 * h + st]);
                P[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag, bfrag, P[mb], 0, 0, 0);
            }
        }
        const float sf = h2f(sv);
        const float bf = h2f(bv) - 128.f * sf;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 xb = *(const float4*)(xsum + 64 * wm + 32 * mb + 8 * j + 4 * h);
                acc[mb][4 * j + 0] = fmaf(bf, xb.x, fmaf(sf, P[mb][4 * j + 0], acc[mb][4 * j + 0]));
                acc[mb][4 * j + 1] = fmaf(bf, xb.y, fmaf(sf, P[mb][4 * j + 1], acc[mb][4 * j + 1]));
                acc[mb][4 * j + 2] = fmaf(bf, xb.z, fmaf(sf, P[mb][4 * j + 2], acc[mb][4 * j + 2]));
                acc[mb][4 * j + 3] = fmaf(bf, xb.w, fmaf(sf, P[mb][4 * j + 3], acc[mb][4 * j + 3]));
            }
        }
        if (g + 1 < G) chunk_store_x(xs_raw[buf ^ 1], xsum_raw[buf ^ 1], xr);
        __syncthreads();
        bw = bw_next;
        sv = sv_next;
        bv = bv_next;
    }
    if (n < a.N) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = 64 * wm + 32 * mb + 8 * (i / 4) + 4 * h + (i % 4);
                if (m < a.M) a.y[(int64_t)m * a.y_row_stride + n] = acc[mb][i];
            }
    }
}

hipError_t launch_chunk_gemm(int bits, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                             const uint16_t* x_bf16, float* y, int M, int N, int K,
                             hipStream_t st) {
    if (bits != 4 || M > CH_MT) return hipErrorInvalidValue;
    ChunkArgs a{};
    a.wq = wq;
    a.s = s;
    a.b = b;
    a.x = x_bf16;
    a.y = y;
    a.M = M;
    a.N = N;
    a.K = K;
    a.x_row_stride = K;
    a.y_row_stride = N;
    const int grid = (N + CH_NT - 1) / CH_NT;
    hipLaunchKernelGGL(chunk_gemm_kernel, dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace qd
