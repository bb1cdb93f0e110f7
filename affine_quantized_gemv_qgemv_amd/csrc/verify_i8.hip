// Verification GEMM on dynamically quantized int8 activations for gfx950:
//     Y[m][n] = sum_k w[n][k] xh[m][k],   xh[m][k] = sx[m] xq[m][k],
// with MLX affine 4-bit weights (w = s q + b, group 64).
//
// discuss.pytorch.kr/t/uzu-mac-iphone-llm-apple-silicon-rust/12363 (uzu),
// section "추측 디코딩 구조" (speculative decoding): the target model checks
// 16-32 drafted tokens in one pass, which makes its projections small GEMMs,
// and runs them on the chip's int8 matrix path with the activations
// quantized to 8 bits on the fly. The page gives no quantization scheme;
// the one taken here is per token and symmetric: sx = max|x| / 127 and
// xq = round(x / sx) with ties to even, in fp32 (a row of zeros: sx = 0,
// xq = 0).
//
// Two launches:
//  1. quantize: one workgroup per token (rows up to a multiple of 16, the
//     extra rows zero) writes the codes, its scale and the per-group code
//     sums to the workspace. Within each block of 16 inputs the codes are
//     stored in the byte order in which the GEMM unpacks the weight codes
//     (below), so an operand load needs no shuffling.
//  2. GEMM: v_mfma_i32_16x16x64_i8, one instruction per group of 64 inputs:
//     A = 16 tokens x 64 codes, B = 64 weight codes x 16 rows, each lane
//     holding 16 bytes of one token / one row in the same k order. The
//     weight codes enter exactly as signed bytes q - 8 (the nibbles spread
//     to bytes, then + 0x78 and ^ 0x80 per byte: no carry crosses a byte),
//     so P = sum (q - 8) xq is an exact integer and per group, in fp32,
//         acc += s P + (b + 8 s) Xsum,   Y = sx acc,
//     with Xsum the group's code sum; the s P terms on the VALU, the bias
//     terms of 4 groups as one v_mfma_f32_16x16x4_f32. A workgroup owns 64
//     rows at M <= 16 (32 above) and its VI_W waves split K into contiguous
//     runs of groups; one activation load then serves every 16-row tile, and
//     a stage's scales and biases arrive as one vector load per row. The
//     waves' partial sums meet in LDS in wave order, so results do not
//     depend on timing. Tokens come in one or two blocks of 16 (M <= 32)
//     sharing each unpacked code word.
#include "common.h"
#include "launch.h"

namespace qd {

typedef int int32x4_t __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int VI_ROWS = 64;   // rows x 16-token blocks per GEMM workgroup: 4 tiles at M <= 16, 2 above
constexpr int VI_W = 8;    // waves per GEMM workgroup (runs of K groups)
constexpr int VI_U = 4;    // groups per pipeline stage (the bias MFMA's K)

// Workspace for Mp token rows (M rounded up to 16) and G = K / 64 groups,
// each part 256-byte aligned:
//   codes int8 [G][Mp][64]: group-major, so 16 tokens of one group are 1 KB
//     contiguous; within each block of 16 inputs permuted as vi_perm gives;
//   code sums fp32 [G][Mp] (exact: at most 64 * 127 in magnitude);
//   scales fp32 [Mp].
struct ViWs {
    int8_t* q;
    float* xsum;
    float* sx;
};

static size_t vi_align(size_t v) { return (v + 255) & ~(size_t)255; }

static ViWs vi_carve(void* ws, int Mp, int K) {
    char* p = (char*)ws;
    ViWs w;
    w.q = (int8_t*)p;
    p += vi_align((size_t)Mp * K);
    w.xsum = (float*)p;
    p += vi_align((size_t)(K / 64) * Mp * 4);
    w.sx = (float*)p;
    return w;
}

size_t verify_i8_workspace_bytes(int M, int K) {
    const int Mp = (M + 15) / 16 * 16;
    return vi_align((size_t)Mp * K) + vi_align((size_t)(K / 64) * Mp * 4) + vi_align((size_t)Mp * 4);
}

// Byte i of a 16-input block holds input P(i) = [0, 2, 4, 6, 1, 3, 5, 7, 8,
// 10, 12, 14, 9, 11, 13, 15][i]: the order of the unpacked weight codes.
__host__ __device__ constexpr int vi_perm(int i) {
    return 8 * (i >> 3) + ((i & 7) < 4 ? 2 * (i & 7) : 2 * ((i & 7) - 4) + 1);
}

// ---------------------------------------------------------------------------
// 1. quantize one token row per workgroup (256 threads)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void verify_i8_quant_kernel(const uint16_t* x, int M, int K, ViWs w,
                                                              int Mp) {
    __shared__ float wmax[4];
    const int m = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool live = m < M;
    const uint16_t* xr = x + (int64_t)min(m, M - 1) * K;
    float amax = 0.f;
    if (live)
        for (int k = threadIdx.x; k < K; k += 256) amax = fmaxf(amax, fabsf(h2f(xr[k])));
    amax = wave_max_f(amax);
    if (lane == 0) wmax[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float sc = __fdiv_rn(amax, 127.0f);   // correctly rounded
    if (threadIdx.x == 0) w.sx[m] = live ? sc : 0.f;
    // thread t takes the blocks of 16 inputs t, t + 256, ...; a group's 4
    // blocks sit in 4 consecutive lanes, which sum its codes
    const int nblk = K / 16;
    for (int b0 = 0; b0 < nblk; b0 += 256) {
        const int blk = b0 + threadIdx.x;
        const bool bl = blk < nblk;
        uint16_t h[16] = {};
        if (live && bl) {
            const uint4 lo = *(const uint4*)(xr + 16 * blk), hi = *(const uint4*)(xr + 16 * blk + 8);
            const uint32_t wd[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
            for (int i = 0; i < 16; ++i) h[i] = (uint16_t)(wd[i >> 1] >> (16 * (i & 1)));
        }
        uint32_t d[4] = {0, 0, 0, 0};
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            // a zero scale (a row of zeros) gives code 0 without dividing
            const int c = amax > 0.f ? (int)rintf(__fdiv_rn(h2f(h[vi_perm(i)]), sc)) : 0;
            d[i >> 2] |= (uint32_t)(c & 0xFF) << (8 * (i & 3));
            sum += c;
        }
        const int g = blk >> 2;
        if (bl)
            *(uint4*)(w.q + ((int64_t)g * Mp + m) * 64 + 16 * (blk & 3)) = make_uint4(d[0], d[1], d[2], d[3]);
        sum += __shfl_xor(sum, 1);
        sum += __shfl_xor(sum, 2);
        if (bl && (blk & 3) == 0) w.xsum[(int64_t)g * Mp + m] = (float)sum;
    }
}

// ---------------------------------------------------------------------------
// 2. the GEMM
// ---------------------------------------------------------------------------
// 16 weight codes (words w0, w1 = inputs 16j..16j+15 of a row) as signed
// bytes q - 8 in the order vi_perm gives.
__device__ __forceinline__ int32x4_t vi_codes(uint32_t w0, uint32_t w1) {
    const uint32_t t0 = w0 & 0x0F0F0F0Fu, u0 = (w0 >> 4) & 0x0F0F0F0Fu;
    const uint32_t t1 = w1 & 0x0F0F0F0Fu, u1 = (w1 >> 4) & 0x0F0F0F0Fu;
    int32x4_t r;
    r[0] = (int)((t0 + 0x78787878u) ^ 0x80808080u);
    r[1] = (int)((u0 + 0x78787878u) ^ 0x80808080u);
    r[2] = (int)((t1 + 0x78787878u) ^ 0x80808080u);
    r[3] = (int)((u1 + 0x78787878u) ^ 0x80808080u);
    return r;
}

// Workgroup: RT 16-row tiles (rows r0 .. r0 + 16 RT - 1), W waves; wave w
// takes groups [w per, min(G, (w + 1) per)) in stages of 4 groups, loading
// stage i + 1 while it multiplies stage i. Lane (n, j): row n of each tile
// and token n of each 16-token block for the operands, inputs 16j .. 16j + 15
// of each group; results for tokens 4j .. 4j + 3 of each block.
// Per stage and tile the code products enter as s P (VALU) and the bias
// terms as one v_mfma_f32_16x16x4_f32 contracting the stage's 4 groups:
// lane (n, j) gives Xsum[token n][group g + j] and (b + 8 s)[row n][group
// g + j]. VSB: a stage's scales and biases as one 8-byte load per row (needs
// G even); otherwise 2-byte loads.
template <int RT, int NB, int W, bool VSB>
__global__ __launch_bounds__(64 * W) void verify_i8_gemm_kernel(
    const uint32_t* wq, const uint16_t* s, const uint16_t* b, ViWs ws, float* y, int M, int N, int K,
    int Mp, int per) {
    constexpr int U = 4;
    __shared__ float red[W][RT * NB * 4][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, j = lane >> 4;
    const int G = K >> 6;
    const int r0 = blockIdx.x * 16 * RT;
    const int rows = min(16 * RT, N - r0);
    const uint32_t rowb = (uint32_t)K / 2;
    // resources over this tile's rows: rows past N read as zero
    const auto wr = buf_rsrc(wq + (int64_t)r0 * (K / 8), (int64_t)rows * rowb);
    const auto sr = buf_rsrc(s + (int64_t)r0 * G, (int64_t)rows * G * 2);
    const auto br = buf_rsrc(b + (int64_t)r0 * G, (int64_t)rows * G * 2);
    const auto qr = buf_rsrc(ws.q, (int64_t)G * Mp * 64);
    const auto xr = buf_rsrc(ws.xsum, (int64_t)G * Mp * 4);
    constexpr uint32_t OOB = 0x7FFFFFF0u;   // past every resource: reads zero, touches nothing

    struct Stage {
        uint2 cw[U][RT];
        int32x4_t a[U][NB];
        float xs[NB];
        uint2 sv[RT], bv[RT];                 // VSB: 4 scales, 4 biases per row
        uint16_t su[U][RT], sj[RT], bj[RT];   // otherwise
    };
    const int gb = wave * per;
    const int ge = min(G, gb + per);

    // every load is issued unconditionally (groups past the run read
    // nothing), so the compiler's count of loads in flight stays exact
    auto load = [&](Stage& t, int g) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = g + u < ge;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const uint32_t off = ok ? (uint32_t)(16 * rt + n) * rowb + (uint32_t)(g + u) * 32u + 8u * j : OOB;
                const auto v = __builtin_amdgcn_raw_buffer_load_b64(wr, (int)off, 0, 0);
                t.cw[u][rt] = make_uint2(v[0], v[1]);
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const uint32_t qo = ok ? ((uint32_t)((g + u) * Mp + 16 * nb + n) * 64u + 16u * j) : OOB;
                const uint4 av = buf_load16(qr, qo);
                t.a[u][nb] = int32x4_t{(int)av.x, (int)av.y, (int)av.z, (int)av.w};
            }
        }
        const bool okj = g + j < ge;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const uint32_t xo = okj ? (uint32_t)((g + j) * Mp + 16 * nb + n) * 4u : OOB;
            t.xs[nb] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, (int)xo, 0, 0));
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const uint32_t rg = (uint32_t)(16 * rt + n) * (uint32_t)G;
            if constexpr (VSB) {
                const uint32_t so = g < ge ? (rg + (uint32_t)g) * 2u : OOB;
                const auto sv = __builtin_amdgcn_raw_buffer_load_b64(sr, (int)so, 0, 0);
                const auto bv = __builtin_amdgcn_raw_buffer_load_b64(br, (int)so, 0, 0);
                t.sv[rt] = make_uint2(sv[0], sv[1]);
                t.bv[rt] = make_uint2(bv[0], bv[1]);
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u)
                    t.su[u][rt] = buf_load2(sr, g + u < ge ? (rg + (uint32_t)(g + u)) * 2u : OOB);
                const uint32_t so = okj ? (rg + (uint32_t)(g + j)) * 2u : OOB;
                t.sj[rt] = buf_load2(sr, so);
                t.bj[rt] = buf_load2(br, so);
            }
        }
    };

    floatx4 acc[RT][NB];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[rt][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
    const int32x4_t zero4 = {0, 0, 0, 0};
    const uint32_t hs = 16u * (uint32_t)(j & 1);   // this lane's half of a scale word

    auto compute = [&](const Stage& t, int g) {
        const bool okj = g + j < ge;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float sc[U], sjv, bjv;
            if constexpr (VSB) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t wd = u < 2 ? t.sv[rt].x : t.sv[rt].y;
                    sc[u] = g + u < ge ? h2f((uint16_t)(wd >> (16 * (u & 1)))) : 0.f;
                }
                sjv = h2f((uint16_t)(((j & 2) ? t.sv[rt].y : t.sv[rt].x) >> hs));
                bjv = h2f((uint16_t)(((j & 2) ? t.bv[rt].y : t.bv[rt].x) >> hs));
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) sc[u] = h2f(t.su[u][rt]);
                sjv = h2f(t.sj[rt]);
                bjv = h2f(t.bj[rt]);
            }
            // w = s (q - 8) + (b + 8 s); a group past the run adds exactly zero
            const float bi = okj ? fmaf(8.f, sjv, bjv) : 0.f;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                acc[rt][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(t.xs[nb], bi, acc[rt][nb], 0, 0, 0);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int32x4_t bq = vi_codes(t.cw[u][rt].x, t.cw[u][rt].y);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int32x4_t P = __builtin_amdgcn_mfma_i32_16x16x64_i8(t.a[u][nb], bq, zero4, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[rt][nb][i] = fmaf(sc[u], (float)P[i], acc[rt][nb][i]);
                }
            }
        }
    };

    Stage A, B;
    load(A, gb);
    for (int g = gb; g < ge; g += 2 * U) {
        load(B, g + U);
        compute(A, g);
        load(A, g + 2 * U);
        if (g + U < ge) compute(B, g + U);
    }

    // partial sums of the W waves, added in wave order
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][(rt * NB + nb) * 4 + i][lane] = acc[rt][nb][i];
    __syncthreads();
    for (int p = wave; p < RT * NB; p += W) {
        const int rt = p / NB, nb = p % NB;
        const int row = r0 + 16 * rt + n;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v = 0.f;
#pragma unroll
            for (int wv = 0; wv < W; ++wv) v += red[wv][p * 4 + i][lane];
            const int t = 16 * nb + 4 * j + i;
            if (t < M && row < N) y[(int64_t)t * N + row] = ws.sx[t] * v;
        }
    }
}

template <int NB, bool VSB>
static void vi_gemm(const uint32_t* wq, const uint16_t* s, const uint16_t* b, ViWs w, float* y, int M,
                    int N, int K, int Mp, int per, hipStream_t st) {
    constexpr int RT = VI_ROWS / 16 / NB;
    const dim3 grid((N + 16 * RT - 1) / (16 * RT));
    hipLaunchKernelGGL((verify_i8_gemm_kernel<RT, NB, VI_W, VSB>), grid, dim3(64 * VI_W), 0, st, wq, s, b,
                       w, y, M, N, K, Mp, per);
}

hipError_t launch_verify_i8(const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                            const uint16_t* x, float* y, int M, int N, int K, void* ws,
                            size_t ws_bytes, hipStream_t st) {
    if (M < 1 || M > 32 || K < 64 || K % 64 != 0 || N < 1) return hipErrorInvalidValue;
    if (ws_bytes < verify_i8_workspace_bytes(M, K)) return hipErrorInvalidValue;
    const int Mp = (M + 15) / 16 * 16;
    const int G = K / 64;
    const ViWs w = vi_carve(ws, Mp, K);
    hipLaunchKernelGGL(verify_i8_quant_kernel, dim3(Mp), dim3(256), 0, st, x, M, K, w, Mp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // runs of whole stages; waves past the last group add nothing
    const int per = ((G + VI_W - 1) / VI_W + VI_U - 1) / VI_U * VI_U;
    const bool vsb = G % 2 == 0;
    if (Mp == 16)
        vsb ? vi_gemm<1, true>(wq, s, b, w, y, M, N, K, Mp, per, st)
            : vi_gemm<1, false>(wq, s, b, w, y, M, N, K, Mp, per, st);
    else
        vsb ? vi_gemm<2, true>(wq, s, b, w, y, M, N, K, Mp, per, st)
            : vi_gemm<2, false>(wq, s, b, w, y, M, N, K, Mp, per, st);
    return hipGetLastError();
}

}  // namespace qd
