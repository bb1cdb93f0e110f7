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
//     weight codes enter as bytes q (the nibbles spread to bytes), so
//     P = sum q xq is an exact integer (|P| <= 64 * 15 * 127 < 2^24) and
//     per group, in fp32,
//         acc += s P + b Xsum,   Y = sx acc,
//     with Xsum the group's code sum; the s P terms on the VALU, the bias
//     terms of 4 groups as one v_mfma_f32_16x16x4_f32. A workgroup owns up
//     to 4 16-row tiles (2 at M > 16) and its 4 or 8 waves split K into
//     contiguous runs of groups; one activation load then serves every tile,
//     and the workgroup's scales and biases are staged in LDS once. The
//     waves' partial sums meet in LDS in wave order, so results do not
//     depend on timing. Tokens come in one or two blocks of 16 (M <= 32)
//     sharing each unpacked code word.
#include "common.h"
#include "launch.h"

namespace qd {

typedef int int32x4_t __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

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
// 1. quantize one token row per workgroup (1024 threads)
// ---------------------------------------------------------------------------
constexpr int VQ_T = 1024;   // threads per token
constexpr int VQ_R = 4;      // dwords of codes per thread and pass

// Thread t makes dword d = t % 4 of 16-input block t / 4 (then t + 1024,
// ...): bytes i = 4d .. 4d + 3 of the block, i.e. inputs vi_perm(i), which
// all lie in one 8-input half of the block (dwords 0, 1: inputs 0..7, 2, 3:
// 8..15), so one 16-byte load serves both passes. With K up to 16 VQ_T VQ_R
// / 4 (16384) the values stay in registers between the max and the codes;
// longer rows are read again. 16 consecutive lanes hold a group's 64 codes
// and sum them.
__device__ __forceinline__ uint4 vq_load(const uint16_t* xr, int e, bool live) {
    // e: index of the dword of codes; its 8 inputs start at input 8 (e / 2)
    return live ? *(const uint4*)(xr + 8 * (int64_t)(e >> 1)) : make_uint4(0, 0, 0, 0);
}

__global__ __launch_bounds__(VQ_T) void verify_i8_quant_kernel(const uint16_t* x, int M, int K, ViWs w,
                                                               int Mp) {
    __shared__ float wmax[VQ_T / 64];
    const int m = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool live = m < M;
    const uint16_t* xr = x + (int64_t)min(m, M - 1) * K;
    const int nd = K / 4;   // dwords of codes in the row
    const bool one_pass = nd <= VQ_T * VQ_R;
    uint4 v[VQ_R];
    float amax = 0.f;
    for (int e0 = 0; e0 < nd; e0 += VQ_T * VQ_R) {
#pragma unroll
        for (int r = 0; r < VQ_R; ++r) {
            const int e = e0 + VQ_T * r + threadIdx.x;
            v[r] = vq_load(xr, e, live && e < nd);
        }
#pragma unroll
        for (int r = 0; r < VQ_R; ++r) {
            const uint32_t wd[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                amax = fmaxf(amax, fmaxf(fabsf(h2f((uint16_t)wd[i])), fabsf(h2f((uint16_t)(wd[i] >> 16)))));
        }
    }
    amax = wave_max_f(amax);
    if (lane == 0) wmax[wave] = amax;
    __syncthreads();
    amax = wmax[0];
#pragma unroll
    for (int i = 1; i < VQ_T / 64; ++i) amax = fmaxf(amax, wmax[i]);
    const float sc = __fdiv_rn(amax, 127.0f);   // correctly rounded
    if (threadIdx.x == 0) w.sx[m] = live ? sc : 0.f;
    const int d = threadIdx.x & 3;   // dword of the block this thread makes
    for (int e0 = 0; e0 < nd; e0 += VQ_T * VQ_R) {
        if (!one_pass) {
#pragma unroll
            for (int r = 0; r < VQ_R; ++r) {
                const int e = e0 + VQ_T * r + threadIdx.x;
                v[r] = vq_load(xr, e, live && e < nd);
            }
        }
#pragma unroll
        for (int r = 0; r < VQ_R; ++r) {
            if (e0 + VQ_T * r >= nd) break;   // uniform: the rest of the pass is past the row
            const int e = e0 + VQ_T * r + threadIdx.x;
            const bool ok = e < nd;
            const uint32_t wd[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
            uint32_t code = 0;
            int sum = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // input vi_perm(4d + i) of the block: position (vi_perm(4d + i) & 7)
                // of the loaded half, which for d = 0, 2 is 2i and for d = 1, 3 is 2i + 1
                const uint16_t h = (uint16_t)(wd[i] >> (16 * (d & 1)));
                // a zero scale (a row of zeros) gives code 0 without dividing
                const int c = amax > 0.f ? (int)rintf(__fdiv_rn(h2f(h), sc)) : 0;
                code |= (uint32_t)(c & 0xFF) << (8 * i);
                sum += c;
            }
            const int blk = e >> 2, g = e >> 4;
            if (ok) *(uint32_t*)(w.q + ((int64_t)g * Mp + m) * 64 + 16 * (blk & 3) + 4 * d) = code;
            sum += __shfl_xor(sum, 1);
            sum += __shfl_xor(sum, 2);
            sum += __shfl_xor(sum, 4);
            sum += __shfl_xor(sum, 8);
            if (ok && (e & 15) == 0) w.xsum[(int64_t)g * Mp + m] = (float)sum;
        }
    }
}

// ---------------------------------------------------------------------------
// 2. the GEMM
// ---------------------------------------------------------------------------
// 16 weight codes (words w0, w1 = 16 consecutive inputs of a row) as bytes
// q in 0..15 (non-negative, so exact as the MFMA's signed int8) in the
// order vi_perm gives.
__device__ __forceinline__ int32x4_t vi_codes(uint32_t w0, uint32_t w1) {
    int32x4_t r;
    r[0] = (int)(w0 & 0x0F0F0F0Fu);
    r[1] = (int)((w0 >> 4) & 0x0F0F0F0Fu);
    r[2] = (int)(w1 & 0x0F0F0F0Fu);
    r[3] = (int)((w1 >> 4) & 0x0F0F0F0Fu);
    return r;
}

// The codes of two groups as loaded (lane (n, j): bytes 16j .. 16j + 15 of
// a row's 64-byte pair of groups, i.e. lanes j = 0, 1 hold the first group,
// j = 2, 3 the second) regrouped by two lane swaps between the wave's
// halves into one MFMA operand per group: afterwards lane j holds, of each
// group, the 16 inputs of block jb = [0, 2, 1, 3][j] (dwords 0, 1 for the
// first group, 2, 3 for the second), as bytes q.
__device__ __forceinline__ void pair_codes(uint4 c, int32x4_t& g0, int32x4_t& g1) {
    const auto a = __builtin_amdgcn_permlane32_swap(c.x, c.z, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(c.y, c.w, false, false);
    g0 = vi_codes(a[0], b[0]);
    g1 = vi_codes(a[1], b[1]);
}

// Workgroup: RT 16-row tiles (rows r0 .. r0 + 16 RT - 1), W waves; wave w
// takes groups [w per, min(G, (w + 1) per)) in stages of 4 groups, loading
// stage i + 1 while it multiplies stage i. Lane (n, j): row n of each tile
// and token n of each 16-token block for the operands, inputs 16 jb ..
// 16 jb + 15 of each group (pair_codes); results for tokens 4j .. 4j + 3 of
// each block.
// Per stage and tile the code products enter as s P (VALU) and the bias
// terms as one v_mfma_f32_16x16x4_f32 contracting the stage's 4 groups:
// lane (n, j) gives Xsum[token n][group g + j] and b[row n][group g + j].
// SBL: the workgroup's scales and biases are first copied to LDS with
// row-contiguous loads and each stage reads its 4 per row from there, so the
// stage's global loads are the codes and the activations alone (per-row
// scale loads would touch as many cache lines as the codes); otherwise (odd
// G, or rows too long for the LDS) one 2-byte global load per group.
constexpr int VI_LDS_MAX = 128 * 1024;

// Halves per LDS row of scales (or biases): G rounded up to 4, plus 4, so
// that the 16 rows one instruction reads fall in different banks.
static inline int vi_sb_stride(int G) { return (G + 3) / 4 * 4 + 4; }

template <int RT, int NB, int W>
static size_t vi_lds_bytes(int G, bool sbl) {
    const size_t red = (size_t)W * RT * NB * 4 * 64 * 4;
    const size_t sb = sbl ? (size_t)2 * 16 * RT * vi_sb_stride(G) * 2 : 0;
    return red > sb ? red : sb;
}

template <int RT, int NB, int W, bool SBL>
__global__ __launch_bounds__(64 * W) void verify_i8_gemm_kernel(
    const uint32_t* wq, const uint16_t* s, const uint16_t* b, ViWs ws, float* y, int M, int N, int K,
    int Mp, int per, int str) {
    constexpr int U = 4;
    extern __shared__ uint4 vi_smem[];
    // the scales and biases [16 RT][str] during the loop, the waves' partial
    // sums [W][RT NB 4][64] after it
    uint16_t* sl = (uint16_t*)vi_smem;
    uint16_t* bl = sl + 16 * RT * str;
    float* red = (float*)vi_smem;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, j = lane >> 4;
    const int jb = ((j & 1) << 1) | (j >> 1);   // the 16-input block of a group lane j holds
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

    if constexpr (SBL) {
        // dword c of row r (G is even), 8 per thread per round, loads first
        const int dpr = G / 2, tot = 16 * RT * dpr;
        for (int i0 = 0; i0 < tot; i0 += 8 * 64 * W) {
            uint32_t sv[8], bv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int i = i0 + e * 64 * W + (int)threadIdx.x;
                const int r = i / dpr, c = i - r * dpr;
                const uint32_t off = i < tot ? ((uint32_t)r * (uint32_t)G + 2u * (uint32_t)c) * 2u : OOB;
                sv[e] = __builtin_amdgcn_raw_buffer_load_b32(sr, (int)off, 0, 0);
                bv[e] = __builtin_amdgcn_raw_buffer_load_b32(br, (int)off, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int i = i0 + e * 64 * W + (int)threadIdx.x;
                if (i < tot) {
                    const int r = i / dpr, c = i - r * dpr;
                    *(uint32_t*)(sl + r * str + 2 * c) = sv[e];
                    *(uint32_t*)(bl + r * str + 2 * c) = bv[e];
                }
            }
        }
        __syncthreads();
    }

    struct Stage {
        uint4 cw[U / 2][RT];   // codes of groups g + 2p, g + 2p + 1 as loaded (see pair_codes)
        int32x4_t a[U][NB];
        float xs[NB];
        uint16_t su[SBL ? 1 : U][RT], bj[RT];   // without SBL: the scales, and lane j's bias
    };
    const int gb = wave * per;
    const int ge = min(G, gb + per);

    // every load is issued unconditionally (groups past the run read
    // nothing), so the compiler's count of loads in flight stays exact
    auto load = [&](Stage& t, int g) {
#pragma unroll
        for (int p = 0; p < U / 2; ++p) {
            // lane (n, j): 16 bytes of row n at byte 16 j of the pair of
            // groups g + 2p, g + 2p + 1, so the 4 lanes of a row read 64
            // contiguous bytes
            const bool ok = g + 2 * p < ge;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const uint32_t off = ok ? (uint32_t)(16 * rt + n) * rowb + (uint32_t)(g + 2 * p) * 32u + 16u * j : OOB;
                t.cw[p][rt] = buf_load16(wr, off);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = g + u < ge;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                // the 16 inputs of block jb of the group, the block pair_codes gives lane j
                const uint32_t qo = ok ? ((uint32_t)((g + u) * Mp + 16 * nb + n) * 64u + 16u * jb) : OOB;
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
        if constexpr (!SBL) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const uint32_t rg = (uint32_t)(16 * rt + n) * (uint32_t)G;
#pragma unroll
                for (int u = 0; u < U; ++u)
                    t.su[u][rt] = buf_load2(sr, g + u < ge ? (rg + (uint32_t)(g + u)) * 2u : OOB);
                t.bj[rt] = buf_load2(br, okj ? (rg + (uint32_t)(g + j)) * 2u : OOB);
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
            float sc[U], bjv;
            if constexpr (SBL) {
                // 4 scales and biases of row 16 rt + n from groups g .. g + 3 (8-byte aligned)
                const int ro = (16 * rt + n) * str + g;
                const uint2 sv = *(const uint2*)(sl + ro);
                const uint2 bv = *(const uint2*)(bl + ro);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t wd = u < 2 ? sv.x : sv.y;
                    sc[u] = g + u < ge ? h2f((uint16_t)(wd >> (16 * (u & 1)))) : 0.f;
                }
                bjv = h2f((uint16_t)(((j & 2) ? bv.y : bv.x) >> hs));
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) sc[u] = h2f(t.su[u][rt]);
                bjv = h2f(t.bj[rt]);
            }
            // w = s q + b; a group past the run adds exactly zero
            const float bi = okj ? bjv : 0.f;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                acc[rt][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(t.xs[nb], bi, acc[rt][nb], 0, 0, 0);
            int32x4_t bqs[U];
#pragma unroll
            for (int p = 0; p < U / 2; ++p) pair_codes(t.cw[p][rt], bqs[2 * p], bqs[2 * p + 1]);
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int32x4_t P = __builtin_amdgcn_mfma_i32_16x16x64_i8(t.a[u][nb], bqs[u], zero4, 0, 0, 0);
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

    // partial sums of the W waves, added in wave order (the LDS held the
    // scales until every wave is past its loop)
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                red[((wave * RT * NB + rt * NB + nb) * 4 + i) * 64 + lane] = acc[rt][nb][i];
    __syncthreads();
    for (int p = wave; p < RT * NB; p += W) {
        const int rt = p / NB, nb = p % NB;
        const int row = r0 + 16 * rt + n;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v = 0.f;
#pragma unroll
            for (int wv = 0; wv < W; ++wv) v += red[((wv * RT * NB + p) * 4 + i) * 64 + lane];
            const int t = 16 * nb + 4 * j + i;
            if (t < M && row < N) y[(int64_t)t * N + row] = ws.sx[t] * v;
        }
    }
}

template <int RT, int NB, int W, bool SBL>
static void vi_gemm(const uint32_t* wq, const uint16_t* s, const uint16_t* b, ViWs w, float* y, int M,
                    int N, int K, int Mp, hipStream_t st) {
    const int G = K / 64;
    // runs of whole stages; waves past the last group add nothing
    const int per = ((G + W - 1) / W + VI_U - 1) / VI_U * VI_U;
    const dim3 grid((N + 16 * RT - 1) / (16 * RT));
    const size_t lds = vi_lds_bytes<RT, NB, W>(G, SBL);
    hipLaunchKernelGGL((verify_i8_gemm_kernel<RT, NB, W, SBL>), grid, dim3(64 * W), lds, st, wq, s, b, w,
                       y, M, N, K, Mp, per, vi_sb_stride(G));
}

template <int NB, int W>
static void vi_gemm_rt(int rt, const uint32_t* wq, const uint16_t* s, const uint16_t* b, ViWs w, float* y,
                       int M, int N, int K, int Mp, hipStream_t st) {
    if constexpr (NB == 1) {
        if (rt >= 4) {
            vi_gemm<4, NB, W, true>(wq, s, b, w, y, M, N, K, Mp, st);
            return;
        }
    }
    if (rt >= 2)
        vi_gemm<2, NB, W, true>(wq, s, b, w, y, M, N, K, Mp, st);
    else
        vi_gemm<1, NB, W, true>(wq, s, b, w, y, M, N, K, Mp, st);
}

hipError_t launch_verify_i8(const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                            const uint16_t* x, float* y, int M, int N, int K, void* ws,
                            size_t ws_bytes, hipStream_t st) {
    if (M < 1 || M > 32 || K < 64 || K % 64 != 0 || N < 1) return hipErrorInvalidValue;
    if (ws_bytes < verify_i8_workspace_bytes(M, K)) return hipErrorInvalidValue;
    const int Mp = (M + 15) / 16 * 16;
    const int G = K / 64;
    const ViWs w = vi_carve(ws, Mp, K);
    hipLaunchKernelGGL(verify_i8_quant_kernel, dim3(Mp), dim3(VQ_T), 0, st, x, M, K, w, Mp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // Tiles per workgroup: as many as the registers allow (4 at M <= 16, 2
    // above), halved while the grid has fewer workgroups than the chip's 256
    // CUs; 8 waves per workgroup on rows of 8192 inputs or more, 4 below
    // (measured on the 7B FFN shapes).
    int rt = Mp == 16 ? 4 : 2;
    while (rt > 1 && (N + 16 * rt - 1) / (16 * rt) < 256) rt /= 2;
    const bool wide = G >= 128;
    const bool sbl = G % 2 == 0 && vi_lds_bytes<4, 1, 8>(G, true) <= VI_LDS_MAX;
    if (!sbl) {
        // odd G or very long rows: scales and biases from global memory
        if (Mp == 16)
            vi_gemm<1, 1, 8, false>(wq, s, b, w, y, M, N, K, Mp, st);
        else
            vi_gemm<1, 2, 8, false>(wq, s, b, w, y, M, N, K, Mp, st);
    } else if (Mp == 16) {
        wide ? vi_gemm_rt<1, 8>(rt, wq, s, b, w, y, M, N, K, Mp, st)
             : vi_gemm_rt<1, 4>(rt, wq, s, b, w, y, M, N, K, Mp, st);
    } else {
        wide ? vi_gemm_rt<2, 8>(rt, wq, s, b, w, y, M, N, K, Mp, st)
             : vi_gemm_rt<2, 4>(rt, wq, s, b, w, y, M, N, K, Mp, st);
    }
    return hipGetLastError();
}

}  // namespace qd
