// Device helpers shared by the libqdecode kernels (gfx950 / CDNA4, wave64).
//
// Weight format ([TF] = jeff.news/article/5193, section "성능과 제약",
// performance and constraints): MLX affine quantization, codes of 4 bits
// (8 for the router), one fp16 scale and one fp16 bias per group of 64
// inputs, w = s*q + b. Codes are packed LSB-first, eight (or four) per
// uint32 along the input dimension.
//
// Arithmetic of the GEMV core
// ---------------------------
// OR-ing a 4-bit code into the low mantissa bits of fp16 1024.0 (0x6400)
// gives exactly 1024 + q; OR-ing it one nibble higher gives 1024 + 16q.
// One v_and_or_b32 therefore turns two codes of a word (the nibbles at
// bits 0 and 16, or 4 and 20) into a packed half2. One v_pk_add_f16 then
// subtracts 1024 + c (or 1024 + 16c) from both halves, which is exact in
// fp16 and leaves the centred codes q - c (or 16 (q - c)) with c the
// centre of the format: 8 for affine 4-bit codes, 128 for 8-bit codes, the
// group's zero point z for Mirai-M. v_dot2_f32_f16 multiplies such a pair
// with two fp16 activations (both products exact in fp32) and adds them
// into an fp32 accumulator; fp32 activations take v_fma_mix_f32 instead.
// Because the offset is gone before anything is summed, the accumulators
// hold sums of (q - c) x whose rounding follows |q - c| |x|, and a weight
// that sits at the centre contributes exactly zero. Per group:
//     sum_k (q_k - c) x_k = acc_1 + acc_16 / 16
// where class "1" holds the codes at nibbles 0, 2, 4, 6 and class "16"
// those at nibbles 1, 3, 5, 7, and the affine epilogue adds
//     s_g * (that sum) + (b_g + c s_g) * (sum of the group's activations),
// which is s_g q + b_g summed against x; the Mirai formats have no second
// term (w = s (q - z), or s q for signed codes).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

namespace qd {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

constexpr uint32_t kMagic16 = 0x64006400u;  // fp16 pair (1024, 1024)
// fp16 pairs -(1024 + c) and -(1024 + 16 c): the centring subtrahends
constexpr uint32_t kNeg1032 = 0xE408E408u;  // 4-bit codes, c = 8, class 1
constexpr uint32_t kNeg1152 = 0xE480E480u;  // 4-bit class 16 (c = 8), and 8-bit codes (c = 128)

// Subtrahend pairs for a per-group centre z in [0, 15] (Mirai-M zero point):
// 0xE400 | z is fp16 -(1024 + z), 0xE400 | 16 z is -(1024 + 16 z).
__device__ __forceinline__ uint32_t neg_pair(uint32_t h) { return h | (h << 16); }

// A value the compiler must keep in a VGPR. Used for the fp16 magic so that
// (w & mask) | magic is selected as one v_and_or_b32 (a VOP3 on gfx9 reads at
// most one SGPR or constant; the mask takes that slot).
__device__ __forceinline__ uint32_t in_vgpr(uint32_t c) {
    uint32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(c));
    return r;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a), __builtin_bit_cast(half2v, b), c,
                                  false);
}

// Packed fp16 add of two half2 (one v_pk_add_f16).
__device__ __forceinline__ uint32_t pk_addh(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, a) + __builtin_bit_cast(half2v, b));
}

// fp32 accumulation of a packed fp16 pair against two fp32 activations
// (two v_fma_mix_f32).
__device__ __forceinline__ float fma_pair(uint32_t p, float x0, float x1, float acc) {
    const half2v h = __builtin_bit_cast(half2v, p);
    acc = fmaf((float)h.x, x0, acc);
    return fmaf((float)h.y, x1, acc);
}

// Raw buffer resource over `bytes` bytes from `base` (32-bit data format
// word, no stride or swizzle). A load through it takes a 32-bit byte offset
// from a VGPR and folds constant offsets into the instruction, so a tile's
// loads need one 32-bit multiply-add per row instead of 64-bit address
// arithmetic per load; a read at or past `bytes` returns zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int64_t bytes) {
    const int n = bytes > 0x7FFFFFFFll ? 0x7FFFFFFF : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint16_t buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}

__device__ __forceinline__ uint8_t buf_load1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

__device__ __forceinline__ float h2f(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ float bf2f(uint16_t h) {
    return __builtin_bit_cast(float, (uint32_t)h << 16);
}

__device__ __forceinline__ uint32_t pack_h2(uint16_t lo, uint16_t hi) {
    return (uint32_t)lo | ((uint32_t)hi << 16);
}

// Activation element kinds accepted by the staging code.
enum XKind : int { X_F16 = 0, X_BF16 = 1, X_F32 = 2 };

__device__ __forceinline__ float load_x(const void* x, int kind, int64_t i) {
    if (kind == X_F16) return h2f(((const uint16_t*)x)[i]);
    if (kind == X_BF16) return bf2f(((const uint16_t*)x)[i]);
    return ((const float*)x)[i];
}

// v from another lane through DPP (CTRL: quad_perm 0xB1 = lane ^ 1, 0x4E =
// lane ^ 2; 0x141 = mirror within each 8 lanes; 0x140 = mirror within each
// row of 16).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the `width` lanes of an aligned lane segment (width a power of two),
// returned to every lane of the segment, without LDS traffic: pairs of lanes,
// then quads, through DPP; 8- and 16-lane groups through the half-row and
// row mirrors (after the previous steps every lane of a group holds the same
// value, so a mirror pairs the groups as an xor would); rows of 16 and halves
// of 32 through v_permlane16_swap / v_permlane32_swap.
template <int WIDTH>
__device__ __forceinline__ float seg_sum(float v) {
    static_assert(WIDTH >= 1 && WIDTH <= 64 && (WIDTH & (WIDTH - 1)) == 0, "segment width");
    if constexpr (WIDTH >= 2) v += dpp_f<0xB1>(v);
    if constexpr (WIDTH >= 4) v += dpp_f<0x4E>(v);
    if constexpr (WIDTH >= 8) v += dpp_f<0x141>(v);
    if constexpr (WIDTH >= 16) v += dpp_f<0x140>(v);
    if constexpr (WIDTH >= 32) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                        false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    if constexpr (WIDTH >= 64) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                        false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return v;
}

// Maximum over the 64 lanes of a wave, in every lane (the same pairings as
// seg_sum<64>).
__device__ __forceinline__ float wave_max_f(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// v + (v of lane ^ OFF) for OFF = 8, 16 or 32: sums lanes that hold the same
// position of different lane groups (row_ror:8 within each row of 16, then
// the row and half swaps).
template <int OFF>
__device__ __forceinline__ float xor_add(float v) {
    static_assert(OFF == 8 || OFF == 16 || OFF == 32, "lane offset");
    if constexpr (OFF == 8) return v + dpp_f<0x128>(v);
    if constexpr (OFF == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                        false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// Activation staging into LDS.
//
// Layout for nc chunks and nb activation vectors:
//   xs[b][q][c]  (uint4; q < QPC per chunk), consecutive chunks at
//                consecutive 16-byte slots so the lanes of a row segment
//                read disjoint banks. Values sit in the order the unpacking
//                produces the code pairs: per word of 4-bit codes the fp16
//                pairs (x0,x4) (x1,x5) (x2,x6) (x3,x7), per two words of
//                8-bit codes (x0,x2) (x1,x3) (x4,x6) (x5,x7); fp32 values
//                (XF = 1) in the same order, one uint4 per four;
//   cs[b][c]     float: the sum of the chunk's activations.
// ---------------------------------------------------------------------------
//
// XF = 2 (rotated activations, see stage_x_rot) keeps the fp16 layout twice:
// planes q < QH hold the fp16 rounding hi of each value, planes QH + q the
// fp16 remainder lo = fp16(v - hi), and cs holds the sums of hi + lo.
template <int BITS, int XF>
struct Stage {
    static constexpr int CC = 128 / BITS;                               // codes per chunk
    static constexpr int QH = BITS == 4 ? 4 : 2;                        // fp16 uint4 per chunk
    static constexpr int QPC = XF == 1 ? CC / 4 : (XF == 2 ? 2 * QH : QH);  // uint4 per chunk
    static constexpr int CSZ = 4;                                       // sum bytes per chunk
    __host__ __device__ static size_t bytes(int nb, int nc) { return (size_t)nb * nc * (QPC * 16 + CSZ); }
    // chunk-major layout for B > 1 vectors (fp16 path, see stage_x_cm)
    __host__ __device__ static size_t bytes_cm(int B, int nc) {
        return (size_t)nc * ((B * QPC + 1) * 16 + (B + 1) * 4);
    }
};

// Slot of chunk c when each lane reads CPL consecutive chunks: chunk c goes
// to (c mod CPL) * (nc / CPL) + c / CPL, so the lanes of a segment read
// consecutive 16-byte slots for each of their CPL chunks (nc is a multiple
// of CPL).
template <int CPL>
__device__ __forceinline__ int xslot(int c, int nc) {
    if constexpr (CPL == 1) return c;
    return (c % CPL) * (nc / CPL) + c / CPL;
}

// Stage chunks [c0, c0 + nc) of activation vector(s) x[b][K] for b < nb into
// lds. xstride = elements between consecutive vectors.
template <int BITS, int XF, int CPL = 1>
__device__ void stage_x(const void* x, int kind, int64_t xstride, int nb, int c0, int nc,
                        uint4* lds) {
    using St = Stage<BITS, XF>;
    constexpr int CC = St::CC;
    constexpr int QPC = St::QPC;
    uint4* xs = lds;
    for (int item = threadIdx.x; item < nb * nc; item += blockDim.x) {
        const int b = item / nc, cc = item - b * nc;
        const int c = xslot<CPL>(cc, nc);   // destination slot of chunk cc
        const int64_t base = (int64_t)b * xstride + (int64_t)(c0 + cc) * CC;
        if constexpr (XF == 0) {
            // fp16 activations, kept as raw bits
            const uint16_t* xp = (const uint16_t*)x + base;
            float s1 = 0.f, s16 = 0.f;
            if constexpr (BITS == 4) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint4 raw = *(const uint4*)(xp + 8 * q);
                    uint16_t h[8];
                    h[0] = raw.x & 0xFFFF; h[1] = raw.x >> 16;
                    h[2] = raw.y & 0xFFFF; h[3] = raw.y >> 16;
                    h[4] = raw.z & 0xFFFF; h[5] = raw.z >> 16;
                    h[6] = raw.w & 0xFFFF; h[7] = raw.w >> 16;
                    uint4 o;
                    o.x = pack_h2(h[0], h[4]);
                    o.y = pack_h2(h[1], h[5]);
                    o.z = pack_h2(h[2], h[6]);
                    o.w = pack_h2(h[3], h[7]);
                    xs[(b * QPC + q) * nc + c] = o;
                    s1 += (h2f(h[0]) + h2f(h[4])) + (h2f(h[2]) + h2f(h[6]));
                    s16 += (h2f(h[1]) + h2f(h[5])) + (h2f(h[3]) + h2f(h[7]));
                }
                float* cs = (float*)(xs + (size_t)nb * QPC * nc);
                cs[b * nc + c] = s1 + s16;
            } else {
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const uint4 raw = *(const uint4*)(xp + 8 * q);   // two words' x (8 values)
                    uint16_t h[8];
                    h[0] = raw.x & 0xFFFF; h[1] = raw.x >> 16;
                    h[2] = raw.y & 0xFFFF; h[3] = raw.y >> 16;
                    h[4] = raw.z & 0xFFFF; h[5] = raw.z >> 16;
                    h[6] = raw.w & 0xFFFF; h[7] = raw.w >> 16;
                    uint4 o;
                    o.x = pack_h2(h[0], h[2]);
                    o.y = pack_h2(h[1], h[3]);
                    o.z = pack_h2(h[4], h[6]);
                    o.w = pack_h2(h[5], h[7]);
                    xs[(b * QPC + q) * nc + c] = o;
#pragma unroll
                    for (int i = 0; i < 8; ++i) s1 += h2f(h[i]);
                }
                float* cs = (float*)(xs + (size_t)nb * QPC * nc);
                cs[b * nc + c] = s1;
            }
        } else {
            float v[CC];
#pragma unroll
            for (int i = 0; i < CC; ++i) v[i] = load_x(x, kind, base + i);
            float sum = 0.f;
#pragma unroll
            for (int i = 0; i < CC; ++i) sum += v[i];
            if constexpr (BITS == 4) {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float* u = v + 8 * w;
                    xs[(b * QPC + 2 * w) * nc + c] =
                        make_uint4(__float_as_uint(u[0]), __float_as_uint(u[4]),
                                   __float_as_uint(u[2]), __float_as_uint(u[6]));
                    xs[(b * QPC + 2 * w + 1) * nc + c] =
                        make_uint4(__float_as_uint(u[1]), __float_as_uint(u[5]),
                                   __float_as_uint(u[3]), __float_as_uint(u[7]));
                }
            } else {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float* u = v + 4 * w;
                    xs[(b * QPC + w) * nc + c] =
                        make_uint4(__float_as_uint(u[0]), __float_as_uint(u[2]),
                                   __float_as_uint(u[1]), __float_as_uint(u[3]));
                }
            }
            float* cs = (float*)(xs + (size_t)nb * QPC * nc);
            cs[b * nc + c] = sum;
        }
    }
}

// Chunk-major staging of B fp16 vectors (the XF = 0 values and sums of
// stage_x, rearranged):
//   xs[c][b][q]  uint4, slot c at a stride of SC = B*QPC + 1 uint4 (the pad
//                puts the 8 lanes of one LDS cycle in distinct banks);
//   cs[c][b]     float, slot c at a stride of B + 1 floats.
// Every (vector, quarter) of a chunk then sits at a compile-time offset from
// the chunk's base, so the reads in group_rows take immediate offsets
// instead of one address add each. Vectors b >= nb are not staged; their
// results are never stored.
template <int BITS, int B, int CPL>
struct StageCm {
    using St = Stage<BITS, 0>;
    static constexpr int CC = St::CC;
    static constexpr int QPC = St::QPC;
    static constexpr int SC = B * QPC + 1;
    static constexpr int NQ = BITS == 4 ? 4 : 2;   // uint4 of fp16 per chunk
    __device__ static __forceinline__ const uint16_t* src(const void* x, int64_t xstride, int nc,
                                                          int c0, int item) {
        const int b = item / nc, cc = item - b * nc;
        return (const uint16_t*)x + (int64_t)b * xstride + (int64_t)(c0 + cc) * CC;
    }
    __device__ static __forceinline__ void put(int nc, uint4* lds, int item, const uint4 (&raw)[NQ]) {
        uint4* xs = lds;
        float* cs = (float*)(xs + (size_t)nc * SC);
        const int b = item / nc, cc = item - b * nc;
        const int c = xslot<CPL>(cc, nc);
        float s1 = 0.f, s16 = 0.f;
        if constexpr (BITS == 4) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 r = raw[q];
                uint16_t h[8];
                h[0] = r.x & 0xFFFF; h[1] = r.x >> 16;
                h[2] = r.y & 0xFFFF; h[3] = r.y >> 16;
                h[4] = r.z & 0xFFFF; h[5] = r.z >> 16;
                h[6] = r.w & 0xFFFF; h[7] = r.w >> 16;
                xs[c * SC + b * QPC + q] = make_uint4(pack_h2(h[0], h[4]), pack_h2(h[1], h[5]),
                                                      pack_h2(h[2], h[6]), pack_h2(h[3], h[7]));
                s1 += (h2f(h[0]) + h2f(h[4])) + (h2f(h[2]) + h2f(h[6]));
                s16 += (h2f(h[1]) + h2f(h[5])) + (h2f(h[3]) + h2f(h[7]));
            }
            cs[c * (B + 1) + b] = s1 + s16;
        } else {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const uint4 r = raw[q];
                uint16_t h[8];
                h[0] = r.x & 0xFFFF; h[1] = r.x >> 16;
                h[2] = r.y & 0xFFFF; h[3] = r.y >> 16;
                h[4] = r.z & 0xFFFF; h[5] = r.z >> 16;
                h[6] = r.w & 0xFFFF; h[7] = r.w >> 16;
                xs[c * SC + b * QPC + q] = make_uint4(pack_h2(h[0], h[2]), pack_h2(h[1], h[3]),
                                                      pack_h2(h[4], h[6]), pack_h2(h[5], h[7]));
#pragma unroll
                for (int i = 0; i < 8; ++i) s1 += h2f(h[i]);
            }
            cs[c * (B + 1) + b] = s1;
        }
    }
};

template <int BITS, int B, int CPL>
__device__ void stage_x_cm(const void* x, int64_t xstride, int nb, int c0, int nc, uint4* lds) {
    using S = StageCm<BITS, B, CPL>;
    for (int item = threadIdx.x; item < nb * nc; item += blockDim.x) {
        uint4 raw[S::NQ];
        const uint16_t* xp = S::src(x, xstride, nc, c0, item);
#pragma unroll
        for (int q = 0; q < S::NQ; ++q) raw[q] = *(const uint4*)(xp + 8 * q);
        S::put(nc, lds, item, raw);
    }
}

// The same with the caller's loads (after_loads) issued behind each
// thread's first activation chunk. Vector-memory counters complete in
// order, so the activation waits do not wait for those loads; the first
// chunk's loads are unconditional (clamped index) and its LDS writes sit in
// a branch without loads, so the compiler's counter bookkeeping stays exact
// (a load under a branch would make it wait for everything at the join).
// Further chunks of a thread (more chunks than threads) wait for all.
template <int BITS, int B, int CPL, typename F>
__device__ __forceinline__ void stage_x_cm_overlap(const void* x, int64_t xstride, int nb, int c0,
                                                   int nc, uint4* lds, F&& after_loads) {
    using S = StageCm<BITS, B, CPL>;
    const int items = nb * nc;
    const int i0 = min((int)threadIdx.x, items - 1);
    uint4 raw[S::NQ];
    {
        const uint16_t* xp = S::src(x, xstride, nc, c0, i0);
#pragma unroll
        for (int q = 0; q < S::NQ; ++q) raw[q] = *(const uint4*)(xp + 8 * q);
    }
    __builtin_amdgcn_sched_barrier(0);
    after_loads();
    __builtin_amdgcn_sched_barrier(0);
    if ((int)threadIdx.x < items) S::put(nc, lds, i0, raw);
    for (int item = threadIdx.x + blockDim.x; item < items; item += blockDim.x) {
        const uint16_t* xp = S::src(x, xstride, nc, c0, item);
#pragma unroll
        for (int q = 0; q < S::NQ; ++q) raw[q] = *(const uint4*)(xp + 8 * q);
        S::put(nc, lds, item, raw);
    }
}

// ---------------------------------------------------------------------------
// Rotation prologue (XF = 2): discuss.pytorch.kr/t/uzu-mac-iphone-llm-apple-
// silicon-rust/12363 (uzu), section "uzu의 모델 변환과 Mirai 양자화 형식"
// (model conversion and the Mirai quantization formats): weights are
// quantized after a random Hadamard transform of block size 32, and the
// transform is fused with RMSNorm and the matmul. Each staged block of 32
// inputs becomes
//     v = 2^-2.5 * r * H_32 * D * (x * gamma),   r = 1 / sqrt(mean(x^2) + eps),
// H_32 the Sylvester Hadamard matrix and D the block's random signs. A pair
// of adjacent lanes takes a block, 16 inputs each: four butterfly stages in
// registers and the last one across the pair (one DPP move and one fma per
// value). Staging runs in two passes over LDS: the first writes the
// unnormalized transform in fp32 while summing x^2 and tracking
// max |H D (x gamma)|; after one reduction the second scales by
// r * 2^-2.5 * 2^e (2^e a power of two that keeps |v| below 2^14) and
// rewrites each lane's own slots in place as two fp16 planes, hi = v rounded
// toward zero and lo = (v - hi) rounded toward zero, so hi + lo is v to about
// 2^-20 relative. The kernel multiplies its result by 2^-e. Blocks are 32
// inputs: one chunk of 4-bit codes or two chunks of 8-bit codes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void fwht16(float (&v)[16]) {
#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
        for (int i = 0; i < 16; i += 2 * h)
#pragma unroll
            for (int j = i; j < i + h; ++j) {
                const float a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
}

// The value of lane ^ 1.
__device__ __forceinline__ float pair_swap(float v) {
    // quad_perm [1, 0, 3, 2]
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}

// 8 consecutive elements of x (f16 or bf16 bits) as fp32.
__device__ __forceinline__ void load8(const uint16_t* p, int kind, float (&o)[8]) {
    const uint4 raw = *(const uint4*)p;
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint16_t a = w[i] & 0xFFFF, b = w[i] >> 16;
        o[2 * i] = kind == X_F16 ? h2f(a) : bf2f(a);
        o[2 * i + 1] = kind == X_F16 ? h2f(b) : bf2f(b);
    }
}

__device__ __forceinline__ void cvt8(uint4 raw, int kind, float (&o)[8]) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint16_t a = w[i] & 0xFFFF, b = w[i] >> 16;
        o[2 * i] = kind == X_F16 ? h2f(a) : bf2f(a);
        o[2 * i + 1] = kind == X_F16 ? h2f(b) : bf2f(b);
    }
}

// hi/lo fp16 pairs of (a, b), and the fp32 sum of hi + lo added to s.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo, float& s) {
    typedef __fp16 fp16x2 __attribute__((ext_vector_type(2)));
    const fp16x2 h = __builtin_amdgcn_cvt_pkrtz(a, b);
    const fp16x2 l = __builtin_amdgcn_cvt_pkrtz(a - (float)h.x, b - (float)h.y);
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, l);
    s = dot2(hi, 0x3C003C00u, s);   // (1.0, 1.0)
    s = dot2(lo, 0x3C003C00u, s);
}

constexpr int kRotMaxB = 8;    // vectors per launch
constexpr int kRotWaves = 16;  // waves per workgroup
// LDS floats the rotation prologue needs besides the staged planes.
constexpr int kRotShared = 2 * kRotMaxB * kRotWaves + 2 * kRotMaxB;

// Stage chunks [c0, c0 + nc) of the rotated x[b][K] (b < nb); gamma (K, x's
// kind) and signs (K/32 words) may be NULL. rs is kRotShared floats of LDS;
// on return rs[kRotMaxB + b] holds 2^-e of vector b. Every thread must call.
// after_loads() runs once per thread, right after the thread's first
// activation loads are issued (or before the first barrier if it has none):
// loads the caller issues there return after the activations (a wave's
// loads return in order), so the transform overlaps their latency.
template <int BITS, int CPL, typename F>
__device__ __forceinline__ void stage_x_rot(const uint16_t* x, int kind, int K, int nb, int c0,
                                            int nc, const uint16_t* gamma, const uint32_t* signs,
                                            float eps, float* rs, uint4* lds, F&& after_loads) {
    bool issued = false;
    using St = Stage<BITS, 2>;
    constexpr int CC = St::CC, QH = St::QH, QPC = St::QPC;
    constexpr int CPB = 32 / CC;   // chunks per block
    const int nblk = nc / CPB;
    uint4* xs = lds;
    float* cs = (float*)(xs + (size_t)nb * QPC * nc);
    float* mulv = rs;                        // [kRotMaxB]
    float* unscale = rs + kRotMaxB;          // [kRotMaxB]
    float* red = rs + 2 * kRotMaxB;          // [2][kRotMaxB][kRotWaves]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    const int hh = lane & 1;                 // half of the block this lane holds
    // Slot i < 4 of this lane's half of block bl: the LDS uint4 that receives
    // its inputs 4i..4i+3 in pass 1 and the planes built from them in pass 2
    // (4-bit: hi and lo planes of words 2hh, 2hh + 1; 8-bit: chunk hh).
    auto slot = [&](int b, int bl, int i) -> uint4* {
        if constexpr (BITS == 4)
            return xs + (size_t)(b * QPC + (i & 1) + 2 * hh + QH * (i >> 1)) * nc +
                   xslot<CPL>(bl, nc);
        else
            return xs + (size_t)(b * QPC + i) * nc + xslot<CPL>(bl * 2 + hh, nc);
    };

    // pass 1: each vector's blocks go to wpb waves, so sums stay per wave
    const int wpb = max(1, nwaves / nb);
    const int ngroups = min(nb, nwaves / wpb);
    if (wave < ngroups * wpb) {
        const int wg = wave % wpb;
        const float sgn = hh ? -1.f : 1.f;
        for (int b = wave / wpb; b < nb; b += ngroups) {
            const uint16_t* xb = x + (int64_t)b * K;
            float ss = 0.f, mx = 0.f;
            // both lanes of a pair run the same iterations
            for (int bl = (wg * 64 + lane) >> 1; bl < nblk; bl += wpb * 32) {
                const int k0 = (c0 + bl * CPB) * CC + 16 * hh;
                const uint32_t sg = signs ? signs[k0 / 32] >> (16 * hh) : 0u;
                float v[16];
                uint4 xr[2], gr[2];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    xr[q] = *(const uint4*)(xb + k0 + 8 * q);
                    if (gamma) gr[q] = *(const uint4*)(gamma + k0 + 8 * q);
                }
                if (!issued) {   // the caller's loads go out behind these
                    __builtin_amdgcn_sched_barrier(0);
                    after_loads();
                    __builtin_amdgcn_sched_barrier(0);
                    issued = true;
                }
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    float t[8], g[8];
                    cvt8(xr[q], kind, t);
                    if (gamma) {
                        cvt8(gr[q], kind, g);
                    } else {
#pragma unroll
                        for (int i = 0; i < 8; ++i) g[i] = 1.f;
                    }
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        ss = fmaf(t[i], t[i], ss);
                        const uint32_t neg = (sg << (31 - (8 * q + i))) & 0x80000000u;
                        v[8 * q + i] = t[i] * __uint_as_float(__float_as_uint(g[i]) ^ neg);
                    }
                }
                fwht16(v);
                // last stage: even lane a + b, odd lane a - b (a the even lane's)
#pragma unroll
                for (int j = 0; j < 16; ++j) v[j] = fmaf(v[j], sgn, pair_swap(v[j]));
#pragma unroll
                for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fabsf(v[j]));
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *slot(b, bl, i) = make_uint4(__float_as_uint(v[4 * i]), __float_as_uint(v[4 * i + 1]),
                                                 __float_as_uint(v[4 * i + 2]), __float_as_uint(v[4 * i + 3]));
            }
            if (gamma && nc * CC < K) {
                // a split chunk range: the norm still covers the whole vector
                for (int kb = wg * 64 + lane; kb < K / 32; kb += wpb * 64) {
                    if (kb * 32 >= c0 * CC && kb * 32 < (c0 + nc) * CC) continue;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float t[8];
                        load8(xb + kb * 32 + 8 * q, kind, t);
#pragma unroll
                        for (int i = 0; i < 8; ++i) ss = fmaf(t[i], t[i], ss);
                    }
                }
            }
            ss = seg_sum<64>(ss);
            mx = wave_max_f(mx);
            if (lane == 0) {
                red[b * kRotWaves + wg] = ss;
                red[(kRotMaxB + b) * kRotWaves + wg] = mx;
            }
        }
    }
    if (!issued) after_loads();
    __syncthreads();
    if (threadIdx.x < nb) {
        const int b = threadIdx.x;
        float S = 0.f, M = 0.f;
        for (int w = 0; w < wpb; ++w) {
            S += red[b * kRotWaves + w];
            M = fmaxf(M, red[(kRotMaxB + b) * kRotWaves + w]);
        }
        constexpr float kNorm = 0.17677669529663688f;   // 2^-2.5
        const float r = gamma ? 1.f / sqrtf(S / (float)K + eps) : 1.f;
        const float bound = r * M * kNorm;              // max |v|, up to rounding
        // bound < 2^E with E from the exponent field; then 2^e bound < 2^14
        int e = 0;
        if (bound > 0.f && bound <= 3.0e38f) {
            const int E = max((int)((__float_as_uint(bound) >> 23) & 0xFF), 1) - 126;
            e = min(max(14 - E, -120), 120);
        }
        mulv[b] = r * __uint_as_float((uint32_t)(e + 127) << 23) * kNorm;
        unscale[b] = __uint_as_float((uint32_t)(127 - e) << 23);
    }
    __syncthreads();

    // pass 2: each lane scales its own 16 values and rewrites its slots as
    // hi/lo planes; class sums of a 4-bit chunk combine across the pair
    for (int t = threadIdx.x; t < 2 * nb * nblk; t += blockDim.x) {
        const int item = t >> 1;   // t & 1 == hh, since blockDim.x is even
        const int b = item / nblk, bl = item - b * nblk;
        const float m = mulv[b];
        float v[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 u = *slot(b, bl, i);
            v[4 * i] = __uint_as_float(u.x) * m;
            v[4 * i + 1] = __uint_as_float(u.y) * m;
            v[4 * i + 2] = __uint_as_float(u.z) * m;
            v[4 * i + 3] = __uint_as_float(u.w) * m;
        }
        float s1 = 0.f, s16 = 0.f;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const float* w = v + 8 * q;
            uint32_t h[4], l[4];
            if constexpr (BITS == 4) {
                // pairs (0,4), (2,6) hold the codes of nibbles 0, 2, 4, 6 (class 1)
                split_pair(w[0], w[4], h[0], l[0], s1);
                split_pair(w[1], w[5], h[1], l[1], s16);
                split_pair(w[2], w[6], h[2], l[2], s1);
                split_pair(w[3], w[7], h[3], l[3], s16);
            } else {
                split_pair(w[0], w[2], h[0], l[0], s1);
                split_pair(w[1], w[3], h[1], l[1], s1);
                split_pair(w[4], w[6], h[2], l[2], s1);
                split_pair(w[5], w[7], h[3], l[3], s1);
            }
            // hi plane of word q -> slot q, lo plane -> slot 2 + q
            *slot(b, bl, q) = make_uint4(h[0], h[1], h[2], h[3]);
            *slot(b, bl, 2 + q) = make_uint4(l[0], l[1], l[2], l[3]);
        }
        if constexpr (BITS == 4) {
            s1 += pair_swap(s1);   // the chunk's 32 inputs span both lanes
            s16 += pair_swap(s16);
            if (hh == 0) cs[b * nc + xslot<CPL>(bl, nc)] = s1 + s16;
        } else {
            cs[b * nc + xslot<CPL>(bl * 2 + hh, nc)] = s1;
        }
    }
}

// Centred code pairs of one word: the four half2 that the dot products take.
// 4-bit: (q0, q4), 16 (q1, q5), (q2, q6), 16 (q3, q7), each minus the
// centre; 8-bit (two words w0, w1): (q0, q2), (q1, q3) of each word.
template <int BITS>
__device__ __forceinline__ void centred_pairs(uint32_t w0, uint32_t w1, uint32_t magic, uint32_t n1,
                                              uint32_t n16, uint32_t (&p)[4]) {
    if constexpr (BITS == 4) {
        (void)w1;
        const uint32_t w8 = w0 >> 8;
        p[0] = pk_addh((w0 & 0x000F000Fu) | magic, n1);    // q0 - c, q4 - c
        p[1] = pk_addh((w0 & 0x00F000F0u) | magic, n16);   // 16 (q1 - c), 16 (q5 - c)
        p[2] = pk_addh((w8 & 0x000F000Fu) | magic, n1);    // q2 - c, q6 - c
        p[3] = pk_addh((w8 & 0x00F000F0u) | magic, n16);   // 16 (q3 - c), 16 (q7 - c)
    } else {
        p[0] = pk_addh((w0 & 0x00FF00FFu) | magic, n1);            // q0 - c, q2 - c
        p[1] = pk_addh(((w0 >> 8) & 0x00FF00FFu) | magic, n1);     // q1 - c, q3 - c
        p[2] = pk_addh((w1 & 0x00FF00FFu) | magic, n1);
        p[3] = pk_addh(((w1 >> 8) & 0x00FF00FFu) | magic, n1);
    }
}

// Partial dot products of NCH consecutive 16-byte code chunks (one lane's
// share of a group) of each of R rows with every activation vector b < B,
// followed by one epilogue into y[r][b]:
//   y[r][b] += sc_r * (sum_k (q_k - c_r) x_k) + bi_r * (sum_k x_k),
// with the centre c_r given by the subtrahend pairs n1_r (class 1) and
// n16_r (class 16; 8-bit codes use n1_r only). The second term is left out
// when XSUM is false. The chunks' activations are read from LDS once and
// shared by the R rows; slot[i] is the staged slot of chunk i.
template <int BITS, int XF, int B, int R, int NCH, bool CM = false, bool XSUM = true>
__device__ __forceinline__ void group_rows(const uint4 (&cw)[NCH][R], const float (&sc)[R],
                                           const float (&bi)[R], const uint32_t (&n1)[R],
                                           const uint32_t (&n16)[R], const uint4* lds,
                                           int nb_staged, int nc, const int (&slot)[NCH],
                                           uint32_t magic, float (&y)[R][B]) {
    using St = Stage<BITS, XF>;
    constexpr int QPC = St::QPC;
    constexpr int QH = St::QH;
    constexpr int NPL = XF == 2 ? 2 : 1;   // fp16 planes: value, or hi and lo
    const uint4* xs = lds;
    static_assert(!CM || XF == 0, "chunk-major staging is for fp16 activations");
    constexpr int SC = B * QPC + 1;   // chunk-major slot stride (uint4)
    const float* cs = CM ? (const float*)(xs + (size_t)nc * SC)
                         : (const float*)(xs + (size_t)nb_staged * QPC * nc);
    float a1[R][B], a16[R][B];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) a1[r][b] = a16[r][b] = 0.f;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        const int c = slot[ch];
        // a 4-bit chunk is 4 steps of one word, an 8-bit chunk 2 steps of two
#pragma unroll
        for (int q = 0; q < QH; ++q) {
            if constexpr (XF == 0 || XF == 2) {
                uint4 xq[NPL][B];   // plane 1 (if any): the fp16 remainders
#pragma unroll
                for (int pl = 0; pl < NPL; ++pl)
#pragma unroll
                    for (int b = 0; b < B; ++b)
                        xq[pl][b] = CM ? xs[c * SC + b * QPC + q] : xs[(b * QPC + pl * QH + q) * nc + c];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint4& w4 = cw[ch][r];
                    uint32_t p[4];
                    if constexpr (BITS == 4)
                        centred_pairs<4>(q == 0 ? w4.x : q == 1 ? w4.y : q == 2 ? w4.z : w4.w, 0u,
                                         magic, n1[r], n16[r], p);
                    else
                        centred_pairs<8>(q == 0 ? w4.x : w4.z, q == 0 ? w4.y : w4.w, magic, n1[r],
                                         n1[r], p);
#pragma unroll
                    for (int pl = 0; pl < NPL; ++pl)
#pragma unroll
                        for (int b = 0; b < B; ++b) {
                            a1[r][b] = dot2(p[0], xq[pl][b].x, a1[r][b]);
                            a16[r][b] = dot2(p[1], xq[pl][b].y, a16[r][b]);
                            a1[r][b] = dot2(p[2], xq[pl][b].z, a1[r][b]);
                            a16[r][b] = dot2(p[3], xq[pl][b].w, a16[r][b]);
                        }
                }
            } else {
                // fp32 activations: 4-bit word q as (x0,x4,x2,x6), (x1,x5,x3,x7);
                // 8-bit words 2q, 2q + 1 as (x0,x2,x1,x3) each
                uint4 xa[B], xb[B];
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    xa[b] = xs[(b * QPC + 2 * q) * nc + c];
                    xb[b] = xs[(b * QPC + 2 * q + 1) * nc + c];
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint4& w4 = cw[ch][r];
                    uint32_t p[4];
                    if constexpr (BITS == 4)
                        centred_pairs<4>(q == 0 ? w4.x : q == 1 ? w4.y : q == 2 ? w4.z : w4.w, 0u,
                                         magic, n1[r], n16[r], p);
                    else
                        centred_pairs<8>(q == 0 ? w4.x : w4.z, q == 0 ? w4.y : w4.w, magic, n1[r],
                                         n1[r], p);
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const float4 fa = *(const float4*)&xa[b];
                        const float4 fb = *(const float4*)&xb[b];
                        if constexpr (BITS == 4) {
                            a1[r][b] = fma_pair(p[0], fa.x, fa.y, a1[r][b]);
                            a1[r][b] = fma_pair(p[2], fa.z, fa.w, a1[r][b]);
                            a16[r][b] = fma_pair(p[1], fb.x, fb.y, a16[r][b]);
                            a16[r][b] = fma_pair(p[3], fb.z, fb.w, a16[r][b]);
                        } else {
                            a1[r][b] = fma_pair(p[0], fa.x, fa.y, a1[r][b]);
                            a16[r][b] = fma_pair(p[1], fa.z, fa.w, a16[r][b]);
                            a1[r][b] = fma_pair(p[2], fb.x, fb.y, a1[r][b]);
                            a16[r][b] = fma_pair(p[3], fb.z, fb.w, a16[r][b]);
                        }
                    }
                }
            }
        }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
        float xsum = 0.f;
        if constexpr (XSUM) {
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch)
                xsum += CM ? cs[slot[ch] * (B + 1) + b] : cs[b * nc + slot[ch]];
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float p = BITS == 4 ? fmaf(a16[r][b], 0.0625f, a1[r][b]) : a1[r][b] + a16[r][b];
            y[r][b] = fmaf(sc[r], p, y[r][b]);
            if constexpr (XSUM) y[r][b] = fmaf(bi[r], xsum, y[r][b]);
        }
    }
}

}  // namespace qd
