// MFMA helpers shared by the prefill kernels (gfx950, v_mfma_f32_32x32x16_bf16).
//
// Operand layouts (verified on the device): for A (32 x 16) and B (16 x 32)
// lane l holds row/column l mod 32 and k = 8 (l div 32) + i, i < 8; the
// 16 results of lane l sit in column l mod 32, rows 8 (i div 4) + 4 (l div 32)
// + (i mod 4).
#pragma once

#include "common.h"

namespace qd {

// uint4 per staged operand row: 8 of data (64 bf16) + 1 of padding, so the 32
// rows an MFMA operand read touches fall in distinct LDS banks.
constexpr int XS_STRIDE = 9;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// 8 codes of one word -> 16-bit (off + q) in natural k order: the nibble in
// the low mantissa of magic (per half: 0x4300 = bf16 128, 0x6400 = fp16 1024).
__device__ __forceinline__ uint4 codes_to_16n(uint32_t w, uint32_t magic) {
    const uint32_t t = w & 0x0F0F0F0Fu;         // q0 q2 q4 q6 in bytes 0..3
    const uint32_t u = (w >> 4) & 0x0F0F0F0Fu;  // q1 q3 q5 q7
    // v_perm_b32(u, t, sel): selector bytes 0..3 pick t's bytes, 4..7 u's, 0x0C gives 0
    const uint32_t p01 = __builtin_amdgcn_perm(u, t, 0x0C040C00u) | magic;
    const uint32_t p23 = __builtin_amdgcn_perm(u, t, 0x0C050C01u) | magic;
    const uint32_t p45 = __builtin_amdgcn_perm(u, t, 0x0C060C02u) | magic;
    const uint32_t p67 = __builtin_amdgcn_perm(u, t, 0x0C070C03u) | magic;
    return make_uint4(p01, p23, p45, p67);
}

// ---------------------------------------------------------------------------
// Centred codes as matrix-core operands: w = s (q - c) + (b + c s), with the
// operand holding q - c exactly, so the fp32 products and sums carry no
// offset and a weight at the centre contributes exactly zero.
//  * fp16 operands: the code in the low mantissa of fp16 1024.0 is 1024 + q;
//    one v_pk_add_f16 with -(1024 + c) leaves q - c (exact in fp16).
//  * bf16 operands (no packed bf16 add on gfx950): a 4-bit code XOR 8, read
//    as a signed nibble, is q - 8; placed in the top half of a byte it reads
//    as the signed byte 16 (q - 8), which v_cvt_f32_i32 (SDWA byte select,
//    sign-extended) converts exactly and v_cvt_pk_bf16_f32 packs exactly
//    (|16 (q - 8)| <= 128 needs 4 significant bits). The factor 16 is taken
//    out of the scale (an exact power of two). An 8-bit code XOR 0x80 is the
//    signed byte q - 128, exact in bf16 (at most 8 significant bits).
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    const bf16x2_t v = {(__bf16)a, (__bf16)b};   // exact for these integers
    return __builtin_bit_cast(uint32_t, v);
}

// Byte I of v as a signed integer, in fp32.
template <int I>
__device__ __forceinline__ float sbyte(uint32_t v) {
    return (float)(int8_t)(v >> (8 * I));
}

// 8 codes of one word, natural k order, as fp16 q - 8.
__device__ __forceinline__ uint4 codes_centred_f16(uint32_t w) {
    const uint4 p = codes_to_16n(w, 0x64006400u);
    return make_uint4(pk_addh(p.x, kNeg1032), pk_addh(p.y, kNeg1032), pk_addh(p.z, kNeg1032),
                      pk_addh(p.w, kNeg1032));
}

// 8 codes of one word, natural k order, as bf16 16 (q - 8).
__device__ __forceinline__ uint4 codes_centred_bf16x16(uint32_t w) {
    const uint32_t c = w ^ 0x88888888u;
    const uint32_t lo = (c << 4) & 0xF0F0F0F0u;   // codes 0, 2, 4, 6 in the top of bytes 0..3
    const uint32_t hi = c & 0xF0F0F0F0u;          // codes 1, 3, 5, 7
    return make_uint4(pk_bf16(sbyte<0>(lo), sbyte<0>(hi)), pk_bf16(sbyte<1>(lo), sbyte<1>(hi)),
                      pk_bf16(sbyte<2>(lo), sbyte<2>(hi)), pk_bf16(sbyte<3>(lo), sbyte<3>(hi)));
}

// The same in the k order [0, 4, 1, 5, 2, 6, 3, 7] (fp16: the magic in a VGPR).
__device__ __forceinline__ uint4 codes_centred_f16_p(uint32_t w, uint32_t magic) {
    return make_uint4(pk_addh((w & 0x000F000Fu) | magic, kNeg1032),
                      pk_addh(((w >> 4) & 0x000F000Fu) | magic, kNeg1032),
                      pk_addh(((w >> 8) & 0x000F000Fu) | magic, kNeg1032),
                      pk_addh(((w >> 12) & 0x000F000Fu) | magic, kNeg1032));
}

__device__ __forceinline__ uint4 codes_centred_bf16x16_p(uint32_t w) {
    const uint32_t c = w ^ 0x88888888u;
    const uint32_t lo = (c << 4) & 0xF0F0F0F0u;
    const uint32_t hi = c & 0xF0F0F0F0u;
    return make_uint4(pk_bf16(sbyte<0>(lo), sbyte<2>(lo)), pk_bf16(sbyte<0>(hi), sbyte<2>(hi)),
                      pk_bf16(sbyte<1>(lo), sbyte<3>(lo)), pk_bf16(sbyte<1>(hi), sbyte<3>(hi)));
}

// ---------------------------------------------------------------------------
// Codes through the fp8 converter: a byte 0000qqqq read as OCP E4M3 is
// exactly q 2^-9 (exponent field 0 or 1 with the code's top bit, mantissa
// its low three bits: the subnormal and first normal binade join up), so
// v_cvt_scalef32_pk_{bf16,f16}_fp8 with scale 2^9 turns two such bytes into
// the codes themselves, exactly, in one instruction. 8 codes of one word,
// natural k order: the nibbles are first spread to bytes (2 ANDs, 1 shift,
// 2 byte permutes), then 4 conversions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint2 codes_to_bytes(uint32_t w) {
    const uint32_t t = w & 0x0F0F0F0Fu;          // q0 q2 q4 q6
    const uint32_t u = (w >> 4) & 0x0F0F0F0Fu;   // q1 q3 q5 q7
    // v_perm_b32(u, t, sel): selector bytes 0..3 pick t's bytes, 4..7 u's
    return make_uint2(__builtin_amdgcn_perm(u, t, 0x05010400u), __builtin_amdgcn_perm(u, t, 0x07030602u));
}

__device__ __forceinline__ uint4 codes_bf16(uint32_t w) {
    const uint2 b = codes_to_bytes(w);
    return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b.x, 512.f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b.x, 512.f, true)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b.y, 512.f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b.y, 512.f, true)));
}

__device__ __forceinline__ uint4 codes_f16(uint32_t w) {
    const uint2 b = codes_to_bytes(w);
    return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.x, 512.f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.x, 512.f, true)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.y, 512.f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.y, 512.f, true)));
}

// 4 8-bit codes of one word, natural order, as two bf16 pairs q - 128.
__device__ __forceinline__ uint2 bytes_centred_bf16(uint32_t w) {
    const uint32_t c = w ^ 0x80808080u;
    return make_uint2(pk_bf16(sbyte<0>(c), sbyte<1>(c)), pk_bf16(sbyte<2>(c), sbyte<3>(c)));
}

// ---------------------------------------------------------------------------
// Bias products on the matrix core: acc[m][n] += X[m] V[n] with fp32 factors
// (a group's row sum and its b + c s). With centred codes this term cancels
// against s P where weights sit near zero, so it must be about as exact as
// an fp32 product. Each factor is split into three bf16 parts a = hi + mid +
// lo (each part the rounding of what the earlier ones leave; every residual
// is exact in fp32, so the parts hold 24 significant bits and miss a by at
// most 2^-27 |a|). The six cross products of weight down to 2^-18 fill six
// K slots of one lane half: A = (xh, xm, xl, xh, xm, xh, 0, 0) against
// B = (vh, vh, vh, vm, vm, vl, 0, 0); the dropped ones (xm vl, xl vm, xl vl)
// are below 2^-26 |x v|. Each product is exact in fp32.
// ---------------------------------------------------------------------------
struct Bf16x3 {
    uint32_t h, m, l;   // bf16 bits in the low half
};

__device__ __forceinline__ uint32_t bf16_bits(float a) {
    return __builtin_bit_cast(uint16_t, (__bf16)a);   // round to nearest even
}

__device__ __forceinline__ Bf16x3 split3_bf16(float a) {
    const uint32_t h = bf16_bits(a);
    const float r1 = a - __uint_as_float(h << 16);
    const uint32_t m = bf16_bits(r1);
    const float r2 = r1 - __uint_as_float(m << 16);
    return {h, m, bf16_bits(r2)};
}

// Row factor as staged in LDS: (hi | mid << 16, lo | hi << 16).
__device__ __forceinline__ uint2 bias_row_parts(float x) {
    const Bf16x3 p = split3_bf16(x);
    return make_uint2(p.h | (p.m << 16), p.l | (p.h << 16));
}

// A operand of one lane half from the staged parts: (xh, xm, xl, xh, xm, xh, 0, 0).
__device__ __forceinline__ uint4 bias_a_operand(uint2 r) {
    return make_uint4(r.x, r.y, (r.x >> 16) | (r.x << 16), 0u);
}

// B operand of one lane half: (vh, vh, vh, vm, vm, vl, 0, 0).
__device__ __forceinline__ uint4 bias_b_operand(float v) {
    const Bf16x3 p = split3_bf16(v);
    return make_uint4(p.h | (p.h << 16), p.h | (p.m << 16), p.m | (p.l << 16), 0u);
}

__device__ __forceinline__ float bf16_pair_sum(uint32_t v, float acc) {
    // v_dot2_f32_bf16 with (1, 1): adds both bf16 halves into an fp32 sum
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v), ones, acc, false);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f2bf_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf2f_bits(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

}  // namespace qd
