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

// ---------------------------------------------------------------------------
// 8-bit codes as matrix-core operands (the router over a token chunk): a
// code XOR 0x80 is the signed byte q - 128, which v_cvt_f32_i32 (SDWA byte
// select, sign-extended) converts exactly and v_cvt_pk_bf16_f32 packs
// exactly (at most 8 significant bits); see bytes_centred_bf16 below.
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

// The same codes in the k order [0, 4, 1, 5, 2, 6, 3, 7] (bytes q0 q4 q1 q5
// and q2 q6 q3 q7 before the conversions).
__device__ __forceinline__ uint2 codes_to_bytes_p(uint32_t w) {
    const uint32_t t = w & 0x0F0F0F0Fu;          // q0 q2 q4 q6
    const uint32_t u = (w >> 4) & 0x0F0F0F0Fu;   // q1 q3 q5 q7
    return make_uint2(__builtin_amdgcn_perm(u, t, 0x06040200u), __builtin_amdgcn_perm(u, t, 0x07050301u));
}

template <bool F16>
__device__ __forceinline__ uint4 codes_p(uint32_t w) {
    const uint2 b = codes_to_bytes_p(w);
    if constexpr (F16)
        return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.x, 512.f, false)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.x, 512.f, true)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.y, 512.f, false)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.y, 512.f, true)));
    else
        return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b.x, 512.f, false)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b.x, 512.f, true)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b.y, 512.f, false)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b.y, 512.f, true)));
}

// 4 8-bit codes of one word, natural order, as two bf16 pairs q - 128.
__device__ __forceinline__ uint2 bytes_centred_bf16(uint32_t w) {
    const uint32_t c = w ^ 0x80808080u;
    return make_uint2(pk_bf16(sbyte<0>(c), sbyte<1>(c)), pk_bf16(sbyte<2>(c), sbyte<3>(c)));
}

// ---------------------------------------------------------------------------
// Bias products on the matrix core: acc[m][n] += X[m] V[n] with fp32 factors
// (a group's row sum and its bias, or b + c s for an operand centred at c).
// Where weights sit near zero (b ~ -q s) this term cancels against s P, so
// it must be about as exact as an fp32 product. Each factor is split into three bf16 parts a = hi + mid +
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
