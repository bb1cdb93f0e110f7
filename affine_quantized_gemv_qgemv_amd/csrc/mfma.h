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

__device__ __forceinline__ float bf16_pair_sum(uint32_t v, float acc) {
    // v_dot2_f32_bf16 with (1, 1): adds both bf16 halves into an fp32 sum
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
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
