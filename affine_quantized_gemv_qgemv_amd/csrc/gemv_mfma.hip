// GEMV of 2..8 activation vectors on the matrix core for gfx950:
// y[b][n] = sum_k w[n][k] x[b][k] with MLX affine 4-bit weights (group 64,
// w = s q + b) and fp16 activations (the launch policy sends batch 3..8
// here).
//
// [TF] jeff.news/article/5193, section "성능과 제약" (performance and
// constraints): 4-bit affine group-64 weights; the decode GEMV is the hot
// contraction. With several activation vectors the packed-dot GEMV spends
// one v_dot2 per code pair and vector, so its VALU work grows with the batch
// until it, not HBM, bounds the kernel. Here the codes go through
// v_mfma_f32_16x16x32_f16 instead:
//
//  * B operand = codes. Lane l of a wave holds column n = l mod 16 (a weight
//    row of the 16-row tile) and the 8 k values 8 (l div 16) + i of each
//    MFMA: exactly one 32-bit word of 8 codes. A step is 128 inputs (two
//    groups, 16 words per row): lane (n, j) loads words 4j..4j+3 of its row
//    with one 16-byte load, and MFMA t of the step takes word 4j + t. The
//    codes are unpacked exactly and centred, (q - 8) in fp16, with the
//    packed-dot GEMV's magic-number pairs, so a weight at its group's bias
//    point adds exactly zero.
//  * A operand = activations, read from LDS. Words 4j + t belong to group
//    j div 2 of the step, so every MFMA mixes the step's two groups across
//    its k blocks. The batch (at most 8) leaves rows 8..15 of A unused, and
//    they take the second group: row m < 8 holds x[m] on the k blocks of
//    group 0 (j < 2) and zero elsewhere, row 8 + m holds x[m] on those of
//    group 1 (j >= 2). Lane (n, j) of the result then holds rows 4j..4j+3,
//    all of group j div 2, so one scale and one bias apply per lane and step:
//        acc[i] += s P[i] + (b + 8 s) Xsum[i],   P = sum (q - 8) x,
//    with Xsum the group sums of the activations, formed while staging.
//  * Rows 4j + i of lanes j and j + 2 are the same vector over the two
//    groups; a lane swap adds them at the end.
//  * K is streamed through LDS in slices (all waves of a workgroup consume a
//    slice, a barrier, the next); F waves share each tile, wave f taking the
//    rounds (4 consecutive steps) f, f + F, ... of every slice, and their
//    partial sums meet in LDS in wave order. Every output is summed in the
//    same order on every run.
//  * Weight loads go through buffer resources based at the tile. A round is
//    4 consecutive steps of a wave: four 16-byte code loads per lane and one
//    16-byte load each for the lane's 8 scales and 8 biases of the round (a
//    2-byte load per lane and step would touch 16 cache lines for 32 useful
//    bytes). Rounds are double-buffered: the next is requested before the
//    current one is used, and the first is in flight while the first slice
//    is staged (weights do not depend on x). K is a multiple of 512.
#include "common.h"
#include "launch.h"

namespace qd {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

struct GemvMfmaArgs {
    const uint32_t* wq;
    const uint16_t* s;
    const uint16_t* b;
    const uint16_t* x;   // [nb][K] fp16 bits
    float* y;            // [nb][N]
    int N, K, nb;
    int steps;           // ceil(K / 128)
    int slice_steps;     // steps staged per slice
    int F;               // waves per tile (K groups)
};

// LDS of one staged step: 8 vectors x 128 fp16 (rows padded to 272 bytes so
// that the 8 vectors of one read fall in different banks), then the group
// sums [half][vector] as floats.
constexpr int GM_ROW = 272;
constexpr int GM_XSUM = 8 * GM_ROW;
constexpr int GM_STEP = GM_XSUM + 64;
constexpr int GM_ZERO = 64;   // zero bytes read by the masked lanes of A
constexpr int GM_SB = 4;      // staging loads in flight per thread

__device__ __forceinline__ f16x8_t as_f16x8(uint4 v) { return __builtin_bit_cast(f16x8_t, v); }

// 8 codes of one word as fp16 pairs (q0, q4), (q1, q5), (q2, q6), (q3, q7),
// centred: a nibble in the low mantissa bits of fp16 1024 is 1024 + q (one
// v_and_or_b32 per pair against the magic, kept in a VGPR), and one packed
// fp16 add of -1032 leaves q - 8 exactly. The activations are staged in the
// same k order [0, 4, 1, 5, 2, 6, 3, 7] within each word.
__device__ __forceinline__ uint4 codes_centred_f16(uint32_t w, uint32_t magic) {
    return make_uint4(pk_addh((w & 0x000F000Fu) | magic, kNeg1032),
                      pk_addh(((w >> 4) & 0x000F000Fu) | magic, kNeg1032),
                      pk_addh(((w >> 8) & 0x000F000Fu) | magic, kNeg1032),
                      pk_addh(((w >> 12) & 0x000F000Fu) | magic, kNeg1032));
}

template <int U>
__global__ __launch_bounds__(1024) void gemv_mfma_kernel(GemvMfmaArgs a) {
    extern __shared__ uint4 smem[];
    char* lds = (char*)smem;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = blockDim.x >> 6;
    const int F = a.F;
    const int f = wave % F;               // this wave's K group
    const int tw = wave / F;              // tile-wave within the workgroup
    const int twg = nwaves / F;
    const int tile = blockIdx.x * twg + tw;
    const int ntiles = (a.N + 15) >> 4;
    const bool has_tile = tile < ntiles;
    const int tl = min(tile, ntiles - 1);
    const int G = a.K / 64;
    const int n = lane & 15, j = lane >> 4;
    const int row = tl * 16 + n;
    const int rowc = min(row, a.N - 1);
    const int lr = rowc - tl * 16;        // row within the tile (clamped)
    const uint32_t rowb = (uint32_t)(a.K / 2);   // code bytes per row
    const int64_t r0 = (int64_t)tl * 16;
    const int tile_rows = min(16, a.N - (int)r0);
    const auto wr = buf_rsrc(a.wq + r0 * (a.K / 8), (int64_t)tile_rows * rowb);
    const auto sr = buf_rsrc(a.s + r0 * G, (int64_t)tile_rows * G * 2);
    const auto br = buf_rsrc(a.b + r0 * G, (int64_t)tile_rows * G * 2);
    const int SS = a.slice_steps;
    const int nsl = (a.steps + SS - 1) / SS;
    char* xs = lds;                                   // [SS][GM_STEP]
    char* zero = lds + (size_t)SS * GM_STEP;          // GM_ZERO bytes of zeros
    float* red = (float*)(zero + GM_ZERO);            // [F - 1][twg][32 lanes][4]
    // A rows: lane (m, j) carries vector m mod 8 on the k blocks of group
    // m div 8; the other lanes read zeros.
    const int am = lane & 15, ab = am & 7;
    const bool a_live = (am >> 3) == (j >> 1) && ab < a.nb;
    const uint32_t a_base = a_live ? (uint32_t)(ab * GM_ROW + 64 * j) : (uint32_t)(SS * GM_STEP);
    const uint32_t a_step = a_live ? (uint32_t)GM_STEP : 0u;
    const uint32_t xsum_off = (uint32_t)(GM_XSUM + ((j >> 1) * 8 + 4 * (j & 1)) * 4);
    const uint32_t hsh = 16u * (uint32_t)(j >> 1);   // this lane's half of a scale pair

    // The wave's rounds run back to back over all slices. A round is U
    // consecutive steps (U 64-byte pieces of each of the tile's rows, read as
    // one contiguous run per row), and the waves of a tile take the rounds of
    // a slice in turn: round r of wave f covers steps (f + r F) U .. + U - 1.
    // A full slice (SS, a multiple of F U) gives every wave R0 rounds; the
    // last slice R1 (per wave).
    const int R0 = SS / (F * U);
    const int ns_last = a.steps - (nsl - 1) * SS;
    const int C1 = (ns_last + U - 1) / U;
    const int R1 = C1 > f ? (C1 - f + F - 1) / F : 0;
    const int T = (nsl - 1) * R0 + R1;   // rounds of this wave

    static_assert(U == 4, "a round's scales and biases are one 16-byte load (8 groups)");
    struct Buf {
        uint4 cw[U];
        uint4 sv, bv;   // the round's 8 scales and 8 biases of this lane's row
    };
    // round (sl, r)'s code chunks, scales and biases. Rounds start at a
    // multiple of 4 steps, so the 8 groups of a round are one aligned 16-byte
    // run of the row's scales (G is a multiple of 8); past the row's end they
    // are never used, past the tile's end the resource returns zeros. Steps
    // past the wave's last one read a clamped, valid step, never consumed.
    const int last0 = (a.steps - 1) & ~(U - 1);   // last round start
    auto issue = [&](Buf& bf, int sl, int r) __attribute__((always_inline)) {
        const int st0 = min(sl * SS + (f + r * F) * U, last0);
        const uint32_t go = 2u * ((uint32_t)lr * G + 2u * (uint32_t)st0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int st = min(st0 + u, a.steps - 1);
            bf.cw[u] = buf_load16(wr, (uint32_t)lr * rowb + (uint32_t)st * 64u + 16u * j);
        }
        bf.sv = buf_load16(sr, go);
        bf.bv = buf_load16(br, go);
    };
    // Staging of slice sl in two halves: stage_load requests the chunks
    // (8 vector slots x 16 chunks per step, so a thread's items decode with
    // shifts; slots past nb and steps past the slice are out of range and
    // cost nothing), stage_store writes them and the group sums. At most
    // GM_SB chunks per thread: the host sizes slices so that one batch covers
    // a slice. Vector-memory counters complete in order, so the activation
    // loads are requested before the next weight round: the stores then
    // wait for the activations only.
    uint4 xv[GM_SB];
    // live == false: every offset out of range (the loads return zeros and
    // touch no memory), so a round can request them unconditionally
    auto stage_load = [&](int sl, bool live) __attribute__((always_inline)) {
        const int s0 = sl * SS;
        const int ns = live ? min(SS, a.steps - s0) : 0;
        const auto xr = buf_rsrc(a.x, (int64_t)a.nb * a.K * 2);
#pragma unroll
        for (int e = 0; e < GM_SB; ++e) {
            const int it = (int)threadIdx.x + e * (int)blockDim.x;
            const int ss = it >> 7, bvec = (it >> 4) & 7, w = it & 15;
            const bool ok = ss < ns && bvec < a.nb;
            const uint32_t k = (uint32_t)(s0 + ss) * 128u + 8u * (uint32_t)w;
            xv[e] = buf_load16(xr, ok ? ((uint32_t)bvec * (uint32_t)a.K + k) * 2u : 0x7FFFFFF0u);
        }
    };
    auto stage_store = [&](int sl) __attribute__((always_inline)) {
        const int ns = min(SS, a.steps - sl * SS);
#pragma unroll
        for (int e = 0; e < GM_SB; ++e) {
            const int it = (int)threadIdx.x + e * (int)blockDim.x;
            const int ss = it >> 7, bvec = (it >> 4) & 7, w = it & 15;
            const uint32_t h[4] = {xv[e].x, xv[e].y, xv[e].z, xv[e].w};
            float sum = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                sum += h2f((uint16_t)(h[q] & 0xFFFF)) + h2f((uint16_t)(h[q] >> 16));
            // the 8 chunks of one group sit in 8 consecutive lanes
            sum = seg_sum<8>(sum);
            if (ss < ns) {
                // the pairs (x0, x4), (x1, x5), (x2, x6), (x3, x7) of the chunk
                const uint4 v = xv[e];
                const uint4 o = make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u),
                                           __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                                           __builtin_amdgcn_perm(v.w, v.y, 0x05040100u),
                                           __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
                *(uint4*)(xs + ss * GM_STEP + bvec * GM_ROW + 16 * w) = o;
                if ((w & 7) == 0) ((float*)(xs + ss * GM_STEP + GM_XSUM))[(w >> 3) * 8 + bvec] = sum;
            }
        }
    };

    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
    const floatx4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    const uint32_t magic = in_vgpr(kMagic16);
    auto consume = [&](const Buf& bf, int sl, int r) __attribute__((always_inline)) {
        const int ns = sl < nsl - 1 ? SS : ns_last;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ss = (f + r * F) * U + u;
            if (ss >= ns) break;   // uniform
            const int st = sl * SS + ss;
            const int gi = 2 * st + (j >> 1);
            const bool ok = gi < G && row < a.N;
            // group 2 u + (j div 2) of the round: word u, half j div 2
            const uint32_t sw = u == 0 ? bf.sv.x : u == 1 ? bf.sv.y : u == 2 ? bf.sv.z : bf.sv.w;
            const uint32_t bw = u == 0 ? bf.bv.x : u == 1 ? bf.bv.y : u == 2 ? bf.bv.z : bf.bv.w;
            const float sc = ok ? h2f((uint16_t)(sw >> hsh)) : 0.f;
            const float bi = ok ? fmaf(8.f, sc, h2f((uint16_t)(bw >> hsh))) : 0.f;   // b + 8 s
            const uint32_t ao = a_base + (uint32_t)ss * a_step;
            floatx4_t P = zero4;
            const uint32_t wd[4] = {bf.cw[u].x, bf.cw[u].y, bf.cw[u].z, bf.cw[u].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint4 av = *(const uint4*)(xs + ao + 16 * t);
                const uint4 bq = codes_centred_f16(wd[t], magic);
                P = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(av), as_f16x8(bq), P, 0, 0, 0);
            }
            const float4 xsv = *(const float4*)(xs + ss * GM_STEP + xsum_off);
            acc[0] = fmaf(bi, xsv.x, fmaf(sc, P[0], acc[0]));
            acc[1] = fmaf(bi, xsv.y, fmaf(sc, P[1], acc[1]));
            acc[2] = fmaf(bi, xsv.z, fmaf(sc, P[2], acc[2]));
            acc[3] = fmaf(bi, xsv.w, fmaf(sc, P[3], acc[3]));
        }
    };
    // Round (sl, r) is the R-th of this wave. When it ends a slice, the next
    // slice is staged after it: its activations are requested before the
    // prefetch of the following round (the stores then wait for them alone),
    // and the barriers keep slice sl's readers and slice sl + 1's writers
    // apart. The activation loads are requested every round (out of range,
    // so free, off the edge): a branch around loads would make the compiler
    // wait for every load in flight where the paths join.
    // one half of the double-buffered walk: prefetch the next round into nx,
    // consume (sl, r) from cu
    auto half = [&](Buf& cu, Buf& nx, int sl, int r, int R) __attribute__((always_inline)) {
        const bool edge = sl < nsl - 1 && r == R0 - 1;
        stage_load(sl + 1, edge);
        int ns = sl, nr = r + 1;
        if (edge) {
            ns = sl + 1;
            nr = 0;
        }
        if (R + 1 >= T) nr = r;   // past the last round: a clamped re-request
        issue(nx, ns, nr);
        consume(cu, sl, r);
        if (edge) {
            __syncthreads();
            stage_store(sl + 1);
            __syncthreads();
        }
    };
    auto advance = [&](int& sl, int& r) {
        if (sl < nsl - 1 && r == R0 - 1) {
            ++sl;
            r = 0;
        } else {
            ++r;
        }
    };
    Buf b0, b1;
    // the first weight round is in flight while the first slice is staged
    stage_load(0, true);
    issue(b0, 0, 0);
    if ((int)threadIdx.x < GM_ZERO / 16) ((uint4*)zero)[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
    stage_store(0);
    __syncthreads();
    // every wave walks the same slice boundaries (R0 rounds per full slice
    // for every wave, so its barriers match the others')
    int sl = 0, r = 0;
    for (int R = 0; R < T; R += 2) {
        half(b0, b1, sl, r, R);
        advance(sl, r);
        if (R + 1 >= T) break;
        half(b1, b0, sl, r, R + 1);
        advance(sl, r);
    }
    // the two groups' halves of each vector: lanes l and l + 32
    float tot[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[i]), __float_as_uint(acc[i]),
                                                         false, false);
        tot[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if (F > 1) {
        if (f > 0 && lane < 32)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[(((f - 1) * twg + tw) * 32 + lane) * 4 + i] = tot[i];
        __syncthreads();
        if (f == 0 && lane < 32)
            for (int g = 1; g < F; ++g)
#pragma unroll
                for (int i = 0; i < 4; ++i) tot[i] += red[(((g - 1) * twg + tw) * 32 + lane) * 4 + i];
    }
    if (f == 0 && lane < 32 && has_tile && row < a.N) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int bvec = 4 * j + i;
            if (bvec < a.nb) a.y[(int64_t)bvec * a.N + row] = tot[i];
        }
    }
}

namespace {
constexpr int GM_U = 4;
}

size_t gemv_mfma_lds(int slice_steps, int F, int nwaves) {
    return (size_t)slice_steps * GM_STEP + GM_ZERO + (size_t)(F - 1) * (nwaves / F) * 32 * 4 * 4;
}

hipError_t launch_gemv_mfma(const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                            const uint16_t* x, float* y, int N, int K, int nb, hipStream_t st) {
    if (nb < 1 || nb > 8 || K % 512 != 0 || N < 1) return hipErrorInvalidValue;
    const DeviceInfo& dev = device_info();
    const int ntiles = (N + 15) / 16;
    const int steps = (K + 127) / 128;
    // K groups per tile: the most (at most 8) that keep the grid of 8-wave
    // workgroups within two per CU; 16-wave workgroups (one staging of x per
    // two tiles) when those still cover every CU
    int F = 1;
    while (F < 8 && (int64_t)ntiles * 2 * F <= (int64_t)dev.cus * 2 * 8) F *= 2;
    const int nwaves = (int64_t)ntiles * F >= (int64_t)dev.cus * 16 ? 16 : 8;
    // slices: the LDS of one CU shared by the workgroups it holds, and one
    // batch of staging loads per thread covering a slice
    const size_t budget =
        std::min<size_t>(dev.max_lds_per_block, dev.lds_per_cu / (nwaves == 16 ? 1 : 2));
    auto slice_cap = [&](int Fc) {
        const size_t fixed = gemv_mfma_lds(0, Fc, nwaves);
        const int lds_cap = budget > fixed ? (int)((budget - fixed) / GM_STEP) : 0;
        return std::min(lds_cap, GM_SB * nwaves * 64 / 128);
    };
    // a multiple of F U: every wave has the same whole rounds in a full slice
    // (fewer waves per tile when a slice cannot hold that)
    while (F > 1 && slice_cap(F) < F * GM_U) F /= 2;
    int cap = slice_cap(F);
    if (cap < F * GM_U) return hipErrorInvalidValue;
    cap = cap / (F * GM_U) * (F * GM_U);
    const int twg = nwaves / F;
    // even slices
    const int nsl = (steps + cap - 1) / cap;
    int SS = (steps + nsl - 1) / nsl;
    SS = (SS + F * GM_U - 1) / (F * GM_U) * (F * GM_U);
    GemvMfmaArgs a{};
    a.wq = wq;
    a.s = s;
    a.b = b;
    a.x = x;
    a.y = y;
    a.N = N;
    a.K = K;
    a.nb = nb;
    a.steps = steps;
    a.slice_steps = SS;
    a.F = F;
    const size_t lds = gemv_mfma_lds(SS, F, nwaves);
    auto kern = gemv_mfma_kernel<GM_U>;
    (void)occupancy((const void*)kern, nwaves * 64, lds);   // sets the dynamic-LDS limit once
    const int grid = (ntiles + twg - 1) / twg;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(nwaves * 64), lds, st, a);
    return hipGetLastError();
}

}  // namespace qd
