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
// Tiling: a workgroup owns 128 rows (the whole chunk) x 64 output columns
// with 8 waves: two column waves (32 columns each, all 128 rows as four 32x32
// MFMA blocks) times four K-sets that take alternate groups of K; the K-sets'
// partial sums are added in LDS at the end, in a fixed order. X is staged in
// LDS a stage of 4 groups at a time (double buffered, one barrier per stage;
// the next stage is read into registers while the current one is consumed),
// together with its per-group row sums. Each lane loads the 16 code bytes it
// feeds to the MFMA (words 4h..4h+3 of its column's group, where h is the
// lane's k-half) into a ring of register slots two stages deep, so weight
// fetches overlap the matrix work; the K order inside a group is permuted
// identically on both operands (step st, half h takes word 4h + st).
//
// Cost notes: a wave64 vector instruction occupies its SIMD for 4 cycles, so
// the per-group vector work (unpacking codes, scaling P) is kept small next
// to the MFMAs: the bias term is done on the matrix core once per stage, the
// MFMA results stay in ordinary VGPRs, and each unpacked code word feeds 16
// MFMAs (four row blocks).
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "mfma.h"

namespace qd {

typedef _Float16 halfx8_c __attribute__((ext_vector_type(8)));

constexpr int CH_NT = 64;    // output columns per workgroup
constexpr int CH_MMAX = 128; // rows per call (the whole chunk)

struct ChunkArgs {
    const uint32_t* wq;
    const uint16_t* s;
    const uint16_t* b;
    const uint16_t* x;   // bf16 [M][K]
    float* y;            // [M][N]
    int M, N, K;
    int ncol_tiles;      // ceil(N / 64)
    int64_t x_row_stride;   // elements between rows of x
    int64_t y_row_stride;   // elements between rows of y
};

// A workgroup owns MT = 32 MB WM rows (one row tile) and 64 columns. LDS
// layout (dynamic): xs[2 buffers][SG groups][MT rows][XS_STRIDE] uint4, then
// xsum[2][MT rows][SG groups] fp32, then (fp16 activations only) the same
// sums transposed, xsumT[2][SG groups][MT rows].
template <int SG, int MT_, bool F16 = false>
struct ChunkLds {
    static constexpr int MT = MT_;
    static constexpr int XS = SG * MT * XS_STRIDE;   // uint4 per buffer
    static constexpr size_t bytes = 2 * (size_t)XS * 16 + (F16 ? 4 : 2) * SG * MT * 4;
};

// Group visited at step g (clamped to the last step) when a workgroup starts
// its walk over K at group rot: workgroups that share an L2 start at
// different places, so they do not all read the same few memory channels at
// once (rows of X and of the codes are a power-of-two number of bytes apart).
__device__ __forceinline__ int rot_group(int g, int G, int rot) {
    g = min(g, G - 1) + rot;
    return g >= G ? g - G : g;
}

// One stage = SG groups of X (MT rows x 64 k each), staged by the first NTS
// of the NT threads (at most 8 per row; a multiple of 64, so whole waves
// stage or skip): TPR = NTS / MT threads share a row; thread part p holds k
// in [64 p / TPR, 64 (p + 1) / TPR) of every group: XPT = 8 / TPR uint4 per
// group.
template <int SG, int MT_, int NT, bool F16 = false>
struct StageIO {
    static constexpr int MT = MT_;
    static constexpr int NTS = NT < 8 * MT ? NT : 8 * MT;
    static constexpr int TPR = NTS / MT;
    static constexpr int XPT = 8 / TPR;
    static_assert(TPR >= 1 && XPT >= 1 && NTS % 64 == 0, "staging split");

    __device__ static __forceinline__ void load(const ChunkArgs& a, int m0, int g0, int G, int rot,
                                                uint4 (&xr)[SG][XPT]) {
        const int t = threadIdx.x;
        if (NTS < NT && t >= NTS) return;
        const int m = m0 + t / TPR, part = t % TPR;
#pragma unroll
        for (int gi = 0; gi < SG; ++gi) {
            const int g = rot_group(g0 + gi, G, rot);
            const uint4* src = (const uint4*)(a.x + (int64_t)min(m, a.M - 1) * a.x_row_stride +
                                              (int64_t)g * 64 + 8 * XPT * part);
#pragma unroll
            for (int i = 0; i < XPT; ++i) xr[gi][i] = src[i];
        }
    }

    __device__ static __forceinline__ void store(uint4* xs, float* xsum, const uint4 (&xr)[SG][XPT],
                                                 float* xsumT = nullptr) {
        // rows past M hold copies of row M - 1 (the loads clamp); they only
        // feed output rows that are never stored
        const int t = threadIdx.x;
        if (NTS < NT && t >= NTS) return;
        const int r = t / TPR, part = t % TPR;
#pragma unroll
        for (int gi = 0; gi < SG; ++gi) {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < XPT; ++i) {
                const uint4 v = xr[gi][i];
                xs[(gi * MT + r) * XS_STRIDE + XPT * part + i] = v;
                if constexpr (F16) {
                    acc = dot2(v.x, 0x3C003C00u, acc);
                    acc = dot2(v.y, 0x3C003C00u, acc);
                    acc = dot2(v.z, 0x3C003C00u, acc);
                    acc = dot2(v.w, 0x3C003C00u, acc);
                } else {
                    acc = bf16_pair_sum(v.x, acc);
                    acc = bf16_pair_sum(v.y, acc);
                    acc = bf16_pair_sum(v.z, acc);
                    acc = bf16_pair_sum(v.w, acc);
                }
            }
            acc = seg_sum<TPR>(acc);   // the TPR adjacent lanes of the row
            xsum[r * SG + gi] = acc;   // every lane of the row stores the same sum
            if constexpr (F16) xsumT[gi * MT + r] = acc;
        }
    }
};

// Calls f(integral_constant<int, I>) for I = 0 .. N-1 (compile-time indices).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// A copy of v that the compiler cannot see through or move out of a loop:
// the per-stage LDS base goes through it so that every per-group offset
// stays a constant folded into the ds_read instruction (otherwise each
// address is hoisted out of the loop and held in a register of its own).
__device__ __forceinline__ int opaque(int v) {
    int r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
    return r;
}

// SG groups per barrier. A K-set of 2 WM waves covers the tile: wave
// (wm, wn) computes rows [32 MB wm, 32 MB (wm + 1)) x columns [32 wn, 32 wn
// + 32) as MB 32x32 MFMA blocks. The workgroup has NKS K-sets, set ks taking
// the groups gi = NKS j + ks of every stage (all sets share the staged X);
// their partial sums meet in LDS at the end. D = depth of each wave's
// register ring of code operands, in groups of the whole walk (a multiple of
// SG): the codes of group g + D are requested right after group g is used.
// The main loop runs whole rounds of D groups with no data-dependent exits
// (an exit inside the round would make the compiler wait for every load in
// flight where the paths join); the last partial round runs with checks.
// Workgroup b takes column tile 8 (b / (8 RT)) + b % 8 and row tile
// (b / 8) % RT, so the RT row tiles of a column tile run on one XCD and share
// its L2 copy of the codes.
//
// XD = stages of X held in registers ahead of LDS: with 1, the next stage is
// read while the current one is consumed; with 2 (small row tiles, whose
// stages hold little matrix work) the stage after that is also in flight.
// F16: fp16 activations; the codes enter an fp16 MFMA as 1024 + q and the
// offset part -1024 s Xsum is added in fp32 per group (in the bias MFMA's
// 16-bit split it would lose too much next to the result); bf16 activations
// fold -128 s into the bias MFMA.
template <int SG, int D, int MB, int WM, int NKS, int XD = 1, bool F16 = false>
__global__ __launch_bounds__(128 * WM * NKS) void chunk_gemm_kernel(ChunkArgs a) {
    static_assert(D % SG == 0 && SG % NKS == 0 && SG == 4, "stage shape");
    constexpr int SPR = D / SG;     // stages per round
    static_assert(XD == 1 || (XD == 2 && SPR % 2 == 0), "X prefetch depth");
    constexpr int JS = SG / NKS;    // groups per stage per wave
    constexpr int DW = D / NKS;     // ring slots per wave
    constexpr int WS = 2 * WM;      // waves per K-set
    constexpr int MT = 32 * MB * WM;
    using L = ChunkLds<SG, MT, F16>;
    using IO = StageIO<SG, MT, 64 * WS * NKS, F16>;
    extern __shared__ uint4 smem[];
    uint4* xs_raw = smem;                                    // [2][XS]
    float* xsum_raw = (float*)(smem + 2 * L::XS);            // [2][MT][SG]
    float* xsumT_raw = xsum_raw + 2 * SG * MT;               // [2][SG][MT] (F16)
    const int RT = (a.M + MT - 1) / MT;                      // row tiles
    const int b = blockIdx.x;
    const int ct = (b / (8 * RT)) * 8 + b % 8;
    const int m0 = ((b / 8) % RT) * MT;
    if (ct >= a.ncol_tiles) return;   // whole workgroup, before any barrier
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wq = wave % WS;                 // wave within the K-set
    const int wm = wq % WM, wn = wq / WM, ks = wave / WS;   // ks < NKS
    const int h = lane >> 5, l32 = lane & 31;
    const int G = a.K / 64;
    const int NS = (G + SG - 1) / SG;
    // workgroups on one XCD are 8 apart in blockIdx.x: spread their starts
    const int rot = (int)((unsigned)(b >> 3) * (unsigned)SG % (unsigned)G);
    const int64_t wpr = a.K / 8;
    const int n = ct * CH_NT + wn * 32 + l32;                // this lane's column
    const int nc = min(n, a.N - 1);
    const uint32_t* wrow = a.wq + (int64_t)nc * wpr + 4 * h;  // words 4h..4h+3 of group 0
    const uint16_t* srow = a.s + (int64_t)nc * G;
    const uint16_t* brow = a.b + (int64_t)nc * G;

    floatx16 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;

    // Ring slot e of this wave holds the step NKS e + ks of the current round
    // (steps count groups in walk order). Scale and bias slots are whole
    // registers (zero-extended): packing two 16-bit values per register would
    // force a wait on each refill.
    uint4 bq[DW];
    uint32_t bs[DW], bb[DW];
#pragma unroll
    for (int e = 0; e < DW; ++e) {
        const int g = rot_group(NKS * e + ks, G, rot);
        bq[e] = *(const uint4*)(wrow + (int64_t)g * 8);
        bs[e] = srow[g];
        bb[e] = brow[g];
    }
    // xr[i]: X of stage st + 1 + i while stage st runs (a ring when XD = 2;
    // stage parity picks the slot, and rounds hold an even number of stages)
    uint4 xr[XD][SG][IO::XPT];
    IO::load(a, m0, 0, G, rot, xr[0]);
    IO::store(xs_raw, xsum_raw, xr[0], xsumT_raw);
    if constexpr (XD == 2) IO::load(a, m0, SG, G, rot, xr[1]);
    __syncthreads();

    // one group (step g, slot e): MFMAs into P, then acc += s P, then the
    // slot is refilled with step g + D. xs: this lane's A-operand row (row
    // 32 MB wm + l32, k-half h) of the group. The bias part, (b - 128 s) Xsum,
    // is added per stage on the matrix core (bias_mfma below).
    auto group = [&](const int g, auto ec, const uint4* xs, const float* xt)
                     __attribute__((always_inline)) {
        constexpr int e = decltype(ec)::value;
        // the 4 steps' B operands, then the row blocks PH at a time (fewer
        // live accumulators than all MB at once)
        constexpr int PH = MB < 2 ? MB : 2;
        const uint32_t wv[4] = {bq[e].x, bq[e].y, bq[e].z, bq[e].w};
        bf16x8_t bfrag[4];
#pragma unroll
        for (int stp = 0; stp < 4; ++stp)
            bfrag[stp] = __builtin_bit_cast(bf16x8_t, codes_to_16n(wv[stp], F16 ? 0x64006400u : 0x43004300u));
        const float sf = h2f((uint16_t)bs[e]);
#pragma unroll
        for (int m0b = 0; m0b < MB; m0b += PH) {
            floatx16 P[PH];
#pragma unroll
            for (int pb = 0; pb < PH; ++pb)
#pragma unroll
                for (int i = 0; i < 16; ++i) P[pb][i] = 0.f;
#pragma unroll
            for (int stp = 0; stp < 4; ++stp) {
#pragma unroll
                for (int pb = 0; pb < PH; ++pb) {
                    const uint4 av = xs[32 * (m0b + pb) * XS_STRIDE + stp];
                    if constexpr (F16)
                        P[pb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            __builtin_bit_cast(halfx8_c, av), __builtin_bit_cast(halfx8_c, bfrag[stp]),
                            P[pb], 0, 0, 0);
                    else
                        P[pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8_t, av), bfrag[stp], P[pb], 0, 0, 0);
                }
            }
            if constexpr (F16) {
                // rows 8 (i / 4) + 4 h + i % 4 of the block: quarter i / 4
                const float mo = -1024.f * sf;
#pragma unroll
                for (int pb = 0; pb < PH; ++pb)
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) {
                        const float4 xq = *(const float4*)(xt + 32 * (m0b + pb) + 8 * qq);
                        const float xv[4] = {xq.x, xq.y, xq.z, xq.w};
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            acc[m0b + pb][4 * qq + j] = fmaf(sf, P[pb][4 * qq + j],
                                                             fmaf(mo, xv[j], acc[m0b + pb][4 * qq + j]));
                    }
            } else {
#pragma unroll
                for (int pb = 0; pb < PH; ++pb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[m0b + pb][i] = fmaf(sf, P[pb][i], acc[m0b + pb][i]);
            }
            __builtin_amdgcn_sched_barrier(0);   // keep the passes apart (registers)
        }
        // finish this group's epilogue here: left alone, the compiler sinks it
        // to the end of the stage and holds several groups' P at once
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) asm volatile("" : "+v"(acc[mb]));
        // refill the slot once its old contents are dead (a refill issued
        // while they are still read makes the compiler copy the slot across
        // the loop back edge, and a copy waits for the load)
        const int gn = rot_group(g + D, G, rot);
        bq[e] = *(const uint4*)(wrow + (int64_t)gn * 8);
        bs[e] = srow[gn];
        bb[e] = brow[gn];
        __builtin_amdgcn_sched_barrier(0);
    };

    // Bias of this wave's groups of one stage: acc += sum_g Xsum_g[m] (b_g -
    // 128 s_g)[n] as one MFMA per row block. Both factors are split into bf16
    // hi + lo parts and the K = 16 slots carry the four cross products: lane
    // half h supplies slots 8h..8h+7 as A = (x_h, x_h) over 4 group slots,
    // with x_0 = hi, x_1 = lo, and B = (hi, lo), so the slots sum to
    // (xhi + xlo)(bhi + blo). Each product is exact in fp32; the parts keep 16
    // significant bits. Group slot j < JS is the wave's j-th group of the
    // stage; slots JS..3 are zero.
    auto bias_mfma = [&](const int st, auto sjc, auto checked, const float* xsum)
                         __attribute__((always_inline)) {
        constexpr int sj = decltype(sjc)::value;
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < JS; ++j) {
            const int e = sj * JS + j;
            const float sf = h2f((uint16_t)bs[e]);
            bv[j] = h2f((uint16_t)bb[e]) - (F16 ? 0.f : 128.f * sf);
            if constexpr (decltype(checked)::value)
                if (st * SG + NKS * j + ks >= G) bv[j] = 0.f;
        }
        auto split = [](float a0, float a1, uint32_t& hi, uint32_t& lo) __attribute__((always_inline)) {
            const bf16x2_t hv = {(__bf16)a0, (__bf16)a1};
            hi = __builtin_bit_cast(uint32_t, hv);
            const bf16x2_t lv = {(__bf16)(a0 - __uint_as_float(hi << 16)),
                                 (__bf16)(a1 - __uint_as_float(hi & 0xFFFF0000u))};
            lo = __builtin_bit_cast(uint32_t, lv);
        };
        uint32_t bh01, bl01, bh23 = 0, bl23 = 0;
        split(bv[0], JS > 1 ? bv[1] : 0.f, bh01, bl01);
        if constexpr (JS > 2) split(bv[2], bv[3], bh23, bl23);
        const bf16x8_t bfrag = __builtin_bit_cast(bf16x8_t, make_uint4(bh01, bh23, bl01, bl23));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            // this set's groups of the row: NKS j + ks (read by address: a
            // select on ks would become branches)
            const float* xrow = xsum + (32 * MB * wm + 32 * mb + l32) * SG;
            float xg[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < JS; ++j) xg[j] = xrow[NKS * j];
            uint32_t xh01, xl01, xh23 = 0, xl23 = 0;
            split(xg[0], JS > 1 ? xg[1] : 0.f, xh01, xl01);
            if constexpr (JS > 2) split(xg[2], xg[3], xh23, xl23);
            const uint32_t a01 = h ? xl01 : xh01, a23 = h ? xl23 : xh23;
            const bf16x8_t afrag = __builtin_bit_cast(bf16x8_t, make_uint4(a01, a23, a01, a23));
            acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag, bfrag, acc[mb], 0, 0, 0);
        }
    };

    // one stage: read the next stage's X into registers (addresses clamp to
    // the last group), bias MFMA, this wave's groups from LDS, store the next
    // stage into the other buffer, barrier
    auto stage = [&](const int st, auto sjc, auto checked) __attribute__((always_inline)) {
        constexpr int sj = decltype(sjc)::value;
        const int buf = st & 1;
        // XD = 1: slot 0 receives stage st + 1; XD = 2: slot st % 2 receives
        // stage st + 2 while slot (st + 1) % 2 holds stage st + 1
        constexpr int ld = XD == 1 ? 0 : sj % 2, sv = XD == 1 ? 0 : (sj + 1) % 2;
        IO::load(a, m0, (st + XD) * SG, G, rot, xr[ld]);
        bias_mfma(st, sjc, checked, xsum_raw + opaque(buf * SG * MT + ks));
        // group j of this wave is stage group NKS j + ks
        const uint4* xs = xs_raw + opaque(buf * L::XS + ks * MT * XS_STRIDE +
                                          (32 * MB * wm + l32) * XS_STRIDE + 4 * h);
        // fp16 only: this lane's accumulator rows of the row sums, group ks
        const float* xt = F16 ? xsumT_raw + opaque(buf * SG * MT + ks * MT + 32 * MB * wm + 4 * h)
                              : nullptr;
        static_for<0, JS>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            const int g = st * SG + NKS * j + ks;
            constexpr std::integral_constant<int, sj * JS + j> ec{};
            const uint4* xsj = xs + NKS * j * MT * XS_STRIDE;
            const float* xtj = F16 ? xt + NKS * j * MT : nullptr;
            if constexpr (decltype(checked)::value) {
                if (g < G) group(g, ec, xsj, xtj);
            } else {
                group(g, ec, xsj, xtj);
            }
        });
        IO::store(xs_raw + (buf ^ 1) * L::XS, xsum_raw + (buf ^ 1) * SG * MT, xr[sv],
                  xsumT_raw + (buf ^ 1) * SG * MT);
        __syncthreads();
    };

    const int rounds = G / D;
    for (int r = 0; r < rounds; ++r)
        static_for<0, SPR>([&](auto sjc) __attribute__((always_inline)) {
            stage(r * SPR + decltype(sjc)::value, sjc, std::false_type{});
        });
    static_for<0, SPR>([&](auto sjc) __attribute__((always_inline)) {
        const int st = rounds * SPR + decltype(sjc)::value;
        if (st < NS) stage(st, sjc, std::true_type{});
    });

    // sum the K-sets in a fixed order (the last stage ended with a barrier:
    // X is no longer read)
    if constexpr (NKS > 1) {
        static_assert((NKS - 1) * WS * MB * 16 * 64 * 4 <= L::bytes, "reduction space");
        float* red = (float*)smem;   // [NKS - 1 sets][WS waves][MB][16][64 lanes]
        if (ks > 0) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    red[((((ks - 1) * WS + wq) * MB + mb) * 16 + i) * 64 + lane] = acc[mb][i];
        }
        __syncthreads();
        if (ks > 0) return;
#pragma unroll
        for (int k2 = 0; k2 < NKS - 1; ++k2)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    acc[mb][i] += red[(((k2 * WS + wq) * MB + mb) * 16 + i) * 64 + lane];
                __builtin_amdgcn_sched_barrier(0);   // bounded loads in flight (registers)
            }
    }
    if (n < a.N) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = m0 + 32 * MB * wm + 32 * mb + 8 * (i / 4) + 4 * h + (i % 4);
                if (m < a.M) a.y[(int64_t)m * a.y_row_stride + n] = acc[mb][i];
            }
    }
}

template <int SG, int D, int MB, int WM, int NKS, bool F16>
static hipError_t launch_chunk_cfg(const ChunkArgs& a, hipStream_t st) {
    constexpr int MT = 32 * MB * WM;
    const int RT = (a.M + MT - 1) / MT;
    const int grid = ((a.ncol_tiles + 7) / 8) * 8 * RT;
    const size_t lds = ChunkLds<SG, MT, F16>::bytes;
    if (lds > device_info().max_lds_per_block) return hipErrorInvalidValue;
    constexpr int threads = 128 * WM * NKS;
    auto kern = chunk_gemm_kernel<SG, D, MB, WM, NKS, 1, F16>;
    (void)occupancy((const void*)kern, threads, lds);  // sets the dynamic-LDS limit once
    hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, st, a);
    return hipGetLastError();
}

hipError_t launch_chunk_gemm(int bits, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                             const uint16_t* x, int xkind, float* y, int M, int N, int K,
                             hipStream_t st) {
    if (bits != 4 || M > CH_MMAX || (xkind != X_F16 && xkind != X_BF16)) return hipErrorInvalidValue;
    ChunkArgs a{};
    a.wq = wq;
    a.s = s;
    a.b = b;
    a.x = x;
    a.y = y;
    a.M = M;
    a.N = N;
    a.K = K;
    a.ncol_tiles = (N + CH_NT - 1) / CH_NT;
    a.x_row_stride = K;
    a.y_row_stride = N;
// Row tiles follow M (measured on K = 4096 -> N = 14336): up to 32 rows, one
// row block per wave and two K-sets (4 waves); up to 64 rows, two row blocks
// and four K-sets; beyond, the whole chunk as four row blocks per wave, 2
// column waves x 4 K-sets = 8 waves (2 per SIMD). All use 4 groups per stage
// and a ring of 8 groups.
    if (xkind == X_F16) {
        if (M <= 32) return launch_chunk_cfg<4, 8, 1, 1, 2, true>(a, st);
        if (M <= 64) return launch_chunk_cfg<4, 8, 2, 1, 4, true>(a, st);
        return launch_chunk_cfg<4, 8, 4, 1, 4, true>(a, st);
    }
    if (M <= 32) return launch_chunk_cfg<4, 8, 1, 1, 2, false>(a, st);
    if (M <= 64) return launch_chunk_cfg<4, 8, 2, 1, 4, false>(a, st);
    return launch_chunk_cfg<4, 8, 4, 1, 4, false>(a, st);
}

}  // namespace qd
