// Prefill-chunk GEMM on bf16 MFMA: Y[m][n] = sum_k w[n][k] X[m][k], M <= 128.
//
// [TF] jeff.news/article/5193, section "내부 구조가 진짜 흥미로운 부분"
// (internals): prompts are processed in chunks of at most 128 tokens so that
// one fetch of a weight serves many rows. Weight format as in the decode
// path ("성능과 제약": affine 4-bit, group 64, w = s*q + b).
//
// Rounding w itself to bf16 would lose too much (8 significant bits), so
// the matrix-core operand is the exact code q (4 bits; mfma.h converts the
// nibbles through the fp8 converter, which maps them exactly): one
// v_mfma_f32_32x32x16_bf16 chain per group of 64 inputs (4 x K=16) yields
//     P_g[m][n] = sum_{k in g} X[m][k] q[n][k]                    (fp32)
// and the epilogue adds
//     acc[m][n] += s[n][g] P_g[m][n] + b[n][g] Xsum_g[m]
// with Xsum_g[m] = sum_{k in g} X[m][k], computed while X is staged: the
// first term as an fp32 FMA per group, the second once per stage on the
// matrix core from three-part bf16 splits of both factors, about as exact
// as an fp32 product (the two terms cancel where weights sit near zero,
// b ~ -q s; the products are exact and the fp32 sums round in proportion to
// |s q x| <= 15 |s x|). fp16 activations run the same on an fp16 MFMA.

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
// to the MFMAs and issued while they run: each row block's MFMA chain is
// followed by the previous block's scaling (independent of it), the bias
// term is done on the matrix core once per stage, the MFMA results stay in
// ordinary VGPRs, and each unpacked code word feeds 16 MFMAs (four row
// blocks).
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
    int gsplit;          // K split: groups per split (blockIdx.y), 0 = whole K
};

// A workgroup owns MT = 32 MB WM rows (one row tile) and 64 columns. LDS
// layout (dynamic): xs[2 buffers][SG groups][MT rows][XS_STRIDE] uint4, then
// the per-group row sums as bias-product parts (bias_row_parts),
// xsum[2][SG groups][MT rows] uint2 (row-contiguous: a lane per row reads
// without bank conflicts).
template <int SG, int MT_, bool F16 = false>
struct ChunkLds {
    static constexpr int MT = MT_;
    static constexpr int XS = SG * MT * XS_STRIDE;   // uint4 per buffer
    static constexpr size_t bytes = 2 * (size_t)XS * 16 + 2 * SG * MT * 8;
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

    __device__ static __forceinline__ void store(uint4* xs, uint2* xsum, const uint4 (&xr)[SG][XPT]) {
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
            xsum[gi * MT + r] = bias_row_parts(acc);   // every lane of the row stores the same
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

// Scales and biases of a workgroup's 64 columns through LDS (SBL): read per
// lane, a column each, every 2-byte value costs its own cache-line access.
// The tile's 64 rows are one contiguous run of 64 G halfwords in each array
// (16-byte aligned: the arrays are, and tiles start every 64 rows), copied
// with 16-byte loads by all NTH threads before the first barrier; the ring
// then reads its values from LDS. In LDS each row is padded by one dword
// (rows of G + 2 halfwords, an odd number of dwords when 8 divides G), so
// the 32 rows a wave reads at once fall in different banks. For whole column
// tiles (N % 64 == 0), 8 | G and G <= CH_SB_GMAX.
constexpr int CH_SB_GMAX = 64;
template <int NTH>
struct ChunkSb {
    static constexpr int KMAX = (16 * CH_SB_GMAX + NTH - 1) / NTH;   // uint4 per thread
    uint4 v[KMAX];
    // all loads issued (indices clamp to the two runs, [8 G] uint4 each).
    // STRIDED (a K split): the tile's rows are rs values apart (the matrix's
    // groups per row) and the copy takes G of them from each row; with
    // 8 | rs and the split starting on a multiple of 8 groups, every row's
    // run stays 16-byte aligned.
    template <bool STRIDED = false>
    __device__ __forceinline__ void load(const uint16_t* s, const uint16_t* b, int G, int rs = 0) {
        const int n8 = 8 * G, upr = G / 8;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int i = min((int)threadIdx.x + NTH * k, 2 * n8 - 1);
            if constexpr (STRIDED) {
                const int arr = i >= n8, j = i - arr * n8;
                const int r = j / upr, c = j - r * upr;
                v[k] = *(const uint4*)((arr ? b : s) + (int64_t)r * rs + 8 * c);
            } else {
                const uint4* src = i < n8 ? (const uint4*)s + i : (const uint4*)b + (i - n8);
                v[k] = *src;
            }
        }
    }
    // dst: [64 rows][G + 2] scales, then the same for the biases
    __device__ __forceinline__ void store(uint32_t* dst, int G) const {
        const int n8 = 8 * G, upr = G / 8, rdw = G / 2 + 1;   // uint4 per row, dwords per LDS row
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int i = threadIdx.x + NTH * k;
            if (i < 2 * n8) {
                const int arr = i >= n8, j = i - arr * n8;
                const int r = j / upr, c = j - r * upr;
                uint32_t* d = dst + (arr * 64 + r) * rdw + 4 * c;
                d[0] = v[k].x;
                d[1] = v[k].y;
                d[2] = v[k].z;
                d[3] = v[k].w;
            }
        }
    }
};

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
// F16: fp16 activations on an fp16 MFMA, else bf16; the operand is the code
// q either way. The bias term b Xsum, of the size of the result, runs on the
// matrix core once per stage.
//
// SBL: scales and biases from an LDS copy (ChunkSb), placed after the
// staging buffers in the dynamic LDS.
//
// KSPL: K split across workgroups. Split blockIdx.y takes the groups
// [y gsplit, min((y + 1) gsplit, K / 64)) and writes its partial Y to slice y
// of a [splits][M][N] array (a.y); chunk_ksum_kernel then adds the slices in
// split order. With SBL the scale/bias copy takes the split's part of each
// row (a strided copy).
template <int SG, int D, int MB, int WM, int NKS, int XD = 1, bool F16 = false, bool SBL = false,
          bool KSPL = false>
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
    uint2* xsum_raw = (uint2*)(smem + 2 * L::XS);            // [2][SG][MT]
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
    const int GR = a.K / 64;   // groups per row of the matrix
    int G = GR, g0 = 0;        // this workgroup's groups: [g0, g0 + G)
    if constexpr (KSPL) {
        g0 = (int)blockIdx.y * a.gsplit;
        G = min(a.gsplit, GR - g0);
        a.x += (int64_t)g0 * 64;
        a.y += (int64_t)blockIdx.y * a.M * a.y_row_stride;
    }
    const int NS = (G + SG - 1) / SG;
    // workgroups on one XCD are 8 apart in blockIdx.x: spread their starts
    const int rot = (int)((unsigned)(b >> 3) * (unsigned)SG % (unsigned)G);
    const int64_t wpr = a.K / 8;
    const int n = ct * CH_NT + wn * 32 + l32;                // this lane's column
    const int nc = min(n, a.N - 1);
    // words 4h..4h+3 of group g0
    const uint32_t* wrow = a.wq + (int64_t)nc * wpr + (int64_t)g0 * 8 + 4 * h;
    // SBL: the tile's copy in LDS ([64 G] scales, then [64 G] biases)
    uint16_t* sbl = (uint16_t*)(smem + L::bytes / 16);
    const uint16_t* srow = SBL ? sbl + (nc - ct * CH_NT) * (G + 2) : a.s + (int64_t)nc * GR + g0;
    const uint16_t* brow = SBL ? sbl + (64 + nc - ct * CH_NT) * (G + 2) : a.b + (int64_t)nc * GR + g0;

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
    // xr[i]: X of stage st + 1 + i while stage st runs (a ring when XD = 2;
    // stage parity picks the slot, and rounds hold an even number of stages)
    uint4 xr[XD][SG][IO::XPT];
    if constexpr (SBL) {
        // X first, then the scale/bias runs, then the codes: a wave's loads
        // return in order, so each store below waits only for its own data
        IO::load(a, m0, 0, G, rot, xr[0]);
        __builtin_amdgcn_sched_barrier(0);
        ChunkSb<128 * WM * NKS> sbc;
        sbc.template load<KSPL>(a.s + (int64_t)ct * CH_NT * GR + g0, a.b + (int64_t)ct * CH_NT * GR + g0,
                                G, GR);
#pragma unroll
        for (int e = 0; e < DW; ++e) bq[e] = *(const uint4*)(wrow + (int64_t)rot_group(NKS * e + ks, G, rot) * 8);
        __builtin_amdgcn_sched_barrier(0);
        IO::store(xs_raw, xsum_raw, xr[0]);
        sbc.store((uint32_t*)sbl, G);
        if constexpr (XD == 2) IO::load(a, m0, SG, G, rot, xr[1]);
        __syncthreads();
#pragma unroll
        for (int e = 0; e < DW; ++e) {
            const int g = rot_group(NKS * e + ks, G, rot);
            bs[e] = srow[g];
            bb[e] = brow[g];
        }
    } else {
#pragma unroll
        for (int e = 0; e < DW; ++e) {
            const int g = rot_group(NKS * e + ks, G, rot);
            bq[e] = *(const uint4*)(wrow + (int64_t)g * 8);
            bs[e] = srow[g];
            bb[e] = brow[g];
        }
        IO::load(a, m0, 0, G, rot, xr[0]);
        IO::store(xs_raw, xsum_raw, xr[0]);
        if constexpr (XD == 2) IO::load(a, m0, SG, G, rot, xr[1]);
        __syncthreads();
    }

    // one group (step g, slot e): the row blocks' MFMA chains in turn into
    // a two-slot ring P; block mb - 1's scaling, acc += s P, is issued after
    // block mb's MFMAs (it does not depend on them, so it runs while they
    // do); then the slot is refilled with step g + D. xs: this lane's
    // A-operand row (row 32 MB wm + l32, k-half h) of the group. The bias
    // part, b Xsum, is added per stage on the matrix core (bias_mfma below).
    auto group = [&](const int g, auto ec, const uint4* xs) __attribute__((always_inline)) {
        constexpr int e = decltype(ec)::value;
        const uint32_t wv[4] = {bq[e].x, bq[e].y, bq[e].z, bq[e].w};
        bf16x8_t bfrag[4];
#pragma unroll
        for (int stp = 0; stp < 4; ++stp)
            bfrag[stp] = __builtin_bit_cast(bf16x8_t, F16 ? codes_f16(wv[stp]) : codes_bf16(wv[stp]));
        // one conversion here: folded into each FMA, the compiler would emit the
        // mixed-precision FMA, which issues at half the rate of a plain one
        float sf = h2f((uint16_t)bs[e]);
        asm volatile("" : "+v"(sf));
        floatx16 P[2];
        auto scale = [&](auto mbc) __attribute__((always_inline)) {
            constexpr int mb = decltype(mbc)::value;
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mb][i] = fmaf(sf, P[mb & 1][i], acc[mb][i]);
        };
        static_for<0, MB>([&](auto mbc) __attribute__((always_inline)) {
            constexpr int mb = decltype(mbc)::value;
#pragma unroll
            for (int i = 0; i < 16; ++i) P[mb & 1][i] = 0.f;
#pragma unroll
            for (int stp = 0; stp < 4; ++stp) {
                const uint4 av = xs[32 * mb * XS_STRIDE + stp];
                if constexpr (F16)
                    P[mb & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        __builtin_bit_cast(halfx8_c, av), __builtin_bit_cast(halfx8_c, bfrag[stp]),
                        P[mb & 1], 0, 0, 0);
                else
                    P[mb & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8_t, av), bfrag[stp], P[mb & 1], 0, 0, 0);
            }
            if constexpr (mb > 0) scale(std::integral_constant<int, mb - 1>{});
        });
        scale(std::integral_constant<int, MB - 1>{});
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

    // Bias of this wave's groups of one stage: acc += sum_g Xsum_g[m] b_g[n]
    // as one MFMA per row block, both factors as three bf16 parts
    // (mfma.h: six exact cross products, within 2^-25 of the fp32 product).
    // Lane half h carries the wave's group j = h of the stage (JS = 2); with
    // one group per wave (JS = 1) half 1 has B = 0. xsum: this lane's staged
    // parts of that group for row 0 of the tile.
    static_assert(JS == 1 || JS == 2, "bias slots");
    auto bias_mfma = [&](const int st, auto sjc, auto checked, const uint2* xsum)
                         __attribute__((always_inline)) {
        constexpr int sj = decltype(sjc)::value;
        float bv[JS];
#pragma unroll
        for (int j = 0; j < JS; ++j) {
            const int e = sj * JS + j;
            bv[j] = h2f((uint16_t)bb[e]);
            if constexpr (decltype(checked)::value)
                if (st * SG + NKS * j + ks >= G) bv[j] = 0.f;
        }
        const float bsel = JS == 2 ? (h ? bv[JS - 1] : bv[0]) : (h ? 0.f : bv[0]);
        const bf16x8_t bfrag = __builtin_bit_cast(bf16x8_t, bias_b_operand(bsel));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const uint2 r = xsum[32 * MB * wm + 32 * mb + l32];
            const bf16x8_t afrag = __builtin_bit_cast(bf16x8_t, bias_a_operand(r));
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
        bias_mfma(st, sjc, checked, xsum_raw + opaque(buf * SG * MT + (ks + (JS == 2 ? NKS * h : 0)) * MT));
        // group j of this wave is stage group NKS j + ks
        const uint4* xs = xs_raw + opaque(buf * L::XS + ks * MT * XS_STRIDE +
                                          (32 * MB * wm + l32) * XS_STRIDE + 4 * h);
        static_for<0, JS>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            const int g = st * SG + NKS * j + ks;
            constexpr std::integral_constant<int, sj * JS + j> ec{};
            const uint4* xsj = xs + NKS * j * MT * XS_STRIDE;
            if constexpr (decltype(checked)::value) {
                if (g < G) group(g, ec, xsj);
            } else {
                group(g, ec, xsj);
            }
        });
        IO::store(xs_raw + (buf ^ 1) * L::XS, xsum_raw + (buf ^ 1) * SG * MT, xr[sv]);
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

// Y = sum of the split slices part[0..splits) ([splits][n] fp32), added in
// split order, so results do not depend on timing. Four elements per thread.
__global__ __launch_bounds__(256) void chunk_ksum_kernel(const float* __restrict__ part,
                                                         float* __restrict__ y, int splits,
                                                         int64_t n) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    if ((n & 3) == 0) {
        float4 acc = *(const float4*)(part + i);
        for (int sp = 1; sp < splits; ++sp) {
            const float4 v = *(const float4*)(part + (int64_t)sp * n + i);
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        *(float4*)(y + i) = acc;
        return;
    }
    for (int64_t j = i; j < min(i + 4, n); ++j) {
        float acc = part[j];
        for (int sp = 1; sp < splits; ++sp) acc += part[(int64_t)sp * n + j];
        y[j] = acc;
    }
}

// K split of a call with fewer than CH_SPLIT_TILES tiles, which would leave
// CUs idle (a short N, e.g. a down projection over a few dozen tokens):
// enough splits that tiles x splits reaches CH_SPLIT_WG workgroups, each
// split at least CH_SPLIT_MIN_G groups and, when 8 | G, a multiple of 8 (the
// scale/bias LDS copy then still applies). Depends on the shape only, so a
// shape always sums in the same order.
constexpr int CH_SPLIT_TILES = 128;
constexpr int CH_SPLIT_WG = 256;
constexpr int CH_SPLIT_MIN_G = 16;

static int chunk_row_tile(int M) { return M <= 32 ? 32 : M <= 64 ? 64 : 128; }

ChunkSplit chunk_split(int M, int N, int K) {
    const int G = K / 64;
    if (M < 1 || N < 1 || G < 1 || M > CH_MMAX) return {1, G};
    const int tiles = ((N + CH_NT - 1) / CH_NT) * ((M + chunk_row_tile(M) - 1) / chunk_row_tile(M));
    const int sp = min((CH_SPLIT_WG + tiles - 1) / tiles, G / CH_SPLIT_MIN_G);
    if (tiles >= CH_SPLIT_TILES || sp <= 1) return {1, G};
    int gs = (G + sp - 1) / sp;
    if (G % 8 == 0) gs = (gs + 7) / 8 * 8;   // splits start on 16-byte scale/bias runs
    return {(G + gs - 1) / gs, gs};
}

size_t chunk_split_workspace_bytes(int M, int N, int K) {
    const ChunkSplit c = chunk_split(M, N, K);
    return c.splits > 1 ? (size_t)c.splits * M * N * sizeof(float) : 0;
}

template <int SG, int D, int MB, int WM, int NKS, bool F16, bool SBL = false, bool KSPL = false>
static hipError_t launch_chunk_cfg(const ChunkArgs& a, hipStream_t st, int splits = 1) {
    constexpr int MT = 32 * MB * WM;
    const int RT = (a.M + MT - 1) / MT;
    const int grid = ((a.ncol_tiles + 7) / 8) * 8 * RT;
    const size_t lds = ChunkLds<SG, MT, F16>::bytes +
                       (SBL ? (size_t)256 * ((KSPL ? a.gsplit : a.K / 64) + 2) : 0);
    if (lds > device_info().max_lds_per_block) return hipErrorInvalidValue;
    constexpr int threads = 128 * WM * NKS;
    auto kern = chunk_gemm_kernel<SG, D, MB, WM, NKS, 1, F16, SBL, KSPL>;
    (void)occupancy((const void*)kern, threads, lds);  // sets the dynamic-LDS limit once
    hipLaunchKernelGGL(kern, dim3(grid, splits), dim3(threads), lds, st, a);
    return hipGetLastError();
}

// The K-split launch: the partial slices go to `part` ([splits][M][N]), then
// one pass adds them into y.
template <int SG, int D, int MB, int WM, int NKS, bool F16>
static hipError_t launch_chunk_split(ChunkArgs a, const ChunkSplit& c, float* part, hipStream_t st) {
    float* y = a.y;
    a.y = part;
    a.gsplit = c.gsplit;
    // the scale/bias copy as unsplit: row tiles up to 64 (the 128-row tile's
    // staging leaves no LDS for it), whole column tiles, 8 | split length
    const int G = a.K / 64;
    hipError_t e;
    if (32 * MB * WM <= 64 && a.N % CH_NT == 0 && G % 8 == 0 && c.gsplit % 8 == 0 &&
        c.gsplit <= CH_SB_GMAX)
        e = launch_chunk_cfg<SG, D, MB, WM, NKS, F16, 32 * MB * WM <= 64, true>(a, st, c.splits);
    else
        e = launch_chunk_cfg<SG, D, MB, WM, NKS, F16, false, true>(a, st, c.splits);
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)a.M * a.N;
    hipLaunchKernelGGL(chunk_ksum_kernel, dim3((unsigned)((n + 1023) / 1024)), dim3(256), 0, st,
                       (const float*)part, y, c.splits, n);
    return hipGetLastError();
}

// Up to 64 rows the tile's scales and biases go through LDS when the column
// tiles are whole and the rows short enough (ChunkSb).
template <int SG, int D, int MB, int WM, int NKS, bool F16>
static hipError_t launch_chunk_sb(const ChunkArgs& a, hipStream_t st) {
    const int G = a.K / 64;
    if (a.N % CH_NT == 0 && G % 8 == 0 && G <= CH_SB_GMAX)
        return launch_chunk_cfg<SG, D, MB, WM, NKS, F16, true>(a, st);
    return launch_chunk_cfg<SG, D, MB, WM, NKS, F16, false>(a, st);
}

hipError_t launch_chunk_gemm(int bits, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                             const uint16_t* x, int xkind, float* y, int M, int N, int K,
                             void* ws, size_t ws_bytes, hipStream_t st) {
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
// and a ring of 8 groups. With a workspace, shapes with few tiles split K
// (chunk_split) on the same configurations.
    const ChunkSplit c = chunk_split(M, N, K);
    if (ws != nullptr && c.splits > 1) {
        if (ws_bytes < chunk_split_workspace_bytes(M, N, K)) return hipErrorInvalidValue;
        float* part = (float*)ws;
        if (xkind == X_F16) {
            if (M <= 32) return launch_chunk_split<4, 8, 1, 1, 2, true>(a, c, part, st);
            if (M <= 64) return launch_chunk_split<4, 8, 2, 1, 4, true>(a, c, part, st);
            return launch_chunk_split<4, 8, 4, 1, 4, true>(a, c, part, st);
        }
        if (M <= 32) return launch_chunk_split<4, 8, 1, 1, 2, false>(a, c, part, st);
        if (M <= 64) return launch_chunk_split<4, 8, 2, 1, 4, false>(a, c, part, st);
        return launch_chunk_split<4, 8, 4, 1, 4, false>(a, c, part, st);
    }
    if (xkind == X_F16) {
        if (M <= 32) return launch_chunk_sb<4, 8, 1, 1, 2, true>(a, st);
        if (M <= 64) return launch_chunk_sb<4, 8, 2, 1, 4, true>(a, st);
        return launch_chunk_cfg<4, 8, 4, 1, 4, true>(a, st);
    }
    if (M <= 32) return launch_chunk_sb<4, 8, 1, 1, 2, false>(a, st);
    if (M <= 64) return launch_chunk_sb<4, 8, 2, 1, 4, false>(a, st);
    return launch_chunk_cfg<4, 8, 4, 1, 4, false>(a, st);
}

}  // namespace qd
