// MoE experts for a prefill chunk (T > 1 tokens) on MFMA, grouped by expert.
//
// [TF] jeff.news/article/5193, section "내부 구조가 진짜 흥미로운 부분"
// (internals): prefill runs in chunks of at most 128 tokens so that one fetch
// of an expert serves many rows; the shared expert's output is combined with
// the routed output. Same readings as the decode path (moe.hip): routed
// outputs weighted by the renormalized router weights, shared output with
// weight one, GELU gate, fp32 intermediates.
//
// Four launches:
//   1. prep: a counting sort of the T*k (token, slot) pairs by expert
//      (offsets, sorted pair list, each pair's position; pairs with an expert
//      id outside [0, E) are dropped), and a table of the experts' 32-row
//      blocks of sorted pairs;
//   2. gate+up: one workgroup per (32-row block, 64 columns of I): two gate
//      waves and two up waves each stream their 32 weight rows against the
//      block's gathered activation rows (staged once in LDS) on the matrix
//      core (exact codes as the operand, as in chunk.hip), then
//      h' = p * GELU(gate) * up is split into bf16 hi + lo (16 significant
//      bits) for the next MFMA. The shared expert adds row blocks of all T
//      tokens with weight one;
//   3. down: one workgroup per (32-row block, 128 columns of H) runs hi and
//      lo MFMA chains against the same codes and writes each pair's output
//      row;
//   4. combine: y[t] = o_shared[t] + sum over the token's slots of its
//      (already weighted) pair rows, in slot order.
// Every expert's weights are read once per 32 of its pairs; nothing uses
// atomics on the data path, so results are run-to-run deterministic. The
// expert kernels have no barrier in their main loop: codes, scales and
// biases run several groups ahead in a register ring and activations a few
// groups ahead, so each wave keeps its loads in flight while it computes.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "mfma.h"

namespace qd {

typedef _Float16 halfx8_t __attribute__((ext_vector_type(8)));

struct PrefillWs {
    int* sorted_pair;   // [T*k] pair ids (t*k + j) grouped by expert
    int* pos;           // [T*k] sorted position of each pair, -1 if dropped
    int* offs;          // [E+1] first sorted position of each expert
    int* rbs;           // [E+1] first 32-row block of each expert
    int4* rbinfo;       // [row blocks] (expert, first sorted row, rows, 0)
    int* stok;          // [T*k] token of each sorted row
    uint16_t* hhi;      // [T*k][I] bf16 high part of h' (sorted rows)
    uint16_t* hlo;      // [T*k][I] bf16 low part
    uint16_t* shhi;     // [T][Is]
    uint16_t* shlo;     // [T][Is]
    float* O;           // [T*k][H] weighted routed outputs (sorted rows)
    float* Os;          // [T][H] shared-expert outputs
};

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Routed 32-row blocks: at most ceil(P / 32) full ones plus one partial block
// per expert.
static int max_row_blocks(int P, int E) { return (P + 31) / 32 + E; }

static PrefillWs carve(void* base, const MoeArgs& m, int T, int k, size_t* total) {
    PrefillWs w{};
    char* p = (char*)base;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* r = p ? p + off : nullptr;
        off = align256(off + bytes);
        return r;
    };
    const size_t P = (size_t)T * k;
    w.sorted_pair = (int*)take(P * 4);
    w.pos = (int*)take(P * 4);
    w.offs = (int*)take(((size_t)m.E + 1) * 4);
    w.rbs = (int*)take(((size_t)m.E + 1) * 4);
    w.rbinfo = (int4*)take((size_t)max_row_blocks((int)P, m.E) * 16);
    w.stok = (int*)take(P * 4);
    w.hhi = (uint16_t*)take(P * m.I * 2);
    w.hlo = (uint16_t*)take(P * m.I * 2);
    w.shhi = (uint16_t*)take((size_t)T * m.Is * 2);
    w.shlo = (uint16_t*)take((size_t)T * m.Is * 2);
    w.O = (float*)take(P * m.H * 4);
    w.Os = (float*)take((size_t)T * m.H * 4);
    if (total) *total = off;
    return w;
}

size_t moe_prefill_workspace_bytes(const MoeArgs& m, int T, int k) {
    size_t total = 0;
    carve(nullptr, m, T, k, &total);
    return total;
}

// ---------------------------------------------------------------------------
// 1. prep
// ---------------------------------------------------------------------------
constexpr int PREP_MAX_PAIRS = 128 * 32;
constexpr int PREP_MAX_E = 1024;

__global__ __launch_bounds__(1024) void moe_prep_kernel(const int32_t* __restrict__ idx, int T,
                                                        int k, int E, PrefillWs w) {
    __shared__ int sidx[PREP_MAX_PAIRS];
    __shared__ int cnt[PREP_MAX_E + 1];
    __shared__ int rbl[PREP_MAX_E + 1];
    const int P = T * k;
    const int tid = threadIdx.x, bs = blockDim.x;
    for (int i = tid; i < P; i += bs) sidx[i] = idx[i];
    for (int e = tid; e <= E; e += bs) cnt[e] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += bs) {
        const int e = sidx[p];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    // exclusive prefix sums of the counts and of their 32-row blocks: a
    // double-buffered Hillis-Steele scan over the E + 1 entries (the last one
    // 0, so entry E receives the totals), log2 steps instead of a serial walk
    {
        __shared__ int sc[2][PREP_MAX_E + 1], sb[2][PREP_MAX_E + 1];
        for (int e = tid; e <= E; e += bs) {
            const int c = e < E ? cnt[e] : 0;
            sc[0][e] = c;
            sb[0][e] = (c + 31) / 32;
        }
        __syncthreads();
        int cur = 0;
        for (int off = 1; off <= E; off <<= 1) {
            for (int e = tid; e <= E; e += bs) {
                sc[cur ^ 1][e] = sc[cur][e] + (e >= off ? sc[cur][e - off] : 0);
                sb[cur ^ 1][e] = sb[cur][e] + (e >= off ? sb[cur][e - off] : 0);
            }
            cur ^= 1;
            __syncthreads();
        }
        // inclusive -> exclusive
        for (int e = tid; e <= E; e += bs) {
            cnt[e] = e ? sc[cur][e - 1] : 0;
            rbl[e] = e ? sb[cur][e - 1] : 0;
        }
    }
    __syncthreads();
    for (int e = tid; e <= E; e += bs) {
        w.offs[e] = cnt[e];
        w.rbs[e] = rbl[e];
    }
    for (int e = tid; e < E; e += bs)
        for (int r = rbl[e]; r < rbl[e + 1]; ++r) {
            const int r0 = cnt[e] + 32 * (r - rbl[e]);
            w.rbinfo[r] = make_int4(e, r0, min(32, cnt[e + 1] - r0), 0);
        }
    __syncthreads();  // offsets are read before the counters advance
    // placement: a slot inside the expert's range from an LDS counter. The
    // order inside an expert's rows does not change any result (every output
    // row is its own dot-product chain), only which row a pair occupies.
    for (int p = tid; p < P; p += bs) {
        const int e = sidx[p];
        if (e >= 0 && e < E) {
            const int ps = atomicAdd(&cnt[e], 1);
            w.pos[p] = ps;
            w.sorted_pair[ps] = p;
            w.stok[ps] = p / k;
        } else {
            w.pos[p] = -1;
        }
    }
}

// ---------------------------------------------------------------------------
// Shared pieces
// ---------------------------------------------------------------------------
template <bool F16>
__device__ __forceinline__ floatx16 mfma16(const uint4& a, const uint4& b, const floatx16& c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8_t, a),
                                                      __builtin_bit_cast(halfx8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Calls f(integral_constant<int, I>) for I = 0 .. N-1 (compile-time indices).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Keeps the compiler from sinking an accumulator update past later groups
// (which would hold several groups' partial products live at once).
__device__ __forceinline__ void pin(floatx16& v) { asm volatile("" : "+v"(v)); }

// A copy of v the compiler cannot see through or hoist out of a loop: keeps
// per-group LDS offsets as immediates on a per-stage base.
__device__ __forceinline__ int opaque_i(int v) {
    int r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
    return r;
}

// The codes enter the matrix core as the codes q themselves (fp16 or bf16,
// through the fp8 converter: mfma.h), in the k order [0, 4, 1, 5, 2, 6, 3, 7].
// The activations are staged in LDS in the same order (perm8 below).

// 8 16-bit values e0..e7 -> e0 e4 e1 e5 e2 e6 e3 e7 (the codes' order).
__device__ __forceinline__ uint4 perm8(uint4 v) {
    // v_perm_b32(src0, src1, sel): selector bytes 0..3 pick src1's bytes, 4..7 src0's
    return make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u),
                      __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                      __builtin_amdgcn_perm(v.w, v.y, 0x05040100u),
                      __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
}

// Both expert kernels: a workgroup of 4 waves owns one 32-row block and 4
// weight-row tiles of 32 (one per wave). The block's activation rows are
// staged in LDS a stage of XSG groups at a time (double buffered, one barrier
// per stage; the next stage is read into registers while the current one is
// consumed), permuted to the codes' k order and with their per-group row
// sums, so each activation byte is fetched once per workgroup rather than
// once per wave. Each wave keeps its codes, scales and biases XD groups
// ahead in a register ring. Per group a wave runs one MFMA chain per
// activation plane on the codes and adds s P; the bias term, b Xsum, is
// added once per stage on the matrix core.
constexpr int XSG = 4;       // groups per stage
static_assert(XSG == 4, "the stage bias runs two groups per MFMA, two MFMAs");
constexpr int XD = 4;        // groups of codes in flight per wave (whole stages)
constexpr int XPF = 1;       // stages of activations in flight (1 or 2)
constexpr int GU_WAVES = 4;  // gate+up workgroup: 2 gate + 2 up waves
constexpr int DN_WAVES = 4;  // down workgroup: 4 column tiles
// two waves per SIMD: two workgroups share a CU, so one's latency-bound
// phases (start, stage barriers) overlap the other's work
constexpr int XWPE = 2;

// LDS: [2 buffers][PLANES][XSG groups][GS] uint4 (a group = 32 rows of
// XS_STRIDE uint4 plus one, so that the staging stores of a row's groups
// start in different banks), then the per-group row sums (over the planes)
// as bias-product parts (bias_row_parts), xsum [2 buffers][XSG][32 rows]
// uint2 (row-contiguous: the lanes of a bias read hit distinct banks).
// NW waves stage: TPG = NW / 2 threads share a (row, group) and each holds
// UPT = 8 / TPG of its 16-byte chunks.
template <int PLANES, bool F16, int NW>
struct XStage {
    static constexpr int GS = 32 * XS_STRIDE + 1;       // uint4 per staged group
    static constexpr int PER = XSG * GS;                // uint4 per plane per buffer
    static constexpr int BUF = PLANES * PER;
    static constexpr int SUMS = 2 * 32 * XSG;          // uint2 (both buffers)
    static constexpr int LDS_UINT4 = 2 * BUF + SUMS / 2;
    static constexpr int TPG = NW / 2;
    static constexpr int UPT = 8 / TPG;
    static_assert(TPG * XSG * 32 == 64 * NW, "staging split");
    // thread t: row t / (TPG XSG), group (t / TPG) % XSG, chunks UPT (t % TPG) ..
    __device__ static __forceinline__ void load(const uint16_t* const (&row)[PLANES], int g0, int G,
                                                uint4 (&r)[PLANES][UPT]) {
        const int part = threadIdx.x % (TPG * XSG);
        const int g = min(g0 + part / TPG, G - 1);
        const int c = UPT * (part % TPG);
#pragma unroll
        for (int pl = 0; pl < PLANES; ++pl) {
            const uint4* src = (const uint4*)(row[pl] + (int64_t)g * 64 + 8 * c);
#pragma unroll
            for (int i = 0; i < UPT; ++i) {
                // a value temporary: a struct copy between pointers becomes a
                // memcpy that keeps the array in scratch memory
                const uint4 v = src[i];
                r[pl][i] = v;
            }
        }
    }
    __device__ static __forceinline__ void store(uint4* buf, uint2* xsum, const uint4 (&r)[PLANES][UPT]) {
        const int rr = threadIdx.x / (TPG * XSG), part = threadIdx.x % (TPG * XSG);
        const int gi = part / TPG, c = UPT * (part % TPG);
        float acc = 0.f;
#pragma unroll
        for (int pl = 0; pl < PLANES; ++pl) {
            uint4* dst = buf + pl * PER + gi * GS + rr * XS_STRIDE + c;
#pragma unroll
            for (int i = 0; i < UPT; ++i) {
                const uint4 v = r[pl][i];
                dst[i] = perm8(v);
                const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc = F16 ? dot2(vv[j], 0x3C003C00u, acc) : bf16_pair_sum(vv[j], acc);
            }
        }
        acc = seg_sum<TPG>(acc);   // the TPG adjacent lanes of (row, group)
        // the TPG threads of (row, group) store the same parts
        xsum[gi * 32 + rr] = bias_row_parts(acc);
    }
};

// Per-wave ring of one weight row's codes, scales and biases (lane: words
// 4h..4h+3 of each group). The scale and bias rows are either global
// memory or a copy in LDS (sb_block below); the codes are always global.
template <int D>
struct CodeRing {
    uint4 q[D];
    uint32_t s[D], b[D];
    const uint32_t* wrow;
    const uint16_t *srow, *brow;
    int G;
    __device__ __forceinline__ void init(const uint32_t* w, const uint16_t* sr, const uint16_t* br, int g) {
        wrow = w;
        srow = sr;
        brow = br;
        G = g;
#pragma unroll
        for (int d = 0; d < D; ++d) fill(d, d);
    }
    // codes only (the scale and bias rows are set later)
    __device__ __forceinline__ void init_q(const uint32_t* w, int g) {
        wrow = w;
        G = g;
#pragma unroll
        for (int d = 0; d < D; ++d) q[d] = *(const uint4*)(wrow + (int64_t)min(d, G - 1) * 8);
    }
    __device__ __forceinline__ void init_sb(const uint16_t* sr, const uint16_t* br) {
        srow = sr;
        brow = br;
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int g = min(d, G - 1);
            s[d] = srow[g];
            b[d] = brow[g];
        }
    }
    __device__ __forceinline__ void fill(int d, int g) {
        g = min(g, G - 1);
        q[d] = *(const uint4*)(wrow + (int64_t)g * 8);
        s[d] = srow[g];
        b[d] = brow[g];
    }
    __device__ __forceinline__ void fill_q(int d, int g) {
        q[d] = *(const uint4*)(wrow + (int64_t)min(g, G - 1) * 8);
    }
};

// Scales and biases of a wave's 32 consecutive weight rows through LDS. Read
// per lane (one row each), every 2-byte value would cost its own cache-line
// access; the rows' values are one contiguous block of 32 G halfwords (64 G
// bytes, 16-byte aligned when the arrays are), so the wave copies each block
// with 16-byte loads, lane after lane, and the ring reads its values from LDS.
// For even G the rows are stored RS = 2 ((G / 2) | 1) halfwords apart (an odd
// number of dwords, so the 32 rows a wave reads at once fall in different
// banks); for odd G they stay G apart. Up to SB_GMAX groups per row (4 loads
// per lane per block); the LDS copy takes 2 x 32 RS halfwords.
constexpr int SB_GMAX = 64;
__host__ __device__ constexpr int sb_row_stride(int G) { return G % 2 ? G : 2 * ((G / 2) | 1); }
struct SbBlock {
    uint4 vs[SB_GMAX / 16], vb[SB_GMAX / 16];
    // issue the loads of both blocks (indices clamp to the block)
    __device__ __forceinline__ void load(const uint16_t* s, const uint16_t* b, int G) {
        const int lane = threadIdx.x & 63, n16 = 4 * G;
#pragma unroll
        for (int k = 0; k < SB_GMAX / 16; ++k) {
            const int i = min(lane + 64 * k, n16 - 1);
            vs[k] = ((const uint4*)s)[i];
            vb[k] = ((const uint4*)b)[i];
        }
    }
    // store them at dst: [32 rows][RS] scales, then the same for the biases
    __device__ __forceinline__ void store(uint16_t* dst, int G) const {
        const int lane = threadIdx.x & 63, n16 = 4 * G, rs = sb_row_stride(G);
        if (G % 2) {
#pragma unroll
            for (int k = 0; k < SB_GMAX / 16; ++k) {
                const int i = lane + 64 * k;
                if (i < n16) {
                    ((uint4*)dst)[i] = vs[k];
                    ((uint4*)dst)[n16 + i] = vb[k];
                }
            }
            return;
        }
        // dword j of a block: row j / (G / 2), column j mod (G / 2)
        const int rdw = G / 2, prdw = rs / 2;
        uint32_t* d = (uint32_t*)dst;
#pragma unroll
        for (int k = 0; k < SB_GMAX / 16; ++k) {
            const int i = lane + 64 * k;
            if (i < n16) {
                const uint32_t ws[4] = {vs[k].x, vs[k].y, vs[k].z, vs[k].w};
                const uint32_t wb[4] = {vb[k].x, vb[k].y, vb[k].z, vb[k].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 4 * i + e, r = j / rdw, c = j - r * rdw;
                    d[r * prdw + c] = ws[e];
                    d[(32 + r) * prdw + c] = wb[e];
                }
            }
        }
    }
};

// Where stream_expert takes the scales and biases from. SbInRing: the ring
// holds them (per lane from global memory, or from an SbBlock copy).
struct SbInRing {
    static constexpr bool staged = false;
    __device__ __forceinline__ void load(int) {}
    __device__ __forceinline__ void store(int) {}
    __device__ __forceinline__ void read(int, uint2&, uint2&) const {}
};

// SbStaged: staged per stage with the activations, for a workgroup of 4 waves
// over 128 consecutive weight rows. Thread t requests the stage's 4 values of
// row t mod 128 in array t / 128 (scales, then biases): those rows lie a few
// cache lines apart, so a wave instruction touches a few lines instead of
// one per lane. They go to LDS with the activations; a lane then reads its
// row's 4 scales and 4 biases with two 8-byte LDS reads.
struct SbStaged {
    static constexpr bool staged = true;
    uint2 (*lds)[2][128];   // [2 buffers][2 arrays][128 rows]
    const uint16_t* row;    // this thread's row of its array
    int G;
    uint32_t v[4];
    __device__ __forceinline__ void load(int st) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = row[min(4 * st + i, G - 1)];
    }
    __device__ __forceinline__ void store(int buf) {
        lds[buf][threadIdx.x / 128][threadIdx.x % 128] = make_uint2(v[0] | (v[1] << 16), v[2] | (v[3] << 16));
    }
    // this lane's row of the workgroup: 32 wave + l32
    __device__ __forceinline__ void read(int buf, uint2& s4, uint2& b4) const {
        const int r = 32 * __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) + (threadIdx.x & 31);
        s4 = lds[buf][0][r];
        b4 = lds[buf][1][r];
    }
};

// Streams the G groups of a wave's weight row against the staged activation
// planes: acc (D layout, 32 rows x this lane's column) += sum over groups of
// s P_g + b Xsum_g, with P_g the group's product on the codes q. The first part
// runs in fp32 per group; the second, once per stage on the matrix core. NQ =
// row quarters (8 rows) that hold data: the per-group scaling skips the
// others. Whole rounds of XD groups run with no
// data-dependent exits (an exit inside a round would make the compiler wait
// for every load in flight where the paths join); the last partial round runs
// with checks.
//
// Prologue: the first stage of activations is requested first, then issue()
// requests the ring's first weights (a wave's loads return in order, so the
// staging waits only for the activations), and finish() runs after the
// staging stores, before the barrier.
template <int PLANES, bool F16, int NW, int NQ, typename Sb, typename Issue, typename Finish>
__device__ __forceinline__ void stream_expert(int G, uint4* lds, const uint16_t* const (&row)[PLANES],
                                              CodeRing<XD>& ring, Sb& sb, floatx16& acc, Issue&& issue,
                                              Finish&& finish) {
    static_assert(!Sb::staged || NW == 4, "staged scales: 4 waves over 128 rows");
    using XS = XStage<PLANES, F16, NW>;
    constexpr int SPR = XD / XSG;
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5, l32 = lane & 31;
    uint2* xsum_raw = (uint2*)(lds + 2 * XS::BUF);
    const int NS = (G + XSG - 1) / XSG;

    // activations run XPF stages ahead. XPF = 2: register set st & 1 receives
    // stage st + 2 while set (st + 1) & 1 holds stage st + 1 until it is
    // stored; XPF = 1: one set, loaded at the stage's start, stored at its end.
    static_assert(XPF == 1 || (XPF == 2 && SPR % 2 == 0), "prefetch depth");
    uint4 xr0[PLANES][XS::UPT], xr1[PLANES][XS::UPT];
    XS::load(row, 0, G, xr0);
    if constexpr (XPF == 2) XS::load(row, XSG, G, xr1);
    sb.load(0);
    __builtin_amdgcn_sched_barrier(0);
    issue();
    __builtin_amdgcn_sched_barrier(0);
    XS::store(lds, xsum_raw, xr0);
    sb.store(0);
    finish();
    __syncthreads();
    auto stage = [&](const int st, auto sjc, auto checked) __attribute__((always_inline)) {
        constexpr int sj = decltype(sjc)::value;   // st mod SPR (rounds hold SPR stages)
        constexpr bool chk = decltype(checked)::value;
        const int buf = st & 1;
        auto& xin = [&]() -> auto& { if constexpr (XPF == 2 && sj % 2 == 1) return xr1; else return xr0; }();
        auto& xout = [&]() -> auto& { if constexpr (XPF == 2 && sj % 2 == 0) return xr1; else return xr0; }();
        XS::load(row, (st + XPF) * XSG, G, xin);
        sb.load(st + 1);
        // staged scales and biases of this stage (4 each, 16-bit halves)
        uint2 s4, b4;
        sb.read(buf, s4, b4);
        auto half16 = [](const uint2& v, int gi) __attribute__((always_inline)) {
            const uint32_t w = gi < 2 ? v.x : v.y;
            return (gi & 1) ? (w >> 16) : (w & 0xFFFFu);
        };
        // bias of the stage's groups as two MFMAs (groups 2p + h on lane
        // half h), both factors as three bf16 parts (mfma.h: six exact cross
        // products per group, within 2^-25 of the fp32 product)
        {
            float bv[4];
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {   // b
                bv[gi] = h2f((uint16_t)(Sb::staged ? half16(b4, gi) : ring.b[sj * XSG + gi]));
                if constexpr (chk)
                    if (st * XSG + gi >= G) bv[gi] = 0.f;
            }
            const uint2* xp = xsum_raw + buf * 32 * XSG + opaque_i(h * 32 + l32);
#pragma unroll
            for (int p = 0; p < 2; ++p)
                acc = mfma16<false>(bias_a_operand(xp[2 * p * 32]),
                                    bias_b_operand(h ? bv[2 * p + 1] : bv[2 * p]), acc);
        }
        const uint4* xs = lds + opaque_i(buf * XS::BUF + l32 * XS_STRIDE + 4 * h);
        // groups in pairs: two independent MFMA chains interleave on the matrix
        // core (one chain alone would wait on each MFMA's result)
        static_for<0, XSG / 2>([&](auto pc) __attribute__((always_inline)) {
            constexpr int g0i = 2 * decltype(pc)::value;
            constexpr int d0 = sj * XSG + g0i, d1 = d0 + 1;
            const int g = st * XSG + g0i;
            if (chk && g >= G) return;
            const bool second = !chk || g + 1 < G;   // uniform
            floatx16 P0, P1;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                P0[i] = 0.f;
                P1[i] = 0.f;
            }
            const uint32_t w0[4] = {ring.q[d0].x, ring.q[d0].y, ring.q[d0].z, ring.q[d0].w};
            const uint32_t w1[4] = {ring.q[d1].x, ring.q[d1].y, ring.q[d1].z, ring.q[d1].w};
#pragma unroll
            for (int stp = 0; stp < 4; ++stp) {
                const uint4 b0 = codes_p<F16>(w0[stp]);
                const uint4 b1 = codes_p<F16>(w1[stp]);
#pragma unroll
                for (int pl = 0; pl < PLANES; ++pl) {
                    P0 = mfma16<F16>(xs[pl * XS::PER + g0i * XS::GS + stp], b0, P0);
                    P1 = mfma16<F16>(xs[pl * XS::PER + (g0i + 1) * XS::GS + stp], b1, P1);
                }
            }
            auto epilogue = [&](const floatx16& P, int d) __attribute__((always_inline)) {
                // one conversion (folded into each FMA the compiler would
                // emit the half-rate mixed-precision form)
                float sf = h2f((uint16_t)(Sb::staged ? half16(s4, d % XSG) : ring.s[d]));
                asm volatile("" : "+v"(sf));
                // rows 8 (i / 4) + 4 h + i % 4: quarter i / 4
#pragma unroll
                for (int i = 0; i < 4 * NQ; ++i) acc[i] = fmaf(sf, P[i], acc[i]);
            };
            epilogue(P0, d0);
            if (second) epilogue(P1, d1);
            pin(acc);
            if constexpr (Sb::staged) {   // the slots' contents are dead now
                ring.fill_q(d0, g + XD);
                ring.fill_q(d1, g + 1 + XD);
            } else {
                ring.fill(d0, g + XD);
                ring.fill(d1, g + 1 + XD);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        XS::store(lds + (buf ^ 1) * XS::BUF, xsum_raw + (buf ^ 1) * 32 * XSG, xout);
        sb.store(buf ^ 1);
        __syncthreads();
    };
    const int rounds = G / XD;
    for (int r = 0; r < rounds; ++r)
        static_for<0, SPR>([&](auto sjc) __attribute__((always_inline)) {
            stage(r * SPR + decltype(sjc)::value, sjc, std::false_type{});
        });
    static_for<0, SPR>([&](auto sjc) __attribute__((always_inline)) {
        const int st = rounds * SPR + decltype(sjc)::value;
        if (st < NS) stage(st, sjc, std::true_type{});
    });
}

// Runs stream_expert with NQ = ceil(M / 8) fixed at compile time.
template <int PLANES, bool F16, int NW, typename Sb, typename Issue, typename Finish>
__device__ __forceinline__ void stream_expert_m(int M, int G, uint4* lds,
                                                const uint16_t* const (&row)[PLANES],
                                                CodeRing<XD>& ring, Sb& sb, floatx16& acc,
                                                Issue&& issue, Finish&& finish) {
    const int nq = (M + 7) / 8;
    if (nq <= 1)
        stream_expert<PLANES, F16, NW, 1>(G, lds, row, ring, sb, acc, issue, finish);
    else if (nq == 2)
        stream_expert<PLANES, F16, NW, 2>(G, lds, row, ring, sb, acc, issue, finish);
    else if (nq == 3)
        stream_expert<PLANES, F16, NW, 3>(G, lds, row, ring, sb, acc, issue, finish);
    else
        stream_expert<PLANES, F16, NW, 4>(G, lds, row, ring, sb, acc, issue, finish);
}

// ---------------------------------------------------------------------------
// 2. gate+up with the GELU gate
// ---------------------------------------------------------------------------
struct GuArgs {
    const uint32_t *gu_q, *sgu_q;
    const uint16_t *gu_s, *gu_b, *sgu_s, *sgu_b;
    const uint16_t* x;   // [T][H] fp16 or bf16 bits
    const float* p;      // [T*k] routing weights in pair order
    int E, H, I, Is, k, T, act;
    int rbmax;           // size of the row-block table
    PrefillWs w;
};

// Workgroup = (32-row block, GT = NW / 2 column tiles of 32): waves 0..GT-1
// the gate rows of tiles GT q + w, waves GT..NW-1 the matching up rows.
// Routed blocks come first (expert from the row-block table), then the
// shared expert's blocks of all T tokens. SBL: scales and biases through
// LDS (SbBlock; dynamic LDS of NW x 128 RS bytes).
template <bool F16, bool SBL>
__global__ __launch_bounds__(64 * GU_WAVES) __attribute__((amdgpu_waves_per_eu(XWPE, XWPE))) void moe_gu_kernel(GuArgs a) {
    constexpr int NW = GU_WAVES, GT = NW / 2;
    __shared__ __align__(16) uint4 lds[XStage<1, F16, NW>::LDS_UINT4];
    __shared__ float zb[GT][32][33];
    extern __shared__ __align__(16) uint4 sbl_raw[];   // SBL: [NW][2][32 G] halfwords
    const int ntc = a.I / 32, ntcs = a.Is / 32;
    const int nq = (ntc + GT - 1) / GT, nqs = (ntcs + GT - 1) / GT;
    const int item = blockIdx.x;
    // both loads issued together: the block record is read speculatively
    // (any index below the table size is valid memory)
    const int R = a.w.rbs[a.E];
    const int4 info = a.w.rbinfo[min(item / nq, a.rbmax - 1)];
    const int items_r = R * nq;
    const int items = items_r + ((a.T + 31) / 32) * nqs;
    if (item >= items) return;   // the whole workgroup leaves together
    const bool shared = item >= items_r;
    int row0, M, q, Iw, ntl;
    const uint32_t* Wq;
    const uint16_t *Ws, *Wb;
    if (!shared) {
        const int rbi = item / nq;
        q = item - rbi * nq;
        const int e = info.x;
        row0 = info.y;
        M = info.z;
        Iw = a.I;
        ntl = ntc;
        const int64_t rows = 2 * (int64_t)a.I;
        Wq = a.gu_q + (int64_t)e * rows * (a.H / 8);
        Ws = a.gu_s + (int64_t)e * rows * (a.H / 64);
        Wb = a.gu_b + (int64_t)e * rows * (a.H / 64);
    } else {
        const int j = item - items_r;
        const int rbk = j / nqs;
        q = j - rbk * nqs;
        row0 = 32 * rbk;
        M = min(32, a.T - row0);
        Iw = a.Is;
        ntl = ntcs;
        Wq = a.sgu_q;
        Ws = a.sgu_s;
        Wb = a.sgu_b;
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int G = a.H / 64;
    const int tile = min(GT * q + wave % GT, ntl - 1);   // clamped: waves past the last tile store nothing
    const int c0 = (wave >= GT ? Iw : 0) + 32 * tile;   // first weight row of this wave
    const int col = c0 + l32;                            // weight row of this lane
    CodeRing<XD> ring;
    SbBlock sbb;
    const int rs = sb_row_stride(G);
    uint16_t* sbl = (uint16_t*)sbl_raw + wave * 64 * rs;   // SBL: this wave's block copy
    auto issue = [&]() __attribute__((always_inline)) {
        if constexpr (SBL) {
            sbb.load(Ws + (int64_t)c0 * G, Wb + (int64_t)c0 * G, G);
            ring.init_q(Wq + (int64_t)col * (a.H / 8) + 4 * h, G);
        } else {
            ring.init(Wq + (int64_t)col * (a.H / 8) + 4 * h, Ws + (int64_t)col * G, Wb + (int64_t)col * G, G);
        }
    };
    auto finish = [&]() __attribute__((always_inline)) {
        if constexpr (SBL) {
            sbb.store(sbl, G);   // read back below by other lanes of this wave only
            ring.init_sb(sbl + l32 * rs, sbl + (32 + l32) * rs);
        }
    };
    // staged row of this thread (rows past M repeat row M - 1; their results
    // are never stored)
    const int sr = min(tid / (NW * 2), M - 1);
    const int tok = shared ? row0 + sr : a.w.stok[row0 + sr];
    const uint16_t* const xrow[1] = {a.x + (int64_t)tok * a.H};
    floatx16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    SbInRing sbr;
    stream_expert_m<1, F16, NW>(M, G, lds, xrow, ring, sbr, acc, issue, finish);

    // up waves -> LDS; each gate wave forms h' = p GELU(gate) up
    if (wave >= GT) {
#pragma unroll
        for (int i = 0; i < 16; ++i) zb[wave - GT][8 * (i / 4) + 4 * h + (i % 4)][l32] = acc[i];
    }
    __syncthreads();
    if (wave >= GT || GT * q + wave >= ntl) return;
    uint16_t* dhi = shared ? a.w.shhi : a.w.hhi;
    uint16_t* dlo = shared ? a.w.shlo : a.w.hlo;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i / 4) + 4 * h + (i % 4);
        if (r < M) {
            const float u = acc[i];
            float gl;
            if (a.act == 1) {
                const float cc = 0.7978845608028654f;
                gl = 0.5f * u * (1.f + tanhf(cc * (u + 0.044715f * u * u * u)));
            } else {
                gl = 0.5f * u * (1.f + erff(u * 0.7071067811865476f));
            }
            const float pw = shared ? 1.f : a.p[a.w.sorted_pair[row0 + r]];
            const float v = pw * gl * zb[wave][r][l32];
            const uint16_t hi = f2bf_rne(v);
            const uint16_t lo = f2bf_rne(v - bf2f_bits(hi));
            const int64_t o = (int64_t)(row0 + r) * Iw + 32 * tile + l32;
            dhi[o] = hi;
            dlo[o] = lo;
        }
    }
}

// ---------------------------------------------------------------------------
// 3. down
// ---------------------------------------------------------------------------
struct DnArgs {
    const uint32_t *dn_q, *sdn_q;
    const uint16_t *dn_s, *dn_b, *sdn_s, *sdn_b;
    int E, H, I, Is, T;
    int rbmax;
    PrefillWs w;
};

// Workgroup = (32-row block, 32 NW columns of H); wave w takes columns
// 32 NW o + 32 w + (0..31). The activation h' arrives as bf16 hi + lo planes,
// so each step runs two MFMAs against the same codes. Scales and biases are
// staged per stage (SbStaged).
__global__ __launch_bounds__(64 * DN_WAVES) __attribute__((amdgpu_waves_per_eu(XWPE, XWPE))) void moe_dn_kernel(DnArgs a) {
    constexpr int NW = DN_WAVES;
    __shared__ __align__(16) uint4 lds[XStage<2, false, NW>::LDS_UINT4];
    __shared__ uint2 sbs_lds[2][2][128];
    const int ntH = (a.H + 32 * NW - 1) / (32 * NW);
    const int item = blockIdx.x;
    const int rbi = item / ntH, o8 = item - rbi * ntH;
    const int R = a.w.rbs[a.E];
    const int4 info = a.w.rbinfo[min(rbi, a.rbmax - 1)];   // speculative, as in gate+up
    const int items = (R + (a.T + 31) / 32) * ntH;
    if (item >= items) return;
    const bool shared = rbi >= R;
    int row0, M, K;
    const uint32_t* Wq;
    const uint16_t *Ws, *Wb, *Ahi, *Alo;
    float* Out;
    if (!shared) {
        const int e = info.x;
        row0 = info.y;
        M = info.z;
        K = a.I;
        Wq = a.dn_q + (int64_t)e * a.H * (a.I / 8);
        Ws = a.dn_s + (int64_t)e * a.H * (a.I / 64);
        Wb = a.dn_b + (int64_t)e * a.H * (a.I / 64);
        Ahi = a.w.hhi;
        Alo = a.w.hlo;
        Out = a.w.O;
    } else {
        row0 = 32 * (rbi - R);
        M = min(32, a.T - row0);
        K = a.Is;
        Wq = a.sdn_q;
        Ws = a.sdn_s;
        Wb = a.sdn_b;
        Ahi = a.w.shhi;
        Alo = a.w.shlo;
        Out = a.w.Os;
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int G = K / 64;
    const int n = 32 * NW * o8 + 32 * wave + l32;
    const int nc = min(n, a.H - 1);
    CodeRing<XD> ring;
    auto issue = [&]() __attribute__((always_inline)) { ring.init_q(Wq + (int64_t)nc * (K / 8) + 4 * h, G); };
    SbStaged sbs;
    sbs.lds = sbs_lds;
    sbs.G = G;
    {
        // thread t stages row t mod 128 of the workgroup (clamped) in array t / 128
        const int srow = min(32 * NW * o8 + (tid & 127), a.H - 1);
        sbs.row = (tid < 128 ? Ws : Wb) + (int64_t)srow * G;
    }
    const int64_t sro = (int64_t)(row0 + min(tid / (NW * 2), M - 1)) * K;
    const uint16_t* const arow[2] = {Ahi + sro, Alo + sro};
    floatx16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    stream_expert_m<2, false, NW>(M, G, lds, arow, ring, sbs, acc, issue, [] {});

    if (n < a.H) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = 8 * (i / 4) + 4 * h + (i % 4);
            if (r < M) Out[(int64_t)(row0 + r) * a.H + n] = acc[i];
        }
    }
}

// ---------------------------------------------------------------------------
// 4. combine
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void moe_combine_kernel(const PrefillWs w, int T, int k, int H,
                                                          float* __restrict__ y) {
    const int t = blockIdx.y;
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T || n >= H) return;
    float v = w.Os[(int64_t)t * H + n];
    for (int j = 0; j < k; ++j) {
        const int ps = w.pos[t * k + j];
        if (ps >= 0) v += w.O[(int64_t)ps * H + n];
    }
    y[(int64_t)t * H + n] = v;
}

hipError_t launch_moe_prefill(const MoeArgs& m, const int32_t* idx, const float* wts, int T, int k,
                              const void* x, int xkind, float* y, void* ws, hipStream_t st) {
    if (T * k > PREP_MAX_PAIRS || m.E > PREP_MAX_E || T > 128) return hipErrorInvalidValue;
    if (m.I % 32 != 0 || m.Is % 32 != 0) return hipErrorInvalidValue;
    const PrefillWs w = carve(ws, m, T, k, nullptr);
    hipLaunchKernelGGL(moe_prep_kernel, dim3(1), dim3(1024), 0, st, idx, T, k, m.E, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    // grids cover the most row blocks the routing can produce; workgroups
    // past the actual count (known on the device) leave at once
    const int rb_max = max_row_blocks(T * k, m.E);
    const int rb_shared = (T + 31) / 32;

    GuArgs ga{};
    ga.gu_q = m.gu_q;
    ga.sgu_q = m.sgu_q;
    ga.gu_s = m.gu_s;
    ga.gu_b = m.gu_b;
    ga.sgu_s = m.sgu_s;
    ga.sgu_b = m.sgu_b;
    ga.x = (const uint16_t*)x;
    ga.p = wts;
    ga.E = m.E;
    ga.H = m.H;
    ga.I = m.I;
    ga.Is = m.Is;
    ga.k = k;
    ga.T = T;
    ga.act = m.act;
    ga.rbmax = rb_max;
    ga.w = w;
    constexpr int GT = GU_WAVES / 2;
    const int gu_items = rb_max * ((m.I / 32 + GT - 1) / GT) + rb_shared * ((m.Is / 32 + GT - 1) / GT);
    // scales and biases through LDS when the rows are short enough (the
    // arrays are 16-byte aligned: the boundary rejects others)
    const int Ggu = m.H / 64;
    const bool sbl = Ggu <= SB_GMAX;
    const size_t sbl_bytes = sbl ? (size_t)GU_WAVES * 128 * sb_row_stride(Ggu) : 0;
    if (xkind == X_F16) {
        if (sbl)
            hipLaunchKernelGGL((moe_gu_kernel<true, true>), dim3(gu_items), dim3(64 * GU_WAVES), sbl_bytes, st, ga);
        else
            hipLaunchKernelGGL((moe_gu_kernel<true, false>), dim3(gu_items), dim3(64 * GU_WAVES), 0, st, ga);
    } else {
        if (sbl)
            hipLaunchKernelGGL((moe_gu_kernel<false, true>), dim3(gu_items), dim3(64 * GU_WAVES), sbl_bytes, st, ga);
        else
            hipLaunchKernelGGL((moe_gu_kernel<false, false>), dim3(gu_items), dim3(64 * GU_WAVES), 0, st, ga);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    DnArgs da{};
    da.dn_q = m.dn_q;
    da.sdn_q = m.sdn_q;
    da.dn_s = m.dn_s;
    da.dn_b = m.dn_b;
    da.sdn_s = m.sdn_s;
    da.sdn_b = m.sdn_b;
    da.E = m.E;
    da.H = m.H;
    da.I = m.I;
    da.Is = m.Is;
    da.T = T;
    da.rbmax = rb_max;
    da.w = w;
    const int ntH = (m.H + 32 * DN_WAVES - 1) / (32 * DN_WAVES);
    hipLaunchKernelGGL(moe_dn_kernel, dim3((rb_max + rb_shared) * ntH), dim3(64 * DN_WAVES), 0, st, da);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    hipLaunchKernelGGL(moe_combine_kernel, dim3((m.H + 255) / 256, T), dim3(256), 0, st, w, T, k,
                       m.H, y);
    return hipGetLastError();
}

}  // namespace qd
