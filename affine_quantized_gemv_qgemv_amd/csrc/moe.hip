// MoE FFN experts of one layer on gfx950: routed + shared experts, GELU gate,
// weighted combine.
//
// [TF] jeff.news/article/5193, section "내부 구조가 진짜 흥미로운 부분"
// (internals): per layer the GPU evaluates the router, uses only the top-8
// experts, runs the resident shared expert and combines the shared and
// routed outputs. Expert weights are 4-bit affine group-64 ("성능과 제약",
// performance and constraints). Reading taken here: the routed outputs are
// weighted by the renormalized router weights, the shared output is added
// with weight one, the gate uses GELU (exact erf or tanh form), and all
// intermediates stay in fp32.
//
// Decode (T == 1) runs two kernels per token:
//   A. gate+up: the (slot, i) row pairs of the selected experts and of the
//      shared expert form one gathered list; a lane segment computes the
//      gate row i and the up row I+i together and writes
//      h = GELU(gate) * up straight from registers. Each selected expert's
//      rows are streamed once.
//   B. down + combine: for output row n, the k routed down rows and the
//      shared down row are one concatenated contraction over
//      k*I + Is inputs, whose activations are staged once in LDS already
//      multiplied by the routing weight of their slot:
//         y[n] = sum_j (p_j h_j) . W_dn[e_j][n] + h_s . W_sdn[n].
//      The combine therefore happens inside the row reduction, with no
//      second pass and no atomics.
// Prefill chunks (T > 1) group (token, slot) pairs by expert and run the
// grouped MFMA kernels of chunk.hip.
//
// The routed decode entry (launch_moe_decode_routed) takes the router
// logits instead of the routing: one wave of every gate+up workgroup that
// has routed rows ranks them from LDS (wave_topk: the same exact top-k and
// weights as the routing kernel, so all workgroups agree), and workgroup 0
// writes the ids and weights for the down pass and the caller. A decode
// layer is then three launches (router, gate+up, down) instead of four.
#include "common.h"
#include "launch.h"
#include "route.h"

#include <mutex>

namespace qd {

__device__ __forceinline__ float gelu_f(float u, int act) {
    if (act == 1) {
        const float c = 0.7978845608028654f;  // sqrt(2 / pi)
        return 0.5f * u * (1.f + tanhf(c * (u + 0.044715f * u * u * u)));
    }
    return 0.5f * u * (1.f + erff(u * 0.7071067811865476f));
}

struct MoeAArgs {
    const uint32_t *gu_q, *sgu_q;
    const uint16_t *gu_s, *gu_b, *sgu_s, *sgu_b;
    const int32_t* idx;   // [k] expert ids of this token (when logits is NULL)
    const float* logits;  // [E] router logits to rank here, or NULL
    int32_t* idx_out;     // [k] ids written by workgroup 0 when ranking here
    float* w_out;         // [k] weights written by workgroup 0 when ranking here
    const void* x;        // [H] activations of this token
    int xkind;
    float* h;             // [k*I + Is]
    int E, H, I, Is, k, act;
};

// ---------------------------------------------------------------------------
// A. gathered gate+up rows with the GELU gate.
// ---------------------------------------------------------------------------
constexpr int MOE_RANK_E = 256;   // experts the in-kernel ranking handles

template <int XF, int LPR, int U, int CPL>
__global__ __launch_bounds__(1024) void moe_gateup_kernel(MoeAArgs a) {
    extern __shared__ uint4 lds[];
    constexpr int RPI = 64 / LPR;  // pairs per wave instruction
    const int C16 = a.H / 32;
    const int G = a.H / 64;
    const int64_t wpr = a.H / 8;
    const int lane = threadIdx.x & 63;
    const int seg = lane / LPR, sl = lane % LPR;
    const int nwaves = blockDim.x >> 6;
    const int gw = blockIdx.x * nwaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int W = gridDim.x * nwaves;
    const int S = (C16 + LPR * CPL - 1) / (LPR * CPL);
    const int npairs = a.k * a.I + a.Is;
    const int ntiles = (npairs + RPI - 1) / RPI;
    const int t0 = (int)((int64_t)ntiles * gw / W);
    const int t1 = (int)((int64_t)ntiles * (gw + 1) / W);

    // The routing: given, or ranked here from the logits. One logit per
    // thread is loaded before the activations are staged, so the two loads
    // overlap, and the ranking then reads only LDS.
    float lv = 0.f;
    if (a.logits && (int)threadIdx.x < a.E) lv = a.logits[threadIdx.x];
    stage_x<4, XF, CPL>(a.x, a.xkind, a.H, 1, 0, C16, lds);
    __shared__ int32_t sidx[32];
    __shared__ float sw[32];
    const int32_t* idx = a.idx;
    // Workgroups whose tiles are all shared-expert rows need no routing;
    // workgroup 0 always ranks, as it writes the ids and weights.
    const int wg_t0 = (int)((int64_t)ntiles * (blockIdx.x * nwaves) / W);
    if (a.logits && (blockIdx.x == 0 || wg_t0 * RPI < a.k * a.I)) {
        __shared__ float lsh[MOE_RANK_E];
        if ((int)threadIdx.x < a.E) lsh[threadIdx.x] = lv;
        __syncthreads();
        if (threadIdx.x < 64) {
            switch ((a.E + 63) >> 6) {   // candidates per lane
                case 1: wave_topk<1>(lsh, a.E, a.k, sidx, sw); break;
                case 2: wave_topk<2>(lsh, a.E, a.k, sidx, sw); break;
                case 3: wave_topk<3>(lsh, a.E, a.k, sidx, sw); break;
                default: wave_topk<4>(lsh, a.E, a.k, sidx, sw); break;
            }
        }
        __syncthreads();
        if (blockIdx.x == 0 && threadIdx.x < a.k) {
            a.idx_out[threadIdx.x] = sidx[threadIdx.x];
            a.w_out[threadIdx.x] = sw[threadIdx.x];
        }
        idx = sidx;
    }
    __syncthreads();
    const uint32_t magic = in_vgpr(kMagic16);

    for (int tile = t0; tile < t1; ++tile) {
        const int p = tile * RPI + seg;
        const bool pv = p < npairs;
        const int pc = pv ? p : npairs - 1;
        // rows of this pair: gate row g0 and up row g1 of matrix (q, s, b)
        const uint32_t* q;
        const uint16_t *sp, *bp;
        int g0, g1;
        bool ok = pv;
        if (pc < a.k * a.I) {
            const int j = pc / a.I, i = pc - j * a.I;
            int e = idx[j];
            if (e < 0 || e >= a.E) {
                ok = false;
                e = 0;
            }
            const int64_t rows_e = 2 * (int64_t)a.I;
            q = a.gu_q + (int64_t)e * rows_e * wpr;
            sp = a.gu_s + (int64_t)e * rows_e * G;
            bp = a.gu_b + (int64_t)e * rows_e * G;
            g0 = i;
            g1 = a.I + i;
        } else {
            const int i = pc - a.k * a.I;
            q = a.sgu_q;
            sp = a.sgu_s;
            bp = a.sgu_b;
            g0 = i;
            g1 = a.Is + i;
        }
        float y[2][1] = {{0.f}, {0.f}};
        for (int s0 = 0; s0 < S; s0 += U) {
            uint4 cw[U][CPL][2];
            uint16_t sr[U][2], br[U][2];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (s0 + u >= S) break;  // uniform
                const int c = min(((s0 + u) * LPR + sl) * CPL, C16 - CPL);
#pragma unroll
                for (int ch = 0; ch < CPL; ++ch) {
                    cw[u][ch][0] = *(const uint4*)(q + (int64_t)g0 * wpr + (int64_t)(c + ch) * 4);
                    cw[u][ch][1] = *(const uint4*)(q + (int64_t)g1 * wpr + (int64_t)(c + ch) * 4);
                }
                sr[u][0] = sp[(int64_t)g0 * G + c / 2];
                br[u][0] = bp[(int64_t)g0 * G + c / 2];
                sr[u][1] = sp[(int64_t)g1 * G + c / 2];
                br[u][1] = bp[(int64_t)g1 * G + c / 2];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (s0 + u >= S) break;
                const int cu = ((s0 + u) * LPR + sl) * CPL;
                const bool live = ok && cu < C16;
                const int c = min(cu, C16 - CPL);
                float sc[2], bi[2];   // scale and centred bias b + 8 s
                const uint32_t n1[2] = {kNeg1032, kNeg1032}, n16[2] = {kNeg1152, kNeg1152};
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    sc[r] = live ? h2f(sr[u][r]) : 0.f;
                    bi[r] = live ? fmaf(8.f, sc[r], h2f(br[u][r])) : 0.f;
                }
                int slot[CPL];
#pragma unroll
                for (int ch = 0; ch < CPL; ++ch) slot[ch] = xslot<CPL>(c + ch, C16);
                group_rows<4, XF, 1, 2, CPL>(cw[u], sc, bi, n1, n16, lds, 1, C16, slot, magic, y);
            }
        }
        const float zg = seg_sum<LPR>(y[0][0]);
        const float zu = seg_sum<LPR>(y[1][0]);
        if (sl == 0 && pv) a.h[p] = ok ? gelu_f(zg, a.act) * zu : 0.f;
    }
}

// ---------------------------------------------------------------------------
// B. down rows of the k selected experts and the shared expert, combined.
// ---------------------------------------------------------------------------
struct MoeBArgs {
    const uint32_t *dn_q, *sdn_q;
    const uint16_t *dn_s, *dn_b, *sdn_s, *sdn_b;
    const int32_t* idx;   // [k]
    const float* p;       // [k]
    const float* h;       // [k*I + Is]
    float* y;             // [H]
    int E, H, I, Is, k;
};

// Chunk c (16 bytes = 32 codes) of the concatenated down row: the routed
// segment j = c / (I/32) of expert idx[j], or the shared expert's row.
// Addresses are those of row 0; row n adds n * qs words and n * gs groups.
struct DnChunk {
    const uint32_t* q;
    const uint16_t *s, *b;
    int qs, gs;
    bool ok;   // false: an expert id outside [0, E) (contributes nothing)
};

// idv: lane j < k holds the expert id of slot j (read with a lane shuffle,
// so every lane of the wave must call this).
__device__ __forceinline__ DnChunk dn_chunk(const MoeBArgs& a, int c, int idv) {
    const int cpe = a.I / 32;
    DnChunk d;
    const int jr = min(c / cpe, a.k - 1);
    const int er = __shfl(idv, jr);
    if (c < a.k * cpe) {
        const int j = c / cpe, cl = c - j * cpe;
        int e = er;
        d.ok = e >= 0 && e < a.E;
        if (!d.ok) e = 0;
        const int64_t mq = (int64_t)e * a.H * (a.I / 8);
        const int64_t mg = (int64_t)e * a.H * (a.I / 64);
        d.q = a.dn_q + mq + (int64_t)cl * 4;
        d.s = a.dn_s + mg + cl / 2;
        d.b = a.dn_b + mg + cl / 2;
        d.qs = a.I / 8;
        d.gs = a.I / 64;
    } else {
        const int cl = c - a.k * cpe;
        d.q = a.sdn_q + (int64_t)cl * 4;
        d.s = a.sdn_s + cl / 2;
        d.b = a.sdn_b + cl / 2;
        d.qs = a.Is / 8;
        d.gs = a.Is / 64;
        d.ok = true;
    }
    return d;
}

// A wave's lanes take LPR-lane segments of one row each (R rows per
// segment); a lane reads CPL consecutive chunks per step. The first step
// batch of the wave's first tile is requested before the activations are
// staged, so the weight fetch overlaps the staging.
constexpr int DN_MAX_WAVES = 12;   // 168 VGPRs: the early-requested chunks live across the staging

template <int LPR, int R, int U, int CPL>
__global__ __launch_bounds__(64 * DN_MAX_WAVES) void moe_down_kernel(MoeBArgs a) {
    extern __shared__ uint4 lds[];
    constexpr int RPI = 64 / LPR;
    constexpr int ROWS = RPI * R;
    const int cpe = a.I / 32;                  // chunks per routed segment
    const int C = a.k * cpe + a.Is / 32;       // chunks of the concatenated row
    using St = Stage<4, 1>;

    const int lane = threadIdx.x & 63;
    const int seg = lane / LPR, sl = lane % LPR;
    const int nwaves = blockDim.x >> 6;
    const int gw = blockIdx.x * nwaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int W = gridDim.x * nwaves;
    const int S = (C + LPR * CPL - 1) / (LPR * CPL);
    const int ntiles = (a.H + ROWS - 1) / ROWS;
    const int t0 = (int)((int64_t)ntiles * gw / W);
    const int t1 = (int)((int64_t)ntiles * (gw + 1) / W);

    // Load order (vector-memory counters complete in order): the routing,
    // this thread's first activation chunk, then the first code batch, so
    // waiting for the first two never waits for code fetches. The loads are
    // unconditional (clamped addresses): a branch around one would make the
    // compiler's counter bookkeeping wait for everything at the join.
    const int ls = min(lane, a.k - 1);   // k <= 32
    const int idv = a.idx[ls];
    const float pv = a.p[ls];
    const int cst = threadIdx.x;   // first staged chunk of this thread
    float4 hv[8];
    {
        const float* hp = a.h + (int64_t)min(cst, C - 1) * 32;
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[i] = *(const float4*)(hp + 4 * i);
    }
    // routing weight of that chunk (all lanes active for the shuffles)
    float scale0;
    {
        const int jr = min(cst / cpe, a.k - 1);
        const int er = __shfl(idv, jr);
        const float pr = __shfl(pv, jr);
        scale0 = cst < a.k * cpe ? ((er >= 0 && er < a.E) ? pr : 0.f) : 1.f;
    }
    __builtin_amdgcn_sched_barrier(0);

    uint4 cw[U][CPL][R];
    uint16_t sr[U][R], br[U][R];
    bool live[U];
    // all U steps are requested (clamped): a data-dependent exit would make
    // the counters at the join conservative
    auto load = [&](int tile, int s0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int cu = ((s0 + u) * LPR + sl) * CPL;
            const int c = min(cu, C - CPL);
            const DnChunk d = dn_chunk(a, c, idv);
            live[u] = cu < C && d.ok;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int n = min(tile * ROWS + r * RPI + seg, a.H - 1);
#pragma unroll
                for (int ch = 0; ch < CPL; ++ch)
                    cw[u][ch][r] = *(const uint4*)(d.q + (int64_t)n * d.qs + 4 * ch);
                sr[u][r] = d.s[(int64_t)n * d.gs];
                br[u][r] = d.b[(int64_t)n * d.gs];
            }
        }
    };
    load(min(t0, ntiles - 1), 0);   // unconditional (see above)
    __builtin_amdgcn_sched_barrier(0);

    // stage h' = (p_j h_j | h_s) (fp32 layout for 4-bit codes); the first
    // chunk straight-line (a loop around it would join its counters with
    // those of later iterations), further ones (more chunks than threads)
    // in a loop
    auto stage_chunk = [&](int c, float scale) __attribute__((always_inline)) {
        float v[32];
#pragma unroll
        for (int i = 0; i < 32; i += 4) {
            const float4 t = hv[i / 4];
            v[i] = t.x * scale;
            v[i + 1] = t.y * scale;
            v[i + 2] = t.z * scale;
            v[i + 3] = t.w * scale;
        }
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) sum += v[i];
        constexpr int QPC = St::QPC;
        const int sl2 = xslot<CPL>(c, C);
#pragma unroll
        for (int w = 0; w < 4; ++w) {   // the pair order of the 4-bit unpack
            const float* u = v + 8 * w;
            lds[(2 * w) * C + sl2] = make_uint4(__float_as_uint(u[0]), __float_as_uint(u[4]),
                                                __float_as_uint(u[2]), __float_as_uint(u[6]));
            lds[(2 * w + 1) * C + sl2] = make_uint4(__float_as_uint(u[1]), __float_as_uint(u[5]),
                                                    __float_as_uint(u[3]), __float_as_uint(u[7]));
        }
        ((float*)(lds + (size_t)QPC * C))[sl2] = sum;
    };
    if (cst < C) stage_chunk(cst, scale0);
    for (int c = cst + (int)blockDim.x; c < C; c += blockDim.x) {
        float scale = 1.f;
        if (c < a.k * cpe) {
            const int j = c / cpe;
            const int e = a.idx[j];
            scale = (e >= 0 && e < a.E) ? a.p[j] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[i] = *(const float4*)(a.h + (int64_t)c * 32 + 4 * i);
        stage_chunk(c, scale);
    }
    __syncthreads();

    const uint32_t magic = in_vgpr(kMagic16);
    for (int tile = t0; tile < t1; ++tile) {
        float y[R][1];
#pragma unroll
        for (int r = 0; r < R; ++r) y[r][0] = 0.f;
        for (int s0 = 0; s0 < S; s0 += U) {
            if (tile != t0 || s0 != 0) load(tile, s0);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (s0 + u >= S) break;
                const int cu = ((s0 + u) * LPR + sl) * CPL;
                const int c = min(cu, C - CPL);
                float sc[R], bi[R];   // scale and centred bias b + 8 s
                uint32_t n1[R], n16[R];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const bool ok = live[u] && (tile * ROWS + r * RPI + seg < a.H);
                    sc[r] = ok ? h2f(sr[u][r]) : 0.f;
                    bi[r] = ok ? fmaf(8.f, sc[r], h2f(br[u][r])) : 0.f;
                    n1[r] = kNeg1032;
                    n16[r] = kNeg1152;
                }
                int slot[CPL];
#pragma unroll
                for (int ch = 0; ch < CPL; ++ch) slot[ch] = xslot<CPL>(c + ch, C);
                group_rows<4, 1, 1, R, CPL>(cw[u], sc, bi, n1, n16, lds, 1, C, slot, magic, y);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int n = tile * ROWS + r * RPI + seg;
            const float v = seg_sum<LPR>(y[r][0]);
            if (sl == 0 && n < a.H) a.y[n] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
size_t moe_decode_workspace_bytes(const MoeArgs& m, int k) {
    return ((size_t)k * m.I + m.Is) * sizeof(float);
}

namespace {

// Launch shapes of the two decode kernels (workgroup waves, rows per tile).
struct MoeCfg {
    int gu_nw, dn_nw, dn_r;
};

MoeCfg moe_cfg() {
    MoeCfg c{4, 0, 1};   // dn_nw 0: sized to the row count
    return c;
}

template <typename Kern>
int grid_for(Kern kern, int threads, size_t lds, int ntiles_waves) {
    const DeviceInfo& dev = device_info();
    const int occ = occupancy((const void*)kern, threads, lds);
    const int want = (ntiles_waves + threads / 64 - 1) / (threads / 64);
    return std::max(1, std::min(want, std::max(1, occ) * dev.cus));
}

template <int XF>
hipError_t launch_gateup(const MoeAArgs& a, hipStream_t st) {
    constexpr int LPR = 32, U = 3, CPL = 1;
    const size_t lds = Stage<4, XF>::bytes(1, a.H / 32);
    if (lds > device_info().max_lds_per_block) return hipErrorInvalidValue;
    const int npairs = a.k * a.I + a.Is;
    const int ntiles = (npairs + (64 / LPR) - 1) / (64 / LPR);
    auto kern = moe_gateup_kernel<XF, LPR, U, CPL>;
    const int threads = 64 * moe_cfg().gu_nw;
    const int grid = grid_for(kern, threads, lds, ntiles);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, st, a);
    return hipGetLastError();
}

template <int R>
hipError_t launch_down_r(const MoeBArgs& a, int nw, hipStream_t st) {
    constexpr int LPR = 64, U = 2, CPL = 2;
    const int C = a.k * (a.I / 32) + a.Is / 32;
    const size_t lds = Stage<4, 1>::bytes(1, C);
    if (lds > device_info().max_lds_per_block) return hipErrorInvalidValue;
    const int ntiles = (a.H + (64 / LPR) * R - 1) / ((64 / LPR) * R);
    auto kern = moe_down_kernel<LPR, R, U, CPL>;
    // Every workgroup stages all k*I + Is activations: at most one per CU,
    // each with just enough waves (up to 12) that the rows spread over all
    // CUs (2816 rows: 256 workgroups of 11 waves rather than 235 of 12).
    const int cus = device_info().cus;
    if (nw <= 0) nw = std::min(DN_MAX_WAVES, std::max(1, (ntiles + cus - 1) / cus));
    const int threads = 64 * nw;
    const int grid = std::min(grid_for(kern, threads, lds, ntiles), device_info().cus);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, st, a);
    return hipGetLastError();
}

hipError_t launch_down(const MoeBArgs& a, hipStream_t st) {
    const MoeCfg c = moe_cfg();
    return launch_down_r<1>(a, c.dn_nw, st);
}

}  // namespace

hipError_t launch_moe_decode(const MoeArgs& m, const int32_t* idx, const float* w, int T, int k,
                             const void* x, int xkind, float* y, void* ws, hipStream_t st) {
    float* h = (float*)ws;
    const size_t esz = xkind == X_F32 ? 4 : 2;
    for (int t = 0; t < T; ++t) {
        MoeAArgs a{};
        a.gu_q = m.gu_q;
        a.sgu_q = m.sgu_q;
        a.gu_s = m.gu_s;
        a.gu_b = m.gu_b;
        a.sgu_s = m.sgu_s;
        a.sgu_b = m.sgu_b;
        a.idx = idx + (int64_t)t * k;
        a.x = (const char*)x + (size_t)t * m.H * esz;
        a.xkind = xkind;
        a.h = h;
        a.E = m.E;
        a.H = m.H;
        a.I = m.I;
        a.Is = m.Is;
        a.k = k;
        a.act = m.act;
        hipError_t e = xkind == X_F16 ? launch_gateup<0>(a, st) : launch_gateup<1>(a, st);
        if (e != hipSuccess) return e;
        MoeBArgs b{};
        b.dn_q = m.dn_q;
        b.sdn_q = m.sdn_q;
        b.dn_s = m.dn_s;
        b.dn_b = m.dn_b;
        b.sdn_s = m.sdn_s;
        b.sdn_b = m.sdn_b;
        b.idx = idx + (int64_t)t * k;
        b.p = w + (int64_t)t * k;
        b.h = h;
        b.y = y + (int64_t)t * m.H;
        b.E = m.E;
        b.H = m.H;
        b.I = m.I;
        b.Is = m.Is;
        b.k = k;
        e = launch_down(b, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_moe_decode_routed(const MoeArgs& m, const float* logits, int k, const void* x,
                                    int xkind, int32_t* idx, float* w, float* y, void* ws,
                                    hipStream_t st) {
    // one logit per thread of a gate+up workgroup
    if (m.E > MOE_RANK_E || m.E > 64 * moe_cfg().gu_nw || k > 32) return hipErrorInvalidValue;
    float* h = (float*)ws;
    MoeAArgs a{};
    a.gu_q = m.gu_q;
    a.sgu_q = m.sgu_q;
    a.gu_s = m.gu_s;
    a.gu_b = m.gu_b;
    a.sgu_s = m.sgu_s;
    a.sgu_b = m.sgu_b;
    a.logits = logits;
    a.idx_out = idx;
    a.w_out = w;
    a.x = x;
    a.xkind = xkind;
    a.h = h;
    a.E = m.E;
    a.H = m.H;
    a.I = m.I;
    a.Is = m.Is;
    a.k = k;
    a.act = m.act;
    hipError_t e = xkind == X_F16 ? launch_gateup<0>(a, st) : launch_gateup<1>(a, st);
    if (e != hipSuccess) return e;
    MoeBArgs b{};
    b.dn_q = m.dn_q;
    b.sdn_q = m.sdn_q;
    b.dn_s = m.dn_s;
    b.dn_b = m.dn_b;
    b.sdn_s = m.sdn_s;
    b.sdn_b = m.sdn_b;
    b.idx = idx;
    b.p = w;
    b.h = h;
    b.y = y;
    b.E = m.E;
    b.H = m.H;
    b.I = m.I;
    b.Is = m.Is;
    b.k = k;
    return launch_down(b, st);
}

// ---------------------------------------------------------------------------
// Allocation-free decode layer: the gate+up activations h live in a scratch
// array of this library, one per device, held until the process ends. Only
// the host touches it, through its device address (looked up once per device;
// the array's name in host code is not that address), which is passed to the
// kernels as their workspace. Every call on a device shares the array, so
// calls that overlap on one device race; h is fully written by gate+up before
// down reads it, so nothing needs clearing between calls.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kMoeNoAllocBytes];

static hipError_t scratch_address(void** out) {
    static void* addr[64];
    static hipError_t err[64];
    static std::once_flag once[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    // with this device current (hipGetDevice above): its copy of the array
    std::call_once(once[dev], [dev] {
        err[dev] = hipGetSymbolAddress(&addr[dev], HIP_SYMBOL(scratch));
    });
    if (err[dev] != hipSuccess) return err[dev];
    *out = addr[dev];
    return hipSuccess;
}

hipError_t launch_moe_decode_routed_noalloc(const MoeArgs& m, const float* logits, int k,
                                            const void* x, int xkind, int32_t* idx, float* w,
                                            float* y, hipStream_t st) {
    if (moe_decode_workspace_bytes(m, k) > kMoeNoAllocBytes) return hipErrorInvalidValue;
    void* ws = nullptr;
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return e;
    return launch_moe_decode_routed(m, logits, k, x, xkind, idx, w, y, ws, st);
}

size_t moe_workspace_bytes(const MoeArgs& m, int T, int k) {
    return std::max(moe_decode_workspace_bytes(m, k), moe_prefill_workspace_bytes(m, T, k));
}

hipError_t launch_moe_experts(const MoeArgs& m, const int32_t* idx, const float* w, int T, int k,
                              const void* x, int xkind, float* y, void* ws, size_t ws_bytes,
                              hipStream_t st) {
    (void)ws_bytes;
    if (T == 1) return launch_moe_decode(m, idx, w, T, k, x, xkind, y, ws, st);
    return launch_moe_prefill(m, idx, w, T, k, x, xkind, y, ws, st);
}

}  // namespace qd
