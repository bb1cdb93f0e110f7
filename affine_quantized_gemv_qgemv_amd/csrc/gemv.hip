// Batch-1..8 affine-quantized GEMV for gfx950: y[b][n] = sum_k w[n][k] x[b][k].
//
// [TF] jeff.news/article/5193, section "성능과 제약" (performance and
// constraints): MLX affine 4-bit weights, group 64, router at 8 bits; section
// "기술 맥락" (technical context): the runtime hand-schedules its quantized
// GEMV. This is that contraction, designed for CDNA4 rather than Metal:
//
//  * Work split. Each 64-lane wave owns a tile of rows. A row is covered by
//    a segment of LPR lanes (LPR in {8, 16, 32, 64}); lane j of a segment
//    reads 16-byte code chunks j, j+LPR, j+2*LPR, ... of its row, so one
//    wave instruction fetches 64/LPR row pieces of LPR*16 contiguous bytes
//    (128 B to 1 KB). Each lane keeps its partial sums in registers; a
//    shuffle reduction over the segment finishes a row.
//  * Activations are staged once per workgroup into LDS in the order the
//    code unpacking produces, with per-chunk sums for the affine epilogue.
//    Workgroups are persistent (one wave of work per resident wave slot)
//    so the staging is paid once per workgroup, not once per tile.
//  * Loads of U steps for R rows are issued back to back before any of them
//    is used, so every wave keeps U*R 16-byte loads per lane in flight.
//  * When the staged activations would not fit LDS, the chunk range is split
//    across a second grid dimension and the partial rows are added into a
//    zeroed y with fp32 atomics.
//
// Weight formats (template parameter FMT); all reduce to the per-group
// epilogue y += s * sum(u x) + c * sum(x) with unsigned codes u:
//  * W_AFFINE: MLX affine (above), fp16 s and c = fp16 b.
//  * W_MIRAI_M and W_MIRAI_L, from discuss.pytorch.kr/t/uzu-mac-iphone-llm-
//    apple-silicon-rust/12363 (uzu), section "uzu의 모델 변환과 Mirai 양자화
//    형식" (model conversion and the Mirai quantization formats): Mirai-M has
//    4-bit codes with a 4-bit zero point z and a bf16 scale per group of 64,
//    w = s (q - z), so c = -s z (exact in fp32: 8 x 4 significant bits);
//    the zero points are packed eight per uint32 along a row's groups.
//    Mirai-L has signed 8-bit codes and a bf16 scale per group, w = s q;
//    flipping each code's top bit gives u = q + 128, so c = -128 s.
//
// Activation modes (template parameter XF): 0 = fp16 (dot2 on packed
// halves), 1 = bf16 staged as fp32 (fma), 2 = the rotation prologue of the
// same page and section (RMSNorm, then a block-32 random Hadamard transform,
// computed while staging and kept as hi/lo fp16 planes; see stage_x_rot).
#include "common.h"
#include "launch.h"

namespace qd {

struct GemvArgs {
    const uint32_t* wq;
    const uint16_t* s;
    const uint16_t* b;
    const void* x;
    float* y;
    int xkind;
    int N, K;
    int nb;              // activation vectors in this launch (<= B)
    int chunks_split;    // chunks per K split (grid dimension y)
    int atomic_out;
    int interleave;      // tile order: 1 = wave w takes tiles w, w + W, ...; 0 = a contiguous block
    const uint8_t* zp;   // Mirai-M zero points, zstride bytes per row
    int zstride;
    const uint32_t* signs;   // XF == 2: rotation signs [K/32] (NULL = none)
    const uint16_t* gamma;   // XF == 2: RMSNorm weight [K] in x's kind (NULL = no norm)
    float eps;
};

// LDS of the rotation prologue (factors per vector and per-wave partial
// sums). Only kernels that call this allocate it.
__device__ __forceinline__ float* rot_shared() {
    __shared__ float buf[kRotShared];
    return buf;
}

enum WFmt : int { W_AFFINE = 0, W_MIRAI_M = 1, W_MIRAI_L = 2 };

// One round of loads: U steps of R rows; a step gives each lane CPL
// consecutive 16-byte chunks of one group.
template <int R, int U, int CPL>
struct Round {
    uint4 cw[U][CPL][R];
    uint16_t sc[U][R], bi[U][R];   // raw scale / bias (or zero-point byte) bits; masked when consumed
};

// Staging for the kernel's activation layout: chunk-major for several fp16
// vectors, the plain layout otherwise.
template <int BITS, int XF, int B, int CPL>
__device__ __forceinline__ void stage_x_any(const void* x, int kind, int64_t xstride, int nb, int c0,
                                            int nc, uint4* lds) {
    if constexpr (XF == 0 && B > 1)
        stage_x_cm<BITS, B, CPL>(x, xstride, nb, c0, nc, lds);
    else
        stage_x<BITS, XF, CPL>(x, kind, xstride, nb, c0, nc, lds);
}

template <int BITS, int XF, int B, int LPR, int R, int U, int WPE, int CPL, int FMT>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(WPE))) void qgemv_kernel(
    GemvArgs a) {
    extern __shared__ uint4 lds[];
    constexpr int CC = 128 / BITS;     // codes per 16-byte chunk
    constexpr int CPG = 64 / CC;       // chunks per group of 64
    constexpr int RPI = 64 / LPR;      // rows per wave instruction
    constexpr int ROWS = RPI * R;      // rows per tile
    constexpr bool CM = XF == 0 && B > 1;   // chunk-major staging (stage_x_cm)
    const int C16 = a.K / CC;
    const int c0 = blockIdx.y * a.chunks_split;
    const int nc = min(a.chunks_split, C16 - c0);
    const int G = a.K / 64;
    const int64_t wpr = (int64_t)a.K * BITS / 32;  // words per row

    const int lane = threadIdx.x & 63;
    const int seg = lane / LPR, sl = lane % LPR;
    const int nwaves = blockDim.x >> 6;
    // wave-uniform: keeps the tile bounds and loop control in scalar registers
    const int gw = blockIdx.x * nwaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int W = gridDim.x * nwaves;
    const int S = (nc + LPR * CPL - 1) / (LPR * CPL);  // steps per row
    const int RPT = (S + U - 1) / U;               // rounds per tile
    const int ntiles = (a.N + ROWS - 1) / ROWS;
    // This wave's tiles: interleaved (all waves together sweep one window of
    // the matrix, as a streaming read does) or a contiguous, balanced block.
    int t0, tstep, ntl;
    if (a.interleave) {
        t0 = gw;
        tstep = W;
        ntl = gw < ntiles ? (ntiles - gw + W - 1) / W : 0;
    } else {
        t0 = (int)((int64_t)ntiles * gw / W);
        tstep = 1;
        ntl = (int)((int64_t)ntiles * (gw + 1) / W) - t0;
    }
    const int nrounds = ntl * RPT;

    // Rotation prologue: LDS for the per-vector factors (only kernels with
    // XF == 2 reference it); rot[kRotMaxB + b] is 2^-e of vector b.
    float* rot = nullptr;
    if constexpr (XF == 2) rot = rot_shared();

    // Loads are unconditional inside a wave-uniform step test: rows past N and
    // chunks past the staged range read a clamped, valid address and get a
    // zero scale and bias, so they add nothing. (Branches around individual
    // loads would make the compiler wait for every load in flight.) Each
    // round's loads go through buffer resources based at the tile's first
    // row, so per-lane offsets are 32-bit and the chunk and step offsets are
    // instruction immediates.
    const uint32_t rowb = (uint32_t)(wpr * 4);   // bytes of codes per row (< 2^24)
    auto issue = [&](Round<R, U, CPL>& buf, int tile, int sg) {
        const int64_t r0 = (int64_t)tile * ROWS;
        const int rlast = a.N - 1 - (int)r0;     // last row of the matrix, tile-relative
        const auto wr = buf_rsrc(a.wq + r0 * wpr, (a.N - r0) * (int64_t)rowb);
        const auto sr = buf_rsrc(a.s + r0 * G, (a.N - r0) * (int64_t)G * 2);
        __amdgpu_buffer_rsrc_t br;
        if constexpr (FMT == W_AFFINE)
            br = buf_rsrc(a.b + r0 * G, (a.N - r0) * (int64_t)G * 2);
        else if constexpr (FMT == W_MIRAI_M)
            br = buf_rsrc(a.zp + r0 * a.zstride, (a.N - r0) * (int64_t)a.zstride);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (sg * U + u >= S) break;  // uniform
            const int c = ((sg * U + u) * LPR + sl) * CPL;
            const int gc = c0 + min(c, nc - CPL);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int lr = min(r * RPI + seg, rlast);
                const uint32_t wo = (uint32_t)__umul24(lr, (int)rowb) + (uint32_t)gc * 16u;
#pragma unroll
                for (int ch = 0; ch < CPL; ++ch) buf.cw[u][ch][r] = buf_load16(wr, wo + 16u * ch);
                const uint32_t go = (uint32_t)__umul24(lr, G) + (uint32_t)(gc / CPG);
                buf.sc[u][r] = buf_load2(sr, 2u * go);
                if constexpr (FMT == W_AFFINE)
                    buf.bi[u][r] = buf_load2(br, 2u * go);
                else if constexpr (FMT == W_MIRAI_M)   // byte holding groups 2j, 2j + 1
                    buf.bi[u][r] = buf_load1(br, (uint32_t)__umul24(lr, a.zstride) +
                                                     (uint32_t)((gc / CPG) / 2));
            }
        }
    };

    float y[R][B];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int bb = 0; bb < B; ++bb) y[r][bb] = 0.f;

    const uint32_t magic = in_vgpr(kMagic16);
    auto consume = [&](const Round<R, U, CPL>& buf, int tile, int sg) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (sg * U + u >= S) break;  // uniform
            const int cu = ((sg * U + u) * LPR + sl) * CPL;
            const int c = min(cu, nc - CPL);
            float sc[R], bi[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const bool ok = (cu < nc) && (tile * ROWS + r * RPI + seg < a.N);
                if constexpr (FMT == W_AFFINE) {
                    sc[r] = ok ? h2f(buf.sc[u][r]) : 0.f;
                    bi[r] = ok ? h2f(buf.bi[u][r]) : 0.f;
                } else if constexpr (FMT == W_MIRAI_M) {
                    const int zsh = (((c0 + c) / CPG) & 1) * 4;
                    const float z = (float)((buf.bi[u][r] >> zsh) & 15u);
                    sc[r] = ok ? bf2f(buf.sc[u][r]) : 0.f;
                    bi[r] = -sc[r] * z;
                } else {
                    sc[r] = ok ? bf2f(buf.sc[u][r]) : 0.f;
                    bi[r] = -128.f * sc[r];
                }
            }
            int slot[CPL];
#pragma unroll
            for (int ch = 0; ch < CPL; ++ch) slot[ch] = xslot<CPL>(c + ch, nc);
            if constexpr (FMT == W_MIRAI_L) {
                uint4 cw[CPL][R];   // signed bytes -> offset-128 unsigned codes
#pragma unroll
                for (int ch = 0; ch < CPL; ++ch)
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const uint4 v = buf.cw[u][ch][r];
                        cw[ch][r] = make_uint4(v.x ^ 0x80808080u, v.y ^ 0x80808080u,
                                               v.z ^ 0x80808080u, v.w ^ 0x80808080u);
                    }
                group_rows<BITS, XF, B, R, CPL, CM>(cw, sc, bi, lds, a.nb, nc, slot, magic, y);
            } else {
                group_rows<BITS, XF, B, R, CPL, CM>(buf.cw[u], sc, bi, lds, a.nb, nc, slot, magic, y);
            }
        }
        if (sg == RPT - 1) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int row = tile * ROWS + r * RPI + seg;
#pragma unroll
                for (int bb = 0; bb < B; ++bb) {
                    float v = seg_sum<LPR>(y[r][bb]);
                    if constexpr (XF == 2) v *= rot[kRotMaxB + bb];
                    y[r][bb] = 0.f;
                    if (sl == 0 && row < a.N && bb < a.nb) {
                        float* dst = a.y + (int64_t)bb * a.N + row;
                        if (a.atomic_out)
                            atomicAdd(dst, v);
                        else
                            *dst = v;
                    }
                }
            }
        }
    };

    // One buffer per wave: a round's loads are all issued before any is used;
    // other waves on the SIMD keep the memory system busy while this one
    // computes.
    Round<R, U, CPL> A;
    if constexpr (XF == 2) {
        // the first weight loads go out behind the activation loads, so the
        // transform runs while they are in flight
        stage_x_rot<BITS, CPL>((const uint16_t*)a.x, a.xkind, a.K, a.nb, c0, nc, a.gamma, a.signs,
                               a.eps, rot, lds, [&]() { if (nrounds > 0) issue(A, t0, 0); });
    } else {
        if (nrounds > 0) issue(A, t0, 0);  // in flight while the activations are staged
        stage_x_any<BITS, XF, B, CPL>(a.x, a.xkind, a.K, a.nb, c0, nc, lds);
    }
    __syncthreads();
    for (int rd = 0; rd < nrounds; ++rd) {
        const int tile = t0 + (rd / RPT) * tstep;
        const int sg = rd - (rd / RPT) * RPT;
        if (rd > 0) issue(A, tile, sg);
        consume(A, tile, sg);
    }
}

__global__ void fill_zero_kernel(float* p, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.f;
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int threads = 256;
    const int64_t blocks = std::min<int64_t>((n + threads - 1) / threads, 4096);
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(threads), 0, st, p, n);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Host-side configuration.
// ---------------------------------------------------------------------------
namespace {

template <int BITS, int XF, int B, int LPR, int R, int U, int WPE, int CPL, int FMT>
hipError_t run_cfg(const GemvArgs& base, int nwaves, hipStream_t st) {
    using St = Stage<BITS, XF>;
    const DeviceInfo& dev = device_info();
    auto kern = qgemv_kernel<BITS, XF, B, LPR, R, U, WPE, CPL, FMT>;
    const int C16 = base.K / St::CC;
    // Split the chunk range when the staged activations exceed the LDS budget
    // per workgroup (half the CU's LDS, so two workgroups stay resident).
    const size_t budget = std::min<size_t>(dev.max_lds_per_block, dev.lds_per_cu / 2);
    int splits = 1;
    // chunks per split: a multiple of 4 so a lane's CPL chunks never straddle
    // a split
    auto per_of = [&](int sp) { return (((C16 + sp - 1) / sp) + 3) & ~3; };
    // the kernel's staging layout (chunk-major for several fp16 vectors)
    auto bytes = [&](int nc) {
        return (XF == 0 && B > 1) ? St::bytes_cm(B, nc) : St::bytes(base.nb, nc);
    };
    while (bytes(per_of(splits)) > budget && splits < C16) ++splits;
    const int per = std::min(per_of(splits), C16);
    splits = (C16 + per - 1) / per;
    const size_t lds = bytes(per);
    if (lds > dev.max_lds_per_block) return hipErrorInvalidValue;

    GemvArgs a = base;
    a.chunks_split = per;
    a.atomic_out = splits > 1;
    if (a.atomic_out) {
        hipError_t e = launch_fill_zero(a.y, (int64_t)a.nb * a.N, st);
        if (e != hipSuccess) return e;
    }
    const int threads = nwaves * 64;
    const int rows_per_tile = (64 / LPR) * R;
    const int ntiles = (a.N + rows_per_tile - 1) / rows_per_tile;
    const int want = (ntiles + nwaves - 1) / nwaves;
    const int occ = occupancy((const void*)kern, threads, lds);
    const int grid = std::max(1, std::min(want, std::max(1, occ) * dev.cus));
    hipLaunchKernelGGL(kern, dim3(grid, splits), dim3(threads), lds, st, a);
    return hipGetLastError();
}

struct Cfg {
    int lpr, r, u, wpe, cpl, nw;
    int il = 0;   // interleaved tile order
};

// Lanes per row: the largest segment width that wastes the fewest lane
// slots on the row's chunk count.
int pick_lpr(int chunks) {
    const int opts[4] = {64, 32, 16, 8};
    int best = 64;
    double best_eff = -1.0;
    for (int o : opts) {
        const int steps = (chunks + o - 1) / o;
        const double eff = (double)chunks / (steps * o);
        if (eff > best_eff + 1e-9) {
            best_eff = eff;
            best = o;
        }
    }
    return best;
}

// Launch policy, from on-device sweeps (graph-replayed, weights cycled through
// HBM). Batch 1 wants every resident wave busy with one or two rounds of
// loads; a lane takes a whole group (two 16-byte chunks, CPL = 2) when the row
// splits evenly, which halves the scale/bias loads and epilogues; larger
// workgroups stage x fewer times but must still cover every CU.
int pow2_floor(int v) {
    int p = 1;
    while (p * 2 <= v) p *= 2;
    return p;
}

Cfg default_cfg(int bits, int xf, int nb, int N, int K) {
    Cfg c;
    c.il = 1;   // waves sweep the matrix together (measured faster on every shape)
    const int chunks = K * bits / 128;
    c.lpr = pick_lpr(chunks);
    c.wpe = 1;
    c.cpl = 1;
    c.nw = 4;
    (void)xf;
    if (nb > 1) {
        // several activation vectors: more rows per tile, so each staged
        // activation read from LDS serves more code words, one step per round
        // (measured on the 70B shapes, K = 8192 and 28672)
        c.u = 1;
        c.nw = 8;
        if (nb <= 4 && K < 16384) {
            c.lpr = 64;
            c.r = 2;
            c.cpl = 2;
        } else if (nb <= 2) {
            c.lpr = 32;
            c.r = 2;
            c.cpl = 2;
            c.nw = 16;
        } else if (nb <= 4) {
            c.lpr = 32;
            c.r = 4;
            c.cpl = 1;
            c.nw = 16;
        } else {
            c.lpr = 32;
            c.r = 2;
            c.cpl = 2;
        }
        return c;
    }
    const bool even = chunks % 128 == 0;   // LPR 64 x CPL 2 covers whole steps
    const int S1 = (chunks + c.lpr - 1) / c.lpr;
    if ((int64_t)N * S1 / (64 / c.lpr) < 4096) {
        // latency regime: one row segment per wave, all steps in one round
        const int s64 = (chunks + 63) / 64;
        if (c.lpr != 64 && (double)chunks / (s64 * 64) > 0.85) c.lpr = 64;
        c.cpl = (c.lpr == 64 && even) ? 2 : 1;
        const int S = (chunks + c.lpr * c.cpl - 1) / (c.lpr * c.cpl);
        c.r = 1;
        c.u = S <= 4 ? 4 : 8;
        const int tiles = N / (64 / c.lpr);
        c.nw = std::max(1, std::min(16, pow2_floor(std::max(1, tiles / 256))));
        // fewer tiles than CUs (a router): 8-wave workgroups share one staging
        // of x instead of every wave staging it alone (measured 16 % faster
        // on a 128-row router)
        if (tiles < 256) c.nw = std::min(8, pow2_floor(std::max(1, tiles)));
        return c;
    }
    if (N >= 16384 && even) {
        // many rows: two rows per tile, whole groups per lane
        c.lpr = 64;
        c.cpl = 2;
        const int S = chunks / 128;
        c.r = 2;
        c.u = S >= 2 ? 2 : 1;
        c.nw = 8;
        return c;
    }
    if (S1 <= 8 || !even) {
        // few rows: one row per tile, up to four steps per round
        if (even && c.lpr == 64) c.cpl = 2;
        c.r = 1;
        c.u = 4;
        c.nw = 16;
        return c;
    }
    c.lpr = 64;
    c.cpl = 2;
    c.r = 2;
    c.u = 1;
    c.nw = 8;
    return c;
}

#define QD_TRY(LPR_, R_, U_, WPE_, CPL_)                                                  \
    if (c.lpr == LPR_ && c.r == R_ && c.u == U_ && c.wpe == WPE_ && c.cpl == CPL_)         \
        return run_cfg<BITS, XF, B, LPR_, R_, U_, WPE_, CPL_, FMT>(a, c.nw, st);
#define QD_LPRS(R_, U_, WPE_)                                                    \
    QD_TRY(64, R_, U_, WPE_, 1) QD_TRY(32, R_, U_, WPE_, 1) QD_TRY(16, R_, U_, WPE_, 1) \
    QD_TRY(8, R_, U_, WPE_, 1)
#define QD_LPRS2(R_, U_, WPE_) QD_TRY(64, R_, U_, WPE_, 2) QD_TRY(32, R_, U_, WPE_, 2)

template <int BITS, int XF, int B, int FMT>
hipError_t run_b(const GemvArgs& a, const Cfg& c, hipStream_t st) {
    if constexpr (B == 1) {
        QD_LPRS(1, 4, 1) QD_LPRS(1, 8, 1)
        QD_LPRS2(2, 1, 1) QD_LPRS2(2, 2, 1) QD_LPRS2(1, 4, 1) QD_LPRS2(1, 8, 1)
#ifdef QD_TUNING
        if constexpr (BITS == 4 && XF == 0 && FMT == W_AFFINE) {
            QD_LPRS(4, 2, 1) QD_LPRS(2, 2, 1) QD_LPRS(4, 1, 1)
            QD_LPRS2(4, 1, 1) QD_LPRS2(1, 2, 1) QD_LPRS2(4, 2, 1) QD_LPRS2(2, 4, 1) QD_LPRS2(8, 1, 1)
            QD_LPRS(2, 4, 1) QD_LPRS(8, 1, 1) QD_LPRS(2, 8, 1) QD_LPRS(8, 2, 1)
            QD_LPRS(1, 4, 4) QD_LPRS(2, 2, 4) QD_LPRS(2, 4, 4) QD_LPRS(4, 1, 4) QD_LPRS(4, 2, 4)
            QD_LPRS(8, 1, 4) QD_LPRS(1, 8, 4)
        }
#endif
    } else if constexpr (B == 2 || B == 4) {
        QD_TRY(64, 2, 1, 1, 2) QD_TRY(32, 2, 1, 1, 2) QD_TRY(32, 4, 1, 1, 1)
#ifdef QD_TUNING
        if constexpr (FMT == W_AFFINE) QD_LPRS(2, 2, 1)
        if constexpr (BITS == 4 && XF == 0 && FMT == W_AFFINE) {
            QD_LPRS(4, 1, 1) QD_LPRS(4, 2, 1) QD_LPRS(2, 1, 1) QD_LPRS(1, 2, 1) QD_LPRS(1, 4, 1)
            QD_LPRS2(2, 1, 1) QD_LPRS2(2, 2, 1) QD_LPRS2(4, 1, 1) QD_LPRS2(1, 2, 1)
        }
#endif
    } else {
        QD_TRY(32, 2, 1, 1, 2)
#ifdef QD_TUNING
        if constexpr (FMT == W_AFFINE) QD_LPRS(1, 2, 1)
        if constexpr (BITS == 4 && XF == 0 && FMT == W_AFFINE) {
            QD_LPRS(2, 1, 1) QD_LPRS(2, 2, 1) QD_LPRS(4, 1, 1) QD_LPRS(1, 1, 1) QD_LPRS(1, 4, 1)
            QD_LPRS2(1, 1, 1) QD_LPRS2(2, 1, 1) QD_LPRS2(1, 2, 1) QD_LPRS2(4, 1, 1)
        }
#endif
    }
    return hipErrorInvalidConfiguration;
}
#undef QD_LPRS2
#undef QD_LPRS
#undef QD_TRY

template <int BITS, int XF, int FMT>
hipError_t run_batch(const GemvArgs& a, const Cfg& c, hipStream_t st) {
    if (a.nb <= 1) return run_b<BITS, XF, 1, FMT>(a, c, st);
    if (a.nb <= 2) return run_b<BITS, XF, 2, FMT>(a, c, st);
    if (a.nb <= 4) return run_b<BITS, XF, 4, FMT>(a, c, st);
    return run_b<BITS, XF, 8, FMT>(a, c, st);
}

}  // namespace

#ifdef QD_TUNING
// Tuning builds only: force a configuration (all zero = the default policy).
// Entry 6 >= 0 forces the tile order alone.
extern "C" int qd_tune_gemv[7] = {0, 0, 0, 0, 1, 4, -1};
#endif

hipError_t launch_gemv(int bits, int fmt, const uint32_t* wq, const uint16_t* s,
                       const uint16_t* b, const uint32_t* zp, const void* x, int xkind, float* y,
                       int N, int K, int batch, hipStream_t st, const GemvRot* rot) {
    if ((fmt == W_MIRAI_M && bits != 4) || (fmt == W_MIRAI_L && bits != 8) ||
        (fmt != W_AFFINE && batch > 8) || (rot && (fmt == W_AFFINE || xkind == X_F32)))
        return hipErrorInvalidValue;
    // a chunk of tokens through 8-bit weights (prefill routers): one
    // matrix-core launch instead of slices of 8
    if (fmt == W_AFFINE && bits == 8 && batch > 8 && (xkind == X_F16 || xkind == X_BF16))
        return launch_gemm8_tokens(wq, s, b, (const uint16_t*)x, xkind, y, N, K, batch, st);
    for (int b0 = 0; b0 < batch; b0 += 8) {
        GemvArgs a{};
        a.wq = wq;
        a.s = s;
        a.b = b;
        const size_t esz = xkind == X_F32 ? 4 : 2;
        a.x = (const char*)x + (size_t)b0 * K * esz;
        a.y = y + (size_t)b0 * N;
        a.xkind = xkind;
        a.N = N;
        a.K = K;
        a.nb = std::min(8, batch - b0);
        a.zp = (const uint8_t*)zp;
        a.zstride = 4 * ((K / 64 + 7) / 8);
        if (rot) {
            a.signs = rot->signs;
            a.gamma = rot->gamma;
            a.eps = rot->eps;
        }
        const int xf = xkind == X_F16 ? 0 : 1;
        Cfg c = default_cfg(bits, xf, a.nb, N, K);
        if (c.cpl == 2 && c.u * c.r > (xf == 0 && !rot ? 4 : 2)) {
            // Rounds of whole groups beyond these sizes exceed the 128 VGPRs of a
            // 1024-thread workgroup once the activations are fp32 or two fp16
            // planes (a spilled load result must wait for its load, which
            // serializes the round): keep eight single-chunk steps, or one
            // step of two rows, in flight instead.
            if (c.r == 1) {
                c.cpl = 1;
                c.u = 8;
            } else {
                c.u = 1;
            }
        }
#ifdef QD_TUNING
        if (qd_tune_gemv[0])
            c = Cfg{qd_tune_gemv[0], qd_tune_gemv[1], qd_tune_gemv[2], qd_tune_gemv[3],
                    qd_tune_gemv[4], qd_tune_gemv[5], c.il};
        if (qd_tune_gemv[6] >= 0) c.il = qd_tune_gemv[6];
#endif
        a.interleave = c.il;
        hipError_t e;
        if (rot)
            e = fmt == W_MIRAI_M ? run_batch<4, 2, W_MIRAI_M>(a, c, st)
                                 : run_batch<8, 2, W_MIRAI_L>(a, c, st);
        else if (fmt == W_MIRAI_M)
            e = xf == 0 ? run_batch<4, 0, W_MIRAI_M>(a, c, st) : run_batch<4, 1, W_MIRAI_M>(a, c, st);
        else if (fmt == W_MIRAI_L)
            e = xf == 0 ? run_batch<8, 0, W_MIRAI_L>(a, c, st) : run_batch<8, 1, W_MIRAI_L>(a, c, st);
        else if (bits == 4)
            e = xf == 0 ? run_batch<4, 0, W_AFFINE>(a, c, st) : run_batch<4, 1, W_AFFINE>(a, c, st);
        else
            e = xf == 0 ? run_batch<8, 0, W_AFFINE>(a, c, st) : run_batch<8, 1, W_AFFINE>(a, c, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace qd
