// Kernel template and launch shapes of the batch-1..8 GEMV; instantiated per
// weight format in gemv_*.hip and driven by launch_gemv (gemv.hip).
//
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
//  * When the staged activations would not fit LDS, each workgroup streams
//    K through LDS in slices: it stages slice 0, runs all of its tiles over
//    it, stages slice 1, and so on. When a matrix has too few tiles to fill
//    the chip, the F wave groups of a workgroup share each tile, group f
//    taking the steps f, f + F, ... of every slice. A tile's row segments
//    are reduced after each slice and added to a per-row partial that the
//    group keeps in LDS; at the end the F partials are summed in group
//    order. Every output is therefore summed in the same order on every run
//    (no atomics, no cleared output, no second launch).
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
#pragma once

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
    int chunks_slice;    // chunks per K slice staged at a time (a multiple of 4)
    int nslices;         // K slices staged one after another
    int slice_lds;       // bytes of LDS before the partials (the staged slice, aligned)
    int part_tiles;      // tiles per tile-wave the partials region holds
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
    if constexpr (XF == 0)
        stage_x_cm<BITS, B, CPL>(x, xstride, nb, c0, nc, lds);
    else
        stage_x<BITS, XF, CPL>(x, kind, xstride, nb, c0, nc, lds);
}

// SL: K is streamed in a.nslices slices (otherwise one slice holds all of K).
// LF: log2 of F, the wave groups that share each tile (group f takes the
// steps f, f + F, ... of every slice).
template <int BITS, int XF, int B, int LPR, int R, int U, int WPE, int CPL, int FMT, bool SL,
          int LF>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(WPE))) void qgemv_kernel(
    GemvArgs a) {
    extern __shared__ uint4 lds[];
    constexpr int CC = 128 / BITS;     // codes per 16-byte chunk
    constexpr int CPG = 64 / CC;       // chunks per group of 64
    constexpr int RPI = 64 / LPR;      // rows per wave instruction
    constexpr int ROWS = RPI * R;      // rows per tile
    constexpr bool CM = XF == 0;   // chunk-major staging of fp16 activations (stage_x_cm)
    const int C16 = a.K / CC;
    const int G = a.K / 64;
    const int64_t wpr = (int64_t)a.K * BITS / 32;  // words per row

    const int lane = threadIdx.x & 63;
    const int seg = lane / LPR, sl = lane % LPR;
    const int nwaves = blockDim.x >> 6;
    // wave-uniform: keeps the tile bounds and loop control in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    constexpr int F = 1 << LF;           // wave groups per tile
    const int f = wave & (F - 1);        // this wave's group
    const int TWG = nwaves >> LF;        // tile-waves per workgroup
    const int tw = wave >> LF;
    const int gw = blockIdx.x * TWG + tw;
    const int W = gridDim.x * TWG;
    const int ntiles = (a.N + ROWS - 1) / ROWS;
    // This tile-wave's tiles, interleaved: tile-wave w takes tiles w, w + W,
    // ..., so all waves together sweep one window of the matrix, as a
    // streaming read does.
    const int t0 = gw, tstep = W;
    const int ntl = gw < ntiles ? (ntiles - gw + W - 1) / W : 0;
    // Partials in LDS unless one pass over K finishes every row:
    // [group][tile-wave][tile of the tile-wave][row][vector]
    const bool direct = F == 1 && a.nslices == 1;
    const int PT = a.part_tiles;
    float* part_base = (float*)((char*)lds + a.slice_lds);
    float* part = part_base + (size_t)(f * TWG + tw) * PT * ROWS * B;

    // Rotation prologue: LDS for the per-vector factors (only kernels with
    // XF == 2 reference it); rot[kRotMaxB + b] is 2^-e of vector b.
    float* rot = nullptr;
    if constexpr (XF == 2) rot = rot_shared();

    // The slice being processed: chunks [c0, c0 + nc); S steps per row for
    // this wave's group (step i of the group is step i F + f of the row),
    // RPT rounds per tile.
    int c0 = 0, nc = 0, S = 0, RPT = 1;

    // Loads are unconditional inside a wave-uniform step test: rows past N and
    // chunks past the staged range read a clamped, valid address and get a
    // zero scale and bias, so they add nothing. (Branches around individual
    // loads would make the compiler wait for every load in flight.) Each
    // round's loads go through buffer resources based at the tile's first
    // row, so per-lane offsets are 32-bit and the chunk and step offsets are
    // instruction immediates.
    const uint32_t rowb = (uint32_t)(wpr * 4);   // bytes of codes per row (< 2^24)
    // all: request every step of the round (the peeled first round, so that
    // no branch sits among the prologue's loads)
    auto issue = [&](Round<R, U, CPL>& buf, int tile, int sg, bool all = false) {
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
            if (!all && sg * U + u >= S) break;  // uniform
            const int c = (((sg * U + u) * F + f) * LPR + sl) * CPL;
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
    // ti: the tile's index among this wave's tiles (its partials slot)
    auto consume = [&](const Round<R, U, CPL>& buf, int tile, int ti, int sg, bool last) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (sg * U + u >= S) break;  // uniform
            const int cu = (((sg * U + u) * F + f) * LPR + sl) * CPL;
            const int c = min(cu, nc - CPL);
            // per row: scale, centred bias and the centring subtrahends
            float sc[R], bi[R];
            uint32_t n1[R], n16[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const bool ok = (cu < nc) && (tile * ROWS + r * RPI + seg < a.N);
                if constexpr (FMT == W_AFFINE) {
                    // w = s q + b = s (q - c) + (b + c s), c = 8 or 128
                    constexpr float cen = BITS == 4 ? 8.f : 128.f;
                    sc[r] = ok ? h2f(buf.sc[u][r]) : 0.f;
                    bi[r] = ok ? fmaf(cen, sc[r], h2f(buf.bi[u][r])) : 0.f;
                    n1[r] = BITS == 4 ? kNeg1032 : kNeg1152;
                    n16[r] = kNeg1152;
                } else if constexpr (FMT == W_MIRAI_M) {
                    // w = s (q - z): centred on the group's zero point
                    const int zsh = (((c0 + c) / CPG) & 1) * 4;
                    const uint32_t z = (buf.bi[u][r] >> zsh) & 15u;
                    sc[r] = ok ? bf2f(buf.sc[u][r]) : 0.f;
                    bi[r] = 0.f;
                    n1[r] = neg_pair(0xE400u | z);
                    n16[r] = neg_pair(0xE400u | (z << 4));
                } else {
                    // signed codes with the top bit flipped: u = q + 128, centre 128
                    sc[r] = ok ? bf2f(buf.sc[u][r]) : 0.f;
                    bi[r] = 0.f;
                    n1[r] = kNeg1152;
                    n16[r] = kNeg1152;
                }
            }
            int slot[CPL];
#pragma unroll
            // c is a multiple of CPL: the lane's chunks sit nc / CPL slots apart
            for (int ch = 0; ch < CPL; ++ch)
                slot[ch] = (int)((unsigned)c / CPL + (unsigned)ch * ((unsigned)nc / CPL));
            constexpr bool XS = FMT == W_AFFINE;   // the Mirai formats have no sum term
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
                group_rows<BITS, XF, B, R, CPL, CM, XS>(cw, sc, bi, n1, n16, lds, a.nb, nc, slot,
                                                         magic, y);
            } else {
                group_rows<BITS, XF, B, R, CPL, CM, XS>(buf.cw[u], sc, bi, n1, n16, lds, a.nb, nc,
                                                         slot, magic, y);
            }
        }
        if (sg == RPT - 1) {
            // the tile's rows over this slice (this group's steps): stored, or
            // added to the group's partial (same wave, same order on every
            // run); a lone group stores the sum after the last slice
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
                        if (direct) {
                            *dst = v;
                        } else {
                            float* pp = part + ((size_t)ti * ROWS + r * RPI + seg) * B + bb;
                            v = *pp + v;
                            if (F == 1 && last)
                                *dst = v;
                            else
                                *pp = v;
                        }
                    }
                }
            }
        }
    };

    // One buffer per wave: a round's loads are all issued before any is used;
    // other waves on the SIMD keep the memory system busy while this one
    // computes.
    Round<R, U, CPL> A;
    auto set_slice = [&](int slc) {
        c0 = slc * a.chunks_slice;
        nc = min(a.chunks_slice, C16 - c0);
        const int srow = (nc + LPR * CPL - 1) / (LPR * CPL);   // steps per row
        S = srow > f ? (srow - f + F - 1) >> LF : 0;           // this group's
        RPT = (S + U - 1) / U;                                 // rounds per tile
    };
    // all of this wave's tiles over the staged slice
    auto run_slice = [&](bool first, bool last) {
        const int nrounds = ntl * RPT;
        for (int rd = 0; rd < nrounds; ++rd) {
            const int ti = rd / RPT;
            const int tile = t0 + ti * tstep;
            const int sg = rd - ti * RPT;
            if (rd > 0 || !first) issue(A, tile, sg);
            consume(A, tile, ti, sg, last);
        }
    };
    // this group's partials start at zero (visible after the first barrier)
    if (!direct)
        for (int e = lane; e < PT * ROWS * B; e += 64) part[e] = 0.f;
    // Slice 0: the first weight loads are in flight while the activations
    // are staged (behind the activation loads when they are rotated, so the
    // transform runs while the weights arrive).
    set_slice(0);
    if constexpr (XF == 2) {
        stage_x_rot<BITS, CPL>((const uint16_t*)a.x, a.xkind, a.K, a.nb, c0, nc, a.gamma,
                               a.signs, a.eps, rot, lds,
                               [&]() { if (ntl > 0) issue(A, t0, 0); });
    } else if constexpr (XF == 0) {
        // behind the activation loads, unconditionally (a wave with no tile
        // requests a clamped one and never uses it)
        stage_x_cm_overlap<BITS, B, CPL>(a.x, a.K, a.nb, c0, nc, lds, [&]() {
            issue(A, min(t0, ntiles - 1), 0, true);
        });
    } else {
        if (ntl > 0) issue(A, t0, 0);
        stage_x_any<BITS, XF, B, CPL>(a.x, a.xkind, a.K, a.nb, c0, nc, lds);
    }
    __syncthreads();
    if constexpr (!SL) {
        run_slice(true, true);
    } else {
        for (int slc = 0;;) {
            const bool last = slc == a.nslices - 1;
            run_slice(slc == 0, last);
            if (last) break;
            // the next slice, staged once every wave is done with this one
            set_slice(++slc);
            __syncthreads();
            if constexpr (XF == 2)
                stage_x_rot<BITS, CPL>((const uint16_t*)a.x, a.xkind, a.K, a.nb, c0, nc, a.gamma,
                                       a.signs, a.eps, rot, lds, []() {});
            else
                stage_x_any<BITS, XF, B, CPL>(a.x, a.xkind, a.K, a.nb, c0, nc, lds);
            __syncthreads();
        }
    }
    if constexpr (F > 1) {
        // the F groups' partials of each row, summed in group order
        __syncthreads();
        if (f == 0) {
            for (int ti = 0; ti < ntl; ++ti) {
                const int tile = t0 + ti * tstep;
                for (int e = lane; e < ROWS * B; e += 64) {
                    const int rl = e / B, bb = e - rl * B;
                    const int row = tile * ROWS + rl;
                    if (row < a.N && bb < a.nb) {
                        float v = 0.f;
                        for (int g = 0; g < F; ++g)
                            v += part_base[((size_t)(g * TWG + tw) * PT + ti) * ROWS * B + e];
                        a.y[(int64_t)bb * a.N + row] = v;
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Launch shapes.
// ---------------------------------------------------------------------------
struct Cfg {
    int lpr, r, u, wpe, cpl, nw;
};

// LDS reserved for the per-row partials when K is streamed in slices.

constexpr size_t kPartReserve = 8192;

template <int BITS, int XF, int B, int LPR, int R, int U, int WPE, int CPL, int FMT>
hipError_t run_cfg(const GemvArgs& base, int nwaves, hipStream_t st) {
    using St = Stage<BITS, XF>;
    const DeviceInfo& dev = device_info();
    const int C16 = base.K / St::CC;
    // Stream K in slices when the staged activations exceed the LDS budget
    // per workgroup (half the CU's LDS, so two workgroups stay resident).
    const size_t budget = std::min<size_t>(dev.max_lds_per_block, dev.lds_per_cu / 2);
    // chunks per slice: a multiple of 4 so a lane's CPL chunks never straddle
    // a slice
    auto per_of = [&](int sp) { return (((C16 + sp - 1) / sp) + 3) & ~3; };
    // the kernel's staging layout (chunk-major for several fp16 vectors)
    auto bytes = [&](int nc) {
        return XF == 0 ? St::bytes_cm(B, nc) : St::bytes(base.nb, nc);
    };
    int slices = 1;
    if (bytes(C16) > budget) {
        slices = 2;
        while (bytes(per_of(slices)) + kPartReserve > budget && slices < C16) ++slices;
    }
    const int per = std::min(per_of(slices), C16);
    slices = (C16 + per - 1) / per;
    const size_t xlds = (bytes(per) + 15) & ~(size_t)15;

    GemvArgs a = base;
    a.chunks_slice = per;
    a.nslices = slices;
    a.slice_lds = (int)xlds;
    a.part_tiles = 0;
    const int threads = nwaves * 64;
    const int rows_per_tile = (64 / LPR) * R;
    const int ntiles = (a.N + rows_per_tile - 1) / rows_per_tile;
    auto kern = slices == 1 ? qgemv_kernel<BITS, XF, B, LPR, R, U, WPE, CPL, FMT, false, 0>
                            : qgemv_kernel<BITS, XF, B, LPR, R, U, WPE, CPL, FMT, true, 0>;
    // resident wave slots with the partials region reserved
    const int occ = std::max(1, occupancy((const void*)kern, threads, xlds + kPartReserve));
    const int slots = occ * dev.cus * nwaves;
    // Sliced fp16 launches of several vectors (few rows over a long K) take
    // F wave groups per tile while the tiles leave resident waves idle
    // (never more groups than a slice has steps per row).
    int F = 1;
    if constexpr (XF == 0 && B > 1) {
        const int steps = (per + LPR * CPL - 1) / (LPR * CPL);
        if (slices > 1)
            while (F < 4 && 2 * F <= nwaves && 2 * F <= steps && (int64_t)ntiles * 2 * F <= slots)
                F *= 2;
        if (F == 2) kern = qgemv_kernel<BITS, XF, B, LPR, R, U, WPE, CPL, FMT, true, 1>;
        if (F == 4) kern = qgemv_kernel<BITS, XF, B, LPR, R, U, WPE, CPL, FMT, true, 2>;
    }
    const int twg = nwaves / F;   // tile-waves per workgroup
    const int want = (ntiles + twg - 1) / twg;
    size_t lds = xlds;
    int grid;
    if (slices == 1 && F == 1) {
        const int occ1 = occupancy((const void*)kern, threads, lds);
        grid = std::max(1, std::min(want, std::max(1, occ1) * dev.cus));
    } else {
        // partial slots of one tile for every wave of a workgroup
        const size_t per_tile = (size_t)nwaves * rows_per_tile * B * sizeof(float);
        grid = std::max(1, std::min(want, occ * dev.cus));
        int pt = (ntiles + grid * twg - 1) / (grid * twg);
        const int cap = std::max<int>(1, (int)(kPartReserve / per_tile));
        if (pt > cap) {   // more workgroups, each with fewer tiles per wave
            grid = (ntiles + twg * cap - 1) / (twg * cap);
            pt = (ntiles + grid * twg - 1) / (grid * twg);
        }
        a.part_tiles = pt;
        lds = xlds + (size_t)pt * per_tile;
    }
    if (lds > dev.max_lds_per_block) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, st, a);
    return hipGetLastError();
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
        QD_LPRS2(2, 1, 1) QD_LPRS2(2, 2, 1) QD_LPRS2(1, 1, 1) QD_LPRS2(1, 2, 1) QD_LPRS2(1, 4, 1)
        QD_LPRS2(1, 8, 1)
    } else if constexpr (B == 2 || B == 4) {
        QD_TRY(64, 2, 1, 1, 2) QD_TRY(32, 2, 1, 1, 2) QD_TRY(32, 4, 1, 1, 1)
    } else {
        QD_TRY(32, 2, 1, 1, 2)
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


// One weight format's instances (each in its own translation unit).
hipError_t gemv_run_affine4(const GemvArgs& a, const Cfg& c, int xf, hipStream_t st);
hipError_t gemv_run_affine8(const GemvArgs& a, const Cfg& c, int xf, hipStream_t st);
hipError_t gemv_run_mirai_m(const GemvArgs& a, const Cfg& c, int xf, hipStream_t st);
hipError_t gemv_run_mirai_l(const GemvArgs& a, const Cfg& c, int xf, hipStream_t st);
hipError_t gemv_run_rot(const GemvArgs& a, const Cfg& c, int fmt, hipStream_t st);

}  // namespace qd
