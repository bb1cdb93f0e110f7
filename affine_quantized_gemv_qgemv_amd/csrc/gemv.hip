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
};

template <int BITS, int XF, int B, int LPR, int R, int U>
__global__ __launch_bounds__(256) void qgemv_kernel(GemvArgs a) {
    extern __shared__ uint4 lds[];
    constexpr int CC = 128 / BITS;     // codes per 16-byte chunk
    constexpr int CPG = 64 / CC;       // chunks per group of 64
    constexpr int RPI = 64 / LPR;      // rows per wave instruction
    constexpr int ROWS = RPI * R;      // rows per tile
    const int C16 = a.K / CC;
    const int c0 = blockIdx.y * a.chunks_split;
    const int nc = min(a.chunks_split, C16 - c0);
    const int G = a.K / 64;
    const int64_t wpr = (int64_t)a.K * BITS / 32;  // words per row

    stage_x<BITS, XF>(a.x, a.xkind, a.K, a.nb, c0, nc, lds);
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int seg = lane / LPR, sl = lane % LPR;
    const int nwaves = blockDim.x >> 6;
    const int wave = threadIdx.x >> 6;
    const int S = (nc + LPR - 1) / LPR;
    const int ntiles = (a.N + ROWS - 1) / ROWS;
    const uint32_t magic = in_vgpr(kMagic16);

    for (int tile = blockIdx.x * nwaves + wave; tile < ntiles; tile += gridDim.x * nwaves) {
        int row[R];
        bool rv[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            row[r] = tile * ROWS + r * RPI + seg;
            rv[r] = row[r] < a.N;
        }
        float y[R][B];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int bb = 0; bb < B; ++bb) y[r][bb] = 0.f;

        for (int s0 = 0; s0 < S; s0 += U) {
            uint4 cw[U][R];
            float sc[U][R], bi[U][R];
            // issue every load of this batch of steps before using any
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = (s0 + u) * LPR + sl;
                const bool cv = (s0 + u < S) && (c < nc);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (cv && rv[r]) {
                        const int gc = c0 + c;
                        cw[u][r] = *(const uint4*)(a.wq + (int64_t)row[r] * wpr + (int64_t)gc * 4);
                        const int64_t gi = (int64_t)row[r] * G + gc / CPG;
                        sc[u][r] = h2f(a.s[gi]);
                        bi[u][r] = h2f(a.b[gi]);
                    } else {
                        cw[u][r] = make_uint4(0, 0, 0, 0);
                        sc[u][r] = 0.f;
                        bi[u][r] = 0.f;
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = (s0 + u) * LPR + sl;
                if ((s0 + u < S) && (c < nc))
                    chunk_rows<BITS, XF, B, R>(cw[u], sc[u], bi[u], lds, a.nb, nc, c, magic, y);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int bb = 0; bb < B; ++bb) {
                const float v = seg_sum<LPR>(y[r][bb]);
                if (sl == 0 && rv[r] && bb < a.nb) {
                    float* dst = a.y + (int64_t)bb * a.N + row[r];
                    if (a.atomic_out)
                        atomicAdd(dst, v);
                    else
                        *dst = v;
                }
            }
        }
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

template <int BITS, int XF, int B, int LPR, int R, int U>
hipError_t run_cfg(const GemvArgs& base, int nwaves, hipStream_t st) {
    using St = Stage<BITS, XF>;
    const DeviceInfo& dev = device_info();
    auto kern = qgemv_kernel<BITS, XF, B, LPR, R, U>;
    const int C16 = base.K / St::CC;
    // Split the chunk range when the staged activations exceed the LDS budget
    // per workgroup (half the CU's LDS, so two workgroups stay resident).
    const size_t budget = std::min<size_t>(dev.max_lds_per_block, dev.lds_per_cu / 2);
    int splits = 1;
    while (St::bytes(base.nb, (C16 + splits - 1) / splits) > budget && splits < C16) ++splits;
    int per = (C16 + splits - 1) / splits;
    splits = (C16 + per - 1) / per;
    const size_t lds = St::bytes(base.nb, per);
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
    int grid = std::min(want, std::max(1, occ) * dev.cus);
    grid = std::max(grid, 1);
    hipLaunchKernelGGL(kern, dim3(grid, splits), dim3(threads), lds, st, a);
    return hipGetLastError();
}

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

template <int BITS, int XF, int B, int R, int U>
hipError_t run_lpr(const GemvArgs& a, int lpr, hipStream_t st) {
    switch (lpr) {
        case 64: return run_cfg<BITS, XF, B, 64, R, U>(a, 4, st);
        case 32: return run_cfg<BITS, XF, B, 32, R, U>(a, 4, st);
        case 16: return run_cfg<BITS, XF, B, 16, R, U>(a, 4, st);
        default: return run_cfg<BITS, XF, B, 8, R, U>(a, 4, st);
    }
}

template <int BITS, int XF>
hipError_t run_batch(const GemvArgs& a, int lpr, hipStream_t st) {
    if (a.nb <= 1) return run_lpr<BITS, XF, 1, 4, 2>(a, lpr, st);
    if (a.nb <= 2) return run_lpr<BITS, XF, 2, 2, 2>(a, lpr, st);
    if (a.nb <= 4) return run_lpr<BITS, XF, 4, 2, 2>(a, lpr, st);
    return run_lpr<BITS, XF, 8, 1, 2>(a, lpr, st);
}

}  // namespace

hipError_t launch_gemv(int bits, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                       const void* x, int xkind, float* y, int N, int K, int batch,
                       hipStream_t st) {
    const int chunks = K * bits / 128;
    const int lpr = pick_lpr(chunks);
    const int per_word = 32 / bits;
    (void)per_word;
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
        hipError_t e;
        if (bits == 4)
            e = xkind == X_F16 ? run_batch<4, 0>(a, lpr, st) : run_batch<4, 1>(a, lpr, st);
        else
            e = xkind == X_F16 ? run_batch<8, 0>(a, lpr, st) : run_batch<8, 1>(a, lpr, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace qd
