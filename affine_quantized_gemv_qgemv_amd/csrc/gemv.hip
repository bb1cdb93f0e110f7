// Batch-1..8 GEMV launch policy: picks a launch shape per (format, batch, N, K)
// and runs the kernel of gemv_kernel.h. Shapes come from on-device sweeps
// (graph-replayed launches, weights cycled through HBM).
#include "gemv_kernel.h"

namespace qd {

namespace {

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

Cfg default_cfg(int bits, int xf, int nb, int N, int K, bool rot) {
    Cfg c;
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
        // few rows: one row per tile, up to four steps per round (no more
        // than a row has: the first round requests all of its steps; eight
        // steps per round measured slower, fewer waves fit)
        if (even && c.lpr == 64) c.cpl = 2;
        c.r = 1;
        c.u = 4;
        if (c.cpl == 2) {
            const int S = chunks / 128;
            c.u = S <= 1 ? 1 : (S <= 2 ? 2 : 4);
        }
        // half-group chunks (rows of an odd number of 2 KB steps, e.g. the
        // 7B down projection K = 14336): two 8-wave workgroups per CU rather
        // than one of 16 (interleaved timings: 9.47 vs 9.66 us)
        c.nw = c.cpl == 2 ? 16 : 8;
        return c;
    }
    // long rows: two rows per tile, one step per round; with 4-bit codes and
    // plain fp16 activations (K = 28672 -> N = 8192) one row per tile and four
    // steps per round instead (interleaved timings: 26.8 vs 27.1 us)
    const bool deep = bits == 4 && xf == 0 && !rot;
    c.lpr = 64;
    c.cpl = 2;
    c.r = deep ? 1 : 2;
    c.u = deep ? 4 : 1;
    c.nw = 8;
    return c;
}

}  // namespace

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
    // three to eight fp16 vectors through 4-bit weights: the matrix-core GEMV
    // (gemv_mfma.hip), eight vectors per launch (70B shapes, K = 8192 and
    // 28672: 78.8 vs 150.7 us per step at batch 8, 75.3 vs 95 at batch 4;
    // at batch 2 the packed-dot kernel stays ahead, 64 vs 71.6)
    if (fmt == W_AFFINE && bits == 4 && batch > 2 && xkind == X_F16 && !rot && K % 512 == 0) {
        for (int b0 = 0; b0 < batch; b0 += 8) {
            const int nb = std::min(8, batch - b0);
            const hipError_t e =
                nb <= 2 ? launch_gemv(bits, fmt, wq, s, b, zp, (const uint16_t*)x + (size_t)b0 * K,
                                      xkind, y + (size_t)b0 * N, N, K, nb, st, nullptr)
                        : launch_gemv_mfma(wq, s, b, (const uint16_t*)x + (size_t)b0 * K,
                                           y + (size_t)b0 * N, N, K, nb, st);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
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
        Cfg c = default_cfg(bits, xf, a.nb, N, K, rot != nullptr);
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
        hipError_t e;
        if (rot)
            e = gemv_run_rot(a, c, fmt, st);
        else if (fmt == W_MIRAI_M)
            e = gemv_run_mirai_m(a, c, xf, st);
        else if (fmt == W_MIRAI_L)
            e = gemv_run_mirai_l(a, c, xf, st);
        else if (bits == 4)
            e = gemv_run_affine4(a, c, xf, st);
        else
            e = gemv_run_affine8(a, c, xf, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace qd
