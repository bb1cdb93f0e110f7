/*
 * Runs every routine of the CPU oracle (oracle/oracle.c) on small seeded
 * inputs, for a build with AddressSanitizer and UndefinedBehaviorSanitizer:
 * any out-of-bounds access, use of uninitialised heap, integer overflow or
 * misaligned access in the oracle aborts the run. It also checks a few exact
 * identities so that a build that computes nothing cannot pass:
 *   y of the GEMV equals the dequantized matrix times x (the same fp64 sums),
 *   the listed-rows GEMV equals the full one on those rows,
 *   top-k ids are distinct and their weights sum to one.
 * Test infrastructure only (it links the oracle, never the HIP library).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/oracle.h"

static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) {   /* xorshift64* */
    st ^= st >> 12; st ^= st << 25; st ^= st >> 27;
    return (uint32_t)((st * 0x2545F4914F6CDD1Dull) >> 32);
}
static uint16_t rnd_f16(double lo, double hi) {   /* an fp16 value in [lo, hi): via float bits */
    const double v = lo + (hi - lo) * (rnd() / 4294967296.0);
    /* round to fp16 by hand: |v| < 65504, normal or subnormal */
    const double av = fabs(v);
    uint16_t sign = v < 0 ? 0x8000 : 0;
    if (av < ldexp(1.0, -24)) return sign;
    int e; frexp(av, &e);                  /* av = m 2^e, m in [0.5, 1) */
    int ex = e - 1;                        /* av in [2^ex, 2^(ex+1)) */
    if (ex < -14) ex = -14;                /* subnormal range */
    const double q = nearbyint(av / ldexp(1.0, ex - 10));   /* 10 fraction bits */
    uint32_t m = (uint32_t)q;
    if (ex == -14 && m < 1024) return (uint16_t)(sign | m);
    if (m == 2048) { m = 1024; ex++; }
    return (uint16_t)(sign | ((ex + 15) << 10) | (m - 1024));
}
static uint16_t rnd_bf16(double lo, double hi) {
    const float f = (float)(lo + (hi - lo) * (rnd() / 4294967296.0));
    uint32_t u; memcpy(&u, &f, 4);
    u += 0x7FFF + ((u >> 16) & 1);
    return (uint16_t)(u >> 16);
}

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

static int gemv_case(int bits, int64_t T, int64_t N, int64_t K) {
    const int64_t W = K * bits / 32, G = K / 64;
    uint32_t* wq = malloc(sizeof(uint32_t) * N * W);
    uint16_t* s = malloc(2 * N * G);
    uint16_t* b = malloc(2 * N * G);
    double* x = malloc(sizeof(double) * T * K);
    double* w = malloc(sizeof(double) * N * K);
    double* y = malloc(sizeof(double) * T * N);
    double* a = malloc(sizeof(double) * T * N);
    int64_t rows[3] = {0, N / 2, N - 1};
    double yr[3 * 8], ar[3 * 8];
    for (int64_t i = 0; i < N * W; ++i) wq[i] = rnd();
    for (int64_t i = 0; i < N * G; ++i) { s[i] = rnd_f16(0.002, 0.02); b[i] = rnd_f16(-0.2, 0.0); }
    for (int64_t i = 0; i < T * K; ++i) x[i] = qo_f16_to_f64(rnd_f16(-2.0, 2.0));
    qo_dequant(bits, wq, s, b, N, K, w);
    qo_gemv(bits, wq, s, b, x, T, N, K, y, a);
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, aa = 0.0;
            for (int64_t k = 0; k < K; ++k) { acc += w[n * K + k] * x[t * K + k]; aa += fabs(w[n * K + k] * x[t * K + k]); }
            CHECK(acc == y[t * N + n]);
            CHECK(fabs(aa - a[t * N + n]) <= 1e-12 * aa);
        }
    qo_gemv_rows(bits, wq, s, b, x, T, N, K, rows, 3, yr, ar);
    for (int64_t t = 0; t < T; ++t)
        for (int r = 0; r < 3; ++r) CHECK(yr[t * 3 + r] == y[t * N + rows[r]]);
    for (int64_t k = 0; k < K; ++k) {
        const int q = qo_code(bits, wq, k);
        CHECK(q >= 0 && q < (1 << bits));
    }
    free(wq); free(s); free(b); free(x); free(w); free(y); free(a);
    return 0;
}

static int route_case(int64_t T, int64_t E, int64_t k) {
    double* l = malloc(sizeof(double) * T * E);
    int32_t* idx = malloc(sizeof(int32_t) * T * k);
    double* p = malloc(sizeof(double) * T * k);
    for (int64_t i = 0; i < T * E; ++i) l[i] = (double)(rnd() % 64) / 8.0;   /* ties happen */
    CHECK(qo_route_topk(l, T, E, k, idx, p) == 0);
    for (int64_t t = 0; t < T; ++t) {
        double sum = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            CHECK(idx[t * k + j] >= 0 && idx[t * k + j] < E);
            for (int64_t i = 0; i < j; ++i) CHECK(idx[t * k + i] != idx[t * k + j]);
            sum += p[t * k + j];
        }
        CHECK(fabs(sum - 1.0) < 1e-12);
    }
    CHECK(qo_route_topk(l, T, E, E + 1, idx, p) == -1);
    free(l); free(idx); free(p);
    return 0;
}

static int moe_case(void) {
    const int64_t E = 5, H = 128, I = 64, Is = 128, T = 3, k = 2;
    qo_moe m;
    m.E = E; m.H = H; m.I = I; m.Is = Is;
    uint32_t* gu_q = malloc(4 * E * 2 * I * H / 8);
    uint32_t* dn_q = malloc(4 * E * H * I / 8);
    uint32_t* sgu_q = malloc(4 * 2 * Is * H / 8);
    uint32_t* sdn_q = malloc(4 * H * Is / 8);
    const int64_t ng[4] = {E * 2 * I * H / 64, E * H * I / 64, 2 * Is * H / 64, H * Is / 64};
    uint16_t* sb[8];
    for (int j = 0; j < 8; ++j) {
        sb[j] = malloc(2 * ng[j / 2]);
        for (int64_t i = 0; i < ng[j / 2]; ++i) sb[j][i] = (j & 1) ? rnd_f16(-0.2, 0.0) : rnd_f16(0.002, 0.02);
    }
    for (int64_t i = 0; i < E * 2 * I * H / 8; ++i) gu_q[i] = rnd();
    for (int64_t i = 0; i < E * H * I / 8; ++i) dn_q[i] = rnd();
    for (int64_t i = 0; i < 2 * Is * H / 8; ++i) sgu_q[i] = rnd();
    for (int64_t i = 0; i < H * Is / 8; ++i) sdn_q[i] = rnd();
    m.gu_q = gu_q; m.dn_q = dn_q; m.sgu_q = sgu_q; m.sdn_q = sdn_q;
    m.gu_s = sb[0]; m.gu_b = sb[1]; m.dn_s = sb[2]; m.dn_b = sb[3];
    m.sgu_s = sb[4]; m.sgu_b = sb[5]; m.sdn_s = sb[6]; m.sdn_b = sb[7];
    double* x = malloc(sizeof(double) * T * H);
    for (int64_t i = 0; i < T * H; ++i) x[i] = qo_f16_to_f64(rnd_f16(-1.0, 1.0));
    int32_t idx[6] = {0, 4, 2, 3, 1, 0};   /* T * k */
    double p[6] = {0.7, 0.3, 0.5, 0.5, 0.9, 0.1};
    double* y = malloc(sizeof(double) * T * H);
    double* a = malloc(sizeof(double) * T * H);
    double* h = malloc(sizeof(double) * T * k * I);
    double* hs = malloc(sizeof(double) * T * Is);
    for (int act = 0; act < 2; ++act) {
        qo_moe_experts(&m, x, T, k, idx, p, act, y, a, h, hs);
        for (int64_t i = 0; i < T * H; ++i) CHECK(isfinite(y[i]) && a[i] >= fabs(y[i]) * 0.0);
        qo_moe_experts(&m, x, T, k, idx, p, act, y, a, NULL, NULL);
    }
    CHECK(qo_gelu(0.0, 0) == 0.0 && qo_gelu(0.0, 1) == 0.0);
    free(gu_q); free(dn_q); free(sgu_q); free(sdn_q);
    for (int j = 0; j < 8; ++j) free(sb[j]);
    free(x); free(y); free(a); free(h); free(hs);
    return 0;
}

static int mirai_case(int fmt, int64_t T, int64_t N, int64_t K) {
    const int bits = fmt == QO_MIRAI_M ? 4 : 8;
    const int64_t W = K * bits / 32, G = K / 64, ZW = (G + 7) / 8;
    uint32_t* wq = malloc(4 * N * W);
    uint16_t* s = malloc(2 * N * G);
    uint32_t* zp = malloc(4 * N * ZW);
    double* x = malloc(sizeof(double) * T * K);
    double* w = malloc(sizeof(double) * N * K);
    double* y = malloc(sizeof(double) * T * N);
    double* a = malloc(sizeof(double) * T * N);
    for (int64_t i = 0; i < N * W; ++i) wq[i] = rnd();
    for (int64_t i = 0; i < N * G; ++i) s[i] = rnd_bf16(0.002, 0.02);
    for (int64_t i = 0; i < N * ZW; ++i) zp[i] = rnd();
    for (int64_t i = 0; i < T * K; ++i) x[i] = qo_f16_to_f64(rnd_f16(-2.0, 2.0));
    qo_mirai_dequant(fmt, wq, s, fmt == QO_MIRAI_M ? zp : NULL, N, K, w);
    qo_mirai_gemv(fmt, wq, s, fmt == QO_MIRAI_M ? zp : NULL, x, T, N, K, NULL, 0, y, a);
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += w[n * K + k] * x[t * K + k];
            CHECK(acc == y[t * N + n]);
        }
    free(wq); free(s); free(zp); free(x); free(w); free(y); free(a);
    return 0;
}

static int rot_attn_case(void) {
    const int64_t K = 96;
    double x[96], r[96], g[96], o[96];
    uint32_t signs[3] = {rnd(), rnd(), rnd()};
    for (int i = 0; i < K; ++i) { x[i] = qo_f16_to_f64(rnd_f16(-3.0, 3.0)); g[i] = 1.0 + 0.01 * i; }
    qo_rht(x, K, signs, r);
    qo_rht(x, K, NULL, o);
    qo_rmsnorm(x, K, g, 1e-6, o);
    qo_rmsnorm(x, K, NULL, 0.0, o);
    double n0 = 0.0, n1 = 0.0;
    for (int i = 0; i < K; ++i) { n0 += x[i] * x[i]; n1 += r[i] * r[i]; }
    CHECK(fabs(n1 - n0) <= 1e-9 * n0 * 32.0 && isfinite(n1));   /* 2^-2.5 H_32 D is orthogonal (H H^T = 32 I): the norm is kept */
    const int64_t Hq = 4, Hkv = 2, D = 64, cap = 40;
    double* q = malloc(sizeof(double) * Hq * D);
    double* kn = malloc(sizeof(double) * Hkv * D);
    double* vn = malloc(sizeof(double) * Hkv * D);
    double* kc = malloc(sizeof(double) * Hkv * cap * D);
    double* vc = malloc(sizeof(double) * Hkv * cap * D);
    double* out = malloc(sizeof(double) * Hq * D);
    double* a = malloc(sizeof(double) * Hq * D);
    for (int64_t i = 0; i < Hq * D; ++i) q[i] = qo_f16_to_f64(rnd_f16(-1.0, 1.0));
    for (int64_t i = 0; i < Hkv * D; ++i) { kn[i] = qo_f16_to_f64(rnd_f16(-1.0, 1.0)); vn[i] = kn[i] * 0.5; }
    for (int64_t i = 0; i < Hkv * cap * D; ++i) { kc[i] = qo_f16_to_f64(rnd_f16(-1.0, 1.0)); vc[i] = -kc[i]; }
    const int64_t cases[4][2] = {{0, 0}, {0, 39}, {40, 5}, {40, 100}};   /* window, pos */
    for (int c = 0; c < 4; ++c) {
        qo_attn_decode(q, kn, vn, kc, vc, Hq, Hkv, D, cap, cases[c][0], cases[c][1], 0.125, out, a);
        for (int64_t i = 0; i < Hq * D; ++i) CHECK(isfinite(out[i]) && a[i] >= 0.0);
        CHECK(qo_attn_slot(cases[c][1], cases[c][0]) >= 0);
    }
    free(q); free(kn); free(vn); free(kc); free(vc); free(out); free(a);
    return 0;
}

int main(void) {
    uint16_t h16[1 << 16];
    double d16[1 << 16];
    for (int i = 0; i < (1 << 16); ++i) h16[i] = (uint16_t)i;
    qo_f16_array(h16, 1 << 16, d16);
    qo_bf16_array(h16, 1 << 16, d16);
    qo_set_threads(2);
    CHECK(qo_get_threads() >= 1);
    const int64_t shapes[4][3] = {{1, 1, 64}, {3, 5, 128}, {8, 17, 704}, {2, 33, 256}};
    for (int i = 0; i < 4; ++i)
        for (int bits = 4; bits <= 8; bits += 4)
            if (gemv_case(bits, shapes[i][0], shapes[i][1], shapes[i][2])) return 1;
    if (route_case(1, 1, 1) || route_case(4, 128, 8) || route_case(3, 33, 33) || route_case(2, 1024, 32))
        return 1;
    if (moe_case()) return 1;
    for (int i = 0; i < 4; ++i)
        if (mirai_case(QO_MIRAI_M, shapes[i][0], shapes[i][1], shapes[i][2]) ||
            mirai_case(QO_MIRAI_L, shapes[i][0], shapes[i][1], shapes[i][2]))
            return 1;
    if (rot_attn_case()) return 1;
    printf("oracle driver ok\n");
    return 0;
}
