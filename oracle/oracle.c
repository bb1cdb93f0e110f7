/*
 * CPU oracle (fp64) for the affine-quantized decode path.
 *
 * TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path. Shares no code
 * with the HIP library. Sources cited below:
 *   [TF]   jeff.news/article/5193 (TurboFieldfare running Gemma 4 26B-A4B on
 *          Apple Silicon), sections "성능과 제약" (performance and constraints)
 *          and "내부 구조가 진짜 흥미로운 부분" (internals).
 *   [uzu]  discuss.pytorch.kr/t/uzu-mac-iphone-llm-apple-silicon-rust/12363
 *          (uzu, an on-device engine), section "uzu의 모델 변환과 Mirai 양자화
 *          형식" (model conversion and the Mirai quantization formats).
 *   [TF] internals section also fixes the KV storage of the decode step:
 *          sliding-window layers keep a bounded circular KV store, full-
 *          attention layers a linear one, and decode attention is exact.
 * Plain loops, fp64 throughout; OpenMP only splits independent output rows
 * (each row's sum is still taken in ascending k).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 0;

void qo_set_threads(int n) { g_threads = n; }

int qo_get_threads(void) {
#ifdef _OPENMP
    return g_threads > 0 ? g_threads : omp_get_max_threads();
#else
    return 1;
#endif
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double qo_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double qo_bf16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xFF;
    int m = h & 0x7F;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133);                /* m * 2^-126 * 2^-7 */
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + m), e - 134);     /* (1 + m/128) * 2^(e-127) */
    return sign ? -v : v;
}

void qo_f16_array(const uint16_t* in, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = qo_f16_to_f64(in[i]);
}

void qo_bf16_array(const uint16_t* in, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = qo_bf16_to_f64(in[i]);
}

/* [TF] performance section: 4-bit (8-bit for the router) codes. Packing
 * reading: code k sits in word k / (32/bits) at bit offset bits*(k mod (32/bits)). */
int qo_code(int bits, const uint32_t* row, int64_t k) {
    int per_word = 32 / bits;
    uint32_t word = row[k / per_word];
    int shift = bits * (int)(k % per_word);
    return (int)((word >> shift) & ((1u << bits) - 1u));
}

/* [TF] performance section: affine quantization with group size 64, w = s*q + b. */
static double weight(int bits, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                     int64_t K, int64_t n, int64_t k) {
    int64_t words = K * bits / 32;
    int64_t groups = K / 64;
    int64_t g = k / 64;
    double sc = qo_f16_to_f64(s[n * groups + g]);
    double bi = qo_f16_to_f64(b[n * groups + g]);
    return sc * (double)qo_code(bits, wq + n * words, k) + bi;
}

void qo_dequant(int bits, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                int64_t N, int64_t K, double* w) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) w[n * K + k] = weight(bits, wq, s, b, K, n, k);
}

/* One output: y = sum_k w[n][k] x[k] in ascending k, a = sum_k |w x|. */
static void row_dot(int bits, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                    const double* x, int64_t K, int64_t n, double* y, double* a) {
    double acc = 0.0, aacc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double prod = weight(bits, wq, s, b, K, n, k) * x[k];
        acc += prod;
        aacc += fabs(prod);
    }
    *y = acc;
    if (a) *a = aacc;
}

void qo_gemv(int bits, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
             const double* x, int64_t T, int64_t N, int64_t K, double* y, double* a) {
    int nt = qo_get_threads();
    (void)nt;
    for (int64_t t = 0; t < T; ++t) {
#pragma omp parallel for schedule(static) num_threads(nt)
        for (int64_t n = 0; n < N; ++n)
            row_dot(bits, wq, s, b, x + t * K, K, n, y + t * N + n, a ? a + t * N + n : NULL);
    }
}

void qo_gemv_rows(int bits, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                  const double* x, int64_t T, int64_t N, int64_t K,
                  const int64_t* rows, int64_t nrows, double* y, double* a) {
    (void)N;
    int nt = qo_get_threads();
    (void)nt;
    for (int64_t t = 0; t < T; ++t) {
#pragma omp parallel for schedule(static) num_threads(nt)
        for (int64_t i = 0; i < nrows; ++i)
            row_dot(bits, wq, s, b, x + t * K, K, rows[i], y + t * nrows + i,
                    a ? a + t * nrows + i : NULL);
    }
}

/*
 * Routing ([TF] top section: only the router's top-8 experts are needed per
 * token; [TF] internals: the router picks the top-8 expert IDs). Taken in
 * the workload's order: softmax over all E logits, select the k largest,
 * renormalize their weights to sum to one. Selection compares the logits
 * themselves (softmax is strictly increasing, so the order is the same);
 * equal logits go to the lower expert index, both for membership and for
 * the order of the k slots.
 */
int qo_route_topk(const double* logits, int64_t T, int64_t E, int64_t k, int32_t* idx, double* p) {
    if (T < 0 || E <= 0 || k <= 0 || k > E) return -1;
    double* prob = (double*)malloc(sizeof(double) * (size_t)E);
    char* taken = (char*)malloc((size_t)E);
    if (!prob || !taken) {
        free(prob);
        free(taken);
        return -1;
    }
    for (int64_t t = 0; t < T; ++t) {
        const double* l = logits + t * E;
        /* softmax over all experts */
        double lmax = l[0];
        for (int64_t e = 1; e < E; ++e)
            if (l[e] > lmax) lmax = l[e];
        double z = 0.0;
        for (int64_t e = 0; e < E; ++e) {
            prob[e] = exp(l[e] - lmax);
            z += prob[e];
        }
        for (int64_t e = 0; e < E; ++e) prob[e] /= z;
        /* k largest, in descending order, ties to the lower index */
        memset(taken, 0, (size_t)E);
        double kept = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            taken[best] = 1;
            idx[t * k + j] = (int32_t)best;
            kept += prob[best];
        }
        /* renormalize over the selected experts */
        for (int64_t j = 0; j < k; ++j) p[t * k + j] = prob[idx[t * k + j]] / kept;
    }
    free(prob);
    free(taken);
    return 0;
}

/* GELU (Hendrycks & Gimpel): exact u * Phi(u), or their tanh approximation. */
double qo_gelu(double u, int variant) {
    if (variant == 1) {
        const double c = sqrt(2.0 / M_PI);
        return 0.5 * u * (1.0 + tanh(c * (u + 0.044715 * u * u * u)));
    }
    return 0.5 * u * (1.0 + erf(u / sqrt(2.0)));
}

/* Gate rows [0, I) and up rows [I, 2I) of z; h_i = GELU(gate_i) * up_i. */
static void gated(const double* z, int64_t I, int act, double* h) {
    for (int64_t i = 0; i < I; ++i) h[i] = qo_gelu(z[i], act) * z[I + i];
}

/*
 * [TF] internals: the GPU runs the resident shared expert, runs the routed
 * experts, then combines the shared and routed outputs. Reading: the routed
 * outputs are weighted by the renormalized router weights and the shared
 * output is added with weight one.
 */
void qo_moe_experts(const qo_moe* w, const double* x, int64_t T, int64_t k,
                    const int32_t* idx, const double* p, int act,
                    double* y, double* a, double* h, double* hs) {
    const int64_t H = w->H, I = w->I, Is = w->Is;
    const int64_t gu_words = 2 * I * (H / 8), gu_groups = 2 * I * (H / 64);
    const int64_t dn_words = H * (I / 8), dn_groups = H * (I / 64);
    double* z = (double*)malloc(sizeof(double) * (size_t)(2 * (I > Is ? I : Is)));
    double* hh = (double*)malloc(sizeof(double) * (size_t)(I > Is ? I : Is));
    double* o = (double*)malloc(sizeof(double) * (size_t)H);
    double* oa = (double*)malloc(sizeof(double) * (size_t)H);
    for (int64_t t = 0; t < T; ++t) {
        const double* xt = x + t * H;
        double* yt = y + t * H;
        double* at = a ? a + t * H : NULL;
        for (int64_t n = 0; n < H; ++n) {
            yt[n] = 0.0;
            if (at) at[n] = 0.0;
        }
        for (int64_t j = 0; j < k; ++j) {
            int64_t e = idx[t * k + j];
            double pj = p[t * k + j];
            qo_gemv(4, w->gu_q + e * gu_words, w->gu_s + e * gu_groups, w->gu_b + e * gu_groups,
                    xt, 1, 2 * I, H, z, NULL);
            gated(z, I, act, hh);
            if (h) memcpy(h + (t * k + j) * I, hh, sizeof(double) * (size_t)I);
            qo_gemv(4, w->dn_q + e * dn_words, w->dn_s + e * dn_groups, w->dn_b + e * dn_groups,
                    hh, 1, H, I, o, oa);
            for (int64_t n = 0; n < H; ++n) {
                yt[n] += pj * o[n];
                if (at) at[n] += pj * oa[n];
            }
        }
        qo_gemv(4, w->sgu_q, w->sgu_s, w->sgu_b, xt, 1, 2 * Is, H, z, NULL);
        gated(z, Is, act, hh);
        if (hs) memcpy(hs + t * Is, hh, sizeof(double) * (size_t)Is);
        qo_gemv(4, w->sdn_q, w->sdn_s, w->sdn_b, hh, 1, H, Is, o, oa);
        for (int64_t n = 0; n < H; ++n) {
            yt[n] += o[n];
            if (at) at[n] += oa[n];
        }
    }
    free(z);
    free(hh);
    free(o);
    free(oa);
}

/*
 * Mirai formats ([uzu] quantization-format section): Mirai-M is asymmetric
 * 4-bit integer quantization with a 4-bit zero point and a bf16 scale per
 * group of 64 inputs; Mirai-L is symmetric 8-bit quantization.
 * Readings where the page is silent:
 *   - Mirai-M: w = s * (q - z), q and z in [0, 15]. The zero points are
 *     packed the way codes are, eight per uint32 along the groups of a row,
 *     LSB-first, each row padded to whole words: zp[N][ceil(G/8)]; padding
 *     nibbles carry no meaning.
 *   - Mirai-L: codes are two's-complement signed bytes packed as the 8-bit
 *     codes are; one bf16 scale per group of 64 (the group size and scale
 *     type of the sibling format); w = s * q.
 */
static double mirai_weight(int fmt, const uint32_t* wq, const uint16_t* s, const uint32_t* zp,
                           int64_t K, int64_t n, int64_t k) {
    const int64_t groups = K / 64;
    const int64_t grp = k / 64;
    double sc = qo_bf16_to_f64(s[n * groups + grp]);
    if (fmt == QO_MIRAI_M) {
        int64_t zwords = (groups + 7) / 8;
        int q = qo_code(4, wq + n * (K / 8), k);
        int z = qo_code(4, zp + n * zwords, grp);
        return sc * (double)(q - z);
    }
    int u = qo_code(8, wq + n * (K / 4), k);
    int q = u >= 128 ? u - 256 : u;
    return sc * (double)q;
}

void qo_mirai_dequant(int fmt, const uint32_t* wq, const uint16_t* s, const uint32_t* zp,
                      int64_t N, int64_t K, double* w) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) w[n * K + k] = mirai_weight(fmt, wq, s, zp, K, n, k);
}

void qo_mirai_gemv(int fmt, const uint32_t* wq, const uint16_t* s, const uint32_t* zp,
                   const double* x, int64_t T, int64_t N, int64_t K,
                   const int64_t* rows, int64_t nrows, double* y, double* a) {
    int nt = qo_get_threads();
    (void)nt;
    int64_t m = rows ? nrows : N;
    for (int64_t t = 0; t < T; ++t) {
        const double* xt = x + t * K;
#pragma omp parallel for schedule(static) num_threads(nt)
        for (int64_t i = 0; i < m; ++i) {
            int64_t n = rows ? rows[i] : i;
            double acc = 0.0, aacc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double prod = mirai_weight(fmt, wq, s, zp, K, n, k) * xt[k];
                acc += prod;
                aacc += fabs(prod);
            }
            y[t * m + i] = acc;
            if (a) a[t * m + i] = aacc;
        }
    }
}

/*
 * Block-32 random Hadamard transform ([uzu] quantization-format section:
 * both Mirai formats suppress outliers with a random Hadamard transform of
 * block size 32 before quantization; the transform is fused into the
 * RMSNorm and matmul kernels). Reading: for each block of 32 consecutive
 * inputs, out = (1/sqrt(32)) * H * D * x with H the Sylvester Hadamard
 * matrix, H[i][j] = (-1)^popcount(i & j), and D = diag(d) the random signs,
 * d_j = -1 where bit j of signs[block] is set. Weights stored in the
 * rotated basis then give W' (H D x) = W x. Written as the plain 32 x 32
 * matrix-vector product (no fast transform).
 */
void qo_rht(const double* x, int64_t K, const uint32_t* signs, double* out) {
    const double c = 1.0 / sqrt(32.0);
    for (int64_t blk = 0; blk < K / 32; ++blk) {
        const double* xb = x + 32 * blk;
        double v[32];
        for (int j = 0; j < 32; ++j) {
            int neg = signs ? (int)((signs[blk] >> j) & 1u) : 0;
            v[j] = neg ? -xb[j] : xb[j];
        }
        for (int i = 0; i < 32; ++i) {
            double acc = 0.0;
            for (int j = 0; j < 32; ++j) acc += (__builtin_popcount((unsigned)(i & j)) & 1) ? -v[j] : v[j];
            out[32 * blk + i] = c * acc;
        }
    }
}

/*
 * RMSNorm (the norm the rotation is fused with, [uzu] same section):
 * out_k = x_k / sqrt(mean_k(x_k^2) + eps) * gamma_k; gamma NULL means 1.
 */
void qo_rmsnorm(const double* x, int64_t K, const double* gamma, double eps, double* out) {
    double ss = 0.0;
    for (int64_t k = 0; k < K; ++k) ss += x[k] * x[k];
    const double r = 1.0 / sqrt(ss / (double)K + eps);
    for (int64_t k = 0; k < K; ++k) out[k] = x[k] * r * (gamma ? gamma[k] : 1.0);
}

/*
 * Decode attention for one new token ([TF] internals section: sliding-window
 * layers keep their keys and values in bounded circular storage, full-
 * attention layers in linear storage, and decode attention is computed
 * exactly). Readings where the page is silent: the token at position pos is
 * stored at slot pos mod window (circular, cap == window) or at slot pos
 * (linear, window == 0); the step first stores the new key and value there,
 * then attends over the occupied slots [0, n) with n = min(pos + 1, window)
 * or pos + 1, which are exactly the positions inside the window. Query head
 * h reads key/value head h / (Hq / Hkv). Plain definition, in fp64:
 *   s_j = scale * sum_d q[h][d] k[hk][j][d],  p = softmax_j(s),
 *   out[h][d] = sum_j p_j v[hk][j][d],  a[h][d] = sum_j p_j |v[hk][j][d]|.
 * kc / vc are [Hkv][cap][D]; they are read, never written (slot_of returns
 * the slot the new token occupies, where k_new / v_new are used instead).
 */
int64_t qo_attn_slot(int64_t pos, int64_t window) { return window > 0 ? pos % window : pos; }

void qo_attn_decode(const double* q, const double* k_new, const double* v_new,
                    const double* kc, const double* vc, int64_t Hq, int64_t Hkv, int64_t D,
                    int64_t cap, int64_t window, int64_t pos, double scale,
                    double* out, double* a) {
    const int64_t n = window > 0 ? (pos + 1 < window ? pos + 1 : window) : pos + 1;
    const int64_t slot = qo_attn_slot(pos, window);
    const int64_t grp = Hq / Hkv;
    double* sc = (double*)malloc(sizeof(double) * (size_t)n);
    for (int64_t h = 0; h < Hq; ++h) {
        const int64_t hk = h / grp;
        const double* qh = q + h * D;
        double smax = -INFINITY;
        for (int64_t j = 0; j < n; ++j) {
            const double* kj = j == slot ? k_new + hk * D : kc + (hk * cap + j) * D;
            double acc = 0.0;
            for (int64_t d = 0; d < D; ++d) acc += qh[d] * kj[d];
            sc[j] = scale * acc;
            if (sc[j] > smax) smax = sc[j];
        }
        double z = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            sc[j] = exp(sc[j] - smax);
            z += sc[j];
        }
        for (int64_t d = 0; d < D; ++d) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                const double* vj = j == slot ? v_new + hk * D : vc + (hk * cap + j) * D;
                acc += sc[j] / z * vj[d];
                aacc += sc[j] / z * fabs(vj[d]);
            }
            out[h * D + d] = acc;
            if (a) a[h * D + d] = aacc;
        }
    }
    free(sc);
}

/*
 * Dynamic int8 activations for the verification GEMM (uzu page on
 * discuss.pytorch.kr, section on speculative decoding: the target model
 * checks 16-32 drafted tokens on the chip's int8 matrix path and quantizes
 * its activations to 8 bits on the fly). The page gives no scheme; the
 * reading taken here: per token (row), symmetric, scale = max |x| / 127 and
 * code = round(x / scale) with ties to even, the scale and the quotients in
 * fp32 (the precision in which the kernel takes the same integer decisions);
 * a row of zeros has scale 0 and codes 0. The quantized activation is
 * scale * code, which fp64 holds exactly.
 */
void qo_quant_i8_rows(const uint16_t* x, int64_t M, int64_t K, int8_t* q, float* scale) {
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* xr = x + m * K;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            const float v = fabsf((float)qo_f16_to_f64(xr[k]));
            if (v > amax) amax = v;
        }
        const float sc = amax / 127.0f;
        scale[m] = sc;
        for (int64_t k = 0; k < K; ++k) {
            const float v = (float)qo_f16_to_f64(xr[k]);
            q[m * K + k] = amax > 0.0f ? (int8_t)rintf(v / sc) : (int8_t)0;
        }
    }
}
