/*
 * CPU oracle for the affine-quantized decode path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may include, link
 * or call this code: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code with the HIP library.
 *
 * Everything is computed in fp64 from the plain definitions, with no
 * blocking, fusion or reordering:
 *   - weight format (TurboFieldfare article, "성능과 제약" / performance
 *     and constraints section): MLX affine quantization, 4-bit codes with
 *     one scale and one bias per group of 64 inputs, router at 8 bits;
 *     w = s*q + b;
 *   - GEMV: y[t][n] = sum over k ascending of w[n][k] * x[t][k];
 *   - routing (same article, top section and "내부 구조" / internals
 *     section: only the router's top-8 experts are used): softmax over
 *     all experts, keep the 8 largest, renormalize over those 8;
 *   - expert block (internals section: the shared-expert output and the
 *     routed output are combined): y = sum_j p_j * down_j(GELU(gate_j x)
 *     * up_j x) + down_s(GELU(gate_s x) * up_s x);
 *   - prefill chunk (internals section: prompts run in chunks of at most
 *     128 tokens): Y[m][n] = sum_k w[n][k] * X[m][k];
 *   - Mirai-M / Mirai-L weights (uzu page on discuss.pytorch.kr, section on
 *     model conversion and the Mirai quantization formats): 4-bit
 *     asymmetric with a zero point and a bf16 scale per group of 64, and
 *     8-bit symmetric.
 *
 * Readings where the pages are silent (nibble order LSB-first; separate
 * fp16 scale and bias arrays [N][K/64]; gate rows before up rows; exact
 * erf GELU by default; ties in the top-k broken towards the lower expert
 * index) are listed with the design notes.
 */
#ifndef QD_ORACLE_H
#define QD_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

double qo_f16_to_f64(uint16_t h);
double qo_bf16_to_f64(uint16_t h);
void qo_f16_array(const uint16_t* in, int64_t n, double* out);
void qo_bf16_array(const uint16_t* in, int64_t n, double* out);

/* Code k of one packed row: bits = 4 or 8; LSB-first inside each uint32. */
int qo_code(int bits, const uint32_t* row, int64_t k);

/* Dequantized matrix w[N][K] in fp64. */
void qo_dequant(int bits, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                int64_t N, int64_t K, double* w);

/* y[T][N] = W x for T activation rows x[T][K]; a[T][N] = sum_k |w*x| (may be NULL). */
void qo_gemv(int bits, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
             const double* x, int64_t T, int64_t N, int64_t K, double* y, double* a);

/* Same, for the listed output rows only: y[T][nrows], a[T][nrows]. */
void qo_gemv_rows(int bits, const uint32_t* wq, const uint16_t* s, const uint16_t* b,
                  const double* x, int64_t T, int64_t N, int64_t K,
                  const int64_t* rows, int64_t nrows, double* y, double* a);

/* Top-k routing of logits[T][E] -> idx[T][k], p[T][k]. Returns 0, or -1 on bad sizes. */
int qo_route_topk(const double* logits, int64_t T, int64_t E, int64_t k, int32_t* idx, double* p);

/* variant 0: exact erf form; 1: tanh approximation. */
double qo_gelu(double u, int variant);

typedef struct {
    int64_t E, H, I, Is;
    const uint32_t *gu_q, *dn_q, *sgu_q, *sdn_q;
    const uint16_t *gu_s, *gu_b, *dn_s, *dn_b, *sgu_s, *sgu_b, *sdn_s, *sdn_b;
} qo_moe;

/*
 * Expert block for T tokens: x[T][H] (fp64), idx/p [T][k].
 * Writes y[T][H] and a[T][H] = sum_j p_j sum_k |Wdn_j h_j| + sum_k |Wdn_s h_s|.
 * h[T][k][I] and hs[T][Is] receive the gated activations when non-NULL.
 */
void qo_moe_experts(const qo_moe* w, const double* x, int64_t T, int64_t k,
                    const int32_t* idx, const double* p, int act,
                    double* y, double* a, double* h, double* hs);

/*
 * Mirai formats (uzu page, quantization-format section): QO_MIRAI_M = 4-bit
 * codes q, bf16 scale s and 4-bit zero point z per group of 64,
 * w = s * (q - z), zp[N][ceil(K/512)] packed eight per word LSB-first;
 * QO_MIRAI_L = signed 8-bit codes, bf16 scale per group of 64, w = s * q
 * (zp unused, may be NULL).
 */
enum { QO_MIRAI_M = 1, QO_MIRAI_L = 2 };

void qo_mirai_dequant(int fmt, const uint32_t* wq, const uint16_t* s, const uint32_t* zp,
                      int64_t N, int64_t K, double* w);

/* y[T][m] and a[T][m] = sum_k |w x| for rows[0..nrows) (m = nrows), or all N rows
 * (m = N) when rows is NULL. */
void qo_mirai_gemv(int fmt, const uint32_t* wq, const uint16_t* s, const uint32_t* zp,
                   const double* x, int64_t T, int64_t N, int64_t K,
                   const int64_t* rows, int64_t nrows, double* y, double* a);

/*
 * Block-32 random Hadamard transform of x[K] (K % 32 == 0):
 * out[32b + i] = 2^-2.5 * sum_j (-1)^popcount(i & j) * d_j * x[32b + j], d_j = -1 where
 * bit j of signs[b] is set (signs NULL = all +1). out must not alias x.
 */
void qo_rht(const double* x, int64_t K, const uint32_t* signs, double* out);

/* RMSNorm: out = x / sqrt(mean(x^2) + eps) * gamma (gamma NULL = 1). */
void qo_rmsnorm(const double* x, int64_t K, const double* gamma, double eps, double* out);

/*
 * Decode attention for one token (TurboFieldfare article, internals section:
 * circular KV storage for sliding-window layers, linear for full attention,
 * exact decode attention). q [Hq][D]; k_new, v_new [Hkv][D]; kc, vc
 * [Hkv][cap][D] (read only: slot qo_attn_slot(pos, window) takes k_new /
 * v_new); window 0 = full attention (linear, pos < cap), else circular with
 * cap == window. out, a [Hq][D]: the attention output and sum_j p_j |v_j|.
 */
int64_t qo_attn_slot(int64_t pos, int64_t window);
void qo_attn_decode(const double* q, const double* k_new, const double* v_new,
                    const double* kc, const double* vc, int64_t Hq, int64_t Hkv, int64_t D,
                    int64_t cap, int64_t window, int64_t pos, double scale,
                    double* out, double* a);

/* Number of OpenMP threads the oracle uses (0 = runtime default). */
/* Per-token symmetric int8 quantization of fp16 activations [M][K]: codes
 * q [M][K] and scales [M] (scale = max|x| / 127, codes rounded to nearest
 * even, in fp32); the quantized activation is scale * q. */
void qo_quant_i8_rows(const uint16_t* x, int64_t M, int64_t K, int8_t* q, float* scale);

void qo_set_threads(int n);
int qo_get_threads(void);

#ifdef __cplusplus
}
#endif
#endif
