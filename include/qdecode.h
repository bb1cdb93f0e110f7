/*
 * libqdecode: affine-quantized decode contractions for AMD Instinct MI355X
 * (gfx950), as hand-written HIP kernels behind a plain C ABI.
 *
 * Sources for what each call computes:
 *   [TF]  jeff.news/article/5193, on TurboFieldfare (Gemma 4 26B-A4B on Apple
 *         Silicon): section "성능과 제약" (performance and constraints) fixes
 *         the weight format -- MLX affine quantization with 4-bit codes and
 *         a scale and a bias per group of 64 inputs, the router at 8 bits;
 *         section "내부 구조가 진짜 흥미로운 부분" (internals) describes the
 *         per-layer flow -- router on the GPU, top-8 expert IDs, a resident
 *         shared expert whose output is combined with the routed output, and
 *         prefill in chunks of at most 128 tokens.
 *   [uzu] fiv.co.kr/repos/uzu-deep-dive.html, sections 4-3 and 4-4 (tensors
 *         checked by shape and dtype; errors returned as values) and 7-1
 *         (a CPU reference matmul that rejects unsupported layouts).
 *   [Mirai] discuss.pytorch.kr/t/uzu-mac-iphone-llm-apple-silicon-rust/12363
 *         (uzu), section "uzu의 모델 변환과 Mirai 양자화 형식" (model
 *         conversion and the Mirai quantization formats): Mirai-M and
 *         Mirai-L, the two weight formats its checkpoints ship in; section
 *         "추측 디코딩 구조" (speculative decoding): drafted tokens verified
 *         in one forward pass.
 *
 * Data layout (all row-major, rows along the output dimension N):
 *   codes   uint32_t wq[N][K*bits/32]; code k of a row sits in word
 *           k/(32/bits) at bit offset bits*(k mod (32/bits)) (LSB first);
 *   scales  fp16 s[N][K/64], biases fp16 b[N][K/64] (raw uint16_t bits);
 *   weight  w[n][k] = s[n][k/64] * q[n][k] + b[n][k/64].
 *
 * Conventions shared by every call:
 *   - Every pointer is a DEVICE pointer (hipMalloc / torch CUDA tensor) that
 *     the caller owns. The library allocates, frees and copies nothing and
 *     never synchronizes; work is enqueued on `stream` (a hipStream_t; NULL
 *     selects the null stream) and is complete once that stream is.
 *   - Inputs must stay unmodified until the stream reaches the call;
 *     outputs must not overlap inputs or each other.
 *   - All arguments are checked before anything is launched. On an error
 *     nothing is written and the status says why; qd_last_error() gives a
 *     thread-local message. A launch failure returns QD_ERR_HIP.
 *   - Pointers must be 16-byte aligned; group_size must be 64; K must be a
 *     multiple of 64 and at most 4194304 (2^22; larger K returns
 *     QD_ERR_UNSUPPORTED: the kernels address a row in 32 bits).
 *   - The calls are stateless and may be issued from several threads.
 */
#ifndef QDECODE_H
#define QDECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QD_OK = 0,
    QD_ERR_INVALID_ARGUMENT = 1, /* null pointer, size out of range, K % 64 != 0 */
    QD_ERR_MISALIGNED = 2,       /* a pointer is not 16-byte aligned */
    QD_ERR_UNSUPPORTED = 3,      /* group_size != 64, dtype or shape not built */
    QD_ERR_WORKSPACE = 4,        /* workspace missing or too small */
    QD_ERR_HIP = 5               /* the HIP runtime reported an error */
} qd_status;

typedef enum { QD_F16 = 0, QD_BF16 = 1 } qd_dtype;

typedef enum { QD_GELU_ERF = 0, QD_GELU_TANH = 1 } qd_act;

typedef void* qd_stream; /* hipStream_t */

/*
 * y[t][n] = sum_k w[n][k] * x[t][k] for t < batch, with 4-bit codes.
 * [TF] performance section (4-bit affine weights, group 64).
 *   wq [N][K/8] uint32, scales/biases [N][K/64] fp16 bits,
 *   x  [batch][K] fp16 (QD_F16) or bf16 (QD_BF16) bits, y [batch][N] fp32.
 *   1 <= batch <= 8, N >= 1, K >= 64, K % 64 == 0, group_size == 64.
 */
qd_status qgemv_affine4(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                        const uint16_t* x, qd_dtype x_dtype, float* y,
                        int32_t N, int32_t K, int32_t batch, int32_t group_size,
                        qd_stream stream);

/*
 * The same contraction with 8-bit codes (the router of a MoE layer:
 * [TF] performance section, router at 8 bits; internals section, router
 * computed on the GPU from resident weights).
 *   wq [N][K/4] uint32; 1 <= batch <= 128 (prefill routers run a whole
 *   chunk of tokens); otherwise as qgemv_affine4.
 */
qd_status qgemv_affine8(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                        const uint16_t* x, qd_dtype x_dtype, float* y,
                        int32_t N, int32_t K, int32_t batch, int32_t group_size,
                        qd_stream stream);

/*
 * Mirai-M weights ([Mirai] quantization-format section: asymmetric 4-bit
 * codes with a 4-bit zero point and a bf16 scale per group of 64):
 *   y[t][n] = sum_k s[n][g] * (q[n][k] - z[n][g]) * x[t][k],  g = k / 64.
 *   wq     [N][K/8] uint32, codes packed as for qgemv_affine4;
 *   scales [N][K/64] bf16 bits;
 *   zeros  [N][ceil(K/512)] uint32: z[n][g] is nibble g mod 8 of word g/8 of
 *          row n (LSB-first); nibbles past the row's last group are ignored;
 *   x [batch][K] fp16 (QD_F16) or bf16 (QD_BF16) bits, y [batch][N] fp32;
 *   1 <= batch <= 8, K % 64 == 0, group_size == 64.
 */
qd_status qgemv_mirai_m(const uint32_t* wq, const uint16_t* scales, const uint32_t* zeros,
                        const uint16_t* x, qd_dtype x_dtype, float* y,
                        int32_t N, int32_t K, int32_t batch, int32_t group_size,
                        qd_stream stream);

/*
 * Mirai-L weights ([Mirai] quantization-format section: symmetric 8-bit):
 *   y[t][n] = sum_k s[n][g] * q[n][k] * x[t][k], q a two's-complement byte.
 *   wq [N][K/4] uint32, four signed codes per word, LSB-first;
 *   scales [N][K/64] bf16 bits (the scale type and group of the sibling
 *   format); otherwise as qgemv_mirai_m.
 */
qd_status qgemv_mirai_l(const uint32_t* wq, const uint16_t* scales,
                        const uint16_t* x, qd_dtype x_dtype, float* y,
                        int32_t N, int32_t K, int32_t batch, int32_t group_size,
                        qd_stream stream);

/*
 * Mirai GEMVs with the rotation prologue ([Mirai] quantization-format
 * section: both formats quantize after a random Hadamard transform of
 * block size 32, fused with RMSNorm and the matmul). For each t:
 *   u = gamma ? x_t / sqrt(mean_k(x_t[k]^2) + eps) * gamma : x_t,
 *   x'[32b + i] = 2^-2.5 * sum_j (-1)^popcount(i & j) * d_j * u[32b + j],
 *   y[t][n] = sum_k w[n][k] * x'[k]   (w as qgemv_mirai_m / qgemv_mirai_l),
 * with d_j = -1 where bit j of signs[b] is set.
 *   signs [K/32] uint32 (NULL = no sign flips), gamma [K] in x's dtype
 *   (NULL = no RMSNorm), eps finite and >= 0; the rest as the plain calls.
 * The rotated activations never leave the kernel: they are formed in fp32
 * and held as two fp16 parts with a per-vector power-of-two prescale.
 */
qd_status qgemv_mirai_m_rht(const uint32_t* wq, const uint16_t* scales, const uint32_t* zeros,
                            const uint32_t* signs, const uint16_t* gamma, float eps,
                            const uint16_t* x, qd_dtype x_dtype, float* y,
                            int32_t N, int32_t K, int32_t batch, int32_t group_size,
                            qd_stream stream);
qd_status qgemv_mirai_l_rht(const uint32_t* wq, const uint16_t* scales,
                            const uint32_t* signs, const uint16_t* gamma, float eps,
                            const uint16_t* x, qd_dtype x_dtype, float* y,
                            int32_t N, int32_t K, int32_t batch, int32_t group_size,
                            qd_stream stream);

/*
 * Top-k routing ([TF] top and internals sections: each token uses only the
 * router's top-8 experts). For each token t: idx[t][0..k) are the experts
 * with the k largest logits in descending order, equal logits going to the
 * lower expert index; weights[t][j] = softmax over all E logits, kept for
 * the k selected experts and renormalized to sum to one (equivalently
 * exp(l_j - l_max) / sum over the k kept of exp(l - l_max)).
 *   logits [T][E] fp32, idx [T][k] int32, weights [T][k] fp32.
 *   1 <= T, 1 <= E <= 1024, 1 <= k <= min(E, 32).
 */
qd_status qmoe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                          int32_t* idx, float* weights, qd_stream stream);

/*
 * One MoE FFN layer's experts ([TF] internals section): for each token t
 * and slot j with e = idx[t][j],
 *   z = W_gu[e] x_t (2I outputs: rows [0,I) gate, rows [I,2I) up),
 *   h = act(z[0:I]) * z[I:2I],  o_j = W_dn[e] h;
 * the shared expert gives o_s the same way, and
 *   y[t] = sum_j weights[t][j] * o_j + o_s.
 * All intermediates stay in fp32. Expert ids outside [0, E) contribute
 * nothing.
 *   gu_q [E][2I][H/8], gu_s/gu_b [E][2I][H/64];
 *   dn_q [E][H][I/8],  dn_s/dn_b [E][H][I/64];
 *   sgu_q [2Is][H/8], sgu_s/sgu_b [2Is][H/64];
 *   sdn_q [H][Is/8],  sdn_s/sdn_b [H][Is/64];
 *   H, I, Is multiples of 64; act selects exact-erf or tanh GELU.
 */
typedef struct {
    int32_t E, H, I, I_shared, group_size;
    qd_act act;
    const uint32_t *gu_q, *dn_q, *sgu_q, *sdn_q;
    const uint16_t *gu_s, *gu_b, *dn_s, *dn_b, *sgu_s, *sgu_b, *sdn_s, *sdn_b;
} qd_moe_weights;

/* Bytes of device workspace qmoe_expert_gemv needs for T tokens and k slots. */
size_t qmoe_expert_workspace_bytes(const qd_moe_weights* w, int32_t T, int32_t k);

/*
 *   idx/weights [T][k] (device, as produced by qmoe_route_topk),
 *   x [T][H] fp16 (QD_F16) or bf16 (QD_BF16) bits, y [T][H] fp32,
 *   workspace: device scratch of at least qmoe_expert_workspace_bytes();
 *   1 <= T <= 128 (a prefill chunk, [TF] internals), 1 <= k <= min(E, 32).
 * T == 1 runs the decode GEMV kernels; T > 1 groups the (token, slot)
 * pairs by expert so each selected expert's weights are read once.
 */
qd_status qmoe_expert_gemv(const qd_moe_weights* w, const int32_t* idx, const float* weights,
                           int32_t T, int32_t k, const void* x, qd_dtype x_dtype, float* y,
                           void* workspace, size_t ws_bytes, qd_stream stream);

/*
 * A whole decode MoE layer for one token ([TF] internals section: router on
 * the GPU, top-8 experts, routed plus shared experts combined):
 * logits = router GEMV (8-bit, as qgemv_affine8), idx / weights = top-k of
 * the logits (as qmoe_route_topk), y = the expert block (as
 * qmoe_expert_gemv with T = 1). Results are bit-identical to those three
 * calls; the ranking runs inside the gate+up kernel, so the layer takes
 * three launches instead of four.
 *   router_q [E][H/4] uint32, router_s / router_b [E][H/64] fp16 bits;
 *   x [H] fp16 or bf16 bits; outputs logits [E], idx [k], weights [k], y [H];
 *   E <= 256, 1 <= k <= min(E, 32); workspace as qmoe_expert_gemv with T = 1
 *   (qmoe_expert_workspace_bytes(w, 1, k) bytes, 16-byte aligned).
 * All buffers are device memory owned by the caller; every output is
 * overwritten. Errors as qmoe_expert_gemv; E > 256 gives QD_ERR_UNSUPPORTED.
 */
qd_status qmoe_layer_decode(const qd_moe_weights* w, const uint32_t* router_q,
                            const uint16_t* router_s, const uint16_t* router_b, int32_t k,
                            const void* x, qd_dtype x_dtype, float* logits, int32_t* idx,
                            float* weights, float* y, void* workspace, size_t ws_bytes,
                            qd_stream stream);

/*
 * qmoe_layer_decode without a workspace argument, for callers that cannot
 * allocate device memory around the call: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation. The gate+up
 * activations (k * I + I_shared floats) go to a scratch array inside the
 * library instead, 4 MiB per device, held by every device the library runs
 * on until the process ends; a layer needing more is rejected with
 * QD_ERR_WORKSPACE before any launch. The call allocates nothing. All calls
 * on one device share that scratch, so calls that may overlap on a device
 * (other streams, other threads) race and must be serialized by the caller.
 * Arguments, outputs and results are those of qmoe_layer_decode, bit for bit.
 */
qd_status qmoe_layer_decode_noalloc(const qd_moe_weights* w, const uint32_t* router_q,
                                    const uint16_t* router_s, const uint16_t* router_b, int32_t k,
                                    const void* x, qd_dtype x_dtype, float* logits, int32_t* idx,
                                    float* weights, float* y, qd_stream stream);

/*
 * One MoE layer over a prefill chunk of T tokens ([TF] internals: a chunk of
 * up to 128 tokens goes through the router at once, and each token's top-8
 * experts and the shared expert are combined): the 8-bit router over the
 * chunk (as qgemv_affine8, router [E][H], E <= 1024), top-k routing (as
 * qmoe_route_topk), then the expert block (as qmoe_expert_gemv). The router
 * splits H across workgroups (128 tokens x 128 experts are only 16 tiles of
 * 32 x 32); its partial logits go to the workspace and the routing adds them
 * in a fixed order, so results do not depend on timing (the logits may differ
 * from a separate qgemv_affine8 call by that summation order).
 *   x [T][H] fp16 or bf16 bits; logits [T][E], idx [T][k], weights [T][k]
 *   and y [T][H] are outputs; 1 <= T <= 128, 1 <= k <= min(E, 32).
 *   workspace: 16-byte aligned device memory of at least
 *   qmoe_layer_prefill_workspace_bytes(w, T, k) bytes (0 for arguments out
 *   of range), overwritten by every call; NULL or too small fails with
 *   QD_ERR_WORKSPACE before any launch.
 * Launches on `stream`: the router, the routing, then the expert block's.
 */
size_t qmoe_layer_prefill_workspace_bytes(const qd_moe_weights* w, int32_t T, int32_t k);
qd_status qmoe_layer_prefill(const qd_moe_weights* w, const uint32_t* router_q,
                             const uint16_t* router_s, const uint16_t* router_b, int32_t k, int32_t T,
                             const void* x, qd_dtype x_dtype, float* logits, int32_t* idx,
                             float* weights, float* y, void* workspace, size_t ws_bytes,
                             qd_stream stream);

/*
 * Prefill chunk ([TF] internals: prompts run in chunks of at most 128 tokens
 * so one fetch of a weight serves many rows):
 *   Y[m][n] = sum_k w[n][k] * X[m][k],  X [M][K] bf16 bits, Y [M][N] fp32.
 *   1 <= M <= 128; 4-bit codes as qgemv_affine4. Runs on bf16 MFMA with the
 *   exact integer codes as the matrix operand and the scales and biases
 *   applied per group in fp32.
 *   workspace: as for qgemm_affine4_verify (same kernel, same split plan):
 *   shapes with few 64-column tiles, such as a down projection, split K
 *   across workgroups and need at least
 *   qgemm_affine4_chunk_workspace_bytes(M, N, K) bytes (16-byte aligned) for
 *   their fp32 partial results, which a second launch adds in split order;
 *   0 bytes (workspace may be NULL) for shapes that run unsplit. NULL or too
 *   small otherwise fails with QD_ERR_WORKSPACE before any launch.
 */
size_t qgemm_affine4_chunk_workspace_bytes(int32_t M, int32_t N, int32_t K);
qd_status qgemm_affine4_chunk(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                              const uint16_t* x, float* y,
                              int32_t M, int32_t N, int32_t K, int32_t group_size,
                              void* workspace, size_t ws_bytes, qd_stream stream);

/*
 * Verification GEMM ([Mirai] speculative-decoding section: the target model
 * checks 16 to 32 drafted tokens in one forward pass, so its projections
 * become GEMMs over a few dozen tokens):
 *   Y[m][n] = sum_k w[n][k] * X[m][k],  X [M][K] fp16 (QD_F16) or bf16
 *   (QD_BF16) bits, Y [M][N] fp32, 1 <= M <= 128; 4-bit codes, scales and
 *   biases as qgemv_affine4. Runs on fp16 / bf16 MFMA with the exact integer
 *   codes as the matrix operand and the scales and biases applied per group
 *   in fp32; built for the 9..64-token range between the GEMV kernels and a
 *   prefill chunk.
 *   workspace: shapes with few 64-column tiles (a short N such as a down
 *   projection) split K across workgroups; their fp32 partial results go to
 *   the workspace, 16-byte aligned, of at least
 *   qgemm_affine4_verify_workspace_bytes(M, N, K) bytes, and a second launch
 *   adds them in a fixed order. That size is 0 for shapes that run unsplit
 *   (and for arguments out of range); then workspace may be NULL. Otherwise
 *   NULL or too small fails with QD_ERR_WORKSPACE before any launch. The
 *   split depends on (M, N, K) only, so results do not depend on timing;
 *   calls that share a workspace must be ordered on a stream.
 */
size_t qgemm_affine4_verify_workspace_bytes(int32_t M, int32_t N, int32_t K);
qd_status qgemm_affine4_verify(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                               const uint16_t* x, qd_dtype x_dtype, float* y,
                               int32_t M, int32_t N, int32_t K, int32_t group_size,
                               void* workspace, size_t ws_bytes, qd_stream stream);

/*
 * Verification GEMM on int8 activations (uzu page on discuss.pytorch.kr,
 * section on speculative decoding: the target model checks 16 to 32 drafted
 * tokens in one pass on the chip's int8 matrix path, quantizing its
 * activations to 8 bits as it goes). The page leaves the scheme open; this
 * call takes it per token and symmetric, in fp32:
 *   sx[m] = max_k |X[m][k]| / 127 (correctly rounded division),
 *   xq[m][k] = X[m][k] / sx[m] rounded to the nearest integer, ties to even
 *   (0 throughout a row of zeros, whose sx is 0),
 *   Y[m][n] = sx[m] * sum_k w[n][k] * xq[m][k],
 * with w[n][k] = s q + b from 4-bit codes, scales and biases as
 * qgemv_affine4. X [M][K] fp16 bits, Y [M][N] fp32, 1 <= M <= 32.
 *   workspace: device memory, 16-byte aligned, of at least
 *   qgemm_affine4_verify_i8_workspace_bytes(M, K) bytes (0 for arguments
 *   out of range); it receives the quantized activations, their per-group
 *   sums and the scales, and is overwritten by every call, so calls that
 *   share one must be ordered on a stream. NULL or too small fails with
 *   QD_ERR_WORKSPACE before any launch.
 * Two launches on `stream` (quantization, then the GEMM); results do not
 * depend on timing.
 */
size_t qgemm_affine4_verify_i8_workspace_bytes(int32_t M, int32_t K);
qd_status qgemm_affine4_verify_i8(const uint32_t* wq, const uint16_t* scales, const uint16_t* biases,
                                  const uint16_t* x, float* y, int32_t M, int32_t N, int32_t K,
                                  int32_t group_size, void* workspace, size_t ws_bytes,
                                  qd_stream stream);

/*
 * Decode attention for one new token ([TF] internals section: sliding-window
 * layers keep keys and values in bounded circular storage, full-attention
 * layers in linear storage, and decode attention is exact).
 *   q [Hq][D], k_new / v_new [Hkv][D]: fp16 bits of the token's query, key
 *   and value (already normed and rotated as the model requires);
 *   k_cache / v_cache [Hkv][cap][D] fp16 bits, read and updated in place:
 *   the token at position pos is stored at slot pos mod window when
 *   window > 0 (circular storage, window == cap) or at slot pos when
 *   window == 0 (linear storage, pos < cap);
 *   out [Hq][D] fp32: for query head h and its key/value head
 *   hk = h / (Hq / Hkv),  out[h] = sum_j softmax_j(scale q_h . k_j) v_j over
 *   the occupied slots j < min(pos + 1, window) (or pos + 1): exactly the
 *   positions inside the window.
 *   D in {64, 128, 256}; Hq / Hkv in {1, 2, 4, 8}; scale finite.
 *   workspace: device scratch of at least qattn_decode_workspace_bytes(Hq,
 *   Hkv, D, cap); that size covers every pos the cache can hold. A call
 *   whose split partials would not fit ws_bytes fails with
 *   QD_ERR_WORKSPACE before any launch (nothing is written).
 * The call first stores k_new / v_new at the token's slot, so the caches
 * must not be read or written by other work until the stream reaches it.
 */
size_t qattn_decode_workspace_bytes(int32_t Hq, int32_t Hkv, int32_t D, int32_t cap);
qd_status qattn_decode(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                       uint16_t* k_cache, uint16_t* v_cache,
                       int32_t Hq, int32_t Hkv, int32_t D, int32_t cap, int32_t window,
                       int32_t pos, float scale, float* out,
                       void* workspace, size_t ws_bytes, qd_stream stream);

/*
 * Measurement: reads `bytes` bytes of device memory at buf once, as the
 * GEMV reads its codes (16-byte buffer loads per lane, waves sweeping the
 * buffer in the GEMV's interleaved order), and does nothing
 * else. Its rate over buffers of a workload's size is the practical HBM read
 * ceiling that the GEMV's achieved bandwidth is compared against. sink (4
 * bytes of device memory, 16-byte aligned) is written (with 0x9E3779B9) only
 * when the XOR of the words one lane loaded equals 0x9E3779B9.
 * Asynchronous on stream.
 */
qd_status qd_stream_read(const void* buf, size_t bytes, uint32_t* sink, qd_stream stream);

/* Human-readable name of a status. */
const char* qd_status_string(qd_status status);

/* Detail of the last error raised on the calling thread ("" if none). */
const char* qd_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* QDECODE_H */
