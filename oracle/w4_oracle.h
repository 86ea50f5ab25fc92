/*
 * w4_oracle.h -- plain, slow CPU oracle of the INT4 weight-quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it, to check and to time the HIP path.
 * It shares no source with the HIP library.
 *
 * Sources (web pages; cited by title and section):
 *   [KERAS]  "INT4 quantization in Keras" (Keras guide), section "How it works",
 *            steps 1-6, and "What Keras does in INT4 mode".
 *   [W4A16]  "INT4量化 / 4-bit Integer Quantization for LLMs", section
 *            "量化原理" (weight quantization formula; activations stay high precision).
 *   [ENCY]   "INT4" concept entry (compassingai), section 4.1 (uniform quantization
 *            formulas, symmetric and asymmetric scale), 4.2 (group quantization),
 *            4.5 (hardware execution schemes A and C).
 *   [BLOG]   hnwysp.cn INT4 article, section 2.1 (Q = round(clamp(v/s,-8,7))) and
 *            6.2 (scale = max|x| / 7).
 *
 * Every function returns 0 on success and a negative value when an input is
 * not finite (non-finite inputs are outside the method's domain) or when an
 * integer range assertion fails.
 *
 * Parity status of each function is stated in the test suite's pin tests:
 * every function below is pinned (brute force, closed forms, invariants or
 * hand-derived golden fixtures).
 */
#ifndef W4_ORACLE_H
#define W4_ORACLE_H
#include <stdint.h>

#define ORC_OK 0
#define ORC_ERR_NONFINITE (-1)
#define ORC_ERR_RANGE (-2)
#define ORC_ERR_ROUNDMODE (-3)
#define ORC_ERR_SHAPE (-4)

/* Symmetric per-output-channel int4 weight quantization and packing.
 * W is [K][N] fp32 row-major (Dense kernel orientation, N output channels).
 * Outputs: packed [N][(K+1)/2] bytes (k even -> low nibble), sw [N] fp32. */
int orc_quantize_weight_sym(const float *W, int64_t K, int64_t N,
                            uint8_t *packed, float *sw);

/* Unpack one signed code (two's complement nibble) from the packed layout. */
int orc_unpack_signed(const uint8_t *packed, int64_t K, int64_t n, int64_t k);

/* Per-row dynamic int8 activation quantization.
 * X is [M][K] fp32.  Outputs Xq [M][K] int8 and sx [M] fp32. */
int orc_quantize_act(const float *X, int64_t M, int64_t K, int8_t *Xq, float *sx);

/* acc[m][n] = sum_k Xq[m][k] * q[n][k]  (exact integer dot product). */
int orc_matmul_i32(const int8_t *Xq, const uint8_t *packed, int64_t M, int64_t K,
                   int64_t N, int32_t *acc);

/* y[m][n] = fl(fl(float(acc)) * fl(sx[m]*sw[n])), then fl(y + b[n]) if bias. */
int orc_dequant(const int32_t *acc, const float *sx, const float *sw,
                const float *bias, int64_t M, int64_t N, float *Y);

/* The whole W4A8 forward: quantize X per row, integer GEMM, dequant (+bias). */
int orc_w4a8_linear(const float *X, int64_t M, int64_t K, int64_t N,
                    const uint8_t *packed, const float *sw, const float *bias,
                    float *Y);

/* ReLU on a layer output, in place: y > 0 ? y : +0. */
int orc_relu(float *Y, int64_t n);

/* AWQ-style channel scales from calibration activations Xcal [M][K]:
 * s_k = 2^min(24, max(0, floor(alpha (E_k - E_med)))), E_k = floor(log2 max_m |x|),
 * alpha = alpha_num / alpha_den. */
int orc_awq_channel_scales(const float *Xcal, int64_t M, int64_t K, int alpha_num,
                           int alpha_den, float *s);

/* bf16 activations divided by s: Xout = bf16(fl(X / s_k)) (bit patterns). */
int orc_awq_scale_bf16(const uint16_t *X, int64_t M, int64_t K, const float *s, uint16_t *Xout);

/* Wout[k][n] = fl(W[k][n] * s[k]). */
int orc_awq_fold_weight(const float *W, int64_t K, int64_t N, const float *s, float *Wout);

/* Xq, sx = per-row int8 quantization of x' = fl(X / s) (s per column k). */
int orc_awq_quantize_act(const float *X, int64_t M, int64_t K, const float *s, int8_t *Xq,
                         float *sx);

/* The W4A8 forward on x' = X / s with weights quantized from W diag(s). */
int orc_w4a8_linear_awq(const float *X, int64_t M, int64_t K, int64_t N, const uint8_t *packed,
                        const float *sw, const float *s, const float *bias, float *Y);

/* Symmetric per-output-channel int8 weight quantization (scale = absmax/127,
 * codes in [-128, 127]).  Outputs Wq [N][K] int8 (channel-major), sw [N]. */
int orc_quantize_weight_w8(const float *W, int64_t K, int64_t N, int8_t *Wq, float *sw);

/* acc[m][n] = sum_k Xq[m][k] * Wq[n][k]  (exact integer dot product). */
int orc_matmul_w8_i32(const int8_t *Xq, const int8_t *Wq, int64_t M, int64_t K, int64_t N,
                      int32_t *acc);

/* The whole W8A8 forward: quantize X per row, integer GEMM, dequant (+bias). */
int orc_w8a8_linear(const float *X, int64_t M, int64_t K, int64_t N, const int8_t *Wq,
                    const float *sw, const float *bias, float *Y);

/* Asymmetric group-wise int4 quantization along K (codes 0..15).
 * Outputs packed [N][(K+1)/2], scales [N][K/g], zeros [N][K/g] (integer-valued). */
int orc_quantize_weight_asym(const float *W, int64_t K, int64_t N, int64_t group,
                             uint8_t *packed, float *scales, float *zeros);

/* Weight dequantization to fp32 W [K][N]: zeros == NULL -> symmetric codes,
 * w = fl(q * s[n]); else asymmetric groups, w = fl(fl(q - zp) * s). */
int orc_dequant_weight(const uint8_t *packed, const float *scales, const float *zeros,
                       int64_t K, int64_t N, int64_t group, float *W);

/* LoRA-style merge: requantize fl(dequant(packed) + delta) with the same scheme
 * (zeros == NULL: symmetric per channel; else asymmetric groups). */
int orc_merge_delta(const uint8_t *packed, const float *scales, const float *zeros,
                    int64_t K, int64_t N, int64_t group, const float *delta,
                    uint8_t *packed_out, float *scales_out, float *zeros_out);

/* GPU-shuffled W4A16 layout (group 128, K % 512 == 0, channels padded to a
 * multiple of 16): wpp [N16/16][K/128][16][64] bytes with 16-byte chunk p of
 * channel c holding canonical chunk p ^ ((c/2) % 4); szpp [N16/16][K/256][16][4]
 * fp32 = (scale, zero) of groups 2u and 2u+1. */
/* The weight part of that layout alone (K % 128 == 0), for any packed int4
 * codes (the W4A8 symmetric ones too), and its inverse. */
int orc_w4_prepack_weights(const uint8_t *packed, int64_t K, int64_t N, uint8_t *wpp);
int orc_w4_unprepack_weights(const uint8_t *wpp, int64_t K, int64_t N, uint8_t *packed);
int orc_w4a16_prepack(const uint8_t *packed, const float *scales, const float *zeros, int64_t K,
                      int64_t N, uint8_t *wpp, float *szpp);
int orc_w4a16_unprepack(const uint8_t *wpp, const float *szpp, int64_t K, int64_t N,
                        uint8_t *packed, float *scales, float *zeros);

/* fp32 -> bf16 round-half-to-even (bit pattern). */
uint16_t orc_bf16_rne(float f);

/* Dequantized bf16 weight w'[k][n] = bf16(fl(float(q - zp) * s)) (bit pattern). */
int orc_w4a16_dequant(const uint8_t *packed, const float *scales, const float *zeros,
                      int64_t K, int64_t N, int64_t group, uint16_t *Wd /* [K][N] */);

/* y[m][n] = sum_k x[m][k] * w'[k][n] evaluated in fp64 (products are exact);
 * absy[m][n] = sum_k |x[m][k] * w'[k][n]| (for the fp32 summation bound).
 * X is bf16 bits [M][K].  absy may be NULL. */
int orc_w4a16_linear(const uint16_t *X, int64_t M, int64_t K, int64_t N,
                     const uint8_t *packed, const float *scales, const float *zeros,
                     int64_t group, double *Y, double *absy);

#endif
