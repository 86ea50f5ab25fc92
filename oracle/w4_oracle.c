/*
 * w4_oracle.c -- plain, slow CPU oracle of the INT4 weight-quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the product path.  It shares no code
 * with the HIP library.  Build: gcc -O2 -ffp-contract=off (no fast-math), so
 * every float operation below is one IEEE-754 binary32 operation rounded to
 * nearest-even, in the order written.
 *
 * Each function follows the formula of the page it cites, one step per line,
 * with no blocking, fusion or reordering.
 */
#include "w4_oracle.h"

#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static int round_mode_ok(void) { return fegetround() == FE_TONEAREST; }

/* Round to the nearest integer, ties to even (the current mode is checked to
 * be round-to-nearest before any call). */
static float rne(float v) { return nearbyintf(v); }

static float clampf(float v, float lo, float hi) {
    if (v < lo) return lo;
    if (v > hi) return hi;
    return v;
}

/* [KERAS] "How it works", step 1: a symmetric absmax scale per output channel;
 * [ENCY] 4.1: symmetric scale = max|x| / (2^(b-1) - 1), i.e. / 7 for b = 4;
 * [BLOG] 6.2: scale = max_val / 7.0.
 * [KERAS] step 2 and [BLOG] 2.1: codes are round(v/s) limited to [-8, 7], two
 * codes per byte.  Packing layout (the pages fix none): column n owns bytes
 * packed[n*ceil(K/2) .. ], byte j holds k = 2j in bits 0-3 and k = 2j+1 in
 * bits 4-7, as two's complement nibbles; a missing last high nibble is 0. */
int orc_quantize_weight_sym(const float *W, int64_t K, int64_t N,
                            uint8_t *packed, float *sw) {
    if (K < 1 || N < 1) return ORC_ERR_SHAPE;
    if (!round_mode_ok()) return ORC_ERR_ROUNDMODE;
    const int64_t KB = (K + 1) / 2;
    for (int64_t n = 0; n < N; ++n) {
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float w = W[k * N + n];
            if (!isfinite(w)) return ORC_ERR_NONFINITE;
            float aw = fabsf(w);
            if (aw > a) a = aw;
        }
        float s = (a == 0.0f) ? 0.0f : a / 7.0f;
        sw[n] = s;
        uint8_t *row = packed + n * KB;
        memset(row, 0, (size_t)KB);
        for (int64_t k = 0; k < K; ++k) {
            int q = 0;
            if (s != 0.0f) {
                float t = W[k * N + n] / s;
                float r = clampf(rne(t), -8.0f, 7.0f);
                q = (int)r;
            }
            uint8_t nib = (uint8_t)(q & 0xF);
            if (k % 2 == 0)
                row[k / 2] |= nib;
            else
                row[k / 2] |= (uint8_t)(nib << 4);
        }
    }
    return ORC_OK;
}

/* Inverse of the packing above ([KERAS] step 4: the packed int4 weights are
 * unpacked to int8 values that stay in the int4 range): nibble >= 8 means
 * nibble - 16. */
int orc_unpack_signed(const uint8_t *packed, int64_t K, int64_t n, int64_t k) {
    const int64_t KB = (K + 1) / 2;
    uint8_t b = packed[n * KB + k / 2];
    int nib = (k % 2 == 0) ? (b & 0xF) : (b >> 4);
    return nib >= 8 ? nib - 16 : nib;
}

static int unpack_unsigned(const uint8_t *packed, int64_t K, int64_t n, int64_t k) {
    const int64_t KB = (K + 1) / 2;
    uint8_t b = packed[n * KB + k / 2];
    return (k % 2 == 0) ? (b & 0xF) : (b >> 4);
}

/* [KERAS] step 3 and "What Keras does": activations are scaled by a dynamic
 * absmax computed at run time and quantized to INT8.  Scale granularity: one
 * per row (per token).  [ENCY] 4.1 with b = 8: scale = max|x| / 127; the int8
 * range is [-128, 127] (INT4-vs-INT8 comparison article, 2.1). */
int orc_quantize_act(const float *X, int64_t M, int64_t K, int8_t *Xq, float *sx) {
    if (M < 1 || K < 1) return ORC_ERR_SHAPE;
    if (!round_mode_ok()) return ORC_ERR_ROUNDMODE;
    for (int64_t m = 0; m < M; ++m) {
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float x = X[m * K + k];
            if (!isfinite(x)) return ORC_ERR_NONFINITE;
            float ax = fabsf(x);
            if (ax > a) a = ax;
        }
        float s = (a == 0.0f) ? 0.0f : a / 127.0f;
        sx[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            int q = 0;
            if (s != 0.0f) {
                float t = X[m * K + k] / s;
                float r = clampf(rne(t), -128.0f, 127.0f);
                q = (int)r;
            }
            Xq[m * K + k] = (int8_t)q;
        }
    }
    return ORC_OK;
}

/* [KERAS] step 5: INT8 x INT8 matrix multiplication accumulated in INT32.
 * Summed in int64 and checked to fit int32. */
int orc_matmul_i32(const int8_t *Xq, const uint8_t *packed, int64_t M, int64_t K,
                   int64_t N, int32_t *acc) {
    if (M < 1 || K < 1 || N < 1) return ORC_ERR_SHAPE;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)Xq[m * K + k] * (int64_t)orc_unpack_signed(packed, K, n, k);
            if (s > INT32_MAX || s < INT32_MIN) return ORC_ERR_RANGE;
            acc[m * N + n] = (int32_t)s;
        }
    }
    return ORC_OK;
}

/* [KERAS] step 6: the result is dequantized with (input_scale *
 * per_channel_kernel_scale): the parenthesised product first, then one
 * multiply with the accumulator; the Dense bias is added afterwards. */
int orc_dequant(const int32_t *acc, const float *sx, const float *sw,
                const float *bias, int64_t M, int64_t N, float *Y) {
    if (M < 1 || N < 1) return ORC_ERR_SHAPE;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            float s = sx[m] * sw[n];
            float a = (float)acc[m * N + n];
            float y = a * s;
            if (bias) y = y + bias[n];
            Y[m * N + n] = y;
        }
    }
    return ORC_OK;
}

int orc_w4a8_linear(const float *X, int64_t M, int64_t K, int64_t N,
                    const uint8_t *packed, const float *sw, const float *bias,
                    float *Y) {
    if (M < 1 || K < 1 || N < 1) return ORC_ERR_SHAPE;
    int8_t *Xq = (int8_t *)malloc((size_t)(M * K));
    float *sx = (float *)malloc((size_t)M * sizeof(float));
    int32_t *acc = (int32_t *)malloc((size_t)(M * N) * sizeof(int32_t));
    int rc = ORC_ERR_SHAPE;
    if (Xq && sx && acc) {
        rc = orc_quantize_act(X, M, K, Xq, sx);
        if (rc == ORC_OK) rc = orc_matmul_i32(Xq, packed, M, K, N, acc);
        if (rc == ORC_OK) rc = orc_dequant(acc, sx, sw, bias, M, N, Y);
    }
    free(Xq);
    free(sx);
    free(acc);
    return rc;
}

/* [KERAS] toy model (section "Quantize a minimal functional model"): the first
 * Dense layer carries activation="relu", applied to the layer output after the
 * bias: y = y if y > 0 else +0 (so -0 becomes +0). */
int orc_relu(float *Y, int64_t n) {
    if (n < 0) return ORC_ERR_SHAPE;
    for (int64_t i = 0; i < n; ++i) {
        float y = Y[i];
        if (!isfinite(y)) return ORC_ERR_NONFINITE;
        Y[i] = (y > 0.0f) ? y : 0.0f;
    }
    return ORC_OK;
}

/* [ENCY] 4.4 (AWQ's core idea): on calibration data, measure the activation
 * magnitude of every input channel; scale up the weights of the important
 * channels, W' = W diag(s), quantize W', and at inference divide the
 * activations by s before quantizing them.  The page fixes neither the
 * magnitude statistic nor the rule from magnitude to s; this oracle takes:
 *   a_k = max_m |Xcal[m][k]|                      (magnitude of channel k),
 *   E_k = floor(log2 a_k)  (E_k = -150 for a_k = 0, below every finite value),
 *   E_med = the lower median of E_k over the K channels,
 *   s_k = 2^e_k, e_k = min(24, max(0, floor(alpha * (E_k - E_med)))),
 * alpha = alpha_num / alpha_den (1/2 by default in the library): a fraction of
 * the log-magnitude excess over the median, as a power of two, so that W * s
 * and x / s are exact in fp32 and bf16. */
static int cmp_int(const void *a, const void *b) {
    const int x = *(const int *)a, y = *(const int *)b;
    return (x > y) - (x < y);
}

int orc_awq_channel_scales(const float *Xcal, int64_t M, int64_t K, int alpha_num,
                           int alpha_den, float *s) {
    if (M < 1 || K < 1 || alpha_num < 0 || alpha_den < 1) return ORC_ERR_SHAPE;
    int *E = (int *)malloc((size_t)K * sizeof(int));
    int *sorted = (int *)malloc((size_t)K * sizeof(int));
    if (!E || !sorted) {
        free(E);
        free(sorted);
        return ORC_ERR_SHAPE;
    }
    int rc = ORC_OK;
    for (int64_t k = 0; k < K && rc == ORC_OK; ++k) {
        float a = 0.0f;
        for (int64_t m = 0; m < M; ++m) {
            float x = Xcal[m * K + k];
            if (!isfinite(x)) {
                rc = ORC_ERR_NONFINITE;
                break;
            }
            if (fabsf(x) > a) a = fabsf(x);
        }
        int ex = 0;
        if (a == 0.0f) {
            E[k] = -150;
        } else {
            frexpf(a, &ex); /* a = f * 2^ex with f in [0.5, 1) */
            E[k] = ex - 1;
        }
        sorted[k] = E[k];
    }
    if (rc == ORC_OK) {
        qsort(sorted, (size_t)K, sizeof(int), cmp_int);
        const int med = sorted[(K - 1) / 2];
        for (int64_t k = 0; k < K; ++k) {
            int d = E[k] - med;
            int e = d > 0 ? (d * alpha_num) / alpha_den : 0;
            if (e > 24) e = 24;
            s[k] = ldexpf(1.0f, e);
        }
    }
    free(E);
    free(sorted);
    return rc;
}

/* W' = W diag(s): row k of W [K][N] times s_k, one rounding each. */
int orc_awq_fold_weight(const float *W, int64_t K, int64_t N, const float *s, float *Wout) {
    if (K < 1 || N < 1) return ORC_ERR_SHAPE;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) Wout[k * N + n] = W[k * N + n] * s[k];
    return ORC_OK;
}

/* Activation side: x' = fl(x / s_k), then [KERAS] step 3 on x'. */
int orc_awq_quantize_act(const float *X, int64_t M, int64_t K, const float *s, int8_t *Xq,
                         float *sx) {
    if (M < 1 || K < 1) return ORC_ERR_SHAPE;
    float *Xs = (float *)malloc((size_t)(M * K) * sizeof(float));
    if (!Xs) return ORC_ERR_SHAPE;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) Xs[m * K + k] = X[m * K + k] / s[k];
    int rc = orc_quantize_act(Xs, M, K, Xq, sx);
    free(Xs);
    return rc;
}

/* bf16 activations for the weight-only path: x' = bf16(fl(x / s_k)) (exact
 * when s_k is a power of two). */
int orc_awq_scale_bf16(const uint16_t *X, int64_t M, int64_t K, const float *s, uint16_t *Xout) {
    if (M < 1 || K < 1) return ORC_ERR_SHAPE;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            uint32_t u = (uint32_t)X[m * K + k] << 16;
            float x;
            memcpy(&x, &u, 4);
            Xout[m * K + k] = orc_bf16_rne(x / s[k]);
        }
    return ORC_OK;
}

/* The W4A8 forward with AWQ scaling: packed / sw quantize W diag(s). */
int orc_w4a8_linear_awq(const float *X, int64_t M, int64_t K, int64_t N, const uint8_t *packed,
                        const float *sw, const float *s, const float *bias, float *Y) {
    if (M < 1 || K < 1 || N < 1) return ORC_ERR_SHAPE;
    int8_t *Xq = (int8_t *)malloc((size_t)(M * K));
    float *sx = (float *)malloc((size_t)M * sizeof(float));
    int32_t *acc = (int32_t *)malloc((size_t)(M * N) * sizeof(int32_t));
    int rc = ORC_ERR_SHAPE;
    if (Xq && sx && acc) {
        rc = orc_awq_quantize_act(X, M, K, s, Xq, sx);
        if (rc == ORC_OK) rc = orc_matmul_i32(Xq, packed, M, K, N, acc);
        if (rc == ORC_OK) rc = orc_dequant(acc, sx, sw, bias, M, N, Y);
    }
    free(Xq);
    free(sx);
    free(acc);
    return rc;
}

/* W8A8, the INT8 path that [KERAS] "How it works" says the INT4 path follows
 * apart from the unpacking: steps 1-6 with 8-bit weight codes.  [ENCY] 4.1
 * with b = 8: symmetric scale = max|x| / (2^(b-1) - 1) = / 127 per output
 * channel; codes are round(W/scale) limited to the int8 range [-128, 127]
 * (INT4-vs-INT8 comparison article, 2.1).  The codes are stored one per byte
 * as int8, channel-major: Wq[n*K + k]. */
int orc_quantize_weight_w8(const float *W, int64_t K, int64_t N, int8_t *Wq, float *sw) {
    if (K < 1 || N < 1) return ORC_ERR_SHAPE;
    if (!round_mode_ok()) return ORC_ERR_ROUNDMODE;
    for (int64_t n = 0; n < N; ++n) {
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float w = W[k * N + n];
            if (!isfinite(w)) return ORC_ERR_NONFINITE;
            float aw = fabsf(w);
            if (aw > a) a = aw;
        }
        float s = (a == 0.0f) ? 0.0f : a / 127.0f;
        sw[n] = s;
        for (int64_t k = 0; k < K; ++k) {
            int q = 0;
            if (s != 0.0f) {
                float t = W[k * N + n] / s;
                float r = clampf(rne(t), -128.0f, 127.0f);
                q = (int)r;
            }
            Wq[n * K + k] = (int8_t)q;
        }
    }
    return ORC_OK;
}

/* [KERAS] step 5 for 8-bit weights: acc[m][n] = sum_k Xq[m][k] * Wq[n][k],
 * summed in int64 and checked to fit int32. */
int orc_matmul_w8_i32(const int8_t *Xq, const int8_t *Wq, int64_t M, int64_t K, int64_t N,
                      int32_t *acc) {
    if (M < 1 || K < 1 || N < 1) return ORC_ERR_SHAPE;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)Xq[m * K + k] * (int64_t)Wq[n * K + k];
            if (s > INT32_MAX || s < INT32_MIN) return ORC_ERR_RANGE;
            acc[m * N + n] = (int32_t)s;
        }
    }
    return ORC_OK;
}

/* The whole W8A8 forward: steps 3, 5 and 6 as in orc_w4a8_linear. */
int orc_w8a8_linear(const float *X, int64_t M, int64_t K, int64_t N, const int8_t *Wq,
                    const float *sw, const float *bias, float *Y) {
    if (M < 1 || K < 1 || N < 1) return ORC_ERR_SHAPE;
    int8_t *Xq = (int8_t *)malloc((size_t)(M * K));
    float *sx = (float *)malloc((size_t)M * sizeof(float));
    int32_t *acc = (int32_t *)malloc((size_t)(M * N) * sizeof(int32_t));
    int rc = ORC_ERR_SHAPE;
    if (Xq && sx && acc) {
        rc = orc_quantize_act(X, M, K, Xq, sx);
        if (rc == ORC_OK) rc = orc_matmul_w8_i32(Xq, Wq, M, K, N, acc);
        if (rc == ORC_OK) rc = orc_dequant(acc, sx, sw, bias, M, N, Y);
    }
    free(Xq);
    free(sx);
    free(acc);
    return rc;
}

/* [W4A16] "量化原理": W_int = round(W/scale + zero_point), dequantized as
 * (W_int - zero_point) * scale, codes 0..15.  [ENCY] 4.1: asymmetric scale =
 * (x_max - x_min) / (2^b - 1) = / 15, x_q = round(x/scale) + zero_point.
 * [ENCY] 4.2: groups of group_size weights, each with its own scale and zero
 * point (32 bits each).  Groups run along K inside one output channel.
 * zero_point = 0 - round(x_min/scale) (integer-valued, stored as fp32, never
 * -0.0, not clamped); the code adds it after rounding.  A group with x_max == x_min uses
 * scale |x_min| (1 if zero), which reconstructs the group exactly. */
int orc_quantize_weight_asym(const float *W, int64_t K, int64_t N, int64_t group,
                             uint8_t *packed, float *scales, float *zeros) {
    if (K < 1 || N < 1 || group < 1 || K % group != 0) return ORC_ERR_SHAPE;
    if (!round_mode_ok()) return ORC_ERR_ROUNDMODE;
    const int64_t KB = (K + 1) / 2;
    const int64_t G = K / group;
    for (int64_t n = 0; n < N; ++n) {
        uint8_t *row = packed + n * KB;
        memset(row, 0, (size_t)KB);
        for (int64_t g = 0; g < G; ++g) {
            float lo = W[(g * group) * N + n], hi = lo;
            for (int64_t k = g * group; k < (g + 1) * group; ++k) {
                float w = W[k * N + n];
                if (!isfinite(w)) return ORC_ERR_NONFINITE;
                if (w < lo) lo = w;
                if (w > hi) hi = w;
            }
            float s;
            if (hi > lo) {
                float range = hi - lo;
                s = range / 15.0f;
            } else {
                s = (lo != 0.0f) ? fabsf(lo) : 1.0f;
            }
            if (!isfinite(s) || s == 0.0f) return ORC_ERR_RANGE;
            float zp = 0.0f - rne(lo / s); /* +0.0 when the rounded value is 0 */
            scales[n * G + g] = s;
            zeros[n * G + g] = zp;
            for (int64_t k = g * group; k < (g + 1) * group; ++k) {
                float t = W[k * N + n] / s;
                float r = rne(t) + zp;
                int q = (int)clampf(r, 0.0f, 15.0f);
                uint8_t nib = (uint8_t)q;
                if (k % 2 == 0)
                    row[k / 2] |= nib;
                else
                    row[k / 2] |= (uint8_t)(nib << 4);
            }
        }
    }
    return ORC_OK;
}

/* [KERAS] "Limitations": the LoRA export path dequantizes the weights, adds
 * the delta and requantizes.  Weight dequantization follows the dequant
 * formulas of the pages: symmetric codes ([KERAS] step 6 applied to the
 * kernel, [BLOG] 6.2): w = fl(q * s); asymmetric groups ([W4A16] "量化原理"):
 * w = fl(fl(q - zp) * s).  Output W [K][N] fp32. */
int orc_dequant_weight(const uint8_t *packed, const float *scales, const float *zeros,
                       int64_t K, int64_t N, int64_t group, float *W) {
    if (K < 1 || N < 1) return ORC_ERR_SHAPE;
    if (zeros && (group < 1 || K % group != 0)) return ORC_ERR_SHAPE;
    for (int64_t k = 0; k < K; ++k) {
        for (int64_t n = 0; n < N; ++n) {
            float w;
            if (zeros) {
                const int64_t G = K / group;
                int q = unpack_unsigned(packed, K, n, k);
                float d = (float)q - zeros[n * G + k / group];
                w = d * scales[n * G + k / group];
            } else {
                int q = orc_unpack_signed(packed, K, n, k);
                w = (float)q * scales[n];
            }
            W[k * N + n] = w;
        }
    }
    return ORC_OK;
}

/* The merge itself: W' = fl(dequant(packed) + delta), then the scheme's
 * quantization of W' (new codes, scales and zero points). */
int orc_merge_delta(const uint8_t *packed, const float *scales, const float *zeros,
                    int64_t K, int64_t N, int64_t group, const float *delta,
                    uint8_t *packed_out, float *scales_out, float *zeros_out) {
    if (K < 1 || N < 1) return ORC_ERR_SHAPE;
    float *W = (float *)malloc((size_t)(K * N) * sizeof(float));
    if (!W) return ORC_ERR_SHAPE;
    int rc = orc_dequant_weight(packed, scales, zeros, K, N, group, W);
    if (rc == ORC_OK) {
        for (int64_t i = 0; i < K * N; ++i) W[i] = W[i] + delta[i];
        if (zeros)
            rc = orc_quantize_weight_asym(W, K, N, group, packed_out, scales_out, zeros_out);
        else
            rc = orc_quantize_weight_sym(W, K, N, packed_out, scales_out);
    }
    free(W);
    return rc;
}

/* A second, GPU-shuffled layout of the W4A16 weights (a "prepacked"
 * format of this library; the pages define none, they only pack two codes per
 * byte).  It is a pure rearrangement of the canonical packed bytes and group
 * tables, defined for group 128, K % 512 == 0; channels are padded to
 * N16 = 16 * ceil(N / 16) with zero bytes / zero table entries:
 *   wpp [N16/16][K/128][16][64] bytes:
 *     wpp[b][t][c][16 p + i] = packed[16 b + c][64 t + 16 (p ^ ((c / 2) % 4)) + i]
 *   szpp [N16/16][K/256][16][4] fp32:
 *     szpp[b][u][c] = { scales[n][2u], zeros[n][2u], scales[n][2u+1], zeros[n][2u+1] },
 *     n = 16 b + c.
 * orc_w4a16_unprepack is the inverse on the first N channels. */
/* The weight part alone (also used for the W4A8 symmetric codes), defined
 * for K % 128 == 0. */
int orc_w4_prepack_weights(const uint8_t *packed, int64_t K, int64_t N, uint8_t *wpp) {
    if (K < 1 || N < 1 || K % 128 != 0) return ORC_ERR_SHAPE;
    const int64_t KB = K / 2, S = K / 128, NB = (N + 15) / 16;
    for (int64_t b = 0; b < NB; ++b)
        for (int64_t t = 0; t < S; ++t)
            for (int64_t c = 0; c < 16; ++c) {
                const int64_t n = 16 * b + c;
                for (int64_t p = 0; p < 4; ++p)
                    for (int64_t i = 0; i < 16; ++i) {
                        const int64_t chunk = p ^ ((c / 2) % 4);
                        uint8_t v = 0;
                        if (n < N) v = packed[n * KB + 64 * t + 16 * chunk + i];
                        wpp[((b * S + t) * 16 + c) * 64 + 16 * p + i] = v;
                    }
            }
    return ORC_OK;
}

int orc_w4_unprepack_weights(const uint8_t *wpp, int64_t K, int64_t N, uint8_t *packed) {
    if (K < 1 || N < 1 || K % 128 != 0) return ORC_ERR_SHAPE;
    const int64_t KB = K / 2, S = K / 128;
    for (int64_t n = 0; n < N; ++n) {
        const int64_t b = n / 16, c = n % 16;
        for (int64_t k2 = 0; k2 < KB; ++k2) {
            const int64_t t = k2 / 64, chunk = (k2 % 64) / 16, i = k2 % 16;
            const int64_t p = chunk ^ ((c / 2) % 4);
            packed[n * KB + k2] = wpp[((b * S + t) * 16 + c) * 64 + 16 * p + i];
        }
    }
    return ORC_OK;
}

int orc_w4a16_prepack(const uint8_t *packed, const float *scales, const float *zeros, int64_t K,
                      int64_t N, uint8_t *wpp, float *szpp) {
    if (K < 1 || N < 1 || K % 512 != 0) return ORC_ERR_SHAPE;
    const int64_t G = K / 128, NB = (N + 15) / 16;
    const int rc = orc_w4_prepack_weights(packed, K, N, wpp);
    if (rc != ORC_OK) return rc;
    for (int64_t b = 0; b < NB; ++b)
        for (int64_t u = 0; u < G / 2; ++u)
            for (int64_t c = 0; c < 16; ++c) {
                const int64_t n = 16 * b + c;
                float *e = szpp + ((b * (G / 2) + u) * 16 + c) * 4;
                e[0] = n < N ? scales[n * G + 2 * u] : 0.0f;
                e[1] = n < N ? zeros[n * G + 2 * u] : 0.0f;
                e[2] = n < N ? scales[n * G + 2 * u + 1] : 0.0f;
                e[3] = n < N ? zeros[n * G + 2 * u + 1] : 0.0f;
            }
    return ORC_OK;
}

int orc_w4a16_unprepack(const uint8_t *wpp, const float *szpp, int64_t K, int64_t N,
                        uint8_t *packed, float *scales, float *zeros) {
    if (K < 1 || N < 1 || K % 512 != 0) return ORC_ERR_SHAPE;
    const int64_t G = K / 128;
    const int rc = orc_w4_unprepack_weights(wpp, K, N, packed);
    if (rc != ORC_OK) return rc;
    for (int64_t n = 0; n < N; ++n) {
        const int64_t b = n / 16, c = n % 16;
        for (int64_t g = 0; g < G; ++g) {
            const float *e = szpp + ((b * (G / 2) + g / 2) * 16 + c) * 4;
            scales[n * G + g] = e[2 * (g % 2)];
            zeros[n * G + g] = e[2 * (g % 2) + 1];
        }
    }
    return ORC_OK;
}

/* Round-to-nearest-even of an fp32 value to the bf16 format (the upper 16 bits
 * of the fp32 encoding).  NaN is kept quiet. */
uint16_t orc_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

static double bf16_to_double(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* [W4A16] "激活值保持高精度" and [ENCY] 4.5 schemes A/C: the int4 weights are
 * dequantized at compute time to a 16-bit float weight, here bf16:
 * w' = bf16(fl(float(q - zp) * s)). */
int orc_w4a16_dequant(const uint8_t *packed, const float *scales, const float *zeros,
                      int64_t K, int64_t N, int64_t group, uint16_t *Wd) {
    if (K < 1 || N < 1 || group < 1 || K % group != 0) return ORC_ERR_SHAPE;
    const int64_t G = K / group;
    for (int64_t k = 0; k < K; ++k) {
        for (int64_t n = 0; n < N; ++n) {
            int q = unpack_unsigned(packed, K, n, k);
            float s = scales[n * G + k / group];
            float zp = zeros[n * G + k / group];
            float d = (float)q - zp;
            float w = d * s;
            Wd[k * N + n] = orc_bf16_rne(w);
        }
    }
    return ORC_OK;
}

/* The W4A16 product: bf16 activations times the dequantized bf16 weights.
 * Each product of two bf16 values is exact in fp64; the fp64 sum is the
 * reference value against which any fp32 summation order is judged. */
int orc_w4a16_linear(const uint16_t *X, int64_t M, int64_t K, int64_t N,
                     const uint8_t *packed, const float *scales, const float *zeros,
                     int64_t group, double *Y, double *absy) {
    if (M < 1 || K < 1 || N < 1 || group < 1 || K % group != 0) return ORC_ERR_SHAPE;
    const int64_t G = K / group;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                int q = unpack_unsigned(packed, K, n, k);
                float s = scales[n * G + k / group];
                float zp = zeros[n * G + k / group];
                float d = (float)q - zp;
                float w = d * s;
                double wd = bf16_to_double(orc_bf16_rne(w));
                double xd = bf16_to_double(X[m * K + k]);
                acc += xd * wd;
                aacc += fabs(xd * wd);
            }
            Y[m * N + n] = acc;
            if (absy) absy[m * N + n] = aacc;
        }
    }
    return ORC_OK;
}
