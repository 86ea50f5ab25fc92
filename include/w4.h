/*
 * w4.h -- C ABI of the MI355X (gfx950) INT4 weight-quantized linear layer.
 *
 * The method (INT4 quantization guide of Keras, "How it works", steps 1-6):
 *   1. each output channel of a weight matrix gets a symmetric absmax scale,
 *   2. weights are rounded into [-8, 7] and packed two per byte,
 *   3. at inference time activations are scaled by a dynamic absmax and
 *      quantized to INT8,
 *   4. the packed INT4 weights are unpacked to INT8 values,
 *   5. an INT8 x INT8 product is accumulated in INT32,
 *   6. the result is dequantized with input_scale * per_channel_kernel_scale.
 * A weight-only variant ("4-bit Integer Quantization for LLMs", quantization
 * principle; "INT4" concept entry, sections 4.1, 4.2 and 4.5) stores
 * asymmetric group-wise codes in [0, 15] with a scale and zero point per group
 * and dequantizes them to 16-bit floats (bf16 here) at compute time.
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller (for
 *     example torch tensors); the library never allocates or frees memory.
 *   - `stream` is a hipStream_t handle (NULL = the default stream).  Every
 *     call is asynchronous on that stream.
 *   - Arguments are checked on the host before anything is launched; on a
 *     failed check the call returns a negative w4_status and launches nothing.
 *     After launching, a launch error is reported as W4_ERR_HIP.
 *   - Row-major layouts throughout.  W is [K][N] (input dim K, N output
 *     channels), X is [M][K], Y is [M][N].
 *   - Packed int4 layout: output channel n owns the (K+1)/2 bytes
 *     packed[n*((K+1)/2) ...]; byte j holds k = 2j in bits 0-3 and k = 2j+1 in
 *     bits 4-7; a missing last high nibble (odd K) is 0.  Signed codes are
 *     two's complement nibbles; unsigned codes are plain nibbles.
 *   - Rounding is round-half-to-even; quotients are correctly rounded fp32
 *     divisions.  Inputs must be finite (non-finite values are a caller error;
 *     results are then unspecified).
 *   - Calls on one stream are ordered; calls that write the same buffers on
 *     different streams race.
 */
#ifndef W4_H
#define W4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4_OK = 0,
    W4_ERR_NULL = -1,      /* a required pointer is NULL                          */
    W4_ERR_SHAPE = -2,     /* a size is < 1, a group_size odd or not dividing K, or too large */
    W4_ERR_ALIGN = -3,     /* a pointer is not aligned to its element size        */
    W4_ERR_SCHEME = -4,    /* unknown quantization scheme                         */
    W4_ERR_WORKSPACE = -5, /* workspace missing or smaller than required          */
    W4_ERR_HIP = -6,       /* the HIP runtime reported an error                   */
    W4_ERR_ARG = -7,       /* an enumerated argument has an unknown value         */
    W4_ERR_SCRATCH = -8    /* w4a8_linear_noalloc: the shape needs more scratch
                              than W4_NOALLOC_SCRATCH_BYTES                       */
} w4_status;

/* Activation applied to a layer's output after dequantization and bias (the
 * Keras guide's toy model: Dense(32, activation="relu")). */
typedef enum {
    W4_ACT_NONE = 0,
    W4_ACT_RELU = 1 /* y > 0 ? y : +0 */
} w4_activation;

typedef enum {
    W4_SYM_PER_CHANNEL = 0, /* signed codes [-8,7], scale = absmax/7 per channel  */
    W4_ASYM_GROUP = 1       /* unsigned codes [0,15], scale + zero point per group */
} w4_scheme;

/* Largest K accepted by the integer paths: |acc| <= 128*8*K must fit int32
 * with the 16x headroom the unpacking uses (16*1024*K < 2^31); the W8A8
 * bound 128*128*K < 2^31 is the same. */
#define W4_MAX_K 131071

/* Quantize a weight matrix and pack it (Keras guide steps 1-2 for
 * W4_SYM_PER_CHANNEL; weight-only page's quantization principle and concept
 * entry 4.1-4.2 for W4_ASYM_GROUP).
 *   W       [K][N] fp32, finite.
 *   scheme  W4_SYM_PER_CHANNEL: group_size must be 0, scales is [N]:
 *             scales[n] = fl(max_k |W[k][n]| / 7) (0 for an all-zero channel),
 *             code = clamp(rne(fl(W / scale)), -8, 7) (0 where scale is 0);
 *             zeros must be NULL.
 *           W4_ASYM_GROUP: group_size even, >= 2, with K % group_size == 0
 *             (else W4_ERR_SHAPE): the two codes of a packed byte then never
 *             belong to two groups, so every group owns whole bytes (K <=
 *             W4_MAX_K also keeps K / group_size <= 65535); groups of
 *             group_size consecutive k inside one channel; scales and zeros
 *             are [N][K/group_size]:
 *               lo, hi = min, max of the group;
 *               scale = fl(fl(hi - lo) / 15) if hi > lo, else |lo| (1 if lo == 0);
 *               zero  = 0 - rne(fl(lo / scale))  (integer-valued fp32, not clamped);
 *               code  = clamp(rne(fl(W / scale)) + zero, 0, 15).
 *   packed  [N][(K+1)/2] bytes, fully written.
 * Returns W4_OK, W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_ALIGN, W4_ERR_SCHEME or W4_ERR_HIP. */
int w4_quantize_weight(const float *W, int64_t K, int64_t N, int scheme,
                       int64_t group_size, uint8_t *packed, float *scales,
                       float *zeros, void *stream);

/* Dequantize packed int4 weights back to fp32 (the dequantization step of
 * the LoRA export path, Keras guide "Limitations"; formulas of step 6 and of
 * the weight-only page's quantization principle).
 *   packed, scales, zeros, scheme, group_size as produced by w4_quantize_weight
 *           (the same group_size rule: even, >= 2, dividing K).
 *   W  [K][N] fp32: fl(code * scale[n]) for W4_SYM_PER_CHANNEL,
 *      fl(fl(code - zero) * scale) for W4_ASYM_GROUP.
 * Returns W4_OK, W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_ALIGN, W4_ERR_SCHEME or W4_ERR_HIP. */
int w4_dequantize_weight(const uint8_t *packed, const float *scales, const float *zeros,
                         int64_t K, int64_t N, int scheme, int64_t group_size, float *W,
                         void *stream);

/* The lossy LoRA merge (Keras guide, "Limitations": dequantize -> add the
 * delta -> requantize):
 *   work = fl(dequant(packed) + delta)   (delta [K][N] fp32, e.g. B @ A),
 *   (packed_out, scales_out, zeros_out) = w4_quantize_weight(work, same scheme).
 *   work  caller-owned device scratch of K*N fp32 (overwritten; must not
 *         overlap any other argument).
 * packed_out / scales_out / zeros_out may be the input arrays (in place): the
 * steps run in order on `stream`.  zeros and zeros_out are NULL for
 * W4_SYM_PER_CHANNEL.
 * Returns W4_OK, W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_ALIGN, W4_ERR_SCHEME or W4_ERR_HIP. */
int w4_merge_delta(const uint8_t *packed, const float *scales, const float *zeros,
                   int64_t K, int64_t N, int scheme, int64_t group_size,
                   const float *delta, uint8_t *packed_out, float *scales_out,
                   float *zeros_out, float *work, void *stream);

/* Per-row dynamic int8 activation quantization (Keras guide step 3).
 *   X   [M][K] fp32, finite.
 *   sx  [M]: sx[m] = fl(max_k |X[m][k]| / 127) (0 for an all-zero row).
 *   Xq  [M][K] int8: clamp(rne(fl(X / sx)), -128, 127) (0 where sx is 0).
 * Returns W4_OK, W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_ALIGN or W4_ERR_HIP. */
int a8_quantize_act(const float *X, int64_t M, int64_t K, int8_t *Xq, float *sx,
                    void *stream);

/* Bytes of device workspace that w4a8_linear, w4a8_linear_q and
 * w4a8_matmul_i32 need for this shape (0 when none is needed); 0 also for
 * invalid sizes. */
size_t w4a8_workspace_bytes(int64_t M, int64_t K, int64_t N);

/* The W4A8 forward (Keras guide steps 3-6), with an optional bias added
 * after dequantization (the Dense layer's bias).
 *   X       [M][K] fp32 activations.
 *   packed  [N][(K+1)/2] signed codes and sw [N] scales from
 *           w4_quantize_weight(..., W4_SYM_PER_CHANNEL, ...); any byte value is
 *           accepted (code -8 included).
 *   bias    [N] fp32 or NULL.
 *   Y       [M][N] fp32: Y = fl(fl(float(acc) * fl(sx[m] * sw[n])) [+ bias[n]]),
 *           acc = sum_k Xq[m][k] * code[n][k] exactly, Xq and sx as in
 *           a8_quantize_act.
 *   workspace  device memory of at least w4a8_workspace_bytes(M, K, N) bytes,
 *           256-byte aligned (may be NULL when that size is 0); its contents
 *           are scratch, overwritten by the call.
 * Returns W4_OK, W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_ALIGN, W4_ERR_WORKSPACE or W4_ERR_HIP. */
int w4a8_linear(const float *X, int64_t M, int64_t K, int64_t N,
                const uint8_t *packed, const float *sw, const float *bias,
                float *Y, void *workspace, size_t workspace_bytes, void *stream);

/* w4a8_linear followed by an activation, fused into the product kernel's
 * epilogue: Y = act(fl(fl(float(acc) * fl(sx[m] * sw[n])) [+ bias[n]])).
 * For M <= 4 (K % 32 == 0, K <= 8192, 16-byte aligned X and packed), and for
 * M <= 16 with K % 128 == 0 and K <= 4096 (16-byte aligned X; with int8
 * weights or shuffled tiles also ceil(M/8)*K <= 4096), the whole decode
 * step -- activation quantization, unpacking,
 * product, dequantization, bias and activation -- is one kernel launch (the
 * workspace is then not touched).
 *   activation  W4_ACT_NONE or W4_ACT_RELU; any other value: W4_ERR_ARG.
 * Other arguments and return codes as w4a8_linear. */
int w4a8_linear_act(const float *X, int64_t M, int64_t K, int64_t N,
                    const uint8_t *packed, const float *sw, const float *bias,
                    int activation, float *Y, void *workspace, size_t workspace_bytes,
                    void *stream);

/* Size of the fixed device scratch of w4a8_linear_noalloc: 16 MiB + 64 KiB.
 * It takes every shape with w4a8_workspace_bytes(M, K, N) up to this size
 * (activation codes and row scales), e.g. a 4096 x 4096 prefill.  Every GPU
 * the library runs on holds one such array from the library's load until the
 * process ends. */
#define W4_NOALLOC_SCRATCH_BYTES (16777216 + 65536)

/* w4a8_linear for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); its scratch is a fixed device array of
 * W4_NOALLOC_SCRATCH_BYTES per GPU inside the library, whose address is looked
 * up once per device, on the first call made with that device current.
 *   X, packed, sw, bias, Y  as w4a8_linear (caller-owned device memory);
 *   stream  the hipStream_t the kernels run on.
 * Results are bit-identical to w4a8_linear.  The scratch keeps the last
 * call's contents, and every call on one GPU uses the same array: calls that
 * overlap on one GPU (other streams, other host threads) race and must be
 * serialized by the caller.
 * Returns W4_OK, W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_ALIGN, W4_ERR_HIP, or
 * W4_ERR_SCRATCH when w4a8_workspace_bytes(M, K, N) exceeds
 * W4_NOALLOC_SCRATCH_BYTES (nothing is launched then). */
int w4a8_linear_noalloc(const float *X, int64_t M, int64_t K, int64_t N,
                        const uint8_t *packed, const float *sw, const float *bias,
                        float *Y, void *stream);

/* The W4A8 forward from already-quantized activations (Keras guide steps 4-6):
 *   Xq [M][K] int8 and sx [M] fp32 (any values); the rest as w4a8_linear. */
int w4a8_linear_q(const int8_t *Xq, const float *sx, const uint8_t *packed,
                  const float *sw, const float *bias, int64_t M, int64_t K,
                  int64_t N, float *Y, void *workspace, size_t workspace_bytes,
                  void *stream);

/* The exact integer product alone (Keras guide steps 4-5), for checking:
 *   acc [M][N] int32 = sum_k Xq[m][k] * code[n][k]. */
int w4a8_matmul_i32(const int8_t *Xq, const uint8_t *packed, int64_t M,
                    int64_t K, int64_t N, int32_t *acc, void *workspace,
                    size_t workspace_bytes, void *stream);

/* ---- AWQ-style activation-aware channel scaling ("INT4" concept entry,
 * section 4.4: measure each input channel's activation magnitude on
 * calibration data, scale the weights of the important channels up,
 * W' = W diag(s), quantize W', and divide the activations by s at inference;
 * x/s times W diag(s) is x W).  The page fixes neither the magnitude
 * statistic nor the rule from magnitude to s; these calls take:
 *   a_k   = max over the calibration rows of |x[m][k]|,
 *   E_k   = floor(log2 a_k) (-150 for an all-zero channel),
 *   E_med = the lower median of E over the K channels,
 *   s_k   = 2^e_k, e_k = min(24, max(0, floor(alpha_num * (E_k - E_med) / alpha_den))).
 * Powers of two make the fold and the activation division exact in fp32 and
 * bf16; only the quantization error changes. */

/* Channel scales s [K] fp32 from calibration activations Xcal [M][K] fp32
 * (finite).  0 <= alpha_num <= 1024, 1 <= alpha_den <= 1024, else W4_ERR_ARG.
 * Returns W4_OK, W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_ARG, W4_ERR_ALIGN or W4_ERR_HIP. */
int awq_channel_scales(const float *Xcal, int64_t M, int64_t K, int alpha_num,
                       int alpha_den, float *s, void *stream);

/* W_out [K][N] = fl(W[k][n] * s[k]) (W_out may be W).  The result is then
 * quantized with w4_quantize_weight (either scheme) or w8_quantize_weight. */
int awq_fold_weight(const float *W, int64_t K, int64_t N, const float *s, float *W_out,
                    void *stream);

/* a8_quantize_act of x' = fl(X[m][k] / s[k]) (s any positive finite values). */
int awq_quantize_act(const float *X, int64_t M, int64_t K, const float *s, int8_t *Xq,
                     float *sx, void *stream);

/* Weight-only path: X_out = bf16_rne(fl(float(X_bf16[m][k]) / s[k])) (bit
 * patterns; exact for power-of-two s), to feed w4a16_linear with weights
 * quantized from W diag(s). */
int awq_scale_act_bf16(const uint16_t *X_bf16, int64_t M, int64_t K, const float *s,
                       uint16_t *X_out, void *stream);

/* The W4A8 forward with AWQ scaling: Y = act(dequant(quant(X / s) . codes)
 * [+ bias]), with packed / sw from w4_quantize_weight(awq_fold_weight(W, s)).
 * The division by s is fused into the activation quantization (into the
 * single-launch decode kernel for M <= 4).  s [K] is 16-byte aligned.
 * Other arguments and return codes as w4a8_linear_act. */
int w4a8_linear_awq(const float *X, int64_t M, int64_t K, int64_t N,
                    const uint8_t *packed, const float *sw, const float *s,
                    const float *bias, int activation, float *Y, void *workspace,
                    size_t workspace_bytes, void *stream);

/* ---- W8A8: the INT8 path that the Keras guide's "How it works" says the
 * INT4 path follows apart from the unpacking (steps 1-6 with 8-bit weight
 * codes; "INT4" concept entry, section 4.1 with b = 8 for the scale). */

/* Symmetric per-output-channel int8 weight quantization.
 *   W   [K][N] fp32, finite.
 *   sw  [N]: sw[n] = fl(max_k |W[k][n]| / 127) (0 for an all-zero channel).
 *   Wq  [N][K] int8, channel-major (one code per byte, no packing):
 *       clamp(rne(fl(W / sw)), -128, 127) (0 where sw is 0).
 * Returns W4_OK, W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_ALIGN or W4_ERR_HIP. */
int w8_quantize_weight(const float *W, int64_t K, int64_t N, int8_t *Wq, float *sw,
                       void *stream);

/* Bytes of device workspace that w8a8_linear and w8a8_matmul_i32 need (0 when
 * none is needed, and for invalid sizes). */
size_t w8a8_workspace_bytes(int64_t M, int64_t K, int64_t N);

/* The W8A8 forward: as w4a8_linear with int8 weight codes Wq [N][K] (any byte
 * values) and scales sw [N] from w8_quantize_weight:
 *   Y = fl(fl(float(acc) * fl(sx[m] * sw[n])) [+ bias[n]]),
 *   acc = sum_k Xq[m][k] * Wq[n][k] exactly.
 * Workspace, alignment and return codes as w4a8_linear. */
int w8a8_linear(const float *X, int64_t M, int64_t K, int64_t N, const int8_t *Wq,
                const float *sw, const float *bias, float *Y, void *workspace,
                size_t workspace_bytes, void *stream);

/* w8a8_linear followed by an activation fused into the epilogue (as
 * w4a8_linear_act; the single-launch decode path covers K <= 4096). */
int w8a8_linear_act(const float *X, int64_t M, int64_t K, int64_t N, const int8_t *Wq,
                    const float *sw, const float *bias, int activation, float *Y,
                    void *workspace, size_t workspace_bytes, void *stream);

/* The exact W8A8 integer product alone, for checking:
 *   acc [M][N] int32 = sum_k Xq[m][k] * Wq[n][k]. */
int w8a8_matmul_i32(const int8_t *Xq, const int8_t *Wq, int64_t M, int64_t K, int64_t N,
                    int32_t *acc, void *workspace, size_t workspace_bytes, void *stream);

/* The weight-only W4A16 forward (weight-only page: activations stay 16-bit,
 * weights are dequantized at compute time; concept entry 4.5, schemes A/C).
 *   X_bf16  [M][K] bf16 bit patterns.
 *   packed  [N][(K+1)/2] unsigned codes; scales, zeros [N][K/group_size] fp32
 *           from w4_quantize_weight(..., W4_ASYM_GROUP, group_size, ...);
 *           group_size even, >= 2, dividing K, else W4_ERR_SHAPE.  Zero
 *           points may be any finite value (the quantizer's are integers).
 *   Y       [M][N] fp32 = sum_k x[m][k] * w'[k][n], with
 *           w' = bf16_rne(fl(fl(float(code) - zero) * scale)), products and
 *           sums in fp32 (the summation order is unspecified; the result is
 *           within K*2^-24 * sum_k |x*w'| of the exact sum).
 * Returns W4_OK, W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_ALIGN or W4_ERR_HIP. */
int w4a16_linear(const uint16_t *X_bf16, int64_t M, int64_t K, int64_t N,
                 const uint8_t *packed, const float *scales, const float *zeros,
                 int64_t group_size, float *Y, void *stream);

/* ---- A second, GPU-shuffled layout of the W4A16 weights (group 128,
 * K % 512 == 0).  The pages only pack two codes per byte; this layout is a
 * pure rearrangement of the canonical arrays into the order the W4A16
 * kernel consumes them, so that every load reads contiguous bytes:
 *   wpp  [N16/16][K/128][16][64] bytes, N16 = 16 * ceil(N / 16):
 *        wpp[b][t][c][16 p + i] = packed[16 b + c][64 t + 16 (p ^ ((c / 2) % 4)) + i]
 *        (zero bytes for the padding channels N .. N16 - 1);
 *   szpp [N16/16][K/256][16][4] fp32:
 *        szpp[b][u][c] = (scales[n][2u], zeros[n][2u], scales[n][2u+1], zeros[n][2u+1]),
 *        n = 16 b + c (zeros for padding channels).
 * w4a16_unprepack inverts it exactly (round-trip identity on the first N
 * channels).  All arrays are device memory; wpp, szpp and packed 16-byte
 * aligned.  group_size must be 128 and K % 512 == 0, else W4_ERR_SHAPE. */

/* Sizes of the shuffled arrays (bytes of wpp, floats of szpp); 0 when the
 * shape is not supported. */
int64_t w4a16_prepacked_weight_bytes(int64_t K, int64_t N);
int64_t w4a16_prepacked_table_floats(int64_t K, int64_t N);

/* Canonical (packed [N][K/2], scales, zeros [N][K/128]) -> (wpp, szpp).
 * Returns W4_OK, W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_ALIGN or W4_ERR_HIP. */
int w4a16_prepack(const uint8_t *packed, const float *scales, const float *zeros,
                  int64_t K, int64_t N, int64_t group_size, uint8_t *wpp, float *szpp,
                  void *stream);

/* (wpp, szpp) -> the canonical arrays of the first N channels. */
int w4a16_unprepack(const uint8_t *wpp, const float *szpp, int64_t K, int64_t N,
                    int64_t group_size, uint8_t *packed, float *scales, float *zeros,
                    void *stream);

/* w4a16_linear on the shuffled layout: the same products in the same order
 * (bit-identical outputs), with contiguous weight and table loads.  X_bf16
 * 16-byte aligned.  Returns as w4a16_linear. */
int w4a16_linear_prepacked(const uint16_t *X_bf16, int64_t M, int64_t K, int64_t N,
                           const uint8_t *wpp, const float *szpp, float *Y, void *stream);

/* ---- The weight part of the same shuffled layout for the W4A8 int4 codes
 * (K % 128 == 0): wpp [N16/16][K/128][16][64] exactly as above; the
 * per-channel scales stay [N].  The product kernels then read every weight
 * tile as contiguous bytes (the decode-batch kernel one 1 KB tile per load).
 * Callers: decode / prefill layers whose weights are converted once. */
int64_t w4_prepacked_weight_bytes(int64_t K, int64_t N);  /* 0 if K % 128 != 0 */
int w4_prepack_weights(const uint8_t *packed, int64_t K, int64_t N, uint8_t *wpp,
                       void *stream);
int w4_unprepack_weights(const uint8_t *wpp, int64_t K, int64_t N, uint8_t *packed,
                         void *stream);

/* w4a8_linear_act on the shuffled codes: the same products and epilogue
 * (bit-identical outputs).  K % 128 == 0 (else W4_ERR_SHAPE), wpp 16-byte
 * aligned; other arguments, workspace and return codes as w4a8_linear_act. */
int w4a8_linear_prepacked(const float *X, int64_t M, int64_t K, int64_t N,
                          const uint8_t *wpp, const float *sw, const float *bias,
                          int activation, float *Y, void *workspace,
                          size_t workspace_bytes, void *stream);

/* Static description of a status code (never NULL). */
const char *w4_status_string(int status);

/* Per-kernel timing for benchmarks and profiling: the next product kernel
 * (the GEMV / GEMM / W4A16 kernel, not the activation or weight quantizers
 * of a multi-kernel call) that an entry point launches from this host thread
 * records `start_event` when it begins executing and `stop_event` when it
 * completes.  Both are hipEvent_t handles created by the caller (either may
 * be NULL; NULL and NULL cancels).  Consumed by that one launch.  Not for
 * use while a stream is being captured into a graph.  Returns W4_OK. */
int w4_time_next_kernel(void *start_event, void *stop_event);

/* Name of the kernel variant the last successful call on this thread launched
 * for its main product (for tests and profiling; never NULL). */
const char *w4_last_path(void);

/* Device symbol (mangled name) of that kernel, e.g. for naming the kernel a
 * benchmark timed; "none" before any successful call on this thread.  The
 * returned string belongs to the HIP runtime. */
const char *w4_last_kernel(void);

/* ---- Measurement helpers (not part of the method): the platform references
 * the layer's timings are read against.  Asynchronous on `stream`.
 *
 * An empty kernel of `blocks` workgroups of 256 threads (1 <= blocks < 2^31):
 * its duration in a graph of back-to-back launches is the fixed cost of one
 * launch.  Returns W4_OK, W4_ERR_SHAPE or W4_ERR_HIP. */
int w4_probe_empty(int64_t blocks, void *stream);

/* A plain streaming read of `bytes` device bytes at `src` (16-byte aligned;
 * 16 <= bytes <= 0x7F000000, bytes % 16 == 0), each byte read once with a
 * 16-byte non-temporal load; `sink` is a device array of 64 uint32 that the
 * kernel writes only if the data's XOR takes one particular value (it keeps
 * the loads from being removed).  Returns W4_OK, W4_ERR_NULL, W4_ERR_SHAPE,
 * W4_ERR_ALIGN or W4_ERR_HIP. */
int w4_probe_read(const void *src, int64_t bytes, uint32_t *sink, void *stream);

/* A plain streaming write of `bytes` device bytes at `dst` (16-byte aligned;
 * 16 <= bytes <= 0x7F000000, bytes % 16 == 0): every 32-bit word becomes
 * `value`, each byte written once with a 16-byte non-temporal store.  The
 * fastest a kernel that only writes those bytes once can go (the prefill
 * product's fp32 output is 4 M N bytes).  Returns W4_OK, W4_ERR_NULL,
 * W4_ERR_SHAPE, W4_ERR_ALIGN or W4_ERR_HIP. */
int w4_probe_write(void *dst, int64_t bytes, uint32_t value, void *stream);

/* Back-to-back int8 MFMAs (v_mfma_i32_16x16x64_i8, 16 independent chains per
 * wave, 8 waves per workgroup, each chain cycling over four activation and
 * four weight operands) for `iters` iterations in each of `blocks` workgroups
 * (1 <= blocks <= 65536; iters >= 4, a multiple of 4).  `ops` (nullable,
 * 16-byte aligned) holds blocks * 512 * 32 int32: thread t of workgroup b
 * takes its 4 + 4 operands from ops[32 (512 b + t) ...]; NULL selects small
 * constant operands.  Wave 0 of workgroup b writes times[4b .. 4b+3] =
 * shader-clock counter at start and end, constant 100 MHz counter at start
 * and end, so the host can read the clock the matrix units ran at (it falls
 * with the operands' switching activity); `sink` is a device array of 64
 * uint32 written only for one particular result.  Returns W4_OK,
 * W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_ALIGN or W4_ERR_HIP. */
int w4_probe_mfma(int64_t blocks, int iters, const int32_t *ops, uint64_t *times, uint32_t *sink,
                  void *stream);

#ifdef __cplusplus
}
#endif

#endif /* W4_H */
