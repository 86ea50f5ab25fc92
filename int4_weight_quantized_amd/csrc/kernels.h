// Host-side launchers of the gfx950 kernels (internal to the library).
// Shapes and pointers are validated by the C ABI layer before any launcher
// runs; each launcher only enqueues work on `st` and returns hipGetLastError().
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

// Optional start/stop events for the next product kernel (per host thread);
// taking them clears them.
struct TimingEvents {
    hipEvent_t start;
    hipEvent_t stop;
};
TimingEvents take_timing_events();

// Remember which kernel the current call launches (its host stub and stream);
// the C ABI layer keeps it as the last kernel once the call succeeded.
void note_kernel(const void *kernel, hipStream_t st);

// Launch a product kernel; if timing events are pending they are attached to
// this dispatch (recorded when the kernel starts and when it completes).
template <typename... KArgs, typename... Args>
inline void launch_main(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shm,
                        hipStream_t st, Args... args) {
    note_kernel(reinterpret_cast<const void *>(kernel), st);
    const TimingEvents ev = take_timing_events();
    if (ev.start || ev.stop)
        hipExtLaunchKernelGGL(kernel, grid, block, shm, st, ev.start, ev.stop, 0u, KArgs(args)...);
    else
        hipLaunchKernelGGL(kernel, grid, block, shm, st, KArgs(args)...);
}

// Which accumulation product a W4A8 kernel writes.
enum class Out { Y, I32 };

struct W4A8Args {
    const float *X;       // fp32 activations [M][K] (fused quantization) or NULL
    const int8_t *Xq;     // int8 activations, natural or P8 layout, or NULL
    const float *sx;      // [M] activation scales (with Xq)
    const uint8_t *packed;  // int4 codes [N][K/2], or int8 codes [N][K] when w8
    const float *sw;
    const float *bias;
    float *Y;
    int32_t *acc;
    int64_t M, K, N;
    Out out;
    bool w8;    // 8-bit weight codes (W8A8): natural-layout activations, no unpacking
    bool relu;  // ReLU after dequantization and bias (Out::Y only)
    const float *act_div;  // per-column divisors of X before quantization (AWQ), or NULL
    bool pp;  // int4 weights in the shuffled tile layout (K % 128 == 0; see w4a16.hip)
};

hipError_t launch_quant_weight_sym(const float *W, int64_t K, int64_t N, uint8_t *packed,
                                   float *sw, hipStream_t st);
hipError_t launch_quant_weight_w8(const float *W, int64_t K, int64_t N, int8_t *Wq, float *sw,
                                  hipStream_t st);
hipError_t launch_quant_weight_asym(const float *W, int64_t K, int64_t N, int64_t group,
                                    uint8_t *packed, float *scales, float *zeros, hipStream_t st);
// W [K][N] = dequantized codes (+ delta [K][N] when non-NULL); zeros == NULL
// selects the symmetric form.
hipError_t launch_dequant_weight(const uint8_t *packed, const float *scales, const float *zeros,
                                 int64_t K, int64_t N, int64_t group, const float *delta,
                                 float *W, hipStream_t st);
// div (nullable): per-column divisors applied before quantization (AWQ).
// step (K % 16 == 0): codes stored chunk-major [K/16][M][16] for the MFMA GEMV.
hipError_t launch_quant_act(const float *X, int64_t M, int64_t K, int8_t *Xq, float *sx, bool p8,
                            hipStream_t st, const float *div = nullptr, bool step = false);
// AWQ-style channel scaling: power-of-two scales from calibration rows, the
// weight fold W diag(s) and the bf16 activation division.
hipError_t launch_awq_scales(const float *Xcal, int64_t M, int64_t K, int num, int den, float *s,
                             hipStream_t st);
hipError_t launch_awq_fold(const float *W, int64_t K, int64_t N, const float *s, float *Wout,
                           hipStream_t st);
hipError_t launch_awq_scale_bf16(const uint16_t *X, int64_t M, int64_t K, const float *s,
                                 uint16_t *Xout, hipStream_t st);
// Natural int8 [M][K] -> P8 (p8) and / or chunk-major (step) order.
hipError_t launch_to_p8(const int8_t *Xq, int64_t M, int64_t K, int8_t *out, hipStream_t st,
                        bool p8 = true, bool step = false);

// M <= 4, K % 32 == 0, K <= 8192 (4096 for 8-bit weights), 16-byte aligned: VALU
// dot4 GEMV.  Uses a.X (fused quantization prologue) when non-NULL, else a.Xq
// (natural layout) + a.sx.
bool gemv_dot4_ok(int64_t M, int64_t K, bool w8);
hipError_t launch_gemv_dot4(const W4A8Args &a, hipStream_t st);

// M <= 64, K % 128 == 0: MFMA GEMV; a.Xq chunk-major [K/16][M][16], P8 order
// inside (natural for 8-bit weights).
hipError_t launch_gemv_mfma(const W4A8Args &a, hipStream_t st);
// MFMA GEMV with the activation quantization in its prologue (a.X fp32,
// Out::Y, no divisors): for gemv_mfma_fused_ok(M, K, w8, pp) shapes.
bool gemv_mfma_fused_ok(int64_t M, int64_t K, bool w8, bool pp);
hipError_t launch_gemv_mfma_fused(const W4A8Args &a, hipStream_t st);

// Any M, K % 128 == 0: LDS-tiled MFMA GEMM; a.Xq in P8 layout (natural for
// 8-bit weights).
hipError_t launch_gemm_mfma(const W4A8Args &a, hipStream_t st);

// Any shape: one thread per output, natural-layout a.Xq (int4 or int8 codes).
hipError_t launch_w4a8_generic(const W4A8Args &a, hipStream_t st);

// W4A16.
bool w4a16_fast_ok(int64_t M, int64_t K, int64_t N, int64_t group);
// group == 128, K % 512 == 0, 16-byte aligned operands: LDS-staged kernel.
bool w4a16_lds_ok(int64_t K, int64_t group);
hipError_t launch_w4a16_lds(const uint16_t *X, int64_t M, int64_t K, int64_t N,
                            const uint8_t *packed, const float *scales, const float *zeros,
                            float *Y, hipStream_t st);
// The same kernel on the GPU-shuffled layout (wpp, szpp from launch_w4a16_prepack).
hipError_t launch_w4a16_prepacked(const uint16_t *X, int64_t M, int64_t K, int64_t N,
                                  const uint8_t *wpp, const float *szpp, float *Y,
                                  hipStream_t st);
hipError_t launch_w4_prepack_weights(const uint8_t *packed, int64_t K, int64_t N, uint8_t *wpp,
                                    hipStream_t st);
hipError_t launch_w4_unprepack_weights(const uint8_t *wpp, int64_t K, int64_t N, uint8_t *packed,
                                      hipStream_t st);
hipError_t launch_w4a16_prepack(const uint8_t *packed, const float *scales, const float *zeros,
                                int64_t K, int64_t N, uint8_t *wpp, float *szpp, hipStream_t st);
hipError_t launch_w4a16_unprepack(const uint8_t *wpp, const float *szpp, int64_t K, int64_t N,
                                  uint8_t *packed, float *scales, float *zeros, hipStream_t st);
hipError_t launch_w4a16_mfma(const uint16_t *X, int64_t M, int64_t K, int64_t N,
                             const uint8_t *packed, const float *scales, const float *zeros,
                             int64_t group, float *Y, hipStream_t st);
hipError_t launch_w4a16_generic(const uint16_t *X, int64_t M, int64_t K, int64_t N,
                                const uint8_t *packed, const float *scales, const float *zeros,
                                int64_t group, float *Y, hipStream_t st);

// Measurement helpers (probe.hip): an empty kernel, a plain streaming read and
// write, and an MFMA clock probe.
hipError_t launch_probe_empty(int64_t blocks, hipStream_t st);
hipError_t launch_probe_read(const uint8_t *src, int64_t bytes, uint32_t *sink, hipStream_t st);
hipError_t launch_probe_write(uint8_t *dst, int64_t bytes, uint32_t value, hipStream_t st);
hipError_t launch_probe_mfma(int64_t blocks, int iters, const int32_t *ops, uint64_t *times,
                             uint32_t *sink, hipStream_t st);

}  // namespace w4
