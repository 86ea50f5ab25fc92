// C ABI of the W4A8 / W4A16 linear layer: argument checks (pure host code,
// before anything is launched) and dispatch to the gfx950 kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/w4.h"
#include "kernels.h"

// Device scratch of w4a8_linear_noalloc: the activation-code workspace of the
// W4A8 paths, held in a fixed array so that the call allocates nothing.  In
// host code this name stands for a host-side shadow, not a device address:
// the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[W4_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local const char *g_last_path = "none";
thread_local hipEvent_t g_time_start = nullptr, g_time_stop = nullptr;
// the kernel the current call launches, and the last one of a successful call
thread_local const void *g_pending_kernel = nullptr, *g_last_kernel = nullptr;

inline bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int hip_status(hipError_t e) { return e == hipSuccess ? W4_OK : W4_ERR_HIP; }

// Status of a launch; the kernel variant's name is recorded only when the
// launch succeeded (w4_last_path reports the last successful call).
int launched(const char *path, hipError_t e) {
    if (e != hipSuccess) return W4_ERR_HIP;
    g_last_path = path;
    g_last_kernel = g_pending_kernel;
    return W4_OK;
}

// Workspace layout: [Xq: M*K bytes, 256-aligned][sx: 4*M bytes, 256-aligned].
size_t ws_bytes(int64_t M, int64_t K) {
    return round_up((size_t)M * (size_t)K, 256) + round_up(4 * (size_t)M, 256);
}

bool shape_ok(int64_t M, int64_t K, int64_t N) {
    if (M < 1 || K < 1 || N < 1) return false;
    if (K > W4_MAX_K) return false;
    const int64_t lim = (int64_t)1 << 40;
    if (M > lim / K || N > lim / K || M > lim / N) return false;
    return true;
}

enum class Src { FP32, Q };

// Shared dispatch of the W4A8 and W8A8 entry points (w8: `packed` holds int8
// codes [N][K]; the MFMA paths then take natural-layout activations).
int w4a8_dispatch(Src src, bool w8, const float *X, const int8_t *Xq, const float *sx,
                  const uint8_t *packed, const float *sw, const float *bias, int64_t M,
                  int64_t K, int64_t N, float *Y, int32_t *acc, void *workspace,
                  size_t workspace_bytes, hipStream_t st, bool relu = false,
                  const float *act_div = nullptr, bool pp = false) {
    using namespace w4;
    W4A8Args a{};
    a.pp = pp;
    a.w8 = w8;
    a.relu = relu;
    a.act_div = act_div;
    a.X = nullptr;
    a.Xq = Xq;
    a.sx = sx;
    a.packed = packed;
    a.sw = sw;
    a.bias = bias;
    a.Y = Y;
    a.acc = acc;
    a.M = M;
    a.K = K;
    a.N = N;
    a.out = acc ? Out::I32 : Out::Y;

    const bool aligned16 =
        aligned(packed, 16) && (src == Src::FP32 ? aligned(X, 16) : aligned(Xq, 16));
    // (the shuffled layout is only accepted with K % 128 == 0 and aligned
    // tiles: the MFMA paths always apply, whatever the alignment of X)
    const bool fast = pp || (aligned16 && (K % 128 == 0));
    int8_t *ws_q = reinterpret_cast<int8_t *>(workspace);
    float *ws_s = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(workspace) +
                                            round_up((size_t)M * (size_t)K, 256));
    hipError_t e;

    // the MFMA GEMV that quantizes the activations itself (one launch)
    const bool fused_ok = fast && src == Src::FP32 && !act_div && !acc && aligned(X, 16) &&
                          gemv_mfma_fused_ok(M, K, w8, pp);
    // Few rows: one VALU GEMV launch (activation quantization fused); from
    // three rows on the fused MFMA GEMV is faster where it applies (measured,
    // graph-replayed, us: M = 3 7B-class 9.0-9.5 -> 8.3, shuffled tiles
    // 9.1-9.5 -> 7.8, Gemma-like shuffled 4.28 -> 3.93, canonical even; int8
    // weights 7B-class 11.95 -> 11.55, Gemma-like 4.95 -> 4.70); at M = 2 the
    // VALU GEMV is faster on every path (7B-class 7.46 against 8.13).
    if (aligned16 && gemv_dot4_ok(M, K, w8) && !(M >= 3 && fused_ok)) {
        if (src == Src::FP32) a.X = X;
        return launched(w8 ? "w8_gemv_dot4" : pp ? "gemv_dot4_prepacked" : "gemv_dot4",
                        launch_gemv_dot4(a, st));
    }
    // Activations for the MFMA paths: P8 layout in the workspace (natural
    // layout for 8-bit weights, which then use pre-quantized input as is).
    if (fast) {
        // Few rows of small K: the MFMA GEMV quantizes the activations itself
        // (one launch instead of two).
        if (fused_ok) {
            a.X = X;
            const char *path = w8   ? "w8_gemv_mfma_fused"
                               : pp ? "gemv_mfma_fused_prepacked"
                                    : "gemv_mfma_fused";
            return launched(path, launch_gemv_mfma_fused(a, st));
        }
        // the MFMA GEMV takes the codes chunk-major, the GEMM row-major
        const bool step = M <= 64;
        if (src == Src::FP32) {
            e = launch_quant_act(X, M, K, ws_q, ws_s, !w8, st, act_div, step);
            if (e != hipSuccess) return W4_ERR_HIP;
            a.sx = ws_s;
            a.Xq = ws_q;
        } else if (!w8 || step) {
            e = launch_to_p8(Xq, M, K, ws_q, st, !w8, step);
            if (e != hipSuccess) return W4_ERR_HIP;
            a.Xq = ws_q;
        }
        if (M <= 64) {
            return launched(w8 ? "w8_gemv_mfma" : pp ? "gemv_mfma_prepacked" : "gemv_mfma",
                            launch_gemv_mfma(a, st));
        }
        return launched(w8 ? "w8_gemm_mfma" : pp ? "gemm_mfma_prepacked" : "gemm_mfma",
                        launch_gemm_mfma(a, st));
    }
    // Anything else: natural layout, one thread per output.
    if (src == Src::FP32) {
        e = launch_quant_act(X, M, K, ws_q, ws_s, false, st, act_div);
        if (e != hipSuccess) return W4_ERR_HIP;
        a.Xq = ws_q;
        a.sx = ws_s;
    }
    return launched(w8 ? "w8a8_generic" : "w4a8_generic", launch_w4a8_generic(a, st));
}

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current and kept per device (each GPU holds its
// own copy of the array at its own address).
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

int scratch_address(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return W4_ERR_HIP;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
                (void)hipGetLastError();
                return W4_ERR_HIP;
            }
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return W4_OK;
}

int check_workspace(int64_t M, int64_t K, void *workspace, size_t bytes) {
    const size_t need = ws_bytes(M, K);
    if (need == 0) return W4_OK;
    if (!workspace || bytes < need) return W4_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return W4_ERR_ALIGN;
    return W4_OK;
}

}  // namespace

void w4::note_kernel(const void *kernel, hipStream_t) { g_pending_kernel = kernel; }

w4::TimingEvents w4::take_timing_events() {
    TimingEvents ev{g_time_start, g_time_stop};
    g_time_start = g_time_stop = nullptr;
    return ev;
}

extern "C" {

int w4_time_next_kernel(void *start_event, void *stop_event) {
    g_time_start = reinterpret_cast<hipEvent_t>(start_event);
    g_time_stop = reinterpret_cast<hipEvent_t>(stop_event);
    return W4_OK;
}

const char *w4_status_string(int status) {
    switch (status) {
        case W4_OK: return "ok";
        case W4_ERR_NULL: return "a required pointer is NULL";
        case W4_ERR_SHAPE: return "invalid shape";
        case W4_ERR_ALIGN: return "misaligned pointer";
        case W4_ERR_SCHEME: return "unknown quantization scheme";
        case W4_ERR_WORKSPACE: return "workspace missing or too small";
        case W4_ERR_HIP: return "HIP runtime error";
        case W4_ERR_ARG: return "unknown value of an enumerated argument";
        case W4_ERR_SCRATCH:
            return "the shape needs more scratch than the no-allocation call's fixed buffer holds";
        default: return "unknown status";
    }
}

const char *w4_last_path(void) { return g_last_path; }

const char *w4_last_kernel(void) {
    if (!g_last_kernel) return "none";
    // the launch's stream may be gone by now; a kernel's symbol is the same on
    // every device, so the null stream (current device) resolves it
    const char *name = hipKernelNameRefByPtr(g_last_kernel, nullptr);
    return name ? name : "unknown";
}

int w4_probe_empty(int64_t blocks, void *stream) {
    if (blocks < 1 || blocks > 0x7FFFFFFF) return W4_ERR_SHAPE;
    return launched("probe_empty",
                    w4::launch_probe_empty(blocks, reinterpret_cast<hipStream_t>(stream)));
}

int w4_probe_mfma(int64_t blocks, int iters, const int32_t *ops, uint64_t *times, uint32_t *sink,
                  void *stream) {
    if (!times || !sink) return W4_ERR_NULL;
    if (blocks < 1 || blocks > 65536 || iters < 4 || iters % 4 != 0) return W4_ERR_SHAPE;
    if (!aligned(times, 8) || !aligned(sink, 4) || (ops && !aligned(ops, 16))) return W4_ERR_ALIGN;
    return launched("probe_mfma", w4::launch_probe_mfma(blocks, iters, ops, times, sink,
                                                        reinterpret_cast<hipStream_t>(stream)));
}

int w4_probe_read(const void *src, int64_t bytes, uint32_t *sink, void *stream) {
    if (!src || !sink) return W4_ERR_NULL;
    if (bytes < 16 || bytes % 16 != 0 || bytes > 0x7F000000) return W4_ERR_SHAPE;
    if (!aligned(src, 16) || !aligned(sink, 4)) return W4_ERR_ALIGN;
    return launched("probe_read",
                    w4::launch_probe_read(static_cast<const uint8_t *>(src), bytes, sink,
                                          reinterpret_cast<hipStream_t>(stream)));
}

int w4_probe_write(void *dst, int64_t bytes, uint32_t value, void *stream) {
    if (!dst) return W4_ERR_NULL;
    if (bytes < 16 || bytes % 16 != 0 || bytes > 0x7F000000) return W4_ERR_SHAPE;
    if (!aligned(dst, 16)) return W4_ERR_ALIGN;
    return launched("probe_write", w4::launch_probe_write(static_cast<uint8_t *>(dst), bytes, value,
                                                          reinterpret_cast<hipStream_t>(stream)));
}

int w4_quantize_weight(const float *W, int64_t K, int64_t N, int scheme, int64_t group_size,
                       uint8_t *packed, float *scales, float *zeros, void *stream) {
    if (!W || !packed || !scales) return W4_ERR_NULL;
    if (!shape_ok(1, K, N)) return W4_ERR_SHAPE;
    if (!aligned(W, 4) || !aligned(scales, 4)) return W4_ERR_ALIGN;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (scheme == W4_SYM_PER_CHANNEL) {
        if (group_size != 0 || zeros) return W4_ERR_SHAPE;
        return launched("quant_weight_sym",
                        w4::launch_quant_weight_sym(W, K, N, packed, scales, st));
    }
    if (scheme == W4_ASYM_GROUP) {
        if (!zeros) return W4_ERR_NULL;
        if (!aligned(zeros, 4)) return W4_ERR_ALIGN;
        if (group_size < 2 || group_size % 2 != 0 || K % group_size != 0) return W4_ERR_SHAPE;
        if (K / group_size > 65535) return W4_ERR_SHAPE;
        return launched("quant_weight_asym",
                        w4::launch_quant_weight_asym(
                            W, K, N, group_size, packed, scales, zeros, st));
    }
    return W4_ERR_SCHEME;
}

// Shared checks of the dequantize and merge entry points: scheme, group and
// pointer alignment of the code / scale / zero-point arrays.
static int dequant_args_ok(const uint8_t *packed, const float *scales, const float *zeros,
                           int64_t K, int64_t N, int scheme, int64_t group_size) {
    if (!packed || !scales) return W4_ERR_NULL;
    if (!shape_ok(1, K, N)) return W4_ERR_SHAPE;
    if (!aligned(scales, 4)) return W4_ERR_ALIGN;
    if (scheme == W4_SYM_PER_CHANNEL) {
        if (group_size != 0 || zeros) return W4_ERR_SHAPE;
        return W4_OK;
    }
    if (scheme == W4_ASYM_GROUP) {
        if (!zeros) return W4_ERR_NULL;
        if (!aligned(zeros, 4)) return W4_ERR_ALIGN;
        if (group_size < 2 || group_size % 2 != 0 || K % group_size != 0) return W4_ERR_SHAPE;
        if (K / group_size > 65535) return W4_ERR_SHAPE;
        return W4_OK;
    }
    return W4_ERR_SCHEME;
}

int w4_dequantize_weight(const uint8_t *packed, const float *scales, const float *zeros,
                         int64_t K, int64_t N, int scheme, int64_t group_size, float *W,
                         void *stream) {
    int rc = dequant_args_ok(packed, scales, zeros, K, N, scheme, group_size);
    if (rc != W4_OK) return rc;
    if (!W) return W4_ERR_NULL;
    if (!aligned(W, 4)) return W4_ERR_ALIGN;
    return launched("dequant_weight",
                    w4::launch_dequant_weight(packed, scales,
                                              scheme == W4_ASYM_GROUP ? zeros : nullptr, K, N,
                                              group_size, nullptr, W,
                                              reinterpret_cast<hipStream_t>(stream)));
}

int w4_merge_delta(const uint8_t *packed, const float *scales, const float *zeros, int64_t K,
                   int64_t N, int scheme, int64_t group_size, const float *delta,
                   uint8_t *packed_out, float *scales_out, float *zeros_out, float *work,
                   void *stream) {
    int rc = dequant_args_ok(packed, scales, zeros, K, N, scheme, group_size);
    if (rc != W4_OK) return rc;
    if (!delta || !packed_out || !scales_out || !work) return W4_ERR_NULL;
    if (scheme == W4_ASYM_GROUP && !zeros_out) return W4_ERR_NULL;
    if (scheme == W4_SYM_PER_CHANNEL && zeros_out) return W4_ERR_SHAPE;
    if (!aligned(delta, 4) || !aligned(scales_out, 4) || !aligned(work, 4) ||
        (zeros_out && !aligned(zeros_out, 4)))
        return W4_ERR_ALIGN;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const bool asym = scheme == W4_ASYM_GROUP;
    hipError_t e = w4::launch_dequant_weight(packed, scales, asym ? zeros : nullptr, K, N,
                                             group_size, delta, work, st);
    if (e != hipSuccess) return W4_ERR_HIP;
    if (asym)
        return launched("merge_delta",
                        w4::launch_quant_weight_asym(work, K, N, group_size, packed_out,
                                                     scales_out, zeros_out, st));
    return launched("merge_delta",
                    w4::launch_quant_weight_sym(work, K, N, packed_out, scales_out, st));
}

int a8_quantize_act(const float *X, int64_t M, int64_t K, int8_t *Xq, float *sx, void *stream) {
    if (!X || !Xq || !sx) return W4_ERR_NULL;
    if (M < 1 || K < 1 || M > 0x7FFFFFFF || K > ((int64_t)1 << 40) / M) return W4_ERR_SHAPE;
    if (!aligned(X, 4) || !aligned(sx, 4)) return W4_ERR_ALIGN;
    return launched("quant_act",
                    w4::launch_quant_act(
                        X, M, K, Xq, sx, false, reinterpret_cast<hipStream_t>(stream)));
}

size_t w4a8_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    if (!shape_ok(M, K, N)) return 0;
    return ws_bytes(M, K);
}

int w4a8_linear_act(const float *X, int64_t M, int64_t K, int64_t N, const uint8_t *packed,
                    const float *sw, const float *bias, int activation, float *Y,
                    void *workspace, size_t workspace_bytes, void *stream) {
    if (!X || !packed || !sw || !Y) return W4_ERR_NULL;
    if (!shape_ok(M, K, N)) return W4_ERR_SHAPE;
    if (activation != W4_ACT_NONE && activation != W4_ACT_RELU) return W4_ERR_ARG;
    if (!aligned(X, 4) || !aligned(sw, 4) || !aligned(Y, 4) || (bias && !aligned(bias, 4)))
        return W4_ERR_ALIGN;
    int rc = check_workspace(M, K, workspace, workspace_bytes);
    if (rc != W4_OK) return rc;
    return w4a8_dispatch(Src::FP32, false, X, nullptr, nullptr, packed, sw, bias, M, K, N, Y,
                         nullptr, workspace, workspace_bytes,
                         reinterpret_cast<hipStream_t>(stream), activation == W4_ACT_RELU);
}

int w4a8_linear_awq(const float *X, int64_t M, int64_t K, int64_t N, const uint8_t *packed,
                    const float *sw, const float *s, const float *bias, int activation, float *Y,
                    void *workspace, size_t workspace_bytes, void *stream) {
    if (!X || !packed || !sw || !s || !Y) return W4_ERR_NULL;
    if (!shape_ok(M, K, N)) return W4_ERR_SHAPE;
    if (activation != W4_ACT_NONE && activation != W4_ACT_RELU) return W4_ERR_ARG;
    if (!aligned(X, 4) || !aligned(sw, 4) || !aligned(Y, 4) || (bias && !aligned(bias, 4)))
        return W4_ERR_ALIGN;
    if (!aligned(s, 16)) return W4_ERR_ALIGN;
    int rc = check_workspace(M, K, workspace, workspace_bytes);
    if (rc != W4_OK) return rc;
    return w4a8_dispatch(Src::FP32, false, X, nullptr, nullptr, packed, sw, bias, M, K, N, Y,
                         nullptr, workspace, workspace_bytes,
                         reinterpret_cast<hipStream_t>(stream), activation == W4_ACT_RELU, s);
}

int awq_channel_scales(const float *Xcal, int64_t M, int64_t K, int alpha_num, int alpha_den,
                       float *s, void *stream) {
    if (!Xcal || !s) return W4_ERR_NULL;
    if (M < 1 || K < 1 || K > W4_MAX_K || M > ((int64_t)1 << 40) / K) return W4_ERR_SHAPE;
    if (alpha_num < 0 || alpha_num > 1024 || alpha_den < 1 || alpha_den > 1024) return W4_ERR_ARG;
    if (!aligned(Xcal, 4) || !aligned(s, 4)) return W4_ERR_ALIGN;
    return launched("awq_scales",
                    w4::launch_awq_scales(Xcal, M, K, alpha_num, alpha_den, s,
                                          reinterpret_cast<hipStream_t>(stream)));
}

int awq_fold_weight(const float *W, int64_t K, int64_t N, const float *s, float *W_out,
                    void *stream) {
    if (!W || !s || !W_out) return W4_ERR_NULL;
    if (!shape_ok(1, K, N)) return W4_ERR_SHAPE;
    if (!aligned(W, 4) || !aligned(s, 4) || !aligned(W_out, 4)) return W4_ERR_ALIGN;
    return launched("awq_fold",
                    w4::launch_awq_fold(W, K, N, s, W_out, reinterpret_cast<hipStream_t>(stream)));
}

int awq_quantize_act(const float *X, int64_t M, int64_t K, const float *s, int8_t *Xq, float *sx,
                     void *stream) {
    if (!X || !s || !Xq || !sx) return W4_ERR_NULL;
    if (M < 1 || K < 1 || M > 0x7FFFFFFF || K > ((int64_t)1 << 40) / M) return W4_ERR_SHAPE;
    if (!aligned(X, 4) || !aligned(sx, 4) || !aligned(s, 4)) return W4_ERR_ALIGN;
    return launched("awq_quant_act",
                    w4::launch_quant_act(X, M, K, Xq, sx, false,
                                         reinterpret_cast<hipStream_t>(stream), s));
}

int awq_scale_act_bf16(const uint16_t *X_bf16, int64_t M, int64_t K, const float *s,
                       uint16_t *X_out, void *stream) {
    if (!X_bf16 || !s || !X_out) return W4_ERR_NULL;
    if (M < 1 || K < 1 || K > ((int64_t)1 << 40) / M) return W4_ERR_SHAPE;
    if (!aligned(X_bf16, 2) || !aligned(X_out, 2) || !aligned(s, 4)) return W4_ERR_ALIGN;
    return launched("awq_scale_bf16",
                    w4::launch_awq_scale_bf16(X_bf16, M, K, s, X_out,
                                              reinterpret_cast<hipStream_t>(stream)));
}

int64_t w4_prepacked_weight_bytes(int64_t K, int64_t N) {
    if (!shape_ok(1, K, N) || K % 128 != 0) return 0;
    return ((N + 15) / 16) * 16 * (K / 2);
}

int w4_prepack_weights(const uint8_t *packed, int64_t K, int64_t N, uint8_t *wpp, void *stream) {
    if (!packed || !wpp) return W4_ERR_NULL;
    if (!shape_ok(1, K, N) || K % 128 != 0) return W4_ERR_SHAPE;
    if (!aligned(packed, 16) || !aligned(wpp, 16)) return W4_ERR_ALIGN;
    return launched("w4_prepack_weights",
                    w4::launch_w4_prepack_weights(
                        packed, K, N, wpp, reinterpret_cast<hipStream_t>(stream)));
}

int w4_unprepack_weights(const uint8_t *wpp, int64_t K, int64_t N, uint8_t *packed, void *stream) {
    if (!packed || !wpp) return W4_ERR_NULL;
    if (!shape_ok(1, K, N) || K % 128 != 0) return W4_ERR_SHAPE;
    if (!aligned(packed, 16) || !aligned(wpp, 16)) return W4_ERR_ALIGN;
    return launched("w4_unprepack_weights",
                    w4::launch_w4_unprepack_weights(wpp, K, N, packed,
                                                    reinterpret_cast<hipStream_t>(stream)));
}

int w4a8_linear_prepacked(const float *X, int64_t M, int64_t K, int64_t N, const uint8_t *wpp,
                          const float *sw, const float *bias, int activation, float *Y,
                          void *workspace, size_t workspace_bytes, void *stream) {
    if (!X || !wpp || !sw || !Y) return W4_ERR_NULL;
    if (!shape_ok(M, K, N) || K % 128 != 0) return W4_ERR_SHAPE;
    if (activation != W4_ACT_NONE && activation != W4_ACT_RELU) return W4_ERR_ARG;
    if (!aligned(X, 4) || !aligned(sw, 4) || !aligned(Y, 4) || (bias && !aligned(bias, 4)) ||
        !aligned(wpp, 16))
        return W4_ERR_ALIGN;
    int rc = check_workspace(M, K, workspace, workspace_bytes);
    if (rc != W4_OK) return rc;
    return w4a8_dispatch(Src::FP32, false, X, nullptr, nullptr, wpp, sw, bias, M, K, N, Y,
                         nullptr, workspace, workspace_bytes,
                         reinterpret_cast<hipStream_t>(stream), activation == W4_ACT_RELU,
                         nullptr, true);
}

int w4a8_linear(const float *X, int64_t M, int64_t K, int64_t N, const uint8_t *packed,
                const float *sw, const float *bias, float *Y, void *workspace,
                size_t workspace_bytes, void *stream) {
    return w4a8_linear_act(X, M, K, N, packed, sw, bias, W4_ACT_NONE, Y, workspace,
                           workspace_bytes, stream);
}

int w4a8_linear_noalloc(const float *X, int64_t M, int64_t K, int64_t N, const uint8_t *packed,
                        const float *sw, const float *bias, float *Y, void *stream) {
    if (!X || !packed || !sw || !Y) return W4_ERR_NULL;
    if (!shape_ok(M, K, N)) return W4_ERR_SHAPE;
    if (ws_bytes(M, K) > (size_t)W4_NOALLOC_SCRATCH_BYTES) return W4_ERR_SCRATCH;
    void *ws = nullptr;
    const int rc = scratch_address(&ws);
    if (rc != W4_OK) return rc;
    // the same dispatch and kernels as w4a8_linear, with the scratch array as
    // the workspace (every byte the kernels read from it is written first in
    // the same call, so nothing needs clearing)
    return w4a8_linear_act(X, M, K, N, packed, sw, bias, W4_ACT_NONE, Y, ws,
                           (size_t)W4_NOALLOC_SCRATCH_BYTES, stream);
}

int w4a8_linear_q(const int8_t *Xq, const float *sx, const uint8_t *packed, const float *sw,
                  const float *bias, int64_t M, int64_t K, int64_t N, float *Y, void *workspace,
                  size_t workspace_bytes, void *stream) {
    if (!Xq || !sx || !packed || !sw || !Y) return W4_ERR_NULL;
    if (!shape_ok(M, K, N)) return W4_ERR_SHAPE;
    if (!aligned(sx, 4) || !aligned(sw, 4) || !aligned(Y, 4) || (bias && !aligned(bias, 4)))
        return W4_ERR_ALIGN;
    int rc = check_workspace(M, K, workspace, workspace_bytes);
    if (rc != W4_OK) return rc;
    return w4a8_dispatch(Src::Q, false, nullptr, Xq, sx, packed, sw, bias, M, K, N, Y, nullptr,
                         workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream));
}

int w4a8_matmul_i32(const int8_t *Xq, const uint8_t *packed, int64_t M, int64_t K, int64_t N,
                    int32_t *acc, void *workspace, size_t workspace_bytes, void *stream) {
    if (!Xq || !packed || !acc) return W4_ERR_NULL;
    if (!shape_ok(M, K, N)) return W4_ERR_SHAPE;
    if (!aligned(acc, 4)) return W4_ERR_ALIGN;
    int rc = check_workspace(M, K, workspace, workspace_bytes);
    if (rc != W4_OK) return rc;
    return w4a8_dispatch(Src::Q, false, nullptr, Xq, nullptr, packed, nullptr, nullptr, M, K, N,
                         nullptr, acc, workspace, workspace_bytes,
                         reinterpret_cast<hipStream_t>(stream));
}

int w8_quantize_weight(const float *W, int64_t K, int64_t N, int8_t *Wq, float *sw,
                       void *stream) {
    if (!W || !Wq || !sw) return W4_ERR_NULL;
    if (!shape_ok(1, K, N)) return W4_ERR_SHAPE;
    if (!aligned(W, 4) || !aligned(sw, 4)) return W4_ERR_ALIGN;
    return launched("quant_weight_w8",
                    w4::launch_quant_weight_w8(
                        W, K, N, Wq, sw, reinterpret_cast<hipStream_t>(stream)));
}

size_t w8a8_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    if (!shape_ok(M, K, N)) return 0;
    return ws_bytes(M, K);
}

int w8a8_linear_act(const float *X, int64_t M, int64_t K, int64_t N, const int8_t *Wq,
                    const float *sw, const float *bias, int activation, float *Y,
                    void *workspace, size_t workspace_bytes, void *stream) {
    if (!X || !Wq || !sw || !Y) return W4_ERR_NULL;
    if (!shape_ok(M, K, N)) return W4_ERR_SHAPE;
    if (activation != W4_ACT_NONE && activation != W4_ACT_RELU) return W4_ERR_ARG;
    if (!aligned(X, 4) || !aligned(sw, 4) || !aligned(Y, 4) || (bias && !aligned(bias, 4)))
        return W4_ERR_ALIGN;
    int rc = check_workspace(M, K, workspace, workspace_bytes);
    if (rc != W4_OK) return rc;
    return w4a8_dispatch(Src::FP32, true, X, nullptr, nullptr,
                         reinterpret_cast<const uint8_t *>(Wq), sw, bias, M, K, N, Y, nullptr,
                         workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream),
                         activation == W4_ACT_RELU);
}

int w8a8_linear(const float *X, int64_t M, int64_t K, int64_t N, const int8_t *Wq,
                const float *sw, const float *bias, float *Y, void *workspace,
                size_t workspace_bytes, void *stream) {
    return w8a8_linear_act(X, M, K, N, Wq, sw, bias, W4_ACT_NONE, Y, workspace, workspace_bytes,
                           stream);
}

int w8a8_matmul_i32(const int8_t *Xq, const int8_t *Wq, int64_t M, int64_t K, int64_t N,
                    int32_t *acc, void *workspace, size_t workspace_bytes, void *stream) {
    if (!Xq || !Wq || !acc) return W4_ERR_NULL;
    if (!shape_ok(M, K, N)) return W4_ERR_SHAPE;
    if (!aligned(acc, 4)) return W4_ERR_ALIGN;
    int rc = check_workspace(M, K, workspace, workspace_bytes);
    if (rc != W4_OK) return rc;
    return w4a8_dispatch(Src::Q, true, nullptr, Xq, nullptr, reinterpret_cast<const uint8_t *>(Wq),
                         nullptr, nullptr, M, K, N, nullptr, acc, workspace, workspace_bytes,
                         reinterpret_cast<hipStream_t>(stream));
}

static bool prepacked_shape_ok(int64_t K, int64_t N, int64_t group_size) {
    return group_size == 128 && K % 512 == 0 && shape_ok(1, K, N);
}

int64_t w4a16_prepacked_weight_bytes(int64_t K, int64_t N) {
    if (!prepacked_shape_ok(K, N, 128)) return 0;
    return ((N + 15) / 16) * 16 * (K / 2);
}

int64_t w4a16_prepacked_table_floats(int64_t K, int64_t N) {
    if (!prepacked_shape_ok(K, N, 128)) return 0;
    return ((N + 15) / 16) * 16 * (K / 128) * 2;
}

int w4a16_prepack(const uint8_t *packed, const float *scales, const float *zeros, int64_t K,
                  int64_t N, int64_t group_size, uint8_t *wpp, float *szpp, void *stream) {
    if (!packed || !scales || !zeros || !wpp || !szpp) return W4_ERR_NULL;
    if (!prepacked_shape_ok(K, N, group_size)) return W4_ERR_SHAPE;
    if (!aligned(packed, 16) || !aligned(scales, 4) || !aligned(zeros, 4) || !aligned(wpp, 16) ||
        !aligned(szpp, 16))
        return W4_ERR_ALIGN;
    return launched("w4a16_prepack",
                    w4::launch_w4a16_prepack(packed, scales, zeros, K, N, wpp, szpp,
                                             reinterpret_cast<hipStream_t>(stream)));
}

int w4a16_unprepack(const uint8_t *wpp, const float *szpp, int64_t K, int64_t N,
                    int64_t group_size, uint8_t *packed, float *scales, float *zeros,
                    void *stream) {
    if (!packed || !scales || !zeros || !wpp || !szpp) return W4_ERR_NULL;
    if (!prepacked_shape_ok(K, N, group_size)) return W4_ERR_SHAPE;
    if (!aligned(packed, 16) || !aligned(scales, 4) || !aligned(zeros, 4) || !aligned(wpp, 16) ||
        !aligned(szpp, 16))
        return W4_ERR_ALIGN;
    return launched("w4a16_unprepack",
                    w4::launch_w4a16_unprepack(wpp, szpp, K, N, packed, scales, zeros,
                                               reinterpret_cast<hipStream_t>(stream)));
}

int w4a16_linear_prepacked(const uint16_t *X_bf16, int64_t M, int64_t K, int64_t N,
                           const uint8_t *wpp, const float *szpp, float *Y, void *stream) {
    if (!X_bf16 || !wpp || !szpp || !Y) return W4_ERR_NULL;
    if (!shape_ok(M, K, N) || !prepacked_shape_ok(K, N, 128)) return W4_ERR_SHAPE;
    if (!aligned(X_bf16, 16) || !aligned(wpp, 16) || !aligned(szpp, 16) || !aligned(Y, 4))
        return W4_ERR_ALIGN;
    return launched("w4a16_lds_prepacked",
                    w4::launch_w4a16_prepacked(X_bf16, M, K, N, wpp, szpp, Y,
                                               reinterpret_cast<hipStream_t>(stream)));
}

int w4a16_linear(const uint16_t *X_bf16, int64_t M, int64_t K, int64_t N, const uint8_t *packed,
                 const float *scales, const float *zeros, int64_t group_size, float *Y,
                 void *stream) {
    if (!X_bf16 || !packed || !scales || !zeros || !Y) return W4_ERR_NULL;
    if (!shape_ok(M, K, N)) return W4_ERR_SHAPE;
    if (group_size < 2 || group_size % 2 != 0 || K % group_size != 0) return W4_ERR_SHAPE;
    if (!aligned(X_bf16, 2) || !aligned(scales, 4) || !aligned(zeros, 4) || !aligned(Y, 4))
        return W4_ERR_ALIGN;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (w4::w4a16_lds_ok(K, group_size) && aligned(X_bf16, 16) && aligned(packed, 16) &&
        aligned(scales, 16) && aligned(zeros, 16)) {
        return launched("w4a16_lds",
                        w4::launch_w4a16_lds(X_bf16, M, K, N, packed, scales, zeros, Y, st));
    }
    if (w4::w4a16_fast_ok(M, K, N, group_size) && aligned(X_bf16, 16) && aligned(packed, 16)) {
        return launched("w4a16_mfma",
                        w4::launch_w4a16_mfma(
                            X_bf16, M, K, N, packed, scales, zeros, group_size, Y, st));
    }
    return launched("w4a16_generic",
                    w4::launch_w4a16_generic(
                        X_bf16, M, K, N, packed, scales, zeros, group_size, Y, st));
}

}  // extern "C"
