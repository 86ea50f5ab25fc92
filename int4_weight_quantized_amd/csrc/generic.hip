// Shape-agnostic kernels: any M, K, N and alignment (for example the Keras
// guide's toy model, K = 10 and K = 32).  One thread per output element.
// W4A8 and W8A8 products: exact int32 sums, then the step-6 dequantization.
#include "common.h"
#include "kernels.h"

namespace w4 {

__device__ __forceinline__ int signed_nibble(const uint8_t *row, int64_t k) {
    const int b = row[k >> 1];
    const int nib = (k & 1) ? (b >> 4) : (b & 0xF);
    return nib >= 8 ? nib - 16 : nib;
}

// W4A8: exact int32 sum of Xq (natural layout) times the signed codes, then
// the dequantization epilogue or the raw accumulator.
__global__ __launch_bounds__(256) void k_w4a8_generic(const int8_t *__restrict__ Xq,
                                                      const float *__restrict__ sx,
                                                      const uint8_t *__restrict__ packed,
                                                      const float *__restrict__ sw,
                                                      const float *__restrict__ bias,
                                                      float *__restrict__ Y,
                                                      int32_t *__restrict__ accout, int64_t M,
                                                      int64_t K, int64_t N, bool relu) {
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    const uint8_t *row = packed + n * ((K + 1) / 2);
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        const int8_t *x = Xq + m * K;
        int acc = 0;
        for (int64_t k = 0; k < K; ++k) acc += (int)x[k] * signed_nibble(row, k);
        if (accout)
            accout[m * N + n] = acc;
        else
            Y[m * N + n] = relu_if(dequant(acc, sx[m], sw[n], bias, (int)n), relu);
    }
}

// W8A8: the same with int8 codes, one per byte (row n holds K bytes).
__global__ __launch_bounds__(256) void k_w8a8_generic(const int8_t *__restrict__ Xq,
                                                      const float *__restrict__ sx,
                                                      const int8_t *__restrict__ Wq,
                                                      const float *__restrict__ sw,
                                                      const float *__restrict__ bias,
                                                      float *__restrict__ Y,
                                                      int32_t *__restrict__ accout, int64_t M,
                                                      int64_t K, int64_t N, bool relu) {
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    const int8_t *row = Wq + n * K;
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        const int8_t *x = Xq + m * K;
        int acc = 0;
        for (int64_t k = 0; k < K; ++k) acc += (int)x[k] * (int)row[k];
        if (accout)
            accout[m * N + n] = acc;
        else
            Y[m * N + n] = relu_if(dequant(acc, sx[m], sw[n], bias, (int)n), relu);
    }
}

hipError_t launch_w4a8_generic(const W4A8Args &a, hipStream_t st) {
    dim3 g((unsigned)((a.N + 255) / 256), (unsigned)(a.M < 65535 ? a.M : 65535));
    if (a.w8)
        launch_main(k_w8a8_generic, g, dim3(256), 0, st, a.Xq, a.sx,
                    reinterpret_cast<const int8_t *>(a.packed), a.sw, a.bias, a.Y,
                    a.out == Out::I32 ? a.acc : nullptr, a.M, a.K, a.N, a.relu);
    else
        launch_main(k_w4a8_generic, g, dim3(256), 0, st, a.Xq, a.sx, a.packed, a.sw, a.bias, a.Y,
                    a.out == Out::I32 ? a.acc : nullptr, a.M, a.K, a.N, a.relu);
    return hipGetLastError();
}

// W4A16: w' = bf16(fl(fl(float(q) - zero) * scale)); fp32 sum in k order.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

__global__ __launch_bounds__(256) void k_w4a16_generic(const uint16_t *__restrict__ X,
                                                       const uint8_t *__restrict__ packed,
                                                       const float *__restrict__ scales,
                                                       const float *__restrict__ zeros,
                                                       float *__restrict__ Y, int64_t M,
                                                       int64_t K, int64_t N, int64_t group) {
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    const int64_t G = K / group;
    const uint8_t *row = packed + n * ((K + 1) / 2);
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
    const uint16_t *x = X + m * K;
    float acc = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        const int b = row[k >> 1];
        const int q = (k & 1) ? (b >> 4) : (b & 0xF);
        const float s = scales[n * G + k / group];
        const float zp = zeros[n * G + k / group];
        const float d = (float)q - zp;
        const float w = d * s;
        const float wb = (float)(__bf16)w;
        const float p = bf16_bits_to_f32(x[k]) * wb;
        acc = acc + p;
    }
    Y[m * N + n] = acc;
    }
}

hipError_t launch_w4a16_generic(const uint16_t *X, int64_t M, int64_t K, int64_t N,
                                const uint8_t *packed, const float *scales, const float *zeros,
                                int64_t group, float *Y, hipStream_t st) {
    dim3 g((unsigned)((N + 255) / 256), (unsigned)(M < 65535 ? M : 65535));
    launch_main(k_w4a16_generic, g, dim3(256), 0, st, X, packed, scales, zeros, Y, M, K, N, group);
    return hipGetLastError();
}

}  // namespace w4
