// Device helpers shared by the gfx950 kernels of the W4A8 / W4A16 linear layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

constexpr int kWave = 64;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Max over the whole block (blockDim.x a multiple of 64); `red` is LDS with
// one float per wave.  Every thread gets the result.
__device__ __forceinline__ float block_max(float v, float *red) {
    v = wave_max(v);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x % kWave) == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < (int)(blockDim.x / kWave); ++i) r = fmaxf(r, red[i]);
    __syncthreads();
    return r;
}

// ------------------------------------------------------------- quantization
// round-half-to-even of a correctly rounded fp32 quotient, limited to [lo, hi];
// a zero scale gives code 0.
__device__ __forceinline__ int quant_code(float v, float s, float lo, float hi) {
    if (s == 0.0f) return 0;
    float t = v / s;  // IEEE division (no fast-math in this build)
    float r = rintf(t);
    r = fminf(fmaxf(r, lo), hi);
    return (int)r;
}

// ------------------------------------------------------------------ unpack
// A packed dword holds 8 signed nibbles for k = 0..7 of a group of 8 (byte i:
// k = 2i low nibble, k = 2i+1 high nibble).  Moving each nibble to the top of
// its byte yields int8 lanes equal to 16*code exactly (two's complement), so
// products can run on int8 hardware and the sum is divided by 16 at the end.
//   lo16: bytes = 16*code for k = 0, 2, 4, 6
//   hi16: bytes = 16*code for k = 1, 3, 5, 7
__device__ __forceinline__ uint32_t lo16(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t hi16(uint32_t w) { return w & 0xF0F0F0F0u; }

// The "P8" activation layout pairs with lo16/hi16: inside every group of 8
// consecutive k the int8 values are stored as [x0 x2 x4 x6 | x1 x3 x5 x7], so
// the even and odd halves line up with lo16 and hi16 of the weight dword.
__device__ __forceinline__ void natural_to_p8(uint32_t lo, uint32_t hi, uint32_t &ev,
                                              uint32_t &od) {
    ev = (lo & 0xFFu) | ((lo >> 8) & 0xFF00u) | ((hi & 0xFFu) << 16) | ((hi << 8) & 0xFF000000u);
    od = ((lo >> 8) & 0xFFu) | ((lo >> 16) & 0xFF00u) | ((hi << 8) & 0xFF0000u) | (hi & 0xFF000000u);
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
           ((uint32_t)(d & 0xFF) << 24);
}

// ---------------------------------------------------------------- epilogue
// Dequantize one int32 accumulator: fl(fl(float(acc)) * fl(sx * sw)) then
// + bias, each step rounded separately (this library is built without
// floating-point contraction).
__device__ __forceinline__ float dequant(int acc, float sx, float sw, const float *bias, int n) {
    float s = sx * sw;
    float y = (float)acc * s;
    if (bias) y = y + bias[n];
    return y;
}

// Map a linear block index to a tile index so that the blocks the hardware
// places on one XCD (consecutive ids go round-robin over the 8 XCDs) get a
// contiguous range of tiles and share that XCD's L2.
__device__ __forceinline__ int xcd_swizzle(int bid, int nblocks) {
    constexpr int kXcd = 8;
    if (nblocks % kXcd != 0) return bid;
    const int per = nblocks / kXcd;
    return (bid % kXcd) * per + bid / kXcd;
}

}  // namespace w4
