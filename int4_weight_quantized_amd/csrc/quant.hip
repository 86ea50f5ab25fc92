// Quantization kernels: symmetric per-channel int4 weights, asymmetric
// group-wise int4 weights and per-row dynamic int8 activations.
//
// Symmetric weights (Keras INT4 guide, "How it works", steps 1-2):
//   scale[n] = fl(max_k |W[k][n]| / 7), code = clamp(rne(fl(W / scale)), -8, 7).
// Asymmetric groups ("4-bit Integer Quantization for LLMs", quantization
// principle; "INT4" concept entry 4.1-4.2):
//   scale = fl(fl(max - min) / 15), zero = 0 - rne(fl(min / scale)),
//   code = clamp(rne(fl(W / scale)) + zero, 0, 15).
// Symmetric int8 weights (the INT8 path that the Keras guide's "How it works"
// says the INT4 path follows; "INT4" concept entry 4.1 with b = 8):
//   scale[n] = fl(max_k |W[k][n]| / 127), code = clamp(rne(fl(W / scale)), -128, 127),
//   stored one per byte, channel-major [N][K].
// Activations (Keras guide step 3): sx[m] = fl(max_k |X[m][k]| / 127),
//   Xq = clamp(rne(fl(X / sx)), -128, 127).
#include "common.h"
#include "kernels.h"

namespace w4 {

// ------------------------------------------------------------------ helpers
__global__ void k_fill_u32(uint32_t *p, int64_t n, uint32_t v) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// ---------------------------------------------------- symmetric int4 weights
// Pass 1: per-column absmax of a [krows x 64] slab, merged with an atomic max
// on the fp32 bit pattern (valid because every value is >= +0).
// Block: 256 threads = 64 columns x 4 row phases.
__global__ __launch_bounds__(256) void k_absmax_cols(const float *__restrict__ W, int64_t K,
                                                     int64_t N, int64_t krows,
                                                     uint32_t *__restrict__ amax) {
    __shared__ float red[4][64];
    const int c = threadIdx.x % 64, ph = threadIdx.x / 64;
    const int64_t col = (int64_t)blockIdx.x * 64 + c;
    const int64_t k0 = (int64_t)blockIdx.y * krows;
    const int64_t k1 = min(K, k0 + krows);
    float m = 0.0f;
    if (col < N) {
        for (int64_t k = k0 + ph; k < k1; k += 4) m = fmaxf(m, fabsf(W[k * N + col]));
    }
    red[ph][c] = m;
    __syncthreads();
    if (ph == 0 && col < N) {
        m = fmaxf(fmaxf(red[0][c], red[1][c]), fmaxf(red[2][c], red[3][c]));
        atomicMax(&amax[col], __float_as_uint(m));
    }
}

// Pass 2: codes of a [128 x 64] tile.  Thread (c, part) owns column c and the
// 32 k values part*32 .. part*32+31 of the tile (16 packed bytes, or 32 int8
// codes); loads are coalesced over the 64 columns of a wave.  `amax` still
// holds absmax bits here.
__global__ __launch_bounds__(256) void k_quant_w8_tile(const float *__restrict__ W, int64_t K,
                                                       int64_t N,
                                                       const uint32_t *__restrict__ amax,
                                                       int8_t *__restrict__ Wq) {
    const int c = threadIdx.x % 64, part = threadIdx.x / 64;
    const int64_t col = (int64_t)blockIdx.x * 64 + c;
    if (col >= N) return;
    const float a = __uint_as_float(amax[col]);
    const float s = (a == 0.0f) ? 0.0f : a / 127.0f;
    const int64_t kbeg = (int64_t)blockIdx.y * 128 + part * 32;
    uint32_t words[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t k = kbeg + 4 * j + b;
            const int q = (k < K) ? quant_code(W[k * N + col], s, -128.0f, 127.0f) : 0;
            v |= (uint32_t)(q & 0xFF) << (8 * b);
        }
        words[j] = v;
    }
    int8_t *dst = Wq + col * K + kbeg;
    if ((K % 16) == 0 && kbeg + 32 <= K && (reinterpret_cast<uintptr_t>(Wq) & 15) == 0) {
        reinterpret_cast<uint4 *>(dst)[0] = uint4{words[0], words[1], words[2], words[3]};
        reinterpret_cast<uint4 *>(dst)[1] = uint4{words[4], words[5], words[6], words[7]};
    } else {
        for (int j = 0; j < 32; ++j)
            if (kbeg + j < K) dst[j] = (int8_t)(words[j / 4] >> (8 * (j % 4)));
    }
}

__global__ __launch_bounds__(256) void k_quant_sym_tile(const float *__restrict__ W, int64_t K,
                                                        int64_t N,
                                                        const uint32_t *__restrict__ amax,
                                                        uint8_t *__restrict__ packed) {
    const int c = threadIdx.x % 64, part = threadIdx.x / 64;
    const int64_t col = (int64_t)blockIdx.x * 64 + c;
    if (col >= N) return;
    const int64_t KB = (K + 1) / 2;
    const float a = __uint_as_float(amax[col]);
    const float s = (a == 0.0f) ? 0.0f : a / 7.0f;
    const int64_t kbeg = (int64_t)blockIdx.y * 128 + part * 32;  // even
    uint8_t bytes[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int64_t k = kbeg + 2 * j;
        int q0 = 0, q1 = 0;
        if (k < K) q0 = quant_code(W[k * N + col], s, -8.0f, 7.0f);
        if (k + 1 < K) q1 = quant_code(W[(k + 1) * N + col], s, -8.0f, 7.0f);
        bytes[j] = (uint8_t)((q0 & 0xF) | ((q1 & 0xF) << 4));
    }
    const int64_t b0 = kbeg / 2;
    uint8_t *dst = packed + col * KB + b0;
    if ((KB % 16) == 0 && b0 + 16 <= KB) {
        uint4 v;
        v.x = bytes[0] | (bytes[1] << 8) | (bytes[2] << 16) | ((uint32_t)bytes[3] << 24);
        v.y = bytes[4] | (bytes[5] << 8) | (bytes[6] << 16) | ((uint32_t)bytes[7] << 24);
        v.z = bytes[8] | (bytes[9] << 8) | (bytes[10] << 16) | ((uint32_t)bytes[11] << 24);
        v.w = bytes[12] | (bytes[13] << 8) | (bytes[14] << 16) | ((uint32_t)bytes[15] << 24);
        *reinterpret_cast<uint4 *>(dst) = v;
    } else {
        for (int j = 0; j < 16; ++j)
            if (b0 + j < KB) dst[j] = bytes[j];
    }
}

// Pass 3: absmax bits -> scale (absmax / qmax, qmax = 7 or 127), in place.
__global__ void k_finalize_sym_scales(uint32_t *__restrict__ amax_to_scale, int64_t N,
                                      float qmax) {
    int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    float a = __uint_as_float(amax_to_scale[n]);
    float s = (a == 0.0f) ? 0.0f : a / qmax;
    reinterpret_cast<float *>(amax_to_scale)[n] = s;
}

// Passes 0-1 (shared by the int4 and int8 forms): clear and fill the absmax
// bits in the scale array.
static void absmax_pass(const float *W, int64_t K, int64_t N, uint32_t *amax, hipStream_t st) {
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, st, amax, N,
                       0u);
    const int64_t krows = 256;
    dim3 g1((unsigned)((N + 63) / 64), (unsigned)((K + krows - 1) / krows));
    hipLaunchKernelGGL(k_absmax_cols, g1, dim3(256), 0, st, W, K, N, krows, amax);
}

hipError_t launch_quant_weight_sym(const float *W, int64_t K, int64_t N, uint8_t *packed,
                                   float *sw, hipStream_t st) {
    uint32_t *amax = reinterpret_cast<uint32_t *>(sw);
    absmax_pass(W, K, N, amax, st);
    dim3 g2((unsigned)((N + 63) / 64), (unsigned)((K + 127) / 128));
    hipLaunchKernelGGL(k_quant_sym_tile, g2, dim3(256), 0, st, W, K, N, amax, packed);
    hipLaunchKernelGGL(k_finalize_sym_scales, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, st,
                       amax, N, 7.0f);
    return hipGetLastError();
}

hipError_t launch_quant_weight_w8(const float *W, int64_t K, int64_t N, int8_t *Wq, float *sw,
                                  hipStream_t st) {
    uint32_t *amax = reinterpret_cast<uint32_t *>(sw);
    absmax_pass(W, K, N, amax, st);
    dim3 g2((unsigned)((N + 63) / 64), (unsigned)((K + 127) / 128));
    hipLaunchKernelGGL(k_quant_w8_tile, g2, dim3(256), 0, st, W, K, N, amax, Wq);
    hipLaunchKernelGGL(k_finalize_sym_scales, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, st,
                       amax, N, 127.0f);
    return hipGetLastError();
}

// ------------------------------------------------ weight dequantization
// W[k][n] = fl(q * s[n]) (symmetric) or fl(fl(q - zp) * s) (asymmetric groups),
// then + delta[k][n] when a delta is given (the LoRA merge's dequantize-and-add
// step; Keras guide, "Limitations").  Thread (c, part) of a block owns column
// c of 64 and 32 consecutive k of a 128-k slab: it reads the column's 16
// packed bytes and writes W (and reads delta) coalesced over the 64 columns.
template <bool ASYM>
__global__ __launch_bounds__(256) void k_dequant_weight(const uint8_t *__restrict__ packed,
                                                        const float *__restrict__ scales,
                                                        const float *__restrict__ zeros,
                                                        const float *__restrict__ delta,
                                                        int64_t K, int64_t N, int64_t group,
                                                        float *__restrict__ W) {
    const int c = threadIdx.x % 64, part = threadIdx.x / 64;
    const int64_t n = (int64_t)blockIdx.x * 64 + c;
    if (n >= N) return;
    const int64_t KB = (K + 1) / 2;
    const int64_t kbeg = (int64_t)blockIdx.y * 128 + part * 32;
    if (kbeg >= K) return;
    const uint8_t *row = packed + n * KB + kbeg / 2;
    uint8_t bytes[16];
    if ((KB % 16) == 0 && kbeg / 2 + 16 <= KB && (reinterpret_cast<uintptr_t>(packed) & 15) == 0) {
        const uint4 v = *reinterpret_cast<const uint4 *>(row);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 16; ++j) bytes[j] = (uint8_t)(w[j / 4] >> (8 * (j % 4)));
    } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) bytes[j] = (kbeg / 2 + j < KB) ? row[j] : 0;
    }
    const int64_t G = ASYM ? K / group : 1;
    for (int j = 0; j < 32; ++j) {
        const int64_t k = kbeg + j;
        if (k >= K) break;
        const int nib = (j & 1) ? (bytes[j / 2] >> 4) : (bytes[j / 2] & 0xF);
        float w;
        if (ASYM) {
            const int64_t gi = n * G + k / group;
            const float d = (float)nib - zeros[gi];
            w = d * scales[gi];
        } else {
            w = (float)(nib >= 8 ? nib - 16 : nib) * scales[n];
        }
        if (delta) w = w + delta[k * N + n];
        W[k * N + n] = w;
    }
}

hipError_t launch_dequant_weight(const uint8_t *packed, const float *scales, const float *zeros,
                                 int64_t K, int64_t N, int64_t group, const float *delta,
                                 float *W, hipStream_t st) {
    dim3 g((unsigned)((N + 63) / 64), (unsigned)((K + 127) / 128));
    if (zeros)
        hipLaunchKernelGGL(k_dequant_weight<true>, g, dim3(256), 0, st, packed, scales, zeros,
                           delta, K, N, group, W);
    else
        hipLaunchKernelGGL(k_dequant_weight<false>, g, dim3(256), 0, st, packed, scales, zeros,
                           delta, K, N, group, W);
    return hipGetLastError();
}

// --------------------------------------------------- asymmetric group int4
// One block per (64 columns, one group).  Thread (c, part): column c, a
// contiguous quarter of the group's byte pairs.  The group size is even.
__global__ __launch_bounds__(256) void k_quant_asym(const float *__restrict__ W, int64_t K,
                                                    int64_t N, int64_t group,
                                                    uint8_t *__restrict__ packed,
                                                    float *__restrict__ scales,
                                                    float *__restrict__ zeros) {
    __shared__ float rlo[4][64], rhi[4][64];
    const int c = threadIdx.x % 64, part = threadIdx.x / 64;
    const int64_t col = (int64_t)blockIdx.x * 64 + c;
    const int64_t g = blockIdx.y;
    const int64_t G = K / group;
    const int64_t k0 = g * group;
    float lo = 0.0f, hi = 0.0f;
    if (col < N) {
        lo = hi = W[k0 * N + col];
        for (int64_t k = k0 + part; k < k0 + group; k += 4) {
            float w = W[k * N + col];
            lo = fminf(lo, w);
            hi = fmaxf(hi, w);
        }
    }
    rlo[part][c] = lo;
    rhi[part][c] = hi;
    __syncthreads();
    if (col >= N) return;
    lo = fminf(fminf(rlo[0][c], rlo[1][c]), fminf(rlo[2][c], rlo[3][c]));
    hi = fmaxf(fmaxf(rhi[0][c], rhi[1][c]), fmaxf(rhi[2][c], rhi[3][c]));
    float s;
    if (hi > lo) {
        float range = hi - lo;
        s = range / 15.0f;
    } else {
        s = (lo != 0.0f) ? fabsf(lo) : 1.0f;
    }
    const float zp = 0.0f - rintf(lo / s);
    if (part == 0) {
        scales[col * G + g] = s;
        zeros[col * G + g] = zp;
    }
    const int64_t KB = (K + 1) / 2;
    const int64_t npairs = group / 2;
    const int64_t per = (npairs + 3) / 4;
    const int64_t p0 = part * per, p1 = min(npairs, p0 + per);
    uint8_t *dst = packed + col * KB + k0 / 2;
    const bool vec = (per % 16 == 0) && (KB % 16 == 0) && ((k0 / 2) % 16 == 0);
    for (int64_t p = p0; p < p1; p += 16) {
        uint8_t bytes[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int64_t pp = p + j;
            uint8_t b = 0;
            if (pp < p1) {
                const int64_t k = k0 + 2 * pp;
                float r0 = rintf(W[k * N + col] / s) + zp;
                float r1 = rintf(W[(k + 1) * N + col] / s) + zp;
                int q0 = (int)fminf(fmaxf(r0, 0.0f), 15.0f);
                int q1 = (int)fminf(fmaxf(r1, 0.0f), 15.0f);
                b = (uint8_t)(q0 | (q1 << 4));
            }
            bytes[j] = b;
        }
        if (vec && p + 16 <= p1) {
            uint4 v;
            v.x = bytes[0] | (bytes[1] << 8) | (bytes[2] << 16) | ((uint32_t)bytes[3] << 24);
            v.y = bytes[4] | (bytes[5] << 8) | (bytes[6] << 16) | ((uint32_t)bytes[7] << 24);
            v.z = bytes[8] | (bytes[9] << 8) | (bytes[10] << 16) | ((uint32_t)bytes[11] << 24);
            v.w = bytes[12] | (bytes[13] << 8) | (bytes[14] << 16) | ((uint32_t)bytes[15] << 24);
            *reinterpret_cast<uint4 *>(dst + p) = v;
        } else {
            for (int j = 0; j < 16 && p + j < p1; ++j) dst[p + j] = bytes[j];
        }
    }
}

hipError_t launch_quant_weight_asym(const float *W, int64_t K, int64_t N, int64_t group,
                                    uint8_t *packed, float *scales, float *zeros, hipStream_t st) {
    dim3 g((unsigned)((N + 63) / 64), (unsigned)(K / group));
    hipLaunchKernelGGL(k_quant_asym, g, dim3(256), 0, st, W, K, N, group, packed, scales, zeros);
    return hipGetLastError();
}

// ------------------------------------------------------ int8 activations
// One block (256 threads) per row.  Pass 1: absmax; pass 2: codes, 8 per
// thread-step (re-reading the row from cache).  P8 = true writes the P8 layout
// (requires K % 8 == 0), otherwise the natural layout.
// With DIV the row is first divided by a per-column divisor, x' = fl(x / div[k])
// (the activation side of AWQ-style channel scaling, "INT4" concept entry 4.4).
// STEP (K % 16 == 0): the codes are stored chunk-major, [K/16][M][16] (the 16
// codes of one 16-k chunk of all rows together), the order in which the MFMA
// GEMV loads them: one load instruction reads 16 consecutive rows x 16 bytes
// of four chunks.
template <bool P8, bool DIV, bool STEP>
__global__ __launch_bounds__(256) void k_quant_act(const float *__restrict__ X, int64_t K,
                                                   int8_t *__restrict__ Xq,
                                                   float *__restrict__ sx,
                                                   const float *__restrict__ div) {
    args_now(X, K, Xq, sx, div);
    const int64_t rows = STEP ? arg_now((int64_t)gridDim.x) : 0;
    __shared__ float red[4];
    const int64_t m = blockIdx.x;
    const float *row = X + m * K;
    const bool vec = ((K % 4) == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0) &&
                     (!DIV || (reinterpret_cast<uintptr_t>(div) & 15) == 0);
    auto dv4 = [&](float4 v, int64_t k0) {
        if (DIV) {
            const float4 d = *reinterpret_cast<const float4 *>(div + k0);
            v.x = v.x / d.x;
            v.y = v.y / d.y;
            v.z = v.z / d.z;
            v.w = v.w / d.w;
        }
        return v;
    };
    auto ld = [&](int64_t k) { return DIV ? row[k] / div[k] : row[k]; };
    float a = 0.0f;
    if (vec) {
        const float4 *r4 = reinterpret_cast<const float4 *>(row);
        for (int64_t i = threadIdx.x; i < K / 4; i += 256) {
            float4 v = dv4(r4[i], 4 * i);
            a = fmaxf(a, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
    } else {
        for (int64_t i = threadIdx.x; i < K; i += 256) a = fmaxf(a, fabsf(ld(i)));
    }
    a = block_max<4>(a, red);
    const float s = (a == 0.0f) ? 0.0f : a / 127.0f;
    if (threadIdx.x == 0) sx[m] = s;
    int8_t *out = Xq + m * K;
    const int64_t ng = (K + 7) / 8;
    auto quantize = [&](auto code) {
        for (int64_t g = threadIdx.x; g < ng; g += 256) {
            const int64_t k0 = g * 8;
            int q[8];
            if (vec && k0 + 8 <= K) {
                const float4 v0 = dv4(reinterpret_cast<const float4 *>(row + k0)[0], k0);
                const float4 v1 = dv4(reinterpret_cast<const float4 *>(row + k0)[1], k0 + 4);
                q[0] = code(v0.x);
                q[1] = code(v0.y);
                q[2] = code(v0.z);
                q[3] = code(v0.w);
                q[4] = code(v1.x);
                q[5] = code(v1.y);
                q[6] = code(v1.z);
                q[7] = code(v1.w);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) q[j] = (k0 + j < K) ? code(ld(k0 + j)) : 0;
            }
            if (STEP) {
                uint2 v;
                if (P8) {
                    v.x = pack4_i8(q[0], q[2], q[4], q[6]);
                    v.y = pack4_i8(q[1], q[3], q[5], q[7]);
                } else {
                    v.x = pack4_i8(q[0], q[1], q[2], q[3]);
                    v.y = pack4_i8(q[4], q[5], q[6], q[7]);
                }
                *reinterpret_cast<uint2 *>(Xq + (k0 / 16) * (rows * 16) + m * 16 + k0 % 16) = v;
            } else if (P8) {
                uint2 v;
                v.x = pack4_i8(q[0], q[2], q[4], q[6]);
                v.y = pack4_i8(q[1], q[3], q[5], q[7]);
                *reinterpret_cast<uint2 *>(out + k0) = v;
            } else if ((K % 8) == 0 && (reinterpret_cast<uintptr_t>(Xq) & 7) == 0) {
                uint2 v;
                v.x = pack4_i8(q[0], q[1], q[2], q[3]);
                v.y = pack4_i8(q[4], q[5], q[6], q[7]);
                *reinterpret_cast<uint2 *>(out + k0) = v;
            } else {
                for (int j = 0; j < 8 && k0 + j < K; ++j) out[k0 + j] = (int8_t)q[j];
            }
        }
    };
    const RowScale q = row_scale(s);
    quantize([&](float v) { return quant_code_row(v, q); });
}

// Register-resident variant for 16-byte aligned rows with K % 8 == 0 and
// K <= 2048 * NG: thread t owns the 8-groups t, t + 256, ... of its row, issues
// all of their loads at once, and keeps them in registers between the absmax
// and the code pass, so the row is read from memory once.  Same codes, scales
// and layouts as k_quant_act.
template <bool P8, bool DIV, bool STEP, int NG>
__global__ __launch_bounds__(256) void k_quant_act_reg(const float *__restrict__ X, int64_t K,
                                                       int8_t *__restrict__ Xq,
                                                       float *__restrict__ sx,
                                                       const float *__restrict__ div) {
    args_now(X, K, Xq, sx, div);
    const int64_t rows = STEP ? arg_now((int64_t)gridDim.x) : 0;
    __shared__ float red[4];
    const int64_t m = blockIdx.x;
    const float *row = X + m * K;
    const int ng = (int)(K / 8);
    float4 v[NG][2];
#pragma unroll
    for (int u = 0; u < NG; ++u) {
        const int g = threadIdx.x + 256 * u;
        if (g < ng) {
            v[u][0] = reinterpret_cast<const float4 *>(row + 8 * g)[0];
            v[u][1] = reinterpret_cast<const float4 *>(row + 8 * g)[1];
        } else {
            v[u][0] = v[u][1] = float4{0.f, 0.f, 0.f, 0.f};
        }
    }
    if (DIV) {
#pragma unroll
        for (int u = 0; u < NG; ++u) {
            const int g = threadIdx.x + 256 * u;
            if (g < ng) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float4 d = reinterpret_cast<const float4 *>(div + 8 * g)[h];
                    v[u][h].x = v[u][h].x / d.x;
                    v[u][h].y = v[u][h].y / d.y;
                    v[u][h].z = v[u][h].z / d.z;
                    v[u][h].w = v[u][h].w / d.w;
                }
            }
        }
    }
    float a = 0.0f;
#pragma unroll
    for (int u = 0; u < NG; ++u)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            a = fmaxf(a, fmaxf(fmaxf(fabsf(v[u][h].x), fabsf(v[u][h].y)),
                               fmaxf(fabsf(v[u][h].z), fabsf(v[u][h].w))));
    // row absmax: integer DPP max of the non-negative values' bits in each
    // wave, then the 4 waves through LDS
    a = wave_max_nonneg(a);
    if ((threadIdx.x % kWave) == 0) red[threadIdx.x / kWave] = a;
    __syncthreads();
    a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = (a == 0.0f) ? 0.0f : div127(a);
    if (threadIdx.x == 0) sx[m] = s;
    auto quantize = [&](auto code) {
#pragma unroll
        for (int u = 0; u < NG; ++u) {
            const int g = threadIdx.x + 256 * u;
            if (g >= ng) continue;
            const float4 v0 = v[u][0], v1 = v[u][1];
            uint2 p;
            if (P8) {
                p.x = pack4_i8(code(v0.x), code(v0.z), code(v1.x), code(v1.z));
                p.y = pack4_i8(code(v0.y), code(v0.w), code(v1.y), code(v1.w));
            } else {
                p.x = pack4_i8(code(v0.x), code(v0.y), code(v0.z), code(v0.w));
                p.y = pack4_i8(code(v1.x), code(v1.y), code(v1.z), code(v1.w));
            }
            const int64_t k0 = 8 * (int64_t)g;
            int8_t *dst = STEP ? Xq + (k0 / 16) * (rows * 16) + m * 16 + k0 % 16
                               : Xq + m * K + k0;
            *reinterpret_cast<uint2 *>(dst) = p;
        }
    };
    if (s >= kFastQuotientMinScale) {  // row-uniform
        // correctly rounded quotient without a division, rounded by one add
        // (|x / s| <= 127.5 for every value of the row)
        const float rs = 1.0f / s;
        quantize([&](float x) { return (int)code_in_low_byte(quotient_rn(x, s, rs)); });
    } else {  // zero or tiny scale
        const RowScale q = row_scale(s);
        quantize([&](float x) { return quant_code_row(x, q); });
    }
}

template <bool P8, bool DIV, bool STEP>
static bool go_quant_act_reg(const float *X, int64_t M, int64_t K, int8_t *Xq, float *sx,
                             hipStream_t st, const float *div) {
    const bool aligned = (reinterpret_cast<uintptr_t>(X) & 15) == 0 &&
                         (reinterpret_cast<uintptr_t>(Xq) & 7) == 0 &&
                         (!DIV || (reinterpret_cast<uintptr_t>(div) & 15) == 0);
    if (!aligned || K % 8 != 0 || K > 2048 * 8) return false;
    const dim3 g((unsigned)M), b(256);
    if (K <= 2048)
        hipLaunchKernelGGL((k_quant_act_reg<P8, DIV, STEP, 1>), g, b, 0, st, X, K, Xq, sx, div);
    else if (K <= 4096)
        hipLaunchKernelGGL((k_quant_act_reg<P8, DIV, STEP, 2>), g, b, 0, st, X, K, Xq, sx, div);
    else if (K <= 8192)
        hipLaunchKernelGGL((k_quant_act_reg<P8, DIV, STEP, 4>), g, b, 0, st, X, K, Xq, sx, div);
    else
        hipLaunchKernelGGL((k_quant_act_reg<P8, DIV, STEP, 8>), g, b, 0, st, X, K, Xq, sx, div);
    return true;
}

template <bool P8, bool STEP>
static void go_quant_act(const float *X, int64_t M, int64_t K, int8_t *Xq, float *sx,
                         hipStream_t st, const float *div) {
    if (div ? go_quant_act_reg<P8, true, STEP>(X, M, K, Xq, sx, st, div)
            : go_quant_act_reg<P8, false, STEP>(X, M, K, Xq, sx, st, div))
        return;
    const dim3 g((unsigned)M), b(256);
    if (div)
        hipLaunchKernelGGL((k_quant_act<P8, true, STEP>), g, b, 0, st, X, K, Xq, sx, div);
    else
        hipLaunchKernelGGL((k_quant_act<P8, false, STEP>), g, b, 0, st, X, K, Xq, sx, div);
}

hipError_t launch_quant_act(const float *X, int64_t M, int64_t K, int8_t *Xq, float *sx, bool p8,
                            hipStream_t st, const float *div, bool step) {
    if (step) {
        if (p8)
            go_quant_act<true, true>(X, M, K, Xq, sx, st, div);
        else
            go_quant_act<false, true>(X, M, K, Xq, sx, st, div);
    } else {
        if (p8)
            go_quant_act<true, false>(X, M, K, Xq, sx, st, div);
        else
            go_quant_act<false, false>(X, M, K, Xq, sx, st, div);
    }
    return hipGetLastError();
}

// ------------------------------------------ AWQ-style channel scaling
// ("INT4" concept entry, section 4.4.)  Channel magnitude a_k = max over the
// calibration rows of |x| (the column-absmax pass above, with the rows of Xcal
// as its K); E_k = floor(log2 a_k) from the fp32 encoding (-150 for a_k = 0);
// E_med = the lower median of E over the channels; s_k = 2^e_k with
// e_k = min(24, max(0, floor(alpha (E_k - E_med)))).  One block: an LDS
// histogram of E (278 bins), a serial scan for the median, then the scales.
__device__ __forceinline__ int floor_log2_bits(uint32_t b) {
    const uint32_t ex = (b >> 23) & 0xFF, man = b & 0x7FFFFF;
    if (ex) return (int)ex - 127;
    if (man) return (31 - __builtin_clz(man)) - 149;  // subnormal
    return -150;                                     // zero
}

__global__ __launch_bounds__(1024) void k_awq_scales(uint32_t *__restrict__ amax_to_s,
                                                     int64_t K, int num, int den) {
    constexpr int kBins = 278;  // E in [-150, 127]
    __shared__ int hist[kBins];
    __shared__ int med;
    for (int i = threadIdx.x; i < kBins; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int64_t k = threadIdx.x; k < K; k += blockDim.x)
        atomicAdd(&hist[floor_log2_bits(amax_to_s[k]) + 150], 1);
    __syncthreads();
    if (threadIdx.x == 0) {
        const int64_t t = (K - 1) / 2;  // 0-based rank of the lower median
        int64_t c = 0;
        int b = 0;
        for (; b < kBins; ++b) {
            c += hist[b];
            if (c > t) break;
        }
        med = b - 150;
    }
    __syncthreads();
    for (int64_t k = threadIdx.x; k < K; k += blockDim.x) {
        const int d = floor_log2_bits(amax_to_s[k]) - med;
        int e = d > 0 ? (d * num) / den : 0;
        e = e > 24 ? 24 : e;
        amax_to_s[k] = (uint32_t)(127 + e) << 23;
    }
}

hipError_t launch_awq_scales(const float *Xcal, int64_t M, int64_t K, int num, int den, float *s,
                             hipStream_t st) {
    uint32_t *amax = reinterpret_cast<uint32_t *>(s);
    absmax_pass(Xcal, M, K, amax, st);
    hipLaunchKernelGGL(k_awq_scales, dim3(1), dim3(1024), 0, st, amax, K, num, den);
    return hipGetLastError();
}

// W'[k][n] = fl(W[k][n] * s[k]) (in place allowed).
__global__ void k_awq_fold(const float *__restrict__ W, int64_t K, int64_t N,
                           const float *__restrict__ s, float *__restrict__ Wout) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < K * N; i += stride)
        Wout[i] = W[i] * s[i / N];
}

static unsigned stride_blocks(int64_t n) {
    const int64_t b = (n + 255) / 256;
    return (unsigned)(b < (1 << 20) ? b : (1 << 20));
}

hipError_t launch_awq_fold(const float *W, int64_t K, int64_t N, const float *s, float *Wout,
                           hipStream_t st) {
    hipLaunchKernelGGL(k_awq_fold, dim3(stride_blocks(K * N)), dim3(256), 0, st, W, K, N, s, Wout);
    return hipGetLastError();
}

// bf16 activations divided by s: bf16_rne(fl(float(x) / s[k])).
__global__ void k_awq_scale_bf16(const uint16_t *__restrict__ X, int64_t M, int64_t K,
                                 const float *__restrict__ s, uint16_t *__restrict__ Xout) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < M * K; i += stride) {
        const float x = __uint_as_float((uint32_t)X[i] << 16);
        const float v = x / s[i % K];
        uint32_t u = __float_as_uint(v);
        if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) {
            Xout[i] = (uint16_t)((u >> 16) | 0x0040u);  // NaN stays a quiet NaN
            continue;
        }
        u += 0x7FFFu + ((u >> 16) & 1u);
        Xout[i] = (uint16_t)(u >> 16);
    }
}

hipError_t launch_awq_scale_bf16(const uint16_t *X, int64_t M, int64_t K, const float *s,
                                 uint16_t *Xout, hipStream_t st) {
    hipLaunchKernelGGL(k_awq_scale_bf16, dim3(stride_blocks(M * K)), dim3(256), 0, st, X, M, K, s,
                       Xout);
    return hipGetLastError();
}

// Natural int8 [M][K] -> P8 layout (K % 8 == 0, 8-byte aligned input).
// (With STEP: into the chunk-major order of k_quant_act<.., STEP>; P8 = false
// only moves the 8-byte groups.)
template <bool P8, bool STEP>
__global__ void k_to_p8(const int8_t *__restrict__ in, int64_t M, int64_t K,
                        int8_t *__restrict__ out) {
    args_now(in, M, K, out);
    const int64_t total8 = M * K / 8;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total8) return;
    uint2 v = reinterpret_cast<const uint2 *>(in)[i];
    uint2 r = v;
    if (P8) natural_to_p8(v.x, v.y, r.x, r.y);
    if (STEP) {
        const int64_t m = i / (K / 8), k0 = (i % (K / 8)) * 8;
        *reinterpret_cast<uint2 *>(out + (k0 / 16) * (M * 16) + m * 16 + k0 % 16) = r;
    } else {
        reinterpret_cast<uint2 *>(out)[i] = r;
    }
}

hipError_t launch_to_p8(const int8_t *Xq, int64_t M, int64_t K, int8_t *out, hipStream_t st,
                        bool p8, bool step) {
    const int64_t total8 = M * K / 8;
    const dim3 g((unsigned)((total8 + 255) / 256)), b(256);
    if (step) {
        if (p8)
            hipLaunchKernelGGL((k_to_p8<true, true>), g, b, 0, st, Xq, M, K, out);
        else
            hipLaunchKernelGGL((k_to_p8<false, true>), g, b, 0, st, Xq, M, K, out);
    } else {
        hipLaunchKernelGGL((k_to_p8<true, false>), g, b, 0, st, Xq, M, K, out);
    }
    return hipGetLastError();
}

}  // namespace w4
