// Decode-shaped W4A8 products (few activation rows, many output channels):
// the packed int4 weights are streamed from HBM once with 128-bit loads and
// unpacked in registers (Keras INT4 guide, "How it works", steps 4-5).
//
//  * k_gemv_dot4  (M <= 4): VALU dot products (v_dot4_i32_i8).  The
//    activation quantization (step 3) is fused into the prologue, so one
//    launch runs steps 3-6.
//  * k_gemv_mfma  (M <= 64): int8 MFMA 16x16x64 with the weight operand
//    unpacked in registers; the activations come pre-quantized in P8 layout.
#include "common.h"
#include "kernels.h"

namespace w4 {

// ------------------------------------------------------------------ dot4
// Block = 256 threads = 16 output channels x 16 lanes.  Lane j of a channel
// streams the 16-byte chunks j, j+16, j+32, ... of that channel's packed row
// (one chunk = 32 codes), so a wave reads 4 rows x 256 contiguous bytes per
// load.  The quantized activations (P8 layout) sit in LDS.
constexpr int kDot4Rows = 16;
constexpr int kDot4Batch = 8;  // chunks in flight per lane

bool gemv_dot4_ok(int64_t M, int64_t K) {
    return M >= 1 && M <= 4 && K % 32 == 0 && M * K <= 48 * 1024;
}

template <int M, bool FUSED, Out OUT>
__global__ __launch_bounds__(256) void k_gemv_dot4(W4A8Args a) {
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ float red[4];
    __shared__ float sxs[4];
    int8_t *xs = reinterpret_cast<int8_t *>(smem);
    const int K = (int)a.K;
    const int64_t KB = a.K / 2;
    const int C = K / 32;  // chunks per row
    const int j = threadIdx.x & 15;
    const int64_t n = (int64_t)blockIdx.x * kDot4Rows + threadIdx.x / 16;
    const bool valid = n < a.N;
    const uint4 *prow = reinterpret_cast<const uint4 *>(a.packed + (valid ? n : 0) * KB);

    // Issue the first batch of weight loads before the prologue so their
    // latency overlaps the activation quantization.
    uint4 wb[kDot4Batch];
#pragma unroll
    for (int u = 0; u < kDot4Batch; ++u) {
        const int c = j + 16 * u;
        wb[u] = (valid && c < C) ? prow[c] : make_uint4(0, 0, 0, 0);
    }

    // Prologue: activations -> LDS in P8 layout, plus their row scales.
    const int ng = K / 8;
    if (FUSED) {
        for (int m = 0; m < M; ++m) {
            const float *row = a.X + (int64_t)m * K;
            const float4 *r4 = reinterpret_cast<const float4 *>(row);
            float amax = 0.0f;
            for (int i = threadIdx.x; i < K / 4; i += 256) {
                float4 v = r4[i];
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
            }
            amax = block_max(amax, red);
            const float s = (amax == 0.0f) ? 0.0f : amax / 127.0f;
            if (threadIdx.x == 0) sxs[m] = s;
            for (int g = threadIdx.x; g < ng; g += 256) {
                const float4 v0 = r4[2 * g], v1 = r4[2 * g + 1];
                uint2 p;
                p.x = pack4_i8(quant_code(v0.x, s, -128.f, 127.f), quant_code(v0.z, s, -128.f, 127.f),
                               quant_code(v1.x, s, -128.f, 127.f), quant_code(v1.z, s, -128.f, 127.f));
                p.y = pack4_i8(quant_code(v0.y, s, -128.f, 127.f), quant_code(v0.w, s, -128.f, 127.f),
                               quant_code(v1.y, s, -128.f, 127.f), quant_code(v1.w, s, -128.f, 127.f));
                *reinterpret_cast<uint2 *>(xs + m * K + 8 * g) = p;
            }
        }
    } else {
        for (int m = 0; m < M; ++m) {
            const uint2 *src = reinterpret_cast<const uint2 *>(a.Xq + (int64_t)m * K);
            for (int g = threadIdx.x; g < ng; g += 256) {
                uint2 v = src[g], p;
                natural_to_p8(v.x, v.y, p.x, p.y);
                *reinterpret_cast<uint2 *>(xs + m * K + 8 * g) = p;
            }
            if (threadIdx.x == 0) sxs[m] = (OUT == Out::Y) ? a.sx[m] : 0.0f;
        }
    }
    __syncthreads();

    int acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0;

    for (int base = 0; base < C; base += 16 * kDot4Batch) {
        uint4 cur[kDot4Batch];
#pragma unroll
        for (int u = 0; u < kDot4Batch; ++u) cur[u] = wb[u];
        if (base + 16 * kDot4Batch < C) {
#pragma unroll
            for (int u = 0; u < kDot4Batch; ++u) {
                const int c = base + 16 * kDot4Batch + j + 16 * u;
                wb[u] = (valid && c < C) ? prow[c] : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < kDot4Batch; ++u) {
            const int c = base + j + 16 * u;
            if (c < C) {
                const uint32_t l0 = lo16(cur[u].x), h0 = hi16(cur[u].x);
                const uint32_t l1 = lo16(cur[u].y), h1 = hi16(cur[u].y);
                const uint32_t l2 = lo16(cur[u].z), h2 = hi16(cur[u].z);
                const uint32_t l3 = lo16(cur[u].w), h3 = hi16(cur[u].w);
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const uint4 *xp = reinterpret_cast<const uint4 *>(xs + m * K + c * 32);
                    const uint4 x0 = xp[0], x1 = xp[1];
                    int t = acc[m];
                    t = __builtin_amdgcn_sdot4((int)l0, (int)x0.x, t, false);
                    t = __builtin_amdgcn_sdot4((int)h0, (int)x0.y, t, false);
                    t = __builtin_amdgcn_sdot4((int)l1, (int)x0.z, t, false);
                    t = __builtin_amdgcn_sdot4((int)h1, (int)x0.w, t, false);
                    t = __builtin_amdgcn_sdot4((int)l2, (int)x1.x, t, false);
                    t = __builtin_amdgcn_sdot4((int)h2, (int)x1.y, t, false);
                    t = __builtin_amdgcn_sdot4((int)l3, (int)x1.z, t, false);
                    t = __builtin_amdgcn_sdot4((int)h3, (int)x1.w, t, false);
                    acc[m] = t;
                }
            }
        }
    }

#pragma unroll
    for (int m = 0; m < M; ++m) {
        int t = acc[m];
        t += __shfl_xor(t, 8, kWave);
        t += __shfl_xor(t, 4, kWave);
        t += __shfl_xor(t, 2, kWave);
        t += __shfl_xor(t, 1, kWave);
        acc[m] = t >> 4;  // undo the x16 of the unpacked weights (exact)
    }
    if (j == 0 && valid) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            if (OUT == Out::I32)
                a.acc[(int64_t)m * a.N + n] = acc[m];
            else
                a.Y[(int64_t)m * a.N + n] = dequant(acc[m], sxs[m], a.sw[n], a.bias, (int)n);
        }
    }
}

template <int M, bool FUSED, Out OUT>
static void go_dot4(const W4A8Args &a, hipStream_t st) {
    dim3 grid((unsigned)((a.N + kDot4Rows - 1) / kDot4Rows));
    hipLaunchKernelGGL((k_gemv_dot4<M, FUSED, OUT>), grid, dim3(256), (size_t)(M * a.K), st, a);
}

template <int M>
static void go_dot4_m(const W4A8Args &a, hipStream_t st) {
    if (a.out == Out::I32)
        go_dot4<M, false, Out::I32>(a, st);
    else if (a.X)
        go_dot4<M, true, Out::Y>(a, st);
    else
        go_dot4<M, false, Out::Y>(a, st);
}

hipError_t launch_gemv_dot4(const W4A8Args &a, hipStream_t st) {
    switch (a.M) {
        case 1: go_dot4_m<1>(a, st); break;
        case 2: go_dot4_m<2>(a, st); break;
        case 3: go_dot4_m<3>(a, st); break;
        default: go_dot4_m<4>(a, st); break;
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------ MFMA
// Block = 4 waves that split K into quarters and cover the same 16*NB output
// channels; the partial int32 sums are added through LDS at the end.
// Per 128-k step a lane loads 16 packed bytes (32 codes) of one channel:
//   lane l: channel n0 + 16*nb + l%16, codes k = 128*s + 32*(l/16) + [0, 32)
// and the matching 2 x 16 P8 activation bytes of row 16*mb + l%16, which
// feed two v_mfma_i32_16x16x64_i8 (the first 16 and the last 16 codes of each
// lane).  The weight and activation operands use identical k slots per lane,
// so the order in which the MFMA consumes the slots does not matter.
// Accumulator layout (16x16 i32): lane l holds rows 4*(l/16)+i, column l%16.
template <int MB, int NB, int D, Out OUT>
__global__ __launch_bounds__(256) void k_gemv_mfma(W4A8Args a) {
    __shared__ v4i red[3][MB * NB][kWave];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int r16 = lane % 16, kq = lane / 16;
    const int64_t K = a.K, KB = a.K / 2, N = a.N, M = a.M;
    const int64_t S = K / 128;
    const int64_t s0 = S * wave / 4, s1 = S * (wave + 1) / 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * NB;

    const uint8_t *bp[NB];
    bool bv[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int64_t col = n0 + 16 * nb + r16;
        bv[nb] = col < N;
        bp[nb] = a.packed + (bv[nb] ? col : 0) * KB + kq * 16;
    }
    const int8_t *ap[MB];
    bool av[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int64_t row = 16 * mb + r16;
        av[mb] = row < M;
        ap[mb] = a.Xq + (av[mb] ? row : 0) * K + kq * 32;
    }

    v4i acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = v4i{0, 0, 0, 0};

    uint4 wbuf[D][NB];
#pragma unroll
    for (int d = 0; d < D; ++d)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            wbuf[d][nb] = (s0 + d < s1 && bv[nb])
                              ? *reinterpret_cast<const uint4 *>(bp[nb] + (s0 + d) * 64)
                              : make_uint4(0, 0, 0, 0);

    for (int64_t s = s0; s < s1; s += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int64_t ss = s + d;
            if (ss < s1) {
                uint4 x0[MB], x1[MB];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    if (av[mb]) {
                        const uint4 *xp = reinterpret_cast<const uint4 *>(ap[mb] + ss * 128);
                        x0[mb] = xp[0];
                        x1[mb] = xp[1];
                    } else {
                        x0[mb] = x1[mb] = make_uint4(0, 0, 0, 0);
                    }
                }
                uint4 w[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    w[nb] = wbuf[d][nb];
                    const int64_t sn = ss + D;
                    wbuf[d][nb] = (sn < s1 && bv[nb])
                                      ? *reinterpret_cast<const uint4 *>(bp[nb] + sn * 64)
                                      : make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const v4i b0 = {(int)lo16(w[nb].x), (int)hi16(w[nb].x), (int)lo16(w[nb].y),
                                    (int)hi16(w[nb].y)};
                    const v4i b1 = {(int)lo16(w[nb].z), (int)hi16(w[nb].z), (int)lo16(w[nb].w),
                                    (int)hi16(w[nb].w)};
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        const v4i a0 = {(int)x0[mb].x, (int)x0[mb].y, (int)x0[mb].z, (int)x0[mb].w};
                        const v4i a1 = {(int)x1[mb].x, (int)x1[mb].y, (int)x1[mb].z, (int)x1[mb].w};
                        acc[mb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, acc[mb][nb], 0, 0, 0);
                        acc[mb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, acc[mb][nb], 0, 0, 0);
                    }
                }
            }
        }
    }

    if (wave > 0) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) red[wave - 1][mb * NB + nb][lane] = acc[mb][nb];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            v4i t = acc[mb][nb] + red[0][mb * NB + nb][lane] + red[1][mb * NB + nb][lane] +
                    red[2][mb * NB + nb][lane];
            const int64_t col = n0 + 16 * nb + r16;
            if (col >= N) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row = 16 * mb + 4 * kq + i;
                if (row >= M) continue;
                const int v = t[i] >> 4;
                if (OUT == Out::I32)
                    a.acc[row * N + col] = v;
                else
                    a.Y[row * N + col] = dequant(v, a.sx[row], a.sw[col], a.bias, (int)col);
            }
        }
    }
}

template <int MB, int NB, int D>
static void go_mfma(const W4A8Args &a, hipStream_t st) {
    dim3 grid((unsigned)((a.N + 16 * NB - 1) / (16 * NB)));
    if (a.out == Out::I32)
        hipLaunchKernelGGL((k_gemv_mfma<MB, NB, D, Out::I32>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((k_gemv_mfma<MB, NB, D, Out::Y>), grid, dim3(256), 0, st, a);
}

hipError_t launch_gemv_mfma(const W4A8Args &a, hipStream_t st) {
    const int mb = (int)((a.M + 15) / 16);
    switch (mb) {
        case 1: go_mfma<1, 2, 4>(a, st); break;
        case 2: go_mfma<2, 2, 4>(a, st); break;
        case 3: go_mfma<3, 2, 2>(a, st); break;
        default: go_mfma<4, 2, 2>(a, st); break;
    }
    return hipGetLastError();
}

}  // namespace w4
