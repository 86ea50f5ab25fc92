// Measurement helpers (not part of the method): the two platform references
// the layer's timings are read against.
//
//  * k_probe_empty: a kernel that does nothing, launched with a chosen grid;
//    its duration in a graph of back-to-back launches is the fixed cost every
//    launch pays (dispatch, wave launch, completion).
//  * k_probe_read: a plain streaming read of `bytes` (16-byte non-temporal
//    buffer loads, 4 per thread, whole 64-byte pieces per quarter-wave), with
//    one conditional store so the loads are kept; the best a kernel that only
//    reads those bytes once can do.
//  * k_probe_write: a plain streaming write of `bytes` (16-byte non-temporal
//    buffer stores, 4 per thread, the same pattern as the read); the best a
//    kernel that only writes those bytes once can do (the prefill GEMM's
//    fp32 output, for one).
//  * k_probe_mfma: back-to-back int8 MFMAs on constant or caller-given
//    (e.g. random) operands, timed with the shader clock and the
//    constant-rate clock: the clock the matrix units run at under that load
//    on this machine, and their rate on such operands.
#include "common.h"
#include "kernels.h"

namespace w4 {

__global__ __launch_bounds__(256) void k_probe_empty() {}

constexpr int kProbeUnroll = 4;  // 16-byte loads per thread

__global__ __launch_bounds__(256) void k_probe_read(const uint8_t *__restrict__ src, int64_t bytes,
                                                   uint32_t *__restrict__ sink) {
    const auto r = make_rsrc(src, bytes);
    const int64_t base = ((int64_t)blockIdx.x * kProbeUnroll * 256) * 16;
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int i = 0; i < kProbeUnroll; ++i) {
        const int64_t off = base + ((int64_t)i * 256 + threadIdx.x) * 16;
        v[i] = bload16_nt(r, off < bytes ? (int)off : kOOB);
    }
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < kProbeUnroll; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    if (x == 0x9E3779B9u) sink[blockIdx.x % 64] = x;  // data-dependent: keeps the loads
}

__global__ __launch_bounds__(256) void k_probe_write(uint8_t *__restrict__ dst, int64_t bytes,
                                                    uint32_t value) {
    const auto r = make_rsrc(dst, bytes);
    const int64_t base = ((int64_t)blockIdx.x * kProbeUnroll * 256) * 16;
    const v4i v = {(int)value, (int)value, (int)value, (int)value};
#pragma unroll
    for (int i = 0; i < kProbeUnroll; ++i) {
        const int64_t off = base + ((int64_t)i * 256 + threadIdx.x) * 16;
        __builtin_amdgcn_raw_buffer_store_b128(v, r, off < bytes ? (int)off : kOOB, 0, kNonTemporal);
    }
}

// Matrix-unit clock and rate: 8 waves per workgroup (two per SIMD), each
// issuing 16 independent v_mfma_i32_16x16x64_i8 per iteration, cycling over
// four activation and four weight operands so consecutive MFMAs see
// different data; wave 0 of each workgroup records the shader-clock and the
// constant 100 MHz counters at its start and end (times[4 b .. 4 b + 3]).
// OPS: each lane loads its 4 + 4 operands (32 int32) from `ops`, e.g. random
// bytes, whose switching activity is that of a real product; else small
// constant operands.
template <bool OPS>
__global__ __launch_bounds__(512) void k_probe_mfma(int iters, const int *__restrict__ ops,
                                                    uint64_t *__restrict__ times,
                                                    uint32_t *__restrict__ sink) {
    const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    const int lane = threadIdx.x % kWave;
    v4i a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (OPS) {
            const int64_t base = ((int64_t)blockIdx.x * 512 + threadIdx.x) * 32 + 8 * j;
            a[j] = v4i{ops[base], ops[base + 1], ops[base + 2], ops[base + 3]};
            b[j] = v4i{ops[base + 4], ops[base + 5], ops[base + 6], ops[base + 7]};
        } else {
            a[j] = v4i{0x01010101 * (lane % 3), 0x02020202, 0x01010101, 0x03030303 * (lane % 2)};
            b[j] = v4i{0x10101010, 0x20202020 * (lane % 2), 0x10101010, 0x30303030};
        }
    }
    v4i acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = v4i{0, 0, 0, 0};
    for (int it = 0; it < iters; it += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i % 4], b[(i / 4 + u) % 4], acc[i],
                                                               0, 0, 0);
    }
    int x = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) x ^= acc[i][0] ^ acc[i][3];
    const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        times[4 * blockIdx.x + 0] = c0;
        times[4 * blockIdx.x + 1] = c1;
        times[4 * blockIdx.x + 2] = r0;
        times[4 * blockIdx.x + 3] = r1;
    }
    if (x == 0x5A5A5A5A) sink[blockIdx.x % 64] = (uint32_t)x;  // keeps the products
}

hipError_t launch_probe_mfma(int64_t blocks, int iters, const int32_t *ops, uint64_t *times,
                             uint32_t *sink, hipStream_t st) {
    if (ops)
        launch_main(k_probe_mfma<true>, dim3((unsigned)blocks), dim3(512), 0, st, iters,
                    (const int *)ops, times, sink);
    else
        launch_main(k_probe_mfma<false>, dim3((unsigned)blocks), dim3(512), 0, st, iters,
                    (const int *)nullptr, times, sink);
    return hipGetLastError();
}

hipError_t launch_probe_empty(int64_t blocks, hipStream_t st) {
    launch_main(k_probe_empty, dim3((unsigned)blocks), dim3(256), 0, st);
    return hipGetLastError();
}

hipError_t launch_probe_read(const uint8_t *src, int64_t bytes, uint32_t *sink, hipStream_t st) {
    const int64_t per_block = (int64_t)kProbeUnroll * 256 * 16;
    launch_main(k_probe_read, dim3((unsigned)((bytes + per_block - 1) / per_block)), dim3(256), 0,
                st, src, bytes, sink);
    return hipGetLastError();
}

hipError_t launch_probe_write(uint8_t *dst, int64_t bytes, uint32_t value, hipStream_t st) {
    const int64_t per_block = (int64_t)kProbeUnroll * 256 * 16;
    launch_main(k_probe_write, dim3((unsigned)((bytes + per_block - 1) / per_block)), dim3(256), 0,
                st, dst, bytes, value);
    return hipGetLastError();
}

}  // namespace w4
