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

}  // namespace w4
