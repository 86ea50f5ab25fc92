// Prefill-shaped W4A8 product (many activation rows): int8 MFMA GEMM with
// LDS-staged tiles (Keras INT4 guide, "How it works", steps 4-6).
//
// Block tile 256 (rows) x 256 (output channels) x 128 (k), 8 waves in a 2x4
// arrangement, each owning a 128x64 sub-tile = 8x4 blocks of
// v_mfma_i32_16x16x64_i8 (accumulators in AGPRs).
//
// Per k-tile the block stages
//   A: 256 rows x 128 int8 activations (P8 layout)  = 32 KB
//   B: 256 channels x 64 packed bytes (128 codes)   = 16 KB
// in one stage of a 3-stage LDS ring, using direct global->LDS loads
// (global_load_lds_dwordx4: lane L of a wave writes LDS[base + 16 L]), so the
// tile after next is in flight while the current one is multiplied.  Rows
// are stored without padding; the 16-byte chunk position inside each row is
// XOR-swizzled so that the fragment reads of 8 consecutive lanes hit 8
// distinct bank groups.  Each wave unpacks its packed B fragments in
// registers (16 * code as int8) and the int32 sums are divided by 16 in the
// epilogue, which also applies the dequantization.
#include "common.h"
#include "kernels.h"

namespace w4 {

constexpr int kBM = 256, kBN = 256, kBK = 128, kStages = 3;
constexpr int kABytes = kBM * kBK;       // 32 KB
constexpr int kBBytes = kBN * kBK / 2;   // 16 KB
constexpr int kStageBytes = kABytes + kBBytes;

typedef __attribute__((address_space(3))) void lds_void;

// Wait until at most N of this wave's vector-memory operations (here: the
// direct global->LDS loads) are outstanding and all its LDS operations are
// done, then join the workgroup barrier.  The "memory" clobber keeps the
// compiler from moving LDS accesses across it.  (The fences of
// __syncthreads would instead drain every outstanding direct load.)
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
    static_assert(N >= 0 && N < 16, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <Out OUT>
__global__ __launch_bounds__(512) void k_gemm_mfma(W4A8Args a) {
    // One array per ring stage: each unrolled iteration below names its
    // stages statically, so the compiler can tell the stage being read from
    // the stages being filled.
    __shared__ __align__(16) uint8_t stage0[kStageBytes];
    __shared__ __align__(16) uint8_t stage1[kStageBytes];
    __shared__ __align__(16) uint8_t stage2[kStageBytes];

    const int64_t M = a.M, N = a.N, K = a.K, KB = a.K / 2;
    const int tiles_n = (int)((N + kBN - 1) / kBN);
    const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
    const int64_t m0 = (int64_t)(tile / tiles_n) * kBM;
    const int64_t n0 = (int64_t)(tile % tiles_n) * kBN;

    const int t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
    const int lane = t % kWave;
    const int r16 = lane % 16, kq = lane / 16;
    const int wm = wave / 4, wn = wave % 4;

    // ---- direct-load sources (buffer loads that write LDS; rows past M and
    // channels past N are outside the descriptors and read as zeros).
    // A: 32 wave-loads of 8 rows x 128 B; this wave issues q = 4*wave + i, i.e.
    // rows 32*wave + 8*i + lane/8.  Stored chunk position lane%8 of a row holds
    // the row's global chunk (lane%8) ^ (lane/8).
    const auto ra = make_rsrc(a.Xq + m0 * K, min((int64_t)kBM, M - m0) * K);
    const int a_voff = (32 * wave + lane / 8) * (int)K + (((lane % 8) ^ (lane / 8)) * 16);
    // B: 16 wave-loads of 16 channels x 64 B; this wave issues q = 2*wave + i,
    // i.e. channels 32*wave + 16*i + lane/4.  Stored position lane%4 holds the
    // channel's global chunk (lane%4) ^ ((lane/8)%4).
    const auto rbs = make_rsrc(a.packed + n0 * KB, min((int64_t)kBN, N - n0) * KB);
    const int b_voff = (32 * wave + lane / 4) * (int)KB + (((lane % 4) ^ ((lane / 8) % 4)) * 16);
    auto issue = [&](uint8_t *st, int kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (lds_void *)(st + (4 * wave + i) * 1024), 16, a_voff,
                8 * i * (int)K + kt * kBK, 0, 0);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rbs, (lds_void *)(st + kABytes + (2 * wave + i) * 1024), 16, b_voff,
                16 * i * (int)KB + kt * (kBK / 2), 0, 0);
    };

    // ---- fragment read offsets inside a stage (row block rb adds rb*2048,
    // channel block nb adds nb*1024).
    int aoff[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
        aoff[h] = (wm * 128 + r16) * 128 + (((2 * kq + h) ^ (r16 % 8)) * 16);
    const int boff = kABytes + (wn * 64 + r16) * 64 + ((kq ^ ((r16 / 2) % 4)) * 16);

    v4i acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    auto compute = [&](const uint8_t *st) {
        v4i b0[4], b1[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const uint4 w = *reinterpret_cast<const uint4 *>(st + boff + nb * 1024);
            b0[nb] = v4i{(int)lo16(w.x), (int)hi16(w.x), (int)lo16(w.y), (int)hi16(w.y)};
            b1[nb] = v4i{(int)lo16(w.z), (int)hi16(w.z), (int)lo16(w.w), (int)hi16(w.w)};
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int rb = 0; rb < 8; ++rb) {
                const uint4 x = *reinterpret_cast<const uint4 *>(st + aoff[h] + rb * 2048);
                const v4i av = {(int)x.x, (int)x.y, (int)x.z, (int)x.w};
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    acc[rb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, h ? b1[nb] : b0[nb],
                                                                        acc[rb][nb], 0, 0, 0);
            }
        }
    };
    // One ring step: tile kt sits in `cur`; the tile two ahead goes into
    // `nxt2` (the stage read in the previous step).  Before the barrier this
    // thread's loads of tile kt must be complete: at most the 6 loads of tile
    // kt+1 may remain outstanding.  The barrier also guarantees that no wave
    // still reads `nxt2`.
    auto step = [&](int kt, int KT, const uint8_t *cur, uint8_t *nxt2) {
        if (kt + 1 < KT)
            wait_and_barrier<6>();
        else
            wait_and_barrier<0>();
        if (kt + 2 < KT) issue(nxt2, kt + 2);
        compute(cur);
    };

    const int KT = (int)(K / kBK);
    issue(stage0, 0);
    if (KT > 1) issue(stage1, 1);
    int kt = 0;
    for (; kt + 3 <= KT; kt += 3) {
        step(kt, KT, stage0, stage2);
        step(kt + 1, KT, stage1, stage0);
        step(kt + 2, KT, stage2, stage1);
    }
    if (kt < KT) step(kt, KT, stage0, stage2);
    if (kt + 1 < KT) step(kt + 1, KT, stage1, stage0);

    // ---- epilogue: rows 4*(lane/16)+i of each 16x16 block, column lane%16.
    float swc[4], bc[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const int64_t col = min(n0 + wn * 64 + nb * 16 + r16, N - 1);
        swc[nb] = (OUT == Out::Y) ? a.sw[col] : 0.0f;
        bc[nb] = (OUT == Out::Y && a.bias) ? a.bias[col] : 0.0f;
    }
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t row = m0 + wm * 128 + rb * 16 + 4 * kq + i;
            if (row >= M) continue;
            const float sxr = (OUT == Out::Y) ? a.sx[row] : 0.0f;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int64_t col = n0 + wn * 64 + nb * 16 + r16;
                if (col >= N) continue;
                const int v = acc[rb][nb][i] >> 4;
                if (OUT == Out::I32) {
                    a.acc[row * N + col] = v;
                } else {
                    const float s = sxr * swc[nb];
                    float y = (float)v * s;
                    if (a.bias) y = y + bc[nb];
                    a.Y[row * N + col] = y;
                }
            }
        }
    }
}

hipError_t launch_gemm_mfma(const W4A8Args &a, hipStream_t st) {
    const int64_t tiles = ((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN);
    if (a.out == Out::I32)
        launch_main(k_gemm_mfma<Out::I32>, dim3((unsigned)tiles), dim3(512), 0, st, a);
    else
        launch_main(k_gemm_mfma<Out::Y>, dim3((unsigned)tiles), dim3(512), 0, st, a);
    return hipGetLastError();
}

}  // namespace w4
