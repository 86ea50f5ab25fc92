// Prefill-shaped W4A8 product (many activation rows): int8 MFMA GEMM with
// LDS-staged tiles (Keras INT4 guide, "How it works", steps 4-6).
//
// Block tile 128 (rows) x 128 (output channels) x 128 (k); 4 waves in a 2x2
// arrangement, each owning a 64x64 sub-tile = 4x4 blocks of
// v_mfma_i32_16x16x64_i8.  Per k-tile the block stages
//   A: 128 rows x 128 int8 activations (P8 layout)  -> LDS, row pitch 144 B
//   B: 128 channels x 64 packed bytes (128 codes)   -> LDS, row pitch 80 B
// (the pitches keep the 16-byte LDS reads of 8 consecutive lanes on distinct
// banks).  Each wave unpacks its B fragments in registers; the next k-tile is
// fetched into registers while the current one is multiplied (two LDS
// buffers, one barrier per k-tile).
#include "common.h"
#include "kernels.h"

namespace w4 {

constexpr int kBM = 128, kBN = 128, kBK = 128;
constexpr int kAP = kBK + 16;      // A row pitch (bytes)
constexpr int kBP = kBK / 2 + 16;  // B row pitch (bytes)

template <Out OUT>
__global__ __launch_bounds__(256) void k_gemm_mfma(W4A8Args a) {
    __shared__ __align__(16) uint8_t As[2][kBM * kAP];
    __shared__ __align__(16) uint8_t Bs[2][kBN * kBP];

    const int64_t M = a.M, N = a.N, K = a.K, KB = a.K / 2;
    const int tiles_n = (int)((N + kBN - 1) / kBN);
    const int nblk = gridDim.x;
    const int tile = xcd_swizzle(blockIdx.x, nblk);
    const int64_t m0 = (int64_t)(tile / tiles_n) * kBM;
    const int64_t n0 = (int64_t)(tile % tiles_n) * kBN;

    const int t = threadIdx.x;
    const int wave = t / kWave, lane = t % kWave;
    const int r16 = lane % 16, kq = lane / 16;
    const int wm = wave / 2, wn = wave % 2;

    // Global -> register staging assignment (raw buffer loads; the
    // descriptors cover this tile's rows / channels, so rows past M and
    // channels past N read zeros and their outputs are not stored).
    // A: 1024 16-byte pieces: piece p = t + 256*i -> row p/8, column (p%8)*16.
    // B: 512 pieces: piece p = t + 256*i -> channel p/4, bytes (p%4)*16.
    const int Ki = (int)K, KBi = (int)KB;
    const auto ra = make_rsrc(a.Xq + m0 * K, min((int64_t)kBM, M - m0) * K);
    const auto rbs = make_rsrc(a.packed + n0 * KB, min((int64_t)kBN, N - n0) * KB);
    int aoff[4], boff[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = t + 256 * i;
        aoff[i] = (p / 8) * Ki + (p % 8) * 16;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = t + 256 * i;
        boff[i] = (p / 4) * KBi + (p % 4) * 16;
    }

    uint4 ra_[4], rb_[2];
    auto fetch = [&](int kt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ra_[i] = bload16(ra, aoff[i] + kt * kBK);
#pragma unroll
        for (int i = 0; i < 2; ++i) rb_[i] = bload16(rbs, boff[i] + kt * (kBK / 2));
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = t + 256 * i;
            *reinterpret_cast<uint4 *>(&As[buf][(p / 8) * kAP + (p % 8) * 16]) = ra_[i];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int p = t + 256 * i;
            *reinterpret_cast<uint4 *>(&Bs[buf][(p / 4) * kBP + (p % 4) * 16]) = rb_[i];
        }
    };

    v4i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    const int KT = (int)(K / kBK);
    fetch(0);
    stash(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int buf = (int)(kt & 1);
        if (kt + 1 < KT) fetch(kt + 1);

        // B fragments of this wave: 4 channel blocks, 16 packed bytes each.
        v4i b0[4], b1[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int c = wn * 64 + nb * 16 + r16;
            const uint4 w = *reinterpret_cast<const uint4 *>(&Bs[buf][c * kBP + kq * 16]);
            b0[nb] = v4i{(int)lo16(w.x), (int)hi16(w.x), (int)lo16(w.y), (int)hi16(w.y)};
            b1[nb] = v4i{(int)lo16(w.z), (int)hi16(w.z), (int)lo16(w.w), (int)hi16(w.w)};
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int r = wm * 64 + mb * 16 + r16;
            const uint4 x0 = *reinterpret_cast<const uint4 *>(&As[buf][r * kAP + kq * 32]);
            const uint4 x1 = *reinterpret_cast<const uint4 *>(&As[buf][r * kAP + kq * 32 + 16]);
            const v4i a0 = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w};
            const v4i a1 = {(int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                acc[mb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0[nb], acc[mb][nb], 0, 0, 0);
                acc[mb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1[nb], acc[mb][nb], 0, 0, 0);
            }
        }
        if (kt + 1 < KT) stash(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int64_t col = n0 + wn * 64 + nb * 16 + r16;
            if (col >= N) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row = m0 + wm * 64 + mb * 16 + 4 * kq + i;
                if (row >= M) continue;
                const int v = acc[mb][nb][i] >> 4;
                if (OUT == Out::I32)
                    a.acc[row * N + col] = v;
                else
                    a.Y[row * N + col] = dequant(v, a.sx[row], a.sw[col], a.bias, (int)col);
            }
        }
    }
}

hipError_t launch_gemm_mfma(const W4A8Args &a, hipStream_t st) {
    const int64_t tiles = ((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN);
    if (a.out == Out::I32)
        launch_main(k_gemm_mfma<Out::I32>, dim3((unsigned)tiles), dim3(256), 0, st, a);
    else
        launch_main(k_gemm_mfma<Out::Y>, dim3((unsigned)tiles), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace w4
