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
// in one stage of a 3-stage LDS ring, using direct buffer->LDS loads
// (buffer_load_dwordx4 ... lds: lane L of a wave writes LDS[M0 + 16 L]), so the
// tile after next is in flight while the current one is multiplied.  Rows
// are stored without padding, with XOR-swizzled 16-byte chunk positions (the
// weight reads are conflict-free on the LDS bank-conflict counter; the
// activation reads show 2-way conflicts, and a conflict-free layout measured
// no faster).  Each wave unpacks its packed B fragments in registers
// (16 * code as int8) and the int32 sums are divided by 16 in the epilogue,
// which also applies the dequantization.
//
// The W8A8 product (the guide's INT8 path: int8 weight codes, natural-order
// activations, no unpacking) runs the same kernel with W8 = true: its weight
// tile (256 channels x 128 int8 codes = 32 KB) has the activation tile's
// shape and uses the same super-row layout and load pattern; a stage is then
// 64 KB, so the ring has 2 stages (the next tile loads while the current one
// is multiplied).
//
// Measured on gfx950: one wave per SIMD issues independent int8 MFMAs at
// about 60% of the unit's rate and two or more at ~94%; VALU instructions
// between MFMAs are not hidden.  Layouts with 16 waves (64x64 per wave) or 4
// waves (128x128 per wave, fragments double-buffered) were not faster than
// this one on the benchmark's data.
#include "common.h"
#include "kernels.h"

namespace w4 {

constexpr int kBM = 256, kBN = 256, kBK = 128;
constexpr int kABytes = kBM * kBK;  // 32 KB

template <bool W8>
struct GemmStage {
    static constexpr int kBBytes = W8 ? kBN * kBK : kBN * kBK / 2;  // 32 or 16 KB
    static constexpr int kBytes = kABytes + kBBytes;
};

// PP: the int4 codes come in the shuffled tile layout, whose 1 KB tiles (16
// channels x 128 k, chunks already at their LDS slots) are exactly the weight
// wave-loads below.
template <Out OUT, bool W8, bool PP = false>
__global__ __launch_bounds__(512) void k_gemm_mfma(W4A8Args args) {
    const W4A8Args a = args_now(args);
    constexpr int kStageBytes = GemmStage<W8>::kBytes;
    // One array per ring stage: each unrolled iteration below names its
    // stages statically, so the compiler can tell the stage being read from
    // the stages being filled.  (8-bit weights use two stages.)
    __shared__ __align__(16) uint8_t stage0[kStageBytes];
    __shared__ __align__(16) uint8_t stage1[kStageBytes];
    __shared__ __align__(16) uint8_t stage2[W8 ? 16 : kStageBytes];

    const int64_t M = a.M, N = a.N, K = a.K, KB = W8 ? a.K : a.K / 2;
    const int tiles_n = (int)((N + kBN - 1) / kBN);
    const int tiles_m = (int)((M + kBM - 1) / kBM);
    // the grid is exactly the tile count (computed here rather than read from
    // the launch's hidden arguments, which would be a second argument load)
    const int tile = xcd_swizzle(blockIdx.x, tiles_m * tiles_n);
    // Tiles in groups of kGroupRows tile rows, walked column by column: the
    // consecutive tiles one XCD takes form a patch of 4 rows (activation
    // panels) by several channel columns (weight panels), so each XCD's L2
    // fetches fewer panels than with whole rows of tiles.
    constexpr int kGroupRows = 4;
    const int group = tile / (kGroupRows * tiles_n);
    const int first_row = group * kGroupRows;
    const int rows_here = min(kGroupRows, tiles_m - first_row);
    const int in_group = tile - group * kGroupRows * tiles_n;
    const int64_t m0 = (int64_t)(first_row + in_group % rows_here) * kBM;
    const int64_t n0 = (int64_t)(in_group / rows_here) * kBN;

    const int t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
    const int lane = t % kWave;
    const int r16 = lane % 16, kq = lane / 16;
    const int wm = wave / 4, wn = wave % 4;

    // ---- direct-load sources (buffer loads that write LDS; rows past M and
    // channels past N are outside the descriptors and read as zeros).  The
    // raw-buffer range check covers the per-lane offset (voffset) only, not
    // the scalar offset, so each lane's row or channel is part of its voffset
    // and the scalar offset holds only the k-tile's position inside that row
    // (kt * 128 + 128 <= K bytes: it never leaves the row).
    // LDS A layout: rows r, r+1 (r even) form a 256-byte super-row; the 16
    // chunks (row parity p, chunk c) sit at slot ((8p + c) ^ ((r/2) % 8)).  A
    // 128-bit LDS read is conflict-free when each 16 consecutive lanes use 16
    // distinct 16-byte slots modulo 256 bytes; the fragment reads (16 rows, one
    // chunk) do.  A: 32 wave-loads of 4 super-rows (1 KB); this wave issues
    // q = 4*wave + i.  Lane s fills slot s%16 of super-row 4q + s/16, i.e.
    // global row 8q + 2(s/16) + (v>>3), chunk v&7, with v = (s%16) ^ ((s/16 + 4q) % 8)
    // = (s%16) ^ (s/16 + 4*(i%2)) since 4q % 8 = 4*(i%2).
    const v4i ra = buffer_desc(a.Xq + m0 * K, min((int64_t)kBM, M - m0) * K);
    int a_voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int v = (lane % 16) ^ (lane / 16 + 4 * (i % 2));
        a_voff[i] = (32 * wave + 8 * i + 2 * (lane / 16) + (v >> 3)) * (int)K + (v & 7) * 16;
    }
    // B: 16 wave-loads of 16 channels x 64 B; this wave issues q = 2*wave + i,
    // i.e. channels 32*wave + 16*i + lane/4.  Stored position lane%4 holds the
    // channel's global chunk (lane%4) ^ ((lane/8)%4).
    // With 8-bit weights the B tile repeats the A pattern (rows = channels,
    // row stride K bytes), so the same per-lane offsets serve both.
    static_assert(!PP || !W8, "shuffled layout of int4 codes");
    const int64_t ST = K / 128;  // 128-k steps (tiles per 16-channel block)
    const v4i rbs = PP ? buffer_desc(a.packed + (n0 / 16) * ST * 1024,
                                     ((min((int64_t)kBN, N - n0) + 15) / 16) * ST * 1024)
                       : buffer_desc(a.packed + n0 * KB, min((int64_t)kBN, N - n0) * KB);
    int b_voff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
        b_voff[i] = (32 * wave + 16 * i + lane / 4) * (int)KB + (((lane % 4) ^ ((lane / 8) % 4)) * 16);
    auto issue = [&](uint8_t *st, int kt) {
        const uint32_t base = lds_addr(st);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dma16(ra, base + (4 * wave + i) * 1024, a_voff[i], kt * kBK);
        if (W8) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dma16(rbs, base + kABytes + (4 * wave + i) * 1024, a_voff[i], kt * kBK);
        } else if (PP) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                dma16(rbs, base + kABytes + (2 * wave + i) * 1024,
                      (2 * wave + i) * (int)ST * 1024 + lane * 16, kt * 1024);
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                dma16(rbs, base + kABytes + (2 * wave + i) * 1024, b_voff[i], kt * (kBK / 2));
        }
    };

    // ---- fragment read offsets inside a stage (row block rb adds rb*2048,
    // channel block nb adds nb*1024).  A: row r = wm*128 + rb*16 + r16, chunk
    // 2*kq + h -> super-row r/2, slot (8*(r16%2) + 2kq + h) ^ ((r16/2) % 8).
    int aoff[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
        aoff[h] = (wm * 64 + r16 / 2) * 256 + (((8 * (r16 % 2) + 2 * kq + h) ^ ((r16 / 2) % 8)) * 16);
    const int boff = kABytes + (wn * 64 + r16) * 64 + ((kq ^ ((r16 / 2) % 4)) * 16);
    // 8-bit weights: channel c = wn*64 + nb*16 + r16 in super-row c/2 (the A
    // formula with wn*32 super-rows per wave column; block nb adds nb*2048)
    int b8off[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
        b8off[h] = kABytes + (wn * 32 + r16 / 2) * 256 +
                   (((8 * (r16 % 2) + 2 * kq + h) ^ ((r16 / 2) % 8)) * 16);

    v4i acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    // One k-tile.  The activation fragments stream through a rolling window
    // of 4 over both halves (the read of the fragment four ahead is issued
    // right after each row block's MFMAs, across the half boundary); 8-bit
    // weights read their second-half fragments between the first half's row
    // blocks (int4 codes are unpacked for both halves up front: spreading the
    // unpack measured no faster); `after_first` (the DMA issue of a later
    // tile) runs after the first row block's MFMAs, so that the matrix pipe
    // starts right after the barrier.
    auto compute = [&](const uint8_t *st, auto after_first) {
        uint4 wraw[4];
        if (!W8) {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
                wraw[nb] = *reinterpret_cast<const uint4 *>(st + boff + nb * 1024);
        }
        // the 16 codes of each channel block per half (16 * code, or the int8
        // codes themselves; those of half 1 are read below)
        v4i b0[4], b1[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            if (W8) {
                const uint4 w = *reinterpret_cast<const uint4 *>(st + b8off[0] + nb * 2048);
                b0[nb] = v4i{(int)w.x, (int)w.y, (int)w.z, (int)w.w};
            } else {
                b0[nb] = v4i{(int)lo16(wraw[nb].x), (int)hi16(wraw[nb].x), (int)lo16(wraw[nb].y),
                             (int)hi16(wraw[nb].y)};
                b1[nb] = v4i{(int)lo16(wraw[nb].z), (int)hi16(wraw[nb].z), (int)lo16(wraw[nb].w),
                             (int)hi16(wraw[nb].w)};
            }
        }
        // fragment i = 8 * half + row block
        auto a_frag = [&](int i) {
            return *reinterpret_cast<const uint4 *>(st + aoff[i / 8] + (i % 8) * 2048);
        };
        uint4 xa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) xa[i] = a_frag(i);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int rb = i % 8;
            const uint4 x = xa[i % 4];
            const v4i av = {(int)x.x, (int)x.y, (int)x.z, (int)x.w};
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
                acc[rb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, i < 8 ? b0[nb] : b1[nb],
                                                                    acc[rb][nb], 0, 0, 0);
            if (i + 4 < 16) xa[i % 4] = a_frag(i + 4);
            if (i < 8) {
                const int nb = i / 2;
                if (W8) {
                    if (i % 2 == 0) {
                        const uint4 w =
                            *reinterpret_cast<const uint4 *>(st + b8off[1] + nb * 2048);
                        b1[nb] = v4i{(int)w.x, (int)w.y, (int)w.z, (int)w.w};
                    }
                }
            }
            if (i == 0) after_first();
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // One ring step: tile kt sits in `cur`; the tile two ahead goes into
    // `nxt2` (the stage read in the previous step).  Before the barrier this
    // thread's loads of tile kt must be complete: at most the 6 loads of tile
    // kt+1 may remain outstanding.  The barrier also guarantees that no wave
    // still reads `nxt2`, so its loads may be issued anywhere in this step.
    auto step = [&](int kt, int KT, const uint8_t *cur, uint8_t *nxt2) {
        if (kt + 1 < KT)
            wait_and_barrier<6>();
        else
            wait_and_barrier<0>();
        compute(cur, [&] {
            if (kt + 2 < KT) issue(nxt2, kt + 2);
        });
    };

    // 8-bit weights, 2-stage ring: tile kt sits in `cur` and is complete
    // (no load outstanding) at the barrier, after which every wave is done
    // with the other stage, which receives tile kt+1.
    auto step2 = [&](int kt, int KT, const uint8_t *cur, uint8_t *nxt) {
        wait_and_barrier<0>();
        compute(cur, [&] {
            if (kt + 1 < KT) issue(nxt, kt + 1);
        });
    };

    const int KT = (int)(K / kBK);
    int kt = 0;
    if (W8) {
        issue(stage0, 0);
        for (; kt + 2 <= KT; kt += 2) {
            step2(kt, KT, stage0, stage1);
            step2(kt + 1, KT, stage1, stage0);
        }
        if (kt < KT) step2(kt, KT, stage0, stage1);
    } else {
        issue(stage0, 0);
        if (KT > 1) issue(stage1, 1);
        for (; kt + 3 <= KT; kt += 3) {
            step(kt, KT, stage0, stage2);
            step(kt + 1, KT, stage1, stage0);
            step(kt + 2, KT, stage2, stage1);
        }
        if (kt < KT) step(kt, KT, stage0, stage2);
        if (kt + 1 < KT) step(kt + 1, KT, stage1, stage0);
    }

    // ---- epilogue.  Dequantize in registers (lane holds rows 4*(lane/16)+i
    // of each 16x16 block, column lane%16), stage one 16-row block of each
    // wave's sub-tile at a time in LDS (the ring is free now) and store rows
    // back contiguously: one store instruction writes 4 rows x 256 bytes.
    float swc[4], bc[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const int64_t col = min(n0 + wn * 64 + nb * 16 + r16, N - 1);
        swc[nb] = (OUT == Out::Y) ? a.sw[col] : 0.0f;
        bc[nb] = (OUT == Out::Y && a.bias) ? a.bias[col] : 0.0f;
    }
    constexpr int kPitch = 68;  // words per staged row (64 + 4 pad)
    static_assert(8 * 16 * kPitch * 4 <= kStageBytes, "staging fits one ring stage");
    uint32_t *stg = reinterpret_cast<uint32_t *>(stage0) + wave * (16 * kPitch);
    wait_and_barrier<0>();  // every wave is done reading the ring
    const int c4 = (lane % 16) * 4;
    const int64_t col = n0 + wn * 64 + c4;
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int lr = 4 * kq + i;  // local row 0..15 of this row block
            const int64_t row = m0 + wm * 128 + rb * 16 + lr;
            const float sxr = (OUT == Out::Y) ? a.sx[min(row, M - 1)] : 0.0f;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int v = W8 ? acc[rb][nb][i] : (acc[rb][nb][i] >> 4);
                uint32_t bits;
                if (OUT == Out::I32) {
                    bits = (uint32_t)v;
                } else {
                    const float sc = sxr * swc[nb];
                    float y = (float)v * sc;
                    if (a.bias) y = y + bc[nb];
                    y = relu_if(y, a.relu);
                    bits = __float_as_uint(y);
                }
                stg[lr * kPitch + nb * 16 + r16] = bits;
            }
        }
        // wave-local exchange through LDS: the writes complete before the reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int lr = 4 * it + lane / 16;
            const int64_t row = m0 + wm * 128 + rb * 16 + lr;
            const uint4 v = *reinterpret_cast<const uint4 *>(&stg[lr * kPitch + c4]);
            if (row >= M) continue;
            uint32_t *dst = (OUT == Out::I32) ? reinterpret_cast<uint32_t *>(a.acc + row * N + col)
                                              : reinterpret_cast<uint32_t *>(a.Y + row * N + col);
            if (col + 3 < N && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
                // written once and never read back here: a non-temporal store
                // keeps the output stream from evicting the weight and
                // activation tiles the other workgroups still read from L2
                const u32x4 w = {v.x, v.y, v.z, v.w};
                __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(dst));
            } else {
                if (col < N) dst[0] = v.x;
                if (col + 1 < N) dst[1] = v.y;
                if (col + 2 < N) dst[2] = v.z;
                if (col + 3 < N) dst[3] = v.w;
            }
        }
        // the reads above complete before the next row block overwrites
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

template <bool W8>
static void go_gemm(const W4A8Args &a, hipStream_t st) {
    const int64_t tiles = ((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN);
    if constexpr (!W8) {
        if (a.pp) {
            launch_main(k_gemm_mfma<Out::Y, false, true>, dim3((unsigned)tiles), dim3(512), 0, st,
                        a);
            return;
        }
    }
    if (a.out == Out::I32)
        launch_main(k_gemm_mfma<Out::I32, W8>, dim3((unsigned)tiles), dim3(512), 0, st, a);
    else
        launch_main(k_gemm_mfma<Out::Y, W8>, dim3((unsigned)tiles), dim3(512), 0, st, a);
}

hipError_t launch_gemm_mfma(const W4A8Args &a, hipStream_t st) {
    if (a.w8)
        go_gemm<true>(a, st);
    else
        go_gemm<false>(a, st);
    return hipGetLastError();
}

}  // namespace w4
