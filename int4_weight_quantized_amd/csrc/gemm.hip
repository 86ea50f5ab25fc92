// Prefill-shaped W4A8 product (many activation rows): int8 MFMA GEMM with
// LDS-staged tiles (Keras INT4 guide, "How it works", steps 4-6).
//
// Block tile 256 (rows) x 256 (output channels) x 128 (k), 16 waves in a 4x4
// arrangement, each owning a 64x64 sub-tile = 4x4 blocks of
// v_mfma_i32_16x16x64_i8.  Four waves per SIMD: one wave alone issues
// independent int8 MFMAs at only about 60% of the unit's rate (measured), two
// or more interleave to full rate, and the extra waves hide LDS latency.
//
// Per k-tile the block stages
//   A: 256 rows x 128 int8 activations (P8 layout)  = 32 KB
//   B: 256 channels x 64 packed bytes (128 codes)   = 16 KB
// in one stage of a 3-stage LDS ring, using direct buffer->LDS loads
// (buffer_load_dwordx4 ... lds: lane L of a wave writes LDS[M0 + 16 L]), so the
// tile after next is in flight while the current one is multiplied.  Rows
// are stored in 64-byte units without padding, with XOR-swizzled 16-byte
// chunk positions so that the fragment reads are free of LDS bank conflicts.  Each wave unpacks its packed B fragments in
// registers (16 * code as int8) and the int32 sums are divided by 16 in the
// epilogue, which also applies the dequantization.
#include "common.h"
#include "kernels.h"

namespace w4 {

constexpr int kBM = 256, kBN = 256, kBK = 128, kStages = 3;
constexpr int kThreads = 1024;  // 16 waves: 4 per SIMD keep the matrix cores fed
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
    static_assert(N >= 0 && N < 64, "vmcnt range (6 bits on gfx9)");
    // lgkmcnt(0) through the builtin, so that the compiler's wait-count
    // tracking knows every earlier LDS read has completed.
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Raw buffer descriptor (gfx9 layout): 48-bit base, stride 0, byte range,
// raw-buffer flags.  Reads outside [0, bytes) return zeros.
__device__ __forceinline__ v4i buffer_desc(const void *base, int64_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    const int n = bytes > kMaxRange ? kMaxRange : (int)bytes;
    return v4i{(int)(uint32_t)p, (int)(uint32_t)((p >> 32) & 0xFFFFu), n, kBufFlags};
}

// One 16-byte buffer load per lane that writes LDS (lane L of the wave writes
// LDS[lds_base + 16 L]).  Written as inline asm so that the compiler's
// wait-count pass, which cannot tell which ring stage such a load fills,
// does not drain all outstanding loads before every LDS read; all waits for
// these loads are explicit (wait_and_barrier).  The asm has no register
// outputs; it sets M0 itself and declares it clobbered.  On gfx9 an LDS
// direct load needs one wait state after an SALU write of M0, hence the nop.
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t lds_base, int voff, int soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 ::"s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)p));
}

template <Out OUT>
__global__ __launch_bounds__(kThreads) void k_gemm_mfma(W4A8Args a) {
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
    // LDS layouts use 64-byte rows: a fragment read (16 rows at one 16-byte
    // chunk per quarter-wave, chunk kq for lanes 16kq..16kq+15) of rows of 64
    // bytes with chunk kq stored at slot kq ^ ((row/2) % 4) is free of bank
    // conflicts (measured with the LDS bank-conflict counter on gfx950).
    // A: two regions of 256 rows x 64 B; region h holds the odd (h = 1) or
    // even (h = 0) 16-byte chunks of each 128-byte activation row, which are
    // the k ranges of MFMA half h.  32 wave-loads of 16 rows (1 KB); this wave
    // issues q = 2*wave + i: region h = wave / 8, rows 16*(q % 16) + lane/4;
    // lane s fills slot s%4 of its row with global chunk
    // 2*((s%4) ^ ((row/2)%4)) + h, and (row/2)%4 = (s/8)%4.
    // B: 16 wave-loads of 16 channels x 64 B; this wave issues q = wave, i.e.
    // channels 16*wave + lane/4; stored position lane%4 holds the channel's
    // global chunk (lane%4) ^ ((lane/8)%4).
    const v4i ra = buffer_desc(a.Xq + m0 * K, min((int64_t)kBM, M - m0) * K);
    const v4i rbs = buffer_desc(a.packed + n0 * KB, min((int64_t)kBN, N - n0) * KB);

    // Epilogue operands (row scales, channel scales, bias of this tile) go to
    // LDS with direct loads at the start, so the epilogue reads them from LDS
    // instead of waiting on global loads.  They are older than every ring load
    // of their wave, so the ring's waits cover them.
    __shared__ __align__(16) float s_sx[kBM], s_sw[kBN], s_bias[kBN];
    const bool ep_dma = ((reinterpret_cast<uintptr_t>(a.sx) | reinterpret_cast<uintptr_t>(a.sw) |
                          reinterpret_cast<uintptr_t>(a.bias)) & 15) == 0;
    if (OUT == Out::Y && ep_dma) {
        if (wave == 0)
            dma16(buffer_desc(a.sx + m0, min((int64_t)kBM, M - m0) * 4), lds_addr(s_sx), 16 * lane, 0);
        if (wave == 1)
            dma16(buffer_desc(a.sw + n0, min((int64_t)kBN, N - n0) * 4), lds_addr(s_sw), 16 * lane, 0);
        if (wave == 2 && a.bias)
            dma16(buffer_desc(a.bias + n0, min((int64_t)kBN, N - n0) * 4), lds_addr(s_bias), 16 * lane, 0);
    }
    auto issue = [&](uint8_t *st, int kt) {
        // The per-lane source offsets are recomputed here from the lane id
        // (a few ALU operations) rather than kept live across the main loop.
        int l = (int)__builtin_amdgcn_workitem_id_x() & (kWave - 1);
        asm volatile("" : "+v"(l));
        const int sw = (l % 4) ^ ((l / 8) % 4);
        const int a_voff = (32 * (wave % 8) + l / 4) * (int)K + 32 * sw + 16 * (wave / 8);
        const int b_voff = (16 * wave + l / 4) * (int)KB + 16 * sw;
        const uint32_t base = lds_addr(st);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            dma16(ra, base + (2 * wave + i) * 1024, a_voff, 16 * i * (int)K + kt * kBK);
        dma16(rbs, base + kABytes + wave * 1024, b_voff, kt * (kBK / 2));
    };
    constexpr int kLoadsPerTile = 3;  // dma16 per wave per k-tile

    // ---- fragment read offsets inside a stage (row block rb adds rb*1024,
    // channel block nb adds nb*1024).  A: row r = wm*64 + rb*16 + r16, chunk
    // 2*kq + h -> region h, slot kq ^ ((r16/2) % 4).  B: channel
    // wn*64 + nb*16 + r16, chunk kq at slot kq ^ ((r16/2) % 4).
    const int swz = (kq ^ ((r16 / 2) % 4)) * 16;
    const int aoff = (wm * 64 + r16) * 64 + swz;
    const int boff = kABytes + (wn * 64 + r16) * 64 + swz;

    v4i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    auto compute = [&](const uint8_t *st) {
        uint4 wraw[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
            wraw[nb] = *reinterpret_cast<const uint4 *>(st + boff + nb * 1024);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // this half's 16 codes of each channel block, unpacked (16 * code)
            v4i bh[4];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const uint32_t p0 = h ? wraw[nb].z : wraw[nb].x;
                const uint32_t p1 = h ? wraw[nb].w : wraw[nb].y;
                bh[nb] = v4i{(int)lo16(p0), (int)hi16(p0), (int)lo16(p1), (int)hi16(p1)};
            }
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const uint4 x =
                    *reinterpret_cast<const uint4 *>(st + h * (kABytes / 2) + aoff + rb * 1024);
                const v4i av = {(int)x.x, (int)x.y, (int)x.z, (int)x.w};
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    acc[rb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bh[nb], acc[rb][nb],
                                                                        0, 0, 0);
            }
        }
    };
    // One ring step: tile kt sits in `cur`; the tile two ahead goes into
    // `nxt2` (the stage read in the previous step).  Before the barrier this
    // thread's loads of tile kt must be complete: at most the loads of tile
    // kt+1 may remain outstanding.  The barrier also guarantees that no wave
    // still reads `nxt2`.
    auto step = [&](int kt, int KT, const uint8_t *cur, uint8_t *nxt2) {
        if (kt + 1 < KT)
            wait_and_barrier<kLoadsPerTile>();
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

    // ---- epilogue.  Dequantize in registers (lane holds rows 4*(lane/16)+i
    // of each 16x16 block, column lane%16), stage one 16-row block of each
    // wave's 64x64 sub-tile at a time in LDS (the ring is free now) and store
    // rows back contiguously: one store instruction writes 4 rows x 256 bytes.
    constexpr int kPitch = 68;  // words per staged row (64 + 4 pad)
    static_assert(8 * 16 * kPitch * 4 <= kStageBytes, "staging of 8 waves fits one ring stage");
    uint32_t *stg = reinterpret_cast<uint32_t *>(wave < 8 ? stage0 : stage1) + (wave % 8) * (16 * kPitch);
    if (OUT == Out::Y && !ep_dma && t < kBM) {  // operands not 16-byte aligned: plain loads
        s_sx[t] = a.sx[min(m0 + t, M - 1)];
        s_sw[t] = a.sw[min(n0 + t, N - 1)];
        s_bias[t] = a.bias ? a.bias[min(n0 + t, N - 1)] : 0.0f;
    }
    wait_and_barrier<0>();  // every wave is done reading the ring
    float swc[4], bc[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        swc[nb] = (OUT == Out::Y) ? s_sw[wn * 64 + nb * 16 + r16] : 0.0f;
        bc[nb] = (OUT == Out::Y && a.bias) ? s_bias[wn * 64 + nb * 16 + r16] : 0.0f;
    }
    const int c4 = (lane % 16) * 4;
    const int64_t col = n0 + wn * 64 + c4;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int lr = 4 * kq + i;  // local row 0..15 of this row block
            const float sxr = (OUT == Out::Y) ? s_sx[wm * 64 + rb * 16 + lr] : 0.0f;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int v = acc[rb][nb][i] >> 4;
                uint32_t bits;
                if (OUT == Out::I32) {
                    bits = (uint32_t)v;
                } else {
                    const float sc = sxr * swc[nb];
                    float y = (float)v * sc;
                    if (a.bias) y = y + bc[nb];
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
            const int64_t row = m0 + wm * 64 + rb * 16 + lr;
            const uint4 v = *reinterpret_cast<const uint4 *>(&stg[lr * kPitch + c4]);
            if (row >= M) continue;
            uint32_t *dst = (OUT == Out::I32) ? reinterpret_cast<uint32_t *>(a.acc + row * N + col)
                                              : reinterpret_cast<uint32_t *>(a.Y + row * N + col);
            if (col + 3 < N && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
                *reinterpret_cast<uint4 *>(dst) = v;
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

hipError_t launch_gemm_mfma(const W4A8Args &a, hipStream_t st) {
    const int64_t tiles = ((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN);
    if (a.out == Out::I32)
        launch_main(k_gemm_mfma<Out::I32>, dim3((unsigned)tiles), dim3(kThreads), 0, st, a);
    else
        launch_main(k_gemm_mfma<Out::Y>, dim3((unsigned)tiles), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace w4
