// Weight-only W4A16 product: unsigned int4 codes with a scale and zero point
// per group of K ("4-bit Integer Quantization for LLMs": activations stay
// 16-bit, weights are dequantized at compute time; "INT4" concept entry 4.5,
// schemes A and C).  Each weight is dequantized in registers to
//   w' = bf16_rne(fl((q - zero) * scale))
// and fed to v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
//
// Block = W waves that split K into W slices and cover 16*NB output channels
// for 16 activation rows.  Per 128-k step a lane loads 16 packed bytes of one
// channel (codes k = 128*s + 32*(l/16) + [0, 32)) and the matching 32 bf16
// activations of row l%16; the 32 codes feed four MFMAs of 8 codes each.
//
// Fast form for groups whose zero point z is an integer in [-112, 128] and
// whose scale has 2^-100 <= |s| < 2^100 (it gives fl(fl(q - z) * s), bit for
// bit; other groups take that direct form), 21 VALU operations per 8 codes:
// one and-or per pair of codes places two nibbles in the mantissas of two
// fp16 1024s (1024 + q, or 1024 + 16 q for a nibble at bits 4-7), one packed
// fp16 add (or fma with 1/16) per pair subtracts 1024 + z (or 64 + z),
// exact since every value involved is an integer below 2048 in magnitude,
// and one mixed-precision fma per code takes the fp16 q - z times the fp32
// scale plus -0, i.e. the single rounding fl((q - z) * s); no product is
// subnormal.  Measured on the 70B-class layer (shuffled tiles, LDS-staged
// kernel, alternated runs on two boxes): its k-loop takes 2-4 % fewer shader
// cycles than an earlier byte form (v_cvt_f32_ubyte of 128 + q - z, then
// fma with s and -128 s; 25 operations per 8 codes).
#include "common.h"
#include "kernels.h"

namespace w4 {

bool w4a16_fast_ok(int64_t M, int64_t K, int64_t N, int64_t group) {
    (void)M;
    (void)N;
    return K % 128 == 0 && group % 32 == 0;
}

__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
    const bf16x2 v = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
    return __builtin_bit_cast(uint32_t, v);
}

// 8 codes of one packed dword -> 4 dwords of bf16 pairs in natural k order.
// Direct form for any zero point: fl(fl(q - z) * s).
__device__ __forceinline__ v4i dequant8_direct(uint32_t w, float s, float zp) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    float fl[4], fh[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float dl = (float)((lo >> (8 * i)) & 0xFFu) - zp;
        const float dh = (float)((hi >> (8 * i)) & 0xFFu) - zp;
        fl[i] = dl * s;
        fh[i] = dh * s;
    }
    return v4i{(int)pk_bf16(fl[0], fh[0]), (int)pk_bf16(fl[1], fh[1]), (int)pk_bf16(fl[2], fh[2]),
               (int)pk_bf16(fl[3], fh[3])};
}

// A group may take the fast form when its zero point is an integer in
// [-112, 128] (1024 + z and 64 + z are then exact fp16 integers and q - z
// stays within [-128, 127]; a fractional zero point must not be rounded
// there) and 2^-100 <= |s| < 2^100 (no product is subnormal or overflows).
__device__ __forceinline__ bool fast_group_ok(float s, float zp) {
    // bitwise &: straight-line compares instead of short-circuit branches,
    // which made the stage's operand reads wait behind the table read
    return (zp >= -112.0f) & (zp <= 128.0f) & (zp == rintf(zp)) & (fabsf(s) < 0x1p100f) &
           (fabsf(s) >= 0x1p-100f);
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Fast form (see above): c0 = (-1024 - z) and c1 = (-64 - z) in both halves,
// nz = -0 (kept opaque so that the fma is not turned into a multiply), mg =
// 0x64006400 (two fp16 1024s, in a register so that each pair takes one
// v_and_or_b32); the kernels set nz and mg once.
__device__ __forceinline__ v4i dequant8_f16(uint32_t w, float s, float nz, half2v c0, half2v c1,
                                            uint32_t mg) {
    const uint32_t w8 = w >> 8;
    const half2v t0 = __builtin_bit_cast(half2v, (w & 0x000F000Fu) | mg);   // 1024 + q, k = 0, 4
    const half2v t1 = __builtin_bit_cast(half2v, (w & 0x00F000F0u) | mg);   // 1024 + 16 q, k = 1, 5
    const half2v t2 = __builtin_bit_cast(half2v, (w8 & 0x000F000Fu) | mg);  // k = 2, 6
    const half2v t3 = __builtin_bit_cast(half2v, (w8 & 0x00F000F0u) | mg);  // k = 3, 7
    const half2v k16 = half2v{(_Float16)0.0625f, (_Float16)0.0625f};
    const half2v d0 = t0 + c0, d2 = t2 + c0;  // q - z, exact
    const half2v d1 = __builtin_elementwise_fma(t1, k16, c1), d3 = __builtin_elementwise_fma(t3, k16, c1);
    const float f0 = fmaf((float)d0.x, s, nz), f4 = fmaf((float)d0.y, s, nz);
    const float f1 = fmaf((float)d1.x, s, nz), f5 = fmaf((float)d1.y, s, nz);
    const float f2 = fmaf((float)d2.x, s, nz), f6 = fmaf((float)d2.y, s, nz);
    const float f3 = fmaf((float)d3.x, s, nz), f7 = fmaf((float)d3.y, s, nz);
    return v4i{(int)pk_bf16(f0, f1), (int)pk_bf16(f2, f3), (int)pk_bf16(f4, f5), (int)pk_bf16(f6, f7)};
}

// c0 of the fast form, -1024 - z in both halves (exact: an integer below
// 2048 in magnitude); c1 = c0 + 960 = -64 - z, also exact
__device__ __forceinline__ half2v zero_point_pair(float zp) {
    const _Float16 e = (_Float16)(-1024.0f - zp);
    return half2v{e, e};
}
constexpr half2v k960 = half2v{(_Float16)960.0f, (_Float16)960.0f};

__device__ __forceinline__ v4f mfma_bf16(uint4 a, v4i b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                   __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

template <int NB, int D, int W, bool G128>
__global__ __launch_bounds__(64 * W) void k_w4a16_mfma(const uint16_t *__restrict__ X,
                                                    const uint8_t *__restrict__ packed,
                                                    const float *__restrict__ scales,
                                                    const float *__restrict__ zeros,
                                                    float *__restrict__ Y, int64_t M, int64_t K64,
                                                    int64_t N, int64_t group) {
    args_now(X, packed, scales, zeros, Y, M, K64, N, group);
    static_assert(W * NB * kWave * 16 <= 160 * 1024, "partial sums must fit in LDS");
    static_assert(4 % D == 0, "ring depth divides the 4-step scale blocks");
    __shared__ v4f red[W][NB][kWave];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int r16 = lane % 16, kq = lane / 16;
    const int K = (int)K64, KB = K / 2, G = (int)(K64 / group);
    const int S = K / 128;
    const int s0 = S * wave / W, s1 = S * (wave + 1) / W;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * NB;
    const int64_t m0 = (int64_t)blockIdx.y * 16;
    const int cols = (int)min((int64_t)(16 * NB), N - n0);
    const int rowsm = (int)min((int64_t)16, M - m0);

    // Descriptors cover exactly this block's channels / rows: channels past N
    // and rows past M read zeros (their outputs are not stored).
    const auto rb = make_rsrc(packed + n0 * KB, (int64_t)cols * KB);
    const auto rs = make_rsrc(scales + n0 * G, (int64_t)cols * G * 4);
    const auto rz = make_rsrc(zeros + n0 * G, (int64_t)cols * G * 4);
    const auto rx = make_rsrc(X + m0 * K, (int64_t)rowsm * K * 2);
    int boff[NB], goff[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        boff[nb] = (16 * nb + r16) * KB + kq * 16;
        goff[nb] = (16 * nb + r16) * G * 4;
    }
    const int xoff = r16 * K * 2 + kq * 64;

    v4f acc[NB];
    // the fast form's constants, set once: two fp16 1024s (a register
    // operand of v_and_or_b32, not a literal) and the addend -0 (opaque, so
    // that the fma is not turned into a multiply)
    uint32_t mg = 0x64006400u;
    float nz = -0.0f;
    asm volatile("" : "+v"(mg), "+v"(nz));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = v4f{0.f, 0.f, 0.f, 0.f};

    // Register ring: weights and activations of the next D steps.
    uint4 wr[D][NB], xr[D][4];
    auto fetch = [&](int d, int ss) {
        const bool ok = ss < s1;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) wr[d][nb] = bload16(rb, ok ? boff[nb] + 64 * ss : kOOB);
        const int xo = ok ? xoff + 256 * ss : kOOB;
#pragma unroll
        for (int q = 0; q < 4; ++q) xr[d][q] = bload16(rx, xo + 16 * q);
    };

    // One step: one wave-uniform vote picks the dequantization path for all
    // NB channel blocks; each block is dequantized right before its 4 MFMAs
    // so only 16 dequantized registers are live at a time.  Steps past s1
    // read zeros (weights, activations and scales) and add nothing.
    auto compute = [&](int d, const float *sc, const float *zp) {
        bool ok = true;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            ok = ok & fast_group_ok(sc[nb], zp[nb]);
        if (__all(ok)) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const half2v c0 = zero_point_pair(zp[nb]), c1 = c0 + k960;
                const uint4 w = wr[d][nb];
                const v4i b0 = dequant8_f16(w.x, sc[nb], nz, c0, c1, mg);
                const v4i b1 = dequant8_f16(w.y, sc[nb], nz, c0, c1, mg);
                const v4i b2 = dequant8_f16(w.z, sc[nb], nz, c0, c1, mg);
                const v4i b3 = dequant8_f16(w.w, sc[nb], nz, c0, c1, mg);
                acc[nb] = mfma_bf16(xr[d][0], b0, acc[nb]);
                acc[nb] = mfma_bf16(xr[d][1], b1, acc[nb]);
                acc[nb] = mfma_bf16(xr[d][2], b2, acc[nb]);
                acc[nb] = mfma_bf16(xr[d][3], b3, acc[nb]);
            }
        } else {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const uint4 w = wr[d][nb];
                const v4i b0 = dequant8_direct(w.x, sc[nb], zp[nb]);
                const v4i b1 = dequant8_direct(w.y, sc[nb], zp[nb]);
                const v4i b2 = dequant8_direct(w.z, sc[nb], zp[nb]);
                const v4i b3 = dequant8_direct(w.w, sc[nb], zp[nb]);
                acc[nb] = mfma_bf16(xr[d][0], b0, acc[nb]);
                acc[nb] = mfma_bf16(xr[d][1], b1, acc[nb]);
                acc[nb] = mfma_bf16(xr[d][2], b2, acc[nb]);
                acc[nb] = mfma_bf16(xr[d][3], b3, acc[nb]);
            }
        }
    };

    if constexpr (G128) {
        // Group = one 128-k step.  The 4 lanes of a channel (kq = 0..3) load
        // the scales and zero points of 4 consecutive steps with one load
        // (16 contiguous bytes per channel) and hand them to each other with
        // ds_bpermute, instead of every lane loading one value per step.
        float ss_cur[NB], zz_cur[NB], ss_nxt[NB], zz_nxt[NB];
        auto fetch_sz = [&](float *sd, float *zd, int sb) {
            const bool ok = sb + kq < s1;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                sd[nb] = bloadf(rs, ok ? goff[nb] + 4 * (sb + kq) : kOOB);
                zd[nb] = bloadf(rz, ok ? goff[nb] + 4 * (sb + kq) : kOOB);
            }
        };
        fetch_sz(ss_cur, zz_cur, s0);
#pragma unroll
        for (int d = 0; d < D; ++d) {
            fetch(d, s0 + d);
            __builtin_amdgcn_sched_barrier(0);
        }
        fetch_sz(ss_nxt, zz_nxt, s0 + 4);
        for (int s = s0; s < s1; s += 4) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int src = (r16 + 16 * j) * 4;
                float sc[NB], zp[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    sc[nb] = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(ss_cur[nb])));
                    zp[nb] = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(zz_cur[nb])));
                }
                compute(j % D, sc, zp);
                fetch(j % D, s + j + D);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                ss_cur[nb] = ss_nxt[nb];
                zz_cur[nb] = zz_nxt[nb];
            }
            fetch_sz(ss_nxt, zz_nxt, s + 8);
        }
    } else {
        // Any group size (a multiple of 32): each lane loads the scale and
        // zero point of its own 32 codes every step.
        float sr[D][NB], zr[D][NB];
        auto fetch_sz = [&](int d, int ss) {
            const bool ok = ss < s1;
            const int g = (ss * 128 + kq * 32) / (int)group;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                sr[d][nb] = bloadf(rs, ok ? goff[nb] + 4 * g : kOOB);
                zr[d][nb] = bloadf(rz, ok ? goff[nb] + 4 * g : kOOB);
            }
        };
#pragma unroll
        for (int d = 0; d < D; ++d) {
            fetch(d, s0 + d);
            fetch_sz(d, s0 + d);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int s = s0; s < s1; s += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                compute(d, sr[d], zr[d]);
                fetch(d, s + d + D);
                fetch_sz(d, s + d + D);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // Partial sums of the W waves meet in LDS; each channel block is summed
    // over the waves in a fixed order (deterministic results).
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) red[wave][nb][lane] = acc[nb];
    __syncthreads();
    for (int nb = wave; nb < NB; nb += W) {
        v4f t = red[0][nb][lane];
        for (int w = 1; w < W; ++w) t += red[w][nb][lane];
        const int64_t col = n0 + 16 * nb + r16;
        if (col >= N) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = m0 + 4 * kq + i;
            if (r < M) Y[r * N + col] = t[i];
        }
    }
}

// ------------------------------------------------ LDS-staged, group 128
// Block = 2 K halves x WPH waves x 16 output channels for 16 activation rows.
// In each half, the packed weights, the activations and the scales and zero
// points of 2 consecutive 128-k steps form one stage; a 3-stage ring per half
// is filled with direct buffer->LDS loads two stages ahead of the one being
// multiplied, so many weight bytes are in flight without holding registers.
// The waves of a half read the same activation stage (fetched once per
// half-block, not once per wave).  The halves' partial sums meet in LDS in a
// fixed order.  WPH is chosen so that the blocks cover the output channels in
// one round over the CUs (the 28672-channel layer: 7 waves per half, 256
// blocks).
//
// LDS layouts (all reads are 16 rows x one 16-byte chunk per quarter-wave,
// conflict-free):
//   W (canonical layout): [16*WPH channels][128 B], the channel's whole
//     128-byte line of the stage (both steps; one 1 KB load covers 8
//     channels' lines), piece 4 j + kq (step j, chunk kq) at slot
//     (4 j + kq) ^ ((channel/2) % 8).  Loading 64-byte halves of 16
//     channels' lines per load instead measured 45.5 -> 43.1 us (median,
//     70B-class layer).
//   W plane j (shuffled layout, step j of the stage): [16*WPH channels][64 B],
//     chunk kq at slot kq ^ ((channel/2) % 4)
//   X plane (j, kq): [16 rows][64 B] = the 32 activations x[r][128 j + 32 kq ..
//     + 32] of each row, 16-byte chunk q at slot q ^ kq ^ ((r/2) % 4) (the
//     quarter-waves kq then read distinct slot columns: conflict-free)
//   S, Z: [16*WPH channels][4 groups] fp32, the 16-byte-aligned group quad
//     that holds the stage's groups (canonical layout: loaded by the first
//     stage of each pair of stages only; the second takes its groups from
//     the first one's registers: 44.3 -> 43.0 us on the 70B-class layer)
constexpr int kLSteps = 2;   // 128-k steps per stage
constexpr int kLStages = 3;  // ring depth per half

// PP: the weights and tables come in the GPU-shuffled layout (see
// w4a16_prepack below): per 16-channel block, each 128-k step is 1 KB of
// weights in the LDS order, and each stage's (scale, zero) pairs of its two
// groups are 256 contiguous bytes; a stage then needs one table with
// ceil(WPH / 4) loads instead of two tables of 16-byte pieces.
template <int WPH, bool PP = false>
struct W4a16Lds {
    static constexpr int kCh = 16 * WPH;                       // channels per block
    static constexpr int kW = kCh * 64 * kLSteps;              // weight bytes per stage
    static constexpr int kX = 4096 * kLSteps;                  // activation bytes per stage
    static constexpr int kSZ = PP ? ((WPH + 3) / 4) * 1024     // per table, whole KB
                                  : ((kCh * 16 + 1023) / 1024) * 1024;
    static constexpr int kTabs = PP ? 1 : 2;
    static constexpr int kStage = kW + kX + kTabs * kSZ;
    static constexpr int kLoadsW = kW / 1024, kLoadsX = kX / 1024, kLoadsSZ = kSZ / 1024;
    static constexpr int kLoads = kLoadsW + kLoadsX + kTabs * kLoadsSZ;
    static constexpr int kPerWave = (kLoads + WPH - 1) / WPH;  // every wave issues as many
    static_assert(2 * kLStages * kStage <= 160 * 1024, "ring fits in LDS");
};

template <int WPH, bool PP>
__global__ __launch_bounds__(128 * WPH) void k_w4a16_lds(const uint16_t *__restrict__ X,
                                                         const uint8_t *__restrict__ packed,
                                                         const float *__restrict__ scales,
                                                         const float *__restrict__ zeros,
                                                         float *__restrict__ Y, int64_t M,
                                                         int64_t K64, int64_t N) {
    args_now(X, packed, scales, zeros, Y, M, K64, N);
    using L = W4a16Lds<WPH, PP>;
    __shared__ __align__(16) uint8_t ring[2 * kLStages * L::kStage];  // [half][stage]
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int half = wave / WPH, wl = wave % WPH;
    const int lane = threadIdx.x % kWave;
    const int r16 = lane % 16, kq = lane / 16;
    const int K = (int)K64, KB = K / 2, G = K / 128;
    const int64_t n0 = (int64_t)blockIdx.x * L::kCh;
    const int64_t m0 = (int64_t)blockIdx.y * 16;
    const int cols = (int)min((int64_t)L::kCh, N - n0);
    const int rowsm = (int)min((int64_t)16, M - m0);

    // Descriptors cover exactly this block's channels / rows: channels past N
    // and rows past M read zeros (their outputs are not stored).
    // (Shuffled layout: this block's 16-channel blocks blk0 .. blk0 + nblk - 1.)
    const int blk0 = (int)blockIdx.x * WPH;
    const int nblk = (int)min((int64_t)WPH, (N + 15) / 16 - blk0);
    const v4i rw = PP ? buffer_desc(packed + (int64_t)blk0 * G * 1024, (int64_t)nblk * G * 1024)
                      : buffer_desc(packed + n0 * KB, (int64_t)cols * KB);
    const v4i rx = buffer_desc(X + m0 * K, (int64_t)rowsm * K * 2);
    const v4i rs = PP ? buffer_desc(scales + (int64_t)blk0 * (G / 2) * 64,
                                    (int64_t)nblk * (G / 2) * 256)
                      : buffer_desc(scales + n0 * G, (int64_t)cols * G * 4);
    const v4i rz = PP ? rs : buffer_desc(zeros + n0 * G, (int64_t)cols * G * 4);

    const int T = G / (2 * kLSteps);    // stages per half
    const int s0 = half * T * kLSteps;  // first step of this half
    uint8_t *const hbase = ring + half * kLStages * L::kStage;

    // Stage t of a half covers steps s0 + 2t, s0 + 2t + 1.  Its 1 KB
    // wave-loads q: weights (canonical: channels 8q + lane/8, both steps;
    // shuffled: step j = q / WPH, block q % WPH), then activations (step, plane kq, row lane/4: 64 contiguous bytes per
    // row), then the scale and
    // zero-point tables (lane = channel within a 64-channel group).
    // Wave wl issues q = wl + WPH*i, i < kPerWave; indices past the end repeat
    // the last load (same data to the same place), so every wave issues the
    // same number of loads and waits on the same count.
    const int sw4 = (lane % 4) ^ ((lane / 8) % 4);  // stored slot -> chunk
    auto issue = [&](int t) {
        const uint32_t base = lds_addr(hbase + (t % kLStages) * L::kStage);
        const int step = s0 + kLSteps * t;
#pragma unroll
        for (int i = 0; i < L::kPerWave; ++i) {
            const int q = min(wl + WPH * i, L::kLoads - 1);
            if (q < L::kLoadsW) {
                if (PP) {  // 1 KB of block q % WPH, step + j, already in LDS order
                    const int j = q / WPH;
                    dma16(rw, base + q * 1024, (q % WPH) * G * 1024 + lane * 16, (step + j) * 1024);
                } else {   // the whole 128-byte lines (both steps) of channels 8q .. 8q + 7
                    const int c = 8 * q + lane / 8;
                    dma16(rw, base + q * 1024, c * KB + 16 * ((lane % 8) ^ ((c / 2) % 8)), step * 64);
                }
            } else if (q < L::kLoadsW + L::kLoadsX) {
                const int qq = q - L::kLoadsW, j = qq / 4, pk = qq % 4, r = lane / 4;
                dma16(rx, base + L::kW + qq * 1024, r * K * 2 + 64 * pk + 16 * (sw4 ^ pk),
                      (step + j) * 256);
            } else if (PP) {
                // 256 B of (scale, zero) pairs per 16-channel block: lane / 16
                // picks the block (4 per load), lane % 16 the channel
                const int qq = q - L::kLoadsW - L::kLoadsX, bq = 4 * qq + lane / 16;
                dma16(rs, base + L::kW + L::kX + qq * 1024, bq * (G / 2) * 256 + (lane % 16) * 16,
                      (step / 2) * 256);
            } else if (step % 4 != 0 && t != 0) {
                // the tables' 16-byte quads hold the groups of two stages: the
                // second stage of a pair takes them from the first one's
                // registers, and its table loads become out-of-range loads
                // (zeros, no memory access) into its own unused table area, so
                // every stage still issues the same number of loads
                const int qq = q - L::kLoadsW - L::kLoadsX;
                const int tab = qq / L::kLoadsSZ, part = qq % L::kLoadsSZ;
                dma16(tab == 0 ? rs : rz, base + L::kW + L::kX + tab * L::kSZ + part * 1024, kOOB, 0);
            } else {
                const int qq = q - L::kLoadsW - L::kLoadsX;
                const int tab = qq / L::kLoadsSZ, part = qq % L::kLoadsSZ;
                dma16(tab == 0 ? rs : rz, base + L::kW + L::kX + tab * L::kSZ + part * 1024,
                      (64 * part + lane) * G * 4, (step / 4) * 16);
            }
        }
    };

    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
    // the fast form's constants, set once (as in the register-ring kernel)
    uint32_t mg = 0x64006400u;
    float nz = -0.0f;
    asm volatile("" : "+v"(mg), "+v"(nz));
    const int ch = 16 * wl + r16;                         // this lane's channel
    const int swz = (kq ^ ((r16 / 2) % 4)) * 16;          // (row/2)%4 = (r16/2)%4
    const int woff = ch * 64 + swz;
    // canonical layout: channel ch's line at (ch / 8) KB + (ch % 8) * 128,
    // piece 4 j + kq at slot (4 j + kq) ^ ((ch / 2) % 8)
    int wline[kLSteps];
#pragma unroll
    for (int j = 0; j < kLSteps; ++j)
        wline[j] = (ch / 8) * 1024 + (ch % 8) * 128 + 16 * ((4 * j + kq) ^ ((ch / 2) % 8));
    const int xoff = L::kW + kq * 1024 + r16 * 64;

    float next_s[2] = {0.f, 0.f}, next_z[2] = {0.f, 0.f};  // the pair's second stage
    // `after_vote` (the DMA issue of stage t + 2) runs once the stage's first
    // LDS reads and the vote are issued, so that those reads start right
    // after the barrier (measured: 1.2 % fewer loop cycles)
    auto compute = [&](int t, auto after_vote) {
        const uint8_t *sb = hbase + (t % kLStages) * L::kStage;
        auto rd_w = [&](int j) {
            return *reinterpret_cast<const uint4 *>(sb + (PP ? j * (L::kCh * 64) + woff : wline[j]));
        };
        auto rd_x = [&](int j, int q) {
            return *reinterpret_cast<const uint4 *>(sb + xoff + 4096 * j + (swz ^ (16 * q)));
        };
        // the first step's operands are read before the tables and the vote
        // (measured: 3.8 % fewer loop cycles together with the branch-free vote)
        const uint4 w_first = rd_w(0);
        uint4 x_first[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) x_first[q] = rd_x(0, q);
        float scs[2], zps[2];
        if (PP) {  // (scale, zero) of the stage's two groups
            const float4 e = *reinterpret_cast<const float4 *>(sb + L::kW + L::kX + ch * 16);
            scs[0] = e.x, zps[0] = e.y, scs[1] = e.z, zps[1] = e.w;
        } else {
            const int g0 = (s0 + kLSteps * t) % 4;  // 0 or 2
            if (g0 == 0 || t == 0) {  // scales / zero points of the quad in this stage
                const float4 sc4 = *reinterpret_cast<const float4 *>(sb + L::kW + L::kX + ch * 16);
                const float4 zp4 =
                    *reinterpret_cast<const float4 *>(sb + L::kW + L::kX + L::kSZ + ch * 16);
                scs[0] = g0 ? sc4.z : sc4.x, scs[1] = g0 ? sc4.w : sc4.y;
                zps[0] = g0 ? zp4.z : zp4.x, zps[1] = g0 ? zp4.w : zp4.y;
                next_s[0] = sc4.z, next_s[1] = sc4.w, next_z[0] = zp4.z, next_z[1] = zp4.w;
            } else {  // from the previous stage's quad
                scs[0] = next_s[0], scs[1] = next_s[1], zps[0] = next_z[0], zps[1] = next_z[1];
            }
        }
        bool ok = true;
#pragma unroll
        for (int j = 0; j < kLSteps; ++j)
            ok = ok & fast_group_ok(scs[j], zps[j]);
        const bool fast = __all(ok);
        after_vote();
#pragma unroll
        for (int j = 0; j < kLSteps; ++j) {
            const uint4 w = j == 0 ? w_first : rd_w(j);
            uint4 xr[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) xr[q] = j == 0 ? x_first[q] : rd_x(j, q);
            v4i b0, b1, b2, b3;
            if (fast) {
                const half2v c0 = zero_point_pair(zps[j]), c1 = c0 + k960;
                b0 = dequant8_f16(w.x, scs[j], nz, c0, c1, mg);
                b1 = dequant8_f16(w.y, scs[j], nz, c0, c1, mg);
                b2 = dequant8_f16(w.z, scs[j], nz, c0, c1, mg);
                b3 = dequant8_f16(w.w, scs[j], nz, c0, c1, mg);
            } else {
                b0 = dequant8_direct(w.x, scs[j], zps[j]);
                b1 = dequant8_direct(w.y, scs[j], zps[j]);
                b2 = dequant8_direct(w.z, scs[j], zps[j]);
                b3 = dequant8_direct(w.w, scs[j], zps[j]);
            }
            acc = mfma_bf16(xr[0], b0, acc);
            acc = mfma_bf16(xr[1], b1, acc);
            acc = mfma_bf16(xr[2], b2, acc);
            acc = mfma_bf16(xr[3], b3, acc);
        }
    };

    // Ring: stages t+1 and t+2 are in flight while stage t is multiplied.
    // Before the barrier of step t this wave's loads of stage t are complete
    // (at most the loads of stage t+1 outstanding); after it, every wave is
    // done with stage t-1, whose slot receives stage t+2.
    issue(0);
    if (T > 1) issue(1);
    for (int t = 0; t < T; ++t) {
        if (t + 1 < T)
            wait_and_barrier<L::kPerWave>();
        else
            wait_and_barrier<0>();
        // the slot of stage t + 2 held stage t - 1, which every wave finished
        // before this barrier; the next barrier's wait still leaves only
        // stage t + 2's loads outstanding
        compute(t, [&] {
            if (t + 2 < T) issue(t + 2);
        });
    }

    // the second half's partial sums, added to the first half's in LDS
    wait_and_barrier<0>();
    v4f *red = reinterpret_cast<v4f *>(ring) + wl * kWave + lane;
    if (half == 1) *red = acc;
    wait_and_barrier<0>();
    if (half == 1) return;
    acc = acc + *red;
    const int64_t col = n0 + ch;
    if (col < N) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = m0 + 4 * kq + i;
            if (r < M) Y[r * N + col] = acc[i];
        }
    }
}

bool w4a16_lds_ok(int64_t K, int64_t group) { return group == 128 && K % (256 * kLSteps) == 0; }

template <int WPH, bool PP>
static void go_w4a16_lds(const uint16_t *X, int64_t M, int64_t K, int64_t N, const uint8_t *packed,
                         const float *scales, const float *zeros, float *Y, hipStream_t st) {
    const int64_t mblocks = (M + 15) / 16;
    for (int64_t mb0 = 0; mb0 < mblocks; mb0 += 65535) {
        const int64_t cnt = (mblocks - mb0) < 65535 ? (mblocks - mb0) : 65535;
        dim3 grid((unsigned)((N + 16 * WPH - 1) / (16 * WPH)), (unsigned)cnt);
        launch_main(k_w4a16_lds<WPH, PP>, grid, dim3(128 * WPH), 0, st, X + mb0 * 16 * K, packed,
                    scales, zeros, Y + mb0 * 16 * N, M - mb0 * 16, K, N);
    }
}

// Waves per half: enough channels per block that the channel blocks of one
// 16-row block fit in one round over the 256 CUs (at most 7 waves per half).
template <bool PP>
static void go_w4a16_wph(const uint16_t *X, int64_t M, int64_t K, int64_t N, const uint8_t *packed,
                         const float *scales, const float *zeros, float *Y, hipStream_t st) {
    const int64_t groups16 = (N + 15) / 16;
    const int64_t wph = (groups16 + 255) / 256;
    switch (wph <= 1 ? 1 : wph <= 2 ? 2 : wph <= 4 ? 4 : 7) {
        case 1: go_w4a16_lds<1, PP>(X, M, K, N, packed, scales, zeros, Y, st); break;
        case 2: go_w4a16_lds<2, PP>(X, M, K, N, packed, scales, zeros, Y, st); break;
        case 4: go_w4a16_lds<4, PP>(X, M, K, N, packed, scales, zeros, Y, st); break;
        default: go_w4a16_lds<7, PP>(X, M, K, N, packed, scales, zeros, Y, st); break;
    }
}

hipError_t launch_w4a16_lds(const uint16_t *X, int64_t M, int64_t K, int64_t N,
                            const uint8_t *packed, const float *scales, const float *zeros,
                            float *Y, hipStream_t st) {
    go_w4a16_wph<false>(X, M, K, N, packed, scales, zeros, Y, st);
    return hipGetLastError();
}

hipError_t launch_w4a16_prepacked(const uint16_t *X, int64_t M, int64_t K, int64_t N,
                                  const uint8_t *wpp, const float *szpp, float *Y,
                                  hipStream_t st) {
    go_w4a16_wph<true>(X, M, K, N, wpp, szpp, nullptr, Y, st);
    return hipGetLastError();
}

// ------------------------------------------------ shuffled-layout conversion
// wpp[b][t][c][16 p + i] = packed[16 b + c][64 t + 16 (p ^ ((c / 2) % 4)) + i]
// (zero for padding channels); szpp[b][u][c] = (s, z) of groups 2u, 2u + 1.
// One thread per 16-byte unit of the destination (prepack) or of the
// canonical arrays (unprepack); 16-byte aligned arrays.  The weight part
// needs K % 128 == 0 (it also serves the W4A8 codes), the tables K % 512 == 0.
__global__ void k_w4_prepack_weights(const uint8_t *__restrict__ packed, int64_t K, int64_t N,
                                     uint8_t *__restrict__ wpp) {
    const int64_t S = K / 128, KB = K / 2, NB = (N + 15) / 16;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < NB * S * 64; u += stride) {
        const int64_t p = u % 4, c = (u / 4) % 16, t = (u / 64) % S, b = u / (64 * S);
        const int64_t n = 16 * b + c, chunk = p ^ ((c / 2) % 4);
        uint4 v = {0u, 0u, 0u, 0u};
        if (n < N) v = *reinterpret_cast<const uint4 *>(packed + n * KB + 64 * t + 16 * chunk);
        reinterpret_cast<uint4 *>(wpp)[u] = v;
    }
}

__global__ void k_w4a16_prepack_tables(const float *__restrict__ scales,
                                       const float *__restrict__ zeros, int64_t K, int64_t N,
                                       float *__restrict__ szpp) {
    const int64_t S = K / 128, NB = (N + 15) / 16;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < NB * (S / 2) * 16;
         e += stride) {
        const int64_t c = e % 16, uu = (e / 16) % (S / 2), b = e / (16 * (S / 2));
        const int64_t n = 16 * b + c;
        float4 v = {0.f, 0.f, 0.f, 0.f};
        if (n < N)
            v = float4{scales[n * S + 2 * uu], zeros[n * S + 2 * uu], scales[n * S + 2 * uu + 1],
                       zeros[n * S + 2 * uu + 1]};
        reinterpret_cast<float4 *>(szpp)[e] = v;
    }
}

__global__ void k_w4_unprepack_weights(const uint8_t *__restrict__ wpp, int64_t K, int64_t N,
                                       uint8_t *__restrict__ packed) {
    const int64_t S = K / 128, KB = K / 2;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < N * (KB / 16);
         u += stride) {
        const int64_t n = u / (KB / 16), off = (u % (KB / 16)) * 16;
        const int64_t b = n / 16, c = n % 16, t = off / 64, chunk = (off % 64) / 16;
        const int64_t p = chunk ^ ((c / 2) % 4);
        reinterpret_cast<uint4 *>(packed)[u] =
            *reinterpret_cast<const uint4 *>(wpp + ((b * S + t) * 16 + c) * 64 + 16 * p);
    }
}

__global__ void k_w4a16_unprepack_tables(const float *__restrict__ szpp, int64_t K, int64_t N,
                                         float *__restrict__ scales, float *__restrict__ zeros) {
    const int64_t S = K / 128;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < N * S; e += stride) {
        const int64_t n = e / S, g = e % S, b = n / 16, c = n % 16;
        const float *src = szpp + ((b * (S / 2) + g / 2) * 16 + c) * 4 + 2 * (g % 2);
        scales[e] = src[0];
        zeros[e] = src[1];
    }
}

static unsigned conv_blocks(int64_t n) {
    const int64_t b = (n + 255) / 256;
    return (unsigned)(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

hipError_t launch_w4_prepack_weights(const uint8_t *packed, int64_t K, int64_t N, uint8_t *wpp,
                                    hipStream_t st) {
    const int64_t units = ((N + 15) / 16) * (K / 128) * 64;
    hipLaunchKernelGGL(k_w4_prepack_weights, dim3(conv_blocks(units)), dim3(256), 0, st, packed, K,
                       N, wpp);
    return hipGetLastError();
}

hipError_t launch_w4_unprepack_weights(const uint8_t *wpp, int64_t K, int64_t N, uint8_t *packed,
                                      hipStream_t st) {
    hipLaunchKernelGGL(k_w4_unprepack_weights, dim3(conv_blocks(N * (K / 32))), dim3(256), 0, st,
                       wpp, K, N, packed);
    return hipGetLastError();
}

hipError_t launch_w4a16_prepack(const uint8_t *packed, const float *scales, const float *zeros,
                                int64_t K, int64_t N, uint8_t *wpp, float *szpp, hipStream_t st) {
    const hipError_t err = launch_w4_prepack_weights(packed, K, N, wpp, st);
    if (err != hipSuccess) return err;
    const int64_t e = ((N + 15) / 16) * (K / 256) * 16;
    hipLaunchKernelGGL(k_w4a16_prepack_tables, dim3(conv_blocks(e)), dim3(256), 0, st, scales,
                       zeros, K, N, szpp);
    return hipGetLastError();
}

hipError_t launch_w4a16_unprepack(const uint8_t *wpp, const float *szpp, int64_t K, int64_t N,
                                  uint8_t *packed, float *scales, float *zeros, hipStream_t st) {
    const hipError_t err = launch_w4_unprepack_weights(wpp, K, N, packed, st);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_w4a16_unprepack_tables, dim3(conv_blocks(N * (K / 128))), dim3(256), 0, st,
                       szpp, K, N, scales, zeros);
    return hipGetLastError();
}

hipError_t launch_w4a16_mfma(const uint16_t *X, int64_t M, int64_t K, int64_t N,
                             const uint8_t *packed, const float *scales, const float *zeros,
                             int64_t group, float *Y, hipStream_t st) {
    constexpr int NB = 4, D = 1, W = 8;
    const int64_t mblocks = (M + 15) / 16;
    for (int64_t mb0 = 0; mb0 < mblocks; mb0 += 65535) {
        const int64_t cnt = (mblocks - mb0) < 65535 ? (mblocks - mb0) : 65535;
        dim3 grid((unsigned)((N + 16 * NB - 1) / (16 * NB)), (unsigned)cnt);
        if (group == 128)
            launch_main(k_w4a16_mfma<NB, D, W, true>, grid, dim3(64 * W), 0, st, X + mb0 * 16 * K,
                        packed, scales, zeros, Y + mb0 * 16 * N, M - mb0 * 16, K, N, group);
        else
            launch_main(k_w4a16_mfma<NB, D, W, false>, grid, dim3(64 * W), 0, st, X + mb0 * 16 * K,
                        packed, scales, zeros, Y + mb0 * 16 * N, M - mb0 * 16, K, N, group);
    }
    return hipGetLastError();
}

}  // namespace w4
