// Decode-shaped W4A8 products (few activation rows, many output channels):
// the packed int4 weights are streamed from HBM once with 128-bit loads and
// unpacked in registers (Keras INT4 guide, "How it works", steps 4-5).  The
// same kernels run the W8A8 product (the guide's INT8 path: int8 weight codes,
// no unpacking) when instantiated with W8 = true.
//
//  * k_gemv_dot4  (M <= 4): VALU dot products (v_dot4_i32_i8).  The
//    activation quantization (step 3) is fused into the prologue, so one
//    launch runs steps 3-6.
//  * k_gemv_mfma  (M <= 64): int8 MFMA 16x16x64 with the weight operand
//    unpacked in registers; the activations come pre-quantized in P8 layout,
//    or, for M <= 16 and short rows, are quantized in the prologue (G > 0).
//
// All global loads are raw buffer loads: out-of-range lanes get zeros from
// the descriptor's range check instead of an exec-mask branch, so a lane's
// loads issue back to back and the vmcnt waits stay in program order.  The
// weights, read exactly once per launch, carry the non-temporal hint where a
// load covers whole cache lines (the dot4 GEMV; the MFMA GEMV on shuffled
// tiles; measured: Gemma-like M = 1 step 3.37 -> 3.05 us, 7B-class 6.34 ->
// 6.08 us); the activations, which every workgroup reads, stay cacheable.
#include "common.h"
#include "kernels.h"

#include <atomic>

namespace w4 {

// ------------------------------------------------------------------ dot4
// Block = ROWS output channels x 16 lanes.  Lane j of a channel streams the
// 16-byte chunks j, j+16, ..., j+16*(UB-1) of that channel's packed row (one
// chunk = 32 codes), so a wave reads 4 rows x 256 contiguous bytes per load.
// Order of work: (1) issue the activation loads, (2) once every wave of the
// block has, issue the weight chunks (all of them, or the first PRE), (3)
// quantize the activations into LDS (P8 layout) while the weights are in
// flight (the barriers wait for LDS only, so the weight loads stay in
// flight), then issue the remaining chunks, (4) dot products, chunk by chunk
// as the loads land, (5) 16-lane DPP sum and epilogue.
// With W8 a 16-byte chunk holds 16 int8 codes (instead of 32 int4 codes) and
// the activations stay in natural order.
constexpr int kDot4MaxK = 8192, kDot4MaxKW8 = 4096;

bool gemv_dot4_ok(int64_t M, int64_t K, bool w8) {
    return M >= 1 && M <= 4 && K % 32 == 0 && K <= (w8 ? kDot4MaxKW8 : kDot4MaxK);
}

// DIV (with FUSED): the activations are divided by per-column divisors
// (a.act_div) before their quantization -- the activation side of AWQ-style
// channel scaling.
// PP: the int4 codes come in the shuffled tile layout (ROWS % 16 == 0, K % 128
// == 0): chunk c of row r of a 16-channel block sits in tile c / 4 at slot
// (c % 4) ^ ((r / 2) % 4), so the 4 rows of a wave still read 256 contiguous
// bytes per tile.
// PRE (FUSED): the lane requests its first PRE weight chunks before the
// activation quantization and the rest right after it (PRE == UB: all
// before).  The quantization's barriers wait for every wave of the block,
// and a wave whose weight requests back up in the CU's memory pipeline
// reaches them late; with one block per CU and half of the chunks requested
// up front the block's codes are ready while the first half streams in.
template <int M, int ROWS, int UB, bool FUSED, Out OUT, bool W8, bool DIV = false,
          bool PP = false, int PRE = UB>
__global__ __launch_bounds__(16 * ROWS) void k_gemv_dot4(W4A8Args args) {
    static_assert(PRE >= 0 && PRE <= UB && (FUSED || PRE == UB), "chunks before the quantization");
    const W4A8Args a = args_now(args);
    constexpr int T = 16 * ROWS;  // threads
    constexpr int KPC = W8 ? 16 : 32;  // codes per 16-byte chunk
    // 8-groups of k per thread (K <= 16 * KPC * UB): pre-quantized input
    constexpr int NG = (2 * KPC * UB / 16 + ROWS - 1) / ROWS;
    // 4-groups of k per thread: fp32 input (spread over every thread, so that
    // the quantization chain each thread runs is as short as it can be)
    constexpr int NQ = (4 * KPC * UB + T - 1) / T;
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ float red[T / kWave][M];
    int8_t *xs = reinterpret_cast<int8_t *>(smem);
    const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
    const int K = (int)a.K, KB = W8 ? K : K / 2, C = K / KPC, G8 = K / 8, G4 = K / 4;
    const int j = t & 15, r = t >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * ROWS;
    const int rows = (int)min((int64_t)ROWS, a.N - n0);

    // (1) activations: fp32 4-group q = t + T*i holds k = 4q .. 4q+3 of each
    // row; int8 8-group g = t + T*i holds k = 8g .. 8g+7.
    float4 xv[M][FUSED ? NQ : 1];
    float4 dv[DIV ? NQ : 1];
    uint2 xn[M][FUSED ? 1 : NG];
    if constexpr (FUSED) {
        const auto rx = make_rsrc(a.X, (int64_t)M * K * 4);
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int q = t + T * i;
                xv[m][i] = bloadf4(rx, q < G4 ? (m * K + 4 * q) * 4 : kOOB);
            }
        if (DIV) {
            // divisors of the thread's 4-groups (out-of-range groups read 0
            // and are replaced by 1 where they are used)
            const auto rd = make_rsrc(a.act_div, (int64_t)K * 4);
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int q = t + T * i;
                dv[i] = bloadf4(rd, q < G4 ? 16 * q : kOOB);
            }
        }
    } else {
        const auto rq = make_rsrc(a.Xq, (int64_t)M * K);
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                const int g = t + T * i;
                xn[m][i] = bload8(rq, g < G8 ? m * K + 8 * g : kOOB);
            }
    }

    // Every wave's activation loads enter the CU's memory pipeline before any
    // wave's weight loads: that pipeline returns data in order, and an
    // activation load queued behind another wave's weight misses would hold
    // the quantization below for an HBM round trip (measured: Gemma-like
    // M = 1 3.08 -> 2.80 us, 7B-class 6.11 -> 5.83 us).  The barrier does not
    // wait for the loads.
    __builtin_amdgcn_sched_barrier(0);
    issue_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // (2) weights of this block's rows: the lane's first PRE chunks here, the
    // rest right after the quantization.
    static_assert(!PP || (ROWS % 16 == 0 && !W8), "shuffled int4 tiles of 16 channels");
    // (shuffled tiles: the block's ROWS / 16 channel blocks of K / 128 tiles
    // each; channels past N are zero padding inside their block)
    const int tiles = K / 128;
    const auto rw = PP ? make_rsrc(a.packed + (n0 / 16) * (int64_t)tiles * 1024,
                                   (int64_t)((rows + 15) / 16) * tiles * 1024)
                       : make_rsrc(a.packed + n0 * KB, (int64_t)rows * KB);
    const int rowoff = PP ? (r / 16) * tiles * 1024 : r * KB;
    const int rr = r % 16;  // row inside the channel block (shuffled tiles)
    uint4 wb[UB];
    auto wload = [&](int u) {
        const int c = j + 16 * u;
        const int off = PP ? rowoff + ((c / 4) * 16 + rr) * 64 + 16 * ((c % 4) ^ ((rr / 2) % 4))
                           : rowoff + 16 * c;
        wb[u] = bload16_nt(rw, c < C ? off : kOOB);
    };
#pragma unroll
    for (int u = 0; u < PRE; ++u) wload(u);

    // Epilogue operands, so their latency hides behind the main work.
    const int64_t n = n0 + r;
    const int64_t nc = r < rows ? n : n0;
    const float swn = (OUT == Out::Y) ? a.sw[nc] : 0.0f;
    const float bn = (OUT == Out::Y && a.bias) ? a.bias[nc] : 0.0f;
    // Keep the scheduler from interleaving the activation math (which waits
    // for the activation loads) with the loads above.
    __builtin_amdgcn_sched_barrier(0);

    // (3) activations -> int8 P8 layout in LDS, scales in registers.
    float sxm[M];
    if constexpr (FUSED && DIV) {
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            if (t + T * i >= G4) dv[i] = float4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
            for (int m = 0; m < M; ++m) {
                xv[m][i].x = xv[m][i].x / dv[i].x;
                xv[m][i].y = xv[m][i].y / dv[i].y;
                xv[m][i].z = xv[m][i].z / dv[i].z;
                xv[m][i].w = xv[m][i].w / dv[i].w;
            }
        }
    }
    if constexpr (FUSED) {
        // row absmax: thread, wave (integer DPP max of the non-negative
        // values' bits), then the block's waves through LDS
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float am = 0.0f;
#pragma unroll
            for (int i = 0; i < NQ; ++i)
                am = fmaxf(am, fmaxf(fmaxf(fabsf(xv[m][i].x), fabsf(xv[m][i].y)),
                                     fmaxf(fabsf(xv[m][i].z), fabsf(xv[m][i].w))));
            am = wave_max_nonneg(am);
            if (lane == 0) red[wave][m] = am;
        }
        lds_barrier();
        // codes of a 4-group (low bytes of c0..c3) into the LDS copy of the
        // row: P8 order [x0 x2 x4 x6 | x1 x3 x5 x7] inside each 8-group, so
        // the group's even k go to bytes 2h, 2h+1 and its odd k to bytes
        // 4+2h, 5+2h of 8-group q/2 (h = q%2); natural order for 8-bit weights
        auto put = [&](int m, int q, uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3) {
            if (W8) {
                *reinterpret_cast<uint32_t *>(xs + m * K + 4 * q) =
                    (c0 & 0xFFu) | ((c1 & 0xFFu) << 8) | ((c2 & 0xFFu) << 16) | (c3 << 24);
            } else {
                int8_t *g = xs + m * K + 8 * (q >> 1) + 2 * (q & 1);
                *reinterpret_cast<uint16_t *>(g) = (uint16_t)((c0 & 0xFFu) | ((c2 & 0xFFu) << 8));
                *reinterpret_cast<uint16_t *>(g + 4) = (uint16_t)((c1 & 0xFFu) | ((c3 & 0xFFu) << 8));
            }
        };
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float am = red[0][m];
#pragma unroll
            for (int w = 1; w < T / kWave; ++w) am = fmaxf(am, red[w][m]);
            const float s = (am == 0.0f) ? 0.0f : div127(am);
            sxm[m] = s;
            if (s >= kFastQuotientMinScale) {  // row-uniform
                // correctly rounded quotient without a division, rounded by
                // one add (|v / s| <= 127.5 for every value of the row)
                const float rs = 1.0f / s;
#pragma unroll
                for (int i = 0; i < NQ; ++i) {
                    const int q = t + T * i;
                    if (q < G4) {
                        const float4 v = xv[m][i];
                        put(m, q, code_in_low_byte(quotient_rn(v.x, s, rs)),
                            code_in_low_byte(quotient_rn(v.y, s, rs)),
                            code_in_low_byte(quotient_rn(v.z, s, rs)),
                            code_in_low_byte(quotient_rn(v.w, s, rs)));
                    }
                }
            } else {  // zero or tiny scale: IEEE division per value
#pragma unroll
                for (int i = 0; i < NQ; ++i) {
                    const int q = t + T * i;
                    if (q < G4) {
                        const float4 v = xv[m][i];
                        put(m, q, (uint32_t)quant_code(v.x, s, -128.f, 127.f),
                            (uint32_t)quant_code(v.y, s, -128.f, 127.f),
                            (uint32_t)quant_code(v.z, s, -128.f, 127.f),
                            (uint32_t)quant_code(v.w, s, -128.f, 127.f));
                    }
                }
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            sxm[m] = (OUT == Out::Y) ? a.sx[m] : 0.0f;
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                const int g = t + T * i;
                if (g < G8) {
                    uint2 p = xn[m][i];
                    if (!W8) natural_to_p8(xn[m][i].x, xn[m][i].y, p.x, p.y);
                    *reinterpret_cast<uint2 *>(xs + m * K + 8 * g) = p;
                }
            }
        }
    }
    lds_barrier();
#pragma unroll
    for (int u = PRE; u < UB; ++u) wload(u);

    // (4) int8 dot products of 16*code with the P8 activations (of the int8
    // codes with the natural-order activations for 8-bit weights).
    int acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0;
#pragma unroll
    for (int u = 0; u < UB; ++u) {
        // Past the end of the row the weights are zero; clamp the LDS read.
        const int cx = min(j + 16 * u, C - 1);
        const uint4 w = wb[u];
        if (W8) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const uint4 x0 = *reinterpret_cast<const uint4 *>(xs + m * K + cx * 16);
                int s = acc[m];
                s = __builtin_amdgcn_sdot4((int)w.x, (int)x0.x, s, false);
                s = __builtin_amdgcn_sdot4((int)w.y, (int)x0.y, s, false);
                s = __builtin_amdgcn_sdot4((int)w.z, (int)x0.z, s, false);
                s = __builtin_amdgcn_sdot4((int)w.w, (int)x0.w, s, false);
                acc[m] = s;
            }
            continue;
        }
        const uint32_t l0 = lo16(w.x), h0 = hi16(w.x), l1 = lo16(w.y), h1 = hi16(w.y);
        const uint32_t l2 = lo16(w.z), h2 = hi16(w.z), l3 = lo16(w.w), h3 = hi16(w.w);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const uint4 *xp = reinterpret_cast<const uint4 *>(xs + m * K + cx * 32);
            const uint4 x0 = xp[0], x1 = xp[1];
            int s = acc[m];
            s = __builtin_amdgcn_sdot4((int)l0, (int)x0.x, s, false);
            s = __builtin_amdgcn_sdot4((int)h0, (int)x0.y, s, false);
            s = __builtin_amdgcn_sdot4((int)l1, (int)x0.z, s, false);
            s = __builtin_amdgcn_sdot4((int)h1, (int)x0.w, s, false);
            s = __builtin_amdgcn_sdot4((int)l2, (int)x1.x, s, false);
            s = __builtin_amdgcn_sdot4((int)h2, (int)x1.y, s, false);
            s = __builtin_amdgcn_sdot4((int)l3, (int)x1.z, s, false);
            s = __builtin_amdgcn_sdot4((int)h3, (int)x1.w, s, false);
            acc[m] = s;
        }
    }

    // (5) sum the 16 lanes of each channel; divide out the 16 of the int4 codes.
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = W8 ? sum16(acc[m]) : (sum16(acc[m]) >> 4);
    if (j == 0 && r < rows) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            if (OUT == Out::I32) {
                a.acc[(int64_t)m * a.N + n] = acc[m];
            } else {
                const float s = sxm[m] * swn;
                float y = (float)acc[m] * s;
                if (a.bias) y = y + bn;
                y = relu_if(y, a.relu);
                a.Y[(int64_t)m * a.N + n] = y;
            }
        }
    }
}

static int device_cus();

// Int4 codes, fused quantization, M <= 2: one block per CU (the fewest channels per
// block, a multiple of 16 up to 64, that needs no more blocks than the device
// has CUs) with half of each lane's chunks requested before the quantization
// (graph-free back-to-back launches, us: 7B-class M = 1 6.10 -> 5.40 with 48
// channels, Gemma-like 3.17 -> 3.00 with 32; with 16 channels and half of
// the chunks early 7B-class 5.68, Gemma-like with a third early 3.57).
// Layers of up to 16 channels per CU keep 16 channels and every chunk up
// front.
template <int M, int UB, bool W8, bool DIV, bool PP>
static bool go_dot4_wide(const W4A8Args &a, hipStream_t st) {
    const int64_t cus = device_cus();
    constexpr int PRE = (UB + 1) / 2;
    const uint32_t shm = (uint32_t)(M * a.K);
    auto go = [&](auto kernel, int rows) {
        launch_main(kernel, dim3((unsigned)((a.N + rows - 1) / rows)), dim3(16 * rows), shm, st,
                    a);
    };
    if (a.N <= 16 * cus) return false;
    if (a.N <= 32 * cus)
        go(k_gemv_dot4<M, 32, UB, true, Out::Y, W8, DIV, PP, PRE>, 32);
    else if (a.N <= 48 * cus)
        go(k_gemv_dot4<M, 48, UB, true, Out::Y, W8, DIV, PP, PRE>, 48);
    else
        go(k_gemv_dot4<M, 64, UB, true, Out::Y, W8, DIV, PP, PRE>, 64);
    return true;
}

template <int M, int ROWS, int UB, bool W8>
static void go_dot4(const W4A8Args &a, hipStream_t st) {
    dim3 grid((unsigned)((a.N + ROWS - 1) / ROWS));
    const uint32_t shm = (uint32_t)(M * a.K);
    // (int4 codes only: with int8 codes it measured slower at 7B-class size,
    // 9.14 -> 9.67 us, and within noise at Gemma-like size; on shuffled tiles
    // faster at 7B-class size, 5.84 -> 5.44 us, slower with three chunks per
    // lane, Gemma-like 2.82 -> 3.06 us)
    if constexpr (M <= 2 && !W8) {
        if (a.pp) {
            if constexpr (UB >= 8) {
                if (go_dot4_wide<M, UB, false, false, true>(a, st)) return;
            }
        } else if (a.out == Out::Y && a.X) {
            if (a.act_div ? go_dot4_wide<M, UB, false, true, false>(a, st)
                          : go_dot4_wide<M, UB, false, false, false>(a, st))
                return;
        }
    }
    if constexpr (!W8) {
        if (a.pp) {  // shuffled layout: fused forward only
            launch_main(k_gemv_dot4<M, ROWS, UB, true, Out::Y, false, false, true>, grid,
                        dim3(16 * ROWS), shm, st, a);
            return;
        }
    }
    if (a.out == Out::I32)
        launch_main(k_gemv_dot4<M, ROWS, UB, false, Out::I32, W8>, grid, dim3(16 * ROWS), shm, st,
                    a);
    else if (a.X && a.act_div)
        launch_main(k_gemv_dot4<M, ROWS, UB, true, Out::Y, W8, true>, grid, dim3(16 * ROWS), shm,
                    st, a);
    else if (a.X)
        launch_main(k_gemv_dot4<M, ROWS, UB, true, Out::Y, W8>, grid, dim3(16 * ROWS), shm, st, a);
    else
        launch_main(k_gemv_dot4<M, ROWS, UB, false, Out::Y, W8>, grid, dim3(16 * ROWS), shm, st,
                    a);
}

// UB = chunks per lane, the smallest instantiated value >= ceil(chunks / 16).
template <int M, bool W8>
static void go_dot4_m(const W4A8Args &a, hipStream_t st) {
    const int64_t ub = (a.K / (W8 ? 16 : 32) + 15) / 16;
    if (ub <= 2)
        go_dot4<M, 16, 2, W8>(a, st);
    else if (ub <= 3)
        go_dot4<M, 16, 3, W8>(a, st);
    else if (ub <= 4)
        go_dot4<M, 16, 4, W8>(a, st);
    else if (ub <= 8)
        go_dot4<M, 16, 8, W8>(a, st);
    else
        go_dot4<M, 16, 16, W8>(a, st);
}

template <bool W8>
static void go_dot4_w(const W4A8Args &a, hipStream_t st) {
    switch (a.M) {
        case 1: go_dot4_m<1, W8>(a, st); break;
        case 2: go_dot4_m<2, W8>(a, st); break;
        case 3: go_dot4_m<3, W8>(a, st); break;
        default: go_dot4_m<4, W8>(a, st); break;
    }
}

hipError_t launch_gemv_dot4(const W4A8Args &a, hipStream_t st) {
    if (a.w8)
        go_dot4_w<true>(a, st);
    else
        go_dot4_w<false>(a, st);
    return hipGetLastError();
}

// ------------------------------------------------------------------ MFMA
// Block = W waves that split K into W slices and cover the same 16*NB output
// channels for 16*MB activation rows; the partial int32 sums meet in LDS
// (integer adds, so their order does not matter).  Many waves per block keep
// enough weight bytes in flight to cover the HBM latency even though a
// decode-batch layer has few output-channel blocks.
// Per 128-k step a lane loads 16 packed bytes (32 codes) of one channel:
//   lane l: channel n0 + 16*nb + l%16, codes k = 128*s + 32*(l/16) + [0, 32)
// and the matching 2 x 16 P8 activation bytes of row 16*mb + l%16 (the
// activations are stored chunk-major, so one load reads 16 consecutive rows
// x 16 bytes of four chunks; rows past M read other chunks' rows or zeros
// and only feed outputs that are not stored), which
// feed two v_mfma_i32_16x16x64_i8 (the first 16 and the last 16 codes of each
// lane).  The weight and activation operands use identical k slots per lane,
// so the order in which the MFMA consumes the slots does not matter.
// With W8 the lane loads the 32 int8 codes of the same k slots (two 16-byte
// loads) and the activations come in natural order.
// Accumulator layout (16x16 i32): lane l holds rows 4*(l/16)+i, column l%16.
// Weights and activations of the next D steps are in flight in a register
// ring while the current step multiplies.  Rows past M and channels past N
// read zeros (their outputs are not stored).
// PP: the int4 codes come in the shuffled tile layout: the (nb, step) load of
// a wave is one contiguous 1 KB tile (lane (r16, kq) takes slot kq ^ ((r16/2)%4)).
// G > 0 (fused activation quantization, M <= 16, K <= 512 G, fp32 X): the
// workgroup quantizes the activation rows itself into LDS, in the same
// chunk-major layout with 16 rows (rows past M get zero codes): wave w takes
// rows w and w + 8 (8 waves) or row w (16 waves), lane l the 8-groups l,
// l + 64, ... of the row; the loads
// of row w precede the weight loads of the first steps, the row absmax is a
// wave reduction, the codes come from the same division-free chain as in the
// dot4 kernel (measured: Gemma-like M = 8 4.90 -> 4.63 us, bit-identical),
// and the codes and row scales go to LDS before one barrier (the first
// weight loads stay in flight).  The main loop
// then reads the activation fragments from LDS.
// LN (whole-line loads, canonical layout): a load above covers half of each
// of 16 channels' 128-byte lines; with LN load 0 of a unit covers the whole
// lines of channels 0-7 of the block and load 1 those of channels 8-15 (lane
// (kq, r): 16-byte piece 2 kq + r / 8 of channel r % 8, resp. 8 + r % 8), and
// lanes r and r ^ 8 then swap one of the two words (a DPP row rotate by 8),
// after which every lane holds pieces 2 kq and 2 kq + 1 of its own channel r.
// For int4 codes a line is two 128-k steps, so the loop runs over pairs of
// steps (K % 256 = 0) and the activation fragments of pair t are the chunks
// 16 t + 4 kq + j, j = 0..3; for int8 codes a line is one step and the pieces
// are the ones the lane loads without LN.  Measured (graph-replayed, rotating
// weights, 7B-class layer): M = 16 step 11.1 -> 10.4 us, M = 24 11.8 -> 11.7,
// M = 48 13.8 -> 14.1 and M = 64 14.8 -> 15.4 (hence int4 LN only up to two
// row blocks); W8 M = 16 14.9 -> 14.6, M = 64 20.4 -> 19.8; fused int4 M = 4
// 9.4 -> 9.1, M = 8 9.8 -> 9.6; fused W8 M = 8 13.4 -> 13.6 before the loads
// were made non-temporal, 13.4 -> 12.5 after (used).
// In the fused kernel (activation fragments from LDS) the next pair's weights
// are requested between the MFMAs of the pair's two halves (fused M = 4
// 9.1 -> 8.9 us, M = 8 9.75 -> 9.5 us); with the activations from HBM / L2
// that order was slower (M = 16 10.45 -> 10.87 us), so there the whole next
// pair is requested after both halves.
template <int MB, int NB, int D, int W, Out OUT, bool W8, bool PP = false, int G = 0, bool LN = false>
__global__ __launch_bounds__(64 * W) void k_gemv_mfma(W4A8Args args) {
    const W4A8Args a = args_now(args);
    constexpr bool FUSED = G > 0;
    static_assert(!FUSED || (MB == 1 && (W == 8 || W == 16) && OUT == Out::Y),
                  "fused: 16 rows, 8 or 16 waves");
    __shared__ __align__(16) int8_t xs[FUSED ? 16 * 512 * G : 16];  // [K/16][16][16]
    __shared__ float sxs[16];
    constexpr int WL = (W8 || LN) ? 2 : 1;  // 16-byte weight loads per lane and unit
    constexpr bool LP = LN && !W8;  // int4 codes: units of two 128-k steps
    constexpr int kPairs = MB * NB;                 // 16x16 output blocks
    constexpr int kPerWave = (kPairs + W - 1) / W;  // epilogue blocks per wave
    __shared__ int red[kPairs * 4 * kWave];         // [pair][i][lane]
    // wave-uniform (scalar) so the K-range loop branches are scalar branches
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int r16 = lane % 16, kq = lane / 16;
    const int K = (int)a.K, KB = W8 ? K : K / 2;
    const int64_t N = a.N, M = a.M;
    const int S = K / 128;
    const int SU = LP ? S / 2 : S;  // loop units: 128-k steps, or pairs of them
    const int s0 = SU * wave / W, s1 = SU * (wave + 1) / W;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * NB;
    const int cols = (int)min((int64_t)(16 * NB), N - n0);

    for (int t = threadIdx.x; t < kPairs * 4 * kWave; t += 64 * W) red[t] = 0;
    if (!FUSED) __syncthreads();  // (fused: the prologue's barrier covers it)

    static_assert(!PP || !W8, "shuffled layout of int4 codes");
    static_assert(!LN || !PP, "whole-line loads: canonical layout");
    const auto rb = PP ? make_rsrc(a.packed + (n0 / 16) * (int64_t)S * 1024,
                                   (int64_t)((cols + 15) / 16) * S * 1024)
                       : make_rsrc(a.packed + n0 * KB, (int64_t)cols * KB);
    const auto ra = make_rsrc(a.Xq, M * K);
    int boff[NB], aoff[MB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        boff[nb] = PP ? nb * S * 1024 + r16 * 64 + 16 * (kq ^ ((r16 / 2) % 4))
                 : LN ? (16 * nb + r16 % 8) * KB + 16 * (2 * kq + r16 / 8)
                      : (16 * nb + r16) * KB + kq * 16 * WL;
    const int wstep = PP ? 1024 : LP ? 128 : 64 * WL;  // bytes per unit
    const int hstep = LN ? 8 * KB : 16;                 // second load of a unit
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) aoff[mb] = ((LP ? 4 : 2) * kq * (int)M + 16 * mb + r16) * 16;
    // activations are chunk-major, [K/16][M][16]: chunk c = 8 s + 2 kq + half
    // (LN with int4 codes: c = 16 t + 4 kq + j for pair t)
    const int achunk = (int)M * 16, astep = (LP ? 16 : 8) * achunk;
    // LDS copy (fused): [K/16][16][16]
    const int xso = ((LP ? 4 : 2) * kq * 16 + r16) * 16, xsstep = LP ? 4096 : 2048;

    v4i acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = v4i{0, 0, 0, 0};

    uint4 wr[D][NB][WL], xr0[D][MB], xr1[D][MB], xr2[D][MB], xr3[D][MB];
    // Weight loads: a shuffled 1 KB tile, or with LN a set of whole 128-byte
    // lines, is read whole by one load and never again, so it streams
    // (non-temporal; with LN, graph-replayed 7B-class M = 16 10.45 -> 10.15 us,
    // M = 24 11.6 -> 11.05, W8 M = 16 14.5 -> 13.05, M = 64 19.9 -> 19.0); a
    // half-line load (canonical layout without LN) leaves the other half of
    // its lines to the next step or the second load, so those stay cached.
    auto wload = [&](const __amdgpu_buffer_rsrc_t &r, int off) {
        return (PP || LN) ? bload16_nt(r, off) : bload16(r, off);
    };
    // weights and the activation fragments of the unit's first half (for LP:
    // the chunks of piece 2 kq), then those of its second half (piece 2 kq + 1)
    auto fetch_wa = [&](int d, int ss) {
        const bool ok = ss < s1;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int h = 0; h < WL; ++h)
                wr[d][nb][h] = wload(rb, ok ? boff[nb] + wstep * ss + hstep * h : kOOB);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if (FUSED) {  // from LDS (16 rows per chunk); steps past s1 hold zero weights
                const int o = xso + xsstep * min(ss, SU - 1);
                xr0[d][mb] = *reinterpret_cast<const uint4 *>(xs + o);
                xr1[d][mb] = *reinterpret_cast<const uint4 *>(xs + o + 256);
            } else {
                const int o = ok ? aoff[mb] + astep * ss : kOOB;
                xr0[d][mb] = bload16(ra, o);
                xr1[d][mb] = bload16(ra, ok ? o + achunk : kOOB);
            }
        }
    };
    auto fetch_b = [&](int d, int ss) {
        if constexpr (LP) {
            const bool ok = ss < s1;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                if (FUSED) {
                    const int o = xso + xsstep * min(ss, SU - 1);
                    xr2[d][mb] = *reinterpret_cast<const uint4 *>(xs + o + 512);
                    xr3[d][mb] = *reinterpret_cast<const uint4 *>(xs + o + 768);
                } else {
                    const int o = ok ? aoff[mb] + astep * ss + 2 * achunk : kOOB;
                    xr2[d][mb] = bload16(ra, o);
                    xr3[d][mb] = bload16(ra, ok ? o + achunk : kOOB);
                }
            }
        }
    };
    auto fetch = [&](int d, int ss) {
        fetch_wa(d, ss);
        fetch_b(d, ss);
    };
    if constexpr (FUSED) {
        // the activation row of the first pass first (every wave's before any
        // wave's weight loads, as in the dot4 kernel: measured Gemma-like
        // M = 8 5.67 -> 4.89 us), then the weights of the first D steps
        const auto rx = make_rsrc(a.X, M * K * 4);
        const int G8 = K / 8;
        float4 va[G], vb[G];
        auto xload = [&](int m) {
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const int g = lane + 64 * i;
                const int off = (m < M && g < G8) ? (m * K + 8 * g) * 4 : kOOB;
                va[i] = bloadf4(rx, off);
                vb[i] = bloadf4(rx, off == kOOB ? kOOB : off + 16);
            }
        };
        xload(wave);
        __builtin_amdgcn_sched_barrier(0);
        issue_barrier();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < D; ++d)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int h = 0; h < WL; ++h)
                    wr[d][nb][h] = wload(rb, s0 + d < s1 ? boff[nb] + wstep * (s0 + d) + hstep * h : kOOB);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int pass = 0; pass < (FUSED ? 16 / W : 1); ++pass) {
            const int m = wave + W * pass;
            if (m < M) {  // wave-uniform
                if (pass == 1) xload(m);  // rows 8 .. 15
                float am = 0.0f;
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    am = fmaxf(am, fmaxf(fmaxf(fabsf(va[i].x), fabsf(va[i].y)),
                                         fmaxf(fabsf(va[i].z), fabsf(va[i].w))));
                    am = fmaxf(am, fmaxf(fmaxf(fabsf(vb[i].x), fabsf(vb[i].y)),
                                         fmaxf(fabsf(vb[i].z), fabsf(vb[i].w))));
                }
                am = wave_max_nonneg(am);
                const float sx = (am == 0.0f) ? 0.0f : div127(am);
                // the codes of an 8-group in P8 order (natural order for 8-bit
                // weights); `code` returns a word whose low byte is the int8 code
                auto put8 = [&](int g, const float4 &v0, const float4 &v1, auto code) {
                    uint2 pq;
                    if (W8) {
                        pq.x = pack4_i8(code(v0.x), code(v0.y), code(v0.z), code(v0.w));
                        pq.y = pack4_i8(code(v1.x), code(v1.y), code(v1.z), code(v1.w));
                    } else {  // P8: [x0 x2 x4 x6 | x1 x3 x5 x7]
                        pq.x = pack4_i8(code(v0.x), code(v0.z), code(v1.x), code(v1.z));
                        pq.y = pack4_i8(code(v0.y), code(v0.w), code(v1.y), code(v1.w));
                    }
                    *reinterpret_cast<uint2 *>(xs + (g / 2) * 256 + m * 16 + (g % 2) * 8) = pq;
                };
                if (sx >= kFastQuotientMinScale) {  // row-uniform
                    // correctly rounded quotient without a division, rounded by
                    // one add (|v / s| <= 127.5 for every value of the row)
                    const float rs = 1.0f / sx;
                    auto code = [&](float v) { return (int)code_in_low_byte(quotient_rn(v, sx, rs)); };
#pragma unroll
                    for (int i = 0; i < G; ++i) {
                        const int g = lane + 64 * i;
                        if (g < G8) put8(g, va[i], vb[i], code);
                    }
                } else {  // zero or tiny scale
                    const RowScale q = row_scale(sx);
                    auto code = [&](float v) { return quant_code_row(v, q); };
#pragma unroll
                    for (int i = 0; i < G; ++i) {
                        const int g = lane + 64 * i;
                        if (g < G8) put8(g, va[i], vb[i], code);
                    }
                }
                if (lane == 0) sxs[m] = sx;
            } else {
                for (int g = lane; g < G8; g += 64)
                    *reinterpret_cast<uint2 *>(xs + (g / 2) * 256 + m * 16 + (g % 2) * 8) = uint2{0, 0};
                if (lane == 0) sxs[m] = 0.0f;
            }
        }
        lds_barrier();  // codes, row scales and the zeroed partial sums (weight loads stay in flight)
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int ss = s0 + d;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int o = xso + xsstep * min(ss, SU - 1);
                xr0[d][mb] = *reinterpret_cast<const uint4 *>(xs + o);
                xr1[d][mb] = *reinterpret_cast<const uint4 *>(xs + o + 256);
                if (LP) {
                    xr2[d][mb] = *reinterpret_cast<const uint4 *>(xs + o + 512);
                    xr3[d][mb] = *reinterpret_cast<const uint4 *>(xs + o + 768);
                }
            }
        }
    } else {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            fetch(d, s0 + d);
            __builtin_amdgcn_sched_barrier(0);  // slot 0 oldest, as in the loop below
        }
    }

    // Epilogue operands of the output blocks this wave stores, loaded early:
    // channel scale and bias of this lane's column, row scales of its 4 rows.
    float swc[kPerWave], bc[kPerWave], sxr[kPerWave][4];
    if (OUT == Out::Y) {
#pragma unroll
        for (int j = 0; j < kPerWave; ++j) {
            const int p = wave + j * W;
            const int mb = min(p, kPairs - 1) / NB, nb = min(p, kPairs - 1) % NB;
            const int64_t col = min(n0 + 16 * nb + r16, N - 1);
            swc[j] = a.sw[col];
            bc[j] = a.bias ? a.bias[col] : 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sxr[j][i] = FUSED ? sxs[4 * kq + i]
                                  : a.sx[min((int64_t)(16 * mb + 4 * kq + i), M - 1)];
        }
    }

    // Each ring slot keeps its registers: its data is consumed (unpacked /
    // fed to the MFMAs) before the slot is refilled with the step D ahead.
    // The body has no per-step branch: steps past s1 hold zeros (out-of-range
    // loads) and add nothing, which keeps the vmcnt bookkeeping exact.
    for (int s = s0; s < s1; s += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if constexpr (LP) {
                // lanes r < 8 keep piece 2 kq of load 0 and take the partner's
                // (piece 2 kq + 1 of the same channel); lanes r >= 8 keep piece
                // 2 kq + 1 of load 1 and take the partner's piece 2 kq.  The
                // first half's MFMAs (piece 2 kq) run before the second half's
                // activations are waited for; fused, the next unit's weights and
                // first half are requested in between.
                uint4 e[NB], o[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    e[nb] = wr[d][nb][0];
                    o[nb] = wr[d][nb][1];
                    swap_halves8(e[nb], o[nb]);
                }
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const uint4 x0 = xr0[d][mb], x1 = xr1[d][mb];
                    const v4i a0 = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w};
                    const v4i a1 = {(int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const uint4 w = e[nb];
                        const v4i b0 = {(int)lo16(w.x), (int)hi16(w.x), (int)lo16(w.y), (int)hi16(w.y)};
                        const v4i b1 = {(int)lo16(w.z), (int)hi16(w.z), (int)lo16(w.w), (int)hi16(w.w)};
                        acc[mb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, acc[mb][nb], 0, 0, 0);
                        acc[mb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, acc[mb][nb], 0, 0, 0);
                    }
                }
                if constexpr (FUSED) {
                    fetch_wa(d, s + d + D);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const uint4 x2 = xr2[d][mb], x3 = xr3[d][mb];
                    const v4i a2 = {(int)x2.x, (int)x2.y, (int)x2.z, (int)x2.w};
                    const v4i a3 = {(int)x3.x, (int)x3.y, (int)x3.z, (int)x3.w};
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const uint4 w = o[nb];
                        const v4i b2 = {(int)lo16(w.x), (int)hi16(w.x), (int)lo16(w.y), (int)hi16(w.y)};
                        const v4i b3 = {(int)lo16(w.z), (int)hi16(w.z), (int)lo16(w.w), (int)hi16(w.w)};
                        acc[mb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, b2, acc[mb][nb], 0, 0, 0);
                        acc[mb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a3, b3, acc[mb][nb], 0, 0, 0);
                    }
                }
                if constexpr (FUSED)
                    fetch_b(d, s + d + D);
                else
                    fetch(d, s + d + D);
                __builtin_amdgcn_sched_barrier(0);
            } else {
                v4i b0[NB], b1[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    if (W8) {
                        uint4 w0 = wr[d][nb][0], w1 = wr[d][nb][WL - 1];
                        if (LN) swap_halves8(w0, w1);
                        b0[nb] = v4i{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w};
                        b1[nb] = v4i{(int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
                    } else {
                        const uint4 w = wr[d][nb][0];
                        b0[nb] = v4i{(int)lo16(w.x), (int)hi16(w.x), (int)lo16(w.y), (int)hi16(w.y)};
                        b1[nb] = v4i{(int)lo16(w.z), (int)hi16(w.z), (int)lo16(w.w), (int)hi16(w.w)};
                    }
                }
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const uint4 x0 = xr0[d][mb], x1 = xr1[d][mb];
                    const v4i a0 = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w};
                    const v4i a1 = {(int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        acc[mb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0[nb], acc[mb][nb], 0, 0, 0);
                        acc[mb][nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1[nb], acc[mb][nb], 0, 0, 0);
                    }
                }
                fetch(d, s + d + D);
                // keep the refill of this slot ahead of the next slot's math
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) atomicAdd(&red[((mb * NB + nb) * 4 + i) * kWave + lane], acc[mb][nb][i]);
    __syncthreads();

#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
        const int p = wave + j * W;
        if (p >= kPairs) break;
        const int mb = p / NB, nb = p % NB;
        const int64_t col = n0 + 16 * nb + r16;
        if (col >= N) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t row = 16 * mb + 4 * kq + i;
            if (row >= M) continue;
            const int v = W8 ? red[(p * 4 + i) * kWave + lane] : (red[(p * 4 + i) * kWave + lane] >> 4);
            if (OUT == Out::I32) {
                a.acc[row * N + col] = v;
            } else {
                const float sc = sxr[j][i] * swc[j];
                float y = (float)v * sc;
                if (a.bias) y = y + bc[j];
                y = relu_if(y, a.relu);
                a.Y[row * N + col] = y;
            }
        }
    }
}

template <int MB, int NB, int D, int W, bool W8>
static void go_mfma(const W4A8Args &a, hipStream_t st) {
    dim3 grid((unsigned)((a.N + 16 * NB - 1) / (16 * NB)));
    if constexpr (!W8) {
        if (a.pp) {
            launch_main(k_gemv_mfma<MB, NB, D, W, Out::Y, false, true>, grid, dim3(64 * W), 0, st,
                        a);
            return;
        }
    }
    // whole-line loads: int8 codes always, int4 codes up to two row blocks
    if constexpr (W8 || MB <= 2) {
        if (W8 || a.K % 256 == 0) {
            if (a.out == Out::I32)
                launch_main(k_gemv_mfma<MB, NB, D, W, Out::I32, W8, false, 0, true>, grid,
                            dim3(64 * W), 0, st, a);
            else
                launch_main(k_gemv_mfma<MB, NB, D, W, Out::Y, W8, false, 0, true>, grid,
                            dim3(64 * W), 0, st, a);
            return;
        }
    }
    if (a.out == Out::I32)
        launch_main(k_gemv_mfma<MB, NB, D, W, Out::I32, W8>, grid, dim3(64 * W), 0, st, a);
    else
        launch_main(k_gemv_mfma<MB, NB, D, W, Out::Y, W8>, grid, dim3(64 * W), 0, st, a);
}

// Launch shape (measured on the 7B-class 4096 x 11008 and the Gemma-like
// 1152 x 6912 layers, M = 8 ... 64): 8 waves, one step in flight per slot
// (D = 1), and the most channel blocks per workgroup (NB <= 4) that still give
// at least 3/4 of the chip's CUs a workgroup.  Every workgroup reads the M x K
// activation codes of its K range, so fewer, wider workgroups read fewer
// bytes, but a layer with few output channels must not leave CUs idle: the
// 7B-class layer takes NB = 3 (230 workgroups; 9.8 -> 8.2 us at M = 16 against
// NB = 4, 172 workgroups), the Gemma-like layer NB = 2 (216; 5.0 -> 3.8 us at
// M = 8).
// CU count per device, cached (atomics: launches may come from several host
// threads; every writer stores the same value)
static int device_cus() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

static int mfma_channel_blocks(int64_t N) {
    const int64_t want = (3 * (int64_t)device_cus()) / 4;
    for (int nb = 4; nb > 1; --nb)
        if ((N + 16 * nb - 1) / (16 * nb) >= want) return nb;
    return 1;
}

template <int MB, bool W8>
static void go_mfma_nb(const W4A8Args &a, hipStream_t st) {
    switch (mfma_channel_blocks(a.N)) {
        case 1: go_mfma<MB, 1, 1, 8, W8>(a, st); break;
        case 2: go_mfma<MB, 2, 1, 8, W8>(a, st); break;
        case 3: go_mfma<MB, 3, 1, 8, W8>(a, st); break;
        default: go_mfma<MB, 4, 1, 8, W8>(a, st); break;
    }
}

template <bool W8>
static void go_mfma_w(const W4A8Args &a, hipStream_t st) {
    const int mb = (int)((a.M + 15) / 16);
    switch (mb) {
        case 1: go_mfma_nb<1, W8>(a, st); break;
        case 2: go_mfma_nb<2, W8>(a, st); break;
        case 3: go_mfma_nb<3, W8>(a, st); break;
        default: go_mfma_nb<4, W8>(a, st); break;
    }
}

// Fused activation quantization (G > 0): worth it while the per-workgroup
// quantization stays small.  With 8 waves each wave quantizes ceil(M / 8)
// rows of K values before its first MFMA; measured against quantizer + GEMV
// (two launches), with the activation loads ahead of the weights and the
// division-free chain, that is faster up to ceil(M / 8) * K = 4096 (7B-class
// M = 8, K = 4096: 11.0 -> 9.85 us) and slower beyond (M = 16, K = 4096:
// 11.1 -> 12.0 us).  The canonical int4 layout takes 16 waves from 8 or 9
// rows on (below), one row per wave, and then every M <= 16 with K <= 4096
// is faster fused (7B-class M = 10, 12, 16: 10.3 -> 9.5, 10.35 -> 9.7,
// 10.65 -> 10.35 us); int8 weights and shuffled tiles keep the bound (fused
// with 16 waves, 7B-class M = 16: int8 13.4-14.0 against 12.95 us for the
// two launches, shuffled 9.85 against 9.65 us).  Rows of up to 2048 k fit in 32 KB of
// LDS (G = 4), up to 4096 k in 64 KB (G = 8).
bool gemv_mfma_fused_ok(int64_t M, int64_t K, bool w8, bool pp) {
    if (!(M >= 1 && M <= 16 && K % 128 == 0 && K <= 4096)) return false;
    return (!w8 && !pp) || ((M + 7) / 8) * K <= 4096;
}

// Two units in flight per wave (D = 2) in the fused kernel: a wave's slice of
// a K <= 4096 layer is a few units, so with D = 2 most of its weights are
// requested before the prologue's quantization.  Measured (graph-replayed,
// rotating weights, us): shuffled tiles 7B-class M = 4 8.65 -> 8.0, M = 8
// 9.3 -> 8.7; whole-line loads M = 4 8.75 -> 8.5, M = 8 even; int8 weights
// Gemma-like M = 4 5.42 -> 5.05, M = 16 7.0 -> 6.67, 7B-class M = 4
// 12.6 -> 12.35; but the half-line int4 loads (K % 256 = 128) Gemma-like
// M = 4, 8, 16 4.5 -> 4.65, 4.7 -> 4.95, 5.7 -> 6.0, so those keep D = 1.
// (In the non-fused kernel D = 2 was slower on every path: 7B-class M = 16
// 10.45 -> 11.46, shuffled 9.8 -> 10.1, int8 14.6 -> 15.3.)
template <int NB, bool W8, int G>
static void go_mfma_fused_g(const W4A8Args &a, hipStream_t st) {
    dim3 grid((unsigned)((a.N + 16 * NB - 1) / (16 * NB)));
    if constexpr (!W8) {
        if (a.pp) {
            launch_main(k_gemv_mfma<1, NB, 2, 8, Out::Y, false, true, G>, grid, dim3(512), 0, st, a);
            return;
        }
        // 16 waves, one activation row each (and twice the waves to spread a
        // short K over), from 8 rows on with whole-line loads and from 9 rows
        // on with half-line loads (graph-replayed, us: 7B-class M = 8
        // 9.48 -> 9.15, Gemma-like M = 12 5.35 -> 5.12, M = 16 5.72 -> 5.38;
        // at M = 4 and Gemma-like M = 8 they were slower: 8.5 -> 9.0,
        // 4.64 -> 4.80)
        if (a.K % 256 == 0) {  // whole-line loads (int4 codes only)
            if (a.M >= 8)
                launch_main(k_gemv_mfma<1, NB, 1, 16, Out::Y, false, false, G, true>, grid,
                            dim3(1024), 0, st, a);
            else
                launch_main(k_gemv_mfma<1, NB, 2, 8, Out::Y, false, false, G, true>, grid,
                            dim3(512), 0, st, a);
            return;
        }
        if (a.M > 8) {
            launch_main(k_gemv_mfma<1, NB, 1, 16, Out::Y, false, false, G>, grid, dim3(1024), 0, st, a);
            return;
        }
    }
    if constexpr (W8) {
        // whole-line loads (non-temporal: 7B-class M = 4 12.6 -> 11.6 us,
        // Gemma-like M = 8 5.29 -> 4.97 us); 16 waves above 8 rows
        // (Gemma-like M = 12 6.08 -> 5.33 us, M = 16 6.47 -> 5.37 us)
        if (a.M > 8)
            launch_main(k_gemv_mfma<1, NB, 1, 16, Out::Y, true, false, G, true>, grid, dim3(1024),
                        0, st, a);
        else
            launch_main(k_gemv_mfma<1, NB, 2, 8, Out::Y, true, false, G, true>, grid, dim3(512), 0,
                        st, a);
        return;
    }
    launch_main(k_gemv_mfma<1, NB, 1, 8, Out::Y, false, false, G>, grid, dim3(512), 0, st, a);
}

template <int NB, bool W8>
static void go_mfma_fused(const W4A8Args &a, hipStream_t st) {
    if (a.K <= 2048)
        go_mfma_fused_g<NB, W8, 4>(a, st);  // K <= 512 G
    else
        go_mfma_fused_g<NB, W8, 8>(a, st);
}

template <bool W8>
static void go_mfma_fused_w(const W4A8Args &a, hipStream_t st) {
    switch (mfma_channel_blocks(a.N)) {
        case 1: go_mfma_fused<1, W8>(a, st); break;
        case 2: go_mfma_fused<2, W8>(a, st); break;
        case 3: go_mfma_fused<3, W8>(a, st); break;
        default: go_mfma_fused<4, W8>(a, st); break;
    }
}

hipError_t launch_gemv_mfma_fused(const W4A8Args &a, hipStream_t st) {
    if (a.w8)
        go_mfma_fused_w<true>(a, st);
    else
        go_mfma_fused_w<false>(a, st);
    return hipGetLastError();
}

hipError_t launch_gemv_mfma(const W4A8Args &a, hipStream_t st) {
    if (a.w8)
        go_mfma_w<true>(a, st);
    else
        go_mfma_w<false>(a, st);
    return hipGetLastError();
}

}  // namespace w4
