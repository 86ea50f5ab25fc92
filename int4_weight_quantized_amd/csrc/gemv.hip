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
// chunk = 32 codes), so a wave reads 4 rows x 256 contiguous bytes per load
// and every weight byte of the block is requested before any arithmetic.
// Order of work: (1) issue the activation loads, (2) issue the weight chunks,
// (3) quantize the activations into LDS (P8 layout) while the weights are in
// flight (the barriers wait for LDS only, so the weight loads stay in
// flight), (4) dot products, chunk by chunk as the loads land, (5) 16-lane
// DPP sum and epilogue.
// With W8 a 16-byte chunk holds 16 int8 codes (instead of 32 int4 codes) and
// the activations stay in natural order.
constexpr int kDot4MaxK = 8192, kDot4MaxKW8 = 4096;

bool gemv_dot4_ok(int64_t M, int64_t K, bool w8) {
    return M >= 1 && M <= 4 && K % 32 == 0 && K <= (w8 ? kDot4MaxKW8 : kDot4MaxK);
}

// DIV (with FUSED): the activations are divided by per-column divisors
// (a.act_div) before their quantization -- the activation side of AWQ-style
// channel scaling.
// PP: the int4 codes come in the shuffled tile layout (ROWS == 16, K % 128 ==
// 0): chunk c of block row r sits in tile c / 4 at slot (c % 4) ^ ((r / 2) % 4),
// so the 4 rows of a wave still read 256 contiguous bytes per tile.
template <int M, int ROWS, int UB, bool FUSED, Out OUT, bool W8, bool DIV = false,
          bool PP = false>
__global__ __launch_bounds__(16 * ROWS) void k_gemv_dot4(W4A8Args args) {
    const W4A8Args a = args_now(args);
    constexpr int T = 16 * ROWS;  // threads
    constexpr int KPC = W8 ? 16 : 32;  // codes per 16-byte chunk
    // 8-groups of k per thread (K <= 16 * KPC * UB)
    constexpr int NG = (2 * KPC * UB / 16 + ROWS - 1) / ROWS;
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ float red[T / kWave][M];
    int8_t *xs = reinterpret_cast<int8_t *>(smem);
    const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
    const int K = (int)a.K, KB = W8 ? K : K / 2, C = K / KPC, G8 = K / 8;
    const int j = t & 15, r = t >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * ROWS;
    const int rows = (int)min((int64_t)ROWS, a.N - n0);

    // (1) activations: group g = t + T*i holds k = 8g .. 8g+7 of each row.
    float4 xa[M][NG], xb[M][NG];
    float4 da[DIV ? NG : 1], db[DIV ? NG : 1];
    uint2 xn[M][NG];
    if (FUSED) {
        const auto rx = make_rsrc(a.X, (int64_t)M * K * 4);
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                const int g = t + T * i;
                const int off = g < G8 ? (m * K + 8 * g) * 4 : kOOB;
                xa[m][i] = bloadf4(rx, off);
                xb[m][i] = bloadf4(rx, off + 16);
            }
        if (DIV) {
            // divisors of the thread's 8-groups (out-of-range groups read 0
            // and are replaced by 1 where they are used)
            const auto rd = make_rsrc(a.act_div, (int64_t)K * 4);
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                const int g = t + T * i;
                da[i] = bloadf4(rd, g < G8 ? 32 * g : kOOB);
                db[i] = bloadf4(rd, g < G8 ? 32 * g + 16 : kOOB);
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

    // (2) weights of this block's rows: all UB chunks of the lane.
    static_assert(!PP || (ROWS == 16 && !W8), "shuffled int4 tiles of 16 channels");
    const auto rw = PP ? make_rsrc(a.packed + (n0 / 16) * (int64_t)(K / 128) * 1024,
                                   (int64_t)(K / 128) * 1024)
                       : make_rsrc(a.packed + n0 * KB, (int64_t)rows * KB);
    const int rowoff = r * KB;
    uint4 wb[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
        const int c = j + 16 * u;
        const int off = PP ? ((c / 4) * 16 + r) * 64 + 16 * ((c % 4) ^ ((r / 2) % 4))
                           : rowoff + 16 * c;
        wb[u] = bload16_nt(rw, c < C ? off : kOOB);
    }

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
    if (FUSED && DIV) {
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            if (t + T * i >= G8) da[i] = db[i] = float4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
            for (int m = 0; m < M; ++m) {
                xa[m][i].x = xa[m][i].x / da[i].x;
                xa[m][i].y = xa[m][i].y / da[i].y;
                xa[m][i].z = xa[m][i].z / da[i].z;
                xa[m][i].w = xa[m][i].w / da[i].w;
                xb[m][i].x = xb[m][i].x / db[i].x;
                xb[m][i].y = xb[m][i].y / db[i].y;
                xb[m][i].z = xb[m][i].z / db[i].z;
                xb[m][i].w = xb[m][i].w / db[i].w;
            }
        }
    }
    if (FUSED) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float am = 0.0f;
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                am = fmaxf(am, fmaxf(fmaxf(fabsf(xa[m][i].x), fabsf(xa[m][i].y)),
                                     fmaxf(fabsf(xa[m][i].z), fabsf(xa[m][i].w))));
                am = fmaxf(am, fmaxf(fmaxf(fabsf(xb[m][i].x), fabsf(xb[m][i].y)),
                                     fmaxf(fabsf(xb[m][i].z), fabsf(xb[m][i].w))));
            }
            am = wave_max_dpp(am);
            if (lane == 0) red[wave][m] = am;
        }
        lds_barrier();
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float am = red[0][m];
#pragma unroll
            for (int w = 1; w < T / kWave; ++w) am = fmaxf(am, red[w][m]);
            const float s = (am == 0.0f) ? 0.0f : am / 127.0f;
            sxm[m] = s;
            // codes of the thread's 8-groups, stored P8: [x0 x2 x4 x6 | x1 x3 x5 x7]
            // (natural order for 8-bit weights)
            auto quantize = [&](auto code) {
#pragma unroll
                for (int i = 0; i < NG; ++i) {
                    const int g = t + T * i;
                    if (g < G8) {
                        const float4 v0 = xa[m][i], v1 = xb[m][i];
                        uint2 p;
                        if (W8) {
                            p.x = pack4_i8(code(v0.x), code(v0.y), code(v0.z), code(v0.w));
                            p.y = pack4_i8(code(v1.x), code(v1.y), code(v1.z), code(v1.w));
                        } else {
                            p.x = pack4_i8(code(v0.x), code(v0.z), code(v1.x), code(v1.z));
                            p.y = pack4_i8(code(v0.y), code(v0.w), code(v1.y), code(v1.w));
                        }
                        *reinterpret_cast<uint2 *>(xs + m * K + 8 * g) = p;
                    }
                }
            };
            if (s >= kFastQuotientMinScale) {  // row-uniform
                const float rs = 1.0f / s;
                quantize([&](float v) { return quant_code_fast(v, s, rs, -128.f, 127.f); });
            } else {
                quantize([&](float v) { return quant_code(v, s, -128.f, 127.f); });
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

template <int M, int ROWS, int UB, bool W8>
static void go_dot4(const W4A8Args &a, hipStream_t st) {
    dim3 grid((unsigned)((a.N + ROWS - 1) / ROWS));
    const uint32_t shm = (uint32_t)(M * a.K);
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
// rows w and w + 8, lane l the 8-groups l, l + 64, ... of the row, the row
// absmax is a wave reduction, and the codes and row scales go to LDS before
// one barrier (the first weight loads are already in flight).  The main loop
// then reads the activation fragments from LDS.
template <int MB, int NB, int D, int W, Out OUT, bool W8, bool PP = false, int G = 0>
__global__ __launch_bounds__(64 * W) void k_gemv_mfma(W4A8Args args) {
    const W4A8Args a = args_now(args);
    constexpr bool FUSED = G > 0;
    static_assert(!FUSED || (MB == 1 && W == 8 && OUT == Out::Y), "fused: 16 rows, 8 waves");
    __shared__ __align__(16) int8_t xs[FUSED ? 16 * 512 * G : 16];  // [K/16][16][16]
    __shared__ float sxs[16];
    constexpr int WL = W8 ? 2 : 1;  // 16-byte weight loads per lane and step
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
    const int s0 = S * wave / W, s1 = S * (wave + 1) / W;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * NB;
    const int cols = (int)min((int64_t)(16 * NB), N - n0);

    for (int t = threadIdx.x; t < kPairs * 4 * kWave; t += 64 * W) red[t] = 0;
    if (!FUSED) __syncthreads();  // (fused: the prologue's barrier covers it)

    static_assert(!PP || !W8, "shuffled layout of int4 codes");
    const auto rb = PP ? make_rsrc(a.packed + (n0 / 16) * (int64_t)S * 1024,
                                   (int64_t)((cols + 15) / 16) * S * 1024)
                       : make_rsrc(a.packed + n0 * KB, (int64_t)cols * KB);
    const auto ra = make_rsrc(a.Xq, M * K);
    int boff[NB], aoff[MB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        boff[nb] = PP ? nb * S * 1024 + r16 * 64 + 16 * (kq ^ ((r16 / 2) % 4))
                      : (16 * nb + r16) * KB + kq * 16 * WL;
    const int wstep = PP ? 1024 : 64 * WL;  // bytes per 128-k step
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) aoff[mb] = (2 * kq * (int)M + 16 * mb + r16) * 16;
    // activations are chunk-major, [K/16][M][16]: chunk c = 8 s + 2 kq + half
    const int achunk = (int)M * 16, astep = 8 * achunk;

    v4i acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = v4i{0, 0, 0, 0};

    uint4 wr[D][NB][WL], xr0[D][MB], xr1[D][MB];
    // Weight loads: a shuffled 1 KB tile is read whole by one load and never
    // again, so it streams (non-temporal); in the canonical layout a load
    // covers half of each 128-byte line (the next step or the second 16-byte
    // load reads the other half), so those lines must stay cached.
    auto wload = [&](const __amdgpu_buffer_rsrc_t &r, int off) {
        return PP ? bload16_nt(r, off) : bload16(r, off);
    };
    auto fetch = [&](int d, int ss) {
        const bool ok = ss < s1;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int h = 0; h < WL; ++h)
                wr[d][nb][h] = wload(rb, ok ? boff[nb] + wstep * ss + 16 * h : kOOB);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if (FUSED) {  // from LDS (16 rows per chunk); steps past s1 hold zero weights
                const int o = (2 * kq * 16 + r16) * 16 + 2048 * min(ss, S - 1);
                xr0[d][mb] = *reinterpret_cast<const uint4 *>(xs + o);
                xr1[d][mb] = *reinterpret_cast<const uint4 *>(xs + o + 256);
            } else {
                const int o = ok ? aoff[mb] + astep * ss : kOOB;
                xr0[d][mb] = bload16(ra, o);
                xr1[d][mb] = bload16(ra, ok ? o + achunk : kOOB);
            }
        }
    };
    if constexpr (FUSED) {
        // weights of the first steps first, then the activation rows
#pragma unroll
        for (int d = 0; d < D; ++d)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int h = 0; h < WL; ++h)
                    wr[d][nb][h] = wload(rb, s0 + d < s1 ? boff[nb] + wstep * (s0 + d) + 16 * h : kOOB);
        __builtin_amdgcn_sched_barrier(0);
        const auto rx = make_rsrc(a.X, M * K * 4);
        const int G8 = K / 8;
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int m = wave + 8 * pass;
            if (m < M) {  // wave-uniform
                float4 va[G], vb[G];
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    const int g = lane + 64 * i;
                    const int off = g < G8 ? (m * K + 8 * g) * 4 : kOOB;
                    va[i] = bloadf4(rx, off);
                    vb[i] = bloadf4(rx, off + 16);
                }
                float am = 0.0f;
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    am = fmaxf(am, fmaxf(fmaxf(fabsf(va[i].x), fabsf(va[i].y)),
                                         fmaxf(fabsf(va[i].z), fabsf(va[i].w))));
                    am = fmaxf(am, fmaxf(fmaxf(fabsf(vb[i].x), fabsf(vb[i].y)),
                                         fmaxf(fabsf(vb[i].z), fabsf(vb[i].w))));
                }
                am = wave_max_dpp(am);
                const float sx = (am == 0.0f) ? 0.0f : am / 127.0f;
                const RowScale q = row_scale(sx);
                auto code = [&](float v) { return quant_code_row(v, q); };
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    const int g = lane + 64 * i;
                    if (g < G8) {
                        const float4 v0 = va[i], v1 = vb[i];
                        uint2 pq;
                        if (W8) {
                            pq.x = pack4_i8(code(v0.x), code(v0.y), code(v0.z), code(v0.w));
                            pq.y = pack4_i8(code(v1.x), code(v1.y), code(v1.z), code(v1.w));
                        } else {  // P8: [x0 x2 x4 x6 | x1 x3 x5 x7]
                            pq.x = pack4_i8(code(v0.x), code(v0.z), code(v1.x), code(v1.z));
                            pq.y = pack4_i8(code(v0.y), code(v0.w), code(v1.y), code(v1.w));
                        }
                        *reinterpret_cast<uint2 *>(xs + (g / 2) * 256 + m * 16 + (g % 2) * 8) = pq;
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
                const int o = (2 * kq * 16 + r16) * 16 + 2048 * min(ss, S - 1);
                xr0[d][mb] = *reinterpret_cast<const uint4 *>(xs + o);
                xr1[d][mb] = *reinterpret_cast<const uint4 *>(xs + o + 256);
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
            {
                v4i b0[NB], b1[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    if (W8) {
                        const uint4 w0 = wr[d][nb][0], w1 = wr[d][nb][WL - 1];
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
// quantization stays small.  Each wave quantizes ceil(M / 8) rows of K values
// before its first MFMA; measured against quantizer + GEMV (two launches) the
// fused kernel is faster up to ceil(M / 8) * K = 3072 (M = 16, K = 1536) and
// slower from 4096 on (M = 8, K = 4096; M = 16, K = 2048).
bool gemv_mfma_fused_ok(int64_t M, int64_t K) {
    return M >= 1 && M <= 16 && K % 128 == 0 && K <= 2048 && ((M + 7) / 8) * K <= 3072;
}

template <int NB, bool W8>
static void go_mfma_fused(const W4A8Args &a, hipStream_t st) {
    constexpr int G = 4;  // K <= 512 G = 2048
    dim3 grid((unsigned)((a.N + 16 * NB - 1) / (16 * NB)));
    if constexpr (!W8) {
        if (a.pp) {
            launch_main(k_gemv_mfma<1, NB, 1, 8, Out::Y, false, true, G>, grid, dim3(512), 0, st, a);
            return;
        }
    }
    launch_main(k_gemv_mfma<1, NB, 1, 8, Out::Y, W8, false, G>, grid, dim3(512), 0, st, a);
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
