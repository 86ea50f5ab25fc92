// Device helpers shared by the gfx950 kernels of the W4A8 / W4A16 linear layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace w4 {

constexpr int kWave = 64;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ buffer loads
// Raw buffer loads: the descriptor carries the byte range, and a load whose
// offset lies outside it returns zeros without touching memory.  This gives
// branch-free predication (no exec-mask branches between loads, so the loads
// of a lane issue back to back).
constexpr int kBufFlags = 0x00020000;  // gfx9 raw-buffer descriptor word 3
constexpr int kMaxRange = 0x7F000000;  // descriptor ranges are capped here
constexpr int kOOB = 0x7FFF0000;       // an offset beyond every range (plus room for +16 .. +48)
constexpr int kNonTemporal = 2;       // cache-policy operand of the buffer builtins: nt

// Callers keep every in-range offset below kMaxRange (the kernels rebase the
// descriptor on the rows a block touches).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const int n = bytes > kMaxRange ? kMaxRange : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, kBufFlags);
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Streaming 16-byte load (non-temporal hint): for data a kernel reads exactly
// once, the packed weights of the decode GEMVs, so that the stream does not
// displace cache lines that are reused.
__device__ __forceinline__ uint4 bload16_nt(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal));
}

__device__ __forceinline__ uint2 bload8(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

__device__ __forceinline__ float4 bloadf4(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ float bloadf(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// ------------------------------------------------------------ DPP reductions
// Cross-lane moves inside a row of 16 lanes (no LDS traffic).
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int kRowRor8 = 0x128;      // row_ror:8 (lane r of a row <- lane r ^ 8)

// Lanes r and r ^ 8 of each row of 16 exchange one word: lanes r < 8 keep e
// and take the partner's e as o, lanes r >= 8 keep o and take the partner's o
// as e (two DPP moves, each writing one half of the row's lanes).
__device__ __forceinline__ void swap_halves8(uint32_t &e, uint32_t &o) {
    const int e0 = (int)e, o0 = (int)o;
    e = (uint32_t)__builtin_amdgcn_update_dpp(e0, o0, kRowRor8, 0xF, 0xC, false);
    o = (uint32_t)__builtin_amdgcn_update_dpp(o0, e0, kRowRor8, 0xF, 0x3, false);
}
__device__ __forceinline__ void swap_halves8(uint4 &e, uint4 &o) {
    swap_halves8(e.x, o.x);
    swap_halves8(e.y, o.y);
    swap_halves8(e.z, o.z);
    swap_halves8(e.w, o.w);
}

// Sum over each row of 16 lanes; every lane of the row gets the sum.
__device__ __forceinline__ int sum16(int v) {
    v += dpp<kQuadSwap1>(v);
    v += dpp<kQuadSwap2>(v);
    v += dpp<kRowHalfMirror>(v);
    v += dpp<kRowMirror>(v);
    return v;
}

__device__ __forceinline__ float fdpp_max(float v, int which) {
    int b = __builtin_bit_cast(int, v), o;
    switch (which) {
        case 0: o = dpp<kQuadSwap1>(b); break;
        case 1: o = dpp<kQuadSwap2>(b); break;
        case 2: o = dpp<kRowHalfMirror>(b); break;
        default: o = dpp<kRowMirror>(b); break;
    }
    return fmaxf(v, __builtin_bit_cast(float, o));
}

// Max over the 64 lanes of a wave (inputs >= 0 or any finite values); the
// result is wave-uniform.
__device__ __forceinline__ float wave_max_dpp(float v) {
    v = fdpp_max(v, 0);
    v = fdpp_max(v, 1);
    v = fdpp_max(v, 2);
    v = fdpp_max(v, 3);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Max over the 64 lanes of a wave of values >= 0 (no NaN), through their bit
// patterns: for non-negative floats the unsigned order of the bits is the
// float order, so each step is one integer max of a DPP-moved operand (no
// canonicalizing float max).  The result is wave-uniform.
__device__ __forceinline__ float wave_max_nonneg(float v) {
    uint32_t b = __float_as_uint(v);
    b = max(b, (uint32_t)dpp<kQuadSwap1>((int)b));
    b = max(b, (uint32_t)dpp<kQuadSwap2>((int)b));
    b = max(b, (uint32_t)dpp<kRowHalfMirror>((int)b));
    b = max(b, (uint32_t)dpp<kRowMirror>((int)b));
    const uint32_t r0 = __builtin_amdgcn_readlane((int)b, 0);
    const uint32_t r1 = __builtin_amdgcn_readlane((int)b, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane((int)b, 32);
    const uint32_t r3 = __builtin_amdgcn_readlane((int)b, 48);
    return __uint_as_float(max(max(r0, r1), max(r2, r3)));
}

// ------------------------------------------------- direct buffer->LDS loads
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
// outputs; the LDS address is an input bound to M0, so the compiler writes M0
// itself and knows that it holds this value.  On gfx9 an LDS direct load needs
// one wait state after an SALU write of M0, hence the nop.
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t lds_base, int voff, int soff) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_base)
                 : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)p));
}

// ----------------------------------------------------------------- barrier
// Workgroup barrier that waits only for this wave's LDS operations: vector
// memory loads issued before it stay in flight (the compiler still waits for
// each loaded register before its first use).  __syncthreads would instead
// drain every outstanding load at the barrier.  The "memory" clobber keeps
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Workgroup barrier that waits for no memory operation: orders the issue of
// the loads before it (in every wave) ahead of the loads after it.
__device__ __forceinline__ void issue_barrier() { asm volatile("s_barrier" ::: "memory"); }

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Max of values >= 0 over a block of kWaves waves; `red` is LDS with one
// float per wave.  Every thread gets the result.  (The wave count is a
// compile-time constant so that no launch argument is read after the barrier.)
template <int kWaves>
__device__ __forceinline__ float block_max(float v, float *red) {
    v = wave_max_dpp(v);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x % kWave) == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) r = fmaxf(r, red[i]);
    __syncthreads();
    return r;
}

// ------------------------------------------------------------- quantization
// round-half-to-even of a correctly rounded fp32 quotient, limited to [lo, hi];
// a zero scale gives code 0.
__device__ __forceinline__ int quant_code(float v, float s, float lo, float hi) {
    if (s == 0.0f) return 0;
    float t = v / s;  // IEEE division (no fast-math in this build)
    float r = rintf(t);
    r = fminf(fmaxf(r, lo), hi);
    return (int)r;
}

// The correctly rounded quotient fl(v / s) without a division: with
// rs = fl(1 / s), q = fl(v * rs) lies within one ulp of v / s, the residual
// v - s*q is exact in one fma and fl(q + residual * rs) is the correctly
// rounded quotient (Markstein's theorem for round-to-nearest; it needs the
// operands away from the subnormal range, hence kFastQuotientMinScale).
constexpr float kFastQuotientMinScale = 0x1p-64f;

__device__ __forceinline__ float quotient_rn(float v, float s, float rs) {
    const float q = v * rs;
    const float r = __builtin_fmaf(-q, s, v);
    return __builtin_fmaf(r, rs, q);
}

// quant_code for a scale s >= kFastQuotientMinScale, with rs = fl(1 / s).
__device__ __forceinline__ int quant_code_fast(float v, float s, float rs, float lo, float hi) {
    float r = rintf(quotient_rn(v, s, rs));
    r = fminf(fmaxf(r, lo), hi);
    return (int)r;
}

// fl(a / 127) for a >= 0 without a division where it is safe: with
// y = fl(1/127), q = fl(a y), r = fma(-q, 127, a) is exact and fma(r, y, q)
// is the correctly rounded quotient (Markstein's theorem; checked for every
// float a in [2^-100, 2^128)).  Smaller a take the IEEE division.
__device__ __forceinline__ float div127(float a) {
    constexpr float y = 1.0f / 127.0f;
    if (a >= 0x1p-100f) {
        const float q = a * y;
        const float r = __builtin_fmaf(-q, 127.0f, a);
        return __builtin_fmaf(r, y, q);
    }
    return a / 127.0f;
}

// Round-half-to-even of t (|t| <= 127.5) to an int8 code in the low byte of
// the result: t + 1.5 * 2^23 lies in [2^23, 2^24), where fp32 values are the
// integers, so the add rounds t to the nearest integer, ties to even; the bit
// pattern of 1.5 * 2^23 ends in a zero byte, so the sum's low byte is that
// integer modulo 256 (checked for every float t with |t| <= 127.5).  The
// quotient of a value of a row by the row's absmax scale never leaves that
// range, so the clamp to [-128, 127] never binds and is not needed.
__device__ __forceinline__ uint32_t code_in_low_byte(float t) {
    return __float_as_uint(t + 12582912.0f);
}

// An activation row's scale, prepared for quant_code_row.  A scale below
// kFastQuotientMinScale is multiplied by 2^100 and so is every value of its row
// (both exact: the scale stays below 2^36 and |x| <= 127.5 s below 2^-57), which
// keeps the real quotient x / s and brings the scale into the range of the
// division-free quotient; a zero scale (all-zero row) gets rs = 0, so every
// code is 0.  One code path for every scale, no per-value division.
struct RowScale {
    float pre, s, rs;
};

__device__ __forceinline__ RowScale row_scale(float s) {
    const float pre = (s < kFastQuotientMinScale) ? 0x1p100f : 1.0f;
    const float ss = s * pre;
    return RowScale{pre, ss, (ss == 0.0f) ? 0.0f : 1.0f / ss};
}

// clamp(rne(fl(v / s)), -128, 127) for the row scale s behind `q`.
__device__ __forceinline__ int quant_code_row(float v, const RowScale &q) {
    return quant_code_fast(v * q.pre, q.s, q.rs, -128.0f, 127.0f);
}

// ------------------------------------------------------------------ unpack
// A packed dword holds 8 signed nibbles for k = 0..7 of a group of 8 (byte i:
// k = 2i low nibble, k = 2i+1 high nibble).  Moving each nibble to the top of
// its byte yields int8 lanes equal to 16*code exactly (two's complement), so
// products can run on int8 hardware and the sum is divided by 16 at the end.
//   lo16: bytes = 16*code for k = 0, 2, 4, 6
//   hi16: bytes = 16*code for k = 1, 3, 5, 7
__device__ __forceinline__ uint32_t lo16(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t hi16(uint32_t w) { return w & 0xF0F0F0F0u; }

// The "P8" activation layout pairs with lo16/hi16: inside every group of 8
// consecutive k the int8 values are stored as [x0 x2 x4 x6 | x1 x3 x5 x7], so
// the even and odd halves line up with lo16 and hi16 of the weight dword.
__device__ __forceinline__ void natural_to_p8(uint32_t lo, uint32_t hi, uint32_t &ev,
                                              uint32_t &od) {
    ev = (lo & 0xFFu) | ((lo >> 8) & 0xFF00u) | ((hi & 0xFFu) << 16) | ((hi << 8) & 0xFF000000u);
    od = ((lo >> 8) & 0xFFu) | ((lo >> 16) & 0xFF00u) | ((hi << 8) & 0xFF0000u) | (hi & 0xFF000000u);
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
           ((uint32_t)(d & 0xFF) << 24);
}

// ---------------------------------------------------------------- epilogue
// Dequantize one int32 accumulator: fl(fl(float(acc)) * fl(sx * sw)) then
// + bias, each step rounded separately (this library is built without
// floating-point contraction).
__device__ __forceinline__ float dequant(int acc, float sx, float sw, const float *bias, int n) {
    float s = sx * sw;
    float y = (float)acc * s;
    if (bias) y = y + bias[n];
    return y;
}

// The Dense layer's ReLU after the bias (Keras guide, toy model): y > 0 ? y : +0
// (a select, not a max, so -0 becomes +0).
__device__ __forceinline__ float relu_if(float y, bool relu) {
    return (relu && !(y > 0.0f)) ? 0.0f : y;
}

// Map a linear block index to a tile index so that the blocks the hardware
// places on one XCD (consecutive ids go round-robin over the 8 XCDs) get a
// contiguous range of tiles and share that XCD's L2.
__device__ __forceinline__ int xcd_swizzle(int bid, int nblocks) {
    constexpr int kXcd = 8;
    if (nblocks % kXcd != 0) return bid;
    const int per = nblocks / kXcd;
    return (bid % kXcd) * per + bid / kXcd;
}

// Kernel arguments are read from memory by scalar loads that the compiler
// places where a value is first used; an argument first used late (an output
// pointer, an epilogue flag) then costs a memory round trip at that point.
// Passing an argument through arg_now at kernel entry puts its load in the
// kernel's first batch of argument loads.
template <typename T>
__device__ __forceinline__ T arg_now(T v) {
    static_assert(sizeof(T) <= 8, "scalar kernel arguments only");
    if constexpr (sizeof(T) == 8) {
        uint64_t u;
        __builtin_memcpy(&u, &v, 8);
        asm volatile("" : "+s"(u));
        __builtin_memcpy(&v, &u, 8);
    } else {
        uint32_t u = 0;
        __builtin_memcpy(&u, &v, sizeof(T));
        asm volatile("" : "+s"(u));
        __builtin_memcpy(&v, &u, sizeof(T));
    }
    return v;
}

// Pointer arguments keep their global address space through the asm (a plain
// integer round trip would turn their loads and stores into flat ones, which
// also count against the LDS wait counter).
template <typename T>
__device__ __forceinline__ T *arg_now(T *p) {
    using GlobalPtr = __attribute__((address_space(1))) T *;
    uint64_t u = (uint64_t)(GlobalPtr)p;
    asm volatile("" : "+s"(u));
    return (T *)(GlobalPtr)u;
}

template <typename... T>
__device__ __forceinline__ void args_now(T &...v) {
    ((v = arg_now(v)), ...);
}

// Every field of the product kernels' argument block, loaded at entry.
__device__ __forceinline__ W4A8Args args_now(W4A8Args a) {
    args_now(a.X, a.Xq, a.sx, a.packed, a.sw, a.bias, a.Y, a.acc, a.M, a.K, a.N, a.out, a.w8,
             a.relu, a.act_div, a.pp);
    return a;
}

}  // namespace w4
