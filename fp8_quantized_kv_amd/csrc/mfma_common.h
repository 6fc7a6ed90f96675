// mfma_common.h -- device helpers shared by the matrix-core decode kernels of
// the 4-bit cache: LDS DMA issue and waits, the 4-bit code unpack into f16
// MFMA operands, and cross-lane reductions.
#pragma once

#include "internal.h"

#pragma clang diagnostic ignored "-Winline-asm"

namespace kvq {
namespace mx {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kTwo24 = 16777216.0f;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return uint32_t(uintptr_t((__attribute__((address_space(3))) const void*)(p)));
}

// 16 bytes per lane from global (SGPR base + VGPR offset) to LDS at
// m0 + 16 * lane.  Issued from asm so the compiler neither tracks nor
// serialises it; completion is awaited with wait_vmcnt.  base and lds must
// be wave-uniform; they are moved to SGPRs here.  STREAM marks the load
// non-temporal, for bytes that nothing reads again within the launch: a
// read-once stream drew about 7.0 TB/s from HBM with that hint and 6.3 TB/s
// without it (2 GiB, LDS DMA, measured on gfx950); bytes that a second wave
// reads again should keep the default policy so the caches serve them.
template <bool STREAM>
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, uint32_t lds) {
    const uint64_t b = uint64_t(uintptr_t(base));
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(b));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(b >> 32));
    const uint64_t sb = (uint64_t(hi) << 32) | lo;
    const uint32_t sl = __builtin_amdgcn_readfirstlane(lds);
    if (STREAM)
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sb), "s"(sl)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sb), "s"(sl)
                     : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// A partial-result store written through to memory (sc0 sc1: system scope)
// rather than left dirty in the L2: the merge launch reads it, never this
// one, and a launch whose L2 holds no dirty partials ends sooner (32768-key
// wave-pair decode 13.7 vs 14.0 us per layer, measured on gfx950).
__device__ __forceinline__ void store_wt(float* p, float v) {
    asm volatile("global_store_dword %0, %1, off sc0 sc1" ::"v"(p), "v"(v) : "memory");
}

// 8 codes of a dword as MFMA k-slots: (c0,c4) (c1,c5)x16 (c2,c6) (c3,c7)x16,
// each the f16 subnormal (code + 8) * 2^-24 (x16 where marked).  Flipping
// bit 3 of every nibble turns two's complement into offset binary.
__device__ __forceinline__ half8_t unpack8(uint32_t w) {
    constexpr uint32_t X = 0x88888888u;
    const uint32_t w2 = w >> 8;
    const u32x4 r = {(w ^ X) & 0x000F000Fu, (w ^ X) & 0x00F000F0u, (w2 ^ X) & 0x000F000Fu, (w2 ^ X) & 0x00F000F0u};
    return __builtin_bit_cast(half8_t, r);
}

// The f16 context operand p * 2^a * (V scale): p = 2^(score - m) <= 2^6 (the
// lazily moving maximum), so with the tile's largest V scale s in
// [2^(-8-a), 2^(9-a)) every product stays below 2^15 and the dominant ones
// above 2^-8 (full f16 precision).  a is a per-wave power-of-two exponent in
// [-7, 9] (p * 2^a <= 2^15); it starts at 0 and moves when a tile's largest
// V scale leaves the window, e.g. for binary16-subnormal scales.  Scales are
// non-negative f16, so their bit patterns order as the values do.
constexpr int kVExpMin = -7, kVExpMax = 9;

// binary16 bits of 2^e (0x10000, above every f16, for e >= 16; 0 below 2^-24).
__device__ __forceinline__ uint32_t f16_bits_pow2(int e) {
    return e >= 16 ? 0x10000u : (e >= -14 ? uint32_t(e + 15) << 10 : (e >= -24 ? 1u << (e + 24) : 0u));
}

// Largest of the four f16 bit patterns held in two dwords.
__device__ __forceinline__ uint32_t max4_u16(uint32_t w0, uint32_t w1) {
    typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
    const u16x2 m = __builtin_elementwise_max(__builtin_bit_cast(u16x2, w0), __builtin_bit_cast(u16x2, w1));
    return max(uint32_t(m[0]), uint32_t(m[1]));
}

// Wave-uniform: does the wave's largest value of x (one f16 bit pattern per
// lane) lie outside [lo, hi)?
__device__ __forceinline__ bool outside_window(uint32_t x, uint32_t lo, uint32_t hi) {
    return __builtin_amdgcn_ballot_w64(x >= lo) == 0ull || __builtin_amdgcn_ballot_w64(x >= hi) != 0ull;
}

// The exponent a for the wave's largest V scale (x: one f16 bit pattern per
// lane), clamped to [kVExpMin, kVExpMax]; a_old if every scale is 0.  The
// scale's exponent e = floor(log2 max) in [-24, 15] is found by a binary
// search on wave ballots (compares against scalars only: no vector registers
// beyond x in this rarely taken path).
__device__ __forceinline__ int v_exponent_for(uint32_t x, int a_old) {
    if (__builtin_amdgcn_ballot_w64(x != 0u) == 0ull) return a_old;
    int lo = -24, hi = 15;  // some lane holds at least 2^lo; none holds 2^(hi + 1)
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (__builtin_amdgcn_ballot_w64(x >= f16_bits_pow2(mid)) != 0ull) lo = mid;
        else hi = mid - 1;
    }
    return min(max(-lo, kVExpMin), kVExpMax);
}

// 2^e for an integer e in [-126, 127], exactly.
__device__ __forceinline__ float pow2i(int e) { return __uint_as_float(uint32_t(e + 127) << 23); }

// The context weights of two keys, each p times its key's f16 V scale, as
// one f16 pair: p0 * lo(s2), p1 * hi(s2), each formed in fp32 from the fp32 p
// (exact but for the fp32 rounding, 2^-24) and rounded to f16 once, rather
// than rounding p to f16 first and the f16 product again (the decode kernels'
// cheaper form, whose error averages out over a decode's many keys but not
// over the few keys of a prompt chunk's first rows).  Plain code, so the
// compiler sees every operand (it picks the instructions and their waits).
__device__ __forceinline__ half2_t ctx_weights(float p0, float p1, uint32_t s2) {
    const half2_t s = __builtin_bit_cast(half2_t, s2);
    return half2_t{_Float16(p0 * float(s[0])), _Float16(p1 * float(s[1]))};
}

__device__ __forceinline__ f32x4 mfma(half8_t a, half8_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float lo_half(uint32_t w) { return float(__builtin_bit_cast(half2_t, w)[0]); }
__device__ __forceinline__ float hi_half(uint32_t w) { return float(__builtin_bit_cast(half2_t, w)[1]); }

// max(a, b, c) and max(a, b) as single instructions, for values that are
// finite or -inf, never NaN (the compiler otherwise quiets each fmaxf
// operand with a v_max of the operand with itself).
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float max2f(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
// Max of the 8 values a lane holds for two 16-key blocks, then over the
// lanes l, l^16, l^32, l^48.
__device__ __forceinline__ float max8f(const float (&x)[2][4]) {
    return max3f(max3f(x[0][0], x[0][1], x[0][2]), max3f(x[0][3], x[1][0], x[1][1]), max2f(x[1][2], x[1][3]));
}
__device__ __forceinline__ float quad_max_nonan(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = max2f(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return max2f(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Max / sum over the lanes l, l^16, l^32, l^48 (the four row-quarters of an
// MFMA output column), with vector-ALU lane swaps rather than LDS.
__device__ __forceinline__ float quad_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// x of lane l ^ 8 within each 16-lane row (DPP row_ror:8; every lane is
// written, so bound_ctrl has no effect -- it lets the move fold into the
// instruction that uses it).
__device__ __forceinline__ float row_xor8(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, true));
}

}  // namespace mx
}  // namespace kvq
