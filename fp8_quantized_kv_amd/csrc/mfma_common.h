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

// 8 codes of a dword as MFMA k-slots: (c0,c4) (c1,c5)x16 (c2,c6) (c3,c7)x16,
// each the f16 subnormal (code + 8) * 2^-24 (x16 where marked).  Flipping
// bit 3 of every nibble turns two's complement into offset binary.
__device__ __forceinline__ half8_t unpack8(uint32_t w) {
    constexpr uint32_t X = 0x88888888u;
    const uint32_t w2 = w >> 8;
    const u32x4 r = {(w ^ X) & 0x000F000Fu, (w ^ X) & 0x00F000F0u, (w2 ^ X) & 0x000F000Fu, (w2 ^ X) & 0x00F000F0u};
    return __builtin_bit_cast(half8_t, r);
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
