// Matrix-core helpers shared by the fused halo-attention kernels (gfx950).
#pragma once

#include "halo_common.h"

namespace halo {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kMaskLogit = -1.0e30f;       // exp2 of (alpha * this) is exactly 0

// Channel fragment of the QK^T MFMA operands: K = 16 uses 4 channels per lane,
// K = 32 uses 8.  Both operands are loaded with the same lane->channel map, so
// the contraction is over exactly the d channels.
template <int D> struct Frag;
template <> struct Frag<16> {
    typedef s16x4 T;
    __device__ static inline f32x4 mma(T a, T b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
};
template <> struct Frag<32> {
    typedef s16x8 T;
    __device__ static inline f32x4 mma(T a, T b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16((bf16x8)a, (bf16x8)b, c, 0, 0, 0);
    }
};

__device__ inline f32x4 mma_k32(s16x8 a, s16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16((bf16x8)a, (bf16x8)b, c, 0, 0, 0);
}

// 32x32 output tile, K = 16 (8 bf16 per lane: lanes 0-31 and 32-63 hold the
// two halves of K for row / column lane & 31).  Lane l holds rows
// 8j + 4(l >> 5) + i (j, i = 0..3) of column l & 31, element 4j + i.
__device__ inline f32x16 mma32_k16(s16x8 a, s16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16((bf16x8)a, (bf16x8)b, c, 0, 0, 0);
}

__device__ inline unsigned pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 p;
    p[0] = (__bf16)lo;
    p[1] = (__bf16)hi;
    return __builtin_bit_cast(unsigned, p);
}

__device__ inline void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Reductions over the four lanes n, n+16, n+32, n+48 (the lanes holding one
// query in the 16x16 MFMA layouts), on the gfx950 cross-row swaps (VALU, no
// LDS traffic).  v_permlane16_swap exchanges the odd 16-lane rows of its
// first operand with the even rows of its second, v_permlane32_swap the upper
// 32 lanes of the first with the lower 32 of the second; fed two copies of one
// value they return both halves of every row pair / wave half.  Written as
// inline asm because this compiler folds the second result of the
// corresponding builtins into the first.  The s_nop gives the two wait states
// a VALU write needs before a permlane reads it.
__device__ inline void swap16(float& a, float& b)
{
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ inline void swap32(float& a, float& b)
{
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ inline float max_over_rows(float x)
{
    float a = x, b = x;
    swap16(a, b);
    a = fmaxf(a, b);
    b = a;
    swap32(a, b);
    return fmaxf(a, b);
}
__device__ inline float sum_over_rows(float x)
{
    float a = x, b = x;
    swap16(a, b);
    a = a + b;
    b = a;
    swap32(a, b);
    return a + b;
}

__device__ inline float max4(f32x4 s)
{
    return fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
}

}  // namespace halo
