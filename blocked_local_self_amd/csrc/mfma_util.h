// Matrix-core helpers shared by the fused halo-attention kernels (gfx950).
#pragma once

#include "halo_common.h"

namespace halo {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

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
// query in the 16x16 MFMA layouts).  The gfx950 row-swap builtins are not
// used: this compiler folds their second result into the first.
__device__ inline float max_over_rows(float x)
{
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}
__device__ inline float sum_over_rows(float x)
{
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

__device__ inline float max4(f32x4 s)
{
    return fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
}

}  // namespace halo
