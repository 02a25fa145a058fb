// Issue-rate probe for gfx950 (a measurement aid, not part of the attention
// path): independent chains of one instruction kind per wave, so the time
// of a launch is set by how fast a SIMD issues that kind.  bench.py
// --issue-rates times the modes and derives per-SIMD rates; they price the
// attention kernels' instruction streams (fp32 FMA, the exp2 of the
// softmax, bf16 MFMA) and show whether MFMA and VALU work of two waves on
// one SIMD overlap.
#include "halo_attn.h"
#include "mfma_util.h"

namespace halo {

constexpr int kProbeChains = 8;      // independent VALU chains per lane
constexpr int kProbeMfmaChains = 4;  // independent MFMA accumulators per wave
constexpr int kProbeWaves = 8;       // waves per workgroup (two per SIMD)

// Modes: 0 FMA, 1 exp2, 2 MFMA 16x16x32 bf16, 3 MFMA 32x32x16 bf16,
// 4 exp2 in waves 0-3 and MFMA 16x16x32 in waves 4-7, 5 exp2 in waves 0-3
// and FMA in waves 4-7.  A mode-4/5 launch does the work of half a mode-1
// launch plus half a mode-2 (mode-0) launch.
__device__ inline void probe_fma(float* x, int iters)
{
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int j = 0; j < kProbeChains; ++j) x[j] = fmaf(x[j], 0.999f, 0.001f);
}

__device__ inline void probe_exp(float* x, int iters)
{
    // x = 2^-x has a stable fixed point near 0.641: no overflow, no denormals
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int j = 0; j < kProbeChains; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
}

template <bool WIDE>
__device__ inline float probe_mfma(int iters, int lane)
{
    const s16x8 a = {(short)(0x3F80 + (lane & 7)), 0, 0, 0, 0, 0, 0, 0};
    const s16x8 b = {0, (short)(0x3F80 + (lane >> 3)), 0, 0, 0, 0, 0, 0};
    float sum = 0.f;
    if constexpr (WIDE) {
        f32x16 acc[kProbeMfmaChains] = {};
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int j = 0; j < kProbeMfmaChains; ++j) acc[j] = mma32_k16(a, b, acc[j]);
#pragma unroll
        for (int j = 0; j < kProbeMfmaChains; ++j) sum += acc[j][0];
    } else {
        f32x4 acc[kProbeMfmaChains] = {};
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int j = 0; j < kProbeMfmaChains; ++j) acc[j] = mma_k32(a, b, acc[j]);
#pragma unroll
        for (int j = 0; j < kProbeMfmaChains; ++j) sum += acc[j][0];
    }
    return sum;
}

__global__ __launch_bounds__(64 * kProbeWaves) void issue_probe_kernel(float* out, int mode, int iters)
{
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    float x[kProbeChains];
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j) x[j] = 0.5f + 0.01f * (float)((lane + j) & 7);
    float sum = 0.f;
    const bool second = wave >= kProbeWaves / 2;       // waves 4-7 (sharing SIMDs with waves 0-3)
    switch (mode) {
    case 0: probe_fma(x, iters); break;
    case 1: probe_exp(x, iters); break;
    case 2: sum = probe_mfma<false>(iters, lane); break;
    case 3: sum = probe_mfma<true>(iters, lane); break;
    case 4:
        if (second) sum = probe_mfma<false>(iters, lane);
        else probe_exp(x, iters);
        break;
    default:
        if (second) probe_fma(x, iters);
        else probe_exp(x, iters);
        break;
    }
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j) sum += x[j];
    out[(int64_t)blockIdx.x * blockDim.x + tid] = sum;      // keeps every chain live
}

}  // namespace halo

extern "C" int halo_attn_probe_issue(int mode, int iters, int workgroups, float* out, void* stream)
{
    if (mode < 0 || mode > 5 || iters < 1 || workgroups < 1) return HALO_ERR_SHAPE;
    if (out == nullptr) return HALO_ERR_NULL;
    hipLaunchKernelGGL(halo::issue_probe_kernel, dim3((unsigned)workgroups), dim3(64 * halo::kProbeWaves), 0,
                       static_cast<hipStream_t>(stream), out, mode, iters);
    return hipGetLastError() == hipSuccess ? HALO_OK : HALO_ERR_HIP;
}
