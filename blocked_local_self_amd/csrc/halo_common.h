// Shared definitions of the halo-attention kernels (gfx950).
//
// Geometry follows "Scaling Local Self-Attention for Parameter Efficient
// Visual Backbones" (HaloNet), section 2.2 with Figures 1 and 2: blocks of
// side `block` tiled from the top-left, window side r = block + 2*halo
// starting at (by*block - halo, bx*block - halo), queries at multiples of the
// query stride.  The relative-table row of displacement (key - query) is
// displacement + c0, c0 = r - 1 + halo, as in the HaloAttention module of the
// pswp.cn blog page (section 4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace halo {

// Everything a kernel needs to know about one call, computed on the host.
struct Geometry {
    int64_t BH;        // batch * heads
    int H, W, d;
    int block, halo, stride;
    int r;             // window side
    int c0;            // table row of displacement 0
    int Ho, Wo;        // output spatial size
    int nbh, nbw;      // blocks per column / row (ceil)
    float scale;       // multiplies q.k and q.rel
    int flags;         // semantic variants (HALO_CENTRED_OFFSET, ...); 0: the pages' reading
};

// Semantic variants (bit values as in include/halo_attn.h).
constexpr int kFlagCentredOffset = 1;   // table row of displacement D is D + r - 1
constexpr int kFlagZeroPad = 2;         // off-image window positions are zero keys and values
constexpr int kFlagCentredMask = 4;     // only keys within h rows and columns of the query
constexpr int kFlagHalfSplit = 8;       // height table on channels [0, d/2), width on [d/2, d)

// The matrix-core forward kernels (selection in kernel_mfma.hip): the
// 16-query tile kernel, the persistent ring kernel, the streaming kernel for
// windows wider than 32 columns, the strip kernel.
enum class MfmaKernel { tile, ring, wide, strip };

// Attributes of the current device, queried through HIP once per device and
// cached (kernel planning runs on every call and must not pay for API calls).
struct DeviceInfo {
    int lds_per_block;   // bytes of dynamic LDS one workgroup may use
    int cus;             // compute units
};
DeviceInfo device_info();

// Raise a kernel's dynamic-LDS limit to `bytes` once per device (a no-op at
// or below the 64 KiB default).
hipError_t ensure_lds_limit(const void* kernel, int bytes);

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// Round to nearest even (the gfx950 conversion instruction rounds that way).
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return static_cast<__bf16>(x); }

}  // namespace halo
