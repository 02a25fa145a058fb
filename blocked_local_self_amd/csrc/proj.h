// Shapes and launchers of the layer's projection kernels (kernel_proj.hip).
#pragma once

#include "halo_common.h"

namespace halo {

struct LayerGeom {
    int64_t NP, NPo;      // pixels in / out: B*H*W, B*Ho*Wo
    int B, H, W, Ho, Wo;
    int C, Cout;          // layer channels in / out
    int heads, d;         // attention heads and channels per head
    int side, side_out;   // block side of the blocked layout, in / out (block, block/stride)
    int layout;           // 0 NHWC, 1 blocked
};

struct ProjPlan {
    int ns;               // weight rows (output channels) per workgroup
    int nslices;          // workgroups per pixel chunk
    int pitch;            // LDS weight row pitch, elements
    int chunk;            // pixels per workgroup
    int lds_bytes;
    int remap_xcd;
    int64_t nwg;
};

// Whether the matrix-core kernels take these shapes (the caller also checks
// that the pointers are 16-byte aligned).
bool proj_in_mfma_supported(const LayerGeom& L, bool bf16);
bool proj_out_mfma_supported(const LayerGeom& L, bool bf16);
// mfma: run the matrix-core kernel (only when supported), else the plain one.
hipError_t launch_proj_in(const void* x, const void* w_q, const void* w_kv, void* q, void* k, void* v,
                          const LayerGeom& L, bool bf16, bool mfma, hipStream_t st);
hipError_t launch_proj_out(const void* attn, const void* w_o, const void* b_o, void* y, const LayerGeom& L, bool bf16,
                           bool mfma, hipStream_t st);

}  // namespace halo
