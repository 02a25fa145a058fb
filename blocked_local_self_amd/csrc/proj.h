// Shapes and launchers of the layer's projection kernels (kernel_proj.hip).
#pragma once

#include "halo_common.h"

namespace halo {

// Division by a run-time constant d >= 1 for dividends below 2^31, by
// multiplication (Granlund and Montgomery, "Division by invariant integers
// using multiplication", 1994): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(n, m) + n) >> l.
struct FastDiv {
    uint32_t d, m, l;
    FastDiv() = default;
    explicit FastDiv(uint32_t dv) : d(dv)
    {
        l = 0;
        while ((1ull << l) < dv) ++l;
        m = (uint32_t)((((1ull << l) - dv) << 32) / dv + 1);
    }
    __device__ __forceinline__ uint32_t div(uint32_t n) const { return (__umulhi(n, m) + n) >> l; }
};

struct LayerGeom {
    int64_t NP, NPo;      // pixels in / out: B*H*W, B*Ho*Wo
    int B, H, W, Ho, Wo;
    int C, Cout;          // layer channels in / out
    int heads, d;         // attention heads and channels per head
    int side, side_out;   // block side of the blocked layout, in / out (block, block/stride)
    int layout;           // 0 NHWC, 1 blocked
    // dividers for the pixel and channel index arithmetic of the
    // matrix-core kernels (pixel counts below 2^31)
    FastDiv fW, fH, fWo, fHo, fbb, fside, fnbx, fnby, fbbo, fsideo, fnbxo, fnbyo, finner, fd;
};

// Fills the dividers of L's sizes (the launchers call it).
void layer_fastdiv(LayerGeom& L);

struct ProjPlan {
    int ns;               // weight rows (output channels) per workgroup
    int nslices;          // workgroups per pixel chunk
    int pitch;            // LDS weight row pitch, elements
    int chunk;            // pixels per workgroup
    int lds_bytes;
    int stage;            // output projection: byte offset of the per-wave row staging (0: direct stores)
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

// The whole layer in one kernel (kernel_layer.hip): bf16, query stride 1,
// d in {16, 32}, block in {4, 8} dividing H and W, window side <= 16,
// C % 32 == 0, C_out % 16 == 0 and C_out <= 256, within one workgroup's LDS.
// The caller checks pointer alignment (16 bytes for x, w_q, w_kv; 8 bytes
// for w_o, b_o, rel_h, rel_w, y).
bool layer_fused_supported(const LayerGeom& L, int block, int halo, int stride, bool bf16);
// Whether AUTO takes the fused kernel where it is supported (by measurement).
bool layer_fused_preferred(const LayerGeom& L, int block, int halo, int stride);
hipError_t launch_layer_fused(const void* x, const void* w_q, const void* w_kv, const void* w_o, const void* b_o,
                              const void* rel_h, const void* rel_w, void* y, const LayerGeom& L, int block, int halo,
                              float scale, hipStream_t s);

}  // namespace halo
