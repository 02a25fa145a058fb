// C ABI of the halo-attention library: argument checks, kernel choice, launch.
// The operation and every convention are documented in include/halo_attn.h.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <utility>
#include <vector>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/halo_attn.h"
#include "halo_common.h"
#include "proj.h"

namespace halo {

DeviceInfo device_info()
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static std::atomic<int> ready[kMaxDevices];
    static DeviceInfo info[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DeviceInfo{64 * 1024, 256};
    if (!ready[dev].load(std::memory_order_acquire)) {
        std::lock_guard<std::mutex> lock(mu);
        if (!ready[dev].load(std::memory_order_relaxed)) {
            int lds = 0, cus = 0;
            if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || lds <= 0)
                lds = 64 * 1024;
            if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
                cus = 256;
            info[dev] = DeviceInfo{lds, cus};
            ready[dev].store(1, std::memory_order_release);
        }
    }
    return info[dev];
}

hipError_t ensure_lds_limit(const void* kernel, int bytes)
{
    if (bytes <= 64 * 1024) return hipSuccess;
    // (kernel, device) pairs already raised; the attribute is per device
    static std::mutex mu;
    static std::vector<std::pair<const void*, int>> done;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    std::lock_guard<std::mutex> lock(mu);
    for (const auto& d : done)
        if (d.first == kernel && d.second == dev) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done.emplace_back(kernel, dev);
    return e;
}

hipError_t launch_generic(const void* q, const void* k, const void* v, const void* rh,
                          const void* rw, void* out, float* lse, const Geometry& g, bool bf16, hipStream_t st);
bool mfma_supported(int d, int r, int block, int stride, bool bf16);
hipError_t launch_mfma(const void* q, const void* k, const void* v, const void* rh,
                       const void* rw, void* out, float* lse, const Geometry& g, int mode,
                       hipStream_t st);
MfmaKernel mfma_select(const Geometry& g, int mode);
int64_t bwd_generic_workspace_floats(const Geometry& g);
hipError_t launch_bwd_generic(const void* q, const void* k, const void* v, const void* rh, const void* rw,
                              const void* out, const void* dout, const float* lse,
                              void* dq, void* dk, void* dv, float* drh, float* drw,
                              void* ws, const Geometry& g, bool bf16, hipStream_t st);
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t st);
bool ring_supported(const Geometry& g);
bool bwd_mfma_supported(const Geometry& g, bool bf16);
int64_t bwd_mfma_rel_rows(const Geometry& g);
int64_t bwd_mfma_kv_floats(const Geometry& g);
int64_t bwd_rel_chunks(int64_t nrows);
hipError_t launch_bwd_mfma(const void* q, const void* k, const void* v, const void* rh, const void* rw,
                           const void* out, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           float* part_kv, float* part_rel, const Geometry& g, hipStream_t st);
hipError_t launch_rel_reduce(const float* part, int64_t nrows, float* part2, float* drh, float* drw,
                             const Geometry& g, hipStream_t st);
bool bwd_tile_supported(const Geometry& g, bool bf16);
int64_t bwd_tile_rel_rows(const Geometry& g);
hipError_t launch_bwd_tile(const void* q, const void* k, const void* v, const void* rh, const void* rw,
                           const void* out, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           float* dsum, float* part_rel, const Geometry& g, hipStream_t st);
}  // namespace halo

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return pa < pb + nb && pb < pa + na;
}

// Checks that need no tensor pointers; shared by the launch and the query.
int check_config(int d, int block, int halo, int stride, int dtype)
{
    if (dtype != HALO_F32 && dtype != HALO_BF16)
        return fail(HALO_ERR_DTYPE, "dtype %d is neither HALO_F32 (0) nor HALO_BF16 (1)", dtype);
    if (d < 1 || d > 128) return fail(HALO_ERR_SHAPE, "d=%d outside [1, 128]", d);
    if (block < 1) return fail(HALO_ERR_SHAPE, "block=%d must be >= 1", block);
    if (halo < 0) return fail(HALO_ERR_SHAPE, "halo=%d must be >= 0", halo);
    if ((int64_t)block + 2 * (int64_t)halo > 256)
        return fail(HALO_ERR_SHAPE, "window side block+2*halo=%lld exceeds 256",
                    (long long)block + 2 * (long long)halo);
    if (stride < 1) return fail(HALO_ERR_SHAPE, "query_stride=%d must be >= 1", stride);
    if (block % stride)
        return fail(HALO_ERR_SHAPE, "query_stride=%d does not divide block=%d", stride, block);
    return HALO_OK;
}

}  // namespace

extern "C" {

const char* halo_attn_last_error(void) { return g_err; }

int halo_attn_abi_version(void) { return HALO_ATTN_ABI_VERSION; }

#ifndef HALO_BUILD_ID
#define HALO_BUILD_ID "unknown"
#endif
const char* halo_attn_build_id(void) { return HALO_BUILD_ID; }

int halo_attn_select_kernel(int d, int block, int halo, int query_stride, int dtype)
{
    g_err[0] = 0;
    const int st = check_config(d, block, halo, query_stride, dtype);
    if (st) return st;
    return halo::mfma_supported(d, block + 2 * halo, block, query_stride, dtype == HALO_BF16)
               ? HALO_KERNEL_MFMA : HALO_KERNEL_GENERIC;
}

}  // extern "C"

namespace {

// Checks shared by every entry point that takes tensors.  Fills g; sets
// empty when a size is zero (the call then has nothing to compute).
int check_sizes(int B, int heads, int H, int W, int d, int block, int halo, int query_stride,
                float scale, int dtype, halo::Geometry& g, bool& empty)
{
    int st = check_config(d, block, halo, query_stride, dtype);
    if (st) return st;
    if (B < 0 || heads < 0 || H < 0 || W < 0)
        return fail(HALO_ERR_SHAPE, "negative size: B=%d heads=%d H=%d W=%d", B, heads, H, W);
    if (H % query_stride || W % query_stride)
        return fail(HALO_ERR_SHAPE, "query_stride=%d must divide H=%d and W=%d", query_stride, H, W);
    if (!std::isfinite(scale)) return fail(HALO_ERR_SHAPE, "scale must be finite");
    const int r = block + 2 * halo;
    g = halo::Geometry{};
    g.d = d; g.block = block; g.halo = halo; g.stride = query_stride;
    g.r = r; g.c0 = r - 1 + halo; g.scale = scale;
    empty = B == 0 || heads == 0 || H == 0 || W == 0;
    if (empty) return HALO_OK;
    // magnitude checks in double first, so the int64 products below cannot overflow
    const double nelem = (double)B * heads * H * W * d;
    const int nbh = (H + block - 1) / block, nbw = (W + block - 1) / block;
    const double nblk = (double)B * heads * nbh * nbw;
    if (nelem >= 1e18)
        return fail(HALO_ERR_SHAPE, "tensor too large (%.3g elements, limit 1e18)", nelem);
    if (nblk >= 2147483648.0)
        return fail(HALO_ERR_SHAPE, "%.0f blocks exceed the 2^31 grid limit", nblk);
    // pixel indices inside one (batch, head) image are 32-bit in the kernels
    if ((double)H * W >= 2147483648.0)
        return fail(HALO_ERR_SHAPE, "H*W=%.0f pixels per image reach the 2^31 limit", (double)H * W);
    g.BH = (int64_t)B * heads; g.H = H; g.W = W;
    g.Ho = H / query_stride; g.Wo = W / query_stride;
    g.nbh = nbh; g.nbw = nbw;
    return HALO_OK;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace of the matrix-core backward, carved in this order (256-byte
// aligned pieces): per-column dk/dv shares, per-workgroup table partials,
// the table reduction's first level, then the forward's lse and out when the
// caller does not pass them.
struct MfmaWs {
    size_t kv, rel, rel2, lse, out, total;
};
MfmaWs mfma_ws(const halo::Geometry& g)
{
    MfmaWs w;
    const int64_t rows = halo::bwd_mfma_rel_rows(g);
    const int64_t e2 = 2 * (int64_t)(2 * g.r - 1) * g.d;
    const int64_t nq = g.BH * g.Ho * g.Wo;
    w.kv = 0;
    w.rel = align256(w.kv + (size_t)halo::bwd_mfma_kv_floats(g) * 4);
    w.rel2 = align256(w.rel + (size_t)(rows * e2) * 4);
    w.lse = align256(w.rel2 + (size_t)(halo::bwd_rel_chunks(rows) * e2) * 4);
    w.out = align256(w.lse + (size_t)nq * 4);
    w.total = align256(w.out + (size_t)(nq * g.d) * 2);
    return w;
}

// Workspace of the 16-query tile backward: D = dout.out per query, one
// table-gradient partial per block, the reduction's first level, then the
// forward's lse and out when the caller does not pass them.
struct TileWs {
    size_t dsum, rel, rel2, lse, out, total;
};
TileWs tile_ws(const halo::Geometry& g)
{
    TileWs w;
    const int64_t rows = halo::bwd_tile_rel_rows(g);
    const int64_t e2 = 2 * (int64_t)(2 * g.r - 1) * g.d;
    const int64_t nq = g.BH * g.Ho * g.Wo;
    w.dsum = 0;
    w.rel = align256(w.dsum + (size_t)nq * 4);
    w.rel2 = align256(w.rel + (size_t)(rows * e2) * 4);
    w.lse = align256(w.rel2 + (size_t)(halo::bwd_rel_chunks(rows) * e2) * 4);
    w.out = align256(w.lse + (size_t)nq * 4);
    w.total = align256(w.out + (size_t)(nq * g.d) * 2);
    return w;
}

// The matrix-core backward of a shape: 1 the strip kernel (windows of at
// most 16 columns over whole blocks), 2 the 16-query tile kernels, 0 none.
int bwd_mfma_path(const halo::Geometry& g, bool bf16)
{
    if (halo::bwd_mfma_supported(g, bf16)) return 1;
    if (halo::bwd_tile_supported(g, bf16)) return 2;
    return 0;
}

size_t bwd_ws_bytes(const halo::Geometry& g, bool bf16)
{
    const size_t gen = (size_t)halo::bwd_generic_workspace_floats(g) * 4;
    switch (bwd_mfma_path(g, bf16)) {
    case 1: return std::max(gen, mfma_ws(g).total);
    case 2: return std::max(gen, tile_ws(g).total);
    default: return gen;
    }
}

// Validates a forward call's kernel, flags and sizes into g.
int fwd_geometry(int B, int heads, int H, int W, int d, int block, int halo, int query_stride, float scale,
                 int dtype, int flags, int kernel, halo::Geometry& g, bool& empty)
{
    if (kernel != HALO_KERNEL_AUTO && kernel != HALO_KERNEL_GENERIC && kernel != HALO_KERNEL_MFMA &&
        kernel != HALO_KERNEL_MFMA_STRIP && kernel != HALO_KERNEL_MFMA_RING)
        return fail(HALO_ERR_SHAPE, "kernel=%d is not a halo_kernel value", kernel);
    if (flags & ~(HALO_CENTRED_OFFSET | HALO_ZERO_PAD | HALO_CENTRED_MASK | HALO_HALF_SPLIT))
        return fail(HALO_ERR_SHAPE, "flags=%d has bits outside the halo_flags values", flags);
    const int st = check_sizes(B, heads, H, W, d, block, halo, query_stride, scale, dtype, g, empty);
    if (st) return st;
    g.flags = flags;
    if (flags & HALO_CENTRED_OFFSET) g.c0 = g.r - 1;
    return HALO_OK;
}

// The forward kernel of a call: mode >= 0 runs the matrix-core launcher in
// that mode (0 the fastest kernel for the shape, 1 the strip kernel, 2 the
// ring kernel), -1 the generic kernel.
int fwd_choice(const halo::Geometry& g, bool bf16, int kernel, int& mode)
{
    // the variants run on the ring kernel and the generic kernel only
    const bool mfma_ok = halo::mfma_supported(g.d, g.r, g.block, g.stride, bf16) &&
                         (g.flags == 0 || halo::ring_supported(g));
    const bool forced = kernel == HALO_KERNEL_MFMA || kernel == HALO_KERNEL_MFMA_STRIP ||
                        kernel == HALO_KERNEL_MFMA_RING;
    if (forced && !mfma_ok)
        return fail(HALO_ERR_UNSUPPORTED,
                    "matrix-core kernel needs bf16, block %% 4 == 0, d in {16,32} with window side <= 40 "
                    "(variants: <= 32) or d = 64 with window side <= 32 (no variants) "
                    "(got bf16=%d d=%d block=%d r=%d flags=%d)",
                    (int)bf16, g.d, g.block, g.r, g.flags);
    if (kernel == HALO_KERNEL_MFMA_STRIP && g.flags)
        return fail(HALO_ERR_UNSUPPORTED, "the strip kernel runs the default semantics only (flags=%d)", g.flags);
    if (kernel == HALO_KERNEL_MFMA_STRIP && g.d == 64)
        return fail(HALO_ERR_UNSUPPORTED, "the strip kernel takes d = 16 and 32 only (d=%d)", g.d);
    if (kernel == HALO_KERNEL_MFMA_STRIP && g.d == 32 && g.r > 32)
        return fail(HALO_ERR_UNSUPPORTED, "the strip kernel takes windows of up to 32 columns at d = 32 (r=%d)", g.r);
    const bool use_mfma = forced || (kernel == HALO_KERNEL_AUTO && mfma_ok);
    mode = !use_mfma ? -1 : kernel == HALO_KERNEL_MFMA_STRIP ? 1 : kernel == HALO_KERNEL_MFMA_RING ? 2 : 0;
    return HALO_OK;
}

}  // namespace

extern "C" {

const char* halo_attn_fwd_kernel_name(int B, int heads, int H, int W, int d, int block, int halo,
                                      int query_stride, int dtype, int flags, int kernel)
{
    g_err[0] = 0;
    halo::Geometry g;
    bool empty = false;
    if (fwd_geometry(B, heads, H, W, d, block, halo, query_stride, 1.0f, dtype, flags, kernel, g, empty))
        return nullptr;
    if (empty) return "none";
    int mode = 0;
    if (fwd_choice(g, dtype == HALO_BF16, kernel, mode)) return nullptr;
    if (mode < 0) return "generic";
    switch (halo::mfma_select(g, mode)) {
    case halo::MfmaKernel::tile: return "tile";
    case halo::MfmaKernel::ring: return "ring";
    case halo::MfmaKernel::wide: return "wide";
    case halo::MfmaKernel::strip: return "strip";
    }
    return "strip";
}

const char* halo_attn_bwd_kernel_name(int B, int heads, int H, int W, int d, int block, int halo,
                                      int query_stride, int dtype, int flags, int kernel)
{
    g_err[0] = 0;
    if (flags & ~(HALO_CENTRED_OFFSET | HALO_ZERO_PAD | HALO_CENTRED_MASK | HALO_HALF_SPLIT)) {
        fail(HALO_ERR_SHAPE, "flags=%d has bits outside the halo_flags values", flags);
        return nullptr;
    }
    if (kernel != HALO_KERNEL_AUTO && kernel != HALO_KERNEL_GENERIC && kernel != HALO_KERNEL_MFMA &&
        kernel != HALO_KERNEL_MFMA_STRIP && kernel != HALO_KERNEL_MFMA_RING) {
        fail(HALO_ERR_SHAPE, "kernel=%d is not a halo_kernel value", kernel);
        return nullptr;
    }
    halo::Geometry g;
    bool empty = false;
    if (check_sizes(B, heads, H, W, d, block, halo, query_stride, 1.0f, dtype, g, empty)) return nullptr;
    g.flags = flags;
    if (flags & HALO_CENTRED_OFFSET) g.c0 = g.r - 1;
    if (empty) return "none";
    const int path = bwd_mfma_path(g, dtype == HALO_BF16);
    if (kernel != HALO_KERNEL_AUTO && kernel != HALO_KERNEL_GENERIC && path == 0) {
        fail(HALO_ERR_UNSUPPORTED, "no matrix-core backward for this shape (d=%d r=%d block=%d flags=%d)",
             d, g.r, block, flags);
        return nullptr;
    }
    if (kernel == HALO_KERNEL_GENERIC || path == 0) return "generic";
    return path == 1 ? "strip" : "tile";
}

int halo_attn_fwd_ex(const void* q, const void* k, const void* v,
                     const void* rel_h, const void* rel_w, void* out, float* lse,
                     int B, int heads, int H, int W, int d,
                     int block, int halo, int query_stride,
                     float scale, int dtype, int flags, int kernel, void* stream)
{
    g_err[0] = 0;
    halo::Geometry g;
    bool empty = false;
    int st = fwd_geometry(B, heads, H, W, d, block, halo, query_stride, scale, dtype, flags, kernel, g, empty);
    if (st) return st;
    if (empty) return HALO_OK;   // nothing to do

    if (!q || !k || !v || !rel_h || !rel_w || !out)
        return fail(HALO_ERR_NULL, "null pointer among q, k, v, rel_h, rel_w, out");
    const size_t nq = (size_t)(g.BH * g.Ho * g.Wo);

    const int r = g.r;
    const size_t esz = dtype == HALO_BF16 ? 2 : 4;
    const size_t in_bytes = (size_t)(g.BH * H * W * d) * esz;
    const size_t tab_bytes = (size_t)(2 * r - 1) * d * esz;
    const size_t out_bytes = (size_t)(g.BH * g.Ho * g.Wo * d) * esz;
    if (overlaps(out, out_bytes, q, in_bytes) || overlaps(out, out_bytes, k, in_bytes) ||
        overlaps(out, out_bytes, v, in_bytes) || overlaps(out, out_bytes, rel_h, tab_bytes) ||
        overlaps(out, out_bytes, rel_w, tab_bytes))
        return fail(HALO_ERR_ALIAS, "out overlaps an input tensor");
    if (lse && (overlaps(lse, nq * 4, q, in_bytes) || overlaps(lse, nq * 4, k, in_bytes) ||
                overlaps(lse, nq * 4, v, in_bytes) || overlaps(lse, nq * 4, rel_h, tab_bytes) ||
                overlaps(lse, nq * 4, rel_w, tab_bytes) || overlaps(lse, nq * 4, out, out_bytes)))
        return fail(HALO_ERR_ALIAS, "lse overlaps an input tensor or out");

    const bool bf16 = dtype == HALO_BF16;
    int mode = 0;
    st = fwd_choice(g, bf16, kernel, mode);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    const hipError_t e = mode >= 0 ? halo::launch_mfma(q, k, v, rel_h, rel_w, out, lse, g, mode, s)
                                   : halo::launch_generic(q, k, v, rel_h, rel_w, out, lse, g, bf16, s);
    if (e != hipSuccess)
        return fail(HALO_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return HALO_OK;
}

int halo_attn_fwd_lse(const void* q, const void* k, const void* v,
                      const void* rel_h, const void* rel_w, void* out, float* lse,
                      int B, int heads, int H, int W, int d,
                      int block, int halo, int query_stride,
                      float scale, int dtype, int kernel, void* stream)
{
    return halo_attn_fwd_ex(q, k, v, rel_h, rel_w, out, lse, B, heads, H, W, d, block, halo, query_stride,
                            scale, dtype, 0, kernel, stream);
}

int halo_attn_fwd_kernel(const void* q, const void* k, const void* v,
                         const void* rel_h, const void* rel_w, void* out,
                         int B, int heads, int H, int W, int d,
                         int block, int halo, int query_stride,
                         float scale, int dtype, int kernel, void* stream)
{
    return halo_attn_fwd_lse(q, k, v, rel_h, rel_w, out, nullptr, B, heads, H, W, d, block, halo,
                             query_stride, scale, dtype, kernel, stream);
}

int halo_attn_fwd(const void* q, const void* k, const void* v,
                  const void* rel_h, const void* rel_w, void* out,
                  int B, int heads, int H, int W, int d,
                  int block, int halo, int query_stride,
                  float scale, int dtype, void* stream)
{
    return halo_attn_fwd_kernel(q, k, v, rel_h, rel_w, out, B, heads, H, W, d, block, halo,
                                query_stride, scale, dtype, HALO_KERNEL_AUTO, stream);
}

long long halo_attn_bwd_workspace_bytes(int B, int heads, int H, int W, int d,
                                        int block, int halo, int query_stride, int dtype)
{
    g_err[0] = 0;
    halo::Geometry g;
    bool empty = false;
    const int st = check_sizes(B, heads, H, W, d, block, halo, query_stride, 1.0f, dtype, g, empty);
    if (st) return st;
    if (empty) return 0;
    return (long long)bwd_ws_bytes(g, dtype == HALO_BF16);
}

int halo_attn_bwd_ex(const void* q, const void* k, const void* v,
                     const void* rel_h, const void* rel_w,
                     const void* out, const void* dout, const float* lse,
                     void* dq, void* dk, void* dv, float* drel_h, float* drel_w,
                     void* workspace, size_t workspace_bytes,
                     int B, int heads, int H, int W, int d,
                     int block, int halo, int query_stride,
                     float scale, int dtype, int flags, int kernel, void* stream)
{
    g_err[0] = 0;
    if (flags & ~(HALO_CENTRED_OFFSET | HALO_ZERO_PAD | HALO_CENTRED_MASK | HALO_HALF_SPLIT))
        return fail(HALO_ERR_SHAPE, "flags=%d has bits outside the halo_flags values", flags);
    if (kernel != HALO_KERNEL_AUTO && kernel != HALO_KERNEL_GENERIC && kernel != HALO_KERNEL_MFMA &&
        kernel != HALO_KERNEL_MFMA_STRIP && kernel != HALO_KERNEL_MFMA_RING)
        return fail(HALO_ERR_SHAPE, "kernel=%d is not a halo_kernel value", kernel);
    halo::Geometry g;
    bool empty = false;
    int st = check_sizes(B, heads, H, W, d, block, halo, query_stride, scale, dtype, g, empty);
    if (st) return st;
    g.flags = flags;
    if (flags & HALO_CENTRED_OFFSET) g.c0 = g.r - 1;
    if (!drel_h || !drel_w) return fail(HALO_ERR_NULL, "null drel_h or drel_w");
    const int r = g.r;
    const size_t tabf = (size_t)(2 * r - 1) * d;
    if (overlaps(drel_h, tabf * 4, drel_w, tabf * 4))
        return fail(HALO_ERR_ALIAS, "drel_h overlaps drel_w");
    hipStream_t s = (hipStream_t)stream;
    if (empty) {   // the gradient of an empty sum: zero tables, nothing else
        hipError_t e = halo::launch_zero_f32(drel_h, (int64_t)tabf, s);
        if (e == hipSuccess) e = halo::launch_zero_f32(drel_w, (int64_t)tabf, s);
        if (e != hipSuccess) return fail(HALO_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
        return HALO_OK;
    }
    if (!q || !k || !v || !rel_h || !rel_w || !dout || !dq || !dk || !dv || !workspace)
        return fail(HALO_ERR_NULL, "null pointer among q, k, v, rel_h, rel_w, dout, dq, dk, dv, workspace");
    if ((out == nullptr) != (lse == nullptr))
        return fail(HALO_ERR_NULL, "pass both out and lse from the forward, or neither");
    const bool bf16 = dtype == HALO_BF16;
    const size_t need = bwd_ws_bytes(g, bf16);
    if (workspace_bytes < need)
        return fail(HALO_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu this call needs",
                    workspace_bytes, need);
    if ((uintptr_t)workspace % 16)
        return fail(HALO_ERR_WORKSPACE, "workspace must be 16-byte aligned");

    const size_t esz = dtype == HALO_BF16 ? 2 : 4;
    const size_t in_bytes = (size_t)(g.BH * H * W * d) * esz;
    const size_t tab_bytes = tabf * esz;
    const size_t out_bytes = (size_t)(g.BH * g.Ho * g.Wo * d) * esz;
    const size_t nq = (size_t)(g.BH * g.Ho * g.Wo);
    const void* ins[8] = {q, k, v, rel_h, rel_w, dout, out, lse};
    const size_t insz[8] = {in_bytes, in_bytes, in_bytes, tab_bytes, tab_bytes, out_bytes,
                            out ? out_bytes : 0, lse ? nq * 4 : 0};
    const void* outs[6] = {dq, dk, dv, drel_h, drel_w, workspace};
    const size_t outsz[6] = {in_bytes, in_bytes, in_bytes, tabf * 4, tabf * 4, need};
    for (int a = 0; a < 6; ++a) {
        for (int b = 0; b < 8; ++b)
            if (overlaps(outs[a], outsz[a], ins[b], insz[b]))
                return fail(HALO_ERR_ALIAS, "an output or the workspace overlaps an input tensor");
        for (int b = a + 1; b < 6; ++b)
            if (overlaps(outs[a], outsz[a], outs[b], outsz[b]))
                return fail(HALO_ERR_ALIAS, "two outputs (or an output and the workspace) overlap");
    }
    const bool aligned = ((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)dout | (uintptr_t)dq |
                          (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)(out ? out : q)) % 16 == 0;
    const int path = aligned ? bwd_mfma_path(g, bf16) : 0;
    if ((kernel == HALO_KERNEL_MFMA || kernel == HALO_KERNEL_MFMA_STRIP || kernel == HALO_KERNEL_MFMA_RING) &&
        path == 0)
        return fail(HALO_ERR_UNSUPPORTED,
                    "matrix-core backward needs bf16, the default semantics, d in {16,32}, 16-byte aligned "
                    "tensors, and a window side <= 32 with block <= 16 (got dtype=%d d=%d r=%d block=%d "
                    "flags=%d)", dtype, d, r, block, flags);
    hipError_t e;
    if (kernel == HALO_KERNEL_GENERIC || path == 0) {
        e = halo::launch_bwd_generic(q, k, v, rel_h, rel_w, out, dout, lse, dq, dk, dv, drel_h, drel_w,
                                     workspace, g, bf16, s);
    } else if (path == 2) {
        const TileWs w = tile_ws(g);
        unsigned char* base = static_cast<unsigned char*>(workspace);
        const void* fo = out;
        const float* fl = lse;
        e = hipSuccess;
        if (lse == nullptr) {   // the forward's out and lse, recomputed into the workspace
            fo = base + w.out;
            fl = reinterpret_cast<float*>(base + w.lse);
            float* wl = reinterpret_cast<float*>(base + w.lse);
            e = halo::mfma_supported(d, r, block, query_stride, bf16)
                    ? halo::launch_mfma(q, k, v, rel_h, rel_w, base + w.out, wl, g, 0, s)
                    : halo::launch_generic(q, k, v, rel_h, rel_w, base + w.out, wl, g, bf16, s);
        }
        float* rel = reinterpret_cast<float*>(base + w.rel);
        if (e == hipSuccess)
            e = halo::launch_bwd_tile(q, k, v, rel_h, rel_w, fo, dout, fl, dq, dk, dv,
                                      reinterpret_cast<float*>(base + w.dsum), rel, g, s);
        if (e == hipSuccess)
            e = halo::launch_rel_reduce(rel, halo::bwd_tile_rel_rows(g), reinterpret_cast<float*>(base + w.rel2),
                                        drel_h, drel_w, g, s);
    } else {
        const MfmaWs w = mfma_ws(g);
        unsigned char* base = static_cast<unsigned char*>(workspace);
        const void* fo = out;
        const float* fl = lse;
        e = hipSuccess;
        if (lse == nullptr) {   // the forward's out and lse, recomputed into the workspace
            fo = base + w.out;
            fl = reinterpret_cast<float*>(base + w.lse);
            float* wl = reinterpret_cast<float*>(base + w.lse);
            // the variants run on the persistent kernel or the generic one
            e = (flags == 0 || halo::ring_supported(g))
                    ? halo::launch_mfma(q, k, v, rel_h, rel_w, base + w.out, wl, g, 0, s)
                    : halo::launch_generic(q, k, v, rel_h, rel_w, base + w.out, wl, g, bf16, s);
        }
        if (e == hipSuccess)
            e = halo::launch_bwd_mfma(q, k, v, rel_h, rel_w, fo, dout, fl, dq, dk, dv,
                                      reinterpret_cast<float*>(base + w.kv), reinterpret_cast<float*>(base + w.rel),
                                      g, s);
        if (e == hipSuccess)
            e = halo::launch_rel_reduce(reinterpret_cast<const float*>(base + w.rel), halo::bwd_mfma_rel_rows(g),
                                        reinterpret_cast<float*>(base + w.rel2), drel_h, drel_w, g, s);
    }
    if (e != hipSuccess)
        return fail(HALO_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return HALO_OK;
}

int halo_attn_bwd_kernel(const void* q, const void* k, const void* v,
                         const void* rel_h, const void* rel_w,
                         const void* out, const void* dout, const float* lse,
                         void* dq, void* dk, void* dv, float* drel_h, float* drel_w,
                         void* workspace, size_t workspace_bytes,
                         int B, int heads, int H, int W, int d,
                         int block, int halo, int query_stride,
                         float scale, int dtype, int kernel, void* stream)
{
    return halo_attn_bwd_ex(q, k, v, rel_h, rel_w, out, dout, lse, dq, dk, dv, drel_h, drel_w, workspace,
                            workspace_bytes, B, heads, H, W, d, block, halo, query_stride, scale, dtype, 0,
                            kernel, stream);
}

int halo_attn_bwd(const void* q, const void* k, const void* v,
                  const void* rel_h, const void* rel_w,
                  const void* out, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, float* drel_h, float* drel_w,
                  void* workspace, size_t workspace_bytes,
                  int B, int heads, int H, int W, int d,
                  int block, int halo, int query_stride,
                  float scale, int dtype, void* stream)
{
    return halo_attn_bwd_kernel(q, k, v, rel_h, rel_w, out, dout, lse, dq, dk, dv, drel_h, drel_w, workspace,
                                workspace_bytes, B, heads, H, W, d, block, halo, query_stride, scale,
                                dtype, HALO_KERNEL_AUTO, stream);
}

}  // extern "C"

// ------------------------------------------------- allocation-free backward

// The backward's workspace for callers that cannot allocate: one array per
// GPU, held for the life of the process.  Its device address is taken once
// per device (hipGetSymbolAddress, with that device current) and cached;
// host code never passes the array's own name to a kernel.
static constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

// Address of `scratch` on the current device, or nullptr with the HIP error
// in `err`.
void* scratch_ptr(int& dev, hipError_t& err)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* ptrs[kMaxDevices] = {};
    err = hipGetDevice(&dev);
    if (err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (ptrs[dev] == nullptr) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return nullptr;
        ptrs[dev] = p;
    }
    err = hipSuccess;
    return ptrs[dev];
}

}  // namespace

extern "C" {

long long halo_attn_noalloc_scratch_bytes(void) { return (long long)kNoAllocScratchBytes; }

int halo_attn_bwd_noalloc(const void* q, const void* k, const void* v,
                          const void* rel_h, const void* rel_w,
                          const void* out, const void* dout, const float* lse,
                          void* dq, void* dk, void* dv, float* drel_h, float* drel_w,
                          int B, int heads, int H, int W, int d,
                          int block, int halo, int query_stride,
                          float scale, int dtype, void* stream)
{
    g_err[0] = 0;
    halo::Geometry g;
    bool empty = false;
    int st = check_sizes(B, heads, H, W, d, block, halo, query_stride, scale, dtype, g, empty);
    if (st) return st;
    const size_t need = empty ? 0 : bwd_ws_bytes(g, dtype == HALO_BF16);
    if (need > kNoAllocScratchBytes)
        return fail(HALO_ERR_WORKSPACE,
                    "this call needs %zu bytes of workspace; the library's static scratch holds %zu "
                    "(use halo_attn_bwd with a caller workspace, or split the batch)",
                    need, kNoAllocScratchBytes);
    int dev = 0;
    hipError_t e = hipSuccess;
    void* ws = scratch_ptr(dev, e);
    if (ws == nullptr) return fail(HALO_ERR_HIP, "static scratch of device %d: %s", dev, hipGetErrorString(e));
    return halo_attn_bwd_ex(q, k, v, rel_h, rel_w, out, dout, lse, dq, dk, dv, drel_h, drel_w, ws,
                            kNoAllocScratchBytes, B, heads, H, W, d, block, halo, query_stride, scale, dtype, 0,
                            HALO_KERNEL_AUTO, stream);
}

}  // extern "C"

// ------------------------------------------------------------------ the layer

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned8(const void* p) { return ((uintptr_t)p & 7u) == 0; }

// Checks of the layer's sizes; fills L (input and output grids).  empty: a
// size is zero, nothing to compute.
int check_layer(int B, int H, int W, int C, int Cout, int heads, int d, int side, int stride, int layout,
                int dtype, halo::LayerGeom& L, bool& empty)
{
    if (dtype != HALO_F32 && dtype != HALO_BF16)
        return fail(HALO_ERR_DTYPE, "dtype %d is neither HALO_F32 (0) nor HALO_BF16 (1)", dtype);
    if (layout != HALO_LAYOUT_NHWC && layout != HALO_LAYOUT_BLOCKED)
        return fail(HALO_ERR_SHAPE, "layout=%d is not a halo_layout value", layout);
    if (B < 0 || H < 0 || W < 0 || C < 0 || Cout < 0 || heads < 0 || d < 0)
        return fail(HALO_ERR_SHAPE, "negative size: B=%d H=%d W=%d C=%d C_out=%d heads=%d d=%d",
                    B, H, W, C, Cout, heads, d);
    if (C > 65536 || Cout > 65536 || (int64_t)heads * d > 4096)
        return fail(HALO_ERR_SHAPE, "channels out of range: C=%d C_out=%d heads*d=%lld (limits 65536, 4096)",
                    C, Cout, (long long)heads * d);
    if (stride < 1 || H % stride || W % stride)
        return fail(HALO_ERR_SHAPE, "query_stride=%d must be >= 1 and divide H=%d, W=%d", stride, H, W);
    L = halo::LayerGeom{};
    L.B = B; L.H = H; L.W = W; L.Ho = H / stride; L.Wo = W / stride;
    L.C = C; L.Cout = Cout; L.heads = heads; L.d = d; L.layout = layout;
    L.side = side; L.side_out = side;
    empty = B == 0 || H == 0 || W == 0 || C == 0 || Cout == 0 || heads == 0 || d == 0;
    if (layout == HALO_LAYOUT_BLOCKED) {
        if (side < 1) return fail(HALO_ERR_SHAPE, "the blocked layout needs block >= 1 (got %d)", side);
        if (H % side || W % side)
            return fail(HALO_ERR_SHAPE, "the blocked layout needs block=%d to divide H=%d and W=%d", side, H, W);
    }
    const double big = (double)B * H * W * std::max(std::max(C, Cout), heads * d);
    if (big >= 1e15) return fail(HALO_ERR_SHAPE, "tensor too large (%.3g elements)", big);
    L.NP = (int64_t)B * H * W;
    L.NPo = (int64_t)B * L.Ho * L.Wo;
    return HALO_OK;
}

}  // namespace

extern "C" {

int halo_attn_layer_proj_in(const void* x, const void* w_q, const void* w_kv, void* q, void* k, void* v,
                            int B, int H, int W, int C, int heads, int d, int block, int layout, int dtype,
                            void* stream)
{
    g_err[0] = 0;
    halo::LayerGeom L;
    bool empty = false;
    int st = check_layer(B, H, W, C, C, heads, d, layout == HALO_LAYOUT_BLOCKED ? block : 1, 1, layout, dtype, L,
                         empty);
    if (st) return st;
    if (empty) return HALO_OK;
    if (!x || !w_q || !w_kv || !q || !k || !v) return fail(HALO_ERR_NULL, "null pointer among x, w_q, w_kv, q, k, v");
    const size_t esz = dtype == HALO_BF16 ? 2 : 4;
    const size_t inner = (size_t)heads * d;
    const size_t xb = (size_t)L.NP * C * esz, wqb = inner * C * esz, wkvb = 2 * inner * C * esz;
    const size_t ob = (size_t)L.NP * inner * esz;
    const void* outs[3] = {q, k, v};
    for (int i = 0; i < 3; ++i) {
        if (overlaps(outs[i], ob, x, xb) || overlaps(outs[i], ob, w_q, wqb) || overlaps(outs[i], ob, w_kv, wkvb))
            return fail(HALO_ERR_ALIAS, "q, k or v overlaps an input");
        for (int j = 0; j < i; ++j)
            if (overlaps(outs[i], ob, outs[j], ob)) return fail(HALO_ERR_ALIAS, "q, k and v overlap each other");
    }
    const bool bf16 = dtype == HALO_BF16;
    const bool mfma = halo::proj_in_mfma_supported(L, bf16) && aligned16(x) && aligned16(w_q) && aligned16(w_kv) &&
                      aligned16(q) && aligned16(k) && aligned16(v);
    const hipError_t e = halo::launch_proj_in(x, w_q, w_kv, q, k, v, L, bf16, mfma, (hipStream_t)stream);
    if (e != hipSuccess) return fail(HALO_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return HALO_OK;
}

int halo_attn_layer_proj_out(const void* attn, const void* w_o, const void* b_o, void* y,
                             int B, int Ho, int Wo, int C_out, int heads, int d, int block_out, int layout, int dtype,
                             void* stream)
{
    g_err[0] = 0;
    halo::LayerGeom L;
    bool empty = false;
    // the output grid is the layer geometry at stride 1 (Ho x Wo pixels)
    int st = check_layer(B, Ho, Wo, C_out, C_out, heads, d, layout == HALO_LAYOUT_BLOCKED ? block_out : 1, 1, layout,
                         dtype, L, empty);
    if (st) return st;
    if (empty) return HALO_OK;
    if (!attn || !w_o || !b_o || !y) return fail(HALO_ERR_NULL, "null pointer among attn, w_o, b_o, y");
    const size_t esz = dtype == HALO_BF16 ? 2 : 4;
    const size_t inner = (size_t)heads * d;
    const size_t ab = (size_t)L.NPo * inner * esz, wb = (size_t)C_out * inner * esz, bb = (size_t)C_out * esz;
    const size_t yb = (size_t)L.NPo * C_out * esz;
    if (overlaps(y, yb, attn, ab) || overlaps(y, yb, w_o, wb) || overlaps(y, yb, b_o, bb))
        return fail(HALO_ERR_ALIAS, "y overlaps an input");
    const bool bf16 = dtype == HALO_BF16;
    const bool mfma = halo::proj_out_mfma_supported(L, bf16) && aligned16(attn) && aligned16(w_o) &&
                      aligned16(b_o) && aligned16(y);
    const hipError_t e = halo::launch_proj_out(attn, w_o, b_o, y, L, bf16, mfma, (hipStream_t)stream);
    if (e != hipSuccess) return fail(HALO_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return HALO_OK;
}

long long halo_attn_layer_workspace_bytes(int B, int H, int W, int heads, int d, int query_stride, int dtype)
{
    g_err[0] = 0;
    halo::LayerGeom L;
    bool empty = false;
    int st = check_layer(B, H, W, 1, 1, heads, d, 1, query_stride, HALO_LAYOUT_NHWC, dtype, L, empty);
    if (st) return st;
    if (empty) return 0;
    const size_t esz = dtype == HALO_BF16 ? 2 : 4;
    const size_t qkv = align256((size_t)L.NP * heads * d * esz);
    return (long long)(3 * qkv + align256((size_t)L.NPo * heads * d * esz));
}

int halo_attn_layer_fwd_ex(const void* x, const void* w_q, const void* w_kv, const void* w_o, const void* b_o,
                           const void* rel_h, const void* rel_w, void* y, void* workspace, size_t workspace_bytes,
                           int B, int H, int W, int C, int C_out, int heads, int d, int block, int halo,
                           int query_stride, float scale, int layout, int dtype, int kernel, void* stream)
{
    g_err[0] = 0;
    if (kernel != HALO_LAYER_KERNEL_AUTO && kernel != HALO_LAYER_KERNEL_FUSED && kernel != HALO_LAYER_KERNEL_SPLIT)
        return fail(HALO_ERR_SHAPE, "kernel=%d is not a halo_layer_kernel value", kernel);
    halo::LayerGeom L;
    bool empty = false;
    if (block < 1) return fail(HALO_ERR_SHAPE, "block=%d must be >= 1", block);
    if (query_stride < 1 || block % query_stride)
        return fail(HALO_ERR_SHAPE, "query_stride=%d must be >= 1 and divide block=%d", query_stride, block);
    int st = check_layer(B, H, W, C, C_out, heads, d, block, query_stride, layout, dtype, L, empty);
    if (st) return st;
    L.side_out = block / query_stride;
    {   // the attention's own checks, before any launch
        halo::Geometry g;
        bool e2 = false;
        st = check_sizes(B, heads, H, W, d, block, halo, query_stride, scale, dtype, g, e2);
        if (st) return st;
    }
    if (empty) return HALO_OK;
    if (!x || !w_q || !w_kv || !w_o || !b_o || !rel_h || !rel_w || !y)
        return fail(HALO_ERR_NULL, "null pointer among x, w_q, w_kv, w_o, b_o, rel_h, rel_w, y");
    const size_t esz = dtype == HALO_BF16 ? 2 : 4;
    const size_t inner = (size_t)heads * d;
    const int r = block + 2 * halo;
    const size_t xb = (size_t)L.NP * C * esz, yb = (size_t)L.NPo * C_out * esz;
    const size_t wqb = inner * C * esz, wkvb = 2 * inner * C * esz, wob = (size_t)C_out * inner * esz,
                 bb = (size_t)C_out * esz, tb = (size_t)(2 * r - 1) * d * esz;
    const void* ins[7] = {x, w_q, w_kv, w_o, b_o, rel_h, rel_w};
    const size_t insz[7] = {xb, wqb, wkvb, wob, bb, tb, tb};
    for (int i = 0; i < 7; ++i)
        if (overlaps(y, yb, ins[i], insz[i])) return fail(HALO_ERR_ALIAS, "y overlaps an input");

    const bool bf16 = dtype == HALO_BF16;
    hipStream_t s = (hipStream_t)stream;
    const bool fused_ok = halo::layer_fused_supported(L, block, halo, query_stride, bf16) && aligned16(x) &&
                          aligned16(w_q) && aligned16(w_kv) && aligned8(w_o) && aligned8(b_o) && aligned8(rel_h) &&
                          aligned8(rel_w) && aligned8(y);
    if (kernel == HALO_LAYER_KERNEL_FUSED && !fused_ok)
        return fail(HALO_ERR_UNSUPPORTED, "the fused layer kernel does not take these arguments");
    if (kernel == HALO_LAYER_KERNEL_FUSED || (kernel == HALO_LAYER_KERNEL_AUTO && fused_ok &&
                                              halo::layer_fused_preferred(L, block, halo, query_stride))) {
        const hipError_t e = halo::launch_layer_fused(x, w_q, w_kv, w_o, b_o, rel_h, rel_w, y, L, block, halo,
                                                      scale, s);
        if (e != hipSuccess) return fail(HALO_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
        return HALO_OK;
    }

    // the split path: q, k, v and the attention output in the workspace
    if (!workspace) return fail(HALO_ERR_NULL, "null workspace");
    const size_t qkv = align256((size_t)L.NP * inner * esz), ab = align256((size_t)L.NPo * inner * esz);
    const size_t need = 3 * qkv + ab;
    if (workspace_bytes < need || ((uintptr_t)workspace & 255u))
        return fail(HALO_ERR_WORKSPACE, "workspace of %zu bytes at %p: need %zu bytes, 256-byte aligned",
                    workspace_bytes, workspace, need);
    for (int i = 0; i < 7; ++i)
        if (overlaps(workspace, need, ins[i], insz[i])) return fail(HALO_ERR_ALIAS, "workspace overlaps an input");
    if (overlaps(workspace, need, y, yb)) return fail(HALO_ERR_ALIAS, "workspace overlaps y");
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    void *q = ws, *k = ws + qkv, *v = ws + 2 * qkv, *attn = ws + 3 * qkv;
    const bool mi = halo::proj_in_mfma_supported(L, bf16) && aligned16(x) && aligned16(w_q) && aligned16(w_kv);
    hipError_t e = halo::launch_proj_in(x, w_q, w_kv, q, k, v, L, bf16, mi, s);
    if (e != hipSuccess) return fail(HALO_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    st = halo_attn_fwd_ex(q, k, v, rel_h, rel_w, attn, nullptr, B, heads, H, W, d, block, halo, query_stride, scale,
                          dtype, 0, HALO_KERNEL_AUTO, stream);
    if (st) return st;
    const bool mo = halo::proj_out_mfma_supported(L, bf16) && aligned16(w_o) && aligned16(b_o) && aligned16(y);
    e = halo::launch_proj_out(attn, w_o, b_o, y, L, bf16, mo, s);
    if (e != hipSuccess) return fail(HALO_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return HALO_OK;
}

int halo_attn_layer_fwd(const void* x, const void* w_q, const void* w_kv, const void* w_o, const void* b_o,
                        const void* rel_h, const void* rel_w, void* y, void* workspace, size_t workspace_bytes,
                        int B, int H, int W, int C, int C_out, int heads, int d, int block, int halo,
                        int query_stride, float scale, int layout, int dtype, void* stream)
{
    return halo_attn_layer_fwd_ex(x, w_q, w_kv, w_o, b_o, rel_h, rel_w, y, workspace, workspace_bytes, B, H, W, C,
                                  C_out, heads, d, block, halo, query_stride, scale, layout, dtype,
                                  HALO_LAYER_KERNEL_AUTO, stream);
}

const char* halo_attn_layer_kernel_name(int B, int H, int W, int C, int C_out, int heads, int d, int block, int halo,
                                        int query_stride, int layout, int dtype, int kernel)
{
    g_err[0] = 0;
    if (kernel != HALO_LAYER_KERNEL_AUTO && kernel != HALO_LAYER_KERNEL_FUSED && kernel != HALO_LAYER_KERNEL_SPLIT) {
        fail(HALO_ERR_SHAPE, "kernel=%d is not a halo_layer_kernel value", kernel);
        return nullptr;
    }
    halo::LayerGeom L;
    bool empty = false;
    if (block < 1) {
        fail(HALO_ERR_SHAPE, "block=%d must be >= 1", block);
        return nullptr;
    }
    if (query_stride < 1 || block % query_stride) {
        fail(HALO_ERR_SHAPE, "query_stride=%d must be >= 1 and divide block=%d", query_stride, block);
        return nullptr;
    }
    if (check_layer(B, H, W, C, C_out, heads, d, block, query_stride, layout, dtype, L, empty)) return nullptr;
    {
        halo::Geometry g;
        bool e2 = false;
        if (check_sizes(B, heads, H, W, d, block, halo, query_stride, 1.0f, dtype, g, e2)) return nullptr;
    }
    if (empty) return "none";
    const bool ok = halo::layer_fused_supported(L, block, halo, query_stride, dtype == HALO_BF16);
    if (kernel == HALO_LAYER_KERNEL_FUSED && !ok) {
        fail(HALO_ERR_UNSUPPORTED, "the fused layer kernel does not take these arguments");
        return nullptr;
    }
    if (kernel == HALO_LAYER_KERNEL_SPLIT) return "split";
    if (kernel == HALO_LAYER_KERNEL_FUSED) return "fused";
    return ok && halo::layer_fused_preferred(L, block, halo, query_stride) ? "fused" : "split";
}

}  // extern "C"
