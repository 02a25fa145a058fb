// C ABI of the halo-attention library: argument checks, kernel choice, launch.
// The operation and every convention are documented in include/halo_attn.h.
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/halo_attn.h"
#include "halo_common.h"

namespace halo {
hipError_t launch_generic(const void* q, const void* k, const void* v, const void* rh,
                          const void* rw, void* out, const Geometry& g, bool bf16, hipStream_t st);
bool mfma_supported(int d, int r, int block, int stride, bool bf16);
hipError_t launch_mfma(const void* q, const void* k, const void* v, const void* rh,
                       const void* rw, void* out, const Geometry& g, bool force_strip, hipStream_t st);
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

int halo_attn_select_kernel(int d, int block, int halo, int query_stride, int dtype)
{
    g_err[0] = 0;
    const int st = check_config(d, block, halo, query_stride, dtype);
    if (st) return st;
    return halo::mfma_supported(d, block + 2 * halo, block, query_stride, dtype == HALO_BF16)
               ? HALO_KERNEL_MFMA : HALO_KERNEL_GENERIC;
}

int halo_attn_fwd_kernel(const void* q, const void* k, const void* v,
                         const void* rel_h, const void* rel_w, void* out,
                         int B, int heads, int H, int W, int d,
                         int block, int halo, int query_stride,
                         float scale, int dtype, int kernel, void* stream)
{
    g_err[0] = 0;
    int st = check_config(d, block, halo, query_stride, dtype);
    if (st) return st;
    if (kernel != HALO_KERNEL_AUTO && kernel != HALO_KERNEL_GENERIC && kernel != HALO_KERNEL_MFMA &&
        kernel != HALO_KERNEL_MFMA_STRIP)
        return fail(HALO_ERR_SHAPE, "kernel=%d is not a halo_kernel value", kernel);
    if (B < 0 || heads < 0 || H < 0 || W < 0)
        return fail(HALO_ERR_SHAPE, "negative size: B=%d heads=%d H=%d W=%d", B, heads, H, W);
    if (H % query_stride || W % query_stride)
        return fail(HALO_ERR_SHAPE, "query_stride=%d must divide H=%d and W=%d", query_stride, H, W);
    if (!std::isfinite(scale)) return fail(HALO_ERR_SHAPE, "scale must be finite");
    if (B == 0 || heads == 0 || H == 0 || W == 0) return HALO_OK;   // empty: nothing to do

    // magnitude checks in double first, so the int64 products below cannot overflow
    const double nelem = (double)B * heads * H * W * d;
    const int nbh = (H + block - 1) / block, nbw = (W + block - 1) / block;
    const double nblk = (double)B * heads * nbh * nbw;
    if (nelem >= 1e18)
        return fail(HALO_ERR_SHAPE, "tensor too large (%.3g elements, limit 1e18)", nelem);
    if (nblk >= 2147483648.0)
        return fail(HALO_ERR_SHAPE, "%.0f blocks exceed the 2^31 grid limit", nblk);
    const int64_t BH = (int64_t)B * heads;
    const int64_t elems = BH * H * W * d;

    if (!q || !k || !v || !rel_h || !rel_w || !out)
        return fail(HALO_ERR_NULL, "null pointer among q, k, v, rel_h, rel_w, out");

    const int r = block + 2 * halo;
    const size_t esz = dtype == HALO_BF16 ? 2 : 4;
    const size_t in_bytes = (size_t)elems * esz;
    const size_t tab_bytes = (size_t)(2 * r - 1) * d * esz;
    const int Ho = H / query_stride, Wo = W / query_stride;
    const size_t out_bytes = (size_t)(BH * Ho * Wo * d) * esz;
    if (overlaps(out, out_bytes, q, in_bytes) || overlaps(out, out_bytes, k, in_bytes) ||
        overlaps(out, out_bytes, v, in_bytes) || overlaps(out, out_bytes, rel_h, tab_bytes) ||
        overlaps(out, out_bytes, rel_w, tab_bytes))
        return fail(HALO_ERR_ALIAS, "out overlaps an input tensor");

    const bool bf16 = dtype == HALO_BF16;
    const bool mfma_ok = halo::mfma_supported(d, r, block, query_stride, bf16);
    if ((kernel == HALO_KERNEL_MFMA || kernel == HALO_KERNEL_MFMA_STRIP) && !mfma_ok)
        return fail(HALO_ERR_UNSUPPORTED,
                    "matrix-core kernel needs bf16, d in {16,32}, window side <= 32 "
                    "(got dtype=%d d=%d r=%d)", dtype, d, r);

    halo::Geometry g;
    g.BH = BH; g.H = H; g.W = W; g.d = d;
    g.block = block; g.halo = halo; g.stride = query_stride;
    g.r = r; g.c0 = r - 1 + halo; g.Ho = Ho; g.Wo = Wo;
    g.nbh = nbh; g.nbw = nbw; g.scale = scale;

    hipStream_t s = (hipStream_t)stream;
    const bool use_mfma = kernel == HALO_KERNEL_MFMA || kernel == HALO_KERNEL_MFMA_STRIP ||
                          (kernel == HALO_KERNEL_AUTO && mfma_ok);
    const hipError_t e = use_mfma ? halo::launch_mfma(q, k, v, rel_h, rel_w, out, g,
                                                      kernel == HALO_KERNEL_MFMA_STRIP, s)
                                  : halo::launch_generic(q, k, v, rel_h, rel_w, out, g, bf16, s);
    if (e != hipSuccess)
        return fail(HALO_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return HALO_OK;
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

}  // extern "C"
