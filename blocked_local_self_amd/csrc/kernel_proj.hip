// The attention layer's projections around the blocked attention, fused with
// the layout changes (gfx950 matrix cores for bf16, a plain kernel otherwise).
//
// The layer is the HaloAttention module of the pswp.cn blog page (section 4):
// to_q and to_kv are linear maps without bias applied to every pixel (to_kv's
// output is k then v), heads are split off the channel axis (channel
// h*d + c is channel c of head h), and after the attention the heads are
// merged the same way and to_out (a linear map with bias) is applied.
// "Scaling Local Self-Attention for Parameter Efficient Visual Backbones",
// appendix D, keeps activations blocked for the whole network and avoids
// reshapes and formatting operations; here the activations stay pixel-major
// with channels last, in image order (NHWC) or in the blocked order of that
// appendix, and the projections read and write the attention's
// [B, heads, H, W, d] tensors directly: the head split and merge and the
// (un)blocking are index arithmetic in the GEMM prologue / epilogue, never a
// separate pass over memory.
//
// Matrix-core GEMMs: one workgroup holds a slice of the weight rows in LDS
// and streams a chunk of pixels.  A wave takes 32 pixels at a time; their
// channels are the B operand (lane n: pixel n, 8 consecutive channels), the
// weight rows the A operand, so lane (n, g) of the 16x16 result holds four
// consecutive output channels of pixel n: one 8-byte store, and a 16x16 tile
// is 16 pixels x 32 contiguous bytes of one head.
#include <algorithm>

#include "mfma_util.h"
#include "proj.h"

namespace halo {

// layer-order pixel p -> image coordinates (b, y, x) of a B x H x W grid
__device__ inline void layer_pixel(int64_t p, const LayerGeom& L, int H, int W, int side, int64_t& b, int& y, int& x)
{
    if (L.layout == 0) {                    // NHWC
        const int64_t row = p / W;
        x = (int)(p - row * W);
        b = row / H;
        y = (int)(row - b * H);
    } else {                                // blocked: [B, H/s, W/s, s*s]
        const int bb = side * side;
        const int64_t blk = p / bb;
        const int in = (int)(p - blk * bb);
        const int p1 = in / side, p2 = in - p1 * side;
        const int nbx = W / side, nby = H / side;
        const int64_t t = blk / nbx;
        const int j = (int)(blk - t * nbx);
        b = t / nby;
        const int i = (int)(t - b * nby);
        y = i * side + p1;
        x = j * side + p2;
    }
}

template <int KCMAX>
__global__ __launch_bounds__(256)
void proj_in_kernel(const __bf16* __restrict__ x, const __bf16* __restrict__ w_q, const __bf16* __restrict__ w_kv,
                    __bf16* __restrict__ q, __bf16* __restrict__ k, __bf16* __restrict__ v, LayerGeom L, ProjPlan p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int C = L.C, kc = C / 32, inner = L.heads * L.d;

    int64_t wg = blockIdx.x;
    if (p.remap_xcd) {
        const int64_t per = p.nwg >> 3;
        wg = (wg & 7) * per + (wg >> 3);
    }
    const int slice = (int)(wg % p.nslices);
    const int64_t chunk = wg / p.nslices;
    const int o0 = slice * p.ns;
    const int ns = min(p.ns, 3 * inner - o0);          // multiple of 16
    const unsigned pitch = (unsigned)p.pitch * 2;        // bytes per LDS weight row

    // weight rows o0 .. o0+ns-1 of [w_q; w_kv]
    for (int e = tid; e < ns * (C / 8); e += 256) {
        const int row = e / (C / 8), ch = e - row * (C / 8);
        const int o = o0 + row;
        const __bf16* src = o < inner ? w_q + (int64_t)o * C : w_kv + (int64_t)(o - inner) * C;
        *reinterpret_cast<u32x4*>(smem + row * pitch + ch * 16) = *reinterpret_cast<const u32x4*>(src + ch * 8);
    }
    __syncthreads();

    const int64_t HW = (int64_t)L.H * L.W;
    const int64_t pwave = chunk * p.chunk + (int64_t)wave * (p.chunk / 4);
    for (int pp = 0; pp < p.chunk / 4; pp += 32) {
        s16x8 bfr[2][KCMAX];
        int64_t dst0[2];
        bool valid[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int64_t pix = pwave + pp + 16 * tt + n;
            valid[tt] = pix < L.NP;
            const int64_t pc = valid[tt] ? pix : L.NP - 1;
#pragma unroll
            for (int ks = 0; ks < KCMAX; ++ks)
                if (ks < kc) bfr[tt][ks] = *reinterpret_cast<const s16x8*>(x + pc * C + 32 * ks + 8 * g);
            int64_t b;
            int yy, xx;
            layer_pixel(pc, L, L.H, L.W, L.side, b, yy, xx);
            dst0[tt] = ((b * L.heads) * HW + (int64_t)yy * L.W + xx) * L.d;   // head 0, channel 0
        }
        for (int ot = 0; ot < ns / 16; ++ot) {
            f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
            const unsigned arow = (unsigned)(16 * ot + n) * pitch + 16u * g;
#pragma unroll
            for (int ks = 0; ks < KCMAX; ++ks)
                if (ks < kc) {
                    const s16x8 a = *reinterpret_cast<const s16x8*>(smem + arow + 64u * ks);
                    acc[0] = mma_k32(a, bfr[0][ks], acc[0]);
                    acc[1] = mma_k32(a, bfr[1][ks], acc[1]);
                }
            // lane (n, g): outputs o .. o+3 of pixel n (one tensor, one head)
            const int o = o0 + 16 * ot + 4 * g;
            const int t = o / inner, oi = o - t * inner;
            const int head = oi / L.d, c = oi - head * L.d;
            __bf16* dst = t == 0 ? q : (t == 1 ? k : v);
            const int64_t off = (int64_t)head * HW * L.d + c;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                if (valid[tt])
                    *reinterpret_cast<u32x2*>(dst + dst0[tt] + off) =
                        u32x2{pack_bf16x2(acc[tt][0], acc[tt][1]), pack_bf16x2(acc[tt][2], acc[tt][3])};
        }
    }
}

template <int KCMAX>
__global__ __launch_bounds__(256)
void proj_out_kernel(const __bf16* __restrict__ attn, const __bf16* __restrict__ w_o, const __bf16* __restrict__ b_o,
                     __bf16* __restrict__ y, LayerGeom L, ProjPlan p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int inner = L.heads * L.d, kc = inner / 32, Co = L.Cout;

    int64_t wg = blockIdx.x;
    if (p.remap_xcd) {
        const int64_t per = p.nwg >> 3;
        wg = (wg & 7) * per + (wg >> 3);
    }
    const int slice = (int)(wg % p.nslices);
    const int64_t chunk = wg / p.nslices;
    const int o0 = slice * p.ns;
    const int ns = min(p.ns, Co - o0);                   // multiple of 16
    const unsigned pitch = (unsigned)p.pitch * 2;

    for (int e = tid; e < ns * (inner / 8); e += 256) {
        const int row = e / (inner / 8), ch = e - row * (inner / 8);
        *reinterpret_cast<u32x4*>(smem + row * pitch + ch * 16) =
            *reinterpret_cast<const u32x4*>(w_o + (int64_t)(o0 + row) * inner + ch * 8);
    }
    __syncthreads();

    const int64_t HWo = (int64_t)L.Ho * L.Wo;
    const int64_t pwave = chunk * p.chunk + (int64_t)wave * (p.chunk / 4);
    for (int pp = 0; pp < p.chunk / 4; pp += 32) {
        s16x8 bfr[2][KCMAX];
        int64_t pixo[2];
        bool valid[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int64_t pix = pwave + pp + 16 * tt + n;
            valid[tt] = pix < L.NPo;
            const int64_t pc = valid[tt] ? pix : L.NPo - 1;
            pixo[tt] = pc;
            int64_t b;
            int yy, xx;
            layer_pixel(pc, L, L.Ho, L.Wo, L.side_out, b, yy, xx);
            const __bf16* src = attn + ((b * L.heads) * HWo + (int64_t)yy * L.Wo + xx) * L.d;
            // merged channel kk = 32 ks + 8 g + j is channel kk % d of head kk / d
#pragma unroll
            for (int ks = 0; ks < KCMAX; ++ks)
                if (ks < kc) {
                    const int kk = 32 * ks + 8 * g, head = kk / L.d, c = kk - head * L.d;
                    bfr[tt][ks] = *reinterpret_cast<const s16x8*>(src + (int64_t)head * HWo * L.d + c);
                }
        }
        for (int ot = 0; ot < ns / 16; ++ot) {
            f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
            const unsigned arow = (unsigned)(16 * ot + n) * pitch + 16u * g;
#pragma unroll
            for (int ks = 0; ks < KCMAX; ++ks)
                if (ks < kc) {
                    const s16x8 a = *reinterpret_cast<const s16x8*>(smem + arow + 64u * ks);
                    acc[0] = mma_k32(a, bfr[0][ks], acc[0]);
                    acc[1] = mma_k32(a, bfr[1][ks], acc[1]);
                }
            const int o = o0 + 16 * ot + 4 * g;
            const u32x2 bb = *reinterpret_cast<const u32x2*>(b_o + o);
            const float b0 = __builtin_bit_cast(float, bb[0] << 16), b1 = __builtin_bit_cast(float, bb[0] & 0xffff0000u);
            const float b2 = __builtin_bit_cast(float, bb[1] << 16), b3 = __builtin_bit_cast(float, bb[1] & 0xffff0000u);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                if (valid[tt])
                    *reinterpret_cast<u32x2*>(y + pixo[tt] * Co + o) =
                        u32x2{pack_bf16x2(acc[tt][0] + b0, acc[tt][1] + b1), pack_bf16x2(acc[tt][2] + b2, acc[tt][3] + b3)};
        }
    }
}

// Plain kernels (fp32, and shapes the matrix-core ones do not take): one
// thread per (pixel, output channel), fp32 accumulation in channel order.
template <typename T>
__global__ __launch_bounds__(256)
void proj_in_generic(const T* __restrict__ x, const T* __restrict__ w_q, const T* __restrict__ w_kv,
                     T* __restrict__ q, T* __restrict__ k, T* __restrict__ v, LayerGeom L)
{
    const int inner = L.heads * L.d, no = 3 * inner;
    const int64_t HW = (int64_t)L.H * L.W;
    const int64_t total = L.NP * no;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t pix = i / no;
        const int o = (int)(i - pix * no);
        const T* w = o < inner ? w_q + (int64_t)o * L.C : w_kv + (int64_t)(o - inner) * L.C;
        const T* xr = x + pix * L.C;
        float acc = 0.f;
        for (int c = 0; c < L.C; ++c) acc = fmaf(to_f32(xr[c]), to_f32(w[c]), acc);
        int64_t b;
        int yy, xx;
        layer_pixel(pix, L, L.H, L.W, L.side, b, yy, xx);
        const int t = o / inner, oi = o - t * inner, head = oi / L.d, c = oi - head * L.d;
        T* dst = t == 0 ? q : (t == 1 ? k : v);
        dst[((b * L.heads + head) * HW + (int64_t)yy * L.W + xx) * L.d + c] = from_f32<T>(acc);
    }
}

template <typename T>
__global__ __launch_bounds__(256)
void proj_out_generic(const T* __restrict__ attn, const T* __restrict__ w_o, const T* __restrict__ b_o,
                      T* __restrict__ y, LayerGeom L)
{
    const int inner = L.heads * L.d, Co = L.Cout;
    const int64_t HWo = (int64_t)L.Ho * L.Wo;
    const int64_t total = L.NPo * Co;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t pix = i / Co;
        const int o = (int)(i - pix * Co);
        int64_t b;
        int yy, xx;
        layer_pixel(pix, L, L.Ho, L.Wo, L.side_out, b, yy, xx);
        const T* w = w_o + (int64_t)o * inner;
        float acc = 0.f;
        for (int kk = 0; kk < inner; ++kk) {
            const int head = kk / L.d, c = kk - head * L.d;
            acc = fmaf(to_f32(attn[((b * L.heads + head) * HWo + (int64_t)yy * L.Wo + xx) * L.d + c]), to_f32(w[kk]), acc);
        }
        y[pix * Co + o] = from_f32<T>(acc + to_f32(b_o[o]));
    }
}

bool proj_in_mfma_supported(const LayerGeom& L, bool bf16)
{
    const int inner = L.heads * L.d;
    return bf16 && L.C % 32 == 0 && L.C <= 512 && L.d % 4 == 0 && inner % 16 == 0;
}

bool proj_out_mfma_supported(const LayerGeom& L, bool bf16)
{
    const int inner = L.heads * L.d;
    return bf16 && inner % 32 == 0 && inner <= 512 && L.d % 8 == 0 && L.Cout % 16 == 0;
}

// Weight rows per workgroup: as many 16-row tiles as fit 64 KiB of LDS.
static ProjPlan proj_plan(int nout, int kdim, int64_t npix)
{
    ProjPlan p{};
    p.pitch = kdim + 8;                                // 16 bytes of padding per row
    const int rows_fit = std::max(16, (64 * 1024 / (p.pitch * 2)) / 16 * 16);
    p.ns = std::min(rows_fit, (nout + 15) / 16 * 16);
    p.nslices = (nout + p.ns - 1) / p.ns;
    p.chunk = 256;                                     // pixels per workgroup: 4 waves x 2 passes x 32
    const int64_t nchunks = (npix + p.chunk - 1) / p.chunk;
    p.nwg = nchunks * p.nslices;
    p.remap_xcd = p.nwg % 8 == 0 ? 1 : 0;
    p.lds_bytes = p.ns * p.pitch * 2;
    return p;
}

static int64_t grid_for(int64_t total)
{
    return std::max<int64_t>(1, std::min<int64_t>((total + 255) / 256, 1 << 20));
}

hipError_t launch_proj_in(const void* x, const void* w_q, const void* w_kv, void* q, void* k, void* v,
                          const LayerGeom& L, bool bf16, bool mfma, hipStream_t st)
{
    if (mfma) {
        const ProjPlan p = proj_plan(3 * L.heads * L.d, L.C, L.NP);
        auto kern = L.C <= 128 ? proj_in_kernel<4> : proj_in_kernel<16>;
        const hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), p.lds_bytes);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)p.nwg), dim3(256), p.lds_bytes, st, (const __bf16*)x,
                           (const __bf16*)w_q, (const __bf16*)w_kv, (__bf16*)q, (__bf16*)k, (__bf16*)v, L, p);
    } else {
        const int64_t blocks = grid_for(L.NP * 3 * L.heads * L.d);
        if (bf16)
            hipLaunchKernelGGL(proj_in_generic<__bf16>, dim3((unsigned)blocks), dim3(256), 0, st, (const __bf16*)x,
                               (const __bf16*)w_q, (const __bf16*)w_kv, (__bf16*)q, (__bf16*)k, (__bf16*)v, L);
        else
            hipLaunchKernelGGL(proj_in_generic<float>, dim3((unsigned)blocks), dim3(256), 0, st, (const float*)x,
                               (const float*)w_q, (const float*)w_kv, (float*)q, (float*)k, (float*)v, L);
    }
    return hipGetLastError();
}

hipError_t launch_proj_out(const void* attn, const void* w_o, const void* b_o, void* y, const LayerGeom& L, bool bf16,
                           bool mfma, hipStream_t st)
{
    if (mfma) {
        const ProjPlan p = proj_plan(L.Cout, L.heads * L.d, L.NPo);
        auto kern = L.heads * L.d <= 128 ? proj_out_kernel<4> : proj_out_kernel<16>;
        const hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), p.lds_bytes);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)p.nwg), dim3(256), p.lds_bytes, st, (const __bf16*)attn,
                           (const __bf16*)w_o, (const __bf16*)b_o, (__bf16*)y, L, p);
    } else {
        const int64_t blocks = grid_for(L.NPo * L.Cout);
        if (bf16)
            hipLaunchKernelGGL(proj_out_generic<__bf16>, dim3((unsigned)blocks), dim3(256), 0, st, (const __bf16*)attn,
                               (const __bf16*)w_o, (const __bf16*)b_o, (__bf16*)y, L);
        else
            hipLaunchKernelGGL(proj_out_generic<float>, dim3((unsigned)blocks), dim3(256), 0, st, (const float*)attn,
                               (const float*)w_o, (const float*)b_o, (float*)y, L);
    }
    return hipGetLastError();
}

}  // namespace halo
