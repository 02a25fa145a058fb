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
#include <type_traits>

#include "mfma_util.h"
#include "proj.h"

namespace halo {

// layer-order pixel p -> image coordinates (b, y, x) of a B x H x W grid
// (out: the output grid), 32-bit with the precomputed dividers
__device__ inline void layer_pixel(uint32_t p, const LayerGeom& L, bool out, uint32_t& b, uint32_t& y, uint32_t& x)
{
    if (L.layout == 0) {                    // NHWC
        const FastDiv& fW = out ? L.fWo : L.fW;
        const FastDiv& fH = out ? L.fHo : L.fH;
        const uint32_t row = fW.div(p);
        x = p - row * fW.d;
        b = fH.div(row);
        y = row - b * fH.d;
    } else {                                // blocked: [B, H/s, W/s, s*s]
        const FastDiv& fbb = out ? L.fbbo : L.fbb;
        const FastDiv& fs = out ? L.fsideo : L.fside;
        const FastDiv& fnbx = out ? L.fnbxo : L.fnbx;
        const FastDiv& fnby = out ? L.fnbyo : L.fnby;
        const uint32_t blk = fbb.div(p);
        const uint32_t in = p - blk * fbb.d;
        const uint32_t p1 = fs.div(in), p2 = in - p1 * fs.d;
        const uint32_t t = fnbx.div(blk);
        const uint32_t j = blk - t * fnbx.d;
        b = fnby.div(t);
        const uint32_t i = t - b * fnby.d;
        y = i * fs.d + p1;
        x = j * fs.d + p2;
    }
}

// the same in 64-bit arithmetic (plain kernels, any size)
__device__ inline void layer_pixel64(int64_t p, const LayerGeom& L, int H, int W, int side, int64_t& b, int& y, int& x)
{
    if (L.layout == 0) {
        const int64_t row = p / W;
        x = (int)(p - row * W);
        b = row / H;
        y = (int)(row - b * H);
    } else {
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

void layer_fastdiv(LayerGeom& L)
{
    const int side = std::max(1, L.side), so = std::max(1, L.side_out);
    L.fW = FastDiv((uint32_t)std::max(1, L.W));
    L.fH = FastDiv((uint32_t)std::max(1, L.H));
    L.fWo = FastDiv((uint32_t)std::max(1, L.Wo));
    L.fHo = FastDiv((uint32_t)std::max(1, L.Ho));
    L.fbb = FastDiv((uint32_t)(side * side));
    L.fside = FastDiv((uint32_t)side);
    L.fnbx = FastDiv((uint32_t)std::max(1, L.W / side));
    L.fnby = FastDiv((uint32_t)std::max(1, L.H / side));
    L.fbbo = FastDiv((uint32_t)(so * so));
    L.fsideo = FastDiv((uint32_t)so);
    L.fnbxo = FastDiv((uint32_t)std::max(1, L.Wo / so));
    L.fnbyo = FastDiv((uint32_t)std::max(1, L.Ho / so));
    L.finner = FastDiv((uint32_t)std::max(1, L.heads * L.d));
    L.fd = FastDiv((uint32_t)std::max(1, L.d));
}

// rows 0..nrows-1 of kdim bf16 each (row r at src(r)) into LDS rows of
// `pitch` bytes, 16 bytes per item, eight items per thread in flight
template <typename Src>
__device__ inline void stage_rows(unsigned char* smem, unsigned pitch, int nrows, int kdim, int tid, Src src)
{
    constexpr int SB = 8;
    const int per_row = kdim / 8, total = nrows * per_row;
    for (int e0 = tid; e0 < total; e0 += 256 * SB) {
        u32x4 buf[SB];
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int e = e0 + 256 * j;
            if (e < total) {
                const int row = e / per_row, ch = e - row * per_row;
                buf[j] = *reinterpret_cast<const u32x4*>(src(row) + ch * 8);
            }
        }
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int e = e0 + 256 * j;
            if (e < total) {
                const int row = e / per_row, ch = e - row * per_row;
                *reinterpret_cast<u32x4*>(smem + row * pitch + ch * 16) = buf[j];
            }
        }
    }
}

// KCMAX: k-steps of 32 channels (the contraction length / 32), exact
template <int KCMAX>
__global__ __launch_bounds__(256)
void proj_in_kernel(const __bf16* __restrict__ x, const __bf16* __restrict__ w_q, const __bf16* __restrict__ w_kv,
                    __bf16* __restrict__ q, __bf16* __restrict__ k, __bf16* __restrict__ v, LayerGeom L, ProjPlan p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int C = L.C, inner = L.heads * L.d;

    int64_t wg = blockIdx.x;
    if (p.remap_xcd) {
        const int64_t per = p.nwg >> 3;
        wg = (wg & 7) * per + (wg >> 3);
    }
    // this workgroup's weight slice, and its share of the pixel chunks
    const int slice = (int)(wg % p.nslices);
    const int64_t g0 = wg / p.nslices, G = p.nwg / p.nslices;
    const int o0 = slice * p.ns;
    const int ns = min(p.ns, 3 * inner - o0);          // multiple of 16
    const unsigned pitch = (unsigned)p.pitch * 2;        // bytes per LDS weight row

    // weight rows o0 .. o0+ns-1 of [w_q; w_kv], staged once (loads issued
    // in batches, so their latencies overlap)
    stage_rows(smem, pitch, ns, C, tid, [&](int row) {
        const int o = o0 + row;
        return o < inner ? w_q + (int64_t)o * C : w_kv + (int64_t)(o - inner) * C;
    });
    __syncthreads();

    const int64_t HW = (int64_t)L.H * L.W;
    const int64_t nchunks = (L.NP + p.chunk - 1) / p.chunk;
    // passes of 32 pixels: pass i of this wave covers chunk g0 + (i/2)*G,
    // pixels wave*64 + (i%2)*32 .. +31 of it
    const int64_t npass = g0 < nchunks ? 2 * ((nchunks - 1 - g0) / G + 1) : 0;
    auto pass_pixel = [&](int64_t i) { return (g0 + (i >> 1) * G) * p.chunk + wave * (p.chunk / 4) + (i & 1) * 32; };
    auto load = [&](int64_t i, s16x8 (&f)[2][KCMAX]) {
        const int64_t pb = pass_pixel(i);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int64_t pix = min(pb + 16 * tt + n, L.NP - 1);
#pragma unroll
            for (int ks = 0; ks < KCMAX; ++ks)
                f[tt][ks] = *reinterpret_cast<const s16x8*>(x + pix * C + 32 * ks + 8 * g);
        }
    };
    s16x8 cur[2][KCMAX], nxt[2][KCMAX];
    if (npass > 0) load(0, cur);
    for (int64_t i = 0; i < npass; ++i) {
        if (i + 1 < npass) load(i + 1, nxt);             // in flight during this pass
        const int64_t pb = pass_pixel(i);
        int64_t dst0[2];
        bool valid[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int64_t pix = pb + 16 * tt + n;
            valid[tt] = pix < L.NP;
            uint32_t b, yy, xx;
            layer_pixel((uint32_t)(valid[tt] ? pix : L.NP - 1), L, false, b, yy, xx);
            dst0[tt] = ((int64_t)b * L.heads * HW + (int64_t)yy * L.W + xx) * L.d;   // head 0, channel 0
        }
        for (int ot = 0; ot < ns / 16; ++ot) {
            f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
            const unsigned arow = (unsigned)(16 * ot + n) * pitch + 16u * g;
#pragma unroll
            for (int ks = 0; ks < KCMAX; ++ks) {
                const s16x8 a = *reinterpret_cast<const s16x8*>(smem + arow + 64u * ks);
                acc[0] = mma_k32(a, cur[0][ks], acc[0]);
                acc[1] = mma_k32(a, cur[1][ks], acc[1]);
            }
            // lane (n, g): outputs o .. o+3 of pixel n (one tensor, one head)
            const int o = o0 + 16 * ot + 4 * g;
            const int t = (int)L.finner.div((uint32_t)o), oi = o - t * inner;
            const int head = (int)L.fd.div((uint32_t)oi), c = oi - head * L.d;
            __bf16* dst = t == 0 ? q : (t == 1 ? k : v);
            const int64_t off = (int64_t)head * HW * L.d + c;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                if (valid[tt])
                    *reinterpret_cast<u32x2*>(dst + dst0[tt] + off) =
                        u32x2{pack_bf16x2(acc[tt][0], acc[tt][1]), pack_bf16x2(acc[tt][2], acc[tt][3])};
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int ks = 0; ks < KCMAX; ++ks) cur[tt][ks] = nxt[tt][ks];
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
    const int inner = L.heads * L.d, Co = L.Cout;

    int64_t wg = blockIdx.x;
    if (p.remap_xcd) {
        const int64_t per = p.nwg >> 3;
        wg = (wg & 7) * per + (wg >> 3);
    }
    const int slice = (int)(wg % p.nslices);
    const int64_t g0 = wg / p.nslices, G = p.nwg / p.nslices;
    const int o0 = slice * p.ns;
    const int ns = min(p.ns, Co - o0);                   // multiple of 16
    const unsigned pitch = (unsigned)p.pitch * 2;
    // output staging (p.stage != 0): this wave's 32 x ns tile, row pitch spitch bytes
    const unsigned spitch = 2u * ns + 16u;
    const unsigned sbase = (unsigned)p.stage + (unsigned)wave * 32u * (2u * (unsigned)p.ns + 16u);
    const int cpr = ns / 8;                              // 16-byte chunks per row (divides 64)
    const int lrow = p.stage ? lane / cpr : 0, lchunk = p.stage ? lane - lrow * cpr : 0;
    const int rstep = p.stage ? 64 / cpr : 1;

    stage_rows(smem, pitch, ns, inner, tid, [&](int row) { return w_o + (int64_t)(o0 + row) * inner; });
    __syncthreads();

    const int64_t HWo = (int64_t)L.Ho * L.Wo;
    const int64_t nchunks = (L.NPo + p.chunk - 1) / p.chunk;
    const int64_t npass = g0 < nchunks ? 2 * ((nchunks - 1 - g0) / G + 1) : 0;
    auto pass_pixel = [&](int64_t i) { return (g0 + (i >> 1) * G) * p.chunk + wave * (p.chunk / 4) + (i & 1) * 32; };
    // merged channel kk = 32 ks + 8 g + j is channel kk % d of head kk / d
    auto load = [&](int64_t i, s16x8 (&f)[2][KCMAX]) {
        const int64_t pb = pass_pixel(i);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int64_t pix = min(pb + 16 * tt + n, L.NPo - 1);
            uint32_t b, yy, xx;
            layer_pixel((uint32_t)pix, L, true, b, yy, xx);
            const __bf16* src = attn + ((int64_t)b * L.heads * HWo + (int64_t)yy * L.Wo + xx) * L.d;
#pragma unroll
            for (int ks = 0; ks < KCMAX; ++ks) {
                const int kk = 32 * ks + 8 * g, head = (int)L.fd.div((uint32_t)kk), c = kk - head * L.d;
                f[tt][ks] = *reinterpret_cast<const s16x8*>(src + (int64_t)head * HWo * L.d + c);
            }
        }
    };
    s16x8 cur[2][KCMAX], nxt[2][KCMAX];
    if (npass > 0) load(0, cur);
    for (int64_t i = 0; i < npass; ++i) {
        if (i + 1 < npass) load(i + 1, nxt);             // in flight during this pass
        const int64_t pb = pass_pixel(i);
        for (int ot = 0; ot < ns / 16; ++ot) {
            f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
            const unsigned arow = (unsigned)(16 * ot + n) * pitch + 16u * g;
#pragma unroll
            for (int ks = 0; ks < KCMAX; ++ks) {
                const s16x8 a = *reinterpret_cast<const s16x8*>(smem + arow + 64u * ks);
                acc[0] = mma_k32(a, cur[0][ks], acc[0]);
                acc[1] = mma_k32(a, cur[1][ks], acc[1]);
            }
            const int o = o0 + 16 * ot + 4 * g;
            const u32x2 bb = *reinterpret_cast<const u32x2*>(b_o + o);
            const float b0 = __builtin_bit_cast(float, bb[0] << 16), b1 = __builtin_bit_cast(float, bb[0] & 0xffff0000u);
            const float b2 = __builtin_bit_cast(float, bb[1] << 16), b3 = __builtin_bit_cast(float, bb[1] & 0xffff0000u);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int64_t pix = pb + 16 * tt + n;
                const u32x2 w = u32x2{pack_bf16x2(acc[tt][0] + b0, acc[tt][1] + b1),
                                      pack_bf16x2(acc[tt][2] + b2, acc[tt][3] + b3)};
                if (p.stage)        // row 16 tt + n of the wave's tile, channels 16 ot + 4 g ..
                    *reinterpret_cast<u32x2*>(smem + sbase + (16 * tt + n) * spitch + 2u * (16 * ot + 4 * g)) = w;
                else if (pix < L.NPo)
                    *reinterpret_cast<u32x2*>(y + pix * Co + o) = w;
            }
        }
        if (p.stage) {
            // whole rows out: lane -> (row lrow + rstep * it, 16-byte chunk lchunk).
            // The tile was written by this wave; LDS runs one wave's accesses in order.
            for (int r = lrow; r < 32; r += rstep) {
                const int64_t pix = pb + r;
                if (pix < L.NPo)
                    *reinterpret_cast<u32x4*>(y + pix * Co + o0 + 8 * lchunk) =
                        *reinterpret_cast<const u32x4*>(smem + sbase + r * spitch + 16u * lchunk);
            }
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int ks = 0; ks < KCMAX; ++ks) cur[tt][ks] = nxt[tt][ks];
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
        layer_pixel64(pix, L, L.H, L.W, L.side, b, yy, xx);
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
        layer_pixel64(pix, L, L.Ho, L.Wo, L.side_out, b, yy, xx);
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
    return bf16 && L.NP < (int64_t(1) << 31) && L.C % 32 == 0 && L.C <= 512 && L.d % 4 == 0 && inner % 16 == 0;
}

bool proj_out_mfma_supported(const LayerGeom& L, bool bf16)
{
    const int inner = L.heads * L.d;
    return bf16 && L.NPo < (int64_t(1) << 31) && inner % 32 == 0 && inner <= 512 && L.d % 8 == 0 && L.Cout % 16 == 0;
}

// Weight rows per workgroup: the fewest slices of 16-row tiles whose rows
// fit 40 KiB of LDS, so that several workgroups share a CU.  The workgroups
// are persistent: each stages its weight slice once and walks every G-th
// chunk of 256 pixels, as many workgroups as the CUs hold at once (the
// slices of one chunk sit next to each other in the XCD-grouped order, so
// they share the chunk's pixels through one L2).
// out_stage: the output projection stages each wave's 32 x ns output tile in
// LDS (row pitch ns*2 + 16 bytes) and writes whole pixel rows with 16-byte
// stores, when a row's 16-byte chunks divide 64 lanes.
static ProjPlan proj_plan(int nout, int kdim, int64_t npix, bool out_stage = false)
{
    ProjPlan p{};
    p.pitch = kdim + 8;                                // 16 bytes of padding per row
    const int rows_fit = std::max(16, (40 * 1024 / (p.pitch * 2)) / 16 * 16);
    const int tiles = (nout + 15) / 16;
    p.nslices = (tiles * 16 + rows_fit - 1) / rows_fit;
    p.ns = (tiles + p.nslices - 1) / p.nslices * 16;
    p.nslices = (nout + p.ns - 1) / p.ns;
    p.chunk = 256;                                     // pixels per chunk: 4 waves x 2 passes x 32
    p.lds_bytes = p.ns * p.pitch * 2;
    if (out_stage && 64 % (p.ns / 8) == 0) {
        p.stage = p.lds_bytes;                          // a multiple of 16: pitch*2 = 2*kdim + 16
        p.lds_bytes += 4 * 32 * (p.ns * 2 + 16);
    }
    const int64_t nchunks = (npix + p.chunk - 1) / p.chunk;
    const int per_cu = std::max(1, std::min(8, 160 * 1024 / std::max(p.lds_bytes, 1)));
    const int64_t slots = std::max<int64_t>(1, (int64_t)per_cu * device_info().cus / p.nslices);
    // equal chunk counts per workgroup, and a multiple of 8 workgroups when
    // there is enough work (the XCD grouping needs it)
    const int64_t rounds = (nchunks + slots - 1) / slots;
    int64_t G = (nchunks + rounds - 1) / rounds;
    if (G >= 8) G = G / 8 * 8;
    G = std::max<int64_t>(1, G);
    p.nwg = G * p.nslices;
    p.remap_xcd = p.nwg % 8 == 0 ? 1 : 0;
    return p;
}

// kernel instantiation for kc k-steps (1..16)
template <typename F>
static auto pick_kc(int kc, F f)
{
    using I = std::integral_constant<int, 1>;
    switch (kc) {
    case 2: return f(std::integral_constant<int, 2>{});
    case 3: return f(std::integral_constant<int, 3>{});
    case 4: return f(std::integral_constant<int, 4>{});
    case 5: return f(std::integral_constant<int, 5>{});
    case 6: return f(std::integral_constant<int, 6>{});
    case 7: return f(std::integral_constant<int, 7>{});
    case 8: return f(std::integral_constant<int, 8>{});
    case 9: return f(std::integral_constant<int, 9>{});
    case 10: return f(std::integral_constant<int, 10>{});
    case 11: return f(std::integral_constant<int, 11>{});
    case 12: return f(std::integral_constant<int, 12>{});
    case 13: return f(std::integral_constant<int, 13>{});
    case 14: return f(std::integral_constant<int, 14>{});
    case 15: return f(std::integral_constant<int, 15>{});
    case 16: return f(std::integral_constant<int, 16>{});
    default: return f(I{});
    }
}

static int64_t grid_for(int64_t total)
{
    return std::max<int64_t>(1, std::min<int64_t>((total + 255) / 256, 1 << 20));
}

hipError_t launch_proj_in(const void* x, const void* w_q, const void* w_kv, void* q, void* k, void* v,
                          const LayerGeom& L0, bool bf16, bool mfma, hipStream_t st)
{
    LayerGeom L = L0;
    layer_fastdiv(L);
    if (mfma) {
        const ProjPlan p = proj_plan(3 * L.heads * L.d, L.C, L.NP);
        auto kern = pick_kc(L.C / 32, [](auto kc) { return proj_in_kernel<decltype(kc)::value>; });
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

hipError_t launch_proj_out(const void* attn, const void* w_o, const void* b_o, void* y, const LayerGeom& L0, bool bf16,
                           bool mfma, hipStream_t st)
{
    LayerGeom L = L0;
    layer_fastdiv(L);
    if (mfma) {
        const ProjPlan p = proj_plan(L.Cout, L.heads * L.d, L.NPo, true);
        auto kern = pick_kc(L.heads * L.d / 32, [](auto kc) { return proj_out_kernel<decltype(kc)::value>; });
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
