// Fused halo-attention kernel on gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// Method ("Scaling Local Self-Attention for Parameter Efficient Visual
// Backbones", section 2.2, Figures 1 and 2; relative logits of section 2.1 in
// the per-axis form of appendix A / the HaloAttention module on the pswp.cn
// blog page, section 4):
//   out[q] = sum_key softmax_key( scale * (q.k + q.rel_h[dy+c0] + q.rel_w[dx+c0]) ) v[key]
// over the in-image keys of the query's (b+2h)^2 block window.
//
// Work decomposition (MI355X-first, not the TPU scheme of the paper):
//  * one workgroup = a strip of `nbx` adjacent blocks of one block row.  The
//    strip's window rows are staged once into LDS with 16-byte coalesced
//    loads (K as [row][col][d], V transposed to [d][row][col]); neighbouring
//    blocks of the strip share the horizontal halo overlap in LDS, and the
//    vertical overlap is served from L2 because vertically adjacent strips
//    of one (batch, head) are mapped onto the same XCD.
//  * a wave owns 16 queries (one MFMA column tile) at a time.  Scores are
//    computed transposed, S^T = K . Q^T, in 16x16 tiles whose 16 rows are 16
//    consecutive window columns of ONE window row.  In the accumulator layout
//    lane (n, g) holds query n and window columns 4g..4g+3 of that row, so
//      - the width term q.rel_w[col] is the same for every row tile and is
//        loaded once as the MFMA accumulator input (masked columns: -1e30);
//      - the height term q.rel_h[row] is one scalar per (lane, tile);
//      - off-image rows are skipped, off-image columns carry -1e30.
//    q.rel_h / q.rel_w for every table row come from two small MFMAs
//    (table . Q^T) and are re-indexed per query through LDS.
//  * softmax: row max over the tile registers + two cross-lane steps; logits
//    are formed in base 2 (alpha = scale*log2 e) with one FMA per score,
//    exponentiated with v_exp_f32 and packed to bf16.  The packed P tile is
//    already the B operand of the P.V MFMA (O^T = V^T . P^T), so P never
//    leaves registers; the row sums come from a second MFMA against ones, so
//    normalisation uses exactly the bf16 weights that multiplied V.
#include <algorithm>

#include "halo_common.h"

namespace halo {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMfmaThreads = 256;            // 4 waves
constexpr int kMfmaWaves = kMfmaThreads / 64;
constexpr float kMaskLogit = -1.0e30f;       // exp2 of (alpha * this) is exactly 0

struct MfmaPlan {
    int nbx;          // blocks per strip
    int nstrips;      // strips per block row
    int SW;           // strip width in pixels (K rows in LDS)
    int SWv;          // pitch of a V^T row in LDS (elements)
    int RP;           // relative-table rows padded to a multiple of 16
    int off_v, off_rel, off_scr;   // byte offsets into dynamic LDS (K at 0)
    int lds_bytes;
    int remap_xcd;    // 1: map consecutive work items onto one XCD
    int64_t nwg;      // workgroups launched
    float alpha;      // scale * log2(e)
};

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

// D: head dim (16 or 32).  NCH: 16-column chunks per window row (r <= 16*NCH).
template <int D, int NCH>
__global__ __launch_bounds__(kMfmaThreads)
void mfma_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                 const __bf16* __restrict__ v, const __bf16* __restrict__ rel_h,
                 const __bf16* __restrict__ rel_w, __bf16* __restrict__ out,
                 Geometry g, MfmaPlan p)
{
    constexpr int MAXR = 16 * NCH;
    constexpr int KPL = D / 4;                 // channels per lane in a QK fragment
    typedef typename Frag<D>::T FragT;
    extern __shared__ __align__(16) unsigned char smem[];
    __bf16* Kl = reinterpret_cast<__bf16*>(smem);                    // [r][SW][D]
    __bf16* Vt = reinterpret_cast<__bf16*>(smem + p.off_v);          // [D][r][SWv]
    __bf16* Rh = reinterpret_cast<__bf16*>(smem + p.off_rel);        // [RP][D]
    __bf16* Rw = Rh + p.RP * D;                                       // [RP][D]

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, gq = lane >> 4;
    float* scr = reinterpret_cast<float*>(smem + p.off_scr) + wave * p.RP * 16;  // [RP][16]

    // ---- which strip: consecutive work items (same image, adjacent block
    // rows) go to the same XCD so the vertical halo overlap hits its L2.
    int64_t wg = blockIdx.x;
    if (p.remap_xcd) {
        const int64_t per = p.nwg >> 3;
        wg = (wg & 7) * per + (wg >> 3);
    }
    const int64_t per_bh = (int64_t)g.nbh * p.nstrips;
    const int64_t bh = wg / per_bh;
    const int rem = (int)(wg - bh * per_bh);
    const int by = rem / p.nstrips;
    const int sx = rem - by * p.nstrips;
    const int bx_first = sx * p.nbx;
    const int nbx_here = min(p.nbx, g.nbw - bx_first);
    const int r = g.r;
    const int wy0 = by * g.block - g.halo;            // window row 0, image coordinates
    const int sx0 = bx_first * g.block - g.halo;      // strip column 0, image coordinates
    const int tlo = max(0, -wy0), thi = min(r, g.H - wy0);   // in-image window rows
    const int SW = p.SW, SWv = p.SWv;
    const int64_t plane = (int64_t)g.H * g.W * D;

    // ---- stage K and V^T of the strip's in-image window rows
    {
        constexpr int CPP = D / 8;                    // 16-byte chunks per pixel
        const __bf16* kb = k + bh * plane;
        const __bf16* vb = v + bh * plane;
        const int total = (thi - tlo) * SW * CPP;
        for (int e = threadIdx.x; e < total; e += kMfmaThreads) {
            const int ch = e % CPP;
            const int pc = e / CPP;
            const int col = pc % SW;
            const int t = tlo + pc / SW;
            const int ix = sx0 + col;
            u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
            if (ix >= 0 && ix < g.W) {
                const int64_t off = ((int64_t)(wy0 + t) * g.W + ix) * D + ch * 8;
                kv = *reinterpret_cast<const u32x4*>(kb + off);
                vv = *reinterpret_cast<const u32x4*>(vb + off);
            }
            *reinterpret_cast<u32x4*>(Kl + ((size_t)(t * SW + col) * D + ch * 8)) = kv;
            const unsigned short* ve = reinterpret_cast<const unsigned short*>(&vv);
            unsigned short* vt = reinterpret_cast<unsigned short*>(Vt);
#pragma unroll
            for (int c = 0; c < 8; ++c)
                vt[((size_t)(ch * 8 + c) * r + t) * SWv + col] = ve[c];
        }
        const int nrel = 2 * r - 1;
        const unsigned short* rhs = reinterpret_cast<const unsigned short*>(rel_h);
        const unsigned short* rws = reinterpret_cast<const unsigned short*>(rel_w);
        unsigned short* rhd = reinterpret_cast<unsigned short*>(Rh);
        unsigned short* rwd = reinterpret_cast<unsigned short*>(Rw);
        for (int e = threadIdx.x; e < p.RP * D; e += kMfmaThreads) {
            const bool in = e < nrel * D;
            rhd[e] = in ? rhs[e] : (unsigned short)0;
            rwd[e] = in ? rws[e] : (unsigned short)0;
        }
    }
    __syncthreads();

    const float alpha = p.alpha;
    const int yb = by * g.block;
    const int nqy = (min(yb + g.block, g.H) - yb + g.stride - 1) / g.stride;
    const s16x8 ones = {0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80, 0x3F80};

    int item = 0;   // running index of 16-query tiles in the strip
    for (int j = 0; j < nbx_here; ++j) {
        const int xb = (bx_first + j) * g.block;
        const int nqx = (min(xb + g.block, g.W) - xb + g.stride - 1) / g.stride;
        const int nq = nqy * nqx;
        const int wcol0 = j * g.block;                // block j's window, strip coordinates
        for (int tq = 0; tq * 16 < nq; ++tq, ++item) {
            if (item % kMfmaWaves != wave) continue;

            // ---- the 16 queries of this tile (lane n; padding lanes reuse query 0)
            const int qi = tq * 16 + n;
            const bool qvalid = qi < nq;
            const int qq = qvalid ? qi : 0;
            const int yl = (qq / nqx) * g.stride, xl = (qq % nqx) * g.stride;
            const int y = yb + yl, x = xb + xl;
            const FragT qf = *reinterpret_cast<const FragT*>(
                q + bh * plane + ((int64_t)y * g.W + x) * D + gq * KPL);

            // ---- relative logits q.rel[row] for every table row, via MFMA;
            // re-indexed per query through the wave's LDS scratch.
            float RH[MAXR];
            f32x4 cinit[NCH];
            for (int pass = 0; pass < 2; ++pass) {
                const __bf16* tab = pass == 0 ? Rh : Rw;
                for (int rt = 0; rt < p.RP / 16; ++rt) {
                    const FragT a = *reinterpret_cast<const FragT*>(tab + (rt * 16 + n) * D + gq * KPL);
                    const f32x4 gr = Frag<D>::mma(a, qf, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int i = 0; i < 4; ++i) scr[(rt * 16 + gq * 4 + i) * 16 + n] = gr[i];
                }
                wave_lds_sync();
                if (pass == 0) {
                    // height term of window row t: table row (r-1-yl) + t
#pragma unroll
                    for (int t = 0; t < MAXR; ++t)
                        RH[t] = t < r ? scr[(r - 1 - yl + t) * 16 + n] : 0.f;
                } else {
                    // width term of window column c = 16*ch + 4g + i (masked: off-image / c >= r)
#pragma unroll
                    for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int c = ch * 16 + gq * 4 + i;
                            const int ix = xb - g.halo + c;
                            const bool ok = c < r && ix >= 0 && ix < g.W;
                            cinit[ch][i] = ok ? scr[(r - 1 - xl + c) * 16 + n] : kMaskLogit;
                        }
                    }
                }
                wave_lds_sync();
            }

            // ---- S^T tiles: 16 window columns of one window row x 16 queries.
            // r <= 16 keeps every tile in registers; wider windows recompute
            // the tiles in a second pass instead of holding 2*MAXR of them.
            auto score = [&](int t, int ch) -> f32x4 {
                const FragT a = *reinterpret_cast<const FragT*>(
                    Kl + ((size_t)(t * SW + wcol0 + ch * 16 + n) * D + gq * KPL));
                return Frag<D>::mma(a, qf, cinit[ch]);
            };
            constexpr bool kKeep = NCH == 1;
            f32x4 S[kKeep ? MAXR : 1][NCH];
            float M = -3.0e38f;
#pragma unroll
            for (int t = 0; t < MAXR; ++t) {
                if (t < tlo || t >= thi) continue;     // uniform across the workgroup
#pragma unroll
                for (int ch = 0; ch < NCH; ++ch) {
                    const f32x4 s = score(t, ch);
                    if (kKeep) S[kKeep ? t : 0][ch] = s;
                    const float tm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
                    M = fmaxf(M, tm + RH[t]);
                }
            }
            M = fmaxf(M, __shfl_xor(M, 16));
            M = fmaxf(M, __shfl_xor(M, 32));
            const float mb = alpha * M;               // base-2 row max

            // ---- P = exp2(alpha*S - mb) in bf16, O^T += V^T . P^T, L += 1 . P^T
            f32x4 O[D / 16], L = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt) O[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            unsigned pw[4];
            unsigned vw[D / 16][4];
            int half = 0;
#pragma unroll
            for (int t = 0; t < MAXR; ++t) {
                if (t < tlo || t >= thi) continue;
                const float c = alpha * RH[t] - mb;
#pragma unroll
                for (int ch = 0; ch < NCH; ++ch) {
                    const f32x4 s = kKeep ? S[kKeep ? t : 0][ch] : score(t, ch);
                    float e[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) e[i] = __builtin_amdgcn_exp2f(fmaf(s[i], alpha, c));
                    pw[half * 2 + 0] = pack_bf16x2(e[0], e[1]);
                    pw[half * 2 + 1] = pack_bf16x2(e[2], e[3]);
#pragma unroll
                    for (int mt = 0; mt < D / 16; ++mt) {
                        const u32x2 vv = *reinterpret_cast<const u32x2*>(
                            Vt + ((size_t)(mt * 16 + n) * r + t) * SWv + wcol0 + ch * 16 + gq * 4);
                        vw[mt][half * 2 + 0] = vv[0];
                        vw[mt][half * 2 + 1] = vv[1];
                    }
                    if (half) {
                        const s16x8 pf = __builtin_bit_cast(s16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
#pragma unroll
                        for (int mt = 0; mt < D / 16; ++mt) {
                            const s16x8 vf = __builtin_bit_cast(s16x8, u32x4{vw[mt][0], vw[mt][1], vw[mt][2], vw[mt][3]});
                            O[mt] = mma_k32(vf, pf, O[mt]);
                        }
                        L = mma_k32(ones, pf, L);
                    }
                    half ^= 1;
                }
            }
            if (half) {   // odd tile count: second half of the K=32 step is zero
                const s16x8 pf = __builtin_bit_cast(s16x8, u32x4{pw[0], pw[1], 0u, 0u});
#pragma unroll
                for (int mt = 0; mt < D / 16; ++mt) {
                    const s16x8 vf = __builtin_bit_cast(s16x8, u32x4{vw[mt][0], vw[mt][1], 0u, 0u});
                    O[mt] = mma_k32(vf, pf, O[mt]);
                }
                L = mma_k32(ones, pf, L);
            }

            // ---- normalise and store: lane (n, g) holds channels 16*mt + 4g + i of query n
            if (qvalid) {
                const float inv = 1.0f / L[0];
                __bf16* op = out + bh * (int64_t)g.Ho * g.Wo * D +
                             ((int64_t)(y / g.stride) * g.Wo + x / g.stride) * D + gq * 4;
#pragma unroll
                for (int mt = 0; mt < D / 16; ++mt) {
                    const u32x2 w = {pack_bf16x2(O[mt][0] * inv, O[mt][1] * inv),
                                     pack_bf16x2(O[mt][2] * inv, O[mt][3] * inv)};
                    *reinterpret_cast<u32x2*>(op + mt * 16) = w;
                }
            }
        }
    }
}

static int round_up(int x, int m) { return (x + m - 1) / m * m; }

// LDS footprint of a strip of nbx blocks.
static MfmaPlan make_plan(const Geometry& g, int nch, int nbx)
{
    MfmaPlan p{};
    p.nbx = nbx;
    p.nstrips = (g.nbw + nbx - 1) / nbx;
    p.SW = std::max(nbx * g.block + 2 * g.halo, (nbx - 1) * g.block + 16 * nch);
    p.SWv = round_up(p.SW, 4);
    p.RP = round_up(2 * g.r - 1, 16);
    const int kb = g.r * p.SW * g.d * 2;
    const int vb = g.d * g.r * p.SWv * 2;
    const int rb = 2 * p.RP * g.d * 2;
    const int sb = kMfmaWaves * p.RP * 16 * 4;
    p.off_v = round_up(kb, 16);
    p.off_rel = round_up(p.off_v + vb, 16);
    p.off_scr = round_up(p.off_rel + rb, 16);
    p.lds_bytes = p.off_scr + sb;
    return p;
}

bool mfma_supported(int d, int r, int block, int stride, bool bf16)
{
    (void)stride;
    return bf16 && (d == 16 || d == 32) && r <= 32 && block % 4 == 0;
}

// Largest dynamic LDS one workgroup may use on the current device.
static int device_lds_limit()
{
    int dev = 0, bytes = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 64 * 1024;
    if (hipDeviceGetAttribute(&bytes, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
        return 64 * 1024;
    return bytes;
}

template <int D, int NCH>
static hipError_t launch_t(const void* q, const void* k, const void* v, const void* rh,
                           const void* rw, void* out, const Geometry& g, hipStream_t st)
{
    // Widest strip that leaves room for two workgroups per CU; narrower
    // strips only when even one block needs more.
    constexpr int kTarget = 80 * 1024;
    const int limit = device_lds_limit();
    int nbx = g.nbw;
    MfmaPlan p = make_plan(g, NCH, nbx);
    while (nbx > 1 && p.lds_bytes > kTarget) p = make_plan(g, NCH, --nbx);
    if (p.lds_bytes > limit) return hipErrorInvalidConfiguration;
    p.nwg = g.BH * g.nbh * p.nstrips;
    p.remap_xcd = (p.nwg % 8 == 0) ? 1 : 0;
    p.alpha = (float)((double)g.scale * 1.4426950408889634);
    auto kern = mfma_kernel<D, NCH>;
    if (p.lds_bytes > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_bytes);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)p.nwg), dim3(kMfmaThreads), p.lds_bytes, st,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v,
                       (const __bf16*)rh, (const __bf16*)rw, (__bf16*)out, g, p);
    return hipGetLastError();
}

hipError_t launch_mfma(const void* q, const void* k, const void* v, const void* rh,
                       const void* rw, void* out, const Geometry& g, hipStream_t st)
{
    const int nch = g.r <= 16 ? 1 : 2;
    if (g.d == 16) return nch == 1 ? launch_t<16, 1>(q, k, v, rh, rw, out, g, st)
                                   : launch_t<16, 2>(q, k, v, rh, rw, out, g, st);
    return nch == 1 ? launch_t<32, 1>(q, k, v, rh, rw, out, g, st)
                    : launch_t<32, 2>(q, k, v, rh, rw, out, g, st);
}

}  // namespace halo
