// Persistent fused halo-attention kernel for windows of at most 16 columns
// (gfx950 matrix cores, bf16 in, fp32 accumulate).
//
// Method: "Scaling Local Self-Attention for Parameter Efficient Visual
// Backbones", section 2.2 with Figures 1 and 2 (blocks, halo windows padded at
// the border, no centred mask, strided queries with stride-1 windows);
// relative logits of section 2.1 in the per-axis form of appendix A, scaled
// and indexed as in the HaloAttention module on the pswp.cn blog page
// (section 4).
//
// Work decomposition (MI355X-first):
//  * one workgroup owns one (batch, head) image strip of `nbx` adjacent block
//    columns and walks down its block rows.  Window rows live in an LDS ring
//    of R + block rows (K as [row][col][d], V transposed to [d][row][col]):
//    the R rows of the current window plus the `block` rows the next window
//    adds.  So the vertical halo overlap is reused in LDS as well as the
//    horizontal one, every K/V pixel of the strip is read from HBM once, and
//    the next rows are fetched (16-byte loads into registers) while the
//    current block row computes, then written to the ring: one barrier per
//    block row, no exposed load latency after the first.
//  * a wave takes QT tiles of 16 queries of one block at a time.  Scores are
//    computed transposed, S^T = K . Q^T, one 16x16 tile per window row (16
//    window columns); lane (n, g) holds query n and columns 4g..4g+3, so the
//    width term q.rel_w[col] is the MFMA accumulator input (masked columns
//    -1e30) and the height term q.rel_h[row] is one register per (lane, row).
//  * the window side R is a compile-time constant: both passes are fully
//    unrolled with static register indices.  Interior block rows run without
//    any row masking; the first and last block rows mask off-image rows.
//  * pass 1 takes the row max; pass 2 recomputes the scores, forms base-2
//    logits with one FMA each, exponentiates (v_exp_f32), packs bf16 P and
//    feeds it straight into the P.V MFMA (O^T = V^T . P^T) and a row-sum MFMA
//    against ones, so normalisation uses exactly the bf16 weights applied to V.
#include <algorithm>
#include <type_traits>

#include "mfma_util.h"

namespace halo {

#ifndef HALO_RING_WAVES
#define HALO_RING_WAVES 8
#endif
#ifndef HALO_RING_QT
#define HALO_RING_QT 2
#endif
constexpr int kRingWaves = HALO_RING_WAVES;
constexpr int kRingThreads = 64 * kRingWaves;
#ifndef HALO_RING_MAXI
#define HALO_RING_MAXI 2      // query groups per wave per block row with prefetched Q
#endif
constexpr int kRingMaxI = HALO_RING_MAXI;

struct RingPlan {
    int nstrips;     // column strips per image
    int nbx;         // block columns per strip
    int SWv;         // strip width in pixels (multiple of 4): LDS row pitch
    int ring;        // LDS ring rows (R + block)
    int RP;          // relative-table rows padded to a multiple of 16
    int groups;      // QT-tile groups per block
    int off_v, off_rel, off_scr, lds_bytes;
    int remap_xcd;
    int64_t nwg;
    float alpha;     // scale * log2(e)
};

template <int D, int R, int QT>
__global__ __launch_bounds__(kRingThreads)
void ring_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                 const __bf16* __restrict__ v, const __bf16* __restrict__ rel_h,
                 const __bf16* __restrict__ rel_w, __bf16* __restrict__ out,
                 Geometry g, RingPlan p)
{
    static_assert(R <= 16, "one 16-column tile per window row");
    constexpr int KPL = D / 4;                 // channels per lane in a QK fragment
    constexpr int CPP = D / 8;                 // 16-byte chunks per pixel
    typedef typename Frag<D>::T FragT;
    extern __shared__ __align__(16) unsigned char smem[];
    const int ring = p.ring, SWv = p.SWv;
    __bf16* Kr = reinterpret_cast<__bf16*>(smem);                    // [ring][SWv][D]
    __bf16* Vr = reinterpret_cast<__bf16*>(smem + p.off_v);          // [D][ring][SWv]
    __bf16* Rh = reinterpret_cast<__bf16*>(smem + p.off_rel);        // [RP][D]
    __bf16* Rw = Rh + p.RP * D;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, gq = lane >> 4;
    const int scr_stride = p.RP * 16;
    float* scr = reinterpret_cast<float*>(smem + p.off_scr) + wave * QT * scr_stride;

    int64_t wg = blockIdx.x;
    if (p.remap_xcd) {
        const int64_t per = p.nwg >> 3;
        wg = (wg & 7) * per + (wg >> 3);
    }
    const int64_t bh = wg / p.nstrips;
    const int sx = (int)(wg - bh * p.nstrips);
    const int bx_first = sx * p.nbx;
    const int nbx_here = min(p.nbx, g.nbw - bx_first);
    const int sx0 = bx_first * g.block - g.halo;      // strip column 0, image coordinates
    const int64_t plane = (int64_t)g.H * g.W * D;
    const __bf16* kb = k + bh * plane;
    const __bf16* vb = v + bh * plane;
    const int ng4 = SWv / 4;

    // ---- relative tables, zero-padded to RP rows
    {
        const int nrel = 2 * R - 1;
        const unsigned short* rhs = reinterpret_cast<const unsigned short*>(rel_h);
        const unsigned short* rws = reinterpret_cast<const unsigned short*>(rel_w);
        unsigned short* rhd = reinterpret_cast<unsigned short*>(Rh);
        unsigned short* rwd = reinterpret_cast<unsigned short*>(Rw);
        for (int e = tid; e < p.RP * D; e += kRingThreads) {
            const bool in = e < nrel * D;
            rhd[e] = in ? rhs[e] : (unsigned short)0;
            rwd[e] = in ? rws[e] : (unsigned short)0;
        }
    }

    // ---- staging of image rows into the ring.  Item e of the row range
    // starting at row0: 4 adjacent pixels x 8 channels (four 16-byte loads per
    // tensor).  Off-image columns are zero; K is stored as is, V transposed in
    // registers to eight 8-byte rows (4 columns of one channel).
    auto load_item = [&](int e, int row0, u32x4 (&kk)[4], u32x4 (&vv)[4]) {
        const int ch = e % CPP;
        const int rest = e / CPP;
        const int c4 = rest % ng4;
        const int iy = row0 + rest / ng4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ix = sx0 + 4 * c4 + j;
            kk[j] = u32x4{0u, 0u, 0u, 0u};
            vv[j] = u32x4{0u, 0u, 0u, 0u};
            if (ix >= 0 && ix < g.W && iy >= 0 && iy < g.H) {
                const int64_t off = ((int64_t)iy * g.W + ix) * D + ch * 8;
                kk[j] = *reinterpret_cast<const u32x4*>(kb + off);
                vv[j] = *reinterpret_cast<const u32x4*>(vb + off);
            }
        }
    };
    auto store_item = [&](int e, int row0, const u32x4 (&kk)[4], const u32x4 (&vv)[4]) {
        const int ch = e % CPP;
        const int rest = e / CPP;
        const int c4 = rest % ng4;
        const int iy = row0 + rest / ng4;
        const int slot = (iy + g.halo + ring) % ring;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<u32x4*>(Kr + ((size_t)(slot * SWv + 4 * c4 + j) * D + ch * 8)) = kk[j];
#pragma unroll
        for (int w = 0; w < 4; ++w) {             // channels 2w (low halves), 2w+1 (high)
            const u32x2 lo = {__builtin_amdgcn_perm(vv[1][w], vv[0][w], 0x05040100u),
                              __builtin_amdgcn_perm(vv[3][w], vv[2][w], 0x05040100u)};
            const u32x2 hi = {__builtin_amdgcn_perm(vv[1][w], vv[0][w], 0x07060302u),
                              __builtin_amdgcn_perm(vv[3][w], vv[2][w], 0x07060302u)};
            *reinterpret_cast<u32x2*>(Vr + ((size_t)(ch * 8 + 2 * w) * ring + slot) * SWv + 4 * c4) = lo;
            *reinterpret_cast<u32x2*>(Vr + ((size_t)(ch * 8 + 2 * w + 1) * ring + slot) * SWv + 4 * c4) = hi;
        }
    };

    // prologue: the first window's rows (off-image rows are stored as zeros)
    {
        const int lo = -g.halo, hi = R - g.halo;
        const int total = (hi - lo) * ng4 * CPP;
        for (int e = tid; e < total; e += kRingThreads) {
            u32x4 kk[4], vv[4];
            load_item(e, lo, kk, vv);
            store_item(e, lo, kk, vv);
        }
    }
    __syncthreads();

    const float alpha = p.alpha;
    s16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (short)0x3F80;
    asm volatile("" : "+v"(ones));   // opaque: kept in registers, never rebuilt
    const int items = nbx_here * p.groups;
    const int rowpitch = SWv * D;                     // elements per ring row of K
    const int64_t qbase = bh * plane;

    // Items (QT-tile groups) of block row `by` taken by this wave: the wave
    // assignment rotates by `items` per block row to balance the waves.
    auto first_item = [&](int byy) {
        const int rot = (int)(((int64_t)byy * items) % kRingWaves);
        return (wave - rot + kRingWaves) % kRingWaves;
    };
    struct Tile {   // one group of QT query tiles
        int xb, wcol0, nqx, nq;
        int qpix[QT];
        int yl[QT], xl[QT];
        bool qvalid[QT];
    };
    auto tile_of = [&](int byy, int it) {
        Tile T;
        const int j = it / p.groups, grp = it - j * p.groups;
        const int yb = byy * g.block;
        const int nqy = (min(yb + g.block, g.H) - yb + g.stride - 1) / g.stride;
        T.xb = (bx_first + j) * g.block;
        T.wcol0 = j * g.block;
        T.nqx = (min(T.xb + g.block, g.W) - T.xb + g.stride - 1) / g.stride;
        T.nq = nqy * T.nqx;
#pragma unroll
        for (int u = 0; u < QT; ++u) {
            const int qi = (grp * QT + u) * 16 + n;
            T.qvalid[u] = qi < T.nq;
            const int qq = T.qvalid[u] ? qi : 0;
            T.yl[u] = (qq / T.nqx) * g.stride;
            T.xl[u] = (qq % T.nqx) * g.stride;
            T.qpix[u] = (yb + T.yl[u]) * g.W + T.xb + T.xl[u];
        }
        return T;
    };
    auto load_q = [&](int byy, FragT (&qf)[kRingMaxI][QT]) {
        const int f = first_item(byy);
#pragma unroll
        for (int ii = 0; ii < kRingMaxI; ++ii) {
            const int it = f + ii * kRingWaves;
            if (byy < g.nbh && it < items) {
                const Tile T = tile_of(byy, it);
#pragma unroll
                for (int u = 0; u < QT; ++u)
                    qf[ii][u] = *reinterpret_cast<const FragT*>(q + qbase + (int64_t)T.qpix[u] * D + gq * KPL);
            }
        }
    };

    auto probs = [&](f32x4 s, float c) -> u32x2 {
        return u32x2{pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s[0], alpha, c)),
                                 __builtin_amdgcn_exp2f(fmaf(s[1], alpha, c))),
                     pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s[2], alpha, c)),
                                 __builtin_amdgcn_exp2f(fmaf(s[3], alpha, c)))};
    };

    // One group of QT query tiles of block row byy.
    auto do_item = [&](int byy, const Tile& T, const FragT (&qf)[QT]) {
        const int yb = byy * g.block;
        const int wy0 = yb - g.halo;
        const int tlo = max(0, -wy0), thi = min(R, g.H - wy0);
        const int base = yb % ring;                   // ring slot of window row 0
        auto slot = [&](int t) { const int s2 = base + t; return s2 >= ring ? s2 - ring : s2; };

        // ---- relative logits: table . Q^T on MFMA, re-indexed per query in LDS
        f32x4 cinit[QT];
        float RH[QT][R];
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const __bf16* tab = pass == 0 ? Rw : Rh;
            for (int rt = 0; rt < p.RP / 16; ++rt) {
                const FragT a = *reinterpret_cast<const FragT*>(tab + (rt * 16 + n) * D + gq * KPL);
#pragma unroll
                for (int u = 0; u < QT; ++u) {
                    const f32x4 gr = Frag<D>::mma(a, qf[u], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int i = 0; i < 4; ++i) scr[u * scr_stride + (rt * 16 + gq * 4 + i) * 16 + n] = gr[i];
                }
            }
            wave_lds_sync();
#pragma unroll
            for (int u = 0; u < QT; ++u) {
                if (pass == 0) {
                    // width term of window column c = 4g + i (masked: off-image, c >= R)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int c = gq * 4 + i;
                        const int ix = T.xb - g.halo + c;
                        const bool ok = c < R && ix >= 0 && ix < g.W;
                        const float val = scr[u * scr_stride + min(R - 1 - T.xl[u] + c, p.RP - 1) * 16 + n];
                        cinit[u][i] = ok ? val : kMaskLogit;
                    }
                } else {
                    // height term of window row t: table row R-1-yl+t (masked: off-image rows,
                    // whose ring rows are zeros)
                    const float* src = scr + u * scr_stride + (R - 1 - T.yl[u]) * 16 + n;
#pragma unroll
                    for (int t = 0; t < R; ++t) RH[u][t] = (t >= tlo && t < thi) ? src[t * 16] : kMaskLogit;
                }
            }
            wave_lds_sync();
        }

        const __bf16* kfrag = Kr + ((size_t)(T.wcol0 + n) * D + gq * KPL);
        const __bf16* vfrag = Vr + (size_t)n * ring * SWv + T.wcol0 + gq * 4;
        auto kload = [&](int t) -> FragT {
            return *reinterpret_cast<const FragT*>(kfrag + (size_t)slot(t) * rowpitch);
        };
        auto vload = [&](int mt, int t) -> u32x2 {
            return *reinterpret_cast<const u32x2*>(vfrag + (size_t)(mt * 16 * ring + slot(t)) * SWv);
        };

        // ---- pass 1: row max over the window (all R rows; masked rows carry -1e30)
        float M[QT];
#pragma unroll
        for (int u = 0; u < QT; ++u) M[u] = -3.0e38f;
#pragma unroll
        for (int t = 0; t < R; ++t) {
            const FragT a = kload(t);
#pragma unroll
            for (int u = 0; u < QT; ++u)
                M[u] = fmaxf(M[u], max4(Frag<D>::mma(a, qf[u], cinit[u])) + RH[u][t]);
        }
        float mb[QT];
        f32x4 O[QT][D / 16], L[QT];
#pragma unroll
        for (int u = 0; u < QT; ++u) {
            M[u] = fmaxf(M[u], __shfl_xor(M[u], 16));
            M[u] = fmaxf(M[u], __shfl_xor(M[u], 32));
            mb[u] = alpha * M[u];
            L[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt) O[u][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

        // ---- pass 2: P = exp2(alpha*S - mb) in bf16; O^T += V^T . P^T, L += 1 . P^T
#pragma unroll
        for (int t = 0; t < R; t += 2) {
            constexpr bool odd = (R % 2) != 0;
            const bool two = !odd || t + 1 < R;
            const FragT a0 = kload(t);
            const FragT a1 = two ? kload(t + 1) : FragT{};
            u32x4 vw[D / 16];
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt) {
                const u32x2 x0 = vload(mt, t);
                const u32x2 x1 = two ? vload(mt, t + 1) : u32x2{0u, 0u};
                vw[mt] = u32x4{x0[0], x0[1], x1[0], x1[1]};
            }
#pragma unroll
            for (int u = 0; u < QT; ++u) {
                const u32x2 p0 = probs(Frag<D>::mma(a0, qf[u], cinit[u]), alpha * RH[u][t] - mb[u]);
                u32x2 p1 = {0u, 0u};
                if (two) p1 = probs(Frag<D>::mma(a1, qf[u], cinit[u]), alpha * RH[u][t + 1] - mb[u]);
                const s16x8 pf = __builtin_bit_cast(s16x8, u32x4{p0[0], p0[1], p1[0], p1[1]});
#pragma unroll
                for (int mt = 0; mt < D / 16; ++mt)
                    O[u][mt] = mma_k32(__builtin_bit_cast(s16x8, vw[mt]), pf, O[u][mt]);
                L[u] = mma_k32(ones, pf, L[u]);
            }
        }

        // ---- normalise and store: lane (n, g) holds channels 16*mt + 4g + i of query n
#pragma unroll
        for (int u = 0; u < QT; ++u) {
            if (!T.qvalid[u]) continue;
            const float inv = 1.0f / L[u][0];
            const int yq = T.qpix[u] / g.W, xq = T.qpix[u] - yq * g.W;
            __bf16* op = out + bh * (int64_t)g.Ho * g.Wo * D +
                         ((int64_t)(yq / g.stride) * g.Wo + xq / g.stride) * D + gq * 4;
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt) {
                const u32x2 w = {pack_bf16x2(O[u][mt][0] * inv, O[u][mt][1] * inv),
                                 pack_bf16x2(O[u][mt][2] * inv, O[u][mt][3] * inv)};
                *reinterpret_cast<u32x2*>(op + mt * 16) = w;
            }
        }
    };

    FragT qcur[kRingMaxI][QT];
    load_q(0, qcur);
    for (int by = 0; by < g.nbh; ++by) {
        // ---- fetch, for the next block row, the window rows it adds (rows
        // past the image bottom are zeros) and its query fragments
        const int nlo = by * g.block + g.block + g.halo;
        const int ntotal = by + 1 < g.nbh ? g.block * ng4 * CPP : 0;
        u32x4 pk[4], pv[4];
        const bool have = tid < ntotal;
        if (have) load_item(tid, nlo, pk, pv);
        FragT qnext[kRingMaxI][QT];
        load_q(by + 1, qnext);

        // ---- compute this block row
        const int f = first_item(by);
#pragma unroll
        for (int ii = 0; ii < kRingMaxI; ++ii) {
            const int it = f + ii * kRingWaves;
            if (it < items) do_item(by, tile_of(by, it), qcur[ii]);
        }
        for (int it = f + kRingMaxI * kRingWaves; it < items; it += kRingWaves) {
            const Tile T = tile_of(by, it);
            FragT qf[QT];
#pragma unroll
            for (int u = 0; u < QT; ++u)
                qf[u] = *reinterpret_cast<const FragT*>(q + qbase + (int64_t)T.qpix[u] * D + gq * KPL);
            do_item(by, T, qf);
        }
#pragma unroll
        for (int ii = 0; ii < kRingMaxI; ++ii)
#pragma unroll
            for (int u = 0; u < QT; ++u) qcur[ii][u] = qnext[ii][u];

        // ---- the next window's new rows go into the ring slots the current
        // window does not use; then one barrier
        if (have) store_item(tid, nlo, pk, pv);
        for (int e = tid + kRingThreads; e < ntotal; e += kRingThreads) {
            u32x4 kk[4], vv[4];
            load_item(e, nlo, kk, vv);
            store_item(e, nlo, kk, vv);
        }
        __syncthreads();
    }
}

static int rup(int x, int m) { return (x + m - 1) / m * m; }

static RingPlan ring_plan(const Geometry& g, int R, int qt, int nbx)
{
    RingPlan p{};
    p.nbx = nbx;
    p.nstrips = (g.nbw + nbx - 1) / nbx;
    p.SWv = rup(std::max(nbx * g.block + 2 * g.halo, (nbx - 1) * g.block + 16), 4);
    p.ring = R + g.block;
    p.RP = rup(2 * R - 1, 16);
    const int side = (g.block + g.stride - 1) / g.stride;
    p.groups = ((side * side + 15) / 16 + qt - 1) / qt;
    const int kb = p.ring * p.SWv * g.d * 2;
    const int vb = g.d * p.ring * p.SWv * 2;
    const int rb = 2 * p.RP * g.d * 2;
    const int sb = kRingWaves * qt * p.RP * 16 * 4;
    p.off_v = rup(kb, 16);
    p.off_rel = rup(p.off_v + vb, 16);
    p.off_scr = rup(p.off_rel + rb, 16);
    p.lds_bytes = p.off_scr + sb;
    return p;
}

static int ring_lds_limit()
{
    int dev = 0, bytes = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 64 * 1024;
    if (hipDeviceGetAttribute(&bytes, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
        return 64 * 1024;
    return bytes;
}

// Plan for these arguments, or nbx = 0 when the ring does not fit in LDS.
static RingPlan ring_choose(const Geometry& g, int qt)
{
    const int limit = ring_lds_limit();
    for (int nbx = g.nbw; nbx >= 1; --nbx) {
        RingPlan p = ring_plan(g, g.r, qt, nbx);
        if (p.lds_bytes <= limit) return p;
    }
    return RingPlan{};
}

template <int D, int R, int QT>
static hipError_t ring_launch_t(const void* q, const void* k, const void* v, const void* rh,
                                const void* rw, void* out, const Geometry& g, hipStream_t st)
{
    RingPlan p = ring_choose(g, QT);
    if (p.nbx == 0) return hipErrorInvalidConfiguration;
    p.nwg = g.BH * p.nstrips;
    p.remap_xcd = (p.nwg % 8 == 0) ? 1 : 0;
    p.alpha = (float)((double)g.scale * 1.4426950408889634);
    auto kern = ring_kernel<D, R, QT>;
    if (p.lds_bytes > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_bytes);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)p.nwg), dim3(kRingThreads), p.lds_bytes, st,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v,
                       (const __bf16*)rh, (const __bf16*)rw, (__bf16*)out, g, p);
    return hipGetLastError();
}

template <int D, int R>
static hipError_t ring_launch_r(const void* q, const void* k, const void* v, const void* rh,
                                const void* rw, void* out, const Geometry& g, hipStream_t st)
{
    const int side = (g.block + g.stride - 1) / g.stride;
    const int tiles = (side * side + 15) / 16;
    if (HALO_RING_QT > 1 && tiles % HALO_RING_QT == 0)
        return ring_launch_t<D, R, HALO_RING_QT>(q, k, v, rh, rw, out, g, st);
    return ring_launch_t<D, R, 1>(q, k, v, rh, rw, out, g, st);
}

// Window sides with a compiled ring kernel.
static bool ring_side(int r) { return r == 8 || r == 10 || r == 12 || r == 14 || r == 16; }

bool ring_supported(const Geometry& g)
{
    if (!ring_side(g.r) || (g.d != 16 && g.d != 32) || g.block % 4 != 0) return false;
    return ring_choose(g, 1).nbx != 0;
}

hipError_t launch_ring(const void* q, const void* k, const void* v, const void* rh,
                       const void* rw, void* out, const Geometry& g, hipStream_t st)
{
#define HALO_RING_CASE(RR)                                                            \
    case RR:                                                                          \
        return g.d == 16 ? ring_launch_r<16, RR>(q, k, v, rh, rw, out, g, st)         \
                         : ring_launch_r<32, RR>(q, k, v, rh, rw, out, g, st);
    switch (g.r) {
        HALO_RING_CASE(8)
        HALO_RING_CASE(10)
        HALO_RING_CASE(12)
        HALO_RING_CASE(14)
        HALO_RING_CASE(16)
    default: return hipErrorInvalidValue;
    }
#undef HALO_RING_CASE
}

}  // namespace halo
