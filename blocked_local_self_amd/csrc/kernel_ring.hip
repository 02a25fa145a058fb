// Persistent fused halo-attention kernel for windows of at most 32 columns
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
//    of R + block rows: the R rows of the current window plus the `block`
//    rows the next window adds.  The vertical halo overlap is reused in LDS as
//    well as the horizontal one, so every K/V pixel of the strip is read from
//    HBM once; the next rows (and the next query fragments) are fetched into
//    registers at the start of a block row and written to the ring once the
//    wave's first group is computed: one barrier per block row.  Rows above
//    or below the image are kept as zero rows, so every block row runs the
//    same code.
//  * workgroups of 4 or 8 waves: with 4, two workgroups share a CU and one's
//    barrier waits overlap the other's compute; the strip width is the widest
//    whose ring fits the LDS share.
//  * LDS layouts are chosen for conflict-free fragment reads: K is
//    [slot][col][d] with the 16-byte chunks of a pixel XOR-swizzled by column
//    bits; V is transposed to [d][slot][col] with the channel pitch padded to
//    4 (mod 64) dwords; the relative-logit scratch has a 20-float row stride.
//  * a wave takes QT tiles of 16 queries of one block at a time.  Scores are
//    computed transposed, S^T = K . Q^T, one 16x16 tile per window row and
//    16-column tile (NCT = 1 or 2 of them); lane (n, g) holds query n and
//    columns 4g..4g+3 of the tile, so the width term q.rel_w[col] is the MFMA
//    accumulator input (masked columns -1e30) and the height term
//    q.rel_h[row] is one scalar per (lane, row).
//  * both passes loop over the in-image window rows only; the height term of
//    a row is read from the conflict-free scratch.
//  * the softmax is shifted by a per-query upper bound on its logits
//    (sum over channels of |q_c| times the running maximum norm of k's chunk
//    of c plus the table maxima of |rel_w_c| and |rel_h_c|, one MFMA) instead
//    of an exact max, so a
//    single pass forms base-2 logits with one FMA each, exponentiates
//    (v_exp_f32), packs bf16 P and feeds it straight into the P.V MFMA
//    (O^T = V^T . P^T) and a row-sum MFMA against ones (normalisation uses
//    exactly the bf16 weights applied to V).  Should the bound overshoot
//    enough for the weight sum to drop below 2^-60, the group is recomputed
//    with the exact row max (an extra pass), so the result is the stable
//    softmax in every case.
#include <algorithm>
#include <type_traits>

#include "mfma_util.h"

namespace halo {

#ifndef HALO_RING_QT
#define HALO_RING_QT 2
#endif
#ifndef HALO_RING_FORCE_WAVES
#define HALO_RING_FORCE_WAVES 0   // 4 or 8 to override the per-shape choice
#endif

constexpr int kLdsPerCU = 160 * 1024;   // gfx950
// Query groups a wave may take per block row (the plan keeps within it).
constexpr int ring_maxi(int nct) { return nct == 1 ? 2 : 4; }
constexpr int kScrStride = 20;        // floats per scratch row (conflict-free writes)
// LDS banks as a 32-bit access sees them: 32 banks of 4 bytes, 32 lanes per
// pass (SQ_LDS_BANK_CONFLICT on gfx950: padding the 32-query scratch by 32
// dwords changed nothing, by 16 removed its conflicts).  The 32-query
// scratch rows hold 16 floats, and a tile's scratch starts 16 banks after
// the previous tile's: lanes n and n + 16 of a pass (the two query tiles)
// then fall in different halves of the banks, both for a row shared by the
// pass and for each query's own height row (row R - 1 - yl, yl = n32 / 8).
constexpr int kScr32Stride = 16;
constexpr unsigned scr32_tile_bytes(int rows) { return (unsigned)(rows * kScr32Stride + 16) * 4; }

// Relative-table rows (padded, multiple of 16) for windows of up to 16*nct
// columns: 2R-1 <= 32*nct - 1 and R-1+16*nct-1 < 32*nct.
constexpr int rel_rows(int nct) { return 32 * nct; }
// Rows of a query tile's scratch: the table-indexed layout (one column tile)
// or the window-indexed layout with a clamp row at each end (two).
constexpr int scr_rows(int nct) { return nct == 1 ? rel_rows(1) : 16 * nct + 2; }

struct RingPlan {
    int nstrips;     // column strips per image
    int nbx;         // block columns per strip
    int SWv;         // strip width in pixels (multiple of 4)
    int ring;        // LDS ring rows (R + block)
    int CP;          // V^T channel pitch in elements (ring*SWv, padded)
    int groups;      // QT-tile groups per block
    int midstage;    // ring of R + block rows: next rows staged mid block row
    int off_v, off_rel, off_scr, off_kn, off_qt, lds_bytes;
    int remap_xcd;
    int64_t nwg;
    float alpha;     // scale * log2(e)
};

template <typename T>
__device__ inline T lds_ld(const unsigned char* base, unsigned off)
{
    return *reinterpret_cast<const T*>(base + off);
}
template <typename T>
__device__ inline void lds_st(unsigned char* base, unsigned off, T val)
{
    *reinterpret_cast<T*>(base + off) = val;
}

// Byte offset, inside a pixel's D channels, of 16-byte chunk `c` of the
// pixel at strip column `col` (XOR swizzle).
template <int D>
__device__ inline unsigned k_chunk(int c, int col)
{
    if (D == 16) return (unsigned)((c ^ ((col >> 3) & 1)) * 16);
    return (unsigned)((c ^ ((col >> 2) & 3)) * 16);
}

// VAR: the semantic variants of g.flags are honoured (a separate
// instantiation, so the default semantics carry none of their tests).
template <int D, int NCT, int QT, int W, bool VAR>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2)))
void ring_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                 const __bf16* __restrict__ v, const __bf16* __restrict__ rel_h,
                 const __bf16* __restrict__ rel_w, __bf16* __restrict__ out,
                 float* __restrict__ lse, Geometry g, RingPlan p)
{
    static_assert(NCT == 1 || NCT == 2, "windows of up to 32 columns");
    const int R = g.r;                         // window side, <= 16 * NCT
    constexpr int kRelTiles = 2 * NCT;
    constexpr int kRelRows = rel_rows(NCT);
    constexpr int kScrRows = scr_rows(NCT);
    constexpr int kRingWaves = W;
    constexpr int kRingMaxI = ring_maxi(NCT);
    constexpr int kRingThreads = 64 * W;
    constexpr int KPL = D / 4;                 // channels per lane in a QK fragment
    constexpr int CPP = D / 8;                 // 16-byte chunks per pixel
    constexpr unsigned PIXB = D * 2;           // bytes per pixel
    typedef typename Frag<D>::T FragT;
    extern __shared__ __align__(16) unsigned char smem[];
    const int ring = p.ring, SWv = p.SWv, CP = p.CP;
    const unsigned rowb_k = (unsigned)SWv * PIXB;            // bytes per K ring row
    const unsigned offv = p.off_v, offrh = p.off_rel, offrw = p.off_rel + kRelRows * D * 2;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, gq = lane >> 4;
    // One column tile, 16 channels, two query tiles: the group's 32 queries
    // go through 32x32 MFMAs (lane = query lane & 31, K half lane >> 5).
    // A K = 16 score tile of 32 keys x 32 queries then costs what a 16x16
    // one does, and one 32x32 P.V MFMA with bf16 ones in rows 16-31 gives
    // the weighted sum and the weight sum together.
    constexpr bool G32 = D == 16 && NCT == 1 && QT == 2 && !VAR;
    const int n32 = lane & 31, g2 = lane >> 5;
    constexpr unsigned scr_u = (unsigned)kScrRows * kScrStride * 4;   // bytes per query tile
    const unsigned scr0 = p.off_scr + wave * QT * scr_u + 4u * n;     // column n of tile 0

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

    // ---- relative tables, zero-padded to kRelRows rows
    {
        const int nrel = 2 * R - 1;
        const unsigned short* rhs = reinterpret_cast<const unsigned short*>(rel_h);
        const unsigned short* rws = reinterpret_cast<const unsigned short*>(rel_w);
        const bool half = VAR && (g.flags & kFlagHalfSplit);   // height on channels < D/2, width on the rest
        for (int e = tid; e < kRelRows * D; e += kRingThreads) {
            const bool in = e < nrel * D;
            const int c = e % D;
            lds_st<unsigned short>(smem, offrh + 2 * e, in && (!half || c < D / 2) ? rhs[e] : (unsigned short)0);
            lds_st<unsigned short>(smem, offrw + 2 * e, in && (!half || c >= D / 2) ? rws[e] : (unsigned short)0);
        }
    }

    // ---- staging of image rows into the ring.  Item e of a range of rows:
    // 4 adjacent pixels x 8 channels (four 16-byte loads per tensor).
    // Off-image pixels are zero; K is stored swizzled, V transposed in
    // registers to eight 8-byte rows (4 columns of one channel).  The running
    // maxima of |k chunk|^2 over everything staged so far feed the softmax
    // shift bound.
    struct Item { int ch, c4, dr; };            // chunk, 4-column group, row within the range
    auto item_of = [&](int e) {
        Item it;
        it.ch = e % CPP;
        const int rest = e / CPP;
        it.dr = rest / ng4;
        it.c4 = rest - it.dr * ng4;
        return it;
    };
    // Running maxima of |k_chunk|^2 (8-channel chunks) over the keys staged
    // so far.  Two sets, by block-row parity: rows staged during block row
    // `by` update set (by+1)&1 while the waves computing block row `by` read
    // set by&1, which is final since the last barrier.  The bound a query
    // sees is therefore independent of wave timing.
    unsigned* kmax_bits = reinterpret_cast<unsigned*>(smem + p.off_kn);
    if (tid < 32) kmax_bits[tid] = 0u;
    const unsigned off_one = p.off_kn + 2 * 16 * 4 + D * 4;     // 32 bytes of bf16 ones
    if (G32 && tid < 8) lds_st<unsigned>(smem, off_one + 4u * tid, 0x3F803F80u);
    __syncthreads();
    auto load_item = [&](const Item& it, int row0, u32x4 (&kk)[4], u32x4 (&vv)[4]) {
        const int iy = row0 + it.dr;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ix = sx0 + 4 * it.c4 + j;
            kk[j] = u32x4{0u, 0u, 0u, 0u};
            vv[j] = u32x4{0u, 0u, 0u, 0u};
            if (ix >= 0 && ix < g.W && iy >= 0 && iy < g.H) {
                const int64_t off = ((int64_t)iy * g.W + ix) * D + it.ch * 8;
                kk[j] = *reinterpret_cast<const u32x4*>(kb + off);
                vv[j] = *reinterpret_cast<const u32x4*>(vb + off);
            }
        }
    };
    auto store_item = [&](const Item& it, int row0, const u32x4 (&kk)[4], const u32x4 (&vv)[4], unsigned* kmax) {
        const int iy = row0 + it.dr;
        const int slot = (iy + g.halo + ring) % ring;
        float nmax = 0.f;                         // max over the 4 pixels of |k chunk|^2
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = 4 * it.c4 + j;
            lds_st<u32x4>(smem, (unsigned)slot * rowb_k + col * PIXB + k_chunk<D>(it.ch, col), kk[j]);
            float ss = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float lo = __builtin_bit_cast(float, kk[j][w] << 16);
                const float hi = __builtin_bit_cast(float, kk[j][w] & 0xffff0000u);
                ss = fmaf(lo, lo, fmaf(hi, hi, ss));
            }
            nmax = fmaxf(nmax, ss);
        }
        atomicMax(&kmax[it.ch], __builtin_bit_cast(unsigned, nmax));   // non-negative: bit order = value order
#pragma unroll
        for (int w = 0; w < 4; ++w) {             // channels 2w (low halves), 2w+1 (high)
            const u32x2 lo = {__builtin_amdgcn_perm(vv[1][w], vv[0][w], 0x05040100u),
                              __builtin_amdgcn_perm(vv[3][w], vv[2][w], 0x05040100u)};
            const u32x2 hi = {__builtin_amdgcn_perm(vv[1][w], vv[0][w], 0x07060302u),
                              __builtin_amdgcn_perm(vv[3][w], vv[2][w], 0x07060302u)};
            const unsigned base = offv + 2u * ((unsigned)slot * SWv + 4 * it.c4);
            lds_st<u32x2>(smem, base + 2u * (unsigned)((it.ch * 8 + 2 * w) * CP), lo);
            lds_st<u32x2>(smem, base + 2u * (unsigned)((it.ch * 8 + 2 * w + 1) * CP), hi);
        }
    };

    // prologue: the first window's rows (off-image rows are stored as zeros)
    {
        const int lo = -g.halo;
        const int total = R * ng4 * CPP;
        for (int e = tid; e < total; e += kRingThreads) {
            u32x4 kk[4], vv[4];
            const Item it = item_of(e);
            load_item(it, lo, kk, vv);
            store_item(it, lo, kk, vv, kmax_bits);
        }
    }
    __syncthreads();

    // relative tables as MFMA A operands: kept in registers for one column
    // tile, read from LDS per use for two (register pressure)
    constexpr int kTabRegs = NCT == 1 ? kRelTiles : 1;
    FragT tabw[kTabRegs], tabh[kTabRegs];
    auto tab_frag = [&](unsigned off, int rt) {
        return lds_ld<FragT>(smem, off + 2u * ((rt * 16 + n) * D + gq * KPL));
    };
    s16x8 tab32w, tab32h;                       // 32x32 A operands: row n32, channels 8*g2..+7
    if constexpr (G32) {
        tab32w = lds_ld<s16x8>(smem, offrw + 2u * (n32 * D + 8 * g2));
        tab32h = lds_ld<s16x8>(smem, offrh + 2u * (n32 * D + 8 * g2));
    } else if constexpr (NCT == 1) {
#pragma unroll
        for (int rt = 0; rt < kRelTiles; ++rt) {
            tabw[rt] = tab_frag(offrw, rt);
            tabh[rt] = tab_frag(offrh, rt);
        }
    }

    // tmax[c] = max_j |rel_w[j][c]| + max_j |rel_h[j][c]| over all table
    // rows, one fp32 per channel in LDS (after the kmax words)
    float* tmax = reinterpret_cast<float*>(smem + p.off_kn + 2 * 16 * 4);
    if (tid < D) {
        float mw = 0.f, mh = 0.f;
        for (int j = 0; j < 2 * R - 1; ++j) {
            mw = fmaxf(mw, fabsf((float)lds_ld<__bf16>(smem, offrw + 2u * (j * D + tid))));
            mh = fmaxf(mh, fabsf((float)lds_ld<__bf16>(smem, offrh + 2u * (j * D + tid))));
        }
        tmax[tid] = mw + mh;
    }
    // geometry of query n of tile u of group grp in a full block (every
    // block but the partial ones at the image's right and bottom edges):
    // {yl, xl, yl*W + xl, (yl/s)*Wo + xl/s}, or yl = -1 past the block's queries
    const int side = g.block / g.stride;
    for (int qi = tid; qi < p.groups * QT * 16; qi += kRingThreads) {   // qi = (grp*QT + u)*16 + n
        const int iy = qi / side, ix = qi - iy * side;
        const bool in = qi < side * side;
        const int yl = iy * g.stride, xl = ix * g.stride;
        lds_st<i32x4>(smem, p.off_qt + 16u * qi,
                      in ? i32x4{yl, xl, yl * g.W + xl, iy * g.Wo + ix} : i32x4{-1, 0, 0, 0});
    }
    __syncthreads();

    const float alpha = p.alpha;
    s16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (short)0x3F80;
    asm volatile("" : "+v"(ones));   // opaque: kept in registers, never rebuilt
    const int items = nbx_here * p.groups;
    const int64_t qbase = bh * plane;

    // Items (QT-tile groups) of block row `byy` taken by this wave: the wave
    // assignment rotates by `items` per block row to balance the waves.
    auto first_item = [&](int byy) {
        const int rot = (int)(((int64_t)byy * items) % kRingWaves);
        return (wave - rot + kRingWaves) % kRingWaves;
    };
    struct Tile {   // one group of QT query tiles
        int xb, wcol0;
        int yl[QT], xl[QT];                   // block-local query position (full resolution)
        int qpix[QT], opix[QT];               // query pixel in the image, output pixel
        bool qvalid[QT];
    };
    // small non-negative integer quotient a / b through an fp32 reciprocal
    // (exact for a < 2^16: (a + 0.5) / b stays > 0.5/b away from integers)
    auto qdiv = [](int a, float rb) { return (int)(((float)a + 0.5f) * rb); };
    // query of this lane in tile u of group grp (block-local index); the
    // 32-query layout has one query per lane (entries [0] of a Tile)
    constexpr int QU = G32 ? 1 : QT;
    auto qindex = [&](int grp, int u) { return G32 ? grp * 32 + n32 : (grp * QT + u) * 16 + n; };
    auto tile_of = [&](int byy, int it) {
        Tile T;
        const int j = it / p.groups, grp = it - j * p.groups;
        const int yb = byy * g.block;
        if (yb + g.block <= g.H && (bx_first + j) * g.block + g.block <= g.W) {   // uniform: full block
            T.xb = (bx_first + j) * g.block;
            T.wcol0 = j * g.block;
            const int qbase0 = yb * g.W + T.xb, obase0 = byy * side * g.Wo + (bx_first + j) * side;
#pragma unroll
            for (int u = 0; u < QU; ++u) {
                const i32x4 e = lds_ld<i32x4>(smem, p.off_qt + 16u * qindex(grp, u));
                T.qvalid[u] = e[0] >= 0;
                T.yl[u] = T.qvalid[u] ? e[0] : 0;
                T.xl[u] = e[1];
                T.qpix[u] = qbase0 + e[2];
                T.opix[u] = obase0 + e[3];
            }
            return T;
        }
        const int nqy = (min(yb + g.block, g.H) - yb + g.stride - 1) / g.stride;
        T.xb = (bx_first + j) * g.block;
        T.wcol0 = j * g.block;
        const int nqx = (min(T.xb + g.block, g.W) - T.xb + g.stride - 1) / g.stride;
        const int nq = nqy * nqx;
        const float rnqx = __builtin_amdgcn_rcpf((float)nqx);   // 1 ulp: ample for qdiv
        const int opix0 = (yb / g.stride) * g.Wo + T.xb / g.stride;   // block % stride == 0
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            const int qi = qindex(grp, u);
            T.qvalid[u] = qi < nq;
            const int qq = T.qvalid[u] ? qi : 0;
            const int iy = qdiv(qq, rnqx), ix = qq - iy * nqx;
            T.yl[u] = iy * g.stride;
            T.xl[u] = ix * g.stride;
            T.qpix[u] = (yb + T.yl[u]) * g.W + T.xb + T.xl[u];
            T.opix[u] = opix0 + iy * g.Wo + ix;
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
                if constexpr (G32) {                  // channels 8*g2..+7 of the lane's query
                    const u32x4 w = *reinterpret_cast<const u32x4*>(q + qbase + (int64_t)T.qpix[0] * D + 8 * g2);
                    qf[ii][0] = __builtin_bit_cast(FragT, u32x2{w[0], w[1]});
                    qf[ii][1] = __builtin_bit_cast(FragT, u32x2{w[2], w[3]});
                } else {
#pragma unroll
                for (int u = 0; u < QT; ++u)
                    qf[ii][u] = *reinterpret_cast<const FragT*>(
                        q + qbase + (int64_t)T.qpix[u] * D + gq * KPL);
                }
            }
        }
    };

    auto probs = [&](f32x4 s, float c) -> u32x2 {
        return u32x2{pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s[0], alpha, c)),
                                 __builtin_amdgcn_exp2f(fmaf(s[1], alpha, c))),
                     pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s[2], alpha, c)),
                                 __builtin_amdgcn_exp2f(fmaf(s[3], alpha, c)))};
    };

    // Output of one group: lane (n, g) holds channels 16*mt + 4g + i of
    // query n of tile u, packed bf16.
    // lse2: the softmax shift plus log2 of the weight sum (base-2 log of
    // the normaliser), when the caller asks for the log normalisers.
    struct Result {
        u32x2 w[QT][D / 16];
        float lse2[QT];
    };
    auto store_result = [&](const Tile& T, const Result& res) {
        if constexpr (G32) {                          // channels 4*g2.. and 8+4*g2.. of the lane's query
            if (!T.qvalid[0]) return;
            __bf16* op = out + bh * (int64_t)g.Ho * g.Wo * D + (int64_t)T.opix[0] * D + 4 * g2;
            *reinterpret_cast<u32x2*>(op) = res.w[0][0];
            *reinterpret_cast<u32x2*>(op + 8) = res.w[1][0];
            if (lse != nullptr && g2 == 0)
                lse[bh * (int64_t)g.Ho * g.Wo + T.opix[0]] = res.lse2[0] * 0.6931471805599453f;
            return;
        }
#pragma unroll
        for (int u = 0; u < QT; ++u) {
            if (!T.qvalid[u]) continue;
            __bf16* op = out + bh * (int64_t)g.Ho * g.Wo * D + (int64_t)T.opix[u] * D + gq * 4;
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt) *reinterpret_cast<u32x2*>(op + mt * 16) = res.w[u][mt];
            if (lse != nullptr && gq == 0)
                lse[bh * (int64_t)g.Ho * g.Wo + T.opix[u]] = res.lse2[u] * 0.6931471805599453f;
        }
    };

    // One group of 32 queries of block row byy in the 32x32 layout (one
    // column tile, 16 channels, no variants).  The steps are those of the
    // 16x16 path below; lane l holds query l & 31 and, of every 32-row
    // operand or result, the rows 8j + 4(l >> 5) + i.
    auto do_item32 = [&](int byy, const Tile& T, const FragT (&qf)[QT], Result& res) {
      if constexpr (G32) {
            const int yb = byy * g.block;
            const int wy0 = yb - g.halo;
            const int tlo = max(0, -wy0), thi = min(R, g.H - wy0);
            const int base = yb % ring;                   // ring slot of window row 0
            auto rslot = [&](int t) -> unsigned {
                const int s2 = base + t;
                return (unsigned)(s2 >= ring ? s2 - ring : s2);
            };
            const u32x2 qa = __builtin_bit_cast(u32x2, qf[0]), qb = __builtin_bit_cast(u32x2, qf[1]);
            const s16x8 q32 = __builtin_bit_cast(s16x8, u32x4{qa[0], qa[1], qb[0], qb[1]});
            const f32x16 zero16 = {};
            static_assert(2 * scr32_tile_bytes(kScrRows) <= QT * scr_u, "within the wave's scratch");
            const unsigned scr32 = p.off_scr + wave * QT * scr_u + (unsigned)(n32 >> 4) * scr32_tile_bytes(kScrRows) +
                                   4u * (n32 & 15);
            constexpr unsigned RS = 4u * kScr32Stride;    // bytes per scratch row

            // ---- relative logits of the 32 table rows, then the width terms
            const f32x16 gw = mma32_k16(tab32w, q32, zero16);
            const f32x16 gh = mma32_k16(tab32h, q32, zero16);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) lds_st<float>(smem, scr32 + RS * (8 * j + 4 * g2 + i), gw[4 * j + i]);
            // width term of window column c = 8j + 4*g2 + i (j = 0, 1); rows
            // 16-31 of a score tile are the second window row: same columns
            // Masked columns (off the image, c < clo or c >= chi, or past the
            // window, c >= R) get the mask value in their scratch rows, which
            // no other column of the query reads: the reads need no selects
            const int clo = g.halo - T.xb, chi = min(R, g.W - T.xb + g.halo);
            const unsigned a0 = scr32 + RS * (R - 1 - T.xl[0]);     // row of column 0
            for (int c = 0; c < clo; ++c) lds_st<float>(smem, a0 + RS * c, kMaskLogit);
            for (int c = chi; c < 16; ++c) lds_st<float>(smem, a0 + RS * c, kMaskLogit);
            f32x16 cinit;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    cinit[4 * j + i] = cinit[8 + 4 * j + i] = lds_ld<float>(smem, a0 + RS * (8 * j + 4 * g2 + i));

            // ---- softmax shift: the bound of the 16x16 path, for 32 queries in
            // one MFMA (a_c in all 32 rows, |q| as B; channels 8*g2..+7 lie in chunk g2)
            float mb;
            {
                const float kn = __builtin_sqrtf(__builtin_bit_cast(float, kmax_bits[16 * (byy & 1) + g2])) *
                                 (1.f + 0x1p-20f);
                s16x8 abound, aq;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float a = kn + tmax[8 * g2 + e];
                    abound[e] = (short)((__builtin_bit_cast(unsigned, a) + 0xffffu) >> 16);   // round up
                    aq[e] = (short)(q32[e] & 0x7fff);
                }
                const float bound = mma32_k16(abound, aq, zero16)[0];
                mb = alpha * (bound + 1e-3f * (1.f + bound));
            }
            // height terms alpha*G - mb -> scratch (after the width reads)
            const int sh = R - 1 - T.yl[0];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    lds_st<float>(smem, scr32 + RS * (8 * j + 4 * g2 + i), fmaf(gh[4 * j + i], alpha, -mb));
            const unsigned rh = scr32 + RS * sh;          // scratch of window row 0
            // row pairs start at even ring slots (see the 16x16 path); the rows
            // a pair adds before tlo or at thi get a height term of -inf
            const int ts = tlo - ((base + tlo) & 1);
            if (ts < tlo) lds_st<float>(smem, rh + RS * ts, -INFINITY);
            if ((thi - ts) & 1) lds_st<float>(smem, rh + RS * thi, -INFINITY);

            // ---- operands: K rows t, t+1 (keys 0-15, 16-31: 16 bytes of chunk
            // g2 per lane); V^T of channel n32 for n32 < 16 and bf16 ones for the
            // weight-sum rows 16-31 (stride 0: the same 32 bytes every row)
            const int kcol = T.wcol0 + (n32 & 15);
            const unsigned kl = (unsigned)kcol * PIXB + k_chunk<D>(g2, kcol) + (unsigned)(n32 >> 4) * rowb_k;
            const bool vlane = n32 < 16;
            const unsigned vl = vlane ? offv + 2u * ((unsigned)n32 * CP + T.wcol0 + 4 * g2) : off_one;
            const unsigned vrow = vlane ? 2u * SWv : 0u;
            struct Ops32 {
                s16x8 a;
                u32x4 v0, v1;
                float c0, c1;
            };
            auto fetch = [&](int t0) {
                Ops32 o;
                const unsigned sl = rslot(t0);
                o.a = lds_ld<s16x8>(smem, kl + sl * rowb_k);
                const unsigned vo = vl + sl * vrow;
                const u32x2 x0 = lds_ld<u32x2>(smem, vo), x1 = lds_ld<u32x2>(smem, vo + 16);
                const u32x2 y0 = lds_ld<u32x2>(smem, vo + vrow), y1 = lds_ld<u32x2>(smem, vo + vrow + 16);
                o.v0 = u32x4{x0[0], x0[1], x1[0], x1[1]};
                o.v1 = u32x4{y0[0], y0[1], y1[0], y1[1]};
                o.c0 = lds_ld<float>(smem, rh + RS * t0);
                o.c1 = lds_ld<float>(smem, rh + RS * (t0 + 1));
                return o;
            };
            f32x16 O, O2;                             // rows t and t+1 of each pair
            auto weighted_sum = [&]() {
                // first: the pair's P.V products start the sums (no zeroed accumulators)
                auto compute = [&](const Ops32& c, auto first) {
                    const f32x16 sc = mma32_k16(c.a, q32, cinit);
                    unsigned pw[8];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float e = j < 2 ? c.c0 : c.c1;
                        pw[2 * j] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sc[4 * j], alpha, e)),
                                                __builtin_amdgcn_exp2f(fmaf(sc[4 * j + 1], alpha, e)));
                        pw[2 * j + 1] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sc[4 * j + 2], alpha, e)),
                                                    __builtin_amdgcn_exp2f(fmaf(sc[4 * j + 3], alpha, e)));
                    }
                    // K order of B (per lane half): columns 4*g2+i, then 8+4*g2+i;
                    // the V^T operand was read in the same order
                    constexpr bool F = decltype(first)::value;
                    O = mma32_k16(__builtin_bit_cast(s16x8, c.v0),
                                  __builtin_bit_cast(s16x8, u32x4{pw[0], pw[1], pw[2], pw[3]}), F ? zero16 : O);
                    O2 = mma32_k16(__builtin_bit_cast(s16x8, c.v1),
                                   __builtin_bit_cast(s16x8, u32x4{pw[4], pw[5], pw[6], pw[7]}), F ? zero16 : O2);
                };
                // pair ts always exists (the block's own rows are in the image)
                Ops32 A = fetch(ts), B = fetch(ts + 2 < thi ? ts + 2 : ts);
                __builtin_amdgcn_sched_barrier(0);
                compute(A, std::true_type{});
                __builtin_amdgcn_sched_barrier(0);
                for (int t = ts + 2; t < thi;) {
                    A = fetch(t + 2 < thi ? t + 2 : t);
                    __builtin_amdgcn_sched_barrier(0);
                    compute(B, std::false_type{});
                    __builtin_amdgcn_sched_barrier(0);
                    t += 2;
                    if (t >= thi) break;
                    B = fetch(t + 2 < thi ? t + 2 : t);
                    __builtin_amdgcn_sched_barrier(0);
                    compute(A, std::false_type{});
                    __builtin_amdgcn_sched_barrier(0);
                    t += 2;
                }
                O += O2;
            };

            weighted_sum();
            float shift = mb;
            if (__any(!(O[8] >= 0x1p-60f))) {
                // exact maximum of the shifted base-2 logits, then shift the
                // stored height terms by it and redo
                float M = -3.0e38f;
                for (int t = ts; t < thi; t += 2) {
                    const f32x16 sc = mma32_k16(lds_ld<s16x8>(smem, kl + rslot(t) * rowb_k), q32, cinit);
                    float m0 = sc[0], m1 = sc[8];
#pragma unroll
                    for (int e = 1; e < 8; ++e) {
                        m0 = fmaxf(m0, sc[e]);
                        m1 = fmaxf(m1, sc[8 + e]);
                    }
                    M = fmaxf(M, fmaxf(fmaf(m0, alpha, lds_ld<float>(smem, rh + RS * t)),
                                       fmaf(m1, alpha, lds_ld<float>(smem, rh + RS * (t + 1)))));
                }
                {
                    float a = M, b = M;
                    swap32(a, b);                         // the query's other lane half
                    M = fmaxf(a, b);
                }
                shift += M;
#pragma unroll
                for (int r2 = 0; r2 < 8; ++r2) {          // window rows 8*g2 .. +7 of the query
                    const unsigned a = rh + RS * (8 * g2 + r2);
                    lds_st<float>(smem, a, lds_ld<float>(smem, a) - M);
                }
                weighted_sum();
            }

            // ---- normalise and pack: rows 0-15 are channels, 16-31 the weight sum
            const float L = O[8];
            if (lse != nullptr) res.lse2[0] = shift + __builtin_amdgcn_logf(L);
            const float inv = __builtin_amdgcn_rcpf(L);
            res.w[0][0] = u32x2{pack_bf16x2(O[0] * inv, O[1] * inv), pack_bf16x2(O[2] * inv, O[3] * inv)};
            res.w[1][0] = u32x2{pack_bf16x2(O[4] * inv, O[5] * inv), pack_bf16x2(O[6] * inv, O[7] * inv)};
      }
    };

    // One group of QT query tiles of block row byy.
    auto do_item = [&](int byy, const Tile& T, const FragT (&qf)[QT], Result& res) {
        if constexpr (G32) {
            do_item32(byy, T, qf, res);
            return;
        }
        const int yb = byy * g.block;
        const int wy0 = yb - g.halo;
        // variants: zero padding keeps every window position (off-image ones
        // are zero rows / columns in LDS); the centred offset moves every
        // table row by -h; the centred mask keeps rows / columns yl..yl+2h
        const bool zpad = VAR && (g.flags & kFlagZeroPad), cmask = VAR && (g.flags & kFlagCentredMask);
        const int coff = VAR ? g.c0 - (R - 1 + g.halo) : 0;
        const int tlo = zpad ? 0 : max(0, -wy0), thi = zpad ? R : min(R, g.H - wy0);
        const int base = yb % ring;                   // ring slot of window row 0

        // ---- relative logits: G = table . Q^T on MFMA (both tables), then
        // re-indexed per query through the scratch (column n of tile u).  One
        // column tile: scratch row = table row, read at row R-1-xl+c.  Two:
        // scratch row = window column / row + 1, written with a clamp to the
        // end rows for table rows no window position uses.  All scratch
        // traffic is this wave's own, and LDS executes one wave's accesses in
        // program order, so no waits are needed between stores and loads.
        f32x4 gw[QT][kRelTiles], gh[QT][kRelTiles];
#pragma unroll
        for (int u = 0; u < QT; ++u)
#pragma unroll
            for (int rt = 0; rt < kRelTiles; ++rt) {
                const FragT aw = NCT == 1 ? tabw[rt] : tab_frag(offrw, rt);
                const FragT ah = NCT == 1 ? tabh[rt] : tab_frag(offrh, rt);
                gw[u][rt] = Frag<D>::mma(aw, qf[u], f32x4{0.f, 0.f, 0.f, 0.f});
                gh[u][rt] = Frag<D>::mma(ah, qf[u], f32x4{0.f, 0.f, 0.f, 0.f});
            }
        // scratch row receiving table row j for a query whose window position
        // 0 sits at table row s0
        auto wrow = [&](int j, int s0) {
            if constexpr (NCT == 1) return j;
            else return min(max(j - s0 + 1, 0), kScrRows - 1);
        };
#pragma unroll
        for (int u = 0; u < QT; ++u) {
            const int sw = R - 1 - T.xl[u] + coff;
#pragma unroll
            for (int rt = 0; rt < kRelTiles; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    lds_st<float>(smem, scr0 + u * scr_u + 4u * kScrStride * wrow(rt * 16 + 4 * gq + i, sw),
                                  gw[u][rt][i]);
        }
        // width term of window column c = 16ct + 4g + i (masked: off-image, c >= R)
        const int clo = zpad ? 0 : g.halo - T.xb, chi = zpad ? R : min(R, g.W - T.xb + g.halo);
        f32x4 cinit[QT][NCT];
#pragma unroll
        for (int u = 0; u < QT; ++u) {
            const int r0 = NCT == 1 ? R - 1 - T.xl[u] + coff : 1;    // scratch row of column 0
            const unsigned a = scr0 + u * scr_u + 4u * kScrStride * (r0 + 4 * gq);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = 16 * ct + 4 * gq + i;
                    const float val = lds_ld<float>(smem, a + 4u * kScrStride * (16 * ct + i));
                    const bool keep = c >= clo && c < chi && (!cmask || (c >= T.xl[u] && c <= T.xl[u] + 2 * g.halo));
                    cinit[u][ct][i] = keep ? val : kMaskLogit;
                }
        }

        // ---- softmax shift: an upper bound on every logit of the query,
        //   sum_c a_c |q_c|,  a_c = max|k_chunk(c)| + max_j |rel_w[j]_c| + max_j |rel_h[j]_c|
        // (|k_chunk(c)|: L2 norm of the 8-channel chunk holding channel c;
        // maxima over the keys staged so far and over all table rows).  As
        // sum_chunks |q_chunk|_1 K_chunk >= sum_chunks |q_chunk|_2 |k_chunk|_2
        // >= q.k, it bounds q.k + q.rel_w[.] + q.rel_h[.] for every key of the
        // window, so exp2 never overflows.  With a_c (rounded up to bf16) in all 16 rows
        // of an MFMA A operand and |q| as B, every lane of a query receives
        // its bound: no cross-lane reduction.  Should the bound overshoot the
        // true maximum so far that the weights' sum falls below 2^-60, the
        // group is redone with the exact maximum.
        FragT abound;
        {
            // this lane's channels gq*KPL .. +KPL-1 lie in chunk gq*KPL/8; the
            // square root gets a relative margin for its rounding
            const float kn = __builtin_sqrtf(__builtin_bit_cast(float, kmax_bits[16 * (byy & 1) + gq * KPL / 8])) *
                             (1.f + 0x1p-20f);
#pragma unroll
            for (int e = 0; e < KPL; ++e) {
                const float a = kn + tmax[gq * KPL + e];
                abound[e] = (short)((__builtin_bit_cast(unsigned, a) + 0xffffu) >> 16);   // round up
            }
        }
        float mb[QT];
#pragma unroll
        for (int u = 0; u < QT; ++u) {
            FragT aq = qf[u];
#pragma unroll
            for (int e = 0; e < KPL; ++e) aq[e] = (short)(aq[e] & 0x7fff);
            const float bound = Frag<D>::mma(abound, aq, f32x4{0.f, 0.f, 0.f, 0.f})[0];
            mb[u] = alpha * (bound + 1e-3f * (1.f + bound));
        }
        // height products, already in shifted base-2 units alpha*G - mb,
        // -> scratch (after the width reads above, in program order)
        unsigned rh0[QT];                             // scratch byte offset of window row 0
#pragma unroll
        for (int u = 0; u < QT; ++u) {
            const int sh = R - 1 - T.yl[u] + coff;
#pragma unroll
            for (int rt = 0; rt < kRelTiles; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = rt * 16 + 4 * gq + i - sh;       // window row of this table row
                    const bool drop = cmask && (t < T.yl[u] || t > T.yl[u] + 2 * g.halo);
                    lds_st<float>(smem, scr0 + u * scr_u + 4u * kScrStride * wrow(rt * 16 + 4 * gq + i, sh),
                                  drop ? -INFINITY : fmaf(gh[u][rt][i], alpha, -mb[u]));
                }
            rh0[u] = scr0 + u * scr_u + 4u * kScrStride * (NCT == 1 ? sh : 1);
        }
        auto rhv = [&](int u, int t) { return lds_ld<float>(smem, rh0[u] + 4u * kScrStride * t); };
        // One column tile: row pairs start at even ring slots, so the second
        // row of a pair is always the next slot (the ring has an even number
        // of rows, the window advances by an even number of rows).  The pair
        // may then begin one row above tlo and end one row past thi-1; those
        // rows get a height term of -inf (weight 0).  Their scratch rows are
        // not otherwise in use once the width terms have been read.
        const int ts = NCT == 1 ? tlo - ((base + tlo) & 1) : tlo;
        if constexpr (NCT == 1) {
#pragma unroll
            for (int u = 0; u < QT; ++u) {
                if (ts < tlo) lds_st<float>(smem, rh0[u] + 4u * kScrStride * ts, -INFINITY);
                if ((thi - ts) & 1) lds_st<float>(smem, rh0[u] + 4u * kScrStride * thi, -INFINITY);
            }
        }

        // lane-constant LDS byte offsets of this lane's K and V^T fragments
        // (column tile ct adds 16 columns; the K swizzle repeats every 16)
        const int kcol = T.wcol0 + n;
        const unsigned kl = (unsigned)kcol * PIXB + (D == 16 ? k_chunk<D>(gq >> 1, kcol) + (gq & 1) * 8
                                                             : k_chunk<D>(gq, kcol));
        const unsigned vl = offv + 2u * ((unsigned)n * CP + T.wcol0 + 4 * gq);
        auto rslot = [&](int t) -> unsigned {         // uniform: ring slot of window row t
            const int s2 = base + t;
            return (unsigned)(s2 >= ring ? s2 - ring : s2);
        };
        auto kload = [&](int t, int ct) -> FragT {
            return lds_ld<FragT>(smem, kl + ct * 16 * PIXB + rslot(t) * rowb_k);
        };
        auto vload = [&](int mt, int t, int ct) -> u32x2 {
            return lds_ld<u32x2>(smem, vl + 2u * ((unsigned)(mt * 16 * CP) + rslot(t) * SWv + 16 * ct));
        };

        // ---- weighted sum: P = exp2(alpha*S + (alpha*rh - mb)) in bf16;
        // O^T += V^T . P^T and L += 1 . P^T, one K=32 step per two score
        // tiles: rows t and t+1 (one column tile, pairs aligned as above)
        // or both column tiles of row t.  Operands of the next
        // step are loaded one step ahead (clamped to the last row).
        constexpr int STEP = NCT == 1 ? 2 : 1;
        f32x4 O[QT][D / 16], L[QT];
        struct Ops {
            FragT a0, a1;
            u32x4 vw[D / 16];
            float c0[QT], c1[QT];
        };
        auto fetch = [&](int t0) {
            Ops o;
            if constexpr (NCT == 1) {                 // rows t0, t0+1: slots s, s+1
                const unsigned ko = kl + rslot(t0) * rowb_k;
                o.a0 = lds_ld<FragT>(smem, ko);
                o.a1 = lds_ld<FragT>(smem, ko + rowb_k);
#pragma unroll
                for (int mt = 0; mt < D / 16; ++mt) {
                    const unsigned vo = vl + 2u * ((unsigned)(mt * 16 * CP) + rslot(t0) * SWv);
                    const u32x2 x0 = lds_ld<u32x2>(smem, vo), x1 = lds_ld<u32x2>(smem, vo + 2u * SWv);
                    o.vw[mt] = u32x4{x0[0], x0[1], x1[0], x1[1]};
                }
#pragma unroll
                for (int u = 0; u < QT; ++u) {
                    const unsigned ro = rh0[u] + 4u * kScrStride * t0;
                    o.c0[u] = lds_ld<float>(smem, ro);
                    o.c1[u] = lds_ld<float>(smem, ro + 4u * kScrStride);
                }
            } else {                                  // row t0, column tiles 0 and 1
                o.a0 = kload(t0, 0);
                o.a1 = kload(t0, 1);
#pragma unroll
                for (int mt = 0; mt < D / 16; ++mt) {
                    const u32x2 x0 = vload(mt, t0, 0), x1 = vload(mt, t0, 1);
                    o.vw[mt] = u32x4{x0[0], x0[1], x1[0], x1[1]};
                }
#pragma unroll
                for (int u = 0; u < QT; ++u) o.c0[u] = o.c1[u] = rhv(u, t0);
            }
            return o;
        };
        auto weighted_sum = [&]() {
#pragma unroll
            for (int u = 0; u < QT; ++u) {
                L[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int mt = 0; mt < D / 16; ++mt) O[u][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            // double-buffered: the operands of the next step are issued before
            // the current step is computed; scheduling barriers keep the
            // compiler from sinking those loads back to their uses
            auto compute = [&](const Ops& c) {
#pragma unroll
                for (int u = 0; u < QT; ++u) {
                    const u32x2 p0 = probs(Frag<D>::mma(c.a0, qf[u], cinit[u][0]), c.c0[u]);
                    const u32x2 p1 = probs(Frag<D>::mma(c.a1, qf[u], cinit[u][NCT - 1]), c.c1[u]);
                    const s16x8 pf = __builtin_bit_cast(s16x8, u32x4{p0[0], p0[1], p1[0], p1[1]});
#pragma unroll
                    for (int mt = 0; mt < D / 16; ++mt)
                        O[u][mt] = mma_k32(__builtin_bit_cast(s16x8, c.vw[mt]), pf, O[u][mt]);
                    L[u] = mma_k32(ones, pf, L[u]);
                }
                if constexpr (QT == 2 && D == 32) {
                    // same idea for 10 MFMAs (two P.V per tile) and 42 VALU
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 11, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 11, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
                }
                if constexpr (QT == 2 && D == 16) {
                    // order the step's 8 MFMAs and 42 VALU instructions so that
                    // the second tile's score MFMAs and the first tile's P.V
                    // MFMAs are issued between exponentials (measured: ~3%)
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);  // VALU
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 11, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 11, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                }
            };
            Ops A = fetch(ts), B;
            for (int t = ts;;) {
                B = fetch(t + STEP < thi ? t + STEP : t);
                __builtin_amdgcn_sched_barrier(0);
                compute(A);
                __builtin_amdgcn_sched_barrier(0);
                t += STEP;
                if (t >= thi) break;
                A = fetch(t + STEP < thi ? t + STEP : t);
                __builtin_amdgcn_sched_barrier(0);
                compute(B);
                __builtin_amdgcn_sched_barrier(0);
                t += STEP;
                if (t >= thi) break;
            }
        };

        float shift[QT];                              // base-2 shift the weights carry
#pragma unroll
        for (int u = 0; u < QT; ++u) shift[u] = mb[u];
        auto need_redo = [&]() {
            bool redo = false;
#pragma unroll
            for (int u = 0; u < QT; ++u) redo |= !(L[u][0] >= 0x1p-60f);
            return __any(redo);
        };
        auto exact_shift = [&]() {
            // exact maximum M of the shifted base-2 logits over the in-image
            // rows, then shift the stored height terms by -M and redo
            float M[QT];
#pragma unroll
            for (int u = 0; u < QT; ++u) M[u] = -3.0e38f;
            for (int t = tlo; t < thi; ++t)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const FragT a = kload(t, ct);
#pragma unroll
                    for (int u = 0; u < QT; ++u)
                        M[u] = fmaxf(M[u], fmaf(max4(Frag<D>::mma(a, qf[u], cinit[u][ct])), alpha, rhv(u, t)));
                }
#pragma unroll
            for (int u = 0; u < QT; ++u) {
                const float m = max_over_rows(M[u]);
                shift[u] += m;
#pragma unroll
                for (int k2 = 0; k2 < NCT; ++k2)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {      // window rows 16k + 4g + i of query n
                        const unsigned a = rh0[u] + 4u * kScrStride * (16 * k2 + 4 * gq + i);
                        lds_st<float>(smem, a, lds_ld<float>(smem, a) - m);
                    }
            }
        };
        if constexpr (D == 32 && NCT == 1) {
            // the second pass reuses the first one's code (a loop with one
            // copy of the weighted sum): fewer registers live (measured: a
            // 36-byte spill down to 8, mid stage -8%)
#pragma clang loop unroll(disable)
            for (int pass = 0;; ++pass) {
                weighted_sum();
                if (pass == 1 || !need_redo()) break;
                exact_shift();
            }
        } else {
            weighted_sum();
            if (need_redo()) {
                exact_shift();
                weighted_sum();
            }
        }

        // ---- normalise and pack
#pragma unroll
        for (int u = 0; u < QT; ++u) {
            if (lse != nullptr) res.lse2[u] = shift[u] + __builtin_amdgcn_logf(L[u][0]);
            const float inv = __builtin_amdgcn_rcpf(L[u][0]);
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt)
                res.w[u][mt] = u32x2{pack_bf16x2(O[u][mt][0] * inv, O[u][mt][1] * inv),
                                     pack_bf16x2(O[u][mt][2] * inv, O[u][mt][3] * inv)};
        }
    };

    const Item my_item = item_of(tid);            // this thread's staging item (fixed)
    FragT qcur[kRingMaxI][QT];
    load_q(0, qcur);
    // Drain these loads now (vmcnt(0)).  Otherwise the first use of qcur
    // inside the block-row loop carries a conservative wait for every vector
    // load in flight, i.e. for the next block row's prefetch.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    for (int by = 0; by < g.nbh; ++by) {
        unsigned* kmax_next = kmax_bits + 16 * ((by + 1) & 1);
        if (tid < 16) atomicMax(&kmax_next[tid], kmax_bits[16 * (by & 1) + tid]);
        // ---- fetch, for the next block row, the window rows it adds (rows
        // past the image bottom are zeros) and its query fragments
        const int nlo = by * g.block + g.block + g.halo;
        const int ntotal = by + 1 < g.nbh ? g.block * ng4 * CPP : 0;
        u32x4 pk[4], pv[4];
        const bool have = tid < ntotal;
        if (have) load_item(my_item, nlo, pk, pv);
        FragT qnext[kRingMaxI][QT];
        load_q(by + 1, qnext);

        // ---- compute this block row.  The next window's new rows go into
        // ring slots the current window does not use, so they are written as
        // soon as the first group is computed: the wait for the prefetch then
        // precedes every output store of the block row (one counter covers
        // vector loads and stores, so a later wait would also wait for the
        // stores to be acknowledged).
        const int f = first_item(by);
        const int it0 = f;
        Result r0;
        Tile T0;
        if (it0 < items) {
            T0 = tile_of(by, it0);
            do_item(by, T0, qcur[0], r0);
        }
        auto stage = [&]() {
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the prefetch and the next queries
            if (have) store_item(my_item, nlo, pk, pv, kmax_next);
            for (int e = tid + kRingThreads; e < ntotal; e += kRingThreads) {
                u32x4 kk[4], vv[4];
                const Item it = item_of(e);
                load_item(it, nlo, kk, vv);
                store_item(it, nlo, kk, vv, kmax_next);
            }
        };
        if (p.midstage) stage();
        if (it0 < items) store_result(T0, r0);
#pragma unroll
        for (int ii = 1; ii < kRingMaxI; ++ii) {
            const int it = f + ii * kRingWaves;
            if (it < items) {
                const Tile T = tile_of(by, it);
                Result r;
                do_item(by, T, qcur[ii], r);
                store_result(T, r);
            }
        }
#pragma unroll
        for (int ii = 0; ii < kRingMaxI; ++ii)
#pragma unroll
            for (int u = 0; u < QT; ++u) qcur[ii][u] = qnext[ii][u];

        if (!p.midstage) {
            // ring of R rows: the new rows replace the ones this window drops
            // once every wave is done with it
            __syncthreads();
            stage();
        }
        __syncthreads();
    }
}

static int rup(int x, int m) { return (x + m - 1) / m * m; }

static int ring_nct(const Geometry& g) { return (g.r + 15) / 16; }

static RingPlan ring_plan(const Geometry& g, int nct, int qt, int waves, int nbx, bool mid)
{
    RingPlan p{};
    p.nbx = nbx;
    p.nstrips = (g.nbw + nbx - 1) / nbx;
    p.SWv = rup(std::max(nbx * g.block + 2 * g.halo, (nbx - 1) * g.block + 16 * nct), 4);
    p.midstage = mid ? 1 : 0;
    p.ring = mid ? g.r + g.block : g.r;
    // V^T channel pitch: at least ring*SWv elements, and (pitch/2) = 4 (mod 64)
    // dwords so the 16 channels of a fragment read land in distinct banks.
    // The 32-query layout (16 channels, one column tile, two query tiles)
    // reads 8 bytes of channel n32 in lanes 0-15 (and bf16 ones in 16-31):
    // pitch/2 = 2 (mod 32) dwords puts those 16 lanes on 32 distinct banks,
    // and the staging stores of chunks 0 and 1 (channels 8 apart) on
    // different banks
    p.CP = p.ring * p.SWv;
    if (g.d == 16 && nct == 1 && qt == 2)
        while (p.CP % 2 || (p.CP / 2) % 32 != 2) ++p.CP;
    else
        while (p.CP % 2 || (p.CP / 2) % 64 != 4) ++p.CP;
    const int side = (g.block + g.stride - 1) / g.stride;
    p.groups = ((side * side + 15) / 16 + qt - 1) / qt;
    const int kb = p.ring * p.SWv * g.d * 2;
    const int vb = g.d * p.CP * 2;
    const int rb = 2 * rel_rows(nct) * g.d * 2;
    const int sb = waves * qt * scr_rows(nct) * kScrStride * 4;
    p.off_v = rup(kb, 16);
    p.off_rel = rup(p.off_v + vb, 16);
    p.off_scr = rup(p.off_rel + rb, 16);
    p.off_kn = rup(p.off_scr + sb, 16);
    // key-chunk norm maxima (2 sets), table maxima, 32 bytes of bf16 ones
    p.off_qt = rup(p.off_kn + 2 * 16 * 4 + g.d * 4 + 32, 16);
    p.lds_bytes = p.off_qt + p.groups * qt * 16 * 16;       // query geometry of a full block
    return p;
}

// LDS a workgroup of `waves` waves may use so that 8 / waves of them share
// a CU (the device limit per workgroup caps it too).
static int ring_lds_limit(int waves)
{
    return std::min(device_info().lds_per_block, kLdsPerCU * waves / 8);
}

static int device_cus() { return device_info().cus; }

// Widest plan that fits in LDS with at least `min_strips` strips per image
// and at most ring_maxi groups per wave per block row, for one ring size, or
// nbx = 0 when even one block column does not fit.
static RingPlan ring_choose1(const Geometry& g, int nct, int qt, int waves, int min_strips, bool mid)
{
    const int limit = ring_lds_limit(waves);
    const int side = (g.block + g.stride - 1) / g.stride;
    const int groups = ((side * side + 15) / 16 + qt - 1) / qt;
    const int nbx_items = ring_maxi(nct) * waves / groups;
    for (int nbx = std::min((g.nbw + min_strips - 1) / min_strips, nbx_items); nbx >= 1; --nbx) {
        if (ring_plan(g, nct, qt, waves, nbx, mid).lds_bytes > limit) continue;
        // as few strips as fit, then equal widths (no narrow remainder strip)
        const int nstrips = (g.nbw + nbx - 1) / nbx;
        return ring_plan(g, nct, qt, waves, (g.nbw + nstrips - 1) / nstrips, mid);
    }
    return RingPlan{};
}

// Expected efficiency of a plan: wave balance (groups per wave on average
// over the most any wave takes) times the share of staged columns in use.
static double ring_score(const Geometry& g, const RingPlan& p, int waves)
{
    if (p.nbx == 0) return 0.0;
    const int items = p.nbx * p.groups;
    const int most = (items + waves - 1) / waves;
    return ((double)items / waves / most) * ((double)p.nbx * g.block / p.SWv);
}

// The ring of R + block rows (staging overlapped with compute, one barrier
// per block row) unless the R-row ring allows a plan that is clearly better.
static RingPlan ring_choose(const Geometry& g, int nct, int qt, int waves, int min_strips = 1)
{
    const RingPlan pm = ring_choose1(g, nct, qt, waves, min_strips, true);
    const RingPlan pr = ring_choose1(g, nct, qt, waves, min_strips, false);
    return ring_score(g, pr, waves) > 1.2 * ring_score(g, pm, waves) ? pr : pm;
}

// Strips per image a 4-wave launch needs for two workgroups on every CU.
static int ring_min_strips4(const Geometry& g)
{
    const int64_t want = 2 * (int64_t)device_cus();
    const int64_t s = (want + g.BH - 1) / g.BH;
    return (int)std::min<int64_t>(std::max<int64_t>(s, 1), g.nbw);
}

// Workgroup size: two 4-wave workgroups per CU overlap one's barrier waits
// with the other's compute, at the price of narrower strips (more halo
// columns staged per useful column).  Take them when the launch has enough
// workgroups to fill both slots of every CU and the price is low.
static int ring_waves(const Geometry& g, int nct, int qt)
{
    if (HALO_RING_FORCE_WAVES == 4)
        return ring_choose(g, nct, qt, 4, ring_min_strips4(g)).nbx ? 4 : 0;
    if (HALO_RING_FORCE_WAVES == 8)
        return ring_choose(g, nct, qt, 8).nbx ? 8 : 0;
    const RingPlan p4 = ring_choose(g, nct, qt, 4, ring_min_strips4(g)), p8 = ring_choose(g, nct, qt, 8);
    if (p8.nbx == 0) return p4.nbx ? 4 : 0;
    if (p4.nbx == 0 || g.BH * p4.nstrips < 2 * (int64_t)device_cus()) return 8;
    const double cost4 = (double)p4.SWv / (p4.nbx * g.block);
    const double cost8 = (double)p8.SWv / (p8.nbx * g.block);
    // measured: the mid-stage shape (d = 32) runs 4% faster on 4 waves at a
    // column-use ratio of 1.2
    return cost4 <= 1.25 * cost8 ? 4 : 8;
}

// Query tiles per group: two when the block's tiles pair up and a window
// row is one column tile, else one (register pressure).
static int ring_qt(const Geometry& g)
{
    const int side = (g.block + g.stride - 1) / g.stride;
    const int tiles = (side * side + 15) / 16;
    return (HALO_RING_QT > 1 && ring_nct(g) == 1 && tiles % HALO_RING_QT == 0) ? HALO_RING_QT : 1;
}

template <int D, int NCT, int QT, int W, bool VAR>
static hipError_t ring_launch_v(const void* q, const void* k, const void* v, const void* rh,
                                const void* rw, void* out, float* lse, const Geometry& g, hipStream_t st)
{
    RingPlan p = W == 4 ? ring_choose(g, NCT, QT, 4, ring_min_strips4(g)) : ring_choose(g, NCT, QT, 8);
    if (p.nbx == 0) return hipErrorInvalidConfiguration;
    p.nwg = g.BH * p.nstrips;
    p.remap_xcd = (p.nwg % 8 == 0) ? 1 : 0;
    p.alpha = (float)((double)g.scale * 1.4426950408889634);
    auto kern = ring_kernel<D, NCT, QT, W, VAR>;
    {
        const hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), p.lds_bytes);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)p.nwg), dim3(64 * W), p.lds_bytes, st,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v,
                       (const __bf16*)rh, (const __bf16*)rw, (__bf16*)out, lse, g, p);
    return hipGetLastError();
}

template <int D, int NCT, int QT, int W>
static hipError_t ring_launch_t(const void* q, const void* k, const void* v, const void* rh,
                                const void* rw, void* out, float* lse, const Geometry& g, hipStream_t st)
{
    return g.flags ? ring_launch_v<D, NCT, QT, W, true>(q, k, v, rh, rw, out, lse, g, st)
                   : ring_launch_v<D, NCT, QT, W, false>(q, k, v, rh, rw, out, lse, g, st);
}

template <int D, int NCT, int QT>
static hipError_t ring_launch_w(const void* q, const void* k, const void* v, const void* rh,
                                const void* rw, void* out, float* lse, const Geometry& g, hipStream_t st)
{
    const int w = ring_waves(g, NCT, QT);
    if (w == 4) return ring_launch_t<D, NCT, QT, 4>(q, k, v, rh, rw, out, lse, g, st);
    if (w == 8) return ring_launch_t<D, NCT, QT, 8>(q, k, v, rh, rw, out, lse, g, st);
    return hipErrorInvalidConfiguration;
}

template <int D>
static hipError_t ring_launch_d(const void* q, const void* k, const void* v, const void* rh,
                                const void* rw, void* out, float* lse, const Geometry& g, hipStream_t st)
{
    if (ring_nct(g) == 2) return ring_launch_w<D, 2, 1>(q, k, v, rh, rw, out, lse, g, st);
    if (ring_qt(g) > 1) return ring_launch_w<D, 1, HALO_RING_QT>(q, k, v, rh, rw, out, lse, g, st);
    return ring_launch_w<D, 1, 1>(q, k, v, rh, rw, out, lse, g, st);
}

bool ring_supported(const Geometry& g)
{
    if (g.r > 32 || (g.d != 16 && g.d != 32) || g.block % 4 != 0) return false;
    if ((int64_t)g.H * g.W >= (int64_t(1) << 31)) return false;   // pixel indices are 32-bit
    return ring_waves(g, ring_nct(g), ring_qt(g)) != 0;
}

hipError_t launch_ring(const void* q, const void* k, const void* v, const void* rh,
                       const void* rw, void* out, float* lse, const Geometry& g, hipStream_t st)
{
    return g.d == 16 ? ring_launch_d<16>(q, k, v, rh, rw, out, lse, g, st)
                     : ring_launch_d<32>(q, k, v, rh, rw, out, lse, g, st);
}

}  // namespace halo
