// Backward pass of halo attention on gfx950 matrix cores (bf16 in, fp32
// accumulate), for windows of at most 16 columns and full blocks.
//
// The pages print no backward; HaloNet's models are trained by gradient
// descent ("Scaling Local Self-Attention for Parameter Efficient Visual
// Backbones", section 4.1), so this is the exact derivative of the forward
// definition (sections 2.1-2.2; logit
//   l = scale * (q.k + q.rel_h[ky - y + c0] + q.rel_w[kx - x + c0])
// as in the HaloAttention module of the pswp.cn blog page, section 4), with
// the forward's per-query log normaliser lse:
//   P = exp(l - lse),  dl = P (dout.v - dout.out),
//   dq = scale sum_keys dl (k + rel_h[row] + rel_w[col]),
//   dk = scale sum_queries dl q,  dv = sum_queries P dout,
//   d rel_h[R] = scale sum dl q over the pairs at row displacement R (d rel_w alike).
//
// One workgroup (4 waves) per (batch, head, block column) walks down the
// column's block rows.  Both tables are staged once.  Per block row:
//  * staging from registers that were loaded during the previous block row:
//    the block's window (K and V as MFMA fragments, K also transposed), Q^T
//    and dout^T of its queries, and dout.out per query;
//  * relative logits of every query against both tables on MFMA, re-indexed
//    per query into a width table (window column -> q.rel_w, masked -1e30
//    off the image or past the window) and a height table (window row ->
//    alpha q.rel_h - lse2, alpha = scale log2 e, lse2 = lse log2 e);
//  * query path (wave per 16-query tile, scores transposed, S^T = K Q^T, so
//    lane (n, g) holds query n and window columns 4g..4g+3 of one row):
//    P = exp2(alpha S^T + height), dP^T = V dout^T, dl = P (dP - D);
//    dq^T += K^T dl^T and, on two more MFMAs against 0/1 operands, the sums
//    of dl over each window row and each window column of the query.  Those
//    sums, re-indexed by table row, give the tables' share of dq (tables^T
//    times sums) and the table gradients (Q^T times sums), both on MFMA with
//    the sums split into bf16 high and low parts; the table gradients stay
//    in registers for the whole walk;
//  * key path (wave per window row, scores in the other orientation,
//    S = Q K^T, so lane (n, g) holds window column n and queries 4g..4g+3):
//    the same P and dl, then dV^T += dout^T P and dK^T += Q^T dl over pairs
//    of query tiles.  The wave owning window row t keeps its sums in
//    registers: row t of one window is row t - block of the next, and block
//    is a multiple of 4, so the same wave owns it.  A row leaves once no
//    later window holds it, as this column's share of that key row; a
//    gather kernel sums, for every key, the shares of the (at most two, for
//    halo < block) block columns whose windows hold it in a fixed order.
// No floating-point atomics anywhere: results are bitwise reproducible.
#include <algorithm>
#include <type_traits>

#include "mfma_util.h"

namespace halo {

constexpr int kBRows = 16;             // LDS window rows (r <= 16)
constexpr int kBCols = 16;             // window columns per row (one MFMA tile, r <= 16)
constexpr int kKtPitch = 264;          // K^T channel pitch (elements, >= 16*16): 132 dwords = 4 (mod 64)
constexpr int kScrStrideB = 20;        // floats per per-wave scratch row
constexpr int kTabRows = 32;           // relative tables padded to 32 rows (2r-1 <= 31)

struct BwdMfmaPlan {
    int nq;                // queries per block (16 * NT)
    int two_phase;         // block columns in two launches: even (phase 0), then odd
    int phase;
    int ncols;             // block columns this launch walks per image
    int qpitch;            // Q^T / dout^T channel pitch (elements)
    int off_v, off_kt, off_tab, off_tabt, off_qt, off_dot, off_rw, off_rh, off_d, off_scr, off_red, lds_bytes;
    int remap_xcd;
    int64_t nwg;
    float alpha;           // scale * log2(e)
};

template <int D>
__device__ inline unsigned bk_chunk(int c, int col)   // same swizzle as the forward ring
{
    if (D == 16) return (unsigned)((c ^ ((col >> 3) & 1)) * 16);
    return (unsigned)((c ^ ((col >> 2) & 3)) * 16);
}

template <typename T>
__device__ inline T bld(const unsigned char* base, unsigned off) { return *reinterpret_cast<const T*>(base + off); }
template <typename T>
__device__ inline void bst(unsigned char* base, unsigned off, T v) { *reinterpret_cast<T*>(base + off) = v; }

// fp32 -> (bf16 high part, bf16 low part) packed pairs: x ~ hi + lo to 2^-16.
__device__ inline void split2(float a, float b, unsigned& hi, unsigned& lo)
{
    hi = pack_bf16x2(a, b);
    const float ah = __builtin_bit_cast(float, hi << 16), bh = __builtin_bit_cast(float, hi & 0xffff0000u);
    lo = pack_bf16x2(a - ah, b - bh);
}

// NT: 16-query tiles per block (1: 4 x 4 queries, 4: 8 x 8 queries).
template <int D, int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 16 ? 2 : 1)))
void bwd_strip_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                      const __bf16* __restrict__ v, const __bf16* __restrict__ rel_h,
                      const __bf16* __restrict__ rel_w, const __bf16* __restrict__ out,
                      const __bf16* __restrict__ dout, const float* __restrict__ lse,
                      __bf16* __restrict__ dq, __bf16* __restrict__ dk, __bf16* __restrict__ dv,
                      float* __restrict__ part_kv, float* __restrict__ part_rel, Geometry g, BwdMfmaPlan p)
{
    constexpr int KPL = D / 4;
    constexpr int CPP = D / 8;                  // 16-byte chunks per pixel
    constexpr unsigned PIXB = D * 2;
    constexpr unsigned ROWB = kBCols * PIXB;    // bytes per K / V row
    constexpr int NQ = 16 * NT;
    constexpr int PX = D == 16 ? 2 : 4;         // pixels per staging item (register budget)
    constexpr int NGX = kBCols / PX;            // items per window row and chunk
    constexpr int KV_ITEMS = kBRows * NGX * CPP;   // staging items (PX pixels x 8 channels): one per thread
    static_assert(KV_ITEMS == 256, "one staging item per thread");
    constexpr int NSLOT = kBRows / 4;           // window rows per wave in the key path
    typedef typename Frag<D>::T FragT;
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, gq = lane >> 4;
    const int r = g.r;
    const float alpha = p.alpha;

    int64_t wg = blockIdx.x;
    if (p.remap_xcd) {
        const int64_t per = p.nwg >> 3;
        wg = (wg & 7) * per + (wg >> 3);
    }
    const int64_t bh = wg / p.ncols;                           // (batch, head)
    const int kcol = (int)(wg - bh * p.ncols);
    const int bx = p.two_phase ? 2 * kcol + p.phase : kcol;     // block column
    const int64_t strip = bh * g.nbw + bx;                     // its share / partial slot
    const int xb = bx * g.block;
    const int wx0 = xb - g.halo;                               // window column origin
    const int clo = max(0, -wx0), chi = min(r, g.W - wx0);     // in-image window columns
    // semantic variants (the forward's flags): zero padding keeps every
    // window position in the softmax (off-image ones are zero in LDS); the
    // centred mask keeps rows / columns yl..yl+2h; the centred offset moves
    // every table row by -h; the half split zeroes table channels
    const bool zpad = g.flags & kFlagZeroPad, cmask = g.flags & kFlagCentredMask;
    const bool half = g.flags & kFlagHalfSplit;
    const int coff = g.c0 - (r - 1 + g.halo);
    const int64_t plane = (int64_t)g.H * g.W * D;
    const int64_t oplane = (int64_t)g.Ho * g.Wo;
    constexpr int SIDE = NT == 1 ? 4 : 8;       // queries per block row / column
    // the query tile this wave owns in the relative and query phases (NT is
    // 1 or 4: at most one per wave)
    const int uown = NT == 4 ? wave : 0;

    // query position of block-local query index qi (row-major over the block's query grid)
    auto qpos = [&](int qi, int& yl, int& xl) {
        const int iy = qi / SIDE;
        yl = iy * g.stride;
        xl = (qi - iy * SIDE) * g.stride;
    };
    // Pixel offsets of query n of tile 0 from the block's first query pixel
    // (lane_q, input resolution) and output pixel (lane_o); tile u lies
    // 16/SIDE query rows further (tile_q, tile_o).  Blocks start at multiples
    // of the stride, so the output pixel of block-local query (iy, ix) is the
    // block's first output pixel + (iy, ix): no division.
    const int lane_q = (n / SIDE) * g.stride * g.W + (n % SIDE) * g.stride;
    const int lane_o = (n / SIDE) * g.Wo + (n % SIDE);
    const int tile_q = (16 / SIDE) * g.stride * g.W, tile_o = (16 / SIDE) * g.Wo;
    auto qpix0 = [&](int byy) -> int64_t { return (int64_t)byy * g.block * g.W + xb; };        // block's first query pixel
    auto opix0 = [&](int byy) -> int64_t { return (int64_t)byy * SIDE * g.Wo + bx * SIDE; };   // its output pixel

    // ------------------------------------------- tables, once per workgroup
    // [32][D] (A operands of table . Q^T) and [D][32] (A operands of tables^T . sums)
    {
        const unsigned short* rhs = reinterpret_cast<const unsigned short*>(rel_h);
        const unsigned short* rws = reinterpret_cast<const unsigned short*>(rel_w);
        const int nrel = 2 * r - 1;
        for (int e = tid; e < kTabRows * D; e += 256) {
            const int row = e / D, c = e - row * D;
            const unsigned short hv = row < nrel && (!half || c < D / 2) ? rhs[row * D + c] : (unsigned short)0;
            const unsigned short wv = row < nrel && (!half || c >= D / 2) ? rws[row * D + c] : (unsigned short)0;
            bst<unsigned short>(smem, p.off_tab + 2u * e, hv);
            bst<unsigned short>(smem, p.off_tab + 2u * (kTabRows * D + e), wv);
            bst<unsigned short>(smem, p.off_tabt + 2u * (c * kTabRows + row), hv);
            bst<unsigned short>(smem, p.off_tabt + 2u * (D * kTabRows + c * kTabRows + row), wv);
        }
    }

    // ------------------------------- inputs of a block row, held in registers
    // K / V: this thread's staging item (window row kv_t, columns
    // PX kv_cx .. +PX-1, channels 8 kv_ch .. +7); queries: the fragments of
    // every query tile (lane n: query 16u+n, channels gq*KPL..) and of the
    // own tile.
    struct Pre {
        u32x4 kk[PX], vv[PX];
        FragT qf[NT], gf[NT], oo;
        float lse2;
    };
    const int kv_ch = tid % CPP, kv_t = (tid / CPP) / NGX, kv_cx = (tid / CPP) % NGX;
    auto prefetch = [&](int byy, Pre& P) {
        const int yb = byy * g.block, wy0 = yb - g.halo;
        {
            const int iy = wy0 + kv_t;
            const __bf16* kb = k + bh * plane;
            const __bf16* vb = v + bh * plane;
#pragma unroll
            for (int j = 0; j < PX; ++j) {
                const int c = PX * kv_cx + j, ix = wx0 + c;
                P.kk[j] = u32x4{0u, 0u, 0u, 0u};
                P.vv[j] = u32x4{0u, 0u, 0u, 0u};
                if (kv_t < r && c < r && iy >= 0 && iy < g.H && ix >= 0 && ix < g.W) {
                    const int64_t off = ((int64_t)iy * g.W + ix) * D + kv_ch * 8;
                    P.kk[j] = *reinterpret_cast<const u32x4*>(kb + off);
                    P.vv[j] = *reinterpret_cast<const u32x4*>(vb + off);
                }
            }
        }
        // uniform block bases plus 32-bit lane offsets
        const __bf16* qb = q + (bh * g.H * g.W + qpix0(byy)) * D;
        const int64_t ob = bh * oplane + opix0(byy);
        const __bf16* gb = dout + ob * D;
        const __bf16* obp = out + ob * D;
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            P.qf[u] = *reinterpret_cast<const FragT*>(qb + ((unsigned)(lane_q + u * tile_q) * D + gq * KPL));
            P.gf[u] = *reinterpret_cast<const FragT*>(gb + ((unsigned)(lane_o + u * tile_o) * D + gq * KPL));
        }
        const unsigned oo = (unsigned)(lane_o + uown * tile_o);
        P.oo = *reinterpret_cast<const FragT*>(obp + (oo * D + gq * KPL));
        P.lse2 = lse[ob + oo] * 1.4426950408889634f;   // base-2
    };

    const unsigned kl = (unsigned)n * PIXB + (D == 16 ? bk_chunk<D>(gq >> 1, n) + (gq & 1) * 8
                                                      : bk_chunk<D>(gq, n));
    auto kfrag = [&](int t) { return bld<FragT>(smem, kl + (unsigned)t * ROWB); };
    auto vfrag = [&](int t) { return bld<FragT>(smem, p.off_v + kl + (unsigned)t * ROWB); };
    const unsigned scr0 = p.off_scr + wave * (kTabRows * kScrStrideB * 4) + 4u * n;
    auto scr = [&](int row) { return scr0 + 4u * kScrStrideB * row; };

    // column-indicator operand: A[m][8g+j] = 1 if window column 4g + (j%4) == m
    u32x4 ecol;
    {
        const unsigned one = (unsigned)0x3F80;
        unsigned w01 = 0, w23 = 0;
        if (n == 4 * gq + 0) w01 |= one;
        if (n == 4 * gq + 1) w01 |= one << 16;
        if (n == 4 * gq + 2) w23 |= one;
        if (n == 4 * gq + 3) w23 |= one << 16;
        ecol = u32x4{w01, w23, w01, w23};
    }

    // table gradients of this wave's queries over the walk: [table][R tile][channel tile]
    f32x4 drelT[2][2][D / 16];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt) drelT[a][b][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // dk^T / dv^T of window rows wave + 4j (lane (n, g): column n, channels
    // 16mt + 4g + i), carried from one block row to the next
    f32x4 akT[NSLOT][D / 16], avT[NSLOT][D / 16];
#pragma unroll
    for (int j = 0; j < NSLOT; ++j)
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt) akT[j][mt] = avT[j][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    Pre P;
    prefetch(0, P);

    for (int by = 0; by < g.nbh; ++by) {
        const int yb = by * g.block;
        const int wy0 = yb - g.halo;                               // window row origin
        const int tlo = max(0, -wy0), thi = min(r, g.H - wy0);     // in-image window rows
        const int qtlo = zpad ? 0 : tlo, qthi = zpad ? r : thi;   // rows in the softmax

        __syncthreads();               // the previous block row is done with LDS

        // ------------------------------------------------------------ staging
        {
            // K, V (swizzled fragment layout) and K^T for window rows 0..kBRows-1,
            // columns 0..15; everything outside the image or the window is zero
            const int t = kv_t, ch = kv_ch;
#pragma unroll
            for (int j = 0; j < PX; ++j) {
                const int c = PX * kv_cx + j;
                bst<u32x4>(smem, (unsigned)t * ROWB + c * PIXB + bk_chunk<D>(ch, c), P.kk[j]);
                bst<u32x4>(smem, p.off_v + (unsigned)t * ROWB + c * PIXB + bk_chunk<D>(ch, c), P.vv[j]);
            }
            // K^T: channel ch*8 + 2w (+1) of the PX columns (PX * 2-byte rows)
            const unsigned base = p.off_kt + 2u * ((unsigned)t * kBCols + PX * kv_cx);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                if constexpr (PX == 4) {
                    const u32x2 lo = {__builtin_amdgcn_perm(P.kk[1][w], P.kk[0][w], 0x05040100u),
                                      __builtin_amdgcn_perm(P.kk[3][w], P.kk[2][w], 0x05040100u)};
                    const u32x2 hi = {__builtin_amdgcn_perm(P.kk[1][w], P.kk[0][w], 0x07060302u),
                                      __builtin_amdgcn_perm(P.kk[3][w], P.kk[2][w], 0x07060302u)};
                    bst<u32x2>(smem, base + 2u * (unsigned)((ch * 8 + 2 * w) * kKtPitch), lo);
                    bst<u32x2>(smem, base + 2u * (unsigned)((ch * 8 + 2 * w + 1) * kKtPitch), hi);
                } else {
                    bst<unsigned>(smem, base + 2u * (unsigned)((ch * 8 + 2 * w) * kKtPitch),
                                  __builtin_amdgcn_perm(P.kk[1][w], P.kk[0][w], 0x05040100u));
                    bst<unsigned>(smem, base + 2u * (unsigned)((ch * 8 + 2 * w + 1) * kKtPitch),
                                  __builtin_amdgcn_perm(P.kk[1][w], P.kk[0][w], 0x07060302u));
                }
            }
        }
        FragT qfa[NT], gfa[NT];
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            qfa[u] = P.qf[u];
            gfa[u] = P.gf[u];
        }
        // the own tile's fragments, picked with wave-uniform selects (no
        // run-time array index)
        FragT qown = P.qf[0], gown = P.gf[0];
#pragma unroll
        for (int u = 1; u < NT; ++u)
            if (uown == u) {
                qown = P.qf[u];
                gown = P.gf[u];
            }
        const float lse2own = P.lse2;
        if (wave < NT) {
            // Q^T and dout^T of the own tile (channel gq*KPL + e, query 16u + n),
            // and D = dout . out of its queries (the four lanes of a query hold
            // a quarter of the channels each)
            float dpart = 0.f;
#pragma unroll
            for (int e = 0; e < KPL; ++e) {
                const unsigned c = gq * KPL + e;
                bst<short>(smem, p.off_qt + 2u * (c * p.qpitch + 16 * uown + n), qown[e]);
                bst<short>(smem, p.off_dot + 2u * (c * p.qpitch + 16 * uown + n), gown[e]);
                dpart = fmaf(__builtin_bit_cast(float, (unsigned)(unsigned short)gown[e] << 16),
                             __builtin_bit_cast(float, (unsigned)(unsigned short)P.oo[e] << 16), dpart);
            }
            const float dsum = sum_over_rows(dpart);
            if (gq == 0) bst<float>(smem, p.off_d + 4u * (16 * uown + n), -dsum);   // stored negated
        }

        // the next block row's inputs, in flight during this one's compute
        if (by + 1 < g.nbh) prefetch(by + 1, P);

        // strided queries, one tile per block: dq is zero at the block's
        // other pixels (the blocks tile the image, so every such pixel is
        // written once; with more tiles a separate pass clears dq first)
        if (NT == 1 && g.stride > 1) {
            constexpr int C4 = D / 4;                       // 8-byte pieces per pixel
            for (int e = tid; e < g.block * g.block * C4; e += 256) {
                const int pix = e / C4, c4 = e - pix * C4;
                const int yy = pix / g.block, xx = pix - yy * g.block;
                if (yy % g.stride || xx % g.stride)
                    *reinterpret_cast<u32x2*>(dq + (bh * g.H * g.W + (int64_t)(yb + yy) * g.W + xb + xx) * D + 4 * c4) =
                        u32x2{0u, 0u};
            }
        }

        // ----------------------------------- relative tables per query tile
        if (wave < NT) {
            const int u = uown;
            const FragT qf = qown;
            int yl, xl;
            qpos(16 * u + n, yl, xl);
            const float lse2 = lse2own;
#pragma unroll
            for (int tab = 0; tab < 2; ++tab) {          // 0: rel_w -> width table, 1: rel_h -> height
                f32x4 gv[2];
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const FragT a = bld<FragT>(smem, p.off_tab + 2u * ((tab == 0 ? kTabRows * D : 0) +
                                                                         (rt * 16 + n) * D + gq * KPL));
                    gv[rt] = Frag<D>::mma(a, qf, f32x4{0.f, 0.f, 0.f, 0.f});
                }
                // scratch row j = table row j, column n = query n
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) bst<float>(smem, scr(rt * 16 + 4 * gq + i), gv[rt][i]);
                // window position w = 4g+i <- table row w - (yl or xl) + r - 1;
                // kept when inside [blo, bhi) (the image, or the whole window
                // under zero padding) and, under the centred mask, within 2h
                // of the query's own position (bitwise tests: no branches)
                const int lo = tab == 0 ? xl : yl;
                const int blo = tab == 0 ? (zpad ? 0 : clo) : qtlo, bhi = tab == 0 ? (zpad ? r : chi) : qthi;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int w = 4 * gq + i;
                    const int row = w - lo + r - 1 + coff;   // in [0, 31) for w < 16
                    const float gval = bld<float>(smem, scr(row));
                    const int keep = (w >= blo) & (w < bhi) & ((int)!cmask | ((w >= lo) & (w <= lo + 2 * g.halo)));
                    if (tab == 0)
                        bst<float>(smem, p.off_rw + 4u * (w * NQ + 16 * u + n), keep ? gval : kMaskLogit);
                    else
                        bst<float>(smem, p.off_rh + 4u * (w * NQ + 16 * u + n), keep ? alpha * gval - lse2 : -INFINITY);
                }
            }
        }
        __syncthreads();

        // ------------------------------------------------------------ query path
        // With one query tile (NT = 1) its row pairs are spread over the four
        // waves and their partial sums added in wave order through LDS;
        // wave 0 then finishes the tile.
        constexpr bool SPLIT = NT == 1;
        if (SPLIT || wave < NT) {
            const int u = uown;
            const FragT qf = qown, gf = gown;
            const float mD = bld<float>(smem, p.off_d + 4u * (16 * u + n));   // -D
            const f32x4 mDn = {mD, mD, mD, mD};         // accumulator start of dP^T: dP - D directly
            f32x4 cinit;
#pragma unroll
            for (int i = 0; i < 4; ++i) cinit[i] = bld<float>(smem, p.off_rw + 4u * ((4 * gq + i) * NQ + 16 * u + n));
            f32x4 dqT[D / 16], ghT = {0.f, 0.f, 0.f, 0.f}, gwT = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt) dqT[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const unsigned ktl = p.off_kt + 2u * ((unsigned)n * kKtPitch + 4 * gq);
            // one K=32 step per two window rows; a last odd row goes alone (its
            // partner's weights and K^T operand are zero)
            auto step = [&](auto two_c, int t0) {
                constexpr bool two = decltype(two_c)::value;
                const int t1 = two ? t0 + 1 : t0;
                const float c0 = bld<float>(smem, p.off_rh + 4u * (t0 * NQ + 16 * u + n));
                const f32x4 s0 = Frag<D>::mma(kfrag(t0), qf, cinit);
                const f32x4 d0 = Frag<D>::mma(vfrag(t0), gf, mDn);     // dP - D
                float l0[4], l1[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 4; ++i) l0[i] = __builtin_amdgcn_exp2f(fmaf(s0[i], alpha, c0)) * d0[i];
                if (two) {
                    const float c1 = bld<float>(smem, p.off_rh + 4u * (t1 * NQ + 16 * u + n));
                    const f32x4 s1 = Frag<D>::mma(kfrag(t1), qf, cinit);
                    const f32x4 d1 = Frag<D>::mma(vfrag(t1), gf, mDn);
#pragma unroll
                    for (int i = 0; i < 4; ++i) l1[i] = __builtin_amdgcn_exp2f(fmaf(s1[i], alpha, c1)) * d1[i];
                }
                const s16x8 lp = __builtin_bit_cast(s16x8, u32x4{pack_bf16x2(l0[0], l0[1]), pack_bf16x2(l0[2], l0[3]),
                                                                 pack_bf16x2(l1[0], l1[1]), pack_bf16x2(l1[2], l1[3])});
#pragma unroll
                for (int mt = 0; mt < D / 16; ++mt) {
                    const unsigned a = ktl + 2u * (unsigned)(mt * 16 * kKtPitch);
                    const u32x2 x0 = bld<u32x2>(smem, a + 2u * (unsigned)(t0 * kBCols));
                    const u32x2 x1 = two ? bld<u32x2>(smem, a + 2u * (unsigned)(t1 * kBCols)) : u32x2{0u, 0u};
                    dqT[mt] = mma_k32(__builtin_bit_cast(s16x8, u32x4{x0[0], x0[1], x1[0], x1[1]}), lp, dqT[mt]);
                }
                const unsigned e0 = n == t0 ? 0x3F803F80u : 0u, e1 = (two && n == t1) ? 0x3F803F80u : 0u;
                ghT = mma_k32(__builtin_bit_cast(s16x8, u32x4{e0, e0, e1, e1}), lp, ghT);
                gwT = mma_k32(__builtin_bit_cast(s16x8, ecol), lp, gwT);
            };
            if constexpr (SPLIT) {
                for (int t0 = qtlo + 2 * wave; t0 < qthi; t0 += 8) {
                    if (t0 + 1 < qthi) step(std::true_type{}, t0);
                    else step(std::false_type{}, t0);
                }
                // lane-major [wave][lane][dq^T tiles, row sums, column sums]
                constexpr int NV = D / 16 + 2;
                const unsigned rbase = p.off_red + 16u * (unsigned)(lane * NV);
#pragma unroll
                for (int mt = 0; mt < D / 16; ++mt)
                    bst<f32x4>(smem, rbase + 16u * (unsigned)(wave * 64 * NV + mt), dqT[mt]);
                bst<f32x4>(smem, rbase + 16u * (unsigned)(wave * 64 * NV + D / 16), ghT);
                bst<f32x4>(smem, rbase + 16u * (unsigned)(wave * 64 * NV + D / 16 + 1), gwT);
                __syncthreads();
                if (wave == 0) {
#pragma unroll
                    for (int w = 1; w < 4; ++w) {
#pragma unroll
                        for (int mt = 0; mt < D / 16; ++mt)
                            dqT[mt] += bld<f32x4>(smem, rbase + 16u * (unsigned)(w * 64 * NV + mt));
                        ghT += bld<f32x4>(smem, rbase + 16u * (unsigned)(w * 64 * NV + D / 16));
                        gwT += bld<f32x4>(smem, rbase + 16u * (unsigned)(w * 64 * NV + D / 16 + 1));
                    }
                }
            } else {
                int t0 = qtlo;
                for (; t0 + 1 < qthi; t0 += 2) step(std::true_type{}, t0);
                if (t0 < qthi) step(std::false_type{}, t0);
            }
          if (!SPLIT || wave == 0) {

            // sums re-indexed by table row (R = w - yl + r - 1 for rows, - xl for
            // columns), zero elsewhere, in this wave's scratch; then
            //   dq^T += table^T . sums  and  drel^T += Q^T . sums^T
            int yl, xl;
            qpos(16 * u + n, yl, xl);
#pragma unroll
            for (int tab = 0; tab < 2; ++tab) {            // 0: rows -> rel_h, 1: columns -> rel_w
                const f32x4 gs = tab == 0 ? ghT : gwT;
                const int sh = (tab == 0 ? yl : xl);
#pragma unroll
                for (int j = 0; j < 8; ++j) bst<float>(smem, scr(8 * gq + j), 0.f);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int w = 4 * gq + i;
                    if (w < r) bst<float>(smem, scr(w - sh + r - 1 + coff), gs[i]);
                }
                // B operand of table^T . sums: lane (n, g) = query n, table rows 8g..8g+7
                float sv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) sv[j] = bld<float>(smem, scr(8 * gq + j));
                unsigned hw[4], lw[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) split2(sv[2 * j], sv[2 * j + 1], hw[j], lw[j]);
                const u32x4 bh4 = {hw[0], hw[1], hw[2], hw[3]}, bl4 = {lw[0], lw[1], lw[2], lw[3]};
                const unsigned tt = p.off_tabt + 2u * ((tab == 0 ? 0 : D * kTabRows) + gq * 8);
#pragma unroll
                for (int mt = 0; mt < D / 16; ++mt) {
                    const s16x8 at = bld<s16x8>(smem, tt + 2u * (unsigned)((mt * 16 + n) * kTabRows));
                    dqT[mt] = mma_k32(at, __builtin_bit_cast(s16x8, bh4), dqT[mt]);
                    dqT[mt] = mma_k32(at, __builtin_bit_cast(s16x8, bl4), dqT[mt]);
                }
                // table gradient: drel^T[c][R] += sum_q Q^T[c][q] sums[R][q]:
                // A = Q^T (lane n': channel, queries 4g'..4g'+3 of tile u),
                // B = sums^T (lane n: table row 16 rt + n, queries 4g..4g+3)
                wave_lds_sync();   // the scratch column reads above are done before the row reads below
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const f32x4 sr = bld<f32x4>(smem, p.off_scr + wave * (kTabRows * kScrStrideB * 4) +
                                                          4u * (kScrStrideB * (rt * 16 + n) + 4 * gq));
                    unsigned h01, l01, h23, l23;
                    split2(sr[0], sr[1], h01, l01);
                    split2(sr[2], sr[3], h23, l23);
                    const s16x4 bhi = __builtin_bit_cast(s16x4, u32x2{h01, h23});
                    const s16x4 blo = __builtin_bit_cast(s16x4, u32x2{l01, l23});
#pragma unroll
                    for (int mt = 0; mt < D / 16; ++mt) {
                        const s16x4 aq = bld<s16x4>(smem, p.off_qt + 2u * ((mt * 16 + n) * p.qpitch + 16 * u + 4 * gq));
                        drelT[tab][rt][mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aq, bhi, drelT[tab][rt][mt], 0, 0, 0);
                        drelT[tab][rt][mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aq, blo, drelT[tab][rt][mt], 0, 0, 0);
                    }
                }
                wave_lds_sync();   // scratch is rewritten by the next table
            }
            // dq = scale * dq^T (lane: query n, channels 16mt + 4g + i)
            __bf16* dp = dq + (bh * g.H * g.W + qpix0(by)) * D + ((unsigned)(lane_q + u * tile_q) * D + gq * 4);
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt)
                *reinterpret_cast<u32x2*>(dp + mt * 16) =
                    u32x2{pack_bf16x2(dqT[mt][0] * g.scale, dqT[mt][1] * g.scale),
                          pack_bf16x2(dqT[mt][2] * g.scale, dqT[mt][3] * g.scale)};
          }
        }

        // the even neighbours' shares of the rows this block row finishes in
        // window slots 0 and 1 (second launch only), in flight during the key
        // path; not where registers are scarcest (d = 16 with 64 queries),
        // which reads them when it needs them
        constexpr bool PRE = !(D == 16 && NT == 4);
        const bool shl = bx >= 1 && n < 2 * g.halo, shr = bx + 1 < g.nbw && n >= g.block;
        f32x4 pk[2][D / 16], pv[2][D / 16];
        auto share_src = [&](int t) {
            const int64_t nb = shl ? strip - 1 : strip + 1;
            const int cn = shl ? n + g.block : n - g.block;
            return part_kv + ((nb * g.H + (wy0 + t)) * r + cn) * (2 * D) + 4 * gq;
        };
        if (PRE && p.phase == 1) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int t = wave + 4 * j;
                if (t < g.block && t >= tlo && t < thi && n >= clo && n < chi && (shl || shr)) {
                    const float* src = share_src(t);
#pragma unroll
                    for (int mt = 0; mt < D / 16; ++mt) {
                        pk[j][mt] = *reinterpret_cast<const f32x4*>(src + 16 * mt);
                        pv[j][mt] = *reinterpret_cast<const f32x4*>(src + D + 16 * mt);
                    }
                }
            }
        }

        // -------------------------------------------------------------- key path
        {
            constexpr int NP = (NT + 1) / 2;             // pairs of query tiles
            // width terms (column n, queries 4g..4g+3 of tile u) and D of those
            // queries, read from LDS per use (register budget)
            auto cw = [&](int u) { return bld<f32x4>(smem, p.off_rw + 4u * (n * NQ + 16 * u + 4 * gq)); };
            auto mDv = [&](int u) { return bld<f32x4>(smem, p.off_d + 4u * (16 * u + 4 * gq)); };   // -D
            // A operands over query pairs: lane n' = channel, queries
            // {4g..4g+3 of u0, of u1}; held in registers, or read from LDS per
            // use where the shares are prefetched (register budget)
            auto pairA = [&](unsigned base, int pr, int mt) {
                const unsigned row = base + 2u * ((mt * 16 + n) * p.qpitch + 4 * gq);
                const u32x2 a0 = bld<u32x2>(smem, row + 2u * (32 * pr));
                u32x2 a1 = {0u, 0u};
                if (2 * pr + 1 < NT) a1 = bld<u32x2>(smem, row + 2u * (32 * pr + 16));
                return __builtin_bit_cast(s16x8, u32x4{a0[0], a0[1], a1[0], a1[1]});
            };
            s16x8 qtA[PRE ? 1 : NP][D / 16], gtA[PRE ? 1 : NP][D / 16];
            if constexpr (!PRE) {
#pragma unroll
                for (int pr = 0; pr < NP; ++pr)
#pragma unroll
                    for (int mt = 0; mt < D / 16; ++mt) {
                        qtA[pr][mt] = pairA(p.off_qt, pr, mt);
                        gtA[pr][mt] = pairA(p.off_dot, pr, mt);
                    }
            }
            // every slot is computed: rows past the window or, without zero
            // padding, off the image have a height term of -inf (weights 0);
            // rows that are neither finished nor carried are never written
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) {
                const int t = wave + 4 * j;
                const FragT kf = kfrag(t), vf = vfrag(t);
#pragma unroll
                for (int pr = 0; pr < NP; ++pr) {
                    unsigned pw[4] = {0u, 0u, 0u, 0u}, lw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int u = 2 * pr + h;
                        if (u >= NT) continue;
                        const f32x4 s = Frag<D>::mma(qfa[u], kf, cw(u));
                        const f32x4 dpv = Frag<D>::mma(gfa[u], vf, mDv(u));   // dP - D
                        const f32x4 c = bld<f32x4>(smem, p.off_rh + 4u * (t * NQ + 16 * u + 4 * gq));
                        float pv[4], lv[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            pv[i] = __builtin_amdgcn_exp2f(fmaf(s[i], alpha, c[i]));
                            lv[i] = pv[i] * dpv[i];
                        }
                        pw[2 * h] = pack_bf16x2(pv[0], pv[1]);
                        pw[2 * h + 1] = pack_bf16x2(pv[2], pv[3]);
                        lw[2 * h] = pack_bf16x2(lv[0], lv[1]);
                        lw[2 * h + 1] = pack_bf16x2(lv[2], lv[3]);
                    }
                    const s16x8 pp = __builtin_bit_cast(s16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
                    const s16x8 lp = __builtin_bit_cast(s16x8, u32x4{lw[0], lw[1], lw[2], lw[3]});
#pragma unroll
                    for (int mt = 0; mt < D / 16; ++mt) {
                        avT[j][mt] = mma_k32(PRE ? pairA(p.off_dot, pr, mt) : gtA[PRE ? 0 : pr][mt], pp, avT[j][mt]);
                        akT[j][mt] = mma_k32(PRE ? pairA(p.off_qt, pr, mt) : qtA[PRE ? 0 : pr][mt], lp, akT[j][mt]);
                    }
                }
            }
        }

        // ------------------------- finished key rows out, the others carried
        // Window row t is in no later window when t < block (the next window
        // starts block rows lower), or in the last block row.  Such a row is
        // this column's sum for key row wy0 + t, for the in-image columns.
        // One launch: every column writes it as its share ([dk(D) | dv(D)]
        // fp32 per window column) for the gather kernel.  Two launches
        // (2 halo <= block, so a key lies in at most two adjacent windows):
        // an even column writes shares only for the window columns an odd
        // neighbour also holds (n < 2h on the left, n >= block on the right)
        // and final dk, dv for the rest; an odd column then adds those
        // shares to its own sums and writes final dk, dv for its whole window.
        {
            const bool last = by + 1 == g.nbh;
#pragma unroll
            for (int j = 0; j < NSLOT; ++j) {
                const int t = wave + 4 * j;
                if ((t < g.block || last) && t >= tlo && t < thi && n >= clo && n < chi) {
                    const int64_t ky = wy0 + t;
                    if (!p.two_phase || (p.phase == 0 && (shl || shr))) {
                        float* dst = part_kv + ((strip * g.H + ky) * r + n) * (2 * D) + 4 * gq;
#pragma unroll
                        for (int mt = 0; mt < D / 16; ++mt) {
                            *reinterpret_cast<f32x4*>(dst + 16 * mt) = akT[j][mt] * g.scale;
                            *reinterpret_cast<f32x4*>(dst + D + 16 * mt) = avT[j][mt];
                        }
                    } else {
                        f32x4 kk4[D / 16], vv4[D / 16];
#pragma unroll
                        for (int mt = 0; mt < D / 16; ++mt) {
                            kk4[mt] = akT[j][mt] * g.scale;
                            vv4[mt] = avT[j][mt];
                        }
                        if (p.phase == 1 && (shl || shr)) {     // the even neighbour's share
                            if (PRE && j < 2 && t < g.block) {   // prefetched
#pragma unroll
                                for (int mt = 0; mt < D / 16; ++mt) {
                                    kk4[mt] += pk[j < 2 ? j : 0][mt];
                                    vv4[mt] += pv[j < 2 ? j : 0][mt];
                                }
                            } else {
                                const float* src = share_src(t);
#pragma unroll
                                for (int mt = 0; mt < D / 16; ++mt) {
                                    kk4[mt] += *reinterpret_cast<const f32x4*>(src + 16 * mt);
                                    vv4[mt] += *reinterpret_cast<const f32x4*>(src + D + 16 * mt);
                                }
                            }
                        }
                        const int64_t o = ((bh * g.H + ky) * g.W + wx0 + n) * D + 4 * gq;
#pragma unroll
                        for (int mt = 0; mt < D / 16; ++mt) {
                            *reinterpret_cast<u32x2*>(dk + o + 16 * mt) =
                                u32x2{pack_bf16x2(kk4[mt][0], kk4[mt][1]), pack_bf16x2(kk4[mt][2], kk4[mt][3])};
                            *reinterpret_cast<u32x2*>(dv + o + 16 * mt) =
                                u32x2{pack_bf16x2(vv4[mt][0], vv4[mt][1]), pack_bf16x2(vv4[mt][2], vv4[mt][3])};
                        }
                    }
                }
            }
            // row t becomes row t - block of the next window: slot j <- j + block/4
            const int m = g.block >> 2;
            if (m == 2) {                  // block 8: plain moves
#pragma unroll
                for (int mt = 0; mt < D / 16; ++mt) {
                    akT[0][mt] = akT[2][mt];
                    avT[0][mt] = avT[2][mt];
                    akT[1][mt] = akT[3][mt];
                    avT[1][mt] = avT[3][mt];
                    akT[2][mt] = avT[2][mt] = akT[3][mt] = avT[3][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            } else
#pragma unroll
            for (int j = 0; j < NSLOT; ++j)
#pragma unroll
                for (int mt = 0; mt < D / 16; ++mt) {
                    f32x4 nk = {0.f, 0.f, 0.f, 0.f}, nv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 1; s < NSLOT; ++s)
                        if (j + s < NSLOT && s == m) {
                            nk = akT[j + s][mt];
                            nv = avT[j + s][mt];
                        }
                    akT[j][mt] = nk;
                    avT[j][mt] = nv;
                }
        }
    }

    // ----------------------------------- the walk's table gradients, once
    __syncthreads();                   // every wave is done with the K / V region
    float* red = reinterpret_cast<float*>(smem);   // [wave][tab][32][D]
#pragma unroll
    for (int tab = 0; tab < 2; ++tab)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i)    // lane (n, g): channel 16mt + 4g + i, table row 16rt + n
                    red[((wave * 2 + tab) * kTabRows + rt * 16 + n) * D + mt * 16 + 4 * gq + i] = drelT[tab][rt][mt][i];
    __syncthreads();
    const int E = (2 * r - 1) * D;
    float* dst = part_rel + strip * 2 * (int64_t)E;
    for (int e = tid; e < 2 * E; e += 256) {
        const int tab = e / E, rr = e - tab * E;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) acc += red[(w * 2 + tab) * kTabRows * D + rr];
        // part layout: table 0 = rel_h (row sums), 1 = rel_w (column sums);
        // half split: the channels a table does not use get no gradient
        const int c = rr % D;
        const bool used = !half || (tab == 0 ? c < D / 2 : c >= D / 2);
        dst[e] = used ? acc * g.scale : 0.f;
    }
}

// dk, dv of every key: the shares of the block columns whose windows hold
// it, summed in increasing column order; one thread per (key, 4 channels).
template <int D>
__global__ __launch_bounds__(256)
void bwd_gather_kernel(const float* __restrict__ part_kv, __bf16* __restrict__ dk, __bf16* __restrict__ dv,
                       Geometry g)
{
    constexpr int G4 = D / 4;
    const int64_t total = g.BH * g.H * g.W * G4;
    // block columns whose window [bx*b - h, bx*b + b + h) holds kx lie
    // within ceil(h/b) columns of kx's own
    const int A = (g.halo + g.block - 1) / g.block;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int c4 = (int)(i % G4);
        const int64_t pix = i / G4;
        const int64_t row = pix / g.W;                 // bh * H + ky
        const int kx = (int)(pix - row * g.W);
        const int64_t bh = row / g.H;
        const int ky = (int)(row - bh * g.H);
        const int bx0 = kx / g.block;
        f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
        for (int bx = max(0, bx0 - A); bx <= min(g.nbw - 1, bx0 + A); ++bx) {
            const int u = kx - (bx * g.block - g.halo);
            if (u < 0 || u >= g.r) continue;
            const float* src = part_kv + (((bh * g.nbw + bx) * g.H + ky) * g.r + u) * (2 * D) + 4 * c4;
            sk += *reinterpret_cast<const f32x4*>(src);
            sv += *reinterpret_cast<const f32x4*>(src + D);
        }
        const int64_t o = pix * D + 4 * c4;
        *reinterpret_cast<u32x2*>(dk + o) = u32x2{pack_bf16x2(sk[0], sk[1]), pack_bf16x2(sk[2], sk[3])};
        *reinterpret_cast<u32x2*>(dv + o) = u32x2{pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3])};
    }
}

static int brup(int x, int m) { return (x + m - 1) / m * m; }

static BwdMfmaPlan bwd_mfma_plan(const Geometry& g)
{
    BwdMfmaPlan p{};
    const int side = g.block / g.stride;
    p.nq = side * side;
    p.qpitch = p.nq + 8;                       // keeps the 8-byte Q^T reads of 16 channels spread
    const int D = g.d;
    const int kb = kBRows * kBCols * D * 2;
    p.off_v = kb;
    p.off_kt = brup(p.off_v + kb, 16);
    p.off_tab = brup(p.off_kt + D * kKtPitch * 2, 16);
    p.off_tabt = brup(p.off_tab + 2 * kTabRows * D * 2, 16);
    p.off_qt = brup(p.off_tabt + 2 * kTabRows * D * 2, 16);
    p.off_dot = brup(p.off_qt + D * p.qpitch * 2, 16);
    p.off_rw = brup(p.off_dot + D * p.qpitch * 2, 16);
    p.off_rh = brup(p.off_rw + kBCols * p.nq * 4, 16);
    p.off_d = brup(p.off_rh + kBRows * p.nq * 4, 16);
    p.off_scr = brup(p.off_d + p.nq * 4, 16);
    p.lds_bytes = p.off_scr + 4 * kTabRows * kScrStrideB * 4;
    // one query tile: the four waves' partial query-path sums
    p.off_red = brup(p.lds_bytes, 16);
    if (p.nq == 16) p.lds_bytes = p.off_red + 4 * 64 * (D / 16 + 2) * 16;
    // the final table reduction reuses the front of LDS (K and V):
    // 4 waves x 2 x 32 x D floats
    p.lds_bytes = std::max(p.lds_bytes, 4 * 2 * kTabRows * D * 4);
    return p;
}

bool bwd_mfma_supported(const Geometry& g, bool bf16)
{
    if (!bf16 || (g.d != 16 && g.d != 32) || g.r > 16) return false;
    if (g.H % g.block || g.W % g.block) return false;          // full blocks only
    const int side = g.block / g.stride;
    if (side % 4) return false;                                // also makes block a multiple of 4
    const int nt = side * side / 16;
    if (nt != 1 && nt != 4) return false;
    if ((int64_t)g.H * g.W * g.d >= (int64_t(1) << 31)) return false;   // 32-bit lane offsets
    return true;
}

// Rows of table-gradient partials the matrix-core backward writes (one per workgroup).
int64_t bwd_mfma_rel_rows(const Geometry& g) { return g.BH * g.nbw; }

// Floats of the per-column dk/dv shares: [BH][nbw][H][r][2d].
int64_t bwd_mfma_kv_floats(const Geometry& g) { return g.BH * g.nbw * (int64_t)g.H * g.r * 2 * g.d; }

template <int D, int NT>
static hipError_t bwd_mfma_t(const void* q, const void* k, const void* v, const void* rh, const void* rw,
                             const void* out, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             float* part_kv, float* part_rel, const Geometry& g, bool two_phase, int phase,
                             hipStream_t st)
{
    BwdMfmaPlan p = bwd_mfma_plan(g);
    p.two_phase = two_phase ? 1 : 0;
    p.phase = phase;
    p.ncols = two_phase ? (g.nbw - phase + 1) / 2 : g.nbw;
    p.nwg = g.BH * p.ncols;
    if (p.nwg == 0) return hipSuccess;
    p.remap_xcd = (p.nwg % 8 == 0) ? 1 : 0;
    p.alpha = (float)((double)g.scale * 1.4426950408889634);
    auto kern = bwd_strip_kernel<D, NT>;
    {
        const hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), p.lds_bytes);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)p.nwg), dim3(256), p.lds_bytes, st,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)rh,
                       (const __bf16*)rw, (const __bf16*)out, (const __bf16*)dout, lse, (__bf16*)dq,
                       (__bf16*)dk, (__bf16*)dv, part_kv, part_rel, g, p);
    return hipGetLastError();
}

// The strip kernel, then the dk/dv shares combined: with 2*halo <= block in
// two launches of the strip kernel (even block columns, then odd ones, which
// add the even columns' shares), otherwise in one launch and a gather.  The
// table partials land in part_rel ([BH*nbw][2][2r-1][d], scaled), ready for
// the fixed-order reduction.
hipError_t launch_zero_bf16(void* p, int64_t n, hipStream_t st);

hipError_t launch_bwd_mfma(const void* q, const void* k, const void* v, const void* rh, const void* rw,
                           const void* out, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           float* part_kv, float* part_rel, const Geometry& g, hipStream_t st)
{
    const int nt = (g.block / g.stride) * (g.block / g.stride) / 16;
    hipError_t e;
    if (g.stride > 1 && nt != 1) {   // dq is zero at the pixels that are not queries
        e = launch_zero_bf16(dq, g.BH * g.H * g.W * g.d, st);
        if (e != hipSuccess) return e;
    }
    const bool two = 2 * g.halo <= g.block;
    auto strip = [&](int phase) {
        if (g.d == 16)
            return nt == 1 ? bwd_mfma_t<16, 1>(q, k, v, rh, rw, out, dout, lse, dq, dk, dv, part_kv, part_rel, g, two,
                                               phase, st)
                           : bwd_mfma_t<16, 4>(q, k, v, rh, rw, out, dout, lse, dq, dk, dv, part_kv, part_rel, g, two,
                                               phase, st);
        return nt == 1 ? bwd_mfma_t<32, 1>(q, k, v, rh, rw, out, dout, lse, dq, dk, dv, part_kv, part_rel, g, two,
                                           phase, st)
                       : bwd_mfma_t<32, 4>(q, k, v, rh, rw, out, dout, lse, dq, dk, dv, part_kv, part_rel, g, two,
                                           phase, st);
    };
    e = strip(0);
    if (e != hipSuccess) return e;
    if (two) return strip(1);
    const int64_t total = g.BH * g.H * g.W * (g.d / 4);
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((total + 255) / 256, 1 << 20));
    if (g.d == 16)
        hipLaunchKernelGGL(bwd_gather_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const float*)part_kv, (__bf16*)dk, (__bf16*)dv, g);
    else
        hipLaunchKernelGGL(bwd_gather_kernel<32>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const float*)part_kv, (__bf16*)dk, (__bf16*)dv, g);
    return hipGetLastError();
}

}  // namespace halo
