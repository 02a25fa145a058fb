// Persistent fused halo-attention forward on gfx950 matrix cores, 16-query
// groups on 16x16 tiles (bf16 in, fp32 accumulate).  The default forward for
// bf16, d in {16, 32}, windows of up to 16 columns, and d = 32 windows of up
// to 20 columns (the 18x18 window of b = 12, h = 3).
//
// Method: "Scaling Local Self-Attention for Parameter Efficient Visual
// Backbones", section 2.2 with Figures 1 and 2 (non-overlapping blocks, halo
// windows padded at the image border, no centred mask, strided queries whose
// windows are the stride-1 ones); relative logits of section 2.1 in the
// per-axis form of appendix A, scaled and indexed as in the HaloAttention
// module on the pswp.cn blog page (section 4):
//   out[q] = sum_key softmax( scale*(q.k + q.rel_h[ky-y+c0] + q.rel_w[kx-x+c0]) ) v[key]
// over the in-image keys of the query's window, c0 = r - 1 + halo.
//
// Why this shape (measured on MI355X): the softmax makes the kernel
// VALU-issue bound -- one FMA, one v_exp_f32 (two FMA issue slots) and half
// a bf16 pack per (query, key) -- while the MFMAs overlap with the VALU work
// of other waves.  So the design spends registers on occupancy (three or
// four waves per SIMD), keeps per-group setup small, and chooses key tiles
// that waste few columns:
//  * PC = 16: a key tile is 16 columns of one window row (windows <= 16
//    wide), two rows per P.V step;
//  * PC = 4: a key tile is a 4x4 patch (4 rows x 4 columns), so a window of
//    18 columns is computed as 20 (1.11x) instead of 32 (1.78x).
// In the S^T = K . Q^T accumulator lane (n, g) holds query n and the tile's
// keys 4g..4g+3: for PC = 16 columns 4g..4g+3 of the row, for PC = 4 row g
// of the patch, columns 0..3.  The width term of those four columns is the
// MFMA accumulator input (the same for every row, loaded once per group);
// the height term (already scaled and shifted) is one scalar per lane and
// tile.
//
// Work decomposition: one workgroup per (image, strip of nbx block columns),
// walking down the block rows.  Window rows of K and V live in an LDS ring;
// every K/V pixel of the strip is read from HBM once.  Either the ring has
// R + block rows and the next block row's rows are written while the
// current one computes (one barrier per block row), or it has R rows and the
// new rows, fetched into registers at the start of the block row, replace
// the dropped ones between two barriers.  Off-image rows are zero rows.
#include <algorithm>
#include <cstdio>
#include <cstdlib>

#include "mfma_util.h"

namespace halo {

struct TilePlan {
    int nstrips;      // column strips per image
    int nbx;          // block columns per strip
    int SWv;          // strip width in pixels (even)
    int ring;         // LDS ring rows (even)
    int CP;           // V^T channel pitch in elements
    int tiles;        // 16-query tiles per full block
    int groups;       // QT-tile groups per full block
    int midstage;     // 1: ring >= R + block rows, next rows staged mid block row
    int jlo;          // first relative-table row any query of a block uses
    int SS;           // scratch floats per query
    int off_v, off_rel, off_scr, off_kn, off_qt, lds_bytes;
    int gmul;         // ceil(2^16 / groups): item / groups = (item * gmul) >> 16 for small items
    int remap_xcd;
    int64_t nwg;
    float alpha;      // scale * log2(e)
};

constexpr int kTileTabTiles = 2;   // 16-row relative-table tiles per group (32 rows from jlo)

template <typename T>
__device__ inline T lds_load(const unsigned char* base, unsigned off)
{
    return *reinterpret_cast<const T*>(base + off);
}
template <typename T>
__device__ inline void lds_store(unsigned char* base, unsigned off, T val)
{
    *reinterpret_cast<T*>(base + off) = val;
}

// Byte offset inside a pixel of 16-byte chunk c, stored at strip column col
// of ring slot `slot` (XOR swizzle, so a fragment read hits distinct banks).
template <int D, int PC>
__device__ inline unsigned tile_chunk(int c, int col, int slot)
{
    if (PC == 4) return (unsigned)((c ^ (slot & 3)) * 16);            // D == 32: 4 chunks per pixel
    if (D == 16) return (unsigned)((c ^ ((col >> 3) & 1)) * 16);
    return (unsigned)((c ^ ((col >> 2) & 3)) * 16);
}

// D: head dim.  PC: columns of a key tile (16 or 4).  NCT: column tiles per
// window row.  NQ: row quads of a window (PC = 4).  QT: 16-query tiles a
// wave carries at once (they share every K and V fragment read from LDS).
// W: waves per workgroup.  WPE: waves per SIMD the register budget targets.
template <int D, int PC, int NCT, int NQ, int QT, int W, int WPE>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(WPE)))
void tile_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                 const __bf16* __restrict__ v, const __bf16* __restrict__ rel_h,
                 const __bf16* __restrict__ rel_w, __bf16* __restrict__ out,
                 float* __restrict__ lse, Geometry g, TilePlan p)
{
    static_assert(PC == 16 || (PC == 4 && D == 32), "4x4 patches are laid out for 32 channels");
    static_assert(PC == 4 || NCT == 1, "one 16-column tile per row");
    constexpr int KPL = D / 4;                 // channels per lane in a QK fragment
    constexpr int CPP = D / 8;                 // 16-byte chunks per pixel
    constexpr unsigned PIXB = D * 2;           // bytes per pixel
    constexpr int kThreads = 64 * W;
    // scratch regions per wave: PC = 16 keeps every tile's height terms in
    // LDS for the whole group; PC = 4 keeps them in registers and reuses one
    constexpr int kScrTiles = PC == 16 ? QT : 1;
    typedef typename Frag<D>::T FragT;
    extern __shared__ __align__(16) unsigned char smem[];

    const int R = g.r;
    const int ring = p.ring, SWv = p.SWv, CP = p.CP;
    const unsigned rowb = (unsigned)SWv * PIXB;          // bytes per K ring row
    const unsigned offv = p.off_v;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, gq = lane >> 4;

    int64_t wg = blockIdx.x;
    if (p.remap_xcd) {   // each XCD takes one contiguous range of (image, strip) items
        const int64_t per = p.nwg >> 3;
        wg = (wg & 7) * per + (wg >> 3);
    }
    const int64_t bh = wg / p.nstrips;
    const int sx = (int)(wg - bh * p.nstrips);
    const int bx_first = sx * p.nbx;
    const int nbx_here = min(p.nbx, g.nbw - bx_first);
    const int sx0 = bx_first * g.block - g.halo;          // strip column 0, image coordinates
    const int64_t plane = (int64_t)g.H * g.W * D;
    const __bf16* kb = k + bh * plane;
    const __bf16* vb = v + bh * plane;
    const int ng2 = SWv / 2;                              // 2-pixel items per row and chunk
    const int side = g.block / g.stride;                  // queries per block side
    const unsigned offrw = p.off_rel, offrh = p.off_rel + 32u * D * 2;

    // ---- zero the K/V area (over-read columns and slots not yet staged must
    // hold finite values); relative tables (32 rows from jlo, zero outside
    // the table) into LDS; the bound maxima; the query geometry of a full
    // block: {yl, xl, yl*W + xl, (yl/s)*Wo + xl/s}, yl = -1 past its queries
    {
        const unsigned words = (unsigned)p.off_v / 16u + (unsigned)(D * CP * 2 + 15) / 16u;
        for (unsigned e = tid; e < words; e += kThreads) lds_store<u32x4>(smem, 16u * e, u32x4{0u, 0u, 0u, 0u});
    }
    for (int e = tid; e < 32 * D; e += kThreads) {
        const int row = p.jlo + e / D;
        const bool in = row >= 0 && row < 2 * R - 1;
        const int src = row * D + e % D;
        lds_store<unsigned short>(smem, offrw + 2u * e,
                                  in ? reinterpret_cast<const unsigned short*>(rel_w)[src] : (unsigned short)0);
        lds_store<unsigned short>(smem, offrh + 2u * e,
                                  in ? reinterpret_cast<const unsigned short*>(rel_h)[src] : (unsigned short)0);
    }
    for (int qi = tid; qi < p.groups * QT * 16; qi += kThreads) {
        const int iy = qi / side, ix = qi - iy * side;
        const bool in = qi < side * side;
        const int yl = iy * g.stride, xl = ix * g.stride;
        lds_store<i32x4>(smem, p.off_qt + 16u * qi,
                         in ? i32x4{yl, xl, yl * g.W + xl, iy * g.Wo + ix} : i32x4{-1, 0, 0, 0});
    }
    unsigned* kmax_bits = reinterpret_cast<unsigned*>(smem + p.off_kn);   // 2 x 16 words
    float* tmax = reinterpret_cast<float*>(smem + p.off_kn + 2 * 16 * 4);  // D floats
    unsigned* tab_bits = reinterpret_cast<unsigned*>(smem + p.off_kn + 2 * 16 * 4 + D * 4);   // 2 x D words
    if (tid < 32) kmax_bits[tid] = 0u;
    if (tid < 2 * D) tab_bits[tid] = 0u;
    __syncthreads();
    // tmax[c] = max_j |rel_w[j][c]| + max_j |rel_h[j][c]| over the whole
    // tables: every thread folds a few entries into LDS maxima (non-negative
    // floats: bit order is value order)
    for (int e = tid; e < (2 * R - 1) * D; e += kThreads) {
        const int c = e % D;
        atomicMax(&tab_bits[c], __builtin_bit_cast(unsigned, fabsf((float)rel_w[e])));
        atomicMax(&tab_bits[D + c], __builtin_bit_cast(unsigned, fabsf((float)rel_h[e])));
    }
    __syncthreads();
    if (tid < D) tmax[tid] = __builtin_bit_cast(float, tab_bits[tid]) + __builtin_bit_cast(float, tab_bits[D + tid]);

    // ---- staging of image rows into the ring.  Item e of a range of rows:
    // 2 adjacent pixels x 8 channels (two 16-byte loads per tensor).  K is
    // stored swizzled; V is transposed in registers into eight 4-byte rows
    // (2 columns of one channel).  Off-image pixels are zero.  The running
    // maxima of |k chunk|^2 feed the softmax shift bound.
    struct Item { int ch, c2, dr; };
    const float rng2 = __builtin_amdgcn_rcpf((float)ng2);
    auto item_of = [&](int e) {                  // e = (dr * ng2 + c2) * CPP + ch
        Item it;
        it.ch = e & (CPP - 1);
        const int rest = e / CPP;
        it.dr = (int)(((float)rest + 0.5f) * rng2);   // exact for rest < 2^16
        it.c2 = rest - it.dr * ng2;
        return it;
    };
    auto load_item = [&](const Item& it, int row0, u32x4 (&kk)[2], u32x4 (&vv)[2]) {
        const int iy = row0 + it.dr;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int ix = sx0 + 2 * it.c2 + j;
            kk[j] = u32x4{0u, 0u, 0u, 0u};
            vv[j] = u32x4{0u, 0u, 0u, 0u};
            if (ix >= 0 && ix < g.W && iy >= 0 && iy < g.H) {
                const int64_t off = ((int64_t)iy * g.W + ix) * D + it.ch * 8;
                kk[j] = *reinterpret_cast<const u32x4*>(kb + off);
                vv[j] = *reinterpret_cast<const u32x4*>(vb + off);
            }
        }
    };
    auto store_item = [&](const Item& it, int row0, const u32x4 (&kk)[2], const u32x4 (&vv)[2], unsigned* kmax) {
        const int iy = row0 + it.dr;
        const int slot = (iy + g.halo + ring) % ring;
        float nmax = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = 2 * it.c2 + j;
            lds_store<u32x4>(smem, (unsigned)slot * rowb + col * PIXB + tile_chunk<D, PC>(it.ch, col, slot), kk[j]);
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
        const unsigned base = offv + 2u * ((unsigned)slot * SWv + 2 * it.c2);
#pragma unroll
        for (int w = 0; w < 4; ++w) {             // channels 2w (low halves), 2w+1 (high)
            const unsigned lo = __builtin_amdgcn_perm(vv[1][w], vv[0][w], 0x05040100u);
            const unsigned hi = __builtin_amdgcn_perm(vv[1][w], vv[0][w], 0x07060302u);
            lds_store<unsigned>(smem, base + 2u * (unsigned)((it.ch * 8 + 2 * w) * CP), lo);
            lds_store<unsigned>(smem, base + 2u * (unsigned)((it.ch * 8 + 2 * w + 1) * CP), hi);
        }
    };

    // prologue: the first window's rows (off-image rows are zeros)
    {
        const int lo = -g.halo;
        const int total = R * ng2 * CPP;
        // two items per thread in flight: both loads issued before the stores
        for (int e = tid; e < total; e += 2 * kThreads) {
            u32x4 kk[2], vv[2], kk2[2], vv2[2];
            const Item it = item_of(e);
            const bool second = e + kThreads < total;
            const Item it2 = item_of(second ? e + kThreads : e);
            load_item(it, lo, kk, vv);
            if (second) load_item(it2, lo, kk2, vv2);
            store_item(it, lo, kk, vv, kmax_bits);
            if (second) store_item(it2, lo, kk2, vv2, kmax_bits);
        }
    }
    __syncthreads();

    const float alpha = p.alpha;
    s16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (short)0x3F80;
    asm volatile("" : "+v"(ones));   // opaque: kept in registers, never rebuilt
    const int items = nbx_here * p.groups;
    const int64_t qbase = bh * plane;
    const int64_t obase = bh * (int64_t)g.Ho * g.Wo;
    // this lane's query row in the wave's scratch regions (one per tile for PC = 16)
    const unsigned scr_n = (unsigned)p.off_scr + 4u * (unsigned)((wave * kScrTiles * 16 + n) * p.SS);
    constexpr unsigned kScrTile = 16u * 4u;   // times SS: bytes per scratch tile region

    // Items (groups of QT tiles) of block row `byy` taken by this wave: the
    // assignment rotates by `items` per block row to balance the waves.
    auto first_item = [&](int byy) {
        const int rot = (int)(((int64_t)byy * items) % W);
        return (wave - rot + W) % W;
    };
    struct Tile {
        int yl, xl;            // lane's query inside the block (full resolution)
        int qpix, opix;        // query pixel in the image, output pixel
        bool qvalid;
    };
    struct Group {
        int xb, wcol0;         // block's first image column, its window's first strip column
        bool two;              // QT == 2: the second tile holds queries
        bool any;              // some lane of the group holds a query
        Tile t[QT];
    };
    // geometry of item `it` (block column it / groups, group it % groups)
    // of block row byy.  Every block uses the query layout of a full block;
    // in a partial block at the image's bottom or right edge the queries
    // outside the image are masked (q read at the block's first pixel,
    // nothing stored).
    auto group_of = [&](int byy, int it) {
        Group G;
        const int j = (int)(((unsigned)it * (unsigned)p.gmul) >> 16);
        const int grp = it - j * p.groups;
        const int yb = byy * g.block;
        G.xb = (bx_first + j) * g.block;
        G.wcol0 = j * g.block;
        const int qb = yb * g.W + G.xb, ob = byy * side * g.Wo + (bx_first + j) * side;
        G.two = QT == 2 && (grp * QT + 1) < p.tiles;
        bool any = false;
#pragma unroll
        for (int u = 0; u < QT; ++u) {
            const i32x4 e = lds_load<i32x4>(smem, p.off_qt + 16u * ((grp * QT + u) * 16 + n));
            const bool in = e[0] >= 0 && yb + e[0] < g.H && G.xb + e[1] < g.W;
            G.t[u].qvalid = in;
            G.t[u].yl = in ? e[0] : 0;
            G.t[u].xl = in ? e[1] : 0;
            G.t[u].qpix = qb + (in ? e[2] : 0);
            G.t[u].opix = ob + e[3];
            any |= in;
        }
        G.any = __any(any);
        return G;
    };
    auto load_q = [&](const Group& G, FragT (&qf)[QT]) {
#pragma unroll
        for (int u = 0; u < QT; ++u)
            qf[u] = *reinterpret_cast<const FragT*>(q + qbase + (int64_t)G.t[u].qpix * D + gq * KPL);
    };

    auto probs = [&](f32x4 s, float c) -> u32x2 {
        return u32x2{pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s[0], alpha, c)),
                                 __builtin_amdgcn_exp2f(fmaf(s[1], alpha, c))),
                     pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s[2], alpha, c)),
                                 __builtin_amdgcn_exp2f(fmaf(s[3], alpha, c)))};
    };

    struct Result {
        u32x2 w[QT][D / 16];
        float lse2[QT];
    };
    auto store_result = [&](const Group& G, const Result& res) {
#pragma unroll
        for (int u = 0; u < QT; ++u) {
            if (!G.t[u].qvalid) continue;
            __bf16* op = out + (obase + G.t[u].opix) * D + gq * 4;
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt) *reinterpret_cast<u32x2*>(op + mt * 16) = res.w[u][mt];
            if (lse != nullptr && gq == 0) lse[obase + G.t[u].opix] = res.lse2[u] * 0.6931471805599453f;
        }
    };

    // softmax-shift bound coefficients of this block row (see do_group)
    FragT abound;
    auto make_abound = [&](int byy) {
        const float kn = __builtin_sqrtf(__builtin_bit_cast(float, kmax_bits[16 * (byy & 1) + gq * KPL / 8])) *
                         (1.f + 0x1p-20f);
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
            const float a = kn + tmax[gq * KPL + e];
            abound[e] = (short)((__builtin_bit_cast(unsigned, a) + 0xffffu) >> 16);   // round up
        }
    };

    // One group: QT tiles of 16 queries of one block of block row byy.
    // Block-row constants: tlo/thi in-image window rows, base ring slot of
    // window row 0.
    auto do_group = [&](int tlo, int thi, int base, const Group& G, const FragT (&qf)[QT], Result& res) {
        const int clo = g.halo - G.xb, chi = min(R, g.W - G.xb + g.halo);   // in-image window columns
        const bool interior = clo <= 0 && chi >= R;
        constexpr int kCols = NCT * PC;

        // ---- per tile: relative logits G = table . Q^T for the 32 table
        // rows from jlo, written to the scratch (query n: entry j - jlo), read
        // back re-indexed by window column (width terms: the MFMA
        // accumulator input) and by window row (height terms, scaled and
        // shifted by the softmax bound).  Masked columns (off the image or
        // past the window) get the mask value in their scratch entries,
        // which no other column of the query reads.  LDS executes one wave's
        // accesses in program order and the scratch is private to the wave,
        // so no waits are needed between the writes and the reads.
        f32x4 cinit[QT][NCT];
        float mb[QT];
        unsigned hbase[QT];                      // scratch byte address of window row 0's height term
        float hq[QT][PC == 4 ? NQ : 1];
#pragma unroll
        for (int u = 0; u < QT; ++u) {
            if (u == 1 && !G.two) {               // no queries: zero weights, no work
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) cinit[u][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
                mb[u] = 0.f;
                hbase[u] = hbase[0];
                if constexpr (PC == 4) {
#pragma unroll
                    for (int rq = 0; rq < NQ; ++rq) hq[u][rq] = -INFINITY;
                }
                continue;
            }
            const unsigned sb = scr_n + (PC == 16 ? (unsigned)u * kScrTile * p.SS : 0u);
            const Tile& T = G.t[u];
            f32x4 gw[kTileTabTiles], gh[kTileTabTiles];
#pragma unroll
            for (int t = 0; t < kTileTabTiles; ++t) {
                const FragT aw = lds_load<FragT>(smem, offrw + 2u * ((16 * t + n) * D + gq * KPL));
                const FragT ah = lds_load<FragT>(smem, offrh + 2u * ((16 * t + n) * D + gq * KPL));
                gw[t] = Frag<D>::mma(aw, qf[u], f32x4{0.f, 0.f, 0.f, 0.f});
                gh[t] = Frag<D>::mma(ah, qf[u], f32x4{0.f, 0.f, 0.f, 0.f});
            }
#pragma unroll
            for (int t = 0; t < kTileTabTiles; ++t) lds_store<f32x4>(smem, sb + 4u * (16 * t + 4 * gq), gw[t]);
            // window column c is c - halo - xl columns from the query: table
            // row c - halo - xl + c0, scratch entry c + cw
            const unsigned wbase = sb + 4u * (unsigned)(g.c0 - g.halo - p.jlo - T.xl);
            if (interior) {
                for (int c = R + gq; c < kCols; c += 4) lds_store<float>(smem, wbase + 4u * c, kMaskLogit);
            } else {
                for (int c = gq; c < kCols; c += 4)
                    if (c < clo || c >= chi) lds_store<float>(smem, wbase + 4u * c, kMaskLogit);
            }
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = PC == 16 ? 4 * gq + i : 4 * ct + i;
                    cinit[u][ct][i] = lds_load<float>(smem, wbase + 4u * c);
                }
            // softmax shift: an upper bound on every logit of the query,
            //   sum_c a_c |q_c|,  a_c = max|k_chunk(c)| + max_j |rel_w[j]_c| + max_j |rel_h[j]_c|
            // (|k_chunk(c)|: L2 norm of the 8-channel chunk holding channel c,
            // maximum over the keys staged so far; tables over all rows).  As
            // sum_chunks |q_chunk|_1 K_chunk >= sum_chunks |q_chunk|_2 |k_chunk|_2
            // >= q.k, it bounds every logit of the window, so exp2 cannot
            // overflow.  With a_c (rounded up to bf16) in all 16 rows of an
            // MFMA A operand and |q| as B, every lane of a query receives its
            // bound.  Should the bound overshoot the true maximum so far that
            // the weight sum falls below 2^-60, the group is redone with the
            // exact maximum.
            {
                FragT aq = qf[u];
#pragma unroll
                for (int e = 0; e < KPL; ++e) aq[e] = (short)(aq[e] & 0x7fff);
                const float bound = Frag<D>::mma(abound, aq, f32x4{0.f, 0.f, 0.f, 0.f})[0];
                mb[u] = alpha * (bound + 1e-3f * (1.f + bound));
            }
            // height terms alpha*G - mb (after the width reads)
#pragma unroll
            for (int t = 0; t < kTileTabTiles; ++t) {
                f32x4 hv;
#pragma unroll
                for (int i = 0; i < 4; ++i) hv[i] = fmaf(gh[t][i], alpha, -mb[u]);
                lds_store<f32x4>(smem, sb + 4u * (16 * t + 4 * gq), hv);
            }
            hbase[u] = sb + 4u * (unsigned)(g.c0 - g.halo - p.jlo - T.yl);
            if constexpr (PC == 4) {
#pragma unroll
                for (int rq = 0; rq < NQ; ++rq) {
                    const int t = 4 * rq + gq;
                    const float hvv = lds_load<float>(smem, hbase[u] + 4u * t);
                    hq[u][rq] = (t >= tlo && t < thi) ? hvv : -INFINITY;
                }
            }
        }

        f32x4 O[QT][D / 16], L[QT];
        float shift[QT];
#pragma unroll
        for (int u = 0; u < QT; ++u) shift[u] = mb[u];
        auto need_redo = [&]() {
            bool redo = false;
#pragma unroll
            for (int u = 0; u < QT; ++u) redo |= !(L[u][0] >= 0x1p-60f) && (u == 0 || G.two);
            return __any(redo);
        };

        if constexpr (PC == 16) {
            // ---- rows in pairs starting at even ring slots (the ring has an
            // even number of rows and the window moves by an even number), so
            // the pair's second row is the next slot; a pair may begin one row
            // above tlo and end one past thi-1: those rows get a height term of
            // -inf.  Their scratch entries are free once the width terms are read.
            const int ts = tlo - ((base + tlo) & 1);
#pragma unroll
            for (int u = 0; u < QT; ++u) {
                if (ts < tlo) lds_store<float>(smem, hbase[u] + 4u * ts, -INFINITY);
                if ((thi - ts) & 1) lds_store<float>(smem, hbase[u] + 4u * thi, -INFINITY);
            }
            const int kcol = G.wcol0 + n;
            const unsigned kl = (unsigned)kcol * PIXB + (D == 16 ? tile_chunk<D, PC>(gq >> 1, kcol, 0) + (gq & 1) * 8
                                                                 : tile_chunk<D, PC>(gq, kcol, 0));
            const unsigned vl = offv + 2u * ((unsigned)n * CP + G.wcol0 + 4 * gq);
            auto rslot = [&](int t) -> unsigned {
                const int s2 = base + t;
                return (unsigned)(s2 >= ring ? s2 - ring : s2);
            };
            struct Ops {
                FragT a0, a1;
                u32x4 vw[D / 16];
                float c0[QT], c1[QT];
            };
            auto fetch = [&](int t0) {
                Ops o;
                const unsigned sl = rslot(t0);
                const unsigned ko = kl + sl * rowb;
                o.a0 = lds_load<FragT>(smem, ko);
                o.a1 = lds_load<FragT>(smem, ko + rowb);
#pragma unroll
                for (int mt = 0; mt < D / 16; ++mt) {
                    const unsigned vo = vl + 2u * ((unsigned)(mt * 16 * CP) + sl * SWv);
                    const u32x2 x0 = lds_load<u32x2>(smem, vo), x1 = lds_load<u32x2>(smem, vo + 2u * SWv);
                    o.vw[mt] = u32x4{x0[0], x0[1], x1[0], x1[1]};
                }
#pragma unroll
                for (int u = 0; u < QT; ++u) {
                    o.c0[u] = lds_load<float>(smem, hbase[u] + 4u * t0);
                    o.c1[u] = lds_load<float>(smem, hbase[u] + 4u * (t0 + 1));
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
                auto compute = [&](const Ops& c) {
#pragma unroll
                    for (int u = 0; u < QT; ++u) {
                        if (u == 1 && !G.two) continue;
                        const u32x2 p0 = probs(Frag<D>::mma(c.a0, qf[u], cinit[u][0]), c.c0[u]);
                        const u32x2 p1 = probs(Frag<D>::mma(c.a1, qf[u], cinit[u][0]), c.c1[u]);
                        const s16x8 pf = __builtin_bit_cast(s16x8, u32x4{p0[0], p0[1], p1[0], p1[1]});
#pragma unroll
                        for (int mt = 0; mt < D / 16; ++mt)
                            O[u][mt] = mma_k32(__builtin_bit_cast(s16x8, c.vw[mt]), pf, O[u][mt]);
                        L[u] = mma_k32(ones, pf, L[u]);
                    }
                };
                Ops A = fetch(ts), B;
                for (int t = ts;;) {
                    B = fetch(t + 2 < thi ? t + 2 : t);
                    __builtin_amdgcn_sched_barrier(0);
                    compute(A);
                    __builtin_amdgcn_sched_barrier(0);
                    t += 2;
                    if (t >= thi) break;
                    A = fetch(t + 2 < thi ? t + 2 : t);
                    __builtin_amdgcn_sched_barrier(0);
                    compute(B);
                    __builtin_amdgcn_sched_barrier(0);
                    t += 2;
                    if (t >= thi) break;
                }
            };
            auto exact_shift = [&]() {
                float M[QT];
#pragma unroll
                for (int u = 0; u < QT; ++u) M[u] = -3.0e38f;
                for (int t = tlo; t < thi; ++t) {
                    const FragT a = lds_load<FragT>(smem, kl + rslot(t) * rowb);
#pragma unroll
                    for (int u = 0; u < QT; ++u)
                        if (u == 0 || G.two)
                            M[u] = fmaxf(M[u], fmaf(max4(Frag<D>::mma(a, qf[u], cinit[u][0])), alpha,
                                                lds_load<float>(smem, hbase[u] + 4u * t)));
                }
#pragma unroll
                for (int u = 0; u < QT; ++u) {
                    if (u == 1 && !G.two) continue;     // its scratch is not its own
                    const float m = max_over_rows(M[u]);
                    shift[u] += m;
                    for (int t = gq; t < R + 1; t += 4) {      // this query's height terms, shared by its lanes
                        const unsigned a = hbase[u] + 4u * t;
                        lds_store<float>(smem, a, lds_load<float>(smem, a) - m);
                    }
                }
            };
#pragma clang loop unroll(disable)
            for (int pass = 0;; ++pass) {
                weighted_sum();
                if (pass == 1 || !need_redo()) break;
                exact_shift();
            }
        } else {
            // ---- 4x4 patches: tile (quad rq, column tile ct) holds rows
            // 4rq..4rq+3 and columns 4ct..4ct+3 of the window.  Key n of the
            // tile (A operand row) is row n >> 2, column n & 3; result lane
            // (n, g) holds row g, columns 0..3.  Rows outside the image or
            // past the window have a height term of -inf (their ring slots
            // hold finite data).  Two tiles per P.V step.
            // the ring has a multiple of 4 rows and window row 0 sits at a
            // slot multiple of 4, so a quad's rows are 4 consecutive slots:
            // address = slot of its first row (uniform) + a lane constant
            // (row n >> 2 for K, row g for V^T; the K swizzle uses slot & 3 = row)
            const unsigned kl = (unsigned)(n >> 2) * rowb + (unsigned)(G.wcol0 + (n & 3)) * PIXB +
                                tile_chunk<D, PC>(gq, 0, n >> 2);
            const unsigned vl = offv + 2u * ((unsigned)n * CP + (unsigned)gq * SWv + G.wcol0);
            auto qslot = [&](int rq) -> unsigned {
                const int s2 = base + 4 * rq;
                return (unsigned)(s2 >= ring ? s2 - ring : s2);
            };
            constexpr int NT = NQ * NCT;               // tiles
            constexpr int NS = (NT + 1) / 2;           // P.V steps
            // software pipeline over the fully unrolled steps: the K
            // fragments of step s+2 and the V fragments of step s+1 are
            // loaded, and the scores of step s+1 computed, before step s's
            // exponentials, so a wave overlaps its own MFMA and LDS latency
            FragT kf[NS][2];
            u32x4 vf[NS][D / 16];
            f32x4 sc[NS][QT][2];
            auto kfetch = [&](int st) {
                const int t0 = 2 * st, t1 = 2 * st + 1 < NT ? 2 * st + 1 : 2 * st;
                kf[st][0] = lds_load<FragT>(smem, kl + qslot(t0 / NCT) * rowb + 4u * (t0 % NCT) * PIXB);
                kf[st][1] = lds_load<FragT>(smem, kl + qslot(t1 / NCT) * rowb + 4u * (t1 % NCT) * PIXB);
            };
            auto vfetch = [&](int st) {
                const int t0 = 2 * st, t1 = 2 * st + 1 < NT ? 2 * st + 1 : 2 * st;
                const unsigned s0 = qslot(t0 / NCT), s1 = qslot(t1 / NCT);
#pragma unroll
                for (int mt = 0; mt < D / 16; ++mt) {
                    const u32x2 x0 = lds_load<u32x2>(smem, vl + 2u * (s0 * SWv + (unsigned)(mt * 16 * CP + 4 * (t0 % NCT))));
                    const u32x2 x1 = lds_load<u32x2>(smem, vl + 2u * (s1 * SWv + (unsigned)(mt * 16 * CP + 4 * (t1 % NCT))));
                    vf[st][mt] = u32x4{x0[0], x0[1], x1[0], x1[1]};
                }
            };
            auto scores = [&](int st) {
                const int t0 = 2 * st, t1 = 2 * st + 1;
#pragma unroll
                for (int u = 0; u < QT; ++u) {
                    if (u == 1 && !G.two) continue;
                    sc[st][u][0] = Frag<D>::mma(kf[st][0], qf[u], cinit[u][t0 % NCT]);
                    if (t1 < NT) sc[st][u][1] = Frag<D>::mma(kf[st][1], qf[u], cinit[u][t1 % NCT]);
                }
            };
            auto weighted_sum = [&]() {
#pragma unroll
                for (int u = 0; u < QT; ++u) {
                    L[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int mt = 0; mt < D / 16; ++mt) O[u][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
                kfetch(0);
                if (NS > 1) kfetch(1);
                vfetch(0);
                scores(0);
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    if (st + 2 < NS) kfetch(st + 2);
                    if (st + 1 < NS) vfetch(st + 1);
                    if (st + 1 < NS) scores(st + 1);
                    __builtin_amdgcn_sched_barrier(0);
                    const int t0 = 2 * st, t1 = 2 * st + 1;
#pragma unroll
                    for (int u = 0; u < QT; ++u) {
                        if (u == 1 && !G.two) continue;
                        const u32x2 p0 = probs(sc[st][u][0], hq[u][t0 / NCT]);
                        u32x2 p1 = u32x2{0u, 0u};
                        if (t1 < NT) p1 = probs(sc[st][u][1], hq[u][t1 / NCT]);
                        const s16x8 pf = __builtin_bit_cast(s16x8, u32x4{p0[0], p0[1], p1[0], p1[1]});
#pragma unroll
                        for (int mt = 0; mt < D / 16; ++mt)
                            O[u][mt] = mma_k32(__builtin_bit_cast(s16x8, vf[st][mt]), pf, O[u][mt]);
                        L[u] = mma_k32(ones, pf, L[u]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            auto exact_shift = [&]() {
                float M[QT];
#pragma unroll
                for (int u = 0; u < QT; ++u) M[u] = -3.0e38f;
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const FragT a = lds_load<FragT>(smem, kl + qslot(t / NCT) * rowb + 4u * (t % NCT) * PIXB);
#pragma unroll
                    for (int u = 0; u < QT; ++u)
                        if (u == 0 || G.two)
                            M[u] = fmaxf(M[u], fmaf(max4(Frag<D>::mma(a, qf[u], cinit[u][t % NCT])), alpha, hq[u][t / NCT]));
                }
#pragma unroll
                for (int u = 0; u < QT; ++u) {
                    const float m = max_over_rows(M[u]);
                    shift[u] += m;
#pragma unroll
                    for (int rq = 0; rq < NQ; ++rq) hq[u][rq] -= m;
                }
            };
#pragma clang loop unroll(disable)
            for (int pass = 0;; ++pass) {
                weighted_sum();
                if (pass == 1 || !need_redo()) break;
                exact_shift();
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

    // ---- the walk down the block rows.  A wave takes items f, f + W, ...
    // of every block row (item = block column * groups + group).
    const int my_e = tid;                             // this thread's first staging item
    FragT qcur[QT];
    Group Gcur = group_of(0, min(first_item(0), items - 1));
    load_q(Gcur, qcur);
    __builtin_amdgcn_s_waitcnt(0x0F70);               // vmcnt(0)
    for (int by = 0; by < g.nbh; ++by) {
        unsigned* kmax_next = kmax_bits + 16 * ((by + 1) & 1);
        if (tid < 16) atomicMax(&kmax_next[tid], kmax_bits[16 * (by & 1) + tid]);
        make_abound(by);
        const int yb = by * g.block;
        const int tlo = max(0, g.halo - yb), thi = min(R, g.H - yb + g.halo);   // in-image window rows
        const int base = yb % ring;                   // ring slot of window row 0
        // ---- fetch the next block row's new window rows (first item per
        // thread into registers; rows past the image are zeros)
        const int nlo = yb + g.block + g.halo;
        const int ntotal = by + 1 < g.nbh ? g.block * ng2 * CPP : 0;
        u32x4 pk[2], pv[2];
        const bool have = my_e < ntotal;
        Item my_it{};
        if (have) {
            my_it = item_of(my_e);
            load_item(my_it, nlo, pk, pv);
        }
        auto stage = [&]() {
            __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0)
            if (have) store_item(my_it, nlo, pk, pv, kmax_next);
            for (int e = my_e + kThreads; e < ntotal; e += kThreads) {
                u32x4 kk[2], vv[2];
                const Item it = item_of(e);
                load_item(it, nlo, kk, vv);
                store_item(it, nlo, kk, vv, kmax_next);
            }
        };
        const int f = first_item(by);
        bool staged = false;
        for (int it = f; it < items; it += W) {
            const Group G = Gcur;
            // the next item's geometry and query fragments (this block row or the next)
            FragT qn[QT];
            if (it + W < items) Gcur = group_of(by, it + W);
            else if (by + 1 < g.nbh) Gcur = group_of(by + 1, min(first_item(by + 1), items - 1));
            load_q(Gcur, qn);
            if (G.any) {
                Result r;
                do_group(tlo, thi, base, G, qcur, r);
                if (p.midstage && !staged) {
                    stage();
                    staged = true;
                }
                store_result(G, r);
            }
#pragma unroll
            for (int u = 0; u < QT; ++u) qcur[u] = qn[u];
        }
        if (f >= items && by + 1 < g.nbh) {           // a wave with no item this block row
            Gcur = group_of(by + 1, min(first_item(by + 1), items - 1));
            load_q(Gcur, qcur);
        }
        if (p.midstage) {
            if (!staged) stage();
        } else {
            // the thread's further staging items: loads issued before the
            // barrier (the compute registers are free here), so their latency
            // overlaps the wait for the other waves' last items
            constexpr int kMore = 2;
            u32x4 mk[kMore][2], mv[kMore][2];
            Item mit[kMore];
            bool mh[kMore];
#pragma unroll
            for (int j = 0; j < kMore; ++j) {
                const int e = my_e + (j + 1) * kThreads;
                mh[j] = e < ntotal;
                if (mh[j]) {
                    mit[j] = item_of(e);
                    load_item(mit[j], nlo, mk[j], mv[j]);
                }
            }
            __syncthreads();
            __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0)
            if (have) store_item(my_it, nlo, pk, pv, kmax_next);
#pragma unroll
            for (int j = 0; j < kMore; ++j)
                if (mh[j]) store_item(mit[j], nlo, mk[j], mv[j], kmax_next);
            for (int e = my_e + (kMore + 1) * kThreads; e < ntotal; e += kThreads) {
                u32x4 kk[2], vv[2];
                const Item it = item_of(e);
                load_item(it, nlo, kk, vv);
                store_item(it, nlo, kk, vv, kmax_next);
            }
        }
        __syncthreads();
    }
}

static int rup(int x, int m) { return (x + m - 1) / m * m; }

// Relative-table rows a block's queries use, from jlo: the largest query
// offset (block - stride) plus the window extent the tiles compute, plus
// the spare row below for PC = 16.
static int tile_rows_needed(const Geometry& g, int pc, int nct)
{
    const int cols = nct * pc;
    const int rows = pc == 16 ? g.r + 1 : rup(g.r, 4);
    return (pc == 16 ? 1 : 0) + g.block - g.stride + std::max(cols, rows);
}

static TilePlan tile_plan(const Geometry& g, int pc, int nct, int qt, int waves, int nbx, bool mid)
{
    TilePlan p{};
    p.nbx = nbx;
    p.nstrips = (g.nbw + nbx - 1) / nbx;
    // strip width: a multiple of 4 plus 2, so the V^T rows of a quad's two
    // lane halves fall in different banks (pitch / 2 = 2 mod 4 dwords);
    // pixels a tile reads past a row come from the next slot (finite data)
    p.SWv = nbx * g.block + 2 * g.halo;
    p.SWv = rup(p.SWv, 2);
    if (pc == 4)
        while (p.SWv % 8 != 4) p.SWv += 2;
    p.midstage = mid ? 1 : 0;
    p.ring = rup(mid ? g.r + g.block : g.r, pc == 4 ? 4 : 2);
    const int over = std::max(0, (nbx - 1) * g.block + nct * pc - p.SWv);   // pixels read past a row
    // V^T channel pitch: >= ring*SWv + over-read, = 2 (mod 8) dwords.  LDS
    // serves 8-byte reads 16 lanes per pass over 32 banks of 4 bytes: the 16
    // channels of a fragment read (lanes 0-15, and 16-31 one slot on) then
    // start 2*odd dwords apart and cover the 32 banks once
    p.CP = rup(p.ring * p.SWv + over, 2);
    while ((p.CP / 2) % 8 != 2 || p.CP % 2) ++p.CP;
    const int side = g.block / g.stride;
    p.tiles = (side * side + 15) / 16;
    p.groups = (p.tiles + qt - 1) / qt;
    p.gmul = (65536 + p.groups - 1) / p.groups;
    // the smallest displacement a block's queries meet is -(halo + block -
    // stride) (table row c0 - halo - block + stride); one spare row below
    // for PC = 16: a row pair may start one row above the window
    p.jlo = g.c0 - g.halo - (g.block - g.stride) - (pc == 16 ? 1 : 0);
    // scratch: 32 entries written by the relative MFMAs; 36 = 4 x odd keeps
    // the 16 queries' rows in distinct banks
    p.SS = 36;
    const int scr_tiles = pc == 16 ? qt : 1;
    const int kb = p.ring * p.SWv * g.d * 2 + over * g.d * 2;
    const int vb = g.d * p.CP * 2;
    p.off_v = rup(kb, 16);
    p.off_rel = rup(p.off_v + vb, 16);
    p.off_scr = p.off_rel + 2 * 32 * g.d * 2;
    p.off_qt = rup(p.off_scr + waves * scr_tiles * 16 * p.SS * 4, 16);
    p.off_kn = p.off_qt + p.groups * qt * 16 * 16;
    p.lds_bytes = p.off_kn + 2 * 16 * 4 + 3 * g.d * 4;   // chunk-norm maxima, tmax, table maxima
    return p;
}

template <int D, int PC, int NCT, int NQ, int QT, int W, int WPE>
static hipError_t tile_launch(const void* q, const void* k, const void* v, const void* rh, const void* rw,
                              void* out, float* lse, const Geometry& g, const TilePlan& plan, hipStream_t st)
{
    TilePlan p = plan;
    p.nwg = g.BH * p.nstrips;
    p.remap_xcd = (p.nwg % 8 == 0) ? 1 : 0;
    p.alpha = (float)((double)g.scale * 1.4426950408889634);
    auto kern = tile_kernel<D, PC, NCT, NQ, QT, W, WPE>;
    {
        const hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), p.lds_bytes);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)p.nwg), dim3(64 * W), p.lds_bytes, st,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v,
                       (const __bf16*)rh, (const __bf16*)rw, (__bf16*)out, lse, g, p);
    return hipGetLastError();
}

// Plan of a shape: tile shape, query tiles per group, waves per workgroup,
// workgroups per CU (their LDS share) and strip width, chosen for whole
// waves of workgroups over the chip and balanced groups per wave; 0 waves
// when nothing fits.
struct TileChoice {
    int waves, per_cu, pc, nct, qt;
    TilePlan plan;
};

#ifndef HALO_TILE_ROWS
#define HALO_TILE_ROWS 0   // 1: also take windows of <= 16 columns (16-column row tiles)
#endif

static bool tile_shape(const Geometry& g, int& pc, int& nct, int& qt)
{
    if (g.r <= 16) {
        if (!HALO_TILE_ROWS) return false;
        pc = 16;
        nct = 1;
    } else if (g.d == 32 && g.r <= 20) {
        pc = 4;
        nct = 5;
    } else {
        return false;
    }
    // two query tiles per wave step where a block has them and the
    // registers allow (4x4 patches need one tile's 5 width vectors)
    const int side = g.block / g.stride;
    qt = pc == 16 && (side * side + 15) / 16 >= 2 ? 2 : 1;
    return tile_rows_needed(g, pc, nct) <= 16 * kTileTabTiles;
}

// (waves per workgroup, workgroups per CU) within the register budget of
// two waves per SIMD.
static const int kTileOpts[][2] = {{4, 2}, {8, 1}};

// Optional plan override for tuning runs:
// HALO_TILE_PLAN="waves,per_cu,nbx,mid[,qt]" (read once per process).
static bool tile_override(int& waves, int& per_cu, int& nbx, int& mid, int& qt)
{
    static int cached[6] = {-1, 0, 0, 0, 0, 0};
    if (cached[0] < 0) {
        const char* e = getenv("HALO_TILE_PLAN");
        int w = 0, k = 0, b = 0, m = 0, t = 0;
        const int got = e ? sscanf(e, "%d,%d,%d,%d,%d", &w, &k, &b, &m, &t) : 0;
        cached[0] = got >= 4 ? 1 : 0;
        cached[1] = w; cached[2] = k; cached[3] = b; cached[4] = m; cached[5] = got == 5 ? t : 0;
    }
    if (!cached[0]) return false;
    waves = cached[1]; per_cu = cached[2]; nbx = cached[3]; mid = cached[4];
    if (cached[5] == 1 || cached[5] == 2) qt = cached[5];
    return true;
}

static TileChoice tile_choose(const Geometry& g)
{
    TileChoice best{};
    int pc = 0, nct = 0, qt = 0;
    if (!tile_shape(g, pc, nct, qt)) return best;
    const int cus = device_info().cus;
    const int lds_dev = device_info().lds_per_block;
    int ow = 0, ok_ = 0, onbx = 0, omid = 0;
    if (tile_override(ow, ok_, onbx, omid, qt)) {
        const bool allowed = (ow == 4 && ok_ == 2) || (ow == 8 && ok_ == 1);
        const TilePlan p = tile_plan(g, pc, nct, qt, ow, std::min(std::max(onbx, 1), g.nbw), omid != 0);
        if (allowed && p.lds_bytes <= std::min(lds_dev, 160 * 1024 / ok_)) {
            best = TileChoice{ow, ok_, pc, nct, qt, p};
            return best;
        }
    }
    double best_score = 0.0;
    for (const auto& o : kTileOpts) {
        const int waves = o[0], per_cu = o[1];
        const int limit = std::min(lds_dev, 160 * 1024 / per_cu);
        for (int mid = 1; mid >= 0; --mid)
            for (int nbx = 1; nbx <= g.nbw; ++nbx) {
                const TilePlan p = tile_plan(g, pc, nct, qt, waves, nbx, mid != 0);
                if (p.lds_bytes > limit) continue;
                const int64_t nwg = g.BH * p.nstrips;
                const int64_t slots = (int64_t)cus * per_cu;
                const int64_t rounds = (nwg + slots - 1) / slots;
                const double fill = (double)nwg / (double)(rounds * slots);
                const int items = nbx * p.groups;
                const int most = (items + waves - 1) / waves;
                const double balance = (double)items / waves / most;
                // staged columns per used column (L2 traffic, staging work)
                const double cols = (double)nbx * g.block / p.SWv;
                const double score = fill * balance * (0.7 + 0.3 * cols) * (mid ? 1.0 : 0.93);
                if (score > best_score * 1.0001) {
                    best_score = score;
                    best = TileChoice{waves, per_cu, pc, nct, qt, p};
                }
            }
    }
    return best;
}

bool tile_supported(const Geometry& g)
{
    if (g.flags != 0 || (g.d != 16 && g.d != 32) || g.block % 4 != 0) return false;
    if ((int64_t)g.H * g.W >= (int64_t(1) << 31)) return false;     // pixel indices are 32-bit
    return tile_choose(g).waves != 0;
}

template <int D, int PC, int NCT, int NQ, int QT>
static hipError_t tile_launch_w(const void* q, const void* k, const void* v, const void* rh, const void* rw,
                                void* out, float* lse, const Geometry& g, const TileChoice& c, hipStream_t st)
{
    if (c.waves == 4) return tile_launch<D, PC, NCT, NQ, QT, 4, 2>(q, k, v, rh, rw, out, lse, g, c.plan, st);
    if (c.waves == 8) return tile_launch<D, PC, NCT, NQ, QT, 8, 2>(q, k, v, rh, rw, out, lse, g, c.plan, st);
    return hipErrorInvalidConfiguration;
}

hipError_t launch_tile(const void* q, const void* k, const void* v, const void* rh, const void* rw,
                       void* out, float* lse, const Geometry& g, hipStream_t st)
{
    const TileChoice c = tile_choose(g);
    if (c.waves == 0) return hipErrorInvalidConfiguration;
    if (c.pc == 4) return c.qt == 2 ? tile_launch_w<32, 4, 5, 5, 2>(q, k, v, rh, rw, out, lse, g, c, st)
                                    : tile_launch_w<32, 4, 5, 5, 1>(q, k, v, rh, rw, out, lse, g, c, st);
    if (g.d == 16) return c.qt == 2 ? tile_launch_w<16, 16, 1, 1, 2>(q, k, v, rh, rw, out, lse, g, c, st)
                                    : tile_launch_w<16, 16, 1, 1, 1>(q, k, v, rh, rw, out, lse, g, c, st);
    return c.qt == 2 ? tile_launch_w<32, 16, 1, 1, 2>(q, k, v, rh, rw, out, lse, g, c, st)
                     : tile_launch_w<32, 16, 1, 1, 1>(q, k, v, rh, rw, out, lse, g, c, st);
}

}  // namespace halo
