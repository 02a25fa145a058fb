// Backward pass of halo attention on gfx950 matrix cores for windows of up
// to 32 columns and any block tiling (partial edge blocks included): bf16
// in, fp32 accumulate, the pages' default semantics.
//
// The pages print no backward; HaloNet's models are trained by gradient
// descent ("Scaling Local Self-Attention for Parameter Efficient Visual
// Backbones", section 4.1), so this is the exact derivative of the forward
// definition (sections 2.1-2.2; logit
//   l = scale * (q.k + q.rel_h[ky - y + c0] + q.rel_w[kx - x + c0])
// as in the HaloAttention module of the pswp.cn blog page, section 4), with
// the forward's per-query log normaliser lse and D = dout.out:
//   P = exp(l - lse),  dl = P (dout.v - D),
//   dq = scale sum_keys dl (k + rel_h[row] + rel_w[col]),
//   dk = scale sum_queries dl q,  dv = sum_queries P dout,
//   d rel_h[R] = scale sum dl q over the pairs at row displacement R (d rel_w alike).
//
// Two kernels, then the table reduction shared with the other backward paths:
//  * bwd_query_kernel: one workgroup per block.  The block's window (K and V,
//    zero off the image) is staged in LDS; waves take 16-query tiles.  Scores
//    are transposed, S^T = K Q^T over 4x4 key patches (lane (n, g): query n,
//    window row 4rq+g, columns 4ct..4ct+3), the width term entering as the
//    MFMA accumulator and the height term (minus lse) as the exponent's
//    addend, as in the forward tile kernel.  dP^T = V dout^T, dl = P (dP - D),
//    dq^T += K^T dl^T on a 16x16x16 MFMA per patch (K^T fragments gathered
//    from the key-major window).  Per query, the sums of dl over each window
//    column and each window row, placed at their table rows, give the
//    tables' share of dq (tables^T times sums) and the table gradients (Q^T
//    times sums), on MFMA with the sums split into bf16 high and low parts.
//    Writes dq, D per query, and one table-gradient partial per workgroup
//    (the waves' partials summed in a fixed order).
//  * bwd_key_kernel: one workgroup per key block, its keys staged as 4x4
//    patches.  The 16-query tiles of the query blocks whose windows reach
//    the key block are shared out over the waves; for its tile a wave takes
//    every patch inside the window, scores in the other orientation
//    (S = Q K^T, lane (n, g): key n, queries 4g..4g+3; relative terms
//    gathered per pair from the tile's table products): P and dl are
//    recomputed, dv^T += dout^T P and dk^T += Q^T dl (Q^T and dout^T as
//    MFMA products with a 0/1 operand).  The waves' sums are added in wave
//    order; every key belongs to one workgroup: dk and dv are written once,
//    with no atomics.
// Every sum runs in a fixed order: results are bitwise reproducible.
#include <algorithm>
#include <type_traits>

#include "mfma_util.h"

namespace halo {

constexpr int kBtWaves = 4;          // waves per workgroup (both kernels)

struct BwdTilePlan {
    // query kernel
    int rp;            // staged window rows and columns (4 * NP)
    int cw;            // staged row pitch in pixels (>= rp, = 4 mod 8)
    int jr;            // table rows in LDS and scratch (16 * JT >= 2r - 1)
    int jp;            // scratch pitch per query (floats)
    int q_off_v, q_off_tab, q_off_scr, q_lds;
    int64_t q_nwg;
    // key kernel
    int k_off_tab, k_off_scr, k_off_red, k_off_nb, k_lds;
    int64_t k_nwg;
    float alpha;       // scale * log2(e)
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ inline f32x4 mma16(s16x4_t a, s16x4_t b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

template <typename T>
__device__ inline T bt_ld(const unsigned char* base, unsigned off) { return *reinterpret_cast<const T*>(base + off); }
template <typename T>
__device__ inline void bt_st(unsigned char* base, unsigned off, T v) { *reinterpret_cast<T*>(base + off) = v; }

// four bf16 values (16-bit patterns) into one MFMA operand
__device__ inline s16x4_t pack4(unsigned short a, unsigned short b, unsigned short c, unsigned short d)
{
    return s16x4_t{(short)a, (short)b, (short)c, (short)d};
}

__device__ inline s16x4_t bf16x4_of(float a, float b, float c, float d)
{
    const u32x2 w{pack_bf16x2(a, b), pack_bf16x2(c, d)};
    return __builtin_bit_cast(s16x4_t, w);
}

// x ~ hi + lo (bf16 each) to 2^-16 relative
__device__ inline void split4(f32x4 x, s16x4_t& hi, s16x4_t& lo)
{
    hi = bf16x4_of(x[0], x[1], x[2], x[3]);
    const u32x2 h = __builtin_bit_cast(u32x2, hi);
    const float h0 = __builtin_bit_cast(float, h[0] << 16), h1 = __builtin_bit_cast(float, h[0] & 0xffff0000u);
    const float h2 = __builtin_bit_cast(float, h[1] << 16), h3 = __builtin_bit_cast(float, h[1] & 0xffff0000u);
    lo = bf16x4_of(x[0] - h0, x[1] - h1, x[2] - h2, x[3] - h3);
}

// a / d for 0 <= a < 2^20 from rd = 1/d (one ulp): (a + 1/2)/d is at least
// 1/(2d) from an integer, far above the rounding error
__device__ inline int bt_div(int a, float rd) { return (int)(((float)a + 0.5f) * rd); }

// Workgroup i runs on XCD i mod 8 (the dispatcher deals them round-robin);
// this bijection gives each XCD one contiguous range of logical blocks, so
// neighbouring blocks, which read the same halo rows and queries, share an
// L2.
__device__ inline int64_t bt_logical(int64_t i, int64_t nwg)
{
    const int64_t q8 = nwg >> 3, r8 = nwg & 7, x = i & 7, j = i >> 3;
    return x * q8 + min(x, r8) + j;
}

// Byte offset of channel chunk `c` (16 bytes) of the staged window pixel in
// row t: chunks rotate with the row so the four rows of a patch spread over
// the banks.
template <int D>
__device__ inline unsigned bt_chunk(int c, int t)
{
    constexpr int CPP = D / 8;
    return (unsigned)((c ^ (t & (CPP - 1))) * 16);
}

// ------------------------------------------------------------------ queries
template <int D, int NP>
__global__ __launch_bounds__(64 * kBtWaves) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_query_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                      const __bf16* __restrict__ v, const __bf16* __restrict__ rel_h,
                      const __bf16* __restrict__ rel_w, const __bf16* __restrict__ out,
                      const __bf16* __restrict__ dout, const float* __restrict__ lse,
                      __bf16* __restrict__ dq, float* __restrict__ dsum, float* __restrict__ part_rel,
                      Geometry g, BwdTilePlan p)
{
    constexpr int KPL = D / 4;                  // channels per lane in a Frag<D> operand
    constexpr int CPP = D / 8;                  // 16-byte chunks per pixel
    constexpr unsigned PIXB = D * 2;
    constexpr int MT = D / 16;                  // 16-channel output tiles
    constexpr int JT = NP <= 4 ? 2 : NP <= 6 ? 3 : 4;   // 16-row table tiles (2r - 1 <= 16 JT)
    typedef typename Frag<D>::T FragT;
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, gq = lane >> 4;
    const int r = g.r;
    const float alpha = p.alpha;
    const float log2e = 1.4426950408889634f;

    const int64_t nblk = (int64_t)g.nbh * g.nbw;
    const int64_t wg = bt_logical(blockIdx.x, p.q_nwg);
    const int64_t bh = wg / nblk;
    const int rem = (int)(wg - bh * nblk);
    const int by = rem / g.nbw, bx = rem - by * g.nbw;
    const int ybeg = by * g.block, xbeg = bx * g.block;
    const int wy0 = ybeg - g.halo, wx0 = xbeg - g.halo;
    const int nqy = (min(ybeg + g.block, g.H) - ybeg + g.stride - 1) / g.stride;
    const int nqx = (min(xbeg + g.block, g.W) - xbeg + g.stride - 1) / g.stride;
    const int nq = nqy * nqx;
    const int tiles = (nq + 15) / 16;
    const float rnqx = __builtin_amdgcn_rcpf((float)nqx);
    const int bs = g.block / g.stride;                  // query rows / columns of a full block
    const int64_t plane = (int64_t)g.H * g.W * D;
    const int64_t oplane = (int64_t)g.Ho * g.Wo;
    const __bf16* qs = q + bh * plane;
    const int cw = p.cw, rp = p.rp, jr = p.jr, jp = p.jp;
    const unsigned rowb = (unsigned)cw * PIXB;
    const unsigned offv = (unsigned)p.q_off_v, offth = (unsigned)p.q_off_tab;
    const unsigned offtw = offth + (unsigned)jr * D * 2;
    const unsigned scr = (unsigned)p.q_off_scr + (unsigned)wave * (unsigned)(16 * jp * 4 + 16 * D * 2);
    const unsigned qtl = scr + (unsigned)(16 * jp * 4);     // this wave's tile of Q, [16][D] bf16

    // ---- stage the window (K and V, zero outside the image or the window)
    // and both tables (zero rows past 2r - 1)
    {
        // SB items per thread in flight: every load of a batch is issued
        // before its stores
        constexpr int SB = 8;
        const int items = rp * rp * CPP;
        const float rrow = __builtin_amdgcn_rcpf((float)(rp * CPP));
        for (int e0 = tid; e0 < items; e0 += SB * 64 * kBtWaves) {
            u32x4 kk[SB], vv[SB];
            unsigned a[SB];
#pragma unroll
            for (int b = 0; b < SB; ++b) {
                const int e = e0 + b * 64 * kBtWaves;
                const int t = bt_div(e, rrow), rr = e - t * (rp * CPP);
                const int c = rr / CPP, ch = rr - c * CPP;
                const int y = wy0 + t, x = wx0 + c;
                kk[b] = u32x4{0u, 0u, 0u, 0u};
                vv[b] = u32x4{0u, 0u, 0u, 0u};
                a[b] = (unsigned)t * rowb + (unsigned)c * PIXB + bt_chunk<D>(ch, t);
                if (e < items && t < r && c < r && y >= 0 && y < g.H && x >= 0 && x < g.W) {
                    const int64_t off = bh * plane + ((int64_t)y * g.W + x) * D + ch * 8;
                    kk[b] = *reinterpret_cast<const u32x4*>(k + off);
                    vv[b] = *reinterpret_cast<const u32x4*>(v + off);
                }
            }
#pragma unroll
            for (int b = 0; b < SB; ++b) {
                if (e0 + b * 64 * kBtWaves >= items) break;
                bt_st<u32x4>(smem, a[b], kk[b]);
                bt_st<u32x4>(smem, offv + a[b], vv[b]);
            }
        }
        const int titems = jr * CPP;
        for (int e = tid; e < 2 * titems; e += 64 * kBtWaves) {
            const int tab = e / titems, rr = e - tab * titems;
            const int j = rr / CPP, ch = rr - j * CPP;
            u32x4 x{0u, 0u, 0u, 0u};
            if (j < 2 * r - 1) x = *reinterpret_cast<const u32x4*>((tab ? rel_w : rel_h) + (int64_t)j * D + ch * 8);
            bt_st<u32x4>(smem, (tab ? offtw : offth) + (unsigned)(j * D + ch * 8) * 2, x);
        }
    }
    __syncthreads();

    // table-gradient partials of this wave: lane (n, g) holds
    // d rel^T[channel 16 mt + 4g + i][table row 16 jt + n]
    f32x4 dRh[MT][JT], dRw[MT][JT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
            dRh[mt][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
            dRw[mt][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    for (int u = wave; u < tiles; u += kBtWaves) {
        // ---- the tile's queries (lane n: query 16u + n)
        const int qi = 16 * u + n;
        const bool valid = qi < nq;
        const int qc = valid ? qi : 0;
        const int iy = bt_div(qc, rnqx), ix = qc - iy * nqx;
        const int y = ybeg + iy * g.stride, x = xbeg + ix * g.stride;
        const int yl = y - wy0, xl = x - wx0;
        const int64_t opix = bh * oplane + (int64_t)(by * bs + iy) * g.Wo + bx * bs + ix;
        FragT qf = *reinterpret_cast<const FragT*>(qs + ((int64_t)y * g.W + x) * D + gq * KPL);
        FragT df = *reinterpret_cast<const FragT*>(dout + opix * D + gq * KPL);
        const FragT of = *reinterpret_cast<const FragT*>(out + opix * D + gq * KPL);
        if (!valid) {
#pragma unroll
            for (int e = 0; e < KPL; ++e) { qf[e] = 0; df[e] = 0; }
        }
        float dpart = 0.f;
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
            const float a = __builtin_bit_cast(float, (unsigned)(unsigned short)df[e] << 16);
            const float b = __builtin_bit_cast(float, (unsigned)(unsigned short)of[e] << 16);
            dpart = fmaf(a, b, dpart);
        }
        const float Dq = sum_over_rows(dpart);
        const float lse2 = lse[opix] * log2e;
        if (valid && gq == 0) dsum[opix] = Dq;
        bt_st<FragT>(smem, qtl + (unsigned)(n * D + gq * KPL) * 2, qf);

        // ---- height terms: alpha q.rel_h[row] - lse2 (-inf off the image,
        // past the window, or for lanes without a query)
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
            const FragT a = bt_ld<FragT>(smem, offth + (unsigned)((16 * jt + n) * D + gq * KPL) * 2);
            bt_st<f32x4>(smem, scr + (unsigned)(n * jp + 16 * jt + 4 * gq) * 4,
                         Frag<D>::mma(a, qf, f32x4{0.f, 0.f, 0.f, 0.f}));
        }
        float hq[NP];
#pragma unroll
        for (int rq = 0; rq < NP; ++rq) {
            const int t = 4 * rq + gq, ky = wy0 + t;
            const bool ok = valid && t < r && ky >= 0 && ky < g.H;
            const int j = ok ? t - yl + g.c0 : 0;
            const float h = bt_ld<float>(smem, scr + (unsigned)(n * jp + j) * 4);
            hq[rq] = ok ? fmaf(h, alpha, -lse2) : -INFINITY;
        }
        // ---- width terms: scratch[query][j] = q.rel_w[j], read in the loop
        // per window column c at entry c - xl + c0 (wbase + 4c) as the score
        // MFMA's accumulator; columns past the window or off the image get
        // the mask value in their entries (no other column reads them)
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
            const FragT a = bt_ld<FragT>(smem, offtw + (unsigned)((16 * jt + n) * D + gq * KPL) * 2);
            bt_st<f32x4>(smem, scr + (unsigned)(n * jp + 16 * jt + 4 * gq) * 4,
                         Frag<D>::mma(a, qf, f32x4{0.f, 0.f, 0.f, 0.f}));
        }
        const unsigned wbase = scr + 4u * (unsigned)(n * jp + g.c0 - xl);
#pragma unroll
        for (int ct = 0; ct < NP; ++ct) {
            const int c = 4 * ct + gq, kx = wx0 + c;
            if (!(c < r && kx >= 0 && kx < g.W)) bt_st<float>(smem, wbase + 4u * c, kMaskLogit);
        }

        // ---- the window, patch by patch
        // 0/1 operands picking channels 16mt..16mt+15: K . sel^T is the
        // patch's channel block as an MFMA result, lane (n, g) = channel
        // 16mt + n of keys 4g..4g+3 (patch row g), i.e. the A operand of
        // dq^T += K^T dS (exact: the products pick single bf16 values)
        FragT selk[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < KPL; ++e) selk[mt][e] = (gq * KPL + e == 16 * mt + n) ? (short)0x3F80 : (short)0;
        f32x4 dQt[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) dQt[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        float rowsum[NP];
#pragma unroll
        for (int rq = 0; rq < NP; ++rq) rowsum[rq] = 0.f;
        // A-operand lane (m, kg): key m of the patch = (row m >> 2, column
        // m & 3), channels kg*KPL..; its K^T (lane (channel n, kg): patch
        // row kg, columns 0..3) comes from an MFMA against selk.  Column tile by column tile: once a tile's
        // columns are done, their sums over the window (and over the four
        // lanes of a query) replace their width terms in the scratch, at the
        // same entries; every other entry is zeroed after the loop, so the
        // scratch then holds the width table's sums by table row.
        const unsigned kA = (unsigned)(n >> 2) * rowb + (unsigned)(n & 3) * PIXB;
#pragma unroll
        for (int ct = 0; ct < NP; ++ct) {
            f32x4 colsum{0.f, 0.f, 0.f, 0.f};
            const f32x4 cin{bt_ld<float>(smem, wbase + 16u * ct), bt_ld<float>(smem, wbase + 16u * ct + 4),
                            bt_ld<float>(smem, wbase + 16u * ct + 8), bt_ld<float>(smem, wbase + 16u * ct + 12)};
#pragma unroll
            for (int rq = 0; rq < NP; ++rq) {
                const int ta = 4 * rq + (n >> 2);      // row of this lane's A-operand key
                const unsigned chA = D == 32 ? bt_chunk<D>(gq, ta) : bt_chunk<D>(gq >> 1, ta) + (gq & 1) * 8;
                const unsigned a = (unsigned)(4 * rq) * rowb + kA + (unsigned)(4 * ct) * PIXB + chA;
                const FragT kf = bt_ld<FragT>(smem, a);
                const FragT vf = bt_ld<FragT>(smem, offv + a);
                const f32x4 s = Frag<D>::mma(kf, qf, cin);
                const f32x4 dp = Frag<D>::mma(vf, df, f32x4{0.f, 0.f, 0.f, 0.f});
                f32x4 ds;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pr = __builtin_amdgcn_exp2f(fmaf(s[i], alpha, hq[rq]));
                    ds[i] = pr * (dp[i] - Dq);
                }
                rowsum[rq] += (ds[0] + ds[1]) + (ds[2] + ds[3]);
                colsum += ds;
                const s16x4_t dsb = bf16x4_of(ds[0], ds[1], ds[2], ds[3]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const f32x4 kc = Frag<D>::mma(kf, selk[mt], f32x4{0.f, 0.f, 0.f, 0.f});
                    dQt[mt] = mma16(bf16x4_of(kc[0], kc[1], kc[2], kc[3]), dsb, dQt[mt]);
                }
            }
            // this tile's column sums (lane g writes column 4ct + g)
#pragma unroll
            for (int i = 0; i < 4; ++i) colsum[i] = sum_over_rows(colsum[i]);
            const float val = gq == 0 ? colsum[0] : gq == 1 ? colsum[1] : gq == 2 ? colsum[2] : colsum[3];
            bt_st<float>(smem, wbase + 4u * (4 * ct + gq), val);
            __builtin_amdgcn_sched_barrier(0);   // schedule one column tile at a time (registers)
        }

        // ---- the lane's query again, from an opaque copy of the tile index:
        // recomputed here rather than kept in registers through the loop
        int uo = u;
        asm volatile("" : "+s"(uo));
        const int qi2 = 16 * uo + n;
        const bool valid2 = qi2 < nq;
        const int qc2 = valid2 ? qi2 : 0;
        const int iy2 = bt_div(qc2, rnqx), ix2 = qc2 - iy2 * nqx;
        const int y2 = ybeg + iy2 * g.stride, x2 = xbeg + ix2 * g.stride;
        const int yl2 = y2 - wy0, xl2 = x2 - wx0;

        // ---- zero the entries outside the in-image window columns (and all
        // of a lane without a query): the scratch is the width table's sums
        {
            const int clo = max(0, -wx0), chi = min(r, g.W - wx0);
            const int jlo = valid2 ? clo - xl2 + g.c0 : jr, jhi = valid2 ? chi - xl2 + g.c0 : jr;
            for (int j = gq; j < jr; j += 4)
                if (j < jlo || j >= jhi) bt_st<float>(smem, scr + (unsigned)(n * jp + j) * 4, 0.f);
        }
        auto table_terms = [&](unsigned offt, f32x4 (&dR)[MT][JT]) {
            // Q^T of the tile: lane (channel 16 mt + n, kg) holds queries 4kg..4kg+3
            s16x4_t qt[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const unsigned b = qtl + (unsigned)((4 * gq) * D + 16 * mt + n) * 2;
                qt[mt] = pack4(bt_ld<unsigned short>(smem, b), bt_ld<unsigned short>(smem, b + D * 2),
                               bt_ld<unsigned short>(smem, b + 2 * D * 2), bt_ld<unsigned short>(smem, b + 3 * D * 2));
            }
#pragma unroll
            for (int jt = 0; jt < JT; ++jt) {
                // dq^T += table^T sums: B lane (query n, kg) = sums at rows 16jt+4kg..
                s16x4_t hi, lo;
                split4(bt_ld<f32x4>(smem, scr + (unsigned)(n * jp + 16 * jt + 4 * gq) * 4), hi, lo);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const unsigned b = offt + (unsigned)((16 * jt + 4 * gq) * D + 16 * mt + n) * 2;
                    const s16x4_t tt = pack4(bt_ld<unsigned short>(smem, b), bt_ld<unsigned short>(smem, b + D * 2),
                                             bt_ld<unsigned short>(smem, b + 2 * D * 2),
                                             bt_ld<unsigned short>(smem, b + 3 * D * 2));
                    dQt[mt] = mma16(tt, lo, mma16(tt, hi, dQt[mt]));
                }
                // d table^T += Q^T sums^T: B lane (table row 16jt+n, kg) = sums of queries 4kg..4kg+3
                f32x4 st;
#pragma unroll
                for (int e = 0; e < 4; ++e) st[e] = bt_ld<float>(smem, scr + (unsigned)((4 * gq + e) * jp + 16 * jt + n) * 4);
                split4(st, hi, lo);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) dR[mt][jt] = mma16(qt[mt], lo, mma16(qt[mt], hi, dR[mt][jt]));
            }
        };
        table_terms(offtw, dRw);
        // ---- the height table likewise (row sums are whole per lane)
        for (int jj = gq; jj < jr / 4; jj += 4)
            bt_st<f32x4>(smem, scr + (unsigned)(n * jp + 4 * jj) * 4, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int rq = 0; rq < NP; ++rq) {
            const int t = 4 * rq + gq, ky = wy0 + t;
            if (valid2 && t < r && ky >= 0 && ky < g.H)
                bt_st<float>(smem, scr + (unsigned)(n * jp + t - yl2 + g.c0) * 4, rowsum[rq]);
        }
        table_terms(offth, dRh);

        if (valid2) {
            __bf16* dp = dq + bh * plane + ((int64_t)y2 * g.W + x2) * D + 4 * gq;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                *reinterpret_cast<u32x2*>(dp + 16 * mt) =
                    u32x2{pack_bf16x2(g.scale * dQt[mt][0], g.scale * dQt[mt][1]),
                          pack_bf16x2(g.scale * dQt[mt][2], g.scale * dQt[mt][3])};
        }
    }

    // ---- the workgroup's table-gradient partial: waves' partials through
    // LDS (the window's space), summed in wave order
    __syncthreads();
    const int E = (2 * r - 1) * D;
    float* red = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int tab = 0; tab < 2; ++tab)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int jt = 0; jt < JT; ++jt) {
                const f32x4 x = tab ? dRw[mt][jt] : dRh[mt][jt];
                const int j = 16 * jt + n;
                *reinterpret_cast<f32x4*>(red + ((wave * 2 + tab) * jr + j) * D + 16 * mt + 4 * gq) = x;
            }
    __syncthreads();
    float* part = part_rel + wg * 2 * E;
    for (int e = tid; e < 2 * E; e += 64 * kBtWaves) {
        const int tab = e / E, rr = e - tab * E;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kBtWaves; ++w) s += red[(w * 2 + tab) * jr * D + rr];
        part[e] = g.scale * s;
    }
}

// --------------------------------------------------------------------- keys
// One workgroup per key block.  The block's keys, cut into PB x PB patches
// of 4x4, are staged once (K and V as B operands: lane (key n, kg) =
// channels kg*KPL..).  The work items are the 16-query tiles of every query
// block whose window reaches the key block, in a fixed order; wave w takes
// items w, w+4, ... and, for its tile, every patch inside that window (the
// patches in registers per pass: two passes for 16 patches at d = 32).
// Patches wholly inside the window and the image take an unmasked path.
// The waves' dk^T and dv^T sums are added in wave order through LDS at the
// end.
template <int D, int PB>
__global__ __launch_bounds__(64 * kBtWaves) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_key_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                    const __bf16* __restrict__ v, const __bf16* __restrict__ rel_h,
                    const __bf16* __restrict__ rel_w, const __bf16* __restrict__ dout,
                    const float* __restrict__ lse, const float* __restrict__ dsum,
                    __bf16* __restrict__ dk, __bf16* __restrict__ dv, Geometry g, BwdTilePlan p)
{
    constexpr int KPL = D / 4;
    constexpr int CPP = D / 8;
    constexpr int MT = D / 16;
    constexpr int NPATCH = PB * PB;
    constexpr int NPASS = (D == 32 && NPATCH > 9) ? 2 : 1;
    constexpr int NPP = (NPATCH + NPASS - 1) / NPASS;
    typedef typename Frag<D>::T FragT;
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, gq = lane >> 4;
    const int r = g.r;
    const float alpha = p.alpha;
    const float log2e = 1.4426950408889634f;

    const int64_t nblk = (int64_t)g.nbh * g.nbw;
    const int64_t wg = bt_logical(blockIdx.x, p.k_nwg);
    const int64_t bh = wg / nblk;
    const int rem = (int)(wg - bh * nblk);
    const int kby = rem / g.nbw, kbx = rem - kby * g.nbw;
    const int kyb = kby * g.block, kxb = kbx * g.block;
    const int nky = min(g.block, g.H - kyb), nkx = min(g.block, g.W - kxb);
    const int bs = g.block / g.stride;
    const int64_t plane = (int64_t)g.H * g.W * D;
    const int64_t oplane = (int64_t)g.Ho * g.Wo;
    const __bf16* qs = q + bh * plane;
    const int jr = p.jr, jp = p.jp;
    const int JT = jr / 16;
    const unsigned offkv = 0;                           // [patch][K, V][16 keys][D] bf16
    const unsigned offth = (unsigned)p.k_off_tab, offtw = offth + (unsigned)jr * D * 2;
    const unsigned scrh = (unsigned)p.k_off_scr + (unsigned)wave * (unsigned)(2 * 16 * jp * 4);
    const unsigned scrw = scrh + (unsigned)(16 * jp * 4);
    constexpr unsigned PATB = 16 * D * 2;               // one patch of K (or V)

    // ---- the key block's patches and both tables (zero past the image, the
    // block, or table row 2r - 1)
    {
        // all of a thread's items in flight at once (loads, then stores)
        constexpr int SB = (NPATCH * 16 * CPP + 64 * kBtWaves - 1) / (64 * kBtWaves);
        u32x4 kk[SB], vv[SB];
        unsigned a[SB];
#pragma unroll
        for (int b = 0; b < SB; ++b) {
            const int e = tid + b * 64 * kBtWaves;
            const int pi = e / (16 * CPP), rr = e - pi * (16 * CPP);
            const int kn = rr / CPP, ch = rr - kn * CPP;
            const int py = pi / PB, px = pi - py * PB;
            const int ly = 4 * py + (kn >> 2), lx = 4 * px + (kn & 3);
            kk[b] = u32x4{0u, 0u, 0u, 0u};
            vv[b] = u32x4{0u, 0u, 0u, 0u};
            a[b] = offkv + (unsigned)pi * 2 * PATB + (unsigned)(kn * D + ch * 8) * 2;
            if (e < NPATCH * 16 * CPP && ly < nky && lx < nkx) {
                const int64_t off = bh * plane + ((int64_t)(kyb + ly) * g.W + kxb + lx) * D + ch * 8;
                kk[b] = *reinterpret_cast<const u32x4*>(k + off);
                vv[b] = *reinterpret_cast<const u32x4*>(v + off);
            }
        }
#pragma unroll
        for (int b = 0; b < SB; ++b) {
            if (tid + b * 64 * kBtWaves >= NPATCH * 16 * CPP) break;
            bt_st<u32x4>(smem, a[b], kk[b]);
            bt_st<u32x4>(smem, a[b] + PATB, vv[b]);
        }
    }
    {
        const int titems = jr * CPP;
        for (int e = tid; e < 2 * titems; e += 64 * kBtWaves) {
            const int tab = e / titems, rr = e - tab * titems;
            const int j = rr / CPP, ch = rr - j * CPP;
            u32x4 x{0u, 0u, 0u, 0u};
            if (j < 2 * r - 1) x = *reinterpret_cast<const u32x4*>((tab ? rel_w : rel_h) + (int64_t)j * D + ch * 8);
            bt_st<u32x4>(smem, (tab ? offtw : offth) + (unsigned)(j * D + ch * 8) * 2, x);
        }
    }
    __syncthreads();

    // 0/1 operands picking channels 16mt..16mt+15: Q . sel^T is Q's channel
    // block as an MFMA result, lane (n, g) = channel 16mt + n of queries
    // 4g..4g+3, i.e. the A operand of the contraction over queries
    FragT sel[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < KPL; ++e) sel[mt][e] = (gq * KPL + e == 16 * mt + n) ? (short)0x3F80 : (short)0;

    const int A = (g.halo + g.block - 1) / g.block;
    const int ny0 = max(0, kby - A), ny1 = min(g.nbh - 1, kby + A);
    const int nx0 = max(0, kbx - A), nx1 = min(g.nbw - 1, kbx + A);
    const int nnx = nx1 - nx0 + 1, nnb = (ny1 - ny0 + 1) * nnx;
    i32x4* nbinfo = reinterpret_cast<i32x4*>(smem + p.k_off_nb);
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        f32x4 dKt[NPP][MT], dVt[NPP][MT];
#pragma unroll
        for (int pp = 0; pp < NPP; ++pp)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                dKt[pp][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
                dVt[pp][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        // the query blocks whose windows reach this key block, in row-major
        // order: {query columns, query count (0: no patch of this pass in
        // the window), patches meeting the window | patches wholly in it
        // and in the image << 16, 16-query tiles}
        for (int b = tid; b < nnb; b += 64 * kBtWaves) {
            const int nby = ny0 + b / nnx, nbx = nx0 + b % nnx;
            const int wy0 = nby * g.block - g.halo, wx0 = nbx * g.block - g.halo;
            unsigned pin = 0u, full = 0u;
#pragma unroll
            for (int pp = 0; pp < NPP; ++pp) {
                const int pi = pass * NPP + pp;
                if (pi >= NPATCH) continue;
                const int y0 = kyb + 4 * (pi / PB), x0 = kxb + 4 * (pi % PB);
                const int y1 = min(y0 + 4, kyb + nky), x1 = min(x0 + 4, kxb + nkx);
                if (max(y0, wy0) < min(y1, wy0 + r) && max(x0, wx0) < min(x1, wx0 + r)) pin |= 1u << pp;
                if (y1 == y0 + 4 && x1 == x0 + 4 && y0 >= wy0 && y1 <= wy0 + r && x0 >= wx0 && x1 <= wx0 + r)
                    full |= 1u << pp;
            }
            const int ybeg = nby * g.block, xbeg = nbx * g.block;
            const int nqy = (min(ybeg + g.block, g.H) - ybeg + g.stride - 1) / g.stride;
            const int nqx = (min(xbeg + g.block, g.W) - xbeg + g.stride - 1) / g.stride;
            const int nq = pin ? nqy * nqx : 0;
            nbinfo[b] = i32x4{nqx, nq, (int)(pin | (full << 16)), (nq + 15) / 16};
        }
        __syncthreads();

        // this wave's items: tiles wave, wave + 4, ... of the query blocks in order
        auto settle = [&](int& b, int& u) {
            while (b < nnb) {
                const int t = bt_ld<int>(smem, (unsigned)p.k_off_nb + 16u * (unsigned)b + 12u);
                if (u < t) break;
                u -= t;
                ++b;
            }
        };
        // the global operands of item (b, u): Q and dout A fragments of
        // query 16u + n, its lse2 and D
        struct ItemIn {
            FragT qa, da;
            float l2, dd;
        };
        auto fetch = [&](int b, int u) {
            ItemIn it;
            const i32x4 info = nbinfo[b];
            const int nqx = info[0], nq = info[1];
            const int nby = ny0 + b / nnx, nbx = nx0 + b % nnx;
            const int qi = min(16 * u + n, nq - 1);
            const int iy = bt_div(qi, __builtin_amdgcn_rcpf((float)nqx)), ix = qi - iy * nqx;
            const int y = nby * g.block + iy * g.stride, x = nbx * g.block + ix * g.stride;
            const int64_t op = bh * oplane + (int64_t)(nby * bs + iy) * g.Wo + nbx * bs + ix;
            it.qa = *reinterpret_cast<const FragT*>(qs + ((int64_t)y * g.W + x) * D + gq * KPL);
            it.da = *reinterpret_cast<const FragT*>(dout + op * D + gq * KPL);
            it.l2 = 16 * u + n < nq ? lse[op] * log2e : INFINITY;
            it.dd = dsum[op];
            return it;
        };
        int cb = 0, cu = wave;
        settle(cb, cu);
        ItemIn cur{};
        if (cb < nnb) cur = fetch(cb, cu);
        while (cb < nnb) {
            int nb2 = cb, nu = cu + kBtWaves;
            settle(nb2, nu);
            ItemIn nxt{};
            if (nb2 < nnb) nxt = fetch(nb2, nu);

            const i32x4 info = nbinfo[cb];
            const int nqx = info[0], nq = info[1];
            const unsigned pin = (unsigned)info[2] & 0xffffu, full = (unsigned)info[2] >> 16;
            const int nby = ny0 + cb / nnx, nbx = nx0 + cb % nnx;
            const int wy0 = nby * g.block - g.halo, wx0 = nbx * g.block - g.halo;
            const int ybeg = nby * g.block, xbeg = nbx * g.block;
            const float rnqx = __builtin_amdgcn_rcpf((float)nqx);
            const int u = cu;
            const FragT qa = cur.qa, da = cur.da;
            // this lane's four queries 16u + 4g + i: lse2 and D (from the
            // lanes that loaded them), and the scratch addresses of their
            // table products at this lane's key of patch (0, 0)
            unsigned hb[4], wb[4];
            float l2[4], dd[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int src = 4 * gq + i;               // lane holding query 16u + 4g + i
                l2[i] = __shfl(cur.l2, src);
                dd[i] = __shfl(cur.dd, src);
                const int qv = min(16 * u + src, nq - 1);
                const int jy = bt_div(qv, rnqx), jx = qv - jy * nqx;
                const int yq = ybeg + jy * g.stride, xq = xbeg + jx * g.stride;
                hb[i] = scrh + 4u * (unsigned)(src * jp + g.c0 - yq + kyb + (n >> 2));
                wb[i] = scrw + 4u * (unsigned)(src * jp + g.c0 - xq + kxb + (n & 3));
            }
            // Q^T and dout^T fragments (lane (channel n, kg) = queries 4kg..4kg+3)
            s16x4_t qt[MT], dt[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const f32x4 a = Frag<D>::mma(qa, sel[mt], f32x4{0.f, 0.f, 0.f, 0.f});
                const f32x4 b = Frag<D>::mma(da, sel[mt], f32x4{0.f, 0.f, 0.f, 0.f});
                qt[mt] = bf16x4_of(a[0], a[1], a[2], a[3]);
                dt[mt] = bf16x4_of(b[0], b[1], b[2], b[3]);
            }
            // q.rel_h[j] and q.rel_w[j] of the tile's queries: scratch[query][j]
            for (int jt = 0; jt < JT; ++jt) {
                const FragT ah = bt_ld<FragT>(smem, offth + (unsigned)((16 * jt + n) * D + gq * KPL) * 2);
                const FragT aw = bt_ld<FragT>(smem, offtw + (unsigned)((16 * jt + n) * D + gq * KPL) * 2);
                bt_st<f32x4>(smem, scrh + (unsigned)(n * jp + 16 * jt + 4 * gq) * 4,
                             Frag<D>::mma(ah, qa, f32x4{0.f, 0.f, 0.f, 0.f}));
                bt_st<f32x4>(smem, scrw + (unsigned)(n * jp + 16 * jt + 4 * gq) * 4,
                             Frag<D>::mma(aw, qa, f32x4{0.f, 0.f, 0.f, 0.f}));
            }
            // one patch: masked (some of its keys outside the window
            // or the image) or not
            auto patch = [&](auto masked, int pp) {
                constexpr bool M = decltype(masked)::value;
                const int pi = pass * NPP + pp;
                const int py = pi / PB, px = pi % PB;
                const unsigned pa = offkv + (unsigned)pi * 2 * PATB + (unsigned)(n * D + gq * KPL) * 2;
                const FragT kb = bt_ld<FragT>(smem, pa);
                const FragT vb = bt_ld<FragT>(smem, pa + PATB);
                bool inw = true;
                if (M) {
                    const int ly = 4 * py + (n >> 2), lx = 4 * px + (n & 3);
                    const int ky = kyb + ly, kx = kxb + lx;
                    inw = ly < nky && lx < nkx && ky >= wy0 && ky < wy0 + r && kx >= wx0 && kx < wx0 + r;
                }
                f32x4 cin;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const unsigned ah = M ? (inw ? hb[i] + 16u * py : scrh) : hb[i] + 16u * py;
                    const unsigned aw = M ? (inw ? wb[i] + 16u * px : scrw) : wb[i] + 16u * px;
                    const float rel = bt_ld<float>(smem, ah) + bt_ld<float>(smem, aw);
                    cin[i] = (!M || inw) ? rel : kMaskLogit;
                }
                const f32x4 s = Frag<D>::mma(qa, kb, cin);
                const f32x4 dp = Frag<D>::mma(da, vb, f32x4{0.f, 0.f, 0.f, 0.f});
                f32x4 pr, ds;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pr[i] = __builtin_amdgcn_exp2f(fmaf(s[i], alpha, -l2[i]));
                    ds[i] = pr[i] * (dp[i] - dd[i]);
                }
                const s16x4_t pb4 = bf16x4_of(pr[0], pr[1], pr[2], pr[3]);
                const s16x4_t db4 = bf16x4_of(ds[0], ds[1], ds[2], ds[3]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    dVt[pp][mt] = mma16(dt[mt], pb4, dVt[pp][mt]);
                    dKt[pp][mt] = mma16(qt[mt], db4, dKt[pp][mt]);
                }
            };
#pragma unroll
            for (int pp = 0; pp < NPP; ++pp) {
                if (!(pin & (1u << pp))) continue;
                if (full & (1u << pp)) patch(std::false_type{}, pp);
                else patch(std::true_type{}, pp);
            }
            cb = nb2;
            cu = nu;
            cur = nxt;
        }

        // ---- sums over the waves in wave order (waves 0-2 through LDS, the
        // last wave adds its own and writes dk, dv); the LDS holds the
        // waves' scratch, free once every wave is past the first barrier
        float* red = reinterpret_cast<float*>(smem + p.k_off_red);
        for (int w = 0; w < kBtWaves; ++w) {
            __syncthreads();
            if (wave != w) continue;
#pragma unroll
            for (int pp = 0; pp < NPP; ++pp)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    f32x4* rk = reinterpret_cast<f32x4*>(red) + ((pp * MT + mt) * 2) * 64 + lane;
                    f32x4* rv = rk + 64;
                    f32x4 ak = dKt[pp][mt], av = dVt[pp][mt];
                    if (w > 0) { ak = *rk + ak; av = *rv + av; }
                    if (w < kBtWaves - 1) {
                        *rk = ak;
                        *rv = av;
                        continue;
                    }
                    // dk, dv: lane (key n, g) holds channels 16mt + 4g..4g+3
                    const int pi = pass * NPP + pp;
                    if (pi >= NPATCH) continue;
                    const int ly = 4 * (pi / PB) + (n >> 2), lx = 4 * (pi % PB) + (n & 3);
                    if (ly >= nky || lx >= nkx) continue;
                    const int64_t off = bh * plane + ((int64_t)(kyb + ly) * g.W + kxb + lx) * D + 16 * mt + 4 * gq;
                    *reinterpret_cast<u32x2*>(dk + off) =
                        u32x2{pack_bf16x2(g.scale * ak[0], g.scale * ak[1]), pack_bf16x2(g.scale * ak[2], g.scale * ak[3])};
                    *reinterpret_cast<u32x2*>(dv + off) =
                        u32x2{pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3])};
                }
        }
        __syncthreads();
    }
}

__global__ void bt_zero_u16(unsigned short* __restrict__ p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// ---------------------------------------------------------------- planning
static int bt_np(int r) { return r <= 16 ? 4 : r <= 20 ? 5 : r <= 24 ? 6 : 8; }

static BwdTilePlan bt_plan(const Geometry& g)
{
    BwdTilePlan p{};
    const int np = bt_np(g.r);
    const int jt = np <= 4 ? 2 : np <= 6 ? 3 : 4;
    p.rp = 4 * np;
    p.cw = p.rp;
    while (p.cw % 8 != 4) ++p.cw;
    p.jr = 16 * jt;
    p.jp = p.jr + 4;
    const int pix = g.d * 2;
    const int kvb = p.rp * p.cw * pix;                 // one staged window (bytes)
    p.q_off_v = kvb;
    p.q_off_tab = 2 * kvb;
    p.q_off_scr = p.q_off_tab + 2 * p.jr * g.d * 2;
    p.q_lds = p.q_off_scr + kBtWaves * (16 * p.jp * 4 + 16 * g.d * 2);
    const int red = kBtWaves * 2 * p.jr * g.d * 4;     // the partials' reduction reuses the window space
    if (red > p.q_off_tab) return BwdTilePlan{};       // does not fit under the tables
    p.q_nwg = g.BH * g.nbh * g.nbw;
    // key kernel: the block's patches (K and V), the tables, the waves'
    // scratch; the wave-order sums of dk^T and dv^T reuse the scratch
    const int pb = (g.block + 3) / 4;
    const int npp = g.d == 32 && pb * pb > 9 ? (pb * pb + 1) / 2 : pb * pb;
    p.k_off_tab = pb * pb * 2 * 16 * g.d * 2;
    p.k_off_scr = p.k_off_tab + 2 * p.jr * g.d * 2;
    p.k_off_red = p.k_off_scr;
    const int scr = kBtWaves * 2 * 16 * p.jp * 4;
    const int redb = npp * (g.d / 16) * 2 * 64 * 16;
    p.k_off_nb = p.k_off_scr + std::max(scr, redb);
    const int A = (g.halo + g.block - 1) / g.block;
    const int nnb = std::min(2 * A + 1, g.nbh) * std::min(2 * A + 1, g.nbw);
    p.k_lds = p.k_off_nb + nnb * 16;
    p.k_nwg = p.q_nwg;
    p.alpha = (float)((double)g.scale * 1.4426950408889634);
    return p;
}

bool bwd_tile_supported(const Geometry& g, bool bf16)
{
    if (!bf16 || g.flags != 0 || (g.d != 16 && g.d != 32) || g.r > 32 || g.block > 16) return false;
    if ((int64_t)g.H * g.W * g.d >= (int64_t(1) << 31)) return false;   // 32-bit offsets inside an image
    // LDS of one gfx950 workgroup (160 KiB): the choice depends on the shape
    // only, so workspace queries need no device
    const BwdTilePlan p = bt_plan(g);
    constexpr int kLds = 160 * 1024;
    return p.q_lds != 0 && p.q_lds <= kLds && p.k_lds <= kLds;
}

// Rows of table-gradient partials the query kernel writes (one per block).
int64_t bwd_tile_rel_rows(const Geometry& g) { return g.BH * g.nbh * g.nbw; }

template <int D, int NP>
static hipError_t bt_query_launch(const void* q, const void* k, const void* v, const void* rh, const void* rw,
                                  const void* out, const void* dout, const float* lse, void* dq, float* dsum,
                                  float* part_rel, const Geometry& g, const BwdTilePlan& p, hipStream_t st)
{
    auto kern = bwd_query_kernel<D, NP>;
    const hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), p.q_lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)p.q_nwg), dim3(64 * kBtWaves), p.q_lds, st,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)rh, (const __bf16*)rw,
                       (const __bf16*)out, (const __bf16*)dout, lse, (__bf16*)dq, dsum, part_rel, g, p);
    return hipGetLastError();
}

template <int D, int PB>
static hipError_t bt_key_launch(const void* q, const void* k, const void* v, const void* rh, const void* rw,
                                const void* dout, const float* lse, const float* dsum, void* dk, void* dv,
                                const Geometry& g, const BwdTilePlan& p, hipStream_t st)
{
    auto kern = bwd_key_kernel<D, PB>;
    const hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), p.k_lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)p.k_nwg), dim3(64 * kBtWaves), p.k_lds, st,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)rh, (const __bf16*)rw,
                       (const __bf16*)dout, lse, dsum, (__bf16*)dk, (__bf16*)dv, g, p);
    return hipGetLastError();
}

template <int D>
static hipError_t bt_query_np(const void* q, const void* k, const void* v, const void* rh, const void* rw,
                              const void* out, const void* dout, const float* lse, void* dq, float* dsum,
                              float* part_rel, const Geometry& g, const BwdTilePlan& p, hipStream_t st)
{
    switch (bt_np(g.r)) {
    case 4: return bt_query_launch<D, 4>(q, k, v, rh, rw, out, dout, lse, dq, dsum, part_rel, g, p, st);
    case 5: return bt_query_launch<D, 5>(q, k, v, rh, rw, out, dout, lse, dq, dsum, part_rel, g, p, st);
    case 6: return bt_query_launch<D, 6>(q, k, v, rh, rw, out, dout, lse, dq, dsum, part_rel, g, p, st);
    default: return bt_query_launch<D, 8>(q, k, v, rh, rw, out, dout, lse, dq, dsum, part_rel, g, p, st);
    }
}

template <int D>
static hipError_t bt_key_pb(const void* q, const void* k, const void* v, const void* rh, const void* rw,
                            const void* dout, const float* lse, const float* dsum, void* dk, void* dv,
                            const Geometry& g, const BwdTilePlan& p, hipStream_t st)
{
    switch ((g.block + 3) / 4) {
    case 1: return bt_key_launch<D, 1>(q, k, v, rh, rw, dout, lse, dsum, dk, dv, g, p, st);
    case 2: return bt_key_launch<D, 2>(q, k, v, rh, rw, dout, lse, dsum, dk, dv, g, p, st);
    case 3: return bt_key_launch<D, 3>(q, k, v, rh, rw, dout, lse, dsum, dk, dv, g, p, st);
    default: return bt_key_launch<D, 4>(q, k, v, rh, rw, dout, lse, dsum, dk, dv, g, p, st);
    }
}

// dq (zeroed first where queries are strided: only query pixels receive a
// gradient), D per query into dsum, table partials, then dk and dv.
hipError_t launch_bwd_tile(const void* q, const void* k, const void* v, const void* rh, const void* rw,
                           const void* out, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           float* dsum, float* part_rel, const Geometry& g, hipStream_t st)
{
    const BwdTilePlan p = bt_plan(g);
    if (g.stride > 1) {
        const int64_t nel = g.BH * (int64_t)g.H * g.W * g.d;
        const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((nel + 255) / 256, 65536));
        hipLaunchKernelGGL(bt_zero_u16, dim3((unsigned)blocks), dim3(256), 0, st, (unsigned short*)dq, nel);
    }
    hipError_t e = g.d == 16 ? bt_query_np<16>(q, k, v, rh, rw, out, dout, lse, dq, dsum, part_rel, g, p, st)
                             : bt_query_np<32>(q, k, v, rh, rw, out, dout, lse, dq, dsum, part_rel, g, p, st);
    if (e != hipSuccess) return e;
    return g.d == 16 ? bt_key_pb<16>(q, k, v, rh, rw, dout, lse, dsum, dk, dv, g, p, st)
                     : bt_key_pb<32>(q, k, v, rh, rw, dout, lse, dsum, dk, dv, g, p, st);
}

}  // namespace halo
