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
#include <type_traits>

#include "mfma_util.h"

namespace halo {

#ifndef HALO_MFMA_WAVES
#define HALO_MFMA_WAVES 4                  // waves per workgroup (upper bound)
#endif
#ifndef HALO_MFMA_LDS_TARGET
#define HALO_MFMA_LDS_TARGET (40 * 1024)   // preferred strip LDS per workgroup
#endif
#ifndef HALO_MFMA_QT
#define HALO_MFMA_QT 0                     // 16-query tiles per wave step; 0 = automatic
#endif
constexpr int kMaxWaves = HALO_MFMA_WAVES;
constexpr int kMaxThreads = 64 * kMaxWaves;

struct MfmaPlan {
    int nbx;          // blocks per strip
    int nstrips;      // strips per block row
    int waves;        // waves per workgroup
    int SWv;          // strip width in pixels, multiple of 4 (row pitch of K and V^T in LDS)
    int RP;           // relative-table rows padded to a multiple of 16
    int off_v, off_rel, off_scr;   // byte offsets into dynamic LDS (K at 0)
    int lds_bytes;
    int remap_xcd;    // 1: map consecutive work items onto one XCD
    int64_t nwg;      // workgroups launched
    float alpha;      // scale * log2(e)
};

// D: head dim (16 or 32).  NCH: 16-column chunks per window row (r <= 16*NCH).
// QT: 16-query tiles a wave carries at once; they share every K and V
// fragment read from LDS and all loop and address arithmetic.
template <int D, int NCH, int QT>
__global__ __launch_bounds__(kMaxThreads)
void mfma_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                 const __bf16* __restrict__ v, const __bf16* __restrict__ rel_h,
                 const __bf16* __restrict__ rel_w, __bf16* __restrict__ out,
                 float* __restrict__ lse, Geometry g, MfmaPlan p)
{
    constexpr int KPL = D / 4;                 // channels per lane in a QK fragment
    typedef typename Frag<D>::T FragT;
    extern __shared__ __align__(16) unsigned char smem[];
    __bf16* Kl = reinterpret_cast<__bf16*>(smem);                    // [r][SWv][D]
    __bf16* Vt = reinterpret_cast<__bf16*>(smem + p.off_v);          // [D][r][SWv]
    __bf16* Rh = reinterpret_cast<__bf16*>(smem + p.off_rel);        // [RP][D]
    __bf16* Rw = Rh + p.RP * D;                                       // [RP][D]

    const int nthreads = p.waves * 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, gq = lane >> 4;
    float* scr = reinterpret_cast<float*>(smem + p.off_scr) + wave * QT * p.RP * 16;  // QT x [RP][16]

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
    const int SWv = p.SWv;
    const int64_t plane = (int64_t)g.H * g.W * D;

    // ---- stage K ([row][col][d]) and V^T ([d][row][col]) of the strip's
    // in-image window rows.  A work item is 4 adjacent pixels x 8 channels:
    // four 16-byte loads per tensor; K is copied as is, V is transposed in
    // registers into eight 8-byte rows (4 columns of one channel).
    {
        constexpr int CPP = D / 8;                    // 16-byte chunks per pixel
        const __bf16* kb = k + bh * plane;
        const __bf16* vb = v + bh * plane;
        const int ng4 = SWv / 4;
        const int total = (thi - tlo) * ng4 * CPP;
        for (int e = threadIdx.x; e < total; e += nthreads) {
            const int ch = e % CPP;
            const int rest = e / CPP;
            const int c4 = rest % ng4;
            const int t = tlo + rest / ng4;
            u32x4 kk[4], vv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int ix = sx0 + 4 * c4 + j;
                kk[j] = u32x4{0u, 0u, 0u, 0u};
                vv[j] = u32x4{0u, 0u, 0u, 0u};
                if (ix >= 0 && ix < g.W) {
                    const int64_t off = ((int64_t)(wy0 + t) * g.W + ix) * D + ch * 8;
                    kk[j] = *reinterpret_cast<const u32x4*>(kb + off);
                    vv[j] = *reinterpret_cast<const u32x4*>(vb + off);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<u32x4*>(Kl + ((size_t)(t * SWv + 4 * c4 + j) * D + ch * 8)) = kk[j];
#pragma unroll
            for (int w = 0; w < 4; ++w) {             // channels 2w (low halves), 2w+1 (high)
                const u32x2 lo = {__builtin_amdgcn_perm(vv[1][w], vv[0][w], 0x05040100u),
                                  __builtin_amdgcn_perm(vv[3][w], vv[2][w], 0x05040100u)};
                const u32x2 hi = {__builtin_amdgcn_perm(vv[1][w], vv[0][w], 0x07060302u),
                                  __builtin_amdgcn_perm(vv[3][w], vv[2][w], 0x07060302u)};
                *reinterpret_cast<u32x2*>(Vt + ((size_t)(ch * 8 + 2 * w) * r + t) * SWv + 4 * c4) = lo;
                *reinterpret_cast<u32x2*>(Vt + ((size_t)(ch * 8 + 2 * w + 1) * r + t) * SWv + 4 * c4) = hi;
            }
        }
        const int nrel = 2 * r - 1;
        const unsigned short* rhs = reinterpret_cast<const unsigned short*>(rel_h);
        const unsigned short* rws = reinterpret_cast<const unsigned short*>(rel_w);
        unsigned short* rhd = reinterpret_cast<unsigned short*>(Rh);
        unsigned short* rwd = reinterpret_cast<unsigned short*>(Rw);
        for (int e = threadIdx.x; e < p.RP * D; e += nthreads) {
            const bool in = e < nrel * D;
            rhd[e] = in ? rhs[e] : (unsigned short)0;
            rwd[e] = in ? rws[e] : (unsigned short)0;
        }
    }
    __syncthreads();

    const float alpha = p.alpha;
    const int yb = by * g.block;
    const int nqy = (min(yb + g.block, g.H) - yb + g.stride - 1) / g.stride;
    const int rp16 = p.RP / 16;
    const int scr_stride = p.RP * 16;
    // all-ones A operand of the row-sum MFMA, built once
    s16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (short)0x3F80;

    int item = 0;   // running index of QT-tile groups in the strip
    for (int j = 0; j < nbx_here; ++j) {
        const int xb = (bx_first + j) * g.block;
        const int nqx = (min(xb + g.block, g.W) - xb + g.stride - 1) / g.stride;
        const int nq = nqy * nqx;
        const int nqt = (nq + 15) / 16;
        const int wcol0 = j * g.block;                // block j's window, strip coordinates
        for (int tq0 = 0; tq0 < nqt; tq0 += QT, ++item) {
            if (item % p.waves != wave) continue;

            // ---- QT tiles of 16 queries (lane n; padding lanes reuse query 0)
            FragT qf[QT];
            bool qvalid[QT];
            int qpix[QT], yl[QT], xl[QT];
#pragma unroll
            for (int u = 0; u < QT; ++u) {
                const int qi = (tq0 + u) * 16 + n;
                qvalid[u] = qi < nq;
                const int qq = qvalid[u] ? qi : 0;
                yl[u] = (qq / nqx) * g.stride;
                xl[u] = (qq % nqx) * g.stride;
                qpix[u] = (yb + yl[u]) * g.W + xb + xl[u];
                qf[u] = *reinterpret_cast<const FragT*>(q + bh * plane + (int64_t)qpix[u] * D + gq * KPL);
            }

            // ---- relative logits q.rel[row] for every table row (MFMA with the
            // table as A operand), re-indexed per query through LDS scratch.
            // Width first: its values become the accumulator input of every
            // score tile.  Height second: read per tile from the scratch.
            f32x4 cinit[QT][NCH];
            for (int pass = 0; pass < 2; ++pass) {
                const __bf16* tab = pass == 0 ? Rw : Rh;
                for (int rt = 0; rt < rp16; ++rt) {
                    const FragT a = *reinterpret_cast<const FragT*>(tab + (rt * 16 + n) * D + gq * KPL);
#pragma unroll
                    for (int u = 0; u < QT; ++u) {
                        const f32x4 gr = Frag<D>::mma(a, qf[u], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                        for (int i = 0; i < 4; ++i) scr[u * scr_stride + (rt * 16 + gq * 4 + i) * 16 + n] = gr[i];
                    }
                }
                wave_lds_sync();
                if (pass == 0) {
                    // width term of window column c = 16*ch + 4g + i; masked when
                    // the column is off-image or past the window (c >= r)
#pragma unroll
                    for (int u = 0; u < QT; ++u) {
#pragma unroll
                        for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int c = ch * 16 + gq * 4 + i;
                                const int ix = xb - g.halo + c;
                                const bool ok = c < r && ix >= 0 && ix < g.W;
                                const float val = scr[u * scr_stride + min(r - 1 - xl[u] + c, p.RP - 1) * 16 + n];
                                cinit[u][ch][i] = ok ? val : kMaskLogit;
                            }
                        }
                    }
                    wave_lds_sync();
                }
            }
            // height term of window row t for tile u: scratch row (r-1-yl) + t
            const float* rh_row[QT];
#pragma unroll
            for (int u = 0; u < QT; ++u) rh_row[u] = scr + u * scr_stride + (r - 1 - yl[u]) * 16 + n;
            const __bf16* kfrag = Kl + ((size_t)(wcol0 + n) * D + gq * KPL);
            auto kload = [&](int t, int ch) -> FragT {
                return *reinterpret_cast<const FragT*>(kfrag + (size_t)(t * SWv + ch * 16) * D);
            };

            // ---- pass 1: row max of the logits (S^T tiles: 16 window columns
            // of one window row x 16 queries; lane (n, g) holds columns 4g..4g+3)
            float M[QT];
#pragma unroll
            for (int u = 0; u < QT; ++u) M[u] = -3.0e38f;
            for (int t = tlo; t < thi; ++t) {
                FragT a[NCH];
#pragma unroll
                for (int ch = 0; ch < NCH; ++ch) a[ch] = kload(t, ch);
#pragma unroll
                for (int u = 0; u < QT; ++u) {
                    const float rh = rh_row[u][t * 16];
#pragma unroll
                    for (int ch = 0; ch < NCH; ++ch)
                        M[u] = fmaxf(M[u], max4(Frag<D>::mma(a[ch], qf[u], cinit[u][ch])) + rh);
                }
            }
            float mb[QT];
#pragma unroll
            for (int u = 0; u < QT; ++u) {
                M[u] = fmaxf(M[u], __shfl_xor(M[u], 16));
                M[u] = fmaxf(M[u], __shfl_xor(M[u], 32));
                mb[u] = alpha * M[u];                  // base-2 row max
            }

            // ---- pass 2: P = exp2(alpha*S - mb) in bf16; O^T += V^T . P^T and
            // L += 1 . P^T, one K=32 step per pair of score tiles
            auto probs = [&](f32x4 s, float c) -> u32x2 {
                return u32x2{pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s[0], alpha, c)),
                                         __builtin_amdgcn_exp2f(fmaf(s[1], alpha, c))),
                             pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s[2], alpha, c)),
                                         __builtin_amdgcn_exp2f(fmaf(s[3], alpha, c)))};
            };
            const __bf16* vfrag = Vt + (size_t)n * r * SWv + wcol0 + gq * 4;
            auto vload = [&](int mt, int t, int ch) -> u32x2 {
                return *reinterpret_cast<const u32x2*>(vfrag + (size_t)(mt * 16 * r + t) * SWv + ch * 16);
            };
            f32x4 O[QT][D / 16], L[QT];
#pragma unroll
            for (int u = 0; u < QT; ++u) {
                L[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int mt = 0; mt < D / 16; ++mt) O[u][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            // one K=32 step: score tiles (t0, ch0) and (t1, ch1); `two` false
            // means the second tile does not exist (zero operands, zero weights)
            auto step = [&](auto two_c, int t0, int ch0, int t1, int ch1) {
                constexpr bool two = decltype(two_c)::value;
                const FragT a0 = kload(t0, ch0);
                FragT a1 = {};
                if (two) a1 = kload(t1, ch1);
                u32x4 vw[D / 16];
#pragma unroll
                for (int mt = 0; mt < D / 16; ++mt) {
                    const u32x2 x0 = vload(mt, t0, ch0);
                    const u32x2 x1 = two ? vload(mt, t1, ch1) : u32x2{0u, 0u};
                    vw[mt] = u32x4{x0[0], x0[1], x1[0], x1[1]};
                }
#pragma unroll
                for (int u = 0; u < QT; ++u) {
                    const float c0 = alpha * rh_row[u][t0 * 16] - mb[u];
                    const u32x2 p0 = probs(Frag<D>::mma(a0, qf[u], cinit[u][ch0]), c0);
                    u32x2 p1 = {0u, 0u};
                    if (two) {
                        const float c1 = alpha * rh_row[u][t1 * 16] - mb[u];
                        p1 = probs(Frag<D>::mma(a1, qf[u], cinit[u][ch1]), c1);
                    }
                    const s16x8 pf = __builtin_bit_cast(s16x8, u32x4{p0[0], p0[1], p1[0], p1[1]});
#pragma unroll
                    for (int mt = 0; mt < D / 16; ++mt)
                        O[u][mt] = mma_k32(__builtin_bit_cast(s16x8, vw[mt]), pf, O[u][mt]);
                    L[u] = mma_k32(ones, pf, L[u]);
                }
            };
            if (NCH == 1) {
                int t = tlo;
                for (; t + 1 < thi; t += 2) step(std::true_type{}, t, 0, t + 1, 0);
                if (t < thi) step(std::false_type{}, t, 0, t, 0);
            } else if (NCH == 2) {
                for (int t = tlo; t < thi; ++t) step(std::true_type{}, t, 0, t, NCH - 1);
            } else {
                // consecutive score tiles of the row-major (row, column chunk)
                // sequence, two per step; a pair may span two rows
                const int ntiles = (thi - tlo) * NCH;
                int tau = 0;
                for (; tau + 1 < ntiles; tau += 2)
                    step(std::true_type{}, tlo + tau / NCH, tau % NCH, tlo + (tau + 1) / NCH, (tau + 1) % NCH);
                if (tau < ntiles) step(std::false_type{}, tlo + tau / NCH, tau % NCH, tlo + tau / NCH, tau % NCH);
            }

            // ---- normalise and store: lane (n, g) holds channels 16*mt + 4g + i of query n
#pragma unroll
            for (int u = 0; u < QT; ++u) {
                if (!qvalid[u]) continue;
                const float inv = 1.0f / L[u][0];
                const int yq = qpix[u] / g.W, xq = qpix[u] - yq * g.W;
                const int64_t opix = bh * (int64_t)g.Ho * g.Wo + (int64_t)(yq / g.stride) * g.Wo + xq / g.stride;
                __bf16* op = out + opix * D + gq * 4;
                if (lse != nullptr && gq == 0)   // natural log of the normaliser: (shift + log2 L) ln 2
                    lse[opix] = (mb[u] + __builtin_amdgcn_logf(L[u][0])) * 0.6931471805599453f;
#pragma unroll
                for (int mt = 0; mt < D / 16; ++mt) {
                    const u32x2 w = {pack_bf16x2(O[u][mt][0] * inv, O[u][mt][1] * inv),
                                     pack_bf16x2(O[u][mt][2] * inv, O[u][mt][3] * inv)};
                    *reinterpret_cast<u32x2*>(op + mt * 16) = w;
                }
            }
            wave_lds_sync();   // scratch is rewritten by the next group
        }
    }
}

static int round_up(int x, int m) { return (x + m - 1) / m * m; }

// LDS footprint of a strip of nbx blocks.
static MfmaPlan make_plan(const Geometry& g, int nch, int qt, int nbx, int waves)
{
    MfmaPlan p{};
    p.nbx = nbx;
    p.waves = waves;
    p.nstrips = (g.nbw + nbx - 1) / nbx;
    // columns the strip's windows cover, and those the last block's 16-wide
    // column tiles read
    p.SWv = round_up(std::max(nbx * g.block + 2 * g.halo, (nbx - 1) * g.block + 16 * nch), 4);
    p.RP = round_up(2 * g.r - 1, 16);
    const int kb = g.r * p.SWv * g.d * 2;
    const int vb = g.d * g.r * p.SWv * 2;
    const int rb = 2 * p.RP * g.d * 2;
    const int sb = waves * qt * p.RP * 16 * 4;
    p.off_v = round_up(kb, 16);
    p.off_rel = round_up(p.off_v + vb, 16);
    p.off_scr = round_up(p.off_rel + rb, 16);
    p.lds_bytes = p.off_scr + sb;
    return p;
}

// Windows up to 32 columns for d in {16, 32}; up to 40 (three column
// chunks, the strip kernel only) for d = 16: a one-block strip's K and V^T
// (r x 48 columns) plus one query tile of scratch per wave stay within LDS.
bool mfma_supported(int d, int r, int block, int stride, bool bf16)
{
    (void)stride;
    return bf16 && block % 4 == 0 && ((d == 16 || d == 32) && r <= 40 || d == 64 && r <= 32);
}

// Largest dynamic LDS one workgroup may use on the current device.
static int device_lds_limit() { return device_info().lds_per_block; }

// 16-query tiles per block, and how many of them a wave carries at once.
static int tiles_per_block(const Geometry& g)
{
    const int side = (g.block + g.stride - 1) / g.stride;
    return (side * side + 15) / 16;
}

static int choose_qt(const Geometry& g)
{
    if (HALO_MFMA_QT > 0) return HALO_MFMA_QT;
    const int t = tiles_per_block(g);
    if (t % 2 == 0) return 2;
    if (t % 3 == 0) return 3;
    return t == 1 ? 1 : 2;
}

template <int D, int NCH, int QT>
static hipError_t launch_t(const void* q, const void* k, const void* v, const void* rh,
                           const void* rw, void* out, float* lse, const Geometry& g, hipStream_t st)
{
    // Strip width: widest strip within the preferred LDS budget; narrower
    // only when even one block needs more.  One wave per QT-tile group of
    // the strip, at most kMaxWaves.
    const int limit = device_lds_limit();
    const int groups_per_block = (tiles_per_block(g) + QT - 1) / QT;
    auto waves_for = [&](int nbx) { return std::min(kMaxWaves, nbx * groups_per_block); };
    int nbx = g.nbw;
    MfmaPlan p = make_plan(g, NCH, QT, nbx, waves_for(nbx));
    while (nbx > 1 && p.lds_bytes > HALO_MFMA_LDS_TARGET) {
        --nbx;
        p = make_plan(g, NCH, QT, nbx, waves_for(nbx));
    }
    if (p.lds_bytes > limit) return hipErrorInvalidConfiguration;
    p.nwg = g.BH * g.nbh * p.nstrips;
    p.remap_xcd = (p.nwg % 8 == 0) ? 1 : 0;
    p.alpha = (float)((double)g.scale * 1.4426950408889634);
    auto kern = mfma_kernel<D, NCH, QT>;
    {
        const hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), p.lds_bytes);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)p.nwg), dim3(64 * p.waves), p.lds_bytes, st,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v,
                       (const __bf16*)rh, (const __bf16*)rw, (__bf16*)out, lse, g, p);
    return hipGetLastError();
}

template <int D, int NCH>
static hipError_t launch_dn(const void* q, const void* k, const void* v, const void* rh,
                            const void* rw, void* out, float* lse, const Geometry& g, hipStream_t st)
{
    hipError_t e;
    switch (choose_qt(g)) {
    case 1: return launch_t<D, NCH, 1>(q, k, v, rh, rw, out, lse, g, st);
    case 3: e = launch_t<D, NCH, 3>(q, k, v, rh, rw, out, lse, g, st); break;
    case 4: e = launch_t<D, NCH, 4>(q, k, v, rh, rw, out, lse, g, st); break;
    default: e = launch_t<D, NCH, 2>(q, k, v, rh, rw, out, lse, g, st); break;
    }
    // a window too large for several query tiles' scratch: one tile per wave
    if (e == hipErrorInvalidConfiguration) e = launch_t<D, NCH, 1>(q, k, v, rh, rw, out, lse, g, st);
    return e;
}

bool ring_supported(const Geometry& g);
hipError_t launch_ring(const void* q, const void* k, const void* v, const void* rh,
                       const void* rw, void* out, float* lse, const Geometry& g, hipStream_t st);
bool wide_supported(const Geometry& g, bool bf16);
hipError_t launch_wide(const void* q, const void* k, const void* v, const void* rh, const void* rw, void* out,
                       float* lse, const Geometry& g, hipStream_t st);

// Matrix-core launch: the persistent ring kernel when it covers the shape,
// the streaming kernel for windows wider than 32 columns, else the strip
// kernel.  force_strip selects the strip kernel regardless.
bool tile_supported(const Geometry& g);
hipError_t launch_tile(const void* q, const void* k, const void* v, const void* rh, const void* rw,
                       void* out, float* lse, const Geometry& g, hipStream_t st);

// mode: 0 the fastest matrix-core kernel for the shape (16-query tile
// kernel, else the persistent ring kernel, the streaming wide kernel, the
// strip kernel); 1 the strip kernel; 2 the ring kernel where it applies
// (else as 0 without the tile kernel).
MfmaKernel mfma_select(const Geometry& g, int mode)
{
    const bool force_strip = mode == 1;
    if (mode == 0 && tile_supported(g)) return MfmaKernel::tile;
    if (!force_strip && ring_supported(g)) return MfmaKernel::ring;
    if (!force_strip && g.flags == 0 && wide_supported(g, true)) return MfmaKernel::wide;
    return MfmaKernel::strip;
}

hipError_t launch_mfma(const void* q, const void* k, const void* v, const void* rh,
                       const void* rw, void* out, float* lse, const Geometry& g, int mode,
                       hipStream_t st)
{
    switch (mfma_select(g, mode)) {
    case MfmaKernel::tile: return launch_tile(q, k, v, rh, rw, out, lse, g, st);
    case MfmaKernel::ring: return launch_ring(q, k, v, rh, rw, out, lse, g, st);
    case MfmaKernel::wide: return launch_wide(q, k, v, rh, rw, out, lse, g, st);
    case MfmaKernel::strip: break;
    }
    const bool wide = g.r > 16;
    if (g.d == 64) return hipErrorInvalidValue;                // 64 channels run on the streaming kernel only
    if (g.d == 32 && g.r > 32) return hipErrorInvalidValue;   // the strip kernel holds 32 columns at d = 32
    if (g.d == 16 && g.r > 32) return launch_dn<16, 3>(q, k, v, rh, rw, out, lse, g, st);
    if (g.d == 16) return wide ? launch_dn<16, 2>(q, k, v, rh, rw, out, lse, g, st)
                               : launch_dn<16, 1>(q, k, v, rh, rw, out, lse, g, st);
    return wide ? launch_dn<32, 2>(q, k, v, rh, rw, out, lse, g, st)
                : launch_dn<32, 1>(q, k, v, rh, rw, out, lse, g, st);
}

}  // namespace halo
