// The whole attention layer in one kernel (bf16): to_q and to_kv, the
// blocked local attention of every head, the head merge and to_out, with
// q, k, v and the attention output kept on chip.
//
// What it computes is the HaloAttention module of the pswp.cn blog page
// (section 4) around the blocked local self-attention of HaloNet ("Scaling
// Local Self-Attention for Parameter Efficient Visual Backbones", section
// 2.2, Figures 1-2): q = x W_q^T and [k | v] = x W_kv^T per pixel, heads
// split off the channel axis (channel h*d + c is channel c of head h), the
// attention of each head over its block's (block + 2 halo)^2 window with
// the relative logits q.rel_h[ky - y + c0] + q.rel_w[kx - x + c0] (c0 =
// r - 1 + halo), off-image keys skipped, then y = attn W_o^T + b_o.  HaloNet
// appendix D keeps activations in the blocked layout and avoids formatting
// passes; here x is read once per window and y written once, in either the
// NHWC or the blocked layout.
//
// One workgroup of four waves per image block.  Per workgroup:
//  - the block's window of x (all C channels) is staged in LDS once;
//  - per head: the head's rows of W_q, W_k, W_v and columns of W_o go to LDS
//    (loaded into registers during the previous head), k and v of every
//    window pixel are projected on the matrix cores into LDS (the waves
//    share the window rows, one 16-key tile per row; a row's x fragments
//    feed both projections), each wave projects
//    the q of its 16 queries into registers, computes the relative logits
//    (rel . q^T on the matrix cores, through a wave-private scratch: the
//    width terms of its key columns become the score MFMA's accumulator
//    input, one height term per window row), the scores K q^T row by row,
//    an exact-max softmax, P V, and adds (o / l) W_o[:, head]^T to its fp32
//    output accumulators;
//  - y = accumulators + b_o, written once.
// Storage points match the three-kernel layer: q, k, v, the probabilities
// and the attention output are rounded to bf16 where that path stores them.
#include <algorithm>

#include "halo_common.h"
#include "mfma_util.h"
#include "proj.h"

namespace halo {

namespace {

template <typename T>
__device__ inline T ld_lds(const unsigned char* base, unsigned off)
{
    return *reinterpret_cast<const T*>(base + off);
}
template <typename T>
__device__ inline void st_lds(unsigned char* base, unsigned off, T val)
{
    *reinterpret_cast<T*>(base + off) = val;
}

__device__ inline f32x4 mma16(s16x4 a, s16x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ inline s16x4 bf16x4_of(f32x4 v)
{
    return __builtin_bit_cast(s16x4, u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
}

constexpr int kLayerWaves = 4;
constexpr int kScrPitch = 20;          // floats per scratch row (the 16 queries + pad)
constexpr int kScrRows = 32;           // table rows per relative table (2r - 1 <= 31)
// 16-byte chunks of W_q, W_k, W_v and 8-byte chunks of W_o a thread carries
// for one head (3 d C / 8 and C_out d / 4 over the workgroup's threads)
constexpr int kMaxQkvChunks = 6;
constexpr int kMaxWoChunks = 4;
constexpr int kMaxKc = 8;              // 32-channel steps of C (C <= 256)

}  // namespace

struct LayerFusedPlan {
    int R, nr;                // window side, window rows the kernel walks (>= R)
    int XP, KP, VP;           // LDS pitches in elements: x row, K row, V^T row
    int WP, OP;               // LDS pitches of the W_q/W_k/W_v rows and the W_o rows
    int off_k, off_v, off_sc, off_w, off_wo, lds;   // byte offsets, total LDS
    int nbh, nbw;             // blocks per column / row
    int tiles;                // 16-query tiles of a block
    float alpha;              // scale * log2(e)
};

// D: channels per head.  NR: window rows (>= r; rows past r are masked).
// NCO: 16-channel tiles of C_out.  A window row is one 16-key tile: key
// column c at lane rows 4g + i of the score tile, columns >= r masked.
template <int D, int NR, int NCO>
__global__ __launch_bounds__(64 * kLayerWaves) void layer_fused_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ w_q, const __bf16* __restrict__ w_kv,
    const __bf16* __restrict__ w_o, const __bf16* __restrict__ b_o, const __bf16* __restrict__ rel_h,
    const __bf16* __restrict__ rel_w, __bf16* __restrict__ y, LayerGeom L, int block, int halo, LayerFusedPlan p)
{
    typedef typename Frag<D>::T FragT;
    constexpr int MT = D / 16;                 // 16-channel tiles of a head
    constexpr int kT = 64 * kLayerWaves;
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int R = p.R, C = L.C, inner = L.heads * D;
    const int kc = C / 32;                     // 32-channel steps of the input projections (<= kMaxKc)

    const int wg = blockIdx.x;
    const int bx = wg % p.nbw;
    const int rest = wg / p.nbw;
    const int by = rest % p.nbh;
    const int img = rest / p.nbh;
    const int y0 = by * block - halo, x0 = bx * block - halo;

    // pixel index of image position (yy, xx) in the layer layout
    auto pix = [&](int yy, int xx) -> int64_t {
        if (L.layout == 0) return ((int64_t)img * L.H + yy) * L.W + xx;
        const int sb = block;
        return (((int64_t)img * p.nbh + yy / sb) * p.nbw + xx / sb) * (sb * sb) + (yy % sb) * sb + xx % sb;
    };

    // ---- the window of x, all channels: slot 16 t + u holds window row t,
    // column u (rows of XP elements); columns >= r, rows >= r and pixels off
    // the image are zero.  Loads go out in batches ahead of their stores.
    {
        constexpr int kStageBatch = 8;
        const int cpr = C / 8;                 // 16-byte chunks per pixel
        const int total = NR * 16 * cpr;
        for (int e0 = 0; e0 < total; e0 += kStageBatch * kT) {
            u32x4 val[kStageBatch];
            unsigned dst[kStageBatch];
#pragma unroll
            for (int j = 0; j < kStageBatch; ++j) {
                const int e = e0 + j * kT + tid;
                const int ps = e / cpr, c8 = e - ps * cpr;
                const int t = ps >> 4, u = ps & 15;
                const int yy = y0 + t, xx = x0 + u;
                val[j] = u32x4{0u, 0u, 0u, 0u};
                dst[j] = e < total ? 2u * (unsigned)(ps * p.XP + c8 * 8) : ~0u;
                if (e < total && t < R && u < R && yy >= 0 && yy < L.H && xx >= 0 && xx < L.W)
                    val[j] = *reinterpret_cast<const u32x4*>(x + pix(yy, xx) * C + c8 * 8);
            }
#pragma unroll
            for (int j = 0; j < kStageBatch; ++j)
                if (dst[j] != ~0u) st_lds<u32x4>(smem, dst[j], val[j]);
        }
    }

    // ---- this wave's 16 queries: block-local position, window pixel slot
    const bool has_tile = wave < p.tiles;
    const int qi = (has_tile ? wave : 0) * 16 + n;
    const int yl = qi / block, xl = qi - yl * block;
    const int qslot = (yl + halo) * 16 + xl + halo;
    const bool qvalid = has_tile && by * block + yl < L.H && bx * block + xl < L.W;
    // key columns 4g + i of this lane: in the window and on the image
    bool colok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = 4 * g + i;
        colok[i] = c < R && x0 + c >= 0 && x0 + c < L.W;
    }
    const int tlo = max(0, -y0), thi = min(R, L.H - y0);    // window rows on the image

    // relative tables as A operands (the channel map of the q fragment):
    // rows 16 jt + n, zero past 2r - 1
    FragT tabh[2], tabw[2];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
        const int row = 16 * jt + n;
        const bool in = row < 2 * R - 1;
        const int rr = in ? row : 0;
        if constexpr (D == 16) {
            u32x2 a = *reinterpret_cast<const u32x2*>(rel_h + rr * D + 4 * g);
            u32x2 b = *reinterpret_cast<const u32x2*>(rel_w + rr * D + 4 * g);
            if (!in) a = b = u32x2{0u, 0u};
            tabh[jt] = __builtin_bit_cast(s16x4, a);
            tabw[jt] = __builtin_bit_cast(s16x4, b);
        } else {
            // channels 4g..4g+3 and 16+4g..16+4g+3 (the q fragment's map)
            u32x2 a0 = *reinterpret_cast<const u32x2*>(rel_h + rr * D + 4 * g);
            u32x2 a1 = *reinterpret_cast<const u32x2*>(rel_h + rr * D + 16 + 4 * g);
            u32x2 b0 = *reinterpret_cast<const u32x2*>(rel_w + rr * D + 4 * g);
            u32x2 b1 = *reinterpret_cast<const u32x2*>(rel_w + rr * D + 16 + 4 * g);
            if (!in) a0 = a1 = b0 = b1 = u32x2{0u, 0u};
            tabh[jt] = __builtin_bit_cast(s16x8, u32x4{a0[0], a0[1], a1[0], a1[1]});
            tabw[jt] = __builtin_bit_cast(s16x8, u32x4{b0[0], b0[1], b1[0], b1[1]});
        }
    }

    f32x4 acc[NCO];
#pragma unroll
    for (int co = 0; co < NCO; ++co) acc[co] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- one head's weights, loaded into registers a head ahead and written
    // to LDS at the head's start: W_q, W_k, W_v rows (16-byte chunks, rows of
    // WP elements), W_o's d columns of the head (8-byte chunks, rows of OP)
    const int cpr = C / 8;
    const int per = D * cpr;                   // 16-byte chunks of one of W_q, W_k, W_v
    const int nq = 3 * per, no = L.Cout * (D / 4);
    u32x4 pq[kMaxQkvChunks];
    u32x2 po[kMaxWoChunks];
    auto prefetch = [&](int hh) {
#pragma unroll
        for (int i = 0; i < kMaxQkvChunks; ++i) {
            const int e = tid + kT * i;
            if (e < nq) {
                const int which = e / per, rem = e - which * per;
                const int r = rem / cpr, c8 = rem - r * cpr;
                const __bf16* src = which == 0 ? w_q + (int64_t)(hh * D + r) * C
                                               : w_kv + (int64_t)((which == 1 ? 0 : inner) + hh * D + r) * C;
                pq[i] = *reinterpret_cast<const u32x4*>(src + 8 * c8);
            }
        }
#pragma unroll
        for (int i = 0; i < kMaxWoChunks; ++i) {
            const int e = tid + kT * i;
            if (e < no) {
                const int co = e / (D / 4), c4 = e - co * (D / 4);
                po[i] = *reinterpret_cast<const u32x2*>(w_o + (int64_t)co * inner + hh * D + 4 * c4);
            }
        }
    };
    auto commit = [&]() {
#pragma unroll
        for (int i = 0; i < kMaxQkvChunks; ++i) {
            const int e = tid + kT * i;
            if (e < nq) {
                const int which = e / per, rem = e - which * per;
                const int r = rem / cpr, c8 = rem - r * cpr;
                st_lds<u32x4>(smem, p.off_w + 2u * (unsigned)((which * D + r) * p.WP + 8 * c8), pq[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < kMaxWoChunks; ++i) {
            const int e = tid + kT * i;
            if (e < no) {
                const int co = e / (D / 4), c4 = e - co * (D / 4);
                st_lds<u32x2>(smem, p.off_wo + 2u * (unsigned)(co * p.OP + 4 * c4), po[i]);
            }
        }
    };
    prefetch(0);
    __syncthreads();                           // the window of x is in LDS

    const unsigned scr = p.off_sc + (unsigned)wave * 2 * kScrRows * kScrPitch * 4;   // height, then width
    const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
    // channel slot of 4-channel group gg of 16-channel tile mt in a K row
    // (and in the q fragment): D = 16 natural; D = 32 pairs groups gg and
    // gg + 4 in 8 adjacent channels
    auto kpos = [](int mt, int gg) { return D == 16 ? 4 * gg : 8 * gg + 4 * mt; };
    const unsigned kb = p.off_k, vb = p.off_v;
    const unsigned wqa = p.off_w, wka = p.off_w + 2u * (unsigned)(D * p.WP), wva = p.off_w + 4u * (unsigned)(D * p.WP);
    // C x 16 contraction of 16 rows of A and 16 of B, both rows of LDS with
    // 8 channels per lane: all fragments loaded before the MFMAs
    auto contract = [&](unsigned aa, unsigned ba) {
        s16x8 fa[kMaxKc], fb[kMaxKc];
#pragma unroll
        for (int kk = 0; kk < kMaxKc; ++kk)
            if (kk < kc) {
                fa[kk] = ld_lds<s16x8>(smem, aa + 64u * kk);
                fb[kk] = ld_lds<s16x8>(smem, ba + 64u * kk);
            }
        f32x4 c = zero4;
#pragma unroll
        for (int kk = 0; kk < kMaxKc; ++kk)
            if (kk < kc) c = mma_k32(fa[kk], fb[kk], c);
        return c;
    };

    for (int h = 0; h < L.heads; ++h) {
        if (h > 0) __syncthreads();            // every wave is done with the previous head's K, V, W
        commit();
        __syncthreads();                       // this head's weights are in LDS
        if (h + 1 < L.heads) prefetch(h + 1);  // in flight behind this head's work

        // ---- k and v of the window's rows, one row per wave at a time: the
        // row's x fragments (lane: pixel n, channels 8g..8g+7 of each
        // 32-channel step) serve as B of K^T = W_k X^T and as A of V = X W_v^T
        for (int t = wave; t < NR; t += kLayerWaves) {
            const unsigned xa = 2u * (unsigned)((t * 16 + n) * p.XP + 8 * g);
            s16x8 xf[kMaxKc];
#pragma unroll
            for (int kk = 0; kk < kMaxKc; ++kk)
                if (kk < kc) xf[kk] = ld_lds<s16x8>(smem, xa + 64u * kk);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const unsigned ka = wka + 2u * (unsigned)((mt * 16 + n) * p.WP + 8 * g);
                const unsigned va = wva + 2u * (unsigned)((mt * 16 + n) * p.WP + 8 * g);
                s16x8 wk[kMaxKc], wv[kMaxKc];
#pragma unroll
                for (int kk = 0; kk < kMaxKc; ++kk)
                    if (kk < kc) {
                        wk[kk] = ld_lds<s16x8>(smem, ka + 64u * kk);
                        wv[kk] = ld_lds<s16x8>(smem, va + 64u * kk);
                    }
                f32x4 ck = zero4, cv = zero4;
#pragma unroll
                for (int kk = 0; kk < kMaxKc; ++kk)
                    if (kk < kc) {
                        ck = mma_k32(wk[kk], xf[kk], ck);     // lane (pixel n, channels 4g..4g+3)
                        cv = mma_k32(xf[kk], wv[kk], cv);     // lane (channel n, pixels 4g..4g+3)
                    }
                st_lds<s16x4>(smem, kb + 2u * (unsigned)((t * 16 + n) * p.KP + kpos(mt, g)), bf16x4_of(ck));
                st_lds<s16x4>(smem, vb + 2u * (unsigned)((mt * 16 + n) * p.VP + t * 16 + 4 * g), bf16x4_of(cv));
            }
        }

        // ---- q of this wave's queries, in the score MFMA's B layout, and the
        // relative logits of table rows 0..31 -> scratch [table][row][query]
        FragT qf{};
        if (has_tile) {
            f32x4 qc[MT];
            const unsigned xa = 2u * (unsigned)(qslot * p.XP + 8 * g);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) qc[mt] = contract(wqa + 2u * (unsigned)((mt * 16 + n) * p.WP + 8 * g), xa);
            if constexpr (D == 16) {
                qf = bf16x4_of(qc[0]);
            } else {
                const u32x2 lo = __builtin_bit_cast(u32x2, bf16x4_of(qc[0]));
                const u32x2 hi = __builtin_bit_cast(u32x2, bf16x4_of(qc[1]));
                qf = __builtin_bit_cast(s16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
            }
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
                const f32x4 gh = Frag<D>::mma(tabh[jt], qf, zero4);
                const f32x4 gw = Frag<D>::mma(tabw[jt], qf, zero4);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const unsigned row = (unsigned)(16 * jt + 4 * g + i);
                    st_lds<float>(smem, scr + 4u * (row * kScrPitch + n), gh[i]);
                    st_lds<float>(smem, scr + 4u * ((kScrRows + row) * kScrPitch + n), gw[i]);
                }
            }
        }
        __syncthreads();                       // k and v of this head are in LDS

        if (has_tile) {
            // width terms of the lane's 4 key columns (the score MFMA's
            // accumulator input; masked columns get the mask logit) and the
            // height term of each window row (-inf for rows off the image)
            f32x4 cinit;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float w = ld_lds<float>(smem, scr + 4u * ((unsigned)(kScrRows + 4 * g + i - xl + R - 1) * kScrPitch + n));
                cinit[i] = colok[i] ? w : kMaskLogit;
            }
            const unsigned hrow0 = scr + 4u * (unsigned)((R - 1 - yl) * kScrPitch + n);
            // ---- scores, one window row per MFMA: lane (query n, columns 4g..4g+3)
            f32x4 S[NR];
            float m = -INFINITY;
#pragma unroll
            for (int t = 0; t < NR; ++t) {
                const FragT a = ld_lds<FragT>(smem, kb + 2u * (unsigned)((t * 16 + n) * p.KP + (D == 16 ? 4 * g : 8 * g)));
                const float hb = ld_lds<float>(smem, hrow0 + 4u * kScrPitch * (unsigned)t);
                const float hh = t >= tlo && t < thi ? hb * p.alpha : -INFINITY;
                const f32x4 sc = Frag<D>::mma(a, qf, cinit);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    S[t][i] = fmaf(sc[i], p.alpha, hh);
                    m = fmaxf(m, S[t][i]);
                }
            }
            m = max_over_rows(m);
            float lsum = 0.f;
            s16x4 P[NR];
#pragma unroll
            for (int t = 0; t < NR; ++t) {
                f32x4 e;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    e[i] = __builtin_amdgcn_exp2f(S[t][i] - m);
                    lsum += e[i];
                }
                P[t] = bf16x4_of(e);
            }
            lsum = sum_over_rows(lsum);
            // ---- O^T = V^T P^T: lane (query n, channels 16 mt + 4g .. +3)
            s16x4 ob[MT];
            const float inv = 1.f / lsum;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                f32x4 o = zero4;
#pragma unroll
                for (int t = 0; t < NR; ++t) {
                    const s16x4 a = ld_lds<s16x4>(smem, vb + 2u * (unsigned)((mt * 16 + n) * p.VP + t * 16 + 4 * g));
                    o = mma16(a, P[t], o);
                }
                ob[mt] = bf16x4_of(o * inv);
            }
            // ---- to_out of this head's channels: Y^T += W_o[:, h D + ...] O^T
#pragma unroll
            for (int co = 0; co < NCO; ++co) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const s16x4 a = ld_lds<s16x4>(smem, p.off_wo + 2u * (unsigned)((co * 16 + n) * p.OP + mt * 16 + 4 * g));
                    acc[co] = mma16(a, ob[mt], acc[co]);
                }
            }
        }
    }

    // ---- y = acc + b_o: lane (query n, output channels 16 co + 4g .. +3)
    if (qvalid) {
        const int64_t op = pix(by * block + yl, bx * block + xl) * L.Cout;
#pragma unroll
        for (int co = 0; co < NCO; ++co) {
            const u32x2 bb = *reinterpret_cast<const u32x2*>(b_o + co * 16 + 4 * g);
            const float b0 = __builtin_bit_cast(float, bb[0] << 16), b1 = __builtin_bit_cast(float, bb[0] & 0xffff0000u);
            const float b2 = __builtin_bit_cast(float, bb[1] << 16), b3 = __builtin_bit_cast(float, bb[1] & 0xffff0000u);
            *reinterpret_cast<u32x2*>(y + op + co * 16 + 4 * g) =
                u32x2{pack_bf16x2(acc[co][0] + b0, acc[co][1] + b1), pack_bf16x2(acc[co][2] + b2, acc[co][3] + b3)};
        }
    }
}

namespace {

int rup_i(int v, int m) { return (v + m - 1) / m * m; }

int layer_nr_template(int r) { return r <= 6 ? 6 : r <= 8 ? 8 : r <= 10 ? 10 : r <= 12 ? 12 : r <= 14 ? 14 : 16; }

LayerFusedPlan layer_fused_plan(const LayerGeom& L, int block, int halo, float scale)
{
    LayerFusedPlan p{};
    p.R = block + 2 * halo;
    p.nr = layer_nr_template(p.R);
    // x rows: C + 8 elements (a 16-pixel operand read of 16 bytes per lane
    // lands 4 dwords apart per pixel: 8 lanes on distinct banks per pass)
    p.XP = L.C + 8;
    // K rows: d + 4 (16 channels) or d + 8 (32): the fragment reads of 16
    // keys fall on distinct banks
    p.KP = L.d == 16 ? 20 : 40;
    // V^T rows: at least the window's 16 nr slots, pitch / 2 = 2 (mod 32) dwords
    p.VP = 16 * p.nr;
    while ((p.VP / 2) % 32 != 2 || p.VP % 2) ++p.VP;
    // weight rows: W_q/W_k/W_v like x rows; W_o rows of d + 4 elements (the
    // 8-byte operand reads of 16 output channels on distinct banks)
    p.WP = L.C + 8;
    p.OP = L.d + 4;
    const int xb = 16 * p.nr * p.XP * 2;
    p.off_k = rup_i(xb, 16);
    p.off_v = rup_i(p.off_k + 16 * p.nr * p.KP * 2, 16);
    p.off_sc = rup_i(p.off_v + L.d * p.VP * 2, 16);
    p.off_w = rup_i(p.off_sc + kLayerWaves * 2 * kScrRows * kScrPitch * 4, 16);
    p.off_wo = rup_i(p.off_w + 3 * L.d * p.WP * 2, 16);
    p.lds = p.off_wo + L.Cout * p.OP * 2;
    p.nbh = L.H / block;
    p.nbw = L.W / block;
    p.tiles = block * block / 16;
    p.alpha = (float)((double)scale * 1.4426950408889634);
    return p;
}

}  // namespace

bool layer_fused_supported(const LayerGeom& L, int block, int halo, int stride, bool bf16)
{
    if (!bf16 || stride != 1) return false;
    if (L.d != 16 && L.d != 32) return false;
    if (block != 4 && block != 8) return false;             // one 16-query tile per wave
    if (L.H % block || L.W % block) return false;
    const int R = block + 2 * halo;
    if (R > 16) return false;                               // 2r - 1 <= 31 table rows, <= 16 key tiles
    if (L.C % 32 || L.C < 32 || L.C > 32 * kMaxKc || L.Cout % 16 || L.Cout < 16 || L.Cout > 256) return false;
    if (L.NP >= ((int64_t)1 << 31) || (int64_t)L.NP * std::max(L.C, L.Cout) >= ((int64_t)1 << 40)) return false;
    // one head's weights in the threads' prefetch registers
    if (3 * L.d * L.C / 8 > kMaxQkvChunks * 64 * kLayerWaves || L.Cout * L.d / 4 > kMaxWoChunks * 64 * kLayerWaves)
        return false;
    const LayerFusedPlan p = layer_fused_plan(L, block, halo, 1.f);
    return p.lds <= 160 * 1024;
}

// The split path (projection kernels around the attention kernel) measured
// faster on every shape tried: this kernel runs one four-wave workgroup per
// compute unit (the window of x fills most of the LDS) and projects k and v
// of every window pixel, (b + 2h)^2 / b^2 times the pixels of the block.
bool layer_fused_preferred(const LayerGeom& L, int block, int halo, int stride)
{
    (void)L; (void)block; (void)halo; (void)stride;
    return false;
}

template <int D, int NR>
static hipError_t layer_fused_nco(const void* x, const void* w_q, const void* w_kv, const void* w_o, const void* b_o,
                                  const void* rel_h, const void* rel_w, void* y, const LayerGeom& L, int block,
                                  int halo, const LayerFusedPlan& p, hipStream_t s)
{
    const int nco = L.Cout / 16;
#define HALO_LAYER_NCO(NC)                                                                                    \
    case NC: {                                                                                                \
        auto kern = layer_fused_kernel<D, NR, NC>;                                                           \
        hipError_t e = ensure_lds_limit((const void*)kern, p.lds);                                           \
        if (e != hipSuccess) return e;                                                                        \
        const int64_t nwg = (int64_t)L.B * p.nbh * p.nbw;                                                    \
        hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(64 * kLayerWaves), p.lds, s,                      \
                           (const __bf16*)x, (const __bf16*)w_q, (const __bf16*)w_kv, (const __bf16*)w_o,   \
                           (const __bf16*)b_o, (const __bf16*)rel_h, (const __bf16*)rel_w, (__bf16*)y, L,    \
                           block, halo, p);                                                                   \
        return hipGetLastError();                                                                             \
    }
    switch (nco) {
        HALO_LAYER_NCO(1) HALO_LAYER_NCO(2) HALO_LAYER_NCO(3) HALO_LAYER_NCO(4) HALO_LAYER_NCO(5)
        HALO_LAYER_NCO(6) HALO_LAYER_NCO(7) HALO_LAYER_NCO(8) HALO_LAYER_NCO(9) HALO_LAYER_NCO(10)
        HALO_LAYER_NCO(11) HALO_LAYER_NCO(12) HALO_LAYER_NCO(13) HALO_LAYER_NCO(14) HALO_LAYER_NCO(15)
        HALO_LAYER_NCO(16)
    }
#undef HALO_LAYER_NCO
    return hipErrorInvalidValue;
}

template <int D>
static hipError_t layer_fused_d(const void* x, const void* w_q, const void* w_kv, const void* w_o, const void* b_o,
                                const void* rel_h, const void* rel_w, void* y, const LayerGeom& L, int block, int halo,
                                const LayerFusedPlan& p, hipStream_t s)
{
    switch (p.nr) {
    case 6: return layer_fused_nco<D, 6>(x, w_q, w_kv, w_o, b_o, rel_h, rel_w, y, L, block, halo, p, s);
    case 8: return layer_fused_nco<D, 8>(x, w_q, w_kv, w_o, b_o, rel_h, rel_w, y, L, block, halo, p, s);
    case 10: return layer_fused_nco<D, 10>(x, w_q, w_kv, w_o, b_o, rel_h, rel_w, y, L, block, halo, p, s);
    case 12: return layer_fused_nco<D, 12>(x, w_q, w_kv, w_o, b_o, rel_h, rel_w, y, L, block, halo, p, s);
    case 14: return layer_fused_nco<D, 14>(x, w_q, w_kv, w_o, b_o, rel_h, rel_w, y, L, block, halo, p, s);
    case 16: return layer_fused_nco<D, 16>(x, w_q, w_kv, w_o, b_o, rel_h, rel_w, y, L, block, halo, p, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_layer_fused(const void* x, const void* w_q, const void* w_kv, const void* w_o, const void* b_o,
                              const void* rel_h, const void* rel_w, void* y, const LayerGeom& L, int block, int halo,
                              float scale, hipStream_t s)
{
    const LayerFusedPlan p = layer_fused_plan(L, block, halo, scale);
    if ((int64_t)L.B * p.nbh * p.nbw >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    if (L.d == 16) return layer_fused_d<16>(x, w_q, w_kv, w_o, b_o, rel_h, rel_w, y, L, block, halo, p, s);
    return layer_fused_d<32>(x, w_q, w_kv, w_o, b_o, rel_h, rel_w, y, L, block, halo, p, s);
}

}  // namespace halo
