// Halo attention for windows wider than 32 columns, and for 64-channel
// heads at any window of up to 32 columns (gfx950 matrix cores, bf16 in,
// fp32 accumulate): the detection setting of "Scaling Local
// Self-Attention for Parameter Efficient Visual Backbones", section 4.6
// (block 32, halo 3: 38x38 windows), with the method of section 2.2
// (Figures 1 and 2) and the relative logits of section 2.1 / appendix A as
// the HaloAttention module on the pswp.cn blog page (section 4) indexes them.
//
// A block this large has more queries than one workgroup should carry and a
// window whose K and V do not fit LDS twice per CU, so:
//  * a workgroup takes one group of query tiles of one block (8 waves x QT
//    tiles of 16 queries); the groups of a block, and neighbouring blocks,
//    are consecutive in the XCD-grouped order, so they read the window's K
//    and V through one L2;
//  * the window streams through LDS in chunks of kWideRows rows (K as
//    [row][col][d], V transposed to [d][row][col], 16*NCH columns);
//  * the softmax is online: per group of two window rows the scores stay in
//    registers, their maximum updates the running maximum of each query,
//    and O and L are rescaled by exp2(old - new) before the group's
//    weights are added.  One pass over the scores, exact result;
//  * scores are transposed, S^T = K . Q^T (lane (n, g): query n, window
//    columns 4g..4g+3 of one 16-column chunk of one row), so the width term
//    q.rel_w[col] is the accumulator input (masked columns -1e30) and the
//    height term q.rel_h[row] is one scalar per (lane, row); both come from
//    MFMAs against the tables, re-indexed per query through LDS.
#include <algorithm>
#include <type_traits>

#include "mfma_util.h"

namespace halo {

#ifndef HALO_WIDE_ROWS
#define HALO_WIDE_ROWS 14
#endif
#ifndef HALO_WIDE_QT
#define HALO_WIDE_QT 1
#endif
#ifndef HALO_WIDE_WAVES
#define HALO_WIDE_WAVES 8
#endif
constexpr int kWideWaves = HALO_WIDE_WAVES;
constexpr int kWideRows = HALO_WIDE_ROWS;   // window rows per LDS chunk

// QK^T operands of this kernel: those of the other kernels for 16 and 32
// channels; for 64, a lane holds 16 consecutive channels (quarter gq of the
// head) and the contraction is two K = 32 MFMAs over its two halves.  Both
// operands use the same lane -> channel map, so the sum runs over exactly the
// d channels.
typedef short s16x16 __attribute__((ext_vector_type(16)));
template <int D> struct WFrag : Frag<D> {};
template <> struct WFrag<64> {
    typedef s16x16 T;
    __device__ static inline f32x4 mma(T a, T b, f32x4 c) {
        const s16x8 a0 = __builtin_shufflevector(a, a, 0, 1, 2, 3, 4, 5, 6, 7);
        const s16x8 a1 = __builtin_shufflevector(a, a, 8, 9, 10, 11, 12, 13, 14, 15);
        const s16x8 b0 = __builtin_shufflevector(b, b, 0, 1, 2, 3, 4, 5, 6, 7);
        const s16x8 b1 = __builtin_shufflevector(b, b, 8, 9, 10, 11, 12, 13, 14, 15);
        return mma_k32(a1, b1, mma_k32(a0, b0, c));
    }
};

struct WidePlan {
    int groups;       // workgroups per block
    int SW;           // LDS row pitch in columns (16 * NCH)
    int RP;           // relative-table rows padded to 16
    int HR;           // height rows kept per query tile (r rounded up to 16)
    int CPv;          // V^T channel pitch in elements (kWideRows * SW, padded)
    int off_v, off_rel, off_hgt, lds_bytes;
    int remap_xcd;
    int64_t nwg;
    float alpha;      // scale * log2(e)
};

template <int D, int NCH, int QT>
__global__ __launch_bounds__(64 * kWideWaves) __attribute__((amdgpu_waves_per_eu(2)))
void wide_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                 const __bf16* __restrict__ v, const __bf16* __restrict__ rel_h,
                 const __bf16* __restrict__ rel_w, __bf16* __restrict__ out,
                 float* __restrict__ lse, Geometry g, WidePlan p)
{
    constexpr int KPL = D / 4;
    constexpr int CPP = D / 8;                // 16-byte chunks per pixel
    typedef typename WFrag<D>::T FragT;
    extern __shared__ __align__(16) unsigned char smem[];
    __bf16* Kc = reinterpret_cast<__bf16*>(smem);                  // [kWideRows][SW][D], swizzled
    // K pixels hold their 16-byte (8-channel) units in an order XOR-ed with
    // bits of the column, so the 16 (8-byte reads) or 8 (16-byte reads)
    // lanes of one LDS pass, which read one unit of consecutive columns, fall
    // on different banks (two lanes per bank pair at d = 16)
    constexpr int KSH = D == 16 ? 2 : D == 32 ? 1 : 0;
    auto kunit = [](int col, int unit) { return (unit ^ ((col >> KSH) & (CPP - 1))) * 8; };
    __bf16* Vc = reinterpret_cast<__bf16*>(smem + p.off_v);        // [D][CPv >= kWideRows * SW]
    __bf16* Rh = reinterpret_cast<__bf16*>(smem + p.off_rel);      // [RP][D]
    __bf16* Rw = Rh + p.RP * D;                                     // [RP][D]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, gq = lane >> 4;
    const int r = g.r, SW = p.SW;
    const float alpha = p.alpha;
    // per-wave scratch of the relative phase (aliases the chunk buffers,
    // which are not in use yet) and the per-query height terms
    float* scr = reinterpret_cast<float*>(smem) + wave * p.RP * 16;                 // [RP][16]
    float* hgt = reinterpret_cast<float*>(smem + p.off_hgt) + wave * QT * p.HR * 16;  // QT x [HR][16]

    int64_t wg = blockIdx.x;
    if (p.remap_xcd) {
        const int64_t per = p.nwg >> 3;
        wg = (wg & 7) * per + (wg >> 3);
    }
    const int grp = (int)(wg % p.groups);
    int64_t rest = wg / p.groups;
    const int bx = (int)(rest % g.nbw);
    rest /= g.nbw;
    const int by = (int)(rest % g.nbh);
    const int64_t bh = rest / g.nbh;
    const int yb = by * g.block, xb = bx * g.block;
    const int wy0 = yb - g.halo, wx0 = xb - g.halo;
    const int tlo = max(0, -wy0), thi = min(r, g.H - wy0);
    const int64_t plane = (int64_t)g.H * g.W * D;
    const int nqy = (min(yb + g.block, g.H) - yb + g.stride - 1) / g.stride;
    const int nqx = (min(xb + g.block, g.W) - xb + g.stride - 1) / g.stride;
    const int nq = nqy * nqx, nqt = (nq + 15) / 16;
    const int tq0 = (grp * kWideWaves + wave) * QT;
    const bool active = tq0 < nqt;              // wave-uniform; idle waves still stage

    // ---- tables
    {
        const int nrel = 2 * r - 1;
        const unsigned short* rhs = reinterpret_cast<const unsigned short*>(rel_h);
        const unsigned short* rws = reinterpret_cast<const unsigned short*>(rel_w);
        unsigned short* rhd = reinterpret_cast<unsigned short*>(Rh);
        unsigned short* rwd = reinterpret_cast<unsigned short*>(Rw);
        for (int e = tid; e < p.RP * D; e += 64 * kWideWaves) {
            const bool in = e < nrel * D;
            rhd[e] = in ? rhs[e] : (unsigned short)0;
            rwd[e] = in ? rws[e] : (unsigned short)0;
        }
    }
    __syncthreads();

    // ---- query tiles (lane n; padding lanes reuse query 0 of the block)
    FragT qf[QT];
    bool qvalid[QT];
    int qpix[QT], yl[QT], xl[QT];
#pragma unroll
    for (int u = 0; u < QT; ++u) {
        const int qi = (tq0 + u) * 16 + n;
        qvalid[u] = active && qi < nq;
        const int qq = qvalid[u] ? qi : 0;
        yl[u] = (qq / nqx) * g.stride;
        xl[u] = (qq % nqx) * g.stride;
        qpix[u] = (yb + yl[u]) * g.W + xb + xl[u];
        qf[u] = *reinterpret_cast<const FragT*>(q + bh * plane + (int64_t)qpix[u] * D + gq * KPL);
    }

    // ---- relative logits of every table row, re-indexed per query: the
    // width term of window column c = 16 ch + 4g + i (accumulator input,
    // -1e30 off the image or past the window) and the height term of window
    // row t (kept in LDS for the stream)
    f32x4 cinit[QT][NCH];
    const int rp16 = p.RP / 16;
    if (active) {
#pragma unroll
        for (int u = 0; u < QT; ++u)
            for (int pass = 0; pass < 2; ++pass) {
                const __bf16* tab = pass == 0 ? Rw : Rh;
                for (int rt = 0; rt < rp16; ++rt) {
                    const FragT a = *reinterpret_cast<const FragT*>(tab + (rt * 16 + n) * D + gq * KPL);
                    const f32x4 gr = WFrag<D>::mma(a, qf[u], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int i = 0; i < 4; ++i) scr[(rt * 16 + gq * 4 + i) * 16 + n] = gr[i];
                }
                wave_lds_sync();
                if (pass == 0) {
#pragma unroll
                    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int c = ch * 16 + gq * 4 + i;
                            const int ix = wx0 + c;
                            const bool ok = c < r && ix >= 0 && ix < g.W;
                            const float val = scr[min(r - 1 - xl[u] + c, p.RP - 1) * 16 + n];
                            cinit[u][ch][i] = ok ? val : kMaskLogit;
                        }
                } else {
                    // height of window row t: scratch row (r-1-yl) + t, in
                    // base-2 units (alpha applied)
                    for (int t = gq; t < r; t += 4)
                        hgt[(u * p.HR + t) * 16 + n] = alpha * scr[(r - 1 - yl[u] + t) * 16 + n];
                }
                wave_lds_sync();
            }
    }
    __syncthreads();                 // the scratch (chunk buffers) is free again

    s16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (short)0x3F80;

    f32x4 O[QT][D / 16], L[QT];
    float M[QT];                      // running maximum of the base-2 logits (per query)
#pragma unroll
    for (int u = 0; u < QT; ++u) {
        L[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt) O[u][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        M[u] = -3.0e38f;
    }
    const __bf16* kbase = k + bh * plane;
    const __bf16* vbase = v + bh * plane;

    for (int c0 = tlo; c0 < thi; c0 += kWideRows) {
        const int c1 = min(thi, c0 + kWideRows);
        // ---- stage window rows c0..c1-1 (chunk row t - c0), columns 0..SW-1;
        // off-image columns and columns past the window are zero
        {
            const int ng4 = SW / 4;
            const int total = (c1 - c0) * ng4 * CPP;
            for (int e = tid; e < total; e += 64 * kWideWaves) {
                const int ch = e % CPP;
                const int rr = e / CPP;
                const int c4 = rr % ng4;
                const int tr = rr / ng4;                       // chunk row
                const int iy = wy0 + c0 + tr;
                u32x4 kk[4], vv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = 4 * c4 + j, ix = wx0 + c;
                    kk[j] = u32x4{0u, 0u, 0u, 0u};
                    vv[j] = u32x4{0u, 0u, 0u, 0u};
                    if (c < r && ix >= 0 && ix < g.W) {
                        const int64_t off = ((int64_t)iy * g.W + ix) * D + ch * 8;
                        kk[j] = *reinterpret_cast<const u32x4*>(kbase + off);
                        vv[j] = *reinterpret_cast<const u32x4*>(vbase + off);
                    }
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<u32x4*>(Kc + ((size_t)(tr * SW + 4 * c4 + j) * D + kunit(4 * c4 + j, ch))) = kk[j];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const u32x2 lo = {__builtin_amdgcn_perm(vv[1][w], vv[0][w], 0x05040100u),
                                      __builtin_amdgcn_perm(vv[3][w], vv[2][w], 0x05040100u)};
                    const u32x2 hi = {__builtin_amdgcn_perm(vv[1][w], vv[0][w], 0x07060302u),
                                      __builtin_amdgcn_perm(vv[3][w], vv[2][w], 0x07060302u)};
                    *reinterpret_cast<u32x2*>(Vc + (size_t)(ch * 8 + 2 * w) * p.CPv + tr * SW + 4 * c4) = lo;
                    *reinterpret_cast<u32x2*>(Vc + (size_t)(ch * 8 + 2 * w + 1) * p.CPv + tr * SW + 4 * c4) = hi;
                }
            }
        }
        __syncthreads();

        if (active) {
            // lane (n, g): column n of a 16-column chunk (the swizzle depends
            // on n only: 16 is a multiple of CPP << KSH), channels g*KPL..+KPL-1
            const __bf16* kfrag0 = Kc + (size_t)n * D + (D == 16 ? kunit(n, gq >> 1) + (gq & 1) * 4
                                                                : kunit(n, D == 32 ? gq : 2 * gq));
            const __bf16* kfrag1 = Kc + (size_t)n * D + (D == 64 ? kunit(n, 2 * gq + 1) : 0);
            auto kload = [&](int tr, int ch) -> FragT {
                const size_t o = (size_t)(tr * SW + ch * 16) * D;
                if constexpr (D == 64) {
                    const s16x8 lo = *reinterpret_cast<const s16x8*>(kfrag0 + o);
                    const s16x8 hi = *reinterpret_cast<const s16x8*>(kfrag1 + o);
                    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
                } else {
                    return *reinterpret_cast<const FragT*>(kfrag0 + o);
                }
            };
            const __bf16* vfrag = Vc + (size_t)n * p.CPv + gq * 4;
            auto vload = [&](int mt, int tr, int ch) -> u32x2 {
                return *reinterpret_cast<const u32x2*>(vfrag + (size_t)mt * 16 * p.CPv + tr * SW + ch * 16);
            };
            // groups of two window rows (the last may hold one)
            for (int t = c0; t < c1; t += 2) {
                const bool two = t + 1 < c1;                  // wave-uniform
                const int tr0 = t - c0, tr1 = two ? tr0 + 1 : tr0;
                FragT a[2][NCH];
#pragma unroll
                for (int ch = 0; ch < NCH; ++ch) {
                    a[0][ch] = kload(tr0, ch);
                    a[1][ch] = kload(tr1, ch);
                }
#pragma unroll
                for (int u = 0; u < QT; ++u) {
                    const float h0 = hgt[(u * p.HR + t) * 16 + n];
                    const float h1 = two ? hgt[(u * p.HR + t + 1) * 16 + n] : -INFINITY;
                    f32x4 s[2][NCH];
                    float mx0 = -3.0e38f, mx1 = -3.0e38f;
#pragma unroll
                    for (int ch = 0; ch < NCH; ++ch) {
                        s[0][ch] = WFrag<D>::mma(a[0][ch], qf[u], cinit[u][ch]);
                        s[1][ch] = WFrag<D>::mma(a[1][ch], qf[u], cinit[u][ch]);
                        mx0 = fmaxf(mx0, max4(s[0][ch]));
                        mx1 = fmaxf(mx1, max4(s[1][ch]));
                    }
                    // base-2 maximum of the group, over the four lanes of the query
                    const float gm = max_over_rows(fmaxf(fmaf(mx0, alpha, h0), two ? fmaf(mx1, alpha, h1) : -3.0e38f));
                    const float mnew = fmaxf(M[u], gm);
                    const float f = __builtin_amdgcn_exp2f(M[u] - mnew);
                    M[u] = mnew;
#pragma unroll
                    for (int mt = 0; mt < D / 16; ++mt) O[u][mt] *= f;
                    L[u] *= f;
                    const float e0 = h0 - mnew, e1 = h1 - mnew;
                    // weights of the group's 2*NCH score tiles, row-major, two per K=32 step
                    unsigned pw[2 * NCH][2];
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int ch = 0; ch < NCH; ++ch) {
                            const float e = j == 0 ? e0 : e1;
                            const f32x4 sv = s[j][ch];
                            pw[j * NCH + ch][0] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sv[0], alpha, e)),
                                                              __builtin_amdgcn_exp2f(fmaf(sv[1], alpha, e)));
                            pw[j * NCH + ch][1] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sv[2], alpha, e)),
                                                              __builtin_amdgcn_exp2f(fmaf(sv[3], alpha, e)));
                        }
#pragma unroll
                    for (int st = 0; st < NCH; ++st) {           // tiles 2st, 2st+1
                        const int ta = 2 * st, tb = 2 * st + 1;
                        const s16x8 pf = __builtin_bit_cast(s16x8, u32x4{pw[ta][0], pw[ta][1], pw[tb][0], pw[tb][1]});
#pragma unroll
                        for (int mt = 0; mt < D / 16; ++mt) {
                            const u32x2 x0 = vload(mt, ta / NCH == 0 ? tr0 : tr1, ta % NCH);
                            const u32x2 x1 = vload(mt, tb / NCH == 0 ? tr0 : tr1, tb % NCH);
                            O[u][mt] = mma_k32(__builtin_bit_cast(s16x8, u32x4{x0[0], x0[1], x1[0], x1[1]}), pf, O[u][mt]);
                        }
                        L[u] = mma_k32(ones, pf, L[u]);
                    }
                }
            }
        }
        __syncthreads();             // the chunk buffers are restaged next
    }

    // ---- normalise and store: lane (n, g) holds channels 16*mt + 4g + i of query n
#pragma unroll
    for (int u = 0; u < QT; ++u) {
        if (!qvalid[u]) continue;
        const float inv = 1.0f / L[u][0];
        const int yq = qpix[u] / g.W, xq = qpix[u] - yq * g.W;
        const int64_t opix = bh * (int64_t)g.Ho * g.Wo + (int64_t)(yq / g.stride) * g.Wo + xq / g.stride;
        __bf16* op = out + opix * D + gq * 4;
        if (lse != nullptr && gq == 0)   // natural log of the normaliser: (max + log2 L) ln 2
            lse[opix] = (M[u] + __builtin_amdgcn_logf(L[u][0])) * 0.6931471805599453f;
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt)
            *reinterpret_cast<u32x2*>(op + mt * 16) = u32x2{pack_bf16x2(O[u][mt][0] * inv, O[u][mt][1] * inv),
                                                            pack_bf16x2(O[u][mt][2] * inv, O[u][mt][3] * inv)};
    }
}

static int wround(int x, int m) { return (x + m - 1) / m * m; }

// Windows of 33..48 columns (three 16-column chunks) for d = 16 and 32
// (two chunk buffers of 14 rows x 48 columns: 43 KB each at d = 32), and
// every window of up to 32 columns (one or two chunks) for d = 64, which
// the other matrix-core kernels do not take (two buffers of 14 rows x 32
// columns x 64 channels: 57 KB each).
bool wide_supported(const Geometry& g, bool bf16)
{
    if (!bf16 || g.block % 4 != 0) return false;
    if (g.d == 64) return g.r <= 32;
    return (g.d == 16 || g.d == 32) && g.r > 32 && g.r <= 48;
}

template <int D, int NCH, int QT>
static hipError_t wide_t(const void* q, const void* k, const void* v, const void* rh, const void* rw, void* out,
                         float* lse, const Geometry& g, hipStream_t st)
{
    WidePlan p{};
    p.SW = 16 * NCH;
    p.RP = wround(2 * g.r - 1, 16);
    p.HR = wround(g.r, 16);
    const int chunk = kWideRows * p.SW * D * 2;
    // V^T channel pitch: (pitch / 2) = 2 (mod 32) dwords, so the 16 channels
    // of a fragment read (8 bytes per lane) cover the 32 banks once
    p.CPv = kWideRows * p.SW;
    while (p.CPv % 2 || (p.CPv / 2) % 32 != 2) ++p.CPv;
    p.off_v = chunk;
    const int scratch = kWideWaves * p.RP * 16 * 4;             // aliases the chunk buffers
    p.off_rel = wround(std::max(chunk + D * p.CPv * 2, scratch), 16);
    p.off_hgt = wround(p.off_rel + 2 * p.RP * D * 2, 16);
    p.lds_bytes = p.off_hgt + kWideWaves * QT * p.HR * 16 * 4;
    const int side = (g.block + g.stride - 1) / g.stride;
    const int nqt = (side * side + 15) / 16;
    p.groups = (nqt + kWideWaves * QT - 1) / (kWideWaves * QT);
    p.nwg = g.BH * g.nbh * g.nbw * p.groups;
    p.remap_xcd = (p.nwg % 8 == 0) ? 1 : 0;
    p.alpha = (float)((double)g.scale * 1.4426950408889634);
    auto kern = wide_kernel<D, NCH, QT>;
    {
        const hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), p.lds_bytes);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)p.nwg), dim3(64 * kWideWaves), p.lds_bytes, st, (const __bf16*)q, (const __bf16*)k,
                       (const __bf16*)v, (const __bf16*)rh, (const __bf16*)rw, (__bf16*)out, lse, g, p);
    return hipGetLastError();
}

hipError_t launch_wide(const void* q, const void* k, const void* v, const void* rh, const void* rw, void* out,
                       float* lse, const Geometry& g, hipStream_t st)
{
    if (g.d == 64) {
        // a block of 9..16 query tiles in one workgroup of two tiles per wave
        // rather than two workgroups (each staging the whole window), the
        // second nearly idle
        const int side = (g.block + g.stride - 1) / g.stride;
        const bool two = (side * side + 15) / 16 > kWideWaves;
        if (g.r <= 16) return two ? wide_t<64, 1, 2>(q, k, v, rh, rw, out, lse, g, st)
                                  : wide_t<64, 1, 1>(q, k, v, rh, rw, out, lse, g, st);
        return two ? wide_t<64, 2, 2>(q, k, v, rh, rw, out, lse, g, st)
                   : wide_t<64, 2, 1>(q, k, v, rh, rw, out, lse, g, st);
    }
    if (g.d == 32) {
        // one workgroup per CU (121 KB of LDS), two waves per SIMD: two query
        // tiles per wave give each wave independent MFMA -> exp -> MFMA chains
        // to interleave (r = 38 at block 32: 189 -> 151 us), where a block
        // has the tiles to keep all eight waves busy; at d = 16 (two
        // workgroups per CU) a second tile per wave measured slower
        const int side = (g.block + g.stride - 1) / g.stride;
        if ((side * side + 15) / 16 >= 2 * kWideWaves) return wide_t<32, 3, 2>(q, k, v, rh, rw, out, lse, g, st);
        return wide_t<32, 3, HALO_WIDE_QT>(q, k, v, rh, rw, out, lse, g, st);
    }
    return wide_t<16, 3, HALO_WIDE_QT>(q, k, v, rh, rw, out, lse, g, st);
}

}  // namespace halo
