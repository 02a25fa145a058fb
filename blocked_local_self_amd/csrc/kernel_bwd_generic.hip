// Backward pass of halo attention: fp32 vector arithmetic, any supported
// shape, deterministic (no floating-point atomics anywhere).
//
// The pages give no backward pass; HaloNet's models are trained by gradient
// descent ("Scaling Local Self-Attention for Parameter Efficient Visual
// Backbones", section 4.1), so these kernels compute the exact derivative of
// the forward definition (sections 2.1-2.2; logit
//   l = scale * (q.k + q.rel_h[ky - y + c0] + q.rel_w[kx - x + c0])
// as in the HaloAttention module of the pswp.cn blog page, section 4):
//   P = softmax(l),  dl = P * (dout.v - dout.out),
//   dq = scale * sum_key dl (k + rel_h[row] + rel_w[col]),
//   dk = scale * sum_query dl q,   dv = sum_query P dout,
//   d rel_h[row] = scale * sum dl q over the (query, key) pairs at that row
//   displacement, likewise d rel_w.
//
// Kernels, in launch order (workspace layout in BwdWork):
//  1. softmax statistics per query (generic forward kernel in STATS mode):
//     lse = log of the normaliser, D = dout . out.
//  2. bwd_q_kernel: one workgroup per query block, one thread per query.
//     The window streams through LDS in chunks; each thread forms P and dl
//     of its keys and accumulates dq.  It also sums scale*dl over every
//     window row and every window column of its query (2r numbers per query,
//     kept in the workspace); after a barrier the workgroup turns those into
//     the block's partial table gradients, each entry summed over the
//     block's queries in a fixed order.
//  3. bwd_kv_kernel: one workgroup per key block (the b x b keys of one
//     block position), one thread per key.  The keys of a block are seen by
//     the queries of the blocks within ceil(h/b) block positions; their
//     query data (q, dout, lse, D) stream through LDS, and each thread sums
//     dk and dv over the queries whose window holds its key.  Keys are
//     owned by exactly one workgroup, so dk and dv need no atomics.
//  4. bwd_rel_reduce_kernel (levels of 32-row sums), then bwd_rel_final_kernel:
//     the partial table gradients summed over blocks in a fixed order, fp32.
#include <algorithm>

#include "halo_common.h"

namespace halo {

hipError_t launch_softmax_stats(const void* q, const void* k, const void* v, const void* rh,
                                const void* rw, const void* dout, float* lse, float* dsum,
                                const Geometry& g, bool bf16, hipStream_t st);

constexpr int kBwdKC = 64;           // keys per LDS chunk (bwd_q_kernel)
constexpr int kBwdQC = 64;           // queries per LDS chunk (bwd_kv_kernel)
constexpr int kBwdThreads = 256;     // upper bound on workgroup size
constexpr int kRelChunk = 32;        // rows summed per thread at each reduction level

// Workspace carve-up of the generic backward, in floats.
struct BwdWork {
    float* lse;      // [BH][Ho][Wo]   log normaliser of the scaled logits
    float* dsum;     // [BH][Ho][Wo]   dout . out
    float* gsum;     // [BH][Ho][Wo][2r]  per query: sum of scale*dl over window row t (t < r), column u (r + u)
    float* part;     // [nblocks][2][(2r-1)*d]  per block table gradients (rel_h, then rel_w)
    float* part2;    // [nchunks][2][(2r-1)*d]
};

// Rows of reduction scratch for nblocks partial rows: every level divides
// the row count by kRelChunk, so twice the first level's rows hold them all.
static int64_t bwd_nchunks(int64_t nblocks) { return 2 * ((nblocks + kRelChunk - 1) / kRelChunk) + 1; }

// Floats of workspace the generic backward needs.
int64_t bwd_generic_workspace_floats(const Geometry& g)
{
    const int64_t nq = g.BH * g.Ho * g.Wo;
    const int64_t nblocks = g.BH * g.nbh * g.nbw;
    const int64_t e2 = 2 * (int64_t)(2 * g.r - 1) * g.d;
    return 2 * nq + nq * 2 * g.r + nblocks * e2 + bwd_nchunks(nblocks) * e2;
}

static BwdWork bwd_carve(const Geometry& g, void* ws)
{
    BwdWork w;
    const int64_t nq = g.BH * g.Ho * g.Wo;
    const int64_t nblocks = g.BH * g.nbh * g.nbw;
    const int64_t e2 = 2 * (int64_t)(2 * g.r - 1) * g.d;
    w.lse = static_cast<float*>(ws);
    w.dsum = w.lse + nq;
    w.gsum = w.dsum + nq;
    w.part = w.gsum + nq * 2 * g.r;
    w.part2 = w.part + nblocks * e2;
    return w;
}

// Query block of workgroup `wg`: slice, block row/column, query grid.
struct QBlock {
    int64_t bh;
    int by, bx, ybeg, xbeg, nqy, nqx;
};
__device__ inline QBlock qblock_of(const Geometry& g, int64_t wg)
{
    QBlock b;
    const int64_t nblk_img = (int64_t)g.nbh * g.nbw;
    b.bh = wg / nblk_img;
    const int rem = (int)(wg - b.bh * nblk_img);
    b.by = rem / g.nbw;
    b.bx = rem - b.by * g.nbw;
    b.ybeg = b.by * g.block;
    b.xbeg = b.bx * g.block;
    b.nqy = (min(b.ybeg + g.block, g.H) - b.ybeg + g.stride - 1) / g.stride;
    b.nqx = (min(b.xbeg + g.block, g.W) - b.xbeg + g.stride - 1) / g.stride;
    return b;
}

template <int DMAX, typename T>
__global__ __launch_bounds__(kBwdThreads)
void bwd_q_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                  const T* __restrict__ rel_h, const T* __restrict__ rel_w,
                  const T* __restrict__ dout, T* __restrict__ dq, Geometry g, BwdWork w)
{
    __shared__ float Ks[kBwdKC][DMAX];
    __shared__ float Vs[kBwdKC][DMAX];
    __shared__ int valid[kBwdKC];

    const int d = g.d, r = g.r, nkeys = r * r;
    const QBlock qb = qblock_of(g, blockIdx.x);
    const int64_t plane = (int64_t)g.H * g.W * d;
    const int64_t qplane = (int64_t)g.Ho * g.Wo;
    const T* qs = q + qb.bh * plane;
    const T* ks = k + qb.bh * plane;
    const T* vs = v + qb.bh * plane;
    const int nq = qb.nqy * qb.nqx;
    const int y0 = qb.ybeg - g.halo, x0 = qb.xbeg - g.halo;
    // semantic variants (the forward's flags): zero padding, centred mask,
    // half-split embedding (height on channels < hhi, width on >= wlo)
    const bool zpad = g.flags & kFlagZeroPad, cmask = g.flags & kFlagCentredMask;
    const int hhi = (g.flags & kFlagHalfSplit) ? d / 2 : d;
    const int wlo = (g.flags & kFlagHalfSplit) ? d / 2 : 0;

    for (int qbase = 0; qbase < nq; qbase += blockDim.x) {
        const int qi = qbase + threadIdx.x;
        const bool active = qi < nq;
        int y = 0, x = 0;
        float qr[DMAX], gr[DMAX], acc[DMAX];
        float lse = 0.f, D = 0.f;
        float* gs = nullptr;
        if (active) {
            y = qb.ybeg + (qi / qb.nqx) * g.stride;
            x = qb.xbeg + (qi % qb.nqx) * g.stride;
            const int64_t opix = qb.bh * qplane + (int64_t)(y / g.stride) * g.Wo + x / g.stride;
            const T* qp = qs + ((int64_t)y * g.W + x) * d;
            const T* gp = dout + opix * d;
#pragma unroll
            for (int c = 0; c < DMAX; ++c) {
                qr[c] = c < d ? to_f32(qp[c]) : 0.f;
                gr[c] = c < d ? to_f32(gp[c]) : 0.f;
            }
            lse = w.lse[opix];
            D = w.dsum[opix];
            gs = w.gsum + opix * 2 * r;
            for (int t = 0; t < 2 * r; ++t) gs[t] = 0.f;
        }
#pragma unroll
        for (int c = 0; c < DMAX; ++c) acc[c] = 0.f;

        int cur_t = -1;
        float rh = 0.f, grow = 0.f;
        const T* rhp = rel_h;
        for (int kbase = 0; kbase < nkeys; kbase += kBwdKC) {
            __syncthreads();
            for (int e = threadIdx.x; e < kBwdKC * d; e += blockDim.x) {
                const int j = e / d, c = e - j * d;
                const int t = kbase + j;
                const int ky = y0 + t / r, kx = x0 + t % r;
                const bool in = t < nkeys && ky >= 0 && ky < g.H && kx >= 0 && kx < g.W;
                const int64_t off = ((int64_t)ky * g.W + kx) * d + c;
                Ks[j][c] = in ? to_f32(ks[off]) : 0.f;
                Vs[j][c] = in ? to_f32(vs[off]) : 0.f;
                if (c == 0) valid[j] = in || (zpad && t < nkeys);
            }
            __syncthreads();
            if (!active) continue;
            const int jn = min(kBwdKC, nkeys - kbase);
            for (int j = 0; j < jn; ++j) {
                if (!valid[j]) continue;
                const int idx = kbase + j;
                const int t = idx / r, u = idx - t * r;
                if (cmask && (y0 + t < y - g.halo || y0 + t > y + g.halo || x0 + u < x - g.halo ||
                              x0 + u > x + g.halo))
                    continue;
                if (t != cur_t) {            // window row changes: flush its sum
                    if (cur_t >= 0) gs[cur_t] = grow;
                    cur_t = t;
                    grow = 0.f;
                    rhp = rel_h + (int64_t)(y0 + t - y + g.c0) * d;
                    float a = 0.f;
#pragma unroll
                    for (int c = 0; c < DMAX; ++c) if (c < hhi) a += qr[c] * to_f32(rhp[c]);
                    rh = a;
                }
                const T* wp = rel_w + (int64_t)(x0 + u - x + g.c0) * d;
                float sc = rh, gv = 0.f;
#pragma unroll
                for (int c = 0; c < DMAX; ++c)
                    if (c < d) {
                        sc += qr[c] * (Ks[j][c] + (c >= wlo ? to_f32(wp[c]) : 0.f));
                        gv += gr[c] * Vs[j][c];
                    }
                const float p = __expf(sc * g.scale - lse);
                const float sdl = g.scale * p * (gv - D);
#pragma unroll
                for (int c = 0; c < DMAX; ++c)
                    if (c < d)
                        acc[c] += sdl * (Ks[j][c] + (c >= wlo ? to_f32(wp[c]) : 0.f) + (c < hhi ? to_f32(rhp[c]) : 0.f));
                grow += sdl;
                gs[r + u] += sdl;            // this thread's own entry
            }
        }
        if (active) {
            if (cur_t >= 0) gs[cur_t] = grow;
            T* dp = dq + qb.bh * plane + ((int64_t)y * g.W + x) * d;
#pragma unroll
            for (int c = 0; c < DMAX; ++c) if (c < d) dp[c] = from_f32<T>(acc[c]);
        }
    }
    __syncthreads();   // every query's row / column sums are written

    // this block's table gradients: entry (table, row R, channel c) sums
    // gsum(query, t) * q_c over the block's queries, t = R - (r-1) + (query's
    // block-local row, or column for rel_w)
    const int E = (2 * r - 1) * d;
    float* part = w.part + (int64_t)blockIdx.x * 2 * E;
    for (int e = threadIdx.x; e < 2 * E; e += blockDim.x) {
        const int tab = e / E, rem = e - tab * E;
        const int R = rem / d, c = rem - R * d;
        float acc = 0.f;
        for (int qi = 0; qi < nq; ++qi) {
            const int iy = qi / qb.nqx, ix = qi - iy * qb.nqx;
            const int yl = iy * g.stride, xl = ix * g.stride;
            // window row (column) whose table row is R for this query
            const int t = R + (tab == 0 ? yl : xl) + g.halo - g.c0;
            if (t < 0 || t >= r) continue;
            const int64_t opix = qb.bh * qplane + (int64_t)(qb.ybeg / g.stride + iy) * g.Wo +
                                 qb.xbeg / g.stride + ix;
            const float gsum = w.gsum[opix * 2 * r + tab * r + t];
            const int64_t qoff = ((int64_t)(qb.ybeg + yl) * g.W + qb.xbeg + xl) * d + c;
            acc += gsum * to_f32(qs[qoff]);
        }
        part[e] = (tab == 0 ? c < hhi : c >= wlo) ? acc : 0.f;   // unused half-split channels: 0
    }
}

template <int DMAX, typename T>
__global__ __launch_bounds__(kBwdThreads)
void bwd_kv_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                   const T* __restrict__ rel_h, const T* __restrict__ rel_w,
                   const T* __restrict__ dout, T* __restrict__ dk, T* __restrict__ dv,
                   Geometry g, BwdWork w)
{
    __shared__ float Qs[kBwdQC][DMAX];
    __shared__ float Gs[kBwdQC][DMAX];
    __shared__ float Ls[kBwdQC], Ds[kBwdQC];
    __shared__ int Ys[kBwdQC], Xs[kBwdQC];

    const int d = g.d;
    const int64_t nblk_img = (int64_t)g.nbh * g.nbw;
    const int64_t bh = blockIdx.x / nblk_img;
    const int rem = (int)(blockIdx.x - bh * nblk_img);
    const int kby = rem / g.nbw, kbx = rem - kby * g.nbw;
    const int kyb = kby * g.block, kxb = kbx * g.block;
    const int nky = min(kyb + g.block, g.H) - kyb, nkx = min(kxb + g.block, g.W) - kxb;
    const int nk = nky * nkx;
    const int64_t plane = (int64_t)g.H * g.W * d;
    const int64_t qplane = (int64_t)g.Ho * g.Wo;
    const T* qs = q + bh * plane;
    const T* gsrc = dout + bh * qplane * d;
    const int A = (g.halo + g.block - 1) / g.block;   // block positions a key's viewers reach
    const bool cmask = g.flags & kFlagCentredMask;
    const int hhi = (g.flags & kFlagHalfSplit) ? d / 2 : d;
    const int wlo = (g.flags & kFlagHalfSplit) ? d / 2 : 0;

    for (int kbase = 0; kbase < nk; kbase += blockDim.x) {
        const int ki = kbase + threadIdx.x;
        const bool active = ki < nk;
        const int ky = kyb + (active ? ki / nkx : 0), kx = kxb + (active ? ki % nkx : 0);
        float kr[DMAX], vr[DMAX], gk[DMAX], gvv[DMAX];
        const int64_t koff = bh * plane + ((int64_t)ky * g.W + kx) * d;
#pragma unroll
        for (int c = 0; c < DMAX; ++c) {
            kr[c] = (active && c < d) ? to_f32(k[koff + c]) : 0.f;
            vr[c] = (active && c < d) ? to_f32(v[koff + c]) : 0.f;
            gk[c] = 0.f;
            gvv[c] = 0.f;
        }
        for (int by = max(0, kby - A); by <= min(g.nbh - 1, kby + A); ++by)
            for (int bx = max(0, kbx - A); bx <= min(g.nbw - 1, kbx + A); ++bx) {
                const int wy0 = by * g.block - g.halo, wx0 = bx * g.block - g.halo;
                const bool mine = active && ky >= wy0 && ky < wy0 + g.r && kx >= wx0 && kx < wx0 + g.r;
                const int ybeg = by * g.block, xbeg = bx * g.block;
                const int nqy = (min(ybeg + g.block, g.H) - ybeg + g.stride - 1) / g.stride;
                const int nqx = (min(xbeg + g.block, g.W) - xbeg + g.stride - 1) / g.stride;
                const int nq = nqy * nqx;
                for (int qc = 0; qc < nq; qc += kBwdQC) {
                    const int qn = min(kBwdQC, nq - qc);
                    __syncthreads();
                    for (int e = threadIdx.x; e < qn * d; e += blockDim.x) {
                        const int j = e / d, c = e - j * d;
                        const int qi = qc + j;
                        const int y = ybeg + (qi / nqx) * g.stride, x = xbeg + (qi % nqx) * g.stride;
                        const int64_t opix = (int64_t)(y / g.stride) * g.Wo + x / g.stride;
                        Qs[j][c] = to_f32(qs[((int64_t)y * g.W + x) * d + c]);
                        Gs[j][c] = to_f32(gsrc[opix * d + c]);
                        if (c == 0) {
                            Ls[j] = w.lse[bh * qplane + opix];
                            Ds[j] = w.dsum[bh * qplane + opix];
                            Ys[j] = y;
                            Xs[j] = x;
                        }
                    }
                    __syncthreads();
                    if (!mine) continue;
                    for (int j = 0; j < qn; ++j) {
                        if (cmask && (ky < Ys[j] - g.halo || ky > Ys[j] + g.halo || kx < Xs[j] - g.halo ||
                                      kx > Xs[j] + g.halo))
                            continue;
                        const T* rhp = rel_h + (int64_t)(ky - Ys[j] + g.c0) * d;
                        const T* rwp = rel_w + (int64_t)(kx - Xs[j] + g.c0) * d;
                        float sc = 0.f, gv = 0.f;
#pragma unroll
                        for (int c = 0; c < DMAX; ++c)
                            if (c < d) {
                                sc += Qs[j][c] * (kr[c] + (c < hhi ? to_f32(rhp[c]) : 0.f) +
                                                  (c >= wlo ? to_f32(rwp[c]) : 0.f));
                                gv += Gs[j][c] * vr[c];
                            }
                        const float p = __expf(sc * g.scale - Ls[j]);
                        const float sdl = g.scale * p * (gv - Ds[j]);
#pragma unroll
                        for (int c = 0; c < DMAX; ++c) {
                            gk[c] += sdl * Qs[j][c];
                            gvv[c] += p * Gs[j][c];
                        }
                    }
                }
            }
        if (active) {
#pragma unroll
            for (int c = 0; c < DMAX; ++c)
                if (c < d) {
                    dk[koff + c] = from_f32<T>(gk[c]);
                    dv[koff + c] = from_f32<T>(gvv[c]);
                }
        }
    }
}

// out[y][e] = sum of in[n][e] over the rows n of chunk y = blockIdx.x
// (rows y*per .. min((y+1)*per, nin) - 1, in increasing order); entry
// e = blockIdx.y * blockDim.x + threadIdx.x < E.
__global__ __launch_bounds__(256)
void bwd_rel_reduce_kernel(const float* __restrict__ in, float* __restrict__ out,
                           int64_t E, int64_t nin, int64_t per)
{
    const int64_t e = (int64_t)blockIdx.y * blockDim.x + threadIdx.x;
    if (e >= E) return;
    const int64_t n0 = (int64_t)blockIdx.x * per;
    const int64_t n1 = min(n0 + per, nin);
    float acc = 0.f;
#pragma unroll 8
    for (int64_t n = n0; n < n1; ++n) acc += in[n * E + e];
    out[(int64_t)blockIdx.x * E + e] = acc;
}

// The two tables' gradients: entry e of the concatenated (rel_h, rel_w) row
// summed over the nin first-level rows in order.
__global__ __launch_bounds__(256)
void bwd_rel_final_kernel(const float* __restrict__ in, float* __restrict__ drh, float* __restrict__ drw,
                          int64_t E, int64_t nin)
{
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= E) return;
    float acc = 0.f;
#pragma unroll 8
    for (int64_t n = 0; n < nin; ++n) acc += in[n * E + e];
    const int64_t half = E / 2;
    if (e < half) drh[e] = acc;
    else drw[e - half] = acc;
}

// D = dout . out per query, from the forward's output (n queries of d channels).
template <typename T>
__global__ __launch_bounds__(256)
void bwd_dsum_kernel(const T* __restrict__ out, const T* __restrict__ dout, float* __restrict__ dsum,
                     int64_t n, int d)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        float acc = 0.f;
        for (int c = 0; c < d; ++c) acc += to_f32(out[i * d + c]) * to_f32(dout[i * d + c]);
        dsum[i] = acc;
    }
}

hipError_t launch_dsum(const void* out, const void* dout, float* dsum, const Geometry& g, bool bf16, hipStream_t st)
{
    const int64_t n = g.BH * g.Ho * g.Wo;
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 65536));
    if (bf16)
        hipLaunchKernelGGL(bwd_dsum_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const __bf16*)out, (const __bf16*)dout, dsum, n, g.d);
    else
        hipLaunchKernelGGL(bwd_dsum_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const float*)out, (const float*)dout, dsum, n, g.d);
    return hipGetLastError();
}

// Zero a buffer of `n` elements of T (the dq pixels strided queries never write).
template <typename T>
__global__ __launch_bounds__(256)
void zero_kernel(T* __restrict__ p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = from_f32<T>(0.f);
}

hipError_t launch_zero_bf16(void* p, int64_t n, hipStream_t st)
{
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 65536));
    hipLaunchKernelGGL(zero_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, st, (__bf16*)p, n);
    return hipGetLastError();
}

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t st)
{
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 65536));
    hipLaunchKernelGGL(zero_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

hipError_t launch_rel_reduce(const float* part, int64_t nrows, float* part2, float* drh, float* drw,
                             const Geometry& g, hipStream_t st);

template <int DMAX, typename T>
static hipError_t bwd_launch_t(const void* q, const void* k, const void* v, const void* rh, const void* rw,
                               const void* dout, void* dq, void* dk, void* dv, float* drh, float* drw,
                               const Geometry& g, const BwdWork& w, hipStream_t st)
{
    const int64_t nblocks = g.BH * g.nbh * g.nbw;
    const int side = (g.block + g.stride - 1) / g.stride;
    const int qthreads = std::min(kBwdThreads, ((side * side + 63) / 64) * 64);
    const int kthreads = std::min(kBwdThreads, ((g.block * g.block + 63) / 64) * 64);
    if (g.stride > 1) {
        const int64_t n = g.BH * g.H * g.W * g.d;
        const int64_t blocks = std::min<int64_t>((n + 255) / 256, 65536);
        hipLaunchKernelGGL(zero_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, st, (T*)dq, n);
    }
    hipLaunchKernelGGL((bwd_q_kernel<DMAX, T>), dim3((unsigned)nblocks), dim3(qthreads), 0, st,
                       (const T*)q, (const T*)k, (const T*)v, (const T*)rh, (const T*)rw, (const T*)dout,
                       (T*)dq, g, w);
    hipLaunchKernelGGL((bwd_kv_kernel<DMAX, T>), dim3((unsigned)nblocks), dim3(kthreads), 0, st,
                       (const T*)q, (const T*)k, (const T*)v, (const T*)rh, (const T*)rw, (const T*)dout,
                       (T*)dk, (T*)dv, g, w);
    return launch_rel_reduce(w.part, g.BH * g.nbh * g.nbw, w.part2, drh, drw, g, st);
}

// Table gradients from partials [nrows][2][(2r-1)*d] (one row per block or
// per workgroup): rows are summed kRelChunk at a time, level after level
// (scratch rows in part2, bwd_rel_chunks(nrows) of them), until at most
// kRelChunk remain; the last level writes the two tables.  Every sum runs in
// a fixed order.
hipError_t launch_rel_reduce(const float* part, int64_t nrows, float* part2, float* drh, float* drw,
                             const Geometry& g, hipStream_t st)
{
    const int64_t E = (int64_t)(2 * g.r - 1) * g.d * 2;
    const unsigned ey = (unsigned)((E + 255) / 256);
    const float* in = part;
    int64_t rows = nrows;
    float* dst = part2;
    while (rows > kRelChunk) {
        const int64_t nch = (rows + kRelChunk - 1) / kRelChunk;
        hipLaunchKernelGGL(bwd_rel_reduce_kernel, dim3((unsigned)nch, ey), dim3(256), 0, st, in, dst, E, rows,
                           (int64_t)kRelChunk);
        in = dst;
        dst += nch * E;
        rows = nch;
    }
    hipLaunchKernelGGL(bwd_rel_final_kernel, dim3(ey), dim3(256), 0, st, in, drh, drw, E, rows);
    return hipGetLastError();
}

int64_t bwd_rel_chunks(int64_t nrows) { return bwd_nchunks(nrows); }

template <typename T>
static hipError_t bwd_launch_dt(const void* q, const void* k, const void* v, const void* rh, const void* rw,
                                const void* dout, void* dq, void* dk, void* dv, float* drh, float* drw,
                                const Geometry& g, const BwdWork& w, hipStream_t st)
{
    if (g.d <= 16) return bwd_launch_t<16, T>(q, k, v, rh, rw, dout, dq, dk, dv, drh, drw, g, w, st);
    if (g.d <= 32) return bwd_launch_t<32, T>(q, k, v, rh, rw, dout, dq, dk, dv, drh, drw, g, w, st);
    if (g.d <= 64) return bwd_launch_t<64, T>(q, k, v, rh, rw, dout, dq, dk, dv, drh, drw, g, w, st);
    return bwd_launch_t<128, T>(q, k, v, rh, rw, dout, dq, dk, dv, drh, drw, g, w, st);
}

// Whole generic backward on `st`: statistics, dq + table partials, dk/dv,
// table reduction.  `ws` holds bwd_generic_workspace_floats(g) floats.
// With the forward's out and lse given, the statistics are lse itself and
// dout . out; otherwise both come from a recomputation of the softmax.
hipError_t launch_bwd_generic(const void* q, const void* k, const void* v, const void* rh, const void* rw,
                              const void* out, const void* dout, const float* lse,
                              void* dq, void* dk, void* dv, float* drh, float* drw,
                              void* ws, const Geometry& g, bool bf16, hipStream_t st)
{
    BwdWork w = bwd_carve(g, ws);
    hipError_t e;
    if (lse != nullptr) {
        w.lse = const_cast<float*>(lse);   // read only
        e = launch_dsum(out, dout, w.dsum, g, bf16, st);
    } else {
        e = launch_softmax_stats(q, k, v, rh, rw, dout, w.lse, w.dsum, g, bf16, st);
    }
    if (e != hipSuccess) return e;
    return bf16 ? bwd_launch_dt<__bf16>(q, k, v, rh, rw, dout, dq, dk, dv, drh, drw, g, w, st)
                : bwd_launch_dt<float>(q, k, v, rh, rw, dout, dq, dk, dv, drh, drw, g, w, st);
}

}  // namespace halo
