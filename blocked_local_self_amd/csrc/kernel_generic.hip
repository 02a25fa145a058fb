// Generic halo-attention kernel: fp32 vector arithmetic, any supported shape.
//
// One workgroup per query block ("Scaling Local Self-Attention for Parameter
// Efficient Visual Backbones", section 2.2, Figure 1).  The block's window is
// streamed through LDS in chunks of KC keys (row-major over the r x r
// window; off-image positions flagged invalid, section 2.2 "padding at image
// borders", and skipped).  Each thread owns one query at a time and keeps an
// online softmax (running max, running sum, rescaled accumulator) so any
// window size works, including windows larger than the image (the global
// attention limit of section 2.2).  Logit, as in the HaloAttention module of
// the pswp.cn blog page (section 4):
//     scale * (q.k + q.rel_h[ky - y + c0] + q.rel_w[kx - x + c0]).
// This is the path for fp32 inputs, for shapes the matrix-core kernel does
// not cover, and a second implementation to cross-check that kernel.
//
// With STATS set the same kernel serves the backward pass: instead of the
// output it writes, per query, the log of the softmax normaliser in logit
// units (lse = m + log l) and dout . out, the two numbers every later
// gradient kernel needs.
#include "halo_common.h"

namespace halo {

constexpr int kGenericKC = 64;        // keys per LDS chunk
constexpr int kGenericThreads = 256;  // upper bound on workgroup size

// lse (may be null in the forward): natural log of each query's softmax
// normaliser, [B*heads][Ho][Wo].
template <int DMAX, typename T, bool STATS>
__global__ __launch_bounds__(kGenericThreads)
void generic_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                    const T* __restrict__ rel_h, const T* __restrict__ rel_w,
                    T* __restrict__ out, Geometry g,
                    const T* __restrict__ dout, float* __restrict__ lse, float* __restrict__ dsum)
{
    __shared__ float Ks[kGenericKC][DMAX];
    __shared__ float Vs[kGenericKC][DMAX];
    __shared__ int valid[kGenericKC];

    const int d = g.d;
    const int64_t nblk_img = (int64_t)g.nbh * g.nbw;
    const int64_t wg = blockIdx.x;
    const int64_t bh = wg / nblk_img;
    const int rem = (int)(wg - bh * nblk_img);
    const int by = rem / g.nbw, bx = rem - by * g.nbw;

    const int64_t plane = (int64_t)g.H * g.W * d;
    const T* qs = q + bh * plane;
    const T* ks = k + bh * plane;
    const T* vs = v + bh * plane;
    T* os = out + bh * (int64_t)g.Ho * g.Wo * d;

    // queries of this block: rows by*block + s*i inside the image
    const int ybeg = by * g.block, xbeg = bx * g.block;
    const int yend = min(ybeg + g.block, g.H), xend = min(xbeg + g.block, g.W);
    const int nqy = (yend - ybeg + g.stride - 1) / g.stride;
    const int nqx = (xend - xbeg + g.stride - 1) / g.stride;
    const int nq = nqy * nqx;
    const int y0 = ybeg - g.halo, x0 = xbeg - g.halo;   // window origin
    const int r = g.r, nkeys = r * r;
    // variants: centred mask; half-split embedding (height on channels
    // [0, d/2), width on [d/2, d))
    const bool cmask = g.flags & kFlagCentredMask;
    const int hlo = 0, hhi = (g.flags & kFlagHalfSplit) ? d / 2 : d;
    const int wlo = (g.flags & kFlagHalfSplit) ? d / 2 : 0;

    for (int qbase = 0; qbase < nq; qbase += blockDim.x) {
        const int qi = qbase + threadIdx.x;
        const bool active = qi < nq;
        int y = 0, x = 0;
        float qr[DMAX], o[DMAX];
        float m = -INFINITY, l = 0.f;
        if (active) {
            y = ybeg + (qi / nqx) * g.stride;
            x = xbeg + (qi % nqx) * g.stride;
            const T* qp = qs + ((int64_t)y * g.W + x) * d;
#pragma unroll
            for (int c = 0; c < DMAX; ++c) qr[c] = c < d ? to_f32(qp[c]) : 0.f;
        }
#pragma unroll
        for (int c = 0; c < DMAX; ++c) o[c] = 0.f;

        for (int kbase = 0; kbase < nkeys; kbase += kGenericKC) {
            __syncthreads();   // previous chunk fully consumed
            for (int e = threadIdx.x; e < kGenericKC * d; e += blockDim.x) {
                const int j = e / d, c = e - j * d;
                const int t = kbase + j;
                const int ky = y0 + t / r, kx = x0 + t % r;
                const bool in = t < nkeys && ky >= 0 && ky < g.H && kx >= 0 && kx < g.W;
                const int64_t off = ((int64_t)ky * g.W + kx) * d + c;
                Ks[j][c] = in ? to_f32(ks[off]) : 0.f;
                Vs[j][c] = in ? to_f32(vs[off]) : 0.f;
                // zero padding: off-image window positions are zero keys and values
                if (c == 0) valid[j] = in || (t < nkeys && (g.flags & kFlagZeroPad));
            }
            __syncthreads();
            if (!active) continue;
            const int jn = min(kGenericKC, nkeys - kbase);
            int cur_ky = INT32_MIN;
            float rh = 0.f;
            for (int j = 0; j < jn; ++j) {
                if (!valid[j]) continue;
                const int t = kbase + j;
                const int ky = y0 + t / r, kx = x0 + t % r;
                if (cmask && (ky < y - g.halo || ky > y + g.halo || kx < x - g.halo || kx > x + g.halo))
                    continue;         // centred mask: only keys within h rows and columns
                if (ky != cur_ky) {   // height term changes once per window row
                    cur_ky = ky;
                    const T* rp = rel_h + (int64_t)(ky - y + g.c0) * d;
                    float acc = 0.f;
#pragma unroll
                    for (int c = 0; c < DMAX; ++c) if (c >= hlo && c < hhi) acc += qr[c] * to_f32(rp[c]);
                    rh = acc;
                }
                const T* wp = rel_w + (int64_t)(kx - x + g.c0) * d;
                float s = rh;
#pragma unroll
                for (int c = 0; c < DMAX; ++c)
                    if (c < d) s += qr[c] * (Ks[j][c] + (c >= wlo ? to_f32(wp[c]) : 0.f));
                s *= g.scale;
                // online softmax update
                if (s > m) {
                    const float corr = __expf(m - s);   // 0 when m = -inf
                    l *= corr;
#pragma unroll
                    for (int c = 0; c < DMAX; ++c) o[c] *= corr;
                    m = s;
                }
                const float p = __expf(s - m);
                l += p;
#pragma unroll
                for (int c = 0; c < DMAX; ++c) o[c] += p * Vs[j][c];
            }
        }
        if (active) {
            const float inv = 1.f / l;
            const int64_t opix = (int64_t)((y / g.stride) * g.Wo + x / g.stride);
            if constexpr (STATS) {
                const T* gp = dout + bh * (int64_t)g.Ho * g.Wo * d + opix * d;
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < DMAX; ++c) if (c < d) acc += to_f32(gp[c]) * o[c];
                const int64_t qo = bh * (int64_t)g.Ho * g.Wo + opix;
                lse[qo] = m + __logf(l);
                dsum[qo] = acc * inv;
            } else {
                T* op = os + opix * d;
#pragma unroll
                for (int c = 0; c < DMAX; ++c) if (c < d) op[c] = from_f32<T>(o[c] * inv);
                if (lse != nullptr) lse[bh * (int64_t)g.Ho * g.Wo + opix] = m + __logf(l);
            }
        }
    }
}

template <int DMAX, typename T, bool STATS = false>
static hipError_t launch_generic_t(const void* q, const void* k, const void* v, const void* rh,
                                   const void* rw, void* out, const Geometry& g, hipStream_t st,
                                   const void* dout = nullptr, float* lse = nullptr, float* dsum = nullptr)
{
    const int64_t nblocks = g.BH * g.nbh * g.nbw;
    const int qmax = ((g.block + g.stride - 1) / g.stride) * ((g.block + g.stride - 1) / g.stride);
    int threads = ((qmax + 63) / 64) * 64;
    if (threads > kGenericThreads) threads = kGenericThreads;
    hipLaunchKernelGGL((generic_kernel<DMAX, T, STATS>), dim3((unsigned)nblocks), dim3(threads), 0, st,
                       (const T*)q, (const T*)k, (const T*)v, (const T*)rh, (const T*)rw, (T*)out, g,
                       (const T*)dout, lse, dsum);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_generic_dt(const void* q, const void* k, const void* v, const void* rh,
                                    const void* rw, void* out, float* lse, const Geometry& g, hipStream_t st)
{
    if (g.d <= 16) return launch_generic_t<16, T>(q, k, v, rh, rw, out, g, st, nullptr, lse);
    if (g.d <= 32) return launch_generic_t<32, T>(q, k, v, rh, rw, out, g, st, nullptr, lse);
    if (g.d <= 64) return launch_generic_t<64, T>(q, k, v, rh, rw, out, g, st, nullptr, lse);
    return launch_generic_t<128, T>(q, k, v, rh, rw, out, g, st, nullptr, lse);
}

// Softmax statistics for the backward pass (lse, dout . out per query).
template <typename T>
static hipError_t launch_stats_dt(const void* q, const void* k, const void* v, const void* rh,
                                  const void* rw, const void* dout, float* lse, float* dsum,
                                  const Geometry& g, hipStream_t st)
{
    if (g.d <= 16) return launch_generic_t<16, T, true>(q, k, v, rh, rw, nullptr, g, st, dout, lse, dsum);
    if (g.d <= 32) return launch_generic_t<32, T, true>(q, k, v, rh, rw, nullptr, g, st, dout, lse, dsum);
    if (g.d <= 64) return launch_generic_t<64, T, true>(q, k, v, rh, rw, nullptr, g, st, dout, lse, dsum);
    return launch_generic_t<128, T, true>(q, k, v, rh, rw, nullptr, g, st, dout, lse, dsum);
}

hipError_t launch_softmax_stats(const void* q, const void* k, const void* v, const void* rh,
                                const void* rw, const void* dout, float* lse, float* dsum,
                                const Geometry& g, bool bf16, hipStream_t st)
{
    return bf16 ? launch_stats_dt<__bf16>(q, k, v, rh, rw, dout, lse, dsum, g, st)
                : launch_stats_dt<float>(q, k, v, rh, rw, dout, lse, dsum, g, st);
}

// Host entry used by the dispatcher; d <= 128 is checked by the caller.
hipError_t launch_generic(const void* q, const void* k, const void* v, const void* rh,
                          const void* rw, void* out, float* lse, const Geometry& g, bool bf16, hipStream_t st)
{
    return bf16 ? launch_generic_dt<__bf16>(q, k, v, rh, rw, out, lse, g, st)
                : launch_generic_dt<float>(q, k, v, rh, rw, out, lse, g, st);
}

}  // namespace halo
