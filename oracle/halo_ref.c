/*
 * Plain fp64 CPU oracle for blocked local self-attention with haloing.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it; the
 * product path never calls it and shares no code with it.
 *
 * What it computes (the per-query definition, written out; no blocking,
 * fusion or reordering):
 *
 *   "Scaling Local Self-Attention for Parameter Efficient Visual Backbones"
 *   (HaloNet), section 2.1: each output pixel is a softmax-weighted sum of
 *   the values in its neighbourhood; the logit of key (a,b) for query (i,j)
 *   is the content term q_ij . k_ab plus the content-geometry term
 *   q_ij . r_{a-i,b-j}, one relative embedding per displacement, shared by
 *   all heads (note 1 of 2.1; appendix A factorises it per axis).
 *   Section 2.2 and Figure 1: the image is cut into non-overlapping b x b
 *   query blocks; a block's neighbourhood is the block plus a band of h
 *   pixels on every side, (b+2h) x (b+2h), with padding at the image border;
 *   no centred attention mask is used.  Section 2.2 and Figure 2: the strided
 *   variant subsamples the queries and keeps the stride-1 neighbourhoods.
 *
 *   The PyTorch HaloAttention module printed on the pswp.cn page
 *   ("Scaling Local Self-Attention..." blog post, section 4 "code") fixes the
 *   concrete form used here: the query is multiplied by the scale before both
 *   the content and the relative term; the relative term is
 *   q . rel_w[...] + q . rel_h[...] with two full-width tables of 2r-1 rows,
 *   r = b + 2h; its pad-and-reshape relative-to-absolute step selects, for a
 *   query at block-local position i and window position j along one axis,
 *   table row r-1+j-i, i.e. row (key - query) + (r-1+h) in image
 *   coordinates; padded (off-image) window positions are meant to be masked
 *   out of the softmax.
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes): off-image keys are excluded from the softmax; H and W need not be
 * multiples of b (tiling starts at the top-left, the last block row/column is
 * partial and keeps the full window geometry); strided queries sit at
 * (s*y', s*x'), displacements measured at full resolution; b % s == 0.
 *
 * Layouts: q, k, v are [B][heads][H][W][d] row-major; rel_h, rel_w are
 * [2r-1][d]; out is [B][heads][H/s][W/s][d].  All fp64.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double dot(const double* a, const double* b, int d)
{
    double acc = 0.0;
    for (int c = 0; c < d; ++c) acc += a[c] * b[c];
    return acc;
}

/*
 * Attention of one query over an explicit set of keys (HaloNet section 2.1):
 *   l_j   = scale * (q . key_j + bias_j)
 *   out   = sum_j softmax(l)_j * val_j
 * keys/vals are arrays of nkeys pointers to d-vectors; bias has nkeys
 * entries; logits is caller scratch of nkeys doubles.  The max is subtracted
 * before exponentiation (the result is unchanged by it).  nkeys must be >= 1.
 */
void halo_ref_set_attention(int d, int nkeys, const double* q,
                            const double* const* keys, const double* bias,
                            const double* const* vals, double scale,
                            double* out, double* logits)
{
    double m = -INFINITY;
    for (int j = 0; j < nkeys; ++j) {
        logits[j] = scale * (dot(q, keys[j], d) + bias[j]);
        if (logits[j] > m) m = logits[j];
    }
    double z = 0.0;
    for (int j = 0; j < nkeys; ++j) {
        logits[j] = exp(logits[j] - m);
        z += logits[j];
    }
    for (int c = 0; c < d; ++c) out[c] = 0.0;
    for (int j = 0; j < nkeys; ++j) {
        const double p = logits[j] / z;
        for (int c = 0; c < d; ++c) out[c] += p * vals[j][c];
    }
}

/* Same argument checks as the library's entry point; returns 0 or -2. */
static int check_shape(int B, int heads, int H, int W, int d, int block,
                       int halo, int stride)
{
    if (B < 0 || heads < 0 || H < 0 || W < 0) return -2;
    if (d < 1 || block < 1 || halo < 0 || stride < 1) return -2;
    if (block % stride != 0 || H % stride != 0 || W % stride != 0) return -2;
    return 0;
}

/*
 * Whole forward pass.  nthreads <= 0 means the OpenMP default.
 * Returns 0 on success, -1 on a null pointer, -2 on a bad shape,
 * -3 when scratch memory cannot be allocated.
 */
int halo_ref_fwd(const double* q, const double* k, const double* v,
                 const double* rel_h, const double* rel_w, double* out,
                 int B, int heads, int H, int W, int d,
                 int block, int halo, int stride, double scale, int nthreads)
{
    if (check_shape(B, heads, H, W, d, block, halo, stride)) return -2;
    const long slices = (long)B * heads;
    if (slices == 0 || H == 0 || W == 0) return 0;
    if (!q || !k || !v || !rel_h || !rel_w || !out) return -1;

    const int r = block + 2 * halo;        /* window side */
    const int c0 = r - 1 + halo;           /* table row of displacement 0 */
    const int Ho = H / stride, Wo = W / stride;
    const long plane = (long)H * W * d;    /* one (batch, head) slice */
    const long oplane = (long)Ho * Wo * d;
#ifdef _OPENMP
    const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    const int nt = 1;
    (void)nthreads;
#endif
    /* per-thread scratch, allocated up front */
    const size_t nk = (size_t)r * r;
    const double** keys = malloc(sizeof(double*) * nk * nt);
    const double** vals = malloc(sizeof(double*) * nk * nt);
    double* bias = malloc(sizeof(double) * nk * nt);
    double* logits = malloc(sizeof(double) * nk * nt);
    if (!keys || !vals || !bias || !logits) {
        free(keys); free(vals); free(bias); free(logits);
        return -3;
    }

#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
#endif
    for (long sl = 0; sl < slices; ++sl) {
#ifdef _OPENMP
        const size_t t = (size_t)omp_get_thread_num();
#else
        const size_t t = 0;
#endif
        const double** tk = keys + t * nk;
        const double** tv = vals + t * nk;
        double* tb = bias + t * nk;
        double* tl = logits + t * nk;
        const double* qs = q + sl * plane;
        const double* ks = k + sl * plane;
        const double* vs = v + sl * plane;
        double* os = out + sl * oplane;
        for (int yo = 0; yo < Ho; ++yo) {
            for (int xo = 0; xo < Wo; ++xo) {
                const int y = yo * stride, x = xo * stride;
                /* block holding the query, and its window origin */
                const int y0 = (y / block) * block - halo;
                const int x0 = (x / block) * block - halo;
                const double* qv = qs + ((long)y * W + x) * d;
                int n = 0;
                for (int ky = y0; ky < y0 + r; ++ky) {
                    if (ky < 0 || ky >= H) continue;      /* off-image row */
                    const double rh = dot(qv, rel_h + (long)(ky - y + c0) * d, d);
                    for (int kx = x0; kx < x0 + r; ++kx) {
                        if (kx < 0 || kx >= W) continue;  /* off-image column */
                        const long off = ((long)ky * W + kx) * d;
                        tk[n] = ks + off;
                        tv[n] = vs + off;
                        tb[n] = rh + dot(qv, rel_w + (long)(kx - x + c0) * d, d);
                        ++n;
                    }
                }
                /* n >= 1: the query pixel lies inside its own window */
                halo_ref_set_attention(d, n, qv, tk, tb, tv, scale,
                                       os + ((long)yo * Wo + xo) * d, tl);
            }
        }
    }
    free(keys);
    free(vals);
    free(bias);
    free(logits);
    return 0;
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int halo_ref_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
