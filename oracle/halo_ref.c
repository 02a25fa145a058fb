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
 * Backward (halo_ref_bwd): the gradient of a scalar loss with respect to
 * q, k, v and both tables, given its gradient with respect to out; the
 * chain rule through the softmax of each query, nothing else.
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
 * Returns log(sum_j exp(l_j)), the log of the softmax normaliser.
 */
double halo_ref_set_attention(int d, int nkeys, const double* q,
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
    return m + log(z);
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
 * Whole forward pass.  nthreads <= 0 means the OpenMP default.  lse may be
 * NULL; otherwise it receives, per query ([B][heads][H/s][W/s]), the log of
 * its softmax normaliser, log sum_j exp(l_j) over its window keys.
 * Returns 0 on success, -1 on a null pointer, -2 on a bad shape,
 * -3 when scratch memory cannot be allocated.
 */
/*
 * Variants of the semantics (flags, OR-ed), for matching other readings of
 * the pages:
 *   HALO_REF_CENTRED_OFFSET (1): table row of displacement D is D + r - 1
 *     (the table's centre row) instead of D + r - 1 + h;
 *   HALO_REF_ZERO_PAD (2): window positions outside the image take part as
 *     zero keys and values (the "padding at image borders" of section 2.2
 *     read literally) instead of being left out;
 *   HALO_REF_CENTRED_MASK (4): a query attends only to the keys of its
 *     window within h rows and h columns of it (the centred (2h+1)^2
 *     neighbourhood of SASA, which section 2.2 says the blocked form
 *     drops);
 *   HALO_REF_HALF_SPLIT (8): the height embedding uses channels [0, d/2) and
 *     the width embedding channels [d/2, d) only (appendix A's factorised
 *     embedding, each half of the channels per axis).
 */
int halo_ref_fwd_ex(const double* q, const double* k, const double* v,
                    const double* rel_h, const double* rel_w, double* out, double* lse,
                    int B, int heads, int H, int W, int d,
                    int block, int halo, int stride, double scale, int flags, int nthreads)
{
    if (check_shape(B, heads, H, W, d, block, halo, stride)) return -2;
    if (flags & ~15) return -2;
    const long slices = (long)B * heads;
    if (slices == 0 || H == 0 || W == 0) return 0;
    if (!q || !k || !v || !rel_h || !rel_w || !out) return -1;

    const int r = block + 2 * halo;        /* window side */
    const int c0 = (flags & 1) ? r - 1 : r - 1 + halo;   /* table row of displacement 0 */
    const int zero_pad = (flags & 2) != 0, centred = (flags & 4) != 0;
    const int hlo = 0, hhi = (flags & 8) ? d / 2 : d;     /* channels of the height term */
    const int wlo = (flags & 8) ? d / 2 : 0, whi = d;     /* and of the width term */
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
    double* zero = calloc((size_t)d, sizeof(double));    /* key and value of a padded position */
    if (!keys || !vals || !bias || !logits || !zero) {
        free(keys); free(vals); free(bias); free(logits); free(zero);
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
                    const int row_in = ky >= 0 && ky < H;
                    if (!row_in && !zero_pad) continue;              /* off-image row */
                    if (centred && (ky < y - halo || ky > y + halo)) continue;
                    const double* rhr = rel_h + (long)(ky - y + c0) * d;
                    const double rh = dot(qv + hlo, rhr + hlo, hhi - hlo);
                    for (int kx = x0; kx < x0 + r; ++kx) {
                        const int in = row_in && kx >= 0 && kx < W;
                        if (!in && !zero_pad) continue;              /* off-image column */
                        if (centred && (kx < x - halo || kx > x + halo)) continue;
                        const long off = ((long)ky * W + kx) * d;
                        tk[n] = in ? ks + off : zero;
                        tv[n] = in ? vs + off : zero;
                        const double* rwr = rel_w + (long)(kx - x + c0) * d;
                        tb[n] = rh + dot(qv + wlo, rwr + wlo, whi - wlo);
                        ++n;
                    }
                }
                /* n >= 1: the query pixel lies inside its own window */
                const double z = halo_ref_set_attention(d, n, qv, tk, tb, tv, scale,
                                                        os + ((long)yo * Wo + xo) * d, tl);
                if (lse) lse[sl * (long)Ho * Wo + (long)yo * Wo + xo] = z;
            }
        }
    }
    free(keys);
    free(vals);
    free(bias);
    free(logits);
    free(zero);
    return 0;
}

/* The pages' default semantics: halo_ref_fwd_ex with no flags. */
int halo_ref_fwd(const double* q, const double* k, const double* v,
                 const double* rel_h, const double* rel_w, double* out, double* lse,
                 int B, int heads, int H, int W, int d,
                 int block, int halo, int stride, double scale, int nthreads)
{
    return halo_ref_fwd_ex(q, k, v, rel_h, rel_w, out, lse, B, heads, H, W, d, block, halo, stride,
                           scale, 0, nthreads);
}

/*
 * Backward of halo_ref_set_attention: the exact gradient of the scalar
 * sum_c g[c] * out[c] with respect to every input, by the chain rule through
 * the softmax.  The pages print no backward pass; HaloNet's models are
 * trained by gradient descent (section 4.1, Nesterov momentum on ImageNet),
 * so this is the derivative of the definition above, written out:
 *   P_j    = softmax(l)_j,  o = sum_j P_j val_j
 *   dl_j   = P_j * (g . val_j - g . o)          (softmax Jacobian)
 *   dq     = scale * sum_j dl_j key_j           (through q . key_j only)
 *   dkey_j = scale * dl_j * q
 *   dval_j = P_j * g
 *   dbias_j = scale * dl_j
 * dq[d], dbias[nkeys] are written; dkeys_j and dvals_j (arrays of nkeys
 * pointers to d-vectors) are ACCUMULATED into (+=), so a key seen by several
 * queries collects every contribution.  scratch holds 2*nkeys doubles.
 */
void halo_ref_set_attention_bwd(int d, int nkeys, const double* q,
                                const double* const* keys, const double* bias,
                                const double* const* vals, double scale,
                                const double* g, double* dq,
                                double* const* dkeys, double* const* dvals,
                                double* dbias, double* scratch)
{
    double* p = scratch;            /* softmax weights */
    double* gv = scratch + nkeys;   /* g . val_j */
    double m = -INFINITY;
    for (int j = 0; j < nkeys; ++j) {
        p[j] = scale * (dot(q, keys[j], d) + bias[j]);
        if (p[j] > m) m = p[j];
    }
    double z = 0.0;
    for (int j = 0; j < nkeys; ++j) {
        p[j] = exp(p[j] - m);
        z += p[j];
    }
    double go = 0.0;                /* g . o = sum_j P_j (g . val_j) */
    for (int j = 0; j < nkeys; ++j) {
        p[j] /= z;
        gv[j] = dot(g, vals[j], d);
        go += p[j] * gv[j];
    }
    for (int c = 0; c < d; ++c) dq[c] = 0.0;
    for (int j = 0; j < nkeys; ++j) {
        const double dl = p[j] * (gv[j] - go);
        dbias[j] = scale * dl;
        for (int c = 0; c < d; ++c) {
            dq[c] += scale * dl * keys[j][c];
            dkeys[j][c] += scale * dl * q[c];
            dvals[j][c] += p[j] * g[c];
        }
    }
}

/*
 * Whole backward pass: given dout (the gradient of a scalar loss with
 * respect to out, same layout as out), the gradients with respect to q, k,
 * v (layouts of the inputs) and to the two tables ([2r-1][d]).  Per query it
 * forms the same key set, biases and table rows as halo_ref_fwd, calls
 * halo_ref_set_attention_bwd, and sends the bias gradient of key j to both
 * tables and to q:  bias_j = q . rel_h[row_j] + q . rel_w[col_j], so
 *   dq += sum_j dbias_j (rel_h[row_j] + rel_w[col_j]),
 *   drel_h[row_j] += dbias_j q,  drel_w[col_j] += dbias_j q.
 * Queries of other (batch, head) slices never share keys, so slices run in
 * parallel; the tables' gradients are summed per slice and then over slices
 * in slice order (results do not depend on the thread count).
 * Returns 0, -1 (null pointer), -2 (bad shape) or -3 (no memory).
 */
int halo_ref_bwd_ex(const double* q, const double* k, const double* v,
                    const double* rel_h, const double* rel_w, const double* dout,
                    double* dq, double* dk, double* dv, double* drel_h, double* drel_w,
                    int B, int heads, int H, int W, int d,
                    int block, int halo, int stride, double scale, int flags, int nthreads)
{
    if (check_shape(B, heads, H, W, d, block, halo, stride)) return -2;
    if (flags & ~15) return -2;
    const int r = block + 2 * halo;
    /* the variants of halo_ref_fwd_ex: same key sets and biases */
    const int c0 = (flags & 1) ? r - 1 : r - 1 + halo;
    const int zero_pad = (flags & 2) != 0, centred = (flags & 4) != 0;
    const int hlo = 0, hhi = (flags & 8) ? d / 2 : d;
    const int wlo = (flags & 8) ? d / 2 : 0, whi = d;
    const long nrel = (long)(2 * r - 1) * d;
    if (!drel_h || !drel_w) return -1;
    for (long e = 0; e < nrel; ++e) drel_h[e] = drel_w[e] = 0.0;
    const long slices = (long)B * heads;
    if (slices == 0 || H == 0 || W == 0) return 0;
    if (!q || !k || !v || !rel_h || !rel_w || !dout || !dq || !dk || !dv) return -1;

    const int Ho = H / stride, Wo = W / stride;
    const long plane = (long)H * W * d;
    const long oplane = (long)Ho * Wo * d;
#ifdef _OPENMP
    const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    const int nt = 1;
    (void)nthreads;
#endif
    const size_t nk = (size_t)r * r;
    const double** keys = malloc(sizeof(double*) * nk * nt);
    const double** vals = malloc(sizeof(double*) * nk * nt);
    double** dkeys = malloc(sizeof(double*) * nk * nt);
    double** dvals = malloc(sizeof(double*) * nk * nt);
    int* rows = malloc(sizeof(int) * 2 * nk * nt);
    double* bias = malloc(sizeof(double) * nk * nt);
    double* dbias = malloc(sizeof(double) * nk * nt);
    double* scratch = malloc(sizeof(double) * 2 * nk * nt);
    double* qgrad = malloc(sizeof(double) * (size_t)d * nt);
    double* part = calloc((size_t)slices * 2 * nrel, sizeof(double));   /* per-slice table grads */
    double* zero = calloc((size_t)d, sizeof(double));             /* key / value of a padded position */
    double* sink = calloc((size_t)2 * d * nt, sizeof(double));    /* their (discarded) gradients */
    if (!keys || !vals || !dkeys || !dvals || !rows || !bias || !dbias || !scratch || !qgrad || !part ||
        !zero || !sink) {
        free(keys); free(vals); free(dkeys); free(dvals); free(rows);
        free(bias); free(dbias); free(scratch); free(qgrad); free(part); free(zero); free(sink);
        return -3;
    }
    for (long e = 0; e < slices * plane; ++e) dq[e] = dk[e] = dv[e] = 0.0;

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
        double** tdk = dkeys + t * nk;
        double** tdv = dvals + t * nk;
        int* trow = rows + t * 2 * nk;
        double* tb = bias + t * nk;
        double* tdb = dbias + t * nk;
        double* ts = scratch + t * 2 * nk;
        double* tq = qgrad + t * d;
        double* ph = part + sl * 2 * nrel;     /* this slice's d rel_h */
        double* pw = ph + nrel;                /* and d rel_w */
        const long so = sl * plane;
        for (int yo = 0; yo < Ho; ++yo) {
            for (int xo = 0; xo < Wo; ++xo) {
                const int y = yo * stride, x = xo * stride;
                const int y0 = (y / block) * block - halo;
                const int x0 = (x / block) * block - halo;
                const double* qv = q + so + ((long)y * W + x) * d;
                int n = 0;
                double* tsink = sink + t * 2 * d;
                for (int ky = y0; ky < y0 + r; ++ky) {
                    const int row_in = ky >= 0 && ky < H;
                    if (!row_in && !zero_pad) continue;
                    if (centred && (ky < y - halo || ky > y + halo)) continue;
                    const int rowh = ky - y + c0;
                    const double rh = dot(qv + hlo, rel_h + (long)rowh * d + hlo, hhi - hlo);
                    for (int kx = x0; kx < x0 + r; ++kx) {
                        const int in = row_in && kx >= 0 && kx < W;
                        if (!in && !zero_pad) continue;
                        if (centred && (kx < x - halo || kx > x + halo)) continue;
                        const int roww = kx - x + c0;
                        const long off = so + ((long)ky * W + kx) * d;
                        tk[n] = in ? k + off : zero;
                        tv[n] = in ? v + off : zero;
                        tdk[n] = in ? dk + off : tsink;
                        tdv[n] = in ? dv + off : tsink + d;
                        tb[n] = rh + dot(qv + wlo, rel_w + (long)roww * d + wlo, whi - wlo);
                        trow[2 * n] = rowh;
                        trow[2 * n + 1] = roww;
                        ++n;
                    }
                }
                halo_ref_set_attention_bwd(d, n, qv, tk, tb, tv, scale,
                                           dout + sl * oplane + ((long)yo * Wo + xo) * d,
                                           tq, tdk, tdv, tdb, ts);
                double* dqv = dq + so + ((long)y * W + x) * d;
                for (int c = 0; c < d; ++c) dqv[c] = tq[c];
                for (int j = 0; j < n; ++j) {
                    const double* rhr = rel_h + (long)trow[2 * j] * d;
                    const double* rwr = rel_w + (long)trow[2 * j + 1] * d;
                    double* ghr = ph + (long)trow[2 * j] * d;
                    double* gwr = pw + (long)trow[2 * j + 1] * d;
                    for (int c = hlo; c < hhi; ++c) {
                        dqv[c] += tdb[j] * rhr[c];
                        ghr[c] += tdb[j] * qv[c];
                    }
                    for (int c = wlo; c < whi; ++c) {
                        dqv[c] += tdb[j] * rwr[c];
                        gwr[c] += tdb[j] * qv[c];
                    }
                }
            }
        }
    }
    for (long sl = 0; sl < slices; ++sl)
        for (long e = 0; e < nrel; ++e) {
            drel_h[e] += part[sl * 2 * nrel + e];
            drel_w[e] += part[sl * 2 * nrel + nrel + e];
        }
    free(keys); free(vals); free(dkeys); free(dvals); free(rows);
    free(bias); free(dbias); free(scratch); free(qgrad); free(part); free(zero); free(sink);
    return 0;
}

/* The backward of the pages' default semantics: halo_ref_bwd_ex with no flags. */
int halo_ref_bwd(const double* q, const double* k, const double* v,
                 const double* rel_h, const double* rel_w, const double* dout,
                 double* dq, double* dk, double* dv, double* drel_h, double* drel_w,
                 int B, int heads, int H, int W, int d,
                 int block, int halo, int stride, double scale, int nthreads)
{
    return halo_ref_bwd_ex(q, k, v, rel_h, rel_w, dout, dq, dk, dv, drel_h, drel_w, B, heads, H, W, d,
                           block, halo, stride, scale, 0, nthreads);
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
