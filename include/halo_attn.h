/*
 * halo_attn.h -- C ABI of the MI355X (gfx950) halo-attention library.
 *
 * The operation: HaloNet's blocked local self-attention with haloing, forward
 * and backward pass, on already projected queries, keys and values ("Scaling
 * Local Self-Attention for Parameter Efficient Visual Backbones").
 *
 *  - Section 2.2, Figure 1: the H x W map is cut into non-overlapping
 *    block x block query blocks, tiled from the top-left (a last block row or
 *    column may be partial when block does not divide H or W).  Every query of
 *    a block attends to the same window: the block plus a halo of `halo`
 *    pixels on every side, side r = block + 2*halo.  Window positions outside
 *    the image are padding and take no part in the softmax.  No centred mask.
 *  - Section 2.1 and appendix A: the logit of key (ky,kx) for query (y,x) is
 *    the content term plus a content-geometry term built from one relative
 *    table per axis, shared by all heads.  The concrete form, as in the
 *    HaloAttention module of the pswp.cn blog page (section 4):
 *        l = scale * ( q.k + q.rel_h[ky - y + c0] + q.rel_w[kx - x + c0] )
 *    with c0 = r - 1 + halo, tables of 2r-1 rows; out = softmax(l) . v over
 *    the in-image window keys.
 *  - Section 2.2, Figure 2: with query_stride s > 1 only the queries at
 *    (s*y', s*x') are computed; their windows are the stride-1 windows.
 *
 * Layouts (all row-major, contiguous, d innermost):
 *   q, k, v      [B][heads][H][W][d]
 *   rel_h, rel_w [2r-1][d]          one pair shared by every batch and head
 *   out          [B][heads][H/s][W/s][d]
 * Element type: all six tensors share `dtype` (HALO_F32 or HALO_BF16).
 * Arithmetic is fp32 (products, sums, softmax) for both dtypes; bf16 results
 * are rounded to nearest even when stored.
 *
 * Memory and ownership: every tensor pointer is a DEVICE pointer allocated
 * by the caller (any allocator; PyTorch tensors are fine).  The library
 * allocates no device memory, keeps no state between calls and never
 * synchronises: work is enqueued on `stream` (a hipStream_t; NULL means the
 * default stream) and the call returns.  `out` must not overlap any input.
 * Device-side faults surface at the caller's next synchronisation.
 *
 * Errors: every argument check runs on the host before any HIP call.  A
 * non-zero status leaves `out` untouched and sets a thread-local message
 * readable with halo_attn_last_error().  A failed launch returns
 * HALO_ERR_HIP.  Nothing is thrown across the ABI.
 */
#ifndef HALO_ATTN_H
#define HALO_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HALO_ATTN_ABI_VERSION 5

typedef enum halo_dtype {
    HALO_F32 = 0,
    HALO_BF16 = 1
} halo_dtype;

/* Which implementation runs.  AUTO picks the fastest one that supports the
 * arguments.  GENERIC is the fp32-vector kernel for every supported shape.
 * MFMA is the fused matrix-core path: bf16, block % 4 == 0, and d in
 * {16, 32} with window side r <= 40 (r <= 32 for the semantic variants) or
 * d == 64 with r <= 32 (default semantics).  Inside it the forward picks,
 * by shape: a persistent kernel of 16-query groups (d in {16, 32} with
 * r <= 16, d == 32 with r <= 20; default semantics); a persistent kernel
 * that walks each image down its block rows with the window rows in an LDS
 * ring (d in {16, 32}, r <= 32, and every semantic variant); a streaming
 * kernel for windows of 33..40 columns and for d == 64; or a kernel that
 * stages each strip of blocks separately (d == 16, or d == 32 with
 * r <= 32).  The backward of d == 64 runs on the generic kernels.
 * MFMA_STRIP forces the last one and MFMA_RING the ring kernel where it
 * applies (for cross-checking; the
 * backward treats both as MFMA).  Asking for a matrix-core path with other
 * arguments returns HALO_ERR_UNSUPPORTED. */
typedef enum halo_kernel {
    HALO_KERNEL_AUTO = 0,
    HALO_KERNEL_GENERIC = 1,
    HALO_KERNEL_MFMA = 2,
    HALO_KERNEL_MFMA_STRIP = 3,
    HALO_KERNEL_MFMA_RING = 4
} halo_kernel;

/* Semantic variants (OR-ed into `flags` of halo_attn_fwd_ex), for matching
 * other readings of the pages.  0 selects the reading documented above.
 *  HALO_CENTRED_OFFSET: table row of displacement D is D + r - 1 (the
 *    table's centre row) instead of D + r - 1 + halo.
 *  HALO_ZERO_PAD: window positions outside the image take part in the
 *    softmax as zero keys and values (section 2.2's "padding at image
 *    borders" read literally) instead of being left out.
 *  HALO_CENTRED_MASK: a query attends only to the keys of its window within
 *    `halo` rows and columns of it: the (2*halo+1)^2 neighbourhood centred
 *    on the query, clipped to the image (SASA; section 2.2 says the blocked
 *    form drops this mask).
 *  HALO_HALF_SPLIT: the height table is applied to channels [0, d/2) of q
 *    and the width table to channels [d/2, d) (appendix A's factorised
 *    embedding, half the channels per axis); the other channels of the
 *    tables are ignored. */
typedef enum halo_flags {
    HALO_CENTRED_OFFSET = 1,
    HALO_ZERO_PAD = 2,
    HALO_CENTRED_MASK = 4,
    HALO_HALF_SPLIT = 8
} halo_flags;

typedef enum halo_status {
    HALO_OK = 0,
    HALO_ERR_NULL = -1,         /* a required pointer is NULL */
    HALO_ERR_SHAPE = -2,        /* sizes inconsistent or out of range */
    HALO_ERR_DTYPE = -3,        /* dtype not HALO_F32 / HALO_BF16 */
    HALO_ERR_UNSUPPORTED = -4,  /* valid, but no kernel handles it */
    HALO_ERR_HIP = -5,          /* the HIP runtime reported an error */
    HALO_ERR_ALIAS = -6,        /* an output overlaps an input or another output */
    HALO_ERR_WORKSPACE = -7     /* workspace too small or misaligned */
} halo_status;

/*
 * Forward pass.  Preconditions (else HALO_ERR_SHAPE):
 *   B, heads, H, W >= 0 (a zero makes the call a no-op returning HALO_OK;
 *   pointers are then not inspected); 1 <= d <= 128; block >= 1;
 *   0 <= halo; r = block + 2*halo <= 256; query_stride >= 1 with
 *   block % query_stride == 0, H % query_stride == 0, W % query_stride == 0;
 *   B*heads*H*W*d < 10^18, H*W < 2^31 (pixel indices inside one image are
 *   32-bit) and the number of blocks B*heads*ceil(H/block)*ceil(W/block)
 *   < 2^31.  scale must be finite (else HALO_ERR_SHAPE); pass
 *   d^-0.5 to follow the HaloAttention module.
 * kernel: a halo_kernel value (else HALO_ERR_SHAPE).
 */
int halo_attn_fwd_kernel(const void* q, const void* k, const void* v,
                         const void* rel_h, const void* rel_w, void* out,
                         int B, int heads, int H, int W, int d,
                         int block, int halo, int query_stride,
                         float scale, int dtype, int kernel, void* stream);

/*
 * halo_attn_fwd_kernel that also writes, per query, the natural log of its
 * softmax normaliser: lse[n][head][y'][x'] = log sum_j exp(l_j) over the
 * query's in-image window keys (fp32, [B][heads][H/s][W/s], caller-owned
 * device memory that must not overlap any other tensor).  lse may be NULL
 * (then this is halo_attn_fwd_kernel).  A training step keeps out and lse
 * for halo_attn_bwd, which then skips recomputing the softmax statistics.
 */
int halo_attn_fwd_lse(const void* q, const void* k, const void* v,
                      const void* rel_h, const void* rel_w, void* out, float* lse,
                      int B, int heads, int H, int W, int d,
                      int block, int halo, int query_stride,
                      float scale, int dtype, int kernel, void* stream);

/*
 * halo_attn_fwd_lse with semantic variants: flags is an OR of halo_flags
 * values (other bits: HALO_ERR_SHAPE).  Variants run on the generic kernel
 * and on the persistent matrix-core kernel; HALO_KERNEL_MFMA_STRIP with
 * flags != 0 returns HALO_ERR_UNSUPPORTED.  halo_attn_bwd_ex is the
 * matching backward.
 */
int halo_attn_fwd_ex(const void* q, const void* k, const void* v,
                     const void* rel_h, const void* rel_w, void* out, float* lse,
                     int B, int heads, int H, int W, int d,
                     int block, int halo, int query_stride,
                     float scale, int dtype, int flags, int kernel, void* stream);

/* halo_attn_fwd_kernel with kernel = HALO_KERNEL_AUTO. */
int halo_attn_fwd(const void* q, const void* k, const void* v,
                  const void* rel_h, const void* rel_w, void* out,
                  int B, int heads, int H, int W, int d,
                  int block, int halo, int query_stride,
                  float scale, int dtype, void* stream);

/*
 * Backward pass: gradients of a scalar loss with respect to q, k, v and both
 * relative tables, given dout = d loss / d out.  The pages print no backward;
 * HaloNet's models are trained by gradient descent (section 4.1), so this is
 * the exact derivative of the forward definition above, with
 * P = softmax(l) over the query's in-image window keys:
 *   dl_j      = P_j (dout . v_j - dout . out)
 *   dq        = scale * sum_j dl_j (k_j + rel_h[row_j] + rel_w[col_j])
 *   dk_j, dv_j = sums over every query whose window holds key j of
 *               scale * dl_j * q and P_j * dout
 *   drel_h[R] = scale * sum of dl_j * q over all (query, key) pairs of all
 *               batches and heads whose row displacement selects row R;
 *               drel_w likewise for columns.
 * out and lse: the forward's output and log normalisers
 * (halo_attn_fwd_lse) for these inputs, or both NULL.  Given, the softmax
 * weights are exp(l - lse) and dout . out comes from out; NULL, both are
 * recomputed from q, k and the tables (an extra pass).
 *
 * Layouts and dtype: q, k, v, rel_h, rel_w as in the forward; dout has out's
 * layout [B][heads][H/s][W/s][d]; dq, dk, dv have q's layout; all of these
 * share `dtype`.  drel_h and drel_w are fp32 [2r-1][d] whatever the dtype
 * (sums over the whole batch).  With query_stride s > 1, dq is zero at the
 * pixels that are not queries.  Table rows no displacement selects get 0.
 * All arithmetic is fp32; bf16 gradients are rounded to nearest even.
 *
 * Workspace: a device buffer of at least halo_attn_bwd_workspace_bytes()
 * bytes, 16-byte aligned, owned by the caller, contents irrelevant on entry
 * and undefined on return (per-query softmax statistics, per-block partial
 * table gradients).  The library allocates nothing.
 *
 * Determinism: no floating-point atomics; every sum runs in a fixed order,
 * so repeated calls give bitwise identical results.
 *
 * Errors as for the forward, plus HALO_ERR_WORKSPACE (workspace too small or
 * misaligned), HALO_ERR_ALIAS when any output or the workspace overlaps an
 * input or another output, and HALO_ERR_NULL when only one of out and lse
 * is given.  drel_h and drel_w must be non-NULL; if a size
 * is zero they are set to zero (the gradient of an empty sum) and no other
 * pointer is inspected.
 *
 * kernel: a halo_kernel value.  GENERIC runs fp32-vector kernels for every
 * supported shape.  MFMA (and MFMA_STRIP, a synonym here) runs the
 * matrix-core backward: bf16, d in {16, 32}, window side r <= 16, block
 * dividing H and W, and (block/query_stride)^2 in {16, 64}; other arguments
 * return HALO_ERR_UNSUPPORTED.  AUTO takes MFMA when it applies.  The
 * matrix-core path keeps, per block column and key row, that column's share
 * of dk and dv in the workspace and sums the shares of every key in a fixed
 * order.
 */
int halo_attn_bwd_kernel(const void* q, const void* k, const void* v,
                         const void* rel_h, const void* rel_w,
                         const void* out, const void* dout, const float* lse,
                         void* dq, void* dk, void* dv, float* drel_h, float* drel_w,
                         void* workspace, size_t workspace_bytes,
                         int B, int heads, int H, int W, int d,
                         int block, int halo, int query_stride,
                         float scale, int dtype, int kernel, void* stream);

/* halo_attn_bwd_kernel for the semantic variants: flags as in
 * halo_attn_fwd_ex (the out and lse passed in must come from the forward
 * with the same flags).  With HALO_HALF_SPLIT the channels a table does not
 * use get a zero gradient. */
int halo_attn_bwd_ex(const void* q, const void* k, const void* v,
                     const void* rel_h, const void* rel_w,
                     const void* out, const void* dout, const float* lse,
                     void* dq, void* dk, void* dv, float* drel_h, float* drel_w,
                     void* workspace, size_t workspace_bytes,
                     int B, int heads, int H, int W, int d,
                     int block, int halo, int query_stride,
                     float scale, int dtype, int flags, int kernel, void* stream);

/* halo_attn_bwd_kernel with kernel = HALO_KERNEL_AUTO. */
int halo_attn_bwd(const void* q, const void* k, const void* v,
                  const void* rel_h, const void* rel_w,
                  const void* out, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, float* drel_h, float* drel_w,
                  void* workspace, size_t workspace_bytes,
                  int B, int heads, int H, int W, int d,
                  int block, int halo, int query_stride,
                  float scale, int dtype, void* stream);

/*
 * halo_attn_bwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight training loops, harnesses that forbid hipMalloc):
 * the same operation, arguments and results as halo_attn_bwd without the
 * workspace arguments.  The workspace is a static array the library holds on
 * every GPU it runs on, halo_attn_noalloc_scratch_bytes() bytes (64 MiB),
 * kept until the process ends; its address is looked up once per device.
 * A call whose workspace (halo_attn_bwd_workspace_bytes) exceeds it returns
 * HALO_ERR_WORKSPACE before any launch (split the batch, or use
 * halo_attn_bwd).  The call allocates nothing and calls no allocating
 * routine.  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (other streams, other host threads) race and
 * must be serialised by the caller.  The array keeps the last call's
 * contents; the backward reads none of it before writing it.
 */
int halo_attn_bwd_noalloc(const void* q, const void* k, const void* v,
                          const void* rel_h, const void* rel_w,
                          const void* out, const void* dout, const float* lse,
                          void* dq, void* dk, void* dv, float* drel_h, float* drel_w,
                          int B, int heads, int H, int W, int d,
                          int block, int halo, int query_stride,
                          float scale, int dtype, void* stream);

/* Bytes of the static workspace halo_attn_bwd_noalloc uses (host-only). */
long long halo_attn_noalloc_scratch_bytes(void);

/* Host-only query: workspace bytes halo_attn_bwd needs for these sizes
 * (0 when a size is zero), or a negative status for invalid arguments. */
long long halo_attn_bwd_workspace_bytes(int B, int heads, int H, int W, int d,
                                        int block, int halo, int query_stride, int dtype);

/*
 * The attention layer around the op: the HaloAttention module on the pswp.cn
 * blog page (section 4).  With inner = heads * d:
 *   q = x W_q^T, [k | v] = x W_kv^T   (to_q, to_kv: no bias; k is the first
 *                                      inner outputs of to_kv, v the rest)
 *   heads split off the channel axis: channel h*d + c is channel c of head h
 *   attn = the blocked attention above (scale, tables, block, halo, stride)
 *   y = merge_heads(attn) W_o^T + b_o (to_out), merged head-major as split.
 * Activations (x, y) stay in a persistent pixel-major layout with channels
 * last (appendix D of the paper keeps the network's activations blocked and
 * avoids formatting operations):
 *   HALO_LAYOUT_NHWC:    [B][H][W][C]
 *   HALO_LAYOUT_BLOCKED: [B][H/s][W/s][s*s][C] with s the block side: pixel
 *                        (i*s + p1, j*s + p2) at [.][i][j][p1*s + p2][.]
 *                        (the blocks flattened row-major).
 * The projections read and write the attention's [B][heads][H][W][d]
 * tensors directly; the head split / merge and the (un)blocking are index
 * arithmetic inside the projection kernels.
 * Weights use the linear-layer layout [out][in]: w_q [inner][C], w_kv
 * [2*inner][C], w_o [C_out][inner], b_o [C_out]; all tensors share `dtype`;
 * accumulation is fp32.  Pointers are device pointers owned by the caller;
 * outputs must not overlap inputs (else HALO_ERR_ALIAS).
 */
typedef enum halo_layout {
    HALO_LAYOUT_NHWC = 0,
    HALO_LAYOUT_BLOCKED = 1
} halo_layout;

/* to_q and to_kv of every pixel of x (layout `layout`, block side `block`
 * for HALO_LAYOUT_BLOCKED) into q, k, v [B][heads][H][W][d].
 * Preconditions: B, H, W, C, heads, d >= 0 (a zero makes the call a no-op);
 * heads*d <= 4096, C <= 65536; for the blocked layout block >= 1 divides H
 * and W.  bf16 with C % 32 == 0, C <= 512, d % 4 == 0 and heads*d % 16 == 0
 * (16-byte aligned pointers) runs on matrix cores, anything else on a plain
 * fp32-accumulating kernel. */
int halo_attn_layer_proj_in(const void* x, const void* w_q, const void* w_kv,
                            void* q, void* k, void* v,
                            int B, int H, int W, int C, int heads, int d,
                            int block, int layout, int dtype, void* stream);

/* Head merge and to_out: attn [B][heads][Ho][Wo][d] -> y [.][C_out] in
 * `layout` (block side `block_out` for HALO_LAYOUT_BLOCKED, which must divide
 * Ho and Wo).  bf16 with heads*d % 32 == 0, heads*d <= 512, d % 8 == 0 and
 * C_out % 16 == 0 (16-byte aligned pointers) runs on matrix cores. */
int halo_attn_layer_proj_out(const void* attn, const void* w_o, const void* b_o, void* y,
                             int B, int Ho, int Wo, int C_out, int heads, int d,
                             int block_out, int layout, int dtype, void* stream);

/* Host-only query: workspace bytes halo_attn_layer_fwd needs (q, k, v and
 * the attention output), 0 when a size is zero, or a negative status. */
long long halo_attn_layer_workspace_bytes(int B, int H, int W, int heads, int d,
                                          int query_stride, int dtype);

/* The whole layer: proj_in, the attention (halo_attn_fwd, kernel AUTO) and
 * proj_out, on `stream`, with q, k, v and the attention output in the
 * caller's workspace (at least halo_attn_layer_workspace_bytes(), 256-byte
 * aligned; contents undefined on return), or the one-kernel fused path
 * where it applies and is the faster (halo_attn_layer_kernel_name tells
 * which; that path uses no workspace and accepts a NULL one; on the shapes
 * measured AUTO takes the split path).  x has
 * B x H x W pixels of C channels, y has B x H/s x W/s pixels of C_out
 * channels (s = query_stride; blocks of side block/s in the blocked
 * layout).  Errors as for the parts, plus HALO_ERR_WORKSPACE. */
int halo_attn_layer_fwd(const void* x, const void* w_q, const void* w_kv,
                        const void* w_o, const void* b_o,
                        const void* rel_h, const void* rel_w, void* y,
                        void* workspace, size_t workspace_bytes,
                        int B, int H, int W, int C, int C_out, int heads, int d,
                        int block, int halo, int query_stride, float scale,
                        int layout, int dtype, void* stream);

/* How halo_attn_layer_fwd_ex computes the layer.  SPLIT: the three steps
 * above, through the workspace.  FUSED: one kernel per image block that
 * stages the block's window of x in LDS and, head by head, projects k and v
 * of the window and q of the block, runs the attention and accumulates
 * to_out in registers, writing y once (HaloNet appendix D: activations stay
 * blocked, no formatting passes; the module of the pswp.cn page, section 4).
 * FUSED takes bf16 with query_stride 1, d in {16, 32}, block in {4, 8}
 * dividing H and W, block + 2*halo <= 16, C % 32 == 0, C_out % 16 == 0,
 * C_out <= 256, a window of x that fits one workgroup's LDS, 16-byte
 * aligned x, w_q, w_kv and 8-byte aligned w_o, b_o, rel_h, rel_w, y.
 * Storage points are the split path's (q, k, v, the probabilities and the
 * attention output rounded to bf16); the softmax uses the exact maximum.
 * It moves about half the split path's HBM bytes but is the slower of the
 * two on the shapes measured, so AUTO takes SPLIT. */
typedef enum halo_layer_kernel {
    HALO_LAYER_KERNEL_AUTO = 0,
    HALO_LAYER_KERNEL_FUSED = 1,
    HALO_LAYER_KERNEL_SPLIT = 2
} halo_layer_kernel;

/* halo_attn_layer_fwd with a halo_layer_kernel value (else HALO_ERR_SHAPE);
 * FUSED with arguments it does not take returns HALO_ERR_UNSUPPORTED.  Only
 * the split path uses (and checks) the workspace: the fused one accepts a
 * NULL workspace. */
int halo_attn_layer_fwd_ex(const void* x, const void* w_q, const void* w_kv,
                           const void* w_o, const void* b_o,
                           const void* rel_h, const void* rel_w, void* y,
                           void* workspace, size_t workspace_bytes,
                           int B, int H, int W, int C, int C_out, int heads, int d,
                           int block, int halo, int query_stride, float scale,
                           int layout, int dtype, int kernel, void* stream);

/* Which path halo_attn_layer_fwd_ex takes for these sizes, with aligned
 * pointers, given a halo_layer_kernel value: "fused", "split", or "none"
 * when a size is zero.  Host only; the string is static.  Invalid arguments,
 * or FUSED where it does not apply: NULL, with halo_attn_last_error()
 * telling why. */
const char* halo_attn_layer_kernel_name(int B, int H, int W, int C, int C_out, int heads, int d,
                                        int block, int halo, int query_stride, int layout, int dtype,
                                        int kernel);

/* Host-only query: the halo_kernel value AUTO would run for these
 * arguments (HALO_KERNEL_GENERIC or HALO_KERNEL_MFMA), or a negative
 * status if the arguments are invalid.  Touches no device. */
int halo_attn_select_kernel(int d, int block, int halo, int query_stride, int dtype);

/*
 * Which forward kernel halo_attn_fwd_ex would run for these arguments:
 * "generic", "tile" (16-query tiles of 4x4 key patches), "ring" (the
 * persistent block-row ring), "wide" (windows wider than 32 columns),
 * "strip", or "none" when a size is zero (nothing to compute).  The
 * arguments mean what they mean there (the scale plays no part).  Queries
 * the current device's compute-unit count and LDS limit, which the
 * matrix-core plans depend on; launches nothing.  The string is static.
 * Invalid arguments: NULL, with halo_attn_last_error() telling why.
 */
const char* halo_attn_fwd_kernel_name(int B, int heads, int H, int W, int d,
                                      int block, int halo, int query_stride,
                                      int dtype, int flags, int kernel);

/*
 * Which backward kernels halo_attn_bwd_ex would run for these arguments
 * with 16-byte-aligned tensors (unaligned ones take the generic kernels):
 * "generic", "strip" (matrix cores, windows of at most 16 columns over
 * whole blocks), "tile" (matrix cores, the 16-query tile kernels), or
 * "none" when a size is zero.  Host only: touches no device.  The string
 * is static.  Invalid arguments: NULL, with halo_attn_last_error() telling
 * why.
 */
const char* halo_attn_bwd_kernel_name(int B, int heads, int H, int W, int d,
                                      int block, int halo, int query_stride,
                                      int dtype, int flags, int kernel);

/* Message for the last non-zero status returned on this thread ("" if none).
 * The pointer stays valid until the next call on this thread. */
const char* halo_attn_last_error(void);

/* HALO_ATTN_ABI_VERSION of the built library. */
int halo_attn_abi_version(void);

/* Identifier of the sources the library was built from: the first 16 hex
 * digits of the SHA-256 over the names and contents of every file in the
 * package's csrc/ directory, in name order ("unknown" when built without it).
 * The Python binding compares it with the sources next to the library and
 * warns when they differ (a library older than its sources).  Static string,
 * owned by the library. */
const char* halo_attn_build_id(void);

/* Measurement aid, not part of the attention path: launches `workgroups`
 * workgroups of 8 waves on `stream`, every lane running independent chains
 * of one instruction kind `iters` times, so a launch's duration gives the
 * rate at which a SIMD issues that kind.  mode: 0 fp32 FMA (8 chains per
 * lane), 1 exp2 (v_exp_f32, 8 chains), 2 bf16 MFMA 16x16x32 (4 accumulators
 * per wave), 3 bf16 MFMA 32x32x16 (4 accumulators), 4 waves 0-3 as mode 1
 * and waves 4-7 as mode 2 (two waves of one SIMD doing different kinds),
 * 5 waves 0-3 as mode 1 and 4-7 as mode 0.  out: device buffer of
 * workgroups * 512 floats, overwritten with values that keep the chains
 * live (meaningless otherwise).  Returns HALO_ERR_SHAPE for a mode outside
 * 0..5 or non-positive counts, HALO_ERR_NULL for a null out, HALO_ERR_HIP
 * when the launch fails; asynchronous otherwise.  bench.py --issue-rates
 * times it. */
int halo_attn_probe_issue(int mode, int iters, int workgroups, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HALO_ATTN_H */
