"""Dense NumPy float64 formulation of halo attention, used to pin the oracle.

It takes a different route from the oracle's per-query loops: every query
attends to *all* H*W pixels of its (batch, head) slice through an additive
mask matrix (0 where the key lies in the query's block window and inside the
image, -inf elsewhere) plus a bias matrix gathered from the full relative
logits q . rel_h^T and q . rel_w^T.  Written from the definition in
"Scaling Local Self-Attention for Parameter Efficient Visual Backbones",
sections 2.1-2.2 (Figures 1 and 2), with the table row (key - query) + r-1+h
that the HaloAttention module on the pswp.cn page uses.  Tiny shapes only.
"""
from __future__ import annotations

import numpy as np


def window_mask_and_index(H: int, W: int, block: int, halo: int, stride: int):
    """For query positions (s*y', s*x') and all keys: membership mask and
    displacement+offset row indices along each axis."""
    r = block + 2 * halo
    c0 = r - 1 + halo
    ys = np.arange(0, H, stride)
    xs = np.arange(0, W, stride)
    qy, qx = np.meshgrid(ys, xs, indexing="ij")
    qy, qx = qy.reshape(-1), qx.reshape(-1)
    ky, kx = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    ky, kx = ky.reshape(-1), kx.reshape(-1)
    by0 = (qy // block) * block - halo          # window origin, per query
    bx0 = (qx // block) * block - halo
    in_y = (ky[None, :] >= by0[:, None]) & (ky[None, :] < by0[:, None] + r)
    in_x = (kx[None, :] >= bx0[:, None]) & (kx[None, :] < bx0[:, None] + r)
    member = in_y & in_x                        # keys are in-image by construction
    row_h = ky[None, :] - qy[:, None] + c0
    row_w = kx[None, :] - qx[:, None] + c0
    return member, row_h, row_w, qy, qx


def halo_attn_dense(q, k, v, rel_h, rel_w, block, halo, stride=1, scale=None):
    q, k, v, rel_h, rel_w = (np.asarray(t, dtype=np.float64) for t in (q, k, v, rel_h, rel_w))
    B, heads, H, W, d = q.shape
    if scale is None:
        scale = d ** -0.5
    member, row_h, row_w, qy, qx = window_mask_and_index(H, W, block, halo, stride)
    nrows = rel_h.shape[0]
    safe_h = np.clip(row_h, 0, nrows - 1)
    safe_w = np.clip(row_w, 0, nrows - 1)
    out = np.zeros((B, heads, H // stride, W // stride, d))
    for n in range(B):
        for hd in range(heads):
            Qs = q[n, hd][qy, qx]                       # [P, d]
            Ks = k[n, hd].reshape(-1, d)                # [H*W, d]
            Vs = v[n, hd].reshape(-1, d)
            rel_logits_h = Qs @ rel_h.T                 # [P, 2r-1]
            rel_logits_w = Qs @ rel_w.T
            P = Qs.shape[0]
            pidx = np.arange(P)[:, None]
            bias = rel_logits_h[pidx, safe_h] + rel_logits_w[pidx, safe_w]
            logits = scale * (Qs @ Ks.T + bias)
            logits = np.where(member, logits, -np.inf)
            logits = logits - logits.max(axis=1, keepdims=True)
            w = np.exp(logits)
            w = w / w.sum(axis=1, keepdims=True)
            out[n, hd] = (w @ Vs).reshape(H // stride, W // stride, d)
    return out


def halo_attn_dense_torch(q, k, v, rel_h, rel_w, block, halo, stride=1, scale=None):
    """The same dense formulation in torch float64, differentiable.

    Used to pin the oracle's backward against torch autograd: the gradient
    comes from autograd through this dense route, not from any hand-written
    derivative.
    """
    import torch
    B, heads, H, W, d = q.shape
    if scale is None:
        scale = d ** -0.5
    member, row_h, row_w, qy, qx = window_mask_and_index(H, W, block, halo, stride)
    nrows = rel_h.shape[0]
    member = torch.as_tensor(member)
    safe_h = torch.as_tensor(np.clip(row_h, 0, nrows - 1))
    safe_w = torch.as_tensor(np.clip(row_w, 0, nrows - 1))
    qy, qx = torch.as_tensor(qy), torch.as_tensor(qx)
    outs = []
    for n in range(B):
        per_head = []
        for hd in range(heads):
            Qs = q[n, hd][qy, qx]
            Ks = k[n, hd].reshape(-1, d)
            Vs = v[n, hd].reshape(-1, d)
            lh = Qs @ rel_h.T
            lw = Qs @ rel_w.T
            bias = torch.gather(lh, 1, safe_h) + torch.gather(lw, 1, safe_w)
            logits = scale * (Qs @ Ks.T + bias)
            logits = logits.masked_fill(~member, float("-inf"))
            w = torch.softmax(logits, dim=1)
            per_head.append((w @ Vs).reshape(H // stride, W // stride, d))
        outs.append(torch.stack(per_head))
    return torch.stack(outs)


def halo_lse_dense(q, k, rel_h, rel_w, block, halo, stride=1, scale=None):
    """Per-query log softmax normaliser, dense formulation (float64)."""
    q, k, rel_h, rel_w = (np.asarray(t, dtype=np.float64) for t in (q, k, rel_h, rel_w))
    B, heads, H, W, d = q.shape
    if scale is None:
        scale = d ** -0.5
    member, row_h, row_w, qy, qx = window_mask_and_index(H, W, block, halo, stride)
    nrows = rel_h.shape[0]
    safe_h = np.clip(row_h, 0, nrows - 1)
    safe_w = np.clip(row_w, 0, nrows - 1)
    out = np.zeros((B, heads, H // stride, W // stride))
    for n in range(B):
        for hd in range(heads):
            Qs = q[n, hd][qy, qx]
            Ks = k[n, hd].reshape(-1, d)
            pidx = np.arange(Qs.shape[0])[:, None]
            bias = (Qs @ rel_h.T)[pidx, safe_h] + (Qs @ rel_w.T)[pidx, safe_w]
            logits = np.where(member, scale * (Qs @ Ks.T + bias), -np.inf)
            m = logits.max(axis=1, keepdims=True)
            lse = m[:, 0] + np.log(np.exp(logits - m).sum(axis=1))
            out[n, hd] = lse.reshape(H // stride, W // stride)
    return out


def halo_layer_module_torch(x, w_q, w_kv, w_o, b_o, rel_h, rel_w, block, halo, heads, scale=None):
    """The HaloAttention layer computed the way the module on the pswp.cn page
    (section 4) orders its steps, in torch float64 on the CPU:
      x [N, C, H, W] is cut into blocks of b*b query pixels; the key/value
      inputs are the (b+2h)^2 windows extracted by a zero-padded unfold; both
      go through the projections (so k, v are projected per window position,
      padded positions included, instead of once per pixel); heads are split;
      logits = (scale q) . k + relative terms; padded window positions are
      masked; softmax; weighted sum of v; heads merged; to_out with its bias;
      blocks put back into [N, C, H, W].
    The relative term of block-local query (y, x) and window position (ty, tx)
    is q . rel_h[ty - y + r - 1] + q . rel_w[tx - x + r - 1] with ty, tx
    counted from the window corner (the same row as (key - query) + r-1+h).
    Stride 1 only, as in the module."""
    import torch
    import torch.nn.functional as F
    t = lambda a: torch.as_tensor(np.asarray(a, dtype=np.float64))
    x, w_q, w_kv, w_o, b_o, rel_h, rel_w = (t(a) for a in (x, w_q, w_kv, w_o, b_o, rel_h, rel_w))
    N, C, H, W = x.shape
    b, r = block, block + 2 * halo
    nby, nbx = H // b, W // b
    inner = w_q.shape[0]
    d = inner // heads
    if scale is None:
        scale = d ** -0.5
    # queries: [N*nby*nbx, b*b, C], block-local pixel p1*b + p2
    q_in = x.reshape(N, C, nby, b, nbx, b).permute(0, 2, 4, 3, 5, 1).reshape(N * nby * nbx, b * b, C)
    # key/value inputs: the zero-padded windows, [N*nblocks, r*r, C]
    win = F.unfold(x, kernel_size=r, stride=b, padding=halo)             # [N, C*r*r, nblocks]
    kv_in = win.reshape(N, C, r * r, nby * nbx).permute(0, 3, 2, 1).reshape(N * nby * nbx, r * r, C)
    inside = F.unfold(torch.ones(1, 1, H, W, dtype=torch.float64), kernel_size=r, stride=b, padding=halo)
    inside = inside.reshape(r * r, nby * nbx).T.repeat(N, 1)             # [N*nblocks, r*r], 1 = in the image
    q = q_in @ w_q.T
    kv = kv_in @ w_kv.T
    k, v = kv[..., :inner], kv[..., inner:]
    heads_first = lambda a: a.reshape(a.shape[0], a.shape[1], heads, d).permute(0, 2, 1, 3)
    q, k, v = heads_first(q) * scale, heads_first(k), heads_first(v)      # [nb, heads, n, d]
    qy = torch.arange(b).repeat_interleave(b)                            # query rows / columns in the block
    qx = torch.arange(b).repeat(b)
    ty = torch.arange(r).repeat_interleave(r)                            # window rows / columns
    tx = torch.arange(r).repeat(r)
    rows_h = ty[None, :] - qy[:, None] + r - 1                           # [b*b, r*r]
    rows_w = tx[None, :] - qx[:, None] + r - 1
    lh = q @ rel_h.T                                                     # [nb, heads, b*b, 2r-1]
    lw = q @ rel_w.T
    rel = (torch.gather(lh, 3, rows_h.expand(lh.shape[0], heads, -1, -1)) +
           torch.gather(lw, 3, rows_w.expand(lw.shape[0], heads, -1, -1)))
    sim = q @ k.transpose(-1, -2) + rel
    sim = sim.masked_fill(inside[:, None, None, :] == 0, float("-inf"))
    out = torch.softmax(sim, dim=-1) @ v                                 # [nb, heads, b*b, d]
    out = out.permute(0, 2, 1, 3).reshape(out.shape[0], b * b, inner)
    y = out @ w_o.T + b_o                                                # [nb, b*b, C_out]
    Co = y.shape[-1]
    y = y.reshape(N, nby, nbx, b, b, Co).permute(0, 5, 1, 3, 2, 4).reshape(N, Co, H, W)
    return y.numpy()
