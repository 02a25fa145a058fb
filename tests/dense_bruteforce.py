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
