"""MI355X-native blocked local self-attention with haloing (HaloNet forward).

``halo_attn_fwd`` marshals PyTorch tensors into the C ABI of
``libhaloattn.so`` (include/halo_attn.h); every step of the computation runs
in the library's HIP kernels on the tensors' device and on the current HIP
stream.  PyTorch provides device memory and streams only.

The operation ("Scaling Local Self-Attention for Parameter Efficient Visual
Backbones", sections 2.1-2.2, Figures 1-2, appendix A; the HaloAttention
module on the pswp.cn blog page, section 4): for every query pixel, softmax
over the in-image keys of its block's (block+2*halo)^2 window of
scale * (q.k + q.rel_h[dy + c0] + q.rel_w[dx + c0]), c0 = block+3*halo-1,
then the weighted sum of v; queries at multiples of ``query_stride``.
``halo_attn_bwd`` is its exact gradient (recomputing every softmax), and
``halo_attention`` joins the two as a differentiable torch function.
``halo_layer_fwd`` is the whole attention layer of that module (to_q, to_kv,
the attention, to_out) on activations kept in a pixel-major, channels-last
layout (image order or the paper's persistent blocks, appendix D), with the
head split / merge and the (un)blocking done inside the projection kernels.
"""
from __future__ import annotations

from . import _native

__all__ = ["halo_attn_fwd", "halo_attn_bwd", "bwd_workspace_bytes", "halo_attention",
           "halo_layer_proj_in", "halo_layer_proj_out", "halo_layer_fwd", "layer_workspace_bytes",
           "select_kernel", "HaloError", "KERNELS", "VARIANTS", "LAYOUTS", "LAYER_KERNELS"]

HaloError = _native.HaloError
# semantic variants (flags of halo_attn_fwd_ex; see include/halo_attn.h)
VARIANTS = {"centred_offset": _native.HALO_CENTRED_OFFSET, "zero_pad": _native.HALO_ZERO_PAD,
            "centred_mask": _native.HALO_CENTRED_MASK, "half_split": _native.HALO_HALF_SPLIT}
LAYOUTS = {"nhwc": _native.HALO_LAYOUT_NHWC, "blocked": _native.HALO_LAYOUT_BLOCKED}
KERNELS = {"auto": _native.HALO_KERNEL_AUTO, "generic": _native.HALO_KERNEL_GENERIC,
           "mfma": _native.HALO_KERNEL_MFMA, "mfma_strip": _native.HALO_KERNEL_MFMA_STRIP,
           "mfma_ring": _native.HALO_KERNEL_MFMA_RING}


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return _native.HALO_F32
    if t.dtype == torch.bfloat16:
        return _native.HALO_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def select_kernel(d: int, block: int, halo: int, query_stride: int = 1, dtype: str = "bf16") -> str:
    """Name of the kernel ``kernel='auto'`` runs for these arguments (host-only)."""
    code = {"fp32": _native.HALO_F32, "bf16": _native.HALO_BF16}[dtype]
    st = _native.load().halo_attn_select_kernel(d, block, halo, query_stride, code)
    if st < 0:
        _native.check(st)
    return {v: k for k, v in KERNELS.items()}[st]


def _flags(variants) -> int:
    flags = 0
    for name in variants:
        if name not in VARIANTS:
            raise ValueError(f"unknown variant {name!r}; expected some of {sorted(VARIANTS)}")
        flags |= VARIANTS[name]
    return flags


def _check_inputs(q, k, v, rel_h, rel_w, block, halo, query_stride, **extra):
    import torch
    tensors = {"q": q, "k": k, "v": v, "rel_h": rel_h, "rel_w": rel_w, **extra}
    for name, t in tensors.items():
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must live on the GPU (got {t.device})")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q's dtype and device")
    if q.dim() != 5 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"q, k, v must share one [B, heads, H, W, d] shape; got "
                         f"{tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    B, heads, H, W, d = q.shape
    r = block + 2 * halo
    if tuple(rel_h.shape) != (2 * r - 1, d) or tuple(rel_w.shape) != (2 * r - 1, d):
        raise ValueError(f"rel_h and rel_w must be {(2 * r - 1, d)}; got "
                         f"{tuple(rel_h.shape)}, {tuple(rel_w.shape)}")
    s = query_stride
    if s < 1 or H % s or W % s:
        raise ValueError(f"query_stride={s} must divide H={H} and W={W}")
    return B, heads, H, W, d


def halo_attn_fwd(q, k, v, rel_h, rel_w, block: int, halo: int, query_stride: int = 1,
                  scale: float | None = None, out=None, kernel: str = "auto", stream=None,
                  return_lse: bool = False, variants=()):
    """Halo attention forward.

    q, k, v: [B, heads, H, W, d] contiguous CUDA(HIP) tensors, float32 or bfloat16.
    rel_h, rel_w: [2*(block+2*halo)-1, d], same dtype and device.
    Returns out [B, heads, H/s, W/s, d] (allocated unless ``out`` is given).
    ``scale=None`` means d**-0.5.  ``kernel`` in {"auto", "generic", "mfma", "mfma_strip"}.
    ``stream``: a torch.cuda.Stream (default: the current stream).
    ``return_lse``: also return lse [B, heads, H/s, W/s] float32, the natural
    log of each query's softmax normaliser (what ``halo_attn_bwd`` reuses).
    ``variants``: names from VARIANTS (other readings of the pages' semantics).
    """
    import torch
    B, heads, H, W, d = _check_inputs(q, k, v, rel_h, rel_w, block, halo, query_stride)
    s = query_stride
    if scale is None:
        scale = float(d) ** -0.5
    oshape = (B, heads, H // s, W // s, d)
    if out is None:
        out = torch.empty(oshape, dtype=q.dtype, device=q.device)
    elif (tuple(out.shape) != oshape or out.dtype != q.dtype or out.device != q.device
          or not out.is_contiguous()):
        raise ValueError(f"out must be a contiguous {oshape} {q.dtype} tensor on {q.device}")
    if kernel not in KERNELS:
        raise ValueError(f"kernel must be one of {sorted(KERNELS)}")
    flags = _flags(variants)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    lse = torch.empty(oshape[:4], dtype=torch.float32, device=q.device) if return_lse else None
    lib = _native.load()
    with torch.cuda.device(q.device):
        st = lib.halo_attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), rel_h.data_ptr(),
                                  rel_w.data_ptr(), out.data_ptr(), lse.data_ptr() if return_lse else None,
                                  B, heads, H, W, d, block, halo, s, float(scale), _dtype_code(q), flags,
                                  KERNELS[kernel], stream.cuda_stream)
    _native.check(st)
    return (out, lse) if return_lse else out


def bwd_workspace_bytes(B: int, heads: int, H: int, W: int, d: int, block: int, halo: int,
                        query_stride: int = 1, dtype: str = "bf16") -> int:
    """Workspace bytes ``halo_attn_bwd`` needs for these sizes (host-only)."""
    code = {"fp32": _native.HALO_F32, "bf16": _native.HALO_BF16}[dtype]
    n = _native.load().halo_attn_bwd_workspace_bytes(B, heads, H, W, d, block, halo, query_stride, code)
    if n < 0:
        _native.check(int(n))
    return int(n)


def halo_attn_bwd(q, k, v, rel_h, rel_w, dout, block: int, halo: int, query_stride: int = 1,
                  scale: float | None = None, out=None, lse=None, kernel: str = "auto",
                  workspace=None, grads=None, stream=None, variants=()):
    """Halo attention backward: gradients given dout = d loss / d out.

    Same tensors and arguments as ``halo_attn_fwd`` plus ``dout``
    [B, heads, H/s, W/s, d] (same dtype).  Returns (dq, dk, dv, drel_h, drel_w):
    dq, dk, dv in q's dtype and layout, drel_h and drel_w float32 [2r-1, d].
    ``workspace``: optional uint8 CUDA tensor of at least
    ``bwd_workspace_bytes(...)`` bytes (allocated here when None).
    ``out``, ``lse``: the forward's output and log normalisers
    (``halo_attn_fwd(..., return_lse=True)``), or both None to recompute them.
    ``grads``: optional preallocated (dq, dk, dv, drel_h, drel_w) to write into.
    ``variants``: as in ``halo_attn_fwd`` (out and lse must come from a
    forward with the same variants).
    """
    import torch
    B, heads, H, W, d = _check_inputs(q, k, v, rel_h, rel_w, block, halo, query_stride, dout=dout)
    s = query_stride
    oshape = (B, heads, H // s, W // s, d)
    if tuple(dout.shape) != oshape:
        raise ValueError(f"dout must be {oshape}; got {tuple(dout.shape)}")
    if (out is None) != (lse is None):
        raise ValueError("pass both out and lse from the forward, or neither")
    if out is not None:
        if (tuple(out.shape) != oshape or out.dtype != q.dtype or out.device != q.device
                or not out.is_contiguous()):
            raise ValueError(f"out must be a contiguous {oshape} {q.dtype} tensor on {q.device}")
        if (tuple(lse.shape) != oshape[:4] or lse.dtype != torch.float32 or lse.device != q.device
                or not lse.is_contiguous()):
            raise ValueError(f"lse must be a contiguous float32 {oshape[:4]} tensor on {q.device}")
    if scale is None:
        scale = float(d) ** -0.5
    if kernel not in KERNELS:
        raise ValueError(f"kernel must be one of {sorted(KERNELS)}")
    dtype = "bf16" if q.dtype == torch.bfloat16 else "fp32"
    need = bwd_workspace_bytes(B, heads, H, W, d, block, halo, s, dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif (workspace.device != q.device or not workspace.is_contiguous()
          or workspace.numel() * workspace.element_size() < need):
        raise ValueError(f"workspace must be a contiguous tensor of >= {need} bytes on {q.device}")
    r = block + 2 * halo
    if grads is None:
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        drh = torch.empty((2 * r - 1, d), dtype=torch.float32, device=q.device)
        drw = torch.empty_like(drh)
    else:
        dq, dk, dv, drh, drw = grads
        for t, like in ((dq, q), (dk, q), (dv, q)):
            if t.shape != like.shape or t.dtype != like.dtype or t.device != q.device or not t.is_contiguous():
                raise ValueError("dq, dk, dv must be contiguous tensors like q")
        for t in (drh, drw):
            if (tuple(t.shape) != (2 * r - 1, d) or t.dtype != torch.float32 or t.device != q.device
                    or not t.is_contiguous()):
                raise ValueError(f"drel_h, drel_w must be contiguous float32 {(2 * r - 1, d)} tensors")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    lib = _native.load()
    with torch.cuda.device(q.device):
        st = lib.halo_attn_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), rel_h.data_ptr(),
                                  rel_w.data_ptr(), out.data_ptr() if out is not None else None,
                                  dout.data_ptr(), lse.data_ptr() if lse is not None else None,
                                  dq.data_ptr(), dk.data_ptr(),
                                  dv.data_ptr(), drh.data_ptr(), drw.data_ptr(), workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(), B, heads, H, W, d,
                                  block, halo, s, float(scale), _dtype_code(q), _flags(variants),
                                  KERNELS[kernel], stream.cuda_stream)
    _native.check(st)
    return dq, dk, dv, drh, drw


def _make_function():
    import torch

    class HaloAttentionFunction(torch.autograd.Function):
        """out = halo_attn_fwd(...); its backward calls halo_attn_bwd."""

        @staticmethod
        def forward(ctx, q, k, v, rel_h, rel_w, block, halo, query_stride, scale, variants):
            out, lse = halo_attn_fwd(q, k, v, rel_h, rel_w, block, halo, query_stride, scale=scale,
                                     return_lse=True, variants=variants)
            ctx.save_for_backward(q, k, v, rel_h, rel_w, out, lse)
            ctx.cfg = (block, halo, query_stride, scale, variants)
            return out

        @staticmethod
        def backward(ctx, dout):
            q, k, v, rel_h, rel_w, out, lse = ctx.saved_tensors
            block, halo, s, scale, variants = ctx.cfg
            dq, dk, dv, drh, drw = halo_attn_bwd(q, k, v, rel_h, rel_w, dout.contiguous(), block, halo,
                                                 s, scale=scale, out=out, lse=lse, variants=variants)
            return dq, dk, dv, drh.to(rel_h.dtype), drw.to(rel_w.dtype), None, None, None, None, None

    return HaloAttentionFunction


_FUNCTION = None


def halo_attention(q, k, v, rel_h, rel_w, block: int, halo: int, query_stride: int = 1,
                   scale: float | None = None, variants=()):
    """Differentiable halo attention (torch autograd) on the library's kernels.

    ``variants``: semantic variants (names from VARIANTS), forward and backward.
    """
    global _FUNCTION
    if _FUNCTION is None:
        _FUNCTION = _make_function()
    if scale is None:
        scale = float(q.shape[-1]) ** -0.5
    return _FUNCTION.apply(q, k, v, rel_h, rel_w, block, halo, query_stride, scale, tuple(variants))


# ---------------------------------------------------------------- the layer

def _check_device_tensors(ref, **tensors):
    import torch
    for name, t in tensors.items():
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda" or t.device != ref.device:
            raise ValueError(f"{name} must live on {ref.device} (got {t.device})")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != ref.dtype:
            raise ValueError(f"{name} must have dtype {ref.dtype} (got {t.dtype})")


def _layer_pixels(x, layout: str, block: int):
    """(B, H, W, C) of activations x in `layout` (block side `block`)."""
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    if layout == "nhwc":
        if x.dim() != 4:
            raise ValueError(f"nhwc activations are [B, H, W, C]; got {tuple(x.shape)}")
        return tuple(x.shape)
    if x.dim() != 5 or x.shape[3] != block * block:
        raise ValueError(f"blocked activations are [B, H/b, W/b, b*b, C] with b={block}; got {tuple(x.shape)}")
    B, nby, nbx, _, C = x.shape
    return B, nby * block, nbx * block, C


def _layer_shape(B, H, W, C, layout, block):
    if layout == "nhwc":
        return (B, H, W, C)
    return (B, H // block, W // block, block * block, C)


def halo_layer_proj_in(x, w_q, w_kv, heads: int, block: int = 1, layout: str = "nhwc", stream=None):
    """to_q and to_kv of every pixel: x in `layout` ([B, H, W, C], or
    [B, H/b, W/b, b*b, C] with b = ``block``), w_q [inner, C], w_kv
    [2*inner, C] -> q, k, v [B, heads, H, W, inner/heads]."""
    import torch
    _check_device_tensors(x, x=x, w_q=w_q, w_kv=w_kv)
    B, H, W, C = _layer_pixels(x, layout, block)
    inner = w_q.shape[0]
    if w_q.dim() != 2 or tuple(w_q.shape) != (inner, C) or tuple(w_kv.shape) != (2 * inner, C) or inner % heads:
        raise ValueError(f"w_q {tuple(w_q.shape)} / w_kv {tuple(w_kv.shape)} do not fit C={C}, heads={heads}")
    d = inner // heads
    q, k, v = (torch.empty((B, heads, H, W, d), dtype=x.dtype, device=x.device) for _ in range(3))
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    with torch.cuda.device(x.device):
        st = _native.load().halo_attn_layer_proj_in(x.data_ptr(), w_q.data_ptr(), w_kv.data_ptr(), q.data_ptr(),
                                                    k.data_ptr(), v.data_ptr(), B, H, W, C, heads, d, block,
                                                    LAYOUTS[layout], _dtype_code(x), stream.cuda_stream)
    _native.check(st)
    return q, k, v


def halo_layer_proj_out(attn, w_o, b_o, block_out: int = 1, layout: str = "nhwc", stream=None):
    """Head merge and to_out: attn [B, heads, Ho, Wo, d], w_o [C_out, heads*d],
    b_o [C_out] -> y in `layout` (blocks of side ``block_out``)."""
    import torch
    _check_device_tensors(attn, attn=attn, w_o=w_o, b_o=b_o)
    if attn.dim() != 5:
        raise ValueError(f"attn must be [B, heads, Ho, Wo, d]; got {tuple(attn.shape)}")
    B, heads, Ho, Wo, d = attn.shape
    Co = w_o.shape[0]
    if w_o.dim() != 2 or w_o.shape[1] != heads * d or tuple(b_o.shape) != (Co,):
        raise ValueError(f"w_o {tuple(w_o.shape)} / b_o {tuple(b_o.shape)} do not fit {heads}x{d} channels")
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    y = torch.empty(_layer_shape(B, Ho, Wo, Co, layout, block_out), dtype=attn.dtype, device=attn.device)
    if stream is None:
        stream = torch.cuda.current_stream(attn.device)
    with torch.cuda.device(attn.device):
        st = _native.load().halo_attn_layer_proj_out(attn.data_ptr(), w_o.data_ptr(), b_o.data_ptr(), y.data_ptr(),
                                                     B, Ho, Wo, Co, heads, d, block_out, LAYOUTS[layout],
                                                     _dtype_code(attn), stream.cuda_stream)
    _native.check(st)
    return y


def layer_workspace_bytes(B: int, H: int, W: int, heads: int, d: int, query_stride: int = 1,
                          dtype: str = "bf16") -> int:
    """Workspace bytes ``halo_layer_fwd`` needs (host-only query)."""
    code = {"fp32": _native.HALO_F32, "bf16": _native.HALO_BF16}[dtype]
    n = _native.load().halo_attn_layer_workspace_bytes(B, H, W, heads, d, query_stride, code)
    if n < 0:
        _native.check(int(n))
    return int(n)


LAYER_KERNELS = {"auto": _native.HALO_LAYER_KERNEL_AUTO, "fused": _native.HALO_LAYER_KERNEL_FUSED,
                 "split": _native.HALO_LAYER_KERNEL_SPLIT}


def halo_layer_fwd(x, w_q, w_kv, w_o, b_o, rel_h, rel_w, block: int, halo: int, heads: int,
                   query_stride: int = 1, scale: float | None = None, layout: str = "nhwc",
                   workspace=None, out=None, stream=None, kernel: str = "auto"):
    """The attention layer: to_q / to_kv, halo attention, head merge, to_out.

    x: [B, H, W, C] ("nhwc") or [B, H/b, W/b, b*b, C] ("blocked", b = block);
    w_q [inner, C], w_kv [2*inner, C], w_o [C_out, inner], b_o [C_out];
    rel_h, rel_w [2*(block+2*halo)-1, inner/heads]; all one dtype on one GPU.
    Returns y in the same layout at the output resolution (H/s x W/s pixels,
    blocks of side block/s).  ``workspace``: an optional uint8 device tensor
    of at least ``layer_workspace_bytes`` bytes (allocated if None).
    ``kernel``: "auto", "fused" (one kernel, nothing between the steps in
    HBM) or "split" (projections and attention as three kernels).
    """
    import torch
    if kernel not in LAYER_KERNELS:
        raise ValueError(f"kernel must be one of {sorted(LAYER_KERNELS)}, got {kernel!r}")
    _check_device_tensors(x, x=x, w_q=w_q, w_kv=w_kv, w_o=w_o, b_o=b_o, rel_h=rel_h, rel_w=rel_w)
    B, H, W, C = _layer_pixels(x, layout, block)
    inner = w_q.shape[0]
    if tuple(w_q.shape) != (inner, C) or tuple(w_kv.shape) != (2 * inner, C) or inner % heads:
        raise ValueError(f"w_q {tuple(w_q.shape)} / w_kv {tuple(w_kv.shape)} do not fit C={C}, heads={heads}")
    d = inner // heads
    Co = w_o.shape[0]
    if w_o.dim() != 2 or w_o.shape[1] != inner or tuple(b_o.shape) != (Co,):
        raise ValueError(f"w_o {tuple(w_o.shape)} / b_o {tuple(b_o.shape)} do not fit inner={inner}")
    s = query_stride
    if s < 1 or block % s or H % s or W % s:
        raise ValueError(f"query_stride={s} must divide block, H and W")
    if scale is None:
        scale = float(d) ** -0.5
    oshape = _layer_shape(B, H // s, W // s, Co, layout, block // s)
    if out is None:
        out = torch.empty(oshape, dtype=x.dtype, device=x.device)
    elif tuple(out.shape) != oshape or out.dtype != x.dtype or out.device != x.device or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {oshape} {x.dtype} tensor on {x.device}")
    dname = "bf16" if x.dtype == torch.bfloat16 else "fp32"
    if workspace is None:
        # the fused path takes none (it needs 16-byte aligned x and weights,
        # 8-byte aligned tables, bias and output, which torch's allocations are)
        aligned = all(t.data_ptr() % 16 == 0 for t in (x, w_q, w_kv)) and \
            all(t.data_ptr() % 8 == 0 for t in (w_o, b_o, rel_h, rel_w, out))
        fused = kernel == "fused" or (kernel == "auto" and aligned and _native.layer_kernel_name(
            B, H, W, C, Co, heads, d, block, halo, s, LAYOUTS[layout], _dtype_code(x)) == "fused")
        if not fused:
            workspace = torch.empty(max(layer_workspace_bytes(B, H, W, heads, d, s, dname), 1), dtype=torch.uint8,
                                    device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with torch.cuda.device(x.device):
        st = _native.load().halo_attn_layer_fwd_ex(
            x.data_ptr(), w_q.data_ptr(), w_kv.data_ptr(), w_o.data_ptr(), b_o.data_ptr(), rel_h.data_ptr(),
            rel_w.data_ptr(), out.data_ptr(), ws_ptr, ws_bytes,
            B, H, W, C, Co, heads, d, block, halo, s, float(scale), LAYOUTS[layout], _dtype_code(x),
            LAYER_KERNELS[kernel], stream.cuda_stream)
    _native.check(st)
    return out
