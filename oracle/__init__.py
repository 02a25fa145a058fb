"""Fp64 CPU oracle for blocked local self-attention with haloing (HaloNet).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only code allowed to import this package.  The GPU
library never imports, links or calls it, and the two share no code.

The arithmetic lives in ``halo_ref.c`` (plain C, fp64), which follows the
per-query definition of HaloNet's blocked local self-attention:
"Scaling Local Self-Attention for Parameter Efficient Visual Backbones",
sections 2.1 (relative dot-product attention, relative embeddings shared by
heads), 2.2 with Figures 1 and 2 (blocking, haloing, padding at the border,
no centred mask, strided queries keep stride-1 neighbourhoods), appendix A
(per-axis factorisation), and the HaloAttention module on the pswp.cn blog
page (scale applied to q before both terms; table row (key - query) + r-1+h;
off-image window positions masked).  The backward (``halo_attn_bwd_ref``) is
the exact derivative of that definition.  This module only marshals numpy
arrays.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB_PATH, build as _build

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        _build()
    lib = ctypes.CDLL(LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.halo_ref_fwd.argtypes = [dp, dp, dp, dp, dp, dp, dp] + [ctypes.c_int] * 8 + [
        ctypes.c_double, ctypes.c_int]
    lib.halo_ref_fwd.restype = ctypes.c_int
    lib.halo_ref_fwd_ex.argtypes = [dp, dp, dp, dp, dp, dp, dp] + [ctypes.c_int] * 8 + [
        ctypes.c_double, ctypes.c_int, ctypes.c_int]
    lib.halo_ref_fwd_ex.restype = ctypes.c_int
    lib.halo_ref_set_attention.argtypes = [
        ctypes.c_int, ctypes.c_int, dp, ctypes.POINTER(dp), dp, ctypes.POINTER(dp),
        ctypes.c_double, dp, dp]
    lib.halo_ref_set_attention.restype = ctypes.c_double
    lib.halo_ref_bwd.argtypes = [dp] * 11 + [ctypes.c_int] * 8 + [ctypes.c_double, ctypes.c_int]
    lib.halo_ref_bwd.restype = ctypes.c_int
    lib.halo_ref_bwd_ex.argtypes = [dp] * 11 + [ctypes.c_int] * 8 + [ctypes.c_double, ctypes.c_int, ctypes.c_int]
    lib.halo_ref_bwd_ex.restype = ctypes.c_int
    lib.halo_ref_set_attention_bwd.argtypes = [
        ctypes.c_int, ctypes.c_int, dp, ctypes.POINTER(dp), dp, ctypes.POINTER(dp),
        ctypes.c_double, dp, dp, ctypes.POINTER(dp), ctypes.POINTER(dp), dp, dp]
    lib.halo_ref_set_attention_bwd.restype = None
    lib.halo_ref_max_threads.argtypes = []
    lib.halo_ref_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    """OpenMP threads the oracle uses by default."""
    return int(_load().halo_ref_max_threads())


# Semantic variants (flags of halo_ref_fwd_ex); see halo_ref.c.
CENTRED_OFFSET, ZERO_PAD, CENTRED_MASK, HALF_SPLIT = 1, 2, 4, 8


def halo_attn_ref(q, k, v, rel_h, rel_w, block: int, halo: int,
                  query_stride: int = 1, scale: float | None = None,
                  threads: int = 0, return_lse: bool = False, flags: int = 0):
    """Forward pass, fp64.

    q, k, v: [B, heads, H, W, d]; rel_h, rel_w: [2*(block+2*halo)-1, d].
    Inputs are converted exactly to float64 (fp32 and bf16 values are exact
    in fp64).  Returns [B, heads, H/s, W/s, d] float64.
    ``scale=None`` means d**-0.5, the value the HaloAttention module uses.
    With ``return_lse`` also returns lse [B, heads, H/s, W/s]: per query,
    log sum_j exp(l_j) over its window keys (the log softmax normaliser).
    ``flags``: OR of CENTRED_OFFSET, ZERO_PAD, CENTRED_MASK, HALF_SPLIT
    (variants of the semantics; 0 = the pages' reading).
    """
    q, k, v, rel_h, rel_w = (_f64(t) for t in (q, k, v, rel_h, rel_w))
    _check(q, k, v, rel_h, rel_w, block, halo, query_stride)
    B, heads, H, W, d = q.shape
    s = query_stride
    if scale is None:
        scale = float(d) ** -0.5
    out = np.zeros((B, heads, H // s, W // s, d), dtype=np.float64)
    lse = np.zeros((B, heads, H // s, W // s), dtype=np.float64) if return_lse else None
    rc = _load().halo_ref_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(rel_h), _ptr(rel_w), _ptr(out),
                                 _ptr(lse) if return_lse else None,
                                 B, heads, H, W, d, block, halo, s, float(scale), int(flags), int(threads))
    if rc != 0:
        raise ValueError(f"halo_ref_fwd failed with status {rc}")
    return (out, lse) if return_lse else out


def _check(q, k, v, rel_h, rel_w, block, halo, query_stride):
    if q.ndim != 5 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"q, k, v must share one 5-D shape, got {q.shape} {k.shape} {v.shape}")
    B, heads, H, W, d = q.shape
    r = block + 2 * halo
    if rel_h.shape != (2 * r - 1, d) or rel_w.shape != (2 * r - 1, d):
        raise ValueError(f"rel tables must be {(2 * r - 1, d)}, got {rel_h.shape} {rel_w.shape}")
    s = query_stride
    if s < 1 or block % s or H % s or W % s:
        raise ValueError("query_stride must divide block, H and W")


def halo_attn_bwd_ref(q, k, v, rel_h, rel_w, dout, block: int, halo: int,
                      query_stride: int = 1, scale: float | None = None,
                      threads: int = 0, flags: int = 0):
    """Backward pass, fp64: gradients of a scalar loss given d loss / d out.

    Same arguments as ``halo_attn_ref`` plus ``dout`` [B, heads, H/s, W/s, d].
    Returns (dq, dk, dv, drel_h, drel_w) as float64 arrays shaped like
    (q, k, v, rel_h, rel_w).  Pixels that are not queries (stride > 1) get a
    zero dq.  The exact derivative of the forward definition (chain rule
    through each query's softmax); see halo_ref.c.  ``flags``: the variants
    of ``halo_attn_ref`` (CENTRED_OFFSET, ZERO_PAD, CENTRED_MASK, HALF_SPLIT).
    """
    q, k, v, rel_h, rel_w, dout = (_f64(t) for t in (q, k, v, rel_h, rel_w, dout))
    _check(q, k, v, rel_h, rel_w, block, halo, query_stride)
    B, heads, H, W, d = q.shape
    s = query_stride
    if dout.shape != (B, heads, H // s, W // s, d):
        raise ValueError(f"dout must be {(B, heads, H // s, W // s, d)}, got {dout.shape}")
    if scale is None:
        scale = float(d) ** -0.5
    dq, dk, dv = (np.zeros(q.shape) for _ in range(3))
    drh, drw = np.zeros(rel_h.shape), np.zeros(rel_w.shape)
    rc = _load().halo_ref_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(rel_h), _ptr(rel_w), _ptr(dout),
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(drh), _ptr(drw),
                                 B, heads, H, W, d, block, halo, s, float(scale), int(flags), int(threads))
    if rc != 0:
        raise ValueError(f"halo_ref_bwd failed with status {rc}")
    return dq, dk, dv, drh, drw


def set_attention_bwd(q, keys, bias, vals, scale: float, g):
    """Gradients of sum(g * set_attention(q, keys, bias, vals, scale)).

    Returns (dq [d], dkeys [n, d], dbias [n], dvals [n, d]); dq covers the
    path through q . keys_j only (bias is an independent input here).
    """
    q, g = _f64(q), _f64(g)
    keys, vals, bias = _f64(keys), _f64(vals), _f64(bias)
    n, d = keys.shape
    if n < 1:
        raise ValueError("need at least one key")
    dp = ctypes.POINTER(ctypes.c_double)
    dkeys, dvals = np.zeros((n, d)), np.zeros((n, d))
    kp = (dp * n)(*[_ptr(keys[j]) for j in range(n)])
    vp = (dp * n)(*[_ptr(vals[j]) for j in range(n)])
    dkp = (dp * n)(*[_ptr(dkeys[j]) for j in range(n)])
    dvp = (dp * n)(*[_ptr(dvals[j]) for j in range(n)])
    dq, dbias = np.zeros(d), np.zeros(n)
    scratch = np.zeros(2 * n)
    _load().halo_ref_set_attention_bwd(d, n, _ptr(q), kp, _ptr(bias), vp, float(scale), _ptr(g),
                                       _ptr(dq), dkp, dvp, _ptr(dbias), _ptr(scratch))
    return dq, dkeys, dbias, dvals


def set_attention(q, keys, bias, vals, scale: float) -> np.ndarray:
    """Softmax attention of one query over an explicit key set.

    q: [d]; keys, vals: [n, d]; bias: [n].  Returns [d]:
    sum_j softmax_j(scale * (q . keys_j + bias_j)) * vals_j.
    """
    q = _f64(q)
    keys, vals, bias = _f64(keys), _f64(vals), _f64(bias)
    n, d = keys.shape
    if n < 1:
        raise ValueError("need at least one key")
    dp = ctypes.POINTER(ctypes.c_double)
    kp = (dp * n)(*[_ptr(keys[j]) for j in range(n)])
    vp = (dp * n)(*[_ptr(vals[j]) for j in range(n)])
    out = np.zeros(d, dtype=np.float64)
    scratch = np.zeros(n, dtype=np.float64)
    _load().halo_ref_set_attention(d, n, _ptr(q), kp, _ptr(bias), vp, float(scale),
                                   _ptr(out), _ptr(scratch))
    return out


# ---------------------------------------------------------------- the layer
# The attention layer around the op: the HaloAttention module on the pswp.cn
# blog page (section 4) projects every pixel with to_q and to_kv (linear maps
# without bias; to_kv's output is k then v), splits the heads, runs the
# blocked attention, merges the heads (head-major: channel h*d + c) and
# applies to_out (a linear map with bias).  Activations stay in one of two
# pixel-major layouts:
#   "nhwc":    [B, H, W, C]
#   "blocked": [B, H/b, W/b, b*b, C], pixel (i*b + p1, j*b + p2) at
#              [., i, j, p1*b + p2, .]: the persistent blocking of appendix D
#              of "Scaling Local Self-Attention for Parameter Efficient Visual
#              Backbones" (blocks flattened row-major, as in the module's
#              rearrange into (p1 p2)).
LAYOUTS = ("nhwc", "blocked")


def to_nhwc(x, layout: str, side: int) -> np.ndarray:
    """Layer activations in `layout` (block side `side`) -> [B, H, W, C]."""
    x = np.asarray(x)
    if layout == "nhwc":
        return x
    if layout != "blocked":
        raise ValueError(f"unknown layout {layout!r}")
    B, nby, nbx, bb, C = x.shape
    if bb != side * side:
        raise ValueError(f"blocked layout needs {side * side} pixels per block, got {bb}")
    return x.reshape(B, nby, nbx, side, side, C).transpose(0, 1, 3, 2, 4, 5).reshape(B, nby * side, nbx * side, C)


def from_nhwc(x, layout: str, side: int) -> np.ndarray:
    """[B, H, W, C] -> layer activations in `layout` (block side `side`)."""
    x = np.asarray(x)
    if layout == "nhwc":
        return x
    if layout != "blocked":
        raise ValueError(f"unknown layout {layout!r}")
    B, H, W, C = x.shape
    if H % side or W % side:
        raise ValueError("the blocked layout needs H and W divisible by the block side")
    return x.reshape(B, H // side, side, W // side, side, C).transpose(0, 1, 3, 2, 4, 5).reshape(
        B, H // side, W // side, side * side, C)


def halo_proj_in_ref(x, w_q, w_kv, heads: int, layout: str = "nhwc", block: int = 1):
    """to_q and to_kv of every pixel, fp64: x (layer layout, C channels),
    w_q [inner, C], w_kv [2*inner, C] -> q, k, v [B, heads, H, W, inner/heads]."""
    xn = _f64(to_nhwc(x, layout, block))
    w_q, w_kv = _f64(w_q), _f64(w_kv)
    B, H, W, C = xn.shape
    inner = w_q.shape[0]
    if w_q.shape != (inner, C) or w_kv.shape != (2 * inner, C) or inner % heads:
        raise ValueError(f"weights {w_q.shape} {w_kv.shape} do not fit C={C}, heads={heads}")
    d = inner // heads

    def split(t):   # [B, H, W, inner] -> [B, heads, H, W, d]
        return np.ascontiguousarray(t.reshape(B, H, W, heads, d).transpose(0, 3, 1, 2, 4))

    kv = xn @ w_kv.T
    return split(xn @ w_q.T), split(kv[..., :inner]), split(kv[..., inner:])


def halo_proj_out_ref(attn, w_o, b_o, layout: str = "nhwc", block: int = 1):
    """Head merge and to_out, fp64: attn [B, heads, Ho, Wo, d], w_o [C, heads*d],
    b_o [C] -> y in the layer layout (block side `block` for "blocked")."""
    attn, w_o, b_o = _f64(attn), _f64(w_o), _f64(b_o)
    B, heads, Ho, Wo, d = attn.shape
    merged = attn.transpose(0, 2, 3, 1, 4).reshape(B, Ho, Wo, heads * d)
    if w_o.shape[1] != heads * d or b_o.shape != (w_o.shape[0],):
        raise ValueError(f"to_out weight {w_o.shape} / bias {b_o.shape} do not fit {heads}x{d} channels")
    return from_nhwc(merged @ w_o.T + b_o, layout, block)


def halo_layer_ref(x, w_q, w_kv, w_o, b_o, rel_h, rel_w, block: int, halo: int, heads: int,
                   query_stride: int = 1, scale: float | None = None, layout: str = "nhwc",
                   threads: int = 0, flags: int = 0) -> np.ndarray:
    """The whole layer, fp64: to_q / to_kv, blocked attention, head merge,
    to_out.  x: [B, H, W, C] ("nhwc") or [B, H/b, W/b, b*b, C] ("blocked");
    returns y in the same layout at the output resolution (blocks of side
    block/query_stride)."""
    q, k, v = halo_proj_in_ref(x, w_q, w_kv, heads, layout, block)
    attn = halo_attn_ref(q, k, v, rel_h, rel_w, block, halo, query_stride, scale, threads, flags=flags)
    return halo_proj_out_ref(attn, w_o, b_o, layout, block // query_stride)
