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
off-image window positions masked).  This module only marshals numpy arrays.
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
    lib.halo_ref_fwd.argtypes = [dp, dp, dp, dp, dp, dp] + [ctypes.c_int] * 8 + [
        ctypes.c_double, ctypes.c_int]
    lib.halo_ref_fwd.restype = ctypes.c_int
    lib.halo_ref_set_attention.argtypes = [
        ctypes.c_int, ctypes.c_int, dp, ctypes.POINTER(dp), dp, ctypes.POINTER(dp),
        ctypes.c_double, dp, dp]
    lib.halo_ref_set_attention.restype = None
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


def halo_attn_ref(q, k, v, rel_h, rel_w, block: int, halo: int,
                  query_stride: int = 1, scale: float | None = None,
                  threads: int = 0) -> np.ndarray:
    """Forward pass, fp64.

    q, k, v: [B, heads, H, W, d]; rel_h, rel_w: [2*(block+2*halo)-1, d].
    Inputs are converted exactly to float64 (fp32 and bf16 values are exact
    in fp64).  Returns [B, heads, H/s, W/s, d] float64.
    ``scale=None`` means d**-0.5, the value the HaloAttention module uses.
    """
    q, k, v, rel_h, rel_w = (_f64(t) for t in (q, k, v, rel_h, rel_w))
    if q.ndim != 5 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"q, k, v must share one 5-D shape, got {q.shape} {k.shape} {v.shape}")
    B, heads, H, W, d = q.shape
    r = block + 2 * halo
    if rel_h.shape != (2 * r - 1, d) or rel_w.shape != (2 * r - 1, d):
        raise ValueError(f"rel tables must be {(2 * r - 1, d)}, got {rel_h.shape} {rel_w.shape}")
    s = query_stride
    if s < 1 or block % s or H % s or W % s:
        raise ValueError("query_stride must divide block, H and W")
    if scale is None:
        scale = float(d) ** -0.5
    out = np.zeros((B, heads, H // s, W // s, d), dtype=np.float64)
    rc = _load().halo_ref_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(rel_h), _ptr(rel_w), _ptr(out),
                              B, heads, H, W, d, block, halo, s, float(scale), int(threads))
    if rc != 0:
        raise ValueError(f"halo_ref_fwd failed with status {rc}")
    return out


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
