"""Seeded synthetic inputs for halo attention.

This module draws random tensors and nothing else: it holds none of the
attention arithmetic, so both the GPU path and the CPU checker can take their
inputs from it.

Recipe (one CPU ``torch.Generator`` per call, seeded): q, k, v are drawn in that
order as N(0, 1) float32 tensors of shape [B, heads, H, W, d]; then rel_h and
rel_w, each [2r-1, d] with r = block + 2*halo, drawn N(0, 1) and multiplied by
d**-0.5 (the initialisation of the relative tables in the HaloAttention module
on the pswp.cn blog page, section 4).  Every tensor is then rounded to the
workload dtype (round-to-nearest-even for bf16), tables included.

For the backward pass, the gradient of the loss with respect to out is drawn
by ``make_grad_output`` from its own seeded generator: N(0, 1) float32 of the
output's shape, rounded to the workload dtype.
"""
from __future__ import annotations

import torch

_DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    try:
        return _DTYPES[name]
    except KeyError:
        raise ValueError(f"unknown dtype {name!r}; expected one of {sorted(_DTYPES)}") from None


def make_inputs(B: int, heads: int, H: int, W: int, d: int, block: int, halo: int,
                dtype: str = "bf16", seed: int = 0, device: str | torch.device = "cpu"):
    """Return (q, k, v, rel_h, rel_w) drawn as described in the module docstring."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    r = block + 2 * halo
    shape = (B, heads, H, W, d)
    q = torch.randn(shape, dtype=torch.float32, generator=g)
    k = torch.randn(shape, dtype=torch.float32, generator=g)
    v = torch.randn(shape, dtype=torch.float32, generator=g)
    rel_h = torch.randn((2 * r - 1, d), dtype=torch.float32, generator=g) * d ** -0.5
    rel_w = torch.randn((2 * r - 1, d), dtype=torch.float32, generator=g) * d ** -0.5
    dt = torch_dtype(dtype)
    return tuple(t.to(dtype=dt).to(device).contiguous() for t in (q, k, v, rel_h, rel_w))


def make_workload_inputs(wl, seed: int = 0, device: str | torch.device = "cpu"):
    """Inputs for a :class:`blocked_local_self_amd.workloads.Workload`."""
    return make_inputs(wl.B, wl.heads, wl.H, wl.W, wl.d, wl.block, wl.halo,
                       dtype=wl.dtype, seed=seed, device=device)


def make_grad_output(B: int, heads: int, Ho: int, Wo: int, d: int, dtype: str = "bf16",
                     seed: int = 0, device: str | torch.device = "cpu"):
    """d loss / d out, [B, heads, Ho, Wo, d], drawn N(0, 1) and rounded to ``dtype``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 0x5EED)
    t = torch.randn((B, heads, Ho, Wo, d), dtype=torch.float32, generator=g)
    return t.to(dtype=torch_dtype(dtype)).to(device).contiguous()


def make_layer_inputs(B: int, H: int, W: int, C: int, heads: int, d: int, block: int, halo: int,
                      C_out: int | None = None, dtype: str = "bf16", seed: int = 0,
                      device: str | torch.device = "cpu"):
    """Inputs of the attention layer: (x, w_q, w_kv, w_o, b_o, rel_h, rel_w).

    One seeded CPU generator; drawn in that order as N(0, 1) float32: x
    [B, H, W, C] (pixel-major, channels last), w_q [inner, C] and w_kv
    [2*inner, C] times C**-0.5, w_o [C_out, inner] times inner**-0.5, b_o
    [C_out] times 0.1, rel_h and rel_w [2r-1, d] times d**-0.5 (inner =
    heads*d, r = block + 2*halo; C_out defaults to C, as in the module); then
    each is rounded to ``dtype``.  The weight scales keep the projections'
    outputs near unit variance.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 0x1A7E)
    inner = heads * d
    Co = C if C_out is None else C_out
    r = block + 2 * halo
    x = torch.randn((B, H, W, C), dtype=torch.float32, generator=g)
    w_q = torch.randn((inner, C), dtype=torch.float32, generator=g) * C ** -0.5
    w_kv = torch.randn((2 * inner, C), dtype=torch.float32, generator=g) * C ** -0.5
    w_o = torch.randn((Co, inner), dtype=torch.float32, generator=g) * inner ** -0.5
    b_o = torch.randn((Co,), dtype=torch.float32, generator=g) * 0.1
    rel_h = torch.randn((2 * r - 1, d), dtype=torch.float32, generator=g) * d ** -0.5
    rel_w = torch.randn((2 * r - 1, d), dtype=torch.float32, generator=g) * d ** -0.5
    dt = torch_dtype(dtype)
    return tuple(t.to(dtype=dt).to(device).contiguous() for t in (x, w_q, w_kv, w_o, b_o, rel_h, rel_w))


def nhwc_to_layout(x: torch.Tensor, layout: str, side: int) -> torch.Tensor:
    """Seeded [B, H, W, C] activations rearranged into the layer's `layout`:
    "nhwc" (unchanged) or "blocked" ([B, H/s, W/s, s*s, C], blocks flattened
    row-major).  Data arrangement only."""
    if layout == "nhwc":
        return x
    if layout != "blocked":
        raise ValueError(f"unknown layout {layout!r}")
    B, H, W, C = x.shape
    return x.reshape(B, H // side, side, W // side, side, C).permute(0, 1, 3, 2, 4, 5).reshape(
        B, H // side, W // side, side * side, C).contiguous()
