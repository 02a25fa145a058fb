"""GPU parity of the attention layer (to_q / to_kv, the blocked attention,
head merge, to_out; the HaloAttention module on the pswp.cn page, section 4)
through the C ABI, against the fp64 oracle (oracle.halo_proj_in_ref,
halo_proj_out_ref, halo_layer_ref) on the same seeded, rounded inputs.

Tolerances, from the arithmetic:
  projections: fp32 accumulation of exact products, one rounding of the
    result to the output dtype: |gpu - ref| <= 2^-8 |ref| + 1e-6 max|ref|
    for bf16 (round to nearest: 2^-9 relative, doubled), 1e-5 relative for
    fp32;
  the whole layer in bf16: q, k, v and the attention output are stored in
    bf16 between the kernels, so the result is compared with the oracle run
    on those same rounding points (project in fp64, round to bf16, attention
    in fp64, round, project): max error <= 2e-2 max|ref| (the attention
    kernel's own bf16 bound); against the unrounded fp64 layer the bound is
    5e-2 max|ref|.  fp32: 1e-4 max|ref|.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from blocked_local_self_amd import (halo_layer_proj_in, halo_layer_proj_out, halo_layer_fwd, halo_attn_fwd,
                                    HaloError, _native)
from blocked_local_self_amd.inputs import make_layer_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rnd(a, dtype):
    """fp64 array rounded to `dtype` the way the kernels store it (RNE)."""
    t = torch.as_tensor(a)
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32).to(torch.float64).numpy()


def check_proj(gpu, want, dtype):
    g = f64(gpu)
    assert np.isfinite(g).all()
    m = float(np.abs(want).max())
    if dtype == "bf16":
        bound = 2.0 ** -8 * np.abs(want) + 1e-6 * m
    else:
        bound = 1e-5 * np.abs(want) + 1e-6 * m
    bad = np.abs(g - want) > bound
    assert not bad.any(), f"{int(bad.sum())} elements off; worst {float(np.abs(g - want).max()):.3g} (max|ref| {m:.3g})"


# (B, H, W, C, heads, d, block, layout): ragged pixel counts (not multiples
# of 32 or 256), both layouts, C from one to several MFMA k-steps, inner
# spanning several 16-row output tiles and slices
PROJ_CASES = [
    (1, 6, 6, 64, 2, 16, 3, "nhwc"),
    (2, 8, 12, 32, 4, 16, 4, "blocked"),
    (1, 16, 16, 128, 8, 16, 8, "nhwc"),
    (3, 8, 8, 96, 2, 32, 8, "blocked"),
    (1, 10, 10, 256, 8, 32, 5, "nhwc"),
    (1, 4, 4, 512, 4, 32, 2, "blocked"),
    (1, 5, 7, 24, 3, 4, 1, "nhwc"),          # not matrix-core shapes: plain kernel
]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("case", PROJ_CASES, ids=lambda c: "x".join(map(str, c)))
def test_proj_in_matches_oracle(case, dtype):
    B, H, W, C, heads, d, block, layout = case
    say("proj_in", case, dtype)
    x, w_q, w_kv, *_ = make_layer_inputs(B, H, W, C, heads, d, block, 1, dtype=dtype, seed=3)
    xl = torch.as_tensor(oracle.from_nhwc(x.float().numpy(), layout, block)).to(x.dtype)
    q, k, v = halo_layer_proj_in(xl.to(DEV).contiguous(), w_q.to(DEV), w_kv.to(DEV), heads, block, layout)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.halo_proj_in_ref(f64(xl), f64(w_q), f64(w_kv), heads, layout, block)
    for got, want in ((q, rq), (k, rk), (v, rv)):
        check_proj(got, want, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("case", PROJ_CASES, ids=lambda c: "x".join(map(str, c)))
def test_proj_out_matches_oracle(case, dtype):
    B, H, W, C, heads, d, block, layout = case
    say("proj_out", case, dtype)
    g = torch.Generator().manual_seed(5)
    attn = torch.randn((B, heads, H, W, d), generator=g).to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    _, _, _, w_o, b_o, _, _ = make_layer_inputs(B, H, W, C, heads, d, block, 1, C_out=C, dtype=dtype, seed=4)
    y = halo_layer_proj_out(attn.to(DEV), w_o.to(DEV), b_o.to(DEV), block, layout)
    torch.cuda.synchronize()
    want = oracle.halo_proj_out_ref(f64(attn), f64(w_o), f64(b_o), layout, block)
    assert tuple(y.shape) == want.shape
    check_proj(y, want, dtype)


def layer_ref_rounded(x, w_q, w_kv, w_o, b_o, rh, rw, block, halo, heads, stride, layout):
    """The oracle with the bf16 storage points of the GPU layer."""
    q, k, v = (rnd(t, "bf16") for t in oracle.halo_proj_in_ref(x, w_q, w_kv, heads, layout, block))
    attn = rnd(oracle.halo_attn_ref(q, k, v, rh, rw, block, halo, stride), "bf16")
    return oracle.halo_proj_out_ref(attn, w_o, b_o, layout, block // stride)


# (B, H, W, C, C_out, heads, d, block, halo, stride, layout)
LAYER_CASES = [
    (2, 16, 16, 64, 64, 4, 16, 8, 3, 1, "nhwc"),
    (1, 24, 16, 128, 128, 8, 16, 8, 2, 1, "blocked"),
    (2, 16, 16, 64, 32, 2, 32, 8, 3, 2, "nhwc"),
    (1, 16, 16, 64, 64, 2, 32, 8, 3, 2, "blocked"),
    (1, 12, 12, 48, 40, 3, 16, 4, 1, 1, "nhwc"),     # plain projections (C_out % 16 != 0, C % 32 != 0)
    (1, 16, 16, 128, 64, 2, 64, 8, 3, 1, "nhwc"),    # 64-channel heads (streaming attention kernel)
]


# (B, H, W, C, C_out, heads, d, block, halo, stride, layout) the fused
# kernel takes: both head widths, blocks of 4 and 8 (one query tile, four),
# windows from 6 to 16 pixels a side (3 to 16 key tiles, padded key tiles
# masked), halo 0, C != heads*d, C_out from one to sixteen 16-channel tiles,
# both layouts, non-square images and several images
FUSED_CASES = [
    (1, 8, 8, 32, 16, 2, 16, 4, 1, 1, "nhwc"),
    (2, 16, 24, 64, 48, 4, 16, 8, 3, 1, "blocked"),
    (1, 16, 16, 96, 64, 3, 32, 8, 4, 1, "nhwc"),
    (1, 12, 8, 64, 128, 4, 32, 4, 6, 1, "nhwc"),
    (2, 16, 16, 192, 128, 8, 16, 8, 2, 1, "blocked"),
    (1, 8, 8, 64, 64, 2, 32, 8, 0, 1, "nhwc"),
]


def run_layer_case(case, dtype, kernel):
    B, H, W, C, Co, heads, d, block, halo, stride, layout = case
    x, w_q, w_kv, w_o, b_o, rh, rw = make_layer_inputs(B, H, W, C, heads, d, block, halo, C_out=Co, dtype=dtype,
                                                       seed=11)
    xl = torch.as_tensor(oracle.from_nhwc(x.float().numpy(), layout, block)).to(x.dtype)
    args = [t.to(DEV).contiguous() for t in (xl, w_q, w_kv, w_o, b_o, rh, rw)]
    y = halo_layer_fwd(*args, block, halo, heads, stride, layout=layout, kernel=kernel)
    torch.cuda.synchronize()
    return y, [f64(t) for t in (xl, w_q, w_kv, w_o, b_o, rh, rw)]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "x".join(map(str, c)))
def test_fused_layer_matches_oracle(case):
    """The one-kernel layer against the oracle with the same bf16 storage
    points, and against the three-kernel path."""
    B, H, W, C, Co, heads, d, block, halo, stride, layout = case
    say("fused layer", case)
    assert _native.layer_kernel_name(B, H, W, C, Co, heads, d, block, halo, stride,
                                     1 if layout == "blocked" else 0, _native.HALO_BF16,
                                     kernel=_native.HALO_LAYER_KERNEL_FUSED) == "fused"
    y, ref_in = run_layer_case(case, "bf16", "fused")
    exact = oracle.halo_layer_ref(*ref_in, block, halo, heads, stride, layout=layout)
    rounded = layer_ref_rounded(*ref_in, block, halo, heads, stride, layout)
    assert tuple(y.shape) == exact.shape
    g = f64(y)
    assert np.isfinite(g).all()
    m = float(np.abs(exact).max())
    e1, e2 = float(np.abs(g - rounded).max()), float(np.abs(g - exact).max())
    say(f"  err vs rounded oracle {e1 / m:.3g}, vs fp64 layer {e2 / m:.3g} (of max|ref| {m:.3g})")
    assert e1 <= 2e-2 * m and e2 <= 5e-2 * m
    y2, _ = run_layer_case(case, "bf16", "split")
    e3 = float((y.float() - y2.float()).abs().max())
    say(f"  fused vs split {e3 / m:.3g}")
    assert e3 <= 2e-2 * m


def test_fused_layer_refuses_what_it_does_not_take():
    x, w_q, w_kv, w_o, b_o, rh, rw = (t.to(DEV) for t in make_layer_inputs(1, 16, 16, 64, 2, 16, 8, 2, seed=1))
    with pytest.raises(HaloError):
        halo_layer_fwd(x, w_q, w_kv, w_o, b_o, rh, rw, 8, 2, 2, 2, kernel="fused")     # query stride 2
    y = halo_layer_fwd(x, w_q, w_kv, w_o, b_o, rh, rw, 8, 2, 2, 2)                     # auto: the split path
    torch.cuda.synchronize()
    assert np.isfinite(f64(y)).all()


@pytest.mark.parametrize("kernel", ["auto", "fused"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("case", LAYER_CASES, ids=lambda c: "x".join(map(str, c)))
def test_layer_matches_oracle(case, dtype, kernel):
    B, H, W, C, Co, heads, d, block, halo, stride, layout = case
    if kernel == "fused" and (dtype == "fp32" or stride != 1 or C % 32 or d not in (16, 32)):
        pytest.skip("a shape the fused kernel does not take (the split path covers it)")
    say("layer", case, dtype, kernel)
    x, w_q, w_kv, w_o, b_o, rh, rw = make_layer_inputs(B, H, W, C, heads, d, block, halo, C_out=Co, dtype=dtype,
                                                       seed=11)
    xl = torch.as_tensor(oracle.from_nhwc(x.float().numpy(), layout, block)).to(x.dtype)
    args = [t.to(DEV).contiguous() for t in (xl, w_q, w_kv, w_o, b_o, rh, rw)]
    y = halo_layer_fwd(*args, block, halo, heads, stride, layout=layout, kernel=kernel)
    torch.cuda.synchronize()
    ref_in = [f64(t) for t in (xl, w_q, w_kv, w_o, b_o, rh, rw)]
    exact = oracle.halo_layer_ref(*ref_in, block, halo, heads, stride, layout=layout)
    assert tuple(y.shape) == exact.shape
    g = f64(y)
    assert np.isfinite(g).all()
    m = float(np.abs(exact).max())
    if dtype == "fp32":
        assert float(np.abs(g - exact).max()) <= 1e-4 * m
    else:
        rounded = layer_ref_rounded(*ref_in, block, halo, heads, stride, layout)
        e1, e2 = float(np.abs(g - rounded).max()), float(np.abs(g - exact).max())
        say(f"  err vs rounded oracle {e1 / m:.3g}, vs fp64 layer {e2 / m:.3g} (of max|ref| {m:.3g})")
        assert e1 <= 2e-2 * m and e2 <= 5e-2 * m


def test_layer_equals_its_parts():
    """The split path of halo_layer_fwd is proj_in, the attention and
    proj_out in sequence: bitwise the same as calling the three entry points."""
    B, H, W, C, heads, d, block, halo = 2, 16, 16, 64, 4, 16, 8, 3
    x, w_q, w_kv, w_o, b_o, rh, rw = (t.to(DEV) for t in make_layer_inputs(B, H, W, C, heads, d, block, halo, seed=2))
    y = halo_layer_fwd(x, w_q, w_kv, w_o, b_o, rh, rw, block, halo, heads, kernel="split")
    q, k, v = halo_layer_proj_in(x, w_q, w_kv, heads)
    attn = halo_attn_fwd(q, k, v, rh, rw, block, halo)
    y2 = halo_layer_proj_out(attn, w_o, b_o)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


def test_layer_full_size_sampled_images():
    """The bench's layer shape (32 images of 64x64, 128 channels, 8 heads of
    16, block 8, halo 3): two whole images against the oracle (images are
    independent, so the oracle runs on them alone)."""
    B, H, W, C, heads, d, block, halo = 32, 64, 64, 128, 8, 16, 8, 3
    x, w_q, w_kv, w_o, b_o, rh, rw = make_layer_inputs(B, H, W, C, heads, d, block, halo, seed=0)
    args = [t.to(DEV) for t in (x, w_q, w_kv, w_o, b_o, rh, rw)]
    say("layer full size", _native.layer_kernel_name(B, H, W, C, C, heads, d, block, halo, 1, 0, _native.HALO_BF16))
    y = halo_layer_fwd(*args, block, halo, heads)
    torch.cuda.synchronize()
    for b in (0, B - 1):
        ref_in = [f64(x[b:b + 1])] + [f64(t) for t in (w_q, w_kv, w_o, b_o, rh, rw)]
        rounded = layer_ref_rounded(*ref_in, block, halo, heads, 1, "nhwc")
        g = f64(y[b:b + 1])
        m = float(np.abs(rounded).max())
        err = float(np.abs(g - rounded).max())
        say(f"  image {b}: err {err / m:.3g} of max|ref| {m:.3g}")
        assert err <= 2e-2 * m


def test_layer_errors_raise():
    x, w_q, w_kv, w_o, b_o, rh, rw = (t.to(DEV) for t in make_layer_inputs(1, 8, 8, 32, 2, 16, 4, 1, seed=1))
    with pytest.raises(ValueError):
        halo_layer_fwd(x, w_q, w_kv, w_o, b_o, rh, rw, 4, 1, 3)        # heads does not divide inner
    with pytest.raises(HaloError):
        halo_layer_fwd(x, w_q, w_kv, w_o, b_o, rh, rw, 4, 1, 2, kernel="split",
                       workspace=torch.empty(16, dtype=torch.uint8, device=DEV))     # too small for the split path
