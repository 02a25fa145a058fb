"""GPU parity of the backward pass: the HIP kernels (through the C ABI)
against the fp64 oracle's backward, on the same seeded inputs.

The pages print no backward; HaloNet's models are trained by gradient
descent ("Scaling Local Self-Attention for Parameter Efficient Visual
Backbones", section 4.1), and the oracle's backward is pinned to finite
differences of the forward definition.  Each gradient tensor is compared
element by element, relative to its own largest magnitude:

    max |gpu - oracle| <= TOL[dtype] * max |oracle|

fp32 inputs: 1e-4 (fp32 sums of up to a few hundred terms, fast exp and
log).  bf16 inputs: 1.5e-2, from the rounding of dq, dk, dv to bf16 (half an
ulp, 2^-9 of the value) on top of fp32 arithmetic, with headroom for the
cancellation in dl = P (dout.v - dout.out).  The table gradients are fp32
for both dtypes but sum over every query of the batch; they are held to the
same relative bound.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from blocked_local_self_amd import halo_attn_bwd, halo_attention, halo_attn_fwd, HaloError, workloads
from blocked_local_self_amd.inputs import make_inputs, make_workload_inputs, make_grad_output

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 1.5e-2}
DEV = "cuda"
NAMES = ["dq", "dk", "dv", "drel_h", "drel_w"]


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def case(B, heads, H, W, d, block, halo, stride, dtype, seed):
    ins = make_inputs(B, heads, H, W, d, block, halo, dtype=dtype, seed=seed)
    g = make_grad_output(B, heads, H // stride, W // stride, d, dtype=dtype, seed=seed)
    return ins, g


def gpu_bwd(ins, g, block, halo, stride, kernel="auto", use_fwd=False):
    """Backward through the C ABI; with use_fwd the forward's out and lse
    (halo_attn_fwd with return_lse) are passed in instead of recomputed."""
    q, k, v, rh, rw = (t.to(DEV) for t in ins)
    extra = {}
    if use_fwd:
        out, lse = halo_attn_fwd(q, k, v, rh, rw, block, halo, stride, return_lse=True)
        extra = {"out": out, "lse": lse}
    res = halo_attn_bwd(q, k, v, rh, rw, g.to(DEV), block, halo, stride, kernel=kernel, **extra)
    torch.cuda.synchronize()
    return [f64(t) for t in res]


def ref_bwd(ins, g, block, halo, stride):
    return oracle.halo_attn_bwd_ref(*(f64(t) for t in ins), f64(g), block, halo, stride)


def compare(got, want, dtype, label=""):
    worst = 0.0
    for name, a, b in zip(NAMES, got, want):
        assert a.shape == b.shape, name
        assert np.isfinite(a).all(), f"{name}: non-finite"
        scale = max(float(np.abs(b).max()), 1e-6)
        rel = float(np.abs(a - b).max()) / scale
        worst = max(worst, rel)
        assert rel <= TOL[dtype], f"{label} {name}: max err {rel:.3e} of max |ref| {scale:.3e}"
    return worst


SMALL = [
    # (B, heads, H, W, d, block, halo, stride)
    (2, 3, 24, 24, 16, 8, 3, 1),
    (1, 2, 24, 24, 32, 8, 3, 1),
    (1, 2, 20, 28, 16, 8, 3, 1),    # ragged last block row and column
    (2, 2, 24, 24, 16, 8, 3, 2),    # strided queries
    (1, 2, 36, 36, 32, 12, 3, 1),   # 18x18 window
    (1, 2, 32, 40, 16, 12, 3, 2),   # ragged + strided + wide window
    (1, 2, 16, 16, 16, 4, 1, 1),
    (1, 1, 16, 16, 16, 8, 0, 1),    # h = 0
    (1, 2, 12, 12, 16, 16, 1, 1),   # block larger than the image
    (1, 1, 20, 20, 16, 2, 5, 1),    # halo wider than a block: keys seen by 5x5 blocks
    (1, 2, 9, 7, 24, 3, 1, 1),      # odd d and block
    (1, 1, 10, 10, 64, 4, 2, 2),
    (1, 1, 6, 6, 128, 2, 1, 1),
]


@pytest.mark.parametrize("use_fwd", [False, True], ids=["recompute", "fwd_lse"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_small_shapes_match_oracle(shape, dtype, use_fwd):
    B, heads, H, W, d, block, halo, stride = shape
    say(f"bwd case {shape} {dtype} use_fwd={use_fwd}")
    ins, g = case(*shape, dtype, seed=sum(shape))
    got = gpu_bwd(ins, g, block, halo, stride, use_fwd=use_fwd, kernel="generic")
    compare(got, ref_bwd(ins, g, block, halo, stride), dtype, str(shape))


def mfma_ok(shape):
    B, heads, H, W, d, block, halo, stride = shape
    side = block // stride
    return (d in (16, 32) and block + 2 * halo <= 16 and H % block == 0 and W % block == 0
            and side % 4 == 0 and side * side in (16, 64))


MFMA_SHAPES = [s for s in SMALL if mfma_ok(s)] + [
    (1, 2, 32, 48, 32, 8, 3, 2),   # d = 32, strided
    (2, 1, 16, 16, 16, 8, 4, 1),   # r = 16, the widest window of the path
    (1, 1, 8, 8, 16, 4, 6, 1),     # r = 16 with 4x4 blocks and stride 1 (one query tile)
]


# Shapes the strip kernel does not take (windows wider than 16 columns,
# partial edge blocks, other query counts per block): the 16-query tile
# backward kernels.
TILE_SHAPES = [
    (1, 2, 36, 36, 32, 12, 3, 1),    # 18x18 windows, whole blocks
    (1, 2, 40, 44, 32, 12, 3, 1),    # 18x18 windows, partial last block row and column
    (1, 2, 20, 28, 16, 8, 3, 1),     # 14x14 windows, partial blocks
    (1, 2, 32, 40, 16, 12, 3, 2),    # partial + strided + 18x18 windows
    (1, 1, 20, 20, 16, 2, 5, 1),     # halo wider than a block: keys seen by 7x7 blocks
    (1, 2, 30, 30, 32, 12, 6, 1),    # r = 24, d = 32
    (1, 1, 40, 40, 16, 16, 8, 1),    # r = 32, d = 16
    (1, 2, 24, 21, 16, 6, 3, 3),     # block 6 (patches cross the block edge), partial, stride 3
    (2, 1, 12, 12, 32, 12, 0, 1),    # h = 0: windows are the blocks
    (1, 2, 40, 36, 32, 16, 4, 1),    # 16 key patches per block at d = 32: two passes of the key kernel
]


@pytest.mark.parametrize("use_fwd", [False, True], ids=["recompute", "fwd_lse"])
@pytest.mark.parametrize("shape", TILE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_tile_backward_matches_oracle(shape, use_fwd):
    B, heads, H, W, d, block, halo, stride = shape
    say(f"bwd tile case {shape} use_fwd={use_fwd}")
    ins, g = case(*shape, "bf16", seed=5 * sum(shape))
    got = gpu_bwd(ins, g, block, halo, stride, use_fwd=use_fwd, kernel="mfma")
    worst = compare(got, ref_bwd(ins, g, block, halo, stride), "bf16", str(shape))
    say(f"  worst relative error {worst:.3e}")


@pytest.mark.parametrize("use_fwd", [False, True], ids=["recompute", "fwd_lse"])
@pytest.mark.parametrize("shape", MFMA_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_matrix_core_backward_matches_oracle(shape, use_fwd):
    B, heads, H, W, d, block, halo, stride = shape
    say(f"bwd mfma case {shape} use_fwd={use_fwd}")
    ins, g = case(*shape, "bf16", seed=3 * sum(shape))
    got = gpu_bwd(ins, g, block, halo, stride, use_fwd=use_fwd, kernel="mfma")
    worst = compare(got, ref_bwd(ins, g, block, halo, stride), "bf16", str(shape))
    say(f"  worst relative error {worst:.3e}")


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_workload_full_size(name):
    wl = workloads.get(name)
    say(f"bwd workload {name}")
    ins = make_workload_inputs(wl, seed=0)
    g = make_grad_output(wl.B, wl.heads, wl.Ho, wl.Wo, wl.d, dtype=wl.dtype, seed=0)
    got = gpu_bwd(ins, g, wl.block, wl.halo, wl.stride, use_fwd=True)
    want = ref_bwd(ins, g, wl.block, wl.halo, wl.stride)
    worst = compare(got, want, wl.dtype, name)
    say(f"  worst relative error {worst:.3e}")


@pytest.mark.parametrize("kernel,shape", [("mfma", (2, 4, 32, 32, 16, 8, 3, 1)),
                                          ("mfma", (1, 3, 40, 44, 32, 12, 3, 1)),
                                          ("generic", (2, 4, 32, 32, 16, 8, 3, 1))])
def test_deterministic(kernel, shape):
    ins, g = case(*shape, "bf16", seed=21)
    a = gpu_bwd(ins, g, *shape[5:], kernel=kernel)
    b = gpu_bwd(ins, g, *shape[5:], kernel=kernel)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("shape", [(1, 1, 40, 40, 16, 20, 6, 1),    # block 20 > 16
                                   (1, 1, 40, 40, 32, 16, 8, 1),    # r = 32 at d = 32: window past LDS
                                   (1, 1, 16, 16, 24, 4, 1, 1)])    # d = 24
def test_matrix_core_backward_refuses_what_it_does_not_cover(shape):
    ins, g = case(*shape, "bf16", seed=1)
    with pytest.raises(HaloError):
        gpu_bwd(ins, g, *shape[5:], kernel="mfma")


def test_autograd_function_matches_direct_call():
    ins, g = case(1, 2, 24, 24, 16, 8, 3, 1, "fp32", seed=22)
    ts = [t.to(DEV).requires_grad_(True) for t in ins]
    out = halo_attention(*ts, 8, 3)
    ref_out = halo_attn_fwd(*(t.detach() for t in ts), 8, 3)
    assert torch.equal(out.detach(), ref_out)
    out.backward(g.to(DEV))
    direct = gpu_bwd(ins, g, 8, 3, 1, use_fwd=True)   # the function keeps the forward's out and lse
    for t, want in zip(ts, direct):
        assert np.array_equal(f64(t.grad), want)


def test_zero_output_gradient_and_constant_values():
    ins, g = case(1, 2, 24, 24, 16, 8, 3, 1, "fp32", seed=23)
    for x in gpu_bwd(ins, torch.zeros_like(g), 8, 3, 1):
        assert not x.any()
    q, k, v, rh, rw = ins
    got = gpu_bwd((q, k, torch.full_like(v, 0.5), rh, rw), g, 8, 3, 1)
    for name, x in zip(NAMES, got):
        if name != "dv":
            assert np.abs(x).max() < 1e-5, name


def test_empty_and_errors_on_gpu():
    q = torch.zeros(0, 2, 8, 8, 16, dtype=torch.bfloat16, device=DEV)
    t = torch.zeros(11, 16, dtype=torch.bfloat16, device=DEV)
    dq, dk, dv, drh, drw = halo_attn_bwd(q, q, q, t, t, q, 4, 1)
    torch.cuda.synchronize()
    assert dq.shape == q.shape and not drh.any() and not drw.any()
    x = torch.zeros(1, 1, 8, 8, 16, dtype=torch.bfloat16, device=DEV)
    small = torch.zeros(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        halo_attn_bwd(x, x, x, t, t, x, 4, 1, workspace=small)
