"""The allocation-free backward (halo_attn_bwd_noalloc, static workspace)
against the workspace-taking halo_attn_bwd, both called through the C ABI
on the same inputs: two calls in a row, the second on a smaller input (the
static array keeps the first call's contents).  The backward is
deterministic (fixed-order sums, no floating-point atomics), so the two
entry points must agree bit for bit."""
import sys

import pytest
import torch

from blocked_local_self_amd import _native, halo_attn_fwd
from blocked_local_self_amd.inputs import make_inputs, make_grad_output

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def grads_of(lib, entry, inp, g, block, halo, stride, dtype, with_lse):
    q, k, v, rh, rw = inp
    B, heads, H, W, d = q.shape
    r = block + 2 * halo
    out = lse = None
    if with_lse:
        out, lse = halo_attn_fwd(q, k, v, rh, rw, block, halo, stride, return_lse=True)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    drh = torch.full((2 * r - 1, d), float("nan"), dtype=torch.float32, device="cuda")
    drw = torch.full_like(drh, float("nan"))
    code = _native.HALO_BF16 if dtype == "bf16" else _native.HALO_F32
    ptr = lambda t: None if t is None else t.data_ptr()
    common = (q.data_ptr(), k.data_ptr(), v.data_ptr(), rh.data_ptr(), rw.data_ptr(), ptr(out), g.data_ptr(),
              ptr(lse), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), drh.data_ptr(), drw.data_ptr())
    sizes = (B, heads, H, W, d, block, halo, stride, float(d) ** -0.5, code, torch.cuda.current_stream().cuda_stream)
    if entry == "noalloc":
        st = lib.halo_attn_bwd_noalloc(*common, *sizes)
    else:
        nws = lib.halo_attn_bwd_workspace_bytes(B, heads, H, W, d, block, halo, stride, code)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
        st = lib.halo_attn_bwd(*common, ws.data_ptr(), ws.numel(), *sizes)
    assert st == 0, _native.last_error()
    torch.cuda.synchronize()
    return dq, dk, dv, drh, drw


SEQUENCES = [
    # two calls in a row, the second smaller: (shape, dtype, lse from the forward)
    [((2, 4, 40, 40, 16, 8, 3, 1), "bf16", False), ((1, 2, 24, 24, 16, 8, 3, 1), "bf16", True)],
    [((1, 3, 32, 32, 32, 8, 3, 1), "bf16", True), ((1, 1, 24, 24, 32, 8, 3, 2), "bf16", False)],
    [((1, 2, 20, 28, 16, 4, 1, 1), "fp32", False), ((1, 1, 12, 12, 16, 4, 1, 2), "fp32", True)],
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=lambda s: "_".join("x".join(map(str, c[0])) for c in s))
def test_noalloc_backward_matches_workspace_backward(seq):
    lib = _native.load()
    for shape, dtype, with_lse in seq:
        print(f"case {shape} {dtype} lse={with_lse}", flush=True)
        sys.stdout.flush()
        B, heads, H, W, d, block, halo, stride = shape
        inp = tuple(t.to("cuda") for t in make_inputs(B, heads, H, W, d, block, halo, dtype=dtype, seed=sum(shape)))
        g = make_grad_output(B, heads, H // stride, W // stride, d, dtype=dtype, seed=3).to("cuda")
        got = grads_of(lib, "noalloc", inp, g, block, halo, stride, dtype, with_lse)
        want = grads_of(lib, "workspace", inp, g, block, halo, stride, dtype, with_lse)
        for a, b in zip(got, want):
            assert torch.isfinite(a).all(), "a gradient element was not written"
            assert torch.equal(a, b)
