"""The C-ABI entry point halo_attn_fwd itself, called through ctypes with
device pointers and the caller's stream (the Python binding goes through
halo_attn_fwd_ex), compared element by element with the fp64 oracle.

Tolerances as in test_parity_gpu: max-abs 1e-4 (fp32), 2e-2 (bf16, fp32
accumulate).  Shapes: the tiny fp32 configuration, a two-image slice of the
early-stage shape (64x64, d = 16, block 8, halo 3) and one image of the
large shape (128x128, d = 32, block 12, halo 3: 18x18 windows, partial edge
blocks) -- "Scaling Local Self-Attention for Parameter Efficient Visual
Backbones", section 2.2.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from blocked_local_self_amd import _native
from blocked_local_self_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = [
    # (B, heads, H, W, d, block, halo, stride, dtype, tol)
    (1, 2, 16, 16, 16, 4, 1, 1, "fp32", 1e-4),
    (1, 2, 64, 64, 16, 8, 3, 1, "bf16", 2e-2),
    (1, 1, 64, 64, 16, 8, 3, 2, "bf16", 2e-2),
    (1, 1, 128, 128, 32, 12, 3, 1, "bf16", 2e-2),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:8])) + "-" + c[8])
def test_halo_attn_fwd_symbol_matches_oracle(case):
    B, heads, H, W, d, block, halo, stride, dtype, tol = case
    print(f"case {case}", flush=True)
    sys.stdout.flush()
    lib = _native.load()
    inp = make_inputs(B, heads, H, W, d, block, halo, dtype=dtype, seed=7)
    q, k, v, rh, rw = (t.to("cuda") for t in inp)
    out = torch.full((B, heads, H // stride, W // stride, d), float("nan"), dtype=q.dtype, device="cuda")
    stream = torch.cuda.current_stream()
    code = _native.HALO_BF16 if dtype == "bf16" else _native.HALO_F32
    st = lib.halo_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), rh.data_ptr(), rw.data_ptr(),
                           out.data_ptr(), B, heads, H, W, d, block, halo, stride, float(d) ** -0.5, code,
                           stream.cuda_stream)
    assert st == 0, _native.last_error()
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all(), "an output element was not written"
    want = oracle.halo_attn_ref(*(t.double().numpy() for t in inp), block, halo, stride)
    err = float(np.abs(got - want).max())
    assert err <= tol, err


@pytest.mark.gpu
def test_kernel_name_query_names_the_launched_kernels():
    """The kernels the query names for the stage shapes (the benchmark reports
    them and keys its traffic records on them)."""
    from blocked_local_self_amd import workloads
    name = lambda wl, kernel=_native.HALO_KERNEL_AUTO: _native.fwd_kernel_name(
        wl.B, wl.heads, wl.H, wl.W, wl.d, wl.block, wl.halo, wl.stride,
        _native.HALO_BF16 if wl.dtype == "bf16" else _native.HALO_F32, kernel=kernel)
    get = workloads.get
    assert name(get("large_bf16_128x128_d32_b12h3")) == "tile"
    assert name(get("large_bf16_128x128_d32_b12h3"), _native.HALO_KERNEL_MFMA_RING) == "ring"
    assert name(get("large_bf16_128x128_d32_b12h3"), _native.HALO_KERNEL_MFMA_STRIP) == "strip"
    for wl in ("early_stage_bf16_64x64_d16_b8h3", "mid_stage_bf16_32x32_d32_b8h3",
               "strided_bf16_64x64_d16_b8h3_s2"):
        assert name(get(wl)) == "ring", wl
    assert name(get("detection_bf16_64x64_d16_b32h3")) == "wide"
    assert name(get("tiny_fp32_16x16_d16_b4h1")) == "generic"
