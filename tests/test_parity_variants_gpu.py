"""GPU parity of the semantic variants (flags of halo_attn_fwd_ex) against
the fp64 oracle's variants, which are pinned to the default semantics in
tests/test_oracle_variants.py.  Same tolerances as the default forward:
1e-4 (fp32, generic kernel), 2e-2 (bf16, persistent matrix-core kernel)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from blocked_local_self_amd import halo_attn_fwd, HaloError, VARIANTS
from blocked_local_self_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2}
LSE_TOL = {"fp32": 1e-4, "bf16": 4e-3}
DEV = "cuda"
ORACLE_FLAG = {"centred_offset": oracle.CENTRED_OFFSET, "zero_pad": oracle.ZERO_PAD,
               "centred_mask": oracle.CENTRED_MASK, "half_split": oracle.HALF_SPLIT}


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


SHAPES = [
    (2, 3, 24, 24, 16, 8, 3, 1),
    (1, 2, 20, 28, 32, 8, 3, 1),    # ragged
    (2, 2, 24, 24, 16, 8, 3, 2),    # strided
    (1, 2, 36, 36, 32, 12, 3, 1),   # 18x18 window (two column tiles)
    (1, 1, 16, 16, 16, 8, 0, 1),    # h = 0
]
VARIANT_SETS = [("centred_offset",), ("zero_pad",), ("centred_mask",), ("half_split",),
                ("zero_pad", "centred_mask"), ("centred_offset", "half_split", "zero_pad")]


@pytest.mark.parametrize("kernel,dtype", [("auto", "bf16"), ("generic", "fp32")])
@pytest.mark.parametrize("variants", VARIANT_SETS, ids=lambda v: "+".join(v))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_variants_match_oracle(shape, variants, kernel, dtype):
    B, heads, H, W, d, block, halo, stride = shape
    print(f"variant case {shape} {variants} {kernel} {dtype}", flush=True)
    inp = make_inputs(B, heads, H, W, d, block, halo, dtype=dtype, seed=sum(shape) + len(variants))
    q, k, v, rh, rw = (t.to(DEV) for t in inp)
    out, lse = halo_attn_fwd(q, k, v, rh, rw, block, halo, stride, kernel=kernel, variants=variants,
                             return_lse=True)
    torch.cuda.synchronize()
    flags = sum(ORACLE_FLAG[n] for n in variants)
    want, want_lse = oracle.halo_attn_ref(*(f64(t) for t in inp), block, halo, stride, return_lse=True,
                                          flags=flags)
    assert np.abs(f64(out) - want).max() <= TOL[dtype]
    assert np.abs(f64(lse) - want_lse).max() <= LSE_TOL[dtype]


def test_variants_refused_where_not_supported():
    q, k, v, rh, rw = (t.to(DEV) for t in make_inputs(1, 1, 16, 16, 16, 8, 3, dtype="bf16", seed=1))
    with pytest.raises(HaloError):
        halo_attn_fwd(q, k, v, rh, rw, 8, 3, kernel="mfma_strip", variants=("zero_pad",))
    with pytest.raises(ValueError):
        halo_attn_fwd(q, k, v, rh, rw, 8, 3, variants=("no_such_variant",))


# ------------------------------------------------------ backward of the variants
BWD_TOL = {"fp32": 1e-4, "bf16": 1.5e-2}   # as for the default backward, relative to max |oracle|


@pytest.mark.parametrize("kernel,dtype", [("mfma", "bf16"), ("generic", "fp32")])
@pytest.mark.parametrize("variants", VARIANT_SETS, ids=lambda v: "+".join(v))
@pytest.mark.parametrize("shape", [(2, 2, 24, 24, 16, 8, 3, 1), (1, 2, 32, 48, 32, 8, 3, 2)],
                         ids=lambda s: "x".join(map(str, s)))
def test_variant_backward_matches_oracle(shape, variants, kernel, dtype):
    from blocked_local_self_amd import halo_attn_bwd
    from blocked_local_self_amd.inputs import make_grad_output
    B, heads, H, W, d, block, halo, stride = shape
    print(f"variant bwd case {shape} {variants} {kernel} {dtype}", flush=True)
    inp = make_inputs(B, heads, H, W, d, block, halo, dtype=dtype, seed=3 * sum(shape) + len(variants))
    g = make_grad_output(B, heads, H // stride, W // stride, d, dtype=dtype, seed=sum(shape))
    q, k, v, rh, rw = (t.to(DEV) for t in inp)
    out, lse = halo_attn_fwd(q, k, v, rh, rw, block, halo, stride, variants=variants, return_lse=True)
    got = halo_attn_bwd(q, k, v, rh, rw, g.to(DEV), block, halo, stride, out=out, lse=lse, kernel=kernel,
                        variants=variants)
    torch.cuda.synchronize()
    flags = sum(ORACLE_FLAG[n] for n in variants)
    want = oracle.halo_attn_bwd_ref(*(f64(t) for t in inp), f64(g), block, halo, stride, flags=flags)
    for name, a, b in zip(["dq", "dk", "dv", "drel_h", "drel_w"], got, want):
        a = f64(a)
        scale = max(float(np.abs(b).max()), 1e-6)
        assert np.abs(a - b).max() <= BWD_TOL[dtype] * scale, name
        if "half_split" in variants and name == "drel_h":
            assert not a[:, d // 2:].any()
        if "half_split" in variants and name == "drel_w":
            assert not a[:, :d // 2].any()
