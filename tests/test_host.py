"""Host-side logic: workload accounting and the seeded input recipe."""
import torch

from blocked_local_self_amd import workloads
from blocked_local_self_amd.inputs import make_inputs, make_workload_inputs


def test_workload_shapes_and_counts():
    w = workloads.get("early_stage_bf16_64x64_d16_b8h3")
    assert w.r == 14 and w.nblocks == 256 * 64
    assert w.flops == 4 * 16 * 196 * 256 * 64 * 64
    assert w.tokens == 32 * 64 * 64
    assert w.alg_bytes == 2 * 16 * 256 * (2 * 4096 + 2 * 4096)
    big = workloads.get("large_bf16_128x128_d32_b12h3")
    assert big.nblocks == 64 * 11 * 11     # ragged: 128 = 10*12 + 8


def test_strided_layer_has_a_quarter_of_the_flops():
    # Section 2.2: stride-2 attention downsampling cuts the layer's FLOPs 4x.
    s1 = workloads.get("early_stage_bf16_64x64_d16_b8h3")
    s2 = workloads.get("strided_bf16_64x64_d16_b8h3_s2")
    assert s2.flops * 4 == s1.flops
    assert s2.tokens * 4 == s1.tokens


def test_flop_convention_reproduces_note_2_ratio():
    # Note 2 of section 2.2: global attention over a 128x128, 64-channel input
    # costs about 28x a 64->64 3x3 convolution.  One N^2*c product against the
    # convolution's multiply-adds gives that ratio.
    n = 128 * 128
    attn = n * n * 64
    conv = 9 * 64 * 64 * n
    assert round(attn / conv) == 28


def test_inputs_are_seeded_and_rounded():
    a = make_inputs(1, 2, 8, 8, 16, 4, 1, dtype="bf16", seed=3)
    b = make_inputs(1, 2, 8, 8, 16, 4, 1, dtype="bf16", seed=3)
    c = make_inputs(1, 2, 8, 8, 16, 4, 1, dtype="bf16", seed=4)
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and torch.equal(x, y)
    assert not torch.equal(a[0], c[0])
    q, k, v, rh, rw = a
    assert q.shape == (1, 2, 8, 8, 16) and rh.shape == (11, 16)
    # tables carry the d**-0.5 initialisation scale
    assert rh.float().std() < 0.6 and q.float().std() > 0.6


def test_fp32_workload_inputs():
    w = workloads.get("tiny_fp32_16x16_d16_b4h1")
    q, k, v, rh, rw = make_workload_inputs(w)
    assert q.dtype == torch.float32 and q.shape == w.shape() and rh.shape == (11, 16)


def test_layer_input_layout_matches_oracle_layout():
    import numpy as np
    import torch
    import oracle
    from blocked_local_self_amd.inputs import make_layer_inputs, nhwc_to_layout
    x = make_layer_inputs(2, 8, 12, 8, 2, 4, 4, 1, dtype="fp32", seed=1)[0]
    for lay in ("nhwc", "blocked"):
        np.testing.assert_array_equal(nhwc_to_layout(x, lay, 4).numpy(), oracle.from_nhwc(x.numpy(), lay, 4))
