"""Pins of the oracle's layer functions (to_q / to_kv, the blocked attention,
head merge, to_out) against what the pages fix.

L1  the layer computed in the order of the HaloAttention module on the pswp.cn
    page (section 4): zero-padded unfold of the input into windows, the
    projections applied to every window position, masks for padded
    positions, heads merged and to_out applied per block
    (tests/dense_bruteforce.halo_layer_module_torch).  The oracle projects
    each pixel once and gathers afterwards: a different route to the same
    numbers.
L2  identity projections reduce the layer to the op (channels = heads*d).
L3  the persistent blocked layout (appendix D) holds the same pixels.
L4  strided queries keep stride-1 windows (section 2.2, Figure 2), so the
    strided layer is the stride-1 layer sampled at every s-th pixel.
L5  with to_out's weight zero the output is the bias at every pixel.
L6  the layer demo on the pswp.cn page (dim 512, block 2, halo 1, 8 heads of
    64 channels) maps an N C H W input to an output of the same shape
    (tests/golden/layer_demo_shapes.json; spatial size cut to 8x8 here).
"""
import json
import os

import numpy as np
import pytest

import oracle
from dense_bruteforce import halo_layer_module_torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _layer_inputs(seed, B, H, W, C, heads, d, block, halo, Cout=None):
    g = np.random.default_rng(seed)
    inner = heads * d
    Cout = C if Cout is None else Cout
    r = block + 2 * halo
    x = g.standard_normal((B, H, W, C))
    w_q = g.standard_normal((inner, C)) * C ** -0.5
    w_kv = g.standard_normal((2 * inner, C)) * C ** -0.5
    w_o = g.standard_normal((Cout, inner)) * inner ** -0.5
    b_o = g.standard_normal(Cout)
    rel_h = g.standard_normal((2 * r - 1, d)) * d ** -0.5
    rel_w = g.standard_normal((2 * r - 1, d)) * d ** -0.5
    return x, w_q, w_kv, w_o, b_o, rel_h, rel_w


@pytest.mark.parametrize("B,H,W,C,heads,d,block,halo,Cout", [
    (2, 8, 8, 12, 2, 8, 4, 1, 12),
    (1, 8, 12, 10, 3, 4, 4, 2, 7),      # non-square, C != inner != Cout
    (1, 6, 6, 5, 1, 6, 2, 1, 5),
])
def test_l1_layer_matches_module_order(B, H, W, C, heads, d, block, halo, Cout):
    x, w_q, w_kv, w_o, b_o, rh, rw = _layer_inputs(7, B, H, W, C, heads, d, block, halo, Cout)
    y = oracle.halo_layer_ref(x, w_q, w_kv, w_o, b_o, rh, rw, block, halo, heads)
    ref = halo_layer_module_torch(x.transpose(0, 3, 1, 2), w_q, w_kv, w_o, b_o, rh, rw, block, halo, heads)
    np.testing.assert_allclose(y, ref.transpose(0, 2, 3, 1), rtol=1e-12, atol=1e-12)


def test_l2_identity_projections_reduce_to_the_op():
    B, H, W, heads, d, block, halo = 2, 8, 8, 2, 4, 4, 1
    C = heads * d
    x, _, _, _, _, rh, rw = _layer_inputs(3, B, H, W, C, heads, d, block, halo)
    eye = np.eye(C)
    y = oracle.halo_layer_ref(x, eye, np.vstack([eye, eye]), eye, np.zeros(C), rh, rw, block, halo, heads)
    qkv = np.ascontiguousarray(x.reshape(B, H, W, heads, d).transpose(0, 3, 1, 2, 4))
    op = oracle.halo_attn_ref(qkv, qkv, qkv, rh, rw, block, halo)
    np.testing.assert_allclose(y, op.transpose(0, 2, 3, 1, 4).reshape(B, H, W, C), rtol=0, atol=1e-15)


@pytest.mark.parametrize("stride", [1, 2])
def test_l3_blocked_layout_holds_the_same_pixels(stride):
    B, H, W, C, heads, d, block, halo = 1, 8, 16, 6, 2, 4, 4, 1
    x, w_q, w_kv, w_o, b_o, rh, rw = _layer_inputs(11, B, H, W, C, heads, d, block, halo)
    y = oracle.halo_layer_ref(x, w_q, w_kv, w_o, b_o, rh, rw, block, halo, heads, stride)
    xb = oracle.from_nhwc(x, "blocked", block)
    assert xb.shape == (B, H // block, W // block, block * block, C)
    # pixel (i*b + p1, j*b + p2) sits at [., i, j, p1*b + p2, .]
    assert np.array_equal(xb[0, 1, 2, 1 * block + 3], x[0, 1 * block + 1, 2 * block + 3])
    yb = oracle.halo_layer_ref(xb, w_q, w_kv, w_o, b_o, rh, rw, block, halo, heads, stride, layout="blocked")
    np.testing.assert_array_equal(yb, oracle.from_nhwc(y, "blocked", block // stride))


def test_l4_strided_layer_samples_the_stride1_layer():
    B, H, W, C, heads, d, block, halo = 1, 8, 8, 6, 2, 4, 4, 2
    x, w_q, w_kv, w_o, b_o, rh, rw = _layer_inputs(5, B, H, W, C, heads, d, block, halo)
    y1 = oracle.halo_layer_ref(x, w_q, w_kv, w_o, b_o, rh, rw, block, halo, heads, 1)
    y2 = oracle.halo_layer_ref(x, w_q, w_kv, w_o, b_o, rh, rw, block, halo, heads, 2)
    np.testing.assert_allclose(y2, y1[:, ::2, ::2], rtol=0, atol=1e-14)


def test_l5_zero_out_weight_gives_the_bias():
    B, H, W, C, heads, d, block, halo = 1, 4, 4, 3, 1, 4, 2, 1
    x, w_q, w_kv, w_o, b_o, rh, rw = _layer_inputs(9, B, H, W, C, heads, d, block, halo)
    y = oracle.halo_layer_ref(x, w_q, w_kv, np.zeros_like(w_o), b_o, rh, rw, block, halo, heads)
    np.testing.assert_array_equal(y, np.broadcast_to(b_o, y.shape))


def test_l6_layer_demo_keeps_the_input_shape():
    g = json.load(open(os.path.join(GOLDEN, "layer_demo_shapes.json")))
    N, C, _, _ = g["input_nchw"]
    H = W = 8
    heads, d, block, halo = g["heads"], g["dim_head"], g["block"], g["halo"]
    x, w_q, w_kv, w_o, b_o, rh, rw = _layer_inputs(1, N, H, W, C, heads, d, block, halo)
    assert rh.shape[0] == g["rel_table_rows"]
    y = oracle.halo_layer_ref(x, w_q, w_kv, w_o, b_o, rh, rw, block, halo, heads)
    assert y.shape == x.shape
    ref = halo_layer_module_torch(x.transpose(0, 3, 1, 2), w_q, w_kv, w_o, b_o, rh, rw, block, halo, heads)
    np.testing.assert_allclose(y, ref.transpose(0, 2, 3, 1), rtol=1e-10, atol=1e-10)


def test_layer_rejects_bad_shapes():
    x, w_q, w_kv, w_o, b_o, rh, rw = _layer_inputs(2, 1, 4, 4, 6, 2, 4, 2, 1)
    with pytest.raises(ValueError):
        oracle.halo_proj_in_ref(x, w_q.T, w_kv, 2)
    with pytest.raises(ValueError):
        oracle.halo_proj_in_ref(x, w_q, w_kv, 3)
    with pytest.raises(ValueError):
        oracle.to_nhwc(x[:, :2, :2].reshape(1, 1, 1, 4, 6), "blocked", 3)
