"""Pins for the oracle's backward pass (no GPU).

The pages print no backward; HaloNet's models are trained by gradient
descent ("Scaling Local Self-Attention for Parameter Efficient Visual
Backbones", section 4.1), so the backward is the exact derivative of the
forward definition.  Each test checks the oracle's hand-written chain rule
against something else: central finite differences of the (separately
pinned) forward oracle over every input entry, torch autograd through an
independent dense formulation, and invariants the softmax fixes.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.dense_bruteforce import halo_attn_dense_torch


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def case(B, heads, H, W, d, block, halo, stride, seed=0):
    r = block + 2 * halo
    q, k, v = (rnd((B, heads, H, W, d), seed + i) for i in range(3))
    rel_h = rnd((2 * r - 1, d), seed + 3, d ** -0.5)
    rel_w = rnd((2 * r - 1, d), seed + 4, d ** -0.5)
    g = rnd((B, heads, H // stride, W // stride, d), seed + 5)
    return [q, k, v, rel_h, rel_w], g


# (H, W, d, block, halo, stride): ragged blocks, h = 0, b = 1, strides,
# windows wider than the image
GEOMS = [
    (8, 8, 3, 4, 1, 1),
    (6, 5, 2, 4, 1, 1),
    (8, 8, 2, 4, 2, 2),
    (6, 6, 2, 3, 0, 1),
    (5, 4, 2, 1, 1, 1),
    (4, 4, 3, 4, 2, 1),
    (6, 6, 2, 2, 1, 2),
]


# ------------------------------------------------------------ B1 finite differences
@pytest.mark.parametrize("H,W,d,block,halo,stride", GEOMS)
def test_b1_matches_central_differences_of_forward(H, W, d, block, halo, stride):
    ins, g = case(1, 2, H, W, d, block, halo, stride, seed=11 * H + W)
    grads = oracle.halo_attn_bwd_ref(*ins, g, block, halo, stride)
    eps = 1e-5

    def loss(args):
        return float((oracle.halo_attn_ref(*args, block, halo, stride) * g).sum())

    for t in range(5):
        fd = np.zeros_like(ins[t])
        for idx in np.ndindex(*ins[t].shape):
            a = [x.copy() for x in ins]
            a[t][idx] += eps
            lp = loss(a)
            a[t][idx] -= 2 * eps
            fd[idx] = (lp - loss(a)) / (2 * eps)
        np.testing.assert_allclose(grads[t], fd, rtol=1e-6, atol=1e-7,
                                   err_msg=["dq", "dk", "dv", "drel_h", "drel_w"][t])


# -------------------------------------------------- B2 autograd, dense formulation
@pytest.mark.parametrize("H,W,d,block,halo,stride",
                         [(8, 8, 4, 4, 1, 1), (10, 7, 3, 4, 2, 1), (12, 12, 4, 4, 2, 2), (9, 9, 2, 3, 3, 3)])
def test_b2_matches_autograd_of_dense_formulation(H, W, d, block, halo, stride):
    ins, g = case(2, 2, H, W, d, block, halo, stride, seed=H * 31 + d)
    want = oracle.halo_attn_bwd_ref(*ins, g, block, halo, stride)
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in ins]
    out = halo_attn_dense_torch(*ts, block, halo, stride)
    (out * torch.tensor(g)).sum().backward()
    for t in range(5):
        np.testing.assert_allclose(want[t], ts[t].grad.numpy(), rtol=0, atol=1e-10)


# ------------------------------------------------------------------ B3 invariants
def test_b3_softmax_shift_invariances():
    # shifting every key of a slice (or every row of one table) by the same
    # vector shifts all logits of a query uniformly: the loss is unchanged, so
    # those gradients sum to zero; the weights sum to one, so the value
    # gradients sum to the output gradient
    H = W = 10; d = 4; block, halo, stride = 4, 2, 1
    ins, g = case(2, 3, H, W, d, block, halo, stride, seed=5)
    dq, dk, dv, drh, drw = oracle.halo_attn_bwd_ref(*ins, g, block, halo, stride)
    np.testing.assert_allclose(dk.sum(axis=(2, 3)), 0, atol=1e-11)
    np.testing.assert_allclose(drh.sum(axis=0), 0, atol=1e-10)
    np.testing.assert_allclose(drw.sum(axis=0), 0, atol=1e-10)
    np.testing.assert_allclose(dv.sum(axis=(2, 3)), g.sum(axis=(2, 3)), atol=1e-11)
    assert np.abs(dk).max() > 1e-2 and np.abs(drh).max() > 1e-2


def test_b3_constant_values_and_zero_gradient():
    H = W = 8; d = 3; block, halo = 4, 1
    ins, g = case(1, 2, H, W, d, block, halo, 1, seed=9)
    # v constant: out is constant whatever the logits, so the gradients that
    # flow through the logits vanish
    ins_c = list(ins)
    ins_c[2] = np.full_like(ins[2], 0.75)
    dq, dk, dv, drh, drw = oracle.halo_attn_bwd_ref(*ins_c, g, block, halo)
    for x in (dq, dk, drh, drw):
        assert np.abs(x).max() < 1e-13
    assert np.abs(dv).max() > 1e-2
    # zero output gradient: every gradient is zero
    for x in oracle.halo_attn_bwd_ref(*ins, np.zeros_like(g), block, halo):
        assert not x.any()


def test_b3_strided_queries_only_get_dq():
    H = W = 8; d = 2; block, halo, stride = 4, 1, 2
    ins, g = case(1, 1, H, W, d, block, halo, stride, seed=3)
    dq = oracle.halo_attn_bwd_ref(*ins, g, block, halo, stride)[0]
    mask = np.zeros((H, W), bool)
    mask[::stride, ::stride] = True
    assert not dq[0, 0][~mask].any()
    assert np.abs(dq[0, 0][mask]).min() > 0


# -------------------------------------------------------------- B4 set semantics
def test_b4_permuting_keys_permutes_their_gradients():
    rng = np.random.default_rng(2)
    n, d = 9, 5
    q, g = rng.standard_normal(d), rng.standard_normal(d)
    keys, vals = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    bias = rng.standard_normal(n)
    dq, dkeys, dbias, dvals = oracle.set_attention_bwd(q, keys, bias, vals, 0.5, g)
    perm = rng.permutation(n)
    dq2, dkeys2, dbias2, dvals2 = oracle.set_attention_bwd(q, keys[perm], bias[perm], vals[perm], 0.5, g)
    np.testing.assert_allclose(dq2, dq, atol=1e-14)
    np.testing.assert_allclose(dkeys2, dkeys[perm], atol=1e-14)
    np.testing.assert_allclose(dbias2, dbias[perm], atol=1e-14)
    np.testing.assert_allclose(dvals2, dvals[perm], atol=1e-14)
    # one key: the output is that value whatever the logit
    dq1, dk1, db1, dv1 = oracle.set_attention_bwd(q, keys[:1], bias[:1], vals[:1], 0.5, g)
    assert not dq1.any() and not dk1.any() and not db1.any()
    np.testing.assert_allclose(dv1[0], g)


def test_bwd_threads_do_not_change_results_and_bad_arguments():
    ins, g = case(3, 2, 9, 9, 3, 4, 1, 1, seed=1)
    a = oracle.halo_attn_bwd_ref(*ins, g, 4, 1, threads=1)
    b = oracle.halo_attn_bwd_ref(*ins, g, 4, 1, threads=4)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    with pytest.raises(ValueError):
        oracle.halo_attn_bwd_ref(*ins, g[:, :, :4], 4, 1)
    with pytest.raises(ValueError):
        oracle.halo_attn_bwd_ref(*ins, g, 4, 1, query_stride=3)
