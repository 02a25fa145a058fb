"""Pins for the oracle's semantic variants (no GPU).

The pages leave several points open (see the readings in the oracle's
header); the variants implement the other readings so that results can be
matched to them.  Each variant is pinned to the pages' default semantics on
transformed inputs, a route that does not go through the variant's code:

  centred table offset  = default with both tables shifted down by h rows;
  zero padding          = default on the image embedded, block-aligned, in a
                          zero canvas wide enough for every window;
  centred (SASA) mask   = default with block 1 (the (2h+1)^2 window centred on
                          each pixel) and the matching slice of the tables;
  half-split embedding  = default with the unused halves of the tables zeroed
                          (appendix A of "Scaling Local Self-Attention for
                          Parameter Efficient Visual Backbones").
"""
import numpy as np
import pytest

import oracle
from oracle import CENTRED_OFFSET, ZERO_PAD, CENTRED_MASK, HALF_SPLIT


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def case(B, heads, H, W, d, block, halo, seed=0):
    r = block + 2 * halo
    q, k, v = (rnd((B, heads, H, W, d), seed + i) for i in range(3))
    rel_h = rnd((2 * r - 1, d), seed + 3, d ** -0.5)
    rel_w = rnd((2 * r - 1, d), seed + 4, d ** -0.5)
    return q, k, v, rel_h, rel_w


GEOMS = [(8, 8, 4, 4, 1, 1), (10, 7, 3, 4, 2, 1), (12, 12, 4, 4, 2, 2), (9, 9, 2, 3, 3, 3), (6, 6, 3, 2, 1, 1)]


@pytest.mark.parametrize("H,W,d,block,halo,stride", GEOMS)
def test_centred_offset_is_default_with_tables_shifted_by_h(H, W, d, block, halo, stride):
    q, k, v, rh, rw = case(2, 2, H, W, d, block, halo, seed=H + W)
    got = oracle.halo_attn_ref(q, k, v, rh, rw, block, halo, stride, flags=CENTRED_OFFSET)
    want = oracle.halo_attn_ref(q, k, v, np.roll(rh, halo, axis=0), np.roll(rw, halo, axis=0),
                                block, halo, stride)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)
    if halo:
        assert np.abs(got - oracle.halo_attn_ref(q, k, v, rh, rw, block, halo, stride)).max() > 1e-3


def test_centred_offset_one_hot_picks_the_displaced_key():
    H = W = 12; d = 4; block, halo = 4, 2
    r = block + 2 * halo
    v = rnd((1, 1, H, W, d), 1)
    q = np.zeros((1, 1, H, W, d)); q[..., 0] = 1.0
    k = np.zeros_like(q)
    for dy, dx in [(0, 0), (1, -2), (-3, 2)]:
        rh = np.zeros((2 * r - 1, d)); rw = np.zeros((2 * r - 1, d))
        rh[r - 1 + dy, 0] = 60.0; rw[r - 1 + dx, 0] = 60.0   # centre row r-1 = displacement 0
        out = oracle.halo_attn_ref(q, k, v, rh, rw, block, halo, scale=1.0, flags=CENTRED_OFFSET)
        for y in range(H):
            for x in range(W):
                y0, x0 = (y // block) * block - halo, (x // block) * block - halo
                ky, kx = y + dy, x + dx
                if 0 <= ky < H and 0 <= kx < W and y0 <= ky < y0 + r and x0 <= kx < x0 + r:
                    np.testing.assert_allclose(out[0, 0, y, x], v[0, 0, ky, kx], atol=1e-9)


@pytest.mark.parametrize("H,W,d,block,halo,stride", GEOMS)
def test_zero_pad_is_default_on_a_zero_canvas(H, W, d, block, halo, stride):
    q, k, v, rh, rw = case(1, 2, H, W, d, block, halo, seed=2 * H + W)
    got = oracle.halo_attn_ref(q, k, v, rh, rw, block, halo, stride, flags=ZERO_PAD)
    m = -(-halo // block) * block                    # block-aligned padding >= h
    pad = lambda t: np.pad(t, ((0, 0), (0, 0), (m, m + block), (m, m + block), (0, 0)))
    full = oracle.halo_attn_ref(pad(q), pad(k), pad(v), rh, rw, block, halo, stride)
    want = full[:, :, m // stride:(m + H) // stride, m // stride:(m + W) // stride]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)
    if halo:
        assert np.abs(got - oracle.halo_attn_ref(q, k, v, rh, rw, block, halo, stride)).max() > 1e-3


@pytest.mark.parametrize("H,W,d,block,halo", [(8, 8, 4, 4, 1), (10, 7, 3, 4, 2), (9, 9, 2, 3, 3), (12, 8, 3, 6, 2)])
def test_centred_mask_is_the_pixel_centred_window(H, W, d, block, halo):
    q, k, v, rh, rw = case(1, 2, H, W, d, block, halo, seed=3 * H + W)
    got = oracle.halo_attn_ref(q, k, v, rh, rw, block, halo, flags=CENTRED_MASK)
    # block 1: window side 2h+1 centred on the pixel, table row D + 3h; the
    # same displacement D reads row D + (block + 3h - 1) of the block tables
    c0 = block + 3 * halo - 1
    sl = slice(c0 - 3 * halo, c0 - 3 * halo + 4 * halo + 1)
    want = oracle.halo_attn_ref(q, k, v, rh[sl], rw[sl], 1, halo)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)
    # with block 1 the mask changes nothing
    np.testing.assert_allclose(oracle.halo_attn_ref(q, k, v, rh[sl], rw[sl], 1, halo, flags=CENTRED_MASK),
                               want, rtol=0, atol=1e-15)


@pytest.mark.parametrize("d", [4, 5, 16])
def test_half_split_is_default_with_zeroed_halves(d):
    H = W = 8; block, halo = 4, 2
    q, k, v, rh, rw = case(2, 1, H, W, d, block, halo, seed=d)
    got = oracle.halo_attn_ref(q, k, v, rh, rw, block, halo, flags=HALF_SPLIT)
    rh2, rw2 = rh.copy(), rw.copy()
    rh2[:, d // 2:] = 0.0
    rw2[:, :d // 2] = 0.0
    np.testing.assert_allclose(got, oracle.halo_attn_ref(q, k, v, rh2, rw2, block, halo), rtol=0, atol=1e-13)


def test_combined_flags_and_bad_flags():
    H = W = 8; d = 4; block, halo = 4, 1
    q, k, v, rh, rw = case(1, 1, H, W, d, block, halo, seed=11)
    got = oracle.halo_attn_ref(q, k, v, rh, rw, block, halo, flags=CENTRED_OFFSET | HALF_SPLIT)
    rh2, rw2 = np.roll(rh, halo, axis=0), np.roll(rw, halo, axis=0)
    rh2[:, d // 2:] = 0.0
    rw2[:, :d // 2] = 0.0
    np.testing.assert_allclose(got, oracle.halo_attn_ref(q, k, v, rh2, rw2, block, halo), rtol=0, atol=1e-13)
    with pytest.raises(ValueError):
        oracle.halo_attn_ref(q, k, v, rh, rw, block, halo, flags=16)


# ------------------------------------------------ backward of the variants
@pytest.mark.parametrize("flags", [CENTRED_OFFSET, ZERO_PAD, CENTRED_MASK, HALF_SPLIT,
                                   ZERO_PAD | CENTRED_MASK | HALF_SPLIT])
@pytest.mark.parametrize("H,W,d,block,halo,stride", [(6, 5, 2, 4, 1, 1), (8, 8, 2, 4, 2, 2)])
def test_variant_backward_matches_central_differences(H, W, d, block, halo, stride, flags):
    ins = list(case(1, 2, H, W, d, block, halo, seed=7 * H + flags))
    g = rnd((1, 2, H // stride, W // stride, d), 99)
    grads = oracle.halo_attn_bwd_ref(*ins, g, block, halo, stride, flags=flags)
    eps = 1e-5

    def loss(a):
        return float((oracle.halo_attn_ref(*a, block, halo, stride, flags=flags) * g).sum())

    for t in range(5):
        fd = np.zeros_like(ins[t])
        for idx in np.ndindex(*ins[t].shape):
            a = [x.copy() for x in ins]
            a[t][idx] += eps
            lp = loss(a)
            a[t][idx] -= 2 * eps
            fd[idx] = (lp - loss(a)) / (2 * eps)
        np.testing.assert_allclose(grads[t], fd, rtol=1e-6, atol=1e-7)
    if flags & HALF_SPLIT:   # unused table channels get no gradient
        assert not grads[3][:, d // 2:].any() and not grads[4][:, :d // 2].any()
