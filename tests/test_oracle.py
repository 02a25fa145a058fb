"""Pins for the fp64 CPU oracle (no GPU).

Each test checks the oracle against something other than itself: a dense
global-attention formulation, closed forms, special cases that reduce to a
library routine, invariants, and the geometry the pages print.  Page
references: "Scaling Local Self-Attention for Parameter Efficient Visual
Backbones" (HaloNet) sections 2.1, 2.2 (Figures 1, 2), 4.3 (Figure 7) and
appendix A; the HaloAttention module on the pswp.cn blog page, section 4.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
from tests.dense_bruteforce import halo_attn_dense, halo_lse_dense

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def case(B, heads, H, W, d, block, halo, seed=0):
    r = block + 2 * halo
    q, k, v = (rnd((B, heads, H, W, d), seed + i) for i in range(3))
    rel_h = rnd((2 * r - 1, d), seed + 3, d ** -0.5)
    rel_w = rnd((2 * r - 1, d), seed + 4, d ** -0.5)
    return q, k, v, rel_h, rel_w


# ---------------------------------------------------------------- P1 brute force
P1_CASES = [
    # (H, W, d, block, halo, stride)
    (8, 8, 4, 4, 1, 1),
    (8, 8, 4, 4, 1, 2),
    (12, 12, 3, 4, 2, 1),
    (12, 12, 3, 4, 2, 2),
    (9, 7, 5, 3, 1, 1),     # b divides neither side exactly? (9 yes, 7 no)
    (10, 10, 4, 4, 2, 2),   # ragged last block row/col
    (10, 6, 2, 4, 0, 1),    # h = 0
    (6, 6, 3, 1, 1, 1),     # b = 1
    (5, 5, 3, 1, 2, 1),     # b = 1, window larger than half the image
    (7, 11, 4, 2, 1, 1),
    (12, 8, 4, 4, 1, 4),    # stride = block
    (4, 4, 2, 3, 2, 1),     # ragged, window covers image
    (12, 12, 6, 3, 0, 3),   # h = 0 with stride 3 (= block): one query per block
]


@pytest.mark.parametrize("H,W,d,block,halo,stride", P1_CASES)
def test_p1_oracle_matches_dense_bruteforce(H, W, d, block, halo, stride):
    if H % stride or W % stride:
        pytest.skip("stride must divide H and W")
    q, k, v, rh, rw = case(2, 2, H, W, d, block, halo, seed=H * 100 + W)
    got = oracle.halo_attn_ref(q, k, v, rh, rw, block, halo, stride)
    want = halo_attn_dense(q, k, v, rh, rw, block, halo, stride)
    assert got.shape == want.shape == (2, 2, H // stride, W // stride, d)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("H,W,d,block,halo,stride", P1_CASES[:8])
def test_p1_lse_matches_dense_bruteforce(H, W, d, block, halo, stride):
    q, k, v, rh, rw = case(2, 2, H, W, d, block, halo, seed=H * 10 + W)
    out, lse = oracle.halo_attn_ref(q, k, v, rh, rw, block, halo, stride, return_lse=True)
    np.testing.assert_allclose(lse, halo_lse_dense(q, k, rh, rw, block, halo, stride), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(out, oracle.halo_attn_ref(q, k, v, rh, rw, block, halo, stride))


def test_p1_lse_of_zero_logits_counts_the_in_image_window():
    # q = 0: every logit is 0, so exp(lse) is the number of in-image window keys
    H = W = 10; block, halo = 4, 2
    q, k, v, rh, rw = case(1, 1, H, W, 3, block, halo, seed=4)
    _, lse = oracle.halo_attn_ref(np.zeros_like(q), k, v, rh, rw, block, halo, return_lse=True)
    r = block + 2 * halo
    for y in range(H):
        for x in range(W):
            y0, x0 = (y // block) * block - halo, (x // block) * block - halo
            n = (min(H, y0 + r) - max(0, y0)) * (min(W, x0 + r) - max(0, x0))
            assert abs(lse[0, 0, y, x] - np.log(n)) < 1e-13


def test_p1_negative_control_wrong_offset_is_detected():
    # A plausible slip -- centring the table at r-1 instead of r-1+h -- must be
    # visible to the brute-force comparison: shifting both tables by h rows
    # emulates it and has to change the output.
    H = W = 8; block, halo, d = 4, 2, 4
    q, k, v, rh, rw = case(1, 1, H, W, d, block, halo, seed=7)
    base = oracle.halo_attn_ref(q, k, v, rh, rw, block, halo)
    rh2, rw2 = np.roll(rh, halo, axis=0), np.roll(rw, halo, axis=0)
    shifted = oracle.halo_attn_ref(q, k, v, rh2, rw2, block, halo)
    assert np.abs(base - shifted).max() > 1e-3


# ------------------------------------------------------ P2 q = 0, rel = 0 -> mean
@pytest.mark.parametrize("H,W,block,halo,stride", [(8, 8, 4, 1, 1), (10, 7, 4, 3, 1), (12, 12, 6, 2, 2)])
def test_p2_zero_query_gives_mean_of_in_image_window(H, W, block, halo, stride):
    d = 3
    _, k, v, _, _ = case(1, 2, H, W, d, block, halo, seed=11)
    r = block + 2 * halo
    q = np.zeros_like(k)
    z = np.zeros((2 * r - 1, d))
    got = oracle.halo_attn_ref(q, k, v, z, z, block, halo, stride)
    for yo in range(H // stride):
        for xo in range(W // stride):
            y, x = yo * stride, xo * stride
            y0 = (y // block) * block - halo
            x0 = (x // block) * block - halo
            win = v[:, :, max(0, y0):min(H, y0 + r), max(0, x0):min(W, x0 + r), :]
            want = win.mean(axis=(2, 3))
            np.testing.assert_allclose(got[:, :, yo, xo], want, rtol=0, atol=1e-13)


def test_p2_unmasked_zero_padding_would_differ():
    # The alternative reading (pad with zeros and keep them in the softmax)
    # gives sum(v)/r^2 at border blocks; the oracle must not.
    H = W = 8; block, halo, d = 4, 2, 2
    _, k, v, _, _ = case(1, 1, H, W, d, block, halo, seed=12)
    r = block + 2 * halo
    z = np.zeros((2 * r - 1, d))
    got = oracle.halo_attn_ref(np.zeros_like(k), k, v, z, z, block, halo)
    padded_mean = v[0, 0, 0:6, 0:6].sum(axis=(0, 1)) / r ** 2
    assert np.abs(got[0, 0, 0, 0] - padded_mean).max() > 1e-3


# ------------------------------------------- P3 one block covers -> global attention
@pytest.mark.parametrize("H,W,block,halo", [(4, 4, 4, 0), (4, 4, 4, 1), (4, 4, 4, 2), (3, 4, 5, 1), (5, 5, 8, 0)])
def test_p3_single_block_is_global_attention_with_bias(H, W, block, halo):
    d = 4
    q, k, v, rh, rw = case(2, 2, H, W, d, block, halo, seed=21)
    r = block + 2 * halo
    c0 = r - 1 + halo
    scale = d ** -0.5
    got = oracle.halo_attn_ref(q, k, v, rh, rw, block, halo, 1, scale)
    # torch's scaled-dot-product attention over all pixels, fp64, with the
    # relative bias as an additive float mask (logit = scale*(q.k + bias)).
    ys, xs = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    ys, xs = ys.reshape(-1), xs.reshape(-1)
    dy = ys[None, :] - ys[:, None] + c0
    dx = xs[None, :] - xs[:, None] + c0
    for n in range(2):
        for hd in range(2):
            Q = q[n, hd].reshape(-1, d)
            bias = np.einsum("pc,pkc->pk", Q, rh[dy]) + np.einsum("pc,pkc->pk", Q, rw[dx])
            t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
            o = torch.nn.functional.scaled_dot_product_attention(
                t(Q), t(k[n, hd].reshape(-1, d)), t(v[n, hd].reshape(-1, d)),
                attn_mask=t(scale * bias), scale=scale)
            np.testing.assert_allclose(got[n, hd].reshape(-1, d), o[0, 0].numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------ P4 b = 1 -> centred sliding window
@pytest.mark.parametrize("H,W,halo", [(6, 6, 1), (7, 5, 2), (4, 9, 3)])
def test_p4_block_one_is_pixel_centred_window(H, W, halo):
    d = 3
    q, k, v, rh, rw = case(1, 1, H, W, d, 1, halo, seed=31)
    scale = d ** -0.5
    got = oracle.halo_attn_ref(q, k, v, rh, rw, 1, halo, 1, scale)
    for y in range(H):
        for x in range(W):
            qv = q[0, 0, y, x]
            logits, vals = [], []
            for dy in range(-halo, halo + 1):
                for dx in range(-halo, halo + 1):
                    yy, xx = y + dy, x + dx
                    if 0 <= yy < H and 0 <= xx < W:
                        # b = 1: r = 2h+1, table row 3h + displacement
                        logits.append(scale * qv @ (k[0, 0, yy, xx] + rh[3 * halo + dy] + rw[3 * halo + dx]))
                        vals.append(v[0, 0, yy, xx])
            w = torch.softmax(torch.tensor(logits, dtype=torch.float64), 0).numpy()
            np.testing.assert_allclose(got[0, 0, y, x], w @ np.array(vals), rtol=0, atol=1e-13)


# ---------------------------------------------- P5 h = 0 -> block-diagonal attention
@pytest.mark.parametrize("H,W,block", [(8, 8, 4), (6, 9, 3), (7, 7, 4)])
def test_p5_zero_halo_is_attention_within_blocks(H, W, block):
    d = 4
    q, k, v, rh, rw = case(1, 2, H, W, d, block, 0, seed=41)
    scale = d ** -0.5
    got = oracle.halo_attn_ref(q, k, v, rh, rw, block, 0, 1, scale)
    c0 = block - 1
    for by in range(0, H, block):
        for bx in range(0, W, block):
            ys, xs = np.meshgrid(np.arange(by, min(by + block, H)), np.arange(bx, min(bx + block, W)), indexing="ij")
            ys, xs = ys.reshape(-1), xs.reshape(-1)
            for hd in range(2):
                Q, K, V = q[0, hd][ys, xs], k[0, hd][ys, xs], v[0, hd][ys, xs]
                bias = (np.einsum("pc,pkc->pk", Q, rh[ys[None, :] - ys[:, None] + c0])
                        + np.einsum("pc,pkc->pk", Q, rw[xs[None, :] - xs[:, None] + c0]))
                w = torch.softmax(torch.from_numpy(scale * (Q @ K.T + bias)), 1).numpy()
                np.testing.assert_allclose(got[0, hd][ys, xs], w @ V, rtol=0, atol=1e-13)


# ------------------------------------------------- P6 strided = subsampled stride 1
@pytest.mark.parametrize("H,W,block,halo,stride", [(8, 8, 4, 1, 2), (12, 12, 6, 2, 3), (12, 8, 4, 3, 4)])
def test_p6_strided_is_subsampled_stride_one(H, W, block, halo, stride):
    q, k, v, rh, rw = case(1, 2, H, W, 3, block, halo, seed=51)
    full = oracle.halo_attn_ref(q, k, v, rh, rw, block, halo, 1)
    sub = oracle.halo_attn_ref(q, k, v, rh, rw, block, halo, stride)
    np.testing.assert_allclose(sub, full[:, :, ::stride, ::stride], rtol=0, atol=1e-14)


# --------------------------------------------------- P7 normalisation and linearity
def test_p7_constant_values_and_linearity():
    H, W, d, block, halo = 9, 10, 4, 4, 2
    q, k, v1, rh, rw = case(1, 2, H, W, d, block, halo, seed=61)
    v2 = rnd(v1.shape, 62)
    ones = oracle.halo_attn_ref(q, k, np.ones_like(v1), rh, rw, block, halo)
    np.testing.assert_allclose(ones, 1.0, rtol=0, atol=1e-14)
    a = 2.5
    lhs = oracle.halo_attn_ref(q, k, a * v1 + v2, rh, rw, block, halo)
    rhs = a * oracle.halo_attn_ref(q, k, v1, rh, rw, block, halo) + oracle.halo_attn_ref(q, k, v2, rh, rw, block, halo)
    np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-13)


# ------------------------------------------------------------- P8 set semantics
def test_p8_permuting_keys_with_their_biases_is_invariant():
    rng = np.random.default_rng(71)
    d, n = 5, 23
    q, keys, vals, bias = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d)), rng.standard_normal(n)
    base = oracle.set_attention(q, keys, bias, vals, 0.7)
    # direct softmax, written out
    l = 0.7 * (keys @ q + bias)
    w = np.exp(l - l.max()); w /= w.sum()
    np.testing.assert_allclose(base, w @ vals, rtol=0, atol=1e-14)
    for t in range(5):
        p = rng.permutation(n)
        np.testing.assert_allclose(oracle.set_attention(q, keys[p], bias[p], vals[p], 0.7), base, rtol=0, atol=1e-14)
    # negative control: permuting keys but not their biases changes the result
    p = rng.permutation(n)
    assert np.abs(oracle.set_attention(q, keys[p], bias, vals[p], 0.7) - base).max() > 1e-6


def test_p8_large_logits_stay_finite():
    # Stable softmax: logits of several hundred must neither overflow nor lose
    # the answer; the dominant key wins.
    rng = np.random.default_rng(72)
    d, n = 4, 10
    q, keys, vals = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))
    bias = np.zeros(n); bias[3] = 2000.0
    out = oracle.set_attention(q, keys, bias, vals, 1.0)
    np.testing.assert_allclose(out, vals[3], rtol=0, atol=1e-14)
    H = W = 8; block, halo = 4, 1
    qq, kk, vv, rh, rw = case(1, 1, H, W, d, block, halo, seed=73)
    got = oracle.halo_attn_ref(qq * 300, kk, vv, rh, rw, block, halo)
    want = halo_attn_dense(qq * 300, kk, vv, rh, rw, block, halo)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-9)


# ------------------------------------------------------- P9 shifts by b only
def test_p9_equivariant_to_block_shifts_only():
    d, block, halo = 3, 3, 1
    rng = np.random.default_rng(81)
    S = 15
    r = block + 2 * halo
    rh, rw = rng.standard_normal((2 * r - 1, d)), rng.standard_normal((2 * r - 1, d))
    content = rng.standard_normal((3, S, S, d))
    def place(shift):
        canvas = rng.standard_normal((3, S + 6, S + 6, d))
        canvas[:, shift:shift + S, shift:shift + S] = content
        return [c[None, None] for c in canvas]
    base = oracle.halo_attn_ref(*[c[None, None] for c in content], rh, rw, block, halo)
    for shift, equal in ((3, True), (6, True), (1, False), (2, False)):
        shifted = oracle.halo_attn_ref(*place(shift), rh, rw, block, halo)
        # interior blocks of the content: windows inside [0, S)
        diffs = []
        for by in range(1, S // block - 1):
            for bx in range(1, S // block - 1):
                ys = slice(by * block, by * block + block)
                xs = slice(bx * block, bx * block + block)
                ys2 = slice(by * block + shift, by * block + block + shift)
                xs2 = slice(bx * block + shift, bx * block + block + shift)
                diffs.append(np.abs(base[0, 0, ys, xs] - shifted[0, 0, ys2, xs2]).max())
        if equal:
            assert max(diffs) < 1e-13
        else:
            assert max(diffs) > 1e-3


# ---------------------------------------------------- P10 relative-table offset
def skew_rows(l: int, r: int) -> np.ndarray:
    """Relative-to-absolute step described by the HaloAttention module on the
    pswp.cn page (section 4): logits against the 2r-1 table rows, one row per
    block-local query position, get a zero column appended, are flattened,
    padded with (2r-1) - l zeros, viewed as (l+1) rows of 2r-1, and the first
    l rows' last r columns are kept.  Feeding each table row's own index
    through it reveals which row lands at (query position i, window position j)."""
    m = 2 * r - 1
    x = np.tile(np.arange(m, dtype=np.float64), (l, 1))           # x[i, c] = c
    x = np.concatenate([x, np.full((l, 1), -1.0)], axis=1)          # pad column
    flat = np.concatenate([x.reshape(-1), np.full(m - l, -1.0)])
    return flat.reshape(l + 1, m)[:l, -r:].astype(int)


@pytest.mark.parametrize("block,halo", [(4, 1), (8, 3), (12, 3), (2, 1), (3, 2)])
def test_p10_table_offset_follows_the_pages_relative_to_absolute_step(block, halo):
    r = block + 2 * halo
    rows = skew_rows(block, r)
    i, j = np.meshgrid(np.arange(block), np.arange(r), indexing="ij")
    assert (rows >= 0).all(), "skew must never select the padding"
    # query at block-local i is pixel o+i, window position j is pixel o-h+j:
    # displacement (key - query) = j - h - i, so the page's row is that + c0
    c0_page = rows - (j - halo - i)
    assert (c0_page == r - 1 + halo).all()


@pytest.mark.parametrize("block,halo,stride", [(4, 1, 1), (3, 2, 1), (4, 2, 2)])
def test_p10_one_hot_tables_pick_the_displaced_key(block, halo, stride):
    # k = 0 and q = e0: the logits are the table entries alone.  A large value
    # at row c0+delta of rel_h (and c0+eps of rel_w) concentrates the softmax
    # on the key at displacement (delta, eps) whenever that key is in the
    # window and in the image.
    H, W, d = 12, 12, 2
    r = block + 2 * halo
    c0 = r - 1 + halo
    rng = np.random.default_rng(91)
    v = rng.standard_normal((1, 1, H, W, d))
    q = np.zeros((1, 1, H, W, d)); q[..., 0] = 1.0
    k = np.zeros_like(q)
    L = 60.0
    total = 0
    for delta, eps in [(0, 0), (1, -1), (-halo, halo), (block + halo - 1, 0), (0, -(block + halo - 1))]:
        rh = np.zeros((2 * r - 1, d)); rw = np.zeros((2 * r - 1, d))
        rh[c0 + delta, 0] = L
        rw[c0 + eps, 0] = L
        out = oracle.halo_attn_ref(q, k, v, rh, rw, block, halo, stride, 1.0)
        checked = 0
        for yo in range(H // stride):
            for xo in range(W // stride):
                y, x = yo * stride, xo * stride
                ky, kx = y + delta, x + eps
                y0 = (y // block) * block - halo
                x0 = (x // block) * block - halo
                if 0 <= ky < H and 0 <= kx < W and y0 <= ky < y0 + r and x0 <= kx < x0 + r:
                    np.testing.assert_allclose(out[0, 0, yo, xo], v[0, 0, ky, kx], rtol=0, atol=1e-12)
                    checked += 1
        total += checked
        if stride == 1:
            assert checked > 0
    assert total > 0


# ------------------------------------------------------------ P11 axis symmetry
def test_p11_transpose_and_reflection():
    H, W, d, block, halo = 8, 12, 3, 4, 2
    q, k, v, rh, rw = case(1, 2, H, W, d, block, halo, seed=101)
    base = oracle.halo_attn_ref(q, k, v, rh, rw, block, halo)
    T = lambda a: np.ascontiguousarray(np.swapaxes(a, 2, 3))
    tr = oracle.halo_attn_ref(T(q), T(k), T(v), rw, rh, block, halo)
    np.testing.assert_allclose(tr, T(base), rtol=0, atol=1e-13)
    # reverse x (W % block == 0): displacement dx -> -dx, so rel_w mirrors about c0
    r = block + 2 * halo
    c0 = r - 1 + halo
    rw_m = np.zeros_like(rw)
    for row in range(2 * halo, 2 * r - 1):          # rows [2h, 2r-2] are the used ones
        rw_m[row] = rw[2 * c0 - row]
    Rx = lambda a: np.ascontiguousarray(a[:, :, :, ::-1])
    refl = oracle.halo_attn_ref(Rx(q), Rx(k), Rx(v), rh, rw_m, block, halo)
    np.testing.assert_allclose(refl, Rx(base), rtol=0, atol=1e-13)


# ------------------------------------------------ P12 appendix A half-split form
def test_p12_half_split_embedding_is_a_special_case():
    # Appendix A: half of a head's channels carry the height embedding and
    # half the width embedding.  Written out directly and compared with the
    # full-width tables padded by zeros.
    H, W, d, block, halo = 8, 8, 4, 4, 1
    r = block + 2 * halo
    c0 = r - 1 + halo
    q, k, v, _, _ = case(1, 1, H, W, d, block, halo, seed=111)
    rng = np.random.default_rng(112)
    eh, ew = rng.standard_normal((2 * r - 1, d // 2)), rng.standard_normal((2 * r - 1, d // 2))
    rh = np.concatenate([eh, np.zeros_like(eh)], 1)
    rw = np.concatenate([np.zeros_like(ew), ew], 1)
    got = oracle.halo_attn_ref(q, k, v, rh, rw, block, halo, 1, 0.5)
    for y in range(H):
        for x in range(W):
            y0, x0 = (y // block) * block - halo, (x // block) * block - halo
            qv = q[0, 0, y, x]
            logits, vals = [], []
            for ky in range(max(0, y0), min(H, y0 + r)):
                for kx in range(max(0, x0), min(W, x0 + r)):
                    geo = qv[: d // 2] @ eh[ky - y + c0] + qv[d // 2:] @ ew[kx - x + c0]
                    logits.append(0.5 * (qv @ k[0, 0, ky, kx] + geo))
                    vals.append(v[0, 0, ky, kx])
            l = np.array(logits); w = np.exp(l - l.max()); w /= w.sum()
            np.testing.assert_allclose(got[0, 0, y, x], w @ np.array(vals), rtol=0, atol=1e-13)


# --------------------------------------------------------- P13 page geometry
def test_p13_figure1_geometry():
    g = json.load(open(os.path.join(GOLDEN, "fig1_geometry.json")))
    H, W, block, halo = g["H"], g["W"], g["block"], g["halo"]
    assert block + 2 * halo == g["window_side"]
    # one-hot values: d = H*W channels, value of pixel p is e_p; with q = 0 and
    # zero tables the output is the uniform mean over the in-image window, so
    # its support is exactly the window's in-image pixels
    d = H * W
    v = np.eye(d).reshape(1, 1, H, W, d)
    k = np.zeros_like(v); q = np.zeros_like(v)
    r = block + 2 * halo
    z = np.zeros((2 * r - 1, d))
    out = oracle.halo_attn_ref(q, k, v, z, z, block, halo, 1, 1.0)
    assert list(out.shape[2:4]) == g["output_hw"]
    nb = [-(-H // block), -(-W // block)]
    assert nb == g["num_blocks"]
    for blk in g["blocks"]:
        (ry0, ry1), (rx0, rx1) = blk["window_rows"], blk["window_cols"]
        assert ry1 - ry0 + 1 == g["window_side"] and rx1 - rx0 + 1 == g["window_side"]
        expect = np.zeros((H, W), bool)
        expect[max(0, ry0):min(H, ry1 + 1), max(0, rx0):min(W, rx1 + 1)] = True
        for (y, x) in blk["queries"]:
            assert (y // block, x // block) == tuple(blk["block"])
            support = out[0, 0, y, x].reshape(H, W) > 1e-12
            assert (support == expect).all()
            np.testing.assert_allclose(out[0, 0, y, x].sum(), 1.0, atol=1e-14)


def test_p13_layer_demo_shapes():
    g = json.load(open(os.path.join(GOLDEN, "layer_demo_shapes.json")))
    N, C, H, W = g["input_nchw"]
    assert g["heads"] * g["dim_head"] == C
    assert 2 * (g["block"] + 2 * g["halo"]) - 1 == g["rel_table_rows"]
    # shape check on a reduced batch of heads (values are not printed on the page)
    B, heads, Hh, Ww, d = g["per_head_qkv_shape"]
    rng = np.random.default_rng(121)
    small = (1, 1, 8, 8, d)
    q, k, v = (rng.standard_normal(small) for _ in range(3))
    rh = rng.standard_normal((g["rel_table_rows"], d))
    out = oracle.halo_attn_ref(q, k, v, rh, rh, g["block"], g["halo"])
    assert out.shape == small
    assert tuple(g["per_head_out_shape"]) == (B, heads, Hh, Ww, d)


# ------------------------------------------------------------------ edge cases
def test_empty_batch_and_bad_arguments():
    r = 6
    z = np.zeros((2 * r - 1, 4))
    e = np.zeros((0, 2, 8, 8, 4))
    out = oracle.halo_attn_ref(e, e, e, z, z, 4, 1)
    assert out.shape == (0, 2, 8, 8, 4)
    x = np.zeros((1, 1, 8, 8, 4))
    with pytest.raises(ValueError):
        oracle.halo_attn_ref(x, x, x, z, z, 4, 1, 3)        # stride does not divide
    with pytest.raises(ValueError):
        oracle.halo_attn_ref(x, x, x, z[:5], z, 4, 1)       # wrong table length


def test_threads_do_not_change_results():
    q, k, v, rh, rw = case(3, 3, 10, 9, 4, 4, 1, seed=131)
    a = oracle.halo_attn_ref(q, k, v, rh, rw, 4, 1, threads=1)
    b = oracle.halo_attn_ref(q, k, v, rh, rw, 4, 1, threads=4)
    assert np.array_equal(a, b)
