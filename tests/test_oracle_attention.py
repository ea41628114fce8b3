"""Pins for the float64 attention oracle.

Checked against: torch's scaled_dot_product_attention on the CPU in float64
(an independent library routine) with and without boolean/additive masks,
logsumexp, the fully-masked-row invariant, single-key rows, convexity of the
output, GQA == repeated KV heads, stride-0 broadcast == materialised expand,
and the DFlash predicate == its dense mask.
"""

import math

import numpy as np
import torch
import torch.nn.functional as F

from oracle import DFlashGeom, attention_full, attention_rows, dflash_dense_mask


def _qkv(B, Sq, Sk, H, KVH, D, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Sq, H, D))
    k = rng.standard_normal((B, Sk, KVH, D))
    v = rng.standard_normal((B, Sk, KVH, D))
    return q, k, v


def _sdpa(q, k, v, scale, attn_mask=None):
    """torch SDPA in float64 with KV heads repeated; returns (B, Sq, H, D)."""
    H, KVH = q.shape[2], k.shape[2]
    G = H // KVH
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    am = None if attn_mask is None else torch.from_numpy(attn_mask)
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=am, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def test_unmasked_matches_sdpa():
    q, k, v = _qkv(2, 37, 53, 4, 2, 16, 0)
    O, lse = attention_full(q, k, v)
    np.testing.assert_allclose(O, _sdpa(q, k, v, 1 / 4), rtol=1e-12, atol=1e-12)
    # LSE against logsumexp of the scores
    s = np.einsum("bqhd,bkhd->bhqk", q, np.repeat(k, 2, axis=2)) / 4
    np.testing.assert_allclose(lse, torch.logsumexp(torch.from_numpy(s), -1).numpy(), rtol=1e-12)


def test_all_keep_mask_equals_unmasked():
    q, k, v = _qkv(1, 20, 30, 2, 2, 8, 1)
    keep = np.ones((1, 1, 1, 128), bool)
    O1, l1 = attention_full(q, k, v, mask=keep)
    O2, l2 = attention_full(q, k, v)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(l1, l2)


def test_mask_and_bias_match_sdpa():
    B, Sq, Sk, H, KVH, D = 2, 33, 70, 6, 3, 16
    q, k, v = _qkv(B, Sq, Sk, H, KVH, D, 2)
    rng = np.random.default_rng(9)
    mask = rng.random((B, H, Sq, 128)) < 0.5
    mask[..., 0] = True  # no fully masked row: SDPA would give NaN there
    bias = rng.standard_normal((B, KVH, 1, 128))
    O, _ = attention_full(q, k, v, scale=0.3, mask=mask, bias=bias)
    G = H // KVH
    add = np.where(mask[..., :Sk], np.repeat(bias, G, axis=1)[..., :Sk], -np.inf)
    np.testing.assert_allclose(O, _sdpa(q, k, v, 0.3, add), rtol=1e-11, atol=1e-12)


def test_fully_masked_row_is_zero():
    q, k, v = _qkv(1, 4, 10, 1, 1, 8, 3)
    mask = np.ones((1, 1, 4, 128), bool)
    mask[0, 0, 2] = False
    O, lse = attention_full(q, k, v, mask=mask)
    assert (O[0, 2, 0] == 0).all() and lse[0, 0, 2] == -np.inf
    assert np.isfinite(lse[0, 0, [0, 1, 3]]).all()


def test_single_key_returns_that_value_row():
    q, k, v = _qkv(1, 3, 10, 2, 1, 8, 4)
    mask = np.zeros((1, 1, 3, 128), bool)
    mask[0, 0, 0, 7] = mask[0, 0, 1, 0] = mask[0, 0, 2, 9] = True
    O, _ = attention_full(q, k, v, mask=mask)
    for r, j in [(0, 7), (1, 0), (2, 9)]:
        np.testing.assert_array_equal(O[0, r, 0], v[0, j, 0])
        np.testing.assert_array_equal(O[0, r, 1], v[0, j, 0])


def test_output_is_convex_combination():
    q, k, v = _qkv(1, 16, 40, 2, 2, 8, 5)
    rng = np.random.default_rng(1)
    mask = rng.random((1, 2, 16, 128)) < 0.4
    mask[..., 3] = True
    O, _ = attention_full(q, k, v, mask=mask)
    for h in range(2):
        for r in range(16):
            sel = mask[0, h, r, :40]
            lo, hi = v[0, sel, h].min(0), v[0, sel, h].max(0)
            assert (O[0, r, h] >= lo - 1e-12).all() and (O[0, r, h] <= hi + 1e-12).all()


def test_gqa_equals_repeated_kv_heads():
    q, k, v = _qkv(1, 12, 20, 8, 2, 8, 6)
    O1, l1 = attention_full(q, k, v)
    O2, l2 = attention_full(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2))
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(l1, l2)


def test_broadcast_equals_expand():
    B, Sq, Sk, H, KVH = 2, 9, 140, 4, 2
    q, k, v = _qkv(B, Sq, Sk, H, KVH, 8, 7)
    rng = np.random.default_rng(2)
    mask = rng.random((B, 1, 1, 256)) < 0.7
    bias = rng.standard_normal((1, KVH, 1, 256))
    O1, l1 = attention_full(q, k, v, mask=mask, bias=bias)
    mx = np.broadcast_to(mask, (B, H, Sq, 256))
    bx = np.repeat(np.broadcast_to(bias, (B, KVH, Sq, 256)), H // KVH, axis=1)
    O2, l2 = attention_full(q, k, v, mask=mx, bias=bx)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(l1, l2)


def test_dflash_geom_equals_its_dense_mask():
    g = DFlashGeom(64, 4, 8, layer_type="sliding", sliding_window=20)
    q, k, v = _qkv(1, g.Sq, g.Sk, 2, 1, 8, 8)
    O1, l1 = attention_full(q, k, v, mask=g)
    d = dflash_dense_mask(g)[None, None]
    O2, l2 = attention_full(q, k, v, mask=d)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(l1, l2)


def test_rows_subset_matches_full():
    q, k, v = _qkv(2, 30, 25, 2, 1, 8, 9)
    O, lse = attention_full(q, k, v, scale=0.5)
    Or, lr = attention_rows(q, k, v, 1, 1, [3, 17, 29], scale=0.5)
    np.testing.assert_array_equal(Or, O[1, [3, 17, 29], 1])
    np.testing.assert_array_equal(lr, lse[1, 1, [3, 17, 29]])
    assert math.isclose(1 / math.sqrt(8), 0.3535533905932738)


# ---------------------------------------------------------------------------
# Huge and infinite biases (readings: finite biases saturate at
# +-FLT_MAX / log2 e, -inf stays -inf and drops the key)

BF16_MIN = -(2.0 - 2.0 ** -7) * 2.0 ** 127   # finfo(bf16).min, from the format


def _one_row(bias_row, kept_row, seed=3):
    Sk = len(bias_row)
    q, k, v = _qkv(1, 1, Sk, 1, 1, 8, seed)
    K = 128 * ((Sk + 127) // 128)
    bias = np.zeros((1, 1, 1, K))
    bias[0, 0, 0, :Sk] = bias_row
    mask = np.zeros((1, 1, 1, K), bool)
    mask[0, 0, 0, :Sk] = kept_row
    O, L = attention_rows(q, k, v, 0, 0, [0], mask=mask, bias=bias)
    return O[0], L[0], v[0, :, 0, :]


def test_sentinel_on_every_kept_key_weighs_them_equally():
    """Every kept key carries finfo(bf16).min: the scores all equal -BIAS_BOUND
    (the dot products vanish beside it), so O is the plain mean of their V rows
    and LSE = -BIAS_BOUND (log of the key count vanishes too)."""
    from oracle.attention import BIAS_BOUND
    kept = np.array([1, 0, 1, 1, 0, 1], bool)
    O, L, V = _one_row(np.full(6, BF16_MIN), kept)
    np.testing.assert_allclose(O, V[kept].mean(axis=0), rtol=0, atol=1e-12)
    assert L == -BIAS_BOUND


def test_sentinel_beside_an_ordinary_key_weighs_nothing():
    O, L, V = _one_row(np.array([BF16_MIN, 0.25, BF16_MIN]), np.ones(3, bool))
    np.testing.assert_allclose(O, V[1], rtol=0, atol=1e-12)


def test_values_beyond_the_bound_saturate_to_one_score():
    """-3e38 and -2.4e38 are both beyond FLT_MAX / log2 e: equal weights;
    -2e38 and -1e38 are not: the larger wins outright."""
    O, _, V = _one_row(np.array([-3.0e38, -2.4e38]), np.ones(2, bool))
    np.testing.assert_allclose(O, V.mean(axis=0), rtol=0, atol=1e-12)
    O, _, V = _one_row(np.array([-2.0e38, -1.0e38]), np.ones(2, bool))
    np.testing.assert_allclose(O, V[1], rtol=0, atol=1e-12)


def test_minus_inf_bias_drops_the_key():
    bias = np.array([0.5, -np.inf, -1.0, 0.0])
    O, L, _ = _one_row(bias, np.ones(4, bool))
    O2, L2, _ = _one_row(np.where(np.isinf(bias), 0.0, bias), np.array([1, 0, 1, 1], bool))
    np.testing.assert_allclose(O, O2, rtol=0, atol=1e-14)
    assert abs(L - L2) < 1e-14
    O, L, _ = _one_row(np.full(3, -np.inf), np.ones(3, bool))
    assert (O == 0).all() and L == -np.inf
