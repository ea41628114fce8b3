"""Pins for the varlen oracle: pad / unpad on a hand-worked example and a
round trip, packed attention against the padded batch (equal lengths) and
against a padded batch with a dense mask that hides the padding (unequal
lengths), the per-sequence block mask against its expansion, and the packed
gradients against central finite differences of the packed forward."""

import numpy as np
import pytest

from oracle import attention_full, dflash_dense_mask, round_multiple
from oracle.blockmask import expand_block_mask
from oracle.varlen import (attention_varlen, attention_varlen_bwd, block_mask_varlen,
                           dflash_varlen_geoms, pad, unpad)


def test_unpad_pad_worked_example():
    x = np.arange(6).reshape(2, 3)
    valid = np.array([[1, 0, 1], [1, 1, 0]], bool)
    packed, idx, cu, mx = unpad(x, valid)
    assert packed.tolist() == [0, 2, 3, 4]
    assert idx.tolist() == [0, 2, 3, 4]
    assert cu.tolist() == [0, 2, 4] and mx == 2
    assert pad(packed, idx, 2, 3).tolist() == [[0, 0, 2], [3, 4, 0]]


def test_unpad_pad_round_trip():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((4, 37, 3, 8))
    valid = rng.random((4, 37)) < 0.6
    valid[2] = False
    packed, idx, cu, mx = unpad(x, valid)
    assert packed.shape == (valid.sum(), 3, 8)
    assert cu[-1] == valid.sum() and mx == valid.sum(axis=1).max()
    np.testing.assert_array_equal(pad(packed, idx, 4, 37), x * valid[:, :, None, None])


def _qkv(total_q, total_k, H, KVH, D, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((total_q, H, D)), rng.standard_normal((total_k, KVH, D)),
            rng.standard_normal((total_k, KVH, D)))


@pytest.mark.parametrize("layer", [dict(), dict(layer_type="sliding", sliding_window=20)])
def test_equal_lengths_match_padded_batch(layer):
    B, bs, NB, C, H, KVH, D = 3, 4, 5, 40, 4, 2, 8
    Sq, Sk = NB * bs, C + NB * bs
    q, k, v = _qkv(B * Sq, B * Sk, H, KVH, D, 1)
    cu_q = np.arange(B + 1) * Sq
    cu_k = np.arange(B + 1) * Sk
    geoms = dflash_varlen_geoms(cu_q, cu_k, bs, **layer)
    o, lse = attention_varlen(q, k, v, cu_q, cu_k, geoms=geoms)
    wo, wl = attention_full(q.reshape(B, Sq, H, D), k.reshape(B, Sk, KVH, D),
                            v.reshape(B, Sk, KVH, D), mask=geoms[0])
    np.testing.assert_allclose(o.reshape(B, Sq, H, D), wo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse.reshape(H, B, Sq).transpose(1, 0, 2), wl, rtol=0, atol=1e-12)
    o2, _ = attention_varlen(q, k, v, cu_q, cu_k)
    wo2, _ = attention_full(q.reshape(B, Sq, H, D), k.reshape(B, Sk, KVH, D),
                            v.reshape(B, Sk, KVH, D))
    np.testing.assert_allclose(o2.reshape(B, Sq, H, D), wo2, rtol=0, atol=1e-12)


def test_unequal_lengths_match_masked_padded_batch():
    """Each sequence padded to the longest, the padding hidden by a dense mask."""
    bs, H, KVH, D = 4, 2, 1, 8
    ctx = [30, 0, 70]
    nb = [3, 2, 1]
    sq = [n * bs for n in nb]
    sk = [c + s for c, s in zip(ctx, sq)]
    cu_q = np.r_[0, np.cumsum(sq)]
    cu_k = np.r_[0, np.cumsum(sk)]
    q, k, v = _qkv(cu_q[-1], cu_k[-1], H, KVH, D, 2)
    geoms = dflash_varlen_geoms(cu_q, cu_k, bs, is_causal=True, layer_type="sliding",
                                sliding_window=25)
    o, lse = attention_varlen(q, k, v, cu_q, cu_k, geoms=geoms)
    B, Mq, Mk = 3, max(sq), max(sk)
    Kr = round_multiple(Mk, 128)
    qp = np.zeros((B, Mq, H, D))
    kp = np.zeros((B, Mk, KVH, D))
    vp = np.zeros((B, Mk, KVH, D))
    mask = np.zeros((B, 1, Mq, Kr), bool)
    for b in range(B):
        qp[b, :sq[b]] = q[cu_q[b]:cu_q[b + 1]]
        kp[b, :sk[b]] = k[cu_k[b]:cu_k[b + 1]]
        vp[b, :sk[b]] = v[cu_k[b]:cu_k[b + 1]]
        mask[b, 0, :sq[b], :sk[b]] = dflash_dense_mask(geoms[b])[:, :sk[b]]
    wo, wl = attention_full(qp, kp, vp, mask=mask)
    for b in range(B):
        np.testing.assert_allclose(o[cu_q[b]:cu_q[b + 1]], wo[b, :sq[b]], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[:, cu_q[b]:cu_q[b + 1]], wl[b, :, :sq[b]], rtol=0,
                                   atol=1e-12)


def test_block_mask_varlen_expands_to_each_sequence():
    bs = 16
    sq = [32, 0, 160, 16]
    ctx = [100, 0, 300, 500]
    cu_q = np.r_[0, np.cumsum(sq)]
    cu_k = np.r_[0, np.cumsum([c + s for c, s in zip(ctx, sq)])]
    geoms = dflash_varlen_geoms(cu_q, cu_k, bs, layer_type="sliding", sliding_window=150)
    kv_num, kv_idx, full_num, full_idx = block_mask_varlen(geoms)
    assert kv_num.shape == (4, 1, 2) and kv_idx.shape == (4, 1, 2, 5)  # 516 keys: 5 tiles
    for b, g in enumerate(geoms):
        nq = -(-g.Sq // 128)
        nk = -(-g.Sk // 128)
        assert (kv_num[b, 0, nq:] == 0).all() and (full_num[b, 0, nq:] == 0).all()
        assert (kv_idx[b, 0, :, nk:] == -1).all()
        if g.Sq == 0:
            continue
        dense = dflash_dense_mask(g)
        dense[:, g.Sk:] = False
        Kr = dense.shape[1]
        got = expand_block_mask(kv_num[b:b + 1, :, :nq], kv_idx[b:b + 1, :, :nq, :Kr // 128],
                                full_num[b:b + 1, :, :nq], full_idx[b:b + 1, :, :nq, :Kr // 128],
                                dense[None, None], g.Sq)
        np.testing.assert_array_equal(got[0, 0], dense)


def test_geoms_reject_non_dflash_lengths():
    with pytest.raises(ValueError):
        dflash_varlen_geoms([0, 10], [0, 30], 4)   # 10 queries, blocks of 4
    with pytest.raises(ValueError):
        dflash_varlen_geoms([0, 8], [0, 4], 4)     # fewer keys than queries


def _fd(fn, x, eps=1e-6):
    g = np.zeros_like(x)
    for i in np.ndindex(x.shape):
        old = x[i]
        x[i] = old + eps
        lp = fn()
        x[i] = old - eps
        lm = fn()
        x[i] = old
        g[i] = (lp - lm) / (2 * eps)
    return g


@pytest.mark.parametrize("layer", [dict(is_causal=True),
                                   dict(is_causal=False, layer_type="sliding",
                                        sliding_window=3)])
def test_varlen_grads_match_finite_differences(layer):
    """Three sequences, the middle one keys without queries: every gradient,
    including the middle sequence's zero dK / dV, against finite differences
    of the packed forward's loss sum(O * dO)."""
    bs, H, KVH, D = 2, 2, 1, 3
    cu_q = np.array([0, 4, 4, 6])
    cu_k = np.array([0, 10, 15, 21])
    q, k, v = _qkv(6, 21, H, KVH, D, 5)
    dout = np.random.default_rng(6).standard_normal((6, H, D))
    geoms = dflash_varlen_geoms(cu_q, cu_k, bs, **layer)
    scale = 0.7

    def loss():
        o, _ = attention_varlen(q, k, v, cu_q, cu_k, scale=scale, geoms=geoms)
        return float((o * dout).sum())

    dq, dk, dv = attention_varlen_bwd(q, k, v, dout, cu_q, cu_k, scale=scale, geoms=geoms)
    np.testing.assert_allclose(dq, _fd(loss, q), rtol=0, atol=1e-7)
    np.testing.assert_allclose(dk, _fd(loss, k), rtol=0, atol=1e-7)
    np.testing.assert_allclose(dv, _fd(loss, v), rtol=0, atol=1e-7)
    assert not dk[10:15].any() and not dv[10:15].any()
    assert np.abs(dk[:10]).max() > 1e-3 and np.abs(dv[15:]).max() > 1e-3
