"""Pins for the kept-key list oracle.

Checked against: a hand-worked 3-row example, the round trip (a key list
expanded back equals the dense mask with keys >= Sk cleared), ordering and
union-count properties, the top-k count invariant (the bits of a list built
from a top-k mask hold exactly min(k, #valid) keys per row), and attention
over the gathered keys with the per-row bits equal to attention over the
dense mask.
"""

import numpy as np
import pytest

from oracle import attention_rows, topk_keep_mask
from oracle.keylist import expand_key_list, key_list


def test_hand_worked_example():
    # 3 rows, 128 keys, Sk = 10: row 0 keeps {1, 4}, row 1 keeps {4, 7, 12},
    # row 2 keeps nothing; key 12 >= Sk is dropped.
    m = np.zeros((1, 1, 3, 128), bool)
    m[0, 0, 0, [1, 4]] = True
    m[0, 0, 1, [4, 7, 12]] = True
    num, keys, bits = key_list(m, 10, 3)
    assert num.tolist() == [[3]]
    assert keys[0, 0, :3].tolist() == [1, 4, 7]
    assert bits[0, 0, :3].tolist() == [0b001, 0b011, 0b010]
    assert (keys[0, 0, 3:] == -1).all() and (bits[0, 0, 3:] == 0).all()


def _random_mask(shape, density, seed):
    rng = np.random.default_rng(seed)
    return rng.random(shape) < density


@pytest.mark.parametrize("shape,rows,Sk", [
    ((2, 3, 4, 256), 4, 256),
    ((2, 3, 4, 256), 4, 200),
    ((1, 2, 1, 384), 5, 300),     # query dim broadcast: every row the same
    ((3, 1, 32, 128), 32, 128),   # 32 rows, the largest row count
    ((1, 1, 1, 128), 1, 0),       # no keys at all
])
def test_round_trip(shape, rows, Sk):
    m = _random_mask(shape, 0.1, sum(shape) + rows)
    num, keys, bits = key_list(m, Sk, rows)
    want = np.broadcast_to(m, shape[:2] + (rows, shape[3])).copy()
    want[..., Sk:] = False
    np.testing.assert_array_equal(expand_key_list(num, keys, bits, rows, shape[3]), want)


def test_order_and_union():
    m = _random_mask((2, 2, 6, 512), 0.05, 7)
    num, keys, bits = key_list(m, 500, 6)
    for b in range(2):
        for h in range(2):
            n = num[b, h]
            listed = keys[b, h, :n]
            assert (np.diff(listed) > 0).all()
            assert n == int(m[b, h, :, :500].any(axis=0).sum())
            assert (bits[b, h, :n] > 0).all() and (bits[b, h, :n] < 2 ** 6).all()


def test_topk_rows_keep_k_keys():
    rng = np.random.default_rng(4)
    B, R, Sk, k = 2, 4, 300, 40
    K = 384
    bias = rng.standard_normal((B, 1, R, K))
    valid = rng.random((B, 1, 1, Sk)) < 0.9
    keep = topk_keep_mask(bias, valid, Sk, k, "f32")
    num, keys, bits = key_list(keep, Sk, R)
    for b in range(B):
        per_row = [sum((int(w) >> r) & 1 for w in bits[b, 0, :num[b, 0]]) for r in range(R)]
        assert per_row == [min(k, int(valid[b, 0, 0].sum()))] * R
        assert num[b, 0] <= R * k


def test_attention_over_gathered_keys():
    """Attention with the dense mask equals attention over only the listed
    keys, each row masked by its bit."""
    rng = np.random.default_rng(5)
    B, Sq, Sk, H, D = 1, 6, 200, 1, 16
    q = rng.standard_normal((B, Sq, H, D))
    k = rng.standard_normal((B, Sk, H, D))
    v = rng.standard_normal((B, Sk, H, D))
    m = _random_mask((1, 1, Sq, 256), 0.08, 6)
    m[0, 0, 2] = False  # a row with no kept key
    want_o, want_l = attention_rows(q, k, v, 0, 0, np.arange(Sq), mask=m)
    num, keys, bits = key_list(m, Sk, Sq)
    n = num[0, 0]
    kg = k[:, keys[0, 0, :n]]
    vg = v[:, keys[0, 0, :n]]
    mg = np.zeros((1, 1, Sq, n), bool)
    for r in range(Sq):
        mg[0, 0, r] = (bits[0, 0, :n].astype(np.int64) >> r) & 1 == 1
    got_o, got_l = attention_rows(q, kg, vg, 0, 0, np.arange(Sq), mask=mg)
    np.testing.assert_allclose(got_o, want_o, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(got_l), np.isneginf(want_l))
    fin = ~np.isneginf(want_l)
    np.testing.assert_allclose(got_l[fin], want_l[fin], rtol=0, atol=1e-12)


def test_rejects_bad_rows():
    m = np.zeros((1, 1, 3, 128), bool)
    with pytest.raises(ValueError):
        key_list(m, 128, 4)
    with pytest.raises(ValueError):
        key_list(np.zeros((1, 1, 33, 128), bool), 128, 33)
