"""Pins for the top-k oracle and the pre-mask normalisation.

Checked against: the O(K^2) rank definition on tiny rows, the kept-count
invariants (exactly min(k, #valid) kept per row; pre-masked keys never kept),
argmax and constant-row special cases, torch.topk where the cut has no tie,
the formats' minimum finite values, and the 128-rounding rule of the pages.
"""

import numpy as np
import pytest
import torch

from oracle import finfo_min, normalize_premask, round_multiple, topk_keep_mask, topk_rank_bruteforce


def test_finfo_min_matches_torch():
    assert finfo_min("bf16") == float(torch.finfo(torch.bfloat16).min)
    assert finfo_min("f32") == float(torch.finfo(torch.float32).min)


def test_round_multiple():
    # (x + m - 1) / m * m, e.g. 8000 keys pad to 8064
    assert [round_multiple(x, 128) for x in (0, 1, 127, 128, 129, 8000, 16384, 65536)] == \
        [0, 128, 128, 128, 256, 8064, 16384, 65536]


def _bf16_values(n, rng, levels=None):
    if levels is not None:
        x = rng.integers(-levels, levels + 1, size=n).astype(np.float32) / 4
    else:
        x = rng.standard_normal(n).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("seed", range(6))
def test_rank_definition_tiny_rows(seed):
    rng = np.random.default_rng(seed)
    K = 40
    for levels in (None, 3, 0):
        x = _bf16_values(K, rng, levels)
        x[rng.integers(K)] = -0.0
        x[rng.integers(K)] = 0.0
        if seed % 2:
            x[rng.integers(K)] = -np.inf
        valid = rng.random(K) < 0.8
        for k in (0, 1, 5, 17, 39, 40, 60):
            got = topk_keep_mask(x[None, None, None, :], valid[None, None, None, :],
                                 K, k, "bf16")[0, 0, 0]
            want = topk_rank_bruteforce(x, valid, k, "bf16")
            np.testing.assert_array_equal(got, want)


def test_kept_count_and_premask():
    rng = np.random.default_rng(3)
    B, H, Q, Sk = 2, 3, 2, 300
    K = round_multiple(Sk, 128)
    bias = _bf16_values(B * H * Q * K, rng).reshape(B, H, Q, K)
    pm = rng.random((B, 1, 1, Sk)) < 0.6
    for k in (0, 1, 50, 170, 400):
        keep = topk_keep_mask(bias, pm, Sk, k, "bf16")
        valid = np.zeros((B, H, Q, K), bool)
        valid[..., :Sk] = np.broadcast_to(pm, (B, H, Q, Sk))
        assert not (keep & ~valid).any()
        np.testing.assert_array_equal(keep.sum(-1), np.minimum(k, valid.sum(-1)))
        if k >= K:
            np.testing.assert_array_equal(keep, valid)


def test_fully_premasked_row_keeps_nothing():
    bias = np.ones((1, 1, 1, 128))
    pm = np.zeros((1, 1, 1, 128), bool)
    assert not topk_keep_mask(bias, pm, 128, 10, "f32").any()


def test_k1_is_argmax_lowest_index():
    rng = np.random.default_rng(5)
    for _ in range(20):
        x = _bf16_values(256, rng, levels=2)
        keep = topk_keep_mask(x[None, None, None], None, 256, 1, "bf16")[0, 0, 0]
        assert keep.sum() == 1 and np.nonzero(keep)[0][0] == int(np.argmax(x))


def test_constant_row_keeps_first_valid():
    x = np.full(256, 0.5)
    valid = np.ones(256, bool)
    valid[[0, 3, 10]] = False
    keep = topk_keep_mask(x[None, None, None], valid[None, None, None], 200, 7, "bf16")[0, 0, 0]
    want = np.zeros(256, bool)
    want[[1, 2, 4, 5, 6, 7, 8]] = True
    np.testing.assert_array_equal(keep, want)


def test_minus_inf_valid_ranks_below_sentinel():
    # valid keys with bias -inf lose to pre-masked keys (set to finfo.min)
    x = np.array([-np.inf, -np.inf, 1.0] + [0.0] * 125)
    valid = np.ones(128, bool)
    valid[3:] = False
    keep = topk_keep_mask(x[None, None, None], valid[None, None, None], 128, 3, "f32")[0, 0, 0]
    # selection = key 2 then two sentinel keys (3, 4); AND valid leaves key 2
    assert np.nonzero(keep)[0].tolist() == [2]


def test_agrees_with_torch_topk_without_ties():
    rng = np.random.default_rng(11)
    K = 1000
    for k in (1, 10, 333, 999):
        x = rng.permutation(K).astype(np.float64)  # distinct values: no tie
        keep = topk_keep_mask(x[None, None, None], None, K, k, "f32")[0, 0, 0]
        idx = torch.topk(torch.from_numpy(x), k, sorted=False).indices.numpy()
        want = np.zeros(K, bool)
        want[idx] = True
        np.testing.assert_array_equal(keep[:K], want)


def test_tail_is_invalid():
    x = np.zeros(256)
    x[200:] = 100.0  # large values beyond seqlen_k must not be chosen
    keep = topk_keep_mask(x[None, None, None], None, 200, 10, "bf16")[0, 0, 0]
    assert keep[:10].all() and keep.sum() == 10


def test_normalize_premask_2d_and_4d():
    m2 = np.array([[1, 1, 0], [1, 0, 1]], bool)
    out = normalize_premask(m2, 2, 3)
    assert out.shape == (2, 1, 1, 128)
    np.testing.assert_array_equal(out[:, 0, 0, :3], m2)
    assert not out[..., 3:].any()
    m4 = np.ones((1, 4, 1, 3), bool)
    assert normalize_premask(m4, 2, 3).shape == (1, 4, 1, 128)
    with pytest.raises(ValueError):
        normalize_premask(np.ones((2, 5), bool), 2, 3)


def test_signed_zeros_tie_by_index():
    # -0 and +0 are the same real number: the lower index wins the tie
    x = np.zeros(128)
    x[0] = -0.0
    x[1] = 0.0
    x[2:] = -1.0
    keep = topk_keep_mask(x[None, None, None], None, 128, 1, "bf16")[0, 0, 0]
    assert np.nonzero(keep)[0].tolist() == [0]
    x[0], x[1] = 0.0, -0.0
    keep = topk_keep_mask(x[None, None, None], None, 128, 1, "bf16")[0, 0, 0]
    assert np.nonzero(keep)[0].tolist() == [0]
