"""GPU parity: dynamic top-k keep masks, bit-exact against the CPU oracle."""

import numpy as np
import pytest
import torch

from gpu_helpers import bsm, oracle, say, synth

pytestmark = pytest.mark.gpu


def _oracle(bias, premask, Sk, k, dt):
    pm = None if premask is None else premask.cpu().numpy()
    return oracle.topk_keep_mask(synth.as_f64(bias), pm, Sk, k, dt)


def _check(bias, premask, Sk, k, dt, what):
    say("topk", what, tuple(bias.shape), Sk, k, dt)
    got = bsm.dynamic_topk_mask(bias.cuda(), None if premask is None else premask.cuda(), Sk, k)
    want = _oracle(bias, premask, Sk, k, dt)
    g = got.cpu().numpy()
    if not np.array_equal(g, want):
        bad = np.argwhere(g != want)
        raise AssertionError(f"{what}: {len(bad)} mismatches, first {bad[:5].tolist()}")


def test_dynamic_topk_config():
    """Dynamic-mask workload: bias (2,4,1,8064) bf16, 2D padding mask, k=2048."""
    cfg = synth.CONFIGS["dynamic_topk_bf16"]
    bias, pad2d = synth.topk_inputs(cfg, seed=0)
    B, Sk = cfg["B"], cfg["Sk"]
    got = bsm.create_mask(bias.cuda(), pad2d.cuda(), B, cfg["Sq"], Sk, cfg["topk"])
    want = oracle.topk_keep_mask(synth.as_f64(bias), oracle.normalize_premask(pad2d.numpy(), B, Sk),
                                 Sk, cfg["topk"], "bf16")
    np.testing.assert_array_equal(got.cpu().numpy(), want)
    assert (got.sum(-1).cpu() == 2048).all()


def test_decode_topk_config():
    """Decode workload: bias (64,32,1,16384) bf16, k=1024 per row."""
    cfg = synth.CONFIGS["decode_swap_bf16"]
    bias, _ = synth.topk_inputs(cfg, seed=0)
    _check(bias, None, cfg["Sk"], cfg["topk"], "bf16", "decode")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("Sk,k", [(128, 0), (128, 1), (128, 128), (128, 500), (1000, 7),
                                  (1000, 999), (1000, 1000), (3000, 1500), (300, 64)])
def test_topk_small(dt, Sk, k):
    kr = bsm.round_multiple(Sk)
    bias = synth.normal_tensor((2, 3, 2, kr), 1, synth.TID_BIAS, dt)
    pm = torch.from_numpy(synth.random_bool((2, 1, 2, Sk), 0.8, 1, synth.TID_MASK))
    _check(bias, None, Sk, k, dt, "plain")
    _check(bias, pm, Sk, k, dt, "premask")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_topk_ties_and_special_values(dt):
    """Heavy ties (a few distinct levels), signed zeros, -inf and the sentinel."""
    rng = np.random.default_rng(5)
    K = 1024
    x = (rng.integers(-3, 4, size=(4, 1, 3, K)) / 4).astype(np.float32)
    x[0, 0, 0, :50] = -0.0
    x[1, 0, 1, 10:20] = -np.inf
    x[2, 0, 2, 5:9] = oracle.finfo_min(dt)
    bias = synth.storage(x, dt)
    pm = torch.from_numpy(rng.random((4, 1, 1, K)) < 0.7)
    for k in (1, 3, 100, 700, 1023):
        _check(bias, None, 1000, k, dt, "ties")
        _check(bias, pm, 1000, k, dt, "ties+premask")


def test_topk_premask_broadcast_and_fully_masked_rows():
    bias = synth.normal_tensor((3, 2, 4, 256), 2, synth.TID_BIAS, "bf16")
    pm = torch.ones((1, 2, 4, 256), dtype=torch.bool)
    pm[0, 1, 2] = False  # a fully pre-masked row keeps nothing
    _check(bias, pm, 256, 30, "bf16", "bcast")
    got = bsm.dynamic_topk_mask(bias.cuda(), pm.cuda(), 256, 30).cpu()
    assert not got[:, 1, 2].any()


@pytest.mark.parametrize("dt,K", [("f32", 20480), ("bf16", 40960)])
def test_topk_rows_beyond_lds(dt, K):
    """Rows too long to keep in LDS take the re-reading path."""
    bias = synth.normal_tensor((1, 2, 1, K), 3, synth.TID_BIAS, dt)
    _check(bias, None, K - 5, 3000, dt, "long")
