"""GPU parity: block masks (DFlash predicate and dense) and the dense DFlash mask,
bit-exact against the CPU oracle."""

import numpy as np
import pytest
import torch

from gpu_helpers import assert_bm_equal, bsm, np_bm, oracle, oracle_geom, say, synth

pytestmark = pytest.mark.gpu

DFLASH_CASES = [
    dict(ctx_len=256, num_blocks=4, block_size=16),
    dict(ctx_len=260, num_blocks=13, block_size=16),
    dict(ctx_len=260, num_blocks=13, block_size=16, is_causal=True),
    dict(ctx_len=260, num_blocks=13, block_size=16, layer_type="sliding", sliding_window=100),
    dict(ctx_len=260, num_blocks=13, block_size=16, is_causal=False, layer_type="sliding",
         sliding_window=37),
    dict(ctx_len=512, num_blocks=16, block_size=16, ctx_end_offset=-40),
    dict(ctx_len=512, num_blocks=16, block_size=16, ctx_end_offset=50, is_causal=True,
         layer_type="sliding", sliding_window=200),
    dict(ctx_len=300, num_blocks=10, block_size=8, ctx_per_block=40),
    dict(ctx_len=999, num_blocks=3, block_size=200, layer_type="sliding", sliding_window=150),
    dict(ctx_len=0, num_blocks=5, block_size=64, is_causal=True),
    dict(ctx_len=200, num_blocks=1, block_size=1),
    dict(ctx_len=4096, num_blocks=256, block_size=16),
    dict(ctx_len=4096, num_blocks=256, block_size=16, layer_type="sliding", sliding_window=2048),
]


def _id(c):
    return "-".join(f"{k}{v}" for k, v in c.items())


@pytest.mark.parametrize("case", DFLASH_CASES, ids=[_id(c) for c in DFLASH_CASES])
def test_pred_block_mask(case):
    d = bsm.DFlash(**case)
    say("pred block mask", case)
    geom = (1, 4, 2, d.Sq, d.Sk, 64)
    got = np_bm(bsm.build_block_mask(geom, pred=d))
    og = oracle_geom(d)
    want = oracle.classify_tiles(oracle.dflash_dense_mask(og)[None, None], og.Sk)
    assert_bm_equal(got, want, str(case))


@pytest.mark.parametrize("case", DFLASH_CASES[:11], ids=[_id(c) for c in DFLASH_CASES[:11]])
def test_dense_dflash_mask_and_dense_builder(case):
    d = bsm.DFlash(**case)
    say("dense dflash", case)
    geom = (1, 4, 2, d.Sq, d.Sk, 64)
    dense = bsm.dflash_dense_mask(geom, d)
    og = oracle_geom(d)
    want = oracle.dflash_dense_mask(og)
    np.testing.assert_array_equal(dense.cpu().numpy(), want)
    got = np_bm(bsm.build_block_mask(geom, mask=dense[None, None]))
    assert_bm_equal(got, np_bm(bsm.build_block_mask(geom, pred=d)), "dense vs pred")


def test_long_context_dense_stand_in():
    """The 2 GiB (1,1,32768,65536) dense form of the long-context mask: the dense
    builder gives exactly the predicate builder's block mask."""
    d = bsm.DFlash(32768, 2048, 16, is_causal=True, layer_type="sliding", sliding_window=4096)
    geom = (1, 32, 8, d.Sq, d.Sk, 128)
    dense = bsm.dflash_dense_mask(geom, d)
    og = oracle_geom(d)
    for t in [0, 77, 255]:
        rows = np.arange(128 * t, 128 * t + 128)
        np.testing.assert_array_equal(dense[128 * t:128 * t + 128].cpu().numpy(),
                                      oracle.dflash_dense_mask(og, rows))
    got = np_bm(bsm.build_block_mask(geom, mask=dense[None, None]))
    del dense
    assert_bm_equal(got, np_bm(bsm.build_block_mask(geom, pred=d)), "dense vs pred")


def _random_tiles(shape, Sk, seed):
    """Bool mask with per-tile structure: empty, full or random tiles."""
    rng = np.random.default_rng(seed)
    Bm, Hm, Qm, K = shape
    m = np.zeros(shape, bool)
    for b in range(Bm):
        for h in range(Hm):
            for qt in range((Qm + 127) // 128):
                for kt in range(K // 128):
                    kind = rng.integers(4)
                    blk = m[b, h, qt * 128:qt * 128 + 128, kt * 128:kt * 128 + 128]
                    if kind == 1:
                        blk[:] = True
                    elif kind == 2:
                        blk[:] = rng.random(blk.shape) < 0.5
                    elif kind == 3:
                        blk[rng.integers(blk.shape[0]), rng.integers(128)] = True
    # garbage past Sk must be ignored
    m[..., Sk:] = rng.random(m[..., Sk:].shape) < 0.5
    return m


DENSE_CASES = [
    # (geometry B,H,KVH,Sq,Sk,D), mask shape
    ((2, 6, 3, 300, 600, 64), (2, 3, 300, 640)),
    ((2, 6, 3, 300, 600, 64), (1, 6, 1, 640)),
    ((2, 6, 3, 300, 600, 64), (2, 1, 300, 640)),
    ((2, 16, 4, 8000, 8000, 128), (2, 4, 1, 8064)),
    ((1, 2, 2, 129, 256, 64), (1, 1, 129, 256)),
    ((3, 2, 1, 1000, 130, 64), (3, 2, 1000, 256)),
]


@pytest.mark.parametrize("geom,shape", DENSE_CASES)
def test_dense_builder_random(geom, shape):
    say("dense builder", geom, shape)
    Sk = geom[4]
    m = _random_tiles(shape, Sk, seed=sum(shape))
    got = np_bm(bsm.build_block_mask(geom, mask=torch.from_numpy(m).cuda()))
    assert_bm_equal(got, oracle.classify_tiles(m, Sk), f"{geom} {shape}")


def test_dense_builder_strided_view():
    """A mask that is a strided view (every other query row) of a larger one."""
    geom = (1, 2, 2, 150, 500, 64)
    big = _random_tiles((1, 2, 300, 512), 500, seed=3)
    t = torch.from_numpy(big).cuda()[:, :, ::2, :]
    got = np_bm(bsm.build_block_mask(geom, mask=t))
    assert_bm_equal(got, oracle.classify_tiles(big[:, :, ::2, :], 500), "strided")


def test_decode_swap_block_mask():
    """(B, H, 1, K) mask under the head-group swap becomes (B, KVH, G rows, K)."""
    geom = (64, 32, 8, 1, 16384, 128)
    rng = np.random.default_rng(0)
    m = rng.random((64, 32, 1, 16384)) < 0.0625
    got = np_bm(bsm.build_block_mask(geom, mask=torch.from_numpy(m).cuda()))
    want = oracle.classify_tiles(m.reshape(64, 8, 4, 16384), 16384)
    assert_bm_equal(got, want, "swap")


def test_empty_queries():
    d = bsm.DFlash(128, 0, 16)
    geom = (1, 2, 2, 0, 128, 64)
    bm = bsm.build_block_mask(geom, pred=d)
    assert bm.kv_indices.shape == (1, 1, 0, 1)
