"""GPU parity: DFlash inference masks -- one draft block after a KV cache of
ctx_len tokens -- block masks bit-exact against the oracle, attention against
the fp64 oracle at the bf16 bars (max|err| <= 2e-2, mean|err| <= 2e-3 on O and
LSE; -inf exactly)."""

import numpy as np
import pytest
import torch

from gpu_helpers import (assert_bm_equal, assert_close, bsm, cuda, np_bm, oracle,
                         oracle_geom, oracle_rows, say, synth)

pytestmark = pytest.mark.gpu

LAYERS = [
    dict(is_causal=None, layer_type="full", sliding_window=0),
    dict(is_causal=None, layer_type="sliding", sliding_window=300),
    dict(is_causal=True, layer_type="full", sliding_window=0),
    dict(is_causal=False, layer_type="sliding", sliding_window=77),
]


def _id(c):
    return "-".join(f"{k}{v}" for k, v in c.items())


@pytest.mark.parametrize("layer", LAYERS, ids=[_id(c) for c in LAYERS])
@pytest.mark.parametrize("ctx_len,block_size", [(1000, 16), (0, 16), (4000, 32), (257, 40)])
def test_inference_block_mask(layer, ctx_len, block_size):
    d = bsm.DFlash.inference(ctx_len, block_size, **layer)
    say("inference block mask", ctx_len, block_size, layer)
    geom = (2, 8, 2, d.Sq, d.Sk, 128)
    got = np_bm(bsm.build_block_mask(geom, pred=d))
    og = oracle.dflash_inference_geom(ctx_len, block_size, **layer)
    assert (og.Sq, og.Sk) == (d.Sq, d.Sk)
    want = oracle.classify_tiles(oracle.dflash_dense_mask(og)[None, None], og.Sk)
    assert_bm_equal(got, want, f"{ctx_len} {block_size} {layer}")


def _check(q, k, v, d, bm, what, heads=None):
    say("inference attention", what, tuple(q.shape), tuple(k.shape))
    o, lse = bsm.masked_attn_fwd(q, k, v, pred=d, block_mask=bm, return_lse=True)
    torch.cuda.synchronize()
    B, Sq, H, D = q.shape
    og = oracle_geom(d)
    rows = np.arange(Sq)
    o_np = o.float().cpu().numpy()
    lse_np = lse.cpu().numpy()
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            want_o, want_l = oracle_rows(q, k, v, b, h, rows, mask=og)
            assert_close(o_np[b, :, h], want_o, "bf16", f"{what} O b={b} h={h}")
            assert_close(lse_np[b, h], want_l, "bf16", f"{what} LSE b={b} h={h}")


@pytest.mark.parametrize("layer", LAYERS, ids=[_id(c) for c in LAYERS])
@pytest.mark.parametrize("block_size,D", [(16, 128), (16, 64), (32, 128), (40, 128)])
def test_inference_attention(layer, block_size, D):
    """16 and 32 draft tokens take the short-query kernel (G heads of a KV group
    on one XCD), 40 the tiled kernels; with and without the block mask."""
    d = bsm.DFlash.inference(1000, block_size, **layer)
    q, k, v = cuda(*synth.qkv(2, d.Sq, d.Sk, 8, 2, D, "bf16", seed=60 + block_size,
                              scale=0.5))
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), pred=d)
    _check(q, k, v, d, bm, f"bs={block_size} D={D} {layer}")
    _check(q, k, v, d, None, f"bs={block_size} D={D} {layer} no bm", heads=[0, 5])


def test_inference_empty_cache():
    d = bsm.DFlash.inference(0, 16, is_causal=True)
    q, k, v = cuda(*synth.qkv(1, d.Sq, d.Sk, 4, 4, 128, "bf16", seed=61))
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), pred=d)
    _check(q, k, v, d, bm, "empty cache")


@pytest.mark.parametrize("layer", [0, 1])
def test_inference_full_size_sampled(layer):
    """B=8 requests, H=32, KVH=8, D=128, 32768 cached tokens, one block of 16;
    sampled (b, h) against the oracle."""
    cfg = synth.CONFIGS["dflash_infer_bf16"]
    lay = cfg["layers"][layer]
    d = bsm.DFlash.inference(cfg["ctx_len"], cfg["block_size"], is_causal=lay["is_causal"],
                             layer_type=lay["layer_type"], sliding_window=lay["window"])
    q, k, v = cuda(*synth.qkv(cfg["B"], d.Sq, d.Sk, cfg["H"], cfg["KVH"], cfg["D"], "bf16",
                              seed=0, scale=cfg["qkv_scale"]))
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), pred=d)
    o, lse = bsm.masked_attn_fwd(q, k, v, pred=d, block_mask=bm, return_lse=True)
    torch.cuda.synchronize()
    og = oracle_geom(d)
    for b, h in ((0, 0), (3, 13), (7, 31)):
        say("oracle", b, h)
        want_o, want_l = oracle_rows(q, k, v, b, h, np.arange(d.Sq), mask=og)
        assert_close(o[b, :, h].float().cpu().numpy(), want_o, "bf16", f"O b={b} h={h}")
        assert_close(lse[b, h].cpu().numpy(), want_l, "bf16", f"LSE b={b} h={h}")
