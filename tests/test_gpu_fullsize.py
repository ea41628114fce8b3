"""GPU parity at the workloads' full sizes, against the fp64 oracle run on a
pool of host processes (tests/oracle_pool.py):

  * DFlash training shape, both layers: every row of every (b, h);
  * long-context DFlash: rows in every (b, h, query tile) -- one in each of
    its four 32-row blocks, placed differently per head and tile -- plus rows
    0, 127, 128 and the last; and the
    head-shared block mask on all 256 query tiles, bit-exact;
  * dynamic top-k: every row of every (b, h);
  * decode with the head-group swap: every (b, h), through the block mask and
    through the kept-key list.

Every mask the oracle uses is its own (its DFlash rule, its top-k), never the
GPU's. Bars: bf16 max |err| <= 2e-2 and mean |err| <= 2e-3 per (b, h), on O and
LSE, -inf LSE matched exactly.
"""

import numpy as np
import pytest
import torch

import oracle_pool
from gpu_helpers import assert_close, bsm, oracle, say, synth

pytestmark = pytest.mark.gpu


def _dflash(name, li):
    cfg = synth.CONFIGS[name]
    layer = cfg["layers"][li]
    d = bsm.DFlash(cfg["ctx_len"], cfg["num_blocks"], cfg["block_size"],
                   is_causal=layer["is_causal"], layer_type=layer["layer_type"],
                   sliding_window=layer["window"])
    q, k, v = [t.cuda() for t in synth.qkv(cfg["B"], d.Sq, d.Sk, cfg["H"], cfg["KVH"],
                                            cfg["D"], cfg["dtype"], seed=0,
                                            scale=cfg["qkv_scale"])]
    return cfg, d, q, k, v


def _check_jobs(o, lse, jobs, results, what):
    """jobs: (..., b, h, rows); results: the oracle's (O, LSE) per job."""
    for job, (want_o, want_l) in zip(jobs, results):
        b, h, rows = job[-3], job[-2], np.asarray(job[-1])
        assert_close(o[b, rows, h], want_o, "bf16", f"{what} O b={b} h={h}")
        assert_close(lse[b, h, rows], want_l, "bf16", f"{what} LSE b={b} h={h}")


@pytest.mark.parametrize("li", [0, 1], ids=["full", "sliding"])
def test_dflash_train_every_row(li):
    name = "dflash_train_bf16"
    cfg, d, q, k, v = _dflash(name, li)
    say("train shape, every row, layer", li)
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), pred=d)
    o, lse = bsm.masked_attn_fwd(q, k, v, pred=d, block_mask=bm, return_lse=True)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    rows = list(range(d.Sq))
    jobs = [(name, li, b, h, rows) for b in range(cfg["B"]) for h in range(cfg["H"])]
    _check_jobs(o, lse, jobs, oracle_pool.run(oracle_pool.dflash_rows, jobs), f"train/{li}")


def _tile_rows(Sq, h):
    """One row in each 32-row block of every 128-row query tile (the rows one
    wave of the attention kernel owns), at head- and tile-dependent places, and
    the first / last rows and the 127 / 128 boundary."""
    rows = {0, 127, 128, Sq - 1}
    for qt in range((Sq + 127) // 128):
        for blk in range(4):
            r = 32 * blk + (h * 11 + qt * 7 + blk * 5) % 32
            if qt * 128 + r < Sq:
                rows.add(qt * 128 + r)
    return sorted(rows)


def test_long_dflash_every_query_tile():
    name = "long_dflash_bf16"
    cfg, d, q, k, v = _dflash(name, 0)
    say("long context, every (b, h, query tile)")
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), pred=d)
    o, lse = bsm.masked_attn_fwd(q, k, v, pred=d, block_mask=bm, return_lse=True)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    jobs = [(name, 0, b, h, _tile_rows(d.Sq, h)) for b in range(cfg["B"])
            for h in range(cfg["H"])]
    _check_jobs(o, lse, jobs, oracle_pool.run(oracle_pool.dflash_rows, jobs), "long")


def test_long_dflash_block_mask_every_tile():
    """The head-shared (1, 1, 256, 512) block mask, all 256 query tiles, against
    the oracle's classification of its own dense rows (SpecForge issue #452,
    Expected Behavior: one copy for all heads)."""
    name = "long_dflash_bf16"
    cfg = synth.CONFIGS[name]
    layer = cfg["layers"][0]
    d = bsm.DFlash(cfg["ctx_len"], cfg["num_blocks"], cfg["block_size"],
                   is_causal=layer["is_causal"], layer_type=layer["layer_type"],
                   sliding_window=layer["window"])
    geom = (cfg["B"], cfg["H"], cfg["KVH"], d.Sq, d.Sk, cfg["D"])
    kvn, kvi, fn, fi = [t.cpu().numpy() for t in bsm.build_block_mask(geom, pred=d)]
    nQ = (d.Sq + 127) // 128
    assert kvi.shape == (1, 1, nQ, (d.Sk + 127) // 128)
    tiles = np.array_split(np.arange(nQ), 16)
    jobs = [(name, 0, [int(t) for t in ts]) for ts in tiles]
    res = oracle_pool.run(oracle_pool.dflash_tile_classes, jobs)
    for ts, classes in zip(tiles, res):
        for t, (part, full) in zip(ts, classes):
            np.testing.assert_array_equal(kvi[0, 0, t, :kvn[0, 0, t]], part, f"tile {t}")
            np.testing.assert_array_equal(fi[0, 0, t, :fn[0, 0, t]], full, f"tile {t}")
            assert (kvi[0, 0, t, kvn[0, 0, t]:] == -1).all()
            assert (fi[0, 0, t, fn[0, 0, t]:] == -1).all()
    assert (int(fn.sum()), int(kvn.sum())) == (7215, 961)


def test_dynamic_topk_every_row():
    name = "dynamic_topk_bf16"
    cfg = synth.CONFIGS[name]
    B, H, KVH, D, Sq, Sk = (cfg[x] for x in ("B", "H", "KVH", "D", "Sq", "Sk"))
    q, k, v = [t.cuda() for t in synth.qkv(B, Sq, Sk, H, KVH, D, "bf16", seed=0)]
    bias, pad2d = synth.topk_inputs(cfg, seed=0)
    bias, pad2d = bias.cuda(), pad2d.cuda()
    say("dynamic top-k, every row")
    mask = bsm.create_mask(bias, pad2d, B, Sq, Sk, cfg["topk"])
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask)
    o, lse = bsm.masked_attn_fwd(q, k, v, mask=mask, bias=bias, block_mask=bm, return_lse=True)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    rows = list(range(Sq))
    jobs = [(name, b, h, rows) for b in range(B) for h in range(H)]
    _check_jobs(o, lse, jobs, oracle_pool.run(oracle_pool.topk_rows, jobs), "dynamic")


def test_decode_every_head():
    """Decode (Sq = 1, head-group swap): every (b, h) against the unswapped
    definition with the oracle's own top-k mask of each batch, through both
    decode paths -- the block mask over key tiles, and the kept-key list with
    the key-gather kernel."""
    name = "decode_swap_bf16"
    cfg = synth.CONFIGS[name]
    B, H, KVH, D, Sk = (cfg[x] for x in ("B", "H", "KVH", "D", "Sk"))
    qc, kc, vc = synth.qkv(B, 1, Sk, H, KVH, D, "bf16", seed=0)
    bias_c, _ = synth.topk_inputs(cfg, seed=0)
    q, k, v, bias = qc.cuda(), kc.cuda(), vc.cuda(), bias_c.cuda()
    say("decode, every (b, h)")
    mask = bsm.dynamic_topk_mask(bias, None, Sk, cfg["topk"])
    geom = bsm.geometry_of(q, k)
    bm = bsm.build_block_mask(geom, mask=mask)
    keys = bsm.build_key_list(geom, mask)
    got = {}
    for path, kw in (("tiles", dict(block_mask=bm)), ("gather", dict(keys=keys))):
        o, lse = bsm.masked_attn_fwd(q, k, v, mask=mask, bias=bias, return_lse=True, **kw)
        torch.cuda.synchronize()
        got[path] = (o.float().cpu().numpy(), lse.cpu().numpy())
    del q, k, v, mask, bm, keys
    masks = oracle_pool.run(oracle_pool.topk_mask_rows, [(name, b) for b in range(B)])
    for b in range(B):
        qb, kb, vb = synth.as_f64(qc[b:b + 1]), synth.as_f64(kc[b:b + 1]), synth.as_f64(vc[b:b + 1])
        bb = synth.as_f64(bias_c[b:b + 1])
        for h in range(H):
            want_o, want_l = oracle.attention_rows(qb, kb, vb, 0, h, [0], mask=masks[b], bias=bb)
            for path, (o, lse) in got.items():
                assert_close(o[b, 0, h][None], want_o, "bf16", f"decode {path} O b={b} h={h}")
                assert_close(lse[b, h], want_l, "bf16", f"decode {path} LSE b={b} h={h}")
