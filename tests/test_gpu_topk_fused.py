"""GPU parity: top-k fused with the block mask and the kept-key list of its mask
(dynamic_topk_fused), bit-exact against the CPU oracle (topk_keep_mask, then
classify_tiles / key_list of that mask in the attention's iteration space)."""

import numpy as np
import pytest
import torch

import oracle_pool
from gpu_helpers import assert_bm_equal, bsm, np_bm, oracle, say, synth
from oracle.keylist import key_list

pytestmark = pytest.mark.gpu


def _iter_view(mask_np, geom):
    """The mask in the attention's iteration space (the swap regroups heads)."""
    B, H, KVH, Sq, Sk, D = geom
    if Sq == 1 and H > KVH and mask_np.shape[1] == H:
        return mask_np.reshape(mask_np.shape[0], KVH, H // KVH, mask_np.shape[3])
    return mask_np


def _rows(geom):
    B, H, KVH, Sq, Sk, D = geom
    return H // KVH if (Sq == 1 and H > KVH) else Sq


def _check(geom, bias, premask, k, dt, want_keys, what, lists=None):
    Sk = geom[4]
    say("topk fused", what, tuple(bias.shape), k, dt)
    mask, bm, keys = bsm.dynamic_topk_fused(geom, bias.cuda(),
                                            None if premask is None else premask.cuda(), k,
                                            want_keys=want_keys)
    torch.cuda.synchronize()
    pm = None if premask is None else premask.numpy()
    want_mask = oracle.topk_keep_mask(synth.as_f64(bias), pm, Sk, k, dt)
    np.testing.assert_array_equal(mask.cpu().numpy(), want_mask, err_msg=f"{what} mask")
    it = _iter_view(want_mask, geom)
    assert_bm_equal(np_bm(bm), oracle.classify_tiles(it, Sk), f"{what} block mask")
    if want_keys:
        gn = keys.num_keys.cpu().numpy()
        gk = keys.key_indices.cpu().numpy()
        gb = keys.row_bits.cpu().numpy().view(np.uint32)
        pairs = lists if lists is not None else [(b, h) for b in range(it.shape[0])
                                                 for h in range(it.shape[1])]
        for b, h in pairs:
            wn, wk, wb = key_list(it[b:b + 1, h:h + 1], Sk, _rows(geom))
            n = int(wn[0, 0])
            assert gn[b, h] == n, f"{what} ({b},{h}) num {gn[b, h]} != {n}"
            np.testing.assert_array_equal(gk[b, h, :n], wk[0, 0, :n])
            np.testing.assert_array_equal(gb[b, h, :n], wb[0, 0, :n])
    return mask, bm, keys


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("k", [0, 1, 100, 5000])
def test_fused_swapped_decode(dt, k):
    """Sq == 1, per-head bias: the 4 heads of a KV group are the 4 rows of one
    block-mask / key-list row; ragged Sk; k = 0 and k >= Sk included."""
    geom = (3, 8, 2, 1, 1000, 128)
    bias = synth.normal_tensor((3, 8, 1, 1024), 90 + k, synth.TID_BIAS, dt)
    _check(geom, bias, None, k, dt, True, f"swap k={k} {dt}")


def test_fused_query_broadcast_with_premask():
    """The dynamic-mask workload's layout: bias (B, KVH, 1, K) broadcast over
    8000 queries, a 2D right-padding pre-mask, k = 2048 (no key list: 8000 rows)."""
    cfg = synth.CONFIGS["dynamic_topk_bf16"]
    bias, pad2d = synth.topk_inputs(cfg, seed=0)
    B, Sk = cfg["B"], cfg["Sk"]
    geom = (B, cfg["H"], cfg["KVH"], cfg["Sq"], Sk, cfg["D"])
    pm = pad2d.as_strided((B, 1, 1, Sk), (pad2d.stride(0), 0, 0, pad2d.stride(1)))
    pm_np = oracle.normalize_premask(pad2d.numpy(), B, Sk)
    say("topk fused dynamic workload")
    mask, bm, _ = bsm.dynamic_topk_fused(geom, bias.cuda(), pm.cuda(), cfg["topk"])
    torch.cuda.synchronize()
    want = oracle.topk_keep_mask(synth.as_f64(bias), pm_np, Sk, cfg["topk"], "bf16")
    np.testing.assert_array_equal(mask.cpu().numpy(), want)
    assert_bm_equal(np_bm(bm), oracle.classify_tiles(want, Sk), "dynamic workload")


def test_fused_pre_masked_rows_and_mask_not_written():
    """A row whose pre-mask hides everything keeps nothing; without a mask
    output the block mask and key list still match the unfused path."""
    geom = (2, 4, 4, 20, 700, 64)
    bias = synth.normal_tensor((2, 4, 20, 768), 91, synth.TID_BIAS, "bf16")
    pm = torch.from_numpy(synth.random_bool((2, 1, 20, 700), 0.7, 91, synth.TID_MASK))
    pm[1, 0, 3] = False
    _check(geom, bias, pm, 50, "bf16", True, "premask rows")
    _, bm2, keys2 = bsm.dynamic_topk_fused(geom, bias.cuda(), pm.cuda(), 50, want_mask=False,
                                           want_keys=True)
    mask = bsm.dynamic_topk_mask(bias.cuda(), pm.cuda(), 700, 50)
    bm = bsm.build_block_mask(geom, mask=mask)
    keys = bsm.build_key_list(geom, mask)
    torch.cuda.synchronize()
    assert_bm_equal(np_bm(bm2), np_bm(bm), "no-mask-output bm")
    assert torch.equal(keys2.num_keys, keys.num_keys)
    n = keys.num_keys.cpu()
    for b in range(2):
        for h in range(4):
            c = int(n[b, h])
            assert torch.equal(keys2.key_indices[b, h, :c], keys.key_indices[b, h, :c])
            assert torch.equal(keys2.row_bits[b, h, :c], keys.row_bits[b, h, :c])


def test_fused_decode_full_size():
    """The decode workload (B=64, H=32, KVH=8, Sk=16384, k=1024): fused outputs
    equal the unfused kernels' in full, the mask equals the oracle's top-k, and
    sampled lists match the oracle's lists of the oracle's mask."""
    cfg = synth.CONFIGS["decode_swap_bf16"]
    B, H, KVH, D, Sk = (cfg[x] for x in ("B", "H", "KVH", "D", "Sk"))
    geom = (B, H, KVH, 1, Sk, D)
    bias, _ = synth.topk_inputs(cfg, seed=0)
    say("topk fused decode full size")
    mask, bm, keys = bsm.dynamic_topk_fused(geom, bias.cuda(), None, cfg["topk"], want_keys=True)
    ref_mask = bsm.dynamic_topk_mask(bias.cuda(), None, Sk, cfg["topk"])
    ref_bm = bsm.build_block_mask(geom, mask=ref_mask)
    ref_keys = bsm.build_key_list(geom, ref_mask)
    torch.cuda.synchronize()
    assert torch.equal(mask, ref_mask)
    assert_bm_equal(np_bm(bm), np_bm(ref_bm), "decode bm")
    assert torch.equal(keys.num_keys, ref_keys.num_keys)
    omask = np.concatenate(oracle_pool.run(oracle_pool.topk_mask_rows,
                                           [("decode_swap_bf16", b) for b in range(B)]))
    np.testing.assert_array_equal(mask.cpu().numpy(), omask)
    it = _iter_view(omask, geom)
    for b, h in ((0, 0), (31, 4), (63, 7)):
        wn, wk, wb = key_list(it[b:b + 1, h:h + 1], Sk, H // KVH)
        n = int(wn[0, 0])
        assert int(keys.num_keys[b, h]) == n
        np.testing.assert_array_equal(keys.key_indices[b, h, :n].cpu().numpy(), wk[0, 0, :n])
        np.testing.assert_array_equal(keys.row_bits[b, h, :n].cpu().numpy().view(np.uint32),
                                      wb[0, 0, :n])
