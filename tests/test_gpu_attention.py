"""GPU parity: masked attention forward against the fp64 CPU oracle.

Bars: bf16 inputs max|err| <= 2e-2 and mean|err| <= 2e-3, f32 inputs
max|err| <= 1e-4, on O and on LSE; -inf LSE (fully masked rows) exactly.
"""

import numpy as np
import pytest
import torch

from gpu_helpers import (assert_close, bsm, cuda, oracle, oracle_geom, oracle_rows,
                         oracle_topk_mask, say, synth)

pytestmark = pytest.mark.gpu


def _run_and_check(q, k, v, dt, mask=None, pred=None, bias=None, bm=None, scale=None,
                   rows=None, heads=None, what=""):
    """Run the GPU path, compare the given rows of every (b, h) with the oracle."""
    say("attention", what, tuple(q.shape), tuple(k.shape), dt)
    o, lse = bsm.masked_attn_fwd(q, k, v, pred=pred, mask=mask, bias=bias, block_mask=bm,
                                 softmax_scale=scale, return_lse=True)
    torch.cuda.synchronize()
    B, Sq, H, D = q.shape
    omask = oracle_geom(pred) if pred is not None else mask
    rows = np.arange(Sq) if rows is None else rows
    heads = range(H) if heads is None else heads
    o_np = o[:, rows].float().cpu().numpy()
    lse_np = lse[:, :, rows].cpu().numpy()
    for b in range(B):
        for h in heads:
            want_o, want_l = oracle_rows(q, k, v, b, h, rows, scale=scale, mask=omask, bias=bias)
            assert_close(o_np[b, :, h, :], want_o, dt, f"{what} O b={b} h={h}")
            assert_close(lse_np[b, h], want_l, dt, f"{what} LSE b={b} h={h}")
    return o, lse


def test_tiny_dflash_fp32():
    """Tiny DFlash case in f32: 256 context + 4 blocks of 16, full layer."""
    cfg = synth.CONFIGS["tiny_dflash_fp32"]
    d = bsm.DFlash(cfg["ctx_len"], cfg["num_blocks"], cfg["block_size"])
    q, k, v = cuda(*synth.qkv(1, d.Sq, d.Sk, 2, 2, 64, "f32", seed=0))
    geom = bsm.geometry_of(q, k)
    bm = bsm.build_block_mask(geom, pred=d)
    assert int(bm.kv_num_blocks.sum()) == 3 and int(bm.full_kv_num_blocks.sum()) == 0
    _run_and_check(q, k, v, "f32", pred=d, bm=bm, what="tiny+bm")
    _run_and_check(q, k, v, "f32", pred=d, what="tiny")


SMALL_DFLASH = [
    dict(ctx_len=260, num_blocks=13, block_size=16),
    dict(ctx_len=260, num_blocks=13, block_size=16, layer_type="sliding", sliding_window=100),
    dict(ctx_len=260, num_blocks=13, block_size=16, is_causal=False, layer_type="sliding",
         sliding_window=37),
    dict(ctx_len=999, num_blocks=3, block_size=200, is_causal=True),
]


@pytest.mark.parametrize("case", SMALL_DFLASH)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_small_dflash(case, D, dt):
    d = bsm.DFlash(**case)
    q, k, v = cuda(*synth.qkv(2, d.Sq, d.Sk, 4, 2, D, dt, seed=1))
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), pred=d)
    _run_and_check(q, k, v, dt, pred=d, bm=bm, what=f"dflash {case} D={D}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("mshape,bshape", [
    ((2, 4, 300, 640), None),
    ((1, 1, 1, 640), (2, 2, 1, 640)),
    ((2, 2, 1, 640), (1, 4, 300, 640)),
    ((1, 4, 300, 640), (2, 1, 1, 640)),
    (None, (2, 2, 300, 640)),
    (None, None),
])
def test_dense_mask_and_bias(dt, mshape, bshape):
    B, Sq, Sk, H, KVH, D = 2, 300, 600, 4, 2, 128
    q, k, v = cuda(*synth.qkv(B, Sq, Sk, H, KVH, D, dt, seed=2))
    mask = bias = None
    if mshape is not None:
        m = synth.random_bool(mshape, 0.3, 2, synth.TID_MASK)
        m[..., 5] = True
        mask = torch.from_numpy(m).cuda()
    if bshape is not None:
        bias = synth.normal_tensor(bshape, 2, synth.TID_BIAS, dt).cuda()
    geom = bsm.geometry_of(q, k)
    bm = bsm.build_block_mask(geom, mask=mask) if mask is not None else None
    _run_and_check(q, k, v, dt, mask=mask, bias=bias, bm=bm, scale=0.07,
                   what=f"dense m={mshape} b={bshape}")
    if mask is not None:
        _run_and_check(q, k, v, dt, mask=mask, bias=bias, scale=0.07, what="dense, no bm")


def test_fully_masked_rows_and_single_keys():
    B, Sq, Sk, H, KVH, D = 1, 200, 300, 2, 1, 64
    q, k, v = cuda(*synth.qkv(B, Sq, Sk, H, KVH, D, "bf16", seed=3))
    m = np.zeros((1, 1, Sq, 384), bool)
    m[0, 0, ::3, 7] = True          # single kept key
    m[0, 0, 1::3, :] = True         # everything kept (and the tail, ignored)
    # rows 2::3 keep nothing
    mask = torch.from_numpy(m).cuda()
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask)
    o, lse = _run_and_check(q, k, v, "bf16", mask=mask, bm=bm, what="masked rows")
    assert (o[0, 2::3].float() == 0).all()
    assert torch.isneginf(lse[0, :, 2::3]).all()
    # a single kept key returns that value row, rounded to bf16
    torch.testing.assert_close(o[0, ::3, 0].float(), v[0, 7:8, 0].float().expand(67, 64),
                               rtol=0, atol=0)


@pytest.mark.parametrize("with_mask", [True, False])
def test_decode_swap_small(with_mask):
    """seqlen_q == 1 with H > KVH runs the head-group swap; compare with the
    unswapped definition."""
    B, Sk, H, KVH, D = 3, 1000, 8, 2, 128
    q, k, v = cuda(*synth.qkv(B, 1, Sk, H, KVH, D, "bf16", seed=4))
    bias = synth.normal_tensor((B, H, 1, 1024), 4, synth.TID_BIAS, "bf16").cuda()
    mask = bm = None
    if with_mask:
        mask = oracle_topk_mask(bias, Sk, 100)
        bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask)
        assert bm.kv_indices.shape == (B, KVH, 1, 8)
    _run_and_check(q, k, v, "bf16", mask=mask, bias=bias, bm=bm, what="swap")


def test_decode_swap_pred():
    d = bsm.DFlash(200, 1, 1)
    q, k, v = cuda(*synth.qkv(2, 1, d.Sk, 8, 2, 64, "bf16", seed=5))
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), pred=d)
    _run_and_check(q, k, v, "bf16", pred=d, bm=bm, what="swap pred")


def test_deterministic():
    d = bsm.DFlash(260, 13, 16, layer_type="sliding", sliding_window=100)
    q, k, v = cuda(*synth.qkv(1, d.Sq, d.Sk, 4, 2, 128, "bf16", seed=6))
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), pred=d)
    o1 = bsm.masked_attn_fwd(q, k, v, pred=d, block_mask=bm)
    o2 = bsm.masked_attn_fwd(q, k, v, pred=d, block_mask=bm)
    assert torch.equal(o1, o2)


# The workloads at full size are compared in test_gpu_fullsize.py.


@pytest.mark.parametrize("layer", ["full", "sliding"])
def test_xcd_grouped_work_mapping(layer):
    """B * KVH * G / 2 = 8 head-pair groups: the two-head kernel's mapping that
    gives each XCD whole groups (the training and long-context shapes take it
    too), on every row."""
    kw = dict(layer_type="sliding", sliding_window=300) if layer == "sliding" else {}
    d = bsm.DFlash(512, 32, 16, **kw)
    q, k, v = cuda(*synth.qkv(2, d.Sq, d.Sk, 8, 4, 128, "bf16", seed=40))
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), pred=d)
    _run_and_check(q, k, v, "bf16", pred=d, bm=bm, what=f"xcd groups {layer}")


@pytest.mark.parametrize("Sq", [1, 7, 20, 32])
@pytest.mark.parametrize("D", [64, 128])
def test_short_query_blocks(Sq, D):
    """At most 32 query rows per (b, h): the key-split kernel, with a per-head
    mask, a query-broadcast bias, ragged Sk and a GQA group of 2."""
    B, Sk, H, KVH = 2, 700, 4, 2
    q, k, v = cuda(*synth.qkv(B, Sq, Sk, H, KVH, D, "bf16", seed=10 + Sq))
    m = synth.random_bool((B, H, Sq, 768), 0.4, 7, synth.TID_MASK)
    m[..., 3] = True
    mask = torch.from_numpy(m).cuda()
    bias = synth.normal_tensor((B, KVH, 1, 768), 7, synth.TID_BIAS, "bf16").cuda()
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask)
    _run_and_check(q, k, v, "bf16", mask=mask, bias=bias, bm=bm, what=f"short Sq={Sq} D={D}")


def test_short_dflash_block():
    """Two draft blocks of 16 (32 queries) against a long context."""
    d = bsm.DFlash(1200, 2, 16, is_causal=True, layer_type="sliding", sliding_window=500)
    q, k, v = cuda(*synth.qkv(1, d.Sq, d.Sk, 8, 2, 128, "bf16", seed=12))
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), pred=d)
    _run_and_check(q, k, v, "bf16", pred=d, bm=bm, what="short dflash")


# ---------------------------------------------------------------------------
# bf16, D = 128, no bias and no dense mask: the two-head interleaved kernel.
# Its visit list splits into a run of plain tiles and a run of tested tiles;
# these cases cover an all-plain list, a single tile, a list with no plain
# tile, ragged query and key ends, and GQA groups of 2 and 4.

@pytest.mark.parametrize("B,Sq,Sk,H,KVH", [
    (1, 256, 512, 2, 1),     # every tile plain
    (2, 100, 128, 4, 2),     # one key tile, rows past Sq in every wave
    (1, 130, 129, 8, 2),     # ragged: 2 query tiles, key tile straddling Sk
    (2, 384, 1000, 4, 1),    # G = 4, ragged keys
])
def test_no_mask_bf16_d128(B, Sq, Sk, H, KVH):
    q, k, v = cuda(*synth.qkv(B, Sq, Sk, H, KVH, 128, "bf16", seed=20 + Sq))
    _run_and_check(q, k, v, "bf16", what=f"no mask B={B} Sq={Sq} Sk={Sk} H={H} KVH={KVH}")


@pytest.mark.parametrize("case", [
    dict(ctx_len=512, num_blocks=16, block_size=16, layer_type="sliding", sliding_window=200),
    dict(ctx_len=300, num_blocks=10, block_size=16),
])
@pytest.mark.parametrize("with_bm", [True, False])
def test_dflash_bf16_d128_block_mask_or_not(case, with_bm):
    """Predicate partial tiles after full ones (with a block mask), or every
    tile tested (without)."""
    d = bsm.DFlash(**case)
    q, k, v = cuda(*synth.qkv(1, d.Sq, d.Sk, 4, 2, 128, "bf16", seed=30))
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), pred=d) if with_bm else None
    _run_and_check(q, k, v, "bf16", pred=d, bm=bm, what=f"dflash bm={with_bm} {case}")


def _fwd_ws_bytes(q, k, v, mask=None, bias=None, bm=None):
    """Workspace bytes the library asks for (0: none would be used)."""
    import ctypes
    a = bsm.AttnArgs()
    a.q, a.k, a.v = bsm.tensor4(q), bsm.tensor4(k), bsm.tensor4(v)
    a.o = q.data_ptr()
    for i in range(4):
        a.o_stride[i] = q.stride(i)
    keep = []
    for name, t in (("mask", mask), ("bias", bias)):
        if t is not None:
            c = bsm.tensor4(t)
            keep.append(c)
            setattr(a, name, ctypes.pointer(c))
    if bm is not None:
        bc = bm.c()
        keep.append(bc)
        a.bm = ctypes.pointer(bc)
    n = ctypes.c_int64(0)
    bsm._check(bsm.lib().attn_fwd_workspace_size(ctypes.byref(bsm.geometry_of(q, k).c()),
                                                 ctypes.byref(a), ctypes.byref(n)))
    return n.value


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mshape,bshape", [
    ((2, 2, 1, 768), (2, 4, 1, 768)),   # per-KV-head mask, per-head bias
    ((1, 1, 1, 768), None),             # one mask row for everything
    (None, (2, 1, 1, 768)),             # bias only, one row per batch
    ((2, 4, 1, 768), (1, 2, 1, 768)),   # per-head mask, per-KV-head bias
])
def test_staged_mask_bias_rows(D, mshape, bshape):
    """Query-broadcast mask / bias folded into staged rows: against the oracle
    on every row, and against the same call without the workspace (the rows
    then come from the mask / bias tensors directly)."""
    B, Sq, Sk, H, KVH = 2, 260, 700, 4, 2
    q, k, v = cuda(*synth.qkv(B, Sq, Sk, H, KVH, D, "bf16", seed=5))
    mask = bias = None
    if mshape is not None:
        m = synth.random_bool(mshape, 0.4, 5, synth.TID_MASK)
        m[..., 128:256] = False                      # an empty key tile
        m[0, 0, 0, 3] = True
        mask = torch.from_numpy(m).cuda()
    if bshape is not None:
        bias = synth.normal_tensor(bshape, 5, synth.TID_BIAS, "bf16").cuda()
    # a per-head block mask goes to the one-head kernel, which stages nothing
    bm = (bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask)
          if mask is not None and mshape[1] != H else None)
    assert _fwd_ws_bytes(q, k, v, mask=mask, bias=bias, bm=bm) > 0
    o, lse = _run_and_check(q, k, v, "bf16", mask=mask, bias=bias, bm=bm, scale=0.09,
                            what=f"staged m={mshape} b={bshape} D={D}")
    o1, lse1 = bsm.masked_attn_fwd(q, k, v, mask=mask, bias=bias, block_mask=bm,
                                   softmax_scale=0.09, return_lse=True, split=False)
    torch.cuda.synchronize()
    assert (o.float() - o1.float()).abs().max().item() <= 2e-2
    fin = torch.isfinite(lse1)
    assert torch.equal(torch.isfinite(lse), fin)
    if fin.any():
        # the two paths round their probabilities to bf16 against different
        # running maxima (one per tile / one per 64 keys); each row sum then
        # carries a relative error of at most 2^-9, so the LSEs may differ by
        # up to 2 * 2^-9
        assert (lse[fin] - lse1[fin]).abs().max().item() <= 2 * 2.0 ** -9


def test_two_head_tile_list_lengths():
    """Query tiles that visit 0, 1, 2, 3, 6 and 6 key tiles (full, partial and
    past Sk mixed) in the two-head kernel: the loop reads each next tile index
    ahead of its use, and odd / even counts end on different slots."""
    B, Sq, Sk, H, KVH, D = 1, 768, 677, 4, 2, 128
    q, k, v = cuda(*synth.qkv(B, Sq, Sk, H, KVH, D, "bf16", seed=31))
    m = np.zeros((1, 1, Sq, 768), bool)
    m[0, 0, 128:256, 256:384] = True                    # one full tile
    m[0, 0, 256:384, 0:128] = True                      # a full and a partial tile
    m[0, 0, 256:384, 600] = True
    m[0, 0, 384:512, 128:256] = True                    # two full, one past Sk
    m[0, 0, 384:512, 384:512] = True
    m[0, 0, 384:512, 640:677] = True
    m[0, 0, 512:640:2, :] = True                        # every tile partial
    m[0, 0, 640:768, :677] = True                       # every tile kept
    mask = torch.from_numpy(m).cuda()
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask)
    n = bm.kv_num_blocks.cpu().numpy().ravel() + bm.full_kv_num_blocks.cpu().numpy().ravel()
    assert list(n) == [0, 1, 2, 3, 6, 6], n
    o, lse = _run_and_check(q, k, v, "bf16", mask=mask, bm=bm, what="tile list lengths")
    assert (o[0, :128].float() == 0).all()
    assert torch.isneginf(lse[0, :, :128]).all()


# ---------------------------------------------------------------------------
# huge and infinite biases: finite values saturate at +-FLT_MAX / log2 e in
# the kernels' log2 units (a kept key carrying the pre-mask sentinel
# finfo.min stays kept), -inf drops the key

BF16_MIN = -(2.0 - 2.0 ** -7) * 2.0 ** 127


def _extreme_bias(shape, seed):
    """A normal bias whose rows (by head and query) are, in turn: every key at
    the sentinel, the sentinel beside five ordinary keys, values beyond the
    bound (-3e38 and -2.4e38), a -inf on every third key, or left as drawn."""
    b = synth.normal(shape, seed, synth.TID_BIAS).astype(np.float64)
    for hb in range(shape[1]):
        for row in range(shape[2]):
            kind = (hb + row) % 5
            r = b[:, hb, row]
            if kind == 0:
                r[:] = BF16_MIN
            elif kind == 1:
                r[:] = BF16_MIN
                r[:, :5] = 0.5
            elif kind == 2:
                r[:, 0::2] = -3.0e38
                r[:, 1::2] = -2.4e38
            elif kind == 3:
                r[:, ::3] = -np.inf
    return b


@pytest.mark.parametrize("dt,Sq,bq", [("bf16", 300, True), ("bf16", 300, False),
                                      ("bf16", 20, True), ("f32", 300, True)])
def test_huge_and_infinite_biases(dt, Sq, bq):
    B, Sk, H, KVH, D = 2, 600, 4, 2, 128
    K = 640
    q, k, v = cuda(*synth.qkv(B, Sq, Sk, H, KVH, D, dt, seed=50))
    # a query-broadcast bias comes with a query-broadcast mask (the staged rows)
    m = synth.random_bool((B, 1, Sq if bq else 1, K), 0.6, 50, synth.TID_MASK)
    m[..., :5] = True
    mask = torch.from_numpy(m).cuda()
    shape = (B, H, Sq, K) if bq else (B, KVH, 1, K)
    bias_np = _extreme_bias(shape, 50)
    bias = torch.from_numpy(bias_np).to(torch.bfloat16 if dt == "bf16" else torch.float32).cuda()
    say("extreme biases", dt, Sq, shape)
    o, lse = bsm.masked_attn_fwd(q, k, v, mask=mask, bias=bias, return_lse=True)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        for h in range(H):
            want_o, want_l = oracle_rows(q, k, v, b, h, np.arange(Sq), mask=mask, bias=bias)
            assert_close(o[b, :, h], want_o, dt, f"extreme O b={b} h={h}")
            huge = np.abs(want_l) > 1e30
            assert np.array_equal(np.isneginf(lse[b, h]), np.isneginf(want_l))
            rel = np.abs(lse[b, h][huge] - want_l[huge]) / np.abs(want_l[huge])
            assert (rel <= 1e-6).all(), f"LSE of saturated rows, rel err {rel.max():.2e}"
            small = ~huge
            assert_close(lse[b, h][small], want_l[small], dt, f"extreme LSE b={b} h={h}")


ONE_HEAD_CASES = [
    # (H, KVH, D, DFlash geometry or None for no mask, Sq, Sk without a mask, block mask)
    (4, 4, 128, dict(ctx_len=260, num_blocks=13, block_size=16), 0, 0, True),  # MHA, ragged
    (4, 4, 128, dict(ctx_len=260, num_blocks=13, block_size=16), 0, 0, False),
    (6, 2, 64, dict(ctx_len=260, num_blocks=13, block_size=16, layer_type="sliding",
                    sliding_window=100), 0, 0, True),                          # G = 3
    (6, 2, 64, dict(ctx_len=260, num_blocks=13, block_size=16, layer_type="sliding",
                    sliding_window=100), 0, 0, False),
    (3, 1, 128, dict(ctx_len=999, num_blocks=3, block_size=200, is_causal=True), 0, 0, True),
    (2, 2, 128, None, 300, 777, False),                                        # MHA, no mask
]


@pytest.mark.parametrize("H,KVH,D,case,Sq,Sk,with_bm", ONE_HEAD_CASES)
def test_odd_group_sizes(H, KVH, D, case, Sq, Sk, with_bm):
    """Odd head groups (MHA, G = 3) without a mask tensor or bias: one head per
    workgroup with 64-key sub-tiles; several query and key tiles, ragged ends."""
    d = bsm.DFlash(**case) if case is not None else None
    if d is not None:
        Sq, Sk = d.Sq, d.Sk
    q, k, v = cuda(*synth.qkv(2, Sq, Sk, H, KVH, D, "bf16", seed=60 + H + D))
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), pred=d) if with_bm else None
    _run_and_check(q, k, v, "bf16", pred=d, bm=bm, what=f"G={H // KVH} D={D} {case}")


ONE_HEAD_AUX = [
    # (H, KVH, D, mask shape, bias shape): heads that no two-head workgroup can
    # pair (odd G), or per-head block masks, with dense masks and / or biases
    (3, 3, 128, (2, 3, 300, 640), None),                  # MHA, per-head mask
    (3, 3, 128, (1, 1, 1, 640), (2, 3, 1, 640)),          # broadcast mask, per-head bias
    (6, 2, 64, (2, 2, 300, 640), (1, 6, 300, 640)),       # G = 3, KV-head mask
    (6, 2, 128, None, (2, 1, 1, 640)),                    # bias only
    (3, 1, 128, (1, 3, 300, 640), (2, 1, 300, 640)),      # G = 3, one KV head
    (4, 2, 128, (2, 4, 300, 640), (2, 2, 300, 640)),      # G = 2, per-head block mask
]


@pytest.mark.parametrize("H,KVH,D,mshape,bshape", ONE_HEAD_AUX)
def test_one_head_mask_and_bias(H, KVH, D, mshape, bshape):
    """One head per workgroup with a dense mask and / or a bias: every row of
    every head, with the mask's own (per-head when it has H heads) block mask
    and without one; ragged query and key tiles (Sq = 300, Sk = 600)."""
    B, Sq, Sk = 2, 300, 600
    q, k, v = cuda(*synth.qkv(B, Sq, Sk, H, KVH, D, "bf16", seed=70 + H + D))
    mask = bias = None
    if mshape is not None:
        m = synth.random_bool(mshape, 0.3, 71, synth.TID_MASK)
        m[..., 5] = True
        mask = torch.from_numpy(m).cuda()
    if bshape is not None:
        bias = synth.normal_tensor(bshape, 71, synth.TID_BIAS, "bf16").cuda()
    what = f"one-head H={H} KVH={KVH} D={D} m={mshape} b={bshape}"
    if mask is not None:
        bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask)
        _run_and_check(q, k, v, "bf16", mask=mask, bias=bias, bm=bm, scale=0.07, what=what)
    _run_and_check(q, k, v, "bf16", mask=mask, bias=bias, scale=0.07, what=what + " no bm")


def test_one_head_fully_masked_rows_and_single_keys():
    B, Sq, Sk, H, KVH, D = 1, 200, 300, 3, 3, 128
    q, k, v = cuda(*synth.qkv(B, Sq, Sk, H, KVH, D, "bf16", seed=72))
    m = np.zeros((1, 1, Sq, 384), bool)
    m[0, 0, ::3, 7] = True          # single kept key
    m[0, 0, 1::3, :] = True         # everything kept (and the tail, ignored)
    # rows 2::3 keep nothing
    mask = torch.from_numpy(m).cuda()
    bias = synth.normal_tensor((1, H, 1, 384), 72, synth.TID_BIAS, "bf16").cuda()
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask)
    o, lse = _run_and_check(q, k, v, "bf16", mask=mask, bias=bias, bm=bm,
                            what="one-head masked rows")
    assert (o[0, 2::3].float() == 0).all()
    assert torch.isneginf(lse[0, :, 2::3]).all()
    torch.testing.assert_close(o[0, ::3, 1].float(), v[0, 7:8, 1].float().expand(67, D),
                               rtol=0, atol=0)
