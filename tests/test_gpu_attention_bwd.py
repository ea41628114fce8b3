"""GPU parity: masked attention backward against the fp64 backward oracle.

The GPU forward produces O and LSE, the GPU backward the gradients; the oracle
recomputes everything from the same stored inputs. Bars (relative to the
largest reference magnitude m = max(1, max|ref|)): bf16 outputs are rounded
to bf16 (relative 2^-9) after float arithmetic, so max |err| <= 2e-2 m and mean
|err| <= 2e-3 m; f32 max |err| <= 1e-4 m.
"""

import numpy as np
import pytest
import torch

import oracle_pool
from gpu_helpers import assert_grad_close as _close
from gpu_helpers import bsm, cuda, oracle_geom, oracle_topk_mask, say, synth
from oracle.attention_bwd import attention_bwd

pytestmark = pytest.mark.gpu


def _dout(shape, dt, seed):
    return synth.normal_tensor(shape, seed, synth.TID_DOUT, dt)


def _run(q, k, v, dt, pred=None, mask=None, bias=None, bm=None, scale=None, need_dbias=False,
         seed=0, what=""):
    say("attention bwd", what, tuple(q.shape), tuple(k.shape), dt)
    o, lse = bsm.masked_attn_fwd(q, k, v, pred=pred, mask=mask, bias=bias, block_mask=bm,
                                 softmax_scale=scale, return_lse=True)
    do = _dout(tuple(q.shape), dt, seed).cuda()
    dq, dk, dv, dbias = bsm.masked_attn_bwd(q, k, v, o, do, lse, pred=pred, mask=mask, bias=bias,
                                            block_mask=bm, softmax_scale=scale,
                                            need_dbias=need_dbias)
    torch.cuda.synchronize()
    return do, dq, dk, dv, dbias


def _check_full(q, k, v, dt, pred=None, mask=None, bias=None, bm=None, scale=None,
                need_dbias=False, seed=0, what=""):
    do, dq, dk, dv, dbias = _run(q, k, v, dt, pred, mask, bias, bm, scale, need_dbias, seed, what)
    om = oracle_geom(pred) if pred is not None else (None if mask is None else mask.cpu().numpy())
    ob = None if bias is None else synth.as_f64(bias)
    rq, rk, rv, rb = attention_bwd(synth.as_f64(q), synth.as_f64(k), synth.as_f64(v),
                                   synth.as_f64(do), scale=scale, mask=om, bias=ob)
    _close(dq.float().cpu().numpy(), rq, dt, f"{what} dq")
    _close(dk.float().cpu().numpy(), rk, dt, f"{what} dk")
    _close(dv.float().cpu().numpy(), rv, dt, f"{what} dv")
    if need_dbias:
        Sk = k.shape[1]
        assert dbias.shape[-1] == Sk
        _close(dbias.float().cpu().numpy(), rb[..., :Sk], dt, f"{what} dbias")


def test_tiny_dflash_fp32():
    cfg = synth.CONFIGS["tiny_dflash_fp32"]
    d = bsm.DFlash(cfg["ctx_len"], cfg["num_blocks"], cfg["block_size"])
    q, k, v = cuda(*synth.qkv(1, d.Sq, d.Sk, 2, 2, 64, "f32", seed=0))
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), pred=d)
    _check_full(q, k, v, "f32", pred=d, bm=bm, what="tiny dflash+bm")
    _check_full(q, k, v, "f32", pred=d, what="tiny dflash")


SMALL_DFLASH = [
    dict(ctx_len=260, num_blocks=13, block_size=16),
    dict(ctx_len=260, num_blocks=13, block_size=16, layer_type="sliding", sliding_window=100),
    dict(ctx_len=999, num_blocks=3, block_size=200, is_causal=True),
]


@pytest.mark.parametrize("case", SMALL_DFLASH)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_small_dflash(case, D, dt):
    d = bsm.DFlash(**case)
    q, k, v = cuda(*synth.qkv(2, d.Sq, d.Sk, 4, 2, D, dt, seed=1))
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), pred=d)
    _check_full(q, k, v, dt, pred=d, bm=bm, seed=1, what=f"dflash {case} D={D}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("mshape,bshape", [
    ((2, 4, 150, 256), (2, 4, 150, 256)),   # full bias: dbias = dS
    ((1, 1, 1, 256), (2, 2, 1, 256)),       # bias per KV head, broadcast over queries
    ((2, 2, 1, 256), (1, 4, 150, 256)),     # bias broadcast over batch
    (None, (1, 1, 1, 256)),                 # one bias row for everything
    (None, None),
])
def test_dense_mask_and_bias(dt, mshape, bshape, D):
    """Dense masks and biases of every broadcast shape, with dbias; bf16 at
    D = 128 takes the matrix-core kernels, the rest the generic ones."""
    B, Sq, Sk, H, KVH = 2, 150, 200, 4, 2
    q, k, v = cuda(*synth.qkv(B, Sq, Sk, H, KVH, D, dt, seed=2))
    mask = bias = None
    if mshape is not None:
        m = synth.random_bool(mshape, 0.3, 2, synth.TID_MASK)
        m[..., 5] = True
        mask = torch.from_numpy(m).cuda()
    if bshape is not None:
        bias = synth.normal_tensor(bshape, 2, synth.TID_BIAS, dt).cuda()
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask) if mask is not None else None
    _check_full(q, k, v, dt, mask=mask, bias=bias, bm=bm, scale=0.07,
                need_dbias=bias is not None, seed=2, what=f"dense m={mshape} b={bshape}")


@pytest.mark.parametrize("H,KVH,per_head_bm", [(3, 3, False), (3, 1, False), (4, 2, True)])
def test_broadcast_mask_bias_single_head_kernels(H, KVH, per_head_bm):
    """Query-broadcast mask and bias where the dQ kernel takes one head per
    workgroup (odd G, or a per-head block mask), reading the folded mask /
    bias rows, with dbias."""
    B, Sq, Sk, D = 2, 150, 200, 128
    q, k, v = cuda(*synth.qkv(B, Sq, Sk, H, KVH, D, "bf16", seed=8))
    mh = H if per_head_bm else 1
    m = synth.random_bool((B, mh, 1, 256), 0.4, 8, synth.TID_MASK)
    m[..., 3] = True
    mask = torch.from_numpy(m).cuda()
    bias = synth.normal_tensor((B, KVH, 1, 256), 8, synth.TID_BIAS, "bf16").cuda()
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask)
    _check_full(q, k, v, "bf16", mask=mask, bias=bias, bm=bm, scale=0.09, need_dbias=True,
                seed=8, what=f"broadcast H={H} KVH={KVH} per-head bm={per_head_bm}")


@pytest.mark.parametrize("H,KVH", [(2, 2), (3, 1)])
def test_one_head_dq_dense_and_dflash(H, KVH):
    """Odd G: the pipelined dQ kernel with one head per workgroup, its waves
    splitting each key tile in halves whose partial dQ are summed at the end.
    A per-query mask and bias with dbias (mask bytes and bias values read per
    tile), a DFlash predicate with its block mask, and no mask; ragged query and
    key tails, so one half of the last key tile lies past Sk."""
    B, Sq, Sk, D = 2, 300, 333, 128
    q, k, v = cuda(*synth.qkv(B, Sq, Sk, H, KVH, D, "bf16", seed=11))
    m = synth.random_bool((B, H, Sq, 384), 0.3, 11, synth.TID_MASK)
    m[..., 5] = True
    mask = torch.from_numpy(m).cuda()
    bias = synth.normal_tensor((B, H, Sq, 384), 11, synth.TID_BIAS, "bf16").cuda()
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask)
    _check_full(q, k, v, "bf16", mask=mask, bias=bias, bm=bm, scale=0.08, need_dbias=True,
                seed=11, what=f"one-head dq dense H={H} KVH={KVH}")
    _check_full(q, k, v, "bf16", seed=11, what=f"one-head dq no mask H={H} KVH={KVH}")
    d = bsm.DFlash(**SMALL_DFLASH[1])
    q, k, v = cuda(*synth.qkv(B, d.Sq, d.Sk, H, KVH, D, "bf16", seed=12))
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), pred=d)
    _check_full(q, k, v, "bf16", pred=d, bm=bm, seed=12, what=f"one-head dq dflash H={H} KVH={KVH}")


def test_one_head_dq_mid_size():
    """H = KVH at a size spanning 8 query and 24 key tiles: every gradient
    against the oracle, DFlash causal layer with its block mask."""
    d = bsm.DFlash(2048, 64, 16, is_causal=True)
    q, k, v = cuda(*synth.qkv(1, d.Sq, d.Sk, 2, 2, 128, "bf16", seed=13))
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), pred=d)
    _check_full(q, k, v, "bf16", pred=d, bm=bm, seed=13, what="one-head dq mid size")


def test_fully_masked_rows():
    B, Sq, Sk, H, KVH, D = 1, 130, 200, 2, 1, 64
    q, k, v = cuda(*synth.qkv(B, Sq, Sk, H, KVH, D, "bf16", seed=3))
    m = np.zeros((1, 1, Sq, 256), bool)
    m[0, 0, ::3, 7] = True
    m[0, 0, 1::3, :] = True
    mask = torch.from_numpy(m).cuda()
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask)
    _check_full(q, k, v, "bf16", mask=mask, bm=bm, seed=3, what="masked rows")


@pytest.mark.parametrize("D,dt", [(128, "bf16"), (64, "f32")])
def test_no_queries_zero_key_grads(D, dt):
    """Sq = 0: no query attends to any key, so dK = dV = 0 (written, not left
    as the allocator's memory)."""
    B, Sk, H, KVH = 2, 50, 4, 2
    q, k, v = cuda(*synth.qkv(B, 0, Sk, H, KVH, D, dt, seed=4))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, 0), dtype=torch.float32, device=q.device)
    say("backward without queries", D, dt)
    dq, dk, dv, _ = bsm.masked_attn_bwd(q, k, v, o, torch.empty_like(q), lse)
    torch.cuda.synchronize()
    assert dq.numel() == 0
    assert (dk == 0).all() and (dv == 0).all()


@pytest.mark.parametrize("with_mask", [True, False])
def test_decode_swap(with_mask):
    """Sq == 1 with H > KVH: the head-group swap, with a per-head bias."""
    B, Sk, H, KVH, D = 3, 300, 8, 2, 128
    q, k, v = cuda(*synth.qkv(B, 1, Sk, H, KVH, D, "bf16", seed=4))
    bias = synth.normal_tensor((B, H, 1, 384), 4, synth.TID_BIAS, "bf16").cuda()
    mask = bm = None
    if with_mask:
        mask = oracle_topk_mask(bias, Sk, 50)
        bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask)
    _check_full(q, k, v, "bf16", mask=mask, bias=bias, bm=bm, need_dbias=True, seed=4,
                what="swap")


def _check_groups(name, li, groups, dq, dk, dv, dbias=None, seed=5, what=""):
    """(b, KV head) groups of a full-size backward against the oracle, head by
    head on the host pool: dQ of the G heads, dK / dV summed over them, and
    (with a bias per KV head, broadcast over queries) dbias."""
    cfg = synth.CONFIGS[name]
    G = cfg["H"] // cfg["KVH"]
    jobs = [(name, li, b, kvh * G + g, seed) for b, kvh in groups for g in range(G)]
    res = oracle_pool.run(oracle_pool.bwd_head, jobs)
    for i, (b, kvh) in enumerate(groups):
        part = res[i * G:(i + 1) * G]
        say("backward group", what, b, kvh)
        rq = np.stack([r[0] for r in part], axis=1)
        rk = sum(r[1] for r in part)
        rv = sum(r[2] for r in part)
        _close(dq[b, :, kvh * G:(kvh + 1) * G].float().cpu().numpy(), rq, "bf16", f"{what} dq")
        _close(dk[b, :, kvh].float().cpu().numpy(), rk, "bf16", f"{what} dk")
        _close(dv[b, :, kvh].float().cpu().numpy(), rv, "bf16", f"{what} dv")
        if dbias is not None:
            rdb = sum(r[3] for r in part)
            _close(dbias[b, kvh, 0].float().cpu().numpy(), rdb, "bf16", f"{what} dbias")


@pytest.mark.parametrize("li", [0, 1], ids=["full", "sliding"])
def test_dflash_train_backward_groups(li):
    """The DFlash training shape, each layer: three (b, KV group)s of the
    backward checked in full against the oracle."""
    name = "dflash_train_bf16"
    cfg = synth.CONFIGS[name]
    layer = cfg["layers"][li]
    d = bsm.DFlash(cfg["ctx_len"], cfg["num_blocks"], cfg["block_size"],
                   is_causal=layer["is_causal"], layer_type=layer["layer_type"],
                   sliding_window=layer["window"])
    q, k, v = cuda(*synth.qkv(cfg["B"], d.Sq, d.Sk, cfg["H"], cfg["KVH"], cfg["D"], "bf16",
                              seed=0, scale=cfg["qkv_scale"]))
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), pred=d)
    do, dq, dk, dv, _ = _run(q, k, v, "bf16", pred=d, bm=bm, seed=5,
                             what=f"dflash train {layer['name']}")
    del q, k, v, do
    _check_groups(name, li, [(0, 0), (1, 5), (0, 7)], dq, dk, dv, what=layer["name"])


def test_dynamic_topk_backward_groups():
    """The dynamic-mask workload (Sq = Sk = 8000, top-2048 of a bias per KV
    head broadcast over queries, 2D padding): backward with dbias; two
    (b, KV group)s in full against the oracle (its own top-k mask), dbias of
    those groups summed over their heads and queries."""
    name = "dynamic_topk_bf16"
    cfg = synth.CONFIGS[name]
    B, H, KVH, D, Sq, Sk = (cfg[x] for x in ("B", "H", "KVH", "D", "Sq", "Sk"))
    q, k, v = cuda(*synth.qkv(B, Sq, Sk, H, KVH, D, "bf16", seed=0))
    bias, pad2d = [t.cuda() for t in synth.topk_inputs(cfg, seed=0)]
    mask = bsm.create_mask(bias, pad2d, B, Sq, Sk, cfg["topk"])
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask)
    do, dq, dk, dv, dbias = _run(q, k, v, "bf16", mask=mask, bias=bias, bm=bm, need_dbias=True,
                                 seed=5, what="dynamic top-k")
    del q, k, v, do
    _check_groups(name, 0, [(0, 1), (1, 3)], dq, dk, dv, dbias, what="dynamic")
