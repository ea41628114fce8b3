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

from gpu_helpers import bsm, cuda, oracle_geom, say, synth
from oracle.attention_bwd import attention_bwd, group_grads

pytestmark = pytest.mark.gpu


def _close(got, want, dt, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    m = max(1.0, float(np.abs(want).max()) if want.size else 1.0)
    err = np.abs(got - want)
    if err.size == 0:
        return
    if dt == "bf16":
        assert err.max() <= 2e-2 * m, f"{what}: max |err| {err.max():.3e} > {2e-2 * m:.3e}"
        assert err.mean() <= 2e-3 * m, f"{what}: mean |err| {err.mean():.3e} > {2e-3 * m:.3e}"
    else:
        assert err.max() <= 1e-4 * m, f"{what}: max |err| {err.max():.3e} > {1e-4 * m:.3e}"


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


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("mshape,bshape", [
    ((2, 4, 150, 256), (2, 4, 150, 256)),   # full bias: dbias = dS
    ((1, 1, 1, 256), (2, 2, 1, 256)),       # bias per KV head, broadcast over queries
    ((2, 2, 1, 256), (1, 4, 150, 256)),     # bias broadcast over batch
    (None, (1, 1, 1, 256)),                 # one bias row for everything
    (None, None),
])
def test_dense_mask_and_bias(dt, mshape, bshape):
    B, Sq, Sk, H, KVH, D = 2, 150, 200, 4, 2, 64
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


def test_fully_masked_rows():
    B, Sq, Sk, H, KVH, D = 1, 130, 200, 2, 1, 64
    q, k, v = cuda(*synth.qkv(B, Sq, Sk, H, KVH, D, "bf16", seed=3))
    m = np.zeros((1, 1, Sq, 256), bool)
    m[0, 0, ::3, 7] = True
    m[0, 0, 1::3, :] = True
    mask = torch.from_numpy(m).cuda()
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask)
    _check_full(q, k, v, "bf16", mask=mask, bm=bm, seed=3, what="masked rows")


@pytest.mark.parametrize("with_mask", [True, False])
def test_decode_swap(with_mask):
    """Sq == 1 with H > KVH: the head-group swap, with a per-head bias."""
    B, Sk, H, KVH, D = 3, 300, 8, 2, 128
    q, k, v = cuda(*synth.qkv(B, 1, Sk, H, KVH, D, "bf16", seed=4))
    bias = synth.normal_tensor((B, H, 1, 384), 4, synth.TID_BIAS, "bf16").cuda()
    mask = bm = None
    if with_mask:
        mask = bsm.dynamic_topk_mask(bias, None, Sk, 50)
        bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask)
    _check_full(q, k, v, "bf16", mask=mask, bias=bias, bm=bm, need_dbias=True, seed=4,
                what="swap")


def test_dflash_train_layer_sampled():
    """The DFlash training shape's sliding layer, one (b, KV group) checked in
    full against the oracle."""
    cfg = synth.CONFIGS["dflash_train_bf16"]
    layer = cfg["layers"][1]
    d = bsm.DFlash(cfg["ctx_len"], cfg["num_blocks"], cfg["block_size"],
                   is_causal=layer["is_causal"], layer_type=layer["layer_type"],
                   sliding_window=layer["window"])
    q, k, v = cuda(*synth.qkv(cfg["B"], d.Sq, d.Sk, cfg["H"], cfg["KVH"], cfg["D"], "bf16",
                              seed=0, scale=cfg["qkv_scale"]))
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), pred=d)
    do, dq, dk, dv, _ = _run(q, k, v, "bf16", pred=d, bm=bm, seed=5, what="dflash train sliding")
    G = cfg["H"] // cfg["KVH"]
    for b, kvh in ((1, 5),):
        say("oracle group", b, kvh)
        rq, rk, rv = group_grads(synth.as_f64(q[b:b + 1]), synth.as_f64(k[b:b + 1]),
                                 synth.as_f64(v[b:b + 1]), synth.as_f64(do[b:b + 1]), 0, kvh,
                                 mask=oracle_geom(d))
        _close(dq[b, :, kvh * G:(kvh + 1) * G].float().cpu().numpy(), rq, "bf16", "dq")
        _close(dk[b, :, kvh].float().cpu().numpy(), rk, "bf16", "dk")
        _close(dv[b, :, kvh].float().cpu().numpy(), rv, "bf16", "dv")
