"""GPU parity: short query blocks with the heads of a KV group packed into one
workgroup and the key tiles split over several workgroups (k_attn_group and
the merge of the splits), against the fp64 oracle at the bf16 bars (max|err|
<= 2e-2, mean|err| <= 2e-3 on O and LSE, -inf exactly), and against the
unsplit launch of the same call."""

import numpy as np
import pytest
import torch

from gpu_helpers import (assert_close, bsm, cuda, oracle, oracle_geom, oracle_rows,
                         oracle_topk_mask, say, synth)

pytestmark = pytest.mark.gpu


def _ws_bytes(q, k, v, **kw):
    """Workspace bytes the library asks for (0: no split)."""
    import ctypes
    geom = bsm.geometry_of(q, k)
    a = bsm.AttnArgs()
    a.q, a.k, a.v = bsm.tensor4(q), bsm.tensor4(k), bsm.tensor4(v)
    a.o = q.data_ptr()
    for i in range(4):
        a.o_stride[i] = q.stride(i)
    keep = []
    for name in ("mask", "bias"):
        t = kw.get(name)
        if t is not None:
            c = bsm.tensor4(t)
            keep.append(c)
            setattr(a, name, ctypes.pointer(c))
    if kw.get("pred") is not None:
        pc = kw["pred"].c()
        keep.append(pc)
        a.pred = ctypes.pointer(pc)
    if kw.get("bm") is not None:
        bc = kw["bm"].c()
        keep.append(bc)
        a.bm = ctypes.pointer(bc)
    n = ctypes.c_int64(0)
    bsm._check(bsm.lib().attn_fwd_workspace_size(ctypes.byref(geom.c()), ctypes.byref(a),
                                                 ctypes.byref(n)))
    return n.value


def _check(q, k, v, what, mask=None, bias=None, pred=None, bm=None, heads=None,
           expect_split=True):
    if expect_split:
        assert _ws_bytes(q, k, v, mask=mask, bias=bias, pred=pred, bm=bm) > 0, what
    say("group attention", what, tuple(q.shape), tuple(k.shape))
    o, lse = bsm.masked_attn_fwd(q, k, v, pred=pred, mask=mask, bias=bias, block_mask=bm,
                                 return_lse=True)
    o1, lse1 = bsm.masked_attn_fwd(q, k, v, pred=pred, mask=mask, bias=bias, block_mask=bm,
                                   return_lse=True, split=False)
    torch.cuda.synchronize()
    B, Sq, H, D = q.shape
    om = oracle_geom(pred) if pred is not None else mask
    rows = np.arange(Sq)
    o_np, lse_np = o.float().cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        for h in (range(H) if heads is None else heads):
            want_o, want_l = oracle_rows(q, k, v, b, h, rows, mask=om, bias=bias)
            assert_close(o_np[b, :, h], want_o, "bf16", f"{what} O b={b} h={h}")
            assert_close(lse_np[b, h], want_l, "bf16", f"{what} LSE b={b} h={h}")
    # split and unsplit launches agree to bf16 rounding
    d = (o.float() - o1.float()).abs().max().item()
    assert d <= 2e-2, f"{what}: split vs unsplit O differ by {d}"
    fin = torch.isfinite(lse1)
    assert torch.equal(torch.isfinite(lse), fin)
    assert (lse[fin] - lse1[fin]).abs().max().item() <= 1e-3 if fin.any() else True


@pytest.mark.parametrize("Sq", [7, 10, 16])
@pytest.mark.parametrize("D", [64, 128])
def test_packed_heads_dense_mask_and_bias(Sq, D):
    """G = 4 heads packed (28, 40 and 64 rows: one or two row blocks, rows past
    G*Sq idle), a per-KV-head mask with its block mask, per-head bias, ragged Sk."""
    B, Sk, H, KVH = 2, 3000, 8, 2
    q, k, v = cuda(*synth.qkv(B, Sq, Sk, H, KVH, D, "bf16", seed=80 + Sq))
    m = synth.random_bool((B, KVH, Sq, 3072), 0.3, 80, synth.TID_MASK)
    m[..., 1000:1300] = False                        # some empty tiles in the list
    m[0, 1, 3] = False                               # a fully masked row of 4 heads
    mask = torch.from_numpy(m).cuda()
    bias = synth.normal_tensor((B, H, Sq, 3072), 80, synth.TID_BIAS, "bf16").cuda()
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask)
    _check(q, k, v, f"packed Sq={Sq} D={D}", mask=mask, bias=bias, bm=bm)


@pytest.mark.parametrize("layer", [dict(), dict(is_causal=True, layer_type="sliding",
                                                sliding_window=500)])
def test_packed_dflash_inference_split(layer):
    """A draft block of 16 against a 6000-token cache, 2 requests: 4 heads x 16
    rows packed (two row blocks), many splits, a window that leaves most splits
    with one tile or none."""
    d = bsm.DFlash.inference(6000, 16, **layer)
    q, k, v = cuda(*synth.qkv(2, d.Sq, d.Sk, 8, 2, 128, "bf16", seed=81, scale=0.5))
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), pred=d)
    _check(q, k, v, f"inference {layer}", pred=d, bm=bm)
    _check(q, k, v, f"inference {layer} no bm", pred=d, heads=[0, 7])


def test_per_head_block_mask_splits_without_packing():
    """A per-head block mask keeps one head per workgroup; the keys still split."""
    B, Sq, Sk, H, KVH, D = 1, 12, 5000, 4, 1, 128
    q, k, v = cuda(*synth.qkv(B, Sq, Sk, H, KVH, D, "bf16", seed=82))
    m = synth.random_bool((B, H, Sq, 5120), 0.05, 82, synth.TID_MASK)
    m[:, 2, :, :4000] = False
    mask = torch.from_numpy(m).cuda()
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask)
    _check(q, k, v, "per-head bm", mask=mask, bm=bm)


@pytest.mark.parametrize("B", [1, 3])
def test_swapped_decode_few_sequences(B):
    """seqlen_q == 1 with few sequences: G rows per KV head after the swap, the
    keys of each split over up to 32 workgroups, top-k mask and bias."""
    Sk, H, KVH, D = 16384, 32, 8, 128
    q, k, v = cuda(*synth.qkv(B, 1, Sk, H, KVH, D, "bf16", seed=83))
    bias = synth.normal_tensor((B, H, 1, Sk), 83, synth.TID_BIAS, "bf16").cuda()
    mask = oracle_topk_mask(bias, Sk, 1024)
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask)
    _check(q, k, v, f"swap B={B}", mask=mask, bias=bias, bm=bm, heads=[0, 5, 31])
    _check(q, k, v, f"swap B={B} no mask", heads=[0, 30])
