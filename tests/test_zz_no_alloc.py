"""GPU check of masked_attn_fwd_noalloc, the forward entry point that allocates
nothing: on the plans that use a workspace (key splits of a few decoding
sequences; staged query-broadcast mask / bias rows), two calls in a row, the
second on a smaller input, each bit-equal to masked_attn_fwd given its own
workspace, and the first call's scratch contents never leaking into the
second's result."""

import pytest
import torch

from gpu_helpers import bsm, cuda, oracle_topk_mask, say, synth

pytestmark = pytest.mark.gpu


def _need(q, k, v, **kw):
    """Workspace bytes masked_attn_fwd asks for these arguments."""
    import ctypes
    geom, a, keep, _, _, _ = bsm._fwd_args(q, k, v, kw.get("pred"), kw.get("mask"),
                                           kw.get("bias"), kw.get("block_mask"), None, True,
                                           None, None, None)
    n = ctypes.c_int64(0)
    bsm._check(bsm.lib().attn_fwd_workspace_size(ctypes.byref(geom.c()), ctypes.byref(a),
                                                  ctypes.byref(n)))
    return n.value


def _decode(B, Sk, seed):
    H, KVH, D = 32, 8, 128
    q, k, v = cuda(*synth.qkv(B, 1, Sk, H, KVH, D, "bf16", seed=seed))
    K = (Sk + 127) // 128 * 128
    bias = synth.normal_tensor((B, H, 1, K), seed, synth.TID_BIAS, "bf16").cuda()
    mask = oracle_topk_mask(bias, Sk, min(1024, Sk // 4))
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask)
    return q, k, v, dict(mask=mask, bias=bias, block_mask=bm)


def _staged(B, Sq, Sk, seed):
    H, KVH, D = 16, 4, 128
    q, k, v = cuda(*synth.qkv(B, Sq, Sk, H, KVH, D, "bf16", seed=seed))
    K = (Sk + 127) // 128 * 128
    bias = synth.normal_tensor((B, KVH, 1, K), seed, synth.TID_BIAS, "bf16").cuda()
    mask = oracle_topk_mask(bias, Sk, Sk // 4)
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask)
    return q, k, v, dict(mask=mask, bias=bias, block_mask=bm)


def _compare(q, k, v, kw, what):
    need = _need(q, k, v, **kw)
    say("noalloc", what, tuple(q.shape), tuple(k.shape), "workspace", need)
    assert 0 < need <= bsm.NOALLOC_SCRATCH_BYTES
    want_o, want_l = bsm.masked_attn_fwd(q, k, v, return_lse=True, **kw)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((q.shape[0], q.shape[2], q.shape[1]), float("nan"), device=q.device)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    bsm.masked_attn_fwd_noalloc(q, k, v, out, lse, **kw)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.equal(out, want_o), f"{what}: O differs"
    assert torch.equal(lse, want_l), f"{what}: LSE differs"


def test_noalloc_decode_splits_twice():
    """Few sequences against a long KV cache: the key splits' partial states
    live in the scratch; the second, smaller call reuses it."""
    _compare(*_decode(4, 30000, 60), "decode B=4 Sk=30000")
    _compare(*_decode(1, 3000, 61), "decode B=1 Sk=3000")


def test_noalloc_staged_rows_twice():
    """A query-broadcast mask and bias folded into staged rows in the
    scratch; the second, smaller call reuses it."""
    _compare(*_staged(2, 700, 6000, 62), "staged B=2 Sq=700 Sk=6000")
    _compare(*_staged(1, 300, 1000, 63), "staged B=1 Sq=300 Sk=1000")


def test_noalloc_without_workspace_plan():
    """A call whose plan uses no workspace runs as masked_attn_fwd does."""
    d = bsm.DFlash(256, 4, 16)
    q, k, v = cuda(*synth.qkv(1, d.Sq, d.Sk, 4, 2, 128, "bf16", seed=64))
    assert _need(q, k, v, pred=d) == 0
    want = bsm.masked_attn_fwd(q, k, v, pred=d)
    out = torch.empty_like(q)
    bsm.masked_attn_fwd_noalloc(q, k, v, out, pred=d)
    torch.cuda.synchronize()
    assert torch.equal(out, want)


def test_noalloc_refuses_a_workspace_and_oversize_plans():
    q, k, v, kw = _decode(1, 3000, 65)
    out = torch.empty_like(q)
    import ctypes
    geom, a, keep, _, _, _ = bsm._fwd_args(q, k, v, None, kw["mask"], kw["bias"],
                                           kw["block_mask"], None, False, out, None, None)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    st = bsm.lib().masked_attn_fwd_noalloc(ctypes.byref(geom.c()), ctypes.byref(a),
                                           bsm._stream(None))
    assert st == bsm.BSM_E_ARG
