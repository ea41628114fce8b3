"""GPU check of the binding's stream= argument: every call made on a side
stream (the library's temporaries allocated on the current stream, the inputs
written there) gives results bit-equal to the same calls on the current
stream. Covers top-k, block mask, key list, the forward with a split
workspace and with a key list, the backward with its workspace and dbias,
unpad (with its read-back of the sequence lengths) and pad."""

import pytest
import torch

from gpu_helpers import bsm, cuda, say, synth

pytestmark = pytest.mark.gpu


def _work(stream):
    outs = []
    # a few decoding sequences: the forward splits keys with a workspace
    B, Sk, H, KVH, D = 2, 20000, 32, 8, 128
    q, k, v = cuda(*synth.qkv(B, 1, Sk, H, KVH, D, "bf16", seed=70))
    bias = synth.normal_tensor((B, H, 1, 20096), 70, synth.TID_BIAS, "bf16").cuda()
    geom = bsm.geometry_of(q, k)
    mask = bsm.dynamic_topk_mask(bias, None, Sk, 512, stream=stream)
    bm = bsm.build_block_mask(geom, mask=mask, stream=stream)
    keys = bsm.build_key_list(geom, mask, stream=stream)
    o, lse = bsm.masked_attn_fwd(q, k, v, mask=mask, bias=bias, block_mask=bm,
                                 return_lse=True, stream=stream)
    og = bsm.masked_attn_fwd(q, k, v, mask=mask, bias=bias, keys=keys, stream=stream)
    outs += [mask, *bm, keys.num_keys, o, lse, og]
    # backward with a full bias and its gradient
    B, Sq, Sk, H, KVH, D = 2, 150, 200, 4, 2, 64
    q, k, v = cuda(*synth.qkv(B, Sq, Sk, H, KVH, D, "bf16", seed=71))
    m = synth.random_bool((B, H, Sq, 256), 0.3, 71, synth.TID_MASK)
    m[..., 5] = True
    mask = torch.from_numpy(m).cuda()
    bias = synth.normal_tensor((B, H, Sq, 256), 71, synth.TID_BIAS, "bf16").cuda()
    bm = bsm.build_block_mask(bsm.geometry_of(q, k), mask=mask, stream=stream)
    o, lse = bsm.masked_attn_fwd(q, k, v, mask=mask, bias=bias, block_mask=bm,
                                 return_lse=True, stream=stream)
    do = synth.normal_tensor(tuple(q.shape), 71, synth.TID_DOUT, "bf16").cuda()
    dq, dk, dv, db = bsm.masked_attn_bwd(q, k, v, o, do, lse, mask=mask, bias=bias,
                                         block_mask=bm, need_dbias=True, stream=stream)
    outs += [o, lse, dq, dk, dv, db]
    # unpad / pad of a ragged batch
    x = synth.normal_tensor((3, 100, 4, 64), 72, synth.TID_DOUT, "bf16").cuda()
    valid = torch.from_numpy(synth.random_bool((3, 100), 0.6, 72, synth.TID_MASK)).cuda()
    packed, idx, cu, mx = bsm.unpad(x, valid, stream=stream)
    back = bsm.pad(packed, idx, 3, 100, stream=stream)
    outs += [packed, idx, cu, back, torch.tensor(mx)]
    torch.cuda.synchronize()
    return outs


def test_side_stream_matches_current_stream():
    say("streams: current")
    ref = _work(None)
    side = torch.cuda.Stream()
    say("streams: side")
    got = _work(side)
    assert len(got) == len(ref)
    for i, (g, r) in enumerate(zip(got, ref)):
        assert g.shape == r.shape and g.dtype == r.dtype, i
        assert torch.equal(g.cpu(), r.cpu()), f"output {i} differs on the side stream"
    # and pad(unpad(x)) is x on the valid rows, zero elsewhere
    x = synth.normal_tensor((3, 100, 4, 64), 72, synth.TID_DOUT, "bf16")
    valid = torch.from_numpy(synth.random_bool((3, 100), 0.6, 72, synth.TID_MASK))
    want = torch.where(valid[:, :, None, None], x, torch.zeros_like(x))
    assert torch.equal(got[-2].cpu(), want)
