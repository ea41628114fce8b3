"""GPU parity: packed variable-length sequences -- unpad / pad and the packing
index bit-exact against oracle.varlen, per-sequence DFlash block masks
bit-exact, packed attention against the fp64 oracle (bf16: max|err| <=
2e-2, mean|err| <= 2e-3; f32: max|err| <= 1e-4; -inf LSE exactly), and its
gradients against the fp64 oracle (the same bars scaled by max(1, max|ref|))."""

import numpy as np
import pytest
import torch

from gpu_helpers import assert_bm_equal, assert_close, assert_grad_close, bsm, np_bm, say, synth
from oracle.attention_bwd import group_grads
from oracle.varlen import (attention_varlen, attention_varlen_bwd, block_mask_varlen,
                           dflash_varlen_geoms, pad, unpad)

pytestmark = pytest.mark.gpu


def test_unpad_pad_match_oracle():
    B, S, H, D = 5, 300, 4, 64
    x = synth.normal_tensor((B, S, H, D), 70, synth.TID_Q, "bf16")
    valid = synth.random_bool((B, S), 0.6, 70, synth.TID_MASK)
    valid[1] = False          # an empty sequence
    valid[3] = True           # a full one
    say("unpad", B, S)
    packed, idx, cu, mx = bsm.unpad(x.cuda(), torch.from_numpy(valid).cuda())
    torch.cuda.synchronize()
    wp, wi, wc, wm = unpad(x.view(torch.int16).numpy(), valid)
    np.testing.assert_array_equal(cu.cpu().numpy(), wc)
    np.testing.assert_array_equal(idx.cpu().numpy(), wi)
    assert mx == wm
    np.testing.assert_array_equal(packed.cpu().view(torch.int16).numpy(), wp)
    back = bsm.pad(packed, idx, B, S)
    np.testing.assert_array_equal(back.cpu().view(torch.int16).numpy(),
                                  pad(wp, wi, B, S))


def _pack(seqs, H, KVH, D, dt, seed):
    """Packed q, k, v and cu arrays for [(queries, keys), ...]."""
    sq = [a for a, _ in seqs]
    sk = [b for _, b in seqs]
    cu_q = np.r_[0, np.cumsum(sq)].astype(np.int32)
    cu_k = np.r_[0, np.cumsum(sk)].astype(np.int32)
    q, k, v = synth.qkv(1, int(cu_q[-1]), int(cu_k[-1]), H, KVH, D, dt, seed=seed, scale=0.5)
    return q[0], k[0], v[0], cu_q, cu_k


def _dflash_seqs(bs, layout):
    """(queries, keys) of DFlash sequences given as (context, blocks)."""
    return [(nb * bs, c + nb * bs) for c, nb in layout]


LAYERS = [dict(), dict(layer_type="sliding", sliding_window=100),
          dict(is_causal=True), dict(is_causal=False, layer_type="sliding", sliding_window=37)]


def _id(c):
    return "-".join(f"{k}{v}" for k, v in c.items()) or "full"


@pytest.mark.parametrize("layer", LAYERS, ids=[_id(c) for c in LAYERS])
def test_varlen_block_mask(layer):
    bs = 16
    seqs = _dflash_seqs(bs, [(100, 2), (0, 0), (300, 10), (4096, 16), (0, 3)])
    cu_q = np.r_[0, np.cumsum([a for a, _ in seqs])].astype(np.int32)
    cu_k = np.r_[0, np.cumsum([b for _, b in seqs])].astype(np.int32)
    vl = bsm.Varlen(torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda(), 8, 2, 128)
    pred = bsm.varlen_dflash(bs, **layer)
    say("varlen block mask", layer)
    got = np_bm(bsm.build_block_mask_varlen(vl, pred))
    want = block_mask_varlen(dflash_varlen_geoms(cu_q, cu_k, bs, **layer))
    assert_bm_equal(got, want, str(layer))


def _check(seqs, H, KVH, D, dt, layer, bs=16, use_bm=True, seed=0, what=""):
    q, k, v, cu_q, cu_k = _pack(seqs, H, KVH, D, dt, seed)
    vl = bsm.Varlen(torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda(), H, KVH, D)
    pred = None if layer is None else bsm.varlen_dflash(bs, **layer)
    bm = bsm.build_block_mask_varlen(vl, pred) if (pred is not None and use_bm) else None
    say("varlen attention", what, seqs, H, KVH, D, dt, layer)
    o, lse = bsm.masked_attn_varlen_fwd(q.cuda(), k.cuda(), v.cuda(), vl, pred=pred,
                                        block_mask=bm, return_lse=True)
    torch.cuda.synchronize()
    geoms = None if layer is None else dflash_varlen_geoms(cu_q, cu_k, bs, **layer)
    wo, wl = attention_varlen(synth.as_f64(q), synth.as_f64(k), synth.as_f64(v), cu_q, cu_k,
                              geoms=geoms)
    assert_close(o.float().cpu().numpy(), wo, dt, f"{what} O")
    assert_close(lse.cpu().numpy(), wl, dt, f"{what} LSE")


@pytest.mark.parametrize("layer", LAYERS, ids=[_id(c) for c in LAYERS])
@pytest.mark.parametrize("H,KVH,D,dt", [(8, 2, 128, "bf16"), (4, 2, 64, "bf16"),
                                        (3, 3, 128, "bf16"), (4, 2, 64, "f32")])
def test_varlen_dflash_attention(layer, H, KVH, D, dt):
    """Two-head kernel (G even), the one-head kernel (G = 1) and the float
    kernel; sequences with no queries, no context, ragged tiles."""
    seqs = _dflash_seqs(16, [(100, 2), (0, 0), (300, 10), (0, 3), (700, 1)])
    _check(seqs, H, KVH, D, dt, layer, what="dflash")


def test_varlen_without_block_mask_and_without_mask():
    seqs = _dflash_seqs(16, [(135, 9), (257, 1), (0, 2)])
    _check(seqs, 8, 2, 128, "bf16", dict(layer_type="sliding", sliding_window=64),
           use_bm=False, what="no bm")
    # no mask: every sequence attends to all its keys (keys may outnumber queries)
    _check([(200, 333), (1, 7), (0, 5), (129, 129)], 8, 2, 128, "bf16", None, what="no mask")
    _check([(200, 333), (1, 7), (129, 129)], 4, 4, 64, "f32", None, what="no mask f32")


def test_varlen_training_shape_sampled():
    """Four DFlash sequences of different lengths packed together (about the
    size of the two-sequence training batch): every row of a few heads."""
    bs = 16
    layout = [(4096, 256), (2048, 128), (1024, 64), (3008, 47)]
    seqs = _dflash_seqs(bs, layout)
    H, KVH, D = 32, 8, 128
    q, k, v, cu_q, cu_k = _pack(seqs, H, KVH, D, "bf16", 3)
    layer = dict(layer_type="sliding", sliding_window=2048)
    vl = bsm.Varlen(torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda(), H, KVH, D)
    pred = bsm.varlen_dflash(bs, **layer)
    bm = bsm.build_block_mask_varlen(vl, pred)
    o, lse = bsm.masked_attn_varlen_fwd(q.cuda(), k.cuda(), v.cuda(), vl, pred=pred,
                                        block_mask=bm, return_lse=True)
    torch.cuda.synchronize()
    geoms = dflash_varlen_geoms(cu_q, cu_k, bs, **layer)
    o_np = o.float().cpu().numpy()
    lse_np = lse.cpu().numpy()
    from oracle import attention_rows
    for b in (1, 3):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        rows = np.unique(np.r_[0, q1 - q0 - 1, np.linspace(0, q1 - q0 - 1, 12).astype(int)])
        for h in (0, 17):
            say("oracle seq", b, "head", h)
            wo, wl = attention_rows(synth.as_f64(q[None, q0:q1]), synth.as_f64(k[None, k0:k1]),
                                    synth.as_f64(v[None, k0:k1]), 0, h, rows, mask=geoms[b])
            assert_close(o_np[q0 + rows, h], wo, "bf16", f"O seq={b} h={h}")
            assert_close(lse_np[h, q0 + rows], wl, "bf16", f"LSE seq={b} h={h}")


def _bwd(seqs, H, KVH, D, dt, layer, bs=16, use_bm=True, seed=0, what=""):
    """GPU forward + backward of packed sequences; returns the inputs, dO and
    the gradients (dq, dk, dv) on the host."""
    q, k, v, cu_q, cu_k = _pack(seqs, H, KVH, D, dt, seed)
    do = synth.normal_tensor(tuple(q.shape), seed, synth.TID_DOUT, dt)
    vl = bsm.Varlen(torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda(), H, KVH, D)
    pred = None if layer is None else bsm.varlen_dflash(bs, **layer)
    bm = bsm.build_block_mask_varlen(vl, pred) if (pred is not None and use_bm) else None
    say("varlen backward", what, seqs if len(seqs) < 8 else len(seqs), H, KVH, D, dt, layer)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    o, lse = bsm.masked_attn_varlen_fwd(qc, kc, vc, vl, pred=pred, block_mask=bm,
                                        return_lse=True)
    dq, dk, dv = bsm.masked_attn_varlen_bwd(qc, kc, vc, o, do.cuda(), lse, vl, pred=pred,
                                            block_mask=bm)
    torch.cuda.synchronize()
    return (q, k, v, do, cu_q, cu_k), tuple(x.float().cpu().numpy() for x in (dq, dk, dv))


def _check_bwd(seqs, H, KVH, D, dt, layer, bs=16, use_bm=True, seed=0, what=""):
    (q, k, v, do, cu_q, cu_k), (dq, dk, dv) = _bwd(seqs, H, KVH, D, dt, layer, bs, use_bm,
                                                   seed, what)
    geoms = None if layer is None else dflash_varlen_geoms(cu_q, cu_k, bs, **layer)
    rq, rk, rv = attention_varlen_bwd(synth.as_f64(q), synth.as_f64(k), synth.as_f64(v),
                                      synth.as_f64(do), cu_q, cu_k, geoms=geoms)
    for b in range(len(seqs)):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        assert_grad_close(dq[q0:q1], rq[q0:q1], dt, f"{what} seq {b} dq")
        assert_grad_close(dk[k0:k1], rk[k0:k1], dt, f"{what} seq {b} dk")
        assert_grad_close(dv[k0:k1], rv[k0:k1], dt, f"{what} seq {b} dv")
        if q1 == q0:          # keys that no query sees: exactly zero
            assert not dk[k0:k1].any() and not dv[k0:k1].any(), f"{what} seq {b}"


@pytest.mark.parametrize("layer", LAYERS, ids=[_id(c) for c in LAYERS])
@pytest.mark.parametrize("H,KVH,D,dt", [(8, 2, 128, "bf16"), (4, 2, 64, "bf16"),
                                        (3, 3, 128, "bf16"), (6, 2, 128, "bf16"),
                                        (4, 2, 64, "f32")])
def test_varlen_dflash_backward(layer, H, KVH, D, dt):
    """Matrix-core backward (bf16) in one launch per kernel, with head pairs
    (even G) and one head per dQ workgroup (G = 1, 3), and the float kernels;
    sequences with no queries (with and without keys), no context, ragged
    tiles."""
    seqs = _dflash_seqs(16, [(100, 2), (0, 0), (300, 10), (50, 0), (0, 3), (700, 1)])
    _check_bwd(seqs, H, KVH, D, dt, layer, what="dflash")


def test_varlen_backward_without_block_mask_and_without_mask():
    seqs = _dflash_seqs(16, [(135, 9), (257, 1), (0, 2)])
    _check_bwd(seqs, 8, 2, 128, "bf16", dict(layer_type="sliding", sliding_window=64),
               use_bm=False, what="no bm")
    _check_bwd([(200, 333), (1, 7), (0, 5), (129, 129)], 8, 2, 128, "bf16", None,
               what="no mask")
    _check_bwd([(200, 333), (1, 7), (129, 129)], 4, 4, 64, "f32", None, what="no mask f32")


def test_varlen_backward_training_shape_sampled():
    """The packed training-size batch of the forward test: every gradient of
    two KV groups of two sequences against the oracle."""
    bs = 16
    seqs = _dflash_seqs(bs, [(4096, 256), (2048, 128), (1024, 64), (3008, 47)])
    H, KVH, D = 32, 8, 128
    layer = dict(layer_type="sliding", sliding_window=2048)
    (q, k, v, do, cu_q, cu_k), (dq, dk, dv) = _bwd(seqs, H, KVH, D, "bf16", layer, seed=3,
                                                   what="training size")
    geoms = dflash_varlen_geoms(cu_q, cu_k, bs, **layer)
    G = H // KVH
    for b in (1, 3):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        for kvh in (0, 5):
            say("oracle seq", b, "group", kvh)
            rq, rk, rv = group_grads(synth.as_f64(q[None, q0:q1]), synth.as_f64(k[None, k0:k1]),
                                     synth.as_f64(v[None, k0:k1]), synth.as_f64(do[None, q0:q1]),
                                     0, kvh, mask=geoms[b])
            w = f"seq {b} group {kvh}"
            assert_grad_close(dq[q0:q1, kvh * G:(kvh + 1) * G], rq, "bf16", f"{w} dq")
            assert_grad_close(dk[k0:k1, kvh], rk, "bf16", f"{w} dk")
            assert_grad_close(dv[k0:k1, kvh], rv, "bf16", f"{w} dv")


def test_varlen_backward_many_sequences():
    """70 short sequences (more than the host work orders take): the kernels'
    own mapping of (sequence, tile) items; with and without a DFlash mask."""
    rng = np.random.default_rng(9)
    layout = [(int(c), int(nb)) for c, nb in zip(rng.integers(0, 90, 70), rng.integers(0, 4, 70))]
    layout = [(c - c % nb if nb else c, nb) for c, nb in layout]   # context a multiple of blocks
    seqs = _dflash_seqs(16, layout)
    _check_bwd(seqs, 8, 2, 128, "bf16", dict(is_causal=True), what="70 seqs dflash")
    _check_bwd(seqs, 3, 1, 128, "bf16", dict(is_causal=True), what="70 seqs dflash G=3")
    _check_bwd([(int(a), int(b)) for a, b in zip(rng.integers(0, 40, 70), rng.integers(0, 60, 70))],
               8, 2, 128, "bf16", None, what="70 seqs no mask")


def test_varlen_backward_queries_without_keys():
    """No mask: a sequence with queries and no keys has zero dQ (its rows keep
    nothing), beside ordinary ones."""
    _check_bwd([(40, 0), (130, 77), (0, 9), (17, 200)], 8, 2, 128, "bf16", None,
               what="queries without keys")
