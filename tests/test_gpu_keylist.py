"""GPU parity: the kept-key list (bit-exact against oracle.keylist) and
attention that visits only the listed keys (against the fp64 attention oracle
with the dense mask, at the bf16 bars: max|err| <= 2e-2, mean|err| <= 2e-3 on O
and LSE, -inf LSE exactly)."""

import numpy as np
import pytest
import torch

import oracle_pool
from gpu_helpers import assert_close, bsm, cuda, oracle_rows, oracle_topk_mask, say, synth
from oracle.keylist import key_list

pytestmark = pytest.mark.gpu


def _iter_mask(mask_np, geom):
    """The mask in the attention's iteration space (the swap regroups heads)."""
    B, H, KVH, Sq, Sk, D = geom
    if Sq == 1 and H > KVH and mask_np.shape[1] == H:
        b, _, _, K = mask_np.shape
        return mask_np.reshape(b, KVH, H // KVH, K)
    return mask_np


def _rows(geom):
    B, H, KVH, Sq, Sk, D = geom
    return H // KVH if (Sq == 1 and H > KVH) else Sq


def _assert_list_equal(got, want, what, pairs=None):
    """Compare num_keys and the first num_keys entries; pairs maps GPU list
    (b, h) to oracle list (b, h), all lists by default."""
    gn = got.num_keys.cpu().numpy()
    gk = got.key_indices.cpu().numpy()
    gb = got.row_bits.cpu().numpy().view(np.uint32)
    wn, wk, wb = want
    if pairs is None:
        pairs = [((b, h), (b, h)) for b in range(wn.shape[0]) for h in range(wn.shape[1])]
    for (b, h), (ob, oh) in pairs:
        n = int(wn[ob, oh])
        assert gn[b, h] == n, f"{what} ({b},{h}): num {gn[b, h]} != {n}"
        np.testing.assert_array_equal(gk[b, h, :n], wk[ob, oh, :n],
                                      err_msg=f"{what} ({b},{h}) keys")
        np.testing.assert_array_equal(gb[b, h, :n], wb[ob, oh, :n],
                                      err_msg=f"{what} ({b},{h}) bits")


LIST_CASES = [
    # geometry (B, H, KVH, Sq, Sk, D), mask shape, density
    ((4, 32, 8, 1, 4096, 128), (4, 32, 1, 4096), 0.06),   # swap: G = 4 rows per KV head
    ((3, 8, 2, 1, 1000, 64), (3, 2, 1, 1024), 0.3),       # swap, mask per KV head (broadcast)
    ((2, 8, 2, 20, 300, 64), (2, 2, 20, 384), 0.2),       # short prefill chunk, ragged Sk
    ((1, 4, 4, 32, 250, 128), (1, 4, 32, 256), 0.05),     # 32 rows, Sk not a multiple of 16
    ((2, 4, 2, 5, 9000, 128), (1, 1, 5, 9088), 0.01),     # broadcast over batch and heads, 3 passes
    ((2, 16, 4, 1, 512, 128), (2, 16, 1, 512), 0.0),      # nothing kept
]


@pytest.mark.parametrize("geom,shape,density", LIST_CASES)
def test_key_list_matches_oracle(geom, shape, density):
    say("key list", geom, shape, density)
    Sk = geom[4]
    m = synth.random_bool(shape, density, 3, synth.TID_MASK)
    m[..., Sk:] = synth.random_bool(m[..., Sk:].shape, 0.5, 4, synth.TID_MASK)  # ignored tail
    kl = bsm.build_key_list(geom, torch.from_numpy(m).cuda())
    torch.cuda.synchronize()
    want = key_list(_iter_mask(m, geom), Sk, _rows(geom))
    assert tuple(kl.key_indices.shape) == want[1].shape
    _assert_list_equal(kl, want, f"{geom} {shape}")


def test_key_list_decode_full_size_sampled():
    """Decode shape (B=64, H=32, KVH=8, Sk=16384, top-1024 per head), built
    from the oracle's top-k masks: lists of sampled (b, KV head) pairs against
    the oracle, and every list's count against the union of its four top-k
    rows."""
    name = "decode_swap_bf16"
    cfg = synth.CONFIGS[name]
    B, H, KVH, D, Sk = (cfg[x] for x in ("B", "H", "KVH", "D", "Sk"))
    geom = (B, H, KVH, 1, Sk, D)
    mask_np = np.concatenate(oracle_pool.run(oracle_pool.topk_mask_rows,
                                             [(name, b) for b in range(B)]))
    kl = bsm.build_key_list(geom, torch.from_numpy(mask_np).cuda())
    torch.cuda.synchronize()
    m = _iter_mask(mask_np, geom)
    union = m[..., :Sk].any(axis=2).sum(axis=-1)
    np.testing.assert_array_equal(kl.num_keys.cpu().numpy(), union)
    pairs = [(0, 0), (17, 3), (40, 7), (63, 5)]
    for b, h in pairs:
        say("oracle key list", b, h)
        want = key_list(m[b:b + 1, h:h + 1], Sk, H // KVH)
        _assert_list_equal(kl, want, "decode", [((b, h), (0, 0))])


def _gather_check(q, k, v, mask, bias, keys, what, heads=None):
    say("gather attention", what, tuple(q.shape), tuple(k.shape))
    o, lse = bsm.masked_attn_fwd(q, k, v, mask=mask, bias=bias, keys=keys, return_lse=True)
    torch.cuda.synchronize()
    B, Sq, H, D = q.shape
    rows = np.arange(Sq)
    heads = range(H) if heads is None else heads
    o_np = o.float().cpu().numpy()
    lse_np = lse.cpu().numpy()
    for b in range(B):
        for h in heads:
            want_o, want_l = oracle_rows(q, k, v, b, h, rows, mask=mask, bias=bias)
            assert_close(o_np[b, :, h, :], want_o, "bf16", f"{what} O b={b} h={h}")
            assert_close(lse_np[b, h], want_l, "bf16", f"{what} LSE b={b} h={h}")
    return o, lse


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("with_bias", [True, False])
def test_gather_decode_swap(D, with_bias):
    """Sq == 1, H > KVH: per-head top-k masks, the list of each KV group's union."""
    B, Sk, H, KVH = 3, 1000, 8, 2
    q, k, v = cuda(*synth.qkv(B, 1, Sk, H, KVH, D, "bf16", seed=30 + D))
    bias = synth.normal_tensor((B, H, 1, 1024), 30, synth.TID_BIAS, "bf16").cuda()
    mask = oracle_topk_mask(bias, Sk, 100)
    keys = bsm.build_key_list(bsm.geometry_of(q, k), mask)
    _gather_check(q, k, v, mask, bias if with_bias else None, keys, f"swap D={D}")


@pytest.mark.parametrize("Sq", [3, 20, 32])
def test_gather_short_prefill(Sq):
    """Short query blocks without the swap: per-query mask rows, a per-KV-head
    bias broadcast over queries, ragged Sk, several list tiles."""
    B, Sk, H, KVH, D = 2, 700, 4, 2, 128
    q, k, v = cuda(*synth.qkv(B, Sq, Sk, H, KVH, D, "bf16", seed=40 + Sq))
    m = synth.random_bool((B, H, Sq, 768), 0.15, 8, synth.TID_MASK)
    m[0, 1, 0] = False            # a row with no kept key
    m[1, :, :, 699] = True        # the last key
    mask = torch.from_numpy(m).cuda()
    bias = synth.normal_tensor((B, KVH, 1, 768), 8, synth.TID_BIAS, "bf16").cuda()
    keys = bsm.build_key_list(bsm.geometry_of(q, k), mask)
    o, lse = _gather_check(q, k, v, mask, bias, keys, f"prefill Sq={Sq}")
    assert (o[0, 0, 1].float() == 0).all() and torch.isneginf(lse[0, 1, 0])


def test_gather_empty_lists():
    B, Sk, H, KVH, D = 2, 300, 8, 2, 128
    q, k, v = cuda(*synth.qkv(B, 1, Sk, H, KVH, D, "bf16", seed=50))
    mask = torch.zeros((B, H, 1, 384), dtype=torch.bool, device="cuda")
    mask[1, 5, 0, 17] = True
    keys = bsm.build_key_list(bsm.geometry_of(q, k), mask)
    assert keys.num_keys.cpu().tolist() == [[0, 0], [0, 1]]
    o, lse = _gather_check(q, k, v, mask, None, keys, "empty")
    assert (o[0].float() == 0).all() and torch.isneginf(lse[0]).all()


def test_gather_list_with_keys_out_of_range():
    """Listed keys outside [0, Sk) are treated as masked: the result is that of
    the mask without them."""
    B, Sk, H, KVH, D = 1, 500, 4, 1, 128
    q, k, v = cuda(*synth.qkv(B, 1, Sk, H, KVH, D, "bf16", seed=51))
    m = synth.random_bool((B, H, 1, 512), 0.1, 9, synth.TID_MASK)
    m[..., Sk:] = False
    geom = bsm.geometry_of(q, k)
    keys = bsm.build_key_list(geom, torch.from_numpy(m).cuda())
    n = int(keys.num_keys[0, 0])
    idx = keys.key_indices[0, 0, :n].cpu().numpy()
    dropped = idx[[1, n // 2]]
    keys.key_indices[0, 0, 1] = Sk + 5
    keys.key_indices[0, 0, n // 2] = -3
    m2 = m.copy()
    m2[..., dropped] = False
    out = bsm.masked_attn_fwd(q, k, v, mask=torch.from_numpy(m).cuda(), keys=keys)
    torch.cuda.synchronize()
    mask2 = torch.from_numpy(m2).cuda()
    for h in range(H):
        want_o, _ = oracle_rows(q, k, v, 0, h, [0], mask=mask2)
        assert_close(out[0, 0, h].float().cpu().numpy()[None], want_o, "bf16", f"h={h}")
