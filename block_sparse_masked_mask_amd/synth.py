"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws numbers and lays them out; it holds none of the masking
or attention arithmetic. The same draws feed the GPU path and the CPU oracle.

Random stream: element block c (CHUNK elements each) of tensor `tensor_id`
under seed s comes from numpy.random.default_rng([s, tensor_id, c]), drawn as
float32 standard normals, then scaled. bf16 storage is torch's round-to-
nearest-even conversion of those float32 values.

The five workloads below are the DFlash and dynamic-mask shapes the pages
describe (a tiny DFlash case; a DFlash training shape with a full-attention and
a sliding-window layer; a long-context DFlash case with one block mask shared by
all heads; dynamic top-k attention with a 2D padding mask; a seqlen_q == 1 decode
case taking the head-group swap).
"""

import numpy as np
import torch

CHUNK = 1 << 22

TID_Q, TID_K, TID_V, TID_BIAS, TID_PADLEN, TID_MASK, TID_DOUT = 1, 2, 3, 4, 5, 6, 7


def normal(shape, seed, tensor_id, scale=1.0):
    """float32 array of N(0, scale^2) draws, chunked as the module states."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    for c, lo in enumerate(range(0, n, CHUNK)):
        hi = min(n, lo + CHUNK)
        rng = np.random.default_rng([seed, tensor_id, c])
        out[lo:hi] = rng.standard_normal(hi - lo, dtype=np.float32)
    if scale != 1.0:
        out *= np.float32(scale)
    return out.reshape(shape)


def normal_range(seed, tensor_id, lo, hi, scale=1.0):
    """float32 elements [lo, hi) of the flat stream that `normal` lays out (the
    same values; only the chunks that overlap the range are drawn, each up to
    the range's end)."""
    out = np.empty(max(0, hi - lo), np.float32)
    for c in range(lo // CHUNK, (hi - 1) // CHUNK + 1 if hi > lo else lo // CHUNK):
        base = c * CHUNK
        a, b = max(lo, base), min(hi, base + CHUNK)
        rng = np.random.default_rng([seed, tensor_id, c])
        out[a - lo:b - lo] = rng.standard_normal(b - base, dtype=np.float32)[a - base:]
    if scale != 1.0:
        out *= np.float32(scale)
    return out


def normal_rows(shape, seed, tensor_id, b, r0, r1, dtype, scale=1.0):
    """Rows [r0, r1) of batch b of the (B, S, X, Y) tensor normal_tensor would
    make, as a (1, r1 - r0, X, Y) tensor in the storage dtype."""
    B, S, X, Y = shape
    row = X * Y
    lo = (b * S + r0) * row
    arr = normal_range(seed, tensor_id, lo, lo + (r1 - r0) * row, scale)
    return storage(arr.reshape(1, r1 - r0, X, Y), dtype)


def storage(arr, dtype):
    """torch CPU tensor in the storage dtype ('bf16' or 'f32')."""
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t.to(torch.float32)
    raise ValueError(dtype)


def normal_tensor(shape, seed, tensor_id, dtype, scale=1.0):
    return storage(normal(shape, seed, tensor_id, scale), dtype)


def as_f64(t):
    """Exact float64 copy of a stored tensor, as a NumPy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def pad_lengths(batch, lo, hi, seed):
    """Per-batch right-padding lengths, uniform integers in [lo, hi]."""
    rng = np.random.default_rng([seed, TID_PADLEN])
    return rng.integers(lo, hi + 1, size=batch)


def padding_mask_2d(seqlen, lengths):
    """(B, seqlen) bool: True for the first seqlen - L_b keys of batch b."""
    k = np.arange(seqlen)[None, :]
    return k < (seqlen - np.asarray(lengths)[:, None])


def random_bool(shape, p_true, seed, tensor_id):
    rng = np.random.default_rng([seed, tensor_id])
    return rng.random(shape) < p_true


# Workload table. DFlash entries: ctx_len C, num_blocks NB, block_size bs
# (queries = NB*bs draft tokens, keys = C + NB*bs), and the layers to run.
CONFIGS = {
    "tiny_dflash_fp32": dict(
        kind="dflash", dtype="f32", B=1, H=2, KVH=2, D=64,
        ctx_len=256, num_blocks=4, block_size=16, qkv_scale=1.0,
        layers=[dict(name="full", is_causal=None, layer_type="full", window=0)],
    ),
    "dflash_train_bf16": dict(
        kind="dflash", dtype="bf16", B=2, H=32, KVH=8, D=128,
        ctx_len=4096, num_blocks=256, block_size=16, qkv_scale=0.5,
        layers=[
            dict(name="full", is_causal=None, layer_type="full", window=0),
            dict(name="sliding", is_causal=None, layer_type="sliding", window=2048),
        ],
    ),
    "long_dflash_bf16": dict(
        kind="dflash", dtype="bf16", B=1, H=32, KVH=8, D=128,
        ctx_len=32768, num_blocks=2048, block_size=16, qkv_scale=1.0,
        layers=[dict(name="sliding_causal", is_causal=1, layer_type="sliding", window=4096)],
    ),
    "dynamic_topk_bf16": dict(
        kind="topk", dtype="bf16", B=2, H=16, KVH=4, D=128, Sq=8000, Sk=8000,
        bias_heads="kvh", bias_q=1, pad_lo=0, pad_hi=1000, topk=2048, qkv_scale=1.0,
    ),
    # inference: one draft block of 16 after a 32K-token cache per request
    "dflash_infer_bf16": dict(
        kind="dflash_infer", dtype="bf16", B=8, H=32, KVH=8, D=128,
        ctx_len=32768, block_size=16, qkv_scale=0.5,
        layers=[dict(name="full", is_causal=None, layer_type="full", window=0),
                dict(name="sliding", is_causal=None, layer_type="sliding", window=4096)],
    ),
    "decode_swap_bf16": dict(
        kind="topk", dtype="bf16", B=64, H=32, KVH=8, D=128, Sq=1, Sk=16384,
        bias_heads="h", bias_q=1, pad_lo=None, pad_hi=None, topk=1024, qkv_scale=1.0,
    ),
}


def qkv(B, Sq, Sk, H, KVH, D, dtype, seed=0, scale=1.0):
    """Q (B,Sq,H,D), K and V (B,Sk,KVH,D) as torch CPU tensors."""
    q = normal_tensor((B, Sq, H, D), seed, TID_Q, dtype, scale)
    k = normal_tensor((B, Sk, KVH, D), seed, TID_K, dtype, scale)
    v = normal_tensor((B, Sk, KVH, D), seed, TID_V, dtype, scale)
    return q, k, v


def round_up_128(x):
    return -(-int(x) // 128) * 128


def topk_inputs(cfg, seed=0):
    """Bias (B, Hb, 1, K_round) and the optional 2D padding mask of a top-k config."""
    B, H, KVH, Sk = cfg["B"], cfg["H"], cfg["KVH"], cfg["Sk"]
    Hb = KVH if cfg["bias_heads"] == "kvh" else H
    kr = round_up_128(Sk)
    bias = normal_tensor((B, Hb, cfg["bias_q"], kr), seed, TID_BIAS, cfg["dtype"])
    pad2d = None
    if cfg.get("pad_hi") is not None:
        lens = pad_lengths(B, cfg["pad_lo"], cfg["pad_hi"], seed)
        pad2d = torch.from_numpy(padding_mask_2d(Sk, lens))
    return bias, pad2d
