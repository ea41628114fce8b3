"""Pins of the backward oracle (oracle.attention_bwd).

The gradients are checked against two things that do not share its formulas:
central finite differences of the forward oracle (oracle.attention), and torch
autograd in float64 on a plain masked-softmax attention. Cases cover GQA
(dK / dV summed over a KV group), a mask with fully masked rows, and biases
broadcast over batch, heads or queries (dbias reduced over the broadcast dims,
flash-sparse-attention PR #190, Changes: mha_bwd), plus a DFlash predicate.
"""

import numpy as np
import pytest
import torch

from oracle.attention import attention_full
from oracle.attention_bwd import attention_bwd
from oracle.dflash import DFlashGeom, dflash_dense_mask

B, SQ, SK, H, KVH, D = 2, 5, 7, 4, 2, 3
KR = 8  # bias / mask key length (>= SK)


def _inputs(seed, mask_kind, bias_shape):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, SQ, H, D))
    k = rng.standard_normal((B, SK, KVH, D))
    v = rng.standard_normal((B, SK, KVH, D))
    dout = rng.standard_normal((B, SQ, H, D))
    mask = None
    if mask_kind == "random":
        mask = rng.random((B, 1, SQ, KR)) < 0.6
        mask[0, 0, 1, :] = False          # a fully masked row
        mask[1, 0, 3, :SK] = False
        mask[1, 0, 3, 2] = True           # a single kept key
    bias = None if bias_shape is None else rng.standard_normal(bias_shape)
    return q, k, v, dout, mask, bias


def _loss(q, k, v, dout, mask, bias, scale):
    o, _ = attention_full(q, k, v, scale=scale, mask=mask, bias=bias)
    return float((o * dout).sum())


def _fd(fn, x, eps=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        lp = fn()
        x[i] = old - eps
        lm = fn()
        x[i] = old
        g[i] = (lp - lm) / (2 * eps)
    return g


CASES = [
    ("none", None),
    ("random", None),
    ("random", (B, H, SQ, KR)),
    ("random", (1, KVH, 1, KR)),
    ("none", (B, 1, 1, KR)),
    ("random", (1, H, SQ, KR)),
]


@pytest.mark.parametrize("mask_kind,bias_shape", CASES)
def test_bwd_matches_finite_differences(mask_kind, bias_shape):
    q, k, v, dout, mask, bias = _inputs(7, mask_kind, bias_shape)
    scale = 0.6
    dq, dk, dv, dbias = attention_bwd(q, k, v, dout, scale=scale, mask=mask, bias=bias)
    loss = lambda: _loss(q, k, v, dout, mask, bias, scale)  # noqa: E731
    np.testing.assert_allclose(dq, _fd(loss, q), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dk, _fd(loss, k), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dv, _fd(loss, v), rtol=1e-6, atol=1e-8)
    if bias is not None:
        np.testing.assert_allclose(dbias, _fd(loss, bias), rtol=1e-6, atol=1e-8)
        assert (dbias[..., SK:] == 0).all()


def _torch_attention(q, k, v, mask, bias, scale):
    """Plain masked softmax attention in torch (float64), rows with no kept
    key giving 0."""
    G = H // KVH
    qt = q.permute(0, 2, 1, 3)                                  # B H Sq D
    kt = k.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)      # B H Sk D
    vt = v.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    s = scale * torch.matmul(qt, kt.transpose(-1, -2))
    if bias is not None:
        bb = bias[..., :SK]
        if bb.shape[1] == KVH and KVH != H:
            bb = bb.repeat_interleave(G, dim=1)
        s = s + bb
    if mask is not None:
        keep = mask[..., :SK].expand(B, H, SQ, SK)
        s = s.masked_fill(~keep, float("-inf"))
    p = torch.softmax(s, dim=-1)
    p = torch.nan_to_num(p, nan=0.0)
    return torch.matmul(p, vt).permute(0, 2, 1, 3)


@pytest.mark.parametrize("mask_kind,bias_shape", CASES)
def test_bwd_matches_torch_autograd(mask_kind, bias_shape):
    q, k, v, dout, mask, bias = _inputs(11, mask_kind, bias_shape)
    scale = 0.45
    dq, dk, dv, dbias = attention_bwd(q, k, v, dout, scale=scale, mask=mask, bias=bias)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    tb = None if bias is None else torch.tensor(bias, dtype=torch.float64, requires_grad=True)
    tm = None if mask is None else torch.tensor(mask)
    o = _torch_attention(tq, tk, tv, tm, tb, scale)
    (o * torch.tensor(dout)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)
    if bias is not None:
        np.testing.assert_allclose(dbias, tb.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_fully_masked_row_has_zero_gradients():
    q, k, v, dout, mask, _ = _inputs(3, "random", None)
    dq, _, _, _ = attention_bwd(q, k, v, dout, mask=mask)
    assert (dq[0, 1] == 0).all()       # row 1 of batch 0 keeps nothing


def test_bwd_dflash_predicate_equals_its_dense_mask():
    g = DFlashGeom(ctx_len=12, num_blocks=3, block_size=4, layer_type="sliding",
                   sliding_window=6)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, g.Sq, 2, 4))
    k = rng.standard_normal((1, g.Sk, 1, 4))
    v = rng.standard_normal((1, g.Sk, 1, 4))
    dout = rng.standard_normal((1, g.Sq, 2, 4))
    dense = dflash_dense_mask(g, np.arange(g.Sq))[None, None]
    a = attention_bwd(q, k, v, dout, mask=g)
    d = attention_bwd(q, k, v, dout, mask=dense)
    for x, y in zip(a[:3], d[:3]):
        np.testing.assert_array_equal(x, y)
