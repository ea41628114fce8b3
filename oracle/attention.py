"""Masked softmax attention in float64 over the kept keys (oracle).

For batch b, head h and query row q (definitions from [FSA-190] Design: bool
mask True = keep, floating bias additive; GQA with the KV head of head h being
h // G, G = H / KVH; aux tensors broadcast over singleton batch / head / query
dims by the ({B|1}, {H|KVH|1}, {Sq|1}, K) contract):

  kept  = { key j < Sk : mask[b', h', q', j] }          (all keys if no mask)
  s_j   = scale * <Q[b, q, h, :], K[b, j, h // G, :]> + bias[b', h', q', j]
  m     = max_{j in kept} s_j
  O     = sum_{j in kept} exp(s_j - m) V[b, j, h // G, :] / sum_{j in kept} exp(s_j - m)
  LSE   = m + log sum_{j in kept} exp(s_j - m)

with b' = b or 0, q' = q or 0 for singleton dims, and h' = h (head dim H),
h // G (head dim KVH) or 0 (head dim 1). A row with no kept key returns O = 0
(the fully-masked-row invariant) and LSE = -inf (log of an empty sum). Masked
positions are left out of the sums, which is the same as giving them score
-inf. The default scale is 1 / sqrt(D).

The mask may also be a DFlashGeom: its rows then come from
oracle.dflash.dflash_dense_mask, shared by every batch and head ([SF-452]
Problem / Expected Behavior).
"""

import math

import numpy as np

from .dflash import DFlashGeom, dflash_dense_mask


# Readings where the pages leave huge and infinite biases open:
#   * a finite bias beyond +-BIAS_BOUND = FLT_MAX / log2(e) (~2.36e38) counts
#     as +-BIAS_BOUND: the bias is taken in log2 units (bias * log2 e) and
#     saturated at the largest finite float32 there. A kept key carrying the
#     pre-mask sentinel finfo(bf16 / f32).min ([FSA-197] Changes) therefore
#     stays kept, and keys that all carry it weigh the same;
#   * a bias of -inf stays -inf: that key contributes nothing, and a row whose
#     kept keys all score -inf is treated as a fully masked row.
_F32_MAX = (2.0 - 2.0 ** -23) * 2.0 ** 127
BIAS_BOUND = _F32_MAX / math.log2(math.e)


def saturate_bias(x):
    """Finite values clipped to [-BIAS_BOUND, BIAS_BOUND]; -inf kept."""
    x = np.asarray(x, np.float64)
    return np.where(np.isneginf(x), x, np.clip(x, -BIAS_BOUND, BIAS_BOUND))


def _aux_rows(t, b, h, rows, H, KVH):
    """Rows of a broadcastable 4D aux tensor for (b, h, rows)."""
    Bt, Ht, Qt, _ = t.shape
    G = H // KVH
    bi = b if Bt > 1 else 0
    if Ht == H:
        hi = h
    elif Ht == KVH:
        hi = h // G
    elif Ht == 1:
        hi = 0
    else:
        raise ValueError(f"aux head dim {Ht} not in (1, {KVH}, {H})")
    if Qt > 1:
        return t[bi, hi, rows, :]
    return np.broadcast_to(t[bi, hi, 0, :], (len(rows), t.shape[3]))


def attention_rows(q, k, v, b, h, rows, scale=None, mask=None, bias=None):
    """O (len(rows), D) and LSE (len(rows),) for batch b, head h, query rows.

    q: (B, Sq, H, D), k/v: (B, Sk, KVH, D) float arrays holding the exact
    stored values; mask: None, a DFlashGeom, or a bool (Bm, Hm, Qm, K>=Sk)
    array; bias: None or a float (Bb, Hb, Qb, K>=Sk) array.
    """
    B, Sq, H, D = q.shape
    Sk, KVH = k.shape[1], k.shape[2]
    G = H // KVH
    rows = np.asarray(rows, np.int64)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    Kh = np.asarray(k[b, :, h // G, :], np.float64)
    Vh = np.asarray(v[b, :, h // G, :], np.float64)
    Q = np.asarray(q[b, rows, h, :], np.float64)
    s = scale * (Q @ Kh.T)
    if bias is not None:
        s = s + saturate_bias(_aux_rows(bias, b, h, rows, H, KVH)[:, :Sk])
    if mask is None:
        kept = np.ones(s.shape, bool)
    elif isinstance(mask, DFlashGeom):
        kept = dflash_dense_mask(mask, rows)[:, :Sk]
    else:
        kept = np.asarray(_aux_rows(np.asarray(mask, bool), b, h, rows, H, KVH)[:, :Sk])
    # every requested row at once: a masked position takes score -inf, so its
    # exp is 0 and it drops out of the max, the sum and the weighted sum of V
    s = np.where(kept, s, -np.inf)
    has = (s > -np.inf).any(axis=1)
    m = np.where(has, s.max(axis=1), 0.0)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    O = np.zeros((len(rows), D))
    lse = np.full(len(rows), -np.inf)
    O[has] = (p[has] @ Vh) / l[has, None]
    lse[has] = m[has] + np.log(l[has])
    return O, lse


def attention_full(q, k, v, scale=None, mask=None, bias=None):
    """O (B, Sq, H, D) and LSE (B, H, Sq) for every row (small sizes only)."""
    q = np.asarray(q, np.float64)
    B, Sq, H, D = q.shape
    O = np.zeros((B, Sq, H, D))
    lse = np.zeros((B, H, Sq))
    rows = np.arange(Sq)
    for b in range(B):
        for h in range(H):
            O[b, :, h, :], lse[b, h, :] = attention_rows(
                q, k, v, b, h, rows, scale=scale, mask=mask, bias=bias)
    return O, lse
