"""Gradients of masked softmax attention in float64 (oracle).

The forward is the one in oracle.attention: on the kept keys of a row,
s_j = scale * <Q_q, K_j> + bias_j and P_j = exp(s_j - LSE); P_j = 0 on masked
keys and on rows with no kept key. For a loss L with dL/dO = dO (the backward
that flash-sparse-attention PR #190 describes under Changes: mha_bwd, and
checks in its backward equivalence tests):

  dV_j   = sum_q P_qj dO_q                 summed over the G heads of a KV group
  dP_qj  = <dO_q, V_j>
  Delta_q = sum_j P_qj dP_qj               (equals <dO_q, O_q>)
  dS_qj  = P_qj (dP_qj - Delta_q)          (0 where P is 0)
  dQ_q   = scale * sum_j dS_qj K_j
  dK_j   = scale * sum_q dS_qj Q_q         summed over the G heads of a KV group
  dbias  = dS, summed over every (b, h, q) that reads the same bias element
           (the broadcast-dim reductions of PR #190, Changes: mha_bwd); its
           key dim keeps the bias's rounded length and is 0 past Sk.

These follow from differentiating the forward definition; the tests pin them
against central finite differences of oracle.attention and against torch
autograd in float64.
"""

import math

import numpy as np

from .attention import _aux_rows, saturate_bias
from .dflash import DFlashGeom, dflash_dense_mask


def head_grads(q, k, v, dout, b, h, scale=None, mask=None, bias=None):
    """dQ (Sq, D), dK (Sk, D), dV (Sk, D) contributions of head h of batch b,
    and dS (Sq, Sk), all float64."""
    q = np.asarray(q, np.float64)
    B, Sq, H, D = q.shape
    Sk, KVH = k.shape[1], k.shape[2]
    G = H // KVH
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rows = np.arange(Sq)
    Q = q[b, :, h, :]
    K = np.asarray(k[b, :, h // G, :], np.float64)
    V = np.asarray(v[b, :, h // G, :], np.float64)
    dO = np.asarray(dout[b, :, h, :], np.float64)
    s = scale * (Q @ K.T)
    if bias is not None:
        s = s + saturate_bias(_aux_rows(bias, b, h, rows, H, KVH)[:, :Sk])
    if mask is None:
        kept = np.ones(s.shape, bool)
    elif isinstance(mask, DFlashGeom):
        kept = dflash_dense_mask(mask, rows)[:, :Sk]
    else:
        kept = np.asarray(_aux_rows(np.asarray(mask, bool), b, h, rows, H, KVH)[:, :Sk])
    P = np.zeros((Sq, Sk))
    for r in range(Sq):
        sel = kept[r] & (s[r] > -np.inf)
        if not sel.any():
            continue
        sr = s[r, sel]
        e = np.exp(sr - sr.max())
        P[r, sel] = e / e.sum()
    dP = dO @ V.T
    delta = (P * dP).sum(axis=1)
    dS = P * (dP - delta[:, None])
    dQ = scale * (dS @ K)
    dK = scale * (dS.T @ Q)
    dV = P.T @ dO
    return dQ, dK, dV, dS


def _reduce_dbias(dbias, dS, b, h, H, KVH, Sk):
    """Add dS (Sq, Sk) of (b, h) into the broadcast-shaped dbias."""
    Bt, Ht, Qt, _ = dbias.shape
    G = H // KVH
    bi = b if Bt > 1 else 0
    hi = h if Ht == H else (h // G if Ht == KVH else 0)
    if Qt > 1:
        dbias[bi, hi, :, :Sk] += dS
    else:
        dbias[bi, hi, 0, :Sk] += dS.sum(axis=0)


def attention_bwd(q, k, v, dout, scale=None, mask=None, bias=None):
    """dQ (B, Sq, H, D), dK and dV (B, Sk, KVH, D) and dbias (bias's shape, or
    None without a bias) for every row (small sizes only)."""
    q = np.asarray(q, np.float64)
    B, Sq, H, D = q.shape
    Sk, KVH = k.shape[1], k.shape[2]
    G = H // KVH
    dq = np.zeros((B, Sq, H, D))
    dk = np.zeros((B, Sk, KVH, D))
    dv = np.zeros((B, Sk, KVH, D))
    dbias = None if bias is None else np.zeros(np.shape(bias))
    for b in range(B):
        for h in range(H):
            dQ, dK, dV, dS = head_grads(q, k, v, dout, b, h, scale, mask, bias)
            dq[b, :, h, :] = dQ
            dk[b, :, h // G, :] += dK
            dv[b, :, h // G, :] += dV
            if dbias is not None:
                _reduce_dbias(dbias, dS, b, h, H, KVH, Sk)
    return dq, dk, dv, dbias


def group_grads(q, k, v, dout, b, kvh, scale=None, mask=None, bias=None):
    """dQ (Sq, G, D) of the G heads of KV head kvh, and their summed dK, dV
    (Sk, D), for one batch element (for sampled checks at larger sizes)."""
    H, KVH = q.shape[2], k.shape[2]
    G = H // KVH
    Sq, D = q.shape[1], q.shape[3]
    Sk = k.shape[1]
    dq = np.zeros((Sq, G, D))
    dk = np.zeros((Sk, D))
    dv = np.zeros((Sk, D))
    for g in range(G):
        dQ, dK, dV, _ = head_grads(q, k, v, dout, b, kvh * G + g, scale, mask, bias)
        dq[:, g, :] = dQ
        dk += dK
        dv += dV
    return dq, dk, dv
