"""Packed variable-length sequences (oracle).

[FSA-197] Changes / Implementation Notes: the attention integration loads a
varlen entry point next to the padded one, and pad / unpad helpers that move
between a padded (B, S, ...) batch with a validity mask and a packed
(total, ...) layout. The pages name these functions without printing them; the
plainest reading, used throughout, is the usual packed layout:

  unpad: keep the valid positions of a padded batch in row-major order;
         indices[i] = flat position b * S + s of packed row i;
         cu_seqlens[b] = number of valid positions in rows 0 .. b-1 (B + 1
         entries), max_seqlen = the longest row.
  pad:   the inverse scatter, zeros at invalid positions.
  varlen attention: sequence b owns query rows cu_q[b] .. cu_q[b+1] and key
         rows cu_k[b] .. cu_k[b+1] of the packed Q and K / V and attends to its
         own keys only -- attention_full applied to each sequence alone.

Per-sequence DFlash geometry (the block mask with one entry per batch element,
Bm = B, instead of one shared copy, [SF-452] traceback / Expected Behavior):
sequence b with Sq_b queries and Sk_b keys is a DFlash sequence of
NB_b = Sq_b / bs draft blocks after C_b = Sk_b - Sq_b context tokens, with the
layer's causality and window shared by every sequence.
"""

import numpy as np

from .attention import attention_full
from .attention_bwd import attention_bwd
from .blockmask import TILE, classify_tiles
from .dflash import DFlashGeom, dflash_dense_mask


def unpad(x, valid):
    """(packed, indices, cu_seqlens, max_seqlen) of x (B, S, ...) and valid (B, S)."""
    x = np.asarray(x)
    valid = np.asarray(valid, bool)
    B, S = valid.shape
    indices = np.flatnonzero(valid.reshape(-1)).astype(np.int32)
    counts = valid.sum(axis=1)
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(counts)
    packed = x.reshape((B * S,) + x.shape[2:])[indices]
    return packed, indices, cu, int(counts.max()) if B else 0


def pad(packed, indices, B, S):
    """(B, S, ...) with packed row i at flat position indices[i], zeros elsewhere."""
    packed = np.asarray(packed)
    out = np.zeros((B * S,) + packed.shape[1:], packed.dtype)
    out[np.asarray(indices)] = packed
    return out.reshape((B, S) + packed.shape[1:])


def seq_lengths(cu):
    cu = np.asarray(cu, np.int64)
    return cu[1:] - cu[:-1]


def dflash_varlen_geoms(cu_q, cu_k, block_size, ctx_per_block=0, ctx_end_offset=0,
                        is_causal=None, layer_type="full", sliding_window=0):
    """DFlashGeom of every sequence: NB_b = Sq_b / bs blocks after C_b = Sk_b - Sq_b
    context tokens (Sq_b must be a multiple of bs and Sk_b >= Sq_b)."""
    out = []
    for sq, sk in zip(seq_lengths(cu_q), seq_lengths(cu_k)):
        if sq % block_size or sk < sq:
            raise ValueError(f"sequence with {sq} queries / {sk} keys is not a DFlash layout")
        out.append(DFlashGeom(int(sk - sq), int(sq // block_size), block_size, ctx_per_block,
                              ctx_end_offset, is_causal, layer_type, sliding_window))
    return out


def attention_varlen(q, k, v, cu_q, cu_k, scale=None, geoms=None):
    """O (total_q, H, D) and LSE (H, total_q) of packed q (total_q, H, D) and
    k, v (total_k, KVH, D); geoms: None (no mask) or a DFlashGeom per sequence."""
    q = np.asarray(q, np.float64)
    total_q, H, D = q.shape
    o = np.zeros((total_q, H, D))
    lse = np.full((H, total_q), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if q1 == q0:
            continue
        mask = None if geoms is None else geoms[b]
        ob, lb = attention_full(q[None, q0:q1], np.asarray(k[None, k0:k1], np.float64),
                                np.asarray(v[None, k0:k1], np.float64), scale=scale, mask=mask)
        o[q0:q1] = ob[0]
        lse[:, q0:q1] = lb[0]
    return o, lse


def attention_varlen_bwd(q, k, v, dout, cu_q, cu_k, scale=None, geoms=None):
    """dQ (total_q, H, D), dK and dV (total_k, KVH, D) of attention_varlen for
    dL/dO = dout: attention_bwd applied to each sequence alone, so a sequence's
    keys get gradient from its own queries only (zero if it has none)."""
    q = np.asarray(q, np.float64)
    total_q, H, D = q.shape
    total_k, KVH = k.shape[0], k.shape[1]
    dq = np.zeros((total_q, H, D))
    dk = np.zeros((total_k, KVH, D))
    dv = np.zeros((total_k, KVH, D))
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if q1 == q0:
            continue
        mask = None if geoms is None else geoms[b]
        gq, gk, gv, _ = attention_bwd(q[None, q0:q1], np.asarray(k[None, k0:k1], np.float64),
                                      np.asarray(v[None, k0:k1], np.float64),
                                      np.asarray(dout[None, q0:q1], np.float64), scale=scale,
                                      mask=mask)
        dq[q0:q1] = gq[0]
        dk[k0:k1] = gk[0]
        dv[k0:k1] = gv[0]
    return dq, dk, dv


def block_mask_varlen(geoms):
    """Block mask (B, 1, nQmax, nKmax) of per-sequence DFlash geometries: row b
    holds sequence b's own tiles (classify_tiles of its dense mask), padded
    with empty query tiles and -1 indices."""
    B = len(geoms)
    nq = [-(-g.Sq // TILE) for g in geoms]
    nk = [-(-g.Sk // TILE) for g in geoms]
    nQ = max(nq, default=0)
    nK = max(nk, default=0)
    kv_num = np.zeros((B, 1, nQ), np.int32)
    kv_idx = np.full((B, 1, nQ, nK), -1, np.int32)
    full_num = np.zeros((B, 1, nQ), np.int32)
    full_idx = np.full((B, 1, nQ, nK), -1, np.int32)
    for b, g in enumerate(geoms):
        if g.Sq == 0:
            continue
        a, i, c, j = classify_tiles(dflash_dense_mask(g)[None, None], g.Sk)
        kv_num[b, 0, :nq[b]] = a[0, 0]
        kv_idx[b, 0, :nq[b], :nk[b]] = i[0, 0]
        full_num[b, 0, :nq[b]] = c[0, 0]
        full_idx[b, 0, :nq[b], :nk[b]] = j[0, 0]
    return kv_num, kv_idx, full_num, full_idx
