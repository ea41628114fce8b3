"""Kept-key list of a dense mask over a few query rows (oracle).

For short query blocks -- the seqlen_q == 1 head-group swap of [FSA-190]
(Design, Implementation Notes: the G heads of a KV group become G query rows
of one KV head) and, generally, any (b, h) with at most 32 rows -- a dense
mask can be handed to the attention as the list of keys that at least one of
the rows keeps, each with a bit per row telling which rows keep it. With a
dynamic top-k mask ([FSA-197] Design: each row keeps window_size keys) the
union over G rows is a small part of the key range, so only those K / V rows
need to be read. The list changes how keys are visited, never which pairs are
kept: expanding it back gives the dense mask.

Definition (per leading index (bm, hm) of a mask in the attention's iteration
space, shape (Bm, Hm, Qm, K_round) with Qm in {1, R}, and R <= 32 rows):
  row r of (bm, hm) reads mask row r if Qm == R, row 0 if Qm == 1;
  key j is listed iff j < Sk and some row r < R keeps it;
  keys[0 .. num) are the listed keys in ascending order;
  bits[p] = sum over rows r that keep keys[p] of 2^r.
"""

import numpy as np

MAX_ROWS = 32


def key_list(mask, seqlen_k, rows):
    """(num (Bm, Hm) int32, keys (Bm, Hm, K) int32, bits (Bm, Hm, K) uint32).

    Entries at positions >= num are -1 in keys and 0 in bits here; the GPU
    builder leaves them unspecified, so comparisons look at [0, num) only.
    """
    m = np.asarray(mask, dtype=bool)
    if m.ndim != 4:
        raise ValueError("mask must be 4D")
    Bm, Hm, Qm, K = m.shape
    if not 1 <= rows <= MAX_ROWS:
        raise ValueError("rows must be in [1, 32]")
    if Qm not in (1, rows):
        raise ValueError("mask query dim must be 1 or rows")
    num = np.zeros((Bm, Hm), np.int32)
    keys = np.full((Bm, Hm, K), -1, np.int32)
    bits = np.zeros((Bm, Hm, K), np.uint32)
    for b in range(Bm):
        for h in range(Hm):
            row_masks = np.zeros((rows, K), bool)
            for r in range(rows):
                row_masks[r] = m[b, h, r if Qm == rows else 0]
            row_masks[:, seqlen_k:] = False
            listed = np.nonzero(row_masks.any(axis=0))[0]
            num[b, h] = len(listed)
            keys[b, h, :len(listed)] = listed
            for p, j in enumerate(listed):
                word = 0
                for r in range(rows):
                    if row_masks[r, j]:
                        word |= 1 << r
                bits[b, h, p] = word
    return num, keys, bits


def expand_key_list(num, keys, bits, rows, K):
    """Dense (Bm, Hm, rows, K) bool mask that a key list stands for."""
    Bm, Hm = num.shape
    out = np.zeros((Bm, Hm, rows, K), bool)
    for b in range(Bm):
        for h in range(Hm):
            for p in range(num[b, h]):
                j = keys[b, h, p]
                for r in range(rows):
                    if (int(bits[b, h, p]) >> r) & 1:
                        out[b, h, r, j] = True
    return out
