"""Tile classification of a dense boolean mask into a block mask (oracle).

[SF-452] traceback: flex_attention's create_block_mask sums the dense mask per
tile and returns a partial-block part and a full-block part; the block mask
carries, per query tile, the number of kept key tiles and their indices
(kv_num_blocks / kv_indices and full_kv_num_blocks / full_kv_indices). [SF-452]
Problem / Expected Behavior: for a head-independent mask one copy (H = 1) is
shared by all heads. [FSA-190] Summary / Design: the key dimension is rounded to
a multiple of 128, which fixes the key-tile width.

Definition (per leading index (bm, hm), query tile qt, key tile kt, 128 x 128):
  rows = [128 qt, min(128 qt + 128, Qm)), keys = [128 kt, 128 kt + 128);
  n    = number of kept (row, key) pairs, keys >= Sk counting as not kept;
  empty iff n == 0, full iff n == len(rows) * 128, partial otherwise.
kv_indices lists the partial tiles in ascending kt, full_kv_indices the full
ones; unused tail entries are -1.
"""

import numpy as np

TILE = 128


def classify_tiles(mask, seqlen_k):
    """Block mask of a dense bool mask of shape (Bm, Hm, Qm, K_round).

    Returns (kv_num_blocks, kv_indices, full_kv_num_blocks, full_kv_indices)
    as int32 arrays of shapes (Bm, Hm, nQm) and (Bm, Hm, nQm, nK).
    """
    m = np.asarray(mask, dtype=bool)
    if m.ndim != 4:
        raise ValueError("mask must be 4D")
    Bm, Hm, Qm, K = m.shape
    if K % TILE:
        raise ValueError("mask key dim must be a multiple of 128")
    nQ = -(-Qm // TILE)
    nK = K // TILE
    m = m.copy()
    m[..., seqlen_k:] = False
    kv_num = np.zeros((Bm, Hm, nQ), np.int32)
    kv_idx = np.full((Bm, Hm, nQ, nK), -1, np.int32)
    full_num = np.zeros((Bm, Hm, nQ), np.int32)
    full_idx = np.full((Bm, Hm, nQ, nK), -1, np.int32)
    for b in range(Bm):
        for h in range(Hm):
            for qt in range(nQ):
                r0, r1 = qt * TILE, min(qt * TILE + TILE, Qm)
                rows = r1 - r0
                band = m[b, h, r0:r1]
                counts = band.reshape(rows, nK, TILE).sum(axis=(0, 2))
                full = np.nonzero(counts == rows * TILE)[0]
                part = np.nonzero((counts > 0) & (counts < rows * TILE))[0]
                kv_num[b, h, qt] = len(part)
                kv_idx[b, h, qt, :len(part)] = part
                full_num[b, h, qt] = len(full)
                full_idx[b, h, qt, :len(full)] = full
    return kv_num, kv_idx, full_num, full_idx


def classify_tile_band(band_rows, seqlen_k):
    """Classes of the key tiles of one query tile, from its dense rows.

    band_rows: bool (rows, K_round) for the rows of one query tile. Returns
    (partial_indices, full_indices) as ascending int arrays. Same definition
    as classify_tiles; used to stream large masks one query tile at a time.
    """
    m = np.asarray(band_rows, dtype=bool).copy()
    rows, K = m.shape
    m[:, seqlen_k:] = False
    nK = K // TILE
    counts = m.reshape(rows, nK, TILE).sum(axis=(0, 2))
    full = np.nonzero(counts == rows * TILE)[0]
    part = np.nonzero((counts > 0) & (counts < rows * TILE))[0]
    return part, full


def expand_block_mask(kv_num, kv_idx, full_num, full_idx, dense, Qm):
    """Dense mask reconstructed from a block mask.

    Full tiles become all True, partial tiles copy `dense` (the mask the block
    mask was built from), every other tile is all False. Shapes as in
    classify_tiles; `dense` is (Bm, Hm, Qm, K_round).
    """
    Bm, Hm, nQ = kv_num.shape
    nK = kv_idx.shape[-1]
    out = np.zeros((Bm, Hm, Qm, nK * TILE), dtype=bool)
    for b in range(Bm):
        for h in range(Hm):
            for qt in range(nQ):
                r0, r1 = qt * TILE, min(qt * TILE + TILE, Qm)
                for kt in full_idx[b, h, qt, :full_num[b, h, qt]]:
                    out[b, h, r0:r1, kt * TILE:(kt + 1) * TILE] = True
                for kt in kv_idx[b, h, qt, :kv_num[b, h, qt]]:
                    out[b, h, r0:r1, kt * TILE:(kt + 1) * TILE] = \
                        dense[b, h, r0:r1, kt * TILE:(kt + 1) * TILE]
    return out
