"""Dynamic top-k keep mask over an additive attention bias (oracle).

[FSA-197] Design / Implementation Notes and the review suggestion on
dynamic_mask: positions the pre-mask marks invalid are first set to the
minimum finite value of the BIAS dtype (torch.finfo(bias.dtype).min, [FSA-197]
Changes), then the window_size largest entries of each row along the key axis
are selected (top-k, unsorted) and a boolean mask is scattered from their
indices.

Readings where the pages leave the step open:
  * ties at the cut go to the lower key index (top-k without sorting does not
    define an order, so one correct answer is fixed here);
  * values compare as real numbers of the bias dtype: -0 == +0; a valid key
    whose bias is -inf ranks below the sentinel of pre-masked keys;
  * keys at or beyond seqlen_k (the round-up-to-128 tail) are invalid;
  * the returned mask is (selected AND valid), so a row keeps exactly
    min(window_size, #valid) keys and a fully pre-masked row keeps none.
NaN biases are outside the contract.
"""

import numpy as np

# Largest finite magnitudes from the formats' definitions:
#   bfloat16: 8 exponent bits, 7 fraction bits -> (2 - 2**-7) * 2**127
#   float32 : 8 exponent bits, 23 fraction bits -> (2 - 2**-23) * 2**127
_FMAX = {
    "bf16": (2.0 - 2.0 ** -7) * 2.0 ** 127,
    "f32": (2.0 - 2.0 ** -23) * 2.0 ** 127,
}


def finfo_min(dtype):
    """Minimum finite value of 'bf16' or 'f32' as a Python float."""
    return -_FMAX[dtype]


def _masked_values(bias_row, valid_row, dtype):
    x = np.where(valid_row, np.asarray(bias_row, np.float64), finfo_min(dtype))
    return x + 0.0  # -0.0 + 0.0 == +0.0: fold the two zeros together


def topk_keep_mask(bias, premask, seqlen_k, k, dtype):
    """Top-k keep mask of a 4D bias (Bb, Hb, Qb, K_round).

    bias: float array holding the exact stored values; premask: None or bool
    array broadcastable to the bias (each dim 1 or equal; last dim seqlen_k
    or K_round); dtype: 'bf16' or 'f32' (the bias dtype, for the sentinel).
    Returns a bool array with the bias's shape.
    """
    if k < 0:
        raise ValueError("k must be >= 0")
    b = np.asarray(bias, np.float64)
    Bb, Hb, Qb, K = b.shape
    valid = np.zeros(b.shape, bool)
    valid[..., :seqlen_k] = True
    if premask is not None:
        pm = np.asarray(premask, bool)
        pmk = np.zeros(pm.shape[:3] + (K,), bool)
        n = min(pm.shape[3], seqlen_k)
        pmk[..., :n] = pm[..., :n]
        valid &= np.broadcast_to(pmk, b.shape)
    out = np.zeros(b.shape, bool)
    idx = np.arange(K)
    for bb in range(Bb):
        for hh in range(Hb):
            for qq in range(Qb):
                x = _masked_values(b[bb, hh, qq], valid[bb, hh, qq], dtype)
                # one stable ordering by (value descending, index ascending)
                order = np.lexsort((idx, -x))
                sel = np.zeros(K, bool)
                sel[order[:k]] = True
                out[bb, hh, qq] = sel & valid[bb, hh, qq]
    return out


def topk_rank_bruteforce(bias_row, valid_row, k, dtype):
    """O(K^2) statement of the same selection for one short row.

    rank(k) = #{m : x_m > x_k} + #{m < k : x_m == x_k}; keep iff
    rank < k and valid. Used to pin topk_keep_mask on tiny rows.
    """
    x = _masked_values(bias_row, valid_row, dtype)
    K = len(x)
    keep = np.zeros(K, bool)
    for a in range(K):
        rank = 0
        for m in range(K):
            if x[m] > x[a] or (m < a and x[m] == x[a]):
                rank += 1
        keep[a] = rank < k and bool(valid_row[a])
    return keep
