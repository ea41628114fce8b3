"""Key-length rounding and pre-mask normalisation (oracle).

[FSA-190] Design / Changes: aux tensors are 4D,
({B|1}, {H|KVH|1}, {Sq|1}, round_multiple(Sk, 128)); only the key dimension is
materialised, padded to the 128-multiple; singleton B/H/Sq broadcast.
[FSA-197] Implementation Notes: a 2D (batch, seq_len) mask with
seq_len == key_len becomes (B, 1, 1, K); a 4D mask must already broadcast to
the bias shape.
"""

import numpy as np


def round_multiple(x, m):
    """Smallest multiple of m that is >= x (x >= 0, m >= 1)."""
    return -(-int(x) // int(m)) * int(m)


def normalize_premask(mask, batch, key_len, k_round=None):
    """Return the pre-mask as a 4D bool array with last dim k_round.

    2D (batch, key_len) -> (batch, 1, 1, k_round); 4D (b, h, q, key_len or
    k_round) -> same leading dims. Keys at or beyond key_len are False
    (never kept). The 2D case with seq_len == query_len != key_len is left
    unsupported: the page's code pads it with ones while its review asks for
    zeros ([FSA-197] review comment on the padding mask), so it raises.
    """
    if k_round is None:
        k_round = round_multiple(key_len, 128)
    m = np.asarray(mask).astype(bool)
    if m.ndim == 2:
        if m.shape != (batch, key_len):
            raise ValueError(
                f"2D mask must be (batch, key_len) = {(batch, key_len)}, got {m.shape}")
        m = m[:, None, None, :]
    if m.ndim != 4:
        raise ValueError("mask must be 2D or 4D")
    if m.shape[3] not in (key_len, k_round):
        raise ValueError("mask last dim must be key_len or round_up(key_len,128)")
    out = np.zeros(m.shape[:3] + (k_round,), dtype=bool)
    out[..., :key_len] = m[..., :key_len]
    return out
