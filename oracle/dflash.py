"""DFlash draft-block attention mask, written out rule by rule (oracle, fp-free).

Layout of one DFlash sequence (the plainest reading of [SF-452] Problem and of
the tiny worked case "draft block j attends to context positions < 64*j + 64"
with 256 context tokens and 4 draft blocks of 16):

  keys    = C context tokens, then NB draft blocks of bs tokens each
            (Sk = C + NB*bs);
  queries = the NB*bs draft tokens (Sq = NB*bs), query q is token i = q % bs of
            draft block j = q // bs.

Visibility of key k from query q (all rules from the cited passages):
  * context key k < C: visible iff k < E_j, where E_j = clamp((j+1)*S + e0,
    0, C) is the end of the context that block j may see ("context blocks
    before current block", [SF-452] Problem; S = C/NB context tokens per block,
    e0 an optional offset, 0 by default);
  * draft key k = C + j'*bs + i': visible iff j' == j ("noise tokens from same
    block", [SF-452] Problem), and, when in-block attention is causal, i' <= i;
  * in-block causality comes from resolve_dflash_is_causal ([SF-905]
    Motivation / Modifications, rule of the maintainer reply item #934);
  * on sliding-attention layers a window with a LEFT bound only applies
    ([SF-905] maintainer reply, #934: the right bound is dropped): with token
    positions pos(context c) = c and pos(draft (j, i)) = E_j + i, a key is
    visible only if pos_q - pos_k < W;
  * keys k >= Sk (the round-up-to-128 tail) are never visible ([FSA-190]
    Implementation Notes, stability fix).

The mask is independent of batch and head ([SF-452] Problem / Expected
Behavior), so it is returned as one (rows, K_round) array.
"""

from dataclasses import dataclass

import numpy as np

from .normalize import round_multiple

FULL = 0
SLIDING = 1


def _is_sliding(layer_type):
    """Layer type: 'full'/0 -> False, 'sliding'/1 -> True, else ValueError."""
    if not isinstance(layer_type, bool):
        if layer_type in ("full", FULL):
            return False
        if layer_type in ("sliding", SLIDING):
            return True
    raise ValueError(f"unknown layer type {layer_type!r}")


def resolve_dflash_is_causal(is_causal, layer_type):
    """In-block causality from the config's is_causal and the layer type.

    [SF-905] Motivation (SGLang rule) and maintainer reply item #934:
      is_causal absent -> bidirectional on full-attention layers, causal on
                          sliding-attention layers;
      is_causal False  -> bidirectional on both;
      is_causal True   -> causal on both.
    is_causal: None (absent), False/True, or the C-style -1/0/1.
    layer_type: 'full'/'sliding' or 0/1. Anything else raises ValueError.
    """
    sliding = _is_sliding(layer_type)
    if is_causal is None:
        return sliding
    if isinstance(is_causal, bool):
        return is_causal
    if is_causal == -1:
        return sliding
    if is_causal in (0, 1):
        return bool(is_causal)
    raise ValueError(f"bad is_causal {is_causal!r}")


@dataclass(frozen=True)
class DFlashGeom:
    """One DFlash sequence geometry plus the layer's mask semantics.

    ctx_len C, num_blocks NB, block_size bs; ctx_per_block S (0 -> C // NB,
    which then requires C % NB == 0); ctx_end_offset e0; is_causal (None /
    bool / -1,0,1); layer_type ('full' / 'sliding'); sliding_window W (used on
    sliding layers only, must be >= 1 there).
    """

    ctx_len: int
    num_blocks: int
    block_size: int
    ctx_per_block: int = 0
    ctx_end_offset: int = 0
    is_causal: object = None
    layer_type: object = "full"
    sliding_window: int = 0

    @property
    def S(self):
        if self.ctx_per_block:
            return self.ctx_per_block
        if self.num_blocks == 0 or self.ctx_len % self.num_blocks:
            raise ValueError("ctx_per_block=0 needs ctx_len % num_blocks == 0")
        return self.ctx_len // self.num_blocks

    @property
    def Sq(self):
        return self.num_blocks * self.block_size

    @property
    def Sk(self):
        return self.ctx_len + self.num_blocks * self.block_size

    @property
    def causal(self):
        return resolve_dflash_is_causal(self.is_causal, self.layer_type)

    @property
    def window(self):
        """W on sliding layers ([SF-905] #934), None (no window) on full ones."""
        if not _is_sliding(self.layer_type):
            return None
        if self.sliding_window < 1:
            raise ValueError("sliding layer needs sliding_window >= 1")
        return int(self.sliding_window)


def _block_context_end(g, j):
    """E_j = clamp((j+1)*S + e0, 0, C) for an integer array j."""
    return np.clip((j + 1) * g.S + g.ctx_end_offset, 0, g.ctx_len)


def dflash_dense_mask(g, rows=None):
    """Dense boolean DFlash mask (True = keep) for the given query rows.

    Returns an array of shape (len(rows), round_up(Sk, 128)); rows defaults to
    all Sq queries. Every element is decided by the rules in the module
    docstring, evaluated independently per (q, k) pair.
    """
    if rows is None:
        rows = np.arange(g.Sq, dtype=np.int64)
    q = np.asarray(rows, dtype=np.int64)[:, None]
    k_round = round_multiple(g.Sk, 128)
    k = np.arange(k_round, dtype=np.int64)[None, :]
    C, bs = g.ctx_len, g.block_size
    W = g.window
    j = q // bs
    i = q % bs
    E = _block_context_end(g, j)
    pos_q = E + i

    # context keys
    is_ctx = k < C
    ctx_keep = is_ctx & (k < E)
    if W is not None:
        ctx_keep &= (pos_q - k) < W

    # draft keys
    kd = k - C
    is_draft = (k >= C) & (k < g.Sk)
    jd = np.where(is_draft, kd // bs, -1)
    idr = np.where(is_draft, kd % bs, 0)
    draft_keep = is_draft & (jd == j)
    if g.causal:
        draft_keep &= idr <= i
    if W is not None:
        pos_k = E + idr  # the key lies in the query's own block
        draft_keep &= (pos_q - pos_k) < W

    return ctx_keep | draft_keep


def dflash_inference_geom(ctx_len, block_size, is_causal=None, layer_type="full",
                          sliding_window=0):
    """Mask geometry of one draft block drafted after ctx_len cached tokens.

    [SF-905] Modifications and the maintainer reply (#935) give inference
    (spec_generate) a default mask built by the same builders as training; the
    pages show no inference shapes. Plainest reading: the block being drafted
    is the last block of a training sequence whose context ends at the cache
    end, so it sees every cached token (E = C), its own bs tokens under the
    layer's in-block causality, and on sliding layers the left-bound window
    with pos(draft i) = C + i. Keys: the C cached tokens, then the block.
    """
    return DFlashGeom(ctx_len, 1, block_size, ctx_per_block=ctx_len, is_causal=is_causal,
                      layer_type=layer_type, sliding_window=sliding_window)

