"""CPU oracle for block-sparse masked attention -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct restatement of what the GPU
path computes. It exists so that tests, the smoke check and the benchmark's
CPU-baseline leg have something independent to compare against. Nothing in the
product path (the HIP library and its Python binding) may import it, and it
imports nothing from the product path: the two share no code. Inputs reach it
as NumPy arrays produced by the seeded generators, never from a GPU result.

Arithmetic is float64 (or exact integers); NumPy's matmul, sort and exp are
used as library primitives, with no blocking, fusion or reordering beyond the
definitions below.

Sources (cited by title and section throughout):
  [SF-452]  SpecForge issue #452, "[Bug] flex_attention BlockMask incorrectly
            created with H=num_heads" (sections: traceback, Problem, Expected
            Behavior).
  [SF-905]  SpecForge PR #905, "Fix DFlash attention masking" (sections:
            Motivation, Modifications, maintainer reply listing #934/#935/#936,
            open question on #934).
  [SF-474]  SpecForge issue #474, "DFlash block mask currently relies on Flex
            Attention only -- request for SDPA / generic attention backend
            support" (Suggestion 2: dense [B,1,Q_LEN,KV_LEN] bool mask).
  [FSA-190] flash-sparse-attention PR #190, "Broadcastable 4D mask/bias,
            128-rounded key length, stride-0 broadcasting, and dbias
            reductions" (sections: Summary, Design, Changes, Implementation
            Notes, Tests).
  [FSA-197] flash-sparse-attention PR #197, "Centralize dynamic mask creation
            for FDMA" (sections: Design, Changes, Implementation Notes, review
            suggestion on dynamic_mask).

Modules:
  dflash     -- DFlash draft-block predicate: is_causal resolution and the dense
                boolean mask (pinned: brute-force rule tables, closed forms);
                the inference geometry of one block after a KV cache (pinned:
                worked example, the last block of a training sequence).
  blockmask  -- 128x128 tile classification into empty / partial / full and
                the inverse expansion (pinned: round trip, per-head identity).
  topk       -- dynamic top-k keep mask over an additive bias (pinned: O(K^2)
                rank formula, kept-count invariants, argmax / constant rows).
  attention  -- float64 softmax attention over the kept keys (pinned: SDPA in
                float64, single-key rows, convexity, GQA and broadcast
                identities).
  attention_bwd -- float64 gradients dQ / dK / dV / dbias of the same
                attention (pinned: central finite differences of the forward
                oracle, torch autograd in float64, broadcast dbias reductions).
  normalize  -- 2D/4D pre-mask normalisation and key-length rounding.
  varlen     -- packed variable-length sequences: pad / unpad, per-sequence
                DFlash geometry, packed attention, its gradients and its
                block mask (pinned: worked example, round trip, padded-batch
                equivalences, finite differences of the packed forward).
  keylist    -- kept-key list of a dense mask over at most 32 query rows, with
                a bit per row (pinned: hand-worked example, round trip,
                top-k count invariant, attention over the gathered keys).

No function here is "parity unpinned" except where its docstring says so.
"""

from .dflash import (  # noqa: F401
    DFlashGeom,
    resolve_dflash_is_causal,
    dflash_dense_mask,
    dflash_inference_geom,
)
from .blockmask import TILE, classify_tiles, expand_block_mask  # noqa: F401
from .topk import finfo_min, topk_keep_mask, topk_rank_bruteforce  # noqa: F401
from .attention import attention_rows, attention_full  # noqa: F401
from .attention_bwd import attention_bwd, group_grads, head_grads  # noqa: F401
from .normalize import round_multiple, normalize_premask  # noqa: F401
from .keylist import key_list, expand_key_list  # noqa: F401
from .varlen import (attention_varlen, attention_varlen_bwd, block_mask_varlen,  # noqa: F401
                     dflash_varlen_geoms, pad, unpad)
