"""Pins for the DFlash oracle (mask rules and tile classification).

Each test checks the oracle against something other than itself: hand-written
tables from the pages' rules (tests/golden), the worked tiny case the pages'
DFlash description gives, closed-form tile and kept-pair counts derived by
interval arithmetic, and special cases that reduce to textbook masks.
"""

import json
import os

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import DFlashGeom, classify_tiles, dflash_dense_mask, resolve_dflash_is_causal
from oracle.blockmask import classify_tile_band, expand_block_mask


def _load_tiny_cases():
    cases, cur = [], None
    for line in open(os.path.join(GOLDEN, "dflash_tiny_masks.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("case"):
            parts = line.split()
            kv = dict(p.split("=") for p in parts[2:])
            ic = {"none": None, "true": True, "false": False}[kv["is_causal"]]
            cur = dict(name=parts[1], is_causal=ic, layer=kv["layer"],
                       window=int(kv["window"]), rows=[])
            cases.append(cur)
        else:
            cur["rows"].append([c == "1" for c in line.replace(" ", "")])
    return cases


TINY = _load_tiny_cases()


def test_is_causal_table():
    tab = json.load(open(os.path.join(GOLDEN, "dflash_is_causal.json")))["table"]
    for e in tab:
        assert resolve_dflash_is_causal(e["is_causal"], e["layer_type"]) == e["causal"]
        # the C-style encoding of the same table
        ic = -1 if e["is_causal"] is None else int(e["is_causal"])
        lt = 0 if e["layer_type"] == "full" else 1
        assert resolve_dflash_is_causal(ic, lt) == e["causal"]


@pytest.mark.parametrize("bad", [("full", 2), ("sliding", -2), ("other", None), (3, 1)])
def test_is_causal_rejects(bad):
    lt, ic = bad
    with pytest.raises(ValueError):
        resolve_dflash_is_causal(ic, lt)


@pytest.mark.parametrize("case", TINY, ids=[c["name"] for c in TINY])
def test_tiny_tables(case):
    g = DFlashGeom(8, 2, 4, is_causal=case["is_causal"], layer_type=case["layer"],
                   sliding_window=case["window"])
    m = dflash_dense_mask(g)
    assert m.shape == (8, 128)
    assert not m[:, 16:].any()
    np.testing.assert_array_equal(m[:, :16], np.array(case["rows"]))


def test_worked_tiny_case():
    """256 context tokens, 4 draft blocks of 16, full layer, is_causal absent:
    draft block j sees context positions < 64*j + 64 and its own block both
    ways, nothing else."""
    g = DFlashGeom(256, 4, 16, layer_type="full")
    m = dflash_dense_mask(g)
    assert m.shape == (64, 384)
    for q in range(64):
        j = q // 16
        want = np.zeros(384, bool)
        want[:64 * j + 64] = True
        want[256 + 16 * j:256 + 16 * j + 16] = True
        np.testing.assert_array_equal(m[q], want)
    assert m.sum() == 11264  # sum_j 16 * (64 (j+1) + 16)


def test_no_context_bidirectional_is_all_keep():
    g = DFlashGeom(0, 1, 48, ctx_per_block=1, layer_type="full", is_causal=False)
    m = dflash_dense_mask(g)
    assert m[:, :48].all() and not m[:, 48:].any()


def test_no_context_causal_is_block_diagonal_causal():
    g = DFlashGeom(0, 3, 40, ctx_per_block=1, layer_type="full", is_causal=True)
    m = dflash_dense_mask(g)[:, :120]
    want = np.zeros((120, 120), bool)
    for j in range(3):
        want[40 * j:40 * j + 40, 40 * j:40 * j + 40] = np.tril(np.ones((40, 40), bool))
    np.testing.assert_array_equal(m, want)


def _window_context_count(E, i, W):
    """Visible context keys of draft token (E_j, i) under a left-bound window W:
    keys c with c < E_j and (E_j + i) - c < W, i.e. c in [max(0, E_j+i-W+1), E_j)."""
    return max(0, E - max(0, E + i - W + 1))


def test_train_shape_kept_pairs():
    """DFlash training shape (C=4096, 256 blocks of 16): kept pairs per head,
    full layer bidirectional and sliding layer causal with W=2048, counted row
    by row from interval lengths."""
    full = DFlashGeom(4096, 256, 16, layer_type="full")
    slid = DFlashGeom(4096, 256, 16, layer_type="sliding", sliding_window=2048)
    want_full = sum(16 * (16 * (j + 1) + 16) for j in range(256))
    want_slid = sum(_window_context_count(16 * (j + 1), i, 2048) + (i + 1)
                    for j in range(256) for i in range(16))
    assert want_full == 8486912
    got_full = got_slid = 0
    for r0 in range(0, 4096, 512):
        rows = np.arange(r0, r0 + 512)
        got_full += int(dflash_dense_mask(full, rows).sum())
        got_slid += int(dflash_dense_mask(slid, rows).sum())
    assert got_full == want_full
    assert got_slid == want_slid


def _closed_form_counts(t, W_tiles):
    """Tiles of query tile t when S = bs = 16 (8 draft blocks per 128-row tile).

    Context tile kt is full iff every row sees all of it: kt <= t-1 (the first
    block of the tile sees only 16 keys of tile t) and, under a window of
    W = 128*W_tiles keys, kt >= t - (W_tiles - 2). Partial: the diagonal
    context tile t, the draft tile, and under a window the two tiles below the
    full run. Derived from E_j = 16(j+1), pos = E_j + i, lower bound pos-W+1.
    """
    if W_tiles is None:
        return t, 2
    span = W_tiles - 2
    full = min(t, span)
    partial = 2 + (t >= span + 1) + (t >= span + 2)
    return full, partial


@pytest.mark.parametrize("layer", ["full", "sliding"])
def test_train_shape_tile_counts(layer):
    g = DFlashGeom(4096, 256, 16, layer_type=layer,
                   sliding_window=2048 if layer == "sliding" else 0)
    m = dflash_dense_mask(g)[None, None]
    kv_num, kv_idx, full_num, full_idx = classify_tiles(m, g.Sk)
    assert kv_num.shape == (1, 1, 32) and kv_idx.shape == (1, 1, 32, 64)
    for t in range(32):
        f, p = _closed_form_counts(t, None if layer == "full" else 16)
        assert (full_num[0, 0, t], kv_num[0, 0, t]) == (f, p), t
    tot = (int(full_num.sum()), int(kv_num.sum()))
    assert tot == ((496, 64) if layer == "full" else (343, 97))
    # round trip: full tiles all True, partial tiles the mask, others empty
    back = expand_block_mask(kv_num, kv_idx, full_num, full_idx, m, g.Sq)
    np.testing.assert_array_equal(back, m)


def test_long_context_tile_counts_sampled():
    """Long-context DFlash (C=32768, 2048 blocks of 16, causal, W=4096):
    closed-form counts on a sample of query tiles, and the 7215 / 961 totals."""
    g = DFlashGeom(32768, 2048, 16, is_causal=True, layer_type="sliding", sliding_window=4096)
    for t in [0, 1, 2, 29, 30, 31, 32, 33, 128, 254, 255]:
        band = dflash_dense_mask(g, np.arange(128 * t, 128 * t + 128))
        part, full = classify_tile_band(band, g.Sk)
        assert (len(full), len(part)) == _closed_form_counts(t, 32), t
        # full run is contiguous and ends right below the diagonal
        if len(full):
            assert full[-1] == t - 1 and full[0] == max(0, t - 30)
        assert 256 + t in part
    full_tot = sum(_closed_form_counts(t, 32)[0] for t in range(256))
    part_tot = sum(_closed_form_counts(t, 32)[1] for t in range(256))
    assert (full_tot, part_tot) == (7215, 961)


def test_head_independent_block_mask_equals_per_head():
    """One block mask shared by all heads equals each head's own block mask."""
    g = DFlashGeom(512, 16, 16, layer_type="sliding", sliding_window=300)
    d = dflash_dense_mask(g)
    per_head = np.broadcast_to(d, (2, 4) + d.shape)
    one = classify_tiles(d[None, None], g.Sk)
    many = classify_tiles(per_head, g.Sk)
    for a, b in zip(one, many):
        assert (b == a).all()


def test_blockmask_golden():
    fx = json.load(open(os.path.join(GOLDEN, "blockmask_tiny.json")))["expected"]
    m = np.zeros((1, 1, 130, 384), bool)
    m[0, 0, :128, :128] = True
    m[0, 0, 5, 200] = True
    m[0, 0, :128, 256:] = True
    m[0, 0, 128:130, :128] = True
    m[0, 0, 128:130, 256:300] = True
    got = classify_tiles(m, 300)
    for name, arr in zip(["kv_num_blocks", "kv_indices", "full_kv_num_blocks",
                          "full_kv_indices"], got):
        np.testing.assert_array_equal(arr, np.array(fx[name]), err_msg=name)


def test_blockmask_round_trip_random():
    rng = np.random.default_rng(7)
    Bm, Hm, Qm, nK, Sk = 2, 3, 300, 5, 600
    m = np.zeros((Bm, Hm, Qm, nK * 128), bool)
    for b in range(Bm):
        for h in range(Hm):
            for qt in range(3):
                for kt in range(nK):
                    kind = rng.integers(3)
                    r0, r1 = qt * 128, min(qt * 128 + 128, Qm)
                    blk = m[b, h, r0:r1, kt * 128:(kt + 1) * 128]
                    if kind == 1:
                        blk[:] = True
                    elif kind == 2:
                        blk[:] = rng.random(blk.shape) < 0.3
    m[..., Sk:] = False
    got = classify_tiles(m, Sk)
    back = expand_block_mask(*got, m, Qm)
    np.testing.assert_array_equal(back, m)
    # a full tile is never listed when it straddles seqlen_k
    assert not (got[3] == Sk // 128).any()


# ---------------------------------------------------------------------------
# inference geometry: one draft block after a KV cache of C tokens


def test_inference_worked_example():
    """C = 5 cached tokens, a block of 3, causal sliding layer with W = 4: token
    i sits at position 5 + i and sees cached keys c with 5 + i - c < 4 and its
    own tokens i' <= i."""
    from oracle import dflash_inference_geom
    g = dflash_inference_geom(5, 3, is_causal=True, layer_type="sliding", sliding_window=4)
    m = dflash_dense_mask(g)
    assert m.shape == (3, 128) and not m[:, 8:].any()
    want = [[0, 0, 1, 1, 1, 1, 0, 0],
            [0, 0, 0, 1, 1, 1, 1, 0],
            [0, 0, 0, 0, 1, 1, 1, 1]]
    np.testing.assert_array_equal(m[:, :8], np.array(want, bool))
    full = dflash_dense_mask(dflash_inference_geom(5, 3))
    assert full[:, :8].all() and not full[:, 8:].any()


@pytest.mark.parametrize("is_causal,layer,window", [
    (None, "full", 0), (None, "sliding", 40), (True, "full", 0), (False, "sliding", 25),
    (True, "sliding", 300),
])
def test_inference_is_last_training_block(is_causal, layer, window):
    """The inference mask equals the last block of a training sequence with the
    same context: its rows, on the context keys and that block's own keys."""
    from oracle import dflash_inference_geom
    C, NB, bs = 240, 6, 16
    train = dflash_dense_mask(DFlashGeom(C, NB, bs, is_causal=is_causal, layer_type=layer,
                                         sliding_window=window))
    last = train[(NB - 1) * bs:NB * bs]
    cols = np.r_[0:C, C + (NB - 1) * bs:C + NB * bs]
    inf = dflash_dense_mask(dflash_inference_geom(C, bs, is_causal, layer, window))
    np.testing.assert_array_equal(inf[:, :C + bs], last[:, cols])
    assert not inf[:, C + bs:].any()
