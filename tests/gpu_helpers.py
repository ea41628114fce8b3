"""Helpers shared by the GPU parity tests (no test functions here)."""

import sys

import numpy as np
import torch

import oracle
from block_sparse_masked_mask_amd import bsm, synth

# tolerances of the fp64 comparison: bf16 path max/mean abs error, f32 max
BF16_MAX, BF16_MEAN, F32_MAX = 2e-2, 2e-3, 1e-4


def say(*a):
    """Print and flush, so a GPU fault still leaves the case name behind."""
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_geom(d):
    return oracle.DFlashGeom(d.ctx_len, d.num_blocks, d.block_size, d.ctx_per_block,
                             d.ctx_end_offset, d.is_causal, d.layer_type, d.sliding_window)


def np_bm(bm):
    return [t.cpu().numpy() for t in bm]


def assert_bm_equal(got, want, msg=""):
    names = ["kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices"]
    for n, a, b in zip(names, got, want):
        a = np.asarray(a)
        b = np.asarray(b)
        assert a.shape == b.shape, f"{msg} {n}: shape {a.shape} vs {b.shape}"
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)[:5]
            raise AssertionError(f"{msg} {n}: {len(np.argwhere(a != b))} mismatches, first "
                                 f"{[(tuple(i), a[tuple(i)], b[tuple(i)]) for i in bad]}")


def assert_close(got, want, dtype, what=""):
    """Elementwise comparison against the fp64 oracle with the stated bars."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    ninf_g, ninf_w = np.isneginf(got), np.isneginf(want)
    assert np.array_equal(ninf_g, ninf_w), f"{what}: -inf pattern differs"
    fin = ~ninf_w
    assert np.isfinite(got[fin]).all(), f"{what}: non-finite values"
    err = np.abs(got[fin] - want[fin])
    if err.size == 0:
        return
    if dtype == "bf16":
        assert err.max() <= BF16_MAX, f"{what}: max |err| {err.max():.3e} > {BF16_MAX}"
        assert err.mean() <= BF16_MEAN, f"{what}: mean |err| {err.mean():.3e} > {BF16_MEAN}"
    else:
        assert err.max() <= F32_MAX, f"{what}: max |err| {err.max():.3e} > {F32_MAX}"


def assert_grad_close(got, want, dt, what):
    """Gradients against the fp64 oracle, the bars scaled by max(1, max|want|):
    bf16 max |err| <= 2e-2 and mean |err| <= 2e-3, f32 max |err| <= 1e-4."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    m = max(1.0, float(np.abs(want).max()) if want.size else 1.0)
    err = np.abs(got - want)
    if err.size == 0:
        return
    if dt == "bf16":
        assert err.max() <= 2e-2 * m, f"{what}: max |err| {err.max():.3e} > {2e-2 * m:.3e}"
        assert err.mean() <= 2e-3 * m, f"{what}: mean |err| {err.mean():.3e} > {2e-3 * m:.3e}"
    else:
        assert err.max() <= 1e-4 * m, f"{what}: max |err| {err.max():.3e} > {1e-4 * m:.3e}"


def batch_slice(t, b):
    """Batch b of a 4D aux tensor that broadcasts over batch when its dim is 1."""
    if t is None:
        return None
    return t[b:b + 1] if t.shape[0] > 1 else t


def oracle_rows(q, k, v, b, h, rows, scale=None, mask=None, bias=None):
    """fp64 oracle O/LSE for batch b, head h and the given rows.

    q/k/v/mask/bias are torch tensors (any device); only batch b is copied to
    the host. mask may also be an oracle.DFlashGeom.
    """
    qb = synth.as_f64(q[b:b + 1])
    kb = synth.as_f64(k[b:b + 1])
    vb = synth.as_f64(v[b:b + 1])
    m = mask
    if isinstance(mask, torch.Tensor):
        m = batch_slice(mask, b).cpu().numpy()
    bi = synth.as_f64(batch_slice(bias, b)) if bias is not None else None
    return oracle.attention_rows(qb, kb, vb, 0, h, rows, scale=scale, mask=m, bias=bi)


def sample_rows(Sq, n, seed):
    """First, last, tile-boundary and random query rows."""
    rng = np.random.default_rng(seed)
    base = {0, Sq - 1, min(127, Sq - 1), min(128, Sq - 1)}
    base |= set(rng.integers(0, Sq, size=n).tolist())
    return np.array(sorted(base))


def oracle_topk_mask(bias, seqlen_k, k, dtype="bf16"):
    """The oracle's top-k keep mask of a stored bias, as a bool tensor on the
    bias's device. Tests that need a top-k mask for attention use this one for
    both the GPU run and the oracle, so the oracle never takes a mask the GPU
    built (the GPU's top-k is compared with it bit for bit elsewhere)."""
    m = oracle.topk_keep_mask(synth.as_f64(bias), None, seqlen_k, k, dtype)
    return torch.from_numpy(m).to(bias.device)


def cuda(*ts):
    return [None if t is None else t.cuda() for t in ts]


__all__ = ["bsm", "synth", "oracle", "say", "oracle_geom", "np_bm", "assert_bm_equal",
           "assert_close", "oracle_rows", "sample_rows", "cuda", "batch_slice",
           "oracle_topk_mask"]
