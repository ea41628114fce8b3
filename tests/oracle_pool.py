"""The fp64 oracle over a pool of host processes, for the full-size parity
tests (test infrastructure only).

Workers draw the workloads' seeded inputs themselves with
block_sparse_masked_mask_amd.synth (the generators the GPU run uses) and build
every mask with the oracle's own functions, so nothing a worker computes comes
from a GPU result. Work goes out in units of (batch, head) or query-tile
ranges; the test compares the returned rows with the GPU's.

The pool's processes are forked from a fork server that tests/conftest.py
starts before the test process touches the GPU, so no process that has used
the GPU forks or execs. Each worker runs one BLAS thread; the pool has as many
workers as the process may use CPUs, at most 16.
"""

import multiprocessing as mp
import os

import numpy as np

_POOL = None
_CACHE = {}
_LIMITS = None

# one BLAS / OpenMP thread per worker (read when the worker first loads NumPy)
_THREAD_ENV = {"OMP_NUM_THREADS": "1", "OPENBLAS_NUM_THREADS": "1", "MKL_NUM_THREADS": "1"}


def start_server():
    """Start the fork server (call before any GPU use in this process)."""
    from multiprocessing import forkserver
    saved = {k: os.environ.get(k) for k in _THREAD_ENV}
    os.environ.update(_THREAD_ENV)
    try:
        # preloading this module hands the server our sys.path
        mp.set_forkserver_preload(["oracle_pool"])
        forkserver.ensure_running()
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def pool():
    global _POOL
    if _POOL is None:
        import atexit
        _POOL = mp.get_context("forkserver").Pool(workers(), initializer=_init)
        atexit.register(close)
    return _POOL


def close():
    global _POOL
    if _POOL is not None:
        _POOL.close()
        _POOL.join()
        _POOL = None


def run(fn, jobs):
    """fn(job) for every job, in order, on the pool."""
    return pool().map(fn, jobs, chunksize=1)


def _init():
    global _LIMITS
    from threadpoolctl import threadpool_limits
    _LIMITS = threadpool_limits(1)


# ---------------------------------------------------------------------------
# inputs, drawn once per worker


def _f32(t):
    """float32 NumPy copy of a stored tensor (exact for bf16 and f32 values)."""
    import torch
    return t.to(torch.float32).numpy()


def dflash_geom(cfg, layer):
    import oracle
    return oracle.DFlashGeom(cfg["ctx_len"], cfg["num_blocks"], cfg["block_size"], 0, 0,
                             layer["is_causal"], layer["layer_type"], layer["window"])


def _dflash(name, li):
    key = ("dflash", name, li)
    if key not in _CACHE:
        from block_sparse_masked_mask_amd import synth
        cfg = synth.CONFIGS[name]
        g = dflash_geom(cfg, cfg["layers"][li])
        qkv_key = ("qkv", name)
        if qkv_key not in _CACHE:
            q, k, v = synth.qkv(cfg["B"], g.Sq, g.Sk, cfg["H"], cfg["KVH"], cfg["D"],
                                cfg["dtype"], seed=0, scale=cfg["qkv_scale"])
            _CACHE[qkv_key] = (_f32(q), _f32(k), _f32(v))
        _CACHE[key] = _CACHE[qkv_key] + (g,)
    return _CACHE[key]


def topk_mask(cfg, bias, pad2d):
    """The oracle's top-k keep mask of a top-k workload (pre-mask normalised
    from the 2D padding mask when there is one)."""
    import oracle
    pre = None
    if pad2d is not None:
        pre = oracle.normalize_premask(np.asarray(pad2d), cfg["B"], cfg["Sk"])
    return oracle.topk_keep_mask(bias, pre, cfg["Sk"], cfg["topk"], cfg["dtype"])


def _topk(name):
    key = ("topk", name)
    if key not in _CACHE:
        from block_sparse_masked_mask_amd import synth
        cfg = synth.CONFIGS[name]
        q, k, v = synth.qkv(cfg["B"], cfg["Sq"], cfg["Sk"], cfg["H"], cfg["KVH"], cfg["D"],
                            cfg["dtype"], seed=0, scale=cfg["qkv_scale"])
        bias_t, pad2d = synth.topk_inputs(cfg, seed=0)
        bias = _f32(bias_t).astype(np.float64)
        mask = topk_mask(cfg, bias, None if pad2d is None else pad2d.numpy())
        _CACHE[key] = (_f32(q), _f32(k), _f32(v), bias, mask)
    return _CACHE[key]


# ---------------------------------------------------------------------------
# jobs (module-level functions, so the pool can name them)


def dflash_rows(job):
    """(name, layer index, b, h, rows) -> oracle (O, LSE) of those rows."""
    import oracle
    name, li, b, h, rows = job
    q, k, v, g = _dflash(name, li)
    return oracle.attention_rows(q, k, v, b, h, np.asarray(rows), mask=g)


def dflash_tile_classes(job):
    """(name, layer index, query tiles) -> [(partial, full)] per tile, from the
    oracle's dense rows of each tile."""
    import oracle
    from oracle.blockmask import classify_tile_band
    from block_sparse_masked_mask_amd import synth
    name, li, tiles = job
    cfg = synth.CONFIGS[name]
    g = dflash_geom(cfg, cfg["layers"][li])
    out = []
    for qt in tiles:
        rows = np.arange(qt * 128, min(qt * 128 + 128, g.Sq))
        band = oracle.dflash_dense_mask(g, rows)
        out.append(classify_tile_band(band, g.Sk))
    return out


def topk_rows(job):
    """(name, b, h, rows) -> oracle (O, LSE) of those rows under the oracle's
    top-k mask and the bias."""
    import oracle
    name, b, h, rows = job
    q, k, v, bias, mask = _topk(name)
    return oracle.attention_rows(q, k, v, b, h, np.asarray(rows), mask=mask, bias=bias)


def topk_mask_rows(job):
    """(name, b) -> the oracle's top-k mask rows of batch b (all heads)."""
    from block_sparse_masked_mask_amd import synth
    name, b = job
    key = ("bias", name)
    if key not in _CACHE:
        cfg = synth.CONFIGS[name]
        bias_t, pad2d = synth.topk_inputs(cfg, seed=0)
        _CACHE[key] = (cfg, _f32(bias_t).astype(np.float64),
                       None if pad2d is None else pad2d.numpy())
    cfg, bias, pad2d = _CACHE[key]
    sub = dict(cfg, B=1)
    return topk_mask(sub, bias[b:b + 1], None if pad2d is None else pad2d[b:b + 1])


def _dout(name, shape, seed, dtype):
    key = ("dout", name, seed)
    if key not in _CACHE:
        from block_sparse_masked_mask_amd import synth
        _CACHE[key] = _f32(synth.normal_tensor(tuple(shape), seed, synth.TID_DOUT, dtype))
    return _CACHE[key]


def bwd_head(job):
    """(name, layer index, b, h, dO seed) -> the oracle's dQ (Sq, D), dK and dV
    (Sk, D) of head h of batch b, and its dS summed over queries (Sk,), under
    the workload's own mask (DFlash rule, or the oracle's top-k and the bias)."""
    from oracle.attention_bwd import head_grads
    from block_sparse_masked_mask_amd import synth
    name, li, b, h, seed = job
    cfg = synth.CONFIGS[name]
    if cfg["kind"] == "dflash":
        q, k, v, g = _dflash(name, li)
        mask, bias = g, None
    else:
        q, k, v, bias, mask = _topk(name)
    do = _dout(name, q.shape, seed, cfg["dtype"])
    dQ, dK, dV, dS = head_grads(q, k, v, do, b, h, mask=mask, bias=bias)
    return dQ, dK, dV, dS.sum(axis=0)

