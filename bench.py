"""Benchmark of the block-sparse masked attention hot path on one MI355X.

One step = one pass of the DFlash training-shape workload through the library:
resolve the layer's in-block causality, build the head-shared block mask from the
DFlash predicate, and run the masked attention forward -- for a full-attention
layer (bidirectional in-block) and a sliding-window layer (causal in-block,
left-bound window 2048). B=2, H=32, KVH=8, D=128, 4096 context tokens + 256 draft
blocks of 16 (Sq=4096 queries, Sk=8192 keys), bf16, Q/K/V ~ 0.5 N(0,1).

value = counted flops of the step / step time, where counted flops are
4 * D * (rows x keys) summed over the non-empty 128x128 tiles of every (b, h)
(QK^T plus PV; exp not counted). The JSON line also carries:
  roofline     -- the attention kernel alone: algorithmic flops per launch over
                  its HIP-event-timed average launch duration, against the bf16
                  dense MFMA peak;
  mask_build   -- the dense-mask block-mask builder on the long-context DFlash
                  mask materialised densely (1 x 1 x 32768 x 65536 bytes), GB/s
                  against HBM peak;
  configs      -- the other workloads at full size: long-context DFlash (TFLOP/s,
                  fraction of peak, device memory), dynamic top-k (TFLOP/s,
                  fraction of peak), decode (GB/s of the tile and the gather
                  path against HBM peak), tiny fp32 (launch time); the
                  backward of the training shape and of the dynamic-mask
                  workload with dbias, and the packed 4-sequence pack forward
                  and backward (ms, TFLOP/s counted);
  cpu_baseline -- the CPU oracle on a pool of one-thread host processes, one
                  per usable core (at most 16), on a bounded random sample of
                  every workload: wall seconds, oracle seconds, extrapolated
                  full-workload seconds; `value` is the training step's.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-configs] [--no-mask-build]
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from block_sparse_masked_mask_amd import bsm, synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
WORKLOAD = "dflash_train_bf16"
METRIC = "masked attn fwd TFLOP/s on kept tiles (% bf16 MFMA peak); mask build GB/s"


# HBM bytes per launch of the attention kernel on this workload, from two
# rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch, averaged over
# both layers) scaled by what the same counters read for a 1 GiB device copy
# (FETCH_SIZE reads 0.5 GiB for it, so x2.0; WRITE_SIZE reads 1 GiB, so x1.0).
# The figure holds only for the kernel sources it was taken on: when their hash
# differs, traffic is reported as null. (The hash moved once without new
# counters, after a header edit that left the kernel's gfx950 code unchanged,
# instruction for instruction.)
ATTN_TRAFFIC = {"sources": ["attn_v2.hip", "attn_pipe.h", "attn_common.h", "bsm_internal.h",
                            "dflash_rows.h"],
                "sha256_16": "ca0ab43dc6590f7e",
                "fetch_kib": 86603.2, "write_kib": 65536.0,
                "fetch_scale": 2.0, "write_scale": 1.0}


def attn_traffic_bytes():
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_TRAFFIC["sources"]:
        with open(os.path.join(ROOT, "block_sparse_masked_mask_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != ATTN_TRAFFIC["sha256_16"]:
        return None
    t = ATTN_TRAFFIC
    return 1024.0 * (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"])


def counted_flops(bm, geom):
    """4*D*rows*keys over non-empty tiles of every (b, h), from a block mask."""
    B, H, KVH, Sq, Sk, D = geom
    kvn, kvi, fn, fi = [t.cpu().numpy() for t in bm]
    Bm, Hm, nQm, nK = kvi.shape
    total = 0
    for b in range(B):
        for h in range(H):
            mb = 0 if Bm == 1 else b
            mh = 0 if Hm == 1 else (h if Hm == H else h // (H // KVH))
            for qt in range((Sq + 127) // 128):
                mq = 0 if nQm == 1 else qt
                rows = min(128, Sq - 128 * qt)
                tiles = list(kvi[mb, mh, mq, :kvn[mb, mh, mq]]) + \
                    list(fi[mb, mh, mq, :fn[mb, mh, mq]])
                for kt in tiles:
                    total += rows * min(128, Sk - 128 * int(kt))
    return 4 * D * total


class Step:
    """The DFlash training-shape step: both layers, block mask + attention."""

    def __init__(self, seed=0):
        cfg = synth.CONFIGS[WORKLOAD]
        self.cfg = cfg
        self.layers = []
        for lay in cfg["layers"]:
            d = bsm.DFlash(cfg["ctx_len"], cfg["num_blocks"], cfg["block_size"],
                           is_causal=lay["is_causal"], layer_type=lay["layer_type"],
                           sliding_window=lay["window"])
            self.layers.append((lay["name"], d))
        d0 = self.layers[0][1]
        self.q, self.k, self.v = [t.cuda() for t in synth.qkv(
            cfg["B"], d0.Sq, d0.Sk, cfg["H"], cfg["KVH"], cfg["D"], "bf16", seed=seed,
            scale=cfg["qkv_scale"])]
        self.geom = bsm.geometry_of(self.q, self.k)
        self.out = [torch.empty_like(self.q) for _ in self.layers]
        self.bms = [bsm.build_block_mask(self.geom, pred=d) for _, d in self.layers]
        self.flops = [counted_flops(bm, self.geom) for bm in self.bms]
        self.attn_events = []

    def run(self, record=False):
        stream = torch.cuda.current_stream()
        for i, (name, d) in enumerate(self.layers):
            bsm.resolve_dflash_is_causal(d.is_causal, d.layer_type)
            bm = bsm.build_block_mask(self.geom, pred=d)
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            bsm.masked_attn_fwd(self.q, self.k, self.v, pred=d, block_mask=bm, out=self.out[i])
            if record:
                e1.record(stream)
                self.attn_events.append((i, e0, e1))


def measure_mask_build(reps=5):
    """Dense builder on the long-context DFlash mask written out densely."""
    d = bsm.DFlash(32768, 2048, 16, is_causal=True, layer_type="sliding", sliding_window=4096)
    geom = bsm.Geometry(1, 32, 8, d.Sq, d.Sk, 128)
    dense = bsm.dflash_dense_mask(geom, d)[None, None]
    bm = bsm.build_block_mask(geom, mask=dense)  # warm
    ref = bsm.build_block_mask(geom, pred=d)
    for a, b in zip(bm, ref):
        if not torch.equal(a, b):
            raise RuntimeError("dense and predicate block masks differ")
    nbytes = dense.numel() + 4 * sum(t.numel() for t in bm)
    ms = _time_ms(lambda: bsm.build_block_mask(geom, mask=dense), reps=reps)
    del dense
    return {"workload": "long_dflash_dense_mask", "shape": [1, 1, d.Sq, 65536],
            "bytes": int(nbytes), "ms": ms, "GB/s": nbytes / ms / 1e6,
            "frac": nbytes / ms / 1e6 / PEAK_HBM_GBS}


def device_info(mib=1024, reps=5):
    """Name, CU count and peak clock of cuda:0, and the GB/s of a plain device
    copy of mib MiB (read + write bytes over the copy time): the measured
    counterpart of the 8 TB/s HBM peak used as the denominator."""
    import ctypes
    props = torch.cuda.get_device_properties(0)
    clock_khz = ctypes.c_int(0)
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        # hipDeviceAttributeClockRate: 5 in hip_runtime_api.h's enum (kHz)
        hip.hipDeviceGetAttribute(ctypes.byref(clock_khz), 5, 0)
    except OSError:
        pass
    n = mib << 20
    src = torch.full((n,), 1, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms = _time_ms(lambda: dst.copy_(src), reps=reps)
    del src, dst
    return {"name": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count,
            "clock_mhz": clock_khz.value / 1000.0, "copy_GB/s": 2 * n / (ms * 1e-3) / 1e9}


def copy_probe(mib=1024, reps=3):
    """Plain device-to-device copy of a known size: the calibration run for the
    HBM byte counters (each copy reads and writes mib MiB)."""
    n = mib << 20
    src = torch.full((n,), 1, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "reps": reps}), flush=True)


def _time_ms(fn, reps=10):
    """Average ms of fn() over reps back-to-back launches (HIP events on the stream)."""
    fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def measure_backward():
    """Backward of the DFlash training shape, both layers: dQ/dK/dV from the
    forward's O and LSE. Counted flops: 2.5x the forward's (the five products
    QK^T, dO V^T, P^T dO, dS^T Q, dS K over the kept tiles)."""
    out = {}
    cfg = synth.CONFIGS["dflash_train_bf16"]
    for lay in cfg["layers"]:
        d = bsm.DFlash(cfg["ctx_len"], cfg["num_blocks"], cfg["block_size"],
                       is_causal=lay["is_causal"], layer_type=lay["layer_type"],
                       sliding_window=lay["window"])
        q, k, v = [t.cuda() for t in synth.qkv(cfg["B"], d.Sq, d.Sk, cfg["H"], cfg["KVH"],
                                               cfg["D"], "bf16", seed=0, scale=cfg["qkv_scale"])]
        geom = bsm.geometry_of(q, k)
        bm = bsm.build_block_mask(geom, pred=d)
        o, lse = bsm.masked_attn_fwd(q, k, v, pred=d, block_mask=bm, return_lse=True)
        do = synth.normal_tensor(tuple(q.shape), 0, synth.TID_DOUT, "bf16").cuda()
        ms = _time_ms(lambda: bsm.masked_attn_bwd(q, k, v, o, do, lse, pred=d, block_mask=bm),
                      reps=10)
        fl = 2.5 * counted_flops(bm, geom)
        out[f"attn_bwd/dflash_train_bf16/{lay['name']}_ms"] = ms
        out[f"attn_bwd/dflash_train_bf16/{lay['name']}_TFLOP/s"] = fl / (ms * 1e-3) / 1e12
        del q, k, v, o, do
    # the dynamic-mask workload: top-k mask, bias per KV head broadcast over
    # queries, and its gradient dbias
    cfg = synth.CONFIGS["dynamic_topk_bf16"]
    B, H, KVH, D, Sq, Sk = (cfg[x] for x in ("B", "H", "KVH", "D", "Sq", "Sk"))
    q, k, v = [t.cuda() for t in synth.qkv(B, Sq, Sk, H, KVH, D, "bf16", seed=0)]
    bias, pad2d = [t.cuda() for t in synth.topk_inputs(cfg, seed=0)]
    mask = bsm.create_mask(bias, pad2d, B, Sq, Sk, cfg["topk"])
    geom = bsm.geometry_of(q, k)
    bm = bsm.build_block_mask(geom, mask=mask)
    o, lse = bsm.masked_attn_fwd(q, k, v, mask=mask, bias=bias, block_mask=bm, return_lse=True)
    do = synth.normal_tensor(tuple(q.shape), 0, synth.TID_DOUT, "bf16").cuda()
    ms = _time_ms(lambda: bsm.masked_attn_bwd(q, k, v, o, do, lse, mask=mask, bias=bias,
                                              block_mask=bm, need_dbias=True), reps=10)
    fl = 2.5 * counted_flops(bm, geom)
    out["attn_bwd/dynamic_topk_bf16_dbias_ms"] = ms
    out["attn_bwd/dynamic_topk_bf16_dbias_TFLOP/s"] = fl / (ms * 1e-3) / 1e12
    del q, k, v, o, do
    return out


def measure_one_head():
    """The DFlash training geometry with MHA (H = KVH = 32, so no head pairs):
    attention on the one-head-per-workgroup kernel, TFLOP/s on kept tiles."""
    out = {}
    cfg = synth.CONFIGS["dflash_train_bf16"]
    for lay in cfg["layers"]:
        d = bsm.DFlash(cfg["ctx_len"], cfg["num_blocks"], cfg["block_size"],
                       is_causal=lay["is_causal"], layer_type=lay["layer_type"],
                       sliding_window=lay["window"])
        q, k, v = [t.cuda() for t in synth.qkv(cfg["B"], d.Sq, d.Sk, 32, 32, cfg["D"], "bf16",
                                               seed=0, scale=cfg["qkv_scale"])]
        geom = bsm.geometry_of(q, k)
        bm = bsm.build_block_mask(geom, pred=d)
        fl = counted_flops(bm, geom)
        o = torch.empty_like(q)
        ms = _time_ms(lambda: bsm.masked_attn_fwd(q, k, v, pred=d, block_mask=bm, out=o), reps=5)
        out[f"attn_one_head/dflash_train_mha_bf16/{lay['name']}_ms"] = ms
        out[f"attn_one_head/dflash_train_mha_bf16/{lay['name']}_TFLOP/s"] = fl / (ms * 1e-3) / 1e12
        del q, k, v, o
    return out


def measure_components():
    """Per-kernel times of the other workloads (parity cases, not the headline)."""
    out = measure_backward()
    out.update(measure_one_head())
    # DFlash block masks from the predicate (integer work, output only)
    for name in ("dflash_train_bf16", "long_dflash_bf16"):
        cfg = synth.CONFIGS[name]
        for lay in cfg["layers"]:
            d = bsm.DFlash(cfg["ctx_len"], cfg["num_blocks"], cfg["block_size"],
                           is_causal=lay["is_causal"], layer_type=lay["layer_type"],
                           sliding_window=lay["window"])
            geom = bsm.Geometry(cfg["B"], cfg["H"], cfg["KVH"], d.Sq, d.Sk, cfg["D"])
            out[f"block_mask_pred/{name}/{lay['name']}_us"] = \
                1e3 * _time_ms(lambda: bsm.build_block_mask(geom, pred=d))
    # long-context attention
    cfg = synth.CONFIGS["long_dflash_bf16"]
    lay = cfg["layers"][0]
    d = bsm.DFlash(cfg["ctx_len"], cfg["num_blocks"], cfg["block_size"], is_causal=lay["is_causal"],
                   layer_type=lay["layer_type"], sliding_window=lay["window"])
    q, k, v = [t.cuda() for t in synth.qkv(cfg["B"], d.Sq, d.Sk, cfg["H"], cfg["KVH"], cfg["D"],
                                           "bf16", seed=0)]
    geom = bsm.geometry_of(q, k)
    bm = bsm.build_block_mask(geom, pred=d)
    fl = counted_flops(bm, geom)
    o = torch.empty_like(q)
    ms = _time_ms(lambda: bsm.masked_attn_fwd(q, k, v, pred=d, block_mask=bm, out=o), reps=3)
    out["attn/long_dflash_bf16_ms"] = ms
    out["attn/long_dflash_bf16_TFLOP/s"] = fl / (ms * 1e-3) / 1e12
    del q, k, v, o
    out.update(measure_dynamic())
    out.update(measure_decode())
    out.update(measure_dflash_infer())
    out.update(measure_varlen())
    return out


VARLEN_LAYOUT = [(4096, 256), (2048, 128), (1024, 64), (3008, 47)]  # (context, blocks)


def measure_varlen():
    """Four DFlash sequences of different lengths packed together (H=32, KVH=8,
    D=128, blocks of 16), both layer types of the training shape: per-sequence
    block mask and packed attention forward and backward, TFLOP/s counted on
    each sequence's kept tiles."""
    out = {}
    cfg = synth.CONFIGS["dflash_train_bf16"]
    H, KVH, D, bs = cfg["H"], cfg["KVH"], cfg["D"], cfg["block_size"]
    sq = [nb * bs for _, nb in VARLEN_LAYOUT]
    sk = [c + nb * bs for c, nb in VARLEN_LAYOUT]
    cu_q = torch.tensor([0] + list(np.cumsum(sq)), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(np.cumsum(sk)), dtype=torch.int32)
    q, k, v = [t[0].cuda() for t in synth.qkv(1, int(cu_q[-1]), int(cu_k[-1]), H, KVH, D, "bf16",
                                               seed=0, scale=cfg["qkv_scale"])]
    vl = bsm.Varlen(cu_q.cuda(), cu_k.cuda(), H, KVH, D)
    for lay in cfg["layers"]:
        pred = bsm.varlen_dflash(bs, is_causal=lay["is_causal"], layer_type=lay["layer_type"],
                                 sliding_window=lay["window"])
        bm = bsm.build_block_mask_varlen(vl, pred)
        kvn, kvi, fn, fi = [t.cpu().numpy() for t in bm]
        fl = 0
        for b in range(len(sq)):
            for qt in range((sq[b] + 127) // 128):
                rows = min(128, sq[b] - 128 * qt)
                for kt in list(kvi[b, 0, qt, :kvn[b, 0, qt]]) + list(fi[b, 0, qt, :fn[b, 0, qt]]):
                    fl += 4 * D * H * rows * min(128, sk[b] - 128 * int(kt))
        o = torch.empty_like(q)
        ms = _time_ms(lambda: bsm.masked_attn_varlen_fwd(q, k, v, vl, pred=pred, block_mask=bm,
                                                         out=o), reps=5)
        out[f"attn_varlen/dflash_4seq_bf16/{lay['name']}_ms"] = ms
        out[f"attn_varlen/dflash_4seq_bf16/{lay['name']}_TFLOP/s"] = fl / (ms * 1e-3) / 1e12
        # backward, one sequence after another (2.5x the forward's counted flops)
        o, lse = bsm.masked_attn_varlen_fwd(q, k, v, vl, pred=pred, block_mask=bm,
                                            return_lse=True)
        do = synth.normal_tensor(tuple(q.shape), 1, synth.TID_DOUT, "bf16").cuda()
        ms = _time_ms(lambda: bsm.masked_attn_varlen_bwd(q, k, v, o, do, lse, vl, pred=pred,
                                                         block_mask=bm), reps=5)
        out[f"attn_varlen_bwd/dflash_4seq_bf16/{lay['name']}_ms"] = ms
        out[f"attn_varlen_bwd/dflash_4seq_bf16/{lay['name']}_TFLOP/s"] = \
            2.5 * fl / (ms * 1e-3) / 1e12
    return out


def measure_dflash_infer():
    """DFlash inference: one draft block of 16 after a 32K-token cache, B=8
    requests, H=32, KVH=8, D=128, full and sliding (W=4096) layers. HBM-bound;
    GB/s counts the K/V rows of the visited key tiles once per (b, KV head)
    plus Q and O."""
    out = {}
    cfg = synth.CONFIGS["dflash_infer_bf16"]
    B, H, KVH, D = (cfg[x] for x in ("B", "H", "KVH", "D"))
    for lay in cfg["layers"]:
        d = bsm.DFlash.inference(cfg["ctx_len"], cfg["block_size"], is_causal=lay["is_causal"],
                                 layer_type=lay["layer_type"], sliding_window=lay["window"])
        q, k, v = [t.cuda() for t in synth.qkv(B, d.Sq, d.Sk, H, KVH, D, "bf16", seed=0,
                                               scale=cfg["qkv_scale"])]
        geom = bsm.geometry_of(q, k)
        bm = bsm.build_block_mask(geom, pred=d)
        tiles = int(bm.kv_num_blocks.sum() + bm.full_kv_num_blocks.sum())
        o = torch.empty_like(q)
        ms = _time_ms(lambda: bsm.masked_attn_fwd(q, k, v, pred=d, block_mask=bm, out=o),
                      reps=10)
        rows = min(tiles * 128, d.Sk)
        nbytes = B * KVH * rows * 2 * D * 2 + 2 * q.numel() * 2
        out[f"attn/dflash_infer_bf16/{lay['name']}_us"] = ms * 1e3
        out[f"attn/dflash_infer_bf16/{lay['name']}_GB/s"] = nbytes / (ms * 1e-3) / 1e9
        del q, k, v, o
    return out


def measure_dynamic():
    """The dynamic-mask workload (B=2, H=16, KVH=4, Sq=Sk=8000, bias (2,4,1,8064),
    2D right padding, top-2048): top-k, dense builder, the fused top-k + block
    mask, and the attention."""
    out = {}
    cfg = synth.CONFIGS["dynamic_topk_bf16"]
    B, H, KVH, D, Sq, Sk = (cfg[x] for x in ("B", "H", "KVH", "D", "Sq", "Sk"))
    q, k, v = [t.cuda() for t in synth.qkv(B, Sq, Sk, H, KVH, D, "bf16", seed=0)]
    bias, pad2d = [t.cuda() for t in synth.topk_inputs(cfg, seed=0)]
    mask = bsm.create_mask(bias, pad2d, B, Sq, Sk, cfg["topk"])
    geom = bsm.geometry_of(q, k)
    bm = bsm.build_block_mask(geom, mask=mask)
    fl = counted_flops(bm, geom)
    o = torch.empty_like(q)
    out["topk/dynamic_topk_bf16_us"] = 1e3 * _time_ms(
        lambda: bsm.create_mask(bias, pad2d, B, Sq, Sk, cfg["topk"], ))
    out["block_mask_dense/dynamic_topk_bf16_us"] = 1e3 * _time_ms(
        lambda: bsm.build_block_mask(geom, mask=mask))
    pm4 = pad2d.as_strided((B, 1, 1, Sk), (pad2d.stride(0), 0, 0, pad2d.stride(1)))
    out["topk_fused_bm/dynamic_topk_bf16_us"] = 1e3 * _time_ms(
        lambda: bsm.dynamic_topk_fused(geom, bias, pm4, cfg["topk"]))
    ms = _time_ms(lambda: bsm.masked_attn_fwd(q, k, v, mask=mask, bias=bias, block_mask=bm,
                                              out=o), reps=5)
    out["attn/dynamic_topk_bf16_ms"] = ms
    out["attn/dynamic_topk_bf16_TFLOP/s"] = fl / (ms * 1e-3) / 1e12
    # the same call without a workspace: mask and bias read per key tile
    ms = _time_ms(lambda: bsm.masked_attn_fwd(q, k, v, mask=mask, bias=bias, block_mask=bm,
                                              out=o, split=False), reps=5)
    out["attn_unstaged/dynamic_topk_bf16_ms"] = ms
    out["attn_unstaged/dynamic_topk_bf16_TFLOP/s"] = fl / (ms * 1e-3) / 1e12
    del q, k, v, o
    return out


def measure_decode():
    """Decode with the head-group swap (B=64, H=32, KVH=8, Sk=16384, per-head
    bias, top-1024): top-k, then either the dense block-mask builder and the
    tile-visiting kernel, or the key-list builder and the key-gather kernel.
    GB/s counts the bytes each path must move: all K/V rows, or the listed ones."""
    out = {}
    cfg = synth.CONFIGS["decode_swap_bf16"]
    B, H, KVH, D, Sk = (cfg[x] for x in ("B", "H", "KVH", "D", "Sk"))
    q = _device_normal((B, 1, H, D), 111)
    k = _device_normal((B, Sk, KVH, D), 112)
    v = _device_normal((B, Sk, KVH, D), 113)
    bias, _ = synth.topk_inputs(cfg, seed=0)
    bias = bias.cuda()
    mask = torch.empty(bias.shape, dtype=torch.bool, device="cuda")
    tk = 1e3 * _time_ms(lambda: bsm.dynamic_topk_mask(bias, None, Sk, cfg["topk"], out=mask))
    out["topk/decode_swap_bf16_us"] = tk
    out["topk/decode_swap_bf16_GB/s"] = (bias.numel() * 2 + mask.numel()) / (tk * 1e-6) / 1e9
    geom = bsm.geometry_of(q, k)
    bm = bsm.build_block_mask(geom, mask=mask)
    bd = 1e3 * _time_ms(lambda: bsm.build_block_mask(geom, mask=mask))
    out["block_mask_dense/decode_swap_bf16_us"] = bd
    o = torch.empty_like(q)
    ms = _time_ms(lambda: bsm.masked_attn_fwd(q, k, v, mask=mask, bias=bias, block_mask=bm,
                                              out=o), reps=5)
    row_bytes = 2 * D * 2  # one K row and one V row, bf16
    kv_bytes = row_bytes * B * KVH * Sk + bias.numel() * 2 + mask.numel() + 2 * q.numel() * 2
    out["attn/decode_swap_bf16_ms"] = ms
    out["attn/decode_swap_bf16_GB/s"] = kv_bytes / (ms * 1e-3) / 1e9
    # key gather
    keys = bsm.build_key_list(geom, mask)
    kb = 1e3 * _time_ms(lambda: bsm.build_key_list(geom, mask))
    listed = int(keys.num_keys.sum())
    out["key_list/decode_swap_bf16_us"] = kb
    out["key_list/decode_swap_bf16_listed_frac"] = listed / (B * KVH * Sk)
    out["key_list/decode_swap_bf16_GB/s"] = (mask.numel() + listed * 8) / (kb * 1e-6) / 1e9
    # top-k fused with the key list (and the block mask), one pass over the bias
    out["topk_fused_keys/decode_swap_bf16_us"] = 1e3 * _time_ms(
        lambda: bsm.dynamic_topk_fused(geom, bias, None, cfg["topk"], want_mask=False,
                                       want_block_mask=False, want_keys=True))
    out["topk_fused_all/decode_swap_bf16_us"] = 1e3 * _time_ms(
        lambda: bsm.dynamic_topk_fused(geom, bias, None, cfg["topk"], want_keys=True))
    mg = _time_ms(lambda: bsm.masked_attn_fwd(q, k, v, mask=mask, bias=bias, keys=keys, out=o),
                  reps=5)
    g_bytes = row_bytes * listed + listed * 8 + bias.numel() * 2 + 2 * q.numel() * 2
    out["attn_gather/decode_swap_bf16_ms"] = mg
    out["attn_gather/decode_swap_bf16_GB/s"] = g_bytes / (mg * 1e-3) / 1e9
    return out


# ---------------------------------------------------------------------------
# the other workloads at full size, in the default line


def _device_normal(shape, seed, scale=1.0):
    """bf16 N(0, scale^2) draws made on the device (torch's generator seeded
    `seed`): the same distribution as the host generator, for inputs too large
    to draw on the host within the run."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    y = x.to(torch.bfloat16)
    del x
    return y


def measure_long_context(reps=3):
    """Long-context DFlash (B=1, H=32, KVH=8, D=128, 32768 queries, 65536 keys,
    causal in-block, window 4096): block mask from the predicate, attention on
    the kept tiles, and the device memory the call needs beyond its tensors."""
    cfg = synth.CONFIGS["long_dflash_bf16"]
    lay = cfg["layers"][0]
    d = bsm.DFlash(cfg["ctx_len"], cfg["num_blocks"], cfg["block_size"], is_causal=lay["is_causal"],
                   layer_type=lay["layer_type"], sliding_window=lay["window"])
    B, H, KVH, D = cfg["B"], cfg["H"], cfg["KVH"], cfg["D"]
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    q = _device_normal((B, d.Sq, H, D), 101)
    k = _device_normal((B, d.Sk, KVH, D), 102)
    v = _device_normal((B, d.Sk, KVH, D), 103)
    o = torch.empty_like(q)
    torch.cuda.synchronize()
    tensors = sum(t.numel() * t.element_size() for t in (q, k, v, o))
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    geom = bsm.geometry_of(q, k)
    bm = bsm.build_block_mask(geom, pred=d)
    bm_bytes = sum(t.numel() * t.element_size() for t in bm)
    bm_us = 1e3 * _time_ms(lambda: bsm.build_block_mask(geom, pred=d))
    fl = counted_flops(bm, geom)
    ms = _time_ms(lambda: bsm.masked_attn_fwd(q, k, v, pred=d, block_mask=bm, out=o), reps=reps)
    torch.cuda.synchronize()
    extra = torch.cuda.max_memory_allocated() - base
    del q, k, v, o
    tf = fl / (ms * 1e-3) / 1e12
    return {"attn_ms": ms, "TFLOP/s": tf, "frac": tf / PEAK_BF16_TFLOPS, "flops": int(fl),
            "block_mask_us": bm_us, "block_mask_bytes": int(bm_bytes),
            "peak_device_bytes": int(tensors + extra), "tensor_bytes": int(tensors),
            "peak_bytes_beyond_tensors": int(extra),
            "dense_mask_bytes_per_head_copy": int(B * H * d.Sq * d.Sk)}


def measure_dynamic_topk(reps=5):
    """Dynamic-mask workload (B=2, H=16, KVH=4, Sq=Sk=8000, bias (2,4,1,8064),
    2D right padding, top-2048): top-k, block mask, attention."""
    cfg = synth.CONFIGS["dynamic_topk_bf16"]
    B, H, KVH, D, Sq, Sk = (cfg[x] for x in ("B", "H", "KVH", "D", "Sq", "Sk"))
    q, k, v = [t.cuda() for t in synth.qkv(B, Sq, Sk, H, KVH, D, "bf16", seed=0)]
    bias, pad2d = [t.cuda() for t in synth.topk_inputs(cfg, seed=0)]
    mask = bsm.create_mask(bias, pad2d, B, Sq, Sk, cfg["topk"])
    geom = bsm.geometry_of(q, k)
    bm = bsm.build_block_mask(geom, mask=mask)
    fl = counted_flops(bm, geom)
    o = torch.empty_like(q)
    topk_us = 1e3 * _time_ms(lambda: bsm.create_mask(bias, pad2d, B, Sq, Sk, cfg["topk"]))
    bm_us = 1e3 * _time_ms(lambda: bsm.build_block_mask(geom, mask=mask))
    ms = _time_ms(lambda: bsm.masked_attn_fwd(q, k, v, mask=mask, bias=bias, block_mask=bm,
                                              out=o), reps=reps)
    del q, k, v, o
    tf = fl / (ms * 1e-3) / 1e12
    return {"attn_ms": ms, "TFLOP/s": tf, "frac": tf / PEAK_BF16_TFLOPS, "flops": int(fl),
            "topk_us": topk_us, "block_mask_us": bm_us}


def measure_decode_swap(reps=5):
    """Decode with the head-group swap (B=64, H=32, KVH=8, Sk=16384, per-head
    bias, top-1024): top-k, then the tile path (block mask + tile-visiting
    kernel, every K/V row read) and the gather path (kept-key list + key-gather
    kernel, listed rows read). GB/s counts the bytes each path must move."""
    cfg = synth.CONFIGS["decode_swap_bf16"]
    B, H, KVH, D, Sk = (cfg[x] for x in ("B", "H", "KVH", "D", "Sk"))
    q = _device_normal((B, 1, H, D), 111)
    k = _device_normal((B, Sk, KVH, D), 112)
    v = _device_normal((B, Sk, KVH, D), 113)
    bias = synth.topk_inputs(cfg, seed=0)[0].cuda()
    mask = torch.empty(bias.shape, dtype=torch.bool, device="cuda")
    topk_us = 1e3 * _time_ms(lambda: bsm.dynamic_topk_mask(bias, None, Sk, cfg["topk"], out=mask))
    geom = bsm.geometry_of(q, k)
    bm = bsm.build_block_mask(geom, mask=mask)
    bm_us = 1e3 * _time_ms(lambda: bsm.build_block_mask(geom, mask=mask))
    o = torch.empty_like(q)
    row_bytes = 2 * D * 2  # one K row and one V row, bf16
    small = bias.numel() * 2 + 2 * q.numel() * 2
    ms = _time_ms(lambda: bsm.masked_attn_fwd(q, k, v, mask=mask, bias=bias, block_mask=bm,
                                              out=o), reps=reps)
    t_bytes = row_bytes * B * KVH * Sk + mask.numel() + small
    keys = bsm.build_key_list(geom, mask)
    kl_us = 1e3 * _time_ms(lambda: bsm.build_key_list(geom, mask))
    listed = int(keys.num_keys.sum())
    mg = _time_ms(lambda: bsm.masked_attn_fwd(q, k, v, mask=mask, bias=bias, keys=keys, out=o),
                  reps=reps)
    g_bytes = row_bytes * listed + listed * 8 + small
    del q, k, v, o
    return {"topk_us": topk_us,
            "tiles": {"block_mask_us": bm_us, "attn_ms": ms, "bytes": int(t_bytes),
                      "GB/s": t_bytes / (ms * 1e-3) / 1e9,
                      "frac": t_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
            "gather": {"key_list_us": kl_us, "attn_ms": mg, "bytes": int(g_bytes),
                       "listed_frac": listed / (B * KVH * Sk),
                       "GB/s": g_bytes / (mg * 1e-3) / 1e9,
                       "frac": g_bytes / (mg * 1e-3) / 1e9 / PEAK_HBM_GBS}}


def measure_tiny(reps=20):
    """Tiny DFlash, fp32 (B=1, H=2, D=64, 64 queries, 320 keys): launch-bound."""
    cfg = synth.CONFIGS["tiny_dflash_fp32"]
    d = bsm.DFlash(cfg["ctx_len"], cfg["num_blocks"], cfg["block_size"])
    q, k, v = [t.cuda() for t in synth.qkv(1, d.Sq, d.Sk, cfg["H"], cfg["KVH"], cfg["D"], "f32",
                                           seed=0)]
    geom = bsm.geometry_of(q, k)
    bm = bsm.build_block_mask(geom, pred=d)
    o = torch.empty_like(q)
    us = 1e3 * _time_ms(lambda: bsm.masked_attn_fwd(q, k, v, pred=d, block_mask=bm, out=o),
                        reps=reps)
    return {"attn_us": us, "block_mask_us": 1e3 * _time_ms(
        lambda: bsm.build_block_mask(geom, pred=d), reps=reps)}


def measure_configs():
    return {"tiny_dflash_fp32": measure_tiny(),
            "long_dflash_bf16": measure_long_context(),
            "dynamic_topk_bf16": measure_dynamic_topk(),
            "decode_swap_bf16": measure_decode_swap(),
            # the backward (training shape; dynamic-mask workload with dbias) and
            # packed sequences (forward and backward)
            "backward": measure_backward(),
            "varlen_dflash_4seq_bf16": measure_varlen()}


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a pool of host processes, one BLAS thread
# each. Workers draw their inputs with the same generator as the GPU run (or,
# for the two workloads whose inputs the GPU run draws on the device, with the
# host generator: the same shapes and distribution) and cache what they reuse.

_WCACHE = {}
_THREAD_ENV = {"OMP_NUM_THREADS": "1", "OPENBLAS_NUM_THREADS": "1", "MKL_NUM_THREADS": "1"}


def host_workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def start_host_pool():
    """The pool of oracle workers. Call before this process touches the GPU:
    the workers come from a fork server started here, never from a process
    that has used the GPU."""
    import multiprocessing as mp
    saved = {k: os.environ.get(k) for k in _THREAD_ENV}
    os.environ.update(_THREAD_ENV)
    try:
        ctx = mp.get_context("forkserver")
        pool = ctx.Pool(host_workers(), initializer=_worker_init)
        manager = ctx.Manager()
    finally:
        for k, val in saved.items():
            if val is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = val
    return pool, manager


def _worker_init():
    from threadpoolctl import threadpool_limits
    _WCACHE["limits"] = threadpool_limits(1)


def _f32(t):
    return t.to(torch.float32).numpy()


def _dflash_geom(name, li):
    import oracle
    cfg = synth.CONFIGS[name]
    lay = cfg["layers"][li]
    return oracle.DFlashGeom(cfg["ctx_len"], cfg["num_blocks"], cfg["block_size"], 0, 0,
                             lay["is_causal"], lay["layer_type"], lay["window"])


def _load(name):
    """Inputs a worker keeps for a workload (whole tensors, or K/V only)."""
    if name in _WCACHE:
        return _WCACHE[name]
    cfg = synth.CONFIGS[name]
    if cfg["kind"] == "dflash":
        g = _dflash_geom(name, 0)
        Sq, Sk = g.Sq, g.Sk
    else:
        Sq, Sk = cfg["Sq"], cfg["Sk"]
    B, H, KVH, D, dt, sc = (cfg[x] for x in ("B", "H", "KVH", "D", "dtype", "qkv_scale"))
    if name == "long_dflash_bf16":   # K/V only; each unit draws its own query rows
        kv = [_f32(synth.normal_tensor((B, Sk, KVH, D), 0, t, dt, sc))
              for t in (synth.TID_K, synth.TID_V)]
        val = (None, kv[0], kv[1])
    else:
        val = tuple(_f32(t) for t in synth.qkv(B, Sq, Sk, H, KVH, D, dt, seed=0, scale=sc))
    if cfg["kind"] == "topk" and name != "decode_swap_bf16":
        bias_t, pad2d = synth.topk_inputs(cfg, seed=0)
        val = val + (_f32(bias_t).astype(np.float64), None if pad2d is None else pad2d.numpy())
    _WCACHE[name] = val
    return val


def _preload(job):
    """Draw a workload's inputs in this worker, then wait at the barrier so that
    every worker takes exactly one preload job."""
    name, barrier = job
    if name != "decode_swap_bf16":
        _load(name)
    barrier.wait()
    return os.getpid()


def _tile_flops(band, Sk, D):
    from oracle.blockmask import classify_tile_band
    part, full = classify_tile_band(band, Sk)
    rows = band.shape[0]
    return 4 * D * rows * sum(min(128, Sk - 128 * int(t)) for t in list(part) + list(full))


def oracle_unit(job):
    """One unit of oracle work; returns (oracle seconds, counted flops). The
    seconds cover the oracle's steps only (dense mask rows or top-k, tile
    classification, attention), not the drawing of inputs."""
    import oracle
    name, li, b, h, qt = job
    cfg = synth.CONFIGS[name]
    D, H = cfg["D"], cfg["H"]
    if cfg["kind"] == "dflash":
        q, k, v = _load(name)
        g = _dflash_geom(name, li)
        r0, r1 = 128 * qt, min(128 * qt + 128, g.Sq)
        sliced = q is None   # this unit's query rows only (batch entry b of a B = 1 workload)
        if sliced:
            q = _f32(synth.normal_rows((cfg["B"], g.Sq, H, D), 0, synth.TID_Q, b, r0, r1,
                                       cfg["dtype"], cfg["qkv_scale"]))
        t0 = time.perf_counter()
        band = oracle.dflash_dense_mask(g, np.arange(r0, r1))
        fl = _tile_flops(band, g.Sk, D)
        if sliced:
            oracle.attention_rows(q, k, v, 0, h, np.arange(r1 - r0), mask=band[None, None])
        else:
            oracle.attention_rows(q, k, v, b, h, np.arange(r0, r1), mask=g)
        return time.perf_counter() - t0, fl
    if name == "dynamic_topk_bf16":
        q, k, v, bias, pad2d = _load(name)
        Sq, Sk, G = cfg["Sq"], cfg["Sk"], H // cfg["KVH"]
        r0, r1 = 128 * qt, min(128 * qt + 128, Sq)
        t0 = time.perf_counter()
        pre = oracle.normalize_premask(pad2d[b:b + 1], 1, Sk)
        m = oracle.topk_keep_mask(bias[b:b + 1, h // G:h // G + 1], pre, Sk, cfg["topk"], "bf16")
        fl = _tile_flops(np.broadcast_to(m[0, 0, 0], (r1 - r0, m.shape[-1])), Sk, D)
        oracle.attention_rows(q[b:b + 1], k[b:b + 1], v[b:b + 1], 0, h, np.arange(r0, r1),
                              mask=m, bias=bias[b:b + 1, h // G:h // G + 1])
        return time.perf_counter() - t0, fl
    # decode: one batch entry, all heads
    B, KVH, Sk = cfg["B"], cfg["KVH"], cfg["Sk"]
    K = synth.round_up_128(Sk)
    q = _f32(synth.normal_rows((B, 1, H, D), 0, synth.TID_Q, b, 0, 1, "bf16"))
    k = _f32(synth.normal_rows((B, Sk, KVH, D), 0, synth.TID_K, b, 0, Sk, "bf16"))
    v = _f32(synth.normal_rows((B, Sk, KVH, D), 0, synth.TID_V, b, 0, Sk, "bf16"))
    bias = _f32(synth.normal_rows((B, H, 1, K), 0, synth.TID_BIAS, b, 0, H, "bf16"))
    bias = bias.astype(np.float64)
    t0 = time.perf_counter()
    m = oracle.topk_keep_mask(bias, None, Sk, cfg["topk"], "bf16")
    for hh in range(H):
        oracle.attention_rows(q, k, v, 0, hh, [0], mask=m, bias=bias)
    return time.perf_counter() - t0, 4 * D * H * Sk


def _units(name):
    """Every unit of a workload: (name, layer, b, h, query tile)."""
    cfg = synth.CONFIGS[name]
    if cfg["kind"] == "dflash":
        nq = -(-_dflash_geom(name, 0).Sq // 128)
        return [(name, li, b, h, qt) for li in range(len(cfg["layers"])) for b in range(cfg["B"])
                for h in range(cfg["H"]) for qt in range(nq)]
    if name == "dynamic_topk_bf16":
        nq = -(-cfg["Sq"] // 128)
        return [(name, 0, b, h, qt) for b in range(cfg["B"]) for h in range(cfg["H"])
                for qt in range(nq)]
    return [(name, 0, b, 0, 0) for b in range(cfg["B"])]


UNIT_DESC = {"tiny_dflash_fp32": "(b, h, 128-row query tile)",
             "dflash_train_bf16": "(layer, b, h, 128-row query tile)",
             "long_dflash_bf16": "(b, h, 128-row query tile)",
             "dynamic_topk_bf16": "(b, h, 128-row query tile) incl. its top-k row",
             "decode_swap_bf16": "(b): top-k of 32 head rows + 32 one-row attentions"}


def cpu_baseline(pool, manager, budgets=None):
    """The fp64 oracle, as it stands, on a bounded random sample of every
    workload's units, run by the pool in waves of one unit per worker. Per
    workload: units done / total, wall seconds of the waves (inputs drawn
    beforehand, except the decode units, which draw their batch entry's K/V),
    the oracle's own seconds summed over units, and the full workload's oracle
    time at this core count extrapolated from the sample. `value` is the
    training-shape step's counted TFLOP/s over that workload's wall time."""
    W = host_workers()
    budgets = budgets or {"tiny_dflash_fp32": 0.0, "dflash_train_bf16": 8.0,
                          "long_dflash_bf16": 5.0, "dynamic_topk_bf16": 5.0,
                          "decode_swap_bf16": 5.0}
    rng = np.random.default_rng(0)
    out = {}
    for name, budget in budgets.items():
        units = _units(name)
        order = rng.permutation(len(units))
        barrier = manager.Barrier(W)
        pool.map(_preload, [(name, barrier)] * W, chunksize=1)
        done = []
        t0 = time.perf_counter()
        i = 0
        while i < len(units) and (not done or time.perf_counter() - t0 < budget):
            done += pool.map(oracle_unit, [units[j] for j in order[i:i + W]], chunksize=1)
            i += W
        wall = time.perf_counter() - t0
        osec = sum(s for s, _ in done)
        fl = sum(f for _, f in done)
        out[name] = {"unit": UNIT_DESC[name], "units_done": len(done), "units_total": len(units),
                     "wall_s": wall, "oracle_s": osec,
                     "est_full_workload_s": len(units) * wall / len(done),
                     "counted_TFLOP/s": fl / wall / 1e12}
    main = out[WORKLOAD]
    return {"value": main["counted_TFLOP/s"], "unit": "TFLOP/s", "cores": W, "kind": "oracle",
            "sample": f"{main['units_done']} random {UNIT_DESC[WORKLOAD]} units of the "
                      f"{WORKLOAD} step on {W} one-thread worker processes, float64, "
                      f"{main['wall_s']:.1f} s wall; per-workload samples under 'configs'",
            "configs": out}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mask-build", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads' full-size lines (long context, dynamic "
                         "top-k, decode, tiny)")
    ap.add_argument("--components", action="store_true",
                    help="also time the other workloads' kernels (top-k, builders, attention)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--backward-only", action="store_true",
                    help="only time the DFlash training-shape backward and print it")
    ap.add_argument("--only", choices=["decode", "dynamic", "infer", "varlen", "one_head",
                                       "components"],
                    help="only time one group of the other workloads' kernels and print it")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the hot path "
              "is measured on a single MI355X; sharding is described, not run.", file=sys.stderr)
        sys.exit(2)
    pool = manager = None
    if not (args.no_cpu_baseline or args.copy_probe or args.backward_only or args.only):
        pool, manager = start_host_pool()   # before this process touches the GPU
    torch.cuda.init()
    if args.copy_probe:
        copy_probe()
        return
    if args.backward_only:
        print(json.dumps(measure_backward()), flush=True)
        return
    if args.only:
        fn = {"decode": measure_decode, "dynamic": measure_dynamic,
              "infer": measure_dflash_infer, "varlen": measure_varlen,
              "one_head": measure_one_head, "components": measure_components}[args.only]
        print(json.dumps(fn()), flush=True)
        return
    step = Step()
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step.run(record=True)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms_step = el * 1e3 / args.steps
    flops_step = sum(step.flops)
    value = flops_step / (ms_step * 1e-3) / 1e12

    attn_ms = [e0.elapsed_time(e1) for _, e0, e1 in step.attn_events]
    attn_flops = [step.flops[i] for i, _, _ in step.attn_events]
    achieved = sum(attn_flops) / (sum(attn_ms) * 1e-3) / 1e12
    per_layer = {}
    for li, (name, _) in enumerate(step.layers):
        ms = [e0.elapsed_time(e1) for i, e0, e1 in step.attn_events if i == li]
        per_layer[name] = {"attn_ms": float(np.mean(ms)), "flops": int(step.flops[li]),
                           "TFLOP/s": step.flops[li] / (np.mean(ms) * 1e-3) / 1e12}
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "B": 2, "H": 32, "KVH": 8, "D": 128,
                   "ctx_len": 4096, "draft_blocks": 256, "block_size": 16,
                   "Sq": 4096, "Sk": 8192, "layers": [n for n, _ in step.layers],
                   "flops_per_step": int(flops_step)},
        "roofline": {"bound": "mfma", "kernel": "k_attn_bf16_v2<128>", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": attn_traffic_bytes(),
                     "avg_launch_ms": float(np.mean(attn_ms)),
                     "flops_per_launch": float(np.mean(attn_flops))},
        "per_layer": per_layer,
        "device": device_info(),
    }
    if not args.no_mask_build:
        line["mask_build"] = measure_mask_build()
    if not args.no_configs:
        del step
        line["configs"] = measure_configs()
    if args.components:
        line["components"] = measure_components()
    if pool is not None:
        line["cpu_baseline"] = cpu_baseline(pool, manager)
        pool.close()
        pool.join()
        manager.shutdown()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
