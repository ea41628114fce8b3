"""C-ABI checks that need no GPU: the library loads, exports every function that
include/bsm.h declares, and its host-only logic (is_causal resolution, block mask
shapes, argument validation) answers without touching a device. Validation
cases use fake, never-dereferenced device addresses and must fail before any
launch."""

import ctypes
import json
import os
import re
import subprocess

import pytest

from conftest import GOLDEN, ROOT

from block_sparse_masked_mask_amd import bsm


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bsm.LIB_PATH):
        from block_sparse_masked_mask_amd.build import build
        build()
    return bsm.lib()


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "bsm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_function(L):
    decl = _declared_functions()
    assert set(decl) == set(bsm.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", bsm.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in decl:
        assert name in syms, name
        assert hasattr(L, name)


def test_struct_sizes_match_header():
    # C layout: pointer 8, two int32, 2 x int64[4]
    assert ctypes.sizeof(bsm.Tensor4) == 80
    assert ctypes.sizeof(bsm.DFlashC) == 56
    assert ctypes.sizeof(bsm.BlockMaskC) == 64
    assert ctypes.sizeof(bsm.KeyListC) == 3 * 8 + 4 * 8
    assert ctypes.sizeof(bsm.AttnArgs) == 3 * 80 + 8 + 32 + 8 + 8 + 7 * 8
    assert ctypes.sizeof(bsm.AttnBwdArgs) == 8 * 80 + 8 + 8 + 5 * 8 + 8 + 8


def test_struct_layouts_match_c_compiler(tmp_path):
    """sizeof and field offsets as the C compiler lays out include/bsm.h."""
    structs = {"bsm_tensor4": bsm.Tensor4, "bsm_dflash": bsm.DFlashC,
               "bsm_block_mask": bsm.BlockMaskC, "bsm_geom": bsm.Geom,
               "bsm_key_list": bsm.KeyListC, "bsm_varlen": bsm.VarlenC,
               "bsm_attn_args": bsm.AttnArgs, "bsm_attn_bwd_args": bsm.AttnBwdArgs}
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "bsm.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    r = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("no C compiler for the header: " + r.stderr[:200])
    got = dict(ln.rsplit(" ", 1) for ln in
               subprocess.run([str(exe)], capture_output=True, text=True, check=True)
               .stdout.splitlines())
    for cname, py in structs.items():
        assert int(got[f"{cname} sizeof"]) == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert int(got[f"{cname} {f}"]) == getattr(py, f).offset, (cname, f)


def test_resolve_is_causal_table(L):
    tab = json.load(open(os.path.join(GOLDEN, "dflash_is_causal.json")))["table"]
    for e in tab:
        ic = -1 if e["is_causal"] is None else int(e["is_causal"])
        lt = 0 if e["layer_type"] == "full" else 1
        assert L.resolve_dflash_is_causal(ic, lt) == int(e["causal"])
    assert L.resolve_dflash_is_causal(2, 0) == bsm.BSM_E_ARG
    assert L.resolve_dflash_is_causal(-1, 2) == bsm.BSM_E_ARG
    assert b"layer_type" in L.bsm_last_error()


def _t4(shape, dtype=bsm.BSM_BOOL, strides=None, data=1 << 20):
    t = bsm.Tensor4()
    t.data = data
    t.dtype = dtype
    t.reserved = 0
    if strides is None:
        strides, acc = [], 1
        for s in reversed(shape):
            strides.insert(0, acc)
            acc *= s
    for i in range(4):
        t.size[i] = shape[i]
        t.stride[i] = strides[i]
    return t


def _shape(L, geom, pred=None, mask=None):
    out = (ctypes.c_int64 * 4)()
    g = bsm.Geom(*geom)
    st = L.block_mask_shape(ctypes.byref(g), ctypes.byref(pred) if pred else None,
                            ctypes.byref(mask) if mask else None, out)
    return st, tuple(out)


def test_block_mask_shapes(L):
    # DFlash: one (1, 1, nQ, nK) block mask for every batch entry and head
    tiny = bsm.DFlash(256, 4, 16).c()
    assert _shape(L, (1, 2, 2, 64, 320, 64), pred=tiny) == (0, (1, 1, 1, 3))
    train = bsm.DFlash(4096, 256, 16).c()
    assert _shape(L, (2, 32, 8, 4096, 8192, 128), pred=train) == (0, (1, 1, 32, 64))
    long = bsm.DFlash(32768, 2048, 16, is_causal=True, layer_type="sliding",
                      sliding_window=4096).c()
    assert _shape(L, (1, 32, 8, 32768, 65536, 128), pred=long) == (0, (1, 1, 256, 512))
    # dense top-k mask (B, KVH, 1, 8064) broadcast over queries
    m = _t4((2, 4, 1, 8064))
    assert _shape(L, (2, 16, 4, 8000, 8000, 128), mask=m) == (0, (2, 4, 1, 63))
    # decode: (B, H, 1, K) under the head-group swap -> (B, KVH, 1 tile of G rows, nK)
    m = _t4((64, 32, 1, 16384))
    assert _shape(L, (64, 32, 8, 1, 16384, 128), mask=m) == (0, (64, 8, 1, 128))
    # no swap when H == KVH
    m = _t4((3, 8, 1, 256))
    assert _shape(L, (3, 8, 8, 1, 200, 64), mask=m) == (0, (3, 8, 1, 2))


@pytest.mark.parametrize("case,code", [
    (dict(mask_shape=(2, 4, 1, 8000)), bsm.BSM_E_SHAPE),      # K not rounded to 128
    (dict(mask_shape=(3, 4, 1, 8064)), bsm.BSM_E_SHAPE),      # batch not B or 1
    (dict(mask_shape=(2, 5, 1, 8064)), bsm.BSM_E_SHAPE),      # head not H, KVH or 1
    (dict(mask_shape=(2, 4, 7, 8064)), bsm.BSM_E_SHAPE),      # query not Sq or 1
    (dict(mask_shape=(2, 4, 1, 8064), dtype=bsm.BSM_BF16), bsm.BSM_E_DTYPE),
    (dict(mask_shape=(2, 4, 1, 8064), strides=(0, 8064, 8064, 1)), bsm.BSM_E_STRIDE),  # expand
    (dict(mask_shape=(2, 4, 1, 8064), strides=(8064 * 4, 8064, 8064, 2)), bsm.BSM_E_STRIDE),
    (dict(mask_shape=(2, 4, 1, 8064), strides=(8064 * 4 + 3, 8064, 8064, 1)), bsm.BSM_E_STRIDE),
    (dict(mask_shape=(2, 4, 1, 8064), data=(1 << 20) + 8), bsm.BSM_E_STRIDE),  # misaligned
])
def test_mask_validation(L, case, code):
    m = _t4(case["mask_shape"], case.get("dtype", bsm.BSM_BOOL), case.get("strides"),
            case.get("data", 1 << 20))
    st, _ = _shape(L, (2, 16, 4, 8000, 8000, 128), mask=m)
    assert st == code, L.bsm_last_error()


def test_geometry_and_source_validation(L):
    d = bsm.DFlash(256, 4, 16).c()
    assert _shape(L, (1, 6, 4, 64, 320, 64), pred=d)[0] == bsm.BSM_E_SHAPE  # H % KVH
    assert _shape(L, (1, 2, 2, 63, 320, 64), pred=d)[0] == bsm.BSM_E_SHAPE  # Sq != NB*bs
    assert _shape(L, (1, 2, 2, 64, 300, 64), pred=d)[0] == bsm.BSM_E_SHAPE  # Sk != C + NB*bs
    assert _shape(L, (1, 2, 2, 64, 320, 64))[0] == bsm.BSM_E_ARG            # no source
    m = _t4((1, 1, 64, 384))
    assert _shape(L, (1, 2, 2, 64, 320, 64), pred=d, mask=m)[0] == bsm.BSM_E_ARG
    bad = bsm.DFlash(250, 4, 16).c()  # C % NB != 0 with derived ctx_per_block
    assert _shape(L, (1, 2, 2, 64, 314, 64), pred=bad)[0] == bsm.BSM_E_ARG
    nowin = bsm.DFlash(256, 4, 16, layer_type="sliding", sliding_window=0).c()
    assert _shape(L, (1, 2, 2, 64, 320, 64), pred=nowin)[0] == bsm.BSM_E_ARG


def _attn_args(geom, dtype=bsm.BSM_BF16, **kw):
    B, H, KVH, Sq, Sk, D = geom
    a = bsm.AttnArgs()
    a.q = _t4((B, Sq, H, D), dtype)
    a.k = _t4((B, Sk, KVH, D), dtype)
    a.v = _t4((B, Sk, KVH, D), dtype)
    a.o = 1 << 21
    for i, s in enumerate(_t4((B, Sq, H, D)).stride):
        a.o_stride[i] = s
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _attn(L, geom, a):
    g = bsm.Geom(*geom)
    return L.masked_attn_fwd(ctypes.byref(g), ctypes.byref(a), None)


def test_attention_validation(L):
    geom = (2, 16, 4, 64, 300, 128)
    a = _attn_args(geom)
    a.k = _t4((2, 300, 4, 128), bsm.BSM_F32)
    assert _attn(L, geom, a) == bsm.BSM_E_DTYPE
    a = _attn_args(geom)
    a.q = _t4((2, 64, 16, 128), bsm.BSM_BF16, strides=(64 * 16 * 128, 16 * 128, 128, 2))
    assert _attn(L, geom, a) == bsm.BSM_E_STRIDE
    geom96 = (2, 16, 4, 64, 300, 96)
    assert _attn(L, geom96, _attn_args(geom96)) == bsm.BSM_E_UNSUPPORTED
    a = _attn_args(geom)
    bias = _t4((2, 4, 1, 384), bsm.BSM_F32)
    a.bias = ctypes.pointer(bias)
    assert _attn(L, geom, a) == bsm.BSM_E_DTYPE       # bias dtype != q dtype
    a = _attn_args(geom)
    bm = bsm.BlockMaskC(1 << 22, 1 << 22, 1 << 22, 1 << 22, 1, 1, 1, 3)
    a.bm = ctypes.pointer(bm)
    assert _attn(L, geom, a) == bsm.BSM_E_ARG         # block mask without a source
    a = _attn_args(geom)
    m = _t4((2, 4, 1, 384))
    a.mask = ctypes.pointer(m)
    bm = bsm.BlockMaskC(1 << 22, 1 << 22, 1 << 22, 1 << 22, 2, 4, 1, 2)
    a.bm = ctypes.pointer(bm)
    assert _attn(L, geom, a) == bsm.BSM_E_SHAPE       # block mask for another geometry
    assert b"block mask" in L.bsm_last_error()


def _kl_shape(L, geom, mask):
    out = (ctypes.c_int64 * 4)()
    st = L.key_list_shape(ctypes.byref(bsm.Geom(*geom)), ctypes.byref(mask), out)
    return st, tuple(out)


def test_key_list_shapes_and_validation(L):
    # decode with the swap: (B, H, 1, K) -> lists per (b, KV head) over G = 4 rows
    dec = (64, 32, 8, 1, 16384, 128)
    assert _kl_shape(L, dec, _t4((64, 32, 1, 16384))) == (0, (64, 8, 4, 16384))
    # mask per KV head under the swap broadcasts over the G rows
    assert _kl_shape(L, dec, _t4((64, 8, 1, 16384))) == (0, (64, 8, 4, 16384))
    # a short prefill chunk without the swap: Sq rows per (b, h)
    assert _kl_shape(L, (2, 8, 2, 20, 300, 64), _t4((2, 2, 20, 384))) == (0, (2, 2, 20, 384))
    # more than 32 rows is outside what a row word holds
    st, _ = _kl_shape(L, (2, 8, 2, 40, 300, 64), _t4((2, 2, 40, 384)))
    assert st == bsm.BSM_E_UNSUPPORTED
    assert _kl_shape(L, dec, _t4((64, 32, 1, 16384), bsm.BSM_BF16))[0] == bsm.BSM_E_DTYPE
    g = bsm.Geom(*dec)
    m = _t4((64, 32, 1, 16384))
    kl = bsm.KeyListC(1 << 22, 1 << 23, 1 << 24, 64, 8, 4, 16384)
    wrong = bsm.KeyListC(1 << 22, 1 << 23, 1 << 24, 64, 8, 2, 16384)
    assert L.build_key_list(ctypes.byref(g), ctypes.byref(m), ctypes.byref(wrong), None) == \
        bsm.BSM_E_SHAPE
    odd = bsm.KeyListC(1 << 22, (1 << 23) + 4, 1 << 24, 64, 8, 4, 16384)
    assert L.build_key_list(ctypes.byref(g), ctypes.byref(m), ctypes.byref(odd), None) == \
        bsm.BSM_E_STRIDE
    null = bsm.KeyListC(None, 1 << 23, 1 << 24, 64, 8, 4, 16384)
    assert L.build_key_list(ctypes.byref(g), ctypes.byref(m), ctypes.byref(null), None) == \
        bsm.BSM_E_ARG
    # attention with a key list: needs the mask and no block mask, bf16 only
    a = _attn_args(dec)
    a.keys = ctypes.pointer(kl)
    assert _attn(L, dec, a) == bsm.BSM_E_ARG
    a.mask = ctypes.pointer(m)
    bm = bsm.BlockMaskC(1 << 22, 1 << 22, 1 << 22, 1 << 22, 64, 8, 1, 128)
    a.bm = ctypes.pointer(bm)
    assert _attn(L, dec, a) == bsm.BSM_E_ARG
    a = _attn_args(dec, dtype=bsm.BSM_F32)
    a.mask, a.keys = ctypes.pointer(m), ctypes.pointer(kl)
    assert _attn(L, dec, a) == bsm.BSM_E_UNSUPPORTED
    a = _attn_args(dec)
    a.mask, a.keys = ctypes.pointer(m), ctypes.pointer(wrong)
    assert _attn(L, dec, a) == bsm.BSM_E_SHAPE
    assert b"key list" in L.bsm_last_error()


def test_topk_validation(L):
    bias = _t4((2, 4, 1, 8064), bsm.BSM_BF16)
    st = L.dynamic_topk_mask(ctypes.byref(bias), None, 8000, -1, 1 << 21, None)
    assert st == bsm.BSM_E_ARG
    st = L.dynamic_topk_mask(ctypes.byref(bias), None, 8100, 10, 1 << 21, None)
    assert st == bsm.BSM_E_SHAPE
    pm = _t4((2, 2, 1, 8000))
    st = L.dynamic_topk_mask(ctypes.byref(bias), ctypes.byref(pm), 8000, 10, 1 << 21, None)
    assert st == bsm.BSM_E_SHAPE
    bad = _t4((2, 4, 1, 8064), bsm.BSM_BOOL)
    st = L.dynamic_topk_mask(ctypes.byref(bad), None, 8000, 10, 1 << 21, None)
    assert st == bsm.BSM_E_DTYPE


def _bwd_args(geom, dtype=bsm.BSM_BF16):
    B, H, KVH, Sq, Sk, D = geom
    a = bsm.AttnBwdArgs()
    for name in ("q", "o", "dout", "dq"):
        setattr(a, name, _t4((B, Sq, H, D), dtype))
    for name in ("k", "v", "dk", "dv"):
        setattr(a, name, _t4((B, Sk, KVH, D), dtype))
    a.lse = 1 << 21
    return a


def _bwd(L, geom, a, ws=None):
    g = bsm.Geom(*geom)
    need = ctypes.c_int64(0)
    assert L.attn_bwd_workspace_size(ctypes.byref(g), ctypes.byref(a), ctypes.byref(need)) == 0
    if ws is None:
        a.workspace, a.workspace_bytes = 1 << 24, need.value
    return L.masked_attn_bwd(ctypes.byref(g), ctypes.byref(a), None), need.value


def test_attention_bwd_validation(L):
    geom = (2, 16, 4, 64, 300, 128)
    a = _bwd_args(geom)
    a.dk = _t4((2, 300, 16, 128), bsm.BSM_BF16)        # dk with H heads instead of KVH
    assert _bwd(L, geom, a)[0] == bsm.BSM_E_SHAPE
    a = _bwd_args(geom)
    a.lse = None
    assert _bwd(L, geom, a)[0] == bsm.BSM_E_ARG
    geom96 = (2, 16, 4, 64, 300, 96)
    assert _bwd(L, geom96, _bwd_args(geom96))[0] == bsm.BSM_E_UNSUPPORTED
    a = _bwd_args(geom)
    db = _t4((2, 4, 1, 384), bsm.BSM_BF16)
    a.dbias = ctypes.pointer(db)                       # dbias without bias
    assert _bwd(L, geom, a)[0] == bsm.BSM_E_ARG
    a = _bwd_args(geom)
    bias = _t4((2, 4, 1, 384), bsm.BSM_BF16)
    dbias = _t4((2, 4, 1, 384), bsm.BSM_BF16)
    a.bias, a.dbias = ctypes.pointer(bias), ctypes.pointer(dbias)
    g = bsm.Geom(*geom)
    need = ctypes.c_int64(0)
    assert L.attn_bwd_workspace_size(ctypes.byref(g), ctypes.byref(a), ctypes.byref(need)) == 0
    # Delta (2*16*64 floats) + the bias accumulator (2*4*384 floats) + the bias
    # folded into one float row per (b, KV head) for the matrix-core kernels
    # (it broadcasts over queries), 256-byte parts
    assert need.value == 2 * 16 * 64 * 4 + 2 * 4 * 384 * 4 + 2 * 4 * 384 * 4
    f32 = _bwd_args(geom, bsm.BSM_F32)                   # f32: the generic kernels, no rows
    fb, fdb = _t4((2, 4, 1, 384), bsm.BSM_F32), _t4((2, 4, 1, 384), bsm.BSM_F32)
    f32.bias, f32.dbias = ctypes.pointer(fb), ctypes.pointer(fdb)
    n32 = ctypes.c_int64(0)
    assert L.attn_bwd_workspace_size(ctypes.byref(g), ctypes.byref(f32), ctypes.byref(n32)) == 0
    assert n32.value == 2 * 16 * 64 * 4 + 2 * 4 * 384 * 4
    a.workspace, a.workspace_bytes = 1 << 24, need.value - 4
    assert L.masked_attn_bwd(ctypes.byref(g), ctypes.byref(a), None) == bsm.BSM_E_ARG
    assert b"workspace" in L.bsm_last_error()
    a.workspace, a.workspace_bytes = (1 << 24) + 16, need.value
    assert L.masked_attn_bwd(ctypes.byref(g), ctypes.byref(a), None) == bsm.BSM_E_ARG
    wrong = _t4((2, 4, 1, 384), bsm.BSM_F32)           # dbias dtype != bias dtype
    a.dbias = ctypes.pointer(wrong)
    assert _bwd(L, geom, a)[0] == bsm.BSM_E_DTYPE


def _varlen(cu_q, cu_k, H=8, KVH=2, D=128, dev_q=1 << 22, dev_k=1 << 23):
    hq = (ctypes.c_int32 * len(cu_q))(*cu_q)
    hk = (ctypes.c_int32 * len(cu_k))(*cu_k)
    vl = bsm.VarlenC(len(cu_q) - 1, H, KVH, D, cu_q[-1], cu_k[-1], dev_q, dev_k,
                     ctypes.addressof(hq), ctypes.addressof(hk))
    return vl, (hq, hk)


def _vl_shape(L, vl, pred):
    out = (ctypes.c_int64 * 4)()
    return L.block_mask_varlen_shape(ctypes.byref(vl), ctypes.byref(pred), out), tuple(out)


def test_varlen_shapes_and_validation(L):
    pred = bsm.varlen_dflash(16).c()
    # three sequences: 2 blocks after 100 tokens, none, 10 blocks after 300
    vl, keep = _varlen([0, 32, 32, 192], [0, 132, 132, 592])
    assert _vl_shape(L, vl, pred) == (0, (3, 1, 2, 4))
    bad, keep2 = _varlen([0, 30, 62], [0, 130, 262])          # 30 queries, blocks of 16
    assert _vl_shape(L, bad, pred)[0] == bsm.BSM_E_SHAPE
    dec, keep3 = _varlen([0, 32, 16], [0, 132, 300])          # decreasing
    assert _vl_shape(L, dec, pred)[0] == bsm.BSM_E_ARG
    odd, keep4 = _varlen([0, 32], [0, 133])                   # 101 context tokens, 2 blocks
    assert _vl_shape(L, odd, pred)[0] == bsm.BSM_E_SHAPE
    fixed = bsm.varlen_dflash(16, ctx_per_block=50).c()       # a fixed S needs no divisibility
    assert _vl_shape(L, odd, fixed)[0] == 0
    whole = bsm.DFlash(100, 2, 16).c()                        # ctx_len / num_blocks given
    assert _vl_shape(L, vl, whole)[0] == bsm.BSM_E_ARG
    total, keep5 = _varlen([0, 32, 32, 192], [0, 132, 132, 592])
    total.total_q = 191
    assert _vl_shape(L, total, pred)[0] == bsm.BSM_E_SHAPE
    # attention: packed tensors are (1, total, heads, D); masks and biases are refused
    a = _attn_args((1, 8, 2, 192, 592, 128))
    m = _t4((1, 1, 192, 640))
    a.mask = ctypes.pointer(m)
    assert L.masked_attn_varlen_fwd(ctypes.byref(vl), ctypes.byref(a), None) == \
        bsm.BSM_E_UNSUPPORTED
    a = _attn_args((2, 8, 2, 96, 296, 128))                   # a padded (B=2) q
    assert L.masked_attn_varlen_fwd(ctypes.byref(vl), ctypes.byref(a), None) == bsm.BSM_E_SHAPE


def test_varlen_bwd_workspace_and_validation(L):
    vl, keep = _varlen([0, 32, 32, 192], [0, 132, 132, 592])
    need = ctypes.c_int64(-1)
    assert L.masked_attn_varlen_bwd_workspace_size(ctypes.byref(vl), ctypes.byref(need)) == 0
    assert need.value == 8 * 32 * 4 + 8 * 160 * 4          # Delta per sequence, 256-aligned
    a = _bwd_args((1, 8, 2, 192, 592, 128))
    a.workspace, a.workspace_bytes = 1 << 24, need.value
    pc = bsm.varlen_dflash(16).c()
    a.pred = ctypes.pointer(pc)
    m = _t4((1, 1, 192, 640))
    a.mask = ctypes.pointer(m)
    assert L.masked_attn_varlen_bwd(ctypes.byref(vl), ctypes.byref(a), None) == \
        bsm.BSM_E_UNSUPPORTED
    a.mask = None
    a.workspace_bytes = need.value - 256
    assert L.masked_attn_varlen_bwd(ctypes.byref(vl), ctypes.byref(a), None) == bsm.BSM_E_ARG
    a.workspace_bytes = need.value
    a.workspace = (1 << 24) + 16                              # not 256-byte aligned
    assert L.masked_attn_varlen_bwd(ctypes.byref(vl), ctypes.byref(a), None) == bsm.BSM_E_ARG
    a.workspace = 1 << 24
    a.lse = None
    assert L.masked_attn_varlen_bwd(ctypes.byref(vl), ctypes.byref(a), None) == bsm.BSM_E_ARG
    a.lse = 1 << 21
    bm = bsm.BlockMaskC(1 << 20, 1 << 20, 1 << 20, 1 << 20, 3, 1, 1, 5)   # nQ is 2
    a.bm = ctypes.pointer(bm)
    assert L.masked_attn_varlen_bwd(ctypes.byref(vl), ctypes.byref(a), None) == bsm.BSM_E_SHAPE
    a.bm = None
    b2 = _bwd_args((2, 8, 2, 96, 296, 128))                    # a padded (B=2) layout
    b2.workspace, b2.workspace_bytes = 1 << 24, need.value
    assert L.masked_attn_varlen_bwd(ctypes.byref(vl), ctypes.byref(b2), None) == bsm.BSM_E_SHAPE
    bad, keep2 = _varlen([0, 30, 62], [0, 130, 262])          # 30 queries, blocks of 16
    c = _bwd_args((1, 8, 2, 62, 262, 128))
    c.workspace, c.workspace_bytes = 1 << 24, 1 << 20
    c.pred = ctypes.pointer(pc)
    assert L.masked_attn_varlen_bwd(ctypes.byref(bad), ctypes.byref(c), None) == bsm.BSM_E_SHAPE


def test_row_copy_validation(L):
    assert L.gather_rows(1 << 20, 48, 1 << 21, 48, 40, 1 << 22, 5, None) == bsm.BSM_E_STRIDE
    assert L.gather_rows(1 << 20, 32, 1 << 21, 64, 64, 1 << 22, 5, None) == bsm.BSM_E_STRIDE
    assert L.scatter_rows(None, 64, 1 << 21, 64, 64, 1 << 22, 5, None) == bsm.BSM_E_ARG
    assert L.gather_rows(None, 64, None, 64, 64, None, 0, None) == 0   # nothing to copy
    assert L.unpad_index(1 << 20, 70000, 10, 10, 1 << 21, 1 << 22, None) == \
        bsm.BSM_E_UNSUPPORTED
    assert L.unpad_index(1 << 20, 4, 100, 50, 1 << 21, 1 << 22, None) == bsm.BSM_E_STRIDE


def test_forward_workspace_sizes(L):
    """Short query blocks with few (b, head) pairs ask for a split workspace."""
    def need(geom, **kw):
        a = _attn_args(geom, **kw)
        n = ctypes.c_int64(-1)
        st = L.attn_fwd_workspace_size(ctypes.byref(bsm.Geom(*geom)), ctypes.byref(a),
                                       ctypes.byref(n))
        return st, n.value
    # inference: 8 requests x 8 KV groups of 4 heads x 16 rows packed, 257 key
    # tiles -> 8 splits of (8, 32, 16) rows x (128 + 2) floats
    geom = (8, 32, 8, 16, 32784, 128)
    assert need(geom) == (0, 8 * 8 * 32 * 16 * 128 * 4 + 8 * 8 * 32 * 16 * 2 * 4)
    # a long prefill (tiled kernels) and a wide decode batch need none
    assert need((2, 32, 8, 4096, 8192, 128)) == (0, 0)
    assert need((64, 32, 8, 1, 16384, 128)) == (0, 0)
    assert need((8, 32, 8, 16, 32784, 128), dtype=bsm.BSM_F32) == (0, 0)
    a = _attn_args(geom)
    a.workspace, a.workspace_bytes = (1 << 24) + 8, 1 << 20
    assert L.masked_attn_fwd(ctypes.byref(bsm.Geom(*geom)), ctypes.byref(a), None) == \
        bsm.BSM_E_ARG  # misaligned workspace


def test_forward_staged_row_workspace(L):
    """Longer queries with a mask / bias that broadcast over the query dim ask
    for one float row per (b, head of the widest rule) and key: the dynamic
    top-k layout (mask and bias per KV head) needs B * KVH * K_round floats; a
    per-head bias makes it B * H; per-query tensors or the predicate need none."""
    geom = (2, 16, 4, 8000, 8000, 128)
    Kr = 8064
    keep = []

    def need(mshape=None, bshape=None, dtype=bsm.BSM_BF16, **kw):
        a = _attn_args(geom, dtype=dtype)
        if mshape is not None:
            m = _t4(mshape, bsm.BSM_BOOL)
            keep.append(m)
            a.mask = ctypes.pointer(m)
        if bshape is not None:
            bt = _t4(bshape, dtype)
            keep.append(bt)
            a.bias = ctypes.pointer(bt)
        for k, v in kw.items():
            setattr(a, k, v)
        n = ctypes.c_int64(-1)
        assert L.attn_fwd_workspace_size(ctypes.byref(bsm.Geom(*geom)), ctypes.byref(a),
                                         ctypes.byref(n)) == 0
        return n.value

    def rows(nrows):
        return (nrows * Kr * 4 + 255) // 256 * 256
    assert need((2, 4, 1, Kr), (2, 4, 1, Kr)) == rows(2 * 4)
    assert need((2, 4, 1, Kr), (2, 16, 1, Kr)) == rows(2 * 16)
    assert need((1, 1, 1, Kr), None) == rows(2 * 1)
    assert need(None, (2, 1, 1, Kr)) == rows(2 * 1)
    assert need((2, 4, 8000, Kr), (2, 4, 1, Kr)) == 0   # per-query mask
    assert need(None, (2, 16, 8000, Kr)) == 0           # per-query bias
    assert need(None, None) == 0
    assert need((2, 4, 1, Kr), (2, 4, 1, Kr), dtype=bsm.BSM_F32) == 0  # f32 kernel


def test_topk_fused_validation(L):
    geom = bsm.Geom(2, 16, 4, 8000, 8000, 128)
    bias = _t4((2, 4, 1, 8064), bsm.BSM_BF16)
    bm = bsm.BlockMaskC(1 << 22, 1 << 22, 1 << 22, 1 << 22, 2, 4, 1, 63)
    # nothing to produce
    assert L.dynamic_topk_fused(ctypes.byref(geom), ctypes.byref(bias), None, 10, None, None,
                                None, None) == bsm.BSM_E_ARG
    # block mask of the wrong shape
    bad = bsm.BlockMaskC(1 << 22, 1 << 22, 1 << 22, 1 << 22, 2, 1, 1, 63)
    assert L.dynamic_topk_fused(ctypes.byref(geom), ctypes.byref(bias), None, 10, None,
                                ctypes.byref(bad), None, None) == bsm.BSM_E_SHAPE
    # a key list needs at most 32 rows per (b, h): 8000 query rows here
    kl = bsm.KeyListC(1 << 22, 1 << 23, 1 << 24, 2, 4, 8000, 8064)
    assert L.dynamic_topk_fused(ctypes.byref(geom), ctypes.byref(bias), None, 10, None, None,
                                ctypes.byref(kl), None) == bsm.BSM_E_UNSUPPORTED
    # per-query bias rows: 8000 distinct mask rows per (b, h)
    per_q = _t4((2, 4, 8000, 8064), bsm.BSM_BF16)
    assert L.dynamic_topk_fused(ctypes.byref(geom), ctypes.byref(per_q), None, 10, 1 << 21,
                                None, None, None) == bsm.BSM_E_UNSUPPORTED
    # rows longer than the register-resident selection
    g2 = bsm.Geom(1, 8, 8, 1, 20000, 128)
    long_bias = _t4((1, 8, 1, 20096), bsm.BSM_BF16)
    assert L.dynamic_topk_fused(ctypes.byref(g2), ctypes.byref(long_bias), None, 10, 1 << 21,
                                None, None, None) == bsm.BSM_E_UNSUPPORTED
    # a bias whose mask does not fit the geometry (head dim 3)
    odd = _t4((2, 3, 1, 8064), bsm.BSM_BF16)
    assert L.dynamic_topk_fused(ctypes.byref(geom), ctypes.byref(odd), None, 10, 1 << 21,
                                None, None, None) == bsm.BSM_E_SHAPE
    assert bm.Bm == 2



def test_noalloc_scratch_size_matches_header(tmp_path):
    src = tmp_path / "scratch.c"
    src.write_text('#include <stdio.h>\n#include "bsm.h"\n'
                   'int main(void) { printf("%lld\\n", (long long)BSM_NOALLOC_SCRATCH_BYTES); '
                   'return 0; }\n')
    exe = tmp_path / "scratch"
    r = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("no C compiler for the header: " + r.stderr[:200])
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    assert int(out) == bsm.NOALLOC_SCRATCH_BYTES == 32 << 20


def test_noalloc_rejects_before_any_launch(L):
    """The entry point without allocation refuses a caller's workspace, and a
    call whose plan needs more than the static scratch, before touching a
    device (the stream argument is never used on these paths)."""
    geom = (2, 32, 8, 1, 16384, 128)
    g = bsm.Geom(*geom)
    a = _attn_args(geom)
    a.workspace, a.workspace_bytes = 1 << 24, 256
    assert L.masked_attn_fwd_noalloc(ctypes.byref(g), ctypes.byref(a), None) == bsm.BSM_E_ARG
    assert b"workspace" in L.bsm_last_error()
    # staged query-broadcast bias rows of (8, 32 heads, 100096 keys) floats: 102.5 MB
    big = (8, 32, 8, 256, 100000, 128)
    g = bsm.Geom(*big)
    a = _attn_args(big)
    bias = _t4((8, 32, 1, 100096), bsm.BSM_BF16)
    a.bias = ctypes.pointer(bias)
    need = ctypes.c_int64(0)
    assert L.attn_fwd_workspace_size(ctypes.byref(g), ctypes.byref(a), ctypes.byref(need)) == 0
    assert need.value == 8 * 32 * 782 * 128 * 4 > bsm.NOALLOC_SCRATCH_BYTES
    assert L.masked_attn_fwd_noalloc(ctypes.byref(g), ctypes.byref(a), None) == \
        bsm.BSM_E_UNSUPPORTED
    assert b"scratch" in L.bsm_last_error()
