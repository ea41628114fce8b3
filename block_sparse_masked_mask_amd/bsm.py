"""Thin Python binding of libbsm.so (include/bsm.h), argument marshalling only.

Every step of the path runs in the library's HIP kernels; torch supplies device
memory, shapes/strides and the current stream. There is no fallback: if the
library is not built, or a call fails, this module raises.

Names follow the C ABI: resolve_dflash_is_causal, block_mask_shape,
build_block_mask, key_list_shape, build_key_list, dynamic_topk_mask,
dflash_dense_mask, masked_attn_fwd, attn_bwd_workspace_size, masked_attn_bwd, plus
create_mask, the 2D/4D pre-mask normalisation of flash-sparse-attention PR #197
(Implementation Notes) done as zero-copy views before dynamic_topk_mask.
"""

import ctypes
import math
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_void_p
from dataclasses import dataclass
from typing import NamedTuple, Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbsm.so")

BSM_OK, BSM_E_ARG, BSM_E_SHAPE, BSM_E_STRIDE, BSM_E_DTYPE, BSM_E_UNSUPPORTED, BSM_E_HIP = \
    0, -1, -2, -3, -4, -5, -6
BSM_BOOL, BSM_BF16, BSM_F32 = 0, 1, 2
# bytes of the static device scratch of masked_attn_fwd_noalloc (BSM_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20

EXPORTS = ("resolve_dflash_is_causal", "block_mask_shape", "build_block_mask",
           "key_list_shape", "build_key_list", "dynamic_topk_mask", "dynamic_topk_fused",
           "dflash_dense_mask",
           "masked_attn_fwd", "masked_attn_fwd_noalloc", "attn_fwd_workspace_size",
           "attn_bwd_workspace_size",
           "masked_attn_bwd",
           "block_mask_varlen_shape", "build_block_mask_varlen", "masked_attn_varlen_fwd",
           "masked_attn_varlen_bwd_workspace_size", "masked_attn_varlen_bwd",
           "unpad_index", "gather_rows", "scatter_rows", "bsm_last_error")


class Tensor4(ctypes.Structure):
    _fields_ = [("data", c_void_p), ("dtype", c_int32), ("reserved", c_int32),
                ("size", c_int64 * 4), ("stride", c_int64 * 4)]


class Geom(ctypes.Structure):
    _fields_ = [(n, c_int64) for n in ("B", "H", "KVH", "Sq", "Sk", "D")]


class DFlashC(ctypes.Structure):
    _fields_ = [("ctx_len", c_int64), ("num_blocks", c_int64), ("block_size", c_int64),
                ("ctx_per_block", c_int64), ("ctx_end_offset", c_int64),
                ("is_causal", c_int32), ("layer_type", c_int32), ("sliding_window", c_int64)]


class BlockMaskC(ctypes.Structure):
    _fields_ = [("kv_num_blocks", c_void_p), ("kv_indices", c_void_p),
                ("full_kv_num_blocks", c_void_p), ("full_kv_indices", c_void_p),
                ("Bm", c_int64), ("Hm", c_int64), ("nQm", c_int64), ("nK", c_int64)]


class KeyListC(ctypes.Structure):
    _fields_ = [("num_keys", c_void_p), ("key_indices", c_void_p), ("row_bits", c_void_p),
                ("Bm", c_int64), ("Hm", c_int64), ("R", c_int64), ("K", c_int64)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("q", Tensor4), ("k", Tensor4), ("v", Tensor4), ("o", c_void_p),
                ("o_stride", c_int64 * 4), ("lse", c_void_p), ("softmax_scale", c_float),
                ("reserved", c_int32), ("pred", POINTER(DFlashC)), ("mask", POINTER(Tensor4)),
                ("bias", POINTER(Tensor4)), ("bm", POINTER(BlockMaskC)),
                ("keys", POINTER(KeyListC)), ("workspace", c_void_p),
                ("workspace_bytes", c_int64)]


class VarlenC(ctypes.Structure):
    _fields_ = [("num_seqs", c_int64), ("H", c_int64), ("KVH", c_int64), ("D", c_int64),
                ("total_q", c_int64), ("total_k", c_int64), ("cu_seqlens_q", c_void_p),
                ("cu_seqlens_k", c_void_p), ("cu_seqlens_q_host", c_void_p),
                ("cu_seqlens_k_host", c_void_p)]


class AttnBwdArgs(ctypes.Structure):
    _fields_ = [("q", Tensor4), ("k", Tensor4), ("v", Tensor4), ("o", Tensor4),
                ("dout", Tensor4), ("lse", c_void_p), ("dq", Tensor4), ("dk", Tensor4),
                ("dv", Tensor4), ("softmax_scale", c_float), ("reserved", c_int32),
                ("pred", POINTER(DFlashC)), ("mask", POINTER(Tensor4)),
                ("bias", POINTER(Tensor4)), ("bm", POINTER(BlockMaskC)),
                ("dbias", POINTER(Tensor4)), ("workspace", c_void_p),
                ("workspace_bytes", c_int64)]


_lib = None


def lib():
    """The loaded libbsm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built: run `python -m block_sparse_masked_mask_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.bsm_last_error.restype = c_char_p
        L.bsm_last_error.argtypes = []
        L.resolve_dflash_is_causal.argtypes = [c_int32, c_int32]
        L.block_mask_shape.argtypes = [POINTER(Geom), POINTER(DFlashC), POINTER(Tensor4),
                                       POINTER(c_int64)]
        L.build_block_mask.argtypes = [POINTER(Geom), POINTER(DFlashC), POINTER(Tensor4),
                                       POINTER(BlockMaskC), c_void_p]
        L.key_list_shape.argtypes = [POINTER(Geom), POINTER(Tensor4), POINTER(c_int64)]
        L.build_key_list.argtypes = [POINTER(Geom), POINTER(Tensor4), POINTER(KeyListC),
                                     c_void_p]
        L.dynamic_topk_mask.argtypes = [POINTER(Tensor4), POINTER(Tensor4), c_int64, c_int64,
                                        c_void_p, c_void_p]
        L.dynamic_topk_fused.argtypes = [POINTER(Geom), POINTER(Tensor4), POINTER(Tensor4),
                                         c_int64, c_void_p, POINTER(BlockMaskC),
                                         POINTER(KeyListC), c_void_p]
        L.dflash_dense_mask.argtypes = [POINTER(Geom), POINTER(DFlashC), c_void_p, c_void_p]
        L.masked_attn_fwd.argtypes = [POINTER(Geom), POINTER(AttnArgs), c_void_p]
        L.masked_attn_fwd_noalloc.argtypes = L.masked_attn_fwd.argtypes
        L.attn_fwd_workspace_size.argtypes = [POINTER(Geom), POINTER(AttnArgs), POINTER(c_int64)]
        L.attn_bwd_workspace_size.argtypes = [POINTER(Geom), POINTER(AttnBwdArgs),
                                              POINTER(c_int64)]
        L.masked_attn_bwd.argtypes = [POINTER(Geom), POINTER(AttnBwdArgs), c_void_p]
        L.block_mask_varlen_shape.argtypes = [POINTER(VarlenC), POINTER(DFlashC),
                                              POINTER(c_int64)]
        L.build_block_mask_varlen.argtypes = [POINTER(VarlenC), POINTER(DFlashC),
                                              POINTER(BlockMaskC), c_void_p]
        L.masked_attn_varlen_fwd.argtypes = [POINTER(VarlenC), POINTER(AttnArgs), c_void_p]
        L.masked_attn_varlen_bwd_workspace_size.argtypes = [POINTER(VarlenC), POINTER(c_int64)]
        L.masked_attn_varlen_bwd.argtypes = [POINTER(VarlenC), POINTER(AttnBwdArgs), c_void_p]
        L.unpad_index.argtypes = [c_void_p, c_int64, c_int64, c_int64, c_void_p, c_void_p,
                                  c_void_p]
        L.gather_rows.argtypes = [c_void_p, c_int64, c_void_p, c_int64, c_int64, c_void_p,
                                  c_int64, c_void_p]
        L.scatter_rows.argtypes = L.gather_rows.argtypes
        for name in EXPORTS[:-1]:
            getattr(L, name).restype = c_int32
        _lib = L
    return _lib


class BsmError(Exception):
    pass


def _check(status):
    if status >= 0:
        return status
    msg = lib().bsm_last_error().decode()
    if status in (BSM_E_ARG, BSM_E_SHAPE, BSM_E_STRIDE, BSM_E_DTYPE):
        raise ValueError(f"bsm status {status}: {msg}")
    raise RuntimeError(f"bsm status {status}: {msg}")


_DT = {torch.bool: BSM_BOOL, torch.uint8: BSM_BOOL, torch.bfloat16: BSM_BF16,
       torch.float32: BSM_F32}


def tensor4(t, dims=4):
    """Tensor4 view of a 4D torch tensor (sizes and element strides as they are)."""
    if t.dim() != dims:
        raise ValueError(f"expected a {dims}D tensor, got {tuple(t.shape)}")
    if t.dtype not in _DT:
        raise ValueError(f"unsupported dtype {t.dtype}")
    x = Tensor4()
    x.data = t.data_ptr() if t.numel() > 0 else None
    x.dtype = _DT[t.dtype]
    x.reserved = 0
    for i in range(4):
        x.size[i] = t.shape[i]
        x.stride[i] = t.stride(i)
    return x


def _stream(stream, *owned):
    """The HIP stream handle to launch on: `stream`, or torch's current stream
    when None. On a stream other than the current one, the launch must see what
    the current stream has queued (inputs written there, outputs zero-filled by
    this module), so `stream` first waits for it; and every tensor this module
    allocated for the call (`owned`: outputs, workspaces, or tuples of them) is
    recorded as used on `stream`, so that torch's caching allocator does not
    hand its memory out again before the launch has completed."""
    cur = torch.cuda.current_stream()
    if stream is None or stream == cur:
        return c_void_p(cur.cuda_stream)
    stream.wait_stream(cur)
    for t in owned:
        for x in (t if isinstance(t, tuple) else (t,)):
            if isinstance(x, torch.Tensor) and x.is_cuda:
                x.record_stream(stream)
    return c_void_p(stream.cuda_stream)


class Geometry(NamedTuple):
    B: int
    H: int
    KVH: int
    Sq: int
    Sk: int
    D: int

    def c(self):
        return Geom(*[int(x) for x in self])


def geometry_of(q, k):
    """Geometry from Q (B, Sq, H, D) and K (B, Sk, KVH, D)."""
    B, Sq, H, D = q.shape
    return Geometry(B, H, k.shape[2], Sq, k.shape[1], D)


@dataclass(frozen=True)
class DFlash:
    """DFlash draft-block mask parameters (see include/bsm.h, bsm_dflash).

    is_causal: None (absent), False or True; layer_type: 'full' or 'sliding'.
    """

    ctx_len: int
    num_blocks: int
    block_size: int
    ctx_per_block: int = 0
    ctx_end_offset: int = 0
    is_causal: Optional[bool] = None
    layer_type: str = "full"
    sliding_window: int = 0

    def c(self):
        ic = -1 if self.is_causal is None else int(bool(self.is_causal))
        lt = {"full": 0, "sliding": 1}.get(self.layer_type, self.layer_type)
        return DFlashC(self.ctx_len, self.num_blocks, self.block_size, self.ctx_per_block,
                       self.ctx_end_offset, ic, lt, self.sliding_window)

    @classmethod
    def inference(cls, ctx_len, block_size, is_causal=None, layer_type="full", sliding_window=0):
        """One draft block after ctx_len cached tokens (the default mask of
        inference): the block sees every cached token, and keys are the cache
        followed by the block's own block_size tokens."""
        return cls(ctx_len, 1, block_size, ctx_per_block=ctx_len, is_causal=is_causal,
                   layer_type=layer_type, sliding_window=sliding_window)

    @property
    def Sq(self):
        return self.num_blocks * self.block_size

    @property
    def Sk(self):
        return self.ctx_len + self.num_blocks * self.block_size


class BlockMask(NamedTuple):
    kv_num_blocks: torch.Tensor
    kv_indices: torch.Tensor
    full_kv_num_blocks: torch.Tensor
    full_kv_indices: torch.Tensor

    def c(self):
        Bm, Hm, nQm, nK = self.kv_indices.shape
        return BlockMaskC(self.kv_num_blocks.data_ptr(), self.kv_indices.data_ptr(),
                          self.full_kv_num_blocks.data_ptr(), self.full_kv_indices.data_ptr(),
                          Bm, Hm, nQm, nK)


class KeyList(NamedTuple):
    """Kept keys of a mask over a short query block: num_keys (Bm, Hm), ascending
    key_indices (Bm, Hm, K) and per-key row words row_bits (Bm, Hm, K, int32
    holding the uint32 bits); entries past num_keys are unspecified."""
    num_keys: torch.Tensor
    key_indices: torch.Tensor
    row_bits: torch.Tensor
    rows: int

    def c(self):
        Bm, Hm, K = self.key_indices.shape
        return KeyListC(self.num_keys.data_ptr(), self.key_indices.data_ptr(),
                        self.row_bits.data_ptr(), Bm, Hm, self.rows, K)


def round_multiple(x, m=128):
    return (int(x) + m - 1) // m * m


def resolve_dflash_is_causal(is_causal, layer_type):
    ic = -1 if is_causal is None else int(bool(is_causal))
    lt = {"full": 0, "sliding": 1}.get(layer_type, layer_type)
    return bool(_check(lib().resolve_dflash_is_causal(ic, lt)))


def block_mask_shape(geom, pred=None, mask=None):
    out = (c_int64 * 4)()
    g = Geometry(*geom).c()
    pc = pred.c() if pred is not None else None
    mc = tensor4(mask) if mask is not None else None
    _check(lib().block_mask_shape(ctypes.byref(g), ctypes.byref(pc) if pc else None,
                                  ctypes.byref(mc) if mc else None, out))
    return tuple(int(x) for x in out)


def build_block_mask(geom, pred=None, mask=None, device=None, stream=None):
    """Block mask of a DFlash predicate or a dense bool mask (four int32 tensors)."""
    shp = block_mask_shape(geom, pred, mask)
    if device is None:
        device = mask.device if mask is not None else torch.device("cuda")
    Bm, Hm, nQm, nK = shp
    bm = BlockMask(torch.empty((Bm, Hm, nQm), dtype=torch.int32, device=device),
                   torch.empty((Bm, Hm, nQm, nK), dtype=torch.int32, device=device),
                   torch.empty((Bm, Hm, nQm), dtype=torch.int32, device=device),
                   torch.empty((Bm, Hm, nQm, nK), dtype=torch.int32, device=device))
    g = Geometry(*geom).c()
    pc = pred.c() if pred is not None else None
    mc = tensor4(mask) if mask is not None else None
    bc = bm.c()
    _check(lib().build_block_mask(ctypes.byref(g), ctypes.byref(pc) if pc else None,
                                  ctypes.byref(mc) if mc else None, ctypes.byref(bc),
                                  _stream(stream, bm)))
    return bm


def key_list_shape(geom, mask):
    out = (c_int64 * 4)()
    mc = tensor4(mask)
    _check(lib().key_list_shape(ctypes.byref(Geometry(*geom).c()), ctypes.byref(mc), out))
    return tuple(int(x) for x in out)


def build_key_list(geom, mask, stream=None):
    """Kept-key list of a bool mask (at most 32 rows per (b, h) after the swap)."""
    Bm, Hm, R, K = key_list_shape(geom, mask)
    dev = mask.device
    kl = KeyList(torch.empty((Bm, Hm), dtype=torch.int32, device=dev),
                 torch.empty((Bm, Hm, K), dtype=torch.int32, device=dev),
                 torch.empty((Bm, Hm, K), dtype=torch.int32, device=dev), R)
    mc = tensor4(mask)
    kc = kl.c()
    _check(lib().build_key_list(ctypes.byref(Geometry(*geom).c()), ctypes.byref(mc),
                                ctypes.byref(kc), _stream(stream, kl)))
    return kl


def dynamic_topk_mask(bias, premask, seqlen_k, k, out=None, stream=None):
    """Top-k keep mask (bool, bias's shape) over a 4D bias."""
    owned = out is None
    if out is None:
        out = torch.empty(bias.shape, dtype=torch.bool, device=bias.device)
    bc = tensor4(bias)
    pc = tensor4(premask) if premask is not None else None
    _check(lib().dynamic_topk_mask(ctypes.byref(bc), ctypes.byref(pc) if pc else None,
                                   int(seqlen_k), int(k),
                                   out.data_ptr() if out.numel() else None,
                                   _stream(stream, out if owned else None)))
    return out


def dynamic_topk_fused(geom, bias, premask, k, want_mask=True, want_block_mask=True,
                       want_keys=False, stream=None):
    """Top-k over `bias` (seqlen_k = geom Sk) and, from the same pass, the block
    mask and / or the kept-key list of its mask. Returns (mask, block_mask, keys)
    with None for what was not asked."""
    g = Geometry(*geom)
    dev = bias.device
    mask = torch.empty(bias.shape, dtype=torch.bool, device=dev) if want_mask else None
    bm = keys = None
    if want_block_mask:
        Bm, Hm, nQm, nK = _mask_bm_shape(g, bias.shape)
        bm = BlockMask(torch.empty((Bm, Hm, nQm), dtype=torch.int32, device=dev),
                       torch.empty((Bm, Hm, nQm, nK), dtype=torch.int32, device=dev),
                       torch.empty((Bm, Hm, nQm), dtype=torch.int32, device=dev),
                       torch.empty((Bm, Hm, nQm, nK), dtype=torch.int32, device=dev))
    if want_keys:
        Bm, Hm, R, K = _mask_kl_shape(g, bias.shape)
        keys = KeyList(torch.empty((Bm, Hm), dtype=torch.int32, device=dev),
                       torch.empty((Bm, Hm, K), dtype=torch.int32, device=dev),
                       torch.empty((Bm, Hm, K), dtype=torch.int32, device=dev), R)
    bc = tensor4(bias)
    pc = tensor4(premask) if premask is not None else None
    bmc = bm.c() if bm is not None else None
    kc = keys.c() if keys is not None else None
    _check(lib().dynamic_topk_fused(ctypes.byref(g.c()), ctypes.byref(bc),
                                    ctypes.byref(pc) if pc else None, int(k),
                                    mask.data_ptr() if mask is not None and mask.numel() else None,
                                    ctypes.byref(bmc) if bmc else None,
                                    ctypes.byref(kc) if kc else None,
                                    _stream(stream, mask, bm, keys)))
    return mask, bm, keys


def _contig_mask4(shape):
    """Tensor4 of a contiguous bool mask of this shape (sizes and strides only)."""
    x = Tensor4()
    x.data = 256
    x.dtype = BSM_BOOL
    x.reserved = 0
    st = 1
    for i in (3, 2, 1, 0):
        x.size[i] = shape[i]
        x.stride[i] = st
        st *= shape[i]
    return x


def _mask_bm_shape(g, shape):
    out = (c_int64 * 4)()
    mc = _contig_mask4(shape)
    _check(lib().block_mask_shape(ctypes.byref(g.c()), None, ctypes.byref(mc), out))
    return tuple(int(x) for x in out)


def _mask_kl_shape(g, shape):
    out = (c_int64 * 4)()
    mc = _contig_mask4(shape)
    _check(lib().key_list_shape(ctypes.byref(g.c()), ctypes.byref(mc), out))
    return tuple(int(x) for x in out)


def create_mask(attention_bias, attention_mask, batch_size, query_len, key_len, window_size,
                stream=None):
    """Normalise a 2D or 4D pre-mask to the bias's 4D contract, then top-k.

    2D (batch, key_len) -> (batch, 1, 1, key_len) view; 4D must already
    broadcast to the bias (dims 1 or equal, last dim key_len or K_round).
    A 2D mask of length query_len != key_len is not supported (the pages
    disagree on whether to pad it with ones or zeros).
    """
    pm = attention_mask
    if pm is not None:
        if pm.dim() == 2:
            if tuple(pm.shape) == (batch_size, key_len):
                pm = pm.as_strided((batch_size, 1, 1, key_len), (pm.stride(0), 0, 0, pm.stride(1)))
            elif pm.shape[1] == query_len:
                raise NotImplementedError("2D mask over query_len != key_len is not supported")
            else:
                raise ValueError(f"2D mask must be (batch, key_len), got {tuple(pm.shape)}")
        elif pm.dim() != 4:
            raise ValueError("mask must be 2D or 4D")
        if pm.dtype != torch.bool:
            raise ValueError("mask must be bool")
    return dynamic_topk_mask(attention_bias, pm, key_len, window_size, stream=stream)


def dflash_dense_mask(geom, pred, out=None, stream=None):
    """Dense (Sq, K_round) bool DFlash mask, written by the library's kernel."""
    g = Geometry(*geom)
    owned = out is None
    if out is None:
        out = torch.empty((g.Sq, round_multiple(g.Sk)), dtype=torch.bool, device="cuda")
    pc = pred.c()
    _check(lib().dflash_dense_mask(ctypes.byref(g.c()), ctypes.byref(pc),
                                   out.data_ptr() if out.numel() else None,
                                   _stream(stream, out if owned else None)))
    return out


def _fwd_args(q, k, v, pred, mask, bias, block_mask, softmax_scale, return_lse, out, lse,
              keys):
    """AttnArgs of a forward call; returns (geometry, args, the ctypes objects
    it points to, out, lse, the tensors allocated here)."""
    geom = geometry_of(q, k)
    owned = []
    if out is None:
        out = torch.empty_like(q)
        owned.append(out)
    if return_lse and lse is None:
        lse = torch.empty((geom.B, geom.H, geom.Sq), dtype=torch.float32, device=q.device)
        owned.append(lse)
    a = AttnArgs()
    a.q, a.k, a.v = tensor4(q), tensor4(k), tensor4(v)
    a.o = out.data_ptr() if out.numel() else None
    for i in range(4):
        a.o_stride[i] = out.stride(i)
    a.lse = lse.data_ptr() if lse is not None else None
    a.softmax_scale = 0.0 if softmax_scale is None else float(softmax_scale)
    a.reserved = 0
    keep = []
    if pred is not None:
        pc = pred.c()
        keep.append(pc)
        a.pred = ctypes.pointer(pc)
    if mask is not None:
        mc = tensor4(mask)
        keep.append(mc)
        a.mask = ctypes.pointer(mc)
    if bias is not None:
        bc = tensor4(bias)
        keep.append(bc)
        a.bias = ctypes.pointer(bc)
    if block_mask is not None:
        bmc = block_mask.c()
        keep.append(bmc)
        a.bm = ctypes.pointer(bmc)
    if keys is not None:
        kc = keys.c()
        keep.append(kc)
        a.keys = ctypes.pointer(kc)
    return geom, a, keep, out, lse, owned


def masked_attn_fwd(q, k, v, pred=None, mask=None, bias=None, block_mask=None,
                    softmax_scale=None, return_lse=False, out=None, lse=None, stream=None,
                    keys=None, split=True, workspace=None):
    """Masked attention forward; returns O (and LSE if return_lse).

    split: allocate (unless given) the workspace attn_fwd_workspace_size asks
    for, which lets short query blocks split their keys over several
    workgroups and folds a query-broadcast mask / bias into staged rows;
    split=False runs without either."""
    geom, a, keep, out, lse, owned = _fwd_args(q, k, v, pred, mask, bias, block_mask,
                                               softmax_scale, return_lse, out, lse, keys)
    gc = geom.c()
    if split:
        if workspace is None:
            need = c_int64(0)
            _check(lib().attn_fwd_workspace_size(ctypes.byref(gc), ctypes.byref(a),
                                                 ctypes.byref(need)))
            if need.value > 0:
                workspace = torch.empty(need.value, dtype=torch.uint8, device=q.device)
                owned.append(workspace)
        if workspace is not None:
            a.workspace = workspace.data_ptr()
            a.workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().masked_attn_fwd(ctypes.byref(gc), ctypes.byref(a),
                                 _stream(stream, *owned)))
    return (out, lse) if return_lse else out


def masked_attn_fwd_noalloc(q, k, v, out, lse=None, pred=None, mask=None, bias=None,
                            block_mask=None, softmax_scale=None, stream=None, keys=None):
    """masked_attn_fwd through the library's entry point that allocates
    nothing: the caller passes O (and LSE, or None), and any workspace comes
    from the library's static device scratch (see NOALLOC_SCRATCH_BYTES).
    Calls that overlap in time on one device share that scratch and race."""
    geom, a, keep, out, lse, _ = _fwd_args(q, k, v, pred, mask, bias, block_mask,
                                           softmax_scale, lse is not None, out, lse, keys)
    _check(lib().masked_attn_fwd_noalloc(ctypes.byref(geom.c()), ctypes.byref(a),
                                         _stream(stream)))
    return out


def masked_attn_bwd(q, k, v, out, dout, lse, pred=None, mask=None, bias=None, block_mask=None,
                    softmax_scale=None, need_dbias=False, stream=None):
    """Masked attention backward; returns (dq, dk, dv, dbias). dbias is None
    unless need_dbias (with a bias); it has the bias's shape, K-dim rounded to
    128, and is returned sliced to Sk like the gradients of PR #190."""
    geom = geometry_of(q, k)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dbias = None
    a = AttnBwdArgs()
    a.q, a.k, a.v = tensor4(q), tensor4(k), tensor4(v)
    a.o, a.dout = tensor4(out), tensor4(dout)
    a.lse = lse.data_ptr() if lse.numel() else None
    a.dq, a.dk, a.dv = tensor4(dq), tensor4(dk), tensor4(dv)
    a.softmax_scale = 0.0 if softmax_scale is None else float(softmax_scale)
    a.reserved = 0
    keep = []
    if pred is not None:
        pc = pred.c()
        keep.append(pc)
        a.pred = ctypes.pointer(pc)
    if mask is not None:
        mc = tensor4(mask)
        keep.append(mc)
        a.mask = ctypes.pointer(mc)
    if bias is not None:
        bc = tensor4(bias)
        keep.append(bc)
        a.bias = ctypes.pointer(bc)
        if need_dbias:
            dbias = torch.empty(bias.shape, dtype=bias.dtype, device=bias.device)
            dc = tensor4(dbias)
            keep.append(dc)
            a.dbias = ctypes.pointer(dc)
    if block_mask is not None:
        bmc = block_mask.c()
        keep.append(bmc)
        a.bm = ctypes.pointer(bmc)
    gc = geom.c()
    nbytes = c_int64(0)
    _check(lib().attn_bwd_workspace_size(ctypes.byref(gc), ctypes.byref(a), ctypes.byref(nbytes)))
    ws = torch.empty(max(nbytes.value, 1), dtype=torch.uint8, device=q.device)
    a.workspace = ws.data_ptr()
    a.workspace_bytes = nbytes.value
    _check(lib().masked_attn_bwd(ctypes.byref(gc), ctypes.byref(a),
                                 _stream(stream, dq, dk, dv, dbias, ws)))
    if dbias is not None:
        dbias = dbias[..., :geom.Sk]
    return dq, dk, dv, dbias


def default_scale(D):
    return 1.0 / math.sqrt(D)


# ---------------------------------------------------------------------------
# packed variable-length sequences


class Varlen:
    """Packed sequences: cu_seqlens_q / cu_seqlens_k (int32, num_seqs + 1) on the
    device, with host copies kept for the library's validation."""

    def __init__(self, cu_seqlens_q, cu_seqlens_k, H, KVH, D):
        self.cu_q = cu_seqlens_q.to(torch.int32).contiguous()
        self.cu_k = cu_seqlens_k.to(torch.int32).contiguous()
        self.cu_q_host = self.cu_q.cpu().contiguous()
        self.cu_k_host = self.cu_k.cpu().contiguous()
        self.H, self.KVH, self.D = int(H), int(KVH), int(D)

    @property
    def num_seqs(self):
        return self.cu_q_host.numel() - 1

    def c(self):
        return VarlenC(self.num_seqs, self.H, self.KVH, self.D, int(self.cu_q_host[-1]),
                       int(self.cu_k_host[-1]), self.cu_q.data_ptr(), self.cu_k.data_ptr(),
                       self.cu_q_host.data_ptr(), self.cu_k_host.data_ptr())


def varlen_dflash(block_size, ctx_per_block=0, ctx_end_offset=0, is_causal=None,
                  layer_type="full", sliding_window=0):
    """DFlash predicate for packed sequences: each sequence's context and block
    count come from its own lengths (ctx_len and num_blocks are 0)."""
    return DFlash(0, 0, block_size, ctx_per_block, ctx_end_offset, is_causal, layer_type,
                  sliding_window)


def block_mask_varlen_shape(varlen, pred):
    out = (c_int64 * 4)()
    vc = varlen.c()
    pc = pred.c()
    _check(lib().block_mask_varlen_shape(ctypes.byref(vc), ctypes.byref(pc), out))
    return tuple(int(x) for x in out)


def build_block_mask_varlen(varlen, pred, stream=None):
    """Per-sequence DFlash block mask (num_seqs, 1, nQmax, nKmax)."""
    Bm, Hm, nQm, nK = block_mask_varlen_shape(varlen, pred)
    dev = varlen.cu_q.device
    bm = BlockMask(torch.empty((Bm, Hm, nQm), dtype=torch.int32, device=dev),
                   torch.empty((Bm, Hm, nQm, nK), dtype=torch.int32, device=dev),
                   torch.empty((Bm, Hm, nQm), dtype=torch.int32, device=dev),
                   torch.empty((Bm, Hm, nQm, nK), dtype=torch.int32, device=dev))
    vc, pc, bc = varlen.c(), pred.c(), bm.c()
    _check(lib().build_block_mask_varlen(ctypes.byref(vc), ctypes.byref(pc), ctypes.byref(bc),
                                         _stream(stream, bm)))
    return bm


def masked_attn_varlen_fwd(q, k, v, varlen, pred=None, block_mask=None, softmax_scale=None,
                           return_lse=False, out=None, stream=None):
    """Attention over packed sequences: q (total_q, H, D), k / v (total_k, KVH, D);
    returns O (total_q, H, D) and, if asked, LSE (H, total_q)."""
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("packed q, k, v must be 3D (rows, heads, D)")
    q4, k4, v4 = q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0)
    owned = out is None
    if out is None:
        out = torch.empty_like(q)
    o4 = out.unsqueeze(0)
    lse = torch.empty((1, q.shape[1], q.shape[0]), dtype=torch.float32,
                      device=q.device) if return_lse else None
    a = AttnArgs()
    a.q, a.k, a.v = tensor4(q4), tensor4(k4), tensor4(v4)
    a.o = o4.data_ptr() if o4.numel() else None
    for i in range(4):
        a.o_stride[i] = o4.stride(i)
    a.lse = lse.data_ptr() if lse is not None else None
    a.softmax_scale = 0.0 if softmax_scale is None else float(softmax_scale)
    a.reserved = 0
    keep = []
    if pred is not None:
        pc = pred.c()
        keep.append(pc)
        a.pred = ctypes.pointer(pc)
    if block_mask is not None:
        bmc = block_mask.c()
        keep.append(bmc)
        a.bm = ctypes.pointer(bmc)
    vc = varlen.c()
    _check(lib().masked_attn_varlen_fwd(ctypes.byref(vc), ctypes.byref(a),
                                        _stream(stream, out if owned else None, lse)))
    return (out, lse[0]) if return_lse else out


def masked_attn_varlen_bwd(q, k, v, out, dout, lse, varlen, pred=None, block_mask=None,
                           softmax_scale=None, stream=None):
    """Backward of masked_attn_varlen_fwd: q, out, dout (total_q, H, D), k, v
    (total_k, KVH, D), lse (H, total_q) as that forward returns it; returns
    (dq, dk, dv) in the packed layouts."""
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        if t.dim() != 3:
            raise ValueError(f"packed {name} must be 3D (rows, heads, D)")
    if lse.dim() != 2 or tuple(lse.shape) != (q.shape[1], q.shape[0]):
        raise ValueError("lse must be (H, total_q)")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    a = AttnBwdArgs()
    a.q, a.k, a.v = tensor4(q.unsqueeze(0)), tensor4(k.unsqueeze(0)), tensor4(v.unsqueeze(0))
    a.o, a.dout = tensor4(out.unsqueeze(0)), tensor4(dout.unsqueeze(0))
    lse = lse.contiguous()
    a.lse = lse.data_ptr() if lse.numel() else None
    a.dq, a.dk, a.dv = tensor4(dq.unsqueeze(0)), tensor4(dk.unsqueeze(0)), tensor4(dv.unsqueeze(0))
    a.softmax_scale = 0.0 if softmax_scale is None else float(softmax_scale)
    a.reserved = 0
    keep = []
    if pred is not None:
        pc = pred.c()
        keep.append(pc)
        a.pred = ctypes.pointer(pc)
    if block_mask is not None:
        bmc = block_mask.c()
        keep.append(bmc)
        a.bm = ctypes.pointer(bmc)
    vc = varlen.c()
    nbytes = c_int64(0)
    _check(lib().masked_attn_varlen_bwd_workspace_size(ctypes.byref(vc), ctypes.byref(nbytes)))
    ws = torch.empty(max(nbytes.value, 1), dtype=torch.uint8, device=q.device)
    a.workspace = ws.data_ptr()
    a.workspace_bytes = nbytes.value
    _check(lib().masked_attn_varlen_bwd(ctypes.byref(vc), ctypes.byref(a),
                                        _stream(stream, dq, dk, dv, ws, lse)))
    return dq, dk, dv


def unpad(x, valid, stream=None):
    """Packed rows of a padded (B, S, ...) tensor: returns (packed, indices,
    cu_seqlens, max_seqlen). The index pass runs on the device; the total is
    read back to size the packed tensor."""
    B, S = valid.shape
    if tuple(x.shape[:2]) != (B, S):
        raise ValueError("x and valid disagree on (batch, seqlen)")
    if valid.dtype != torch.bool or valid.stride(1) != 1:
        raise ValueError("valid must be a bool tensor with contiguous rows")
    xc = x.contiguous()
    cu = torch.empty(B + 1, dtype=torch.int32, device=x.device)
    idx = torch.empty(max(B * S, 1), dtype=torch.int32, device=x.device)
    _check(lib().unpad_index(valid.data_ptr() if valid.numel() else None, B, S,
                             valid.stride(0), cu.data_ptr(), idx.data_ptr(),
                             _stream(stream, xc, cu, idx)))
    if stream is not None:
        # the read-back runs on the current stream: order it after the index pass
        torch.cuda.current_stream().wait_stream(stream)
    cu_host = cu.cpu()
    total = int(cu_host[-1])
    lens = cu_host[1:] - cu_host[:-1]
    row_shape = tuple(x.shape[2:])
    row_bytes = xc[0, 0].numel() * xc.element_size() if B * S else 0
    packed = torch.empty((total,) + row_shape, dtype=x.dtype, device=x.device)
    if total:
        _check(lib().gather_rows(xc.data_ptr(), row_bytes, packed.data_ptr(), row_bytes,
                                 row_bytes, idx.data_ptr(), total, _stream(stream, packed)))
    return packed, idx[:total], cu, int(lens.max()) if B else 0


def pad(packed, indices, B, S, stream=None):
    """(B, S, ...) zeros with packed row i at flat position indices[i]."""
    pc = packed.contiguous()
    out = torch.zeros((B, S) + tuple(packed.shape[1:]), dtype=packed.dtype, device=packed.device)
    n = pc.shape[0]
    if n:
        row_bytes = pc[0].numel() * pc.element_size()
        _check(lib().scatter_rows(pc.data_ptr(), row_bytes, out.data_ptr(), row_bytes,
                                  row_bytes, indices.data_ptr(), n, _stream(stream, pc, out)))
    return out

