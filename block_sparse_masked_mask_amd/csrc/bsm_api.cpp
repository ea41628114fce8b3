// Host side of the C ABI declared in include/bsm.h: argument validation, the
// broadcast / head-group-swap view rewrites, and kernel launches on the caller's
// stream. No device memory is allocated here and nothing synchronises the host.
//
// Shape contract (flash-sparse-attention PR #190, Design and Changes): aux
// tensors are 4D ({B|1}, {H|KVH|1}, {Sq|1}, round_multiple(Sk, 128)) with a
// contiguous last dim; size-1 dims broadcast by stride 0; nothing is implicitly
// unsqueezed or expanded. Swapped path (PR #190, Design / Implementation Notes):
// with Sq == 1 and H > KVH the G heads of a KV group become G query rows of that
// KV head, by rewriting strides only, and the LSE write-back follows the same
// view.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <utility>
#include <vector>

#include "bsm.h"
#include "bsm_internal.h"
#include "dflash_rows.h"

using namespace bsm;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int64_t round_multiple(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

int elem_size(int32_t dt) { return dt == BSM_BOOL ? 1 : (dt == BSM_BF16 ? 2 : 4); }

struct Geo {
  int64_t B, H, KVH, Sq, Sk, D, G, Kr, nQ, nK;
  bool swap;
};

int check_geom(const bsm_geom* g, Geo& o) {
  if (!g) return fail(BSM_E_ARG, "geom is NULL");
  if (g->B < 0 || g->H < 1 || g->KVH < 1 || g->Sq < 0 || g->Sk < 0 || g->D < 1)
    return fail(BSM_E_SHAPE, "bad geometry B=%lld H=%lld KVH=%lld Sq=%lld Sk=%lld D=%lld",
                (long long)g->B, (long long)g->H, (long long)g->KVH, (long long)g->Sq,
                (long long)g->Sk, (long long)g->D);
  if (g->H % g->KVH)
    return fail(BSM_E_SHAPE, "H=%lld is not a multiple of KVH=%lld", (long long)g->H,
                (long long)g->KVH);
  if (g->Sq > INT32_MAX / 2 || g->Sk > INT32_MAX / 2 || g->B > 65535 || g->H > 65535)
    return fail(BSM_E_UNSUPPORTED, "geometry beyond the library's size limits");
  o.B = g->B;
  o.H = g->H;
  o.KVH = g->KVH;
  o.Sq = g->Sq;
  o.Sk = g->Sk;
  o.D = g->D;
  o.G = g->H / g->KVH;
  o.Kr = round_multiple(g->Sk, kTile);
  o.nK = o.Kr / kTile;
  o.nQ = (g->Sq + kTile - 1) / kTile;
  o.swap = g->Sq == 1 && g->H > g->KVH;
  return BSM_OK;
}

int resolve_causal(int32_t is_causal, int32_t layer_type) {
  if (layer_type != 0 && layer_type != 1) return -1;
  if (is_causal == -1) return layer_type == 1;
  if (is_causal == 0 || is_causal == 1) return is_causal;
  return -1;
}

int check_dflash(const bsm_dflash* d, const Geo& g, DFlashRule& r) {
  if (d->ctx_len < 0 || d->num_blocks < 0 || d->block_size < 1 || d->ctx_per_block < 0)
    return fail(BSM_E_ARG, "bad DFlash sizes ctx_len=%lld num_blocks=%lld block_size=%lld",
                (long long)d->ctx_len, (long long)d->num_blocks, (long long)d->block_size);
  const int c = resolve_causal(d->is_causal, d->layer_type);
  if (c < 0)
    return fail(BSM_E_ARG, "bad is_causal=%d / layer_type=%d", d->is_causal, d->layer_type);
  int64_t S = d->ctx_per_block;
  if (S == 0 && d->num_blocks > 0) {
    if (d->ctx_len % d->num_blocks)
      return fail(BSM_E_ARG, "ctx_per_block=0 needs ctx_len %% num_blocks == 0");
    S = d->ctx_len / d->num_blocks;
  }
  if (g.Sq != d->num_blocks * d->block_size)
    return fail(BSM_E_SHAPE, "DFlash needs Sq == num_blocks*block_size (%lld != %lld)",
                (long long)g.Sq, (long long)(d->num_blocks * d->block_size));
  if (g.Sk != d->ctx_len + d->num_blocks * d->block_size)
    return fail(BSM_E_SHAPE, "DFlash needs Sk == ctx_len + num_blocks*block_size");
  if (d->layer_type == 1 && d->sliding_window < 1)
    return fail(BSM_E_ARG, "sliding layer needs sliding_window >= 1");
  r.C = d->ctx_len;
  r.bs = d->block_size;
  r.S = S;
  r.e0 = d->ctx_end_offset;
  r.W = d->layer_type == 1 ? d->sliding_window : 0;
  r.causal = c;
  r.pad = 0;
  return BSM_OK;
}

// Stride rules common to every 4D view: last dim contiguous, no negative
// stride, no 0 stride on a dim of size > 1, 16-byte aligned rows.
int check_strides(const bsm_tensor4* t, const char* name, int esz) {
  if (t->reserved != 0) return fail(BSM_E_ARG, "%s.reserved must be 0", name);
  if (t->size[3] > 1 && t->stride[3] != 1)
    return fail(BSM_E_STRIDE, "%s: last dim must be contiguous", name);
  for (int i = 0; i < 3; ++i) {
    if (t->stride[i] < 0) return fail(BSM_E_STRIDE, "%s: negative stride", name);
    if (t->size[i] > 1 && t->stride[i] == 0)
      return fail(BSM_E_STRIDE, "%s: stride 0 on dim %d of size %lld (no implicit expand)",
                  name, i, (long long)t->size[i]);
    if (t->size[i] > 1 && (t->stride[i] * esz) % 16)
      return fail(BSM_E_STRIDE, "%s: dim %d stride is not a multiple of 16 bytes", name, i);
  }
  if ((uintptr_t)t->data % 16) return fail(BSM_E_STRIDE, "%s: data not 16-byte aligned", name);
  for (int i = 0; i < 4; ++i)
    if (t->size[i] < 0) return fail(BSM_E_SHAPE, "%s: negative size", name);
  return BSM_OK;
}

int64_t numel(const bsm_tensor4* t) {
  return t->size[0] * t->size[1] * t->size[2] * t->size[3];
}

// Aux tensor (mask / bias) in the attention's iteration space.
struct Aux {
  AuxView view;
  int64_t Bm, Hm, Qm;  // sizes in that space
};

int check_aux(const bsm_tensor4* t, const char* name, const Geo& g, int32_t dtype, Aux& a) {
  if (t->dtype != dtype)
    return fail(BSM_E_DTYPE, "%s: dtype %d, expected %d", name, t->dtype, dtype);
  const int esz = elem_size(dtype);
  int e = check_strides(t, name, esz);
  if (e) return e;
  if (t->size[3] != g.Kr)
    return fail(BSM_E_SHAPE, "%s: last dim %lld must be round_multiple(Sk,128)=%lld", name,
                (long long)t->size[3], (long long)g.Kr);
  if (t->size[0] != g.B && t->size[0] != 1)
    return fail(BSM_E_SHAPE, "%s: dim 0 must be B or 1", name);
  if (t->size[1] != g.H && t->size[1] != g.KVH && t->size[1] != 1)
    return fail(BSM_E_SHAPE, "%s: dim 1 must be H, KVH or 1", name);
  if (t->size[2] != g.Sq && t->size[2] != 1)
    return fail(BSM_E_SHAPE, "%s: dim 2 must be Sq or 1", name);
  if (!t->data && numel(t) > 0) return fail(BSM_E_ARG, "%s: data is NULL", name);
  const int64_t sb = t->size[0] == 1 ? 0 : t->stride[0];
  const int64_t sh = t->size[1] == 1 ? 0 : t->stride[1];
  const int64_t sq = t->size[2] == 1 ? 0 : t->stride[2];
  a.view.data = t->data;
  a.view.sb = sb;
  a.Bm = t->size[0];
  if (!g.swap) {
    a.view.h_mode = t->size[1] == g.H ? 1 : (t->size[1] == g.KVH ? 2 : 0);
    a.view.sh = sh;
    a.view.sq = sq;
    a.view.q_bcast = t->size[2] == 1;
    a.Hm = t->size[1];
    a.Qm = t->size[2];
  } else if (t->size[1] == g.H) {
    // (Bm, H, 1, K) viewed as (Bm, KVH, G, K): head kvh*G + g -> row g of kvh
    a.view.h_mode = 1;
    a.view.sh = g.G * t->stride[1];
    a.view.sq = t->stride[1];
    a.view.q_bcast = 0;
    a.Hm = g.KVH;
    a.Qm = g.G;
  } else if (t->size[1] == g.KVH) {
    a.view.h_mode = 1;
    a.view.sh = sh;
    a.view.sq = 0;
    a.view.q_bcast = 1;
    a.Hm = g.KVH;
    a.Qm = 1;
  } else {
    a.view.h_mode = 0;
    a.view.sh = 0;
    a.view.sq = 0;
    a.view.q_bcast = 1;
    a.Hm = 1;
    a.Qm = 1;
  }
  return BSM_OK;
}

// Heads and query rows of the attention's iteration space.
int64_t iter_heads(const Geo& g) { return g.swap ? g.KVH : g.H; }
int64_t iter_rows(const Geo& g) { return g.swap ? g.G : g.Sq; }

int expected_bm(const Geo& g, const bsm_dflash* pred, const Aux* mask, int64_t out[4]) {
  if (pred) {
    out[0] = 1;
    out[1] = 1;
    out[2] = g.nQ;  // the predicate's rows (Sq == 1 under the swap: one tile)
    out[3] = g.nK;
  } else {
    out[0] = mask->Bm;
    out[1] = mask->Hm;
    out[2] = (mask->Qm + kTile - 1) / kTile;
    out[3] = g.nK;
  }
  return BSM_OK;
}

int bm_head_mode(const Geo& g, int64_t Hm) {
  const int64_t Hi = iter_heads(g);
  const int64_t KVHi = g.KVH;
  return Hm == Hi ? 1 : (Hm == KVHi ? 2 : 0);
}

// Key-list dims of a bool mask: its (Bm, Hm) in the iteration space, the
// iteration rows R (<= 32) and K_round.
constexpr int64_t kMaxListRows = 32;

int key_list_dims(const Geo& g, const bsm_tensor4* mask, Aux& a, int64_t out[4]) {
  if (!mask) return fail(BSM_E_ARG, "mask is NULL");
  int e = check_aux(mask, "mask", g, BSM_BOOL, a);
  if (e) return e;
  const int64_t R = iter_rows(g);
  if (R > kMaxListRows)
    return fail(BSM_E_UNSUPPORTED, "key list needs at most 32 rows per (b, h), got %lld",
                (long long)R);
  out[0] = a.Bm;
  out[1] = a.Hm;
  out[2] = R;
  out[3] = g.Kr;
  return BSM_OK;
}

int check_key_list(const bsm_key_list* kl, const int64_t shp[4]) {
  if (kl->Bm != shp[0] || kl->Hm != shp[1] || kl->R != shp[2] || kl->K != shp[3])
    return fail(BSM_E_SHAPE, "key list dims (%lld,%lld,%lld,%lld) expected (%lld,%lld,%lld,%lld)",
                (long long)kl->Bm, (long long)kl->Hm, (long long)kl->R, (long long)kl->K,
                (long long)shp[0], (long long)shp[1], (long long)shp[2], (long long)shp[3]);
  if (shp[0] * shp[1] > 0 &&
      (!kl->num_keys || (shp[3] > 0 && (!kl->key_indices || !kl->row_bits))))
    return fail(BSM_E_ARG, "key list buffer is NULL");
  if ((uintptr_t)kl->key_indices % 16 || (uintptr_t)kl->row_bits % 16)
    return fail(BSM_E_STRIDE, "key list arrays must be 16-byte aligned");
  return BSM_OK;
}

int check_tensor_qkv(const bsm_tensor4* t, const char* name, int64_t d0, int64_t d1,
                     int64_t d2, int64_t d3, int32_t dtype) {
  if (t->dtype != dtype) return fail(BSM_E_DTYPE, "%s: dtype mismatch", name);
  if (t->size[0] != d0 || t->size[1] != d1 || t->size[2] != d2 || t->size[3] != d3)
    return fail(BSM_E_SHAPE, "%s: sizes (%lld,%lld,%lld,%lld) expected (%lld,%lld,%lld,%lld)",
                name, (long long)t->size[0], (long long)t->size[1], (long long)t->size[2],
                (long long)t->size[3], (long long)d0, (long long)d1, (long long)d2,
                (long long)d3);
  int e = check_strides(t, name, elem_size(dtype));
  if (e) return e;
  if (!t->data && numel(t) > 0) return fail(BSM_E_ARG, "%s: data is NULL", name);
  return BSM_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BSM_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return BSM_OK;
}

}  // namespace

int bsm::set_error(int code, const char* msg) {
  g_err = msg;
  return code;
}

extern "C" {

const char* bsm_last_error(void) { return g_err.c_str(); }

int resolve_dflash_is_causal(int32_t is_causal, int32_t layer_type) {
  const int c = resolve_causal(is_causal, layer_type);
  if (c < 0)
    return fail(BSM_E_ARG, "bad is_causal=%d / layer_type=%d", is_causal, layer_type);
  return c;
}

int block_mask_shape(const bsm_geom* geom, const bsm_dflash* pred, const bsm_tensor4* mask,
                     int64_t out_shape[4]) {
  Geo g;
  int e = check_geom(geom, g);
  if (e) return e;
  if (!out_shape) return fail(BSM_E_ARG, "out_shape is NULL");
  if ((pred == nullptr) == (mask == nullptr))
    return fail(BSM_E_ARG, "exactly one of pred and mask must be given");
  if (pred) {
    DFlashRule r;
    e = check_dflash(pred, g, r);
    if (e) return e;
    return expected_bm(g, pred, nullptr, out_shape);
  }
  if (mask->dtype != BSM_BOOL) return fail(BSM_E_DTYPE, "mask must be BSM_BOOL");
  Aux a;
  e = check_aux(mask, "mask", g, BSM_BOOL, a);
  if (e) return e;
  return expected_bm(g, nullptr, &a, out_shape);
}

int build_block_mask(const bsm_geom* geom, const bsm_dflash* pred, const bsm_tensor4* mask,
                     const bsm_block_mask* out, hipStream_t stream) {
  int64_t shp[4];
  int e = block_mask_shape(geom, pred, mask, shp);
  if (e) return e;
  if (!out) return fail(BSM_E_ARG, "out is NULL");
  if (out->Bm != shp[0] || out->Hm != shp[1] || out->nQm != shp[2] || out->nK != shp[3])
    return fail(BSM_E_SHAPE, "block mask dims (%lld,%lld,%lld,%lld) expected (%lld,%lld,%lld,%lld)",
                (long long)out->Bm, (long long)out->Hm, (long long)out->nQm, (long long)out->nK,
                (long long)shp[0], (long long)shp[1], (long long)shp[2], (long long)shp[3]);
  const int64_t rows = shp[0] * shp[1] * shp[2];
  if (rows > 0 && (!out->kv_num_blocks || !out->full_kv_num_blocks ||
                   (shp[3] > 0 && (!out->kv_indices || !out->full_kv_indices))))
    return fail(BSM_E_ARG, "block mask buffer is NULL");
  if (shp[3] > 65536) return fail(BSM_E_UNSUPPORTED, "more than 65536 key tiles");
  Geo g;
  check_geom(geom, g);
  if (pred) {
    DFlashRule r;
    check_dflash(pred, g, r);
    return hip_status(launch_block_mask_pred(r, g.Sq, g.Sk, shp[2], shp[3], out->kv_num_blocks,
                                             out->kv_indices, out->full_kv_num_blocks,
                                             out->full_kv_indices, stream),
                      "block_mask_pred");
  }
  Aux a;
  check_aux(mask, "mask", g, BSM_BOOL, a);
  DenseMaskView v;
  v.data = reinterpret_cast<const uint8_t*>(a.view.data);
  v.sb = a.view.sb;
  v.sh = a.view.sh;
  v.sq = a.view.sq;
  v.Bm = a.Bm;
  v.Hm = a.Hm;
  v.Qm = a.Qm;
  v.K = g.Kr;
  v.Sk = g.Sk;
  return hip_status(launch_block_mask_dense(v, out->kv_num_blocks, out->kv_indices,
                                            out->full_kv_num_blocks, out->full_kv_indices,
                                            stream),
                    "block_mask_dense");
}

}  // extern "C"

namespace {

// Validation and parameters of a top-k over `bias` (shared by the plain and the
// fused entry points); p.out is left null.
int fill_topk(const bsm_tensor4* bias, const bsm_tensor4* premask, int64_t seqlen_k, int64_t k,
              TopkParams& p) {
  if (!bias) return fail(BSM_E_ARG, "bias is NULL");
  if (k < 0) return fail(BSM_E_ARG, "k must be >= 0 (got %lld)", (long long)k);
  if (seqlen_k < 0) return fail(BSM_E_ARG, "seqlen_k must be >= 0");
  if (bias->dtype != BSM_BF16 && bias->dtype != BSM_F32)
    return fail(BSM_E_DTYPE, "bias must be bf16 or f32");
  int e = check_strides(bias, "bias", elem_size(bias->dtype));
  if (e) return e;
  const int64_t Kr = round_multiple(seqlen_k, kTile);
  if (bias->size[3] != Kr)
    return fail(BSM_E_SHAPE, "bias last dim %lld must be round_multiple(seqlen_k,128)=%lld",
                (long long)bias->size[3], (long long)Kr);
  const int64_t n = numel(bias);
  if (n > 0 && !bias->data) return fail(BSM_E_ARG, "bias data is NULL");
  if (bias->size[0] * bias->size[1] * bias->size[2] > INT32_MAX)
    return fail(BSM_E_UNSUPPORTED, "too many rows");
  p = TopkParams{};
  p.bias = bias->data;
  p.b_sb = bias->size[0] == 1 ? 0 : bias->stride[0];
  p.b_sh = bias->size[1] == 1 ? 0 : bias->stride[1];
  p.b_sq = bias->size[2] == 1 ? 0 : bias->stride[2];
  p.Bb = bias->size[0];
  p.Hb = bias->size[1];
  p.Qb = bias->size[2];
  p.K = Kr;
  p.Sk = seqlen_k;
  p.k = k;
  p.is_bf16 = bias->dtype == BSM_BF16;
  p.pm = nullptr;
  if (premask) {
    if (premask->dtype != BSM_BOOL) return fail(BSM_E_DTYPE, "premask must be BSM_BOOL");
    if (premask->reserved != 0) return fail(BSM_E_ARG, "premask.reserved must be 0");
    for (int i = 0; i < 3; ++i)
      if (premask->size[i] != 1 && premask->size[i] != bias->size[i])
        return fail(BSM_E_SHAPE, "premask dim %d must be 1 or %lld", i, (long long)bias->size[i]);
    if (premask->size[3] != seqlen_k && premask->size[3] != Kr)
      return fail(BSM_E_SHAPE, "premask last dim must be seqlen_k or round_multiple(seqlen_k,128)");
    if (premask->size[3] > 1 && premask->stride[3] != 1)
      return fail(BSM_E_STRIDE, "premask: last dim must be contiguous");
    for (int i = 0; i < 3; ++i) {
      if (premask->stride[i] < 0) return fail(BSM_E_STRIDE, "premask: negative stride");
      if (premask->size[i] > 1 && premask->stride[i] == 0)
        return fail(BSM_E_STRIDE, "premask: stride 0 on dim %d of size > 1", i);
    }
    if (!premask->data && numel(premask) > 0) return fail(BSM_E_ARG, "premask data is NULL");
    p.pm = reinterpret_cast<const uint8_t*>(premask->data);
    p.p_sb = premask->size[0] == 1 ? 0 : premask->stride[0];
    p.p_sh = premask->size[1] == 1 ? 0 : premask->stride[1];
    p.p_sq = premask->size[2] == 1 ? 0 : premask->stride[2];
    p.pK = premask->size[3];
  }
  return BSM_OK;
}

}  // namespace

extern "C" {

int dynamic_topk_mask(const bsm_tensor4* bias, const bsm_tensor4* premask, int64_t seqlen_k,
                      int64_t k, uint8_t* out_mask, hipStream_t stream) {
  TopkParams p;
  int e = fill_topk(bias, premask, seqlen_k, k, p);
  if (e) return e;
  const int64_t n = numel(bias);
  if (n > 0 && !out_mask) return fail(BSM_E_ARG, "out_mask is NULL");
  p.out = out_mask;
  if (n == 0) return BSM_OK;
  return hip_status(launch_topk(p, stream), "dynamic_topk_mask");
}

int dynamic_topk_fused(const bsm_geom* geom, const bsm_tensor4* bias, const bsm_tensor4* premask,
                       int64_t k, uint8_t* out_mask, const bsm_block_mask* out_bm,
                       const bsm_key_list* out_keys, hipStream_t stream) {
  Geo g;
  int e = check_geom(geom, g);
  if (e) return e;
  if (!out_mask && !out_bm && !out_keys) return fail(BSM_E_ARG, "no output requested");
  TopkFusedParams fp{};
  if ((e = fill_topk(bias, premask, g.Sk, k, fp.t))) return e;
  if (!topk_fused_applies(fp.t))
    return fail(BSM_E_UNSUPPORTED, "fused top-k handles rows of up to 16384 bf16 / 8192 f32 keys");
  // the mask this top-k writes: contiguous, the bias's sizes, seen in the
  // attention's iteration space
  bsm_tensor4 mt{};
  mt.data = out_mask ? out_mask : reinterpret_cast<const void*>((uintptr_t)256);
  mt.dtype = BSM_BOOL;
  for (int i = 0; i < 4; ++i) mt.size[i] = bias->size[i];
  mt.stride[3] = 1;
  mt.stride[2] = mt.size[3];
  mt.stride[1] = mt.size[2] * mt.stride[2];
  mt.stride[0] = mt.size[1] * mt.stride[1];
  Aux a;
  if ((e = check_aux(&mt, "top-k mask", g, BSM_BOOL, a))) return e;
  if (a.Qm > 32)
    return fail(BSM_E_UNSUPPORTED, "fused top-k needs at most 32 distinct mask rows per (b, h)");
  if (out_mask && (uintptr_t)out_mask % 16) return fail(BSM_E_STRIDE, "out_mask not 16-byte aligned");
  fp.t.out = out_mask;
  fp.m_sb = a.view.sb;
  fp.m_sh = a.view.sh;
  fp.m_sq = a.view.q_bcast ? 0 : a.view.sq;
  fp.Bm = a.Bm;
  fp.Hm = a.Hm;
  fp.Qm = (int32_t)a.Qm;
  fp.R = (int32_t)iter_rows(g);
  if (out_bm) {
    int64_t shp[4];
    expected_bm(g, nullptr, &a, shp);
    if (out_bm->Bm != shp[0] || out_bm->Hm != shp[1] || out_bm->nQm != shp[2] ||
        out_bm->nK != shp[3])
      return fail(BSM_E_SHAPE, "block mask dims do not match the top-k mask");
    if (shp[0] * shp[1] > 0 && (!out_bm->kv_num_blocks || !out_bm->full_kv_num_blocks ||
                                (shp[3] > 0 && (!out_bm->kv_indices || !out_bm->full_kv_indices))))
      return fail(BSM_E_ARG, "block mask buffer is NULL");
    fp.kv_num = out_bm->kv_num_blocks;
    fp.kv_idx = out_bm->kv_indices;
    fp.full_num = out_bm->full_kv_num_blocks;
    fp.full_idx = out_bm->full_kv_indices;
    fp.nK = shp[3];
  }
  if (out_keys) {
    int64_t shp[4];
    Aux ka;
    if ((e = key_list_dims(g, &mt, ka, shp))) return e;
    if ((e = check_key_list(out_keys, shp))) return e;
    fp.l_num = out_keys->num_keys;
    fp.l_idx = out_keys->key_indices;
    fp.l_bits = out_keys->row_bits;
  }
  if (fp.Qm == 0) return BSM_OK;  // no rows
  return hip_status(launch_topk_fused(fp, stream), "dynamic_topk_fused");
}

int key_list_shape(const bsm_geom* geom, const bsm_tensor4* mask, int64_t out_shape[4]) {
  Geo g;
  int e = check_geom(geom, g);
  if (e) return e;
  if (!out_shape) return fail(BSM_E_ARG, "out_shape is NULL");
  Aux a;
  return key_list_dims(g, mask, a, out_shape);
}

int build_key_list(const bsm_geom* geom, const bsm_tensor4* mask, const bsm_key_list* out,
                   hipStream_t stream) {
  Geo g;
  int e = check_geom(geom, g);
  if (e) return e;
  if (!out) return fail(BSM_E_ARG, "out is NULL");
  Aux a;
  int64_t shp[4];
  if ((e = key_list_dims(g, mask, a, shp))) return e;
  if ((e = check_key_list(out, shp))) return e;
  if (shp[0] * shp[1] > INT32_MAX) return fail(BSM_E_UNSUPPORTED, "too many key lists");
  KeyListParams p{};
  p.mask = reinterpret_cast<const uint8_t*>(a.view.data);
  p.sb = a.view.sb;
  p.sh = a.view.sh;
  p.sq = a.view.sq;
  p.Bm = a.Bm;
  p.Hm = a.Hm;
  p.K = g.Kr;
  p.Sk = g.Sk;
  p.R = (int32_t)shp[2];
  p.Qm = (int32_t)a.Qm;
  p.num = out->num_keys;
  p.idx = out->key_indices;
  p.bits = out->row_bits;
  return hip_status(launch_key_list(p, stream), "build_key_list");
}

int dflash_dense_mask(const bsm_geom* geom, const bsm_dflash* pred, uint8_t* out_mask,
                      hipStream_t stream) {
  Geo g;
  int e = check_geom(geom, g);
  if (e) return e;
  if (!pred) return fail(BSM_E_ARG, "pred is NULL");
  DFlashRule r;
  e = check_dflash(pred, g, r);
  if (e) return e;
  if (g.Sq * g.Kr > 0 && !out_mask) return fail(BSM_E_ARG, "out_mask is NULL");
  if ((uintptr_t)out_mask % 16) return fail(BSM_E_STRIDE, "out_mask not 16-byte aligned");
  return hip_status(launch_dflash_dense(r, g.Sq, g.Sk, g.Kr, out_mask, stream), "dflash_dense");
}

}  // extern "C"

namespace {

// ---- shared by the attention forward and backward

struct AttnInputs {
  DFlashRule rule{};
  Aux mk{}, bs{};
  BlockMaskView bmv{};
};

// Mask source, bias and block mask of an attention call.
int check_attn_aux(const Geo& g, int32_t dt, const bsm_dflash* pred, const bsm_tensor4* mask,
                   const bsm_tensor4* bias, const bsm_block_mask* bm, float softmax_scale,
                   AttnInputs& in) {
  int e;
  if (pred && mask) return fail(BSM_E_ARG, "give at most one of pred and mask");
  if (std::isnan(softmax_scale)) return fail(BSM_E_ARG, "softmax_scale is NaN");
  if (pred && (e = check_dflash(pred, g, in.rule))) return e;
  if (mask && (e = check_aux(mask, "mask", g, BSM_BOOL, in.mk))) return e;
  if (bias && (e = check_aux(bias, "bias", g, dt, in.bs))) return e;
  if (bm) {
    if (!pred && !mask) return fail(BSM_E_ARG, "a block mask needs pred or mask");
    int64_t shp[4];
    expected_bm(g, pred, &in.mk, shp);
    if (bm->Bm != shp[0] || bm->Hm != shp[1] || bm->nQm != shp[2] || bm->nK != shp[3])
      return fail(BSM_E_SHAPE, "block mask dims (%lld,%lld,%lld,%lld) do not match this call "
                  "(%lld,%lld,%lld,%lld)", (long long)bm->Bm, (long long)bm->Hm,
                  (long long)bm->nQm, (long long)bm->nK, (long long)shp[0], (long long)shp[1],
                  (long long)shp[2], (long long)shp[3]);
    if (shp[0] * shp[1] * shp[2] > 0 &&
        (!bm->kv_num_blocks || !bm->full_kv_num_blocks ||
         (shp[3] > 0 && (!bm->kv_indices || !bm->full_kv_indices))))
      return fail(BSM_E_ARG, "block mask buffer is NULL");
    in.bmv.kv_num = bm->kv_num_blocks;
    in.bmv.kv_idx = bm->kv_indices;
    in.bmv.full_num = bm->full_kv_num_blocks;
    in.bmv.full_idx = bm->full_kv_indices;
    in.bmv.Bm = bm->Bm;
    in.bmv.Hm = bm->Hm;
    in.bmv.nQm = bm->nQm;
    in.bmv.nK = bm->nK;
    in.bmv.h_mode = bm_head_mode(g, bm->Hm);
  }
  return BSM_OK;
}

// (b, q, h) element strides of a (B, Sq, H, D) tensor in the iteration space:
// under the swap, head kvh*G + i of a KV group is row i of KV head kvh.
void qlike_strides(const Geo& g, const int64_t* st, int64_t& sb, int64_t& sq, int64_t& sh) {
  sb = st[0];
  if (!g.swap) {
    sq = st[1];
    sh = st[2];
  } else {
    sq = st[2];
    sh = g.G * st[2];
  }
}

void fill_params(const Geo& g, const bsm_tensor4& q, const bsm_tensor4& k,
                 const bsm_tensor4& v, void* o, const int64_t* o_stride, float* lse,
                 float softmax_scale, bool has_pred, bool has_mask, bool has_bias,
                 bool has_bm, const AttnInputs& in, AttnParams& p) {
  p = AttnParams{};
  p.q = q.data;
  p.k = k.data;
  p.v = v.data;
  p.o = o;
  p.lse = lse;
  p.k_sb = k.stride[0];
  p.k_sk = k.stride[1];
  p.k_sh = k.stride[2];
  p.v_sb = v.stride[0];
  p.v_sk = v.stride[1];
  p.v_sh = v.stride[2];
  p.B = (int32_t)g.B;
  p.Sk = (int32_t)g.Sk;
  p.nK = (int32_t)g.nK;
  qlike_strides(g, q.stride, p.q_sb, p.q_sq, p.q_sh);
  if (o_stride) qlike_strides(g, o_stride, p.o_sb, p.o_sq, p.o_sh);
  p.KVH = (int32_t)g.KVH;
  if (!g.swap) {
    p.lse_sb = g.H * g.Sq;
    p.lse_sh = g.Sq;
    p.lse_sq = 1;
    p.H = (int32_t)g.H;
    p.G = (int32_t)g.G;
    p.Sq = (int32_t)g.Sq;
  } else {
    p.lse_sb = g.H;
    p.lse_sh = g.G;
    p.lse_sq = 1;
    p.H = (int32_t)g.KVH;
    p.G = 1;
    p.Sq = (int32_t)g.G;
  }
  p.nQ = (p.Sq + kTile - 1) / kTile;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)g.D);
  p.scale_log2 = scale * 1.4426950408889634f;
  p.mask_kind = has_pred ? 1 : (has_mask ? 2 : 0);
  p.pred_row0 = g.swap && has_pred;
  p.rule = in.rule;
  p.mask = in.mk.view;
  p.bias = in.bs.view;
  p.has_bias = has_bias;
  p.has_bm = has_bm;
  p.bm = in.bmv;
}

// Float workspace of the backward: Delta (B*H*Sq), then the dbias accumulator
// (the bias's element count) when dbias is requested; each part 256-byte aligned.
int64_t bwd_delta_bytes(const Geo& g) { return round_multiple(g.B * g.H * g.Sq * 4, 256); }
int64_t bwd_workspace_bytes(const Geo& g, const bsm_tensor4* bias, const bsm_tensor4* dbias) {
  int64_t n = bwd_delta_bytes(g);
  if (bias && dbias) n += round_multiple(numel(bias) * 4, 256);
  return n;
}

}  // namespace

namespace {

// Short query blocks on the packed / split kernel: the G heads of a KV group
// share a workgroup when their rows fit (G * Sq <= 64) and their block-mask
// row is shared; a launch with fewer than 384 workgroups splits each tile list
// into up to 32 parts of at least ~4 tiles, given a workspace for the partials.
struct GroupPlan {
  int pack, splits;
  int64_t ws_o_bytes, ws_bytes;
};

GroupPlan group_plan(const AttnParams& p, int D) {
  GroupPlan g{1, 1, 0, 0};
  if (p.G > 1 && (int64_t)p.Sq * p.G <= 64 && !(p.has_bm && p.bm.h_mode == 1)) g.pack = p.G;
  const int64_t base = (int64_t)p.B * (p.H / g.pack);
  if (base > 0 && base < 384) {
    int64_t S = (512 + base - 1) / base;
    const int64_t cap = p.nK / 4 > 1 ? p.nK / 4 : 1;
    S = S < cap ? S : cap;
    g.splits = (int)(S < 32 ? S : 32);
  }
  if (g.splits > 1) {
    const int64_t rows = (int64_t)g.splits * p.B * p.H * p.Sq;
    g.ws_o_bytes = round_multiple(rows * D * 4, 256);
    g.ws_bytes = g.ws_o_bytes + round_multiple(rows * 2 * 4, 256);
  }
  return g;
}

// Validation and parameters shared by masked_attn_fwd and its workspace query.
// Sets `empty` when there is nothing to compute.
int prepare_fwd(const bsm_geom* geom, const bsm_attn_args* a, Geo& g, AttnParams& p,
                bool& empty) {
  int e = check_geom(geom, g);
  if (e) return e;
  if (!a) return fail(BSM_E_ARG, "args is NULL");
  if (a->reserved != 0) return fail(BSM_E_ARG, "args.reserved must be 0");
  if (g.D != 64 && g.D != 128)
    return fail(BSM_E_UNSUPPORTED, "head dim %lld not supported (64 or 128)", (long long)g.D);
  const int32_t dt = a->q.dtype;
  if (dt != BSM_BF16 && dt != BSM_F32) return fail(BSM_E_DTYPE, "q must be bf16 or f32");
  if ((e = check_tensor_qkv(&a->q, "q", g.B, g.Sq, g.H, g.D, dt))) return e;
  if ((e = check_tensor_qkv(&a->k, "k", g.B, g.Sk, g.KVH, g.D, dt))) return e;
  if ((e = check_tensor_qkv(&a->v, "v", g.B, g.Sk, g.KVH, g.D, dt))) return e;
  {
    bsm_tensor4 o{};
    o.data = a->o;
    o.dtype = dt;
    o.size[0] = g.B;
    o.size[1] = g.Sq;
    o.size[2] = g.H;
    o.size[3] = g.D;
    for (int i = 0; i < 4; ++i) o.stride[i] = a->o_stride[i];
    if ((e = check_tensor_qkv(&o, "o", g.B, g.Sq, g.H, g.D, dt))) return e;
  }
  AttnInputs in;
  if ((e = check_attn_aux(g, dt, a->pred, a->mask, a->bias, a->bm, a->softmax_scale, in)))
    return e;
  int64_t klist[4] = {0, 0, 0, 0};
  if (a->keys) {
    if (!a->mask || a->bm)
      return fail(BSM_E_ARG, "a key list needs the mask it was built from and no block mask");
    if (dt != BSM_BF16) return fail(BSM_E_UNSUPPORTED, "key-gather attention is bf16 only");
    Aux ka;
    if ((e = key_list_dims(g, a->mask, ka, klist))) return e;
    if ((e = check_key_list(a->keys, klist))) return e;
  }
  if (a->workspace_bytes < 0) return fail(BSM_E_ARG, "workspace_bytes < 0");
  if (a->workspace_bytes > 0 && (!a->workspace || (uintptr_t)a->workspace % 256))
    return fail(BSM_E_ARG, "workspace is NULL or not 256-byte aligned");
  empty = g.B == 0 || g.Sq == 0;
  if (empty) return BSM_OK;
  fill_params(g, a->q, a->k, a->v, a->o, a->o_stride, a->lse, a->softmax_scale, a->pred,
              a->mask, a->bias, a->bm, in, p);
  if (a->keys) {
    p.gather = 1;
    p.keys.num = a->keys->num_keys;
    p.keys.idx = a->keys->key_indices;
    p.keys.bits = a->keys->row_bits;
    p.keys.Bm = klist[0];
    p.keys.Hm = klist[1];
    p.keys.K = klist[3];
    p.keys.h_mode = bm_head_mode(g, klist[1]);
    if (!short_query_applies(p, (int)g.D))
      return fail(BSM_E_UNSUPPORTED, "key-gather attention: K/V too large for 32-bit offsets");
  }
  return BSM_OK;
}

}  // namespace

extern "C" {

int attn_fwd_workspace_size(const bsm_geom* geom, const bsm_attn_args* a, int64_t* bytes) {
  if (!bytes) return fail(BSM_E_ARG, "bytes is NULL");
  Geo g;
  AttnParams p{};
  bool empty = false;
  int e = prepare_fwd(geom, a, g, p, empty);
  if (e) return e;
  *bytes = 0;
  if (empty || p.gather || a->q.dtype != BSM_BF16) return BSM_OK;
  if (short_query_applies(p, (int)g.D))
    *bytes = group_plan(p, (int)g.D).ws_bytes;
  else if (attn_v2_applies(p, (int)g.D) && staged_aux_applies(p))
    *bytes = staged_aux_bytes(p);
  return BSM_OK;
}

int masked_attn_fwd(const bsm_geom* geom, const bsm_attn_args* a, hipStream_t stream) {
  Geo g;
  AttnParams p{};
  bool empty = false;
  int e = prepare_fwd(geom, a, g, p, empty);
  if (e) return e;
  if (empty) return BSM_OK;
  const int D = (int)g.D;
  if (p.gather) return hip_status(launch_attn_gather(p, D, stream), "masked_attn_fwd");
  hipError_t he;
  if (a->q.dtype == BSM_BF16) {
    if (short_query_applies(p, D)) {
      const GroupPlan gp = group_plan(p, D);
      p.pack = gp.pack;
      p.splits = gp.splits > 1 && a->workspace_bytes >= gp.ws_bytes ? gp.splits : 1;
      if (p.splits > 1) {
        char* ws = static_cast<char*>(a->workspace);
        p.ws_o = reinterpret_cast<float*>(ws);
        p.ws_ml = reinterpret_cast<float*>(ws + gp.ws_o_bytes);
      }
      he = launch_attn_group(p, D, stream);
    } else if (attn_v2_applies(p, D)) {
      he = hipSuccess;
      if (staged_aux_applies(p) && a->workspace_bytes >= staged_aux_bytes(p))
        he = launch_aux_combine(p, a->workspace, stream);
      if (he == hipSuccess) he = launch_attn_bf16_v2(p, D, stream);
    } else if (attn_h1_applies(p, D)) {
      he = launch_attn_bf16_h1(p, D, stream);
    } else {
      he = launch_attn_bf16(p, D, stream);
    }
  } else {
    he = launch_attn_f32(p, D, stream);
  }
  return hip_status(he, "masked_attn_fwd");
}

}  // extern "C"

namespace {

// Kernel parameters of a padded backward call (workspace pointers aside).
void bwd_params(const Geo& g, const bsm_attn_bwd_args* a, const AttnInputs& in,
                AttnBwdParams& p) {
  p = AttnBwdParams{};
  fill_params(g, a->q, a->k, a->v, const_cast<void*>(a->o.data), a->o.stride,
              const_cast<float*>(a->lse),
              a->softmax_scale, a->pred, a->mask, a->bias, a->bm, in, p.f);
  p.scale = p.f.scale_log2 / 1.4426950408889634f;
  p.dout = a->dout.data;
  qlike_strides(g, a->dout.stride, p.do_sb, p.do_sq, p.do_sh);
  p.dq = const_cast<void*>(a->dq.data);
  qlike_strides(g, a->dq.stride, p.dq_sb, p.dq_sq, p.dq_sh);
  p.dk = const_cast<void*>(a->dk.data);
  p.dk_sb = a->dk.stride[0];
  p.dk_sk = a->dk.stride[1];
  p.dk_sh = a->dk.stride[2];
  p.dv = const_cast<void*>(a->dv.data);
  p.dv_sb = a->dv.stride[0];
  p.dv_sk = a->dv.stride[1];
  p.dv_sh = a->dv.stride[2];
}

// Bytes of the folded mask / bias rows the matrix-core backward reads when
// both broadcast over queries (the forward's staged rows), or 0: bf16, D =
// 128, and the pipelined dQ kernel (K / V offsets within 32 bits).
int64_t bwd_staged_bytes(const AttnBwdParams& p, int64_t D, int32_t dt) {
  const AttnParams& f = p.f;
  if (dt != BSM_BF16 || D != 128 || !attn_bwd_mfma_applies(p, 128) || !staged_aux_applies(f))
    return 0;
  if ((int64_t)f.Sk * f.k_sk * 2 >= ((int64_t)1 << 31) ||
      (int64_t)f.Sk * f.v_sk * 2 >= ((int64_t)1 << 31))
    return 0;
  return staged_aux_bytes(f);
}

}  // namespace

extern "C" {

int attn_bwd_workspace_size(const bsm_geom* geom, const bsm_attn_bwd_args* a, int64_t* bytes) {
  Geo g;
  int e = check_geom(geom, g);
  if (e) return e;
  if (!a || !bytes) return fail(BSM_E_ARG, "args or bytes is NULL");
  int64_t n = bwd_workspace_bytes(g, a->bias, a->dbias);
  if ((a->mask || a->bias) && g.B > 0) {
    AttnInputs in;
    if ((e = check_attn_aux(g, a->q.dtype, a->pred, a->mask, a->bias, a->bm, a->softmax_scale,
                            in)))
      return e;
    AttnBwdParams p;
    bwd_params(g, a, in, p);
    n += bwd_staged_bytes(p, g.D, a->q.dtype);
  }
  *bytes = n;
  return BSM_OK;
}

int masked_attn_bwd(const bsm_geom* geom, const bsm_attn_bwd_args* a, hipStream_t stream) {
  Geo g;
  int e = check_geom(geom, g);
  if (e) return e;
  if (!a) return fail(BSM_E_ARG, "args is NULL");
  if (a->reserved != 0) return fail(BSM_E_ARG, "args.reserved must be 0");
  if (g.D != 64 && g.D != 128)
    return fail(BSM_E_UNSUPPORTED, "head dim %lld not supported (64 or 128)", (long long)g.D);
  const int32_t dt = a->q.dtype;
  if (dt != BSM_BF16 && dt != BSM_F32) return fail(BSM_E_DTYPE, "q must be bf16 or f32");
  if ((e = check_tensor_qkv(&a->q, "q", g.B, g.Sq, g.H, g.D, dt))) return e;
  if ((e = check_tensor_qkv(&a->k, "k", g.B, g.Sk, g.KVH, g.D, dt))) return e;
  if ((e = check_tensor_qkv(&a->v, "v", g.B, g.Sk, g.KVH, g.D, dt))) return e;
  if ((e = check_tensor_qkv(&a->o, "o", g.B, g.Sq, g.H, g.D, dt))) return e;
  if ((e = check_tensor_qkv(&a->dout, "dout", g.B, g.Sq, g.H, g.D, dt))) return e;
  if ((e = check_tensor_qkv(&a->dq, "dq", g.B, g.Sq, g.H, g.D, dt))) return e;
  if ((e = check_tensor_qkv(&a->dk, "dk", g.B, g.Sk, g.KVH, g.D, dt))) return e;
  if ((e = check_tensor_qkv(&a->dv, "dv", g.B, g.Sk, g.KVH, g.D, dt))) return e;
  if (!a->lse && g.B * g.H * g.Sq > 0) return fail(BSM_E_ARG, "lse is NULL");
  AttnInputs in;
  if ((e = check_attn_aux(g, dt, a->pred, a->mask, a->bias, a->bm, a->softmax_scale, in)))
    return e;
  if (a->dbias) {
    if (!a->bias) return fail(BSM_E_ARG, "dbias needs bias");
    const bsm_tensor4* b = a->bias;
    const bsm_tensor4* d = a->dbias;
    for (int i = 0; i < 4; ++i)
      if (d->size[i] != b->size[i]) return fail(BSM_E_SHAPE, "dbias: sizes must equal bias's");
    if (d->dtype != dt) return fail(BSM_E_DTYPE, "dbias: dtype must equal bias's");
    if ((e = check_strides(d, "dbias", elem_size(dt)))) return e;
    if (!d->data && numel(d) > 0) return fail(BSM_E_ARG, "dbias: data is NULL");
  }
  AttnBwdParams p;
  bwd_params(g, a, in, p);
  const int64_t staged = g.B > 0 ? bwd_staged_bytes(p, g.D, dt) : 0;
  const int64_t need = bwd_workspace_bytes(g, a->bias, a->dbias) + staged;
  if (a->workspace_bytes < need)
    return fail(BSM_E_ARG, "workspace of %lld bytes, %lld needed", (long long)a->workspace_bytes,
                (long long)need);
  if (need > 0 && (!a->workspace || (uintptr_t)a->workspace % 256))
    return fail(BSM_E_ARG, "workspace is NULL or not 256-byte aligned");
  if (g.B == 0) return BSM_OK;

  char* ws = static_cast<char*>(a->workspace);
  p.delta = reinterpret_cast<float*>(ws);
  p.delta_sb = (int64_t)p.f.H * p.f.Sq;
  p.delta_sh = p.f.Sq;
  DbiasOut dout{};
  hipError_t he = hipSuccess;
  if (a->dbias) {
    float* acc = reinterpret_cast<float*>(ws + bwd_delta_bytes(g));
    // the accumulator: contiguous float with the bias's sizes, seen like the bias
    bsm_tensor4 t{};
    t.data = acc;
    t.dtype = BSM_F32;
    for (int i = 0; i < 4; ++i) t.size[i] = a->bias->size[i];
    t.stride[3] = 1;
    t.stride[2] = t.size[3];
    t.stride[1] = t.size[2] * t.stride[2];
    t.stride[0] = t.size[1] * t.stride[1];
    Aux av;
    if ((e = check_aux(&t, "dbias workspace", g, BSM_F32, av))) return e;
    p.dbias_acc = acc;
    p.dbias = av.view;
    he = launch_fill_zero(acc, numel(&t), stream);
    if (he != hipSuccess) return hip_status(he, "masked_attn_bwd");
    dout.acc = acc;
    dout.out = const_cast<void*>(a->dbias->data);
    dout.n0 = t.size[0];
    dout.n1 = t.size[1];
    dout.n2 = t.size[2];
    dout.K = t.size[3];
    dout.Sk = g.Sk;
    dout.s0 = a->dbias->size[0] == 1 ? 0 : a->dbias->stride[0];
    dout.s1 = a->dbias->size[1] == 1 ? 0 : a->dbias->stride[1];
    dout.s2 = a->dbias->size[2] == 1 ? 0 : a->dbias->stride[2];
    dout.is_bf16 = dt == BSM_BF16;
  }
  if (staged > 0) {
    // the folded rows go after Delta and the dbias accumulator
    he = launch_aux_combine(p.f, ws + bwd_workspace_bytes(g, a->bias, a->dbias), stream);
    if (he != hipSuccess) return hip_status(he, "masked_attn_bwd");
  }
  he = launch_attn_bwd(p, (int)g.D, dt == BSM_BF16, stream);
  if (he == hipSuccess && a->dbias) he = launch_dbias_out(dout, stream);
  return hip_status(he, "masked_attn_bwd");
}

}  // extern "C"

// ---- packed variable-length sequences

namespace {

struct VarlenInfo {
  int64_t B, maxSq, maxSk, nQ, nK;
};

int check_varlen(const bsm_varlen* vl, VarlenInfo& vi) {
  if (!vl) return fail(BSM_E_ARG, "varlen is NULL");
  if (vl->num_seqs < 0 || vl->H < 1 || vl->KVH < 1 || vl->D < 1 || vl->total_q < 0 ||
      vl->total_k < 0)
    return fail(BSM_E_SHAPE, "bad varlen sizes");
  if (vl->H % vl->KVH)
    return fail(BSM_E_SHAPE, "H=%lld is not a multiple of KVH=%lld", (long long)vl->H,
                (long long)vl->KVH);
  if (vl->num_seqs > 65535 || vl->H > 65535 || vl->total_q > INT32_MAX / 2 ||
      vl->total_k > INT32_MAX / 2)
    return fail(BSM_E_UNSUPPORTED, "varlen sizes beyond the library's size limits");
  const int64_t B = vl->num_seqs;
  if (!vl->cu_seqlens_q_host || !vl->cu_seqlens_k_host || !vl->cu_seqlens_q ||
      !vl->cu_seqlens_k)
    return fail(BSM_E_ARG, "cu_seqlens arrays (device and host) are required");
  const int32_t* cq = vl->cu_seqlens_q_host;
  const int32_t* ck = vl->cu_seqlens_k_host;
  if (cq[0] != 0 || ck[0] != 0) return fail(BSM_E_ARG, "cu_seqlens must start at 0");
  vi.B = B;
  vi.maxSq = vi.maxSk = 0;
  for (int64_t b = 0; b < B; ++b) {
    const int64_t sq = (int64_t)cq[b + 1] - cq[b];
    const int64_t sk = (int64_t)ck[b + 1] - ck[b];
    if (sq < 0 || sk < 0) return fail(BSM_E_ARG, "cu_seqlens must be nondecreasing");
    vi.maxSq = sq > vi.maxSq ? sq : vi.maxSq;
    vi.maxSk = sk > vi.maxSk ? sk : vi.maxSk;
  }
  if (cq[B] != vl->total_q || ck[B] != vl->total_k)
    return fail(BSM_E_SHAPE, "cu_seqlens end at %d / %d, total_q / total_k are %lld / %lld",
                cq[B], ck[B], (long long)vl->total_q, (long long)vl->total_k);
  vi.nQ = (vi.maxSq + kTile - 1) / kTile;
  vi.nK = (vi.maxSk + kTile - 1) / kTile;
  return BSM_OK;
}

// Per-sequence DFlash rule: the shared fields, C and (when 0) S left to the
// kernels; every sequence must have a DFlash layout.
int check_dflash_varlen(const bsm_dflash* d, const bsm_varlen* vl, DFlashRule& r) {
  if (d->ctx_len != 0 || d->num_blocks != 0)
    return fail(BSM_E_ARG, "varlen DFlash: ctx_len and num_blocks must be 0 (per sequence)");
  if (d->block_size < 1 || d->ctx_per_block < 0)
    return fail(BSM_E_ARG, "bad DFlash block_size / ctx_per_block");
  const int c = resolve_causal(d->is_causal, d->layer_type);
  if (c < 0)
    return fail(BSM_E_ARG, "bad is_causal=%d / layer_type=%d", d->is_causal, d->layer_type);
  if (d->layer_type == 1 && d->sliding_window < 1)
    return fail(BSM_E_ARG, "sliding layer needs sliding_window >= 1");
  const int32_t* cq = vl->cu_seqlens_q_host;
  const int32_t* ck = vl->cu_seqlens_k_host;
  for (int64_t b = 0; b < vl->num_seqs; ++b) {
    const int64_t sq = (int64_t)cq[b + 1] - cq[b];
    const int64_t sk = (int64_t)ck[b + 1] - ck[b];
    if (sq % d->block_size || sk < sq)
      return fail(BSM_E_SHAPE, "sequence %lld (%lld queries, %lld keys) is not a DFlash layout "
                  "with blocks of %lld", (long long)b, (long long)sq, (long long)sk,
                  (long long)d->block_size);
    const int64_t nb = sq / d->block_size;
    if (d->ctx_per_block == 0 && nb > 0 && (sk - sq) % nb)
      return fail(BSM_E_SHAPE, "sequence %lld: ctx_per_block=0 needs its context (%lld) to be a "
                  "multiple of its %lld blocks", (long long)b, (long long)(sk - sq),
                  (long long)nb);
  }
  r.C = 0;
  r.bs = d->block_size;
  r.S = d->ctx_per_block;
  r.e0 = d->ctx_end_offset;
  r.W = d->layer_type == 1 ? d->sliding_window : 0;
  r.causal = c;
  r.pad = 0;
  return BSM_OK;
}

int check_copy(const void* src, int64_t src_stride, void* dst, int64_t dst_stride,
               int64_t row_bytes, const int32_t* idx, int64_t n) {
  if (n < 0 || row_bytes < 0) return fail(BSM_E_ARG, "negative row count or size");
  if (n == 0 || row_bytes == 0) return BSM_OK;
  if (!src || !dst || !idx) return fail(BSM_E_ARG, "src, dst or indices is NULL");
  if (row_bytes % 16 || src_stride % 16 || dst_stride % 16 || (uintptr_t)src % 16 ||
      (uintptr_t)dst % 16)
    return fail(BSM_E_STRIDE, "rows, strides and pointers must be multiples of 16 bytes");
  if (src_stride < row_bytes || dst_stride < row_bytes)
    return fail(BSM_E_STRIDE, "row stride smaller than the row");
  return BSM_OK;
}

}  // namespace

extern "C" {

int block_mask_varlen_shape(const bsm_varlen* vl, const bsm_dflash* pred, int64_t out_shape[4]) {
  VarlenInfo vi;
  int e = check_varlen(vl, vi);
  if (e) return e;
  if (!pred || !out_shape) return fail(BSM_E_ARG, "pred or out_shape is NULL");
  DFlashRule r;
  if ((e = check_dflash_varlen(pred, vl, r))) return e;
  if (vi.nK > 65536) return fail(BSM_E_UNSUPPORTED, "more than 65536 key tiles");
  out_shape[0] = vi.B;
  out_shape[1] = 1;
  out_shape[2] = vi.nQ;
  out_shape[3] = vi.nK;
  return BSM_OK;
}

int build_block_mask_varlen(const bsm_varlen* vl, const bsm_dflash* pred,
                            const bsm_block_mask* out, hipStream_t stream) {
  int64_t shp[4];
  int e = block_mask_varlen_shape(vl, pred, shp);
  if (e) return e;
  if (!out) return fail(BSM_E_ARG, "out is NULL");
  if (out->Bm != shp[0] || out->Hm != shp[1] || out->nQm != shp[2] || out->nK != shp[3])
    return fail(BSM_E_SHAPE, "block mask dims (%lld,%lld,%lld,%lld) expected (%lld,%lld,%lld,%lld)",
                (long long)out->Bm, (long long)out->Hm, (long long)out->nQm, (long long)out->nK,
                (long long)shp[0], (long long)shp[1], (long long)shp[2], (long long)shp[3]);
  if (shp[0] * shp[2] > 0 && (!out->kv_num_blocks || !out->full_kv_num_blocks ||
                              (shp[3] > 0 && (!out->kv_indices || !out->full_kv_indices))))
    return fail(BSM_E_ARG, "block mask buffer is NULL");
  DFlashRule r;
  check_dflash_varlen(pred, vl, r);
  return hip_status(launch_block_mask_pred_varlen(r, vl->cu_seqlens_q, vl->cu_seqlens_k, shp[0],
                                                  shp[2], shp[3], out->kv_num_blocks,
                                                  out->kv_indices, out->full_kv_num_blocks,
                                                  out->full_kv_indices, stream),
                    "build_block_mask_varlen");
}

}  // extern "C"

namespace {

// Heaviest-first order of a packed launch's (sequence, query tile) items, from
// the host copies of cu_seqlens: the cost of an item is the number of key
// tiles its rows see -- under the DFlash predicate the tiles spanned by the
// context interval of its first row up to the context end of its last row,
// plus those of its draft keys (the rows' intervals are monotone in the row);
// without a mask, all of the sequence's key tiles. The order is an estimate
// only: every item is still computed from the block mask or the predicate.
// Leaves n = 0 (the kernel's own order) past kMaxOrder items or 64 sequences.
void varlen_order(const bsm_varlen* vl, const VarlenInfo& vi, const DFlashRule* rule,
                  WorkOrder& ord) {
  ord.n = 0;
  if (vi.B > 64 || vi.nQ > 1024) return;
  std::vector<std::pair<int64_t, int>> items;  // (-cost, b << 10 | qt)
  for (int64_t b = 0; b < vi.B; ++b) {
    const int64_t Sq = vl->cu_seqlens_q_host[b + 1] - vl->cu_seqlens_q_host[b];
    const int64_t Sk = vl->cu_seqlens_k_host[b + 1] - vl->cu_seqlens_k_host[b];
    const int64_t nQ = (Sq + kTile - 1) / kTile;
    const int64_t nK = (Sk + kTile - 1) / kTile;
    DFlashRule r{};
    if (rule) {  // the sequence's own geometry, as the kernels complete it
      r = *rule;
      r.C = Sk - Sq;
      const int64_t nb = Sq / r.bs;
      if (r.S == 0) r.S = nb > 0 ? r.C / nb : 0;
    }
    for (int64_t qt = 0; qt < nQ; ++qt) {
      int64_t cost = nK;
      if (rule) {
        const RowIv a = dflash_row(r, qt * kTile);
        const RowIv z = dflash_row(r, std::min(Sq, (qt + 1) * kTile) - 1);
        auto span = [](int64_t lo, int64_t hi) {
          return hi > lo ? (hi - 1) / kTile - lo / kTile + 1 : (int64_t)0;
        };
        cost = span(a.lo1, std::max(a.hi1, z.hi1)) + span(a.lo2, z.hi2);
      }
      items.emplace_back(-cost, (int)((b << 10) | qt));
    }
  }
  if ((int64_t)items.size() > kMaxOrder) return;
  std::stable_sort(items.begin(), items.end(),
                   [](const std::pair<int64_t, int>& x, const std::pair<int64_t, int>& y) {
                     return x.first < y.first;
                   });
  for (size_t i = 0; i < items.size(); ++i) ord.item[i] = (uint16_t)items[i].second;
  ord.n = (int32_t)items.size();
}

// (sequence, key tile) items of the dK / dV kernel over packed sequences,
// heaviest first: a key tile's cost is the number of the sequence's query
// tiles whose rows keep any of its keys (every one without a DFlash rule).
void varlen_key_order(const bsm_varlen* vl, const VarlenInfo& vi, const DFlashRule* rule,
                      WorkOrder& ord) {
  ord.n = 0;
  if (vi.B > 64 || vi.nK > 1024) return;
  std::vector<std::pair<int64_t, int>> items;  // (-cost, b << 10 | kt)
  for (int64_t b = 0; b < vi.B; ++b) {
    const int64_t Sq = vl->cu_seqlens_q_host[b + 1] - vl->cu_seqlens_q_host[b];
    const int64_t Sk = vl->cu_seqlens_k_host[b + 1] - vl->cu_seqlens_k_host[b];
    const int64_t nQ = (Sq + kTile - 1) / kTile;
    const int64_t nK = (Sk + kTile - 1) / kTile;
    std::vector<int64_t> cost(nK, rule ? 0 : nQ);
    if (rule) {
      DFlashRule r = *rule;  // the sequence's own geometry, as the kernels complete it
      r.C = Sk - Sq;
      const int64_t nb = Sq / r.bs;
      if (r.S == 0) r.S = nb > 0 ? r.C / nb : 0;
      auto add = [&](int64_t lo, int64_t hi) {
        hi = std::min(hi, Sk);
        for (int64_t kt = lo / kTile; hi > lo && kt <= (hi - 1) / kTile; ++kt) ++cost[kt];
      };
      for (int64_t qt = 0; qt < nQ; ++qt) {
        const RowIv a = dflash_row(r, qt * kTile);
        const RowIv z = dflash_row(r, std::min(Sq, (qt + 1) * kTile) - 1);
        add(a.lo1, std::max(a.hi1, z.hi1));
        add(a.lo2, z.hi2);
      }
    }
    for (int64_t kt = 0; kt < nK; ++kt) items.emplace_back(-cost[kt], (int)((b << 10) | kt));
  }
  if ((int64_t)items.size() > kMaxOrder) return;
  std::stable_sort(items.begin(), items.end(),
                   [](const std::pair<int64_t, int>& x, const std::pair<int64_t, int>& y) {
                     return x.first < y.first;
                   });
  for (size_t i = 0; i < items.size(); ++i) ord.item[i] = (uint16_t)items[i].second;
  ord.n = (int32_t)items.size();
}

}  // namespace

extern "C" {

int masked_attn_varlen_fwd(const bsm_varlen* vl, const bsm_attn_args* a, hipStream_t stream) {
  VarlenInfo vi;
  int e = check_varlen(vl, vi);
  if (e) return e;
  if (!a) return fail(BSM_E_ARG, "args is NULL");
  if (a->reserved != 0) return fail(BSM_E_ARG, "args.reserved must be 0");
  if (vl->D != 64 && vl->D != 128)
    return fail(BSM_E_UNSUPPORTED, "head dim %lld not supported (64 or 128)", (long long)vl->D);
  if (a->mask || a->bias || a->keys)
    return fail(BSM_E_UNSUPPORTED, "varlen attention takes a DFlash predicate or no mask");
  const int32_t dt = a->q.dtype;
  if (dt != BSM_BF16 && dt != BSM_F32) return fail(BSM_E_DTYPE, "q must be bf16 or f32");
  if ((e = check_tensor_qkv(&a->q, "q", 1, vl->total_q, vl->H, vl->D, dt))) return e;
  if ((e = check_tensor_qkv(&a->k, "k", 1, vl->total_k, vl->KVH, vl->D, dt))) return e;
  if ((e = check_tensor_qkv(&a->v, "v", 1, vl->total_k, vl->KVH, vl->D, dt))) return e;
  {
    bsm_tensor4 o{};
    o.data = a->o;
    o.dtype = dt;
    o.size[0] = 1;
    o.size[1] = vl->total_q;
    o.size[2] = vl->H;
    o.size[3] = vl->D;
    for (int i = 0; i < 4; ++i) o.stride[i] = a->o_stride[i];
    if ((e = check_tensor_qkv(&o, "o", 1, vl->total_q, vl->H, vl->D, dt))) return e;
  }
  if (std::isnan(a->softmax_scale)) return fail(BSM_E_ARG, "softmax_scale is NaN");
  AttnInputs in;
  if (a->pred && (e = check_dflash_varlen(a->pred, vl, in.rule))) return e;
  if (a->bm) {
    if (!a->pred) return fail(BSM_E_ARG, "a block mask needs pred");
    const bsm_block_mask* bm = a->bm;
    if (bm->Bm != vi.B || bm->Hm != 1 || bm->nQm != vi.nQ || bm->nK != vi.nK)
      return fail(BSM_E_SHAPE, "block mask dims do not match these sequences");
    if (vi.B * vi.nQ > 0 && (!bm->kv_num_blocks || !bm->full_kv_num_blocks ||
                             (vi.nK > 0 && (!bm->kv_indices || !bm->full_kv_indices))))
      return fail(BSM_E_ARG, "block mask buffer is NULL");
    in.bmv.kv_num = bm->kv_num_blocks;
    in.bmv.kv_idx = bm->kv_indices;
    in.bmv.full_num = bm->full_kv_num_blocks;
    in.bmv.full_idx = bm->full_kv_indices;
    in.bmv.Bm = bm->Bm;
    in.bmv.Hm = 1;
    in.bmv.nQm = bm->nQm;
    in.bmv.nK = bm->nK;
    in.bmv.h_mode = 0;
  }
  if (vi.B == 0 || vl->total_q == 0) return BSM_OK;

  // Geometry of the launch: one "batch" per sequence, the longest sequence's
  // tile counts, and the packed tensors' row strides with batch strides 0.
  Geo g{};
  g.B = vi.B;
  g.H = vl->H;
  g.KVH = vl->KVH;
  g.Sq = vl->total_q;
  g.Sk = vl->total_k;
  g.D = vl->D;
  g.G = vl->H / vl->KVH;
  g.swap = false;
  AttnParams p;
  fill_params(g, a->q, a->k, a->v, a->o, a->o_stride, a->lse, a->softmax_scale, a->pred,
              false, false, a->bm, in, p);
  p.q_sb = p.k_sb = p.v_sb = p.o_sb = 0;
  p.lse_sb = 0;
  p.lse_sh = vl->total_q;
  p.lse_sq = 1;
  p.Sq = (int32_t)vi.maxSq;
  p.nQ = (int32_t)vi.nQ;
  p.Sk = (int32_t)vl->total_k;  // bounds the 32-bit offset checks
  p.nK = (int32_t)vi.nK;
  p.varlen = 1;
  p.cu_q = vl->cu_seqlens_q;
  p.cu_k = vl->cu_seqlens_k;
  hipError_t he;
  if (dt == BSM_BF16) {
    if (attn_v2_applies(p, (int)g.D)) {
      WorkOrder ord;
      varlen_order(vl, vi, a->pred ? &p.rule : nullptr, ord);
      he = launch_attn_bf16_v2(p, (int)g.D, stream, &ord);
    } else if (attn_h1_applies(p, (int)g.D)) {
      he = launch_attn_bf16_h1(p, (int)g.D, stream);
    } else {
      he = launch_attn_bf16(p, (int)g.D, stream);
    }
  } else {
    he = launch_attn_f32(p, (int)g.D, stream);
  }
  return hip_status(he, "masked_attn_varlen_fwd");
}

}  // extern "C"

namespace {

// Rows r0 .. r0 + n - 1 of a packed (1, rows, heads, D) tensor, as a batch of one.
bsm_tensor4 seq_rows(const bsm_tensor4& t, int64_t r0, int64_t n) {
  bsm_tensor4 s = t;
  s.size[1] = n;
  if (t.data && n > 0)
    s.data = static_cast<const char*>(t.data) + r0 * t.stride[1] * elem_size(t.dtype);
  return s;
}

// Delta of sequence b of a varlen backward: H * Sq_b floats, 256-byte aligned.
int64_t varlen_delta_bytes(const bsm_varlen* vl, int64_t b) {
  const int64_t sq = (int64_t)vl->cu_seqlens_q_host[b + 1] - vl->cu_seqlens_q_host[b];
  return round_multiple(vl->H * sq * 4, 256);
}

}  // namespace

extern "C" {

int masked_attn_varlen_bwd_workspace_size(const bsm_varlen* vl, int64_t* bytes) {
  VarlenInfo vi;
  int e = check_varlen(vl, vi);
  if (e) return e;
  if (!bytes) return fail(BSM_E_ARG, "bytes is NULL");
  int64_t n = 0;
  for (int64_t b = 0; b < vi.B; ++b) n += varlen_delta_bytes(vl, b);
  *bytes = n;
  return BSM_OK;
}

int masked_attn_varlen_bwd(const bsm_varlen* vl, const bsm_attn_bwd_args* a,
                           hipStream_t stream) {
  VarlenInfo vi;
  int e = check_varlen(vl, vi);
  if (e) return e;
  if (!a) return fail(BSM_E_ARG, "args is NULL");
  if (a->reserved != 0) return fail(BSM_E_ARG, "args.reserved must be 0");
  if (vl->D != 64 && vl->D != 128)
    return fail(BSM_E_UNSUPPORTED, "head dim %lld not supported (64 or 128)", (long long)vl->D);
  if (a->mask || a->bias || a->dbias)
    return fail(BSM_E_UNSUPPORTED, "varlen backward takes a DFlash predicate or no mask");
  const int32_t dt = a->q.dtype;
  if (dt != BSM_BF16 && dt != BSM_F32) return fail(BSM_E_DTYPE, "q must be bf16 or f32");
  const int64_t tq = vl->total_q, tk = vl->total_k;
  if ((e = check_tensor_qkv(&a->q, "q", 1, tq, vl->H, vl->D, dt))) return e;
  if ((e = check_tensor_qkv(&a->k, "k", 1, tk, vl->KVH, vl->D, dt))) return e;
  if ((e = check_tensor_qkv(&a->v, "v", 1, tk, vl->KVH, vl->D, dt))) return e;
  if ((e = check_tensor_qkv(&a->o, "o", 1, tq, vl->H, vl->D, dt))) return e;
  if ((e = check_tensor_qkv(&a->dout, "dout", 1, tq, vl->H, vl->D, dt))) return e;
  if ((e = check_tensor_qkv(&a->dq, "dq", 1, tq, vl->H, vl->D, dt))) return e;
  if ((e = check_tensor_qkv(&a->dk, "dk", 1, tk, vl->KVH, vl->D, dt))) return e;
  if ((e = check_tensor_qkv(&a->dv, "dv", 1, tk, vl->KVH, vl->D, dt))) return e;
  if (!a->lse && vl->H * tq > 0) return fail(BSM_E_ARG, "lse is NULL");
  if (std::isnan(a->softmax_scale)) return fail(BSM_E_ARG, "softmax_scale is NaN");
  DFlashRule vrule{};
  if (a->pred && (e = check_dflash_varlen(a->pred, vl, vrule))) return e;
  const bsm_block_mask* bm = a->bm;
  if (bm) {
    if (!a->pred) return fail(BSM_E_ARG, "a block mask needs pred");
    if (bm->Bm != vi.B || bm->Hm != 1 || bm->nQm != vi.nQ || bm->nK != vi.nK)
      return fail(BSM_E_SHAPE, "block mask dims do not match these sequences");
    if (vi.B * vi.nQ > 0 && (!bm->kv_num_blocks || !bm->full_kv_num_blocks ||
                             (vi.nK > 0 && (!bm->kv_indices || !bm->full_kv_indices))))
      return fail(BSM_E_ARG, "block mask buffer is NULL");
  }
  int64_t need = 0;
  for (int64_t b = 0; b < vi.B; ++b) need += varlen_delta_bytes(vl, b);
  if (a->workspace_bytes < need)
    return fail(BSM_E_ARG, "workspace of %lld bytes, %lld needed", (long long)a->workspace_bytes,
                (long long)need);
  if (need > 0 && (!a->workspace || (uintptr_t)a->workspace % 256))
    return fail(BSM_E_ARG, "workspace is NULL or not 256-byte aligned");

  // bf16, D = 128: one launch of each matrix-core kernel over every sequence
  // (sequence mode, as the packed forward), after Delta over the packed rows
  // (H x total_q floats, within the per-sequence workspace's size).
  if (dt == BSM_BF16 && vl->D == 128 && vi.B > 0 && tq > 0 &&
      tk * a->k.stride[1] * 2 < ((int64_t)1 << 31) && tk * a->v.stride[1] * 2 < ((int64_t)1 << 31) &&
      vi.maxSq * a->q.stride[1] * 2 < ((int64_t)1 << 31) &&
      vi.maxSq * a->dout.stride[1] * 2 < ((int64_t)1 << 31)) {
    AttnInputs in;
    in.rule = vrule;
    if (bm) {
      in.bmv.kv_num = bm->kv_num_blocks;
      in.bmv.kv_idx = bm->kv_indices;
      in.bmv.full_num = bm->full_kv_num_blocks;
      in.bmv.full_idx = bm->full_kv_indices;
      in.bmv.Bm = bm->Bm;
      in.bmv.Hm = 1;
      in.bmv.nQm = bm->nQm;
      in.bmv.nK = bm->nK;
      in.bmv.h_mode = 0;
    }
    Geo g{};
    g.B = vi.B;
    g.H = vl->H;
    g.KVH = vl->KVH;
    g.Sq = tq;
    g.Sk = tk;
    g.D = vl->D;
    g.G = vl->H / vl->KVH;
    g.swap = false;
    AttnBwdParams p{};
    fill_params(g, a->q, a->k, a->v, const_cast<void*>(a->o.data), a->o.stride,
                const_cast<float*>(a->lse), a->softmax_scale, a->pred != nullptr, false, false,
                bm != nullptr, in, p.f);
    p.f.q_sb = p.f.k_sb = p.f.v_sb = p.f.o_sb = 0;
    p.f.lse_sb = 0;
    p.f.lse_sh = tq;
    p.f.lse_sq = 1;
    p.f.Sq = (int32_t)vi.maxSq;
    p.f.nQ = (int32_t)vi.nQ;
    p.f.Sk = (int32_t)tk;  // bounds the 32-bit offset checks
    p.f.nK = (int32_t)vi.nK;
    p.f.varlen = 1;
    p.f.cu_q = vl->cu_seqlens_q;
    p.f.cu_k = vl->cu_seqlens_k;
    p.scale = p.f.scale_log2 / 1.4426950408889634f;
    p.dout = a->dout.data;
    p.do_sb = 0;
    p.do_sq = a->dout.stride[1];
    p.do_sh = a->dout.stride[2];
    p.dq = const_cast<void*>(a->dq.data);
    p.dq_sb = 0;
    p.dq_sq = a->dq.stride[1];
    p.dq_sh = a->dq.stride[2];
    p.dk = const_cast<void*>(a->dk.data);
    p.dk_sb = 0;
    p.dk_sk = a->dk.stride[1];
    p.dk_sh = a->dk.stride[2];
    p.dv = const_cast<void*>(a->dv.data);
    p.dv_sb = 0;
    p.dv_sk = a->dv.stride[1];
    p.dv_sh = a->dv.stride[2];
    p.delta = static_cast<float*>(a->workspace);
    p.delta_sb = 0;
    p.delta_sh = tq;
    // Delta: the packed rows as one batch of total_q rows, (H, total_q)
    AttnBwdParams pd = p;
    pd.f.B = 1;
    pd.f.Sq = (int32_t)tq;
    pd.f.varlen = 0;
    WorkOrder qord, kord;
    varlen_order(vl, vi, a->pred ? &p.f.rule : nullptr, qord);
    varlen_key_order(vl, vi, a->pred ? &p.f.rule : nullptr, kord);
    hipError_t he = launch_attn_bwd_delta(pd, 128, 1, stream);
    if (he == hipSuccess) he = launch_attn_bwd_mfma(p, stream, &qord, &kord);
    return hip_status(he, "masked_attn_varlen_bwd");
  }

  // Otherwise each sequence is a padded batch of one: its rows of the packed
  // tensors, its DFlash geometry (C_b = Sk_b - Sq_b context tokens, NB_b =
  // Sq_b / bs blocks), its row of the block mask, and its LSE columns.
  char* ws = static_cast<char*>(a->workspace);
  const int32_t* cq = vl->cu_seqlens_q_host;
  const int32_t* ck = vl->cu_seqlens_k_host;
  for (int64_t b = 0; b < vi.B; ++b) {
    const int64_t q0 = cq[b], sq = (int64_t)cq[b + 1] - cq[b];
    const int64_t k0 = ck[b], sk = (int64_t)ck[b + 1] - ck[b];
    char* delta = ws;
    ws += varlen_delta_bytes(vl, b);
    if (sq == 0 && sk == 0) continue;
    bsm_geom gb{1, vl->H, vl->KVH, sq, sk, vl->D};
    Geo g;
    if ((e = check_geom(&gb, g))) return e;
    g.swap = false;  // the forward over packed sequences applies no swap
    bsm_dflash pb{};
    const bool pred = a->pred && sq > 0;
    if (pred) {
      pb = *a->pred;
      pb.ctx_len = sk - sq;
      pb.num_blocks = sq / a->pred->block_size;
    }
    AttnInputs in;
    if ((e = check_attn_aux(g, dt, pred ? &pb : nullptr, nullptr, nullptr, nullptr,
                            a->softmax_scale, in)))
      return e;
    const bool has_bm = bm && pred;
    if (has_bm) {
      in.bmv.kv_num = bm->kv_num_blocks + b * vi.nQ;
      in.bmv.kv_idx = bm->kv_indices + b * vi.nQ * vi.nK;
      in.bmv.full_num = bm->full_kv_num_blocks + b * vi.nQ;
      in.bmv.full_idx = bm->full_kv_indices + b * vi.nQ * vi.nK;
      in.bmv.Bm = 1;
      in.bmv.Hm = 1;
      in.bmv.nQm = vi.nQ;  // query tiles past this sequence's are never visited
      in.bmv.nK = vi.nK;   // the row stride of the index lists
      in.bmv.h_mode = 0;
    }
    const bsm_tensor4 q = seq_rows(a->q, q0, sq), k = seq_rows(a->k, k0, sk);
    const bsm_tensor4 v = seq_rows(a->v, k0, sk), o = seq_rows(a->o, q0, sq);
    const bsm_tensor4 dout = seq_rows(a->dout, q0, sq), dq = seq_rows(a->dq, q0, sq);
    const bsm_tensor4 dk = seq_rows(a->dk, k0, sk), dv = seq_rows(a->dv, k0, sk);
    AttnBwdParams p{};
    fill_params(g, q, k, v, const_cast<void*>(o.data), o.stride,
                a->lse ? const_cast<float*>(a->lse) + q0 : nullptr, a->softmax_scale, pred,
                false, false, has_bm, in, p.f);
    p.f.lse_sb = 0;
    p.f.lse_sh = tq;  // (1, H, total_q): this sequence's columns
    p.f.lse_sq = 1;
    p.scale = p.f.scale_log2 / 1.4426950408889634f;
    p.dout = dout.data;
    qlike_strides(g, dout.stride, p.do_sb, p.do_sq, p.do_sh);
    p.dq = const_cast<void*>(dq.data);
    qlike_strides(g, dq.stride, p.dq_sb, p.dq_sq, p.dq_sh);
    p.dk = const_cast<void*>(dk.data);
    p.dk_sb = dk.stride[0];
    p.dk_sk = dk.stride[1];
    p.dk_sh = dk.stride[2];
    p.dv = const_cast<void*>(dv.data);
    p.dv_sb = dv.stride[0];
    p.dv_sk = dv.stride[1];
    p.dv_sh = dv.stride[2];
    p.delta = reinterpret_cast<float*>(delta);
    p.delta_sb = (int64_t)p.f.H * p.f.Sq;
    p.delta_sh = p.f.Sq;
    const hipError_t he = launch_attn_bwd(p, (int)g.D, dt == BSM_BF16, stream);
    if (he != hipSuccess) return hip_status(he, "masked_attn_varlen_bwd");
  }
  return BSM_OK;
}

int unpad_index(const uint8_t* valid, int64_t batch, int64_t seqlen, int64_t row_stride,
                int32_t* cu_seqlens, int32_t* indices, hipStream_t stream) {
  if (batch < 0 || seqlen < 0) return fail(BSM_E_ARG, "negative batch or seqlen");
  if (batch > 65535 || batch * seqlen >= ((int64_t)1 << 31))
    return fail(BSM_E_UNSUPPORTED, "batch * seqlen must stay below 2^31");
  if (!cu_seqlens) return fail(BSM_E_ARG, "cu_seqlens is NULL");
  if (batch * seqlen > 0 && (!valid || !indices)) return fail(BSM_E_ARG, "valid or indices is NULL");
  if (batch > 1 && row_stride < seqlen) return fail(BSM_E_STRIDE, "row_stride below seqlen");
  return hip_status(launch_unpad_index(valid, batch, seqlen, row_stride, cu_seqlens, indices,
                                       stream),
                    "unpad_index");
}

int gather_rows(const void* src, int64_t src_stride, void* dst, int64_t dst_stride,
                int64_t row_bytes, const int32_t* indices, int64_t n, hipStream_t stream) {
  int e = check_copy(src, src_stride, dst, dst_stride, row_bytes, indices, n);
  if (e) return e;
  return hip_status(launch_copy_rows(src, src_stride, dst, dst_stride, row_bytes, indices, n,
                                     false, stream),
                    "gather_rows");
}

int scatter_rows(const void* src, int64_t src_stride, void* dst, int64_t dst_stride,
                 int64_t row_bytes, const int32_t* indices, int64_t n, hipStream_t stream) {
  int e = check_copy(src, src_stride, dst, dst_stride, row_bytes, indices, n);
  if (e) return e;
  return hip_status(launch_copy_rows(src, src_stride, dst, dst_stride, row_bytes, indices, n,
                                     true, stream),
                    "scatter_rows");
}

}  // extern "C"
