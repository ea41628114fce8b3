// Internal interfaces between the host API (bsm_api.cpp) and the HIP kernels.
// All sizes are validated by the host API before a launcher is called; the
// launchers only map work onto grids and return hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsm {

constexpr int kTile = 128;  // query and key tile edge

// DFlash predicate, resolved on the host: per-row kept keys are two
// half-open intervals, [lo1, hi1) in the context and [lo2, hi2) in the row's
// own draft block (see dflash_row in dflash_rows.h).
struct DFlashRule {
  int64_t C;      // context tokens
  int64_t bs;     // draft block size
  int64_t S;      // context tokens per block
  int64_t e0;     // context end offset
  int64_t W;      // left-bound window, 0 = none
  int32_t causal; // in-block causality
  int32_t pad;
};

// Device-side block mask view in the attention's iteration space.
struct BlockMaskView {
  const int32_t* kv_num;
  const int32_t* kv_idx;
  const int32_t* full_num;
  const int32_t* full_idx;
  int64_t Bm, Hm, nQm, nK;
  int32_t h_mode;  // 0: head index 0, 1: h, 2: h / G
  int32_t pad;
};

// Kept-key list view in the attention's iteration space: for list (bk, hk),
// num[bk * Hm + hk] keys at idx / bits + (bk * Hm + hk) * K.
struct KeyListView {
  const int32_t* num;
  const int32_t* idx;
  const uint32_t* bits;
  int64_t Bm, Hm, K;
  int32_t h_mode;  // 0: head index 0, 1: h, 2: h / G
  int32_t pad;
};

// Aux tensor (mask or bias) addressed as base + b*sb + hidx*sh + q*sq + k,
// with stride 0 on broadcast dims and hidx chosen by h_mode.
struct AuxView {
  const void* data;
  int64_t sb, sh, sq;
  int32_t h_mode;  // 0: 0, 1: h, 2: h / G
  int32_t q_bcast; // 1 if the query dim broadcasts
};

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_sb, q_sq, q_sh;
  int64_t k_sb, k_sk, k_sh;
  int64_t v_sb, v_sk, v_sh;
  int64_t o_sb, o_sq, o_sh;
  int64_t lse_sb, lse_sh, lse_sq;
  int32_t B, H, KVH, G, Sq, Sk, nQ, nK;
  float scale_log2;  // softmax scale * log2(e)
  int32_t mask_kind; // 0 none, 1 DFlash predicate, 2 dense mask
  int32_t pred_row0; // predicate evaluated at query 0 for every row (swap)
  DFlashRule rule;
  AuxView mask;
  AuxView bias;
  int32_t has_bias;
  int32_t has_bm;
  BlockMaskView bm;
  int32_t gather;   // visit the keys of `keys` instead of key tiles
  int32_t varlen;   // packed sequences: cu_q / cu_k give each one's rows
  KeyListView keys;
  const int32_t* cu_q;
  const int32_t* cu_k;
  // short query blocks (k_attn_group): heads packed per workgroup (1 or G),
  // key-tile splits per (b, head group), and the float partials of the splits
  int32_t pack;
  int32_t splits;
  float* ws_o;   // (splits, B, H, Sq, D)
  float* ws_ml;  // (splits, B, H, Sq, 2): running max (log2 units), row sum
  // Staged mask and bias (bf16 long-query kernel): when both broadcast over
  // the query dim, they are folded into one float row per (b, head) -- the
  // bias in log2 units where the mask keeps a key below Sk, -inf elsewhere --
  // whose 128-key slices travel to LDS with each K/V tile.
  int32_t staged;
  int32_t cb_hmode;     // head rule of the rows: 0 one row, 1 per head, 2 per KV head
  const float* cb;      // (B, Hc, nK * 128) floats, contiguous
  int64_t cb_sb, cb_sh; // element strides of b and of the row's head
};

// Backward: the forward's view plus the incoming gradient, the gradient
// outputs and the float scratch (all in the kernels' iteration space, i.e.
// after the head-group swap when it applies).
struct AttnBwdParams {
  AttnParams f;             // q, k, v, o, lse, geometry, mask, bias, block mask
  const void* dout;
  int64_t do_sb, do_sq, do_sh;
  void* dq;
  int64_t dq_sb, dq_sq, dq_sh;
  void* dk;
  int64_t dk_sb, dk_sk, dk_sh;
  void* dv;
  int64_t dv_sb, dv_sk, dv_sh;
  float* delta;             // rowsum(dO * O): row q of (b, h) at b * delta_sb + h * delta_sh + q
  float* dbias_acc;         // float accumulator of dbias, or null
  AuxView dbias;            // dbias_acc addressed like the bias
  float scale;              // softmax scale (natural units)
  int32_t pad;
  int64_t delta_sb, delta_sh;  // (B, H, Sq) contiguous: H * Sq, Sq; packed: 0, total_q
};

// Float dbias accumulator -> dbias (bias dtype, caller strides), original
// (unswapped) index space; keys >= Sk get 0.
struct DbiasOut {
  const float* acc;         // contiguous (n0, n1, n2, K)
  void* out;
  int64_t n0, n1, n2, K, Sk;
  int64_t s0, s1, s2;       // out element strides (last dim contiguous)
  int32_t is_bf16;
  int32_t pad;
};

struct DenseMaskView {
  const uint8_t* data;
  int64_t sb, sh, sq;
  int64_t Bm, Hm, Qm, K;  // K = K_round
  int64_t Sk;
};

// Kept-key list builder: mask (bm, hm, r) rows at data + bm*sb + hm*sh + r*sq
// (sq unused when Qm == 1), R rows, keys < Sk of K_round.
struct KeyListParams {
  const uint8_t* mask;
  int64_t sb, sh, sq;
  int64_t Bm, Hm, K, Sk;
  int32_t R, Qm;
  int32_t* num;
  int32_t* idx;
  uint32_t* bits;
};

struct TopkParams {
  const void* bias;
  int64_t b_sb, b_sh, b_sq;
  int64_t Bb, Hb, Qb, K;  // K = K_round
  int64_t Sk;
  const uint8_t* pm;      // nullable
  int64_t p_sb, p_sh, p_sq, pK;
  int64_t k;
  uint8_t* out;
  int32_t is_bf16;
};

hipError_t launch_block_mask_pred(const DFlashRule& r, int64_t Sq, int64_t Sk,
                                  int64_t nQ, int64_t nK, int32_t* kv_num,
                                  int32_t* kv_idx, int32_t* full_num,
                                  int32_t* full_idx, hipStream_t s);
// one block-mask row per (sequence, query tile); rule.C is completed per
// sequence from cu_q / cu_k, and rule.S too when it is 0
hipError_t launch_block_mask_pred_varlen(const DFlashRule& r, const int32_t* cu_q,
                                         const int32_t* cu_k, int64_t B, int64_t nQ,
                                         int64_t nK, int32_t* kv_num, int32_t* kv_idx,
                                         int32_t* full_num, int32_t* full_idx, hipStream_t s);
// packing helpers: cu_seqlens / indices of a (batch, seqlen) validity mask,
// and 16-byte row copies through an index list (scatter: dst[idx[i]] = src[i])
hipError_t launch_unpad_index(const uint8_t* valid, int64_t batch, int64_t seqlen,
                              int64_t row_stride, int32_t* cu, int32_t* idx, hipStream_t s);
hipError_t launch_copy_rows(const void* src, int64_t src_stride, void* dst, int64_t dst_stride,
                            int64_t row_bytes, const int32_t* idx, int64_t n, bool scatter,
                            hipStream_t s);
hipError_t launch_dflash_dense(const DFlashRule& r, int64_t Sq, int64_t Sk,
                               int64_t K, uint8_t* out, hipStream_t s);
hipError_t launch_block_mask_dense(const DenseMaskView& m, int32_t* kv_num,
                                   int32_t* kv_idx, int32_t* full_num,
                                   int32_t* full_idx, hipStream_t s);
hipError_t launch_topk(const TopkParams& p, hipStream_t s);

// Top-k fused with the block mask and / or the kept-key list of its mask
// (t.out nullable). The mask is contiguous with the bias's sizes; (m_sb, m_sh,
// m_sq) are its element strides in the attention's iteration space (m_sq = 0
// when Qm == 1), Bm x Hm lists of Qm <= 32 distinct rows, R iteration rows.
struct TopkFusedParams {
  TopkParams t;
  int64_t m_sb, m_sh, m_sq;
  int64_t Bm, Hm;
  int32_t Qm, R;
  int32_t* kv_num;   // block mask (Bm, Hm, 1, nK), or null
  int32_t* kv_idx;
  int32_t* full_num;
  int32_t* full_idx;
  int64_t nK;
  int32_t* l_num;    // key list (Bm, Hm, K), or null
  int32_t* l_idx;
  uint32_t* l_bits;
};
bool topk_fused_applies(const TopkParams& p);  // rows short enough for registers
hipError_t launch_topk_fused(const TopkFusedParams& fp, hipStream_t s);
hipError_t launch_key_list(const KeyListParams& p, hipStream_t s);
hipError_t launch_attn_bf16(const AttnParams& p, int D, hipStream_t s);
hipError_t launch_attn_f32(const AttnParams& p, int D, hipStream_t s);
// pipelined bf16 kernel: two heads of a KV group per workgroup
bool attn_v2_applies(const AttnParams& p, int D);
// Staged mask / bias rows for the pipelined kernel: whether they apply, the
// workspace they take, and the pass that writes them (sets p.staged, p.cb...).
bool staged_aux_applies(const AttnParams& p);
int64_t staged_aux_bytes(const AttnParams& p);
hipError_t launch_aux_combine(AttnParams& p, void* ws, hipStream_t s);
// Order in which a packed (varlen) launch of the pipelined kernel takes its
// (sequence, query tile) items: item[i] = b << 10 | qt, heaviest first; each
// item spans KVH * G / 2 workgroups (the backward's dK / dV kernel: (sequence,
// key tile) items b << 10 | kt, KVH workgroups each). n = 0: the kernel's own
// order.
constexpr int kMaxOrder = 1024;
struct WorkOrder {
  int32_t n;
  uint16_t item[kMaxOrder];
};
hipError_t launch_attn_bf16_v2(const AttnParams& p, int D, hipStream_t s,
                               const WorkOrder* order = nullptr);
// bf16, one head per workgroup, 64-key sub-tiles, two workgroups per CU (no
// mask tensor, no bias, not packed)
bool attn_h1_applies(const AttnParams& p, int D);
hipError_t launch_attn_bf16_h1(const AttnParams& p, int D, hipStream_t s);
// backward: rowsum(dO * O), then dQ and dK / dV (+ dbias accumulation)
hipError_t launch_attn_bwd(const AttnBwdParams& p, int D, int is_bf16, hipStream_t s);
// rowsum(dO * O) alone, row (b, h, q) at delta[(b * H + h) * Sq + q]
hipError_t launch_attn_bwd_delta(const AttnBwdParams& p, int D, int is_bf16, hipStream_t s);
hipError_t launch_fill_zero(float* x, int64_t n, hipStream_t s);
// bf16 matrix-core dQ and dK / dV (D = 128); for packed sequences (f.varlen)
// only without a mask tensor or bias, K / V offsets within 32 bits
bool attn_bwd_mfma_applies(const AttnBwdParams& p, int D);
// (packed: optional host orders of (b, query tile) and (b, key tile) items)
hipError_t launch_attn_bwd_mfma(const AttnBwdParams& p, hipStream_t s,
                                const WorkOrder* dq_order = nullptr,
                                const WorkOrder* dkdv_order = nullptr);
hipError_t launch_dbias_out(const DbiasOut& d, hipStream_t s);
// bf16 short query blocks (at most 32 query rows per (b, h)): the packed /
// split kernel (p.pack, p.splits set; the merge of the splits' partial states
// follows when p.splits > 1), and the key-gather kernel for a kept-key list
bool short_query_applies(const AttnParams& p, int D);
hipError_t launch_attn_group(const AttnParams& p, int D, hipStream_t s);
hipError_t launch_attn_gather(const AttnParams& p, int D, hipStream_t s);

// Sets the thread's error string (bsm_last_error) and returns `code`.
int set_error(int code, const char* msg);

}  // namespace bsm
