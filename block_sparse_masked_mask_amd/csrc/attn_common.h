// Shared pieces of the masked attention kernels: which key tiles a query tile
// visits, and where its mask / bias rows live.
//
// Broadcast rules (flash-sparse-attention PR #190, Design and Changes): an aux
// tensor's batch / query dims broadcast by stride 0 when of size 1, and its head
// dim is H (index h), KVH (index h / G) or 1 (index 0). The block mask follows
// the same head rule and is shared by every query tile when it has one query
// tile row (nQm == 1).
#pragma once

#include "bsm_internal.h"
#include "dflash_rows.h"

namespace bsm {

// An additive bias in the log2 units the kernels' softmax works in, finite
// values saturated at the largest finite float: a bias beyond
// +-FLT_MAX / log2(e) (~2.36e38; the finfo(bf16 / f32).min pre-mask sentinel
// of flash-sparse-attention PR #197, Changes, is one) scores as that bound, so
// a kept key carrying it stays kept and keys that all carry it weigh the
// same. A bias of -inf stays -inf: that key contributes nothing.
__device__ inline float bias_log2(float b) {
  const float x = fminf(fmaxf(b * 1.4426950408889634f, -3.402823466e38f), 3.402823466e38f);
  return b == -INFINITY ? b : x;
}
// the same saturation in natural units (the backward's scores)
__device__ inline float bias_nat(float b) {
  const float x = fminf(fmaxf(b, -2.3586575e38f), 2.3586575e38f);
  return b == -INFINITY ? b : x;
}

__device__ inline int64_t head_index(int mode, int h, int G) {
  return mode == 0 ? 0 : (mode == 1 ? h : h / G);
}

__device__ inline const uint8_t* aux_row(const AuxView& a, int64_t elem, int b, int h,
                                         int G, int q) {
  const int64_t off = (int64_t)b * a.sb + head_index(a.h_mode, h, G) * a.sh +
                      (a.q_bcast ? 0 : (int64_t)q) * a.sq;
  return reinterpret_cast<const uint8_t*>(a.data) + off * elem;
}

// One sequence of a launch. Padded batches: batch b's rows start at 0 and
// every batch has the launch's Sq / Sk. Packed (varlen) launches: sequence b
// owns query rows cu_q[b] .. cu_q[b+1] and key rows cu_k[b] .. cu_k[b+1] of
// one packed batch (batch strides 0), and a DFlash rule is completed per
// sequence: C_b = Sk_b - Sq_b context tokens, NB_b = Sq_b / bs blocks, and
// S_b = C_b / NB_b unless the launch fixes it (rule.S > 0).
struct SeqView {
  int64_t q0, k0;  // first packed query row / key row
  int Sq, Sk, nQ, nK;
  DFlashRule rule;
};

__device__ inline SeqView seq_view(const AttnParams& p, int b) {
  SeqView s;
  s.rule = p.rule;
  if (p.varlen) {
    const int a = p.cu_q[b], e = p.cu_q[b + 1];
    const int c = p.cu_k[b], d = p.cu_k[b + 1];
    s.q0 = a;
    s.k0 = c;
    s.Sq = e - a;
    s.Sk = d - c;
    if (p.mask_kind == 1) {  // 32-bit arithmetic: packed sizes stay below 2^30
      const int C = s.Sk - s.Sq;
      const int nb = s.Sq / (int)p.rule.bs;
      s.rule.C = C;
      if (p.rule.S == 0) s.rule.S = nb > 0 ? C / nb : 0;
    }
  } else {
    s.q0 = 0;
    s.k0 = 0;
    s.Sq = p.Sq;
    s.Sk = p.Sk;
  }
  s.nQ = (s.Sq + kTile - 1) / kTile;
  s.nK = (s.Sk + kTile - 1) / kTile;
  return s;
}

// Key tiles visited by query tile qt of (b, h): first the full tiles, then the
// partial ones. Without a block mask every key tile is visited, as partial when
// a mask is present and as full otherwise.
struct TileList {
  const int32_t* full;
  const int32_t* part;
  int nfull, npart;

  // nK: key tiles of the sequence when there is no block mask (-1: p.nK)
  __device__ inline void init(const AttnParams& p, int b, int h, int qt, int nK = -1) {
    if (nK < 0) nK = p.nK;
    if (p.has_bm) {
      const BlockMaskView& m = p.bm;
      const int64_t mb = m.Bm == 1 ? 0 : b;
      const int64_t mh = head_index(m.h_mode, h, p.G);
      const int64_t mq = m.nQm == 1 ? 0 : qt;
      const int64_t r = (mb * m.Hm + mh) * m.nQm + mq;
      nfull = m.full_num[r];
      npart = m.kv_num[r];
      full = m.full_idx + r * m.nK;
      part = m.kv_idx + r * m.nK;
    } else {
      full = part = nullptr;
      if (p.mask_kind == 0) {
        nfull = nK;
        npart = 0;
      } else {
        nfull = 0;
        npart = nK;
      }
    }
  }
  __device__ inline int count() const { return nfull + npart; }
  // key tile of visit i, and whether it is full (no mask test needed)
  __device__ inline int tile(int i, bool& is_full) const {
    is_full = i < nfull;
    // read through the constant address space: with a uniform index the load
    // is a scalar one, which neither waits for nor is waited on by vector loads
    typedef const __attribute__((address_space(4))) int32_t cint32;
    int kt;
    if (is_full)
      kt = full ? ((cint32*)full)[i] : i;
    else
      kt = part ? ((cint32*)part)[i - nfull] : i - nfull;
    return __builtin_amdgcn_readfirstlane(kt);  // uniform across the workgroup
  }
};

}  // namespace bsm
