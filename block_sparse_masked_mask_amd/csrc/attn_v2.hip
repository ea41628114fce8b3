// Masked attention forward, bf16, pipelined variant for gfx950.
//
// Same arithmetic as k_attn_bf16 (attn.hip): S^T = K Q^T and O^T += V^T P^T on
// v_mfma_f32_32x32x16_bf16 with a float online softmax, full tiles without a
// mask test, partial tiles testing the DFlash row intervals or the mask bytes,
// additive bias, keys >= Sk never kept (flash-sparse-attention PR #190, Design;
// SpecForge issue #452). What changes is how K and V reach the matrix cores:
//
//  * 512 threads = 8 waves: waves 0-3 take 128 query rows of head h, waves 4-7
//    the same rows of head h+1 of the same KV group, so one K/V tile in LDS
//    feeds two heads. Used when both heads share the block mask row (a block
//    mask broadcast over heads, or over the heads of a KV group).
//  * K and V tiles go from HBM/L2 straight into LDS with 16-byte LDS-DMA loads
//    (global_load_lds_dwordx4: each wave instruction fills 1 KiB of LDS), double
//    buffered: the loads of tile i+1 are in flight while tile i is computed.
//  * Both tiles stay row-major ([key][d]). Rows are XOR-swizzled in 16-byte
//    chunks (the swizzle is applied to the global addresses, since an LDS-DMA
//    instruction writes 64 consecutive 16-byte slots), chosen so that the rows
//    one LDS read cycle touches land in distinct banks (attn_pipe.h).
//  * V^T operands come from ds_read_b64_tr_b16: in each 16-lane group, lane
//    4e + g points at 4 d-values of key row e; the hardware hands lane 4g + s
//    the 4 keys of d-value s. Two such reads give a lane the 8 consecutive keys
//    of one d column that the MFMA A operand needs, with no transpose pass.
//  * Work items (b, KV group pair, query tile) are laid out so that each XCD
//    keeps the query tiles of the same (b, kvh) (one L2 per XCD) and runs the
//    heaviest query tiles first.
//  * A tile's softmax takes one max over its 128 keys; the LDS operand reads
//    run several MFMAs ahead (K five, V three) and the exponentials of the
//    tile's second half issue between the PV MFMAs of its first half. The
//    mask / bias path, short of registers for that, takes two halves of 64.
//  * The running max of a row is raised only when it grows by more than 2^8
//    (otherwise O is not rescaled), row sums come from dot2 on the bf16
//    probabilities the PV product uses, and tiles that need no mask test, no
//    bias and have all rows valid take a leaner softmax.
#include <math.h>

#include <type_traits>

#include "attn_common.h"
#include "attn_pipe.h"
#include "bsm_internal.h"
#include "dflash_rows.h"

namespace bsm {
namespace {

using namespace pipe;

// Per-row-block state of a wave: its 32 query rows.
template <int D>
struct RowBlock {
  bf16x8 qf[D / 16];       // Q operand: row n, d = 16 s + 8 hh + [0, 8)
  f32x16 oacc[D / 32];     // O^T accumulators
  float m_run, l_run;      // running max (log2 units) and sum
  RowIv32 iv;              // DFlash kept-key intervals of the row
  const uint8_t* mrow;     // mask row or null
  const uint16_t* brow;    // bias row or null
  bool qvalid;
};

// One key tile: S^T of all four 32-key chunks, one max (and at most one
// rescale) per row, then the probabilities and PV of the first 64 keys, with
// the second half's exponentials issued between the first half's PV MFMAs.
// The LDS operand reads are kept several MFMAs ahead of their use.
// SLOT: which of the two K and V buffers of lds holds the tile; a constant
// (0, 1) makes every LDS operand address a lane offset plus an immediate, -1
// takes it from slot_rt
template <int D, int RB, int MODE, int SLOT>
__device__ inline void compute_tile(const char* lds, int slot_rt, const AttnParams& p, int kt,
                                    bool is_full, RowBlock<D>* rbk, const LaneOffs<D>& off,
                                    int lane, int Sk, const float* cbrow) {
  constexpr int NS = D / 16;
  constexpr int NDC = D / 32;
  const int hh = lane >> 5;
  const int k0 = kt * kTile;
  const bool check_k = k0 + kTile > Sk;
  const bool check_mask = !is_full && p.mask_kind != 0;
  // K slot SLOT at SLOT * TB; the V slots' extra 2 * TB is in the lane offsets
  constexpr int TB = kTile * D * 2;
  const int slot = SLOT >= 0 ? SLOT : slot_rt;
  const char* kbase = lds + slot * TB;
  const char* vbase = lds + slot * TB;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // S^T for the tile's four 32-key chunks
  f32x16 sacc[RB][4];
  auto kop = [&](int i) {
    const int c = i / NS, s = i % NS;
    return *reinterpret_cast<const bf16x8*>(kbase + off.k[s] + c * 32 * D * 2);
  };
  {
    constexpr int PK = 5;  // K operands in flight
    bf16x8 ka[PK];
#pragma unroll
    for (int j = 0; j < PK; ++j) ka[j] = kop(j);
#pragma unroll
    for (int i = 0; i < 4 * NS; ++i) {
      const int c = i / NS, s = i % NS;
      const bf16x8 a = ka[i % PK];
      if (i + PK < 4 * NS) ka[i % PK] = kop(i + PK);
#pragma unroll
      for (int r = 0; r < RB; ++r)
        sacc[r][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            a, rbk[r].qf[s], s == 0 ? f32x16{} : sacc[r][c], 0, 0, 0);
    }
    // keep PK operand reads in flight ahead of the MFMAs (left alone, the
    // scheduler issues each read right before its MFMA)
    __builtin_amdgcn_sched_group_barrier(0x100, PK, 0);
#pragma unroll
    for (int i = 0; i < 4 * NS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, RB, 0);
      if (i + PK < 4 * NS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  }
  // V operand i of a half: d-chunk dc = i / 4, key chunk c = (i / 2) % 2,
  // 16-key step sb = i % 2; two transposed reads of 4 keys each
  auto vop = [&](int half, int i) {
    const int dc = i / 4, c = (i / 2) % 2, sb = i % 2;
    const int kb = (2 * half + c) * 32 + 16 * sb;
    const char* a0 = vbase + off.v[dc] + kb * D * 2;
    const char* a1 = a0 + 4 * D * 2;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a1));
    return __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo),
                                   __builtin_bit_cast(bf16x4, hi), 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // the first V operands load while the softmax runs
  constexpr int NV = 4 * NDC;  // V operands per half
  constexpr int PV = 3;        // V operands in flight
  bf16x8 va[PV];
#pragma unroll
  for (int j = 0; j < PV; ++j) va[j] = vop(j / NV, j % NV);

  // scores in log2 units, masked keys at -inf; one max (and at most one
  // rescale) per row and tile
  bool plain[RB];
  float m_use[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    RowBlock<D>& R = rbk[r];
    plain[r] = MODE != 2 && !check_k && !check_mask && R.brow == nullptr && R.qvalid;
    float mloc = -INFINITY;
    if (MODE == 2) {
      // the tile's slice of the folded mask / bias row: -inf drops a key
      // (masked or past Sk); rows past Sq compute values nobody stores
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const float4 c0 = *reinterpret_cast<const float4*>(cbrow + kc * 32 + 16 * sb + 8 * hh);
          const float4 c1 =
              *reinterpret_cast<const float4*>(cbrow + kc * 32 + 16 * sb + 8 * hh + 4);
          const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int u = 8 * sb + e;
            const float sv = fmaf(sacc[r][kc][u], p.scale_log2, cv[e]);
            sacc[r][kc][u] = sv;
            mloc = fmaxf(mloc, sv);
          }
        }
      }
    } else if (plain[r]) {
      // raw scores: the scale is folded into the exponent below
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int u = 0; u < 16; ++u) mloc = fmaxf(mloc, sacc[r][kc][u]);
      mloc *= p.scale_log2;
    } else {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const int kb = k0 + kc * 32 + 16 * sb + 8 * hh;  // 8 consecutive keys
          float bv[8];
          if (MODE == 1 && R.brow) {
            const uint4 raw = *reinterpret_cast<const uint4*>(R.brow + kb);
            const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
              bv[e] = bias_log2(bf16_to_f32((uint16_t)(wv[e >> 1] >> (16 * (e & 1)))));
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) bv[e] = 0.f;
          }
          uint32_t mbits = 0xFFu;
          if (check_mask) {
            if (MODE == 1 && p.mask_kind == 2) {
              uint2 mb = make_uint2(0, 0);
              if (R.mrow) mb = *reinterpret_cast<const uint2*>(R.mrow + kb);
              mbits = 0;
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const uint32_t byte = ((e < 4 ? mb.x : mb.y) >> (8 * (e & 3))) & 0xFFu;
                mbits |= (byte != 0u ? 1u : 0u) << e;
              }
            } else {
              mbits = range_bits(R.iv.lo1, R.iv.hi1, kb) | range_bits(R.iv.lo2, R.iv.hi2, kb);
            }
          }
          if (!R.qvalid) mbits = 0;
          if (check_k) mbits &= range_bits(0, Sk, kb);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int u = 8 * sb + e;
            float sv = sacc[r][kc][u] * p.scale_log2 + bv[e];
            sv = ((mbits >> e) & 1u) ? sv : -INFINITY;
            sacc[r][kc][u] = sv;
            mloc = fmaxf(mloc, sv);
          }
        }
      }
    }
    mloc = max_pair(mloc);
    // conditional rescale (see kRescaleLog2)
    const bool grow = mloc > R.m_run + kRescaleLog2;
    if (__ballot(grow)) {
      const float m_new = grow ? mloc : R.m_run;
      // 1 where the max is kept (also for rows still at -inf: -inf - -inf is NaN)
      const float alpha = grow ? __builtin_amdgcn_exp2f(R.m_run - m_new) : 1.f;
      R.l_run *= alpha;
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) R.oacc[dc] *= alpha;
      R.m_run = m_new;
    }
    m_use[r] = R.m_run == -INFINITY ? 0.f : R.m_run;
  }

  // probabilities of key chunks 2 * half and 2 * half + 1, as the PV product's
  // B operand, and their bf16 row sum
  auto probs = [&](int half, bf16x8 (&pf)[RB][2][2]) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const float mul = plain[r] ? p.scale_log2 : 1.f;
      float lsum = rbk[r].l_run;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const int u = 8 * sb + e;
            const float x0 = __builtin_amdgcn_exp2f(fmaf(sacc[r][2 * half + c][u], mul, -m_use[r]));
            const float x1 =
                __builtin_amdgcn_exp2f(fmaf(sacc[r][2 * half + c][u + 1], mul, -m_use[r]));
            const bf16x2 pr = {(__bf16)x0, (__bf16)x1};
            pf[r][c][sb][e] = pr[0];
            pf[r][c][sb][e + 1] = pr[1];
            // row sum of the bf16 probabilities the PV product uses
            lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsum, false);
          }
        }
      }
      rbk[r].l_run = lsum;
    }
  };
  auto pv = [&](int half, const bf16x8 (&pf)[RB][2][2]) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int dc = i / 4, c = (i / 2) % 2, sb = i % 2;
      // operand g of the tile; the next half's operands follow on
      const int g = half * NV + i;
      const bf16x8 a = va[g % PV];
      if (g + PV < 2 * NV) va[g % PV] = vop((g + PV) / NV, (g + PV) % NV);
#pragma unroll
      for (int r = 0; r < RB; ++r)
        rbk[r].oacc[dc] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[r][c][sb], rbk[r].oacc[dc], 0, 0, 0);
    }
  };
  bf16x8 pf0[RB][2][2], pf1[RB][2][2];
  probs(0, pf0);
  __builtin_amdgcn_sched_barrier(0);
  // the second half's exponentials can issue under the first half's PV MFMAs
  pv(0, pf0);
  probs(1, pf1);
  pv(1, pf1);
  // PV MFMAs of the first half with the second half's exponentials between
  // them, V operand reads PV operands ahead
#pragma unroll
  for (int i = 0; i < 2 * NV; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, RB, 1);
    if (i + PV < 2 * NV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    if (i < NV) __builtin_amdgcn_sched_group_barrier(0x002, 6, 1);
  }
}

// The mask / bias path (MODE 1), which has no registers for a whole tile's
// scores: the tile in two halves of 64 keys, each with its own max.
// SLOT: which of the two K and V buffers of lds holds the tile; a constant
// (0, 1) makes every LDS operand address a lane offset plus an immediate, -1
// takes it from slot_rt
template <int D, int RB, int MODE, int SLOT>
__device__ inline void compute_tile_halves(const char* lds, int slot_rt, const AttnParams& p,
                                           int kt, bool is_full, RowBlock<D>* rbk,
                                           const LaneOffs<D>& off, int lane, int Sk,
                                           const float* cbrow) {
  constexpr int NS = D / 16;
  constexpr int NDC = D / 32;
  const int hh = lane >> 5;
  const int k0 = kt * kTile;
  const bool check_k = k0 + kTile > Sk;
  const bool check_mask = !is_full && p.mask_kind != 0;
  // K slot SLOT at SLOT * TB; the V slots' extra 2 * TB is in the lane offsets
  constexpr int TB = kTile * D * 2;
  const int slot = SLOT >= 0 ? SLOT : slot_rt;
  const char* kbase = lds + slot * TB;
  const char* vbase = lds + slot * TB;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

#pragma unroll
  for (int half = 0; half < 2; ++half) {
    f32x16 sacc[RB][2];
    // K operand i of this half: chunk c = i / NS, k-step s = i % NS
    auto kop = [&](int i) {
      const int c = i / NS, s = i % NS;
      return *reinterpret_cast<const bf16x8*>(kbase + off.k[s] + (2 * half + c) * 32 * D * 2);
    };
    bf16x8 ka = kop(0);
#pragma unroll
    for (int i = 0; i < 2 * NS; ++i) {
      const int c = i / NS, s = i % NS;
      const bf16x8 a = ka;
      if (i + 1 < 2 * NS) ka = kop(i + 1);
#pragma unroll
      for (int r = 0; r < RB; ++r)
        sacc[r][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            a, rbk[r].qf[s], s == 0 ? f32x16{} : sacc[r][c], 0, 0, 0);
    }
    // V operand i of this half: d-chunk dc = i / 4, key chunk c = (i / 2) % 2,
    // 16-key step sb = i % 2; two transposed reads of 4 keys each
    auto vop = [&](int i) {
      const int dc = i / 4, c = (i / 2) % 2, sb = i % 2;
      const int kb = (2 * half + c) * 32 + 16 * sb;
      const char* a0 = vbase + off.v[dc] + kb * D * 2;
      const char* a1 = a0 + 4 * D * 2;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a1));
      return __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo),
                                     __builtin_bit_cast(bf16x4, hi), 0, 1, 2, 3, 4, 5, 6, 7);
    };
    // the first V operands load while the softmax runs
    bf16x8 va0 = vop(0);
    bf16x8 va1 = vop(1);

    bf16x8 pf[RB][2][2];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      RowBlock<D>& R = rbk[r];
      const bool plain = MODE != 2 && !check_k && !check_mask && R.brow == nullptr && R.qvalid;
      float mloc = -INFINITY;
      if (MODE == 2) {
        // the tile's slice of the folded mask / bias row: -inf drops a key
        // (masked or past Sk); rows past Sq compute values nobody stores
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int kc = 2 * half + c;
#pragma unroll
          for (int sb = 0; sb < 2; ++sb) {
            const float4 c0 = *reinterpret_cast<const float4*>(cbrow + kc * 32 + 16 * sb + 8 * hh);
            const float4 c1 =
                *reinterpret_cast<const float4*>(cbrow + kc * 32 + 16 * sb + 8 * hh + 4);
            const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int u = 8 * sb + e;
              const float sv = fmaf(sacc[r][c][u], p.scale_log2, cv[e]);
              sacc[r][c][u] = sv;
              mloc = fmaxf(mloc, sv);
            }
          }
        }
      } else if (plain) {
        // raw scores: the scale is folded into the exponent below
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int u = 0; u < 16; ++u) mloc = fmaxf(mloc, sacc[r][c][u]);
        mloc *= p.scale_log2;
      } else {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int kc = 2 * half + c;
#pragma unroll
          for (int sb = 0; sb < 2; ++sb) {
            const int kb = k0 + kc * 32 + 16 * sb + 8 * hh;  // 8 consecutive keys
            float bv[8];
            if (MODE == 1 && R.brow) {
              const uint4 raw = *reinterpret_cast<const uint4*>(R.brow + kb);
              const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
              for (int e = 0; e < 8; ++e)
                bv[e] = bias_log2(bf16_to_f32((uint16_t)(wv[e >> 1] >> (16 * (e & 1)))));
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) bv[e] = 0.f;
            }
            uint32_t mbits = 0xFFu;
            if (check_mask) {
              if (MODE == 1 && p.mask_kind == 2) {
                uint2 mb = make_uint2(0, 0);
                if (R.mrow) mb = *reinterpret_cast<const uint2*>(R.mrow + kb);
                mbits = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                  const uint32_t byte = ((e < 4 ? mb.x : mb.y) >> (8 * (e & 3))) & 0xFFu;
                  mbits |= (byte != 0u ? 1u : 0u) << e;
                }
              } else {
                mbits = range_bits(R.iv.lo1, R.iv.hi1, kb) | range_bits(R.iv.lo2, R.iv.hi2, kb);
              }
            }
            if (!R.qvalid) mbits = 0;
            if (check_k) mbits &= range_bits(0, Sk, kb);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int u = 8 * sb + e;
              float sv = sacc[r][c][u] * p.scale_log2 + bv[e];
              sv = ((mbits >> e) & 1u) ? sv : -INFINITY;
              sacc[r][c][u] = sv;
              mloc = fmaxf(mloc, sv);
            }
          }
        }
      }
      mloc = max_pair(mloc);
      // conditional rescale (see kRescaleLog2)
      const bool grow = mloc > R.m_run + kRescaleLog2;
      if (__ballot(grow)) {
        const float m_new = grow ? mloc : R.m_run;
        // 1 where the max is kept (also for rows still at -inf: -inf - -inf is NaN)
        const float alpha = grow ? __builtin_amdgcn_exp2f(R.m_run - m_new) : 1.f;
        R.l_run *= alpha;
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) R.oacc[dc] *= alpha;
        R.m_run = m_new;
      }
      const float m_use = R.m_run == -INFINITY ? 0.f : R.m_run;
      const float mul = plain ? p.scale_log2 : 1.f;
      float lsum = R.l_run;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const int u = 8 * sb + e;
            const float x0 = __builtin_amdgcn_exp2f(fmaf(sacc[r][c][u], mul, -m_use));
            const float x1 = __builtin_amdgcn_exp2f(fmaf(sacc[r][c][u + 1], mul, -m_use));
            const bf16x2 pr = {(__bf16)x0, (__bf16)x1};
            pf[r][c][sb][e] = pr[0];
            pf[r][c][sb][e + 1] = pr[1];
            // row sum of the bf16 probabilities the PV product uses
            lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsum, false);
          }
        }
      }
      R.l_run = lsum;
    }
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int i = 0; i < 4 * NDC; ++i) {
      const int dc = i / 4, c = (i / 2) % 2, sb = i % 2;
      const bf16x8 a = va0;
      va0 = va1;
      if (i + 2 < 4 * NDC) va1 = vop(i + 2);
#pragma unroll
      for (int r = 0; r < RB; ++r)
        rbk[r].oacc[dc] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[r][c][sb], rbk[r].oacc[dc], 0, 0, 0);
    }
  }
}

// MODE 0: no mask tensor and no bias (the DFlash predicate or nothing);
// 1: mask / bias rows read per tile; 2: staged rows (p.staged)
template <int D, int RB, int MODE>
__global__ __launch_bounds__(512 / RB, 1) void k_attn_bf16_v2(AttnParams p, int nWork,
                                                               const WorkOrder order) {
  using C = V2Ctx<D, RB>;
  constexpr int NS = C::NS;
  constexpr int NDC = C::NDC;
  constexpr int WPH = C::NW / 2;  // waves per head
  // K tiles (slots 0, 1), then V tiles (slots 0, 1)
  constexpr int TB = kTile * D * 2;
  __shared__ __align__(1024) char s_kv[4 * TB];
  // the K and V slots
  auto kslot = [&](int sl) { return s_kv + sl * TB; };
  auto vslot = [&](int sl) { return s_kv + (2 + sl) * TB; };
  __shared__ __align__(16) float s_cb[2][2][kTile];  // staged rows: buffer, head of the pair

  // Work items: (head-pair group, query tile). Workgroup L runs on XCD L % 8.
  // When the groups split evenly over the XCDs, XCD x takes groups
  // [x * gx, (x + 1) * gx) and walks them query tile first, heaviest tile first
  // (longest-processing-time order, since a query tile's cost grows with its
  // index under these masks); otherwise each XCD takes a contiguous range.
  const int L = blockIdx.x;
  const int xcd = L % kXcds;
  const int pairs = p.G / 2;
  const int ngrp = nWork / p.nQ;
  int qt, grp;
  if (p.varlen && order.n > 0) {
    // Packed sequences, items in the host's order (heaviest first, by their
    // visible key tiles): KVH * pairs workgroups per item, (KV head, pair)
    // fastest, so a (b, KV head)'s work stays on one XCD.
    const int per = p.KVH * pairs;
    const int it = order.item[L / per];
    const int b = it >> 10;
    qt = it & 1023;
    grp = b * per + L % per;
  } else if (p.varlen) {
    // Packed sequences differ in cost: spread each sequence's groups over the
    // XCDs (group g on XCD g % 8 when the group count is a multiple of 8) and
    // run every group's heaviest (last) query tiles first; tiles past a
    // sequence's end exit at once.
    grp = L % ngrp;
    qt = p.nQ - 1 - L / ngrp;
  } else if (ngrp % kXcds == 0) {
    const int gx = ngrp / kXcds;
    const int li = L / kXcds;
    qt = p.nQ - 1 - li / gx;
    grp = xcd * gx + li % gx;
  } else {
    const int per = nWork / kXcds;
    const int rem = nWork % kXcds;
    const int wi = xcd * per + (xcd < rem ? xcd : rem) + L / kXcds;
    qt = p.nQ - 1 - wi % p.nQ;
    grp = wi / p.nQ;
  }
  const int hp = grp % pairs;
  grp /= pairs;
  const int kvh = grp % p.KVH;
  const int b = grp / p.KVH;
  const SeqView seq = seq_view(p, b);
  if (qt >= seq.nQ) return;  // past a packed sequence's end (uniform)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int h = kvh * p.G + 2 * hp + w / WPH;

  RowBlock<D> rbk[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    RowBlock<D>& R = rbk[r];
    const int q = qt * kTile + ((w % WPH) * RB + r) * 32 + n;
    R.qvalid = q < seq.Sq;
    const __bf16* qrow = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.q_sb +
                         (seq.q0 + q) * p.q_sq + (int64_t)h * p.q_sh;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      R.qf[s] = R.qvalid ? *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * hh) : bf16x8{};
    R.iv = RowIv32{0, 0, 0, 0};
    if (p.mask_kind == 1) {
      const RowIv v = dflash_row(seq.rule, p.pred_row0 ? 0 : q);
      R.iv = RowIv32{(int)v.lo1, (int)v.hi1, (int)v.lo2, (int)v.hi2};
    }
    R.mrow = (MODE == 1 && p.mask_kind == 2 && R.qvalid) ? aux_row(p.mask, 1, b, h, p.G, q)
                                                         : nullptr;
    R.brow = (MODE == 1 && p.has_bias && R.qvalid)
        ? reinterpret_cast<const uint16_t*>(aux_row(p.bias, 2, b, h, p.G, q)) : nullptr;
#pragma unroll
    for (int i = 0; i < NDC; ++i) R.oacc[i] = f32x16{};
    R.m_run = -INFINITY;
    R.l_run = 0.f;
  }
  const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k) + (int64_t)b * p.k_sb +
                        seq.k0 * p.k_sk + (int64_t)kvh * p.k_sh;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(p.v) + (int64_t)b * p.v_sb +
                        seq.k0 * p.v_sk + (int64_t)kvh * p.v_sh;
  LaneOffs<D> off;
  off.init(lane, 2 * TB);
  Loader<D, RB> ld;
  ld.init(kbase, vbase, p.k_sk, p.v_sk, seq.Sk, w, lane);

  // Staged rows: wave 0 loads the tile's 128-key slice of both heads' rows
  // (lanes 0-31 head h, 32-63 head h + 1, 16 bytes each) with the K/V tile.
  const __amdgpu_buffer_rsrc_t cbr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(MODE == 2 ? p.cb + (int64_t)b * p.cb_sb : nullptr), 0,
      MODE == 2 ? (int)(p.cb_sb * 4) : 0, 0x00020000);
  uint32_t cboff = 0;
  if (MODE == 2) {
    const int hs = kvh * p.G + 2 * hp + (lane >> 5);
    const int64_t hc = p.cb_hmode == 1 ? hs : (p.cb_hmode == 2 ? hs / p.G : 0);
    cboff = (uint32_t)(hc * p.cb_sh * 4 + (lane & 31) * 16);
  }
  auto issue_cb = [&](int slot, int kt) {
    if (MODE == 2 && w == 0)
      dma16(cbr, reinterpret_cast<char*>(&s_cb[slot][0][0]), cboff + (uint32_t)kt * (kTile * 4));
  };

  TileList tl;
  tl.init(p, b, kvh * p.G + 2 * hp, qt, seq.nK);  // identical for both heads of the pair
  const int ntiles = tl.count();
  bool full_cur = false, full_nxt = false;
  int kt_cur = ntiles > 0 ? tl.tile(0, full_cur) : 0;
  // the next tile's index is read one step ahead, so that its load has a
  // whole tile to arrive in
  int kt_nxt = ntiles > 1 ? tl.tile(1, full_nxt) : 0;
  if (ntiles > 0) {
    ld.issue_at(kslot(0), vslot(0), kt_cur, wu);
    issue_cb(0, kt_cur);
  }
  // One barrier per tile: it publishes tile i (every wave has awaited its own
  // loads of it) and frees the other buffer (every wave has finished tile
  // i - 1), so the loads of tile i + 1 go out right after it and overlap the
  // whole of tile i's compute.
  auto step = [&](auto slot_c, int it) {
    constexpr int SLOT = decltype(slot_c)::value;
    const int cs = SLOT >= 0 ? SLOT : (it & 1);  // slot of tile it
    wait_vmcnt<0>();
    barrier();
    if (it + 1 < ntiles) {
      ld.issue_at(kslot(cs ^ 1), vslot(cs ^ 1), kt_nxt, wu);
      issue_cb(cs ^ 1, kt_nxt);
    }
    bool full_nn = false;
    const int kt_nn = it + 2 < ntiles ? tl.tile(it + 2, full_nn) : 0;
    if constexpr (MODE == 1)
      compute_tile_halves<D, RB, MODE, SLOT>(s_kv, cs, p, kt_cur, full_cur, rbk, off, lane,
                                             seq.Sk, &s_cb[cs][w / WPH][0]);
    else
      compute_tile<D, RB, MODE, SLOT>(s_kv, cs, p, kt_cur, full_cur, rbk, off, lane, seq.Sk,
                                      &s_cb[cs][w / WPH][0]);
    kt_cur = kt_nxt;
    full_cur = full_nxt;
    kt_nxt = kt_nn;
    full_nxt = full_nn;
  };
  if constexpr (MODE == 0) {
    // fixed slots: no address arithmetic per LDS read
    for (int it = 0; it < ntiles; it += 2) {
      step(std::integral_constant<int, 0>{}, it);
      if (it + 1 < ntiles) step(std::integral_constant<int, 1>{}, it + 1);
    }
  } else {
    // the mask / bias paths keep one copy (two would not fit the registers)
    for (int it = 0; it < ntiles; ++it) step(std::integral_constant<int, -1>{}, it);
  }

#pragma unroll
  for (int r = 0; r < RB; ++r) {
    RowBlock<D>& R = rbk[r];
    const int q = qt * kTile + ((w % WPH) * RB + r) * 32 + n;
    const float l_tot = R.l_run + __shfl_xor(R.l_run, 32, 64);
    if (R.qvalid) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      __bf16* orow = reinterpret_cast<__bf16*>(p.o) + (int64_t)b * p.o_sb +
                     (seq.q0 + q) * p.o_sq + (int64_t)h * p.o_sh;
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(R.oacc[dc][4 * g + e] * inv);
          *reinterpret_cast<bf16x4*>(orow + dc * 32 + 8 * g + 4 * hh) = v4;
        }
      }
      if (p.lse && hh == 0) {
        const float lse =
            l_tot > 0.f ? (R.m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
        p.lse[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + (seq.q0 + q) * p.lse_sq] = lse;
      }
    }
  }
}

// Folded mask / bias rows: cb[b][hc][k] = bias * log2(e) (0 without a bias)
// where the mask keeps key k < Sk, -inf elsewhere. Four keys per thread.
__global__ __launch_bounds__(256) void k_aux_combine(AttnParams p, float* cb, int Hc) {
  const int K4 = p.nK * (kTile / 4);
  const int64_t n = (int64_t)p.B * Hc * K4;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int k0 = (int)(i % K4) * 4;
    const int64_t r = i / K4;
    const int hc = (int)(r % Hc);
    const int b = (int)(r / Hc);
    // an iteration-space head whose row this is
    const int h = p.cb_hmode == 1 ? hc : (p.cb_hmode == 2 ? hc * p.G : 0);
    const uint8_t* mrow = p.mask_kind == 2 ? aux_row(p.mask, 1, b, h, p.G, 0) : nullptr;
    const uint16_t* brow =
        p.has_bias ? reinterpret_cast<const uint16_t*>(aux_row(p.bias, 2, b, h, p.G, 0)) : nullptr;
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = k0 + e;
      const bool keep = k < p.Sk && (mrow == nullptr || mrow[k] != 0);
      o[e] = keep ? (brow ? bias_log2(bf16_to_f32(brow[k])) : 0.f) : -INFINITY;
    }
    *reinterpret_cast<float4*>(cb + r * ((int64_t)p.nK * kTile) + k0) =
        make_float4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace

namespace {
// head rule and head count of the folded rows
void staged_heads(const AttnParams& p, int& hmode, int& Hc) {
  const int mm = p.mask_kind == 2 ? p.mask.h_mode : 0;
  const int bm = p.has_bias ? p.bias.h_mode : 0;
  hmode = (mm == 1 || bm == 1) ? 1 : ((mm == 2 || bm == 2) ? 2 : 0);
  Hc = hmode == 1 ? p.H : (hmode == 2 ? p.KVH : 1);
}
}  // namespace

bool staged_aux_applies(const AttnParams& p) {
  if (p.varlen || p.gather || p.mask_kind == 1) return false;
  if (p.mask_kind != 2 && !p.has_bias) return false;
  if (p.mask_kind == 2 && !p.mask.q_bcast) return false;
  if (p.has_bias && !p.bias.q_bcast) return false;
  int hmode, Hc;
  staged_heads(p, hmode, Hc);
  return (int64_t)Hc * p.nK * kTile * 4 < ((int64_t)1 << 31);  // 32-bit buffer offsets
}

int64_t staged_aux_bytes(const AttnParams& p) {
  int hmode, Hc;
  staged_heads(p, hmode, Hc);
  const int64_t n = (int64_t)p.B * Hc * p.nK * kTile * 4;
  return (n + 255) / 256 * 256;
}

hipError_t launch_aux_combine(AttnParams& p, void* ws, hipStream_t s) {
  int hmode, Hc;
  staged_heads(p, hmode, Hc);
  p.staged = 1;
  p.cb_hmode = hmode;
  p.cb = static_cast<const float*>(ws);
  p.cb_sh = (int64_t)p.nK * kTile;
  p.cb_sb = Hc * p.cb_sh;
  const int64_t n = (int64_t)p.B * Hc * p.nK * (kTile / 4);
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_aux_combine, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256),
                     0, s, p, static_cast<float*>(ws), Hc);
  return hipGetLastError();
}

bool attn_v2_applies(const AttnParams& p, int D) {
  if (D != 64 && D != 128) return false;
  // 32-bit buffer offsets within one (b, kv head)
  if ((int64_t)p.Sk * p.k_sk * 2 >= (int64_t)1 << 31) return false;
  if ((int64_t)p.Sk * p.v_sk * 2 >= (int64_t)1 << 31) return false;
  if (p.G % 2) return false;
  if (p.has_bm && p.bm.h_mode == 1) return false;  // per-head tile lists
  return true;
}

hipError_t launch_attn_bf16_v2(const AttnParams& p, int D, hipStream_t s,
                               const WorkOrder* order) {
  static const WorkOrder kNoOrder{};  // n = 0
  const WorkOrder& ord = (order && p.varlen) ? *order : kNoOrder;
  const int nWork = ord.n > 0 ? ord.n * p.KVH * (p.G / 2) : p.B * p.KVH * (p.G / 2) * p.nQ;
  if (nWork == 0) return hipSuccess;
  constexpr int RB = 1;  // one 32-row block per wave (the 512-thread layout)
  const dim3 grid(nWork);
  const int mode = p.staged ? 2 : ((p.mask_kind == 2 || p.has_bias) ? 1 : 0);
  if (D == 128) {
    constexpr int NT = V2Ctx<128, RB>::NT;
    if (mode == 2)
      hipLaunchKernelGGL((k_attn_bf16_v2<128, RB, 2>), grid, dim3(NT), 0, s, p, nWork, ord);
    else if (mode == 1)
      hipLaunchKernelGGL((k_attn_bf16_v2<128, RB, 1>), grid, dim3(NT), 0, s, p, nWork, ord);
    else
      hipLaunchKernelGGL((k_attn_bf16_v2<128, RB, 0>), grid, dim3(NT), 0, s, p, nWork, ord);
  } else {
    constexpr int NT = V2Ctx<64, RB>::NT;
    if (mode == 2)
      hipLaunchKernelGGL((k_attn_bf16_v2<64, RB, 2>), grid, dim3(NT), 0, s, p, nWork, ord);
    else if (mode == 1)
      hipLaunchKernelGGL((k_attn_bf16_v2<64, RB, 1>), grid, dim3(NT), 0, s, p, nWork, ord);
    else
      hipLaunchKernelGGL((k_attn_bf16_v2<64, RB, 0>), grid, dim3(NT), 0, s, p, nWork, ord);
  }
  return hipGetLastError();
}

}  // namespace bsm
