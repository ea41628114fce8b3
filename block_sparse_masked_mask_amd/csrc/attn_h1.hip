// Masked attention forward, bf16, one head per workgroup (gfx950), with
// 64-key sub-tiles: no mask, the DFlash predicate, or a dense bool mask and /
// or an additive bias read row by row.
//
// Same arithmetic as k_attn_bf16_v2 (S^T = K Q^T and O^T += V^T P^T on
// v_mfma_f32_32x32x16_bf16, float online softmax with the running max raised
// only past kRescaleLog2, full tiles without a mask test; flash-sparse-
// attention PR #190, Design; SpecForge issue #452). The layout differs:
//
//  * 256 threads = 4 waves take the 128 query rows of one head (32 each); a
//    block-mask tile of 128 keys is visited as two sub-tiles of 64 keys.
//  * K and V sub-tiles are double buffered in 64 KiB of LDS (LDS-DMA loads,
//    the swizzled row layout of attn_pipe.h), so two workgroups share a CU.
//    The two waves on each SIMD then belong to different workgroups with no
//    barrier between them: they drift out of step, and one's softmax runs
//    while the other's MFMAs do, without any explicit scheduling.
//  * Work items (b, head, query tile) keep the heads of a (b, KV head) on one
//    XCD (one L2 per XCD) and run the heaviest query tiles first.
#include <math.h>

#include <type_traits>

#include "attn_common.h"
#include "attn_pipe.h"
#include "bsm_internal.h"
#include "dflash_rows.h"

namespace bsm {
namespace {

using namespace pipe;

constexpr int kSub = 64;  // keys per sub-tile

// Loads of one K or V sub-tile by the workgroup's 4 waves (16-byte LDS-DMA
// chunks). Chunk j of a lane lies 256 / (D / 8) * j rows below chunk 0; the
// swizzles depend only on low row bits that this leaves alone, so each chunk
// adds a scalar offset to one vector offset per tensor.
template <int D>
struct SubLoader {
  static constexpr int CPR = D / 8;
  static constexpr int LOADS = kSub * D * 2 / (256 * 16);
  static constexpr int ROWS = 256 / CPR;
  uint32_t koff, voff, kstep, vstep, ksub, vsub;
  __amdgpu_buffer_rsrc_t kr, vr;

  __device__ inline void init(const void* kbase, const void* vbase, int64_t k_sk, int64_t v_sk,
                              int Sk, int w, int lane) {
    kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(kbase), 0,
                                           (int)((int64_t)Sk * k_sk * 2), 0x00020000);
    vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(vbase), 0,
                                           (int)((int64_t)Sk * v_sk * 2), 0x00020000);
    const int f = w * 64 + lane;
    const int r = f / CPR;
    const int c = f % CPR;
    koff = (uint32_t)(r * k_sk * 2 + ((c ^ swz_k<D>(r)) * 16));
    voff = (uint32_t)(r * v_sk * 2 + ((c ^ swz_v<D>(r)) * 16));
    kstep = (uint32_t)(ROWS * k_sk * 2);
    vstep = (uint32_t)(ROWS * v_sk * 2);
    ksub = (uint32_t)(kSub * k_sk * 2);
    vsub = (uint32_t)(kSub * v_sk * 2);
  }
  // sub-tile st (keys 64 st ..) into the LDS bytes at lk and lv (w uniform)
  __device__ inline void issue(char* lk, char* lv, int st, int w) const {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int slot = (j * 4 + w) * 64 * 16;
      dma16(kr, lk + slot, koff, (uint32_t)j * kstep + (uint32_t)st * ksub);
      dma16(vr, lv + slot, voff, (uint32_t)j * vstep + (uint32_t)st * vsub);
    }
  }
};

template <int D>
struct H1Row {
  bf16x8 qf[D / 16];
  f32x16 oacc[D / 32];
  float m_run, l_run;
  RowIv32 iv;
  const uint8_t* mrow;   // mask row or null
  const uint16_t* brow;  // bias row or null
  bool qvalid;
};

// One 64-key sub-tile (keys k0 ..) in buffer SLOT: S^T of its two 32-key
// chunks, one max (and at most one rescale) per row, the probabilities, PV.
// MODE 1: the row's dense mask bytes and / or bias values enter the scores.
template <int D, int MODE, int SLOT>
__device__ __attribute__((always_inline)) inline void sub_tile(const char* lds,
                                                               const AttnParams& p, int k0,
                                                               bool is_full, H1Row<D>& R,
                                                               const LaneOffs<D>& off, int lane,
                                                               int Sk) {
  constexpr int NS = D / 16;
  constexpr int NDC = D / 32;
  constexpr int SB = kSub * D * 2;  // bytes of one sub-tile
  const int hh = lane >> 5;
  const bool check_k = k0 + kSub > Sk;
  const bool check_mask = !is_full && p.mask_kind != 0;
  const char* kbase = lds + SLOT * SB;
  const char* vbase = lds + SLOT * SB;  // the V buffers' 2 * SB is in the lane offsets
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  f32x16 sacc[2];
  {
    auto kop = [&](int i) {
      const int c = i / NS, s = i % NS;
      return *reinterpret_cast<const bf16x8*>(kbase + off.k[s] + c * 32 * D * 2);
    };
    constexpr int PK = 5;
    bf16x8 ka[PK];
#pragma unroll
    for (int j = 0; j < PK; ++j) ka[j] = kop(j);
#pragma unroll
    for (int i = 0; i < 2 * NS; ++i) {
      const int c = i / NS, s = i % NS;
      const bf16x8 a = ka[i % PK];
      if (i + PK < 2 * NS) ka[i % PK] = kop(i + PK);
      sacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, R.qf[s], s == 0 ? f32x16{} : sacc[c],
                                                        0, 0, 0);
    }
    pin_reads_ahead<2 * NS, PK, 1, 1>();
  }
  // V operand i: key chunk c = i / (2 NDC), d-chunk dc = (i / 2) % NDC,
  // 16-key step sb = i % 2
  auto vop = [&](int i) {
    const int c = i / (2 * NDC), dc = (i / 2) % NDC, sb = i % 2;
    const char* a0 = vbase + off.v[dc] + (c * 32 + 16 * sb) * D * 2;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0 + 4 * D * 2));
    return __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo),
                                   __builtin_bit_cast(bf16x4, hi), 0, 1, 2, 3, 4, 5, 6, 7);
  };
  constexpr int NPV = 4 * NDC;
  constexpr int PV = 3;
  bf16x8 va[PV];
#pragma unroll
  for (int j = 0; j < PV; ++j) va[j] = vop(j);

  const bool plain = !check_k && !check_mask && R.qvalid && (MODE == 0 || R.brow == nullptr);
  float mloc = -INFINITY;
  if (plain) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int u = 0; u < 16; ++u) mloc = fmaxf(mloc, sacc[c][u]);
    mloc *= p.scale_log2;
  } else {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int kb = k0 + c * 32 + 16 * sb + 8 * hh;  // 8 consecutive keys
        float bv[8];
        if (MODE == 1 && R.brow) {
          bias8_log2(R.brow + kb, bv);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) bv[e] = 0.f;
        }
        uint32_t mbits = 0xFFu;
        if (check_mask) {
          if (MODE == 1 && p.mask_kind == 2) {
            uint2 mb = make_uint2(0, 0);
            if (R.mrow) mb = *reinterpret_cast<const uint2*>(R.mrow + kb);
            mbits = byte_bits8(mb);
          } else {
            mbits = range_bits(R.iv.lo1, R.iv.hi1, kb) | range_bits(R.iv.lo2, R.iv.hi2, kb);
          }
        }
        if (!R.qvalid) mbits = 0;
        if (check_k) mbits &= range_bits(0, Sk, kb);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int u = 8 * sb + e;
          float sv = sacc[c][u] * p.scale_log2 + bv[e];
          sv = ((mbits >> e) & 1u) ? sv : -INFINITY;
          sacc[c][u] = sv;
          mloc = fmaxf(mloc, sv);
        }
      }
    }
  }
  mloc = max_pair(mloc);
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
  bf16x8 pf[2][2];
  float lsum = R.l_run;
  auto probs = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int u = 8 * sb + e;
        const float x0 = __builtin_amdgcn_exp2f(fmaf(sacc[c][u], mul, -m_use));
        const float x1 = __builtin_amdgcn_exp2f(fmaf(sacc[c][u + 1], mul, -m_use));
        const bf16x2 pr = {(__bf16)x0, (__bf16)x1};
        pf[c][sb][e] = pr[0];
        pf[c][sb][e + 1] = pr[1];
        lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsum, false);
      }
    }
  };
  probs(0);
  __builtin_amdgcn_sched_barrier(0);
  // PV chunk by chunk (each accumulator sees the keys in order), with chunk
  // 1's probabilities issued between chunk 0's MFMAs
#pragma unroll
  for (int i = 0; i < NPV; ++i) {
    const int c = i / (2 * NDC), dc = (i / 2) % NDC, sb = i % 2;
    const bf16x8 a = va[i % PV];
    if (i + PV < NPV) va[i % PV] = vop(i + PV);
    R.oacc[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[c][sb], R.oacc[dc], 0, 0, 0);
    if (i == 0) probs(1);
  }
  R.l_run = lsum;
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * PV, 0);
#pragma unroll
  for (int i = 0; i < NPV; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i + PV < NPV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    if (i < 2 * NDC) __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
  }
}

template <int D, int MODE>
__global__ __launch_bounds__(256, 2) void k_attn_bf16_h1(AttnParams p, int nWork) {
  constexpr int NS = D / 16;
  constexpr int NDC = D / 32;
  constexpr int SB = kSub * D * 2;
  __shared__ __align__(1024) char s_kv[4 * SB];  // K sub-tiles 0, 1, then V sub-tiles 0, 1

  // Work items (b, head, query tile), workgroup L on XCD L % 8. When the
  // (b, KV head) groups split evenly over the XCDs, XCD x takes groups
  // [x gx, (x + 1) gx) and walks them query tile first, heaviest first;
  // otherwise each XCD takes a contiguous range of (group, query tile, head).
  const int L = blockIdx.x;
  const int xcd = L % kXcds;
  const int ngrp = p.B * p.KVH;
  int qt, grp, hg;
  if (ngrp % kXcds == 0) {
    const int gx = ngrp / kXcds;
    const int li = L / kXcds;
    const int per_q = gx * p.G;
    qt = p.nQ - 1 - li / per_q;
    const int rem = li % per_q;
    grp = xcd * gx + rem / p.G;
    hg = rem % p.G;
  } else {
    const int per = nWork / kXcds;
    const int rem8 = nWork % kXcds;
    const int wi = xcd * per + (xcd < rem8 ? xcd : rem8) + L / kXcds;
    hg = wi % p.G;
    qt = p.nQ - 1 - (wi / p.G) % p.nQ;
    grp = wi / (p.G * p.nQ);
  }
  const int kvh = grp % p.KVH;
  const int b = grp / p.KVH;
  const int h = kvh * p.G + hg;
  const SeqView seq = seq_view(p, b);
  if (qt >= seq.nQ) return;  // past a packed sequence's end (uniform)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int q = qt * kTile + w * 32 + n;

  H1Row<D> R;
  R.qvalid = q < seq.Sq;
  {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.q_sb +
                         (seq.q0 + q) * p.q_sq + (int64_t)h * p.q_sh;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      R.qf[s] = R.qvalid ? *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * hh) : bf16x8{};
  }
  R.mrow = (MODE == 1 && p.mask_kind == 2 && R.qvalid) ? aux_row(p.mask, 1, b, h, p.G, q)
                                                        : nullptr;
  R.brow = (MODE == 1 && p.has_bias && R.qvalid)
               ? reinterpret_cast<const uint16_t*>(aux_row(p.bias, 2, b, h, p.G, q))
               : nullptr;
  R.iv = RowIv32{0, 0, 0, 0};
  if (p.mask_kind == 1) {
    const RowIv v = dflash_row(seq.rule, p.pred_row0 ? 0 : q);
    R.iv = RowIv32{(int)v.lo1, (int)v.hi1, (int)v.lo2, (int)v.hi2};
  }
#pragma unroll
  for (int i = 0; i < NDC; ++i) R.oacc[i] = f32x16{};
  R.m_run = -INFINITY;
  R.l_run = 0.f;

  const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k) + (int64_t)b * p.k_sb +
                        seq.k0 * p.k_sk + (int64_t)kvh * p.k_sh;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(p.v) + (int64_t)b * p.v_sb +
                        seq.k0 * p.v_sk + (int64_t)kvh * p.v_sh;
  LaneOffs<D> off;
  off.init(lane, 2 * SB);
  SubLoader<D> ld;
  ld.init(kbase, vbase, p.k_sk, p.v_sk, seq.Sk, w, lane);
  auto kslot = [&](int sl) { return s_kv + sl * SB; };
  auto vslot = [&](int sl) { return s_kv + (2 + sl) * SB; };

  TileList tl;
  tl.init(p, b, h, qt, seq.nK);
  const int nsub = 2 * tl.count();
  // sub-tile j: half j % 2 of visit j / 2
  bool full_cur = false, full_nxt = false, full_nn = false;
  int kt_cur = nsub > 0 ? tl.tile(0, full_cur) : 0;
  int kt_nxt = kt_cur;
  full_nxt = full_cur;
  // the next visit's tile, read a visit ahead of its first load
  int kt_nn = nsub > 2 ? tl.tile(1, full_nn) : 0;
  if (nsub > 0) ld.issue(kslot(0), vslot(0), 2 * kt_cur, wu);
  // One barrier per sub-tile: it publishes sub-tile j and frees the other
  // buffer, so the loads of j + 1 overlap the compute of j.
  auto step = [&](auto slot_c, int j) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_c)::value;
    wait_vmcnt<0>();
    barrier();
    // visit and half of sub-tile j + 1
    if (j + 1 < nsub) {
      if ((j & 1) == 1) {  // sub-tile j + 1 opens visit (j + 1) / 2
        kt_nxt = kt_nn;
        full_nxt = full_nn;
        kt_nn = j + 3 < nsub ? tl.tile((j + 3) >> 1, full_nn) : 0;
      }
      ld.issue(kslot(SLOT ^ 1), vslot(SLOT ^ 1), 2 * kt_nxt + ((j + 1) & 1), wu);
    }
    sub_tile<D, MODE, SLOT>(s_kv, p, kt_cur * kTile + (j & 1) * kSub, full_cur, R, off, lane, seq.Sk);
    kt_cur = kt_nxt;
    full_cur = full_nxt;
  };
  for (int j = 0; j < nsub; j += 2) {
    step(std::integral_constant<int, 0>{}, j);
    step(std::integral_constant<int, 1>{}, j + 1);
  }

  const float l_tot = R.l_run + __shfl_xor(R.l_run, 32, 64);
  if (R.qvalid) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    __bf16* orow = reinterpret_cast<__bf16*>(p.o) + (int64_t)b * p.o_sb + (seq.q0 + q) * p.o_sq +
                   (int64_t)h * p.o_sh;
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
      const float lse = l_tot > 0.f ? (R.m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
      p.lse[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + (seq.q0 + q) * p.lse_sq] = lse;
    }
  }
}

}  // namespace

bool attn_h1_applies(const AttnParams& p, int D) {
  if (D != 64 && D != 128) return false;
  if (p.staged) return false;
  // 32-bit buffer offsets within one (b, kv head)
  if ((int64_t)p.Sk * p.k_sk * 2 >= (int64_t)1 << 31) return false;
  if ((int64_t)p.Sk * p.v_sk * 2 >= (int64_t)1 << 31) return false;
  return true;
}

hipError_t launch_attn_bf16_h1(const AttnParams& p, int D, hipStream_t s) {
  const int nWork = p.B * p.H * p.nQ;
  if (nWork == 0) return hipSuccess;
  const bool aux = p.mask_kind == 2 || p.has_bias;
  if (D == 128) {
    if (aux)
      hipLaunchKernelGGL((k_attn_bf16_h1<128, 1>), dim3(nWork), dim3(256), 0, s, p, nWork);
    else
      hipLaunchKernelGGL((k_attn_bf16_h1<128, 0>), dim3(nWork), dim3(256), 0, s, p, nWork);
  } else {
    if (aux)
      hipLaunchKernelGGL((k_attn_bf16_h1<64, 1>), dim3(nWork), dim3(256), 0, s, p, nWork);
    else
      hipLaunchKernelGGL((k_attn_bf16_h1<64, 0>), dim3(nWork), dim3(256), 0, s, p, nWork);
  }
  return hipGetLastError();
}

}  // namespace bsm
