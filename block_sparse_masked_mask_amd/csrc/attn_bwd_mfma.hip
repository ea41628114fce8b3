// Masked attention backward on the bf16 matrix cores (gfx950), D = 128: the
// training path of the DFlash layers (no mask or the DFlash predicate) and of
// masked calls with a dense bool mask and / or an additive bias, with dbias.
//
// Same gradients as the generic kernels (attn_bwd.hip; flash-sparse-attention
// PR #190, Changes: mha_bwd): P = exp(s - LSE) on kept keys, dS = P (dP - Delta)
// with dP = dO V^T and Delta = rowsum(dO * O); dQ = scale dS K, dK = scale dS^T Q,
// dV = P^T dO, all products on v_mfma_f32_32x32x16_bf16 with float accumulation
// and P, dS rounded to bf16 as MFMA operands.
//
//  * dQ: one workgroup per (b, h, query tile), 4 waves of 32 rows; K and V tiles
//    go through LDS. Per 32-key chunk: S^T = K Q^T and dP^T = V dO^T with Q and
//    dO rows held in registers, then dQ^T += K^T dS^T with K^T from transposed
//    LDS reads. Keys are permuted (bits 2 and 3 of the MFMA row swapped) so that
//    a lane's accumulators hold 8 consecutive keys of its row: the B-operand
//    layout of the dQ product, and the layout the row's interval test uses.
//  * dK / dV: one workgroup per (b, KV head, key tile), 4 waves of 32 keys,
//    visiting every (head of the group, query tile) whose tile is not empty.
//    Per 32-row block: S = Q K^T and dP = dO V^T with the wave's K and V rows
//    held in registers and query rows permuted the same way, then
//    dV^T += dO^T P and dK^T += Q^T dS with transposed LDS reads of dO and Q.
//    Partial tiles use a keep-bit table of the query tile built in LDS (one
//    64-key word per row and half tile) from the predicate or the mask bytes.
//  * Bias: added to the scores in log2 units (bias_log2) wherever P is formed.
//    dbias = dS summed over the dims where the bias broadcasts: the dK / dV
//    workgroup holds every (head of its group, query) of its keys, so a bias
//    broadcast over queries is summed per key in a register and added once
//    per target row (float atomics only across workgroups: batches or KV
//    groups sharing a bias row); a bias per query takes one atomic add per
//    (query, key) and head.
//  * A mask and / or bias that broadcast over queries can come folded into one
//    float row per (b, head of the broadcast) (f.staged: the bias in log2
//    units, -inf where the mask drops a key or past Sk; [FSA-190] Design),
//    which both kernels read in place of keep bits and bias values.
//  * Packed sequences (f.varlen, the two-head dQ kernel and dK / dV): a work
//    item reads its sequence's rows, keys and DFlash geometry through
//    seq_view, items come in the host's order (heaviest first) when given, and
//    those past a sequence's tiles exit at once ([FSA-197] Changes: varlen).
#include <math.h>

#include "attn_common.h"
#include "attn_pipe.h"
#include "block_scan.h"
#include "bsm_internal.h"
#include "dflash_rows.h"

namespace bsm {
namespace {

using namespace pipe;

constexpr int kD = 128;
constexpr int kNS = kD / 16;    // 16-wide d steps
constexpr int kNDC = kD / 32;   // 32-wide d chunks
constexpr int kRowB = kD * 2;   // bytes per bf16 row
constexpr int kAhead = 3;       // row operands (d-steps) read ahead of their MFMAs
constexpr int kTrAhead = 2;     // transposed operands read ahead
constexpr int kThreads = 256;
constexpr int kMaxVisits = 4096;  // (head, query tile) positions listed in LDS by dK / dV

// 128 x 128 bf16 tile in LDS, rows swizzled in 16-byte chunks like the forward's
// K tiles (conflict-free row reads).
struct Tile {
  __bf16 e[kTile * kD];
};

// Cooperative copy of rows r0 .. r0+127 of a (rows, stride) bf16 matrix into t;
// rows >= nrows are zero.
__device__ inline void load_tile(Tile& t, const __bf16* base, int64_t stride, int r0, int nrows,
                                 int tid) {
#pragma unroll
  for (int j = 0; j < kTile * kD / 8 / kThreads; ++j) {
    const int f = j * kThreads + tid;
    const int r = f / (kD / 8);
    const int c = f % (kD / 8);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r0 + r < nrows)
      v = *reinterpret_cast<const uint4*>(base + (int64_t)(r0 + r) * stride + c * 8);
    *reinterpret_cast<uint4*>(reinterpret_cast<char*>(t.e) + r * kRowB +
                              ((c ^ swz_k<kD>(r)) * 16)) = v;
  }
}

// 16-byte chunk swizzle of a tile row: the K-tile one, or (VSW) the V-tile one
// the LDS-DMA loader applies to its second tensor.
template <bool VSW>
__device__ inline int swz(int r) {
  return VSW ? swz_v<kD>(r) : swz_k<kD>(r);
}

// Row operand (A of a 32x32x16 MFMA): rows rb*32 + perm_row(n), d-step s.
template <bool VSW = false>
__device__ inline bf16x8 row_op(const __bf16* t, int rb, int s, int lane) {
  const int row = rb * 32 + perm_row(lane & 31);
  const int hh = lane >> 5;
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(t) + row * kRowB +
                                          (((2 * s + hh) ^ swz<VSW>(row)) * 16));
}
__device__ inline bf16x8 row_op(const Tile& t, int rb, int s, int lane) {
  return row_op<false>(t.e, rb, s, lane);
}

// Transposed operand (A of a 32x32x16 MFMA over the tile's rows): d = 32 dc +
// (lane % 32), rows kb .. kb+15 of the tile with lane holding 8 consecutive
// rows (two 4-row transposed reads).
template <bool VSW = false>
__device__ inline bf16x8 col_op(const __bf16* t, int dc, int kb, int lane) {
  const int blk = lane >> 4;
  const int e4 = (lane >> 2) & 3;
  const int g4 = lane & 3;
  const int chunk = 4 * dc + 2 * (blk & 1) + (g4 >> 1);
  const int row0 = kb + 8 * (blk >> 1) + e4;
  const int row1 = row0 + 4;
  const char* b = reinterpret_cast<const char*>(t);
  const char* a0 = b + row0 * kRowB + ((chunk ^ swz<VSW>(row0)) * 16) + (g4 & 1) * 8;
  const char* a1 = b + row1 * kRowB + ((chunk ^ swz<VSW>(row1)) * 16) + (g4 & 1) * 8;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a1));
  return __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi),
                                 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ inline bf16x8 col_op(const Tile& t, int dc, int kb, int lane) {
  return col_op<false>(t.e, dc, kb, lane);
}

__device__ inline bf16x8 pack8(const float* x) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[e];
  return r;
}

// ---------------------------------------------------------------- dQ

// AUX: the call has a dense mask and / or a bias (their code compiles out otherwise)
template <bool AUX>
__global__ __launch_bounds__(kThreads, 2) void k_bwd_dq_mfma(AttnBwdParams P) {
  const AttnParams& f = P.f;
  __shared__ __align__(1024) Tile sk;
  __shared__ __align__(1024) Tile sv;
  const int qt = blockIdx.x % f.nQ;
  const int bh = blockIdx.x / f.nQ;
  const int h = bh % f.H;
  const int b = bh / f.H;
  const int kvh = h / f.G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int q = qt * kTile + 32 * w + n;
  const bool qvalid = q < f.Sq;

  // this lane's row: Q and dO operands (B of S^T = K Q^T and dP^T = V dO^T)
  bf16x8 qf[kNS], df[kNS];
  {
    const __bf16* qr = reinterpret_cast<const __bf16*>(f.q) + (int64_t)b * f.q_sb +
                       (int64_t)q * f.q_sq + (int64_t)h * f.q_sh;
    const __bf16* dr = reinterpret_cast<const __bf16*>(P.dout) + (int64_t)b * P.do_sb +
                       (int64_t)q * P.do_sq + (int64_t)h * P.do_sh;
#pragma unroll
    for (int s = 0; s < kNS; ++s) {
      qf[s] = qvalid ? *reinterpret_cast<const bf16x8*>(qr + 16 * s + 8 * hh) : bf16x8{};
      df[s] = qvalid ? *reinterpret_cast<const bf16x8*>(dr + 16 * s + 8 * hh) : bf16x8{};
    }
  }
  const float lse2 =
      qvalid ? f.lse[(int64_t)b * f.lse_sb + (int64_t)h * f.lse_sh + (int64_t)q * f.lse_sq] *
                   kLog2e
             : -INFINITY;
  const float delta = qvalid ? P.delta[(int64_t)b * P.delta_sb + (int64_t)h * P.delta_sh + q] : 0.f;
  const bool live = lse2 != -INFINITY;  // rows with no kept key have zero gradients
  const uint8_t* mrow = (AUX && f.mask_kind == 2 && qvalid) ? aux_row(f.mask, 1, b, h, f.G, q) : nullptr;
  const uint16_t* brow = (AUX && f.has_bias && qvalid)
      ? reinterpret_cast<const uint16_t*>(aux_row(f.bias, 2, b, h, f.G, q)) : nullptr;
  RowIv32 iv{0, 0, 0, 0};
  if (f.mask_kind == 1) {
    const RowIv v = dflash_row(f.rule, f.pred_row0 ? 0 : q);
    iv = RowIv32{(int)v.lo1, (int)v.hi1, (int)v.lo2, (int)v.hi2};
  }
  f32x16 dq[kNDC];
#pragma unroll
  for (int i = 0; i < kNDC; ++i) dq[i] = f32x16{};

  const __bf16* kbase = reinterpret_cast<const __bf16*>(f.k) + (int64_t)b * f.k_sb +
                        (int64_t)kvh * f.k_sh;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(f.v) + (int64_t)b * f.v_sb +
                        (int64_t)kvh * f.v_sh;
  TileList tl;
  tl.init(f, b, h, qt);
  const int ntiles = tl.count();
  for (int it = 0; it < ntiles; ++it) {
    bool full;
    const int kt = tl.tile(it, full);
    const int k0 = kt * kTile;
    __syncthreads();  // previous tile's readers are done
    load_tile(sk, kbase, f.k_sk, k0, f.Sk, tid);
    load_tile(sv, vbase, f.v_sk, k0, f.Sk, tid);
    __syncthreads();
    const bool test = !full || k0 + kTile > f.Sk || !qvalid;
#pragma unroll
    for (int c = 0; c < kTile / 32; ++c) {
      f32x16 st = f32x16{}, dpt = f32x16{};
#pragma unroll
      for (int s = 0; s < kNS; ++s) {
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_op(sk, c, s, lane), qf[s], st, 0, 0, 0);
        dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_op(sv, c, s, lane), df[s], dpt, 0, 0,
                                                      0);
      }
      // lane: row q, keys k0 + 32 c + 16 sb + 8 hh + e (e = 0..7) for value 8 sb + e
      float ds[16];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int kb = k0 + 32 * c + 16 * sb + 8 * hh;
        uint32_t bits = 0xFFu;
        if (test) {
          // partial tiles test the row's predicate intervals or mask bytes;
          // keys past Sk and rows past Sq keep nothing
          if (!full && f.mask_kind == 1)
            bits = range_bits(iv.lo1, iv.hi1, kb) | range_bits(iv.lo2, iv.hi2, kb);
          if (AUX && !full && f.mask_kind == 2)
            bits = mrow ? byte_bits8(*reinterpret_cast<const uint2*>(mrow + kb)) : 0u;
          bits &= range_bits(0, f.Sk, kb);
          if (!qvalid) bits = 0;
        }
        float bv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (AUX && brow) bias8_log2(brow + kb, bv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int u = 8 * sb + e;
          const float pr = (live && ((bits >> e) & 1u))
                               ? __builtin_amdgcn_exp2f(fmaf(st[u], f.scale_log2, bv[e] - lse2))
                               : 0.f;
          ds[u] = pr * (dpt[u] - delta);
        }
      }
      const bf16x8 d0 = pack8(ds), d1 = pack8(ds + 8);
#pragma unroll
      for (int dc = 0; dc < kNDC; ++dc) {
        dq[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(col_op(sk, dc, 32 * c, lane), d0, dq[dc],
                                                         0, 0, 0);
        dq[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(col_op(sk, dc, 32 * c + 16, lane), d1,
                                                         dq[dc], 0, 0, 0);
      }
    }
  }
  // dQ^T accumulators: lane holds d = 32 dc + 8 (r / 4) + 4 hh + r % 4 of row q
  if (qvalid) {
    __bf16* out = reinterpret_cast<__bf16*>(P.dq) + (int64_t)b * P.dq_sb + (int64_t)q * P.dq_sq +
                  (int64_t)h * P.dq_sh;
#pragma unroll
    for (int dc = 0; dc < kNDC; ++dc) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(dq[dc][4 * g + e] * P.scale);
        *reinterpret_cast<bf16x4*>(out + dc * 32 + 8 * g + 4 * hh) = v4;
      }
    }
  }
}

// ------------------------------------------------- dQ, pipelined
//
// The layout of the pipelined forward (attn_v2.hip): 512 threads, K and V
// tiles reach LDS by LDS-DMA, double buffered, V with its transposed-read
// swizzle. Per 32-key chunk: S^T = K Q^T, dP^T = V dO^T, dS, then
// dQ^T += K^T dS^T. HP = 2: waves 0-3 take 128 query rows of head h and waves
// 4-7 the same rows of head h + 1 of the same KV group (their block-mask row is
// shared), each wave all 128 keys of a tile. HP = 1 (odd G, per-head block
// masks): one head, waves 0-3 take keys 0-63 of every tile and waves 4-7 keys
// 64-127 for the same 128 rows, and the two partial dQ^T are summed through
// LDS at the end.

// Per-lane LDS byte offsets of the operand reads, computed once. A 32-key chunk
// adds 32 rows, a 16-key step 16 rows: neither changes a swizzle.
struct DqOffs {
  uint32_t krow[kNS];   // K rows (A of S^T): row perm_row(n), chunk 2 s + hh
  uint32_t vrow[kNS];   // V rows (A of dP^T), V swizzle
  uint32_t kc0[kNDC];   // K^T (A of dQ^T): first and second transposed reads
  uint32_t kc1[kNDC];   //   of d chunk dc at key 0
  __device__ inline void init(int lane) {
    const int hh = lane >> 5;
    const int row = perm_row(lane & 31);
#pragma unroll
    for (int s = 0; s < kNS; ++s) {
      krow[s] = (uint32_t)(row * kRowB + (((2 * s + hh) ^ swz_k<kD>(row)) * 16));
      vrow[s] = (uint32_t)(row * kRowB + (((2 * s + hh) ^ swz_v<kD>(row)) * 16));
    }
    const int blk = lane >> 4;
    const int e4 = (lane >> 2) & 3;
    const int g4 = lane & 3;
    const int row0 = 8 * (blk >> 1) + e4;
    const int row1 = row0 + 4;
#pragma unroll
    for (int dc = 0; dc < kNDC; ++dc) {
      const int chunk = 4 * dc + 2 * (blk & 1) + (g4 >> 1);
      kc0[dc] = (uint32_t)(row0 * kRowB + ((chunk ^ swz_k<kD>(row0)) * 16) + (g4 & 1) * 8);
      kc1[dc] = (uint32_t)(row1 * kRowB + ((chunk ^ swz_k<kD>(row1)) * 16) + (g4 & 1) * 8);
    }
  }
};

template <bool AUX, int HP>
__global__ __launch_bounds__(512, 1) void k_bwd_dq_pair(AttnBwdParams P, int nWork,
                                                        const WorkOrder order) {
  static_assert(HP == 1 || HP == 2, "one or two heads per workgroup");
  constexpr int NC = HP == 2 ? kTile / 32 : kTile / 64;  // 32-key chunks per wave and tile
  const AttnParams& f = P.f;
  __shared__ __align__(1024) Tiles<kD> buf0;
  __shared__ __align__(1024) Tiles<kD> buf1;

  // work items (b, KV-group head pair or head, query tile) as in the pipelined forward
  const int L = blockIdx.x;
  const int xcd = L % kXcds;
  const int pairs = f.G / HP;
  const int ngrp = nWork / f.nQ;
  int qt, grp;
  if (f.varlen && order.n > 0) {
    // packed sequences, items (b, query tile) in the host's order (heaviest
    // first), KVH * pairs workgroups per item
    const int per = f.KVH * pairs;
    const int it = order.item[L / per];
    qt = it & 1023;
    grp = (it >> 10) * per + L % per;
  } else if (f.varlen) {
    // every group's heaviest (last) query tiles first, groups spread over the
    // XCDs; tiles past a sequence's end exit at once
    grp = L % ngrp;
    qt = f.nQ - 1 - L / ngrp;
  } else if (ngrp % kXcds == 0) {
    const int gx = ngrp / kXcds;
    const int li = L / kXcds;
    qt = f.nQ - 1 - li / gx;
    grp = xcd * gx + li % gx;
  } else {
    const int per = nWork / kXcds;
    const int rem = nWork % kXcds;
    const int wi = xcd * per + (xcd < rem ? xcd : rem) + L / kXcds;
    qt = f.nQ - 1 - wi % f.nQ;
    grp = wi / f.nQ;
  }
  const int hp = grp % pairs;
  grp /= pairs;
  const int kvh = grp % f.KVH;
  const int b = grp / f.KVH;
  // a packed sequence's rows, keys and DFlash geometry (the batch itself otherwise)
  const SeqView seq = seq_view(f, b);
  if (qt >= seq.nQ) return;  // past a packed sequence's end (uniform)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int h0 = kvh * f.G + HP * hp;
  const int h = HP == 2 ? h0 + (w >> 2) : h0;
  // the key half of every tile (one head); wave-uniform, kept in a scalar register
  const int kh = HP == 2 ? 0 : __builtin_amdgcn_readfirstlane(w >> 2);
  const int q = qt * kTile + 32 * (w & 3) + n;  // row within the sequence
  const bool qvalid = q < seq.Sq;
  const int64_t qg = seq.q0 + q;                 // row of the (packed) tensors

  bf16x8 qf[kNS], df[kNS];
  {
    const __bf16* qr = reinterpret_cast<const __bf16*>(f.q) + (int64_t)b * f.q_sb +
                       qg * f.q_sq + (int64_t)h * f.q_sh;
    const __bf16* dr = reinterpret_cast<const __bf16*>(P.dout) + (int64_t)b * P.do_sb +
                       qg * P.do_sq + (int64_t)h * P.do_sh;
#pragma unroll
    for (int s = 0; s < kNS; ++s) {
      qf[s] = qvalid ? *reinterpret_cast<const bf16x8*>(qr + 16 * s + 8 * hh) : bf16x8{};
      df[s] = qvalid ? *reinterpret_cast<const bf16x8*>(dr + 16 * s + 8 * hh) : bf16x8{};
    }
  }
  const float lse2 =
      qvalid ? f.lse[(int64_t)b * f.lse_sb + (int64_t)h * f.lse_sh + qg * f.lse_sq] *
                   kLog2e
             : -INFINITY;
  const float delta =
      qvalid ? P.delta[(int64_t)b * P.delta_sb + (int64_t)h * P.delta_sh + qg] : 0.f;
  const bool live = lse2 != -INFINITY;
  const bool staged = AUX && f.staged;  // mask and bias folded into one float row
  const uint8_t* mrow =
      (AUX && !staged && f.mask_kind == 2 && qvalid) ? aux_row(f.mask, 1, b, h, f.G, q) : nullptr;
  const uint16_t* brow = (AUX && !staged && f.has_bias && qvalid)
      ? reinterpret_cast<const uint16_t*>(aux_row(f.bias, 2, b, h, f.G, q)) : nullptr;
  const float* cbrow = staged ? f.cb + (int64_t)b * f.cb_sb +
                                    (f.cb_hmode == 1 ? h : (f.cb_hmode == 2 ? h / f.G : 0)) * f.cb_sh
                              : nullptr;
  RowIv32 iv{0, 0, 0, 0};
  if (f.mask_kind == 1) {
    const RowIv v = dflash_row(seq.rule, f.pred_row0 ? 0 : q);
    iv = RowIv32{(int)v.lo1, (int)v.hi1, (int)v.lo2, (int)v.hi2};
  }
  f32x16 dq[kNDC];
#pragma unroll
  for (int i = 0; i < kNDC; ++i) dq[i] = f32x16{};

  DqOffs off;
  off.init(lane);
  Loader<kD, 1> ld;
  ld.init(reinterpret_cast<const __bf16*>(f.k) + (int64_t)b * f.k_sb + seq.k0 * f.k_sk +
              (int64_t)kvh * f.k_sh,
          reinterpret_cast<const __bf16*>(f.v) + (int64_t)b * f.v_sb + seq.k0 * f.v_sk +
              (int64_t)kvh * f.v_sh,
          f.k_sk, f.v_sk, seq.Sk, w, lane);
  TileList tl;
  tl.init(f, b, h0, qt, seq.nK);  // identical for both heads of a pair
  const int ntiles = tl.count();
  bool full_cur = false;
  int kt_cur = ntiles > 0 ? tl.tile(0, full_cur) : 0;
  // Q, dO, LSE and Delta have arrived before the first DMA goes out, so no
  // wait for them inside the loop also waits for a tile
  wait_vmcnt<0>();
  if (ntiles > 0) ld.issue(buf0, kt_cur, w);
  for (int it = 0; it < ntiles; ++it) {
    const Tiles<kD>& cur = (it & 1) ? buf1 : buf0;
    Tiles<kD>& nxt = (it & 1) ? buf0 : buf1;
    bool full_nxt = false;
    const int kt_nxt = it + 1 < ntiles ? tl.tile(it + 1, full_nxt) : 0;
    wait_vmcnt<0>();
    barrier();
    if (it + 1 < ntiles) ld.issue(nxt, kt_nxt, w);

    const int k0 = kt_cur * kTile + 32 * NC * kh;
    const bool test = !full_cur || k0 + 32 * NC > seq.Sk || !qvalid;
    const char* kb = reinterpret_cast<const char*>(cur.k) + 32 * NC * kh * kRowB;
    const char* vb = reinterpret_cast<const char*>(cur.v) + 32 * NC * kh * kRowB;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      f32x16 st = f32x16{}, dpt = f32x16{};
      // row operands kAhead d-steps ahead
      bf16x8 ka[kAhead], va[kAhead];
#pragma unroll
      for (int j = 0; j < kAhead; ++j) {
        ka[j] = *reinterpret_cast<const bf16x8*>(kb + off.krow[j] + c * 32 * kRowB);
        va[j] = *reinterpret_cast<const bf16x8*>(vb + off.vrow[j] + c * 32 * kRowB);
      }
#pragma unroll
      for (int s = 0; s < kNS; ++s) {
        const bf16x8 a = ka[s % kAhead], v = va[s % kAhead];
        if (s + kAhead < kNS) {
          ka[s % kAhead] =
              *reinterpret_cast<const bf16x8*>(kb + off.krow[s + kAhead] + c * 32 * kRowB);
          va[s % kAhead] =
              *reinterpret_cast<const bf16x8*>(vb + off.vrow[s + kAhead] + c * 32 * kRowB);
        }
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], st, 0, 0, 0);
        dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v, df[s], dpt, 0, 0, 0);
      }
      pin_reads_ahead<kNS, kAhead, 2, 2>();
      // lane: row q, keys k0 + 32 c + 16 sb + 8 hh + e for value 8 sb + e
      float ds[16];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int kbk = k0 + 32 * c + 16 * sb + 8 * hh;
        uint32_t bits = 0xFFu;
        if (test) {
          if (!full_cur && f.mask_kind == 1)
            bits = range_bits(iv.lo1, iv.hi1, kbk) | range_bits(iv.lo2, iv.hi2, kbk);
          if (AUX && !staged && !full_cur && f.mask_kind == 2)
            bits = mrow ? byte_bits8(*reinterpret_cast<const uint2*>(mrow + kbk)) : 0u;
          bits &= range_bits(0, seq.Sk, kbk);
          if (!qvalid) bits = 0;
        }
        float bv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (staged) {
          // the folded row: bias in log2 units, -inf where the mask drops a key
          const float4 c0 = *reinterpret_cast<const float4*>(cbrow + kbk);
          const float4 c1 = *reinterpret_cast<const float4*>(cbrow + kbk + 4);
          bv[0] = c0.x, bv[1] = c0.y, bv[2] = c0.z, bv[3] = c0.w;
          bv[4] = c1.x, bv[5] = c1.y, bv[6] = c1.z, bv[7] = c1.w;
        } else if (AUX && brow) {
          bias8_log2(brow + kbk, bv);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int u = 8 * sb + e;
          // computed, then selected: a branch per element would split the
          // block the MFMAs overlap with
          const float ex = __builtin_amdgcn_exp2f(fmaf(st[u], f.scale_log2, bv[e] - lse2));
          const float pr = (live && ((bits >> e) & 1u)) ? ex : 0.f;
          ds[u] = pr * (dpt[u] - delta);
        }
      }
      const bf16x8 d0 = pack8(ds), d1 = pack8(ds + 8);
      // K^T operand i = (d chunk i / 2, 16 keys i % 2), kTrAhead ahead
      auto kop = [&](int i) {
        const int rows = (32 * c + 16 * (i % 2)) * kRowB;
        const i16x4 lo =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(kb + off.kc0[i / 2] + rows));
        const i16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(kb + off.kc1[i / 2] + rows));
        return __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo),
                                       __builtin_bit_cast(bf16x4, hi), 0, 1, 2, 3, 4, 5, 6, 7);
      };
      constexpr int NQ = 2 * kNDC;
      bf16x8 kq[kTrAhead];
#pragma unroll
      for (int j = 0; j < kTrAhead; ++j) kq[j] = kop(j);
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const bf16x8 a = kq[i % kTrAhead];
        if (i + kTrAhead < NQ) kq[i % kTrAhead] = kop(i + kTrAhead);
        dq[i / 2] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, (i % 2) ? d1 : d0, dq[i / 2], 0, 0, 0);
      }
      pin_reads_ahead<NQ, kTrAhead, 2, 1>();
    }
    kt_cur = kt_nxt;
    full_cur = full_nxt;
  }
  if (HP == 1) {
    // waves 4-7 hand their partial dQ^T to waves 0-3 through the (now idle)
    // first K / V buffer: 4 waves x 64 lanes x 64 floats = its 64 KiB
    static_assert(sizeof(Tiles<kD>) == 4 * 64 * 4 * kNDC * 16, "reduction buffer size");
    float4* red = reinterpret_cast<float4*>(&buf0);
    __syncthreads();  // every wave is done with the tiles
    if (kh == 1) {
#pragma unroll
      for (int dc = 0; dc < kNDC; ++dc)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          red[(((w & 3) * kNDC + dc) * 4 + g) * 64 + lane] =
              make_float4(dq[dc][4 * g], dq[dc][4 * g + 1], dq[dc][4 * g + 2], dq[dc][4 * g + 3]);
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int dc = 0; dc < kNDC; ++dc)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 o = red[(((w & 3) * kNDC + dc) * 4 + g) * 64 + lane];
        dq[dc][4 * g] += o.x, dq[dc][4 * g + 1] += o.y;
        dq[dc][4 * g + 2] += o.z, dq[dc][4 * g + 3] += o.w;
      }
  }
  if (qvalid) {
    __bf16* out = reinterpret_cast<__bf16*>(P.dq) + (int64_t)b * P.dq_sb + qg * P.dq_sq +
                  (int64_t)h * P.dq_sh;
#pragma unroll
    for (int dc = 0; dc < kNDC; ++dc) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(dq[dc][4 * g + e] * P.scale);
        *reinterpret_cast<bf16x4*>(out + dc * 32 + 8 * g + 4 * hh) = v4;
      }
    }
  }
}

// ---------------------------------------------------------------- dK / dV

__device__ inline int tile_class_of(const AttnParams& f, int b, int h, int qt, int kt) {
  if (!f.has_bm) return f.mask_kind == 0 ? 2 : 1;
  const BlockMaskView& m = f.bm;
  const int64_t mb = m.Bm == 1 ? 0 : b;
  const int64_t mh = head_index(m.h_mode, h, f.G);
  const int64_t mq = m.nQm == 1 ? 0 : qt;
  const int64_t r = (mb * m.Hm + mh) * m.nQm + mq;
  auto find = [&](const int32_t* idx, int cnt) {
    int lo = 0, hi = cnt;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      const int v = idx[mid];
      if (v == kt) return true;
      if (v < kt) lo = mid + 1; else hi = mid;
    }
    return false;
  };
  if (find(m.full_idx + r * m.nK, m.full_num[r])) return 2;
  if (find(m.kv_idx + r * m.nK, m.kv_num[r])) return 1;
  return 0;
}

// Per-lane LDS byte offsets of the dK / dV kernel's operand reads, computed
// once: Q rows (K swizzle) and dO rows (V swizzle) as A operands of S and dP,
// and the transposed reads of dO (V swizzle: the second read is 4 rows down)
// and of Q (K swizzle: its own offset). A 32-row block or a 16-row step adds
// rows without changing a swizzle.
struct DkdvOffs {
  uint32_t qrow[kNS], drow[kNS];
  uint32_t dc0[kNDC];
  uint32_t qc0[kNDC], qc1[kNDC];
  __device__ inline void init(int lane) {
    const int hh = lane >> 5;
    const int row = perm_row(lane & 31);
#pragma unroll
    for (int s = 0; s < kNS; ++s) {
      qrow[s] = (uint32_t)(row * kRowB + (((2 * s + hh) ^ swz_k<kD>(row)) * 16));
      drow[s] = (uint32_t)(row * kRowB + (((2 * s + hh) ^ swz_v<kD>(row)) * 16));
    }
    const int blk = lane >> 4;
    const int e4 = (lane >> 2) & 3;
    const int g4 = lane & 3;
    const int row0 = 8 * (blk >> 1) + e4;
    const int row1 = row0 + 4;
#pragma unroll
    for (int dc = 0; dc < kNDC; ++dc) {
      const int chunk = 4 * dc + 2 * (blk & 1) + (g4 >> 1);
      dc0[dc] = (uint32_t)(row0 * kRowB + ((chunk ^ swz_v<kD>(row0)) * 16) + (g4 & 1) * 8);
      qc0[dc] = (uint32_t)(row0 * kRowB + ((chunk ^ swz_k<kD>(row0)) * 16) + (g4 & 1) * 8);
      qc1[dc] = (uint32_t)(row1 * kRowB + ((chunk ^ swz_k<kD>(row1)) * 16) + (g4 & 1) * 8);
    }
  }
};

template <bool AUX>
__global__ __launch_bounds__(kThreads, 1) void k_bwd_dkdv_mfma(AttnBwdParams P,
                                                               const WorkOrder order) {
  const AttnParams& f = P.f;
  // two slots: Q tile (.k) and dO tile (.v) of a visited (head, query tile), with
  // its rows' LSE (log2 units), Delta and the key test's keep bits; the loads of
  // the next visit go out while the current one is computed
  __shared__ __align__(1024) Tiles<kD> buf[2];
  __shared__ float s_lse2[2][kTile];
  __shared__ float s_delta[2][kTile];
  __shared__ uint64_t s_keep[2][kTile][2];  // keep bits: row, 64-key half
  __shared__ float s_bias[2][kTile];        // a query-broadcast bias row (log2 units)
  // key tile major, lowest key tile first: under causal-like masks the low key
  // tiles are seen by the most query tiles, so the longest work items start
  // first; packed sequences take the host's order of (b, key tile) items
  // (heaviest first), KVH workgroups per item
  int kt, kvh, b;
  if (f.varlen && order.n > 0) {
    const int it = order.item[blockIdx.x / f.KVH];
    kt = it & 1023;
    b = it >> 10;
    kvh = blockIdx.x % f.KVH;
  } else {
    kt = blockIdx.x / (f.B * f.KVH);
    const int bk = blockIdx.x % (f.B * f.KVH);
    kvh = bk % f.KVH;
    b = bk / f.KVH;
  }
  // a packed sequence's rows, keys and DFlash geometry (the batch itself otherwise)
  const SeqView seq = seq_view(f, b);
  if (kt >= seq.nK) return;  // past a packed sequence's end (uniform)
  const int k0 = kt * kTile;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int key = k0 + 32 * w + n;  // this lane's key (column of S, dP, P, dS)
  const int64_t kg = seq.k0 + key;   // its row of the (packed) K, V, dK, dV
  const bool kvalid = key < seq.Sk;
  const bool test_k = k0 + kTile > seq.Sk;

  // the lane's K and V rows: B operands of S = Q K^T and dP = dO V^T
  bf16x8 kf[kNS], vf[kNS];
  {
    const __bf16* kr = reinterpret_cast<const __bf16*>(f.k) + (int64_t)b * f.k_sb +
                       kg * f.k_sk + (int64_t)kvh * f.k_sh;
    const __bf16* vr = reinterpret_cast<const __bf16*>(f.v) + (int64_t)b * f.v_sb +
                       kg * f.v_sk + (int64_t)kvh * f.v_sh;
#pragma unroll
    for (int s = 0; s < kNS; ++s) {
      kf[s] = kvalid ? *reinterpret_cast<const bf16x8*>(kr + 16 * s + 8 * hh) : bf16x8{};
      vf[s] = kvalid ? *reinterpret_cast<const bf16x8*>(vr + 16 * s + 8 * hh) : bf16x8{};
    }
  }
  f32x16 dk[kNDC], dv[kNDC];
#pragma unroll
  for (int i = 0; i < kNDC; ++i) dk[i] = dv[i] = f32x16{};
  DkdvOffs off;
  off.init(lane);

  // visits: positions pos = g * nQ + qt whose tile (qt, kt) of head g is not empty
  const int end = f.G * f.nQ;
  // Up to kMaxVisits positions, the workgroup classifies them all first, one
  // thread per position (the block-mask lookups run side by side, not one
  // dependent search per visit), and keeps the non-empty ones in order in LDS.
  __shared__ uint16_t s_vis[kMaxVisits];  // pos << 2 | class
  __shared__ int s_scan[kThreads / 64];
  const bool listed = end <= kMaxVisits;
  int nvis = 0;
  if (listed) {
    for (int base = 0; base < end; base += kThreads) {
      const int ps = base + tid;
      const int c = (ps < end && ps % f.nQ < seq.nQ)
                        ? tile_class_of(f, b, kvh * f.G + ps / f.nQ, ps % f.nQ, kt) : 0;
      int tot;
      const int o = block_excl_sum<kThreads / 64>(c != 0 ? 1 : 0, s_scan, tot);
      if (c != 0) s_vis[nvis + o] = (uint16_t)((ps << 2) | c);
      nvis += tot;
    }
    __syncthreads();
  }
  auto listed_visit = [&](int i, int& cls) {
    const int v = __builtin_amdgcn_readfirstlane((int)s_vis[i]);
    cls = v & 3;
    return v >> 2;
  };
  auto next_visit = [&](int pos, int& cls) {
    for (; pos < end; ++pos) {
      if (pos % f.nQ >= seq.nQ) continue;
      cls = __builtin_amdgcn_readfirstlane(
          tile_class_of(f, b, kvh * f.G + pos / f.nQ, pos % f.nQ, kt));
      if (cls != 0) return pos;
    }
    return end;
  };
  // Row data of a visit: its rows' LSE (log2 units) and Delta are loaded into
  // registers (thread tid < 128: row q0 + tid) before the visit's tiles go out
  // and the current visit is computed, and reach LDS slot sl, with the key
  // test's keep bits and a query-broadcast bias row, after it, so that no wait
  // for them holds up the matrix work.
  struct RowPre {
    float lse, dl;  // natural-log LSE, converted when stored
  };
  // every thread loads row q0 + tid % 128, clamped into the sequence (a visit
  // has at least one row): no branch, so nothing waits for the values until
  // they are stored
  auto load_rows = [&](int pos) {
    const int h = kvh * f.G + pos / f.nQ;
    const int q = min((pos % f.nQ) * kTile + (tid & (kTile - 1)), seq.Sq - 1);
    const int64_t qg = seq.q0 + q;
    return RowPre{f.lse[(int64_t)b * f.lse_sb + (int64_t)h * f.lse_sh + qg * f.lse_sq],
                  P.delta[(int64_t)b * P.delta_sb + (int64_t)h * P.delta_sh + qg]};
  };
  auto store_rows = [&](int sl, int pos, int cls, const RowPre& r) {
    const int h = kvh * f.G + pos / f.nQ;
    const int q0 = (pos % f.nQ) * kTile;
    if (tid < kTile) {
      // rows past Sq or without a kept key get +inf: their probabilities
      // exp2(x - inf) come out 0 with no test per element
      const bool ok = q0 + tid < seq.Sq;
      const float l2 = r.lse * kLog2e;
      s_lse2[sl][tid] = (ok && l2 != -INFINITY) ? l2 : INFINITY;
      s_delta[sl][tid] = ok ? r.dl : 0.f;
    }
    if (AUX && f.staged) {
      // mask and bias folded into one float row: the tile's 128-key slice
      if (tid < kTile) {
        const int64_t hc = f.cb_hmode == 1 ? h : (f.cb_hmode == 2 ? h / f.G : 0);
        s_bias[sl][tid] = f.cb[(int64_t)b * f.cb_sb + hc * f.cb_sh + k0 + tid];
      }
    } else if (AUX && f.has_bias && f.bias.q_bcast && tid < kTile) {
      const uint16_t* br = reinterpret_cast<const uint16_t*>(aux_row(f.bias, 2, b, h, f.G, 0));
      s_bias[sl][tid] = bias_log2(bf16_to_f32(br[k0 + tid]));
    }
    if (AUX && f.staged) {
      // no keep bits: the folded row drops masked keys and keys >= Sk
    } else if (AUX && f.mask_kind == 2 && (cls == 1 || test_k)) {
      // keep bits from the mask bytes of row tid / 2, keys of half tid % 2
      const int r = tid >> 1, half = tid & 1;
      const int q = q0 + r;
      uint64_t bits = 0;
      if (q < seq.Sq) {
        const uint8_t* mr = aux_row(f.mask, 1, b, h, f.G, q) + k0 + 64 * half;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t kb = k0 + 64 * half + 8 * j;
          const uint32_t mb = cls == 1 ? byte_bits8(*reinterpret_cast<const uint2*>(mr + 8 * j))
                                       : 0xFFu;
          bits |= (uint64_t)(mb & range_bits(0, seq.Sk, kb)) << (8 * j);
        }
      }
      s_keep[sl][r][half] = bits;
    } else if (cls == 1 || test_k) {  // keep bits: row tid / 2, keys of half tid % 2
      const int r = tid >> 1, half = tid & 1;
      const int q = q0 + r;
      uint64_t bits = 0;
      if (q < seq.Sq) {
        int lo1 = 0, hi1 = seq.Sk, lo2 = 0, hi2 = 0;
        if (cls == 1 && f.mask_kind == 1) {
          const RowIv v = dflash_row(seq.rule, f.pred_row0 ? 0 : q);
          lo1 = (int)v.lo1;
          hi1 = (int)v.hi1;
          lo2 = (int)v.lo2;
          hi2 = (int)v.hi2;
        }
        hi1 = hi1 < seq.Sk ? hi1 : seq.Sk;
        hi2 = hi2 < seq.Sk ? hi2 : seq.Sk;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int kb = k0 + 64 * half + 8 * j;
          bits |= (uint64_t)(range_bits(lo1, hi1, kb) | range_bits(lo2, hi2, kb)) << (8 * j);
        }
      }
      s_keep[sl][r][half] = bits;
    }
  };
  // the Q and dO tiles of visit pos into LDS tiles tq, tdo (LDS-DMA)
  auto issue_tiles = [&](__bf16* tq, __bf16* tdo, int pos) {
    const int h = kvh * f.G + pos / f.nQ;
    Loader<kD, 2> ld;
    ld.init(reinterpret_cast<const __bf16*>(f.q) + (int64_t)b * f.q_sb + seq.q0 * f.q_sq +
                (int64_t)h * f.q_sh,
            reinterpret_cast<const __bf16*>(P.dout) + (int64_t)b * P.do_sb + seq.q0 * P.do_sq +
                (int64_t)h * P.do_sh,
            f.q_sq, P.do_sq, seq.Sq, w, lane);
    ld.issue(tq, tdo, pos % f.nQ, w);
  };

  // the visit after visit `it` (at position pos), or end
  auto following = [&](int it, int pos, int& cls) {
    if (listed) return it + 1 < nvis ? listed_visit(it + 1, cls) : end;
    return next_visit(pos + 1, cls);
  };
  // dbias of a query-broadcast bias: this lane's key summed over the rows of
  // the visits whose heads share one bias row (db_h: such a head, -1: none)
  float dbacc = 0.f;
  int db_h = -1;
  auto db_flush = [&]() {
    const float t = dbacc + __shfl_xor(dbacc, 32, 64);
    if (db_h >= 0 && hh == 0 && kvalid)
      atomicAdd(reinterpret_cast<float*>(const_cast<uint8_t*>(aux_row(P.dbias, 4, b, db_h, f.G, 0))) +
                    key, t);
    dbacc = 0.f;
  };
  const bool db_rows = AUX && P.dbias_acc != nullptr && !f.bias.q_bcast;
  int cls = 0;
  int pos = listed ? (nvis > 0 ? listed_visit(0, cls) : end) : next_visit(0, cls);
  if (pos < end) {
    store_rows(0, pos, cls, load_rows(pos));
    issue_tiles(buf[0].k, buf[0].v, pos);
  }
  for (int it = 0; pos < end; ++it) {
    const int sl = it & 1;
    wait_vmcnt<0>();   // this visit's tiles and row data (this thread's share)
    __syncthreads();   // everyone's share; slot sl ^ 1 is free
    int ncls = 0;
    const int npos = following(it, pos, ncls);
    const RowPre pre = load_rows(npos < end ? npos : pos);
    // One visit: the next visit's tiles go out into slot sl ^ 1 (fq, fdo) while
    // this one's (tq, tdo) are computed. As restrict parameters the slots tell
    // the compiler that the LDS reads do not touch the tiles in flight, so it
    // does not wait for those loads before them.
    auto visit = [&](const char* __restrict__ tq, const char* __restrict__ tdo,
                     __bf16* __restrict__ fq, __bf16* __restrict__ fdo)
                     __attribute__((always_inline)) {
    if (npos < end) issue_tiles(fq, fdo, npos);
    const bool test = !(AUX && f.staged) && (cls == 1 || test_k);
    const int vh = kvh * f.G + pos / f.nQ;  // this visit's head and first row
    const int vq0 = (pos % f.nQ) * kTile;
    if (AUX && P.dbias_acc && f.bias.q_bcast) {
      if (db_h >= 0 && head_index(P.dbias.h_mode, vh, f.G) != head_index(P.dbias.h_mode, db_h, f.G))
        db_flush();
      db_h = vh;
    }
    auto ld8 = [](const char* a) { return *reinterpret_cast<const bf16x8*>(a); };
    auto tr8 = [](const char* a0, const char* a1) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a1));
      return __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo),
                                     __builtin_bit_cast(bf16x4, hi), 0, 1, 2, 3, 4, 5, 6, 7);
    };
#pragma unroll
    for (int rb = 0; rb < kTile / 32; ++rb) {
      const int rbo = rb * 32 * kRowB;
      f32x16 s = f32x16{}, dp = f32x16{};
      // row operands kAhead d-steps ahead
      bf16x8 qa[kAhead], da[kAhead];
#pragma unroll
      for (int j = 0; j < kAhead; ++j) {
        qa[j] = ld8(tq + off.qrow[j] + rbo);
        da[j] = ld8(tdo + off.drow[j] + rbo);
      }
#pragma unroll
      for (int ds_ = 0; ds_ < kNS; ++ds_) {
        const bf16x8 a = qa[ds_ % kAhead], d = da[ds_ % kAhead];
        if (ds_ + kAhead < kNS) {
          qa[ds_ % kAhead] = ld8(tq + off.qrow[ds_ + kAhead] + rbo);
          da[ds_ % kAhead] = ld8(tdo + off.drow[ds_ + kAhead] + rbo);
        }
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[ds_], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(d, vf[ds_], dp, 0, 0, 0);
      }
      pin_reads_ahead<kNS, kAhead, 2, 2>();
      // the first transposed operands load while P and dS are computed
      // (operand i = (d chunk i / 2, 16 rows i % 2))
      auto dop = [&](int i) {
        const int o = rbo + 16 * (i % 2) * kRowB;
        return tr8(tdo + off.dc0[i / 2] + o, tdo + off.dc0[i / 2] + o + 4 * kRowB);
      };
      auto qop = [&](int i) {
        const int o = rbo + 16 * (i % 2) * kRowB;
        return tr8(tq + off.qc0[i / 2] + o, tq + off.qc1[i / 2] + o);
      };
      bf16x8 dca[kTrAhead], qca[kTrAhead];
#pragma unroll
      for (int j = 0; j < kTrAhead; ++j) {
        dca[j] = dop(j);
        qca[j] = qop(j);
      }
      // lane: key, rows rb*32 + 16 st + 8 hh + e for value u = 8 st + e
      float pv[16], dsv[16];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int r0 = rb * 32 + 16 * st + 8 * hh;
        const float4 la = *reinterpret_cast<const float4*>(&s_lse2[sl][r0]);
        const float4 lb = *reinterpret_cast<const float4*>(&s_lse2[sl][r0 + 4]);
        const float4 da4 = *reinterpret_cast<const float4*>(&s_delta[sl][r0]);
        const float4 db4 = *reinterpret_cast<const float4*>(&s_delta[sl][r0 + 4]);
        const float l2[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
        const float dl[8] = {da4.x, da4.y, da4.z, da4.w, db4.x, db4.y, db4.z, db4.w};
        // keep bits of this lane's key for the 8 rows, read together (a
        // branch per element would split the block the MFMAs overlap with)
        uint32_t bits = 0xFFu;
        if (test) {
          const int kk = 32 * w + n;  // key within the tile
          bits = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            bits |= (uint32_t)((s_keep[sl][r0 + e][kk >> 6] >> (kk & 63)) & 1u) << e;
        }
        // the bias of (row, this lane's key) in log2 units
        float bv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (AUX && (f.staged || f.has_bias)) {
          if (f.staged || f.bias.q_bcast) {
            const float bk = s_bias[sl][32 * w + n];
#pragma unroll
            for (int e = 0; e < 8; ++e) bv[e] = bk;
          } else if (kvalid) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int q = vq0 + r0 + e;
              if (q < seq.Sq)
                bv[e] = bias_log2(bf16_to_f32(reinterpret_cast<const uint16_t*>(
                    aux_row(f.bias, 2, b, vh, f.G, q))[key]));
            }
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int u = 8 * st + e;
          const float ex = __builtin_amdgcn_exp2f(
              fmaf(s[u], f.scale_log2, AUX ? bv[e] - l2[e] : -l2[e]));
          const float pr = (test && !((bits >> e) & 1u)) ? 0.f : ex;
          pv[u] = pr;
          dsv[u] = pr * (dp[u] - dl[e]);
        }
        if (AUX && P.dbias_acc) {
          if (!db_rows) {
#pragma unroll
            for (int e = 0; e < 8; ++e) dbacc += dsv[8 * st + e];
          } else if (kvalid) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int q = vq0 + r0 + e;
              if (q < seq.Sq && dsv[8 * st + e] != 0.f)
                atomicAdd(reinterpret_cast<float*>(const_cast<uint8_t*>(
                              aux_row(P.dbias, 4, b, vh, f.G, q))) + key,
                          dsv[8 * st + e]);
            }
          }
        }
      }
      const bf16x8 p0 = pack8(pv), p1 = pack8(pv + 8);
      const bf16x8 s0 = pack8(dsv), s1 = pack8(dsv + 8);
      // dV^T += dO^T P and dK^T += Q^T dS: operand i = (dc, half j), kTrAhead ahead
      constexpr int NT = 2 * kNDC;
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const int dc = i / 2, j = i % 2;
        const bf16x8 a = dca[i % kTrAhead], qb = qca[i % kTrAhead];
        if (i + kTrAhead < NT) {
          dca[i % kTrAhead] = dop(i + kTrAhead);
          qca[i % kTrAhead] = qop(i + kTrAhead);
        }
        dv[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, j ? p1 : p0, dv[dc], 0, 0, 0);
        dk[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qb, j ? s1 : s0, dk[dc], 0, 0, 0);
      }
      pin_reads_ahead<NT, kTrAhead, 4, 2>();
    }
    };
    visit(reinterpret_cast<const char*>(buf[sl].k), reinterpret_cast<const char*>(buf[sl].v),
          buf[sl ^ 1].k, buf[sl ^ 1].v);
    if (npos < end) store_rows(sl ^ 1, npos, ncls, pre);
    pos = npos;
    cls = ncls;
  }
  if (AUX && P.dbias_acc && f.bias.q_bcast) db_flush();
  // dK^T / dV^T accumulators: lane holds d = 32 dc + 8 (r / 4) + 4 hh + r % 4 of its key
  if (kvalid) {
    __bf16* ko = reinterpret_cast<__bf16*>(P.dk) + (int64_t)b * P.dk_sb + kg * P.dk_sk +
                 (int64_t)kvh * P.dk_sh;
    __bf16* vo = reinterpret_cast<__bf16*>(P.dv) + (int64_t)b * P.dv_sb + kg * P.dv_sk +
                 (int64_t)kvh * P.dv_sh;
#pragma unroll
    for (int dc = 0; dc < kNDC; ++dc) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 a, c;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = (__bf16)(dk[dc][4 * g + e] * P.scale);
          c[e] = (__bf16)dv[dc][4 * g + e];
        }
        *reinterpret_cast<bf16x4*>(ko + dc * 32 + 8 * g + 4 * hh) = a;
        *reinterpret_cast<bf16x4*>(vo + dc * 32 + 8 * g + 4 * hh) = c;
      }
    }
  }
}

}  // namespace

bool attn_bwd_mfma_applies(const AttnBwdParams& p, int D) {
  // the dK / dV kernel's tile loads use 32-bit offsets within one (b, head)
  return D == kD && !p.f.varlen && (p.f.has_bias || !p.dbias_acc) &&
         (int64_t)p.f.Sq * p.f.q_sq * 2 < ((int64_t)1 << 31) &&
         (int64_t)p.f.Sq * p.do_sq * 2 < ((int64_t)1 << 31);
}

hipError_t launch_attn_bwd_mfma(const AttnBwdParams& p, hipStream_t s, const WorkOrder* dq_order,
                                const WorkOrder* dkdv_order) {
  static const WorkOrder kNoOrder{};  // n = 0
  const AttnParams& f = p.f;
  const WorkOrder& oq = (dq_order && f.varlen) ? *dq_order : kNoOrder;
  const WorkOrder& ok = (dkdv_order && f.varlen) ? *dkdv_order : kNoOrder;
  const int64_t nq = (int64_t)f.B * f.H * f.nQ;
  const int64_t nk = ok.n > 0 ? (int64_t)ok.n * f.KVH : (int64_t)f.B * f.KVH * f.nK;
  // the pipelined dQ kernel needs K / V offsets within 32 bits; it takes head
  // pairs when G is even and the pair shares its block-mask row, else one head
  const bool piped = (int64_t)f.Sk * f.k_sk * 2 < ((int64_t)1 << 31) &&
                     (int64_t)f.Sk * f.v_sk * 2 < ((int64_t)1 << 31);
  const int hp = (f.G % 2 == 0 && !(f.has_bm && f.bm.h_mode == 1)) ? 2 : 1;
  const bool aux = f.has_bias || f.mask_kind == 2;
  // packed sequences: only the pipelined dQ kernel and the dK / dV kernel read
  // a sequence's rows and keys, and neither takes a mask tensor or bias there
  if (f.varlen && (!piped || aux)) return hipErrorInvalidValue;
  if (nq > 0) {
    const int nWork = oq.n > 0 ? oq.n * f.KVH * (f.G / hp)
                               : (int)((int64_t)f.B * f.KVH * (f.G / hp) * f.nQ);
    if (piped && hp == 2 && aux)
      hipLaunchKernelGGL((k_bwd_dq_pair<true, 2>), dim3(nWork), dim3(512), 0, s, p, nWork, oq);
    else if (piped && hp == 2)
      hipLaunchKernelGGL((k_bwd_dq_pair<false, 2>), dim3(nWork), dim3(512), 0, s, p, nWork, oq);
    else if (piped && aux)
      hipLaunchKernelGGL((k_bwd_dq_pair<true, 1>), dim3(nWork), dim3(512), 0, s, p, nWork, oq);
    else if (piped)
      hipLaunchKernelGGL((k_bwd_dq_pair<false, 1>), dim3(nWork), dim3(512), 0, s, p, nWork, oq);
    else if (aux)
      hipLaunchKernelGGL(k_bwd_dq_mfma<true>, dim3(nq), dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL(k_bwd_dq_mfma<false>, dim3(nq), dim3(kThreads), 0, s, p);
  }
  if (nk > 0) {
    if (aux)
      hipLaunchKernelGGL(k_bwd_dkdv_mfma<true>, dim3(nk), dim3(kThreads), 0, s, p, ok);
    else
      hipLaunchKernelGGL(k_bwd_dkdv_mfma<false>, dim3(nk), dim3(kThreads), 0, s, p, ok);
  }
  return hipGetLastError();
}

}  // namespace bsm
