// Masked attention forward, bf16, for short query blocks: at most 32 query rows
// per (b, h) -- the seqlen_q == 1 head-group swap gives G rows per KV head
// (flash-sparse-attention PR #190, Design: swapped path), prefill chunks of a
// few tokens, a draft block against a long KV cache.
//
// Such a launch streams K and V and does little arithmetic on them, so the
// work inside a workgroup is split along the keys instead of the queries: 4
// waves share each 128-key K/V tile (LDS-DMA double buffering as in
// attn_v2.hip), wave w takes keys 32w .. 32w+31 of every tile for all the rows,
// keeps its own online-softmax state, and the four partial (max, sum, O) states
// are merged through LDS at the end. The mask bytes and bias values a wave
// needs for the next tile are loaded together with that tile's DMA, so the wait
// for one covers the other. Across workgroups:
//  * the heads of a KV group whose block-mask row is shared (a head-shared or
//    per-KV-head block mask, or none) are packed: row r of the workgroup is
//    query r % Sq of head h0 + r / Sq, up to 64 rows in two 32-row blocks, so
//    each K/V tile enters LDS once per KV group;
//  * the tile list of a (b, KV group) is cut into S contiguous parts, one per
//    workgroup; each part's unnormalised O, running max and row sum go to a
//    float workspace and k_split_merge combines them (the online-softmax merge
//    of partial results: weights 2^(m_s - m*)).
// Without packing or splitting (pack = 1, S = 1) a workgroup is one (b, h).
// The heads of the mask / bias / DFlash row follow each row's own head and
// query (flash-sparse-attention PR #190, Design: broadcast rules; SpecForge
// issue #452: head-shared block masks).
#include <math.h>

#include "attn_common.h"
#include "attn_pipe.h"
#include "bsm_internal.h"
#include "dflash_rows.h"

namespace bsm {
namespace {

using namespace pipe;

constexpr int kGWaves = 4;
constexpr int kGRB = 512 / (64 * kGWaves);  // Loader layout for 256 threads

// Mask / bias words of one lane, one row block, one tile: keys kb .. kb+7 for
// sb = 0, 1 with kb = k0 + 32 w + 16 sb + 8 hh.
struct GAux {
  uint4 bias[2];
  uint2 mask[2];
};

template <int RB>
__device__ inline void load_gaux(int kt, int w, int hh, const uint8_t* const (&mrow)[RB],
                                 const uint16_t* const (&brow)[RB], GAux (&a)[RB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int kb = kt * kTile + 32 * w + 16 * sb + 8 * hh;
      a[rb].bias[sb] =
          brow[rb] ? *reinterpret_cast<const uint4*>(brow[rb] + kb) : make_uint4(0, 0, 0, 0);
      a[rb].mask[sb] =
          mrow[rb] ? *reinterpret_cast<const uint2*>(mrow[rb] + kb) : make_uint2(0, 0);
    }
}

// RB: 32-row blocks of the workgroup. With RB = 2, SPLIT gives each row block
// its own four waves (512 threads, two waves per SIMD, one row block each);
// otherwise every wave carries all RB row blocks.
template <int D, int RB, bool SPLIT>
__global__ __launch_bounds__(64 * kGWaves * (SPLIT ? 2 : 1), 1) void k_attn_group(AttnParams p) {
  constexpr int NS = D / 16;
  constexpr int NDC = D / 32;
  constexpr int ROWS = 32 * RB;
  constexpr int WRB = SPLIT ? 1 : RB;  // row blocks of one wave
  static_assert(!SPLIT || RB == 2, "split row blocks come in pairs");
  __shared__ __align__(1024) Tiles<D> buf[2];
  __shared__ float s_m[kGWaves][ROWS];
  __shared__ float s_l[kGWaves][ROWS];

  // Workgroup i runs on XCD i % 8: each XCD takes a contiguous range of work
  // items, so the splits of one (b, KV group) share an L2.
  int id;
  {
    const int nwg = gridDim.x;
    const int x = blockIdx.x % kXcds;
    const int qx = nwg / kXcds, rx = nwg % kXcds;
    id = (x < rx ? x * (qx + 1) : rx * (qx + 1) + (x - rx) * qx) + blockIdx.x / kXcds;
  }
  const int S = p.splits;
  const int sp = id % S;
  id /= S;
  const int ngrp = p.H / p.pack;
  const int h0 = (id % ngrp) * p.pack;
  const int b = id / ngrp;
  const int kvh = h0 / p.G;
  const int R = p.pack * p.Sq;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;             // loader slot of the wave
  const int kw = SPLIT ? (w & 3) : w;  // the wave's 32 keys of each tile
  const int rb0 = SPLIT ? (w >> 2) : 0;  // the wave's first row block
  const int n = lane & 31;
  const int hh = lane >> 5;

  // this lane's rows: r = 32 (rb0 + rb) + n is query r % Sq of head h0 + r / Sq
  bf16x8 qf[WRB][NS];
  RowIv32 iv[WRB];
  const uint8_t* mrow[WRB];
  const uint16_t* brow[WRB];
  bool rvalid[WRB];
#pragma unroll
  for (int rb = 0; rb < WRB; ++rb) {
    const int r = 32 * (rb0 + rb) + n;
    rvalid[rb] = r < R;
    const int q = rvalid[rb] ? r % p.Sq : 0;
    const int h = h0 + (rvalid[rb] ? r / p.Sq : 0);
    const __bf16* qrow = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.q_sb +
                         (int64_t)q * p.q_sq + (int64_t)h * p.q_sh;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      qf[rb][s] =
          rvalid[rb] ? *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * hh) : bf16x8{};
    iv[rb] = RowIv32{0, 0, 0, 0};
    if (p.mask_kind == 1) {
      const RowIv v = dflash_row(p.rule, p.pred_row0 ? 0 : q);
      iv[rb] = RowIv32{(int)v.lo1, (int)v.hi1, (int)v.lo2, (int)v.hi2};
    }
    mrow[rb] = (p.mask_kind == 2 && rvalid[rb]) ? aux_row(p.mask, 1, b, h, p.G, q) : nullptr;
    brow[rb] = (p.has_bias && rvalid[rb])
        ? reinterpret_cast<const uint16_t*>(aux_row(p.bias, 2, b, h, p.G, q)) : nullptr;
  }
  const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k) + (int64_t)b * p.k_sb +
                        (int64_t)kvh * p.k_sh;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(p.v) + (int64_t)b * p.v_sb +
                        (int64_t)kvh * p.v_sh;
  Loader<D, SPLIT ? 1 : kGRB> ld;
  ld.init(kbase, vbase, p.k_sk, p.v_sk, p.Sk, w, lane);

  f32x16 oacc[WRB][NDC];
  float m_run[WRB], l_run[WRB];
#pragma unroll
  for (int rb = 0; rb < WRB; ++rb) {
#pragma unroll
    for (int i = 0; i < NDC; ++i) oacc[rb][i] = f32x16{};
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
  }
  const int blk = lane >> 4;
  const int e4 = (lane >> 2) & 3;
  const int g4 = lane & 3;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // this split's part of the tile list (the list is shared by the packed heads)
  TileList tl;
  tl.init(p, b, h0, 0);
  const int ntot = tl.count();
  const int t0 = (int)((int64_t)sp * ntot / S);
  const int t1 = (int)((int64_t)(sp + 1) * ntot / S);
  bool full_cur = false;
  int kt_cur = t0 < t1 ? tl.tile(t0, full_cur) : 0;
  GAux aux_cur[WRB], aux_nxt[WRB];
  if (t0 < t1) {
    ld.issue(buf[0], kt_cur, w);
    load_gaux<WRB>(kt_cur, kw, hh, mrow, brow, aux_cur);
  }
  for (int it = t0; it < t1; ++it) {
    const Tiles<D>& t = buf[(it - t0) & 1];
    Tiles<D>& nxt = buf[(it - t0 + 1) & 1];
    bool full_nxt = false;
    const int kt_nxt = it + 1 < t1 ? tl.tile(it + 1, full_nxt) : 0;
    wait_vmcnt<0>();
    barrier();
    if (it + 1 < t1) {
      ld.issue(nxt, kt_nxt, w);
      load_gaux<WRB>(kt_nxt, kw, hh, mrow, brow, aux_nxt);
    }
    const int k0 = kt_cur * kTile;
    const int krow = kw * 32 + perm_row(n);
    f32x16 sc[WRB];
#pragma unroll
    for (int rb = 0; rb < WRB; ++rb) sc[rb] = f32x16{};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(t.k + krow * D +
                                                        (((2 * s + hh) ^ swz_k<D>(krow)) * 8));
#pragma unroll
      for (int rb = 0; rb < WRB; ++rb)
        sc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[rb][s], sc[rb], 0, 0, 0);
    }
    const bool check_k = k0 + kTile > p.Sk;
    const bool check_mask = !full_cur && p.mask_kind != 0;
    bf16x8 pf[WRB][2];
#pragma unroll
    for (int rb = 0; rb < WRB; ++rb) {
      float mloc = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int kb = k0 + 32 * kw + 16 * sb + 8 * hh;
        uint32_t mbits = 0xFFu;
        if (check_mask) {
          if (p.mask_kind == 2) {
            const uint2 mb = aux_cur[rb].mask[sb];
            mbits = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint32_t byte = ((e < 4 ? mb.x : mb.y) >> (8 * (e & 3))) & 0xFFu;
              mbits |= (byte != 0u ? 1u : 0u) << e;
            }
          } else {
            mbits = range_bits(iv[rb].lo1, iv[rb].hi1, kb) | range_bits(iv[rb].lo2, iv[rb].hi2, kb);
          }
        }
        if (!rvalid[rb]) mbits = 0;
        if (check_k) mbits &= range_bits(0, p.Sk, kb);
        const uint4 bw = aux_cur[rb].bias[sb];
        const uint32_t wv[4] = {bw.x, bw.y, bw.z, bw.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int u = 8 * sb + e;
          const float bv = bias_log2(bf16_to_f32((uint16_t)(wv[e >> 1] >> (16 * (e & 1)))));
          float sv = fmaf(sc[rb][u], p.scale_log2, bv);
          sv = ((mbits >> e) & 1u) ? sv : -INFINITY;
          sc[rb][u] = sv;
          mloc = fmaxf(mloc, sv);
        }
      }
      mloc = max_pair(mloc);
      const bool grow = mloc > m_run[rb] + kRescaleLog2;
      const float m_new = grow ? mloc : m_run[rb];
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run[rb] - m_new) : 1.f;
      if (__ballot(grow)) {
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) oacc[rb][dc] *= alpha;
      }
      m_run[rb] = m_new;
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      float lsum = l_run[rb] * alpha;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float x0 = __builtin_amdgcn_exp2f(sc[rb][8 * sb + e] - m_use);
          const float x1 = __builtin_amdgcn_exp2f(sc[rb][8 * sb + e + 1] - m_use);
          const bf16x2 pr = {(__bf16)x0, (__bf16)x1};
          pf[rb][sb][e] = pr[0];
          pf[rb][sb][e + 1] = pr[1];
          lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsum, false);
        }
      }
      l_run[rb] = lsum;
    }
    // O^T += V^T P^T over this wave's 32 keys; one V operand serves both row blocks
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int kb = kw * 32 + 16 * sb;
        const int chunk = 4 * dc + 2 * (blk & 1) + (g4 >> 1);
        const int row0 = kb + 8 * (blk >> 1) + e4;
        const int row1 = row0 + 4;
        const __bf16* a0 = t.v + row0 * D + ((chunk ^ swz_v<D>(row0)) * 8) + (g4 & 1) * 4;
        const __bf16* a1 = t.v + row1 * D + ((chunk ^ swz_v<D>(row1)) * 8) + (g4 & 1) * 4;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a1));
        const bf16x8 a = __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo),
                                                 __builtin_bit_cast(bf16x4, hi), 0, 1, 2, 3, 4,
                                                 5, 6, 7);
#pragma unroll
        for (int rb = 0; rb < WRB; ++rb)
          oacc[rb][dc] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[rb][sb], oacc[rb][dc], 0, 0, 0);
      }
    }
#pragma unroll
    for (int rb = 0; rb < WRB; ++rb) aux_cur[rb] = aux_nxt[rb];
    kt_cur = kt_nxt;
    full_cur = full_nxt;
  }

  // merge the four waves' partial states through LDS (both tile buffers are
  // free now: [wave][row][D] floats fill them exactly when RB = 2, D = 128)
  barrier();
  float* sO = reinterpret_cast<float*>(&buf[0]);
#pragma unroll
  for (int rb = 0; rb < WRB; ++rb) {
    const int r = 32 * (rb0 + rb) + n;
    const float l_pair = l_run[rb] + __shfl_xor(l_run[rb], 32, 64);
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(&sO[((int64_t)kw * ROWS + r) * D + dc * 32 + 8 * g + 4 * hh]) =
            make_float4(oacc[rb][dc][4 * g], oacc[rb][dc][4 * g + 1], oacc[rb][dc][4 * g + 2],
                        oacc[rb][dc][4 * g + 3]);
    if (hh == 0) {
      s_m[kw][r] = m_run[rb];
      s_l[kw][r] = l_pair;
    }
  }
  __syncthreads();
  // each wave finishes 32 / RB ... all rows: lanes (n, hh) of wave w cover row
  // r = 32 rb + n and d-chunks dc = w, w + 4, ...
#pragma unroll
  for (int rb = 0; rb < WRB; ++rb) {
    const int r = 32 * (rb0 + rb) + n;
    if (!rvalid[rb]) continue;
    float mstar = -INFINITY;
#pragma unroll
    for (int i = 0; i < kGWaves; ++i) mstar = fmaxf(mstar, s_m[i][r]);
    float f[kGWaves];
    float lstar = 0.f;
#pragma unroll
    for (int i = 0; i < kGWaves; ++i) {
      const float mi = s_m[i][r];
      f[i] = mi == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mi - mstar);
      lstar += f[i] * s_l[i][r];
    }
    const int q = r % p.Sq;
    const int h = h0 + r / p.Sq;
    const float inv = lstar > 0.f ? 1.f / lstar : 0.f;
    __bf16* orow = reinterpret_cast<__bf16*>(p.o) + (int64_t)b * p.o_sb + (int64_t)q * p.o_sq +
                   (int64_t)h * p.o_sh;
    const int64_t prow = (((int64_t)sp * p.B + b) * p.H + h) * p.Sq + q;
    for (int dc = kw; dc < NDC; dc += kGWaves) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = dc * 32 + 8 * g + 4 * hh;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < kGWaves; ++i) {
          const float4 v = *reinterpret_cast<const float4*>(&sO[((int64_t)i * ROWS + r) * D + d0]);
          acc.x += f[i] * v.x;
          acc.y += f[i] * v.y;
          acc.z += f[i] * v.z;
          acc.w += f[i] * v.w;
        }
        if (S == 1) {
          bf16x4 o4 = {(__bf16)(acc.x * inv), (__bf16)(acc.y * inv), (__bf16)(acc.z * inv),
                       (__bf16)(acc.w * inv)};
          *reinterpret_cast<bf16x4*>(orow + d0) = o4;
        } else {
          *reinterpret_cast<float4*>(p.ws_o + prow * D + d0) = acc;
        }
      }
    }
    if (kw == 0 && hh == 0) {
      if (S == 1) {
        if (p.lse)
          p.lse[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + (int64_t)q * p.lse_sq] =
              lstar > 0.f ? (mstar + __builtin_amdgcn_logf(lstar)) * kLn2 : -INFINITY;
      } else {
        p.ws_ml[2 * prow] = mstar;
        p.ws_ml[2 * prow + 1] = lstar;
      }
    }
  }
}

// One wave per (b, h, q) row: combine the S partial states of the row.
template <int D>
__global__ __launch_bounds__(256) void k_split_merge(AttnParams p) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nrows = (int64_t)p.B * p.H * p.Sq;
  if (row >= nrows) return;
  const int lane = threadIdx.x & 63;
  const int q = (int)(row % p.Sq);
  const int h = (int)((row / p.Sq) % p.H);
  const int b = (int)(row / ((int64_t)p.Sq * p.H));
  const int S = p.splits;
  const int64_t stride = nrows;  // rows per split
  float mstar = -INFINITY;
  for (int s = 0; s < S; ++s) mstar = fmaxf(mstar, p.ws_ml[2 * (s * stride + row)]);
  constexpr int E = D / 64;  // elements per lane
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float lstar = 0.f;
  for (int s = 0; s < S; ++s) {
    const int64_t pr = s * stride + row;
    const float ms = p.ws_ml[2 * pr];
    const float f = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - mstar);
    lstar += f * p.ws_ml[2 * pr + 1];
    const float* o = p.ws_o + pr * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += f * o[e];
  }
  const float inv = lstar > 0.f ? 1.f / lstar : 0.f;
  __bf16* orow = reinterpret_cast<__bf16*>(p.o) + (int64_t)b * p.o_sb + (int64_t)q * p.o_sq +
                 (int64_t)h * p.o_sh + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) orow[e] = (__bf16)(acc[e] * inv);
  if (p.lse && lane == 0)
    p.lse[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + (int64_t)q * p.lse_sq] =
        lstar > 0.f ? (mstar + __builtin_amdgcn_logf(lstar)) * kLn2 : -INFINITY;
}

}  // namespace

bool short_query_applies(const AttnParams& p, int D) {
  if (D != 64 && D != 128) return false;
  if (p.Sq > 32 || p.varlen) return false;
  // 32-bit buffer offsets within one (b, kv head)
  if ((int64_t)p.Sk * p.k_sk * 2 >= (int64_t)1 << 31) return false;
  if ((int64_t)p.Sk * p.v_sk * 2 >= (int64_t)1 << 31) return false;
  return true;
}

hipError_t launch_attn_group(const AttnParams& p, int D, hipStream_t s) {
  const int64_t nwg = (int64_t)p.B * (p.H / p.pack) * p.splits;
  if (nwg == 0) return hipSuccess;
  const int rb = p.pack * p.Sq > 32 ? 2 : 1;
  const dim3 blk(64 * kGWaves), blk2(128 * kGWaves);
  if (D == 128) {
    if (rb == 2)
      hipLaunchKernelGGL((k_attn_group<128, 2, true>), dim3((unsigned)nwg), blk2, 0, s, p);
    else
      hipLaunchKernelGGL((k_attn_group<128, 1, false>), dim3((unsigned)nwg), blk, 0, s, p);
  } else {
    if (rb == 2)
      hipLaunchKernelGGL((k_attn_group<64, 2, true>), dim3((unsigned)nwg), blk2, 0, s, p);
    else
      hipLaunchKernelGGL((k_attn_group<64, 1, false>), dim3((unsigned)nwg), blk, 0, s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const int64_t rows = (int64_t)p.B * p.H * p.Sq;
  const unsigned grid = (unsigned)((rows + 3) / 4);
  if (D == 128)
    hipLaunchKernelGGL(k_split_merge<128>, dim3(grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(k_split_merge<64>, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace bsm
