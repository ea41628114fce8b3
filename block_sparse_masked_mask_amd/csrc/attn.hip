// Masked scaled-dot-product attention forward for gfx950.
//
// For each (b, h, query tile) the kernel visits only the key tiles its block mask
// lists (full ones first, without a mask test; then partial ones, testing the
// DFlash predicate's two per-row key intervals or reading the mask bytes), adds
// the additive bias, and keeps a float online softmax (flash-sparse-attention
// PR #190, Design: bool mask True = keep, float bias additive, stride-0 broadcast;
// SpecForge issue #452: one block mask shared by all heads). Keys >= Sk never
// contribute; K and V are read unpadded (PR #190, Implementation Notes). A row
// with no kept key returns O = 0 and LSE = -inf.
//
// bf16 kernel (k_attn_bf16): 256 threads = 4 waves, one 128-query tile; wave w
// owns queries 32w..32w+31. Per 128-key tile:
//   * K is staged in LDS row-major ([key][d], padded pitch) and V transposed
//     ([d][key], padded pitch), the transpose done in registers on the way in
//     (4 keys x 8 d per work item);
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16, 4 chunks of 32 keys. The K rows fed
//     to the MFMA are permuted (bits 2 and 3 of the row swapped) so that each
//     lane ends up holding 8 consecutive keys per 16-key step of one query row:
//     the lane's query is lane % 32, the scores are already laid out as the
//     B operand of the P V product, and row reductions need one cross-lane step;
//   * online softmax in float with exp2 (scale * log2 e folded in); the row
//     rescale is a per-lane scalar because each lane owns one query row;
//   * O^T += V^T P^T on the same MFMA, V^T read as 16-byte rows from LDS.
// f32 kernel (k_attn_f32): true float products on the vector ALU, 16 queries per
// workgroup, 16 threads per query each owning D/16 dims (dot products summed
// across the 16 lanes by DPP); K and V tiles of 64 keys staged in LDS.
#include <math.h>

#include "attn_common.h"
#include "attn_pipe.h"
#include "bsm_internal.h"
#include "dflash_rows.h"

namespace bsm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Row permutation of the K operand: swap bits 2 and 3 of the row index.
__device__ inline int perm_row(int n) { return (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1); }

template <int D>
struct Bf16Smem {
  static constexpr int KP = D + 8;    // K tile pitch in bf16 elements
  static constexpr int VP = kTile + 8;  // V^T tile pitch in bf16 elements
  __bf16 k[kTile * KP];
  __bf16 vt[D * VP];
};

template <int D>
__global__ __launch_bounds__(256, 2) void k_attn_bf16(AttnParams p) {
  constexpr int KP = Bf16Smem<D>::KP;
  constexpr int VP = Bf16Smem<D>::VP;
  constexpr int NS = D / 16;  // k-steps of the QK^T contraction
  constexpr int NDC = D / 32; // 32-wide d chunks of O^T
  __shared__ __align__(16) Bf16Smem<D> sm;

  const int qt = (int)gridDim.x - 1 - (int)blockIdx.x;  // heaviest tiles first
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const SeqView seq = seq_view(p, b);
  if (qt >= seq.nQ) return;  // past a packed sequence's end (uniform)
  const int q = qt * kTile + w * 32 + n;
  const bool qvalid = q < seq.Sq;
  const int kvh = h / p.G;

  // Q fragment: lane holds row q, d = 16 s + 8 hh + [0, 8)
  bf16x8 qf[NS];
  {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.q_sb +
                         (seq.q0 + q) * p.q_sq + (int64_t)h * p.q_sh;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (qvalid)
        qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * hh);
      else
        qf[s] = bf16x8{};
    }
  }
  RowIv iv{0, 0, 0, 0};
  if (p.mask_kind == 1) iv = dflash_row(seq.rule, p.pred_row0 ? 0 : q);
  const uint8_t* mrow =
      (p.mask_kind == 2 && qvalid) ? aux_row(p.mask, 1, b, h, p.G, q) : nullptr;
  const uint16_t* brow = (p.has_bias && qvalid)
      ? reinterpret_cast<const uint16_t*>(aux_row(p.bias, 2, b, h, p.G, q)) : nullptr;

  const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k) + (int64_t)b * p.k_sb +
                        seq.k0 * p.k_sk + (int64_t)kvh * p.k_sh;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(p.v) + (int64_t)b * p.v_sb +
                        seq.k0 * p.v_sk + (int64_t)kvh * p.v_sh;

  f32x16 oacc[NDC];
#pragma unroll
  for (int i = 0; i < NDC; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  TileList tl;
  tl.init(p, b, h, qt, seq.nK);
  const int ntiles = tl.count();
  for (int it = 0; it < ntiles; ++it) {
    bool is_full;
    const int kt = tl.tile(it, is_full);
    const int64_t k0 = (int64_t)kt * kTile;
    const bool check_k = k0 + kTile > seq.Sk;
    const bool check_mask = !is_full && p.mask_kind != 0;

    __syncthreads();  // previous tile's LDS reads are done
    // K tile -> LDS, row-major
    for (int c = tid; c < kTile * D / 8; c += 256) {
      const int r = c / (D / 8);
      const int c8 = c % (D / 8);
      const int64_t key = k0 + r;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (key < seq.Sk) val = *reinterpret_cast<const uint4*>(kbase + key * p.k_sk + c8 * 8);
      *reinterpret_cast<uint4*>(&sm.k[r * KP + c8 * 8]) = val;
    }
    // V tile -> LDS, transposed: item = 4 keys x 8 dims
    for (int c = tid; c < (kTile / 4) * (D / 8); c += 256) {
      const int oct = c % (D / 8);
      const int kq = c / (D / 8);
      uint32_t rw[4][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t key = k0 + 4 * kq + j;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (key < seq.Sk) val = *reinterpret_cast<const uint4*>(vbase + key * p.v_sk + oct * 8);
        rw[j][0] = val.x;
        rw[j][1] = val.y;
        rw[j][2] = val.z;
        rw[j][3] = val.w;
      }
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const int wd = d >> 1;
        uint32_t lo, hi;
        if (d & 1) {
          lo = (rw[0][wd] >> 16) | (rw[1][wd] & 0xFFFF0000u);
          hi = (rw[2][wd] >> 16) | (rw[3][wd] & 0xFFFF0000u);
        } else {
          lo = (rw[0][wd] & 0xFFFFu) | (rw[1][wd] << 16);
          hi = (rw[2][wd] & 0xFFFFu) | (rw[3][wd] << 16);
        }
        *reinterpret_cast<uint2*>(&sm.vt[(oct * 8 + d) * VP + 4 * kq]) = make_uint2(lo, hi);
      }
    }
    __syncthreads();

    // Two halves of 64 keys: S^T = K Q^T (lane's scores are keys
    // 16 (u/8) + 8 hh + u%8 of each 32-key chunk), online softmax, O^T += V^T P^T.
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x16 sacc[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int kc = 2 * half + c;
        sacc[c] = f32x16{};
        const __bf16* krow = &sm.k[(kc * 32 + perm_row(n)) * KP + 8 * hh];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + 16 * s);
          sacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[c], 0, 0, 0);
        }
      }
      pipe::pin_reads_ahead<2 * NS, 3, 1, 1>();

      // scale, bias, mask; row max over this half
      float mloc = -INFINITY;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int kc = 2 * half + c;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int64_t kb = k0 + kc * 32 + 16 * st + 8 * hh;  // 8 consecutive keys
          float bv[8];
          if (brow) {
            const uint4 raw = *reinterpret_cast<const uint4*>(brow + kb);
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
            if (p.mask_kind == 2) {
              uint2 mb = make_uint2(0, 0);
              if (mrow) mb = *reinterpret_cast<const uint2*>(mrow + kb);
              mbits = 0;
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const uint32_t byte = ((e < 4 ? mb.x : mb.y) >> (8 * (e & 3))) & 0xFFu;
                mbits |= (byte != 0u ? 1u : 0u) << e;
              }
            } else {
              mbits = 0;
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const int64_t key = kb + e;
                const bool keep =
                    (key >= iv.lo1 && key < iv.hi1) || (key >= iv.lo2 && key < iv.hi2);
                mbits |= (keep ? 1u : 0u) << e;
              }
            }
          }
          if (!qvalid) mbits = 0;
          if (check_k) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (kb + e >= seq.Sk) mbits &= ~(1u << e);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int u = 8 * st + e;
            float sv = sacc[c][u] * p.scale_log2 + bv[e];
            sv = ((mbits >> e) & 1u) ? sv : -INFINITY;
            sacc[c][u] = sv;
            mloc = fmaxf(mloc, sv);
          }
        }
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      const float m_new = fmaxf(m_run, mloc);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float lsum = 0.f;
      bf16x8 pf[2][2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float e = fast_exp2(sacc[c][u] - m_use);
          lsum += e;
          pf[c][u >> 3][u & 7] = (__bf16)e;
        }
      }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) oacc[dc] *= alpha;

#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
        const __bf16* vrow = &sm.vt[(dc * 32 + n) * VP + 8 * hh];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int kc = 2 * half + c;
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(vrow + kc * 32 + 16 * st);
            oacc[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[c][st], oacc[dc], 0, 0, 0);
          }
        }
      }
      pipe::pin_reads_ahead<4 * NDC, 3, 1, 1>();
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (qvalid) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    __bf16* orow = reinterpret_cast<__bf16*>(p.o) + (int64_t)b * p.o_sb +
                   (seq.q0 + q) * p.o_sq + (int64_t)h * p.o_sh;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(oacc[dc][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + dc * 32 + 8 * g + 4 * hh) = v4;
      }
    }
    if (p.lse && hh == 0) {
      const float lse = l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
      p.lse[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + (seq.q0 + q) * p.lse_sq] = lse;
    }
  }
}

// ---------------------------------------------------------------------------
// float path: vector-ALU products, 16 queries x (16 threads per query), so
// that short query blocks still spread over many workgroups

// x of another lane of the same 16-lane row (DPP control CTRL), one VALU op
template <int CTRL>
__device__ inline float dpp_swap(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// sum over the 16 lanes of a row: quad xor 1 and xor 2 (quad_perm [1,0,3,2],
// [2,3,0,1]), then the two quads of each half row (row_half_mirror) and the
// two halves (row_mirror)
__device__ inline float row16_sum(float x) {
  x += dpp_swap<0xB1>(x);
  x += dpp_swap<0x4E>(x);
  x += dpp_swap<0x141>(x);
  x += dpp_swap<0x140>(x);
  return x;
}
constexpr int kF32Tpq = 16;                 // threads per query
constexpr int kF32Rows = 256 / kF32Tpq;    // queries per workgroup
constexpr int kF32Keys = 64;

template <int D>
__global__ __launch_bounds__(256) void k_attn_f32(AttnParams p) {
  constexpr int DS = D / kF32Tpq;  // dims per thread
  constexpr int P = D + 4;    // LDS pitch in floats
  __shared__ __align__(16) float sk[kF32Keys * P];
  __shared__ __align__(16) float sv[kF32Keys * P];

  const int rt = blockIdx.x;  // block of kF32Rows rows
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int part = tid & (kF32Tpq - 1);
  const SeqView seq = seq_view(p, b);
  if (rt * kF32Rows >= seq.Sq) return;  // past a packed sequence's end (uniform)
  const int q = rt * kF32Rows + tid / kF32Tpq;
  const bool qvalid = q < seq.Sq;
  const int kvh = h / p.G;
  const int qt = (rt * kF32Rows) / kTile;

  float qv[DS];
  {
    const float* qrow = reinterpret_cast<const float*>(p.q) + (int64_t)b * p.q_sb +
                        (seq.q0 + q) * p.q_sq + (int64_t)h * p.q_sh + part * DS;
#pragma unroll
    for (int i = 0; i < DS; ++i) qv[i] = qvalid ? qrow[i] : 0.f;
  }
  RowIv iv{0, 0, 0, 0};
  if (p.mask_kind == 1) iv = dflash_row(seq.rule, p.pred_row0 ? 0 : q);
  const uint8_t* mrow =
      (p.mask_kind == 2 && qvalid) ? aux_row(p.mask, 1, b, h, p.G, q) : nullptr;
  const float* brow = (p.has_bias && qvalid)
      ? reinterpret_cast<const float*>(aux_row(p.bias, 4, b, h, p.G, q)) : nullptr;
  const float* kbase = reinterpret_cast<const float*>(p.k) + (int64_t)b * p.k_sb +
                       seq.k0 * p.k_sk + (int64_t)kvh * p.k_sh;
  const float* vbase = reinterpret_cast<const float*>(p.v) + (int64_t)b * p.v_sb +
                       seq.k0 * p.v_sk + (int64_t)kvh * p.v_sh;

  float o[DS];
#pragma unroll
  for (int i = 0; i < DS; ++i) o[i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  TileList tl;
  tl.init(p, b, h, qt, seq.nK);
  const int ntiles = tl.count();
  for (int it = 0; it < ntiles; ++it) {
    bool is_full;
    const int kt = tl.tile(it, is_full);
    const bool check_mask = !is_full && p.mask_kind != 0;
    for (int half = 0; half < kTile / kF32Keys; ++half) {
      const int64_t k0 = (int64_t)kt * kTile + half * kF32Keys;
      __syncthreads();
      for (int c = tid; c < kF32Keys * D / 4; c += 256) {
        const int r = c / (D / 4);
        const int c4 = c % (D / 4);
        const int64_t key = k0 + r;
        float4 kv4 = make_float4(0, 0, 0, 0), vv4 = make_float4(0, 0, 0, 0);
        if (key < seq.Sk) {
          kv4 = *reinterpret_cast<const float4*>(kbase + key * p.k_sk + c4 * 4);
          vv4 = *reinterpret_cast<const float4*>(vbase + key * p.v_sk + c4 * 4);
        }
        *reinterpret_cast<float4*>(&sk[r * P + c4 * 4]) = kv4;
        *reinterpret_cast<float4*>(&sv[r * P + c4 * 4]) = vv4;
      }
      __syncthreads();
      // fully unrolled key loops: s[] stays in registers
      float s[kF32Keys];
      float mloc = -INFINITY;
#pragma unroll
      for (int j = 0; j < kF32Keys; ++j) {
        const float* kr = &sk[j * P + part * DS];
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < DS; ++i) acc = fmaf(qv[i], kr[i], acc);
        acc = row16_sum(acc);  // the query's 16 threads are one DPP row
        const int64_t key = k0 + j;
        float sc = acc * p.scale_log2;
        if (brow && key < seq.Sk) sc += bias_log2(brow[key]);
        bool keep = qvalid && key < seq.Sk;
        if (keep && check_mask) {
          if (p.mask_kind == 2)
            keep = mrow[key] != 0;
          else
            keep = (key >= iv.lo1 && key < iv.hi1) || (key >= iv.lo2 && key < iv.hi2);
        }
        sc = keep ? sc : -INFINITY;
        s[j] = sc;
        mloc = fmaxf(mloc, sc);
      }
      const float m_new = fmaxf(m_run, mloc);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DS; ++i) o[i] *= alpha;
#pragma unroll
      for (int j = 0; j < kF32Keys; ++j) {
        const float e = exp2f(s[j] - m_use);
        l_run += e;
        const float* vr = &sv[j * P + part * DS];
#pragma unroll
        for (int i = 0; i < DS; ++i) o[i] = fmaf(e, vr[i], o[i]);
      }
      m_run = m_new;
    }
  }
  if (qvalid) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* orow = reinterpret_cast<float*>(p.o) + (int64_t)b * p.o_sb + (seq.q0 + q) * p.o_sq +
                  (int64_t)h * p.o_sh + part * DS;
#pragma unroll
    for (int i = 0; i < DS; ++i) orow[i] = o[i] * inv;
    if (p.lse && part == 0)
      p.lse[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + (seq.q0 + q) * p.lse_sq] =
          l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnParams& p, int D, hipStream_t s) {
  const dim3 grid((unsigned)p.nQ, (unsigned)p.H, (unsigned)p.B);
  if (D == 128)
    hipLaunchKernelGGL(k_attn_bf16<128>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(k_attn_bf16<64>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnParams& p, int D, hipStream_t s) {
  const unsigned rt = (unsigned)((p.Sq + kF32Rows - 1) / kF32Rows);
  const dim3 grid(rt, (unsigned)p.H, (unsigned)p.B);
  if (D == 128)
    hipLaunchKernelGGL(k_attn_f32<128>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(k_attn_f32<64>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace bsm
