// Masked attention backward, generic path (any dtype of the library, D = 64 or
// 128): one wave per query row for dQ and one wave per key for dK / dV, lanes
// across the head dim, float arithmetic throughout.
//
// What it computes (gradients of the forward of flash-sparse-attention PR
// #190, Design, with the broadcast dbias reductions of its Changes: mha_bwd):
// with P = exp(s - LSE) on kept keys (0 elsewhere, 0 on rows whose LSE is
// -inf), dP = dO V^T, Delta = rowsum(dO * O) and dS = P * (dP - Delta):
//   dQ = scale * dS K,  dK = scale * dS^T Q,  dV = P^T dO   (dK, dV summed over
//   the G heads of a KV group), dbias += dS over every (b, h, q) that reads the
//   element. Rows and key tiles are visited exactly as the forward does: key
//   tiles from the block mask (full ones without a test), keys >= Sk never.
#include <math.h>

#include "attn_common.h"
#include "bsm_internal.h"
#include "dflash_rows.h"

namespace bsm {
namespace {

constexpr int kWavesPerBlock = 4;

__device__ inline float ld_elem(const uint16_t* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}
__device__ inline float ld_elem(const float* p, int64_t i) { return p[i]; }
__device__ inline void st_elem(uint16_t* p, int64_t i, float x) {
  p[i] = __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ inline void st_elem(float* p, int64_t i, float x) { p[i] = x; }

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Per-lane slice of a D-vector: d = lane + 64 t.
template <int D>
struct Vec {
  static constexpr int N = D / 64;
  float x[N];
};

template <typename T, int D>
__device__ inline Vec<D> load_vec(const T* row, int lane) {
  Vec<D> v;
#pragma unroll
  for (int t = 0; t < Vec<D>::N; ++t) v.x[t] = ld_elem(row, lane + 64 * t);
  return v;
}

template <int D>
__device__ inline float dot(const Vec<D>& a, const Vec<D>& b) {
  float s = 0.f;
#pragma unroll
  for (int t = 0; t < Vec<D>::N; ++t) s = fmaf(a.x[t], b.x[t], s);
  return wave_sum(s);
}

// Is key j of row q kept on a partial tile (the mask test of the forward)?
__device__ inline bool kept_partial(const AttnParams& f, const RowIv& iv, const uint8_t* mrow,
                                    int64_t j) {
  if (f.mask_kind == 1) return (j >= iv.lo1 && j < iv.hi1) || (j >= iv.lo2 && j < iv.hi2);
  if (f.mask_kind == 2) return mrow[j] != 0;
  return true;
}

// Class of tile (qt, kt) for head h: 0 empty, 1 partial, 2 full.
__device__ inline int tile_class(const AttnParams& f, int b, int h, int qt, int kt) {
  if (!f.has_bm) return f.mask_kind == 0 ? 2 : 1;
  const BlockMaskView& m = f.bm;
  const int64_t mb = m.Bm == 1 ? 0 : b;
  const int64_t mh = head_index(m.h_mode, h, f.G);
  const int64_t mq = m.nQm == 1 ? 0 : qt;
  const int64_t r = (mb * m.Hm + mh) * m.nQm + mq;
  // both lists are ascending
  auto find = [&](const int32_t* idx, int n) {
    int lo = 0, hi = n;
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

__device__ inline float bias_at(const AttnParams& f, int b, int h, int q, int64_t j, bool bf16) {
  if (!f.has_bias) return 0.f;
  const uint8_t* row = aux_row(f.bias, bf16 ? 2 : 4, b, h, f.G, q);
  return bias_nat(bf16 ? ld_elem(reinterpret_cast<const uint16_t*>(row), j)
                       : ld_elem(reinterpret_cast<const float*>(row), j));
}

// Products of the 16 bytes a lane holds of O and dO (8 bf16 or 4 floats), summed.
template <typename T>
__device__ inline float dot16(uint4 a, uint4 b) {
  const uint32_t x[4] = {a.x, a.y, a.z, a.w};
  const uint32_t y[4] = {b.x, b.y, b.z, b.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (sizeof(T) == 2) {
      s = fmaf(__uint_as_float(x[i] << 16), __uint_as_float(y[i] << 16), s);
      s = fmaf(__uint_as_float(x[i] & 0xFFFF0000u), __uint_as_float(y[i] & 0xFFFF0000u), s);
    } else {
      s = fmaf(__uint_as_float(x[i]), __uint_as_float(y[i]), s);
    }
  }
  return s;
}

// Delta = rowsum(dO * O), one row per D * sizeof(T) / 16 lanes (16-byte loads).
template <typename T, int D>
__global__ __launch_bounds__(256) void k_bwd_delta(AttnBwdParams p) {
  constexpr int LPR = D * (int)sizeof(T) / 16;  // lanes per row
  constexpr int EPL = 16 / (int)sizeof(T);      // elements per lane
  const AttnParams& f = p.f;
  const int64_t nrows = (int64_t)f.B * f.H * f.Sq;
  const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  float s = 0.f;
  if (row < nrows) {
    const int q = (int)(row % f.Sq);
    const int64_t bh = row / f.Sq;
    const int h = (int)(bh % f.H);
    const int b = (int)(bh / f.H);
    const T* o = reinterpret_cast<const T*>(f.o) + b * f.o_sb + q * f.o_sq + h * f.o_sh;
    const T* dO = reinterpret_cast<const T*>(p.dout) + b * p.do_sb + q * p.do_sq + h * p.do_sh;
    s = dot16<T>(*reinterpret_cast<const uint4*>(o + c * EPL),
                 *reinterpret_cast<const uint4*>(dO + c * EPL));
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  if (row < nrows && c == 0) p.delta[row] = s;
}

template <typename T, int D>
__global__ __launch_bounds__(64 * kWavesPerBlock) void k_bwd_dq(AttnBwdParams p) {
  const AttnParams& f = p.f;
  constexpr bool kBf16 = sizeof(T) == 2;
  const int64_t row = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= (int64_t)f.B * f.H * f.Sq) return;
  const int q = (int)(row % f.Sq);
  const int64_t bh = row / f.Sq;
  const int h = (int)(bh % f.H);
  const int b = (int)(bh / f.H);
  const int kvh = h / f.G;
  const float lse = f.lse[b * f.lse_sb + h * f.lse_sh + q * f.lse_sq];
  const float delta = p.delta[row];
  const Vec<D> qv = load_vec<T, D>(
      reinterpret_cast<const T*>(f.q) + b * f.q_sb + q * f.q_sq + h * f.q_sh, lane);
  const Vec<D> dov = load_vec<T, D>(
      reinterpret_cast<const T*>(p.dout) + b * p.do_sb + q * p.do_sq + h * p.do_sh, lane);
  const T* kb = reinterpret_cast<const T*>(f.k) + b * f.k_sb + kvh * f.k_sh;
  const T* vb = reinterpret_cast<const T*>(f.v) + b * f.v_sb + kvh * f.v_sh;
  RowIv iv{0, 0, 0, 0};
  if (f.mask_kind == 1) iv = dflash_row(f.rule, f.pred_row0 ? 0 : q);
  const uint8_t* mrow = f.mask_kind == 2 ? aux_row(f.mask, 1, b, h, f.G, q) : nullptr;
  Vec<D> dq;
#pragma unroll
  for (int t = 0; t < Vec<D>::N; ++t) dq.x[t] = 0.f;
  if (lse != -INFINITY) {
    TileList tl;
    tl.init(f, b, h, q / kTile);
    for (int i = 0; i < tl.count(); ++i) {
      bool full;
      const int kt = tl.tile(i, full);
      const int64_t j1 = min((int64_t)(kt + 1) * kTile, (int64_t)f.Sk);
      for (int64_t j = (int64_t)kt * kTile; j < j1; ++j) {
        if (!full && !kept_partial(f, iv, mrow, j)) continue;
        const Vec<D> kv = load_vec<T, D>(kb + j * f.k_sk, lane);
        const Vec<D> vv = load_vec<T, D>(vb + j * f.v_sk, lane);
        const float s = p.scale * dot(qv, kv) + bias_at(f, b, h, q, j, kBf16);
        const float pr = expf(s - lse);
        const float ds = pr * (dot(dov, vv) - delta);
#pragma unroll
        for (int t = 0; t < Vec<D>::N; ++t) dq.x[t] = fmaf(ds, kv.x[t], dq.x[t]);
      }
    }
  }
  T* out = reinterpret_cast<T*>(p.dq) + b * p.dq_sb + q * p.dq_sq + h * p.dq_sh;
#pragma unroll
  for (int t = 0; t < Vec<D>::N; ++t) st_elem(out, lane + 64 * t, p.scale * dq.x[t]);
}

template <typename T, int D>
__global__ __launch_bounds__(64 * kWavesPerBlock) void k_bwd_dkdv(AttnBwdParams p) {
  const AttnParams& f = p.f;
  constexpr bool kBf16 = sizeof(T) == 2;
  const int64_t key = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (key >= (int64_t)f.B * f.KVH * f.Sk) return;
  const int64_t j = key % f.Sk;
  const int64_t bk = key / f.Sk;
  const int kvh = (int)(bk % f.KVH);
  const int b = (int)(bk / f.KVH);
  const int kt = (int)(j / kTile);
  const Vec<D> kv = load_vec<T, D>(
      reinterpret_cast<const T*>(f.k) + b * f.k_sb + j * f.k_sk + kvh * f.k_sh, lane);
  const Vec<D> vv = load_vec<T, D>(
      reinterpret_cast<const T*>(f.v) + b * f.v_sb + j * f.v_sk + kvh * f.v_sh, lane);
  Vec<D> dk, dv;
#pragma unroll
  for (int t = 0; t < Vec<D>::N; ++t) dk.x[t] = dv.x[t] = 0.f;
  for (int g = 0; g < f.G; ++g) {
    const int h = kvh * f.G + g;
    for (int qt = 0; qt < f.nQ; ++qt) {
      const int cls = tile_class(f, b, h, qt, kt);
      if (cls == 0) continue;
      const int q1 = min((qt + 1) * kTile, f.Sq);
      for (int q = qt * kTile; q < q1; ++q) {
        const float lse = f.lse[b * f.lse_sb + h * f.lse_sh + q * f.lse_sq];
        if (lse == -INFINITY) continue;
        if (cls == 1) {
          RowIv iv{0, 0, 0, 0};
          if (f.mask_kind == 1) iv = dflash_row(f.rule, f.pred_row0 ? 0 : q);
          const uint8_t* mrow = f.mask_kind == 2 ? aux_row(f.mask, 1, b, h, f.G, q) : nullptr;
          if (!kept_partial(f, iv, mrow, j)) continue;
        }
        const Vec<D> qv = load_vec<T, D>(
            reinterpret_cast<const T*>(f.q) + b * f.q_sb + q * f.q_sq + h * f.q_sh, lane);
        const Vec<D> dov = load_vec<T, D>(
            reinterpret_cast<const T*>(p.dout) + b * p.do_sb + q * p.do_sq + h * p.do_sh, lane);
        const float s = p.scale * dot(qv, kv) + bias_at(f, b, h, q, j, kBf16);
        const float pr = expf(s - lse);
        const float delta = p.delta[((int64_t)b * f.H + h) * f.Sq + q];
        const float ds = pr * (dot(dov, vv) - delta);
#pragma unroll
        for (int t = 0; t < Vec<D>::N; ++t) {
          dv.x[t] = fmaf(pr, dov.x[t], dv.x[t]);
          dk.x[t] = fmaf(ds, qv.x[t], dk.x[t]);
        }
        if (p.dbias_acc && lane == 0)
          atomicAdd(reinterpret_cast<float*>(
                        const_cast<uint8_t*>(aux_row(p.dbias, 4, b, h, f.G, q))) + j, ds);
      }
    }
  }
  T* dko = reinterpret_cast<T*>(p.dk) + b * p.dk_sb + j * p.dk_sk + kvh * p.dk_sh;
  T* dvo = reinterpret_cast<T*>(p.dv) + b * p.dv_sb + j * p.dv_sk + kvh * p.dv_sh;
#pragma unroll
  for (int t = 0; t < Vec<D>::N; ++t) {
    st_elem(dko, lane + 64 * t, p.scale * dk.x[t]);
    st_elem(dvo, lane + 64 * t, dv.x[t]);
  }
}

__global__ void k_fill_zero(float* x, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) x[i] = 0.f;
}

__global__ void k_dbias_out(DbiasOut d) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = d.n0 * d.n1 * d.n2 * d.K;
  if (i >= n) return;
  const int64_t k = i % d.K;
  int64_t r = i / d.K;
  const int64_t i2 = r % d.n2;
  r /= d.n2;
  const int64_t i1 = r % d.n1;
  const int64_t i0 = r / d.n1;
  const float x = k < d.Sk ? d.acc[i] : 0.f;
  const int64_t o = i0 * d.s0 + i1 * d.s1 + i2 * d.s2 + k;
  if (d.is_bf16)
    st_elem(reinterpret_cast<uint16_t*>(d.out), o, x);
  else
    st_elem(reinterpret_cast<float*>(d.out), o, x);
}

template <typename T, int D>
hipError_t launch_typed(const AttnBwdParams& p, hipStream_t s) {
  const dim3 blk(64 * kWavesPerBlock);
  const int64_t rows = (int64_t)p.f.B * p.f.H * p.f.Sq;
  const int64_t keys = (int64_t)p.f.B * p.f.KVH * p.f.Sk;
  if (rows == 0) {
    // no query attends to any key: dK = dV = 0, written by the row kernel's empty loop
    if (keys > 0)
      hipLaunchKernelGGL((k_bwd_dkdv<T, D>), dim3((keys + kWavesPerBlock - 1) / kWavesPerBlock),
                         blk, 0, s, p);
    return hipGetLastError();
  }
  constexpr int kDeltaRows = 256 / (D * (int)sizeof(T) / 16);  // rows per delta block
  hipLaunchKernelGGL((k_bwd_delta<T, D>), dim3((rows + kDeltaRows - 1) / kDeltaRows), dim3(256),
                     0, s, p);
  if (sizeof(T) == 2 && attn_bwd_mfma_applies(p, D)) return launch_attn_bwd_mfma(p, s);
  hipLaunchKernelGGL((k_bwd_dq<T, D>), dim3((rows + kWavesPerBlock - 1) / kWavesPerBlock), blk,
                     0, s, p);
  if (keys > 0)
    hipLaunchKernelGGL((k_bwd_dkdv<T, D>), dim3((keys + kWavesPerBlock - 1) / kWavesPerBlock),
                       blk, 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const AttnBwdParams& p, int D, int is_bf16, hipStream_t s) {
  if (is_bf16)
    return D == 128 ? launch_typed<uint16_t, 128>(p, s) : launch_typed<uint16_t, 64>(p, s);
  return D == 128 ? launch_typed<float, 128>(p, s) : launch_typed<float, 64>(p, s);
}

hipError_t launch_attn_bwd_delta(const AttnBwdParams& p, int D, int is_bf16, hipStream_t s) {
  const int64_t rows = (int64_t)p.f.B * p.f.H * p.f.Sq;
  if (rows == 0) return hipSuccess;
  const int epr = D * (is_bf16 ? 2 : 4) / 16;  // lanes per row
  const dim3 grid((unsigned)((rows + 256 / epr - 1) / (256 / epr)));
  if (is_bf16) {
    if (D == 128)
      hipLaunchKernelGGL((k_bwd_delta<uint16_t, 128>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((k_bwd_delta<uint16_t, 64>), grid, dim3(256), 0, s, p);
  } else {
    if (D == 128)
      hipLaunchKernelGGL((k_bwd_delta<float, 128>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((k_bwd_delta<float, 64>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* x, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_zero, dim3((n + 255) / 256), dim3(256), 0, s, x, n);
  return hipGetLastError();
}

hipError_t launch_dbias_out(const DbiasOut& d, hipStream_t s) {
  const int64_t n = d.n0 * d.n1 * d.n2 * d.K;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_dbias_out, dim3((n + 255) / 256), dim3(256), 0, s, d);
  return hipGetLastError();
}

}  // namespace bsm
