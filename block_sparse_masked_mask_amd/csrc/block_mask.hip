// Block-mask builders for gfx950.
//
// A block mask splits the (query x key) plane into 128 x 128 tiles and lists,
// per query tile, the key tiles that are partial (some pairs kept) and full (all
// pairs kept), ascending and -1 padded -- the partial/full split flex_attention's
// create_block_mask returns (SpecForge issue #452, traceback), built here without
// its dense (B, H, Q, K) temporary and with one copy shared across heads
// (issue #452, Expected Behavior). Keys >= Sk never count as kept
// (flash-sparse-attention PR #190, Implementation Notes).
//
//  * k_block_mask_pred: DFlash predicate -> block mask. One workgroup per query
//    tile; per-row kept keys are two intervals, so a tile's kept-pair count is a
//    sum of interval overlaps and no mask byte is ever formed. Integer / ALU work.
//  * k_dflash_dense: the same predicate written out as a dense bool mask (the
//    dense SDPA-style mask of SpecForge issue #474, Suggestion 2). HBM-write bound.
//  * k_bm_dense_classify + k_bm_compact: dense bool mask -> block mask. The
//    classify pass is the HBM-bound one: each workgroup streams a 128-row x
//    1024-key strip with 16-byte loads (one wave-wide load covers one row's
//    1024 contiguous bytes, 8 lanes per key tile), folds any/all per lane with
//    word arithmetic, reduces per tile with wave ballots and writes a class code
//    per tile into kv_indices. The compact pass turns each row of codes into the
//    two ascending index lists with ballot prefix counts.
#include "bsm_internal.h"
#include "dflash_rows.h"

namespace bsm {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// Exclusive prefix count of `flag` over the workgroup in thread order.
// Every thread must call it. `tot` receives the workgroup total.
__device__ inline int block_flag_scan(bool flag, int* s_wave, int& tot) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const unsigned long long bal = __ballot(flag);
  const int pre = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) s_wave[w] = __popcll(bal);
  __syncthreads();
  int off = 0;
  tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int t = s_wave[i];
    off += i < w ? t : 0;
    tot += t;
  }
  __syncthreads();
  return off + pre;
}

// Writes the partial/full lists of one query tile from per-tile class codes
// (0 empty, 1 partial, 2 full) provided by code_of(kt).
template <typename CodeFn>
__device__ inline void compact_row(int nK, CodeFn code_of, int32_t* prow,
                                   int32_t* frow, int32_t* pnum, int32_t* fnum) {
  __shared__ int s_wave[2][kWaves];
  int np = 0, nf = 0;
  for (int base = 0; base < nK; base += kThreads) {
    const int kt = base + threadIdx.x;
    const int c = kt < nK ? code_of(kt) : 0;
    int tp, tf;
    const int op = block_flag_scan(c == 1, s_wave[0], tp);
    const int of = block_flag_scan(c == 2, s_wave[1], tf);
    if (c == 1) prow[np + op] = kt;
    if (c == 2) frow[nf + of] = kt;
    np += tp;
    nf += tf;
  }
  for (int kt = np + threadIdx.x; kt < nK; kt += kThreads) prow[kt] = -1;
  for (int kt = nf + threadIdx.x; kt < nK; kt += kThreads) frow[kt] = -1;
  if (threadIdx.x == 0) {
    *pnum = np;
    *fnum = nf;
  }
}

// Partial / full key tiles of query tile qt of one DFlash sequence of Sq
// queries whose keys fill nKs tiles; the row holds nK entries (nK >= nKs, the
// rest empty). A query tile past the sequence's end has no tiles.
__device__ inline void pred_tile_row(const DFlashRule& r, int64_t Sq, int qt, int nKs, int nK,
                                     int32_t* kv_num, int32_t* kv_idx, int32_t* full_num,
                                     int32_t* full_idx) {
  __shared__ int64_t s_iv[kTile][4];
  const int64_t r0 = (int64_t)qt * kTile;
  const int64_t left = Sq - r0;
  const int rows = (int)(left < 0 ? 0 : (left < kTile ? left : kTile));
  for (int t = threadIdx.x; t < rows; t += kThreads) {
    const RowIv v = dflash_row(r, r0 + t);
    s_iv[t][0] = v.lo1;
    s_iv[t][1] = v.hi1;
    s_iv[t][2] = v.lo2;
    s_iv[t][3] = v.hi2;
  }
  __syncthreads();
  auto code_of = [&](int kt) {
    if (kt >= nKs) return 0;
    const int64_t k0 = (int64_t)kt * kTile;
    int64_t cnt = 0;
    for (int t = 0; t < rows; ++t)
      cnt += iv_overlap(s_iv[t][0], s_iv[t][1], k0, kTile) +
             iv_overlap(s_iv[t][2], s_iv[t][3], k0, kTile);
    return cnt == 0 ? 0 : (cnt == (int64_t)rows * kTile ? 2 : 1);
  };
  compact_row(nK, code_of, kv_idx, full_idx, kv_num, full_num);
}

__global__ __launch_bounds__(kThreads) void k_block_mask_pred(
    DFlashRule r, int64_t Sq, int nK, int32_t* kv_num, int32_t* kv_idx,
    int32_t* full_num, int32_t* full_idx) {
  const int qt = blockIdx.x;
  pred_tile_row(r, Sq, qt, nK, nK, kv_num + qt, kv_idx + (int64_t)qt * nK, full_num + qt,
                full_idx + (int64_t)qt * nK);
}

// Packed sequences: workgroup (qt, b) builds row (b, qt) from sequence b's own
// geometry (C_b = Sk_b - Sq_b, S_b = C_b / NB_b unless fixed).
__global__ __launch_bounds__(kThreads) void k_block_mask_pred_varlen(
    DFlashRule r, const int32_t* cu_q, const int32_t* cu_k, int nQ, int nK,
    int32_t* kv_num, int32_t* kv_idx, int32_t* full_num, int32_t* full_idx) {
  const int qt = blockIdx.x;
  const int b = blockIdx.y;
  const int64_t Sq = cu_q[b + 1] - cu_q[b];
  const int64_t Sk = cu_k[b + 1] - cu_k[b];
  DFlashRule sr = r;
  sr.C = Sk - Sq;
  if (r.S == 0) {
    const int64_t nb = Sq / r.bs;
    sr.S = nb > 0 ? sr.C / nb : 0;
  }
  const int64_t row = (int64_t)b * nQ + qt;
  pred_tile_row(sr, Sq, qt, (int)((Sk + kTile - 1) / kTile), nK, kv_num + row,
                kv_idx + row * nK, full_num + row, full_idx + row * nK);
}

__global__ __launch_bounds__(kThreads) void k_dflash_dense(DFlashRule r, int64_t Sq,
                                                          int64_t K, uint8_t* out) {
  const int64_t chunks = K / 16;
  for (int64_t q = blockIdx.x; q < Sq; q += gridDim.x) {
    const RowIv v = dflash_row(r, q);
    uint8_t* row = out + q * K;
    for (int64_t c = threadIdx.x; c < chunks; c += kThreads) {
      const int64_t k0 = c * 16;
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t x = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int64_t k = k0 + 4 * j + b;
          const bool keep = (k >= v.lo1 && k < v.hi1) || (k >= v.lo2 && k < v.hi2);
          x |= (uint32_t)keep << (8 * b);
        }
        w[j] = x;
      }
      *reinterpret_cast<uint4*>(row + k0) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// 1 iff some byte of x is zero (exact for every byte value).
__device__ inline uint32_t has_zero_byte(uint32_t x) {
  return ((x - 0x01010101u) & ~x & 0x80808080u) != 0u;
}

constexpr int kStripKeys = 1024;  // keys per strip: 64 lanes x 16 bytes
constexpr int kRowsInFlight = 8;

template <bool kVec>
__global__ __launch_bounds__(kThreads) void k_bm_dense_classify(
    DenseMaskView m, int nQm, int nK, int nStrips, int32_t* codes) {
  int64_t id = blockIdx.x;
  const int ks = (int)(id % nStrips);
  id /= nStrips;
  const int qt = (int)(id % nQm);
  id /= nQm;
  const int64_t hm = id % m.Hm;
  const int64_t bm = id / m.Hm;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t key0 = (int64_t)ks * kStripKeys + lane * 16;
  const bool active = key0 < m.K;
  // bytes of this lane's 16 keys that lie below Sk
  uint32_t kmask[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t x = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) x |= (key0 + 4 * j + b < m.Sk ? 0xFFu : 0u) << (8 * b);
    kmask[j] = x;
  }
  const int64_t r0 = (int64_t)qt * kTile;
  const int rows = (int)(m.Qm - r0 < kTile ? m.Qm - r0 : kTile);
  const uint8_t* base = m.data + bm * m.sb + hm * m.sh + r0 * m.sq + key0;
  uint32_t any = 0, zero = 0;
  for (int rb = w; rb < rows; rb += kWaves * kRowsInFlight) {
    uint4 x[kRowsInFlight];
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u) {
      const int r = rb + u * kWaves;
      x[u] = make_uint4(0, 0, 0, 0);
      if (active && r < rows) {
        const uint8_t* p = base + (int64_t)r * m.sq;
        if (kVec) {
          x[u] = *reinterpret_cast<const uint4*>(p);
        } else {
          uint32_t t[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            t[j] = (uint32_t)p[4 * j] | ((uint32_t)p[4 * j + 1] << 8) |
                   ((uint32_t)p[4 * j + 2] << 16) | ((uint32_t)p[4 * j + 3] << 24);
          x[u] = make_uint4(t[0], t[1], t[2], t[3]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u) {
      if (rb + u * kWaves < rows) {
        const uint32_t a = x[u].x & kmask[0], b = x[u].y & kmask[1];
        const uint32_t c = x[u].z & kmask[2], d = x[u].w & kmask[3];
        any |= a | b | c | d;
        zero |= has_zero_byte(a) | has_zero_byte(b) | has_zero_byte(c) | has_zero_byte(d);
      }
    }
  }
  __shared__ unsigned long long s_any[kWaves], s_zero[kWaves];
  const unsigned long long ab = __ballot(any != 0u);
  const unsigned long long zb = __ballot(zero != 0u);
  if (lane == 0) {
    s_any[w] = ab;
    s_zero[w] = zb;
  }
  __syncthreads();
  if (threadIdx.x < kStripKeys / kTile) {
    const int t = threadIdx.x;
    const int kt = ks * (kStripKeys / kTile) + t;
    if (kt < nK) {
      unsigned long long a = 0, z = 0;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) {
        a |= s_any[i];
        z |= s_zero[i];
      }
      const bool tany = ((a >> (8 * t)) & 0xFFull) != 0ull;
      const bool tfull = ((z >> (8 * t)) & 0xFFull) == 0ull;
      const int code = !tany ? 0 : (tfull ? 2 : 1);
      codes[((bm * m.Hm + hm) * nQm + qt) * (int64_t)nK + kt] = code;
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_bm_compact(int nK, int32_t* kv_num,
                                                        int32_t* kv_idx,
                                                        int32_t* full_num,
                                                        int32_t* full_idx) {
  extern __shared__ uint8_t s_code[];
  const int64_t row = blockIdx.x;
  int32_t* prow = kv_idx + row * nK;
  for (int kt = threadIdx.x; kt < nK; kt += kThreads) s_code[kt] = (uint8_t)prow[kt];
  __syncthreads();
  auto code_of = [&](int kt) { return (int)s_code[kt]; };
  compact_row(nK, code_of, prow, full_idx + row * nK, kv_num + row, full_num + row);
}

}  // namespace

hipError_t launch_block_mask_pred(const DFlashRule& r, int64_t Sq, int64_t Sk,
                                  int64_t nQ, int64_t nK, int32_t* kv_num,
                                  int32_t* kv_idx, int32_t* full_num,
                                  int32_t* full_idx, hipStream_t s) {
  (void)Sk;
  if (nQ == 0) return hipSuccess;
  hipLaunchKernelGGL(k_block_mask_pred, dim3((unsigned)nQ), dim3(kThreads), 0, s, r,
                     Sq, (int)nK, kv_num, kv_idx, full_num, full_idx);
  return hipGetLastError();
}

hipError_t launch_block_mask_pred_varlen(const DFlashRule& r, const int32_t* cu_q,
                                         const int32_t* cu_k, int64_t B, int64_t nQ,
                                         int64_t nK, int32_t* kv_num, int32_t* kv_idx,
                                         int32_t* full_num, int32_t* full_idx, hipStream_t s) {
  if (B == 0 || nQ == 0) return hipSuccess;
  hipLaunchKernelGGL(k_block_mask_pred_varlen, dim3((unsigned)nQ, (unsigned)B), dim3(kThreads),
                     0, s, r, cu_q, cu_k, (int)nQ, (int)nK, kv_num, kv_idx, full_num, full_idx);
  return hipGetLastError();
}

hipError_t launch_dflash_dense(const DFlashRule& r, int64_t Sq, int64_t Sk,
                               int64_t K, uint8_t* out, hipStream_t s) {
  (void)Sk;
  if (Sq == 0 || K == 0) return hipSuccess;
  const int64_t grid = Sq < 65536 ? Sq : 65536;
  hipLaunchKernelGGL(k_dflash_dense, dim3((unsigned)grid), dim3(kThreads), 0, s, r, Sq,
                     K, out);
  return hipGetLastError();
}

hipError_t launch_block_mask_dense(const DenseMaskView& m, int32_t* kv_num,
                                   int32_t* kv_idx, int32_t* full_num,
                                   int32_t* full_idx, hipStream_t s) {
  const int64_t nQm = (m.Qm + kTile - 1) / kTile;
  const int64_t nK = m.K / kTile;
  const int64_t rows = m.Bm * m.Hm * nQm;
  if (rows == 0) return hipSuccess;
  if (nK > 0) {
    const int64_t nStrips = (m.K + kStripKeys - 1) / kStripKeys;
    const int64_t grid = rows * nStrips;
    const bool vec = ((uintptr_t)m.data % 16 == 0) && (m.sb % 16 == 0) &&
                     (m.sh % 16 == 0) && (m.sq % 16 == 0);
    if (vec)
      hipLaunchKernelGGL(k_bm_dense_classify<true>, dim3((unsigned)grid), dim3(kThreads),
                         0, s, m, (int)nQm, (int)nK, (int)nStrips, kv_idx);
    else
      hipLaunchKernelGGL(k_bm_dense_classify<false>, dim3((unsigned)grid),
                         dim3(kThreads), 0, s, m, (int)nQm, (int)nK, (int)nStrips,
                         kv_idx);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_bm_compact, dim3((unsigned)rows), dim3(kThreads), (size_t)nK, s,
                     (int)nK, kv_num, kv_idx, full_num, full_idx);
  return hipGetLastError();
}

}  // namespace bsm
