// Kept-key list of a dense mask over a short query block (at most 32 rows per
// (b, h) in the attention's iteration space), for the key-gather decode.
//
// For each (bm, hm) the list holds, in ascending order, the keys j < Sk that at
// least one of the R rows keeps, and per listed key a word whose bit r says
// whether row r keeps it. Under the seqlen_q == 1 head-group swap
// (flash-sparse-attention PR #190, Design) the rows are the G heads of a KV
// group, so with a dynamic top-k mask (PR #197, Design) the list is the union
// of G top-k sets: a small part of the key range.
//
// One workgroup per (bm, hm) streams the R mask rows once, 16 contiguous bytes
// per thread per row and 16384 keys per pass (a decode row of 16K keys is one
// pass: one load round trip, one scan), ORs the rows into per-key words, and
// compacts the keys with a non-zero word by a workgroup prefix count.
#include "block_scan.h"
#include "bsm_internal.h"

namespace bsm {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kPer = 16;                 // keys per thread per pass
constexpr int kPass = kThreads * kPer;   // keys per pass

__device__ inline uint32_t byte_of(const uint4& v, int e) {
  const uint32_t w = e < 4 ? v.x : (e < 8 ? v.y : (e < 12 ? v.z : v.w));
  return (w >> (8 * (e & 3))) & 0xFFu;
}

__global__ __launch_bounds__(kThreads) void k_key_list(KeyListParams p) {
  __shared__ int s_wave[kWaves];
  const int64_t bm = blockIdx.x / p.Hm;
  const int64_t hm = blockIdx.x % p.Hm;
  const uint8_t* base = p.mask + bm * p.sb + hm * p.sh;
  const int64_t out0 = (int64_t)blockIdx.x * p.K;
  const int nrows = p.Qm == 1 ? 1 : p.R;
  const uint32_t all_rows = p.R >= 32 ? 0xFFFFFFFFu : ((1u << p.R) - 1u);
  int taken = 0;
  for (int64_t c0 = 0; c0 < p.Sk; c0 += kPass) {
    const int64_t k0 = c0 + (int64_t)threadIdx.x * kPer;
    uint32_t w[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) w[e] = 0;
    if (k0 < p.Sk) {
      // k0 is a multiple of 16 below Sk <= K (a multiple of 128): the 16
      // bytes lie inside the row
      // four rows' loads in flight at a time
      for (int r0 = 0; r0 < nrows; r0 += 4) {
        uint4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[i] = r0 + i < nrows ? *reinterpret_cast<const uint4*>(base + (r0 + i) * p.sq + k0)
                                : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < kPer; ++e)
            w[e] |= (byte_of(v[i], e) != 0u ? 1u : 0u) << ((r0 + i) & 31);
      }
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        if (p.Qm == 1) w[e] = w[e] ? all_rows : 0u;
        if (k0 + e >= p.Sk) w[e] = 0u;
      }
    }
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) cnt += w[e] != 0u;
    int tot;
    int pos = taken + block_excl_sum<kWaves>(cnt, s_wave, tot);
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      if (w[e]) {
        p.idx[out0 + pos] = (int32_t)(k0 + e);
        p.bits[out0 + pos] = w[e];
        ++pos;
      }
    }
    taken += tot;
  }
  if (threadIdx.x == 0) p.num[blockIdx.x] = taken;
}

}  // namespace

hipError_t launch_key_list(const KeyListParams& p, hipStream_t s) {
  const int64_t n = p.Bm * p.Hm;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_key_list, dim3((unsigned)n), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace bsm
