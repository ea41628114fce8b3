// Packing helpers for variable-length sequences (flash-sparse-attention PR
// #197, Changes: the integration's pad / unpad): the packing index of a padded
// batch's validity mask, and row copies through an index list.
//
// unpad_index runs three small passes: per-row counts of valid positions, one
// workgroup turning the counts into cu_seqlens, and per-row compaction that
// writes each valid position's flat index at cu_seqlens[b] + its rank in the
// row. Row copies move 16 bytes per thread.
#include "block_scan.h"
#include "bsm_internal.h"

namespace bsm {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__global__ __launch_bounds__(kThreads) void k_row_counts(const uint8_t* valid, int64_t seqlen,
                                                         int64_t row_stride, int32_t* cu) {
  __shared__ int s_wave[kWaves];
  const int b = blockIdx.x;
  const uint8_t* row = valid + (int64_t)b * row_stride;
  int cnt = 0;
  for (int64_t s = threadIdx.x; s < seqlen; s += kThreads) cnt += row[s] != 0;
  int tot;
  block_excl_sum<kWaves>(cnt, s_wave, tot);
  if (threadIdx.x == 0) cu[b + 1] = tot;
}

// cu[1 .. B] hold counts; make them running totals and set cu[0] = 0.
__global__ __launch_bounds__(kThreads) void k_scan_counts(int32_t* cu, int64_t B) {
  __shared__ int s_wave[kWaves];
  int carry = 0;
  for (int64_t c0 = 0; c0 < B; c0 += kThreads) {
    const int64_t i = c0 + threadIdx.x;
    const int v = i < B ? cu[i + 1] : 0;
    int tot;
    const int ex = block_excl_sum<kWaves>(v, s_wave, tot);
    if (i < B) cu[i + 1] = carry + ex + v;
    carry += tot;
  }
  if (threadIdx.x == 0) cu[0] = 0;
}

__global__ __launch_bounds__(kThreads) void k_row_compact(const uint8_t* valid, int64_t seqlen,
                                                          int64_t row_stride, const int32_t* cu,
                                                          int32_t* idx) {
  __shared__ int s_wave[kWaves];
  const int b = blockIdx.x;
  const uint8_t* row = valid + (int64_t)b * row_stride;
  int base = cu[b];
  for (int64_t s0 = 0; s0 < seqlen; s0 += kThreads) {
    const int64_t s = s0 + threadIdx.x;
    const int f = s < seqlen && row[s] != 0;
    int tot;
    const int ex = block_excl_sum<kWaves>(f, s_wave, tot);
    if (f) idx[base + ex] = (int32_t)((int64_t)b * seqlen + s);
    base += tot;
  }
}

template <bool kScatter>
__global__ __launch_bounds__(kThreads) void k_copy_rows(const char* src, int64_t src_stride,
                                                        char* dst, int64_t dst_stride,
                                                        int64_t chunks, const int32_t* idx,
                                                        int64_t n) {
  const int64_t total = n * chunks;
  for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * kThreads) {
    const int64_t i = t / chunks;
    const int64_t c = t - i * chunks;
    const int64_t j = idx[i];
    const int64_t so = (kScatter ? i : j) * src_stride + c * 16;
    const int64_t dof = (kScatter ? j : i) * dst_stride + c * 16;
    *reinterpret_cast<uint4*>(dst + dof) = *reinterpret_cast<const uint4*>(src + so);
  }
}

}  // namespace

hipError_t launch_unpad_index(const uint8_t* valid, int64_t batch, int64_t seqlen,
                              int64_t row_stride, int32_t* cu, int32_t* idx, hipStream_t s) {
  if (batch > 0) {
    hipLaunchKernelGGL(k_row_counts, dim3((unsigned)batch), dim3(kThreads), 0, s, valid, seqlen,
                       row_stride, cu);
  }
  hipLaunchKernelGGL(k_scan_counts, dim3(1), dim3(kThreads), 0, s, cu, batch);
  if (batch > 0) {
    hipLaunchKernelGGL(k_row_compact, dim3((unsigned)batch), dim3(kThreads), 0, s, valid,
                       seqlen, row_stride, cu, idx);
  }
  return hipGetLastError();
}

hipError_t launch_copy_rows(const void* src, int64_t src_stride, void* dst, int64_t dst_stride,
                            int64_t row_bytes, const int32_t* idx, int64_t n, bool scatter,
                            hipStream_t s) {
  const int64_t chunks = row_bytes / 16;
  const int64_t total = n * chunks;
  if (total == 0) return hipSuccess;
  int64_t grid = (total + kThreads - 1) / kThreads;
  if (grid > 65536) grid = 65536;
  const char* sp = static_cast<const char*>(src);
  char* dp = static_cast<char*>(dst);
  if (scatter)
    hipLaunchKernelGGL(k_copy_rows<true>, dim3((unsigned)grid), dim3(kThreads), 0, s, sp,
                       src_stride, dp, dst_stride, chunks, idx, n);
  else
    hipLaunchKernelGGL(k_copy_rows<false>, dim3((unsigned)grid), dim3(kThreads), 0, s, sp,
                       src_stride, dp, dst_stride, chunks, idx, n);
  return hipGetLastError();
}

}  // namespace bsm
