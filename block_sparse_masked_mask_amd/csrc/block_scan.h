// Workgroup-wide exclusive prefix sum in thread order (wave scan by shuffles,
// then one LDS word per wave).
#pragma once

#include <hip/hip_runtime.h>

namespace bsm {

// Every thread of the NW-wave workgroup must call it; s_wave holds NW ints of
// LDS. Returns the sum of v over the threads before this one; tot receives the
// workgroup total.
template <int NW>
__device__ inline int block_excl_sum(int v, int* s_wave, int& tot) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wave[w] = x;
  __syncthreads();
  int off = 0;
  tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int t = s_wave[i];
    off += i < w ? t : 0;
    tot += t;
  }
  __syncthreads();
  return off + x - v;
}

}  // namespace bsm
