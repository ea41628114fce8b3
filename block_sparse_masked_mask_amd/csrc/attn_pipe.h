// Building blocks shared by the pipelined bf16 attention kernels (gfx950):
// vector types, the K/V tile layout in LDS with its 16-byte-chunk swizzles, the
// LDS-DMA tile loader, a fence-free workgroup barrier, and small helpers of the
// online softmax.
#pragma once

#include "attn_common.h"
#include "bsm_internal.h"

namespace bsm {
namespace pipe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kXcds = 8;

__device__ inline int perm_row(int n) { return (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1); }
// 16-byte chunk swizzles of the K and V tiles (row r). For D = 128 both are
// conflict-free whether the LDS serves 8 lanes x 16 bytes (32 banks) or
// 16 lanes x 16 bytes (64 banks) of a ds_read_b128 per cycle, and the same for
// the 16 / 32 lanes of a transposed 8-byte read; D = 64 rows hold only 8 chunks.
template <int D>
__device__ inline int swz_k(int r) {
  return D == 128 ? perm_row(r & 15) : ((r & 3) | ((r >> 1) & 4));
}
template <int D>
__device__ inline int swz_v(int r) {
  return D == 128 ? (((r & 3) << 2) | (r & 2)) : ((r & 3) << 1);
}
__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// vmcnt <= n, other counters unconstrained (gfx9 encoding)
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N < 64, "vmcnt field is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// One 16-byte LDS-DMA load per lane: the global bytes at buffer offset
// voff + soff go to LDS at lds + 16 * lane (lds must be wave-uniform; the
// compiler puts it in m0). Offsets past the resource's range load zeros.
// Completion is awaited explicitly with wait_vmcnt before the barrier that
// publishes a buffer. The compiler also waits for all outstanding LDS-DMA
// loads (vmcnt(0)) before each transposing LDS read, since it cannot tell the
// buffers apart; in these kernels the next tile's load has landed by then.
__device__ inline void dma16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff,
                             uint32_t soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, (int)voff, (int)soff, 0, 0);
}

template <int D>
struct Tiles {
  __bf16 k[kTile * D];
  __bf16 v[kTile * D];
};

// NT threads per workgroup (RB = 512 / NT, the name of the 32-row query blocks
// per wave in the two-head kernel).
template <int D, int RB>
struct V2Ctx {
  static constexpr int NT = 512 / RB;                      // threads per workgroup
  static constexpr int NW = NT / 64;                       // waves
  static constexpr int CPR = D / 8;                        // 16-byte chunks per row
  static constexpr int LOADS = kTile * D * 2 / (NT * 16);  // per tensor per thread
  static constexpr int NS = D / 16;
  static constexpr int NDC = D / 32;
};

// Byte offsets (within one (b, kv head)) of this thread's LDS-DMA chunks of
// key tile 0; tile kt adds kt * 128 rows. Rows >= Sk fall outside the buffer
// resource's range and load as zeros.
template <int D, int RB>
struct Loader {
  using C = V2Ctx<D, RB>;
  uint32_t koff[C::LOADS];
  uint32_t voff[C::LOADS];
  uint32_t ktile_bytes, vtile_bytes;  // bytes per 128 rows
  __amdgpu_buffer_rsrc_t kr, vr;

  __device__ inline void init(const void* kbase, const void* vbase, int64_t k_sk, int64_t v_sk,
                              int Sk, int w, int lane) {
    constexpr int CPR = C::CPR;
    kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(kbase), 0,
                                           (int)((int64_t)Sk * k_sk * 2), 0x00020000);
    vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(vbase), 0,
                                           (int)((int64_t)Sk * v_sk * 2), 0x00020000);
    ktile_bytes = (uint32_t)(kTile * k_sk * 2);
    vtile_bytes = (uint32_t)(kTile * v_sk * 2);
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) {
      const int f = (j * C::NW + w) * 64 + lane;
      const int r = f / CPR;
      const int c = f % CPR;
      koff[j] = (uint32_t)(r * k_sk * 2 + ((c ^ swz_k<D>(r)) * 16));
      voff[j] = (uint32_t)(r * v_sk * 2 + ((c ^ swz_v<D>(r)) * 16));
    }
  }

  // K and V tile kt into the LDS bytes at lk0 and lv0 (workgroup-uniform
  // addresses; w uniform too, so every destination address is scalar)
  __device__ inline void issue_at(char* lk0, char* lv0, int kt, int w) const {
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) {
      const int slot = (j * C::NW + w) * 64 * 16;
      dma16(kr, lk0 + slot, koff[j] + (uint32_t)kt * ktile_bytes);
      dma16(vr, lv0 + slot, voff[j] + (uint32_t)kt * vtile_bytes);
    }
  }
  __device__ inline void issue(Tiles<D>& t, int kt, int w) const { issue(t.k, t.v, kt, w); }
  // the same into separate K and V tiles of LDS (kTile * D elements each)
  __device__ inline void issue(__bf16* tk, __bf16* tv, int kt, int w) const {
    const int wu = __builtin_amdgcn_readfirstlane(w);
    issue_at(reinterpret_cast<char*>(tk), reinterpret_cast<char*>(tv), kt, wu);
  }
};

// Per-lane byte offsets of the LDS operand reads of the bf16 MFMA kernels,
// computed once: the K operand of d-step s in key chunk 0 (chunk c adds 32
// rows), and the first transposed V read of d-chunk dc at key 0 (the key step
// adds rows). K rows are permuted by perm_row so that a lane's S^T values are
// 8 consecutive keys per 16-key step, the B-operand layout of the PV product.
// The swizzles depend only on a row's low bits, which the added rows leave
// alone. vbase: byte offset of the V tiles from the K tiles, folded in so that
// per-read immediates stay small.
template <int D>
struct LaneOffs {
  uint32_t k[D / 16];
  uint32_t v[D / 32];
  __device__ inline void init(int lane, uint32_t vbase) {
    const int n = lane & 31;
    const int hh = lane >> 5;
    const int row = perm_row(n);
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      k[s] = (uint32_t)((row * D + (((2 * s + hh) ^ swz_k<D>(row)) * 8)) * 2);
    // transposed reads: in each 16-lane group, lane 4e + g reads 4 d-values of
    // key row e (and e + 4 for the second read)
    const int blk = lane >> 4;
    const int e4 = (lane >> 2) & 3;
    const int g4 = lane & 3;
    const int row0 = 8 * (blk >> 1) + e4;
#pragma unroll
    for (int dc = 0; dc < D / 32; ++dc) {
      const int chunk = 4 * dc + 2 * (blk & 1) + (g4 >> 1);
      v[dc] = vbase + (uint32_t)((row0 * D + ((chunk ^ swz_v<D>(row0)) * 8) + (g4 & 1) * 4) * 2);
    }
  }
};

// Scheduling hint for an unrolled MFMA loop of N steps, each issuing M MFMAs
// and R LDS reads for the step A ahead (A steps' reads issued up front): keeps
// the reads A steps ahead of their MFMAs. Left alone, the scheduler moves each
// read next to its MFMA and the wave waits out the LDS latency there.
template <int N, int A, int R, int M, int SYNC = 0>
__device__ inline void pin_reads_ahead() {
  __builtin_amdgcn_sched_group_barrier(0x100, A * R, SYNC);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, M, SYNC);
    if (i + A < N) __builtin_amdgcn_sched_group_barrier(0x100, R, SYNC);
  }
}

// Workgroup barrier without a memory fence: LDS-DMA completion is awaited
// explicitly with wait_vmcnt, and a fence would wait for the prefetch as well.
__device__ inline void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Row intervals in 32 bits (keys < 2^31 here).
struct RowIv32 {
  int lo1, hi1, lo2, hi2;
};

// Keep bits of keys kb .. kb+7 that lie in [lo, hi).
__device__ inline uint32_t range_bits(int lo, int hi, int kb) {
  int a = lo - kb, c = hi - kb;
  a = a < 0 ? 0 : (a > 8 ? 8 : a);
  c = c < 0 ? 0 : (c > 8 ? 8 : c);
  return ((1u << c) - 1u) & ~((1u << a) - 1u);
}

// Keep bits of 8 mask bytes (nonzero = keep), byte e -> bit e.
__device__ inline uint32_t byte_bits8(uint2 mb) {
  uint32_t bits = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t byte = ((e < 4 ? mb.x : mb.y) >> (8 * (e & 3))) & 0xFFu;
    bits |= (byte != 0u ? 1u : 0u) << e;
  }
  return bits;
}

// 8 consecutive bf16 bias values (16-byte aligned) in log2 units, saturated
// like every attention kernel reads a bias (bias_log2).
__device__ inline void bias8_log2(const uint16_t* p, float (&out)[8]) {
  const uint4 raw = *reinterpret_cast<const uint4*>(p);
  const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = bias_log2(bf16_to_f32((uint16_t)(wv[e >> 1] >> (16 * (e & 1)))));
}

// max of x over lanes l and l ^ 32 (the two lanes that share a query row)
__device__ inline float max_pair(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// A row's running max is raised only when a new score exceeds it by more than
// this many powers of two; until then probabilities are taken against the
// stale max and stay below 2^kRescaleLog2 (exact after the final division, which
// uses the same max for the sum and for O).
constexpr float kRescaleLog2 = 8.0f;

}  // namespace pipe
}  // namespace bsm
