// Dynamic top-k keep mask for gfx950: one workgroup per bias row, radix select.
//
// What it computes (flash-sparse-attention PR #197, Design / Implementation
// Notes and the review suggestion on dynamic_mask): positions the pre-mask marks
// invalid take the bias dtype's minimum finite value, the k largest entries of
// the row are selected, and out = selected AND valid. Keys >= Sk are invalid
// (PR #190, Implementation Notes). Ties at the cut go to the lower key index;
// -0 and +0 compare equal.
//
// How: every value is mapped to an unsigned key whose integer order is the
// value order (sign bit set -> bitwise NOT, else set the sign bit; -0 folded to
// +0 first). The k-th largest key T is then found and the row written in index
// order: keys > T are selected, and of the keys == T the `need` lowest-indexed
// ones, found with a workgroup prefix count taken in index order.
//  * k_topk_reg (rows up to 16K bf16 / 8K f32 keys): the row stays in
//    registers, 16 contiguous bytes per thread per 4 KiB segment (coalesced
//    loads and stores); T comes from a radix select with 12-bit digits, so
//    the histogram atomics of a concentrated row rarely hit the same bin.
//  * k_topk (longer rows): T is found one 8-bit digit at a time, most
//    significant first, from LDS histograms of the digit among the keys that
//    share the prefix found so far; the keys stay in LDS when they fit,
//    otherwise each pass re-reads the row.
#include "block_scan.h"
#include "bsm_internal.h"

namespace bsm {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kPer = 16;  // keys per thread per chunk
constexpr int kChunk = kThreads * kPer;

template <typename KeyT>
struct KeyTraits;

template <>
struct KeyTraits<uint16_t> {
  static constexpr int kBits = 16;
  // order-preserving key of a bf16 bit pattern
  __device__ static uint16_t key(uint16_t b) {
    if ((b & 0x7FFFu) == 0) b = 0;
    return (b & 0x8000u) ? (uint16_t)~b : (uint16_t)(b | 0x8000u);
  }
  // key of the sentinel finfo(bfloat16).min = -(2 - 2^-7) * 2^127 (bits 0xFF7F)
  __device__ static uint16_t sentinel() { return (uint16_t)~(uint16_t)0xFF7Fu; }
};

template <>
struct KeyTraits<uint32_t> {
  static constexpr int kBits = 32;
  __device__ static uint32_t key(uint32_t b) {
    if ((b & 0x7FFFFFFFu) == 0) b = 0;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  }
  // finfo(float32).min = -(2 - 2^-23) * 2^127 (bits 0xFF7FFFFF)
  __device__ static uint32_t sentinel() { return ~0xFF7FFFFFu; }
};

template <typename KeyT, bool kCache>
__global__ __launch_bounds__(kThreads) void k_topk(TopkParams p) {
  using Tr = KeyTraits<KeyT>;
  extern __shared__ __align__(16) unsigned char s_dyn[];
  __shared__ uint32_t s_hist[256];
  __shared__ int s_wave[kWaves];
  __shared__ uint32_t s_sel[2];  // chosen digit, count of keys above it

  KeyT* s_keys = reinterpret_cast<KeyT*>(s_dyn);
  const int64_t row = blockIdx.x;
  const int64_t qb = row % p.Qb;
  const int64_t hb = (row / p.Qb) % p.Hb;
  const int64_t bb = row / (p.Qb * p.Hb);
  const KeyT* brow = reinterpret_cast<const KeyT*>(p.bias) + bb * p.b_sb + hb * p.b_sh + qb * p.b_sq;
  const uint8_t* prow = p.pm ? p.pm + bb * p.p_sb + hb * p.p_sh + qb * p.p_sq : nullptr;
  uint8_t* orow = p.out + row * p.K;
  const int64_t K = p.K;
  const KeyT sent = Tr::sentinel();

  auto valid = [&](int64_t k) -> bool {
    return k < p.Sk && (prow == nullptr || (k < p.pK && prow[k] != 0));
  };
  // keys of 16 consecutive positions starting at k0 (k0 % 16 == 0, k0 < K)
  auto load16 = [&](int64_t k0, KeyT* out) {
    if (kCache) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) out[i] = s_keys[k0 + i];
    } else {
      constexpr int kVecs = kPer * sizeof(KeyT) / 16;
      const uint4* src = reinterpret_cast<const uint4*>(brow + k0);
#pragma unroll
      for (int v = 0; v < kVecs; ++v) {
        const uint4 x = src[v];
        const KeyT* e = reinterpret_cast<const KeyT*>(&x);
#pragma unroll
        for (int i = 0; i < 16 / (int)sizeof(KeyT); ++i) {
          const int64_t kk = k0 + v * (16 / sizeof(KeyT)) + i;
          out[v * (16 / sizeof(KeyT)) + i] = valid(kk) ? Tr::key(e[i]) : sent;
        }
      }
    }
  };

  const int64_t keff = p.k < K ? p.k : K;
  if (keff == 0 || keff == K) {
    // nothing or everything selected: out = valid (or nothing)
    for (int64_t k0 = (int64_t)threadIdx.x * kPer; k0 < K; k0 += kChunk) {
      uint32_t w[4] = {0, 0, 0, 0};
      if (keff == K) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) w[i / 4] |= (uint32_t)valid(k0 + i) << (8 * (i % 4));
      }
      *reinterpret_cast<uint4*>(orow + k0) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    return;
  }

  if (kCache) {
    constexpr int kVecs = kPer * sizeof(KeyT) / 16;
    for (int64_t k0 = (int64_t)threadIdx.x * kPer; k0 < K; k0 += kChunk) {
      const uint4* src = reinterpret_cast<const uint4*>(brow + k0);
#pragma unroll
      for (int v = 0; v < kVecs; ++v) {
        const uint4 x = src[v];
        const KeyT* e = reinterpret_cast<const KeyT*>(&x);
        KeyT kk[16 / sizeof(KeyT)];
#pragma unroll
        for (int i = 0; i < 16 / (int)sizeof(KeyT); ++i) {
          const int64_t pos = k0 + v * (16 / sizeof(KeyT)) + i;
          kk[i] = valid(pos) ? Tr::key(e[i]) : sent;
        }
        *reinterpret_cast<uint4*>(s_keys + k0 + v * (16 / sizeof(KeyT))) =
            *reinterpret_cast<const uint4*>(kk);
      }
    }
  }

  // ---- radix select of the keff-th largest key ----
  uint32_t prefix = 0;      // digits found so far, in place
  uint32_t rem = (uint32_t)keff;
  for (int shift = Tr::kBits - 8; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += kThreads) s_hist[i] = 0;
    __syncthreads();  // also orders the LDS key fill before the first pass
    const int hs = shift + 8;  // bits above this digit must equal the prefix
    for (int64_t k0 = (int64_t)threadIdx.x * kPer; k0 < K; k0 += kChunk) {
      KeyT kk[kPer];
      load16(k0, kk);
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const uint32_t key = (uint32_t)kk[i];
        const bool match = hs >= Tr::kBits || ((key ^ prefix) >> hs) == 0;
        if (match) atomicAdd(&s_hist[(key >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l covers digits 255-4l .. 252-4l (descending)
      const int lane = threadIdx.x;
      uint32_t c[4];
      uint32_t sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = s_hist[255 - 4 * lane - j];
        sum += c[j];
      }
      uint32_t incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      const uint32_t excl = incl - sum;
      if (excl < rem && rem <= incl) {
        uint32_t above = excl;
        int d = 255 - 4 * lane;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (above + c[j] >= rem) {
            d = 255 - 4 * lane - j;
            break;
          }
          above += c[j];
        }
        s_sel[0] = (uint32_t)d;
        s_sel[1] = above;
      }
    }
    __syncthreads();
    prefix |= s_sel[0] << shift;
    rem -= s_sel[1];
    __syncthreads();  // s_sel / s_hist reuse
  }
  const uint32_t T = prefix;
  const int need = (int)rem;  // keys equal to T to take, lowest index first

  // ---- write pass, index order ----
  int taken = 0;
  for (int64_t base = 0; base < K; base += kChunk) {
    const int64_t k0 = base + (int64_t)threadIdx.x * kPer;
    KeyT kk[kPer];
    int neq = 0;
    if (k0 < K) {
      load16(k0, kk);
#pragma unroll
      for (int i = 0; i < kPer; ++i) neq += (uint32_t)kk[i] == T;
    }
    int tot;
    int r = taken + block_excl_sum<kWaves>(neq, s_wave, tot);
    if (k0 < K) {
      uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const uint32_t key = (uint32_t)kk[i];
        bool sel = key > T;
        if (key == T) {
          sel = r < need;
          ++r;
        }
        w[i / 4] |= (uint32_t)(sel && valid(k0 + i)) << (8 * (i % 4));
      }
      *reinterpret_cast<uint4*>(orow + k0) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    taken += tot;
  }
}

constexpr size_t kCacheMax = 64 * 1024;

// Register-resident selection for rows of up to NSEG * 256 * (16 / sizeof(KeyT))
// keys: each thread keeps its keys in registers throughout; the threshold
// comes from a wide-digit radix select (below). Segment s of a row is the 4 KiB
// block [s * SEG, (s + 1) * SEG); thread t owns the 16 contiguous bytes at
// t * EPL of every segment, so each load and each store of a segment is one
// coalesced wave-wide access. The index-order prefix count of keys equal to the
// threshold is one workgroup scan of NSEG counters per thread (segment-major,
// then thread order). t is the thread's index in its group of 256 threads
// (sm belongs to the group); on return bit i of sel[s] says whether key
// s * SEG + t * EPL + i is kept (selected and valid). Every thread of the
// workgroup must call it: its barriers are workgroup-wide, so groups that
// share a workgroup run it together, each on its own row and LDS.
template <int NSEG>
struct SelectSmem {
  uint32_t hist[4096];
  uint32_t scan[kWaves];
  uint32_t sel[2];
  int wsum[NSEG][kWaves];
};

template <typename KeyT, int NSEG, bool HAS_PM>
__device__ inline void select_row(const TopkParams& p, const KeyT* brow, const uint8_t* prow,
                                  int t, SelectSmem<NSEG>& sm, uint32_t (&sel)[NSEG]) {
  using Tr = KeyTraits<KeyT>;
  constexpr int EPL = 16 / sizeof(KeyT);  // keys per 16-byte load
  constexpr int SEG = kThreads * EPL;
  uint32_t* s_hist = sm.hist;
  uint32_t* s_scan = sm.scan;
  uint32_t* s_sel = sm.sel;
  auto& s_wsum = sm.wsum;

  const int K = (int)p.K;
  const int lane = t & 63;
  const int w = t >> 6;
  const KeyT sent = Tr::sentinel();
  auto valid = [&](int k) -> bool {
    return k < p.Sk && (!HAS_PM || (k < p.pK && prow[k] != 0));
  };

  uint4 raw[NSEG];
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    const int k0 = s * SEG + t * EPL;
    raw[s] = k0 < K ? *reinterpret_cast<const uint4*>(brow + k0) : make_uint4(0, 0, 0, 0);
  }
  KeyT kk[NSEG][EPL];
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    const KeyT* e = reinterpret_cast<const KeyT*>(&raw[s]);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      kk[s][i] = valid(s * SEG + t * EPL + i) ? Tr::key(e[i]) : sent;
  }

  // The k-th largest key T, by radix select with wide digits: 12 bits first
  // (4096 LDS bins, so the few exponent values a bias row concentrates in are
  // still spread over many bins and the LDS atomics rarely collide), then the
  // remaining 4 (bf16) or 12 + 8 (f32) bits among the keys that share the
  // prefix found so far. After each histogram the bins are scanned from the
  // top (16 per thread, one workgroup scan) to find the digit at which the
  // running count reaches the remaining k.
  const int keff = p.k < K ? (int)p.k : K;
  uint32_t prefix = 0;
  uint32_t rem = (uint32_t)keff;
  if (keff > 0 && keff < K) {
    int hi_bits = Tr::kBits;  // bits above the current digit are fixed
    while (hi_bits > 0) {
      const int dw = hi_bits >= 12 ? 12 : hi_bits;
      const int sh = hi_bits - dw;
      const int nb = 1 << dw;
      const uint32_t dmask = (uint32_t)nb - 1u;
      for (int i = t; i < nb; i += kThreads) s_hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int s = 0; s < NSEG; ++s) {
        if (s * SEG + t * EPL < K) {
#pragma unroll
          for (int i = 0; i < EPL; ++i) {
            const uint32_t key = (uint32_t)kk[s][i];
            const bool match = hi_bits >= Tr::kBits ||
                               ((key ^ prefix) >> (sh + dw)) == 0;
            if (match) atomicAdd(&s_hist[(key >> sh) & dmask], 1u);
          }
        }
      }
      __syncthreads();
      // thread t sums bins nb-1-16t .. nb-16-16t (descending digit order)
      const int per = nb >= 16 * kThreads ? nb / kThreads : 16;
      const int first = nb - 1 - per * t;
      uint32_t c = 0;
      for (int j = 0; j < per; ++j) {
        const int d = first - j;
        c += d >= 0 ? s_hist[d] : 0u;
      }
      uint32_t incl = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      if (lane == 63) s_scan[w] = incl;
      __syncthreads();
      uint32_t off = 0;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) off += i < w ? s_scan[i] : 0u;
      incl += off;
      const uint32_t excl = incl - c;
      if (c > 0 && excl < rem && rem <= incl) {
        uint32_t above = excl;
        int dsel = first;
        for (int j = 0; j < per; ++j) {
          const int d = first - j;
          const uint32_t cd = s_hist[d];
          if (above + cd >= rem) {
            dsel = d;
            break;
          }
          above += cd;
        }
        s_sel[0] = (uint32_t)dsel;
        s_sel[1] = above;
      }
      __syncthreads();
      prefix |= s_sel[0] << sh;
      rem -= s_sel[1];
      hi_bits = sh;
      __syncthreads();  // s_hist / s_scan / s_sel reuse
    }
  }
  const uint32_t T = prefix;
  const int cnt_gt = keff - (int)rem;  // #{key > T}
  const int need = keff - cnt_gt;  // keys equal to T to take, lowest index first

  // prefix counts of keys == T in index order (segment-major, then thread)
  int excl[NSEG];
  if (keff > 0 && keff < K) {
    int incl[NSEG];
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      int c = 0;
      if (s * SEG + t * EPL < K) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) c += (uint32_t)kk[s][i] == T;
      }
      excl[s] = c;
      int x = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      incl[s] = x;
      if (lane == 63) s_wsum[s][w] = x;
    }
    __syncthreads();
    int base = 0;
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      int off = base;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) {
        const int v = s_wsum[s][i];
        off += i < w ? v : 0;
        base += v;
      }
      excl[s] = off + incl[s] - excl[s];
    }
  }

#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    const int k0 = s * SEG + t * EPL;
    uint32_t bits = 0;  // one bit per key
    if (k0 < K) {
      int r = excl[s];
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const uint32_t key = (uint32_t)kk[s][i];
        const bool eq = key == T;
        bool pick = key > T || (eq && r < need);
        r += eq ? 1 : 0;
        pick = keff >= K ? true : (keff == 0 ? false : pick);
        bits |= (uint32_t)(pick && valid(k0 + i)) << i;
      }
    }
    sel[s] = bits;
  }
}

// Writes the keep bytes of one row from select_row's bits.
template <typename KeyT, int NSEG>
__device__ inline void write_row(uint8_t* orow, int K, int t, const uint32_t (&sel)[NSEG]) {
  constexpr int EPL = 16 / sizeof(KeyT);
  constexpr int SEG = kThreads * EPL;
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    const int k0 = s * SEG + t * EPL;
    if (k0 >= K) continue;
    const uint32_t bits = sel[s];
    if (EPL == 8) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= ((bits >> i) & 1u) << (8 * i);
        hi |= ((bits >> (i + 4)) & 1u) << (8 * i);
      }
      *reinterpret_cast<uint2*>(orow + k0) = make_uint2(lo, hi);
    } else {
      uint32_t v = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) v |= ((bits >> i) & 1u) << (8 * i);
      *reinterpret_cast<uint32_t*>(orow + k0) = v;
    }
  }
}

template <typename KeyT, int NSEG, bool HAS_PM>
__global__ __launch_bounds__(kThreads) void k_topk_reg(TopkParams p) {
  const int64_t row = blockIdx.x;
  const int64_t qb = row % p.Qb;
  const int64_t hb = (row / p.Qb) % p.Hb;
  const int64_t bb = row / (p.Qb * p.Hb);
  const KeyT* brow = reinterpret_cast<const KeyT*>(p.bias) + bb * p.b_sb + hb * p.b_sh + qb * p.b_sq;
  const uint8_t* prow = p.pm ? p.pm + bb * p.p_sb + hb * p.p_sh + qb * p.p_sq : nullptr;
  __shared__ SelectSmem<NSEG> sm;
  uint32_t sel[NSEG];
  select_row<KeyT, NSEG, HAS_PM>(p, brow, prow, (int)threadIdx.x, sm, sel);
  write_row<KeyT, NSEG>(p.out + row * p.K, (int)p.K, (int)threadIdx.x, sel);
}

// Top-k fused with what is built from its mask. One workgroup per (bm, hm) of
// the mask in the attention's iteration space selects its Qm (<= 32) distinct
// mask rows in turn (small workgroups: the selection is latency-bound and
// gains from many resident workgroups), writes them if asked, and keeps per
// owned key a word of the rows that keep it (thread t owns the same keys in
// every row). Then, without reading the mask back:
//  * block mask: the kept pairs of each 128-key tile (popcounts of its words)
//    classify it empty / partial / full over the Qm rows, and the two lists
//    are compacted in ascending order;
//  * key list: the keys with a non-zero word, ascending, with the word (all R
//    rows when the mask broadcasts over queries), by a prefix count per
//    segment.
template <typename KeyT, int NSEG, bool HAS_PM>
__global__ __launch_bounds__(kThreads) void k_topk_fused(TopkFusedParams fp) {
  constexpr int EPL = 16 / sizeof(KeyT);
  constexpr int SEG = kThreads * EPL;
  constexpr int KMAX = NSEG * SEG;
  __shared__ SelectSmem<NSEG> sm;
  __shared__ int s_codes[KMAX / kTile];
  __shared__ int s_wave[2][kWaves];
  const TopkParams& p = fp.t;
  const int64_t lb = blockIdx.x / fp.Hm;
  const int64_t lh = blockIdx.x % fp.Hm;
  const int K = (int)p.K;
  const int t = threadIdx.x;
  // per owned key (thread t owns the same keys in every row): bit r = row r keeps it
  uint32_t rw[NSEG][EPL];
#pragma unroll
  for (int s = 0; s < NSEG; ++s)
#pragma unroll
    for (int i = 0; i < EPL; ++i) rw[s][i] = 0;
  for (int r = 0; r < fp.Qm; ++r) {
    // mask row of (lb, lh, r) in the contiguous (Bb, Hb, Qb, K) mask, and the
    // bias / pre-mask rows it comes from
    const int64_t mrow = (lb * fp.m_sb + lh * fp.m_sh + (int64_t)r * fp.m_sq) / p.K;
    const int64_t qb = mrow % p.Qb;
    const int64_t hb = (mrow / p.Qb) % p.Hb;
    const int64_t bb = mrow / (p.Qb * p.Hb);
    const KeyT* brow =
        reinterpret_cast<const KeyT*>(p.bias) + bb * p.b_sb + hb * p.b_sh + qb * p.b_sq;
    const uint8_t* prow = p.pm ? p.pm + bb * p.p_sb + hb * p.p_sh + qb * p.p_sq : nullptr;
    uint32_t sel[NSEG];
    select_row<KeyT, NSEG, HAS_PM>(p, brow, prow, t, sm, sel);
    if (p.out) write_row<KeyT, NSEG>(p.out + mrow * p.K, K, t, sel);
#pragma unroll
    for (int s = 0; s < NSEG; ++s)
#pragma unroll
      for (int i = 0; i < EPL; ++i) rw[s][i] |= ((sel[s] >> i) & 1u) << r;
  }

  const int64_t li = blockIdx.x;  // list / block-mask row (lb, lh), query tile 0
  if (fp.kv_num) {
    const int nK = (int)fp.nK;
    constexpr int TPT = kTile / EPL;  // threads owning one 128-key tile
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      int c = 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) c += __popc(rw[s][i]);
#pragma unroll
      for (int o = TPT / 2; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
      const int kt = (s * SEG + t * EPL) / kTile;
      if (t % TPT == 0 && kt < nK) s_codes[kt] = c == 0 ? 0 : (c == fp.Qm * kTile ? 2 : 1);
    }
    __syncthreads();
    int np = 0, nf = 0;
    int32_t* prow_o = fp.kv_idx + li * nK;
    int32_t* frow_o = fp.full_idx + li * nK;
    for (int base = 0; base < nK; base += kThreads) {
      const int kk = base + t;
      const int cc = kk < nK ? s_codes[kk] : 0;
      int tp, tf;
      const int op = block_excl_sum<kWaves>(cc == 1, s_wave[0], tp);
      const int of = block_excl_sum<kWaves>(cc == 2, s_wave[1], tf);
      if (cc == 1) prow_o[np + op] = kk;
      if (cc == 2) frow_o[nf + of] = kk;
      np += tp;
      nf += tf;
    }
    for (int kk = np + t; kk < nK; kk += kThreads) prow_o[kk] = -1;
    for (int kk = nf + t; kk < nK; kk += kThreads) frow_o[kk] = -1;
    if (t == 0) {
      fp.kv_num[li] = np;
      fp.full_num[li] = nf;
    }
  }
  if (fp.l_num) {
    // segment-major, then thread order = ascending key order
    const uint32_t all_rows = fp.R >= 32 ? 0xFFFFFFFFu : ((1u << fp.R) - 1u);
    int taken = 0;
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      const int k0 = s * SEG + t * EPL;
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) cnt += rw[s][i] != 0u;
      int tot;
      int pos = taken + block_excl_sum<kWaves>(cnt, s_wave[0], tot);
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const uint32_t wd = fp.Qm == 1 ? all_rows : rw[s][i];
        if (rw[s][i]) {
          fp.l_idx[li * p.K + pos] = k0 + i;
          fp.l_bits[li * p.K + pos] = wd;
          ++pos;
        }
      }
      taken += tot;
    }
    if (t == 0) fp.l_num[li] = taken;
  }
}

template <typename KeyT, bool HAS_PM>
bool launch_fused2(const TopkFusedParams& fp, hipStream_t s) {
  constexpr int SEG = kThreads * (16 / sizeof(KeyT));
  const int nseg = (int)((fp.t.K + SEG - 1) / SEG);
  const dim3 grid((unsigned)(fp.Bm * fp.Hm)), block(kThreads);
  switch (nseg) {
    case 1: hipLaunchKernelGGL((k_topk_fused<KeyT, 1, HAS_PM>), grid, block, 0, s, fp); return true;
    case 2: hipLaunchKernelGGL((k_topk_fused<KeyT, 2, HAS_PM>), grid, block, 0, s, fp); return true;
    case 3:
    case 4: hipLaunchKernelGGL((k_topk_fused<KeyT, 4, HAS_PM>), grid, block, 0, s, fp); return true;
    case 5: case 6: case 7:
    case 8: hipLaunchKernelGGL((k_topk_fused<KeyT, 8, HAS_PM>), grid, block, 0, s, fp); return true;
    default: return false;
  }
}

template <typename KeyT, bool HAS_PM>
bool launch_reg2(const TopkParams& p, unsigned rows, hipStream_t s) {
  constexpr int SEG = kThreads * (16 / sizeof(KeyT));
  const int nseg = (int)((p.K + SEG - 1) / SEG);
  const dim3 grid(rows), block(kThreads);
  switch (nseg) {
    case 1: hipLaunchKernelGGL((k_topk_reg<KeyT, 1, HAS_PM>), grid, block, 0, s, p); return true;
    case 2: hipLaunchKernelGGL((k_topk_reg<KeyT, 2, HAS_PM>), grid, block, 0, s, p); return true;
    case 3:
    case 4: hipLaunchKernelGGL((k_topk_reg<KeyT, 4, HAS_PM>), grid, block, 0, s, p); return true;
    case 5: case 6: case 7:
    case 8: hipLaunchKernelGGL((k_topk_reg<KeyT, 8, HAS_PM>), grid, block, 0, s, p); return true;
    default: return false;
  }
}

template <typename KeyT>
bool launch_reg(const TopkParams& p, unsigned rows, hipStream_t s) {
  return p.pm ? launch_reg2<KeyT, true>(p, rows, s) : launch_reg2<KeyT, false>(p, rows, s);
}

}  // namespace

bool topk_fused_applies(const TopkParams& p) {
  const int64_t maxk = p.is_bf16 ? 8 * kThreads * 8 : 8 * kThreads * 4;
  return p.K <= maxk;
}

hipError_t launch_topk_fused(const TopkFusedParams& fp, hipStream_t s) {
  if (fp.Bm * fp.Hm == 0 || fp.t.K == 0) return hipSuccess;
  bool ok;
  if (fp.t.is_bf16)
    ok = fp.t.pm ? launch_fused2<uint16_t, true>(fp, s) : launch_fused2<uint16_t, false>(fp, s);
  else
    ok = fp.t.pm ? launch_fused2<uint32_t, true>(fp, s) : launch_fused2<uint32_t, false>(fp, s);
  return ok ? hipGetLastError() : hipErrorInvalidValue;
}

hipError_t launch_topk(const TopkParams& p, hipStream_t s) {
  const int64_t rows = p.Bb * p.Hb * p.Qb;
  if (rows == 0 || p.K == 0) return hipSuccess;
  if (p.is_bf16 ? launch_reg<uint16_t>(p, (unsigned)rows, s)
                : launch_reg<uint32_t>(p, (unsigned)rows, s))
    return hipGetLastError();
  const size_t ksz = p.is_bf16 ? 2 : 4;
  const size_t bytes = (size_t)p.K * ksz;
  const bool cache = bytes <= kCacheMax;
  const dim3 grid((unsigned)rows), block(kThreads);
  if (p.is_bf16) {
    if (cache)
      hipLaunchKernelGGL((k_topk<uint16_t, true>), grid, block, bytes, s, p);
    else
      hipLaunchKernelGGL((k_topk<uint16_t, false>), grid, block, 0, s, p);
  } else {
    if (cache)
      hipLaunchKernelGGL((k_topk<uint32_t, true>), grid, block, bytes, s, p);
    else
      hipLaunchKernelGGL((k_topk<uint32_t, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace bsm
