// Masked attention forward, bf16, key-gather mode for short query blocks: at
// most 32 query rows per (b, h) -- under the seqlen_q == 1 head-group swap the
// G heads of a KV group (flash-sparse-attention PR #190, Design: swapped path)
// -- whose mask is given as a kept-key list (key_list.hip): the keys any row
// keeps, with a word of row bits per key. With a dynamic top-k mask (PR #197,
// Design) the list is a small part of the keys, and only those K / V rows
// cross HBM.
//
// The gathered rows are scattered, so what bounds the kernel is how many of
// them are in flight, not the bytes. Each of the 8 waves of a workgroup
// therefore streams the list on its own, with no barrier until the end: wave w
// takes chunks w, w + 8, w + 16, ... of 32 consecutive list positions, and
// while it computes one chunk the next one loads --
//  * its K rows straight into registers (the MFMA A operand of a lane is 8
//    d-values of one key, a 16-byte load),
//  * its V rows into the wave's own LDS slot by LDS-DMA (the PV product needs
//    them transposed, which ds_read_b64_tr_b16 does from row-major rows),
//  * the row-bits words and the lane's bias values,
// all by buffer loads whose range check turns listed keys outside [0, Sk)
// into zero rows (they are masked out as well). The keys themselves are
// loaded a chunk earlier still, one per lane, and handed between lanes with
// ds_bpermute. Each wave keeps its own online-softmax state; the 8 partial
// states are merged through LDS at the end.
#include <math.h>

#include "attn_common.h"
#include "attn_pipe.h"
#include "bsm_internal.h"

namespace bsm {
namespace {

using namespace pipe;

constexpr int kGaWaves = 8;
constexpr int kChunk = 32;  // list positions per chunk

// One chunk's per-lane inputs but its K rows, loaded while the chunk before is
// computed.
struct GaChunk {
  uint32_t word;       // row-bits word of position lane & 31
  uint32_t kvalid;     // bit u: position u of the lane (below) is listed, key in [0, Sk)
  uint32_t bias[16];   // bf16 bias of the lane's row at its position u (low half)
  int kkey;            // key of position perm_row(n): the lane's K row
};

// The lane's 16 positions in a chunk: u = 8 sb + e -> 16 sb + 8 hh + e, the
// keys of its S^T values (the K rows are read in perm_row order).
__device__ inline int ga_pos(int u, int hh) { return 16 * (u >> 3) + 8 * hh + (u & 7); }

// value v of lane (base + off) / 4, base a lane-dependent byte address, off a
// constant (it goes in the instruction's offset field instead of a register
// per use); lanes 0-31 and 32-63 hold the same 32 keys / words
__device__ inline int ga_from(int v, int base, int off) {
  return __builtin_amdgcn_ds_bpermute(base + off, v);
}

template <int D>
struct GaCtx {
  static constexpr int NS = D / 16;
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;         // rows per DMA instruction
  static constexpr int NDMA = kChunk / RPI;    // DMA instructions per chunk
  __amdgpu_buffer_rsrc_t kr, vr;               // K, V rows of (b, kvh)
  __amdgpu_buffer_rsrc_t br;                   // bias rows of (b, h) from query row 0
  uint32_t boff;                               // the lane's bias row: byte offset in br
  bool has_bias;
  uint32_t krow, vrow;                         // bytes per K / V row
  uint32_t nkeys;                              // Sk
  int n, hh, lane, wu;
  bool qvalid;
};

// Issue the loads of chunk ch (keyv: its keys, lane l holding position l & 31)
// into set c and the LDS slot vfill, but its K rows (ga_load_k).
template <int D>
__device__ __attribute__((always_inline)) inline void ga_load(const GaCtx<D>& x, int keyv,
                                                              const uint32_t* lbits, int ch,
                                                              int nlist, char* vfill,
                                                              GaChunk& c) {
  constexpr int NS = D / 16;
  constexpr int CPR = GaCtx<D>::CPR;
  constexpr int RPI = GaCtx<D>::RPI;
  constexpr int NDMA = GaCtx<D>::NDMA;
  const int pos0 = ch * kChunk;
  // V rows by LDS-DMA: instruction j fills rows RPI j .. RPI j + RPI - 1 of the
  // slot, 16-byte chunk c of row r from the swizzled source chunk
#pragma unroll
  for (int j = 0; j < NDMA; ++j) {
    const int r = RPI * j + x.lane / CPR;
    const int cc = x.lane % CPR;
    const int key = ga_from(keyv, (x.lane / CPR) * 4, RPI * j * 4);
    const uint32_t off = (uint32_t)key < x.nkeys
        ? (uint32_t)key * x.vrow + (uint32_t)((cc ^ swz_v<D>(r)) * 16) : 0x80000000u;
    dma16(x.vr, vfill + j * 1024, off);
  }
  c.kkey = ga_from(keyv, perm_row(x.n) * 4, 0);
  // row-bits word of position lane & 31
  {
    const int pos = pos0 + (x.lane & 31);
    c.word = pos < nlist ? lbits[pos] : 0u;
  }
  // listed positions with keys in range, and the lane's bias values
  uint32_t kv = 0;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int pu = ga_pos(u, x.hh);
    const int key = ga_from(keyv, 32 * x.hh, ga_pos(u, 0) * 4);
    const bool ok = pos0 + pu < nlist && (uint32_t)key < x.nkeys;
    kv |= (ok ? 1u : 0u) << u;
    // out-of-range offsets read as zeros (rows past Sq, unlisted keys)
    const uint32_t off = ok && x.qvalid ? x.boff + (uint32_t)key * 2 : 0x80000000u;
    c.bias[u] = x.has_bias ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(x.br, off, 0, 0) : 0u;
  }
  c.kvalid = kv;
}

// The 32 query rows in LDS, shared by the waves: byte offset of 16-byte chunk
// c of row n, chunks XOR-swizzled by row so that the 32 rows one read touches
// fall in distinct banks.
template <int D>
__device__ inline int ga_qoff(int n, int c) {
  return (n * (D / 8) + (c ^ (n & (D / 8 - 1)))) * 16;
}

// The lane's K row of a chunk (key kkey) into k.
template <int D>
__device__ inline void ga_load_k(const GaCtx<D>& x, int kkey, bf16x8 (&k)[D / 16]) {
  const uint32_t base = (uint32_t)kkey < x.nkeys ? (uint32_t)kkey * x.krow : 0x80000000u;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const uint32_t off = base == 0x80000000u ? base : base + (uint32_t)((16 * s + 8 * x.hh) * 2);
    k[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(x.kr, off, 0, 0));
  }
}

// Per-wave online-softmax state of the 32 rows.
template <int D>
struct GaState {
  f32x16 oacc[D / 32];
  float m_run, l_run;
};

// Chunk c (V rows in the LDS slot vuse) into the wave's state.
// The K registers then receive the next chunk's K rows (when there is one).
template <int D>
__device__ __attribute__((always_inline)) inline void ga_compute(const GaCtx<D>& x,
                                                                 const AttnParams& p,
                                                                 const char* qs,
                                                                 const GaChunk& c,
                                                                 const char* vuse,
                                                                 bf16x8 (&k)[D / 16],
                                                                 bool next, int kkey_next,
                                                                 GaState<D>& st) {
  constexpr int NS = D / 16;
  constexpr int NDC = D / 32;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  f32x16 sc{};
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const bf16x8 qv = *reinterpret_cast<const bf16x8*>(qs + ga_qoff<D>(x.n, 2 * s + x.hh));
    sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[s], qv, sc, 0, 0, 0);
  }
  if (next) ga_load_k<D>(x, kkey_next, k);
  // keep bits of the lane's 16 positions: listed, key in range, row bit set
  uint32_t mbits = 0;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const uint32_t word = (uint32_t)ga_from((int)c.word, 32 * x.hh, ga_pos(u, 0) * 4);
    mbits |= ((word >> x.n) & 1u) << u;
  }
  mbits &= c.kvalid;
  if (!x.qvalid) mbits = 0;
  float mloc = -INFINITY;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const float bv = bias_log2(__uint_as_float(c.bias[u] << 16));
    float sv = fmaf(sc[u], p.scale_log2, bv);
    sv = ((mbits >> u) & 1u) ? sv : -INFINITY;
    sc[u] = sv;
    mloc = fmaxf(mloc, sv);
  }
  mloc = max_pair(mloc);
  const bool grow = mloc > st.m_run + kRescaleLog2;
  if (__ballot(grow)) {
    const float m_new = grow ? mloc : st.m_run;
    const float alpha = grow ? __builtin_amdgcn_exp2f(st.m_run - m_new) : 1.f;
    st.l_run *= alpha;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) st.oacc[dc] *= alpha;
    st.m_run = m_new;
  }
  const float m_use = st.m_run == -INFINITY ? 0.f : st.m_run;
  float lsum = st.l_run;
  bf16x8 pf[2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float x0 = __builtin_amdgcn_exp2f(sc[8 * sb + e] - m_use);
      const float x1 = __builtin_amdgcn_exp2f(sc[8 * sb + e + 1] - m_use);
      const bf16x2 pr = {(__bf16)x0, (__bf16)x1};
      pf[sb][e] = pr[0];
      pf[sb][e + 1] = pr[1];
      lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsum, false);
    }
  }
  st.l_run = lsum;
  // O^T += V^T P^T over the chunk's 32 positions
  const int blk = x.lane >> 4;
  const int e4 = (x.lane >> 2) & 3;
  const int g4 = x.lane & 3;
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int chunk = 4 * dc + 2 * (blk & 1) + (g4 >> 1);
      const int row0 = 16 * sb + 8 * (blk >> 1) + e4;
      const int row1 = row0 + 4;
      const char* a0 = vuse + (row0 * D + ((chunk ^ swz_v<D>(row0)) * 8) + (g4 & 1) * 4) * 2;
      const char* a1 = vuse + (row1 * D + ((chunk ^ swz_v<D>(row1)) * 8) + (g4 & 1) * 4) * 2;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a1));
      const bf16x8 a = __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo),
                                               __builtin_bit_cast(bf16x4, hi), 0, 1, 2, 3, 4,
                                               5, 6, 7);
      st.oacc[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[sb], st.oacc[dc], 0, 0, 0);
    }
  }
}

// One step of a wave's stream: chunk t (inputs in pend, V rows in slot vuse)
// is computed while chunk t + 1 loads into pend and slot vfill (when it
// exists) and the keys of chunk t + 3 load (key1, key2: the keys of chunks
// t + 1 and t + 2). As restrict parameters, vfill and vuse tell the
// compiler that the LDS reads do not touch the slot in flight.
template <int D>
__device__ __attribute__((always_inline)) inline void ga_step(
    char* __restrict__ vfill, const char* __restrict__ vuse, const GaCtx<D>& x,
    const char* __restrict__ qs, const AttnParams& p, const int32_t* lidx, const uint32_t* lbits,
    int nlist, int t, int nmine, int& key1, int& key2, GaChunk& pend, bf16x8 (&k)[D / 16],
    GaState<D>& st) {
  wait_vmcnt<0>();
  // chunk t's inputs, copied only now that their loads have landed (a copy
  // the scheduler could move up would wait for every load in flight)
  const GaChunk cur = pend;
  GaChunk& nxt = pend;
  const int w = x.wu;
  if (t + 1 < nmine) ga_load<D>(x, key1, lbits, w + kGaWaves * (t + 1), nlist, vfill, nxt);
  key1 = key2;
  key2 = -1;
  if (t + 3 < nmine) {
    const int pos = (w + kGaWaves * (t + 3)) * kChunk + (x.lane & 31);
    key2 = pos < nlist ? lidx[pos] : -1;
  }
  ga_compute<D>(x, p, qs, cur, vuse, k, t + 1 < nmine, nxt.kkey, st);
}

template <int D>
__global__ __launch_bounds__(64 * kGaWaves, 1) void k_attn_gather(AttnParams p) {
  constexpr int NS = D / 16;
  constexpr int NDC = D / 32;
  constexpr int CB = kChunk * D * 2;  // bytes of one V slot
  // one LDS array: the V slots, the Q rows, the merge's max / sum (separate
  // arrays would get per-array alias tags from the compiler that replace the
  // ones telling the LDS reads from the loads in flight)
  constexpr int QB = 32 * D * 2;
  __shared__ __align__(1024) char s_lds[kGaWaves * 2 * CB + QB + 2 * kGaWaves * 32 * 4];
  char* const s_v = s_lds;
  char* const s_q = s_lds + kGaWaves * 2 * CB;
  float (*s_ml)[kGaWaves][32] = reinterpret_cast<float (*)[kGaWaves][32]>(s_q + QB);

  // Workgroup i runs on XCD i % 8; each XCD takes a contiguous range of (b, h).
  int id;
  {
    const int nwg = gridDim.x;
    const int xi = blockIdx.x % kXcds;
    const int qx = nwg / kXcds, rx = nwg % kXcds;
    id = (xi < rx ? xi * (qx + 1) : rx * (qx + 1) + (xi - rx) * qx) + blockIdx.x / kXcds;
  }
  const int h = id % p.H;
  const int b = id / p.H;
  const int kvh = h / p.G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;

  GaCtx<D> x;
  x.lane = lane;
  x.n = lane & 31;
  x.hh = lane >> 5;
  x.wu = __builtin_amdgcn_readfirstlane(w);
  const int q = x.n;
  x.qvalid = q < p.Sq;

  {
    // Q rows into LDS: thread i writes 16-byte chunk i % (D / 8) of row i / (D / 8)
    constexpr int CPR = D / 8;
    for (int i = tid; i < 32 * CPR; i += 64 * kGaWaves) {
      const int r = i / CPR, c = i % CPR;
      bf16x8 v{};
      if (r < p.Sq)
        v = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(p.q) +
                                             (int64_t)b * p.q_sb + (int64_t)r * p.q_sq +
                                             (int64_t)h * p.q_sh + 8 * c);
      *reinterpret_cast<bf16x8*>(s_q + ga_qoff<D>(r, c)) = v;
    }
  }
  x.has_bias = p.has_bias != 0;
  x.boff = 0;
  x.br = __builtin_amdgcn_make_buffer_rsrc(nullptr, 0, 0, 0x00020000);
  if (x.has_bias) {
    // query row q's bias row lies q * sq elements past row 0's (the launch
    // checks that every offset fits below 2^31)
    x.br = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(aux_row(p.bias, 2, b, h, p.G, 0)), 0, 0x7FFFFFFF, 0x00020000);
    x.boff = (uint32_t)((int64_t)q * p.bias.sq * 2);
  }
  const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k) + (int64_t)b * p.k_sb +
                        (int64_t)kvh * p.k_sh;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(p.v) + (int64_t)b * p.v_sb +
                        (int64_t)kvh * p.v_sh;
  x.kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(kbase), 0,
                                           (int)((int64_t)p.Sk * p.k_sk * 2), 0x00020000);
  x.vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(vbase), 0,
                                           (int)((int64_t)p.Sk * p.v_sk * 2), 0x00020000);
  x.krow = (uint32_t)(p.k_sk * 2);
  x.vrow = (uint32_t)(p.v_sk * 2);
  x.nkeys = (uint32_t)p.Sk;

  const KeyListView& kl = p.keys;
  const int64_t li = (kl.Bm == 1 ? 0 : (int64_t)b) * kl.Hm + head_index(kl.h_mode, h, p.G);
  int nlist = kl.num[li];
  nlist = __builtin_amdgcn_readfirstlane(nlist < 0 ? 0 : (nlist > kl.K ? (int)kl.K : nlist));
  const int32_t* lidx = kl.idx + li * kl.K;
  const uint32_t* lbits = kl.bits + li * kl.K;
  const int nch = (nlist + kChunk - 1) / kChunk;
  const int wu = x.wu;
  const int nmine = nch > wu ? (nch - wu + kGaWaves - 1) / kGaWaves : 0;

  GaState<D> st;
#pragma unroll
  for (int i = 0; i < NDC; ++i) st.oacc[i] = f32x16{};
  st.m_run = -INFINITY;
  st.l_run = 0.f;

  char* const slot0 = s_v + (wu * 2) * CB;  // the wave's two V slots
  // the Q rows are in LDS (every wave passes this barrier, chunks or not)
  __syncthreads();
  if (nmine > 0) {
    // keys of the first three chunks; the first chunk's loads
    auto key_of = [&](int t) {
      const int pos = (wu + kGaWaves * t) * kChunk + (lane & 31);
      return t < nmine && pos < nlist ? lidx[pos] : -1;
    };
    int key0 = key_of(0);
    int key1 = key_of(1);
    int key2 = key_of(2);
    GaChunk pend;
    bf16x8 kregs[NS];
    wait_vmcnt<0>();
    ga_load<D>(x, key0, lbits, wu, nlist, slot0, pend);
    ga_load_k<D>(x, pend.kkey, kregs);
    // chunk t in slot t & 1
    for (int t = 0; t < nmine; ++t) {
      const int par = t & 1;
      ga_step<D>(slot0 + (par ^ 1) * CB, slot0 + par * CB, x, s_q, p, lidx, lbits, nlist, t,
                 nmine, key1, key2, pend, kregs, st);
    }
  }

  // merge the waves' partial states through LDS (every slot is free after the
  // barrier)
  __syncthreads();
  float* sO = reinterpret_cast<float*>(s_v);  // [wave][row][D]
  const float l_pair = st.l_run + __shfl_xor(st.l_run, 32, 64);
  const int n = x.n, hh = x.hh;
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(&sO[(w * 32 + n) * D + dc * 32 + 8 * g + 4 * hh]) =
          make_float4(st.oacc[dc][4 * g], st.oacc[dc][4 * g + 1], st.oacc[dc][4 * g + 2],
                      st.oacc[dc][4 * g + 3]);
  if (hh == 0) {
    s_ml[0][w][n] = st.m_run;
    s_ml[1][w][n] = l_pair;
  }
  __syncthreads();
  float mstar = -INFINITY;
#pragma unroll
  for (int i = 0; i < kGaWaves; ++i) mstar = fmaxf(mstar, s_ml[0][i][n]);
  float f[kGaWaves];
  float lstar = 0.f;
#pragma unroll
  for (int i = 0; i < kGaWaves; ++i) {
    const float mi = s_ml[0][i][n];
    f[i] = mi == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mi - mstar);
    lstar += f[i] * s_ml[1][i][n];
  }
  if (x.qvalid) {
    const float inv = lstar > 0.f ? 1.f / lstar : 0.f;
    __bf16* orow = reinterpret_cast<__bf16*>(p.o) + (int64_t)b * p.o_sb + (int64_t)q * p.o_sq +
                   (int64_t)h * p.o_sh;
    // wave w writes d-quads w, w + 8, ... of the row (4 d-values per lane half)
    for (int dq = w; dq < D / 8; dq += kGaWaves) {
      const int d0 = 8 * dq + 4 * hh;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int i = 0; i < kGaWaves; ++i) {
        const float4 v = *reinterpret_cast<const float4*>(&sO[(i * 32 + n) * D + d0]);
        acc.x += f[i] * v.x;
        acc.y += f[i] * v.y;
        acc.z += f[i] * v.z;
        acc.w += f[i] * v.w;
      }
      bf16x4 o4 = {(__bf16)(acc.x * inv), (__bf16)(acc.y * inv), (__bf16)(acc.z * inv),
                   (__bf16)(acc.w * inv)};
      *reinterpret_cast<bf16x4*>(orow + d0) = o4;
    }
    if (p.lse && w == 0 && hh == 0) {
      const float lse = lstar > 0.f ? (mstar + __builtin_amdgcn_logf(lstar)) * kLn2 : -INFINITY;
      p.lse[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + (int64_t)q * p.lse_sq] = lse;
    }
  }
}

}  // namespace

hipError_t launch_attn_gather(const AttnParams& p, int D, hipStream_t s) {
  const int nwg = p.B * p.H;
  if (nwg == 0) return hipSuccess;
  const dim3 blk(64 * kGaWaves);
  if (D == 128)
    hipLaunchKernelGGL(k_attn_gather<128>, dim3(nwg), blk, 0, s, p);
  else
    hipLaunchKernelGGL(k_attn_gather<64>, dim3(nwg), blk, 0, s, p);
  return hipGetLastError();
}

}  // namespace bsm
