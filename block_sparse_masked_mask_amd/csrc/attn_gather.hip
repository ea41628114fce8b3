// Masked attention forward, bf16, key-gather mode for short query blocks: at
// most 32 query rows per (b, h) -- under the seqlen_q == 1 head-group swap the
// G heads of a KV group (flash-sparse-attention PR #190, Design: swapped path)
// -- whose mask is given as a kept-key list (key_list.hip): the keys any row
// keeps, with a word of row bits per key. With a dynamic top-k mask (PR #197,
// Design) the list is a small part of the keys, and only those K / V rows
// cross HBM.
//
// The work is split along the list as in attn_group.hip: 4 waves share each
// "tile" of 128 consecutive list positions (LDS-DMA double buffered), wave w
// takes positions 32w .. 32w+31 for all the rows with its own online-softmax
// state, and the four partial states are merged through LDS at the end. Each
// DMA chunk is fetched from the K / V row of its position's key (positions past
// the list's end, or keys outside [0, Sk), fall outside the buffer resource and
// load as zeros), the mask bit of a (row, position) pair is bit `row` of the
// position's row word, and the bias is gathered per key. The key indices a
// tile's DMA needs are loaded two tiles ahead, so no load waits on another
// inside the loop.
#include <math.h>

#include "attn_common.h"
#include "attn_pipe.h"
#include "bsm_internal.h"

namespace bsm {
namespace {

using namespace pipe;

constexpr int kDecWaves = 4;
constexpr int kDecRB = 512 / (64 * kDecWaves);  // V2Ctx layout for 256 threads

// LDS-DMA loader of gathered rows: load j of this thread moves 16-byte chunk
// c_j of tile row r_j (the Loader layout); its source row is the key at list
// position 128 t + r_j.
template <int D>
struct GatherLoader {
  using C = V2Ctx<D, kDecRB>;
  uint32_t kc[C::LOADS], vc[C::LOADS];  // swizzled chunk byte offset in the row
  int row[C::LOADS];
  uint32_t krow, vrow;                  // bytes per K / V row
  uint32_t nkeys;
  __amdgpu_buffer_rsrc_t kr, vr;

  __device__ inline void init(const void* kbase, const void* vbase, int64_t k_sk, int64_t v_sk,
                              int Sk, int w, int lane) {
    constexpr int CPR = C::CPR;
    kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(kbase), 0,
                                           (int)((int64_t)Sk * k_sk * 2), 0x00020000);
    vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(vbase), 0,
                                           (int)((int64_t)Sk * v_sk * 2), 0x00020000);
    krow = (uint32_t)(k_sk * 2);
    vrow = (uint32_t)(v_sk * 2);
    nkeys = (uint32_t)Sk;
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) {
      const int f = (j * C::NW + w) * 64 + lane;
      const int r = f / CPR;
      const int c = f % CPR;
      row[j] = r;
      kc[j] = (uint32_t)((c ^ swz_k<D>(r)) * 16);
      vc[j] = (uint32_t)((c ^ swz_v<D>(r)) * 16);
    }
  }

  // keys of this thread's rows of tile t (-1 past the list's end)
  __device__ inline void keys(const int32_t* lidx, int t, int nlist, int (&key)[C::LOADS]) const {
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) {
      const int pos = t * kTile + row[j];
      key[j] = pos < nlist ? lidx[pos] : -1;
    }
  }

  // Offsets at or past 2^31 exceed the resource's range (Sk rows, < 2^31
  // bytes), so such chunks load as zeros.
  __device__ inline void issue(Tiles<D>& t, const int (&key)[C::LOADS], int w) const {
    w = __builtin_amdgcn_readfirstlane(w);  // keeps the LDS destinations scalar
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) {
      const int slot = (j * C::NW + w) * 64;
      const bool in = (uint32_t)key[j] < nkeys;
      const uint32_t ok = in ? (uint32_t)key[j] * krow + kc[j] : 0x80000000u;
      const uint32_t ov = in ? (uint32_t)key[j] * vrow + vc[j] : 0x80000000u;
      dma16(kr, reinterpret_cast<char*>(t.k + slot * 8), ok);
      dma16(vr, reinterpret_cast<char*>(t.v + slot * 8), ov);
    }
  }
};

// Gathered-key aux of one lane for one tile: list positions
// 128 t + 32 w + 16 sb + 8 hh + e (e < 8) -- their keys, row words and the
// lane's bias values at those keys.
struct GatherKeys {
  int4 key[2][2];
};
struct GatherAux {
  uint4 bits[2][2];
  uint16_t bias[16];
  int4 key[2][2];
};

__device__ inline void load_gather_keys(const int32_t* lidx, int t, int w, int hh,
                                        GatherKeys& g) {
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int pos = t * kTile + 32 * w + 16 * sb + 8 * hh;
    g.key[sb][0] = *reinterpret_cast<const int4*>(lidx + pos);
    g.key[sb][1] = *reinterpret_cast<const int4*>(lidx + pos + 4);
  }
}

__device__ inline int key_at(const int4 (&k)[2][2], int u) {
  const int4 v = k[u >> 3][(u >> 2) & 1];
  const int e = u & 3;
  return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
}

__device__ inline void load_gather_aux(const uint32_t* lbits, const uint16_t* brow, int Sk,
                                       int t, int w, int hh, const GatherKeys& g,
                                       GatherAux& a) {
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int pos = t * kTile + 32 * w + 16 * sb + 8 * hh;
    a.bits[sb][0] = *reinterpret_cast<const uint4*>(lbits + pos);
    a.bits[sb][1] = *reinterpret_cast<const uint4*>(lbits + pos + 4);
    a.key[sb][0] = g.key[sb][0];
    a.key[sb][1] = g.key[sb][1];
  }
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int key = key_at(g.key, u);
    a.bias[u] = (brow && (uint32_t)key < (uint32_t)Sk) ? brow[key] : (uint16_t)0;
  }
}

template <int D>
__global__ __launch_bounds__(64 * kDecWaves, 1) void k_attn_gather(AttnParams p) {
  constexpr int NS = D / 16;
  constexpr int NDC = D / 32;
  __shared__ __align__(1024) Tiles<D> buf0;
  __shared__ __align__(1024) Tiles<D> buf1;

  // Workgroup i runs on XCD i % 8; each XCD takes a contiguous range of (b, h).
  int id;
  {
    const int nwg = gridDim.x;
    const int x = blockIdx.x % kXcds;
    const int qx = nwg / kXcds, rx = nwg % kXcds;
    id = (x < rx ? x * (qx + 1) : rx * (qx + 1) + (x - rx) * qx) + blockIdx.x / kXcds;
  }
  const int h = id % p.H;
  const int b = id / p.H;
  const int kvh = h / p.G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int q = n;
  const bool qvalid = q < p.Sq;

  bf16x8 qf[NS];
  {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.q_sb +
                         (int64_t)q * p.q_sq + (int64_t)h * p.q_sh;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      qf[s] = qvalid ? *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * hh) : bf16x8{};
  }
  const uint16_t* brow = (p.has_bias && qvalid)
      ? reinterpret_cast<const uint16_t*>(aux_row(p.bias, 2, b, h, p.G, q)) : nullptr;
  const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k) + (int64_t)b * p.k_sb +
                        (int64_t)kvh * p.k_sh;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(p.v) + (int64_t)b * p.v_sb +
                        (int64_t)kvh * p.v_sh;
  GatherLoader<D> gl;
  gl.init(kbase, vbase, p.k_sk, p.v_sk, p.Sk, w, lane);

  f32x16 oacc[NDC];
#pragma unroll
  for (int i = 0; i < NDC; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  // transposed-read lane roles
  const int blk = lane >> 4;
  const int e4 = (lane >> 2) & 3;
  const int g4 = lane & 3;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  const KeyListView& kl = p.keys;
  const int64_t li = (kl.Bm == 1 ? 0 : (int64_t)b) * kl.Hm + head_index(kl.h_mode, h, p.G);
  int nlist = kl.num[li];
  nlist = __builtin_amdgcn_readfirstlane(nlist < 0 ? 0 : (nlist > kl.K ? (int)kl.K : nlist));
  const int32_t* lidx = kl.idx + li * kl.K;
  const uint32_t* lbits = kl.bits + li * kl.K;
  const int ntiles = (nlist + kTile - 1) / kTile;
  GatherAux ga_cur, ga_nxt;
  int dkey[V2Ctx<D, kDecRB>::LOADS];  // DMA keys of the next tile to issue
  GatherKeys gk;                      // lane keys of the next tile's aux loads
  if (ntiles > 0) {
    gl.keys(lidx, 0, nlist, dkey);
    gl.issue(buf0, dkey, w);
    load_gather_keys(lidx, 0, w, hh, gk);
    load_gather_aux(lbits, brow, p.Sk, 0, w, hh, gk, ga_cur);
    if (ntiles > 1) {
      gl.keys(lidx, 1, nlist, dkey);
      load_gather_keys(lidx, 1, w, hh, gk);
    }
  }
  for (int it = 0; it < ntiles; ++it) {
    const Tiles<D>& t = (it & 1) ? buf1 : buf0;
    Tiles<D>& nxt = (it & 1) ? buf0 : buf1;
    wait_vmcnt<0>();
    barrier();
    if (it + 1 < ntiles) {
      gl.issue(nxt, dkey, w);
      load_gather_aux(lbits, brow, p.Sk, it + 1, w, hh, gk, ga_nxt);
      if (it + 2 < ntiles) {
        gl.keys(lidx, it + 2, nlist, dkey);
        load_gather_keys(lidx, it + 2, w, hh, gk);
      }
    }

    // S^T for this wave's 32 list positions
    const int row = w * 32 + perm_row(n);
    f32x16 sc{};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(t.k + row * D +
                                                        (((2 * s + hh) ^ swz_k<D>(row)) * 8));
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sc, 0, 0, 0);
    }
    // scale, bias, mask
    float mloc = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int pb = it * kTile + 32 * w + 16 * sb + 8 * hh;
      uint32_t mbits = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint4 wq = ga_cur.bits[sb][e >> 2];
        const uint32_t word =
            (e & 3) == 0 ? wq.x : ((e & 3) == 1 ? wq.y : ((e & 3) == 2 ? wq.z : wq.w));
        const int key = key_at(ga_cur.key, 8 * sb + e);
        const bool keep = ((word >> q) & 1u) && (uint32_t)key < (uint32_t)p.Sk;
        mbits |= (keep ? 1u : 0u) << e;
      }
      mbits &= range_bits(0, nlist, pb);
      if (!qvalid) mbits = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int u = 8 * sb + e;
        const float bv = bias_log2(bf16_to_f32(ga_cur.bias[u]));
        float sv = fmaf(sc[u], p.scale_log2, bv);
        sv = ((mbits >> e) & 1u) ? sv : -INFINITY;
        sc[u] = sv;
        mloc = fmaxf(mloc, sv);
      }
    }
    mloc = max_pair(mloc);
    const bool grow = mloc > m_run + kRescaleLog2;
    const float m_new = grow ? mloc : m_run;
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
    if (__ballot(grow)) {
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) oacc[dc] *= alpha;
    }
    m_run = m_new;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    float lsum = l_run * alpha;
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
    l_run = lsum;
    // O^T += V^T P^T over this wave's 32 keys
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int kb = w * 32 + 16 * sb;
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
        oacc[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[sb], oacc[dc], 0, 0, 0);
      }
    }
    ga_cur = ga_nxt;
  }

  // merge the four waves' partial states through LDS (tiles are free now)
  barrier();
  float* sO = reinterpret_cast<float*>(&buf0);           // [wave][row][D]
  float* sM = reinterpret_cast<float*>(&buf1);           // [wave][row]
  float* sL = sM + kDecWaves * 32;                       // [wave][row]
  const float l_pair = l_run + __shfl_xor(l_run, 32, 64);
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<float4*>(&sO[(w * 32 + n) * D + dc * 32 + 8 * g + 4 * hh]) =
          make_float4(oacc[dc][4 * g], oacc[dc][4 * g + 1], oacc[dc][4 * g + 2],
                      oacc[dc][4 * g + 3]);
  if (hh == 0) {
    sM[w * 32 + n] = m_run;
    sL[w * 32 + n] = l_pair;
  }
  __syncthreads();
  float mstar = -INFINITY;
#pragma unroll
  for (int i = 0; i < kDecWaves; ++i) mstar = fmaxf(mstar, sM[i * 32 + n]);
  float f[kDecWaves];
  float lstar = 0.f;
#pragma unroll
  for (int i = 0; i < kDecWaves; ++i) {
    const float mi = sM[i * 32 + n];
    f[i] = mi == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mi - mstar);
    lstar += f[i] * sL[i * 32 + n];
  }
  if (qvalid) {
    const float inv = lstar > 0.f ? 1.f / lstar : 0.f;
    __bf16* orow = reinterpret_cast<__bf16*>(p.o) + (int64_t)b * p.o_sb + (int64_t)q * p.o_sq +
                   (int64_t)h * p.o_sh;
    for (int dc = w; dc < NDC; dc += kDecWaves) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = dc * 32 + 8 * g + 4 * hh;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < kDecWaves; ++i) {
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
  const dim3 blk(64 * kDecWaves);
  if (D == 128)
    hipLaunchKernelGGL(k_attn_gather<128>, dim3(nwg), blk, 0, s, p);
  else
    hipLaunchKernelGGL(k_attn_gather<64>, dim3(nwg), blk, 0, s, p);
  return hipGetLastError();
}

}  // namespace bsm
