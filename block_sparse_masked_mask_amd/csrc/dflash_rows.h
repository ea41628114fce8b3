// Kept keys of one DFlash query row as two half-open key intervals.
//
// Rules (SpecForge issue #452, Problem; SpecForge PR #905, Motivation and
// maintainer reply #934): query q is token i = q % bs of draft block
// j = q / bs. It sees context keys below E_j = clamp((j+1)*S + e0, 0, C) and the
// draft tokens of its own block (i' <= i when in-block attention is causal).
// A sliding layer adds a window with a left bound only: with token positions
// pos(context c) = c and pos(draft (j, i)) = E_j + i, a key is kept only if
// pos_q - pos_k < W, i.e. context keys c >= E_j + i - W + 1 and draft tokens
// i' >= i - W + 1. Every kept key of the row is therefore in
//   [lo1, hi1)  (context)   or   [lo2, hi2)  (own draft block),
// two disjoint intervals below Sk = C + NB*bs.
#pragma once

#include "bsm_internal.h"

namespace bsm {

struct RowIv {
  int64_t lo1, hi1, lo2, hi2;
};

__host__ __device__ inline RowIv dflash_row(const DFlashRule& r, int64_t q) {
  const int64_t j = q / r.bs;
  const int64_t i = q - j * r.bs;
  int64_t E = (j + 1) * r.S + r.e0;
  E = E < 0 ? 0 : (E > r.C ? r.C : E);
  RowIv iv;
  int64_t lo_c = 0, lo_d = 0;
  if (r.W > 0) {
    lo_c = E + i - r.W + 1;
    lo_c = lo_c < 0 ? 0 : lo_c;
    lo_d = i - r.W + 1;
    lo_d = lo_d < 0 ? 0 : lo_d;
  }
  iv.lo1 = lo_c;
  iv.hi1 = E > lo_c ? E : lo_c;  // empty when the window passes E_j
  const int64_t base = r.C + j * r.bs;
  iv.lo2 = base + lo_d;
  iv.hi2 = base + (r.causal ? i + 1 : r.bs);
  return iv;
}

// Number of keys of [lo, hi) inside [k0, k0 + n).
__host__ __device__ inline int64_t iv_overlap(int64_t lo, int64_t hi, int64_t k0,
                                              int64_t n) {
  const int64_t a = lo > k0 ? lo : k0;
  const int64_t b = hi < k0 + n ? hi : k0 + n;
  return b > a ? b - a : 0;
}

}  // namespace bsm
