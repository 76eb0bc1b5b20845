// topk.h -- one token's top-k and gates in one thread (internal to libmoe;
// the fused top-k + permute kernel uses it, topk_rank_kernel computes the
// same values with a lane per expert).
//
// "271,104 Routes", section 2: topk on the logits, then softmax over the k
// selected logits (the renormalised gate); "MoE Inference Visualized",
// "Expert Execution": without renormalisation the gate is the full softmax
// probability.  Ties go to the lower expert index.
#pragma once

#include "common.h"

namespace moe {

// (a, ia) precedes (b, ib) in the selection order: larger logit first, lower
// expert index first among equal logits.
__device__ __forceinline__ bool precedes(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

// Top-k of one token: row(e) is logit e of the token (e < E).  A single
// insertion pass keeps the k best in slot order (KMAX: the smallest power of
// two >= k); then gates: exp(l - max) over the selected (renorm) or over all
// E logits, summed in increasing index.  EMAX > 0 unrolls the passes over e
// for E <= EMAX (row then indexes registers with constants); EMAX = 0 loops.
template <int KMAX, int EMAX, typename Row>
__device__ __forceinline__ void topk_token(Row row, int E, int k, int renorm, int (&bi)[KMAX],
                                           float (&gate)[KMAX]) {
  float bv[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    bv[j] = 0.0f;
    bi[j] = 0;
  }
  int filled = 0;
  auto insert = [&](int e) {
    float cv = row(e);
    int ci = e;
    // branch-free insertion: the displaced entry moves one slot down
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const bool take = (j < k) & ((j >= filled) | precedes(cv, ci, bv[j], bi[j]));
      const float ov = bv[j];
      const int oi = bi[j];
      bv[j] = take ? cv : ov;
      bi[j] = take ? ci : oi;
      cv = take ? ov : cv;
      ci = take ? oi : ci;
    }
    filled = filled < k ? filled + 1 : k;
  };
  if constexpr (EMAX > 0) {
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      if (e < E) insert(e);
  } else {
    for (int e = 0; e < E; ++e) insert(e);
  }
  const float m = bv[0];
  float ex[KMAX];
  float denom = 0.0f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    ex[j] = j < k ? expf(bv[j] - m) : 0.0f;
    if (renorm) denom += ex[j];
  }
  if (!renorm) {
    if constexpr (EMAX > 0) {
#pragma unroll
      for (int e = 0; e < EMAX; ++e)
        if (e < E) denom += expf(row(e) - m);
    } else {
      for (int e = 0; e < E; ++e) denom += expf(row(e) - m);
    }
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) gate[j] = ex[j] / denom;
}

}  // namespace moe
