// Column slicing of the backward's reverse sweep (bwd.hip), shared with the workspace layout (api.hip).
#pragma once
#include "sdm_internal.h"

namespace sdm {

// The fast sweep (W, R <= 128 terms: one lane group per term) takes 8-column slices when 16-column ones give fewer
// than 512 workgroups: each workgroup's reverse sweep is one chain of per-token memory round trips, so two chains
// per CU (256 CUs) hide half of each other's latency. Otherwise, and in the general sweep, 16 columns.
inline bool bwd_fast(const Dims& D) { return D.W <= 128 && D.R <= 128; }
inline int bwd_cols(const Dims& D) {
  if (!bwd_fast(D)) return 16;
  const long long s16 = (long long)D.S * ((D.d + 15) / 16);
  return s16 < 512 ? 8 : 16;
}
inline int bwd_nsl(const Dims& D) {
  const int c = bwd_cols(D);
  return (D.d + c - 1) / c;
}

}  // namespace sdm
