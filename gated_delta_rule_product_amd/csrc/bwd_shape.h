// Column slicing of the backward's reverse sweep (bwd.hip), shared with the workspace layout (api.hip).
#pragma once
#include "sdm_internal.h"

namespace sdm {

// The fast sweep (W, R <= 128 terms: one lane group per term) takes 16-column slices (64-byte float32 row pieces)
// when a workgroup of them can run two tokens at once (W, R <= 64), or when they give at least 512 workgroups.
// Otherwise 8-column slices: each workgroup's reverse sweep is one chain of memory round trips, and two chains per
// CU (256 CUs) hide part of each other's latency. (65,536 slots, W = R = 64, 4 streams: 16 columns with two tokens
// a step 10.8 ms, 8 columns 12.2 ms; one token a step, 8 columns 12.8 ms.) The general sweep: 16 columns.
inline bool bwd_fast(const Dims& D) { return D.W <= 128 && D.R <= 128; }
inline int bwd_cols(const Dims& D) {
  if (!bwd_fast(D)) return 16;
  const long long s16 = (long long)D.S * ((D.d + 15) / 16);
  return (D.W <= 64 && D.R <= 64) || s16 >= 512 ? 16 : 8;
}
inline int bwd_nsl(const Dims& D) {
  const int c = bwd_cols(D);
  return (D.d + c - 1) / c;
}
// The fast sweep's BWD_FAST_GROUPS term groups are LPG = cols / 4 lanes each, 64 / LPG to a wave. A token needs a
// block of wb whole waves with a group per term (wb = ceil(max(W, R) LPG / 64)); the workgroup holds as many such
// blocks as fit and runs that many consecutive tokens at once when they address disjoint slots.
constexpr int BWD_FAST_GROUPS = 128;
inline int bwd_wave_block(const Dims& D) {
  const int lpg = bwd_cols(D) / 4, m = D.W > D.R ? D.W : D.R;
  return (m * lpg + 63) / 64;
}
inline int bwd_group_tokens(const Dims& D) {
  if (!bwd_fast(D) || (long long)D.T >= (1LL << 27)) return 1;  // entries hold the token index in 27 bits
  return BWD_FAST_GROUPS * (bwd_cols(D) / 4) / 64 / bwd_wave_block(D);
}

}  // namespace sdm
