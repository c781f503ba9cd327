// Wavefront-level exact selection for the product-key top-k: every 64-lane wave selects, from keys held in its
// registers, the k smallest 64-bit keys (ascending key = best first) and writes them sorted to LDS.
//
// Selection is a most-significant-bit-first radix select on the key, counted with wave ballots (integer counts,
// order independent, so the result is exact and repeatable): the high 32 bits first, then, only if equal high
// parts straddle the cut, the low 32 bits among them. The selected keys are compacted with ballot prefix counts and
// placed at their rank (number of selected keys smaller than them; keys are unique).
#pragma once
#include "sdm_internal.h"

namespace sdm {

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ uint64_t lanes_below_mask() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Radix select of the `need`-th smallest value (1-based) of one 32-bit field among keys flagged `in`.
// On return *need holds the rank of the selected value among the flagged keys equal to it.
template <int N, bool HIGH>
__device__ __forceinline__ uint32_t radix_select32(const uint64_t (&key)[N], const bool (&in)[N], int* need) {
  uint32_t res = 0;
  int nd = *need;
  for (int bit = 31; bit >= 0; --bit) {
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const uint32_t v = HIGH ? (uint32_t)(key[j] >> 32) : (uint32_t)key[j];
      const bool p = in[j] && ((v >> bit) == (res >> bit));
      cnt += __popcll(__ballot(p));
    }
    if (cnt < nd) {
      res |= 1u << bit;
      nd -= cnt;
    }
  }
  *need = nd;
  return res;
}

// Selects the k smallest of the wave's keys (key[j] of every lane; unused slots hold ~0ull, k <= number of used
// slots), writes them ascending to out[0..k). scratch: >= k entries of this wave's LDS. Wave-uniform k.
template <int N>
__device__ void wave_select_sorted(const uint64_t (&key)[N], int k, uint64_t* scratch, uint64_t* out) {
  bool all[N];
#pragma unroll
  for (int j = 0; j < N; ++j) all[j] = true;
  int need = k;
  const uint32_t hi = radix_select32<N, true>(key, all, &need);
  // keys with high part == hi: how many?
  int eq = 0;
#pragma unroll
  for (int j = 0; j < N; ++j) eq += __popcll(__ballot((uint32_t)(key[j] >> 32) == hi));
  bool sel[N];
  if (eq > need) {
    bool tie[N];
#pragma unroll
    for (int j = 0; j < N; ++j) tie[j] = (uint32_t)(key[j] >> 32) == hi;
    int need2 = need;
    const uint32_t lo = radix_select32<N, false>(key, tie, &need2);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const uint32_t h = (uint32_t)(key[j] >> 32);
      sel[j] = h < hi || (h == hi && (uint32_t)key[j] <= lo);
    }
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) sel[j] = (uint32_t)(key[j] >> 32) <= hi;
  }
  // compaction
  const uint64_t below = lanes_below_mask();
  int base = 0;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const uint64_t m = __ballot(sel[j]);
    if (sel[j]) scratch[base + __popcll(m & below)] = key[j];
    base += __popcll(m);
  }
  wave_sync();
  // rank placement
  for (int i = lane_id(); i < k; i += 64) {
    const uint64_t v = scratch[i];
    int r = 0;
    for (int m = 0; m < k; ++m) r += scratch[m] < v;
    out[r] = v;
  }
  wave_sync();
}

}  // namespace sdm
