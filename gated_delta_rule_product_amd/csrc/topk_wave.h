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

// Radix select of the `need`-th smallest value (1-based) of one 32-bit field among keys flagged `in`, most
// significant bit first. The class of keys sharing the prefix decided so far shrinks with every bit; as soon as the
// whole class is needed (class size == remaining need) the selection is decided: it is every flagged key whose
// field, shifted right by *shift, is <= res >> *shift, and the loop stops (about log2 of the key count bits for
// distinct values instead of 32). If the loop runs to bit 0 the class is the keys whose field equals res and
// *need is the number of them still to take.
template <int N, bool HIGH>
__device__ __forceinline__ uint32_t radix_select32(const uint64_t (&key)[N], const bool (&in)[N], int* need,
                                                   int* shift, int* csize) {
  uint32_t res = 0;
  int nd = *need, cs = *csize, sh = 0;
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
      cs -= cnt;
    } else {
      cs = cnt;
    }
    sh = bit;
    if (cs == nd) break;
  }
  *need = nd;
  *shift = sh;
  *csize = cs;
  return res;
}

// Selects the k smallest of the wave's keys (key[j] of every lane; unused slots hold ~0ull, k <= number of used
// slots), writes them ascending to out[0..k). scratch: >= k + 8 entries of this wave's LDS, not overlapping out.
// Wave-uniform k.
template <int N>
__device__ void wave_select_sorted(const uint64_t (&key)[N], int k, uint64_t* scratch, uint64_t* out) {
  bool all[N];
#pragma unroll
  for (int j = 0; j < N; ++j) all[j] = true;
  int need = k, shift = 0, csize = 64 * N;
  const uint32_t hi = radix_select32<N, true>(key, all, &need, &shift, &csize);
  bool sel[N];
  if (csize == need) {  // decided on the high halves
#pragma unroll
    for (int j = 0; j < N; ++j) sel[j] = ((uint32_t)(key[j] >> 32) >> shift) <= (hi >> shift);
  } else {              // equal high halves straddle the cut: select among them on the low halves
    bool tie[N];
#pragma unroll
    for (int j = 0; j < N; ++j) tie[j] = (uint32_t)(key[j] >> 32) == hi;
    int need2 = need, shift2 = 0, csize2 = csize;
    const uint32_t lo = radix_select32<N, false>(key, tie, &need2, &shift2, &csize2);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const uint32_t h = (uint32_t)(key[j] >> 32);
      sel[j] = h < hi || (h == hi && ((uint32_t)key[j] >> shift2) <= (lo >> shift2));
    }
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
  // pad to a multiple of 8 with the largest key (never below a selected one)
  const int kpad = (k + 7) & ~7;
  for (int i = k + lane_id(); i < kpad; i += 64) scratch[i] = ~0ull;
  wave_sync();
  // rank placement: each selected key's rank is the number of selected keys below it (8 reads in flight)
  for (int i = lane_id(); i < k; i += 64) {
    const uint64_t v = scratch[i];
    int r = 0;
    for (int m = 0; m < kpad; m += 8) {
      uint64_t x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = scratch[m + u];
#pragma unroll
      for (int u = 0; u < 8; ++u) r += x[u] < v;
    }
    out[r] = v;
  }
  wave_sync();
}

}  // namespace sdm
