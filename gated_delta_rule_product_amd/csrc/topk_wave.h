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

// 16 bytes of a sub-key row and element e of it as fp64 (exact widening).
template <typename A> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static double at(const uint4& x, int e) {
    const uint32_t w = e == 0 ? x.x : e == 1 ? x.y : e == 2 ? x.z : x.w;
    return (double)__uint_as_float(w);
  }
};
template <> struct Vec16<bf16_t> {
  static constexpr int N = 8;
  __device__ static double at(const uint4& x, int e) {
    const uint32_t w = (e >> 1) == 0 ? x.x : (e >> 1) == 1 ? x.y : (e >> 1) == 2 ? x.z : x.w;
    return (double)__uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
};

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

// Selects the k smallest of the wave's keys (key[j] of every lane; unused slots hold ~0ull, which no used key
// equals; k <= number of used slots), writes them ascending to out[0..k). scratch: >= k + 8 entries of this wave's
// LDS, not overlapping out. Wave-uniform k.
template <int N>
__device__ void wave_select_sorted(const uint64_t (&key)[N], int k, uint64_t* scratch, uint64_t* out) {
  bool all[N];
  int nused = 0;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    all[j] = true;
    nused += __popcll(__ballot(key[j] != ~0ull));
  }
  int need = k, shift = 0, csize = 64 * N;
  bool sel[N];
  if (nused == k) {  // every used key is selected (e.g. k_p = n_f): only the order is left to find
#pragma unroll
    for (int j = 0; j < N; ++j) sel[j] = key[j] != ~0ull;
  } else {
    const uint32_t hi = radix_select32<N, true>(key, all, &need, &shift, &csize);
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

// Exact top-k of one query (the method and its exactness: topk_device.h), in two parts that may run on different
// waves. wave_factor_topk: factor f's scores (the fp64 FMA chain in coordinate order, rounded to float32) for every
// sub-key (NPL per lane, lane l owns l + 64 j) and its top k_p by wave selection, into fsc/fid[f * kpmax + p].
// wave_merge_topk: the candidate tuples of `cand` (CPL per lane) with float32 slot scores summed left to right,
// selected by (score, position sum, candidate index); writes ids[r] (slot ids, best first) and wts[r] (softmax of
// the k slot scores: fp64 exponentials, per-lane partial sums in a fixed order and a fixed butterfly) to LDS.
// scratch and sorted: the calling wave's selection buffers.
template <typename A, int NPL>
__device__ void wave_factor_topk(const Dims& D, const TopkPlan& P, int f, const A* qv, const A* tab, float* fsc,
                                 uint16_t* fid, uint64_t* scratch, uint64_t* sorted) {
  constexpr int VEC = Vec16<A>::N;
  const int lane = lane_id();
  const int dk = D.dk, n = D.widths[f], kpmax = P.kpmax;
  double acc[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) acc[j] = 0.0;
  for (int c0 = 0; c0 < dk; c0 += VEC) {
    uint4 rv[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int i = lane + 64 * j;
      rv[j] = i < n ? *(const uint4*)(tab + (long long)i * dk + c0) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const double x = to_d<A>(qv[f * dk + c0 + e]);
#pragma unroll
      for (int j = 0; j < NPL; ++j) acc[j] = fma(x, Vec16<A>::at(rv[j], e), acc[j]);
    }
  }
  uint64_t key[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int i = lane + 64 * j;
    key[j] = i < n ? (((uint64_t)desc_key((float)acc[j]) << 32) | (uint32_t)i) : ~0ull;
  }
  wave_select_sorted<NPL>(key, P.kp[f], scratch, sorted);
  for (int p = lane; p < P.kp[f]; p += 64) {
    const uint64_t kk = sorted[p];
    fsc[f * kpmax + p] = desc_key_value((uint32_t)(kk >> 32));
    fid[f * kpmax + p] = (uint16_t)(uint32_t)kk;
  }
  wave_sync();
}

template <int CPL>
__device__ void wave_merge_topk(const Dims& D, const TopkPlan& P, const uint64_t* cand, const float* fsc,
                                const uint16_t* fid, uint64_t* scratch, uint64_t* sorted, int32_t* ids, float* wts) {
  const int lane = lane_id();
  const int F = D.F, k = P.k, kpmax = P.kpmax;
  uint64_t ck[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = lane + 64 * j;
    uint64_t key = ~0ull;
    if (c < P.ncand) {
      const uint64_t tup = cand[c];
      int p = (int)(tup & 0xFFFF);
      float S = fsc[p];
      int ps = p;
      for (int f = 1; f < F; ++f) {
        p = (int)((tup >> (16 * f)) & 0xFFFF);
        S = S + fsc[f * kpmax + p];  // float32 sum, left to right
        ps += p;
      }
      key = ((uint64_t)desc_key(S) << 32) | ((uint64_t)ps << 20) | (uint64_t)c;
    }
    ck[j] = key;
  }
  wave_select_sorted<CPL>(ck, k, scratch, sorted);
  const double m = (double)desc_key_value((uint32_t)(sorted[0] >> 32));
  double zpart = 0.0;
  for (int r = lane; r < k; r += 64) {
    const uint64_t kk = sorted[r];
    const uint64_t tup = cand[(int)(kk & 0xFFFFF)];
    long long id = 0;
    for (int f = 0; f < F; ++f) id = id * D.widths[f] + fid[f * kpmax + (int)((tup >> (16 * f)) & 0xFFFF)];
    ids[r] = (int32_t)id;
    zpart += exp((double)desc_key_value((uint32_t)(kk >> 32)) - m);
  }
  double z = zpart;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) z += __shfl_xor(z, o);
  for (int r = lane; r < k; r += 64) wts[r] = (float)(exp((double)desc_key_value((uint32_t)(sorted[r] >> 32)) - m) / z);
  wave_sync();
}

}  // namespace sdm
