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
// The search may start below bit 31: bits above `top` are then res0's (zero at and below top), every flagged key
// at or below that prefix shares it, and *csize counts the keys with it.
template <int N, bool HIGH>
__device__ __forceinline__ uint32_t radix_select32(const uint64_t (&key)[N], const bool (&in)[N], int* need,
                                                   int* shift, int* csize, int top = 31, uint32_t res0 = 0) {
  uint32_t res = res0;
  int nd = *need, cs = *csize, sh = 0;
  for (int bit = top; bit >= 0; --bit) {
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

extern "C" __device__ __attribute__((const)) unsigned int __ockl_wfred_and_u32(unsigned int);
extern "C" __device__ __attribute__((const)) unsigned int __ockl_wfred_or_u32(unsigned int);

// Where a radix search over the high halves of the wave's keys (key[j] of every lane, unused slots ~0ull) for the
// k smallest may start. When at least k lanes hold a used key, the largest lane minimum bounds the k-th smallest
// high half (each of those lanes holds a key at or below it): keys above it are never selected, so the high bits
// shared by every used key at or below it (wave AND == wave OR) decide nothing and the search starts below them.
// Sets *top (the highest bit left to search; -1: every such key shares the whole high half), *res0 (the shared
// prefix, zero at and below top) and *csize (keys with that prefix); leaves them at 31, 0 and 64 N when bit 31
// already differs. Wave-uniform k.
template <int N>
__device__ __forceinline__ void radix_start(const uint64_t (&key)[N], int k, int* top, uint32_t* res0, int* csize) {
  uint32_t lmin = ~0u;
  bool has = false;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    if (key[j] != ~0ull) {
      lmin = min(lmin, (uint32_t)(key[j] >> 32));
      has = true;
    }
  }
  const uint32_t bound = __popcll(__ballot(has)) >= k ? __ockl_wfred_max_u32(has ? lmin : 0u) : ~0u;
  uint32_t andv = ~0u, orv = 0u;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const uint32_t h = (uint32_t)(key[j] >> 32);
    if (key[j] != ~0ull && h <= bound) { andv &= h; orv |= h; }
  }
  andv = __ockl_wfred_and_u32(andv);
  orv = __ockl_wfred_or_u32(orv);
  const uint32_t diff = andv ^ orv;
  *top = 31;
  *res0 = 0;
  *csize = 64 * N;
  if (diff == 0 || (diff >> 31) == 0) {
    const int t = diff ? 31 - __clz(diff) : -1;  // highest differing bit
    const int s = t + 1;                         // 1..31, or 0
    const uint32_t r0 = andv & ~((1u << s) - 1u);
    int cs = 0;  // keys with that prefix (every key at or below the bound, maybe more)
#pragma unroll
    for (int j = 0; j < N; ++j) cs += __popcll(__ballot(((uint32_t)(key[j] >> 32) >> s) == (r0 >> s)));
    *top = t;
    *res0 = r0;
    *csize = cs;
  }
}

// The k-th smallest high half of the wave's used keys (unused slots ~0ull; 1 <= k <= used count): the radix search
// from radix_start; when it stops early, the largest high half of the decided class is the k-th.
template <int N>
__device__ __forceinline__ uint32_t wave_kth_high(const uint64_t (&key)[N], int k) {
  int top, csize;
  uint32_t res0;
  radix_start<N>(key, k, &top, &res0, &csize);
  bool all[N];
#pragma unroll
  for (int j = 0; j < N; ++j) all[j] = true;
  int need = k, shift = 0;
  const uint32_t hi = radix_select32<N, true>(key, all, &need, &shift, &csize, top, res0);
  uint32_t km = 0;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const uint32_t h = (uint32_t)(key[j] >> 32);
    if (key[j] != ~0ull && (h >> shift) <= (hi >> shift)) km = max(km, h);
  }
  return __ockl_wfred_max_u32(km);
}

// Selects the k smallest of the wave's keys (key[j] of every lane; unused slots hold ~0ull, which no used key
// equals; k <= number of used slots), writes them ascending to out[0..k). RB: selected keys read per batch in the
// rank placement (more reads in flight, a larger pad). scratch: >= k + RB entries of this wave's LDS, not
// overlapping out. Wave-uniform k.
template <int N, int RB = 8>
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
    int top;
    uint32_t res0;
    radix_start<N>(key, k, &top, &res0, &csize);
    const uint32_t hi = radix_select32<N, true>(key, all, &need, &shift, &csize, top, res0);
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
  // pad to a multiple of RB with the largest key (never below a selected one)
  const int kpad = (k + RB - 1) & ~(RB - 1);
  for (int i = k + lane_id(); i < kpad; i += 64) scratch[i] = ~0ull;
  wave_sync();
  // rank placement: each selected key's rank is the number of selected keys below it (RB reads in flight)
  for (int i = lane_id(); i < k; i += 64) {
    const uint64_t v = scratch[i];
    int r = 0;
    for (int m = 0; m < kpad; m += RB) {
      uint64_t x[RB];
#pragma unroll
      for (int u = 0; u < RB; ++u) x[u] = scratch[m + u];
#pragma unroll
      for (int u = 0; u < RB; ++u) r += x[u] < v;
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
// the k slot scores: fp64 exponentials, per-lane partial sums in a fixed order, then a fixed cross-lane order) to LDS.
// scratch and sorted: the calling wave's selection buffers.

// One block of factor f's coordinates, loaded ahead of its use: PB pieces of 16 bytes (VEC coordinates) of each of
// this lane's sub-key rows and the same pieces of the query (every lane holds them). The loads are unconditional
// (row and coordinate clamped into the tables) so that no select waits on them; a piece past dk is loaded from the
// last valid coordinates and skipped where it is used. A caller may issue the first block early and do other work
// while it arrives.
template <typename A, int NPL> struct FactorBlock {
  static constexpr int PB = NPL >= 4 ? 2 : 8 / NPL;
  uint4 rv[PB][NPL];
  uint4 qx[PB];
};

// Requires dk a multiple of VEC (16-byte rows) and 16-byte aligned tab and qv.
template <typename A, int NPL>
__device__ __forceinline__ void factor_load(const Dims& D, int f, const A* qv, const A* tab, int c0,
                                            FactorBlock<A, NPL>& B) {
  constexpr int VEC = Vec16<A>::N;
  const int lane = lane_id(), dk = D.dk, n = D.widths[f];
  // 0 in every lane but not known uniform: the query pieces load as vector loads (counted with the row loads)
  const int zero = (int)__builtin_amdgcn_mbcnt_lo(0u, 0u);
#pragma unroll
  for (int p = 0; p < FactorBlock<A, NPL>::PB; ++p) {
    const int c = min(c0 + p * VEC, dk - VEC);
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int i = min(lane + 64 * j, n - 1);
      B.rv[p][j] = *(const uint4*)(tab + (long long)i * dk + c);
    }
    B.qx[p] = *(const uint4*)(qv + f * dk + c + zero);
  }
}

// B holds factor f's first block (factor_load at c0 = 0).
template <typename A, int NPL>
__device__ void wave_factor_topk(const Dims& D, const TopkPlan& P, int f, const A* qv, const A* tab, float* fsc,
                                 uint16_t* fid, uint64_t* scratch, uint64_t* sorted, FactorBlock<A, NPL>& B) {
  constexpr int VEC = Vec16<A>::N, PB = FactorBlock<A, NPL>::PB;
  const int lane = lane_id();
  const int dk = D.dk, n = D.widths[f], kpmax = P.kpmax;
  double acc[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) acc[j] = 0.0;
  for (int c0 = 0; c0 < dk; c0 += PB * VEC) {
    if (c0 > 0) factor_load<A, NPL>(D, f, qv, tab, c0, B);
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      if (c0 + p * VEC < dk) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const double x = Vec16<A>::at(B.qx[p], e);
#pragma unroll
          for (int j = 0; j < NPL; ++j) acc[j] = fma(x, Vec16<A>::at(B.rv[p][j], e), acc[j]);
        }
      }
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

constexpr int MERGE_RB = 32;  // rank-placement batch of the merge's selection (its scratch: >= k + MERGE_RB)

// A lower bound L on the k-th largest slot score of a two-factor candidate table (fq: the factor scores [2][kpmax],
// best first): a block of position tuples p_f < a_f with a_0 a_1 = k (a_f <= k_p) lies in the table (prod(p_f + 1)
// <= k) and holds k candidates, each scoring at least the block's last corner (float32 addition is monotone);
// candidates below L are not in the top k. The blocks tried: 1 x k, k x 1, and a_0 a power of two dividing k.
// -inf for other factor counts: with more, the corners of such blocks sit far down the factor lists and the bound
// keeps most of the table (three factors, 64 slots: no gain, 5 % slower).
__device__ __forceinline__ float merge_lower_bound(const TopkPlan& P, int F, int k, const float* fq, int kpmax) {
  if (F != 2) return -INFINITY;
  // one block per lane, their corners read at once: lane 0 k x 1, lane 1 1 x k, lane i >= 2 2^(i-1) x k / 2^(i-1)
  const int lane = lane_id();
  int a0 = 0, a1 = 0;
  if (lane == 0) {
    a0 = k;
    a1 = 1;
  } else if (lane == 1) {
    a0 = 1;
    a1 = k;
  } else if (lane < 31) {
    a0 = 1 << (lane - 1);
    a1 = (k & (a0 - 1)) == 0 ? k >> (lane - 1) : 0;
  }
  float S = -INFINITY;
  if (a1 >= 1 && a0 <= P.kp[0] && a1 <= P.kp[1] && a0 <= k) {
    S = fq[a0 - 1] + fq[kpmax + a1 - 1];
    if (!(S == S)) S = -INFINITY;
  }
  return desc_key_value(__ockl_wfred_min_u32(desc_key(S)));  // the largest
}

// The k smallest candidate keys, ascending, into sorted (wave_select_sorted): ck[j] the keys (~0ull unused) and
// keep[j] whether the candidate scores at or above a lower bound on the k-th largest score (all of them when there
// is no bound, bounded = false). When at least k and at most min(256, ccap) are kept, they are compacted into cbuf
// (this wave's, ccap uint64 entries, not overlapping scratch or sorted) and selected from at most four a lane;
// otherwise from all CPL a lane.
template <int CPL, int RB>
__device__ void select_kept_candidates(const uint64_t (&ck)[CPL], const bool (&keep)[CPL], bool bounded, int k,
                                       uint64_t* cbuf, int ccap, uint64_t* scratch, uint64_t* sorted) {
  const int lane = lane_id();
  int m2 = 0;
  if (bounded) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) m2 += __popcll(__ballot(keep[j]));
  }
  if (m2 >= k && m2 <= 256 && m2 <= ccap) {
    const uint64_t below = lanes_below_mask();
    int base = 0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const uint64_t bm = __ballot(keep[j]);
      if (keep[j]) cbuf[base + __popcll(bm & below)] = ck[j];
      base += __popcll(bm);
    }
    wave_sync();
    uint64_t ck4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ck4[j] = lane + 64 * j < m2 ? cbuf[lane + 64 * j] : ~0ull;
    wave_sync();
    if (m2 <= 64) {
      uint64_t ck1[1] = {ck4[0]};
      wave_select_sorted<1, RB>(ck1, k, scratch, sorted);
    } else if (m2 <= 128) {
      uint64_t ck2[2] = {ck4[0], ck4[1]};
      wave_select_sorted<2, RB>(ck2, k, scratch, sorted);
    } else {
      wave_select_sorted<4, RB>(ck4, k, scratch, sorted);
    }
  } else {
    wave_select_sorted<CPL, RB>(ck, k, scratch, sorted);
  }
}

// A double moved between lanes by a DPP control (two 32-bit moves; all lanes active).
template <int CTRL> __device__ __forceinline__ double dpp_d(double x) {
  const uint64_t u = __double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xf, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xf, 0xf, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// Lane l's double, as a wave-uniform value (constant l).
template <int L> __device__ __forceinline__ double readlane_d(double x) {
  const uint64_t u = __double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, L);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), L);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// The sum of the 64 lanes' values in a fixed order, the same on every lane: inside each row of 16 lanes by DPP
// moves (pairs, quads, then rotations by 4 and 8), then the row sums of lanes 0, 16, 32 and 48 in row order.
__device__ __forceinline__ double wave_sum_d(double x) {
  x += dpp_d<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_d<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_d<0x124>(x);  // row_ror:4
  x += dpp_d<0x128>(x);  // row_ror:8
  return ((readlane_d<0>(x) + readlane_d<16>(x)) + readlane_d<32>(x)) + readlane_d<48>(x);
}

// Softmax of the k selected slot scores, best first (score(r): the float32 score of rank r), as the decode step
// computes it: fp64 exponentials relative to the best score, rank r = lane + 64 u kept on lane `lane`, per-lane
// partial sums in u order, then wave_sum_d; wts[r] receives the float32 weight. One wave; every lane active.
template <typename ScoreFn>
__device__ __forceinline__ void wave_rank_softmax(int k, ScoreFn score, float* wts) {
  const int lane = lane_id();
  const double m = (double)score(0);
  constexpr int RPL = MAX_K / 64;
  double ex[RPL];
  double zpart = 0.0;
#pragma unroll
  for (int u = 0; u < RPL; ++u) {
    const int r = lane + 64 * u;
    ex[u] = 0.0;
    if (64 * u < k && r < k) {
      ex[u] = exp((double)score(r) - m);
      zpart += ex[u];
    }
  }
  const double z = wave_sum_d(zpart);
#pragma unroll
  for (int u = 0; u < RPL; ++u) {
    const int r = lane + 64 * u;
    if (64 * u < k && r < k) wts[r] = (float)(ex[u] / z);
  }
}

// cbuf: this wave's compaction buffer for the two-factor bound (select_kept_candidates; NULL: select among all).
template <int CPL>
__device__ void wave_merge_topk(const Dims& D, const TopkPlan& P, const uint64_t* cand, const float* fsc,
                                const uint16_t* fid, uint64_t* scratch, uint64_t* sorted, int32_t* ids, float* wts,
                                uint64_t* cbuf = nullptr, int ccap = 0) {
  const int lane = lane_id();
  const int F = D.F, k = P.k, kpmax = P.kpmax;
  // every candidate's tuple, then the factor scores one factor at a time over all of them (the LDS reads of a
  // step in flight together); each slot score is still the float32 sum over factors left to right
  uint64_t tup[CPL];
  float S[CPL];
  int ps[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) tup[j] = cand[min(lane + 64 * j, P.ncand - 1)];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    ps[j] = (int)(tup[j] & 0xFFFF);
    S[j] = fsc[ps[j]];
  }
  for (int f = 1; f < F; ++f) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int p = (int)((tup[j] >> (16 * f)) & 0xFFFF);
      S[j] = S[j] + fsc[f * kpmax + p];
      ps[j] += p;
    }
  }
  const float L = cbuf ? merge_lower_bound(P, F, k, fsc, kpmax) : -INFINITY;
  uint64_t ck[CPL];
  bool keep[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = lane + 64 * j;
    ck[j] = c < P.ncand ? ((uint64_t)desc_key(S[j]) << 32) | ((uint64_t)ps[j] << 20) | (uint64_t)c : ~0ull;
    keep[j] = c < P.ncand && S[j] >= L;
  }
  select_kept_candidates<CPL, MERGE_RB>(ck, keep, L > -INFINITY, k, cbuf, ccap, scratch, sorted);
  for (int r = lane; r < k; r += 64) {
    const uint64_t t = cand[(int)(sorted[r] & 0xFFFFF)];
    long long id = 0;
    for (int f = 0; f < F; ++f) id = id * D.widths[f] + fid[f * kpmax + (int)((t >> (16 * f)) & 0xFFFF)];
    ids[r] = (int32_t)id;
  }
  wave_rank_softmax(k, [&](int r) { return desc_key_value((uint32_t)(sorted[r] >> 32)); }, wts);
  wave_sync();
}

}  // namespace sdm
