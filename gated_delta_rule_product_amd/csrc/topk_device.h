// Exact product-key top-k of one query, computed by one workgroup (shared by the top-k and decode kernels).
//
// Method (sparse-delta-memory CHANGELOG.md 2.0.0, "Upgrading from v1" and "New"): the slot score is the float32
// sum of the factor scores and the top-k is exact; equal slot scores go to the larger rank sum, then the larger
// first rank. Here a factor score is the float32 rounding of an fp64 FMA chain in coordinate order, and ranks are
// per-factor positions p_f under (score descending, index ascending), p_f = 0 best.
//
// Exactness of the candidate set: if slot a is at a position <= slot b's in every factor (and differs), a's slot
// score is >= b's (float32 addition is monotone) and its position sum is smaller, so a precedes b. A slot with
// prod(p_f + 1) > k is therefore preceded by at least k others and cannot be in the top k; every slot of the top k
// lies among the tuples with prod(p_f + 1) <= k (the candidate table), and those need only the best
// min(k, n_f) sub-keys of each factor.
#pragma once
#include "sdm_internal.h"

namespace sdm {

// Number of position tuples (p_1..p_{F-1}) with p_f < kp[f] and prod_{f >= 1}(p_f + 1) <= budget.
__device__ inline int cand_count_rest(const TopkPlan& P, int F, int budget) {
  if (F == 1) return 1;
  const int l1 = min(P.kp[1], budget);
  if (F == 2) return l1;
  int n = 0;
  for (int p1 = 0; p1 < l1; ++p1) {
    const int b1 = budget / (p1 + 1);
    const int l2 = min(P.kp[2], b1);
    if (F == 3) {
      n += l2;
      continue;
    }
    for (int p2 = 0; p2 < l2; ++p2) n += min(P.kp[3], b1 / (p2 + 1));
  }
  return n;
}

// Writes those tuples after first position p0, in lexicographic order, to out[0..) (at most `room` entries).
__device__ inline void cand_emit_rest(const TopkPlan& P, int F, int p0, int budget, uint64_t* out, int room) {
  int n = 0;
  if (F == 1) {
    if (n < room) out[n] = (uint64_t)p0;
    return;
  }
  const int l1 = min(P.kp[1], budget);
  for (int p1 = 0; p1 < l1; ++p1) {
    const uint64_t t1 = (uint64_t)p0 | ((uint64_t)p1 << 16);
    if (F == 2) {
      if (n < room) out[n] = t1;
      ++n;
      continue;
    }
    const int b1 = budget / (p1 + 1);
    const int l2 = min(P.kp[2], b1);
    for (int p2 = 0; p2 < l2; ++p2) {
      const uint64_t t2 = t1 | ((uint64_t)p2 << 32);
      if (F == 3) {
        if (n < room) out[n] = t2;
        ++n;
        continue;
      }
      const int l3 = min(P.kp[3], b1 / (p2 + 1));
      for (int p3 = 0; p3 < l3; ++p3) {
        if (n < room) out[n] = t2 | ((uint64_t)p3 << 48);
        ++n;
      }
    }
  }
}

// The whole block builds the candidate table of plan P in lexicographic order: thread i takes first positions
// p_0 = i, i + NT, ...; an exclusive scan of their counts gives each first position its output range.
// scratch: >= kp[0] + 1 ints (LDS). Ends with a barrier.
template <int NT>
__device__ void build_cand_table(const TopkPlan& P, int F, uint64_t* out, int* scratch) {
  const int tid = threadIdx.x;
  for (int p0 = tid; p0 < P.kp[0]; p0 += NT) scratch[p0] = cand_count_rest(P, F, P.k / (p0 + 1));
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < P.kp[0]; ++i) {
      const int c = scratch[i];
      scratch[i] = run;
      run += c;
    }
  }
  __syncthreads();
  for (int p0 = tid; p0 < P.kp[0]; p0 += NT) {
    const int o = scratch[p0];
    if (o < MAX_CAND) cand_emit_rest(P, F, p0, P.k / (p0 + 1), out + o, MAX_CAND - o);
  }
  __syncthreads();
}

// The same table built by NT threads without a serial step, in two phases with a block barrier between them
// (the caller's). Phase 1: thread t computes the output offset of first positions p_0 = t, t + NT, ... as the sum
// of the counts of the smaller first positions, offs[p_0], and offs[kp[0]] = ncand. Phase 2: two factors, every
// entry e by one thread (its first position found by binary search in offs); otherwise every first position's
// tuples by one thread. offs: >= kp[0] + 1 ints (LDS).
// With kp[0] <= 64 the first wave of the NT threads (t < 64) does phase 1 alone: one count per lane and a wave
// prefix sum (lane shuffles).
__device__ inline void cand_offsets(const TopkPlan& P, int F, int* offs, int t, int NT) {
  if (P.kp[0] <= 64) {
    if (t < 64) {
      int c = t < P.kp[0] ? cand_count_rest(P, F, P.k / (t + 1)) : 0;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(c, o, 64);
        if (t >= o) c += y;
      }
      if (t < P.kp[0]) offs[t + 1] = c;  // inclusive sum of first positions <= t = offset of t + 1
      if (t == 0) offs[0] = 0;
    }
    return;
  }
  for (int p0 = t; p0 < P.kp[0]; p0 += NT) {
    int o = 0;
    for (int q = 0; q < p0; ++q) o += cand_count_rest(P, F, P.k / (q + 1));
    offs[p0] = o;
  }
  if (t == 0) offs[P.kp[0]] = P.ncand;
}
__device__ inline void cand_emit(const TopkPlan& P, int F, const int* offs, uint64_t* out, int t, int NT) {
  if (F == 2) {
    for (int e = t; e < P.ncand; e += NT) {
      int lo = 0, hi = P.kp[0];  // the last p0 with offs[p0] <= e (counts are >= 1, offsets increase)
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offs[mid] <= e) lo = mid; else hi = mid;
      }
      out[e] = (uint64_t)lo | ((uint64_t)(e - offs[lo]) << 16);
    }
    return;
  }
  for (int p0 = t; p0 < P.kp[0]; p0 += NT)
    if (offs[p0] < MAX_CAND) cand_emit_rest(P, F, p0, P.k / (p0 + 1), out + offs[p0], MAX_CAND - offs[p0]);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts right by 1, 2, 4 and 8 lanes inside each
// row of 16 (lanes shifted in from outside the row read 0), then the last lane of row 0 and of row 2 added to rows
// 1 and 3, then the last lane of row 1 added to rows 2 and 3. All lanes active.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Two factors with kp[0] <= 64 and at most 64 tuples after any first position: one wave builds the whole table,
// with no barrier and no search. Lane p_0 counts its tuples, the wave prefix sum gives its output offset, and it
// writes them (lexicographic order, the same table as cand_offsets + cand_emit).
__device__ inline bool cand_one_wave(const TopkPlan& P, int F) {
  return F == 2 && P.kp[0] <= 64 && min(P.kp[1], P.k) <= 64;
}
__device__ inline void cand_table_wave(const TopkPlan& P, uint64_t* out, int lane) {
  const int c = lane < P.kp[0] ? min(P.kp[1], P.k / (lane + 1)) : 0;
  const int o = wave_inclusive_sum(c) - c;
  for (int p1 = 0; p1 < c; ++p1) out[o + p1] = (uint64_t)lane | ((uint64_t)p1 << 16);
}

// LDS bytes of one topk_query workspace (8-byte aligned regions).
__host__ __device__ inline size_t topk_lds_bytes(int F, int dk, const TopkPlan& P) {
  size_t n = 0;
  n += (size_t)F * dk * 8;                                              // query (fp64)
  n += (size_t)(P.nf_pow2 > P.cand_pow2 ? P.nf_pow2 : P.cand_pow2) * 8;  // sort keys
  n += (size_t)F * P.kpmax * 8;                                        // kept factor scores + sub-key ids
  n += (size_t)P.k * 16;                                               // result ids, scores, exp values
  return n;
}

struct TopkLds {
  double* q;
  uint64_t* keys;
  float* fsc;
  int32_t* fid;
  int32_t* rid;
  float* rsc;
  double* rexp;
};

__device__ inline TopkLds topk_lds_carve(unsigned char* base, int F, int dk, const TopkPlan& P) {
  TopkLds L;
  size_t o = 0;
  L.q = (double*)(base + o);
  o += (size_t)F * dk * 8;
  L.keys = (uint64_t*)(base + o);
  o += (size_t)(P.nf_pow2 > P.cand_pow2 ? P.nf_pow2 : P.cand_pow2) * 8;
  L.fsc = (float*)(base + o);
  o += (size_t)F * P.kpmax * 4;
  L.fid = (int32_t*)(base + o);
  o += (size_t)F * P.kpmax * 4;
  L.rexp = (double*)(base + o);
  o += (size_t)P.k * 8;
  L.rid = (int32_t*)(base + o);
  o += (size_t)P.k * 4;
  L.rsc = (float*)(base + o);
  return L;
}

// All NT threads of the block call this. On return (after a barrier) L.rid[0..k) / L.rsc[0..k) hold the top-k
// slot ids and float32 slot scores, best first.
template <typename A, int NT>
__device__ void topk_query(const A* __restrict__ q, const A* __restrict__ sub, const int* widths, int F, int dk,
                           const TopkPlan& P, const uint64_t* __restrict__ cand, const TopkLds& L) {
  const int tid = threadIdx.x;
  for (int c = tid; c < F * dk; c += NT) L.q[c] = to_d<A>(q[c]);
  __syncthreads();
  size_t off = 0;
  for (int f = 0; f < F; ++f) {
    const int n = widths[f];
    const int np2 = pow2_ceil(n);
    const A* tab = sub + off * dk;
    const double* qf = L.q + f * dk;
    for (int i = tid; i < np2; i += NT) {
      uint64_t key = ~0ull;
      if (i < n) {
        const A* row = tab + (size_t)i * dk;
        double acc = 0.0;
        for (int c = 0; c < dk; ++c) acc = fma(qf[c], to_d<A>(row[c]), acc);
        key = ((uint64_t)desc_key((float)acc) << 32) | (uint32_t)i;
      }
      L.keys[i] = key;
    }
    __syncthreads();
    bitonic_sort_u64<NT>(L.keys, np2);
    for (int p = tid; p < P.kp[f]; p += NT) {
      const uint64_t k = L.keys[p];
      L.fid[f * P.kpmax + p] = (int32_t)(uint32_t)k;
      L.fsc[f * P.kpmax + p] = desc_key_value((uint32_t)(k >> 32));
    }
    __syncthreads();
    off += n;
  }
  for (int c = tid; c < P.cand_pow2; c += NT) {
    uint64_t key = ~0ull;
    if (c < P.ncand) {
      const uint64_t tup = cand[c];
      int p = (int)(tup & 0xFFFF);
      float S = L.fsc[p];
      int ps = p;
      for (int f = 1; f < F; ++f) {
        p = (int)((tup >> (16 * f)) & 0xFFFF);
        S = S + L.fsc[f * P.kpmax + p];  // float32 sum, left to right
        ps += p;
      }
      // ascending key = (slot score descending, position sum ascending, lexicographic positions ascending)
      key = ((uint64_t)desc_key(S) << 32) | ((uint64_t)ps << 20) | (uint64_t)c;
    }
    L.keys[c] = key;
  }
  __syncthreads();
  bitonic_sort_u64<NT>(L.keys, P.cand_pow2);
  for (int r = tid; r < P.k; r += NT) {
    const uint64_t key = L.keys[r];
    const uint64_t tup = cand[(int)(key & 0xFFFFF)];
    long long id = 0;
    for (int f = 0; f < F; ++f) id = id * widths[f] + L.fid[f * P.kpmax + (int)((tup >> (16 * f)) & 0xFFFF)];
    L.rid[r] = (int32_t)id;
    L.rsc[r] = desc_key_value((uint32_t)(key >> 32));
  }
  __syncthreads();
}

// Softmax over the k selected scores (fp64, max-subtracted, sequential sum); weights into w (may alias nothing
// in L). All threads call; ends with a barrier.
template <int NT>
__device__ void topk_softmax(const TopkLds& L, int k, float* w) {
  const int tid = threadIdx.x;
  const double m = (double)L.rsc[0];  // best first: the maximum
  for (int r = tid; r < k; r += NT) L.rexp[r] = exp((double)L.rsc[r] - m);
  __syncthreads();
  __shared__ double s_z;
  if (tid == 0) {
    double z = 0.0;
    for (int r = 0; r < k; ++r) z += L.rexp[r];
    s_z = z;
  }
  __syncthreads();
  const double z = s_z;
  for (int r = tid; r < k; r += NT) w[r] = (float)(L.rexp[r] / z);
  __syncthreads();
}

}  // namespace sdm
