// Exact product-key top-k kernels: the candidate table and the batched top-k (write keys and read queries).
#include <cstdlib>
#include <cstring>

#include "sdm_internal.h"
#include "topk_device.h"
#include "topk_wave.h"

namespace sdm {

// One block per plan builds its candidate table (see build_cand_table).
__global__ __launch_bounds__(256) void cand_table_kernel(TopkPlan p0, TopkPlan p1, int F, uint64_t* __restrict__ tables) {
  __shared__ int scratch[MAX_K + 1];
  const TopkPlan& P = blockIdx.x == 0 ? p0 : p1;
  build_cand_table<256>(P, F, tables + (size_t)blockIdx.x * MAX_CAND, scratch);
}

hipError_t launch_cand_tables(const TopkPlan* plans, int nkinds, int F, uint64_t* tables, hipStream_t st) {
  hipLaunchKernelGGL(cand_table_kernel, dim3(nkinds), dim3(256), 0, st, plans[0], plans[nkinds > 1 ? 1 : 0], F,
                     tables);
  return hipGetLastError();
}

template <typename A>
__global__ __launch_bounds__(TOPK_NT) void topk_kernel(Dims D, TopkArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int kind = blockIdx.y;
  const TopkPlan& P = a.plan[kind];
  const int tn = a.tn ? a.tn : D.T;  // token window [a.t0, a.t0 + tn) of every batch row
  const int h = (int)(blockIdx.x % D.H);
  const long long btw = blockIdx.x / D.H;
  const int t = a.t0 + (int)(btw % tn);
  const int b = (int)(btw / tn);
  const long long row = ((long long)b * D.T + t) * D.H + h;
  const int Fdk = D.F * D.dk;
  long long sumn = 0;
  for (int f = 0; f < D.F; ++f) sumn += D.widths[f];
  const A* q = (const A*)a.queries[kind] + row * Fdk;
  const A* sub = (const A*)a.subkeys + (long long)h * sumn * D.dk;
  TopkLds L = topk_lds_carve(lds, D.F, D.dk, P);
  topk_query<A, TOPK_NT>(q, sub, D.widths, D.F, D.dk, P, a.cand[kind], L);
  const int k = P.k;
  if (a.stream_major) {
    const long long so = (((long long)b * D.H + h) * D.T + t) * k;
    for (int r = threadIdx.x; r < k; r += TOPK_NT) a.ids[kind][so + r] = L.rid[r];
    if (a.user_ids[kind])
      for (int r = threadIdx.x; r < k; r += TOPK_NT) a.user_ids[kind][row * k + r] = L.rid[r];
    topk_softmax<TOPK_NT>(L, k, a.vals[kind] + so);
  } else {
    for (int r = threadIdx.x; r < k; r += TOPK_NT) a.ids[kind][row * k + r] = L.rid[r];
    if (a.vals[kind])
      for (int r = threadIdx.x; r < k; r += TOPK_NT) a.vals[kind][row * k + r] = L.rsc[r];
  }
}

// ------------------------------------------------------------------------------------------- wave-level top-k
// One wave scores QW query rows (same head and kind) against every sub-key with the fp64 FMA chain, each lane
// owning NPL sub-keys (its rows read as 16-byte vectors and reused across the QW queries), selects each factor's
// top min(k, n_f) exactly (wave_select_sorted), then merges the candidate tuples (CPL per lane) the same way.
// Queries per wave for NPL sub-keys per lane (QW * NPL <= 16 keeps the fp64 accumulators at 32 registers). Narrow
// factors (NPL <= 2) take 4 queries: the per-wave LDS of 16 (the factor lists of every query are kept until the
// merge) allowed only one 4-wave block per CU, and the selections, which are latency-bound, ran at one wave per
// SIMD (three-factor workload: 1.87 -> 0.65 ms per kind). The filtered scoring of wide factors (NPL >= 8) takes 2:
// its MFMA tiles reload the factor's sub-key table per wave, so a second query halves that traffic, while 4 would
// cost occupancy (1,048,576 slots: 1.46 -> 1.03 ms per 32,768 queries; 4 queries: 1.36 ms).
__host__ __device__ constexpr int wave_qw(int npl, bool mf = false) {
  return (mf && npl >= 8) ? 2 : npl <= 2 ? 4 : 16 / npl < 1 ? 1 : 16 / npl;
}
template <int NPL, bool MF = false> struct WaveTile { static constexpr int QW = wave_qw(NPL, MF); };

// Whether the selection buffers of a wave in block mode (shared score rows; see factor_topk_filtered) live in its own
// score rows of 256 NPL bytes, which are free once a query's candidates are scored exactly: a factor's selection
// scratch [KS + 8] and sorted output [KS] (uint64) in the query's row, the merge's compaction buffer [256], scratch
// and sorted output in the wave's QW rows. KS = max(k_p max, k).
__host__ __device__ inline bool topk2_rows_scratch(int kpmax, int k, int QW, int NPL, bool shared_scores) {
  const int KS = kpmax > k ? kpmax : k;
  const int R = 256 * NPL;
  return shared_scores && (2 * KS + 8) * 8 <= R && (256 + 2 * KS + 8) * 8 <= QW * R;
}

// Per-wave LDS: factor scores [QW][64 NPL] (float; block mode: in the workgroup's shared rows), kept factor lists
// [QW][F][kpmax] (float score + uint16 id), selection scratch [KS + 8] and sorted output [KS] (uint64) unless they
// live in the score rows. The filtered scoring lists its candidates in each query's score row.
__host__ __device__ inline size_t topk2_wave_lds(int F, int kpmax, int k, int QW, int NPL, bool shared_scores = false) {
  const int KS = kpmax > k ? kpmax : k;
  size_t n = shared_scores ? 0 : (size_t)QW * 64 * NPL * 4;
  n += (size_t)QW * F * kpmax * 6;
  n = (n + 7) & ~(size_t)7;
  return n + (topk2_rows_scratch(kpmax, k, QW, NPL, shared_scores) ? 0 : (size_t)(2 * KS + 8) * 8);
}

// ------------------------------------------------------------------------------------------- filtered scoring
// For bf16 activations the factor scores are first computed with bf16 MFMA (float32 accumulation) as a filter, and
// only the sub-keys that can still be among a factor's top k_p are scored exactly (the fp64 chain that defines the
// score). With s the defined score (float32 rounding of the fp64 chain) and s^ the MFMA score, every product of two
// bf16 values is exact in float32, so |s - s^| <= E with
//   E = (dk + 2) 2^-23 |x| |c| (1 + 2^-20) + dk 2^-125 (|x| + |c| + 1)
// (x the query slice, c the sub-key row, |.| Euclidean norms): dk float32 additions in any order, truncating or
// rounding, the final rounding of s, and flushed subnormal inputs or products. Let v be the smallest of the k_p
// largest s^ and E_max the largest bound of the row: those k_p sub-keys have s >= s^ - E >= v - E_max, so the k_p-th
// largest s is >= v - E_max, every member of the true top k_p has s >= v - E_max and therefore s^ + E >= v - E_max.
// Keeping the sub-keys with s^ + E >= v - E_max loses none of them, and the exact selection among the kept ones
// (usually k_p or a few more) equals the selection among all.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Largest Euclidean norm of the sub-key rows of each factor (fp64 sum of squares, rounded up to float32; +inf when a
// row holds an infinity or a NaN): snmax[h][f]. One block per (factor, head); the maximum is order independent.
__global__ __launch_bounds__(256) void subkey_maxnorm_kernel(const bf16_t* __restrict__ sub, Dims D,
                                                             float* __restrict__ snmax) {
  __shared__ float wmax[4];
  const int f = blockIdx.x, h = blockIdx.y, dk = D.dk;
  long long off = 0, sumn = 0;
  for (int g = 0; g < D.F; ++g) {
    if (g < f) off += D.widths[g];
    sumn += D.widths[g];
  }
  const bf16_t* tab = sub + ((long long)h * sumn + off) * dk;
  float m = 0.0f;
  for (int i = threadIdx.x; i < D.widths[f]; i += 256) {
    const bf16_t* r = tab + (long long)i * dk;
    double s2 = 0.0;
    for (int c = 0; c < dk; ++c) {
      const double y = (double)bf16_to_f(r[c]);
      s2 = fma(y, y, s2);
    }
    const float nr = __double2float_ru(sqrt(s2) * (1.0 + 0x1p-40));
    m = nr == nr ? fmaxf(m, nr) : INFINITY;  // a row with a NaN counts as unbounded
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) snmax[h * D.F + f] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
}

__device__ __forceinline__ bf16x8_t load_bf16x8(const bf16_t* p) {
  const uint4 v = *(const uint4*)p;
  return __builtin_bit_cast(bf16x8_t, v);
}

// One factor of the wave's QW queries by the filtered scoring: MFMA tiles of 16 queries (nq used) x 16 sub-keys,
// one error bound per query (from the query norm and the factor's largest sub-key norm), thresholds, exact fp64
// re-score of the kept sub-keys, exact top-k_p. Writes fsc/fid like the direct path.
// Requires n % 16 == 0 and dk % 32 == 0, dk <= 128.
//
// Block mode (NW > 1): the NW waves of the workgroup hold NW * QW <= 16 consecutive queries, the rows of one MFMA
// tile; wave w computes tiles w, w + NW, ... for all of them (each sub-key tile is read once per workgroup) into
// the shared score buffer scs [NW QW][64 NPL]; qb/nqb are the workgroup's first query and query count, row0 the
// wave's first row, and qf/nq the wave's own queries. Every wave calls this (nq may be 0): it has two barriers.
template <int NPL, int QW, int NW = 1>
__device__ void factor_topk_filtered(const Dims& D, const TopkArgs& a, int f, int n, const bf16_t* tab,
                                     const bf16_t* qf, long long qstride, int nq, float* scs, float* fsc,
                                     uint16_t* fid, uint64_t* scratch, uint64_t* sorted, int kpmax,
                                     const bf16_t* qb = nullptr, int nqb = 0, int row0 = 0) {
  constexpr int KBMAX = 4;
  constexpr bool BLK = NW > 1;
  const int lane = threadIdx.x & 63;
  const int dk = D.dk, F = D.F;
  const int KB = dk / 32;
  const int ql = lane & 15, pt = lane >> 4;
  const int kind = blockIdx.y;
  const int kp = a.plan[kind].kp[f];
  const int wv = BLK ? (int)(threadIdx.x >> 6) : 0;
  const bf16_t* qa_base = BLK ? qb : qf;  // the MFMA rows: the workgroup's queries or the wave's
  const int nqa = BLK ? nqb : nq;
  // query fragments (A operand: row = query, 8 consecutive elements of a 32-wide block) and squared norms
  bf16x8_t qa[KBMAX];
  double nx2 = 0.0;
  static_for<KBMAX>([&](auto kc) {
    constexpr int kb = decltype(kc)::value;
    if (kb < KB) {
      if (ql < nqa) {
        qa[kb] = load_bf16x8(qa_base + ql * qstride + kb * 32 + pt * 8);
        const uint4 w = __builtin_bit_cast(uint4, qa[kb]);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double lo = (double)__uint_as_float(ws[e] << 16), hi = (double)__uint_as_float(ws[e] & 0xFFFF0000u);
          nx2 = fma(lo, lo, nx2);
          nx2 = fma(hi, hi, nx2);
        }
      } else {
        qa[kb] = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
      }
    }
  });
  nx2 += __shfl_xor(nx2, 16, 64);
  nx2 += __shfl_xor(nx2, 32, 64);
  // MFMA scores of tile T: lane l holds queries 4 (l / 16) + r (r < 4) for sub-key 16 T + l % 16
  // tiles in batches of TB whose B-operand loads are issued together (the table sits in L2: latency, not bandwidth)
  constexpr int TB = BLK ? 4 : NPL >= 8 ? 8 : 2;
  const int ntile = n / 16;
  for (int T0 = 0; T0 < ntile; T0 += TB * NW) {
    bf16x8_t bv[TB][2];
    static_for<TB>([&](auto tc) {
      constexpr int u = decltype(tc)::value;
      const bf16_t* row = tab + (long long)(min(T0 + u * NW + wv, ntile - 1) * 16 + ql) * dk + pt * 8;
      bv[u][0] = load_bf16x8(row);
      if (KB > 1) bv[u][1] = load_bf16x8(row + 32);
    });
    // the batch's MFMAs first (tiles past the end score the last tile again and are not stored), then the stores
    f32x4_t acc[TB];
    static_for<TB>([&](auto tc) {
      constexpr int u = decltype(tc)::value;
      const bf16_t* row = tab + (long long)(min(T0 + u * NW + wv, ntile - 1) * 16 + ql) * dk + pt * 8;
      acc[u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[0], bv[u][0], acc[u], 0, 0, 0);
      if (KB > 1) acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[1], bv[u][1], acc[u], 0, 0, 0);
      static_for<KBMAX - 2>([&](auto kc) {  // dk = 96, 128: the remaining blocks, loaded here
        constexpr int kb = decltype(kc)::value + 2;
        if (kb < KB)
          acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kb], load_bf16x8(row + kb * 32), acc[u], 0, 0, 0);
      });
    });
    // D row 4 (lane / 16) + r = query, column lane % 16 = sub-key in the tile; a lane's four rows are all stored or
    // none unless the tile's last query falls inside them
    if (4 * pt + 4 <= nqa) {
      static_for<TB>([&](auto tc) {
        constexpr int u = decltype(tc)::value;
        const int T = T0 + u * NW + wv;
        if (T < ntile) {
#pragma unroll
          for (int r = 0; r < 4; ++r) scs[(4 * pt + r) * 64 * NPL + T * 16 + ql] = acc[u][r];
        }
      });
    } else if (4 * pt < nqa) {
      static_for<TB>([&](auto tc) {
        constexpr int u = decltype(tc)::value;
        const int T = T0 + u * NW + wv;
        if (T < ntile) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (4 * pt + r < nqa) scs[(4 * pt + r) * 64 * NPL + T * 16 + ql] = acc[u][r];
        }
      });
    }
  }
  if constexpr (BLK) {
    __syncthreads();  // every tile's scores in LDS
    scs += row0 * 64 * NPL;  // this wave's queries
  } else {
    wave_sync();
  }
  // E bounds |s - s^| for every sub-key of the factor (its norm <= the factor's largest norm): a true top-k_p
  // member j has s_j >= (k_p-th largest s) >= L - E for any L with k_p sub-keys at s^ >= L, hence s^_j >= L - 2E;
  // any sub-key below that threshold has s < L - E and is not a member (ties included)
  const double cmax = (double)a.snorm[(long long)blockIdx.z * F + f];
  const uint64_t below = lanes_below_mask();
  const int KS = a.plan[kind].kpmax > a.plan[kind].k ? a.plan[kind].kpmax : a.plan[kind].k;
  const bool rows_scratch = topk2_rows_scratch(a.plan[kind].kpmax, a.plan[kind].k, QW, NPL, BLK);
  for (int q = 0; q < nq; ++q) {
    // the lane index taken afresh each query (an empty asm hides its value): the compiler otherwise hoists the
    // per-slot sub-key indices and bounds derived from it out of this loop and spills them to scratch memory
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const double nx = sqrt(__shfl(nx2, row0 + q, 64)) * (1.0 + 0x1p-40);
    const double E = (dk + 2) * 0x1p-23 * nx * cmax * (1.0 + 0x1p-20) + dk * 0x1p-125 * (nx + cmax + 1.0);
    // Every s^ is finite when |x| |c| <= 2^127: each partial sum of the MFMA, in any order, is at most
    // sum_i |x_i c_i| (1 + 2^-24)^dk <= |x| |c| (1 + 2^-17) for dk <= 128 (Cauchy-Schwarz), far below the float32
    // maximum. Otherwise (large or non-finite inputs: the norm of a non-finite row is +inf, a NaN query gives a NaN
    // bound) every sub-key is kept and scored exactly.
    const bool anybad = __ballot(!(E <= 1e300 && nx * cmax <= 0x1p127)) != 0ull;
    // The query's score row (256 NPL bytes) is read into registers first and then holds, in turn, the candidate keys
    // of the first stage (uint64, up to 32 NPL), the candidates kept for exact scoring (uint16) and, in block mode
    // when they fit, the selection buffers.
    float* srow = scs + q * 64 * NPL;
    uint64_t* row64 = (uint64_t*)srow;
    uint16_t* klist = (uint16_t*)srow;
    float sv[NPL];  // the lane's s^ (-inf past the factor), kept for the compaction below
#pragma unroll
    for (int j = 0; j < NPL; ++j) sv[j] = srow[lane + 64 * j];  // inside the row buffer: read without a bound
    float lmax = -INFINITY, lmax2 = -INFINITY;  // the lane's largest and second largest s^
    // a factor filling the row (the usual case) takes no per-element bound checks: the compiler would otherwise keep
    // the sixteen loop-invariant lane masks of i < n in scalar registers, which spill
    const bool full = n == 64 * NPL;
    auto lane_max = [&](auto fc) {
      constexpr bool FULL = decltype(fc)::value;
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        if (!FULL) sv[j] = lane + 64 * j < n ? sv[j] : -INFINITY;
        lmax2 = fmaxf(lmax2, fminf(lmax, sv[j]));
        lmax = fmaxf(lmax, sv[j]);
      }
    };
    if (full)
      lane_max(std::true_type{});
    else
      lane_max(std::false_type{});
    // Wide factors first keep only the sub-keys that can reach a value L that at least k_p of them reach in s^:
    // the k_p-th largest lane maximum (k_p <= 64 lanes hold a value at least that large), or the ceil(k_p / 2)-th
    // largest lane second maximum (that many lanes hold two values at least that large; every lane holds at least
    // four sub-keys here), whichever is larger: usually a small fraction of the factor.
    int mA = n;
    float thrA = -INFINITY;
    if constexpr (NPL >= 8) {
      auto kth_largest = [&](float v, int need) -> float {  // the need-th largest v over the wave's lanes
        if (need >= 64) return desc_key_value(__ockl_wfred_max_u32(desc_key(v)));  // the smallest
        const uint64_t lk[1] = {((uint64_t)desc_key(v) << 32) | (uint32_t)lane};
        return desc_key_value(wave_kth_high<1>(lk, need));
      };
      const float L = fmaxf(kth_largest(lmax, kp), kth_largest(lmax2, (kp + 1) / 2));
      thrA = (anybad || kp > 64) ? -INFINITY : __double2float_rd((double)L - 2.0 * E);
      if (!anybad) {  // (otherwise every sub-key is a candidate, taken from the registers)
        // the candidates listed as (s^ bits, index), up to 32 NPL of them
        wave_sync();  // every lane has read its scores before the list overwrites the row
        mA = 0;
        auto list = [&](auto fc) {
          constexpr bool FULL = decltype(fc)::value;
#pragma unroll
          for (int j = 0; j < NPL; ++j) {
            const int i = lane + 64 * j;
            const bool kept = (FULL || i < n) && sv[j] >= thrA;
            const uint64_t bm = __ballot(kept);
            const int pos = mA + __popcll(bm & below);
            if (kept && pos < 32 * NPL) row64[pos] = ((uint64_t)__float_as_uint(sv[j]) << 32) | (uint32_t)i;
            mA += __popcll(bm);
          }
        };
        if (full)
          list(std::true_type{});
        else
          list(std::false_type{});
        wave_sync();
      }
    }
    const bool listed = NPL >= 8 && !anybad && mA <= 32 * NPL;
    // approximate keys of the candidates, the k_p best approximate scores (radix select, stopped once decided),
    // v = the smallest of them; keep every candidate with s^ >= v - 2E
    // LISTED: the first stage's keys from the row (mA <= 32 NPL); otherwise from the registers: every sub-key of the
    // factor that the first stage kept (narrow factors: all of them), NS = NPL
    auto stage_b = [&](auto nsc, auto listed) -> int {
      constexpr int NS = decltype(nsc)::value;
      constexpr bool LISTED = decltype(listed)::value;
      uint64_t key[NS];
      if constexpr (LISTED) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const uint64_t kj = row64[min(lane + 64 * j, 32 * NPL - 1)];
          const uint64_t kd = ((uint64_t)desc_key(__uint_as_float((uint32_t)(kj >> 32))) << 32) | (uint32_t)kj;
          key[j] = lane + 64 * j < mA ? kd : ~0ull;
        }
      } else {
        static_assert(NS == NPL, "keys from the registers: one a sub-key");
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const int i = lane + 64 * j;
          key[j] = i < n && (NPL < 8 || anybad || sv[j] >= thrA) ? ((uint64_t)desc_key(sv[j]) << 32) | (uint32_t)i
                                                                : ~0ull;
        }
      }
      const uint32_t kmax = wave_kth_high<NS>(key, kp);
      const float thr = anybad ? -INFINITY : __double2float_rd((double)desc_key_value(kmax) - 2.0 * E);
      wave_sync();  // every lane has read its candidates before the kept list overwrites them
      int m = 0;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const bool kept = key[j] != ~0ull && (anybad || desc_key_value((uint32_t)(key[j] >> 32)) >= thr);
        const uint64_t bm = __ballot(kept);
        if (kept) klist[m + __popcll(bm & below)] = (uint16_t)(uint32_t)key[j];
        m += __popcll(bm);
      }
      return m;
    };
    int m;
    if constexpr (NPL >= 8) {
      if (listed && mA <= 128)
        m = stage_b(std::integral_constant<int, 2>{}, std::true_type{});
      else if (listed && mA <= 256)
        m = stage_b(std::integral_constant<int, 4>{}, std::true_type{});
      else if (NPL > 8 && listed)
        m = stage_b(std::integral_constant<int, 8>{}, std::true_type{});
      else
        m = stage_b(std::integral_constant<int, NPL>{}, std::false_type{});
    } else {
      m = stage_b(std::integral_constant<int, NPL>{}, std::false_type{});
    }
    wave_sync();
    // exact scores of the kept sub-keys (the fp64 chain), then the exact top k_p among them
    const bf16_t* xq = qf + q * qstride;
    auto exact_key = [&](int r) -> uint64_t {
      const int i = klist[r];
      const uint4* y = (const uint4*)(tab + (long long)i * dk);
      const uint4* xv4 = (const uint4*)xq;
      double acc = 0.0;
      // 32 coordinates a round (dk % 32 == 0): the round's loads in flight together, then its FMAs in order
      for (int p0 = 0; p0 < dk / 8; p0 += 4) {
        uint4 xv[4], yv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          xv[u] = xv4[p0 + u];
          yv[u] = y[p0 + u];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc = fma(Vec16<bf16_t>::at(xv[u], e), Vec16<bf16_t>::at(yv[u], e), acc);
      }
      return ((uint64_t)desc_key((float)acc) << 32) | (uint32_t)i;
    };
    // the selection buffers: the row's, once every exact key is in registers, or the wave's own
    uint64_t* scr = rows_scratch ? row64 : scratch;
    uint64_t* srt = rows_scratch ? row64 + KS + 8 : sorted;
    if (m <= 64) {
      uint64_t ek[1] = {lane < m ? exact_key(lane) : ~0ull};
      wave_sync();
      wave_select_sorted<1>(ek, kp, scr, srt);
    } else if (m <= 128) {
      uint64_t ek[2];
      ek[0] = exact_key(lane);
      ek[1] = lane + 64 < m ? exact_key(lane + 64) : ~0ull;
      wave_sync();
      wave_select_sorted<2>(ek, kp, scr, srt);
    } else {
      uint64_t ek[NPL];
#pragma unroll
      for (int j = 0; j < NPL; ++j) ek[j] = lane + 64 * j < m ? exact_key(lane + 64 * j) : ~0ull;
      wave_sync();
      wave_select_sorted<NPL>(ek, kp, scr, srt);
    }
    for (int p = lane; p < kp; p += 64) {
      const uint64_t kk = srt[p];
      fsc[(q * F + f) * kpmax + p] = desc_key_value((uint32_t)(kk >> 32));
      fid[(q * F + f) * kpmax + p] = (uint16_t)(uint32_t)kk;
    }
    wave_sync();
  }
  if constexpr (BLK) __syncthreads();  // the next factor's tiles overwrite the shared scores
}

// Waves per workgroup: 4; the filtered scoring of wide factors uses 8 waves of 2 queries, so that one MFMA tile of 16
// queries covers the workgroup and each sub-key tile is read once per workgroup (block mode of
// factor_topk_filtered, scores in a shared LDS buffer).
// Waves per workgroup in block mode (NW * QW rows of the MFMA tile, <= 16). Four waves of 2 queries leave half of
// each MFMA tile's rows unused and read the sub-key table once per 8 queries, but their 50 KB of LDS lets three
// workgroups share a CU where the 100 KB of eight waves allowed one: the selections, which set the time, then run at
// 3 waves per SIMD instead of 2 (1,048,576 slots, 131,072 queries: 2.56 -> 1.87 ms; two waves: 2.01 ms).
constexpr int TOPK_BLK_NW = 4;
constexpr int TOPK_WIDE_WPE = 1;  // waves-per-SIMD hint of the kernels with NPL > 4 (their register budget)
template <int NPL, bool MF> struct Topk2Waves {
  static constexpr bool BLK = MF && WaveTile<NPL, true>::QW == 2;
  static constexpr int NW = BLK ? TOPK_BLK_NW : 4;
};

// QW1: one query per wave (few rows, e.g. a decode step: parallelism over queries rather than reuse of sub-key rows).
template <typename A, int NPL, int CPL, bool MF, bool QW1>
__global__ __launch_bounds__((64 * Topk2Waves<NPL, MF>::NW)) __attribute__((amdgpu_waves_per_eu((NPL <= 4 || (MF && !QW1)) ? 4 : TOPK_WIDE_WPE))) void topk2_kernel(Dims D, TopkArgs a) {
  constexpr int QW = QW1 ? 1 : WaveTile<NPL, MF>::QW;
  constexpr int NW = QW1 ? 4 : Topk2Waves<NPL, MF>::NW;
  constexpr bool BLK = !QW1 && Topk2Waves<NPL, MF>::BLK;  // block mode of the filtered scoring
  constexpr int VEC = Vec16<A>::N;
  extern __shared__ __align__(16) unsigned char lds[];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int kind = blockIdx.y, h = blockIdx.z;
  const TopkPlan& P = a.plan[kind];
  const int F = D.F, dk = D.dk, k = P.k, kpmax = P.kpmax;
  // rows bt of the token window [a.t0, a.t0 + tn) of every batch row: (b, t) = (bt / tn, a.t0 + bt % tn)
  const int tn = a.tn ? a.tn : D.T;
  const long long BT = (long long)D.B * tn;
  auto grow = [&](long long bt) { return (bt / tn) * D.T + a.t0 + bt % tn; };  // b T + t
  const long long bt0 = ((long long)blockIdx.x * NW + wv) * QW;
  const uint64_t* cand = a.cand[kind];
  const size_t shared_scs = BLK ? (size_t)NW * QW * 64 * NPL * 4 : 0;  // block mode: [NW QW][64 NPL] scores
  if constexpr (QW1) {  // few rows: the block builds its kind's candidate table itself (no separate launch)
    uint64_t* ctab = (uint64_t*)(lds + 4 * topk2_wave_lds(F, kpmax, k, QW, NPL));
    build_cand_table<256>(P, F, ctab, (int*)(ctab + P.ncand));
    cand = ctab;
  }
  if (!BLK && bt0 >= BT) return;  // no block-wide barriers below: idle waves may leave
  const int KS = kpmax > k ? kpmax : k;
  unsigned char* wl = lds + shared_scs + (size_t)wv * topk2_wave_lds(F, kpmax, k, QW, NPL, BLK);
  float* scs = BLK ? (float*)lds : (float*)wl;              // [QW][64 NPL] (block mode: the shared buffer)
  float* fsc = (float*)(wl + (BLK ? 0 : (size_t)QW * 64 * NPL * 4));  // [QW][F][kpmax]
  uint16_t* fid = (uint16_t*)(fsc + QW * F * kpmax);        // [QW][F][kpmax]
  uint64_t* scratch = (uint64_t*)(wl + (((BLK ? 0 : (size_t)QW * 64 * NPL * 4) + (size_t)QW * F * kpmax * 6 + 7) &
                                        ~(size_t)7));
  uint64_t* sorted = scratch + KS + 8;                      // (unused when the score rows hold them)
  long long sumn = 0;
  for (int f = 0; f < F; ++f) sumn += D.widths[f];
  const A* sub = (const A*)a.subkeys + (long long)h * sumn * dk;
  const int Fdk = F * dk;
  const int nq = (int)max(0LL, min((long long)QW, BT - bt0));
  // the rows of bt0 + q are consecutive (a window of several batch rows is a multiple of 16 tokens)
  const A* qbase = (const A*)a.queries[kind] + (grow(bt0) * D.H + h) * Fdk;
  const long long qstride = (long long)D.H * Fdk;

  long long off = 0;
  for (int f = 0; f < F; ++f) {
    const int n = D.widths[f];
    const A* tab = sub + off * dk;
    if constexpr (MF && BLK) {
      const long long bb = (long long)blockIdx.x * NW * QW;  // the workgroup's first row
      const bf16_t* qb = (const bf16_t*)a.queries[kind] + (grow(bb) * D.H + h) * Fdk + f * dk;
      factor_topk_filtered<NPL, QW, NW>(D, a, f, n, (const bf16_t*)tab, (const bf16_t*)qbase + f * dk, qstride, nq,
                                        scs, fsc, fid, scratch, sorted, kpmax, qb,
                                        (int)max(0LL, min((long long)NW * QW, BT - bb)), wv * QW);
      off += n;
      continue;
    } else if constexpr (MF) {
      factor_topk_filtered<NPL, QW>(D, a, f, n, (const bf16_t*)tab,
                                    (const bf16_t*)qbase + f * dk, qstride, nq, scs, fsc, fid, scratch, sorted,
                                    kpmax);
      off += n;
      continue;
    }
    double acc[QW][NPL];
#pragma unroll
    for (int q = 0; q < QW; ++q)
#pragma unroll
      for (int j = 0; j < NPL; ++j) acc[q][j] = 0.0;
    for (int c0 = 0; c0 < dk; c0 += VEC) {
      uint4 rv[NPL];
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const int i = lane + 64 * j;
        rv[j] = i < n ? *(const uint4*)(tab + (long long)i * dk + c0) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
#pragma unroll
        for (int q = 0; q < QW; ++q) {
          const long long qq = q < nq ? q : 0;
          const double x = to_d<A>(qbase[qq * qstride + f * dk + c0 + e]);
#pragma unroll
          for (int j = 0; j < NPL; ++j) acc[q][j] = fma(x, Vec16<A>::at(rv[j], e), acc[q][j]);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < QW; ++q)
#pragma unroll
      for (int j = 0; j < NPL; ++j) scs[q * 64 * NPL + lane + 64 * j] = (float)acc[q][j];
    wave_sync();
    for (int q = 0; q < nq; ++q) {
      int lane = threadIdx.x & 63;  // taken afresh (see factor_topk_filtered): nothing derived from it is hoisted
      asm volatile("" : "+v"(lane));
      uint64_t key[NPL];
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const int i = lane + 64 * j;
        key[j] = i < n ? (((uint64_t)desc_key(scs[q * 64 * NPL + i]) << 32) | (uint32_t)i) : ~0ull;
      }
      wave_select_sorted<NPL>(key, P.kp[f], scratch, sorted);
      for (int p = lane; p < P.kp[f]; p += 64) {
        const uint64_t kk = sorted[p];
        fsc[(q * F + f) * kpmax + p] = desc_key_value((uint32_t)(kk >> 32));
        fid[(q * F + f) * kpmax + p] = (uint16_t)(uint32_t)kk;
      }
      wave_sync();
    }
    off += n;
  }

  // the merge's compaction buffer: this wave's factor-score rows, free once every factor is done (in block mode with
  // the selection buffers in the rows: their first 256 entries, the merge's scratch and sorted output after them)
  uint64_t* cbuf = (uint64_t*)(scs + (BLK ? wv * QW * 64 * NPL : 0));
  const bool rows_scratch = topk2_rows_scratch(kpmax, k, QW, NPL, BLK);
  const int ccap = rows_scratch ? 256 : QW * 64 * NPL / 2;  // uint64 entries
  if (rows_scratch) {
    scratch = cbuf + 256;
    sorted = scratch + KS + 8;
  }
  for (int q = 0; q < nq; ++q) {
    int lane = threadIdx.x & 63;  // taken afresh (see factor_topk_filtered): nothing derived from it is hoisted
    asm volatile("" : "+v"(lane));
    // candidates below a lower bound on the k-th slot score (two factors) are not selected from
    const float L = ccap >= 128 ? merge_lower_bound(P, F, k, fsc + q * F * kpmax, kpmax) : -INFINITY;
    // the candidates in groups of up to 8 a lane: the group's tuples (loads in flight together), then the factor
    // scores one factor at a time; each slot score is the float32 sum over factors left to right
    constexpr int MB = CPL < 8 ? CPL : 8;
    uint64_t ck[CPL];
    bool keep[CPL];
    static_for<CPL / MB>([&](auto gc) {
      constexpr int j0 = decltype(gc)::value * MB;
      uint64_t tup[MB];
#pragma unroll
      for (int u = 0; u < MB; ++u) tup[u] = cand[min(lane + 64 * (j0 + u), P.ncand - 1)];
      float S[MB];
      int ps[MB];
#pragma unroll
      for (int u = 0; u < MB; ++u) {
        ps[u] = (int)(tup[u] & 0xFFFF);
        S[u] = fsc[(q * F) * kpmax + ps[u]];
      }
      for (int f = 1; f < F; ++f) {
#pragma unroll
        for (int u = 0; u < MB; ++u) {
          const int p = (int)((tup[u] >> (16 * f)) & 0xFFFF);
          S[u] = S[u] + fsc[(q * F + f) * kpmax + p];
          ps[u] += p;
        }
      }
#pragma unroll
      for (int u = 0; u < MB; ++u) {
        const int c = lane + 64 * (j0 + u);
        ck[j0 + u] = c < P.ncand ? ((uint64_t)desc_key(S[u]) << 32) | ((uint64_t)ps[u] << 20) | (uint64_t)c : ~0ull;
        keep[j0 + u] = c < P.ncand && S[u] >= L;
      }
    });
    select_kept_candidates<CPL, 8>(ck, keep, L > -INFINITY, k, cbuf, ccap, scratch, sorted);
    const long long bt = bt0 + q;
    const long long b = bt / tn, t = a.t0 + bt % tn;
    const long long row = (b * D.T + t) * D.H + h;
    const double m = (double)desc_key_value((uint32_t)(sorted[0] >> 32));
    double zpart = 0.0, e0 = 0.0;  // e0: the exponential of this lane's first rank, kept for the weights
    for (int r = lane; r < k; r += 64) {
      const uint64_t kk = sorted[r];
      const uint64_t tup = cand[(int)(kk & 0xFFFFF)];
      long long id = 0;
      for (int f = 0; f < F; ++f)
        id = id * D.widths[f] + fid[(q * F + f) * kpmax + (int)((tup >> (16 * f)) & 0xFFFF)];
      const float sc = desc_key_value((uint32_t)(kk >> 32));
      if (a.stream_major) {
        const long long so = ((b * D.H + h) * D.T + t) * k;
        a.ids[kind][so + r] = (int32_t)id;
        if (a.user_ids[kind]) a.user_ids[kind][row * k + r] = (int32_t)id;
        const double ex = exp((double)sc - m);
        if (r == lane) e0 = ex;
        zpart += ex;
      } else {
        a.ids[kind][row * k + r] = (int32_t)id;
        if (a.vals[kind]) a.vals[kind][row * k + r] = sc;
      }
    }
    if (a.stream_major) {
      // softmax normaliser: per-lane partial sums (fixed order), then a fixed butterfly across the wave
      double z = zpart;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) z += __shfl_xor(z, o);
      const long long so = ((b * D.H + h) * D.T + t) * k;
      for (int r = lane; r < k; r += 64) {
        const double ex = r == lane ? e0 : exp((double)desc_key_value((uint32_t)(sorted[r] >> 32)) - m);
        a.vals[kind][so + r] = (float)(ex / z);
      }
    }
    wave_sync();
  }
}

template <typename A, int NPL, int CPL, bool MF, bool QW1>
static void launch_topk2_k(dim3 grid, size_t lds, hipStream_t st, const Dims& D, const TopkArgs& a) {
  (void)hipFuncSetAttribute((const void*)topk2_kernel<A, NPL, CPL, MF, QW1>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  constexpr int NW = QW1 ? 4 : Topk2Waves<NPL, MF>::NW;
  hipLaunchKernelGGL((topk2_kernel<A, NPL, CPL, MF, QW1>), grid, dim3(64 * NW), lds, st, D, a);
}

template <typename A, int NPL>
static bool launch_topk2_npl(const Dims& D, const TopkArgs& a, hipStream_t st, int cpl, size_t lds, bool mf) {
  const int QW = a.one_query_per_wave ? 1 : (mf ? WaveTile<NPL, true>::QW : WaveTile<NPL>::QW);
  const long long BT = (long long)D.B * (a.tn ? a.tn : D.T);
  const long long tiles = (BT + QW - 1) / QW;
  const int NW = (!a.one_query_per_wave && mf) ? Topk2Waves<NPL, true>::NW : 4;
  dim3 grid((unsigned)((tiles + NW - 1) / NW), (unsigned)a.nkinds, (unsigned)D.H);
  auto go = [&](auto mfc, auto qw1c) {
    constexpr bool MFV = decltype(mfc)::value, QW1V = decltype(qw1c)::value;
    if (cpl == 4) launch_topk2_k<A, NPL, 4, MFV, QW1V>(grid, lds, st, D, a);
    else if (cpl == 8) launch_topk2_k<A, NPL, 8, MFV, QW1V>(grid, lds, st, D, a);
    else launch_topk2_k<A, NPL, 16, MFV, QW1V>(grid, lds, st, D, a);
  };
  if (a.one_query_per_wave) {
    go(std::false_type{}, std::true_type{});
    return true;
  }
  if constexpr (sizeof(A) == 2) {
    if (mf) {
      go(std::true_type{}, std::false_type{});
      return true;
    }
  }
  go(std::false_type{}, std::false_type{});
  return true;
}

// The filtered (MFMA) scoring serves bf16 activations with factor widths that are multiples of 16 and
// dk in {32, 64, 96, 128}. By default (SDM_SCORING_AUTO) it runs when a factor has at least 512 sub-keys: below that
// the direct fp64 chain over every sub-key costs no more than the filter's extra selection and re-scoring (measured:
// 256 and 64 sub-keys per factor are as fast or faster direct; 1024 sub-keys are about twice as fast filtered).
// The config's topk_scoring forces either kernel; both return the same ids and scores.
static bool topk_filtered(const Dims& D, const TopkArgs& a) {
  if (D.scoring == SDM_SCORING_DIRECT) return false;
  if (D.act != SDM_BF16 || a.snorm == nullptr) return false;
  if (D.dk % 32 != 0 || D.dk > 128) return false;
  int nmax = 0;
  for (int f = 0; f < D.F; ++f) {
    if (D.widths[f] % 16 != 0) return false;
    nmax = D.widths[f] > nmax ? D.widths[f] : nmax;
  }
  for (int q = 0; q < a.nkinds; ++q)
    if (((uintptr_t)a.queries[q]) % 16 != 0) return false;
  if (D.scoring == SDM_SCORING_FILTERED) return true;
  return nmax >= 512;
}

template <typename A>
static bool launch_topk2(const Dims& D, const TopkArgs& a, hipStream_t st) {
  int nfmax = 0;
  for (int f = 0; f < D.F; ++f) nfmax = D.widths[f] > nfmax ? D.widths[f] : nfmax;
  int npl = 1;
  while (npl * 64 < nfmax) npl <<= 1;
  if (npl > 16) return false;
  int ncand = 0, kpmax = 0, kmax = 0;
  for (int q = 0; q < a.nkinds; ++q) {
    ncand = a.plan[q].ncand > ncand ? a.plan[q].ncand : ncand;
    kpmax = a.plan[q].kpmax > kpmax ? a.plan[q].kpmax : kpmax;
    kmax = a.plan[q].k > kmax ? a.plan[q].k : kmax;
  }
  if (ncand > 1024 || kpmax > 1024) return false;
  if ((D.dk * (int)sizeof(A)) % 16 != 0 || ((uintptr_t)a.subkeys) % 16 != 0) return false;
  const int cpl = ncand <= 256 ? 4 : ncand <= 512 ? 8 : 16;
  const bool mf = !a.one_query_per_wave && topk_filtered(D, a);
  const int QW = a.one_query_per_wave ? 1 : wave_qw(npl, mf);
  // block mode of the filtered scoring (TOPK_BLK_NW waves of 2 queries, shared [2 TOPK_BLK_NW][64 npl] scores) for
  // wide factors
  const bool blk = mf && QW == 2;
  size_t lds = 0;
  for (int q = 0; q < a.nkinds; ++q) {
    size_t l = blk ? (size_t)TOPK_BLK_NW * QW * 64 * npl * 4 +
                         TOPK_BLK_NW * topk2_wave_lds(D.F, a.plan[q].kpmax, a.plan[q].k, QW, npl, true)
                   : 4 * topk2_wave_lds(D.F, a.plan[q].kpmax, a.plan[q].k, QW, npl);
    if (a.one_query_per_wave) l += (size_t)a.plan[q].ncand * 8 + (size_t)(a.plan[q].kp[0] + 1) * 4;
    lds = l > lds ? l : lds;
  }
  if (lds > 128 * 1024) return false;
  if (mf) {
    hipLaunchKernelGGL(subkey_maxnorm_kernel, dim3((unsigned)D.F, (unsigned)D.H), dim3(256), 0, st,
                       (const bf16_t*)a.subkeys, D, a.snorm);
  }
  switch (npl) {
    case 1: return launch_topk2_npl<A, 1>(D, a, st, cpl, lds, mf);
    case 2: return launch_topk2_npl<A, 2>(D, a, st, cpl, lds, mf);
    case 4: return launch_topk2_npl<A, 4>(D, a, st, cpl, lds, mf);
    case 8: return launch_topk2_npl<A, 8>(D, a, st, cpl, lds, mf);
    default: return launch_topk2_npl<A, 16>(D, a, st, cpl, lds, mf);
  }
}

hipError_t launch_topk(const Dims& D, const TopkArgs& a, hipStream_t st) {
  const long long rows = (long long)D.B * (a.tn ? a.tn : D.T) * D.H;
  if (rows == 0) return hipSuccess;
  const bool done = D.act == SDM_BF16 ? launch_topk2<bf16_t>(D, a, st) : launch_topk2<float>(D, a, st);
  if (done) return hipGetLastError();
  if (a.one_query_per_wave) {  // the block-level kernel reads the candidate tables from the workspace
    const hipError_t e = launch_cand_tables(a.plan, a.nkinds, D.F, (uint64_t*)a.cand[0], st);
    if (e != hipSuccess) return e;
  }
  size_t lds = 0;
  for (int q = 0; q < a.nkinds; ++q) {
    size_t l = topk_lds_bytes(D.F, D.dk, a.plan[q]);
    if (l > lds) lds = l;
  }
  dim3 grid((unsigned)rows, (unsigned)a.nkinds);
  if (D.act == SDM_BF16)
    hipLaunchKernelGGL(topk_kernel<bf16_t>, grid, dim3(TOPK_NT), lds, st, D, a);
  else
    hipLaunchKernelGGL(topk_kernel<float>, grid, dim3(TOPK_NT), lds, st, D, a);
  return hipGetLastError();
}

}  // namespace sdm
