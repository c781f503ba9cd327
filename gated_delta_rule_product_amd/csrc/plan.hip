// Chunk plan: everything of a chunk that does not depend on the bank, for every (stream, chunk) in parallel.
//
// Chunked form of the per-token recurrence (gated delta rule restricted to the selected rows; sparse-delta-memory
// CHANGELOG.md 2.0.0: a chunked write/read whose chunk size changes results only through rounding, with an
// IEEE-float32 triangular ("WY") solve and a "dual" product inside the op). For a chunk of tokens 0..C-1 with bank
// M_0 at its start, let gamma_j(s -> t) be the product of alpha_u over the chunk's tokens u in (s, t] that write
// slot j. Then
//   h_t = sum_{j in S_t} w_tj gamma_j(0 -> t-1) M_0[j]       (write gather, coefficient a_tj)
//   g_t = sum_{j in R_t} rho_tj gamma_j(0 -> t) M_0[j]       (read gather, coefficient b_tj)
//   K_ts = sum_{j in S_t and S_s} w_tj w_sj gamma_j(s -> t-1)             for s < t
//   Q_ts = sum_{j in R_t and S_s} rho_tj w_sj gamma_j(s -> t)             for s <= t
//   delta = T (diag(beta) V - diag(alpha beta) H),  T = (I + diag(alpha beta) K)^-1  (unit lower triangular)
//   out_t = g_t + sum_s Q_ts delta_s,
// and each written row ends as the in-order application of M[j] <- alpha_s M[j] + w_sj delta_s over its events.
// The kernel sorts the chunk's write events by (slot, token) and writes the chunk region of chunk_layout: the
// gather terms (slot, a) and (slot, b), T and Q as row-sorted sparse lists, and the slot segments with their
// events. T is solved in IEEE float32 by forward substitution, row after row, over the nonzero entries of each row
// of diag(alpha beta) K only. Every floating-point sum runs in a fixed order (bitwise repeatable); the only atomics
// are integer bit sets in LDS.
//
// Parallel structure (one 512-thread workgroup per chunk): gather terms are computed one thread per term; the few
// terms that meet an earlier event of the same slot are flagged in per-token bit masks, and one thread per token
// then adds their K and Q contributions in term order. Row nonzero masks, counts and offsets of the sparse T/Q lists
// come from wave ballots and prefix sums.
#include "sdm_internal.h"

namespace sdm {

// Number of keys the event sort works on: the chunk's events padded to 4096 or 8192 (C W <= 8192).
__host__ __device__ inline int plan_sort_n(int CW) { return CW <= 4096 ? 4096 : 8192; }

constexpr int PLAN_HIST_BYTES = (PLAN_NT / 64) * 256 * 4;

// LDS layout of the plan kernel (16-byte aligned parts).
struct PlanLds {
  size_t keys, sslot, sev, pos, scode, sA, sB, kmask, qmask, rmask, roff, lev, loff, tot, hist, bytes;
  int kwm, qwm;  // 64-bit words per token of the K / Q term masks
};

__host__ __device__ inline PlanLds plan_lds(int C, int W, int R) {
  const size_t CW = (size_t)C * W;
  PlanLds L;
  size_t keys = (size_t)plan_sort_n((int)CW) * 8;           // sort keys; later write weights, then dense rows
  if ((size_t)C * C * 4 > keys) keys = (size_t)C * C * 4;
  L.kwm = (W + 63) / 64;
  L.qwm = (R + 63) / 64;
  size_t o = 0;
  L.keys = o;  o += align16((long long)keys);
  L.sslot = o; o += align16((long long)CW * 4);
  L.sev = o;   o += align16((long long)CW * 2);
  L.pos = o;   o += align16((long long)CW * 2);
  L.scode = o; o += align16((long long)CW * 2);
  L.sA = o;    o += align16((long long)C * 4);
  L.sB = o;    o += align16((long long)C * 4);
  L.kmask = o; o += align16((long long)C * L.kwm * 8);
  L.qmask = o; o += align16((long long)C * L.qwm * 8);
  L.rmask = o; o += align16((long long)C * 2 * 8);
  L.roff = o;  o += align16((long long)(C + 1) * 4);
  L.lev = o;   o += align16((long long)C * 4);
  L.loff = o;  o += align16((long long)(C + 2) * 4);
  L.tot = o;   o += align16(3 * 8 * 4 + 16);
  // radix sort: per-wave digit counts, then offsets (8 KiB); in the slot array, free during the sort, when it is
  // that large
  L.hist = CW * 4 >= (size_t)PLAN_HIST_BYTES ? L.sslot : o;
  if (CW * 4 < (size_t)PLAN_HIST_BYTES) o += PLAN_HIST_BYTES;
  L.bytes = o;
  return L;
}

__host__ __device__ inline size_t plan_lds_bytes(int C, int W, int R) { return plan_lds(C, W, R).bytes; }

// Orders this wave's LDS accesses before and after it (program order within one wave).
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ uint64_t lanes_below() {
  const int l = threadIdx.x & 63;
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_up(v, o, 64);
    if (lane >= o) v += x;
  }
  return v;
}

// Exclusive prefix sums of three per-thread counts over the workgroup (thread order); totals in t0..t2.
__device__ inline void block_excl_scan3(int& a, int& b, int& c, int* tot, int& t0, int& t1, int& t2) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ia = wave_incl_scan(a), ib = wave_incl_scan(b), ic = wave_incl_scan(c);
  if (lane == 63) {
    tot[wv] = ia;
    tot[8 + wv] = ib;
    tot[16 + wv] = ic;
  }
  __syncthreads();
  int ba = 0, bb = 0, bc = 0;
  t0 = t1 = t2 = 0;
  for (int w = 0; w < PLAN_NT / 64; ++w) {
    if (w < wv) {
      ba += tot[w];
      bb += tot[8 + w];
      bc += tot[16 + w];
    }
    t0 += tot[w];
    t1 += tot[8 + w];
    t2 += tot[16 + w];
  }
  a = ba + ia - a;
  b = bb + ib - b;
  c = bc + ic - c;
  __syncthreads();
}

// ------------------------------------------------------------------------------------------- event sort
// Bitonic sort of NS = 512 * EPT 64-bit keys (ascending) held in LDS. Wave w owns the contiguous block of
// BW = 64 * EPT keys [w BW, (w + 1) BW); lane l holds its keys j * 64 + l (j < EPT) in registers. Merge steps whose
// partner lies in the same lane run on registers, steps with partner distance < 64 on lane shuffles, and only the
// steps across wave blocks (distance >= BW) go through LDS with workgroup barriers (6 of the 78 steps for 4096 keys).

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
  const int lo = __shfl_xor((int)(uint32_t)x, m, 64);
  const int hi = __shfl_xor((int)(uint32_t)(x >> 32), m, 64);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// One merge step (block size SIZE, partner distance STRIDE < BW) on the lane's registers.
template <int EPT, int SIZE, int STRIDE>
__device__ __forceinline__ void sort_step_reg(uint64_t (&v)[EPT], int gbase, int lane) {
  if constexpr (STRIDE >= 64) {
    constexpr int S = STRIDE / 64;
    static_for<EPT>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      if constexpr ((j & S) == 0) {
        const bool up = ((gbase + j * 64) & SIZE) == 0;
        const uint64_t x = v[j], y = v[j | S];
        const bool sw = (x > y) == up;
        v[j] = sw ? y : x;
        v[j | S] = sw ? x : y;
      }
    });
  } else {
    const bool lower = (lane & STRIDE) == 0;
    static_for<EPT>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const uint64_t x = v[j];
      const uint64_t y = shfl_xor_u64(x, STRIDE);
      const bool up = ((gbase + j * 64 + lane) & SIZE) == 0;
      const bool keep_min = lower == up;
      const bool xl = x < y;
      v[j] = (keep_min == xl) ? x : y;
    });
  }
}

// All steps of block size SIZE with partner distance < BW, largest distance first.
template <int EPT, int SIZE, int LST>
__device__ __forceinline__ void sort_steps_reg(uint64_t (&v)[EPT], int gbase, int lane) {
  sort_step_reg<EPT, SIZE, (1 << LST)>(v, gbase, lane);
  if constexpr (LST > 0) sort_steps_reg<EPT, SIZE, LST - 1>(v, gbase, lane);
}

template <int N>
constexpr int ilog2() { return N <= 1 ? 0 : 1 + ilog2<N / 2>(); }

template <int EPT>
__device__ void sort_keys(uint64_t* keys) {
  constexpr int BW = 64 * EPT;
  constexpr int NS = BW * (PLAN_NT / 64);
  constexpr int LOG_BW = ilog2<BW>();
  constexpr int LOG_NS = ilog2<NS>();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int gbase = wv * BW;
  uint64_t v[EPT];
  static_for<EPT>([&](auto jc) { v[decltype(jc)::value] = keys[gbase + decltype(jc)::value * 64 + lane]; });
  // block sizes 2 .. BW: inside the wave
  static_for<LOG_BW>([&](auto a) {
    constexpr int lsz = decltype(a)::value + 1;
    sort_steps_reg<EPT, (1 << lsz), lsz - 1>(v, gbase, lane);
  });
  // block sizes 2 BW .. NS: distances >= BW through LDS, the rest in registers
  static_for<LOG_NS - LOG_BW>([&](auto a) {
    constexpr int lsz = LOG_BW + 1 + decltype(a)::value;
    constexpr int size = 1 << lsz;
    static_for<EPT>([&](auto jc) { keys[gbase + decltype(jc)::value * 64 + lane] = v[decltype(jc)::value]; });
    __syncthreads();
    for (int stride = size >> 1; stride >= BW; stride >>= 1) {
      for (int i = threadIdx.x; i < NS / 2; i += PLAN_NT) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t x = keys[lo], y = keys[hi];
        if ((x > y) == up) {
          keys[lo] = y;
          keys[hi] = x;
        }
      }
      __syncthreads();
    }
    static_for<EPT>([&](auto jc) { v[decltype(jc)::value] = keys[gbase + decltype(jc)::value * 64 + lane]; });
    sort_steps_reg<EPT, size, LOG_BW - 1>(v, gbase, lane);
  });
  __syncthreads();  // every wave has read its block before the sorted keys overwrite it
  static_for<EPT>([&](auto jc) { keys[gbase + decltype(jc)::value * 64 + lane] = v[decltype(jc)::value]; });
  __syncthreads();
}

// Stable LSD radix sort of the first E of NS = 512 * EPT 32-bit keys (slot << EB | event index) on their slot bits
// [EB, EB + sbits), 8-bit digits: the events come out ordered by (slot, event index), as the 64-bit bitonic sort
// orders them, in a fraction of its steps. Wave w takes keys [w BW, (w + 1) BW) in rows j of 64 (index
// w BW + j 64 + lane), the order a stable pass keeps: in each row a key's rank among equal digits comes from the
// digit bits' ballots, plus the wave's running count of that digit (the digit's lowest lane adds the row's count);
// an exclusive scan in (digit, wave) order then gives every (wave, digit) its first output index. loc: E entries of
// scratch for the keys' ranks within their wave and digit. Keys ping-pong between src and dst; returns the buffer
// holding the result.
template <int EPT>
__device__ uint32_t* radix_sort_keys(uint32_t* src, uint32_t* dst, uint16_t* loc, int* hist, int* tot, int E, int EB,
                                     int sbits) {
  constexpr int BW = 64 * EPT;
  constexpr int NWV = PLAN_NT / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint64_t below = lanes_below();
  int* wh = hist + wv * 256;
  for (int shift = EB; shift < EB + sbits; shift += 8) {
    const int bits = EB + sbits - shift < 8 ? EB + sbits - shift : 8;
    const uint32_t dmask = (1u << bits) - 1u;
    for (int i = lane; i < 256; i += 64) wh[i] = 0;
    wave_sync_lds();
#pragma unroll 1
    for (int j = 0; j < EPT; ++j) {
      const int i = wv * BW + j * 64 + lane;
      const bool real = i < E;
      const uint32_t d = (src[i] >> shift) & dmask;
      uint64_t m = __ballot(real);
      for (int b = 0; b < bits; ++b) {
        const uint64_t bb = __ballot((d >> b) & 1u);
        m &= ((d >> b) & 1u) ? bb : ~bb;
      }
      if (real) {
        const int cur = wh[d];
        loc[i] = (uint16_t)(cur + __popcll(m & below));
        if ((m & below) == 0ull) wh[d] = cur + __popcll(m);  // the digit's lowest lane in this row
      }
      wave_sync_lds();
    }
    __syncthreads();
    // first output index of every (wave, digit): digits in order, waves in order within a digit (threads 0..255
    // own the digits; the others read along and write nothing)
    {
      const int d = threadIdx.x & 255;
      int c[NWV], sum = 0;
#pragma unroll
      for (int w = 0; w < NWV; ++w) { c[w] = hist[w * 256 + d]; sum += c[w]; }
      const int incl = wave_incl_scan(sum);
      if (lane == 63 && threadIdx.x < 256) tot[wv] = incl;
      __syncthreads();
      if (threadIdx.x < 256) {
        int base = incl - sum;
        for (int w = 0; w < wv; ++w) base += tot[w];
#pragma unroll
        for (int w = 0; w < NWV; ++w) { hist[w * 256 + d] = base; base += c[w]; }
      }
    }
    __syncthreads();
#pragma unroll 1
    for (int j = 0; j < EPT; ++j) {
      const int i = wv * BW + j * 64 + lane;
      if (i < E) {
        const uint32_t k = src[i];
        dst[wh[(k >> shift) & dmask] + loc[i]] = k;
      }
    }
    __syncthreads();
    uint32_t* t = src; src = dst; dst = t;
  }
  return src;
}

// Lower bounds of Q slots j[q] in the sorted slots s[0..E) (E >= 1), the searches interleaved: every step halves the
// same range length for all of them (branch-free), so their LDS reads go out together.
template <int Q>
__device__ __forceinline__ void lower_bound_slots(const int32_t* s, int E, const int (&j)[Q], int (&out)[Q]) {
  int base[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) base[q] = 0;
  for (int n = E; n > 1;) {
    const int half = n >> 1;
#pragma unroll
    for (int q = 0; q < Q; ++q) base[q] = s[base[q] + half] < j[q] ? base[q] + half : base[q];
    n -= half;
  }
#pragma unroll
  for (int q = 0; q < Q; ++q) out[q] = base[q] + (s[base[q]] < j[q] ? 1 : 0);
}

// Lower bound of slot j in the sorted slots s[0..E).
__device__ __forceinline__ int lower_bound_slot(const int32_t* s, int E, int j) {
  int l = 0, r = E;
  while (l < r) {
    const int m = (l + r) >> 1;
    if (s[m] < j) l = m + 1; else r = m;
  }
  return l;
}

// Row-sorted sparse compaction of the dense rows 0..Cc-1 (columns 0..t of row t, C <= 128) into ptr / out; returns
// nnz. ptr[t] are absolute offsets (base + running count). Rows are counted with wave ballots (one wave per row),
// offset by a wave prefix sum, and emitted in column order. All threads call; ends with a barrier.
__device__ inline int compact_rows(const float* dense, int C, int Cc, uint64_t* rmask, int* roff, int* tot,
                                   int32_t* ptr, Ent* out, int base) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int t = wv; t < Cc; t += PLAN_NT / 64) {
    const bool nz0 = lane < C && lane <= t && dense[t * C + lane] != 0.0f;
    const bool nz1 = lane + 64 < C && lane + 64 <= t && dense[t * C + lane + 64] != 0.0f;
    const uint64_t m0 = __ballot(nz0), m1 = __ballot(nz1);
    if (lane == 0) {
      rmask[2 * t] = m0;
      rmask[2 * t + 1] = m1;
    }
  }
  __syncthreads();
  if (wv == 0) {  // row offsets: rows 2 lane and 2 lane + 1
    const int r0 = 2 * lane, r1 = 2 * lane + 1;
    const int c0 = r0 < Cc ? __popcll(rmask[2 * r0]) + __popcll(rmask[2 * r0 + 1]) : 0;
    const int c1 = r1 < Cc ? __popcll(rmask[2 * r1]) + __popcll(rmask[2 * r1 + 1]) : 0;
    const int incl = wave_incl_scan(c0 + c1);
    const int ex = incl - c0 - c1;
    if (r0 < Cc) { roff[r0] = ex; ptr[r0] = base + ex; }
    if (r1 < Cc) { roff[r1] = ex + c0; ptr[r1] = base + ex + c0; }
    if (lane == 63) { ptr[Cc] = base + incl; tot[0] = incl; }
  }
  __syncthreads();
  const int total = tot[0];
  const uint64_t below = lanes_below();
  for (int t = wv; t < Cc; t += PLAN_NT / 64) {
    const uint64_t m0 = rmask[2 * t], m1 = rmask[2 * t + 1];
    const int o = base + roff[t];
    if ((m0 >> lane) & 1) {
      Ent x;
      x.col = lane;
      x.val = dense[t * C + lane];
      out[o + __popcll(m0 & below)] = x;
    }
    if ((m1 >> lane) & 1) {
      Ent x;
      x.col = lane + 64;
      x.val = dense[t * C + lane + 64];
      out[o + __popcll(m0) + __popcll(m1 & below)] = x;
    }
  }
  __syncthreads();
  return total;
}

template <typename A>
__global__ __launch_bounds__(PLAN_NT) void plan_kernel(Dims D, PlanArgs a) {
  if (a.abort && *a.abort) return;  // shared-bank conflict: no work (uniform over the grid)
  extern __shared__ __align__(16) unsigned char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int st = blockIdx.y;
  const int ch = a.ch0 + blockIdx.x;
  const int b = st / D.H, h = st % D.H;
  const int W = D.W, R = D.R, C = D.C;
  const int t0 = ch * C;
  const int Cc = min(C, D.T - t0);
  const int E = Cc * W;
  const int NS = plan_sort_n(C * W);
  const long long cidx = (long long)st * D.nch + ch;
  const long long wbase = ((long long)st * D.T + t0) * W;  // [S][T][W] offset of the chunk's first event
  const long long rbase = ((long long)st * D.T + t0) * R;
  const ChunkLayout CL = chunk_layout(C, W, R);
  unsigned char* reg = a.chunks + cidx * CL.bytes;
  Pair* pw = (Pair*)(reg + CL.wpairs);
  Pair* pr = (Pair*)(reg + CL.rpairs);
  int16_t* wlast = (int16_t*)(reg + CL.wlast);
  int32_t* tptr = (int32_t*)(reg + CL.ptrs);
  int32_t* qptr = tptr + (C + 1);
  Ent* lists = (Ent*)(reg + CL.lists);
  Seg* segs = (Seg*)(reg + CL.scat);
  MSeg* msegs = (MSeg*)(reg + CL.multi);

  const PlanLds PL = plan_lds(C, W, R);
  uint64_t* keys = (uint64_t*)(lds + PL.keys);
  // after the sort: write weights in sorted event order, behind the dense rows when both fit in the sort keys'
  // area (then K and Q read them there instead of from global memory)
  const int swoff = (int)align16((long long)C * C * 4);
  const bool swkeep = swoff + (long long)C * W * 4 <= (long long)NS * 8;
  float* sw = (float*)(lds + PL.keys + (swkeep ? swoff : 0));
  float* dense = (float*)(lds + PL.keys);  // after the segments: K, T, Q rows
  int32_t* sslot = (int32_t*)(lds + PL.sslot);
  uint16_t* sev = (uint16_t*)(lds + PL.sev);
  uint16_t* pos = (uint16_t*)(lds + PL.pos);
  int16_t* scode = (int16_t*)(lds + PL.scode);  // last-event code per sorted event
  float* sA = (float*)(lds + PL.sA);
  float* sB = (float*)(lds + PL.sB);
  unsigned long long* kmask = (unsigned long long*)(lds + PL.kmask);
  unsigned long long* qmask = (unsigned long long*)(lds + PL.qmask);
  uint64_t* rmask = (uint64_t*)(lds + PL.rmask);
  int* roff = (int*)(lds + PL.roff);
  int* lev = (int*)(lds + PL.lev);
  int* loff = (int*)(lds + PL.loff);
  int* tot = (int*)(lds + PL.tot);

  // 1. write events -> sort keys (slot, event index); gates of the chunk; empty term masks. Slot and event index
  //    packed in 32 bits when they fit (radix sort), else 64-bit keys (bitonic sort).
  const int EB = NS == 4096 ? 12 : 13;
  const int SB = D.N > 1 ? 64 - __clzll((unsigned long long)(D.N - 1)) : 1;  // bits of the largest slot
  const bool radix = SB + EB <= 32;
  uint32_t* keys32 = (uint32_t*)keys;
  for (int e = tid; e < NS; e += PLAN_NT) {
    if (radix) {
      keys32[e] = e < E ? ((uint32_t)a.widx[wbase + e] << EB) | (uint32_t)e : ~0u;
    } else {
      uint64_t key = ~0ull;
      if (e < E) key = ((uint64_t)(uint32_t)a.widx[wbase + e] << 32) | (uint32_t)e;
      keys[e] = key;
    }
  }
  for (int t = tid; t < C; t += PLAN_NT) {
    float al = 1.0f, be = 0.0f;
    if (t < Cc) {
      const long long g = ((long long)b * D.T + t0 + t) * D.H + h;
      al = to_f<A>(((const A*)a.alpha)[g]);
      be = to_f<A>(((const A*)a.beta)[g]);
    }
    sA[t] = al;
    sB[t] = be;
  }
  for (int i = tid; i < C * PL.kwm; i += PLAN_NT) kmask[i] = 0ull;
  for (int i = tid; i < C * PL.qwm; i += PLAN_NT) qmask[i] = 0ull;
  __syncthreads();
  if (radix) {
    const uint32_t* sorted = NS == 4096
        ? radix_sort_keys<8>(keys32, keys32 + NS, pos, (int*)(lds + PL.hist), tot, E, EB, SB)
        : radix_sort_keys<16>(keys32, keys32 + NS, pos, (int*)(lds + PL.hist), tot, E, EB, SB);
    for (int e = tid; e < E; e += PLAN_NT) {
      const uint32_t k = sorted[e];
      const uint32_t ev = k & ((1u << EB) - 1u);
      sslot[e] = (int32_t)(k >> EB);
      sev[e] = (uint16_t)ev;
      pos[ev] = (uint16_t)e;
    }
  } else {
    if (NS == 4096) sort_keys<8>(keys); else sort_keys<16>(keys);
    for (int e = tid; e < E; e += PLAN_NT) {
      const uint64_t k = keys[e];
      sslot[e] = (int32_t)(k >> 32);
      sev[e] = (uint16_t)(k & 0xFFFF);
      pos[k & 0xFFFF] = (uint16_t)e;
    }
  }
  __syncthreads();
  {  // write weights in sorted event order (loads issued together: the flat loads may not pass the LDS stores)
    constexpr int GB = 8;
    for (int e0 = tid; e0 < E; e0 += PLAN_NT * GB) {
      float wv8[GB];
      static_for<GB>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        wv8[k] = a.wwt[wbase + sev[min(e0 + k * PLAN_NT, E - 1)]];
      });
      static_for<GB>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        if (e0 + k * PLAN_NT < E) sw[e0 + k * PLAN_NT] = wv8[k];
      });
    }
  }

  // 2. segments (runs of equal slots) and the multi-event table: ids by a workgroup prefix sum over contiguous
  //    ranges of the sorted events.
  const int per = (E + PLAN_NT - 1) / PLAN_NT;
  const int lo = min(E, tid * per), hi = min(E, lo + per);
  int g0 = 0, m0 = 0, me0 = 0, nseg = 0, nmseg = 0, nmev = 0;
  {
    for (int e = lo; e < hi; ++e) {
      const bool first = e == 0 || sslot[e] != sslot[e - 1];
      const bool multi = !first || (e + 1 < E && sslot[e + 1] == sslot[e]);
      g0 += first;
      m0 += first && multi;
      me0 += multi;
    }
    block_excl_scan3(g0, m0, me0, tot, nseg, nmseg, nmev);  // includes barriers (sw visible after it)
  }
  if (tid == 0) {
    ChunkCounts cc;
    cc.nnzT = cc.nnzQ = 0;
    cc.nseg = nseg;
    cc.nev = E;
    cc.nmseg = nmseg;
    cc.nmev = nmev;
    cc.pad0 = cc.pad1 = 0;
    a.counts[cidx] = cc;
  }
  Ev* ev = (Ev*)(segs + nseg);
  Ev* mev = (Ev*)(msegs + nmseg);
  {
    int g = g0 - 1;   // segment id of the element before lo
    int m = m0 - 1;   // multi-event segment id of the element before lo
    int me = me0;     // next multi-event event slot
    for (int e = lo; e < hi; ++e) {
      const bool first = e == 0 || sslot[e] != sslot[e - 1];
      const bool last = e == E - 1 || sslot[e + 1] != sslot[e];
      const bool multi = !(first && last);
      if (first) {
        ++g;
        if (a.scat) segs[g].slot = sslot[e];
        if (multi) {
          ++m;
          msegs[m].slot = sslot[e];
          msegs[m].beg = me;
          msegs[m].pad = 0;
        }
      }
      if (last && a.scat) segs[g].end = e + 1;
      const int evi = sev[e];
      Ev x;
      x.w = sw[e];
      x.tok = evi / W;
      if (a.evcode) x.tok |= (evi % W) << 16;
      if (a.scat) ev[e] = x;
      if (multi) {
        mev[me++] = x;
        if (last) msegs[m].end = me;
      }
      scode[e] = (int16_t)(!last ? -1 : (multi ? m : -2));
    }
  }
  __syncthreads();

  // 3. write-gather terms (slot, a_ti), one thread per term; terms meeting an earlier event of their slot are
  //    flagged. Then K (dense rows): one thread per token adds its flagged terms' contributions in term order.
  for (int i = tid; i < C * C; i += PLAN_NT) dense[i] = 0.0f;
  {
    constexpr int GB = 8;
    for (int v0 = tid; v0 < E; v0 += PLAN_NT * GB) {
      float wt8[GB];
      static_for<GB>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        wt8[k] = a.wwt[wbase + min(v0 + k * PLAN_NT, E - 1)];
      });
      static_for<GB>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        const int evi = v0 + k * PLAN_NT;
        if (evi < E) {
          const int e = pos[evi];
          const int slot = sslot[e];
          float prod = 1.0f;
          bool has = false;
          for (int e2 = e - 1; e2 >= 0 && sslot[e2] == slot; --e2) {
            prod *= sA[sev[e2] / W];
            has = true;
          }
          Pair p;
          p.slot = slot;
          p.coef = wt8[k] * prod;
          pw[term_pos(evi / W, evi % W, W, a.lanemajor)] = p;
          wlast[code_pos(evi / W, evi % W, W, a.lanemajor)] = scode[e];
          if (has) {
            const int t = evi / W, i = evi % W;
            atomicOr(&kmask[t * PL.kwm + (i >> 6)], 1ull << (i & 63));
          }
        }
      });
    }
  }
  __syncthreads();
  for (int t = tid; t < Cc; t += PLAN_NT) {
    for (int wd = 0; wd < PL.kwm; ++wd) {
      uint64_t mk = kmask[t * PL.kwm + wd];
      while (mk) {
        const int i = wd * 64 + __ffsll((unsigned long long)mk) - 1;
        mk &= mk - 1;
        const int evi = t * W + i;
        const int e = pos[evi];
        const int slot = sslot[e];
        const float wt = swkeep ? sw[e] : a.wwt[wbase + evi];
        float prod = 1.0f;
        for (int e2 = e - 1; e2 >= 0 && sslot[e2] == slot; --e2) {
          const int s = sev[e2] / W;
          dense[t * C + s] += wt * (swkeep ? sw[e2] : a.wwt[wbase + sev[e2]]) * prod;
          prod *= sA[s];
        }
      }
    }
  }
  __syncthreads();

  // 4. L = diag(alpha beta) K (unit diagonal) with the nonzero mask of each row (one wave per row), then
  //    T = (I + L)^-1 in place by forward substitution, rows grouped by dependency level (a row after every row it
  //    uses): one wave per row (lane s holds columns s and s + 64), summing over the row's nonzero entries in
  //    increasing order.
  for (int t = wv; t < Cc; t += PLAN_NT / 64) {
    const float ab = sA[t] * sB[t];
    bool nz0 = false, nz1 = false;
    if (lane < C) {
      float& x = dense[t * C + lane];
      if (lane < t) { x *= ab; nz0 = x != 0.0f; }
      else if (lane == t) x = 1.0f;
    }
    if (lane + 64 < C) {
      float& x = dense[t * C + lane + 64];
      if (lane + 64 < t) { x *= ab; nz1 = x != 0.0f; }
      else if (lane + 64 == t) x = 1.0f;
    }
    const uint64_t m0 = __ballot(nz0), m1 = __ballot(nz1);
    if (lane == 0) {
      rmask[2 * t] = m0;
      rmask[2 * t + 1] = m1;
    }
  }
  __syncthreads();
  // levels of the rows' dependency graph (row t needs the rows of its mask): wave 0, lane l holds rows l, l + 64
  if (wv == 0) {
    const int r0 = lane, r1 = lane + 64;
    const uint64_t a0 = r0 < Cc ? rmask[2 * r0] : 0ull, a1 = r0 < Cc ? rmask[2 * r0 + 1] : 0ull;
    const uint64_t b0 = r1 < Cc ? rmask[2 * r1] : 0ull, b1 = r1 < Cc ? rmask[2 * r1 + 1] : 0ull;
    if (r0 < C) lev[r0] = 0;
    if (r1 < C) lev[r1] = 0;
    wave_sync_lds();
    for (int it = 0; it < C; ++it) {  // Jacobi sweeps: converges in (depth + 1) sweeps
      int n0 = 0, n1 = 0;
      for (int half = 0; half < 2; ++half) {
        uint64_t m = half ? a1 : a0;
        while (m) {
          const int c = half * 64 + __ffsll((unsigned long long)m) - 1;
          m &= m - 1;
          n0 = max(n0, lev[c] + 1);
        }
        m = half ? b1 : b0;
        while (m) {
          const int c = half * 64 + __ffsll((unsigned long long)m) - 1;
          m &= m - 1;
          n1 = max(n1, lev[c] + 1);
        }
      }
      const bool changed = (r0 < C && n0 != lev[r0]) || (r1 < C && n1 != lev[r1]);
      wave_sync_lds();
      if (r0 < C) lev[r0] = n0;
      if (r1 < C) lev[r1] = n1;
      wave_sync_lds();
      if (__ballot(changed) == 0ull) break;
    }
    const int l0 = r0 < Cc ? lev[r0] : 0, l1 = r1 < Cc ? lev[r1] : 0;
    int maxlev = max(l0, l1);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) maxlev = max(maxlev, __shfl_xor(maxlev, o, 64));
    // rows of each level in increasing order: list roff[loff[v] .. loff[v + 1])
    const uint64_t below = lanes_below();
    int base = 0;
    for (int v = 1; v <= maxlev; ++v) {
      const uint64_t q0 = __ballot(l0 == v && r0 < Cc), q1 = __ballot(l1 == v && r1 < Cc);
      if (l0 == v && r0 < Cc) roff[base + __popcll(q0 & below)] = r0;
      if (l1 == v && r1 < Cc) roff[base + __popcll(q0) + __popcll(q1 & below)] = r1;
      if (lane == 0) loff[v] = base;
      base += __popcll(q0) + __popcll(q1);
    }
    if (lane == 0) {
      loff[maxlev + 1] = base;
      tot[0] = maxlev;
    }
  }
  __syncthreads();
  const int nlev = tot[0];
  for (int v = 1; v <= nlev; ++v) {  // rows of one level are independent: one wave per row
    for (int k = loff[v] + wv; k < loff[v + 1]; k += PLAN_NT / 64) {
      const int t = roff[k];
      const uint64_t mk0 = rmask[2 * t], mk1 = rmask[2 * t + 1];
      float acc0 = 0.0f, acc1 = 0.0f;
      for (int half = 0; half < 2; ++half) {
        uint64_t mk = half ? mk1 : mk0;
        while (mk) {
          const int m = half * 64 + __ffsll((unsigned long long)mk) - 1;
          mk &= mk - 1;
          const float l = dense[t * C + m];
          if (lane <= m) acc0 += l * dense[m * C + lane];
          if (lane + 64 <= m) acc1 += l * dense[m * C + lane + 64];
        }
      }
      wave_sync_lds();
      if (lane < t) dense[t * C + lane] = -acc0;
      if (lane + 64 < t) dense[t * C + lane + 64] = -acc1;
    }
    __syncthreads();
  }
  // read-gather terms (slot, b_ti), one thread per term, flagging the terms that meet an earlier write of their slot
  {
    constexpr int QB = 4;  // read terms per thread per batch (their loads issued together)
    const int nth = PLAN_NT;
    const int nx = Cc * R;
    for (int x0 = tid; x0 < nx; x0 += nth * QB) {
      int jj[QB];
      float rr[QB];
      static_for<QB>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        const int x = min(x0 + k * nth, nx - 1);
        jj[k] = a.ridx[rbase + x];
        rr[k] = a.rwt[rbase + x];
      });
      int lbs[QB];
      lower_bound_slots<QB>(sslot, E, jj, lbs);
      static_for<QB>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        const int x = x0 + k * nth;
        if (x < nx) {
          const int t = x / R;
          const int j = jj[k];
          const int l = lbs[k];
          float prod = 1.0f;
          if (l < E && sslot[l] == j && sev[l] / W <= t) {
            int e1 = l;
            while (e1 + 1 < E && sslot[e1 + 1] == j && sev[e1 + 1] / W <= t) ++e1;
            for (int e2 = e1; e2 >= l; --e2) prod *= sA[sev[e2] / W];
            const int i = x % R;
            atomicOr(&qmask[t * PL.qwm + (i >> 6)], 1ull << (i & 63));
          }
          Pair p;
          p.slot = j;
          p.coef = rr[k] * prod;
          pr[term_pos(t, x % R, R, a.lanemajor)] = p;
        }
      });
    }
  }
  __syncthreads();
  const int nnzT = compact_rows(dense, C, Cc, rmask, roff, tot, tptr, lists, 0);

  // 5. Q (dense rows): one thread per token adds its flagged read terms' contributions in term order.
  for (int i = tid; i < C * C; i += PLAN_NT) dense[i] = 0.0f;
  __syncthreads();
  for (int t = tid; t < Cc; t += PLAN_NT) {
    for (int wd = 0; wd < PL.qwm; ++wd) {
      uint64_t mk = qmask[t * PL.qwm + wd];
      while (mk) {
        const int i = wd * 64 + __ffsll((unsigned long long)mk) - 1;
        mk &= mk - 1;
        const long long x = (long long)t * R + i;
        const int j = a.ridx[rbase + x];
        const float rho = a.rwt[rbase + x];
        const int l = lower_bound_slot(sslot, E, j);
        int e1 = l;
        while (e1 + 1 < E && sslot[e1 + 1] == j && sev[e1 + 1] / W <= t) ++e1;
        float prod = 1.0f;
        for (int e2 = e1; e2 >= l; --e2) {
          const int s = sev[e2] / W;
          dense[t * C + s] += rho * (swkeep ? sw[e2] : a.wwt[wbase + sev[e2]]) * prod;
          prod *= sA[s];
        }
      }
    }
  }
  __syncthreads();
  const int nnzQ = compact_rows(dense, C, Cc, rmask, roff, tot, qptr, lists, nnzT);
  if (tid == 0) {
    a.counts[cidx].nnzT = nnzT;
    a.counts[cidx].nnzQ = nnzQ;
  }
}

hipError_t launch_plan(const Dims& D, const PlanArgs& a, hipStream_t st) {
  if (D.S == 0 || D.T == 0) return hipSuccess;
  const size_t lds = plan_lds_bytes(D.C, D.W, D.R);
  dim3 grid((unsigned)(a.chn ? a.chn : D.nch), (unsigned)D.S);
  if (D.act == SDM_BF16) {
    (void)hipFuncSetAttribute((const void*)plan_kernel<bf16_t>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(plan_kernel<bf16_t>, grid, dim3(PLAN_NT), lds, st, D, a);
  } else {
    (void)hipFuncSetAttribute((const void*)plan_kernel<float>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(plan_kernel<float>, grid, dim3(PLAN_NT), lds, st, D, a);
  }
  return hipGetLastError();
}

}  // namespace sdm
