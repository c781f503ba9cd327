// Single-token decode step, after the step's exact top-k (the wave-level top-k kernel, one query per wave): the
// gated delta-rule update of the W write rows and the read of the R read rows. One workgroup per (stream, 64-byte
// column slice); its 64 lane groups of 4 lanes hold one row slice each (16 bytes per lane), so a step spreads over
// streams x slices workgroups.
//
// Successor bank (lumen PR #29, "Donating is a permission, not a demand"): bank_out == bank_in writes the successor
// in place; a distinct bank_out first receives a copy of bank_in (launch_copy, same stream) and then the same body
// runs: rows are read from bank_in before any row is written, the W updated rows are stored into bank_out, and
// the read takes its rows from bank_out. Both forms therefore execute identical arithmetic on identical values
// and produce identical bits. Per-token work is O((W + R) d) as in the pages' cost model; the copy is O(N d).
#include "sdm_internal.h"
#include "topk_device.h"
#include "topk_wave.h"

namespace sdm {

template <typename Bk> struct DLane;
template <> struct DLane<float> {
  static constexpr int EPL = 4;
  __device__ static void load(const float* p, float* v) {
    const float4 x = *(const float4*)p;
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  }
  __device__ static void store(float* p, const float* v) { *(float4*)p = make_float4(v[0], v[1], v[2], v[3]); }
};
template <> struct DLane<bf16_t> {
  static constexpr int EPL = 8;
  __device__ static void load(const bf16_t* p, float* v) {
    const uint4 x = *(const uint4*)p;
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  __device__ static void store(bf16_t* p, const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f_to_bf16(v[2 * i]) | ((uint32_t)f_to_bf16(v[2 * i + 1]) << 16);
    *(uint4*)p = make_uint4(w[0], w[1], w[2], w[3]);
  }
};


// Sums the 64 lane groups' partial rows in a fixed order: each wave's 16 groups in order into part4[wave], then
// (by the caller) the 4 wave sums in order. Starts and ends with a barrier.
template <int COLS>
__device__ __forceinline__ void reduce_groups(float (*part)[COLS], float (*part4)[COLS]) {
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid < 4 * COLS) {
    const int w = tid / COLS, c = tid % COLS;
    float s = 0.0f;
    for (int gg = 16 * w; gg < 16 * w + 16; ++gg) s += part[gg][c];
    part4[w][c] = s;
  }
  __syncthreads();
}

// RPG = rows per lane group (W, R <= 64 RPG).
template <typename A, typename Bk, int RPG>
__global__ __launch_bounds__(DECODE_NT) void decode_update_kernel(Dims D, DecodeArgs a) {
  constexpr int EPL = DLane<Bk>::EPL;
  constexpr int COLS = 4 * EPL;
  constexpr int NG = DECODE_NT / 4;
  __shared__ float part[NG][COLS];
  __shared__ float part4[DECODE_NT / 64][COLS];
  __shared__ float sdel[COLS];
  const int tid = threadIdx.x;
  const int g = tid >> 2, q = tid & 3;
  const int st = blockIdx.y;  // stream b * H + h; with one token the [B, 1, H] row index equals st
  const int col0 = blockIdx.x * COLS;
  const int col = col0 + q * EPL;
  const bool valid = col < D.d;
  const long long rowsd = D.rows * D.ld;
  const Bk* bin = (const Bk*)a.bank_in + (long long)st * rowsd;
  Bk* bout = (Bk*)a.bank_out + (long long)st * rowsd;
  const int32_t* wid = a.wid + (long long)st * D.W;
  const float* wwt = a.wwt + (long long)st * D.W;
  const int32_t* rid = a.rid + (long long)st * D.R;
  const float* rwt = a.rwt + (long long)st * D.R;
  const float al = to_f<A>(((const A*)a.alpha)[st]);
  const float be = to_f<A>(((const A*)a.beta)[st]);

  // r = sum_i w_i M[S_i]: group g takes rows g, g + 64, ... (kept in registers for the update)
  float m[RPG][EPL];
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int u = 0; u < RPG; ++u) {
    const int i = g + NG * u;
    if (valid && i < D.W) DLane<Bk>::load(bin + (long long)wid[i] * D.ld + col, m[u]);
  }
#pragma unroll
  for (int u = 0; u < RPG; ++u) {
    const int i = g + NG * u;
    if (valid && i < D.W) {
      const float wi = wwt[i];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] += wi * m[u][e];
    }
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) part[g][q * EPL + e] = acc[e];
  reduce_groups<COLS>(part, part4);
  if (tid < COLS && col0 + tid < D.d) {  // delta = beta (v - alpha r)
    const float r = part4[0][tid] + part4[1][tid] + part4[2][tid] + part4[3][tid];
    sdel[tid] = be * (to_f<A>(((const A*)a.values)[(long long)st * D.d + col0 + tid]) - al * r);
  }
  __syncthreads();
  // M[S_i] <- alpha M[S_i] + w_i delta, rounded to the bank dtype, into the successor
#pragma unroll
  for (int u = 0; u < RPG; ++u) {
    const int i = g + NG * u;
    if (valid && i < D.W) {
      const float wi = wwt[i];
      float y[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) y[e] = al * m[u][e] + wi * sdel[q * EPL + e];
      DLane<Bk>::store(bout + (long long)wid[i] * D.ld + col, y);
    }
  }
  __syncthreads();  // the updated rows are visible to the read below
  // out = sum_i rho_i M'[R_i], read from the successor after the write
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
#pragma unroll
  for (int u = 0; u < RPG; ++u) {
    const int i = g + NG * u;
    if (valid && i < D.R) DLane<Bk>::load(bout + (long long)rid[i] * D.ld + col, m[u]);
  }
#pragma unroll
  for (int u = 0; u < RPG; ++u) {
    const int i = g + NG * u;
    if (valid && i < D.R) {
      const float ri = rwt[i];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] += ri * m[u][e];
    }
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) part[g][q * EPL + e] = acc[e];
  reduce_groups<COLS>(part, part4);
  if (tid < COLS && col0 + tid < D.d) {
    const float o = part4[0][tid] + part4[1][tid] + part4[2][tid] + part4[3][tid];
    ((A*)a.out)[(long long)st * D.d + col0 + tid] = from_f<A>(o);
  }
}

template <typename A, typename Bk, int RPG>
static void launch_decode_r(const Dims& D, const DecodeArgs& a, hipStream_t st) {
  constexpr int COLS = 4 * DLane<Bk>::EPL;
  dim3 grid((unsigned)((D.d + COLS - 1) / COLS), (unsigned)D.S);
  hipLaunchKernelGGL((decode_update_kernel<A, Bk, RPG>), grid, dim3(DECODE_NT), 0, st, D, a);
}

template <typename A, typename Bk>
static hipError_t launch_decode_t(const Dims& D, const DecodeArgs& a, hipStream_t st) {
  const int rows = D.W > D.R ? D.W : D.R;  // <= MAX_K = 512
  if (rows <= 64) launch_decode_r<A, Bk, 1>(D, a, st);
  else if (rows <= 128) launch_decode_r<A, Bk, 2>(D, a, st);
  else if (rows <= 256) launch_decode_r<A, Bk, 4>(D, a, st);
  else launch_decode_r<A, Bk, 8>(D, a, st);
  return hipGetLastError();
}

hipError_t launch_decode(const Dims& D, const DecodeArgs& a, hipStream_t st) {
  if (D.S == 0) return hipSuccess;
  if (D.act == SDM_BF16)
    return D.bank == SDM_BF16 ? launch_decode_t<bf16_t, bf16_t>(D, a, st) : launch_decode_t<bf16_t, float>(D, a, st);
  return D.bank == SDM_BF16 ? launch_decode_t<float, bf16_t>(D, a, st) : launch_decode_t<float, float>(D, a, st);
}

// ------------------------------------------------------------------------------------------- one-launch step
// The step in one workgroup per stream (b, h): the block builds both candidate tables in LDS, the four waves
// score and select the factors of both queries, waves 0 and 1 merge them into the write and read top-k, then all
// four waves gather, update and read the rows in
// column passes of 64 lanes x 16 bytes: wave w takes write rows and read rows w, w + 4, ... (W, R <= 64). All row
// loads of a pass come from bank_in and complete before any row of the pass is written; a read row whose slot is
// also written this step is updated in registers with the same arithmetic and rounding as the stored row, so the
// read sees the successor's values (write then read, as the per-token recurrence) and a donated step equals a
// copied one bit for bit. r and out are summed per wave in row order, then over the waves in order.
struct StepLds {
  uint64_t* ctab[2];
  int* offs[2];
  float* fsc[2];
  uint16_t* fid[2];
  uint64_t* scratch[4];  // per wave
  uint64_t* sorted[4];
  int32_t *wid, *rid, *rmatch;
  float *wwt, *rwt;
  float* part;  // [2][4][64 EPL]: the waves' partial sums of r, then of out
  size_t bytes;
};

__host__ __device__ inline StepLds step_lds(unsigned char* base, const Dims& D, const TopkPlan* P, int epl) {
  StepLds L;
  size_t o = 0;
  auto take = [&](size_t b) {
    unsigned char* p = base + o;
    o = (o + b + 15) & ~(size_t)15;
    return p;
  };
  int KS = 0;
  for (int q = 0; q < 2; ++q) {
    L.ctab[q] = (uint64_t*)take((size_t)P[q].ncand * 8);
    L.offs[q] = (int*)take((size_t)(P[q].kp[0] + 1) * 4);
    L.fsc[q] = (float*)take((size_t)D.F * P[q].kpmax * 4);
    L.fid[q] = (uint16_t*)take((size_t)D.F * P[q].kpmax * 2);
    const int ks = P[q].kpmax > P[q].k ? P[q].kpmax : P[q].k;
    KS = ks > KS ? ks : KS;
  }
  for (int w = 0; w < 4; ++w) {
    L.scratch[w] = (uint64_t*)take((size_t)(KS + MERGE_RB) * 8);
    L.sorted[w] = (uint64_t*)take((size_t)KS * 8);
  }
  L.wid = (int32_t*)take((size_t)D.W * 4);
  L.wwt = (float*)take((size_t)D.W * 4);
  L.rid = (int32_t*)take((size_t)D.R * 4);
  L.rwt = (float*)take((size_t)D.R * 4);
  L.rmatch = (int32_t*)take((size_t)D.R * 4);
  L.part = (float*)take((size_t)2 * 4 * 64 * epl * 4);
  L.bytes = o;
  return L;
}

// A 16-byte row piece (EPL elements of the bank dtype) as floats.
template <typename Bk> __device__ __forceinline__ void piece_unpack(const w16_t& x, float* v);
template <> __device__ __forceinline__ void piece_unpack<float>(const w16_t& x, float* v) {
  v[0] = __uint_as_float(x.x); v[1] = __uint_as_float(x.y); v[2] = __uint_as_float(x.z); v[3] = __uint_as_float(x.w);
}
template <> __device__ __forceinline__ void piece_unpack<bf16_t>(const w16_t& x, float* v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(x[i] << 16);
    v[2 * i + 1] = __uint_as_float(x[i] & 0xFFFF0000u);
  }
}

constexpr int STEP_NT = 256;
constexpr int STEP_RPW = 16;  // rows of each kind per wave: W, R <= 64

// The rows of one step of one stream, after its top-k (L: ids, weights; rmatch and part are scratch): every wave
// gathers write rows and read rows w, w + 4, ... (W, R <= 64) of a column pass of 64 lanes x 16 bytes from bin, all
// of a pass's loads complete before any row of the pass is written; r = sum_i w_i M[S_i] per wave in row order,
// then over the waves in order; delta = beta (v - alpha r); the updated write rows go to bout (rounded to the bank
// dtype); a read row whose slot is also written this step is updated in registers with the same arithmetic and
// rounding, so the read sees the successor; out = sum_j rho_j M'[R_j] per wave, then over the waves. values and
// out point at the stream-row's d elements. Starts after a barrier that made L visible; every wave calls it.
template <typename A, typename Bk>
__device__ __forceinline__ void step_rows(const Dims& D, const StepLds& L, const Bk* bin, Bk* bout, const A* values,
                                          A* out, float al, float be) {
  constexpr int EPL = DLane<Bk>::EPL;
  constexpr int COLW = 64 * EPL;
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  float* part = L.part;
  for (int c0 = 0; c0 < D.d; c0 += COLW) {
    const int col = c0 + lane * EPL;
    const bool valid = col < D.d;
    // the value piece first (used after the barrier below; loaded now so that its latency hides behind the rows)
    float va[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) va[e] = valid ? to_f<A>(values[col + e]) : 0.0f;
    w16_t wr[STEP_RPW], rr[STEP_RPW];
    static_for<STEP_RPW>([&](auto u) {
      const int i = wv + 4 * u;
      wr[u] = w16_t{0u, 0u, 0u, 0u};
      if (valid && i < D.W) wr[u] = *(const w16_t*)(bin + (long long)L.wid[i] * D.ld + col);
    });
    static_for<STEP_RPW>([&](auto u) {
      const int j = wv + 4 * u;
      rr[u] = w16_t{0u, 0u, 0u, 0u};
      if (valid && j < D.R) rr[u] = *(const w16_t*)(bin + (long long)L.rid[j] * D.ld + col);
    });
    if (c0 == 0) {
      // while the rows load: read slots that are also written this step (the slots of one top-k are distinct);
      // read slot j is compared with the write slots by the 4 consecutive threads 4 j .. 4 j + 3, each scanning a
      // quarter, then combined. Read after the barrier below, in the output.
      for (int j0 = 0; j0 < D.R; j0 += STEP_NT / 4) {
        const int j = j0 + (tid >> 2), qt = tid & 3;
        const int s = j < D.R ? L.rid[j] : -1;
        int mi = -1;
        for (int i = qt; i < D.W; i += 4) mi = L.wid[i] == s ? i : mi;
        mi = max(mi, __shfl_xor(mi, 1, 64));
        mi = max(mi, __shfl_xor(mi, 2, 64));
        if (qt == 0 && j < D.R) L.rmatch[j] = mi;
      }
    }
    // r = sum_i w_i M[S_i]: this wave's rows in order
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
    static_for<STEP_RPW>([&](auto u) {
      const int i = wv + 4 * u;
      if (i < D.W) {
        const float wi = L.wwt[i];
        float m[EPL];
        piece_unpack<Bk>(wr[u], m);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += wi * m[e];
      }
    });
#pragma unroll
    for (int e = 0; e < EPL; ++e) part[wv * COLW + lane * EPL + e] = acc[e];
    // every read row of this pass has arrived before the barrier, so no row written below can reach it
#pragma unroll
    for (int u = 0; u < STEP_RPW; ++u) asm volatile("" ::"v"(rr[u]));
    __syncthreads();
    // delta = beta (v - alpha r) for this lane's columns (the same in every wave)
    float dl[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int c = lane * EPL + e;
      const float r = part[c] + part[COLW + c] + part[2 * COLW + c] + part[3 * COLW + c];
      dl[e] = valid ? be * (va[e] - al * r) : 0.0f;
    }
    // M[S_i] <- alpha M[S_i] + w_i delta, rounded to the bank dtype, into the successor
    static_for<STEP_RPW>([&](auto u) {
      const int i = wv + 4 * u;
      if (valid && i < D.W) {
        const float wi = L.wwt[i];
        float m[EPL];
        piece_unpack<Bk>(wr[u], m);
        float y[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) y[e] = fmaf(wi, dl[e], al * m[e]);
        DLane<Bk>::store(bout + (long long)L.wid[i] * D.ld + col, y);
      }
    });
    // out = sum_j rho_j M'[R_j], M' the successor (rows written this step updated as above)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
    static_for<STEP_RPW>([&](auto u) {
      const int j = wv + 4 * u;
      if (j < D.R) {
        float m[EPL];
        piece_unpack<Bk>(rr[u], m);
        const int mi = L.rmatch[j];
        if (mi >= 0) {
          const float wi = L.wwt[mi];
#pragma unroll
          for (int e = 0; e < EPL; ++e) m[e] = bank_round<Bk>(fmaf(wi, dl[e], al * m[e]));
        }
        const float rj = L.rwt[j];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += rj * m[e];
      }
    });
    float* opart = part + 4 * COLW;  // a second buffer: no barrier needed between reading r's parts and this
#pragma unroll
    for (int e = 0; e < EPL; ++e) opart[wv * COLW + lane * EPL + e] = acc[e];
    __syncthreads();
    if (wv == 0 && valid) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int c = lane * EPL + e;
        const float o = opart[c] + opart[COLW + c] + opart[2 * COLW + c] + opart[3 * COLW + c];
        out[col + e] = from_f<A>(o);
      }
    }
    if (c0 + COLW < D.d) __syncthreads();  // the partial sums are reused by the next pass
  }
}

template <typename A, typename Bk, int NPL, int CPL>
__global__ __launch_bounds__(STEP_NT) void decode_step_kernel(Dims D, DecodeArgs a) {
  constexpr int EPL = DLane<Bk>::EPL;
  extern __shared__ __align__(16) unsigned char lds[];
  const StepLds L = step_lds(lds, D, a.plan, EPL);
  // the wave index as a scalar: plan fields picked by wave then load as scalar loads (a vector load of them would
  // queue behind the sub-key loads issued early below and wait for them)
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int st = blockIdx.x;  // stream b * H + h; with one token the [B, 1, H] row index equals st
  const int h = st % D.H;
  // (members picked by kind or wave with conditionals, not indexed: a runtime index into a struct's array puts the
  // struct in scratch memory)
  auto pick2 = [](auto x0, auto x1, int i) { return i ? x1 : x0; };
  auto pick4 = [](auto x0, auto x1, auto x2, auto x3, int i) { return i < 2 ? (i ? x1 : x0) : (i == 2 ? x2 : x3); };
  // factor top-k of both queries: task kind * F + f on wave task % 4. Each wave issues the loads of its first
  // task's first block now; they arrive while the candidate tables are built.
  long long sumn = 0;
  for (int f = 0; f < D.F; ++f) sumn += D.widths[f];
  const A* subh = (const A*)a.subkeys + (long long)h * sumn * D.dk;
  auto task_in = [&](int task, int* f, const A** qv, const A** tab) {
    const int kind = task / D.F;
    *f = task % D.F;
    long long off = 0;
    for (int g = 0; g < *f; ++g) off += D.widths[g];
    *qv = (const A*)pick2(a.queries[0], a.queries[1], kind) + (long long)st * D.F * D.dk;
    *tab = subh + off * D.dk;
  };
  FactorBlock<A, NPL> fb;
  if (wv < 2 * D.F) {
    int f;
    const A *qv, *tab;
    task_in(wv, &f, &qv, &tab);
    factor_load<A, NPL>(D, f, qv, tab, 0, fb);
  }
  // candidate tables: threads 0-127 build the write table, 128-255 the read table (small tables: waves 0 and 2)
  {
    const int kind = wv >> 1, t = tid & 127;
    const TopkPlan& P = kind ? a.plan[1] : a.plan[0];
    if (cand_one_wave(a.plan[0], D.F) && cand_one_wave(a.plan[1], D.F)) {
      if (t < 64) cand_table_wave(P, pick2(L.ctab[0], L.ctab[1], kind), lane);
    } else {
      cand_offsets(P, D.F, pick2(L.offs[0], L.offs[1], kind), t, 128);
      __syncthreads();
      cand_emit(P, D.F, pick2(L.offs[0], L.offs[1], kind), pick2(L.ctab[0], L.ctab[1], kind), t, 128);
    }
  }
  uint64_t* wscr = pick4(L.scratch[0], L.scratch[1], L.scratch[2], L.scratch[3], wv);
  uint64_t* wsrt = pick4(L.sorted[0], L.sorted[1], L.sorted[2], L.sorted[3], wv);
  for (int task = wv; task < 2 * D.F; task += 4) {
    const int kind = task / D.F;
    int f;
    const A *qv, *tab;
    task_in(task, &f, &qv, &tab);
    if (task != wv) factor_load<A, NPL>(D, f, qv, tab, 0, fb);
    const TopkPlan& P = kind ? a.plan[1] : a.plan[0];
    wave_factor_topk<A, NPL>(D, P, f, qv, tab, pick2(L.fsc[0], L.fsc[1], kind), pick2(L.fid[0], L.fid[1], kind),
                             wscr, wsrt, fb);
  }
  __syncthreads();  // factor lists and candidate tables complete
  if (wv < 2) {  // merges: wave 0 the write query, wave 1 the read query
    const int kind = wv;
    const TopkPlan& P = kind ? a.plan[1] : a.plan[0];
    int32_t* ids = kind ? L.rid : L.wid;
    // (no lower-bound prefilter here: at one step's latency its compaction costs more than the smaller select saves;
    // 128 streams, 32 x 32 sub-keys: 9.2 k cycles with it, 7.9 k without)
    wave_merge_topk<CPL>(D, P, pick2(L.ctab[0], L.ctab[1], kind), pick2(L.fsc[0], L.fsc[1], kind),
                         pick2(L.fid[0], L.fid[1], kind), wscr, wsrt, ids, kind ? L.rwt : L.wwt);
    int32_t* uid = pick2(a.user_ids[0], a.user_ids[1], kind);
    if (uid)
      for (int r = lane; r < P.k; r += 64) uid[(long long)st * P.k + r] = ids[r];
  }
  __syncthreads();
  const float al = to_f<A>(((const A*)a.alpha)[st]);
  const float be = to_f<A>(((const A*)a.beta)[st]);
  const long long rowsd = D.rows * D.ld;
  step_rows<A, Bk>(D, L, (const Bk*)a.bank_in + (long long)st * rowsd, (Bk*)a.bank_out + (long long)st * rowsd,
                   (const A*)a.values + (long long)st * D.d, (A*)a.out + (long long)st * D.d, al, be);
}

static void step_shape(const Dims& D, const DecodeArgs& a, int* npl, int* cpl) {
  int nfmax = 0;
  for (int f = 0; f < D.F; ++f) nfmax = D.widths[f] > nfmax ? D.widths[f] : nfmax;
  *npl = 1;
  while (*npl * 64 < nfmax) *npl <<= 1;
  const int nc = a.plan[0].ncand > a.plan[1].ncand ? a.plan[0].ncand : a.plan[1].ncand;
  *cpl = nc <= 256 ? 4 : nc <= 512 ? 8 : 16;
}

bool decode_step_fits(const Dims& D, const DecodeArgs& a) {
  int npl, cpl;
  step_shape(D, a, &npl, &cpl);
  const int epl = D.bank == SDM_BF16 ? 8 : 4;
  if (npl > 4 || D.W > 4 * STEP_RPW || D.R > 4 * STEP_RPW) return false;
  for (int q = 0; q < 2; ++q)
    if (a.plan[q].ncand > 64 * cpl || a.plan[q].kpmax > 1024) return false;
  const int esz = D.act == SDM_BF16 ? 2 : 4;
  if ((D.dk * esz) % 16 != 0 || ((uintptr_t)a.subkeys) % 16 != 0) return false;
  if (((uintptr_t)a.queries[0]) % 16 != 0 || ((uintptr_t)a.queries[1]) % 16 != 0) return false;
  return step_lds(nullptr, D, a.plan, epl).bytes <= 64 * 1024;
}

template <typename A, typename Bk, int NPL, int CPL>
static void launch_step_k(const Dims& D, const DecodeArgs& a, size_t lds, hipStream_t st) {
  (void)hipFuncSetAttribute((const void*)decode_step_kernel<A, Bk, NPL, CPL>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL((decode_step_kernel<A, Bk, NPL, CPL>), dim3((unsigned)D.S), dim3(STEP_NT), lds, st, D, a);
}

template <typename A, typename Bk>
static hipError_t launch_step_t(const Dims& D, const DecodeArgs& a, hipStream_t st) {
  int npl, cpl;
  step_shape(D, a, &npl, &cpl);
  const size_t lds = step_lds(nullptr, D, a.plan, DLane<Bk>::EPL).bytes;
  auto go = [&](auto nplc) {
    constexpr int NPL = decltype(nplc)::value;
    if (cpl == 4) launch_step_k<A, Bk, NPL, 4>(D, a, lds, st);
    else if (cpl == 8) launch_step_k<A, Bk, NPL, 8>(D, a, lds, st);
    else launch_step_k<A, Bk, NPL, 16>(D, a, lds, st);
  };
  if (npl == 1) go(std::integral_constant<int, 1>{});
  else if (npl == 2) go(std::integral_constant<int, 2>{});
  else go(std::integral_constant<int, 4>{});
  return hipGetLastError();
}

hipError_t launch_decode_step(const Dims& D, const DecodeArgs& a, hipStream_t st) {
  if (D.S == 0) return hipSuccess;
  if (D.act == SDM_BF16)
    return D.bank == SDM_BF16 ? launch_step_t<bf16_t, bf16_t>(D, a, st) : launch_step_t<bf16_t, float>(D, a, st);
  return D.bank == SDM_BF16 ? launch_step_t<float, bf16_t>(D, a, st) : launch_step_t<float, float>(D, a, st);
}

// ------------------------------------------------------------------------------------------- multi-step decode
// K consecutive decode steps of every stream in one launch, after the batched top-k of all K tokens (ids and
// float32 slot scores, row-major [B, K, H, k]; the top-k reads no bank, so all K run in parallel beforehand). One
// workgroup per stream runs its K steps in order: per step, waves 0 and 1 form the write and read weights exactly
// as the one-launch step does (wave_rank_softmax on the same scores), then step_rows. Step k + 1 reads the rows
// step k wrote (every wave waits for its own stores, then a barrier), so the result is K one-launch steps, bit for
// bit (the same arithmetic on the same values in the same order).
__host__ __device__ inline StepLds steps_lds(unsigned char* base, const Dims& D, int epl) {
  StepLds L = {};  // only the fields the steps kernel uses are set
  size_t o = 0;
  auto take = [&](size_t b) {
    unsigned char* p = base + o;
    o = (o + b + 15) & ~(size_t)15;
    return p;
  };
  L.wid = (int32_t*)take((size_t)D.W * 4);
  L.wwt = (float*)take((size_t)D.W * 4);
  L.rid = (int32_t*)take((size_t)D.R * 4);
  L.rwt = (float*)take((size_t)D.R * 4);
  L.rmatch = (int32_t*)take((size_t)D.R * 4);
  L.part = (float*)take((size_t)2 * 4 * 64 * epl * 4);
  L.bytes = o;
  return L;
}

template <typename A, typename Bk>
__global__ __launch_bounds__(STEP_NT) void decode_steps_kernel(Dims D, DecodeArgs a, int K) {
  extern __shared__ __align__(16) unsigned char lds[];
  const StepLds L = steps_lds(lds, D, DLane<Bk>::EPL);
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int st = blockIdx.x, b = st / D.H, h = st % D.H;
  const long long rowsd = D.rows * D.ld;
  const Bk* bin = (const Bk*)a.bank_in + (long long)st * rowsd;
  Bk* bout = (Bk*)a.bank_out + (long long)st * rowsd;
  // waves 0 and 1 hold the next step's write / read ids and scores in registers (lane r: rank r; k <= 64), loaded
  // one step ahead so that their latency hides behind the current step's rows
  const int kk = wv ? D.R : D.W;
  const int32_t* gid = wv ? a.rid : a.wid;
  const float* gsc = wv ? a.rwt : a.wwt;
  int32_t nid = 0;
  float nsc = 0.0f;
  auto fetch = [&](int k) {
    const long long row = ((long long)b * K + k) * D.H + h;
    if (wv < 2 && lane < kk) {
      nid = gid[row * kk + lane];
      nsc = gsc[row * kk + lane];
    }
  };
  fetch(0);
  for (int k = 0; k < K; ++k) {
    const long long row = ((long long)b * K + k) * D.H + h;
    if (wv < 2) {  // wave 0: the write ids and weights, wave 1: the read ones
      int32_t* ids = wv ? L.rid : L.wid;
      int32_t* uid = wv ? a.user_ids[1] : a.user_ids[0];
      if (lane < kk) {
        ids[lane] = nid;
        if (uid) uid[row * kk + lane] = nid;
      }
      const float s0 = __shfl(nsc, 0, 64);
      const float mine = nsc;
      wave_rank_softmax(kk, [&](int r) { return r == 0 ? s0 : mine; }, wv ? L.rwt : L.wwt);
      if (k + 1 < K) fetch(k + 1);
    }
    __syncthreads();
    const float al = to_f<A>(((const A*)a.alpha)[row]);
    const float be = to_f<A>(((const A*)a.beta)[row]);
    step_rows<A, Bk>(D, L, k == 0 ? bin : bout, bout, (const A*)a.values + row * D.d, (A*)a.out + row * D.d, al, be);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's row stores have completed before any wave reads them next step
    __syncthreads();
  }
}

template <typename A, typename Bk>
static hipError_t launch_steps_t(const Dims& D, const DecodeArgs& a, int K, hipStream_t st) {
  const size_t lds = steps_lds(nullptr, D, DLane<Bk>::EPL).bytes;
  hipLaunchKernelGGL((decode_steps_kernel<A, Bk>), dim3((unsigned)D.S), dim3(STEP_NT), lds, st, D, a, K);
  return hipGetLastError();
}

hipError_t launch_decode_steps(const Dims& D, const DecodeArgs& a, int K, hipStream_t st) {
  if (D.S == 0 || K == 0) return hipSuccess;
  if (D.act == SDM_BF16)
    return D.bank == SDM_BF16 ? launch_steps_t<bf16_t, bf16_t>(D, a, K, st) : launch_steps_t<bf16_t, float>(D, a, K, st);
  return D.bank == SDM_BF16 ? launch_steps_t<float, bf16_t>(D, a, K, st) : launch_steps_t<float, float>(D, a, K, st);
}

__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const uint4*)src, (uint4*)dst, n);
  return hipGetLastError();
}

}  // namespace sdm
