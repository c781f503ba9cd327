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
// events. T is solved in IEEE float32 by forward substitution, row after row. Every sum runs in a fixed order
// (bitwise repeatable; no atomics).
#include "sdm_internal.h"

namespace sdm {

__host__ __device__ inline size_t plan_lds_bytes(int C, int W) {
  const size_t CW = (size_t)C * W;
  size_t keys = (size_t)pow2_ceil((int)CW) * 8;
  const size_t dense = (size_t)C * C * 4;
  if (dense > keys) keys = dense;
  return keys + CW * 4 /*sslot*/ + CW * 2 /*sev*/ + CW * 2 /*pos*/ + (size_t)C * 12 /*alpha, beta, flags*/ +
         (size_t)PLAN_NT * 4 * 3 /*scans*/ + 16;
}

// Row-sorted sparse compaction of the dense rows 0..Cc-1 (columns 0..t for row t) into ptr / out; returns nnz.
// ptr[t] are absolute offsets (base + running count). All threads call; ends with a barrier.
__device__ inline int compact_rows(const float* dense, int C, int Cc, int* scan, int32_t* ptr, Ent* out, int base) {
  const int tid = threadIdx.x;
  for (int t = tid; t < Cc; t += PLAN_NT) {
    int n = 0;
    for (int s = 0; s <= t; ++s) n += dense[t * C + s] != 0.0f;
    scan[t] = n;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int t = 0; t < Cc; ++t) {
      const int c = scan[t];
      scan[t] = run;
      ptr[t] = base + run;
      run += c;
    }
    ptr[Cc] = base + run;
    scan[PLAN_NT - 1] = run;
  }
  __syncthreads();
  const int total = scan[PLAN_NT - 1];
  for (int t = tid; t < Cc; t += PLAN_NT) {
    int o = base + scan[t];
    for (int s = 0; s <= t; ++s) {
      const float v = dense[t * C + s];
      if (v != 0.0f) {
        Ent x;
        x.col = s;
        x.val = v;
        out[o++] = x;
      }
    }
  }
  __syncthreads();
  return total;
}

template <typename A>
__global__ __launch_bounds__(PLAN_NT) void plan_kernel(Dims D, PlanArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int tid = threadIdx.x;
  const int st = blockIdx.y;
  const int ch = blockIdx.x;
  const int b = st / D.H, h = st % D.H;
  const int W = D.W, R = D.R, C = D.C;
  const int t0 = ch * C;
  const int Cc = min(C, D.T - t0);
  const int E = Cc * W;
  const int Ep2 = pow2_ceil(E);
  const long long CW = (long long)C * W;
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

  size_t keys_bytes = (size_t)pow2_ceil((int)CW) * 8;
  if ((size_t)C * C * 4 > keys_bytes) keys_bytes = (size_t)C * C * 4;
  uint64_t* keys = (uint64_t*)lds;
  float* dense = (float*)lds;
  int32_t* sslot = (int32_t*)(lds + keys_bytes);
  uint16_t* sev = (uint16_t*)(sslot + CW);
  uint16_t* pos = sev + CW;
  float* sA = (float*)(pos + CW + (CW & 1));
  float* sB = sA + C;
  int32_t* sHasL = (int32_t*)(sB + C);
  int32_t* scan = sHasL + C;
  int32_t* scanM = scan + PLAN_NT;   // multi-event segment starts per thread range
  int32_t* scanE = scanM + PLAN_NT;  // multi-event events per thread range
  __shared__ int s_nseg, s_nmseg;
  MSeg* msegs = (MSeg*)(reg + CL.multi);

  // 1. write events -> sort keys (slot, event index); gates of the chunk.
  for (int e = tid; e < Ep2; e += PLAN_NT) {
    uint64_t key = ~0ull;
    if (e < E) key = ((uint64_t)(uint32_t)a.widx[wbase + e] << 32) | (uint32_t)e;
    keys[e] = key;
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
    sHasL[t] = 0;
  }
  __syncthreads();
  bitonic_sort_u64<PLAN_NT>(keys, Ep2);
  for (int e = tid; e < E; e += PLAN_NT) {
    const uint64_t k = keys[e];
    sslot[e] = (int32_t)(k >> 32);
    sev[e] = (uint16_t)(k & 0xFFFF);
    pos[k & 0xFFFF] = (uint16_t)e;
  }
  __syncthreads();

  // 2. segments (runs of equal slots) and the multi-event table: ids by block scans over contiguous ranges.
  const int per = (E + PLAN_NT - 1) / PLAN_NT;
  const int lo = min(E, tid * per), hi = min(E, lo + per);
  {
    int cnt = 0, cm = 0, ce = 0;
    for (int e = lo; e < hi; ++e) {
      const bool first = e == 0 || sslot[e] != sslot[e - 1];
      const bool multi = !first || (e + 1 < E && sslot[e + 1] == sslot[e]);
      cnt += first;
      cm += first && multi;
      ce += multi;
    }
    scan[tid] = cnt;
    scanM[tid] = cm;
    scanE[tid] = ce;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0, rm = 0, re = 0;
    for (int i = 0; i < PLAN_NT; ++i) {
      const int c = scan[i], m = scanM[i], x = scanE[i];
      scan[i] = run;
      scanM[i] = rm;
      scanE[i] = re;
      run += c;
      rm += m;
      re += x;
    }
    ChunkCounts cc;
    cc.nnzT = cc.nnzQ = 0;
    cc.nseg = run;
    cc.nev = E;
    cc.nmseg = rm;
    cc.nmev = re;
    cc.pad0 = cc.pad1 = 0;
    a.counts[cidx] = cc;
    s_nseg = run;
    s_nmseg = rm;
  }
  __syncthreads();
  const int nseg = s_nseg;
  Ev* ev = (Ev*)(segs + nseg);
  Ev* mev = (Ev*)(msegs + s_nmseg);
  {
    int g = scan[tid] - 1;   // segment id of the element before lo
    int m = scanM[tid] - 1;  // multi-event segment id of the element before lo
    int me = scanE[tid];     // next multi-event event slot
    for (int e = lo; e < hi; ++e) {
      const bool first = e == 0 || sslot[e] != sslot[e - 1];
      const bool last = e == E - 1 || sslot[e + 1] != sslot[e];
      const bool multi = !(first && last);
      if (first) {
        ++g;
        segs[g].slot = sslot[e];
        if (multi) {
          ++m;
          msegs[m].slot = sslot[e];
          msegs[m].beg = me;
          msegs[m].pad = 0;
        }
      }
      if (last) segs[g].end = e + 1;
      const int evi = sev[e];
      Ev x;
      x.w = a.wwt[wbase + evi];
      x.tok = evi / W;
      ev[e] = x;
      if (multi) {
        mev[me++] = x;
        if (last) msegs[m].end = me;
      }
      wlast[evi] = (int16_t)(!last ? -1 : (multi ? m : -2));
    }
  }
  __syncthreads();

  // 3. K (dense rows in LDS) and the write-gather terms (slot, a_ti); one thread per token, events in order.
  for (int i = tid; i < C * C; i += PLAN_NT) dense[i] = 0.0f;
  __syncthreads();
  for (int t = tid; t < Cc; t += PLAN_NT) {
    int has = 0;
    for (int i = 0; i < W; ++i) {
      const int evi = t * W + i;
      const int e = pos[evi];
      const int slot = sslot[e];
      const float wt = a.wwt[wbase + evi];
      float prod = 1.0f;
      for (int e2 = e - 1; e2 >= 0 && sslot[e2] == slot; --e2) {
        const int s = sev[e2] / W;
        dense[t * C + s] += wt * a.wwt[wbase + sev[e2]] * prod;
        prod *= sA[s];
        has = 1;
      }
      Pair p;
      p.slot = slot;
      p.coef = wt * prod;
      pw[evi] = p;
    }
    sHasL[t] = has;
  }
  __syncthreads();

  // 4. T = (I + L)^-1 with L = diag(alpha beta) K, in place, row after row (IEEE float32).
  for (int i = tid; i < Cc * C; i += PLAN_NT) {
    const int t = i / C, s = i % C;
    if (s < t) dense[i] *= sA[t] * sB[t];
    else if (s == t) dense[i] = 1.0f;
  }
  __syncthreads();
  for (int t = 1; t < Cc; ++t) {
    if (!sHasL[t]) continue;  // row t of T is e_t
    const int s = tid;
    float acc = 0.0f;
    if (s < t) {
      for (int m = s; m < t; ++m) {
        const float l = dense[t * C + m];
        if (l != 0.0f) acc += l * dense[m * C + s];
      }
    }
    __syncthreads();
    if (s < t) dense[t * C + s] = -acc;
    __syncthreads();
  }
  const int nnzT = compact_rows(dense, C, Cc, scan, tptr, lists, 0);

  // 5. Q (dense rows) and the read-gather terms (slot, b_ti).
  for (int i = tid; i < C * C; i += PLAN_NT) dense[i] = 0.0f;
  __syncthreads();
  for (int t = tid; t < Cc; t += PLAN_NT) {
    for (int i = 0; i < R; ++i) {
      const int j = a.ridx[rbase + (long long)t * R + i];
      const float rho = a.rwt[rbase + (long long)t * R + i];
      int l = 0, r = E;  // lower bound of j in sslot
      while (l < r) {
        const int m = (l + r) >> 1;
        if (sslot[m] < j) l = m + 1; else r = m;
      }
      float prod = 1.0f;
      if (l < E && sslot[l] == j && sev[l] / W <= t) {
        int e1 = l;
        while (e1 + 1 < E && sslot[e1 + 1] == j && sev[e1 + 1] / W <= t) ++e1;
        for (int e2 = e1; e2 >= l; --e2) {
          const int s = sev[e2] / W;
          dense[t * C + s] += rho * a.wwt[wbase + sev[e2]] * prod;
          prod *= sA[s];
        }
      }
      Pair p;
      p.slot = j;
      p.coef = rho * prod;
      pr[(long long)t * R + i] = p;
    }
  }
  __syncthreads();
  const int nnzQ = compact_rows(dense, C, Cc, scan, qptr, lists, nnzT);
  if (tid == 0) {
    a.counts[cidx].nnzT = nnzT;
    a.counts[cidx].nnzQ = nnzQ;
  }
}

hipError_t launch_plan(const Dims& D, const PlanArgs& a, hipStream_t st) {
  if (D.S == 0 || D.T == 0) return hipSuccess;
  const size_t lds = plan_lds_bytes(D.C, D.W);
  dim3 grid((unsigned)D.nch, (unsigned)D.S);
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
