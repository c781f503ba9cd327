// The serial chunk loop: bank gather, delta solve, read output and in-order segmented scatter.
//
// Column slices of the bank are independent (every coefficient comes from the bank-independent plan), so one
// workgroup owns one (stream, 64-byte column slice) pair and runs every chunk of its stream in order with no
// synchronisation beyond its own barriers. Per chunk (notation of plan.hip):
//   A  gather  H[t] = sum_i a_ti M_0[S_ti],  G[t] = sum_i b_ti M_0[R_ti]     (HBM: W + R row slices per token)
//   B  solve   U_t = beta_t v_t - alpha_t beta_t H[t];  delta_t = sum_s T_ts U_s      (T from the plan)
//   C  read    out_t = G[t] + sum_s Q_ts delta_s                             (act dtype)
//   D  scatter per written slot j, its events in token order: M[j] <- alpha_s M[j] + w_sj delta_s, one read and
//              one write of the row slice (HBM: W row slices per token); a bfloat16 row is rounded after every
//              event, as the per-token recurrence stores it (bank_round)
// A group of 4 lanes moves one 64-byte row slice (16 bytes per lane). In phase A each group accumulates one token's
// terms in order (no cross-lane reduction), with its row loads back to back. Blocks are mapped so that
// neighbouring column slices of a stream run on the same XCD and share its L2 (a 128-byte L2 line holds two
// 64-byte slices).
//
// Two variants: STAGED copies each chunk's plan region into LDS in batched coalesced passes (gather terms and
// lists before A, the scatter part before D); the direct variant reads it from global memory (used when the
// region does not fit in LDS, e.g. chunk 128). Every global load stream is issued in batches so that many loads
// are in flight per lane.
#include "sdm_internal.h"

namespace sdm {

template <typename Bk> struct Lane;
template <> struct Lane<float> {
  static constexpr int EPL = 4;
  __device__ static void load(const float* p, float* v) {
    const float4 x = *(const float4*)p;
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  }
  __device__ static void store(float* p, const float* v) { *(float4*)p = make_float4(v[0], v[1], v[2], v[3]); }
  __device__ static void unpack(const uint4& x, float* v) {
    v[0] = __uint_as_float(x.x); v[1] = __uint_as_float(x.y); v[2] = __uint_as_float(x.z); v[3] = __uint_as_float(x.w);
  }
};
template <> struct Lane<bf16_t> {
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
  __device__ static void unpack(const uint4& x, float* v) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};

constexpr int PREF = 8;  // uint4 per thread of register prefetch (64 KiB per 512-thread block)

__host__ __device__ inline size_t loop_region_lds(int C, int W, int R) {
  const ChunkLayout CL = chunk_layout(C, W, R);
  const long long r1 = CL.wpairs_bytes + CL.wlast_bytes + CL.rpairs_bytes + CL.ptrs_bytes + CL.lists_cap;
  return (size_t)(r1 > CL.scat_cap ? r1 : CL.scat_cap);
}

__host__ __device__ inline size_t loop_lds_bytes(int C, int W, int R, int cols, bool staged) {
  size_t n = (size_t)C * cols * 4 * 3 + (size_t)C * 8;
  if (staged) n = align16(n) + loop_region_lds(C, W, R);
  return n;
}

template <typename A, typename Bk, bool STAGED>
__global__ __launch_bounds__(LOOP_NT) void loop_kernel(Dims D, LoopArgs a, int nslices) {
  if (a.abort && *a.abort) return;  // shared-bank conflict: no work (uniform over the grid)
  constexpr int EPL = Lane<Bk>::EPL;
  constexpr int COLS = 4 * EPL;  // columns per 64-byte slice
  constexpr int NW = LOOP_NT / 64;
  extern __shared__ __align__(16) unsigned char lds[];
  const int C = D.C, W = D.W, R = D.R;
  float* sH = (float*)lds;              // [C][COLS]  H, then U
  float* sG = sH + C * COLS;            // [C][COLS]
  float* sD = sG + C * COLS;            // [C][COLS]  delta
  float* sA = sD + C * COLS;            // [C]
  float* sB = sA + C;                   // [C]
  unsigned char* sReg = lds + align16((long long)C * COLS * 4 * 3 + (long long)C * 8);

  // XCD-aware mapping: blocks b, b+8, b+16, ... run on one XCD; give them consecutive work units.
  const int nblk = gridDim.x;
  int w = blockIdx.x;
  if ((nblk & 7) == 0) w = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int st = w / nslices, slice = w % nslices;
  const int b = st / D.H, h = st % D.H;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int q = lane & 3, grp = lane >> 2;  // 16 groups of 4 lanes per wave
  const int col0 = slice * COLS;
  const int mycol = col0 + q * EPL;
  const bool valid = mycol < D.d;
  const long long rowsd = D.rows * D.ld;
  Bk* bank = (Bk*)a.bank + bank_of(D, st) * rowsd;
  const A* alpha = (const A*)a.alpha;
  const A* beta = (const A*)a.beta;
  const A* values = (const A*)a.values;
  A* out = (A*)a.out;
  const ChunkLayout CL = chunk_layout(C, W, R);
  const long long CW = (long long)C * W;

  const int ch1 = a.ch1 ? a.ch1 : D.nch;  // chunks [a.ch0, ch1)
  ChunkCounts cnt = a.counts[(long long)st * D.nch + a.ch0];
  for (int ch = a.ch0; ch < ch1; ++ch) {
    const int t0 = ch * C;
    const int Cc = min(C, D.T - t0);
    const long long cidx = (long long)st * D.nch + ch;
    const unsigned char* greg = a.chunks + cidx * CL.bytes;
    const ChunkCounts next = a.counts[ch + 1 < ch1 ? cidx + 1 : cidx];
    // region pointers (LDS copy or global)
    const unsigned char* reg = greg;
    if (STAGED) {
      const int n16 =
          (int)((CL.lists + (long long)(cnt.nnzT + cnt.nnzQ) * 8 + 15) >> 4);
      const uint4* src = (const uint4*)greg;
      uint4* dst = (uint4*)sReg;
      for (int i0 = 0; i0 < n16; i0 += LOOP_NT * PREF) {  // batches of PREF loads per thread in flight
        uint4 tmp[PREF];
#pragma unroll
        for (int k = 0; k < PREF; ++k) tmp[k] = src[min(i0 + tid + k * LOOP_NT, n16 - 1)];  // clamped: in bounds
#pragma unroll
        for (int k = 0; k < PREF; ++k) {
          const int i = i0 + tid + k * LOOP_NT;
          if (i < n16) dst[i] = tmp[k];
        }
      }
      reg = sReg;
    }
    for (int t = tid; t < Cc; t += LOOP_NT) {
      const long long g = ((long long)b * D.T + t0 + t) * D.H + h;
      sA[t] = to_f<A>(alpha[g]);
      sB[t] = to_f<A>(beta[g]);
    }
    if (STAGED) __syncthreads();
    const Pair* pw = (const Pair*)(reg + CL.wpairs);
    const Pair* pr = (const Pair*)(reg + CL.rpairs);
    const int32_t* tptr = (const int32_t*)(reg + CL.ptrs);
    const int32_t* qptr = tptr + (C + 1);
    const Ent* lists = (const Ent*)(reg + CL.lists);

    // value rows of this chunk and slice (bank-independent): loaded now, used in B
    constexpr int VPT = (128 * COLS + LOOP_NT - 1) / LOOP_NT;  // per thread, chunk <= 128
    float vreg[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int idx = tid + k * LOOP_NT;
      const int t = idx / COLS, c = idx % COLS;
      vreg[k] = 0.0f;
      if (t < Cc && col0 + c < D.d) {
        const long long g = ((long long)b * D.T + t0 + t) * D.H + h;
        vreg[k] = to_f<A>(values[g * D.d + col0 + c]);
      }
    }
    // A: gathers. Waves 0..3 take the write terms (H), waves 4..7 the read terms (G); group = token.
    {
      const int kind = wv >> 2;
      const int n = kind ? R : W;
      const Pair* base = kind ? pr : pw;
      float* dst = kind ? sG : sH;
      for (int t = (wv & 3) * 16 + grp; t < Cc; t += 64) {
        float acc[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
        if (valid) {
          const Pair* pp = base + (long long)t * n;
          constexpr int GB = 12;  // row loads in flight per lane
          for (int i0 = 0; i0 < n; i0 += GB) {
            uint4 raw[GB];
            float cf[GB];
#pragma unroll
            for (int u = 0; u < GB; ++u) {
              const int i = i0 + u;
              cf[u] = 0.0f;
              if (i < n) {
                const Pair p = pp[i];
                cf[u] = p.coef;
                raw[u] = *(const uint4*)(bank + (long long)p.slot * D.ld + mycol);
              }
            }
#pragma unroll
            for (int u = 0; u < GB; ++u) {
              if (i0 + u < n) {
                float v[EPL];
                Lane<Bk>::unpack(raw[u], v);
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[e] += cf[u] * v[e];
              }
            }
          }
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) dst[t * COLS + q * EPL + e] = acc[e];
      }
    }
    const int s16 = (int)(((long long)(cnt.nseg + cnt.nev) * 8 + 15) >> 4);
    __syncthreads();
    // B: U = beta v - alpha beta H (in place), then delta = T U.
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int idx = tid + k * LOOP_NT;
      const int t = idx / COLS, c = idx % COLS;
      if (t < Cc && col0 + c < D.d) sH[idx] = sB[t] * vreg[k] - sA[t] * sB[t] * sH[idx];
    }
    __syncthreads();
    for (int idx = tid; idx < Cc * COLS; idx += LOOP_NT) {
      const int t = idx / COLS, c = idx % COLS;
      float d = 0.0f;
      for (int e = tptr[t]; e < tptr[t + 1]; ++e) d += lists[e].val * sH[lists[e].col * COLS + c];
      sD[idx] = d;
    }
    __syncthreads();
    // C: read output.
    for (int idx = tid; idx < Cc * COLS; idx += LOOP_NT) {
      const int t = idx / COLS, c = idx % COLS;
      if (col0 + c < D.d) {
        float o = sG[idx];
        for (int e = qptr[t]; e < qptr[t + 1]; ++e) o += lists[e].val * sD[lists[e].col * COLS + c];
        const long long g = ((long long)b * D.T + t0 + t) * D.H + h;
        out[g * D.d + col0 + c] = from_f<A>(o);
      }
    }
    // D: in-order segmented scatter, one 64-byte row slice per group of 4 lanes.
    const Seg* segs = (const Seg*)(greg + CL.scat);
    if (STAGED) {
      __syncthreads();  // the LDS region is reused
      uint4* dst = (uint4*)sReg;
      const uint4* src = (const uint4*)(greg + CL.scat);
      for (int i0 = 0; i0 < s16; i0 += LOOP_NT * PREF) {
        uint4 tmp[PREF];
#pragma unroll
        for (int k = 0; k < PREF; ++k) tmp[k] = src[min(i0 + tid + k * LOOP_NT, s16 - 1)];
#pragma unroll
        for (int k = 0; k < PREF; ++k) {
          const int i = i0 + tid + k * LOOP_NT;
          if (i < s16) dst[i] = tmp[k];
        }
      }
      __syncthreads();
      segs = (const Seg*)sReg;
    }
    const Ev* ev = (const Ev*)(segs + cnt.nseg);
    // snapshot rows of this stream's chunk: row (t, i) = [t * W + i] * d
    Bk* snap = a.snap ? (Bk*)a.snap + ((long long)st * D.T + t0) * D.W * D.d + mycol : nullptr;
    if (valid) {
      constexpr int UB = 8;
      for (int sg0 = wv * 16 + grp; sg0 < cnt.nseg; sg0 += NW * 16 * UB) {
        float m[UB][EPL];
        int beg[UB], end[UB];
        Bk* p[UB];
#pragma unroll
        for (int u = 0; u < UB; ++u) {
          const int sg = sg0 + u * NW * 16;
          beg[u] = end[u] = 0;
          p[u] = nullptr;
          if (sg < cnt.nseg) {
            const Seg sgm = segs[sg];
            beg[u] = sg > 0 ? segs[sg - 1].end : 0;
            end[u] = sgm.end;
            p[u] = bank + (long long)sgm.slot * D.ld + mycol;
            Lane<Bk>::load(p[u], m[u]);
          }
        }
#pragma unroll
        for (int u = 0; u < UB; ++u) {
          if (p[u]) {
            for (int e = beg[u]; e < end[u]; ++e) {
              const Ev x = ev[e];
              const int tk = x.tok & 0xFFFF;
              if (snap) Lane<Bk>::store(snap + ((long long)tk * D.W + (x.tok >> 16)) * D.d, m[u]);
              const float al = sA[tk];
#pragma unroll
              for (int k = 0; k < EPL; ++k) m[u][k] = bank_round<Bk>(al * m[u][k] + x.w * sD[tk * COLS + q * EPL + k]);
            }
            Lane<Bk>::store(p[u], m[u]);
          }
        }
      }
    }
    cnt = next;
    __syncthreads();
  }
}

// Word 3 of a raw buffer resource on gfx9 (32-bit data format, no swizzle, offsets in bytes).
constexpr int BUF_RSRC_WORD3 = 0x00020000;
// A byte offset past every buffer range used here (ranges are kept below it): an access there is dropped by the
// hardware range check (a store writes nothing), also with 16 or 32 bytes added.
constexpr uint32_t BUF_OOB = 0xFFFFFF00u;

// EPL activation elements of a row as raw words (one 16- or 32-byte load), converted to floats later.
template <typename A, int EPL>
struct ActRaw {
  static constexpr int NW = (EPL * (int)sizeof(A) + 15) / 16;
  static_assert(EPL * sizeof(A) == 16 || EPL * sizeof(A) == 32 || EPL * sizeof(A) == 8, "row piece of 8, 16 or 32 bytes");
  w16_t w[NW];
  __device__ __forceinline__ void load(const A* p) {
    if constexpr (EPL * sizeof(A) == 8) {
      const uint2 x = *(const uint2*)p;
      w[0] = w16_t{x.x, x.y, 0u, 0u};
    } else {
#pragma unroll
      for (int i = 0; i < NW; ++i) w[i] = ((const w16_t*)p)[i];
    }
  }
  __device__ __forceinline__ void pack(const float (&v)[EPL]) {
    if constexpr (sizeof(A) == 4) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) w[e / 4][e % 4] = __float_as_uint(v[e]);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; e += 2)
        w[e / 8][(e % 8) / 2] = (uint32_t)f_to_bf16(v[e]) | ((uint32_t)f_to_bf16(v[e + 1]) << 16);
    }
  }
  // buffer store of the words at byte offset off (one 8-, 16- or two 16-byte stores)
  __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off) const {
    if constexpr (EPL * sizeof(A) == 8) {
      __builtin_amdgcn_raw_buffer_store_b64((unsigned int __attribute__((ext_vector_type(2)))){w[0].x, w[0].y}, r,
                                            (int)off, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < NW; ++i) __builtin_amdgcn_raw_buffer_store_b128(w[i], r, (int)(off + 16 * i), 0, 0);
    }
  }
  __device__ __forceinline__ void unpack(float (&v)[EPL]) const {
    if constexpr (sizeof(A) == 4) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) v[e] = __uint_as_float(w[e / 4][e % 4]);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const uint32_t x = w[e / 8][(e % 8) / 2];
        v[e] = __uint_as_float((e & 1) ? (x & 0xFFFF0000u) : (x << 16));
      }
    }
  }
};

// ------------------------------------------------------------------------------------------- held-row variant
// For chunks with C a power of two, 8 <= C <= 128, and at most 32 write and 32 read terms per part (float32
// banks): the 128 lane groups split every token's write terms, and its read terms, in gpt = 128 / C equal parts;
// each group keeps its gathered write rows M_0[S_ti] in registers, and the group holding a slot's last event of the
// chunk applies the slot's events to that row and stores it (no second read of the bank). A slot written once needs
// only the holder's own term; slots written more than once take their events from the plan's multi-event table.
// H and G are summed per part, then over the parts in order (lane shuffles; bitwise repeatable); the part-0 group
// of each token then computes its U, delta and output row slices.
//
// Memory pipeline per chunk: the write terms (slot, coefficient, int16 last-event code) and the read terms sit in
// LDS, staged during the previous chunk (write terms double-buffered). The 32 read rows of a lane are issued first;
// then a sliding window consumes read row u (the oldest load) into G and issues held write row u into the same
// registers, so 32 row loads stay in flight per lane. T/Q lists and multi-event tables larger than their LDS areas are read from the
// plan region in HBM instead.
template <typename Bk> struct Hold { static constexpr int N = 32; };  // float32 banks only (see launch_loop_t)
constexpr int HELD_LISTS_LDS = 8 * 1024;   // T and Q entries kept in LDS
constexpr int HELD_MULTI_LDS = 8 * 1024;   // multi-event table kept in LDS
constexpr int HELD_MROWS = 256;            // held row slices (64 bytes) of multi-event slots kept in LDS

// one LDS buffer of write terms: pairs [C * W], then int16 last-event codes [C * W] (the plan region's first two
// sections, same layout)
__host__ __device__ inline long long held_wterm_bytes(int C, int W) {
  return align16((long long)C * W * 8) + align16((long long)C * W * 2);
}

__host__ __device__ inline long long held_small_bytes(int C, int cols) {
  return align16((long long)2 * C * cols * 4 + (long long)C * 8);
}

// LDS: U and delta [C][cols], gates [C]; two write-term buffers; the read terms [C * R]; T/Q row pointers and
// lists; the multi-event table; held row slices of slots written more than once.
__host__ __device__ inline size_t loop_held_lds_bytes(int C, int W, int R, int cols) {
  return (size_t)(held_small_bytes(C, cols) + 2 * held_wterm_bytes(C, W) + align16((long long)C * R * 8) +
                  align16((long long)2 * (C + 1) * 4) + HELD_LISTS_LDS + HELD_MULTI_LDS + HELD_MROWS * 64);
}

// Copies n16 16-byte words from global to LDS, NB loads in flight per thread.
template <int NB>
__device__ __forceinline__ void stage16(const uint4* __restrict__ src, uint4* dst, int n16) {
  const int tid = threadIdx.x;
  for (int i0 = 0; i0 < n16; i0 += LOOP_NT * NB) {
    uint4 tmp[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) tmp[k] = src[min(i0 + tid + k * LOOP_NT, n16 - 1)];  // clamped: in bounds
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int i = i0 + tid + k * LOOP_NT;
      if (i < n16) dst[i] = tmp[k];
    }
  }
}

// Sliding window over the 32 row registers of a lane: step U consumes read row U (the oldest load in flight) into
// G, then issues held write row U into the same registers. Lanes without a term load row 0 and ignore it: the
// number of loads in flight is fixed, which keeps the waits exact.
template <int U, int N, bool FULL>
struct Window {
  template <typename Bk>
  __device__ __forceinline__ static void run(uint4 (&row)[N], const Pair* pr, float (&g)[Lane<Bk>::EPL],
                                             const Pair* pw, const Bk* bank, uint32_t ld, int mycol, bool act,
                                             uint32_t amask, int tpr, int tpw) {
    // term slots are read unconditionally (inside the LDS areas) and masked to row 0 when not valid: no branch
    const float cf = pr[U].coef;
    const uint32_t m = amask & ((FULL || U < tpw) ? ~0u : 0u);
    const uint64_t off = (uint64_t)((uint32_t)pw[U].slot & m) * ld + ((uint32_t)mycol & m);
    if (FULL || (act && U < tpr)) {  // FULL: no branch (lanes without a token accumulate row 0, never used)
      float v[Lane<Bk>::EPL];
      Lane<Bk>::unpack(row[U], v);
#pragma unroll
      for (int e = 0; e < Lane<Bk>::EPL; ++e) g[e] += cf * v[e];
    }
    row[U] = *(const uint4*)(bank + off);
    __builtin_amdgcn_sched_barrier(0);  // keep the steps in order: one row in, one row out
    Window<U + 1, N, FULL>::run(row, pr, g, pw, bank, ld, mycol, act, amask, tpr, tpw);
  }
};
template <int N, bool FULL>
struct Window<N, N, FULL> {
  template <typename Bk>
  __device__ __forceinline__ static void run(uint4 (&)[N], const Pair*, float (&)[Lane<Bk>::EPL], const Pair*,
                                             const Bk*, uint32_t, int, bool, uint32_t, int, int) {}
};

// Four activation elements as floats / from floats (value and output row slices of a lane).
template <typename A> struct Act4;
template <> struct Act4<float> {
  __device__ static void load(const float* p, float (&v)[4]) {
    const float4 x = *(const float4*)p;
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  }
  __device__ static void store(float* p, const float (&v)[4]) { *(float4*)p = make_float4(v[0], v[1], v[2], v[3]); }
};
template <> struct Act4<bf16_t> {
  __device__ static void load(const bf16_t* p, float (&v)[4]) {
    const uint2 x = *(const uint2*)p;
    v[0] = __uint_as_float(x.x << 16); v[1] = __uint_as_float(x.x & 0xFFFF0000u);
    v[2] = __uint_as_float(x.y << 16); v[3] = __uint_as_float(x.y & 0xFFFF0000u);
  }
  __device__ static void store(bf16_t* p, const float (&v)[4]) {
    uint2 x;
    x.x = (uint32_t)from_f<bf16_t>(v[0]) | ((uint32_t)from_f<bf16_t>(v[1]) << 16);
    x.y = (uint32_t)from_f<bf16_t>(v[2]) | ((uint32_t)from_f<bf16_t>(v[3]) << 16);
    *(uint2*)p = x;
  }
};

// FULL: every part has exactly 32 write and 32 read terms (no per-row term-count test). SNAP: also the backward's
// snapshot (a.snap; the plan tagged every event with its term index): a slot's only event stores its held row (the
// chunk-start row, the row before that event), and a slot written more than once stores its running row before
// each of its events.
template <typename A, typename Bk, bool FULL, bool SNAP, int SM = SNAP_BANK>
__global__ __launch_bounds__(LOOP_NT) void loop_held_kernel(Dims D, LoopArgs a, int nslices) {
  if (a.abort && *a.abort) return;  // shared-bank conflict: no work (uniform over the grid)
  constexpr int EPL = Lane<Bk>::EPL;
  static_assert(EPL == 4, "held rows are float32 row slices of 4 elements per lane");
  constexpr int COLS = 4 * EPL;
  constexpr int HOLD = Hold<Bk>::N;
  extern __shared__ __align__(16) unsigned char lds[];
  const int C = D.C, W = D.W, R = D.R;
  const int gpt = 128 / C;
  const int tpw = W / gpt, tpr = R / gpt;
  float* sH = (float*)lds;                  // [C][COLS]  U
  float* sD = sH + C * COLS;                // [C][COLS]  delta
  float* sA = sD + C * COLS;                // [C]
  const ChunkLayout CL = chunk_layout(C, W, R);
  const long long WT = held_wterm_bytes(C, W);
  unsigned char* sW0 = lds + held_small_bytes(C, COLS);
  unsigned char* sR = sW0 + 2 * WT;                         // read terms [C * R]
  const long long RT = align16((long long)C * R * 8);
  unsigned char* sLst = sR + RT;                            // T/Q row pointers, then lists (plan region layout)
  const long long ptrs_b = align16((long long)2 * (C + 1) * 4);
  MSeg* msegs_lds = (MSeg*)(sLst + ptrs_b + HELD_LISTS_LDS);
  w16_t* sM = (w16_t*)((unsigned char*)msegs_lds + HELD_MULTI_LDS);  // [HELD_MROWS][4] held rows of multi slots
  const int32_t* tptr = (const int32_t*)sLst;
  const int32_t* qptr = tptr + (C + 1);

  const int nblk = gridDim.x;
  int w = blockIdx.x;
  if ((nblk & 7) == 0) w = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int st = w / nslices, slice = w % nslices;
  const int b = st / D.H, h = st % D.H;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int q = lane & 3, grp = lane >> 2;
  const int G = wv * 16 + grp;              // lane group 0..127
  const int gt = G / gpt, part = G % gpt;   // its token and part
  const int col0 = slice * COLS;
  const int mycol = col0 + q * EPL;
  const bool valid = mycol < D.d;
  Bk* bank = (Bk*)a.bank + bank_of(D, st) * D.rows * D.ld;
  const uint32_t ld = (uint32_t)D.ld;
  const A* alpha = (const A*)a.alpha;
  const A* beta = (const A*)a.beta;
  const A* values = (const A*)a.values;
  A* out = (A*)a.out;
  const int nw16 = (int)(WT >> 4);          // <= 2560: C * W <= 4096
  const int nr16 = (int)(RT >> 4);          // <= 2048: C * R <= 4096
  constexpr int NWP = 5;                    // 16-byte words of the next write terms per thread
  constexpr int NRP = 4;                    // 16-byte words of the next read terms per thread
  constexpr int NST = 4;                    // 16-byte words of row pointers, lists and multi-event table per thread

  // write and read terms of the first chunk
  const int ch1 = a.ch1 ? a.ch1 : D.nch;  // chunks [a.ch0, ch1)
  {
    const unsigned char* g0 = a.chunks + ((long long)st * D.nch + a.ch0) * CL.bytes;
    stage16<NWP>((const uint4*)g0, (uint4*)sW0, nw16);
    stage16<NRP>((const uint4*)(g0 + CL.rpairs), (uint4*)sR, nr16);
  }
  __syncthreads();

  ChunkCounts cnt = a.counts[(long long)st * D.nch + a.ch0];
  for (int ch = a.ch0; ch < ch1; ++ch) {
    const int t0 = ch * C;
    const int Cc = min(C, D.T - t0);
    const long long cidx = (long long)st * D.nch + ch;
    const unsigned char* greg = a.chunks + cidx * CL.bytes;
    const bool more = ch + 1 < ch1;
    const ChunkCounts next = a.counts[more ? cidx + 1 : cidx];
    const bool act = valid && gt < Cc;
    const bool lead = part == 0 && act;     // computes U, delta and the output of token gt's row slice
    unsigned char* sWc = sW0 + ((ch - a.ch0) & 1) * WT;
    unsigned char* sWn = sW0 + ((ch - a.ch0 + 1) & 1) * WT;
    const Pair* pw = (const Pair*)sWc + gt * W + part * tpw;
    const int16_t* wl = (const int16_t*)(sWc + align16((long long)C * W * 8)) + gt * W + part * tpw;

    // 1) read rows: terms from LDS, 32 loads in flight
    const Pair* pr = (const Pair*)sR + gt * R + part * tpr;
    uint4 row[HOLD];
    const uint32_t amask = act ? ~0u : 0u;
#pragma unroll
    for (int u = 0; u < HOLD; ++u) {
      const uint32_t m = amask & ((FULL || u < tpr) ? ~0u : 0u);
      const uint64_t off = (uint64_t)((uint32_t)pr[u].slot & m) * ld + ((uint32_t)mycol & m);
      row[u] = *(const uint4*)(bank + off);
      if ((u & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    }
    // 2) gates and the value row slice of the token (used by its part-0 group), loaded by every lane without a
    //    branch and converted only after H: a use right after the load would wait for every row load before it
    const long long grow = ((long long)b * D.T + t0 + min(gt, Cc - 1)) * D.H + h;  // token gt's (b, t, h) row
    const A raw_a = alpha[grow], raw_b = beta[grow];
    ActRaw<A, 4> raw_v;
    raw_v.load(values + grow * D.d + mycol);
    const A raw_sa = alpha[((long long)b * D.T + t0 + min(tid, Cc - 1)) * D.H + h];
    // 3) window: read rows into G, held write rows into the same registers
    float gacc[EPL], hacc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) gacc[e] = hacc[e] = 0.0f;
    Window<0, HOLD, FULL>::run(row, pr, gacc, pw, bank, ld, mycol, act, amask, tpr, tpw);
    // 4) small loads behind the held rows: this chunk's row pointers, lists and multi-event table
    const long long lbytes = (long long)(cnt.nnzT + cnt.nnzQ) * 8;
    const bool llds = lbytes <= HELD_LISTS_LDS;
    const long long mbytes = (long long)cnt.nmseg * 16 + (long long)cnt.nmev * 8;
    const bool mlds = mbytes <= HELD_MULTI_LDS;
    const int n1 = (int)((ptrs_b + (llds ? lbytes : 0) + 15) >> 4);
    const int n12 = n1 + (mlds ? (int)((mbytes + 15) >> 4) : 0);  // <= NST * LOOP_NT
    const w16_t* src1 = (const w16_t*)(greg + CL.ptrs);
    const w16_t* src2 = (const w16_t*)(greg + CL.multi) - n1;
    w16_t stg[NST];
    static_for<NST>([&](auto k) {
      const int i = min(tid + k * LOOP_NT, n12 - 1);  // n12 >= 1: the row pointers are never empty
      stg[k] = i < n1 ? src1[i] : src2[i];
    });
    // 5) H from the held rows
#pragma unroll
    for (int u = 0; u < HOLD; ++u) {
      const float cf = pw[u].coef;
      if (FULL || (act && u < tpw)) {
        float v[EPL];
        Lane<Bk>::unpack(row[u], v);
#pragma unroll
        for (int e = 0; e < EPL; ++e) hacc[e] += cf * v[e];
      }
    }
    // parts of a token are the gpt consecutive groups (4 gpt consecutive lanes of one wave): sum them in order
    for (int p = 1; p < gpt; ++p) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float hx = __shfl_down(hacc[e], 4 * p, 64);
        const float gx = __shfl_down(gacc[e], 4 * p, 64);
        if (part == 0) {
          hacc[e] += hx;
          gacc[e] += gx;
        }
      }
    }
    // 6) U = beta v - alpha beta H; staged words to LDS (the next write terms go to the free buffer)
    if (lead) {
      const float ga = to_f<A>(raw_a), gb = to_f<A>(raw_b);
      float va[4];
      raw_v.unpack(va);
#pragma unroll
      for (int e = 0; e < EPL; ++e) sH[gt * COLS + q * EPL + e] = gb * va[e] - ga * gb * hacc[e];
    }
    if (tid < Cc) sA[tid] = to_f<A>(raw_sa);
    {
      w16_t* dst1 = (w16_t*)sLst;
      w16_t* dst2 = (w16_t*)msegs_lds - n1;
      static_for<NST>([&](auto k) {
        const int i = tid + k * LOOP_NT;
        if (i < n12) {
          if (i < n1) dst1[i] = stg[k]; else dst2[i] = stg[k];
        }
      });
    }
    __syncthreads();  // U, gates, lists and the multi-event table in LDS; every wave has taken its read terms
    // next chunk's write and read terms (their LDS areas are free now)
    w16_t wpf[NWP], rpf[NRP];
    {
      const unsigned char* gn = more ? greg + CL.bytes : greg;  // last chunk: loaded, never stored
      static_for<NWP>([&](auto k) { wpf[k] = ((const w16_t*)gn)[min(tid + k * LOOP_NT, nw16 - 1)]; });
      static_for<NRP>([&](auto k) { rpf[k] = ((const w16_t*)(gn + CL.rpairs))[min(tid + k * LOOP_NT, nr16 - 1)]; });
    }
    // lists and the multi-event table through typed pointers (LDS, or the plan region when they did not fit): a
    // pointer that may be either compiles to flat loads, whose waits also cover every global load and store
    const Ent* lists_l = (const Ent*)(sLst + ptrs_b);
    const Ent* lists_g = (const Ent*)(greg + CL.lists);
    // 7) delta = T U
    if (lead) {
      float d[EPL] = {0.0f, 0.0f, 0.0f, 0.0f};
      auto trow = [&](const Ent* lists) {
        for (int e = tptr[gt]; e < tptr[gt + 1]; ++e) {
          const Ent x = lists[e];
          const float4 u = *(const float4*)(sH + x.col * COLS + q * EPL);
          d[0] += x.val * u.x; d[1] += x.val * u.y; d[2] += x.val * u.z; d[3] += x.val * u.w;
        }
      };
      if (llds) trow(lists_l); else trow(lists_g);
      *(float4*)(sD + gt * COLS + q * EPL) = make_float4(d[0], d[1], d[2], d[3]);
    }
    static_for<NWP>([&](auto k) {
      const int i = tid + k * LOOP_NT;
      if (more && i < nw16) ((w16_t*)sWn)[i] = wpf[k];
    });
    static_for<NRP>([&](auto k) {
      const int i = tid + k * LOOP_NT;
      if (more && i < nr16) ((w16_t*)sR)[i] = rpf[k];
    });
    __syncthreads();  // delta in LDS
    // 8) scatter: a slot's only event is applied by its holder and stored; the held row slices of slots written more
    //    than once go to LDS (when they fit) and are finished in step 10, one slot per lane group
    const bool mrows = cnt.nmseg <= HELD_MROWS;
    const MSeg* msegs_g = (const MSeg*)(greg + CL.multi);
    // snapshot rows of this stream: row (t, i) at (t * W + i) * d, through a buffer resource (base in scalar
    // registers, 32-bit lane offsets: the held rows leave few vector registers); SM = SNAP_BF16: bfloat16 rows (each
    // float rounded to nearest even), 8 bytes per lane instead of 16; SNAP_FP8 / SNAP_INT4: the 4 lanes of a lane
    // group hold one 16-column group, whose scale comes from their largest magnitude (two DPP moves inside the
    // quad); a lane stores its 4 elements (4 or 2 bytes) and the group's first lane the scale byte
    constexpr bool QS = SM == SNAP_FP8 || SM == SNAP_INT4;
    constexpr uint32_t SES = SM == SNAP_BF16 ? 2u : 4u;  // bytes per snapshot element (SNAP_BANK, SNAP_BF16)
    __amdgpu_buffer_rsrc_t rsnap, rscale;
    if constexpr (SNAP && !QS)
      rsnap = __builtin_amdgcn_make_buffer_rsrc((void*)((char*)a.snap + (long long)st * D.T * D.W * D.d * SES),
                                                (short)0, (int)(uint32_t)((unsigned long long)D.T * D.W * D.d * SES),
                                                BUF_RSRC_WORD3);
    if constexpr (SNAP && QS) {
      const unsigned long long rows_s = (unsigned long long)D.T * D.W;  // snapshot rows per stream
      const unsigned long long eb = snap_row_elem_bytes(SM, D.d), sb = snap_row_scale_bytes(D.d);
      rsnap = __builtin_amdgcn_make_buffer_rsrc((void*)((char*)a.snap + st * rows_s * eb), (short)0,
                                                (int)(uint32_t)(rows_s * eb), BUF_RSRC_WORD3);
      rscale = __builtin_amdgcn_make_buffer_rsrc(
          (void*)((char*)a.snap + (unsigned long long)D.S * rows_s * eb + st * rows_s * sb), (short)0,
          (int)(uint32_t)(rows_s * sb), BUF_RSRC_WORD3);
    }
    auto snap_row = [&](int t, int i) -> uint32_t { return (uint32_t)(t0 + t) * (uint32_t)W + (uint32_t)i; };
    auto snap_store = [&](uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3, uint32_t srow) {
      if constexpr (SM == SNAP_BANK) {
        __builtin_amdgcn_raw_buffer_store_b128(w16_t{x0, x1, x2, x3}, rsnap,
                                               (int)((srow * (uint32_t)D.d + (uint32_t)mycol) * SES), 0, 0);
      } else if constexpr (SM == SNAP_BF16) {
        const uint32_t lo = (uint32_t)f_to_bf16(__uint_as_float(x0)) | ((uint32_t)f_to_bf16(__uint_as_float(x1)) << 16);
        const uint32_t hi = (uint32_t)f_to_bf16(__uint_as_float(x2)) | ((uint32_t)f_to_bf16(__uint_as_float(x3)) << 16);
        typedef unsigned int u32x2_t __attribute__((__vector_size__(2 * sizeof(unsigned int))));
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{lo, hi}, rsnap,
                                              (int)((srow * (uint32_t)D.d + (uint32_t)mycol) * SES), 0, 0);
      } else {
        const float v[4] = {__uint_as_float(x0), __uint_as_float(x1), __uint_as_float(x2), __uint_as_float(x3)};
        float am = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
        am = fmaxf(am, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(am), 0xB1, 0xf, 0xf, false)));
        am = fmaxf(am, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(am), 0x4E, 0xf, 0xf, false)));
        uint32_t word = 0, sbyte = 0;
        if (am > 0.0f) {
          const int e = snap_scale_exp(am, SM == SNAP_FP8 ? 8 : 2);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float x = ldexpf(v[k], -e);
            word |= (SM == SNAP_FP8 ? e4m3_encode(x) : ((uint32_t)(int)rintf(x) & 0xFu)) << ((SM == SNAP_FP8 ? 8 : 4) * k);
          }
          sbyte = (uint32_t)min(max(e + 127, 0), 255);
        }
        const uint32_t el = srow * (uint32_t)D.d + (uint32_t)mycol;  // element index
        if constexpr (SM == SNAP_FP8)
          __builtin_amdgcn_raw_buffer_store_b32(word, rsnap, (int)el, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)word, rsnap, (int)(el / 2), 0, 0);
        if (q == 0)
          __builtin_amdgcn_raw_buffer_store_b8((unsigned char)sbyte, rscale,
                                               (int)(srow * (uint32_t)(D.d / SNAP_GROUP) + (uint32_t)mycol / SNAP_GROUP),
                                               0, 0);
      }
    };
    if (act) {
      const float4 dg = *(const float4*)(sD + gt * COLS + q * EPL);
      const float ag = sA[gt];
#pragma unroll
      for (int u = 0; u < HOLD; ++u) {
        if (FULL || u < tpw) {
          const int code = wl[u];
          if (code == -2) {  // the slot's only event: own token, own weight
            if constexpr (SNAP) snap_store(row[u].x, row[u].y, row[u].z, row[u].w, snap_row(gt, part * tpw + u));
            float m[EPL];
            Lane<Bk>::unpack(row[u], m);
            const Pair p = pw[u];
            m[0] = ag * m[0] + p.coef * dg.x; m[1] = ag * m[1] + p.coef * dg.y;
            m[2] = ag * m[2] + p.coef * dg.z; m[3] = ag * m[3] + p.coef * dg.w;
            Lane<Bk>::store(bank + ((uint64_t)(uint32_t)p.slot * ld + (uint32_t)mycol), m);
          } else if (code >= 0) {
            if (mrows) {
              sM[code * 4 + q] = w16_t{row[u].x, row[u].y, row[u].z, row[u].w};
            } else {  // rare (many multi-event slots): events read from the plan region
              float m[EPL];
              Lane<Bk>::unpack(row[u], m);
              const MSeg sg = msegs_g[code];
              const Ev* mev = (const Ev*)(msegs_g + cnt.nmseg);
              for (int e = sg.beg; e < sg.end; ++e) {
                const Ev x = mev[e];
                const int tk = SNAP ? (x.tok & 0xFFFF) : x.tok;
                if constexpr (SNAP)
                  snap_store(__float_as_uint(m[0]), __float_as_uint(m[1]), __float_as_uint(m[2]), __float_as_uint(m[3]),
                             snap_row(tk, x.tok >> 16));
                const float al = sA[tk];
#pragma unroll
                for (int k = 0; k < EPL; ++k) m[k] = al * m[k] + x.w * sD[tk * COLS + q * EPL + k];
              }
              Lane<Bk>::store(bank + ((uint64_t)(uint32_t)pw[u].slot * ld + (uint32_t)mycol), m);
            }
          }
        }
      }
    }
    // 9) read output: out = G + Q delta
    if (lead) {
      float o[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = gacc[e];
      auto qrow = [&](const Ent* lists) {
        for (int e = qptr[gt]; e < qptr[gt + 1]; ++e) {
          const Ent x = lists[e];
          const float4 dd = *(const float4*)(sD + x.col * COLS + q * EPL);
          o[0] += x.val * dd.x; o[1] += x.val * dd.y; o[2] += x.val * dd.z; o[3] += x.val * dd.w;
        }
      };
      if (llds) qrow(lists_l); else qrow(lists_g);
      Act4<A>::store(out + grow * D.d + mycol, o);
    }
    // 10) slots written more than once: their events in token order on the held row slice, one store
    if (mrows) {
      __syncthreads();  // held row slices in LDS
      auto finish = [&](const MSeg* msegs) {
        const Ev* mev = (const Ev*)(msegs + cnt.nmseg);
        for (int i = G; i < cnt.nmseg; i += 128) {
          const MSeg sg = msegs[i];
          const w16_t x0 = sM[i * 4 + q];
          float m[EPL] = {__uint_as_float(x0.x), __uint_as_float(x0.y), __uint_as_float(x0.z), __uint_as_float(x0.w)};
          for (int e = sg.beg; e < sg.end; ++e) {
            const Ev x = mev[e];
            const int tk = SNAP ? (x.tok & 0xFFFF) : x.tok;
            if constexpr (SNAP)
              if (valid)
                snap_store(__float_as_uint(m[0]), __float_as_uint(m[1]), __float_as_uint(m[2]), __float_as_uint(m[3]),
                           snap_row(tk, x.tok >> 16));
            const float al = sA[tk];
            const float4 dd = *(const float4*)(sD + tk * COLS + q * EPL);
            m[0] = al * m[0] + x.w * dd.x; m[1] = al * m[1] + x.w * dd.y;
            m[2] = al * m[2] + x.w * dd.z; m[3] = al * m[3] + x.w * dd.w;
          }
          if (valid) Lane<Bk>::store(bank + ((uint64_t)(uint32_t)sg.slot * ld + (uint32_t)mycol), m);
        }
      };
      if (mlds) finish(msegs_lds); else finish(msegs_g);
    }
    cnt = next;
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------- narrow variant
// One lane per 16-byte row piece and one workgroup per (stream, 16-byte column slice): four times the workgroups
// of the 64-byte slices, for streams whose rows are short (bf16 banks, small head_dim) or whose chunk gives a
// 64-byte lane group more terms than it can hold. The gpt = 512 / C consecutive lanes of a token split its W write
// and R read terms (at most 16 of each per lane). A lane keeps its own terms in registers (they are not shared
// with other lanes): the next chunk's read terms are loaded during the delta phase; a chunk's write terms and read
// rows are issued first, then a sliding window turns each consumed read row's registers into a held write row. H and G are
// summed over the parts of a token in order by lane shuffles, the token's first lane computes U, delta and the
// output piece, and the lane holding a slot's last event of the chunk applies the slot's events and stores it.
constexpr int NARROW_HOLD = 16;
constexpr int NARROW_NST = 8;                // 16-byte words of row pointers, lists and multi-event table per thread
constexpr int NARROW_STAGE_LDS = NARROW_NST * LOOP_NT * 16;  // their LDS area, filled by direct global-to-LDS loads
constexpr int NARROW_MROWS = 1024;           // held rows of multi-event slots kept in LDS (16 bytes each)

__host__ __device__ inline long long narrow_small_bytes(int C, int epl) {
  return align16((long long)2 * C * epl * 4 + (long long)C * 4);
}

// LDS: U and delta [C][epl], gates [C]; T/Q row pointers, lists and the multi-event table (one contiguous area);
// held rows of slots written more than once.
__host__ __device__ inline size_t loop_narrow_lds_bytes(int C, int epl) {
  return (size_t)(narrow_small_bytes(C, epl) + NARROW_STAGE_LDS + NARROW_MROWS * 16);
}

// EPL activation elements (4 or 8) as floats / from floats.
template <typename A, int EPL>
__device__ __forceinline__ void act_load(const A* p, float (&v)[EPL]) {
  static_for<EPL / 4>([&](auto k) {
    float t[4];
    Act4<A>::load(p + 4 * k, t);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * k + e] = t[e];
  });
}
template <typename A, int EPL>
__device__ __forceinline__ void act_store(A* p, const float (&v)[EPL]) {
  static_for<EPL / 4>([&](auto k) {
    float t[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = v[4 * k + e];
    Act4<A>::store(p + 4 * k, t);
  });
}

// A lane's gather terms of one chunk: NARROW_HOLD (slot, coefficient) pairs, and for write terms their int16
// last-event codes. FULL: exactly NARROW_HOLD terms, stored lane-major (term_pos, code_pos): word k of the lane is
// word k * 512 + lane of the section, one coalesced load; pp and cp are the sections. Otherwise pp and cp point at
// the lane's first term (token-major) and n terms are loaded one by one, the rest repeating the last.
struct NarrowTerms {
  w16_t p[NARROW_HOLD / 2];  // pairs (slot, coef bits) two per word
  w16_t c[2];                // int16 codes, eight per word (write terms only)
};
template <bool FULL, bool CODES>
__device__ __forceinline__ void narrow_load_terms(NarrowTerms& t, const Pair* pp, const int16_t* cp, int n) {
  if (FULL) {
    static_for<NARROW_HOLD / 2>([&](auto k) { t.p[k] = ((const w16_t*)pp)[k * LOOP_NT + threadIdx.x]; });
    if (CODES) static_for<2>([&](auto k) { t.c[k] = ((const w16_t*)cp)[k * LOOP_NT + threadIdx.x]; });
  } else {
    static_for<NARROW_HOLD / 2>([&](auto k) {
      const uint2 a = *(const uint2*)(pp + min(2 * (int)k, n - 1));
      const uint2 b = *(const uint2*)(pp + min(2 * (int)k + 1, n - 1));
      t.p[k] = w16_t{a.x, a.y, b.x, b.y};
    });
    if (CODES)
      static_for<2>([&](auto k) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo = (uint16_t)cp[min(8 * (int)k + 2 * j, n - 1)];
          const uint32_t hi = (uint16_t)cp[min(8 * (int)k + 2 * j + 1, n - 1)];
          w[j] = lo | (hi << 16);
        }
        t.c[k] = w16_t{w[0], w[1], w[2], w[3]};
      });
  }
}
template <int U> __device__ __forceinline__ uint32_t term_slot(const NarrowTerms& t) { return t.p[U / 2][(U & 1) * 2]; }
template <int U> __device__ __forceinline__ float term_coef(const NarrowTerms& t) {
  return __uint_as_float(t.p[U / 2][(U & 1) * 2 + 1]);
}
template <int U> __device__ __forceinline__ int term_code(const NarrowTerms& t) {
  return (int)(int16_t)(uint16_t)(t.c[U / 8][(U & 7) / 2] >> (16 * (U & 1)));
}

// A 16-byte row piece held as a native vector, as floats.
template <typename Bk> __device__ __forceinline__ void unpack_w(const w16_t& x, float* v);
template <> __device__ __forceinline__ void unpack_w<float>(const w16_t& x, float* v) {
  v[0] = __uint_as_float(x.x); v[1] = __uint_as_float(x.y); v[2] = __uint_as_float(x.z); v[3] = __uint_as_float(x.w);
}
template <> __device__ __forceinline__ void unpack_w<bf16_t>(const w16_t& x, float* v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(x[i] << 16);
    v[2 * i + 1] = __uint_as_float(x[i] & 0xFFFF0000u);
  }
}

template <typename Bk> __device__ __forceinline__ w16_t pack_w(const float* v);
template <> __device__ __forceinline__ w16_t pack_w<float>(const float* v) {
  return w16_t{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
}
template <> __device__ __forceinline__ w16_t pack_w<bf16_t>(const float* v) {
  w16_t x;
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = (uint32_t)f_to_bf16(v[2 * i]) | ((uint32_t)f_to_bf16(v[2 * i + 1]) << 16);
  return x;
}


template <typename A, typename Bk, bool FULL>
__global__ __launch_bounds__(LOOP_NT) void loop_narrow_kernel(Dims D, LoopArgs a, int nslices) {
  if (a.abort && *a.abort) return;  // shared-bank conflict: no work (uniform over the grid)
  constexpr int EPL = Lane<Bk>::EPL;
  constexpr int HOLD = NARROW_HOLD;
  extern __shared__ __align__(16) unsigned char lds[];
  const int C = D.C, W = D.W, R = D.R;
  const int lg = __builtin_ctz(LOOP_NT / C);  // log2 of gpt
  const int gpt = 1 << lg;
  const int tpw = W >> lg, tpr = R >> lg;
  float* sU = (float*)lds;   // [C][EPL]
  float* sD = sU + C * EPL;  // [C][EPL]
  float* sA = sD + C * EPL;  // [C]
  const ChunkLayout CL = chunk_layout(C, W, R);
  unsigned char* sLst = lds + narrow_small_bytes(C, EPL);  // T/Q row pointers, lists, then the multi-event table
  const long long ptrs_b = align16((long long)2 * (C + 1) * 4);
  w16_t* sM = (w16_t*)(sLst + NARROW_STAGE_LDS);           // held rows of multi-event slots
  const int32_t* tptr = (const int32_t*)sLst;
  const int32_t* qptr = tptr + (C + 1);

  const int nblk = gridDim.x;
  int w = blockIdx.x;
  if ((nblk & 7) == 0) w = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int st = w / nslices, slice = w % nslices;
  const int b = st / D.H, h = st % D.H;
  const int tid = threadIdx.x;
  const int gt = tid >> lg, part = tid & (gpt - 1);  // token and part of this lane
  const int mycol = slice * EPL;
  const bool valid = mycol < D.d;
  // the stream's bank as a buffer resource: 32-bit byte offsets (the path requires < 4 GiB per stream), and any
  // access beyond the stream's rows is dropped by the hardware range check
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((Bk*)a.bank + bank_of(D, st) * D.rows * D.ld), (short)0,
      (int)(uint32_t)((unsigned long long)D.rows * D.ld * sizeof(Bk)), BUF_RSRC_WORD3);
  const uint32_t ldb = (uint32_t)(D.ld * sizeof(Bk));
  const uint32_t colb = (uint32_t)(mycol * sizeof(Bk));
  const A* alpha = (const A*)a.alpha;
  const A* beta = (const A*)a.beta;
  const A* values = (const A*)a.values;
  A* out = (A*)a.out;
  const long long woff = FULL ? 0 : (long long)gt * W + part * tpw;  // this lane's first write term (token-major)
  const long long roff = FULL ? 0 : (long long)gt * R + part * tpr;

  NarrowTerms rt;
  const int ch1 = a.ch1 ? a.ch1 : D.nch;  // chunks [a.ch0, ch1)
  {
    const unsigned char* g0 = a.chunks + ((long long)st * D.nch + a.ch0) * CL.bytes;
    narrow_load_terms<FULL, false>(rt, (const Pair*)(g0 + CL.rpairs) + roff, nullptr, tpr);
#pragma unroll
    for (int i = 0; i < NARROW_HOLD / 2; ++i) asm volatile("" : "+v"(rt.p[i]));  // arrived before the loop
  }

  ChunkCounts cnt = a.counts[(long long)st * D.nch + a.ch0];
  for (int ch = a.ch0; ch < ch1; ++ch) {
    const int t0 = ch * C;
    const int Cc = min(C, D.T - t0);
    const long long cidx = (long long)st * D.nch + ch;
    const unsigned char* greg = a.chunks + cidx * CL.bytes;
    const bool more = ch + 1 < ch1;
    const ChunkCounts next = a.counts[more ? cidx + 1 : cidx];
    const bool act = valid && gt < Cc;
    const bool lead = part == 0 && act;
    const uint32_t amask = act ? ~0u : 0u;

    // 1) write terms (needed from the first window step on), then the read rows, all in flight
    NarrowTerms wt;
    narrow_load_terms<FULL, true>(wt, (const Pair*)greg + woff, (const int16_t*)(greg + CL.wlast) + woff, tpw);
    w16_t row[HOLD];
    static_for<HOLD>([&](auto u) {
      const uint32_t m = amask & ((FULL || u < tpr) ? ~0u : 0u);
      row[u] = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)((term_slot<decltype(u)::value>(rt) & m) * ldb + (colb & m)), 0, 0);
    });
    // 2) window: read row u into G, then held write row u into its registers
    float gacc[EPL], hacc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) gacc[e] = hacc[e] = 0.0f;
    static_for<HOLD>([&](auto u) {
      if (FULL || (act && u < tpr)) {
        const float cf = term_coef<decltype(u)::value>(rt);
        float v[EPL];
        unpack_w<Bk>(row[u], v);
#pragma unroll
        for (int e = 0; e < EPL; ++e) gacc[e] += cf * v[e];
      }
      // pin G here: the read row's registers are free before the held row is loaded into them
#pragma unroll
      for (int e = 0; e < EPL; ++e) asm volatile("" : "+v"(gacc[e]));
      const uint32_t m = amask & ((FULL || u < tpw) ? ~0u : 0u);
      row[u] = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)((term_slot<decltype(u)::value>(wt) & m) * ldb + (colb & m)), 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
    // 3) behind the held rows: gates and the value piece of the token (its first lane), loaded by every lane without
    //    a branch and converted only after H, so that no wait for them is placed ahead of the held rows
    const long long grow = ((long long)b * D.T + t0 + min(gt, Cc - 1)) * D.H + h;
    const A raw_a = alpha[grow], raw_b = beta[grow];
    ActRaw<A, EPL> raw_v;
    raw_v.load(values + grow * D.d + mycol);
    const A raw_sa = alpha[((long long)b * D.T + t0 + min(tid, Cc - 1)) * D.H + h];
    // 4) this chunk's row pointers, lists and multi-event table into LDS by direct loads, issued behind the held
    //    rows: a direct load still in flight makes the compiler wait for every load before the next use of a
    //    loaded register, which here is H's first held row, which the direct loads follow. Word i of the area:
    //    row pointers and lists for i < n1, then the multi-event table. Each wave fills 64 consecutive words per
    //    step (the LDS address of a step is uniform over the wave); lanes past n12 repeat the last word inside the
    //    area.
    const long long lbytes = (long long)(cnt.nnzT + cnt.nnzQ) * 8;
    const bool llds = ptrs_b + lbytes <= NARROW_STAGE_LDS;
    const int n1 = (int)((ptrs_b + (llds ? lbytes : 0) + 15) >> 4);
    const long long mbytes = (long long)cnt.nmseg * 16 + (long long)cnt.nmev * 8;
    const bool mlds = (long long)n1 * 16 + mbytes <= NARROW_STAGE_LDS;
    const int n12 = n1 + (mlds ? (int)((mbytes + 15) >> 4) : 0);  // <= NARROW_NST * LOOP_NT
    {
      const w16_t* src1 = (const w16_t*)(greg + CL.ptrs);
      const w16_t* src2 = (const w16_t*)(greg + CL.multi) - n1;
      const int wbase = tid & ~63;
#pragma unroll
      for (int k = 0; k < NARROW_NST; ++k) {
        const int i = min(tid + k * LOOP_NT, n12 - 1);  // n12 >= 1: the row pointers are never empty
        const w16_t* src = i < n1 ? src1 + i : src2 + i;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                         (__attribute__((address_space(3))) void*)(sLst + (k * LOOP_NT + wbase) * 16),
                                         16, 0, 0);
      }
    }
    // 5) H from the held rows; the parts of a token summed by a fixed shuffle tree
    static_for<HOLD>([&](auto u) {
      if (FULL || (act && u < tpw)) {
        const float cf = term_coef<decltype(u)::value>(wt);
        float v[EPL];
        unpack_w<Bk>(row[u], v);
#pragma unroll
        for (int e = 0; e < EPL; ++e) hacc[e] += cf * v[e];
      }
      // keep the row packed until the scatter (its unpacked values are not carried over)
      asm volatile("" : "+v"(row[u]));
      __builtin_amdgcn_sched_barrier(0);
    });
    for (int o = gpt >> 1; o > 0; o >>= 1) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        hacc[e] += __shfl_down(hacc[e], o, 64);
        gacc[e] += __shfl_down(gacc[e], o, 64);
      }
    }
    // 6) U = beta v - alpha beta H
    if (lead) {
      const float ga = to_f<A>(raw_a), gb = to_f<A>(raw_b);
      float va[EPL];
      raw_v.unpack(va);
      float u4[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) u4[e] = gb * va[e] - ga * gb * hacc[e];
      static_for<EPL / 4>([&](auto k) {
        *(float4*)(sU + gt * EPL + 4 * k) = make_float4(u4[4 * k], u4[4 * k + 1], u4[4 * k + 2], u4[4 * k + 3]);
      });
    }
    if (tid < Cc) sA[tid] = to_f<A>(raw_sa);
    __syncthreads();  // U, gates, lists and the multi-event table in LDS (the barrier waits for the direct loads)
    // next chunk's read terms (last chunk: this chunk's again, never used)
    NarrowTerms rn;
    {
      const unsigned char* gn = more ? greg + CL.bytes : greg;
      narrow_load_terms<FULL, false>(rn, (const Pair*)(gn + CL.rpairs) + roff, nullptr, tpr);
    }
    // lists and the multi-event table are read through typed pointers (LDS, or the plan region when they did not
    // fit): a pointer that may be either would compile to flat loads, whose waits also cover every global load
    const Ent* lists_l = (const Ent*)(sLst + ptrs_b);
    const Ent* lists_g = (const Ent*)(greg + CL.lists);
    // 7) delta = T U: the gpt lanes of a token take every gpt-th entry of its row, then a fixed shuffle tree
    {
      float d[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) d[e] = 0.0f;
      auto trow = [&](const Ent* lists) {
        const int e1 = tptr[gt + 1];
        for (int e = tptr[gt] + part; e < e1; e += gpt) {
          const Ent x = lists[e];
          static_for<EPL / 4>([&](auto k) {
            const float4 u = *(const float4*)(sU + x.col * EPL + 4 * k);
            d[4 * k] += x.val * u.x; d[4 * k + 1] += x.val * u.y; d[4 * k + 2] += x.val * u.z; d[4 * k + 3] += x.val * u.w;
          });
        }
      };
      if (act) {
        if (llds) trow(lists_l); else trow(lists_g);
      }
      for (int o = gpt >> 1; o > 0; o >>= 1) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) d[e] += __shfl_down(d[e], o, 64);
      }
      if (lead)
        static_for<EPL / 4>([&](auto k) {
          *(float4*)(sD + gt * EPL + 4 * k) = make_float4(d[4 * k], d[4 * k + 1], d[4 * k + 2], d[4 * k + 3]);
        });
    }
    // the next read terms have arrived by now (they were issued before the delta products): taking them here, ahead
    // of the stores, lets the next chunk start its row loads without waiting for this chunk's stores
#pragma unroll
    for (int i = 0; i < NARROW_HOLD / 2; ++i) asm volatile("" : "+v"(rn.p[i]));
    __syncthreads();  // delta in LDS
    // 8) scatter: a slot's only event is applied by its holder; the held rows of slots written more than once go to
    //    LDS (when they fit) and are finished below, one slot per thread. Every lane issues the same number of
    //    stores: a store that must not happen goes to an offset past the buffer's range, which the hardware drops
    //    (so the compiler can count the loads and stores in flight exactly and never has to wait for all of them).
    const bool mrows = cnt.nmseg <= NARROW_MROWS;
    const MSeg* msegs_lds = (const MSeg*)(sLst + (long long)n1 * 16);
    const MSeg* msegs_g = (const MSeg*)(greg + CL.multi);
    {
      float dg[EPL];
#pragma unroll
      for (int k = 0; k < EPL; ++k) dg[k] = sD[gt * EPL + k];
      const float ag = sA[gt];
      static_for<HOLD>([&](auto u) {
        constexpr int U = decltype(u)::value;
        const bool has = act && (FULL || U < tpw);
        const int code = has ? term_code<U>(wt) : -1;
        float m[EPL];
        unpack_w<Bk>(row[u], m);
        if (code >= 0 && !mrows) {  // rare (many multi-event slots): events read from the plan region
          const MSeg sg = msegs_g[code];
          const Ev* mev = (const Ev*)(msegs_g + cnt.nmseg);
          for (int e = sg.beg; e < sg.end; ++e) {
            const Ev x = mev[e];
            const float al = sA[x.tok];
#pragma unroll
            for (int k = 0; k < EPL; ++k) m[k] = bank_round<Bk>(al * m[k] + x.w * sD[x.tok * EPL + k]);
          }
        } else {  // own token, own weight (used when the slot's only event is this one)
          const float wgt = term_coef<U>(wt);
#pragma unroll
          for (int k = 0; k < EPL; ++k) m[k] = ag * m[k] + wgt * dg[k];
          if (code >= 0) sM[code] = row[u];
        }
        const bool st = code == -2 || (code >= 0 && !mrows);
        const uint32_t off = st ? term_slot<U>(wt) * ldb + colb : BUF_OOB;
        __builtin_amdgcn_raw_buffer_store_b128(pack_w<Bk>(m), rb, (int)off, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    // 9) read output: out = G + Q delta (every lane stores; only a token's first lane inside the range)
    {
      float o[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = gacc[e];
      auto qrow = [&](const Ent* lists) {
        for (int e = qptr[gt]; e < qptr[gt + 1]; ++e) {
          const Ent x = lists[e];
          static_for<EPL / 4>([&](auto k) {
            const float4 dd = *(const float4*)(sD + x.col * EPL + 4 * k);
            o[4 * k] += x.val * dd.x; o[4 * k + 1] += x.val * dd.y; o[4 * k + 2] += x.val * dd.z; o[4 * k + 3] += x.val * dd.w;
          });
        }
      };
      if (lead) {
        if (llds) qrow(lists_l); else qrow(lists_g);
      }
      // rows of this chunk and head: token t at byte (t H d + mycol) * sizeof(A) from the chunk's first row
      const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(out + (((long long)b * D.T + t0) * D.H + h) * D.d), (short)0,
          (int)(uint32_t)((unsigned long long)Cc * D.H * D.d * sizeof(A)), BUF_RSRC_WORD3);
      const uint32_t oo = lead ? (uint32_t)(((long long)gt * D.H * D.d + mycol) * sizeof(A)) : BUF_OOB;
      ActRaw<A, EPL> ov;
      ov.pack(o);
      ov.store(ro, oo);
    }
    // 10) slots written more than once: events in token order on the held row, one store (a fixed number of
    //     iterations per thread; the rows past nmseg are not stored)
    if (mrows && valid) {
      __syncthreads();  // held rows in LDS
      auto finish = [&](const MSeg* msegs) {
        const Ev* mev = (const Ev*)(msegs + cnt.nmseg);
#pragma unroll
        for (int r = 0; r < NARROW_MROWS / LOOP_NT; ++r) {
          const int i = tid + r * LOOP_NT;
          const bool in = i < cnt.nmseg;
          const MSeg sg = msegs[in ? i : 0];
          float m[EPL];
          unpack_w<Bk>(sM[i], m);
          const int e1 = in ? sg.end : sg.beg;
          for (int e = sg.beg; e < e1; ++e) {
            const Ev x = mev[e];
            const float al = sA[x.tok];
#pragma unroll
            for (int k = 0; k < EPL; ++k) m[k] = bank_round<Bk>(al * m[k] + x.w * sD[x.tok * EPL + k]);
          }
          const uint32_t off = in ? (uint32_t)sg.slot * ldb + colb : BUF_OOB;
          __builtin_amdgcn_raw_buffer_store_b128(pack_w<Bk>(m), rb, (int)off, 0, 0);
        }
      };
      if (mlds) finish(msegs_lds); else finish(msegs_g);
    }
    rt = rn;
    cnt = next;
    __syncthreads();
  }
}

// The narrow variant: chunk a power of two in [8, 128], every token's terms split evenly over gpt = 512 / C lanes
// with at most 16 of each kind per lane.
bool loop_narrow_path(const Dims& D) {
  const bool pow2 = (D.C & (D.C - 1)) == 0;
  if (!pow2 || D.C < 8 || D.C > 128) return false;
  const int gpt = LOOP_NT / D.C;
  const int epl = D.bank == SDM_BF16 ? 8 : 4;
  const unsigned long long bytes = (unsigned long long)D.rows * D.ld * (D.bank == SDM_BF16 ? 2 : 4);
  const unsigned long long obytes = (unsigned long long)D.C * D.H * D.d * (D.act == SDM_BF16 ? 2 : 4);
  return bytes < BUF_OOB && obytes < BUF_OOB && D.d % epl == 0 && D.W % gpt == 0 && D.R % gpt == 0 && D.W >= gpt && D.R >= gpt &&
         D.W / gpt <= NARROW_HOLD && D.R / gpt <= NARROW_HOLD && loop_narrow_lds_bytes(D.C, epl) <= 160 * 1024;
}

bool loop_narrow_lanemajor(const Dims& D) {
  const int gpt = LOOP_NT / D.C;
  return loop_narrow_path(D) && D.W == NARROW_HOLD * gpt && D.R == NARROW_HOLD * gpt;
}

// The held-row variant serves float32 banks whose chunk fits its lane-group split and LDS budget.
bool loop_held_path(const Dims& D) {
  if (D.bank != SDM_F32) return false;
  constexpr int COLS = 4 * Lane<float>::EPL;
  const bool pow2 = (D.C & (D.C - 1)) == 0;
  if (!pow2 || D.C < 8 || D.C > 128) return false;
  const int gpt = 128 / D.C;
  return D.W % gpt == 0 && D.R % gpt == 0 && D.W / gpt <= Hold<float>::N && D.R / gpt <= Hold<float>::N &&
         D.W >= gpt && D.R >= gpt && loop_held_lds_bytes(D.C, D.W, D.R, COLS) <= 160 * 1024;
}

// The held-row variant can also write the snapshot when a stream's snapshot fits 32-bit byte offsets.
bool loop_held_snap_ok(const Dims& D) {
  return loop_held_path(D) && (unsigned long long)D.T * D.W * D.d * 4 < BUF_OOB;
}

long long loop_workgroups(const Dims& D, bool snapshot) {
  const int epl = D.bank == SDM_BF16 ? 8 : 4;  // bank elements in 16 bytes
  if (D.bank == SDM_F32 && (snapshot ? loop_held_snap_ok(D) : loop_held_path(D)))
    return (long long)D.S * ((D.d + 15) / 16);
  if (loop_narrow_path(D) && !snapshot) return (long long)D.S * (D.d / epl);
  return (long long)D.S * ((D.d + 4 * epl - 1) / (4 * epl));
}

template <typename A, typename Bk>
static hipError_t launch_loop_t(const Dims& D, const LoopArgs& a, hipStream_t st) {
  constexpr int COLS = 4 * Lane<Bk>::EPL;
  const int nslices = (D.d + COLS - 1) / COLS;
  const long long nblk = (long long)D.S * nslices;
  const size_t staged = loop_lds_bytes(D.C, D.W, D.R, COLS, true);
  const int gpt = 128 / D.C;
  if constexpr (sizeof(Bk) == 4) {
    if (a.snap ? loop_held_snap_ok(D) : loop_held_path(D)) {
      const size_t lds = loop_held_lds_bytes(D.C, D.W, D.R, COLS);
      const bool full = D.W / gpt == Hold<Bk>::N && D.R / gpt == Hold<Bk>::N;
      auto go = [&](auto kern) {
        (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(LOOP_NT), lds, st, D, a, nslices);
      };
      if (a.snap && a.snap_mode == SNAP_BF16) {
        if (full) go(loop_held_kernel<A, Bk, true, true, SNAP_BF16>); else go(loop_held_kernel<A, Bk, false, true, SNAP_BF16>);
      } else if (a.snap && a.snap_mode == SNAP_FP8) {
        if (full) go(loop_held_kernel<A, Bk, true, true, SNAP_FP8>); else go(loop_held_kernel<A, Bk, false, true, SNAP_FP8>);
      } else if (a.snap && a.snap_mode == SNAP_INT4) {
        if (full) go(loop_held_kernel<A, Bk, true, true, SNAP_INT4>); else go(loop_held_kernel<A, Bk, false, true, SNAP_INT4>);
      } else if (a.snap) {
        if (full) go(loop_held_kernel<A, Bk, true, true>); else go(loop_held_kernel<A, Bk, false, true>);
      } else {
        if (full) go(loop_held_kernel<A, Bk, true, false>); else go(loop_held_kernel<A, Bk, false, false>);
      }
      return hipGetLastError();
    }
  }
  if (loop_narrow_path(D) && !a.snap) {
    const size_t lds = loop_narrow_lds_bytes(D.C, Lane<Bk>::EPL);
    const int ns = D.d / Lane<Bk>::EPL;
    const long long nb = (long long)D.S * ns;
    const int g = LOOP_NT / D.C;
    if (loop_narrow_lanemajor(D)) {  // the plan wrote the terms lane-major
      (void)hipFuncSetAttribute((const void*)loop_narrow_kernel<A, Bk, true>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      hipLaunchKernelGGL((loop_narrow_kernel<A, Bk, true>), dim3((unsigned)nb), dim3(LOOP_NT), lds, st, D, a, ns);
    } else {
      (void)hipFuncSetAttribute((const void*)loop_narrow_kernel<A, Bk, false>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      hipLaunchKernelGGL((loop_narrow_kernel<A, Bk, false>), dim3((unsigned)nb), dim3(LOOP_NT), lds, st, D, a, ns);
    }
    return hipGetLastError();
  }
  if (staged <= 150 * 1024) {
    (void)hipFuncSetAttribute((const void*)loop_kernel<A, Bk, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)staged);
    hipLaunchKernelGGL((loop_kernel<A, Bk, true>), dim3((unsigned)nblk), dim3(LOOP_NT), staged, st, D, a, nslices);
  } else {
    const size_t lds = loop_lds_bytes(D.C, D.W, D.R, COLS, false);
    hipLaunchKernelGGL((loop_kernel<A, Bk, false>), dim3((unsigned)nblk), dim3(LOOP_NT), lds, st, D, a, nslices);
  }
  return hipGetLastError();
}

hipError_t launch_loop(const Dims& D, const LoopArgs& a, hipStream_t st) {
  if (D.S == 0 || D.T == 0) return hipSuccess;
  if (D.act == SDM_BF16)
    return D.bank == SDM_BF16 ? launch_loop_t<bf16_t, bf16_t>(D, a, st) : launch_loop_t<bf16_t, float>(D, a, st);
  return D.bank == SDM_BF16 ? launch_loop_t<float, bf16_t>(D, a, st) : launch_loop_t<float, float>(D, a, st);
}

}  // namespace sdm
