// Internal declarations shared by the SDM HIP translation units: validated dimensions, workspace layout, device
// helpers (bfloat16 conversion, order-preserving sort keys, LDS bitonic sort) and kernel launch wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <utility>
#include <stddef.h>
#include <stdint.h>

#include "sdm.h"

namespace sdm {

constexpr int MAX_F = 4;
constexpr int MAX_K = 512;           // num_writes, num_reads, top-k k
constexpr int MAX_NF = 4096;         // sub-keys per factor
constexpr int MAX_CAND = 4096;       // candidate tuples prod(p_f + 1) <= k
constexpr int MAX_FDK = 1024;        // F * dk
constexpr int MAX_CHUNK = 128;       // chunk_size
constexpr int MAX_CHUNK_EVENTS = 8192;  // chunk_size * num_writes
constexpr int MAX_CHUNK_SIZE = 65536;   // requested chunk_size (larger chunks run as equal sub-chunks)
constexpr int TOPK_NT = 256;
constexpr int PLAN_NT = 512;
constexpr int LOOP_NT = 512;
constexpr int DECODE_NT = 256;

typedef uint16_t bf16_t;

// Validated problem dimensions (host and device).
struct Dims {
  int B, T, H, F, dk, d, W, R, C;
  int widths[MAX_F];
  int act, bank;        // sdm_dtype
  long long N;          // slots per head
  long long rows;       // bank rows per stream
  long long ld;         // bank row stride (elements)
  int nch;              // chunks per stream
  int S;                // streams = B * H
  int shared;           // the B streams of a head share one bank (bank [H, rows, ld])
  int scoring;          // SDM_SCORING_*: which factor-scoring kernel the batched top-k uses
};

// Bank index of stream st = b * H + h: st itself, or h with a shared bank.
__host__ __device__ inline long long bank_of(const Dims& D, int st) { return D.shared ? st % D.H : st; }

// Per-query-kind top-k plan: kept positions per factor and the candidate table.
struct TopkPlan {
  int k;
  int kp[MAX_F];        // min(k, n_f)
  int kpmax;
  int ncand;            // tuples with prod(p_f + 1) <= k, p_f < kp[f]
  int cand_pow2;
  int nf_pow2;          // next power of two of max n_f
};

// One scatter event of a chunk: (weight, chunk-local token), sorted by (slot, token).
struct Ev {
  float w;
  int32_t tok;  // chunk-local token; with PlanArgs::evcode also the event's term index in bits 16..31
};

// One sparse entry (column, value) of a row-sorted list: T = (I + diag(alpha beta) K)^-1 or the read coupling Q.
struct Ent {
  int32_t col;
  float val;
};

// A gather term: bank row `slot` times `coef`.
struct Pair {
  int32_t slot;
  float coef;
};

// A written slot of a chunk and the exclusive end of its events in the chunk's event list.
struct Seg {
  int32_t slot;
  int32_t end;
};

// Per-chunk plan region (byte offsets; every part 16-byte aligned). Written by the plan kernel, read by the loop.
//   wpairs [C*W] write gather terms (slot, a)                               (token-major, fixed size)
//   wlast  [C*W] int16 per write term: -1 if it is not its slot's last event in the chunk; -2 if it is the slot's
//          only event; else the index of the slot in the multi-event table (< C W / 2 <= 4096)
//   rpairs [C*R] read gather terms (slot, b)                                (token-major, fixed size)
//   ptrs   tptr[C+1], qptr[C+1] row starts of the two lists                  (fixed size)
//   lists  T entries [nnzT] immediately followed by Q entries [nnzQ]         (packed; capacity C(C+1))
//   scat   segments [nseg] immediately followed by events [E]                 (packed; capacity 2 C W)
//   multi  slots written more than once: MSeg [nmseg] then their events Ev [nmev] (packed; capacity 3 C W / 2)
struct ChunkLayout {
  long long wpairs, wlast, rpairs, ptrs, lists, scat, multi, bytes;
  long long wpairs_bytes, wlast_bytes, rpairs_bytes, ptrs_bytes, lists_cap, scat_cap, multi_cap;
};
__host__ __device__ inline long long align16(long long x) { return (x + 15) & ~15LL; }
__host__ __device__ inline ChunkLayout chunk_layout(int C, int W, int R) {
  ChunkLayout L;
  L.wpairs = 0;
  L.wpairs_bytes = align16((long long)C * W * 8);
  L.wlast = L.wpairs + L.wpairs_bytes;
  L.wlast_bytes = align16((long long)C * W * 2);
  L.rpairs = L.wlast + L.wlast_bytes;
  L.rpairs_bytes = align16((long long)C * R * 8);
  L.ptrs = L.rpairs + L.rpairs_bytes;
  L.ptrs_bytes = align16((long long)2 * (C + 1) * 4);
  L.lists = L.ptrs + L.ptrs_bytes;
  L.lists_cap = align16((long long)C * (C + 1) * 8);
  L.scat = L.lists + L.lists_cap;
  L.scat_cap = align16((long long)2 * C * W * 8);
  L.multi = L.scat + L.scat_cap;
  L.multi_cap = align16((long long)C * W / 2 * 16 + (long long)C * W * 8);
  L.bytes = L.multi + L.multi_cap;
  return L;
}

// A slot written more than once in a chunk: its events are mev[beg, end) of the multi-event table.
struct MSeg {
  int32_t slot, beg, end, pad;
};

// Per-chunk counts written by the plan.
struct ChunkCounts {
  int32_t nnzT, nnzQ, nseg, nev, nmseg, nmev, pad0, pad1;
};

// ------------------------------------------------------------------------------------------- device helpers
// A 16-byte word as a native vector (plain loads and stores; HIP's uint4 struct is copied with memcpy, which can
// keep arrays of it out of registers).
typedef unsigned int w16_t __attribute__((ext_vector_type(4)));

// Calls f(std::integral_constant<int, K>{}) for K = 0 .. N-1 in order: indices into register arrays stay compile-time
// constants from the start (a plain unrolled loop is unrolled only after the arrays' promotion to registers is
// attempted, and a barrier between their definition and use can then leave them in scratch memory).
template <typename F, int... K>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, K...>) {
  (f(std::integral_constant<int, K>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ float bf16_to_f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bfloat16, round to nearest even (finite inputs).
__device__ __forceinline__ bf16_t f_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t v) { return bf16_to_f(v); }

template <typename T> __device__ __forceinline__ double to_d(T v) { return (double)to_f<T>(v); }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) { return f_to_bf16(v); }

// Backward snapshot modes: the rows in the bank dtype, or a float32 bank's rows as bfloat16, fp8 or int4.
enum { SNAP_BANK = 0, SNAP_BF16 = 1, SNAP_FP8 = 2, SNAP_INT4 = 3 };
// Quantized snapshots (fp8, int4) of float32 rows: groups of SNAP_GROUP columns, each with a power-of-two scale 2^e
// stored as the byte e + 127 (after all elements of all streams: [S][T][W][d / SNAP_GROUP]); elements [S][T][W][d]
// as OCP FP8 E4M3 bytes (fp8) or int4 nibbles in [-7, 7] (two per byte, the even column in the low nibble), each the
// format's nearest value to x / 2^e, ties to even. e is the smallest exponent with (the group's largest magnitude)
// / 2^e <= 448 (E4M3's largest value) or <= 7 (int4).
constexpr int SNAP_GROUP = 16;
// Bytes of a stream's snapshot elements (T W rows) and scales, per row of d columns.
__host__ __device__ inline unsigned long long snap_row_elem_bytes(int mode, int d) {
  return mode == SNAP_FP8 ? (unsigned long long)d : (unsigned long long)d / 2;
}
__host__ __device__ inline unsigned long long snap_row_scale_bytes(int d) { return (unsigned long long)d / SNAP_GROUP; }

// The scale exponent of a group with largest magnitude amax > 0 (a normal float): amax = m 2^e0 with m in [1, 2);
// qmax = 1.75 * 2^k (k = 8 for E4M3, 2 for int4), so amax / 2^(e0 - k) = m 2^k <= qmax exactly when m <= 1.75.
__device__ __forceinline__ int snap_scale_exp(float amax, int k) {
  const uint32_t u = __float_as_uint(amax);
  const int e0 = (int)((u >> 23) & 0xFF) - 127;
  return e0 - k + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
}
// Nearest OCP E4M3 byte to v (|v| <= 448), ties to even.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t sgn = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  if (a < 0.015625f) return sgn | (uint32_t)rintf(a * 512.0f);  // subnormals (spacing 2^-9); 8 is 2^-6 (E = 1)
  const uint32_t u = __float_as_uint(a);
  const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);            // round the 23-bit mantissa to 3 bits
  return sgn | ((((r >> 23) - 120u) << 3) | ((r >> 20) & 7u));    // exponent field: e + 7 = (r >> 23) - 127 + 7
}
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
  const uint32_t E = (b >> 3) & 15u, M = b & 7u;
  const float a = E == 0 ? (float)M * 0.001953125f : __uint_as_float(((E + 120u) << 23) | (M << 20));
  return (b & 0x80u) ? -a : a;
}

// A bank row value after one write event, as the per-token recurrence stores it: float32 rows keep every bit,
// bfloat16 rows are rounded to nearest even after every event (a slot written several times in one chunk goes
// through the same roundings as when its events come one token at a time).
template <typename Bk> __device__ __forceinline__ float bank_round(float v);
template <> __device__ __forceinline__ float bank_round<float>(float v) { return v; }
template <> __device__ __forceinline__ float bank_round<bf16_t>(float v) {
  return __uint_as_float((uint32_t)f_to_bf16(v) << 16);
}

// Sort key half for "larger float first": ascending order of the returned value = descending order of x.
// -0 and +0 map to the same key (they compare equal).
__device__ __forceinline__ uint32_t desc_key(float x) {
  if (x == 0.0f) x = 0.0f;
  uint32_t u = __float_as_uint(x);
  uint32_t m = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // ascending map
  return ~m;
}
__device__ __forceinline__ float desc_key_value(uint32_t k) {
  uint32_t m = ~k;
  uint32_t u = (m & 0x80000000u) ? (m & 0x7FFFFFFFu) : ~m;
  return __uint_as_float(u);
}

// Ascending bitonic sort of n (a power of two) 64-bit keys in LDS by the whole block. Ends with a barrier.
template <int NT>
__device__ __forceinline__ void bitonic_sort_u64(uint64_t* keys, int n) {
  const int tid = threadIdx.x;
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (n >> 1); i += NT) {
        int lo = 2 * i - (i & (stride - 1));
        int hi = lo + stride;
        bool up = (lo & size) == 0;
        uint64_t a = keys[lo], b = keys[hi];
        if ((a > b) == up) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

__host__ __device__ inline int pow2_ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// ------------------------------------------------------------------------------------------- workspace layout
struct WsLayout {
  size_t cand;                                 // uint64 [2][MAX_CAND]: write then read candidate tables
  size_t snorm;                                // float [H][F]: largest sub-key norm of each factor
  size_t widx, wwt, ridx, rwt;                 // [S][T][W|R] slot ids and softmax weights, stream-major
  size_t chunks;                               // [S * nch] chunk plan regions (chunk_layout)
  size_t counts;                               // [S * nch] ChunkCounts
  size_t owner, conflict;                      // shared bank: int32 [H][N] first stream of each slot; int32 flag
  size_t part;                                 // backward: float [slices][S][T][W + R + 2] per-slice dot products
  size_t mrho;                                 // backward: float [S][T][W] read weight of the same slot, or 0
  size_t gent, gcnt, giter, gn;                // backward: token grouping of the fast sweep (bwd_group_kernel)
  size_t mread;                                // backward: float [S][T][R] 1 if the read slot is also written
  size_t ds;                                   // backward: float [S][T][W + R] slot-score gradients
  size_t sgpart;                               // backward: float [row blocks][H][sum n_f][dk] sub-key partial sums
  size_t total;
};

// ------------------------------------------------------------------------------------------- launch wrappers
// Candidate tuples (p_0..p_{F-1}) with prod(p_f + 1) <= k, p_f < kp[f], in lexicographic order; p_f in bits
// [16 f, 16 f + 16) of each entry. One launch builds the tables of `nkinds` plans (table q at tables + q*MAX_CAND).
hipError_t launch_cand_tables(const TopkPlan* plans, int nkinds, int F, uint64_t* tables, hipStream_t st);

// Top-k of every row of one or two query tensors. For kind q (0, 1): queries[q], k = plan[q].k.
//  stream_major != 0: ids/weights go to ws arrays [S][T][k] (+ optional user ids [B,T,H,k]);
//  otherwise ids/scores go to [B,T,H,k].
struct TopkArgs {
  const void* queries[2];
  const void* subkeys;
  const uint64_t* cand[2];
  TopkPlan plan[2];
  int nkinds;
  int stream_major;
  int32_t* ids[2];       // stream-major ids or user ids
  float* vals[2];        // stream-major weights (softmax) or user scores (may be NULL)
  int32_t* user_ids[2];  // optional user ids [B,T,H,k] in stream-major mode
  float* snorm;          // workspace [H][F]: largest sub-key norms for the filtered (MFMA) scoring, or NULL
  int one_query_per_wave;  // few rows (a decode step): one query per wave
  // token window: tokens [t0, t0 + tn) of every batch row (tn = 0: the whole sequence). With B > 1 a window's tn is
  // a multiple of 16, so the query rows a wave or a workgroup takes never straddle two batch rows.
  int t0, tn;
};
hipError_t launch_topk(const Dims& D, const TopkArgs& a, hipStream_t st);

struct PlanArgs {
  const int32_t* widx; const float* wwt; const int32_t* ridx; const float* rwt;
  const void* alpha; const void* beta;
  unsigned char* chunks;  // [S * nch] regions of chunk_layout(C, W, R).bytes
  ChunkCounts* counts;    // [S * nch]
  int scat;               // also write the slot segments and their events (read by loop_kernel only)
  int lanemajor;          // write the gather terms lane-major for the narrow loop (term_pos)
  const int32_t* abort;   // if not NULL and *abort != 0: do nothing (shared-bank conflict)
  int evcode;             // events also carry their term index (Ev::tok bits 16..31), for the snapshot
  int ch0 = 0, chn = 0;   // chunks [ch0, ch0 + chn) of every stream (chn = 0: all of them)
};

// Position of gather term i (of n per token) of chunk-local token t in a chunk's term section. Token-major: t n + i.
// Lane-major (the narrow chunk loop with 16 terms of each kind per lane): lane L = t gpt + i / 16 (gpt = n / 16)
// keeps its terms j = i % 16 as 8 words of two (slot, coefficient) pairs, and word k of all 512 lanes is
// contiguous, so a lane's k-th load is one coalesced 16-byte word: pair index (k * 512 + L) * 2 + j % 2.
__host__ __device__ inline int term_pos(int t, int i, int n, bool lanemajor) {
  if (!lanemajor) return t * n + i;
  const int L = t * (n >> 4) + (i >> 4), j = i & 15;
  return (((j >> 1) * LOOP_NT + L) << 1) + (j & 1);
}
// Position of the int16 last-event code of write term i of token t: token-major t n + i; lane-major as 2 words of
// 8 codes per lane, word k of all lanes contiguous: ((j / 8) * 512 + L) * 8 + j % 8.
__host__ __device__ inline int code_pos(int t, int i, int n, bool lanemajor) {
  if (!lanemajor) return t * n + i;
  const int L = t * (n >> 4) + (i >> 4), j = i & 15;
  return (((j >> 3) * LOOP_NT + L) << 3) + (j & 7);
}
hipError_t launch_plan(const Dims& D, const PlanArgs& a, hipStream_t st);

struct LoopArgs {
  const void* alpha; const void* beta; const void* values;
  const unsigned char* chunks;
  const ChunkCounts* counts;
  void* bank; void* out;
  const int32_t* abort;   // if not NULL and *abort != 0: do nothing (shared-bank conflict)
  void* snap;             // if not NULL: [S][T][W][d] bank dtype, the row of every write event before it (the
                          // held-row or the segmented loop writes it; needs PlanArgs::evcode)
  int snap_mode;          // SNAP_*: the snapshot's rows as stored (float32 bank, held-row loop only for 1-3)
  int ch0 = 0, ch1 = 0;   // chunks [ch0, ch1) of every stream (ch1 = 0: to the last); the bank holds the state
                          // after chunk ch0 - 1
};
hipError_t launch_loop(const Dims& D, const LoopArgs& a, hipStream_t st);
// True if launch_loop runs the held-row variant (which reads last-event codes, not slot segments).
bool loop_held_path(const Dims& D);
// True if launch_loop runs the held-row variant for a call that writes the snapshot.
bool loop_held_snap_ok(const Dims& D);
// True if launch_loop runs the narrow variant (16-byte column slices; also reads last-event codes).
bool loop_narrow_path(const Dims& D);
// Workgroups launch_loop starts (one per stream and column slice), for a call with or without a snapshot.
long long loop_workgroups(const Dims& D, bool snapshot);
// True if it runs the narrow variant with 16 terms of each kind per lane, which reads lane-major terms.
bool loop_narrow_lanemajor(const Dims& D);

// Backward of the write/read (bwd.hip). Ids and weights are the forward's (recomputed top-k, stream-major).
struct BwdArgs {
  const int32_t* widx; const float* wwt; const int32_t* ridx; const float* rwt;  // [S][T][W|R]
  const void* wkeys; const void* rq; const void* subkeys;                         // activation dtype
  const void* alpha; const void* beta; const void* values; const void* gout;      // activation dtype
  void* bank;             // [S][rows][ld] bank dtype: after the forward on entry, before it on return
  const void* snap;       // [S][T][W][d] bank dtype, or the snapshot of snap_mode
  int snap_mode;          // SNAP_*: the snapshot's rows as stored (a float32 bank restored from them for 1-3)
  void* gbank;            // [S][rows][ld]: gradient w.r.t. the bank after the call in, before the call out (float32,
                          // or bfloat16 with grad_bf16)
  int grad_bf16;          // the bank gradient kept in bfloat16 (a bfloat16 bank; the fast reverse sweep only)
  float* gwkeys; float* grq; float* gvalues; float* galpha; float* gbeta; float* gsub;
  float* part; float* ds; float* sgpart;  // workspace
  float* mrho;            // workspace [S][T][W]: rho of the read term of the same token and slot as write term i, or 0
  float* mread;           // workspace [S][T][R]: 1 if read term j's slot is also written by the token, else 0
  // workspace, the fast sweep's token grouping (NULL: one token per iteration): gent [S][T] the entries of each
  // block of G tokens, gcnt [S][ceil(T / G)] their number, giter [S][T] every stream's entries in order, gn [S]
  // their number. An entry is (first token << 4) | token count.
  int32_t* gent; int32_t* gcnt; int32_t* giter; int32_t* gn;
};
// Slices of 16 columns the backward sweep splits a row into, and the row blocks of the sub-key sums.
inline int bwd_slices(const Dims& D) { return (D.d + 15) / 16; }
// Token rows per block of the sub-key sums: a multiple of 16 giving about 256 blocks per head (at least 16 rows).
inline int bwd_row_block_rows(const Dims& D) {
  const int want = (D.B * D.T + 255) / 256;
  return want <= 16 ? 16 : (want + 15) / 16 * 16;
}
inline int bwd_row_blocks(const Dims& D) {
  const int r = bwd_row_block_rows(D);
  return (D.B * D.T + r - 1) / r;
}
hipError_t launch_bwd(const Dims& D, const BwdArgs& a, hipStream_t st);

struct DecodeArgs {
  const void* values; const void* alpha; const void* beta;
  const void* bank_in; void* bank_out; void* out;
  const int32_t* wid; const float* wwt;  // [S][W] write slots and weights (top-k of the step)
  const int32_t* rid; const float* rwt;  // [S][R] read slots and weights
  // the one-launch step computes the top-k itself from these
  const void* queries[2];                // write keys, read queries [S][F dk]
  const void* subkeys;
  TopkPlan plan[2];
  int32_t* user_ids[2];                  // optional [S][W|R] slot ids
};
hipError_t launch_decode(const Dims& D, const DecodeArgs& a, hipStream_t st);
// The whole step (top-k, update, read) in one launch, one workgroup per stream; false if the shape does not fit
// (then nothing is launched).
bool decode_step_fits(const Dims& D, const DecodeArgs& a);
hipError_t launch_decode_step(const Dims& D, const DecodeArgs& a, hipStream_t st);
// K consecutive steps per stream (inputs [B, K, H, ...]) after the batched top-k of all K tokens: a.wid / a.rid hold
// the ids and a.wwt / a.rwt the float32 slot scores (not weights), row-major [B, K, H, W|R]. Bitwise equal to K
// one-launch steps; needs the shapes decode_step_fits accepts.
hipError_t launch_decode_steps(const Dims& D, const DecodeArgs& a, int K, hipStream_t st);
hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t st);
// Shared bank: owner[h][slot] = -1 for every slot, flag = 0; then every addressed slot is claimed by its stream and
// a slot claimed by two streams of a head sets the flag.
hipError_t launch_shared_check(const Dims& D, const int32_t* widx, const int32_t* ridx, int32_t* owner,
                               int32_t* flag, hipStream_t st);


}  // namespace sdm
