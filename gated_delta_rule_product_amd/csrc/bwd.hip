// Backward of the write/read: gradients of the write keys, read queries, values, both gates, the sub-keys and the
// bank before the call; the bank itself steps back to its state before the call. sparse-delta-memory CHANGELOG.md
// 2.0.0: "Deterministic" (every gradient bitwise repeatable, no float atomics), "New" (exact product-key top-k with
// a deterministic sparse backward), "Known limitations" (the first backward restores the bank in place).
//
// The reverse-mode derivative of the per-token recurrence (write: r = sum_i w_i P_i, delta = beta (v - alpha r),
// M[S_i] <- alpha P_i + w_i delta; then the read out = sum_j rho_j M[R_j]), tokens in reverse, with G the adjoint
// of the bank (the gradient buffer, updated in place):
//   read:   d rho_j = <dout, M[R_j]>,  G[R_j] += rho_j dout
//   write:  g_i = G[S_i],  D = sum_i w_i g_i,  dv = beta D,  d beta = <D, v - alpha r>,
//           d alpha = sum_i <g_i, P_i> - beta <D, r>,  d w_i = <g_i, delta> - alpha beta <D, P_i>,
//           G[S_i] <- alpha g_i - alpha beta w_i D,  M[S_i] <- P_i  (the bank steps back one token)
//   weights: softmax derivative d s_i = w_i (d w_i - sum_k w_k d w_k); scores: a slot score is the sum of its factor
//           scores <x^(f), C_f[i_f]>, so d x^(f) = sum_i d s_i C_f[i_f] and d C_f[i] = sum d s x^(f) over the terms
//           whose factor-f sub-key is i.
// P_i (the row of S_i before the token's write) is the forward's snapshot. G, M and D are column-local, so one
// workgroup runs one (stream, 16-column slice) over every token; only the dot products cross slices: each slice
// writes its partial sums and a second kernel adds them over the slices in order. Every sum has a fixed order.
#include "bwd_shape.h"
#include "sdm_internal.h"
#include "topk_wave.h"  // wave_sync, lanes_below_mask

namespace sdm {

constexpr int BWD_NT = 512;
constexpr int BWD_COLS = 16;  // columns per slice: 128 groups of 4 lanes, 4 columns per lane

// Four consecutive bank elements: raw bits (for the restore) and floats.
template <typename Bk> struct Raw4;
template <> struct Raw4<float> {
  typedef w16_t T;
  __device__ static T load(const float* p) { return *(const w16_t*)p; }
  __device__ static void store(float* p, T x) { *(w16_t*)p = x; }
  __device__ static void unpack(T x, float* v) {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __uint_as_float(x[k]);
  }
};
typedef unsigned int w8_t __attribute__((ext_vector_type(2)));  // 8 bytes as a native vector (not a struct)
template <> struct Raw4<bf16_t> {
  typedef w8_t T;
  __device__ static T load(const bf16_t* p) { return *(const w8_t*)p; }
  __device__ static void store(bf16_t* p, T x) { *(w8_t*)p = x; }
  __device__ static void unpack(T x, float* v) {
    v[0] = __uint_as_float(x[0] << 16);
    v[1] = __uint_as_float(x[0] & 0xFFFF0000u);
    v[2] = __uint_as_float(x[1] << 16);
    v[3] = __uint_as_float(x[1] & 0xFFFF0000u);
  }
};

// An activation element through a 32-bit word: the float itself, or for bfloat16 the aligned 4-byte word that
// contains it (never crossing a page), its half picked where the value is used. A 16-bit value kept in a
// loop-carried register gets re-masked by the compiler right after its load, which makes it wait for that load.
template <typename A> struct Word;
template <> struct Word<float> {
  __device__ static uint32_t load(const float* p) { return __float_as_uint(*p); }
  __device__ static float get(uint32_t w, const float*) { return __uint_as_float(w); }
};
template <> struct Word<bf16_t> {
  __device__ static uint32_t load(const bf16_t* p) { return *(const uint32_t*)((uintptr_t)p & ~(uintptr_t)3); }
  __device__ static float get(uint32_t w, const bf16_t* p) {
    return __uint_as_float(((uintptr_t)p & 2) ? (w & 0xFFFF0000u) : (w << 16));
  }
};

__device__ __forceinline__ float sum4_lanes(float x) {  // over the 4 lanes of a group; equal on all four
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x;
}
// DPP lane moves (VALU, no LDS round trip): within quads (quad_perm) and rotations within rows of 16 lanes.
template <int CTRL> __device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_QUAD_XOR1 = 0xB1, DPP_QUAD_XOR2 = 0x4E, DPP_ROW_ROR4 = 0x124, DPP_ROW_ROR8 = 0x128;

template <int L> __device__ __forceinline__ float sum_group_lanes(float x) {  // over the L lanes of a group
  if (L >= 2) x += dpp_f<DPP_QUAD_XOR1>(x);
  if (L >= 4) x += dpp_f<DPP_QUAD_XOR2>(x);
  return x;
}

// Over the groups of a wave, per column quad: the sum of the lanes with this lane's index mod L (L = 2 or 4 lanes
// per group), in a fixed order; every lane ends with its class's sum.
template <int L> __device__ __forceinline__ float sum_wave_groups(float x) {
  if (L == 2) x += dpp_f<DPP_QUAD_XOR2>(x);  // the other group of the quad
  x += dpp_f<DPP_ROW_ROR4>(x);               // the row's other quads
  x += dpp_f<DPP_ROW_ROR8>(x);
  x += __shfl_xor(x, 16);                    // the other rows
  x += __shfl_xor(x, 32);
  return x;
}

__host__ __device__ inline size_t bwd_sweep_lds(int W) { return (size_t)W * (2 * BWD_COLS + 2) * 4 + 8 * BWD_COLS * 4; }

template <typename A, typename Bk>
__global__ __launch_bounds__(BWD_NT) void bwd_sweep_kernel(Dims D, BwdArgs a, int nsl) {
  extern __shared__ __align__(16) float lds_f[];
  const int W = D.W, R = D.R, T = D.T, d = D.d;
  float* sG = lds_f;                      // [W][16] g_i
  float* sP = sG + W * BWD_COLS;          // [W][16] P_i
  float* sW = sP + W * BWD_COLS;          // [W] w_i
  float* sGP = sW + W;                    // [W] slice partial <g_i, P_i>
  float* sDel = sGP + W;                  // [16] D
  float* sRr = sDel + BWD_COLS;           // [16] r
  float* sDt = sRr + BWD_COLS;            // [16] delta
  float* sSc = sDt + BWD_COLS;            // [2]  slice partials of d alpha and d beta

  const int nblk = gridDim.x;
  int wk = blockIdx.x;
  if ((nblk & 7) == 0) wk = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);  // XCD-aware: slices of a stream together
  const int st = wk / nsl, slice = wk % nsl;
  const int b = st / D.H, h = st % D.H;
  const int tid = threadIdx.x, grp = tid >> 2, q = tid & 3;
  const int col = slice * BWD_COLS + q * 4;
  const bool valid = col < d;  // d % 4 == 0: a lane's four columns are all inside or all outside
  const int P = W + R + 2;
  Bk* bank = (Bk*)a.bank + (long long)st * D.rows * D.ld;
  float* gbank = (float*)a.gbank + (long long)st * D.rows * D.ld;
  const Bk* snap = (const Bk*)a.snap + (long long)st * T * W * d;
  const A* gout = (const A*)a.gout;
  const A* values = (const A*)a.values;

  for (int t = T - 1; t >= 0; --t) {
    const long long so = (long long)st * T + t;             // stream-major token index
    const long long row = ((long long)b * T + t) * D.H + h;  // [B, T, H] row
    const float al = to_f<A>(((const A*)a.alpha)[row]);
    const float be = to_f<A>(((const A*)a.beta)[row]);
    float* part = a.part + ((long long)slice * D.S * T + so) * P;
    float dout[4] = {0.f, 0.f, 0.f, 0.f};
    if (valid) {
#pragma unroll
      for (int k = 0; k < 4; ++k) dout[k] = to_f<A>(gout[row * d + col + k]);
    }
    // the read: d rho partials, G[R_j] += rho_j dout
    for (int j = grp; j < R; j += BWD_NT / 4) {
      const int slot = a.ridx[so * R + j];
      const float rho = a.rwt[so * R + j];
      float m[4] = {0.f, 0.f, 0.f, 0.f};
      if (valid) {
        Raw4<Bk>::unpack(Raw4<Bk>::load(bank + (long long)slot * D.ld + col), m);
        float* gp = gbank + (long long)slot * D.ld + col;
        float4 g = *(float4*)gp;
        g.x += rho * dout[0]; g.y += rho * dout[1]; g.z += rho * dout[2]; g.w += rho * dout[3];
        *(float4*)gp = g;
      }
      const float dot = sum4_lanes(((dout[0] * m[0] + dout[1] * m[1]) + dout[2] * m[2]) + dout[3] * m[3]);
      if (q == 0) part[W + j] = dot;
    }
    __syncthreads();
    // the write, first half: g_i and P_i of the slice into LDS
    for (int i = grp; i < W; i += BWD_NT / 4) {
      const int slot = a.widx[so * W + i];
      float g[4] = {0.f, 0.f, 0.f, 0.f}, p[4] = {0.f, 0.f, 0.f, 0.f};
      if (valid) {
        const float4 gv = *(const float4*)(gbank + (long long)slot * D.ld + col);
        g[0] = gv.x; g[1] = gv.y; g[2] = gv.z; g[3] = gv.w;
        Raw4<Bk>::unpack(Raw4<Bk>::load(snap + ((long long)t * W + i) * d + col), p);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        sG[i * BWD_COLS + q * 4 + k] = g[k];
        sP[i * BWD_COLS + q * 4 + k] = p[k];
      }
      const float gp = sum4_lanes(((g[0] * p[0] + g[1] * p[1]) + g[2] * p[2]) + g[3] * p[3]);
      if (q == 0) {
        sGP[i] = gp;
        sW[i] = a.wwt[so * W + i];
      }
    }
    __syncthreads();
    // D and r per column, sum of <g_i, P_i>, each in term order
    if (tid < BWD_COLS) {
      float s = 0.f;
      for (int i = 0; i < W; ++i) s += sW[i] * sG[i * BWD_COLS + tid];
      sDel[tid] = s;
    } else if (tid < 2 * BWD_COLS) {
      const int c = tid - BWD_COLS;
      float s = 0.f;
      for (int i = 0; i < W; ++i) s += sW[i] * sP[i * BWD_COLS + c];
      sRr[c] = s;
    } else if (tid == 2 * BWD_COLS) {
      float s = 0.f;
      for (int i = 0; i < W; ++i) s += sGP[i];
      sSc[0] = s;
    }
    __syncthreads();
    // delta, dv and the gate partials (one wave: columns on lanes 0..15)
    if (tid < 64) {
      const int c = tid & (BWD_COLS - 1);
      const int cc = slice * BWD_COLS + c;
      const bool cv = tid < BWD_COLS && cc < d;
      const float Dl = sDel[c], r = sRr[c];
      const float v = cv ? to_f<A>(values[row * d + cc]) : 0.f;
      const float e = v - al * r;  // v - alpha r
      float db = cv ? Dl * e : 0.f;
      float rd = cv ? Dl * r : 0.f;
      if (cv) {
        sDt[c] = be * e;
        a.gvalues[row * d + cc] = be * Dl;
      } else if (tid < BWD_COLS) {
        sDt[c] = 0.f;
      }
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) {  // fixed tree over the 16 columns
        db += __shfl_xor(db, o);
        rd += __shfl_xor(rd, o);
      }
      if (tid == 0) {
        part[W + R] = sSc[0] - be * rd;
        part[W + R + 1] = db;
      }
    }
    __syncthreads();
    // the write, second half: d w_i partials, G[S_i] <- alpha g_i - alpha beta w_i D, M[S_i] <- P_i
    const float ab = al * be;
    for (int i = grp; i < W; i += BWD_NT / 4) {
      float g[4], p[4], dl[4], Dl[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        g[k] = sG[i * BWD_COLS + q * 4 + k];
        p[k] = sP[i * BWD_COLS + q * 4 + k];
        dl[k] = sDt[q * 4 + k];
        Dl[k] = sDel[q * 4 + k];
      }
      const float gd = sum4_lanes(((g[0] * dl[0] + g[1] * dl[1]) + g[2] * dl[2]) + g[3] * dl[3]);
      const float Dp = sum4_lanes(((Dl[0] * p[0] + Dl[1] * p[1]) + Dl[2] * p[2]) + Dl[3] * p[3]);
      if (q == 0) part[i] = gd - ab * Dp;
      if (valid) {
        const int slot = a.widx[so * W + i];
        const float cw = ab * sW[i];
        *(float4*)(gbank + (long long)slot * D.ld + col) =
            make_float4(al * g[0] - cw * Dl[0], al * g[1] - cw * Dl[1], al * g[2] - cw * Dl[2], al * g[3] - cw * Dl[3]);
        Raw4<Bk>::store(bank + (long long)slot * D.ld + col, Raw4<Bk>::load(snap + ((long long)t * W + i) * d + col));
      }
    }
    __syncthreads();
  }
}

// For every write term (t, i): the weight rho_j of the read term of the same token with the same slot, or 0; for
// every read term: 1 if the token also writes its slot (slots are distinct within one token's writes and within its
// reads, so there is at most one match). One wave per token.
__global__ __launch_bounds__(64) void bwd_match_kernel(Dims D, BwdArgs a) {
  __shared__ int32_t srs[MAX_K], sws[MAX_K];
  __shared__ float srho[MAX_K];
  const long long so = blockIdx.x;
  const int W = D.W, R = D.R;
  for (int j = threadIdx.x; j < R; j += 64) {
    srs[j] = a.ridx[so * R + j];
    srho[j] = a.rwt[so * R + j];
  }
  for (int i = threadIdx.x; i < W; i += 64) sws[i] = a.widx[so * W + i];
  __syncthreads();
  for (int i = threadIdx.x; i < W; i += 64) {
    const int slot = sws[i];
    float r = 0.f;
    for (int j = 0; j < R; ++j)
      if (srs[j] == slot) r = srho[j];
    a.mrho[so * W + i] = r;
  }
  for (int j = threadIdx.x; j < R; j += 64) {
    const int slot = srs[j];
    float f = 0.f;
    for (int i = 0; i < W; ++i)
      if (sws[i] == slot) f = 1.f;
    a.mread[so * R + j] = f;
  }
}

// The same sweep for W, R <= 128 (one write and one read term per lane group), two barriers and one HBM load round
// trip per step. A step takes one token, or a run of consecutive tokens with pairwise disjoint slots (at most one
// per block of wb waves; bwd_group_kernel), each token on its own block with its own step's arithmetic: the read
// rows, their G rows and the write terms' G rows of the step's tokens are loaded together; the snapshot rows, gates,
// output gradient and values of the next step and the ids of the one after are loaded a step ahead (read-only data)
// and kept raw until used (a conversion next to its load would make the compiler wait for every earlier load). A
// write slot that the token also reads gets the read's G update (rho_j dout, rho_j from bwd_match_kernel) added in
// registers, since its loaded G row predates that update. Sums over a token's write terms: a fixed shuffle tree
// inside each wave, then every lane adds the wave partials of its token's block, for its own columns, in order (the
// same sums on every lane, so no barrier for a broadcast). Every store of a step comes after its last use of loaded
// data: loads and stores share one memory counter, and a wait for a load issued before a store would also wait for
// the store. So the read's G update is stored with the write's, and not at all when the token also writes that slot
// (the write's G row includes it). The next step's row loads follow the end-of-step barrier, after every store of
// this step in the workgroup's program order (one CU: its vector memory pipeline keeps that order).
// LPG lanes per term group (4 columns each): slices of 4 LPG columns, BWD_FAST_GROUPS groups.
// Sk: the snapshot's element type (Bk, or bfloat16 rows of a float32 bank, which restore the bank widened). SQ:
// SNAP_FP8 / SNAP_INT4 for a quantized snapshot of a float32 bank (Sk unused): a lane reads its 4 elements (4 or 2
// bytes) and its 16-column group's scale byte, and the bank is restored from the dequantized values.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
template <int SQ> struct SnapQ {  // the raw snapshot piece of a lane: x = elements, y = scale byte
  typedef u32x2_t T;
  __device__ static T load(const unsigned char* el, const unsigned char* sc, long long row, int d, int col) {
    const long long e = row * d + col;
    const uint32_t x = SQ == SNAP_FP8 ? *(const uint32_t*)(el + e) : (uint32_t)*(const uint16_t*)(el + e / 2);
    return u32x2_t{x, (uint32_t)sc[row * (d / SNAP_GROUP) + col / SNAP_GROUP]};
  }
  __device__ static void unpack(T r, float* v) {
    const float s = ldexpf(1.0f, (int)r.y - 127);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float q = SQ == SNAP_FP8 ? e4m3_decode((r.x >> (8 * k)) & 0xFFu)
                                     : (float)((int)(((r.x >> (4 * k)) & 0xFu) << 28) >> 28);
      v[k] = q * s;
    }
  }
};

// Four consecutive entries of the adjoint bank (the bank gradient): float32, or bfloat16 (the bank dtype of a
// bfloat16 bank, CHANGELOG 2.0.0 "Deterministic": float32 accumulation is the opt-in), rounded at every store.
template <typename Gk> struct GRow;
template <> struct GRow<float> {
  __device__ static float4 load(const float* p) { return *(const float4*)p; }
  __device__ static void store(float* p, float4 v) { *(float4*)p = v; }
  __device__ static float round(float v) { return v; }
};
template <> struct GRow<bf16_t> {
  __device__ static float4 load(const bf16_t* p) {
    const u32x2_t w = *(const u32x2_t*)p;
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                       __uint_as_float(w.y & 0xFFFF0000u));
  }
  __device__ static void store(bf16_t* p, float4 v) {
    *(u32x2_t*)p = u32x2_t{(uint32_t)f_to_bf16(v.x) | ((uint32_t)f_to_bf16(v.y) << 16),
                           (uint32_t)f_to_bf16(v.z) | ((uint32_t)f_to_bf16(v.w) << 16)};
  }
  __device__ static float round(float v) { return bank_round<bf16_t>(v); }
};

template <typename A, typename Bk, int LPG, typename Sk = Bk, int SQ = SNAP_BANK, typename Gk = float>
__global__ __launch_bounds__(BWD_FAST_GROUPS * LPG) void bwd_sweep_fast_kernel(Dims D, BwdArgs a, int nsl, int wb) {
  constexpr int COLS = 4 * LPG, NW = BWD_FAST_GROUPS * LPG / 64;
  constexpr bool QS = SQ == SNAP_FP8 || SQ == SNAP_INT4;
  __shared__ __align__(16) float sRedD[NW][COLS];
  __shared__ __align__(16) float sRedR[NW][COLS];
  __shared__ float sRedGP[NW];
  typedef typename Raw4<Bk>::T RawT;
  typedef typename std::conditional<QS, typename SnapQ<SQ>::T, typename Raw4<Sk>::T>::type RawS;
  typedef typename Raw4<A>::T ARaw;
  const int W = D.W, R = D.R, T = D.T, d = D.d;
  const int nblk = gridDim.x;
  int wk = blockIdx.x;
  if ((nblk & 7) == 0) wk = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int st = wk / nsl, slice = wk % nsl;
  const int b = st / D.H, h = st % D.H;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, grp = tid / LPG, q = tid % LPG;
  const int col = slice * COLS + q * 4;
  const bool valid = col < d;
  // token blocks of wb waves: block `sub` takes the iteration's sub-th token, its group lgrp that token's terms
  const int sub = wv / wb, lgrp = grp - sub * wb * (64 / LPG);
  const bool blk_ok = (sub + 1) * wb <= NW;               // a whole block (waves past the last one idle)
  const int jr = min(lgrp, R - 1), jw = min(lgrp, W - 1);  // clamped term indices: every lane loads in range
  const int P = W + R + 2;
  Bk* bank = (Bk*)a.bank + (long long)st * D.rows * D.ld;
  Gk* gbank = (Gk*)a.gbank + (long long)st * D.rows * D.ld;
  const Sk* snap = (const Sk*)a.snap + (long long)st * T * W * d;
  // quantized snapshot: the elements of every stream, then the scale bytes of every stream
  const unsigned long long qrows = (unsigned long long)T * W;
  const unsigned char* qel = (const unsigned char*)a.snap + (QS ? st * qrows * snap_row_elem_bytes(SQ, d) : 0);
  const unsigned char* qsc = (const unsigned char*)a.snap +
                             (QS ? (unsigned long long)D.S * qrows * snap_row_elem_bytes(SQ, d) +
                                       st * qrows * snap_row_scale_bytes(d)
                                 : 0);
  const A* gout = (const A*)a.gout;
  const A* values = (const A*)a.values;
  const A* alpha = (const A*)a.alpha;
  const A* beta = (const A*)a.beta;
  const int zero = (int)__builtin_amdgcn_mbcnt_lo(0u, 0u);  // 0, not provably uniform: keeps the gate loads vector
  const int dcol = valid ? col : 0;

  auto load_ids = [&](int t, int& rs, float& rho, int& ws, float& w, float& mr, float& mw) {
    const long long so = (long long)st * T + t;
    rs = a.ridx[so * R + jr];
    rho = a.rwt[so * R + jr];
    ws = a.widx[so * W + jw];
    w = a.wwt[so * W + jw];
    mr = a.mrho[so * W + jw];
    mw = a.mread[so * R + jr];
  };
  // (separate variables, not a struct: a struct copy becomes a byte-wise memcpy that needs the loaded data at once;
  // 16-bit values in 32-bit words: kept in 16 bits the compiler re-masks them right after their load)
  auto load_tok = [&](int t, uint32_t& al_, uint32_t& be_, ARaw& v_, ARaw& dout_, RawS& sp_) {
    const long long row = ((long long)b * T + t) * D.H + h;
    al_ = Word<A>::load(alpha + row + zero);
    be_ = Word<A>::load(beta + row + zero);
    dout_ = Raw4<A>::load(gout + row * d + dcol);
    v_ = Raw4<A>::load(values + row * d + dcol);
    if constexpr (QS)
      sp_ = SnapQ<SQ>::load(qel, qsc, (long long)t * W + jw, d, dcol);
    else
      sp_ = Raw4<Sk>::load(snap + ((long long)t * W + jw) * d + dcol);
  };

  // iterations: entry (first token << 4) | number of tokens; the tokens of one entry are consecutive, in
  // decreasing order, and address pairwise disjoint slots (bwd_group_kernel); without grouping, one token each
  // (the entry is then the token itself)
  const bool grouped = a.giter != nullptr;
  const int niter = grouped ? a.gn[st] : T;
  auto entry = [&](int it) -> int32_t {
    it = min(it, niter - 1);  // past the last: the last again (its loads stay in range; it stores nothing)
    return grouped ? a.giter[(long long)st * T + it] : T - 1 - it;
  };
  auto first_tok = [&](int32_t e) { return grouped ? e >> 4 : e; };
  auto tok_of = [&](int32_t e) { return blk_ok ? max(first_tok(e) - sub, 0) : first_tok(e); };
  int32_t e0 = entry(0), e1 = entry(1), e2 = entry(2);

  int rs, ws, rs1, ws1;
  float rho, w, mr, mw, rho1, w1, mr1, mw1;
  uint32_t c_al, c_be;
  ARaw c_v, c_dout;
  RawS c_sp;
  load_ids(tok_of(e0), rs, rho, ws, w, mr, mw);
  load_ids(tok_of(e1), rs1, rho1, ws1, w1, mr1, mw1);
  load_tok(tok_of(e0), c_al, c_be, c_v, c_dout, c_sp);
  // the loop's first values in before it starts: a load still in flight on the way in would make the loop head wait
  // for everything outstanding, the previous token's stores included, on every token
  asm volatile("" ::"v"(rs), "v"(ws), "v"(rho), "v"(w), "v"(mr), "v"(mw), "v"(rs1), "v"(ws1), "v"(rho1), "v"(w1),
               "v"(mr1), "v"(mw1), "v"(c_al), "v"(c_be), "v"(c_v), "v"(c_dout), "v"(c_sp));

  for (int it = 0; it < niter; ++it) {
    const int t = tok_of(e0);
    const bool act = blk_ok && sub < (grouped ? (e0 & 15) : 1);  // this block has a token in this iteration
    const bool hasR = act && lgrp < R, hasW = act && lgrp < W;
    const int32_t e3 = entry(it + 3);
    const long long so = (long long)st * T + t;
    const long long row = ((long long)b * T + t) * D.H + h;
    float* part = a.part + ((long long)slice * D.S * T + so) * P;
    // this token's rows (clamped ids: in range on every lane)
    const RawT rb = Raw4<Bk>::load(bank + (long long)rs * D.ld + dcol);
    float4 rg = GRow<Gk>::load(gbank + (long long)rs * D.ld + dcol);
    const float4 wg = GRow<Gk>::load(gbank + (long long)ws * D.ld + dcol);
    // ahead: the next iteration's inputs and snapshot rows, the ids of the one after
    uint32_t n_al, n_be;
    ARaw n_v, n_dout;
    RawS n_sp;
    int rs2, ws2;
    float rho2, w2, mr2, mw2;
    load_tok(tok_of(e1), n_al, n_be, n_v, n_dout, n_sp);
    load_ids(tok_of(e2), rs2, rho2, ws2, w2, mr2, mw2);
    const float al = Word<A>::get(c_al, alpha + row), be = Word<A>::get(c_be, beta + row);
    float dout[4], v[4];
    Raw4<A>::unpack(c_dout, dout);
    Raw4<A>::unpack(c_v, v);
    if (!valid) dout[0] = dout[1] = dout[2] = dout[3] = v[0] = v[1] = v[2] = v[3] = 0.f;
    // the read: d rho partial, G[R_j] += rho_j dout (stored at the end of the token)
    float m[4];
    Raw4<Bk>::unpack(rb, m);
    const float rdot = sum_group_lanes<LPG>(((dout[0] * m[0] + dout[1] * m[1]) + dout[2] * m[2]) + dout[3] * m[3]);
    rg.x += rho * dout[0]; rg.y += rho * dout[1]; rg.z += rho * dout[2]; rg.w += rho * dout[3];
    // the write: g_i (plus this token's read update of the same slot), P_i
    float g[4] = {GRow<Gk>::round(wg.x + mr * dout[0]), GRow<Gk>::round(wg.y + mr * dout[1]),
                  GRow<Gk>::round(wg.z + mr * dout[2]), GRow<Gk>::round(wg.w + mr * dout[3])}, pp[4];
    if constexpr (QS)
      SnapQ<SQ>::unpack(c_sp, pp);
    else
      Raw4<Sk>::unpack(c_sp, pp);
    if (!valid) pp[0] = pp[1] = pp[2] = pp[3] = 0.f;
    // the looked-ahead values are in (issued before this token's rows, which were just waited for): take them
    // here, before any store, so that moving them into place at the end of the token waits for nothing
    asm volatile("" ::"v"(rs2), "v"(ws2), "v"(rho2), "v"(w2), "v"(mr2), "v"(mw2), "v"(n_al), "v"(n_be), "v"(n_v),
                 "v"(n_dout), "v"(n_sp));
    // sums over the write terms: D = sum w g, r = sum w P, sum <g, P>
    float cD[4], cR[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      cD[k] = hasW ? w * g[k] : 0.f;
      cR[k] = hasW ? w * pp[k] : 0.f;
    }
    float gp = hasW ? sum_group_lanes<LPG>(((g[0] * pp[0] + g[1] * pp[1]) + g[2] * pp[2]) + g[3] * pp[3]) : 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // over the groups of the wave (fixed order; lanes 0..LPG-1 are used)
      cD[k] = sum_wave_groups<LPG>(cD[k]);
      cR[k] = sum_wave_groups<LPG>(cR[k]);
    }
    gp = sum_wave_groups<LPG>(gp);
    if (lane < LPG) {
      *(float4*)&sRedD[wv][lane * 4] = make_float4(cD[0], cD[1], cD[2], cD[3]);
      *(float4*)&sRedR[wv][lane * 4] = make_float4(cR[0], cR[1], cR[2], cR[3]);
      if (lane == 0) sRedGP[wv] = gp;
    }
    __syncthreads();
    // D, r and delta of this lane's four columns (the block's wave partials in order, on every lane alike)
    float Dl[4] = {0.f, 0.f, 0.f, 0.f}, r[4] = {0.f, 0.f, 0.f, 0.f}, dl[4];
    const int k0 = blk_ok ? sub * wb : 0;
    for (int k = k0; k < k0 + wb; ++k) {
      const float4 x = *(const float4*)&sRedD[k][q * 4];
      const float4 y = *(const float4*)&sRedR[k][q * 4];
      Dl[0] += x.x; Dl[1] += x.y; Dl[2] += x.z; Dl[3] += x.w;
      r[0] += y.x; r[1] += y.y; r[2] += y.z; r[3] += y.w;
    }
    float e[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      e[k] = v[k] - al * r[k];  // v - alpha r
      dl[k] = be * e[k];
    }
    if (act && lgrp == 0) {  // dv, and the slice partials of d alpha and d beta (LPG lanes x 4 columns)
      if (valid)
        *(float4*)(a.gvalues + row * d + col) = make_float4(be * Dl[0], be * Dl[1], be * Dl[2], be * Dl[3]);
      const float db = sum_group_lanes<LPG>(((Dl[0] * e[0] + Dl[1] * e[1]) + Dl[2] * e[2]) + Dl[3] * e[3]);
      const float rd = sum_group_lanes<LPG>(((Dl[0] * r[0] + Dl[1] * r[1]) + Dl[2] * r[2]) + Dl[3] * r[3]);
      if (q == 0) {
        float gps = 0.f;
        for (int k = k0; k < k0 + wb; ++k) gps += sRedGP[k];
        part[W + R] = gps - be * rd;
        part[W + R + 1] = db;
      }
    }
    // the read's stores (its G row only if the token does not also write the slot)
    if (hasR) {
      if (q == 0) part[W + lgrp] = rdot;
      if (valid && mw == 0.f) GRow<Gk>::store(gbank + (long long)rs * D.ld + col, rg);
    }
    // d w partials, G[S_i] <- alpha g_i - alpha beta w_i D, M[S_i] <- P_i
    if (hasW) {
      const float ab = al * be;
      const float gd = sum_group_lanes<LPG>(((g[0] * dl[0] + g[1] * dl[1]) + g[2] * dl[2]) + g[3] * dl[3]);
      const float Dp = sum_group_lanes<LPG>(((Dl[0] * pp[0] + Dl[1] * pp[1]) + Dl[2] * pp[2]) + Dl[3] * pp[3]);
      if (q == 0) part[lgrp] = gd - ab * Dp;
      if (valid) {
        const float cw = ab * w;
        GRow<Gk>::store(gbank + (long long)ws * D.ld + col, make_float4(
            al * g[0] - cw * Dl[0], al * g[1] - cw * Dl[1], al * g[2] - cw * Dl[2], al * g[3] - cw * Dl[3]));
        if constexpr (std::is_same<Sk, Bk>::value && !QS)
          Raw4<Bk>::store(bank + (long long)ws * D.ld + col, c_sp);
        else  // a float32 bank from bfloat16 or quantized snapshot rows (pp: the widened values)
          *(float4*)(bank + (long long)ws * D.ld + col) = make_float4(pp[0], pp[1], pp[2], pp[3]);
      }
    }
    // next iteration
    rs = rs1; rho = rho1; ws = ws1; w = w1; mr = mr1; mw = mw1;
    rs1 = rs2; rho1 = rho2; ws1 = ws2; w1 = w2; mr1 = mr2; mw1 = mw2;
    c_al = n_al; c_be = n_be; c_v = n_v; c_dout = n_dout; c_sp = n_sp;
    e0 = e1; e1 = e2; e2 = e3;
    __syncthreads();
  }
}

// One workgroup per token row (stream-major): slice sums, gate gradients, softmax derivative (slot-score gradients
// into the workspace), and the key and query gradients d x^(f) = sum_i d s_i C_f[i_f] (terms in order).
template <typename A>
__global__ __launch_bounds__(256) void bwd_token_kernel(Dims D, BwdArgs a, int nsl) {
  __shared__ float sd[MAX_K * 2 + 2];
  __shared__ float swt[MAX_K * 2];              // the terms' softmax weights (write, then read)
  __shared__ float sm[2];
  __shared__ uint16_t ssub[MAX_K * 2][MAX_F];  // factor sub-key of every term (n_f <= 4096)
  const long long so = blockIdx.x;
  const int T = D.T, W = D.W, R = D.R, P = W + R + 2;
  const int st = (int)(so / T), t = (int)(so % T);
  const int b = st / D.H, h = st % D.H;
  const long long row = ((long long)b * T + t) * D.H + h;
  // slice partials added in slice order (eight loads a thread in flight), the weights and slot ids alongside
  constexpr int NB = 8;
  for (int p = threadIdx.x; p < P; p += 256) {
    float s = 0.f;
    int sl = 0;
    for (; sl + NB <= nsl; sl += NB) {
      float v[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) v[u] = a.part[((long long)(sl + u) * D.S * T + so) * P + p];
#pragma unroll
      for (int u = 0; u < NB; ++u) s += v[u];
    }
    for (; sl < nsl; ++sl) s += a.part[((long long)sl * D.S * T + so) * P + p];
    sd[p] = s;
  }
  int sid = 0;  // the slot id of term threadIdx.x (W + R <= 256 here; the loop below covers more)
  for (int i = threadIdx.x; i < W + R; i += 256) {
    swt[i] = i < W ? a.wwt[so * W + i] : a.rwt[so * R + (i - W)];
    sid = i < W ? a.widx[so * W + i] : a.ridx[so * R + (i - W)];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a.galpha[row] = sd[W + R];
    a.gbeta[row] = sd[W + R + 1];
    float m = 0.f;
    for (int i = 0; i < W; ++i) m += swt[i] * sd[i];
    sm[0] = m;
  } else if (threadIdx.x == 64) {
    float m = 0.f;
    for (int j = 0; j < R; ++j) m += swt[W + j] * sd[W + j];
    sm[1] = m;
  }
  __syncthreads();
  float* ds = a.ds + so * (W + R);
  for (int i = threadIdx.x; i < W + R; i += 256) {
    const bool wr = i < W;
    const float v = swt[i] * (sd[i] - sm[wr ? 0 : 1]);
    sd[i] = v;
    ds[i] = v;
    // mixed radix, factor 0 most significant (slot ids are below 2^31)
    int id = W + R <= 256 ? sid : (wr ? a.widx[so * W + i] : a.ridx[so * R + (i - W)]);
    for (int f = D.F - 1; f >= 0; --f) {
      ssub[i][f] = (uint16_t)(id % D.widths[f]);
      id /= D.widths[f];
    }
  }
  __syncthreads();
  long long sumn = 0;
  for (int f = 0; f < D.F; ++f) sumn += D.widths[f];
  const A* sub = (const A*)a.subkeys + (long long)h * sumn * D.dk;
  const int Fdk = D.F * D.dk;
  for (int x = threadIdx.x; x < 2 * Fdk; x += 256) {
    const int kind = x >= Fdk;
    const int fc = x - kind * Fdk;
    const int f = fc / D.dk, c = fc % D.dk;
    long long off = 0;
    for (int g = 0; g < f; ++g) off += D.widths[g];
    const int n = kind ? R : W, i0 = kind ? W : 0;
    const A* subc = sub + off * D.dk + c;
    float acc = 0.f;
    int i = 0;
    for (; i + NB <= n; i += NB) {  // the terms in order, eight sub-key loads in flight
      float y[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) y[u] = to_f<A>(subc[(long long)ssub[i0 + i + u][f] * D.dk]);
#pragma unroll
      for (int u = 0; u < NB; ++u) acc += sd[i0 + i + u] * y[u];
    }
    for (; i < n; ++i) acc += sd[i0 + i] * to_f<A>(subc[(long long)ssub[i0 + i][f] * D.dk]);
    (kind ? a.grq : a.gwkeys)[row * Fdk + fc] = acc;
  }
}

// Sub-key partial sums of one block of token rows of head h (rows ordered b-major; bwd_row_block_rows each),
// factor f, `cb` columns: one wave, lane c owns column c of every sub-key of the factor (LDS accumulators), terms in
// order. The factor-f sub-key of every term and the slot-score gradients of 16 rows at a time are staged in LDS.
constexpr int BWD_SK_ROWS = 16;

template <typename A>
__global__ __launch_bounds__(64) void bwd_subkey_kernel(Dims D, BwdArgs a, int cb, int ncb, int rows_per_block) {
  extern __shared__ __align__(16) float acc[];  // [n_f][cb], then ids [16][W + R] and ds [16][W + R]
  const int rb = blockIdx.x, h = blockIdx.y, f = blockIdx.z / ncb, cblk = blockIdx.z % ncb;
  const int n = D.widths[f], lane = threadIdx.x;
  const int W = D.W, R = D.R, T = D.T, Fdk = D.F * D.dk, K = W + R;
  int32_t* sid = (int32_t*)(acc + (size_t)n * cb);
  float* sds = (float*)(sid + BWD_SK_ROWS * K);
  const int c = cblk * cb + lane;
  const bool on = lane < cb && c < D.dk;
  for (int i = lane; i < n * cb; i += 64) acc[i] = 0.f;
  long long stride = 1, off = 0, sumn = 0;
  for (int g = D.F - 1; g > f; --g) stride *= D.widths[g];
  for (int g = 0; g < f; ++g) off += D.widths[g];
  for (int g = 0; g < D.F; ++g) sumn += D.widths[g];
  const int r0 = rb * rows_per_block, r1 = min(r0 + rows_per_block, D.B * T);
  for (int q0 = r0; q0 < r1; q0 += BWD_SK_ROWS) {
    const int nr = min(BWD_SK_ROWS, r1 - q0);
    __syncthreads();  // the previous rows' staging is consumed
    // the terms' slot ids and gradients, SKL loads a lane in flight together, then the factor-f sub-keys (32-bit
    // divisions here, in parallel, not in the serial sums; slot ids and stride are below 2^31)
    constexpr int SKL = 8;
    const int ne = nr * K, istride = (int)stride;
    for (int e0 = lane; e0 < ne; e0 += 64 * SKL) {
      int slot[SKL];
      float dsv[SKL];
#pragma unroll
      for (int u = 0; u < SKL; ++u) {
        const int e = min(e0 + 64 * u, ne - 1);
        const int rr = e / K, i = e % K;
        const int r = q0 + rr, b = r / T, t = r % T;
        const long long so = ((long long)b * D.H + h) * T + t;
        slot[u] = i < W ? a.widx[so * W + i] : a.ridx[so * R + (i - W)];
        dsv[u] = a.ds[so * K + i];
      }
#pragma unroll
      for (int u = 0; u < SKL; ++u) {
        const int e = e0 + 64 * u;
        if (e < ne) {
          sid[e] = (slot[u] / istride) % n;
          sds[e] = dsv[u];
        }
      }
    }
    float xw[BWD_SK_ROWS], xr[BWD_SK_ROWS];
#pragma unroll
    for (int rr = 0; rr < BWD_SK_ROWS; ++rr) {
      xw[rr] = xr[rr] = 0.f;
      if (rr < nr && on) {
        const int r = q0 + rr, b = r / T, t = r % T;
        const long long row = ((long long)b * T + t) * D.H + h;
        xw[rr] = to_f<A>(((const A*)a.wkeys)[row * Fdk + f * D.dk + c]);
        xr[rr] = to_f<A>(((const A*)a.rq)[row * Fdk + f * D.dk + c]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < BWD_SK_ROWS; ++rr) {
      if (rr < nr) {
        for (int i = 0; i < K; ++i) {
          const int sf = sid[rr * K + i];
          if (on) acc[sf * cb + lane] += sds[rr * K + i] * (i < W ? xw[rr] : xr[rr]);
        }
      }
    }
  }
  __syncthreads();
  if (on)
    for (int i = 0; i < n; ++i) a.sgpart[(((long long)rb * D.H + h) * sumn + off + i) * D.dk + c] = acc[i * cb + lane];
}

// Sub-key partial sums of one block of token rows, by sub-key: the block's terms are counting-sorted by their
// factor-f sub-key (stable: a sub-key's terms keep their order), then each sub-key's run of terms is summed in a
// register in that order, with the same additions as bwd_subkey_kernel's (so the same bits), and stored once;
// sub-keys without a term store zero. Four waves: the count on every thread, the scan and the placement on wave 0
// (chunks of 64 terms, lanes with the same sub-key matched by ballots on its bits), the sub-keys split between the
// waves by where their buckets start. Lane c owns column 64 cblk + c. For blocks of at most BWD_SKS_ROWS rows and
// BWD_SKS_TERMS terms and at most 4096 sub-keys a factor (the old one-wave kernel serves the rest).
constexpr int BWD_SKS_TERMS = 8192, BWD_SKS_ROWS = 64;
inline size_t bwd_subkey_sorted_lds(int nmax, int rows, int K) {
  const size_t nt = (size_t)rows * K;
  return (size_t)align16(3LL * nmax * 4) + (size_t)align16((long long)nt * 2) + nt * 8 + (size_t)rows * 2 * 64 * 4;
}

template <typename A>
__global__ __launch_bounds__(256) void bwd_subkey_sorted_kernel(Dims D, BwdArgs a, int ncb, int rows_per_block) {
  extern __shared__ __align__(16) unsigned char skl[];
  const int rb = blockIdx.x, h = blockIdx.y, f = blockIdx.z / ncb, cblk = blockIdx.z % ncb;
  const int n = D.widths[f], tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int W = D.W, R = D.R, T = D.T, Fdk = D.F * D.dk, K = W + R;
  const int r0 = rb * rows_per_block, nr = max(0, min(rows_per_block, D.B * T - r0));
  const int nt = nr * K;
  int* hist = (int*)skl;                                               // [n] terms per sub-key
  int* start = hist + n;                                               // [n] bucket starts (advanced)
  int* bstart = start + n;                                             // [n] bucket starts
  uint16_t* tsf = (uint16_t*)(skl + align16(3LL * n * 4));            // [nt] sub-key of term e
  // [nt] terms by sub-key, packed (sub-key << 20) | (row 2 + query << 13) | term (12 + 7 + 13 bits)
  uint32_t* sorted = (uint32_t*)((unsigned char*)tsf + align16((long long)nt * 2));
  float* tds = (float*)(sorted + nt);                                  // [nt] slot-score gradients
  float* xs = tds + nt;                                                // [nr][2][64] key / query column values
  long long stride = 1, off = 0, sumn = 0;
  for (int g = D.F - 1; g > f; --g) stride *= D.widths[g];
  for (int g = 0; g < f; ++g) off += D.widths[g];
  for (int g = 0; g < D.F; ++g) sumn += D.widths[g];
  for (int i = tid; i < n; i += 256) hist[i] = 0;
  // the terms' sub-keys and gradients (eight loads a thread in flight; slot ids and stride below 2^31)
  constexpr int SKL = 8;
  const int istride = (int)stride;
  for (int e0 = tid; e0 < nt; e0 += 256 * SKL) {
    int slot[SKL];
    float dsv[SKL];
#pragma unroll
    for (int u = 0; u < SKL; ++u) {
      const int e = min(e0 + 256 * u, nt - 1);
      const int rr = e / K, i = e % K;
      const int r = r0 + rr, b = r / T, t = r % T;
      const long long so = ((long long)b * D.H + h) * T + t;
      slot[u] = i < W ? a.widx[so * W + i] : a.ridx[so * R + (i - W)];
      dsv[u] = a.ds[so * K + i];
    }
#pragma unroll
    for (int u = 0; u < SKL; ++u) {
      const int e = e0 + 256 * u;
      if (e < nt) {
        tsf[e] = (uint16_t)((slot[u] / istride) % n);
        tds[e] = dsv[u];
      }
    }
  }
  const int c = cblk * 64 + lane;
  const bool on = c < D.dk;
  for (int rr = wv; rr < nr; rr += 4) {
    const int r = r0 + rr, b = r / T, t = r % T;
    const long long row = ((long long)b * T + t) * D.H + h;
    xs[(rr * 2) * 64 + lane] = on ? to_f<A>(((const A*)a.wkeys)[row * Fdk + f * D.dk + c]) : 0.f;
    xs[(rr * 2 + 1) * 64 + lane] = on ? to_f<A>(((const A*)a.rq)[row * Fdk + f * D.dk + c]) : 0.f;
  }
  __syncthreads();
  for (int e = tid; e < nt; e += 256) atomicAdd(&hist[tsf[e]], 1);  // integer counts: order independent
  __syncthreads();
  if (wv == 0) {
    // exclusive scan of the counts, 64 sub-keys a step
    int carry = 0;
    for (int i0 = 0; i0 < n; i0 += 64) {
      const int i = i0 + lane;
      const int v = i < n ? hist[i] : 0;
      int incl = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      if (i < n) start[i] = bstart[i] = carry + incl - v;
      carry += __shfl(incl, 63, 64);
    }
    wave_sync();
    // stable placement, 64 terms a step in term order
    int nb = 0;
    while ((1 << nb) < n) ++nb;
    const uint64_t below = lanes_below_mask();
    for (int e0 = 0; e0 < nt; e0 += 64) {
      const int e = e0 + lane;
      const bool ok = e < nt;
      const int s = ok ? tsf[e] : 0;
      uint64_t m = __ballot(ok);
      for (int bt = 0; bt < nb; ++bt) {
        const bool one = ((s >> bt) & 1) != 0;
        const uint64_t bb = __ballot(one);
        m &= one ? bb : ~bb;
      }
      const int s0 = start[s];  // every lane reads before any lane advances a bucket
      wave_sync();
      if (ok) {
        const int rr = e / K;
        const uint32_t xo = (uint32_t)(rr * 2 + (e - rr * K < W ? 0 : 1));
        sorted[s0 + __popcll(m & below)] = ((uint32_t)s << 20) | (xo << 13) | (uint32_t)e;
      }
      if (ok && (m & ~below & ~(1ull << lane)) == 0) start[s] = s0 + __popcll(m);  // the group's last lane
      wave_sync();
    }
  }
  __syncthreads();
  // the sums: wave w takes the sub-keys whose bucket starts in [w nt / 4, (w + 1) nt / 4) (the last wave also those
  // starting at nt: empty ones), each bucket's terms in order, branch-free within a bucket; empty buckets store zero
  float* outc = a.sgpart + (((long long)rb * D.H + h) * sumn + off) * D.dk + c;
  const int lo = (int)((long long)wv * nt / 4), hi = wv == 3 ? nt + 1 : (int)((long long)(wv + 1) * nt / 4);
  constexpr int RB = 4;
  for (int sk = 0; sk < n; ++sk) {
    const int b = bstart[sk];
    if (b < lo || b >= hi) continue;
    const int cnt = hist[sk];
    float acc = 0.f;
    int i = b;
    for (; i + RB <= b + cnt; i += RB) {
      uint32_t pk[RB];
      float dv[RB], xv[RB];
#pragma unroll
      for (int u = 0; u < RB; ++u) pk[u] = sorted[i + u];
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        dv[u] = tds[pk[u] & 0x1FFF];
        xv[u] = xs[((pk[u] >> 13) & 0x7F) * 64 + lane];
      }
#pragma unroll
      for (int u = 0; u < RB; ++u) acc += dv[u] * xv[u];
    }
    for (; i < b + cnt; ++i) {
      const uint32_t pk = sorted[i];
      acc += tds[pk & 0x1FFF] * xs[((pk >> 13) & 0x7F) * 64 + lane];
    }
    if (on) outc[(long long)sk * D.dk] = acc;  // 0 for an empty bucket
  }
}

__global__ __launch_bounds__(256) void bwd_subkey_sum_kernel(const float* __restrict__ sgpart, float* __restrict__ gsub,
                                                             long long n, int nrb) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  int rb = 0;
  for (; rb + 8 <= nrb; rb += 8) {  // the blocks in order, eight loads in flight
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = sgpart[(long long)(rb + u) * n + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; rb < nrb; ++rb) s += sgpart[(long long)rb * n + i];
  gsub[i] = s;
}

// Token grouping of the fast sweep. Tokens are cut, in decreasing order, into blocks of G; within a block, runs of
// consecutive tokens whose slot sets (read and write ids) are pairwise disjoint are greedy-grown from its first
// token. The tokens of a run touch disjoint bank and gradient rows, so the sweep takes them in one step, each with
// the arithmetic of its own step (the same results, bit for bit). One workgroup per (stream, block).
constexpr int BWD_MAX_G = 16;
__global__ __launch_bounds__(64) void bwd_group_kernel(Dims D, BwdArgs a, int G, int nb) {
  __shared__ int32_t sl[BWD_MAX_G][2 * 128];
  __shared__ int32_t conf[BWD_MAX_G][BWD_MAX_G];
  const int st = blockIdx.x / nb, g = blockIdx.x % nb;
  const int W = D.W, R = D.R, T = D.T, n = W + R;
  const int t0 = T - 1 - g * G;     // the block's first (largest) token
  const int nv = min(G, t0 + 1);    // its tokens: t0, t0 - 1, ..., t0 - nv + 1
  for (int i = threadIdx.x; i < BWD_MAX_G * BWD_MAX_G; i += 64) conf[i / BWD_MAX_G][i % BWD_MAX_G] = 0;
  for (int i = threadIdx.x; i < nv * n; i += 64) {
    const int k = i / n, e = i % n;
    const long long so = (long long)st * T + (t0 - k);
    sl[k][e] = e < R ? a.ridx[so * R + e] : a.widx[so * W + (e - R)];
  }
  __syncthreads();
  // conf[k0][k1], k0 < k1: the block's tokens k0 and k1 address a common slot
  for (int i = threadIdx.x; i < nv * nv * n; i += 64) {
    const int k0 = i / (nv * n), k1 = (i / n) % nv, e = i % n;
    if (k0 >= k1) continue;
    const int32_t x = sl[k1][e];
    bool hit = false;
    for (int f = 0; f < n; ++f) hit |= sl[k0][f] == x;
    if (hit) conf[k0][k1] = 1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int runs = 0;
    for (int k = 0; k < nv;) {
      int size = 1;
      for (; k + size < nv; ++size) {
        bool ok = true;
        for (int m = k; m < k + size; ++m) ok = ok && conf[m][k + size] == 0;
        if (!ok) break;
      }
      a.gent[(long long)st * T + g * G + runs] = ((t0 - k) << 4) | size;
      ++runs;
      k += size;
    }
    a.gcnt[(long long)st * nb + g] = runs;
  }
}

// Every stream's entries in order (the blocks' runs, compacted): an exclusive scan of the run counts. One
// workgroup per stream.
__global__ __launch_bounds__(256) void bwd_group_scan_kernel(Dims D, BwdArgs a, int G, int nb) {
  __shared__ int32_t ssum[256];
  __shared__ int32_t base;
  const int st = blockIdx.x, tid = threadIdx.x, T = D.T;
  if (tid == 0) base = 0;
  __syncthreads();
  for (int c0 = 0; c0 < nb; c0 += 256) {
    const int g = c0 + tid;
    const int c = g < nb ? a.gcnt[(long long)st * nb + g] : 0;
    ssum[tid] = c;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {  // inclusive scan
      const int v = tid >= o ? ssum[tid - o] : 0;
      __syncthreads();
      ssum[tid] += v;
      __syncthreads();
    }
    const int pos = base + ssum[tid] - c;
    for (int e = 0; e < c; ++e) a.giter[(long long)st * T + pos + e] = a.gent[(long long)st * T + g * G + e];
    __syncthreads();  // every thread has read base
    if (tid == 255) base += ssum[255];
    __syncthreads();
  }
  if (tid == 0) a.gn[st] = base;
}

template <typename A, typename Bk>
static hipError_t launch_bwd_t(const Dims& D, const BwdArgs& a, hipStream_t st) {
  const int nsl = bwd_nsl(D);
  if (bwd_fast(D)) {
    hipLaunchKernelGGL(bwd_match_kernel, dim3((unsigned)((long long)D.S * D.T)), dim3(64), 0, st, D, a);
    const int G = bwd_group_tokens(D), wb = bwd_wave_block(D);
    if (G > BWD_MAX_G || wb < 1 || wb * 64 > BWD_FAST_GROUPS * (bwd_cols(D) / 4))
      return hipErrorInvalidValue;  // never: W, R <= 128
    if (G > 1) {
      const int nb = (D.T + G - 1) / G;
      hipLaunchKernelGGL(bwd_group_kernel, dim3((unsigned)((long long)D.S * nb)), dim3(64), 0, st, D, a, G, nb);
      hipLaunchKernelGGL(bwd_group_scan_kernel, dim3((unsigned)D.S), dim3(256), 0, st, D, a, G, nb);
    }
    const dim3 grid((unsigned)((long long)D.S * nsl));
    auto fast = [&](auto sk, auto sq) {  // sk: a value of the snapshot's element type; sq: its mode
      using Sk = decltype(sk);
      constexpr int SQ = decltype(sq)::value;
      auto go = [&](auto gk) {  // gk: a value of the bank gradient's element type
        using Gk = decltype(gk);
        if (bwd_cols(D) == 8)
          hipLaunchKernelGGL((bwd_sweep_fast_kernel<A, Bk, 2, Sk, SQ, Gk>), grid, dim3(BWD_FAST_GROUPS * 2), 0, st, D,
                             a, nsl, wb);
        else
          hipLaunchKernelGGL((bwd_sweep_fast_kernel<A, Bk, 4, Sk, SQ, Gk>), grid, dim3(BWD_FAST_GROUPS * 4), 0, st, D,
                             a, nsl, wb);
      };
      if constexpr (std::is_same<Bk, bf16_t>::value && SQ == SNAP_BANK)
        if (a.grad_bf16) {
          go(bf16_t{});
          return;
        }
      go(float{});
    };
    if (std::is_same<Bk, float>::value && a.snap_mode == SNAP_BF16)
      fast(bf16_t{}, std::integral_constant<int, SNAP_BANK>{});  // bfloat16 snapshot rows of a float32 bank
    else if (std::is_same<Bk, float>::value && a.snap_mode == SNAP_FP8)
      fast(Bk{}, std::integral_constant<int, SNAP_FP8>{});
    else if (std::is_same<Bk, float>::value && a.snap_mode == SNAP_INT4)
      fast(Bk{}, std::integral_constant<int, SNAP_INT4>{});
    else
      fast(Bk{}, std::integral_constant<int, SNAP_BANK>{});
  } else {
    const size_t lds = bwd_sweep_lds(D.W);
    (void)hipFuncSetAttribute((const void*)bwd_sweep_kernel<A, Bk>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
    hipLaunchKernelGGL((bwd_sweep_kernel<A, Bk>), dim3((unsigned)((long long)D.S * nsl)), dim3(BWD_NT), lds, st, D, a,
                       nsl);
  }
  hipLaunchKernelGGL((bwd_token_kernel<A>), dim3((unsigned)((long long)D.S * D.T)), dim3(256), 0, st, D, a, nsl);
  const int nrb = bwd_row_blocks(D), rpb = bwd_row_block_rows(D);
  long long sumn = 0;
  int nmax = 0;
  for (int f = 0; f < D.F; ++f) {
    sumn += D.widths[f];
    nmax = max(nmax, D.widths[f]);
  }
  const int K = D.W + D.R;
  if (nmax <= 4096 && rpb <= BWD_SKS_ROWS && (long long)rpb * K <= BWD_SKS_TERMS) {
    const int ncb2 = (D.dk + 63) / 64;
    const size_t l2 = bwd_subkey_sorted_lds(nmax, rpb, K);
    (void)hipFuncSetAttribute((const void*)bwd_subkey_sorted_kernel<A>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)l2);
    hipLaunchKernelGGL((bwd_subkey_sorted_kernel<A>), dim3((unsigned)nrb, (unsigned)D.H, (unsigned)(D.F * ncb2)),
                       dim3(256), l2, st, D, a, ncb2, rpb);
    const long long n = (long long)D.H * sumn * D.dk;
    hipLaunchKernelGGL(bwd_subkey_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.sgpart, a.gsub,
                       n, nrb);
    return hipGetLastError();
  }
  const size_t stage = (size_t)BWD_SK_ROWS * (D.W + D.R) * 8;  // <= 128 KiB (W, R <= 512)
  const size_t budget = 150 * 1024 - stage;                     // >= 22 KiB: n_f * 4 <= 16 KiB always fits
  int cb = 64;
  while (cb > 1 && (size_t)nmax * cb * 4 > budget) cb >>= 1;
  const int ncb = (D.dk + cb - 1) / cb;
  const size_t slds = (size_t)nmax * cb * 4 + stage;
  (void)hipFuncSetAttribute((const void*)bwd_subkey_kernel<A>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)slds);
  hipLaunchKernelGGL((bwd_subkey_kernel<A>), dim3((unsigned)nrb, (unsigned)D.H, (unsigned)(D.F * ncb)), dim3(64), slds,
                     st, D, a, cb, ncb, rpb);
  const long long n = (long long)D.H * sumn * D.dk;
  hipLaunchKernelGGL(bwd_subkey_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.sgpart, a.gsub, n,
                     nrb);
  return hipGetLastError();
}

hipError_t launch_bwd(const Dims& D, const BwdArgs& a, hipStream_t st) {
  if (D.S == 0 || D.T == 0) return hipSuccess;
  if (D.act == SDM_BF16)
    return D.bank == SDM_BF16 ? launch_bwd_t<bf16_t, bf16_t>(D, a, st) : launch_bwd_t<bf16_t, float>(D, a, st);
  return D.bank == SDM_BF16 ? launch_bwd_t<float, bf16_t>(D, a, st) : launch_bwd_t<float, float>(D, a, st);
}

}  // namespace sdm
