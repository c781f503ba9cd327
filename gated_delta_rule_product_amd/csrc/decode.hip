// Single-token decode step: one workgroup per stream (b, h) does both exact top-k selections, the gated
// delta-rule update of the W write rows and the read of the R read rows.
//
// Successor bank (lumen PR #29, "Donating is a permission, not a demand"): bank_out == bank_in writes the successor
// in place; a distinct bank_out first receives a copy of bank_in (launch_copy, same stream) and then the same body
// runs: rows are read from bank_in before any row is written, the W updated rows are stored into bank_out, and
// the read takes its rows from bank_out. Both forms therefore execute identical arithmetic on identical values
// and produce identical bits. Per-token work is O((W + R) d) as in the pages' cost model; the copy is O(N d).
#include "sdm_internal.h"
#include "topk_device.h"

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

__host__ __device__ inline size_t decode_lds_bytes(const Dims& D, const TopkPlan& pw, const TopkPlan& pr, int EPL) {
  size_t t = topk_lds_bytes(D.F, D.dk, pw);
  const size_t t2 = topk_lds_bytes(D.F, D.dk, pr);
  if (t2 > t) t = t2;
  t = (t + 15) & ~(size_t)15;
  t += (size_t)(D.W + D.R) * 8;             // ids + weights
  t += (size_t)DECODE_NT * EPL * 4;         // partial sums
  t += (size_t)DECODE_NT * EPL * 4;         // delta of one column pass
  return t + 16;
}

template <typename A, typename Bk>
__global__ __launch_bounds__(DECODE_NT) void decode_kernel(Dims D, DecodeArgs a) {
  constexpr int EPL = DLane<Bk>::EPL;
  extern __shared__ __align__(16) unsigned char lds[];
  const int tid = threadIdx.x;
  const int st = blockIdx.x;  // stream b * H + h; with one token the [B, 1, H] row index equals st
  const int h = st % D.H;
  const long long row = st;
  long long sumn = 0;
  for (int f = 0; f < D.F; ++f) sumn += D.widths[f];
  const A* sub = (const A*)a.subkeys + (long long)h * sumn * D.dk;
  const int Fdk = D.F * D.dk;

  size_t tb = topk_lds_bytes(D.F, D.dk, a.plan[0]);
  const size_t tb2 = topk_lds_bytes(D.F, D.dk, a.plan[1]);
  if (tb2 > tb) tb = tb2;
  tb = (tb + 15) & ~(size_t)15;
  int32_t* sWid = (int32_t*)(lds + tb);
  float* sWw = (float*)(sWid + D.W);
  int32_t* sRid = (int32_t*)(sWw + D.W);
  float* sRw = (float*)(sRid + D.R);
  float* part = (float*)(((uintptr_t)(sRw + D.R) + 15) & ~(uintptr_t)15);
  float* sdel = part + DECODE_NT * EPL;

  // 1. addressing (bank-independent)
  {
    TopkLds L = topk_lds_carve(lds, D.F, D.dk, a.plan[0]);
    topk_query<A, DECODE_NT>((const A*)a.wkeys + row * Fdk, sub, D.widths, D.F, D.dk, a.plan[0], a.cand[0], L);
    for (int r = tid; r < D.W; r += DECODE_NT) {
      sWid[r] = L.rid[r];
      if (a.widx) a.widx[row * D.W + r] = L.rid[r];
    }
    topk_softmax<DECODE_NT>(L, D.W, sWw);
  }
  {
    TopkLds L = topk_lds_carve(lds, D.F, D.dk, a.plan[1]);
    topk_query<A, DECODE_NT>((const A*)a.rq + row * Fdk, sub, D.widths, D.F, D.dk, a.plan[1], a.cand[1], L);
    for (int r = tid; r < D.R; r += DECODE_NT) {
      sRid[r] = L.rid[r];
      if (a.ridx) a.ridx[row * D.R + r] = L.rid[r];
    }
    topk_softmax<DECODE_NT>(L, D.R, sRw);
  }
  const float al = to_f<A>(((const A*)a.alpha)[row]);
  const float be = to_f<A>(((const A*)a.beta)[row]);
  const A* v = (const A*)a.values + row * D.d;
  A* out = (A*)a.out + row * D.d;
  const long long rowsd = D.rows * D.ld;
  const Bk* bin = (const Bk*)a.bank_in + (long long)st * rowsd;
  Bk* bout = (Bk*)a.bank_out + (long long)st * rowsd;

  // 2. column passes: lanes of EPL columns; RG row groups of LPR lanes each.
  const int nlane = D.d / EPL;
  const int LPR = nlane < DECODE_NT ? nlane : DECODE_NT;
  const int RG = DECODE_NT / LPR;
  const int cl = tid % LPR, rg = tid / LPR;
  const bool act = rg < RG;
  for (int lane0 = 0; lane0 < nlane; lane0 += LPR) {
    const int ln = lane0 + cl;
    const bool on = act && ln < nlane;
    const int col = ln * EPL;
    // r = sum_i w_i M[S_i]
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
    if (on) {
      for (int i = rg; i < D.W; i += RG) {
        float m[EPL];
        DLane<Bk>::load(bin + (long long)sWid[i] * D.ld + col, m);
        const float wi = sWw[i];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += wi * m[e];
      }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) part[(rg * LPR + cl) * EPL + e] = acc[e];
    __syncthreads();
    if (rg == 0 && on) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float r = 0.0f;
        for (int g = 0; g < RG; ++g) r += part[(g * LPR + cl) * EPL + e];
        sdel[cl * EPL + e] = be * (to_f<A>(v[col + e]) - al * r);
      }
    }
    __syncthreads();
    // M[S_i] <- alpha M[S_i] + w_i delta, rounded to the bank dtype, into the successor
    if (on) {
      for (int i = rg; i < D.W; i += RG) {
        const long long o = (long long)sWid[i] * D.ld + col;
        float m[EPL];
        DLane<Bk>::load(bin + o, m);
        const float wi = sWw[i];
#pragma unroll
        for (int e = 0; e < EPL; ++e) m[e] = al * m[e] + wi * sdel[cl * EPL + e];
        DLane<Bk>::store(bout + o, m);
      }
    }
    __syncthreads();
    // out = sum_i rho_i M'[R_i], read from the successor after the write
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
    if (on) {
      for (int i = rg; i < D.R; i += RG) {
        float m[EPL];
        DLane<Bk>::load(bout + (long long)sRid[i] * D.ld + col, m);
        const float ri = sRw[i];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += ri * m[e];
      }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) part[(rg * LPR + cl) * EPL + e] = acc[e];
    __syncthreads();
    if (rg == 0 && on) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float o = 0.0f;
        for (int g = 0; g < RG; ++g) o += part[(g * LPR + cl) * EPL + e];
        out[col + e] = from_f<A>(o);
      }
    }
    __syncthreads();
  }
}

template <typename A, typename Bk>
static hipError_t launch_decode_t(const Dims& D, const DecodeArgs& a, hipStream_t st) {
  const size_t lds = decode_lds_bytes(D, a.plan[0], a.plan[1], DLane<Bk>::EPL);
  (void)hipFuncSetAttribute((const void*)decode_kernel<A, Bk>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL((decode_kernel<A, Bk>), dim3((unsigned)D.S), dim3(DECODE_NT), lds, st, D, a);
  return hipGetLastError();
}

hipError_t launch_decode(const Dims& D, const DecodeArgs& a, hipStream_t st) {
  if (D.S == 0) return hipSuccess;
  if (D.act == SDM_BF16)
    return D.bank == SDM_BF16 ? launch_decode_t<bf16_t, bf16_t>(D, a, st) : launch_decode_t<bf16_t, float>(D, a, st);
  return D.bank == SDM_BF16 ? launch_decode_t<float, bf16_t>(D, a, st) : launch_decode_t<float, float>(D, a, st);
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
