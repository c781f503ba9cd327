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
