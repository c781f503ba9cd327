// The serial chunk loop: bank gather, delta solve, read output and in-order segmented scatter.
//
// Column slices of the bank are independent (every coefficient comes from the bank-independent plan), so one
// workgroup owns one (stream, 64-byte column slice) pair and runs every chunk of its stream in order with no
// synchronisation beyond its own barriers. Per chunk (notation of plan.hip):
//   A  gather  H[t] = sum_i a_ti M_0[S_ti],  G[t] = sum_i b_ti M_0[R_ti]           (HBM: W + R row slices/token)
//   B  solve   delta_t = beta_t v_t - alpha_t beta_t H[t] - sum_m L_tm delta_m      (forward substitution)
//   C  read    out_t = G[t] + sum_s Q_ts delta_s                                   (act dtype)
//   D  scatter per written slot j, its events in token order: M[j] <- alpha_s M[j] + w_sj delta_s, one read and
//              one write of the row slice, rounded once to the bank dtype            (HBM: W row slices/token)
// Each group of 4 lanes moves one 64-byte row slice (16 bytes per lane). Blocks are mapped so that neighbouring
// column slices of a stream run on the same XCD and share its L2 (a 128-byte L2 line holds two 64-byte slices).
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
};

template <typename A, typename Bk>
__global__ __launch_bounds__(LOOP_NT) void loop_kernel(Dims D, LoopArgs a, int nslices) {
  constexpr int EPL = Lane<Bk>::EPL;
  constexpr int COLS = 4 * EPL;  // columns per 64-byte slice
  constexpr int NW = LOOP_NT / 64;
  extern __shared__ __align__(16) unsigned char lds[];
  float* sH = (float*)lds;              // [C][COLS]
  float* sG = sH + D.C * COLS;          // [C][COLS]
  float* sD = sG + D.C * COLS;          // [C][COLS]
  float* sA = sD + D.C * COLS;          // [C]
  float* sB = sA + D.C;                 // [C]

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
  const long long rowsd = D.rows * (long long)D.d;
  Bk* bank = (Bk*)a.bank + (long long)st * rowsd;
  const A* alpha = (const A*)a.alpha;
  const A* beta = (const A*)a.beta;
  const A* values = (const A*)a.values;
  A* out = (A*)a.out;
  const int W = D.W, R = D.R, C = D.C;
  const long long CW = (long long)C * W;
  const long long lcap = chunk_lents(D), qcap = chunk_qents(D);

  for (int ch = 0; ch < D.nch; ++ch) {
    const int t0 = ch * C;
    const int Cc = min(C, D.T - t0);
    const long long cidx = (long long)st * D.nch + ch;
    for (int t = tid; t < Cc; t += LOOP_NT) {
      const long long g = ((long long)b * D.T + t0 + t) * D.H + h;
      sA[t] = to_f<A>(alpha[g]);
      sB[t] = to_f<A>(beta[g]);
    }
    // A: gathers, one token per wave at a time.
    for (int t = wv; t < Cc; t += NW) {
      const long long wrow = ((long long)st * D.T + t0 + t) * W;
      const long long rrow = ((long long)st * D.T + t0 + t) * R;
      float accH[EPL], accG[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) accH[e] = accG[e] = 0.0f;
      if (valid) {
#pragma unroll 4
        for (int i = grp; i < W; i += 16) {
          const int slot = a.widx[wrow + i];
          const float cf = a.wcoef[wrow + i];
          float v[EPL];
          Lane<Bk>::load(bank + (long long)slot * D.d + mycol, v);
#pragma unroll
          for (int e = 0; e < EPL; ++e) accH[e] += cf * v[e];
        }
#pragma unroll 4
        for (int i = grp; i < R; i += 16) {
          const int slot = a.ridx[rrow + i];
          const float cf = a.rcoef[rrow + i];
          float v[EPL];
          Lane<Bk>::load(bank + (long long)slot * D.d + mycol, v);
#pragma unroll
          for (int e = 0; e < EPL; ++e) accG[e] += cf * v[e];
        }
      }
      // reduce over the 16 groups of the wave (lanes with equal q), fixed order
#pragma unroll
      for (int off = 4; off < 64; off <<= 1) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          accH[e] += __shfl_xor(accH[e], off);
          accG[e] += __shfl_xor(accG[e], off);
        }
      }
      if (grp == 0) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          sH[t * COLS + q * EPL + e] = accH[e];
          sG[t * COLS + q * EPL + e] = accG[e];
        }
      }
    }
    __syncthreads();
    // B: forward substitution, one thread per column.
    if (tid < COLS && col0 + tid < D.d) {
      const int c = tid;
      const int32_t* lp = a.lptr + cidx * (C + 1);
      const Ent* le = a.lent + cidx * lcap;
      for (int t = 0; t < Cc; ++t) {
        const long long g = ((long long)b * D.T + t0 + t) * D.H + h;
        const float v = to_f<A>(values[g * D.d + col0 + c]);
        float u = sB[t] * v - sA[t] * sB[t] * sH[t * COLS + c];
        for (int e = lp[t]; e < lp[t + 1]; ++e) u -= le[e].val * sD[le[e].col * COLS + c];
        sD[t * COLS + c] = u;
      }
    }
    __syncthreads();
    // C: read output.
    {
      const int32_t* qp = a.qptr + cidx * (C + 1);
      const Ent* qe = a.qent + cidx * qcap;
      for (int idx = tid; idx < Cc * COLS; idx += LOOP_NT) {
        const int t = idx / COLS, c = idx % COLS;
        if (col0 + c < D.d) {
          float o = sG[t * COLS + c];
          for (int e = qp[t]; e < qp[t + 1]; ++e) o += qe[e].val * sD[qe[e].col * COLS + c];
          const long long g = ((long long)b * D.T + t0 + t) * D.H + h;
          out[g * D.d + col0 + c] = from_f<A>(o);
        }
      }
    }
    // D: in-order segmented scatter, one 64-byte row slice per group of 4 lanes.
    if (valid) {
      const int nseg = a.nseg[cidx];
      const int32_t* sslot = a.seg_slot + cidx * CW;
      const int32_t* sst = a.seg_start + cidx * (CW + 1);
      const Ev* ev = a.ev + cidx * CW;
#pragma unroll 2
      for (int sg = wv * 16 + grp; sg < nseg; sg += NW * 16) {
        Bk* p = bank + (long long)sslot[sg] * D.d + mycol;
        float m[EPL];
        Lane<Bk>::load(p, m);
        for (int e = sst[sg]; e < sst[sg + 1]; ++e) {
          const Ev x = ev[e];
          const float al = sA[x.tok];
#pragma unroll
          for (int k = 0; k < EPL; ++k) m[k] = al * m[k] + x.w * sD[x.tok * COLS + q * EPL + k];
        }
        Lane<Bk>::store(p, m);
      }
    }
    __syncthreads();
  }
}

template <typename A, typename Bk>
static hipError_t launch_loop_t(const Dims& D, const LoopArgs& a, hipStream_t st) {
  constexpr int COLS = 4 * Lane<Bk>::EPL;
  const int nslices = (D.d + COLS - 1) / COLS;
  const long long nblk = (long long)D.S * nslices;
  const size_t lds = (size_t)D.C * COLS * 4 * 3 + (size_t)D.C * 8;
  hipLaunchKernelGGL((loop_kernel<A, Bk>), dim3((unsigned)nblk), dim3(LOOP_NT), lds, st, D, a, nslices);
  return hipGetLastError();
}

hipError_t launch_loop(const Dims& D, const LoopArgs& a, hipStream_t st) {
  if (D.S == 0 || D.T == 0) return hipSuccess;
  if (D.act == SDM_BF16)
    return D.bank == SDM_BF16 ? launch_loop_t<bf16_t, bf16_t>(D, a, st) : launch_loop_t<bf16_t, float>(D, a, st);
  return D.bank == SDM_BF16 ? launch_loop_t<float, bf16_t>(D, a, st) : launch_loop_t<float, float>(D, a, st);
}

}  // namespace sdm
