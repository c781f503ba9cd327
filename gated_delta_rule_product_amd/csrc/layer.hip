// The layer around the write/read op: its dense maps (projections in, output projection out) and its gates.
//
// Dense maps (sparse-delta-memory README.md, usage example and "Behavior changes": a layer call runs the
// projections, the top-k and the bank copy before the op): Y = X W^T with X [M, K] and W [N, K] bfloat16,
// row-major (the weight in out-features x in-features order), float32 accumulation on the matrix cores, the result
// rounded to bfloat16. The output columns are split into up to GEMM_MAXSEG contiguous destinations (write keys,
// read queries, values, gate inputs), so one launch feeds the op's separate input tensors directly.
//
// Gates (README "ideas": the gated delta rule of Gated DeltaNet, with FLA's A/dt parameterisation): per (token,
// head) the forget gate alpha = exp(-exp(A_log[h]) * softplus(a + dt_bias[h])) and the input gate
// beta = sigmoid(b), from the two gate inputs a and b of the projection, in float32, rounded to bfloat16.
#include "layer.h"

namespace sdm {

typedef __bf16 gemm_bf16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float gemm_f32x4_t;

// One workgroup (4 waves) per 128 x 128 output tile; wave (wm, wn) computes rows 64 wm .. + 64 and columns
// 64 wn .. + 64 as 4 x 4 MFMA tiles of 16 x 16 (v_mfma_f32_16x16x32_bf16). Operand fragments come straight from
// global memory (16 bytes per lane: 8 consecutive K elements of one row), the next K step's fragments loaded while
// the current step multiplies. Rows and columns past M or N load row M - 1 or N - 1 (never stored). K % 32 == 0.
//
// MFMA 16x16x32 bf16 lane layout: A lane l holds row l % 16, K elements 8 (l / 16) .. + 8 of the 32-wide step; B
// lane l holds column l % 16, the same K elements; the result lane l holds column l % 16, rows 4 (l / 16) + r.
// The epilogue shared by both dense-map kernels: acc[i][j][r] is the element at row m0 + 16 i + 4 (lane / 16) + r,
// column n0 + 16 j + lane % 16; column n goes to the segment whose range holds it.
__device__ __forceinline__ void gemm_store(const GemmArgs& g, const gemm_f32x4_t (&acc)[4][4], int m0, int n0,
                                           int lane) {
  const int ql = lane & 15;
  if (g.f32) {  // float32 results (parameter and input gradients)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 16 * j + ql;
      if (n >= g.N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + 16 * i + 4 * (lane >> 4) + r;
          if (m < g.M) g.f32[(long long)m * g.f32ld + n] = acc[i][j][r];
        }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + 16 * j + ql;
    if (n >= g.N) continue;
    // the segment holding column n, picked with constant indices (a runtime index into the argument's array
    // would copy it to scratch memory)
    bf16_t* dst = g.seg[0].dst + n;
    long long ld = g.seg[0].ld;
#pragma unroll
    for (int q = 1; q < GEMM_MAXSEG; ++q)
      if (q < g.nseg && n >= g.seg[q - 1].end) {
        dst = g.seg[q].dst + (n - g.seg[q - 1].end);
        ld = g.seg[q].ld;
      }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * i + 4 * (lane >> 4) + r;
        if (m < g.M) dst[(long long)m * ld] = f_to_bf16(acc[i][j][r]);
      }
  }
}

constexpr int GEMM_NT = 256;
__global__ __launch_bounds__(GEMM_NT) void gemm_bf16_kernel(GemmArgs g) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int m0 = blockIdx.y * 128 + (wv & 1) * 64, n0 = blockIdx.x * 128 + (wv >> 1) * 64;
  const int ql = lane & 15, kq = (lane >> 4) * 8;
  const bf16_t* ap[4];
  const bf16_t* bp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ap[i] = g.x + (long long)min(m0 + 16 * i + ql, g.M - 1) * g.K + kq;
    bp[i] = g.w + (long long)min(n0 + 16 * i + ql, g.N - 1) * g.K + kq;
  }
  gemm_f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = gemm_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  gemm_bf16x8_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = __builtin_bit_cast(gemm_bf16x8_t, *(const uint4*)ap[i]);
    b[i] = __builtin_bit_cast(gemm_bf16x8_t, *(const uint4*)bp[i]);
  }
  for (int k = 32; k <= g.K; k += 32) {
    gemm_bf16x8_t an[4], bn[4];
    const int kk = k < g.K ? k : 0;  // the last step reloads step 0 (in bounds, unused)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      an[i] = __builtin_bit_cast(gemm_bf16x8_t, *(const uint4*)(ap[i] + kk));
      bn[i] = __builtin_bit_cast(gemm_bf16x8_t, *(const uint4*)(bp[i] + kk));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = an[i];
      b[i] = bn[i];
    }
  }
  gemm_store(g, acc, m0, n0, lane);
}

// LDS-tiled dense map (K % 64 == 0): one workgroup per 128 x 128 output tile, K in steps of 64, two LDS buffers.
// Step k multiplies buffer k % 2 while the tile of step k + 1, loaded from global memory into registers during step
// k - 1, is written into the other buffer, and the loads of step k + 2 are issued; one barrier per step separates a
// buffer's reads from its next writes. Tiles: 128 rows x 64 K elements of A and of B, 16 bytes per thread and load
// (8 threads per 128-byte row segment); wave (wm, wn) owns rows 64 wm .., columns 64 wn .. as 4 x 4 MFMA tiles of
// 16 x 16, two 32-wide K halves per step. LDS rows are 72 elements apart (144 bytes), which spreads a fragment
// read's 16 rows over all banks. Rows past M or N load row M - 1 or N - 1 and are never stored. Workgroups map to
// tiles so that the tiles on one XCD (workgroup id mod 8) are consecutive in row-major tile order, sharing A rows
// in that XCD's L2.
constexpr int GT_LD = 72;
constexpr int GT_BUF = 128 * GT_LD;  // elements of one operand tile
constexpr size_t GEMM_LDS = (size_t)4 * GT_BUF * sizeof(bf16_t);  // A and B, two buffers each: 73,728 bytes
__global__ __launch_bounds__(GEMM_NT) void gemm_bf16_lds_kernel(GemmArgs g) {
  extern __shared__ __align__(16) bf16_t gsm[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ntn = gridDim.x, total = gridDim.x * gridDim.y;
  int tile = blockIdx.x + ntn * blockIdx.y;
  if (total % 8 == 0) tile = (tile % 8) * (total / 8) + tile / 8;
  const int bm = (tile / ntn) * 128, bn = (tile % ntn) * 128;
  // this thread's 4 copy chunks per operand: chunk c = tid + 256 u -> row c / 8, K piece (c % 8) * 8
  const bf16_t* ag[4];
  const bf16_t* bg[4];
  int lds_off[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = tid + 256 * u, row = c >> 3, kp = (c & 7) * 8;
    ag[u] = g.x + (long long)min(bm + row, g.M - 1) * g.K + kp;
    bg[u] = g.w + (long long)min(bn + row, g.N - 1) * g.K + kp;
    lds_off[u] = row * GT_LD + kp;
  }
  gemm_bf16x8_t ar[4], br[4];  // native vectors: a union-based uint4 array carried across steps lands in scratch
  // step 0's tile straight into buffer 0, step 1's into registers
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    ar[u] = *(const gemm_bf16x8_t*)ag[u];
    br[u] = *(const gemm_bf16x8_t*)bg[u];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    *(gemm_bf16x8_t*)&gsm[lds_off[u]] = ar[u];
    *(gemm_bf16x8_t*)&gsm[2 * GT_BUF + lds_off[u]] = br[u];
  }
  const int k1 = 64 < g.K ? 64 : 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    ar[u] = *(const gemm_bf16x8_t*)(ag[u] + k1);
    br[u] = *(const gemm_bf16x8_t*)(bg[u] + k1);
  }
  gemm_f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = gemm_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int wm = (wv & 1) * 64, wn = (wv >> 1) * 64;
  const int ql = lane & 15, kq = (lane >> 4) * 8;
  int cur = 0;
  for (int k0 = 0; k0 < g.K; k0 += 64) {
    __syncthreads();  // buffer cur is written; the other buffer's last reads (step k0 - 64) are done
    const int nxt = cur ^ 1;
    if (k0 + 64 < g.K) {  // step k0 + 64's tile into the other buffer, then step k0 + 128's loads
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        *(gemm_bf16x8_t*)&gsm[nxt * GT_BUF + lds_off[u]] = ar[u];
        *(gemm_bf16x8_t*)&gsm[(2 + nxt) * GT_BUF + lds_off[u]] = br[u];
      }
      const int kn = k0 + 128 < g.K ? k0 + 128 : k0;  // past the end: reload a tile in bounds (unused)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        ar[u] = *(const gemm_bf16x8_t*)(ag[u] + kn);
        br[u] = *(const gemm_bf16x8_t*)(bg[u] + kn);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // the copies and loads go out before this step's MFMAs
    const bf16_t* As = gsm + cur * GT_BUF;
    const bf16_t* Bs = gsm + (2 + cur) * GT_BUF;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      gemm_bf16x8_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = *(const gemm_bf16x8_t*)&As[(wm + 16 * i + ql) * GT_LD + 32 * h + kq];
        b[i] = *(const gemm_bf16x8_t*)&Bs[(wn + 16 * i + ql) * GT_LD + 32 * h + kq];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    cur = nxt;
  }
  gemm_store(g, acc, bm + wm, bn + wn, lane);
}

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t st) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  dim3 grid((unsigned)((g.N + 127) / 128), (unsigned)((g.M + 127) / 128));
  if (g.K % 64 == 0) {
    (void)hipFuncSetAttribute((const void*)gemm_bf16_lds_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)GEMM_LDS);
    hipLaunchKernelGGL(gemm_bf16_lds_kernel, grid, dim3(GEMM_NT), GEMM_LDS, st, g);
  }
  else
    hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(GEMM_NT), 0, st, g);
  return hipGetLastError();
}

// softplus(x) = log(1 + e^x), for large x equal to x in float32
__device__ __forceinline__ float softplus_f(float x) { return x > 20.0f ? x : log1pf(expf(x)); }

__global__ __launch_bounds__(256) void gates_kernel(const bf16_t* ga, const bf16_t* gb, int ldg, const float* a_log,
                                                    const float* dt_bias, long long S, int H, bf16_t* alpha,
                                                    bf16_t* beta) {
  const long long s = (long long)blockIdx.x * 256 + threadIdx.x;
  if (s >= S) return;
  const long long row = s / H;
  const int h = (int)(s - row * H);
  const float a = bf16_to_f(ga[row * ldg + h]), b = bf16_to_f(gb[row * ldg + h]);
  const float decay = expf(a_log[h]) * softplus_f(a + dt_bias[h]);
  alpha[s] = f_to_bf16(expf(-decay));
  beta[s] = f_to_bf16(1.0f / (1.0f + expf(-b)));
}

// A 64 x 64 tile per workgroup through LDS (rows padded to 65 elements): reads coalesced along in's rows, writes
// along out's rows.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16_t* in, int R, int C, long long ldi,
                                                             bf16_t* out, int Rp, long long ldo) {
  __shared__ bf16_t t[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4 threads
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    t[i][tx] = (r < R && c < C) ? in[(long long)r * ldi + c] : (bf16_t)0;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < C && r < Rp) out[(long long)c * ldo + r] = t[tx][i];
  }
}

hipError_t launch_transpose_bf16(const bf16_t* in, int R, int C, long long ldi, bf16_t* out, int Rp, long long ldo,
                                 hipStream_t st) {
  if (C == 0 || Rp == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)((C + 63) / 64), (unsigned)((Rp + 63) / 64)), dim3(256),
                     0, st, in, R, C, ldi, out, Rp, ldo);
  return hipGetLastError();
}

// One thread per element of d p. The gate derivatives in float32 from the bfloat16 gate inputs (alpha recomputed,
// not the rounded one): z = a + dt_bias, A = exp(a_log), d a = d alpha * alpha * (-A) * sigmoid(z),
// d b = d beta * beta * (1 - beta); the d a_log term d alpha * alpha * (-A * softplus(z)).
__global__ __launch_bounds__(256) void layer_grad_assemble_kernel(GateBwdArgs g) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= g.M * g.ldp) return;
  const long long m = i / g.ldp;
  const int c = (int)(i - m * g.ldp);
  const int HP = g.HP, Hd = g.Hd, H = g.H;
  float v = 0.f;
  if (c < HP) {
    v = g.gk[m * HP + c];
  } else if (c < 2 * HP) {
    v = g.gq[m * HP + c - HP];
  } else if (c < 2 * HP + Hd) {
    v = g.gv[m * Hd + c - 2 * HP];
  } else if (c < 2 * HP + Hd + H) {
    const int h = c - 2 * HP - Hd;
    const float a = bf16_to_f(g.gin[m * 2 * H + h]);
    const float z = a + g.dt_bias[h], A = expf(g.a_log[h]);
    const float sp = softplus_f(z), alpha = expf(-A * sp), sig = 1.0f / (1.0f + expf(-z));
    const float da = g.galpha[m * H + h];
    v = da * alpha * (-A) * sig;
    g.tparam[m * H + h] = da * alpha * (-A * sp);
    g.tparam[g.M * H + m * H + h] = v;
  } else if (c < 2 * HP + Hd + 2 * H) {
    const int h = c - 2 * HP - Hd - H;
    const float b = bf16_to_f(g.gin[m * 2 * H + H + h]);
    const float beta = 1.0f / (1.0f + expf(-b));
    v = g.gbeta[m * H + h] * beta * (1.0f - beta);
  }
  g.dp[i] = f_to_bf16(v);
}

hipError_t launch_layer_grad_assemble(const GateBwdArgs& g, hipStream_t st) {
  const long long n = g.M * g.ldp;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(layer_grad_assemble_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, g);
  return hipGetLastError();
}

// One workgroup per (head, parameter): thread t adds rows t, t + 256, ... in order, then a fixed tree over threads.
__global__ __launch_bounds__(256) void layer_param_sums_kernel(const float* tparam, long long M, int H,
                                                               float* grad_a_log, float* grad_dt_bias) {
  __shared__ float s[256];
  const int h = blockIdx.x, which = blockIdx.y, t = threadIdx.x;
  const float* src = tparam + (long long)which * M * H + h;
  float acc = 0.f;
  for (long long m = t; m < M; m += 256) acc += src[m * H];
  s[t] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (t < o) s[t] += s[t + o];
    __syncthreads();
  }
  if (t == 0) (which == 0 ? grad_a_log : grad_dt_bias)[h] = s[0];
}

hipError_t launch_layer_param_sums(const float* tparam, long long M, int H, float* grad_a_log, float* grad_dt_bias,
                                   hipStream_t st) {
  if (H == 0) return hipSuccess;
  hipLaunchKernelGGL(layer_param_sums_kernel, dim3((unsigned)H, 2), dim3(256), 0, st, tparam, M, H, grad_a_log,
                     grad_dt_bias);
  return hipGetLastError();
}

// One thread per 16-byte piece of a slot row of one head: the piece is read once and stored into every batch row.
__global__ __launch_bounds__(256) void bank_broadcast_kernel(const unsigned char* init, unsigned char* bank, int B,
                                                             int H, long long N, long long rows, long long pieces,
                                                             long long ldb) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;  // (h, j, piece)
  if (i >= (long long)H * N * pieces) return;
  const long long hp = i / pieces, p = i - hp * pieces;
  const long long h = hp / N, j = hp - h * N;
  const uint4 v = *(const uint4*)(init + (h * rows + j) * ldb + 16 * p);
  for (int b = 0; b < B; ++b) *(uint4*)(bank + (((long long)b * H + h) * rows + j) * ldb + 16 * p) = v;
}

hipError_t launch_bank_broadcast(const void* init, void* bank, int B, int H, long long N, long long rows, int d,
                                 long long ld, int esize, hipStream_t st) {
  const long long pieces = (long long)d * esize / 16;
  const long long n = (long long)H * N * pieces;
  if (n == 0 || B == 0) return hipSuccess;
  hipLaunchKernelGGL(bank_broadcast_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     (const unsigned char*)init, (unsigned char*)bank, B, H, N, rows, pieces, ld * esize);
  return hipGetLastError();
}

// One thread per 4 columns of a slot row of one head, the batch rows added in order.
// Four consecutive float32 or bfloat16 gradient entries, widened.
__device__ inline float4 load4(const float* p) { return *(const float4*)p; }
__device__ inline float4 load4(const bf16_t* p) {
  const uint2 w = *(const uint2*)p;
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                     __uint_as_float(w.y & 0xFFFF0000u));
}

template <typename G>
__global__ __launch_bounds__(256) void bank_grad_sum_kernel(const G* gb, float* gi, int B, int H, long long N,
                                                            long long rows, long long quads, long long ld) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;  // (h, j, quad)
  if (i >= (long long)H * N * quads) return;
  const long long hq = i / quads, q = i - hq * quads;
  const long long h = hq / N, j = hq - h * N;
  float4 acc = load4(gb + (h * rows + j) * ld + 4 * q);
  for (int b = 1; b < B; ++b) {
    const float4 v = load4(gb + (((long long)b * H + h) * rows + j) * ld + 4 * q);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  *(float4*)(gi + (h * rows + j) * ld + 4 * q) = acc;
}

hipError_t launch_bank_grad_sum(const void* grad_bank, bool bf16, float* grad_init, int B, int H, long long N,
                                long long rows, int d, long long ld, hipStream_t st) {
  const long long quads = d / 4;
  const long long n = (long long)H * N * quads;
  if (n == 0 || B == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL(bank_grad_sum_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)grad_bank, grad_init, B,
                       H, N, rows, quads, ld);
  else
    hipLaunchKernelGGL(bank_grad_sum_kernel<float>, grid, dim3(256), 0, st, (const float*)grad_bank, grad_init, B, H,
                       N, rows, quads, ld);
  return hipGetLastError();
}

hipError_t launch_gates(const bf16_t* ga, const bf16_t* gb, int ldg, const float* a_log, const float* dt_bias,
                        long long S, int H, bf16_t* alpha, bf16_t* beta, hipStream_t st) {
  if (S == 0) return hipSuccess;
  hipLaunchKernelGGL(gates_kernel, dim3((unsigned)((S + 255) / 256)), dim3(256), 0, st, ga, gb, ldg, a_log, dt_bias,
                     S, H, alpha, beta);
  return hipGetLastError();
}

}  // namespace sdm
