// Launchers of the layer's dense maps and gates (layer.hip).
#pragma once
#include "sdm_internal.h"

namespace sdm {

// Output columns [previous end, end) of a dense map go to dst, row stride ld elements.
struct GemmSeg {
  int end;
  bf16_t* dst;
  int ld;
};
constexpr int GEMM_MAXSEG = 5;
// Y = X W^T: X [M, K], W [N, K] bfloat16 row-major, K % 32 == 0; nseg segments cover [0, N) (bfloat16 results),
// or, with f32 set, float32 results in f32[m * f32ld + n] (the segments unused).
struct GemmArgs {
  const bf16_t* x;
  const bf16_t* w;
  int M, N, K;
  int nseg;
  GemmSeg seg[GEMM_MAXSEG];
  float* f32;
  long long f32ld;
};
hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t st);
// alpha, beta [S] from gate inputs ga[row * ldg + h], gb[row * ldg + h] (S = rows * H).
hipError_t launch_gates(const bf16_t* ga, const bf16_t* gb, int ldg, const float* a_log, const float* dt_bias,
                        long long S, int H, bf16_t* alpha, bf16_t* beta, hipStream_t st);

// out[c * ldo + r] = in[r * ldi + c] for r < R, c < C, and 0 for R <= r < Rp (bfloat16; a zero-padded transpose).
hipError_t launch_transpose_bf16(const bf16_t* in, int R, int C, long long ldi, bf16_t* out, int Rp, long long ldo,
                                 hipStream_t st);
// The layer backward's assembly of d p [M, ldp] (bfloat16): columns [0, HP) d keys, [HP, 2 HP) d queries,
// [2 HP, 2 HP + Hd) d values (the op's float32 gradients, rounded), then d a and d b per head from the op's d alpha,
// d beta, the gate inputs gin [M, 2 H] (a then b) and the gate parameters, zeros up to ldp; tparam [2][M][H] the
// per-row terms of d a_log and d dt_bias.
struct GateBwdArgs {
  const float* gk; const float* gq; const float* gv; const float* galpha; const float* gbeta;
  const bf16_t* gin; const float* a_log; const float* dt_bias;
  bf16_t* dp; float* tparam;
  long long M; int H, HP, Hd, ldp;
};
hipError_t launch_layer_grad_assemble(const GateBwdArgs& g, hipStream_t st);
// grad_a_log[h] = sum over m of tparam[0][m][h], grad_dt_bias[h] = sum of tparam[1][m][h] (a fixed order).
hipError_t launch_layer_param_sums(const float* tparam, long long M, int H, float* grad_a_log, float* grad_dt_bias,
                                   hipStream_t st);

// The layer's per-sequence bank copy: bank[b, h, j, :d] = init[h, j, :d] for every batch row b and slot j < N (rows
// ld elements apart in both; esize 2 or 4 bytes; d * esize a multiple of 16).
hipError_t launch_bank_broadcast(const void* init, void* bank, int B, int H, long long N, long long rows, int d,
                                 long long ld, int esize, hipStream_t st);
// grad_init[h, j, c] = sum over b = 0, 1, ... B-1 (in that order, float32) of grad_bank[b, h, j, c], j < N, c < d
// (grad_bank float32, or bfloat16 with bf16; d a multiple of 4).
hipError_t launch_bank_grad_sum(const void* grad_bank, bool bf16, float* grad_init, int B, int H, long long N,
                                long long rows, int d, long long ld, hipStream_t st);

}  // namespace sdm
