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
// Y = X W^T: X [M, K], W [N, K] bfloat16 row-major, K % 32 == 0; nseg segments cover [0, N).
struct GemmArgs {
  const bf16_t* x;
  const bf16_t* w;
  int M, N, K;
  int nseg;
  GemmSeg seg[GEMM_MAXSEG];
};
hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t st);
// alpha, beta [S] from gate inputs ga[row * ldg + h], gb[row * ldg + h] (S = rows * H).
hipError_t launch_gates(const bf16_t* ga, const bf16_t* gb, int ldg, const float* a_log, const float* dt_bias,
                        long long S, int H, bf16_t* alpha, bf16_t* beta, hipStream_t st);

// The layer's per-sequence bank copy: bank[b, h, j, :d] = init[h, j, :d] for every batch row b and slot j < N (rows
// ld elements apart in both; esize 2 or 4 bytes; d * esize a multiple of 16).
hipError_t launch_bank_broadcast(const void* init, void* bank, int B, int H, long long N, long long rows, int d,
                                 long long ld, int esize, hipStream_t st);
// grad_init[h, j, c] = sum over b = 0, 1, ... B-1 (in that order, float32) of grad_bank[b, h, j, c], j < N, c < d
// (grad_bank float32, or bfloat16 with bf16; d a multiple of 4).
hipError_t launch_bank_grad_sum(const void* grad_bank, bool bf16, float* grad_init, int B, int H, long long N,
                                long long rows, int d, long long ld, hipStream_t st);

}  // namespace sdm
