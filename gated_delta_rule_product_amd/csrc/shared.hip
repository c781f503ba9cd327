// Shared-bank disjointness check (sparse-delta-memory CHANGELOG.md 2.0.0, "Behavior changes": several streams over
// one shared bank must say so, which asserts that their slots are disjoint). After the top-k, every slot addressed
// by stream (b, h), written or read, is claimed for b in an owner table of head h; a slot that another stream of
// the head has claimed sets the conflict flag, which makes the plan and the chunk loop do nothing. The flag is
// order independent (it is set iff some slot is addressed by two streams of a head), so the check is
// deterministic; the claims are integer compare-and-swap operations.
#include "sdm_internal.h"

namespace sdm {

// owner[i] = -1 for i < n; flag = 0 (plain stores: no memset node when the call is captured into a graph)
__global__ __launch_bounds__(256) void shared_clear_kernel(int32_t* __restrict__ owner, long long n,
                                                           int32_t* __restrict__ flag) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) owner[i] = -1;
  if (blockIdx.x == 0 && threadIdx.x == 0) *flag = 0;
}

// One thread per address: stream-major ids [S][T][k] (s = b * H + h), k = W for the write ids and R for the read ids
__global__ __launch_bounds__(256) void shared_claim_kernel(Dims D, const int32_t* __restrict__ widx,
                                                           const int32_t* __restrict__ ridx,
                                                           int32_t* __restrict__ owner, int32_t* __restrict__ flag) {
  const long long nw = (long long)D.S * D.T * D.W, nr = (long long)D.S * D.T * D.R;
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nw + nr) return;
  const bool w = i < nw;
  const long long j = w ? i : i - nw;
  const long long per = (long long)D.T * (w ? D.W : D.R);  // addresses per stream
  const int s = (int)(j / per);
  const int b = s / D.H, h = s % D.H;
  const int slot = w ? widx[j] : ridx[j];
  const int old = atomicCAS(&owner[(long long)h * D.N + slot], -1, b);
  if (old != -1 && old != b) atomicOr(flag, 1);
}

hipError_t launch_shared_check(const Dims& D, const int32_t* widx, const int32_t* ridx, int32_t* owner,
                               int32_t* flag, hipStream_t st) {
  const long long n = (long long)D.H * D.N;
  long long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(shared_clear_kernel, dim3((unsigned)blocks), dim3(256), 0, st, owner, n, flag);
  const long long na = (long long)D.S * D.T * (D.W + D.R);
  if (na > 0)
    hipLaunchKernelGGL(shared_claim_kernel, dim3((unsigned)((na + 255) / 256)), dim3(256), 0, st, D, widx, ridx,
                       owner, flag);
  return hipGetLastError();
}

}  // namespace sdm
