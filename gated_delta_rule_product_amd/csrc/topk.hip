// Exact product-key top-k kernels: the candidate table and the batched top-k (write keys and read queries).
#include "sdm_internal.h"
#include "topk_device.h"

namespace sdm {

// One thread enumerates, in lexicographic order, the position tuples with prod(p_f + 1) <= k and p_f < kp[f]
// (an odometer that skips the rest of a digit's range once the prefix product exceeds k).
__global__ void cand_table_kernel(TopkPlan P, int F, uint64_t* __restrict__ table) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int p[MAX_F] = {0, 0, 0, 0};
  int c = 0;
  while (true) {
    long long prod = 1;
    for (int f = 0; f < F; ++f) prod *= p[f] + 1;
    if (prod <= P.k && c < MAX_CAND) {
      uint64_t t = 0;
      for (int f = 0; f < F; ++f) t |= (uint64_t)p[f] << (16 * f);
      table[c++] = t;
    }
    int f = F - 1;
    for (; f >= 0; --f) {
      ++p[f];
      long long pp = 1;
      for (int g = 0; g <= f; ++g) pp *= p[g] + 1;
      if (p[f] < P.kp[f] && pp <= P.k) break;
      p[f] = 0;
    }
    if (f < 0) break;
  }
}

hipError_t launch_cand_table(const TopkPlan& p, int F, uint64_t* table, hipStream_t st) {
  hipLaunchKernelGGL(cand_table_kernel, dim3(1), dim3(64), 0, st, p, F, table);
  return hipGetLastError();
}

template <typename A>
__global__ __launch_bounds__(TOPK_NT) void topk_kernel(Dims D, TopkArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int kind = blockIdx.y;
  const TopkPlan& P = a.plan[kind];
  const long long row = blockIdx.x;  // (b * T + t) * H + h
  const int h = (int)(row % D.H);
  const long long bt = row / D.H;
  const int t = (int)(bt % D.T);
  const int b = (int)(bt / D.T);
  const int Fdk = D.F * D.dk;
  long long sumn = 0;
  for (int f = 0; f < D.F; ++f) sumn += D.widths[f];
  const A* q = (const A*)a.queries[kind] + row * Fdk;
  const A* sub = (const A*)a.subkeys + (long long)h * sumn * D.dk;
  TopkLds L = topk_lds_carve(lds, D.F, D.dk, P);
  topk_query<A, TOPK_NT>(q, sub, D.widths, D.F, D.dk, P, a.cand[kind], L);
  const int k = P.k;
  if (a.stream_major) {
    const long long so = (((long long)b * D.H + h) * D.T + t) * k;
    for (int r = threadIdx.x; r < k; r += TOPK_NT) a.ids[kind][so + r] = L.rid[r];
    if (a.user_ids[kind])
      for (int r = threadIdx.x; r < k; r += TOPK_NT) a.user_ids[kind][row * k + r] = L.rid[r];
    topk_softmax<TOPK_NT>(L, k, a.vals[kind] + so);
  } else {
    for (int r = threadIdx.x; r < k; r += TOPK_NT) a.ids[kind][row * k + r] = L.rid[r];
    if (a.vals[kind])
      for (int r = threadIdx.x; r < k; r += TOPK_NT) a.vals[kind][row * k + r] = L.rsc[r];
  }
}

hipError_t launch_topk(const Dims& D, const TopkArgs& a, hipStream_t st) {
  const long long rows = (long long)D.B * D.T * D.H;
  if (rows == 0) return hipSuccess;
  size_t lds = 0;
  for (int q = 0; q < a.nkinds; ++q) {
    size_t l = topk_lds_bytes(D.F, D.dk, a.plan[q]);
    if (l > lds) lds = l;
  }
  dim3 grid((unsigned)rows, (unsigned)a.nkinds);
  if (D.act == SDM_BF16)
    hipLaunchKernelGGL(topk_kernel<bf16_t>, grid, dim3(TOPK_NT), lds, st, D, a);
  else
    hipLaunchKernelGGL(topk_kernel<float>, grid, dim3(TOPK_NT), lds, st, D, a);
  return hipGetLastError();
}

}  // namespace sdm
