// Prefill path (a chunk of many tokens): token->expert grouping and the
// grouped expert GEMMs.
#include "device.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// Deterministic token->expert grouping by one workgroup of 1024 threads:
// histogram (LDS integer atomics: the counts do not depend on their order),
// exclusive scan, then one thread per expert walks the pairs in (token, slot)
// order, so pairs of an expert appear in ascending token order.  Rockchip-NPU
// plan §8.4: one fetched expert serves every row of the chunk that chose it.
__global__ __launch_bounds__(1024) void sort_kernel(const int32_t* __restrict__ ids, int T, int K, int E,
                                                   int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv) {
  extern __shared__ int32_t sh[];  // cnt[E], off[E+1]
  int32_t* cnt = sh;
  int32_t* off = sh + E;
  const int tid = threadIdx.x, n = T * K;
  for (int e = tid; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += blockDim.x) {
    const int e = ids[i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (tid == 0) {  // E <= 1024: a serial scan is cheaper than its barriers
    int run = 0;
    for (int e = 0; e < E; ++e) {
      off[e] = run;
      run += cnt[e];
    }
    off[E] = run;
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    counts[e] = cnt[e];
    offsets[e] = off[e];
    int pos = off[e];
    for (int i = 0; i < n; ++i)
      if (ids[i] == e) {
        perm[pos] = i;
        inv[i] = pos;
        ++pos;
      }
  }
  if (tid == 0) offsets[E] = off[E];
}

}  // namespace

hipError_t launch_sort(const int32_t* ids, int T, int K, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                       int32_t* inv, hipStream_t s) {
  const size_t lds = (size_t)(2 * E + 1) * 4;
  sort_kernel<<<1, 1024, lds, s>>>(ids, T, K, E, counts, offsets, perm, inv);
  return hipGetLastError();
}

size_t prefill_workspace_bytes(int T, int d, int E, int K, int f, int fs) {
  (void)T; (void)d; (void)E; (void)K; (void)f; (void)fs;
  return 256;
}

void prefill_carve(PrefillArgs& p, char* ws, int T, int d, int E, int K, int f, int fs) {
  (void)p; (void)ws; (void)T; (void)d; (void)E; (void)K; (void)f; (void)fs;
}

hipError_t launch_prefill(const PrefillArgs& p, hipStream_t s) {
  (void)p; (void)s;
  return hipErrorNotSupported;
}

}  // namespace moe
