// Slot matcher support on gfx950: longest common prefixes of token lists.
//
// One workgroup per pair (prompt vs slot, or slot vs slot): the first index
// where the two lists differ, scanned 1024 tokens at a time with an early
// exit once a mismatch is seen. The decision rule itself runs on the host
// over the handful of lengths this produces.
#include "common.h"
#include "launch.h"

namespace sve {

__global__ __launch_bounds__(256) void lcp_kernel(LcpArgs args) {
  const int p = blockIdx.x;
  const int32_t* a = args.a[p];
  const int32_t* b = args.b[p];
  const int n = args.n[p];
  __shared__ int found;
  if (threadIdx.x == 0) found = n;
  __syncthreads();
  for (int base = 0; base < n; base += 1024) {
    int local = n;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = base + threadIdx.x + 256 * u;
      if (j < n && a[j] != b[j]) local = min(local, j);
    }
    if (local < n) atomicMin(&found, local);
    __syncthreads();
    const bool stop = found < n;
    __syncthreads();
    if (stop) break;
  }
  if (threadIdx.x == 0) args.out[p] = found;
}

hipError_t launch_lcp(const LcpArgs& args, hipStream_t st) {
  if (args.npairs == 0) return hipSuccess;
  hipLaunchKernelGGL(lcp_kernel, dim3(args.npairs), dim3(256), 0, st, args);
  return hipGetLastError();
}

}  // namespace sve
