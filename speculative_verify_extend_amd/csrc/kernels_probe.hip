// Measurement probes: a plain streaming read and a plain copy of device
// memory. They set the measured HBM ceilings next to the published peak and
// calibrate the hardware traffic counters (a copy of known size moves a
// known number of bytes).
#include "common.h"
#include "launch.h"

namespace sve {

// Each thread issues U independent 16-byte loads per step, grid-stride over
// the buffer, and folds them into one value so the loads stay live.
template <int U>
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
  const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  uint32_t accv = 0;
  size_t i = tid;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) accv ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = src[i];
    accv ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  sink[tid] = accv;
}

__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4* __restrict__ src,
                                                         u32x4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

hipError_t launch_probe_read(const void* src, size_t bytes, int blocks, int unroll, void* sink,
                             hipStream_t st) {
  const size_t n16 = bytes / 16;
  const dim3 g(blocks), b(256);
  switch (unroll) {
    case 1: hipLaunchKernelGGL(probe_read_kernel<1>, g, b, 0, st, (const u32x4*)src, n16, (uint32_t*)sink); break;
    case 2: hipLaunchKernelGGL(probe_read_kernel<2>, g, b, 0, st, (const u32x4*)src, n16, (uint32_t*)sink); break;
    case 8: hipLaunchKernelGGL(probe_read_kernel<8>, g, b, 0, st, (const u32x4*)src, n16, (uint32_t*)sink); break;
    default: hipLaunchKernelGGL(probe_read_kernel<4>, g, b, 0, st, (const u32x4*)src, n16, (uint32_t*)sink); break;
  }
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t st) {
  hipLaunchKernelGGL(probe_copy_kernel, dim3(blocks), dim3(256), 0, st, (const u32x4*)src,
                     (u32x4*)dst, bytes / 16);
  return hipGetLastError();
}

}  // namespace sve
