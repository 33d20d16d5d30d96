// Measurement probes: the achievable ceilings of this chip next to its
// published peaks, and a kernel of known traffic to calibrate the hardware
// counters. None of them is part of the computation.
//
//   streaming read, three ways: plain 16-byte loads, the same with the
//     nontemporal hint, and direct global-to-LDS loads (buffer_load ... lds,
//     which hold no registers while in flight); grid, workgroup size and
//     loads in flight per wave are the caller's, so a sweep finds the best
//     launch shape for a given byte count;
//   a cache-resident direct-to-LDS fill (a small region read over and over:
//     the rate one CU fills LDS from L2);
//   plain copy (counter calibration: a known number of bytes each way);
//   compute: v_mfma_f32_16x16x32_bf16, v_mfma_f32_32x32x16_bf16 and
//     v_mfma_f32_16x16x32_f16 issue rates, v_exp_f32 throughput, and LDS
//     read bandwidth (ds_read_b128).
#include "common.h"
#include "launch.h"

namespace sve {

// Each thread issues U independent 16-byte loads per step, grid-stride over
// the buffer, and folds them into one value so the loads stay live.
template <int U, bool NT>
__global__ __launch_bounds__(1024) void probe_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t accv = 0;
  size_t i = tid;
  auto ld = [&](size_t j) -> u32x4 {
    if constexpr (NT)
      return __builtin_nontemporal_load(src + j);
    else
      return src[j];
  };
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld(i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) accv ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = ld(i);
    accv ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  sink[tid] = accv;
}

// Direct global-to-LDS streaming read: wave w of a workgroup takes the
// 1 KB chunks c = (block * W + w) + k * (grid * W), each one wave-wide
// 16-byte buffer load into its own ring of U LDS slots; at most U loads are
// in flight per wave (the wait before reusing a slot covers only the oldest).
// The data is not consumed: the probe measures how fast HBM fills LDS.
template <int U>
__global__ __launch_bounds__(1024) void probe_read_lds_kernel(const uint8_t* __restrict__ src,
                                                              size_t bytes,
                                                              uint32_t* __restrict__ sink) {
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];  // [W][U][1024]
  const int W = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const size_t nchunks = bytes >> 10;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(src), (short)0, (int)min(bytes, (size_t)0x7FFFFFFF), kBufWord3);
  uint8_t* mine = ring + (size_t)wave * U * 1024;
  size_t c = (size_t)blockIdx.x * W + wave;
  const size_t stride = (size_t)gridDim.x * W;
  int n = 0;
  for (; c < nchunks; c += stride, ++n) {
    if (n >= U) wait_vmem<U - 1>();  // the slot's previous load has landed
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(mine + (n % U) * 1024), 16,
                                             lane * 16, (int)(c << 10), 0, 0);
  }
  wait_vmem<0>();
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = (uint32_t)n + mine[lane];
}

// Cache-resident direct-to-LDS fill: every wave streams 32 KB tiles of a
// small region (tile (block * W + wave) + t, cycling over the region), each
// tile as 32 one-KB requests into two 16 KB halves of its own LDS, waiting
// for a half's previous requests before refilling it (at most 32 KB in
// flight per wave). With a region that fits in L2 this is the rate at which
// one CU can fill LDS from L2 (the bound of a workgroup that reads every
// tile once for few rows). The data is not consumed.
__global__ __launch_bounds__(256) void probe_l2_lds_kernel(const uint8_t* __restrict__ src,
                                                           size_t bytes, int tiles,
                                                           uint32_t* __restrict__ sink) {
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];  // [W][2][16 KB]
  const int W = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(src), (short)0, (int)bytes, kBufWord3);
  const int ntile = (int)(bytes >> 15);
  int tt = (int)(((size_t)blockIdx.x * W + wave) % ntile);
  uint8_t* mine = ring + (size_t)wave * 32768;
  for (int t = 0; t < tiles; ++t) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (t > 0) wait_vmem<16>();  // this half's previous requests have landed
#pragma unroll
      for (int u = 0; u < 16; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(mine + h * 16384 + u * 1024), 16,
                                                 lane * 16, tt * 32768 + h * 16384 + u * 1024, 0,
                                                 0);
    }
    tt = tt + 1 == ntile ? 0 : tt + 1;
  }
  wait_vmem<0>();
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = (uint32_t)tiles + mine[lane];
}

__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4* __restrict__ src,
                                                         u32x4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// ---- compute probes: blocks of 256 threads (4 waves), `iters` iterations
// each; per wave and iteration: 8 matrix products (eight independent
// accumulators), 64 exponentials (eight independent chains of 8), or 8 LDS
// reads of 16 bytes per lane ----------------------------------------------------
constexpr int kProbeChains = 8;

template <int KIND>
__global__ __launch_bounds__(256) void probe_compute_kernel(int iters, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  uint32_t out = 0;
  if constexpr (KIND == 0 || KIND == 1 || KIND == 2) {
    // operands from the lane index: finite, nonzero, never rewritten
    u32x4 av = {0x3F803F80u + (uint32_t)lane, 0x3F003F00u, 0x3E803E80u, 0x3F403F40u};
    if constexpr (KIND == 2) av = u32x4{0x3C003C00u + (uint32_t)lane, 0x38003800u, 0x3A003A00u,
                                         0x3B003B00u};
    if constexpr (KIND == 1) {
      typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
      f32x16 acc[kProbeChains];
#pragma unroll
      for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
      const bf16x8 a = as_bf16x8(av);
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int c = 0; c < kProbeChains; ++c)
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[c], 0, 0, 0);
#pragma unroll
      for (int c = 0; c < kProbeChains; ++c) out ^= __float_as_uint(acc[c][0]);
    } else {
      f32x4 acc[kProbeChains];
#pragma unroll
      for (int c = 0; c < kProbeChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int c = 0; c < kProbeChains; ++c) {
          if constexpr (KIND == 0) {
            acc[c] = mfma16x16x32(as_bf16x8(av), as_bf16x8(av), acc[c]);
          } else {
            typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av),
                                                            __builtin_bit_cast(f16x8, av), acc[c],
                                                            0, 0, 0);
          }
        }
#pragma unroll
      for (int c = 0; c < kProbeChains; ++c) out ^= __float_as_uint(acc[c][0]);
    }
  } else if constexpr (KIND == 3) {
    // x <- 2^(-x) stays in (0, 1] and converges (no overflow, no denormals)
    float x[kProbeChains];
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) x[c] = 0.01f * (float)(lane + c);
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < kProbeChains; ++c) x[c] = __builtin_amdgcn_exp2f(-x[c]);
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) out ^= __float_as_uint(x[c]);
  } else {
    // LDS reads: each lane walks 16-byte slots of a 64 KB buffer (every
    // lane of a read on a distinct 16-byte slot, no bank conflicts)
    __shared__ __attribute__((aligned(16))) u32x4 lds[4096];
    for (int i = threadIdx.x; i < 4096; i += 256) lds[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
    __syncthreads();
    u32x4 acc = {0u, 0u, 0u, 0u};
    int base = (threadIdx.x >> 6) * 1024 + lane;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const u32x4 v = lds[(base + 64 * r) & 4095];
        acc[0] ^= v[0];
        acc[1] += v[1];
      }
      base += 512;
    }
    out = acc[0] ^ acc[1];
  }
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = out;
}

hipError_t launch_probe_read(const void* src, size_t bytes, int blocks, int threads, int unroll,
                             int mode, void* sink, hipStream_t st) {
  const dim3 g(blocks), b(threads);
  uint32_t* sk = (uint32_t*)sink;
  if (mode == 3) {
    const size_t lds = (size_t)(threads / 64) * 32768;
    hipError_t e = hipFuncSetAttribute((const void*)probe_l2_lds_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(probe_l2_lds_kernel, g, b, lds, st, (const uint8_t*)src, bytes, 8 * unroll,
                       sk);
    return hipGetLastError();
  }
  if (mode == 2) {
    const size_t lds = (size_t)(threads / 64) * unroll * 1024;
    auto go = [&](auto kern) {
      // rings beyond the default 64 KB of dynamic LDS need the attribute
      hipError_t e = hipFuncSetAttribute((const void*)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kern, g, b, lds, st, (const uint8_t*)src, bytes, sk);
      return hipGetLastError();
    };
    switch (unroll) {
      case 1: return go(probe_read_lds_kernel<1>);
      case 2: return go(probe_read_lds_kernel<2>);
      case 4: return go(probe_read_lds_kernel<4>);
      case 8: return go(probe_read_lds_kernel<8>);
      default: return go(probe_read_lds_kernel<16>);
    }
  }
  const u32x4* s = (const u32x4*)src;
  const size_t n16 = bytes / 16;
#define SVE_PROBE_READ(U)                                                         \
  if (mode == 1)                                                                  \
    hipLaunchKernelGGL((probe_read_kernel<U, true>), g, b, 0, st, s, n16, sk);    \
  else                                                                            \
    hipLaunchKernelGGL((probe_read_kernel<U, false>), g, b, 0, st, s, n16, sk)
  switch (unroll) {
    case 1: SVE_PROBE_READ(1); break;
    case 2: SVE_PROBE_READ(2); break;
    case 4: SVE_PROBE_READ(4); break;
    case 8: SVE_PROBE_READ(8); break;
    default: SVE_PROBE_READ(16); break;
  }
#undef SVE_PROBE_READ
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t st) {
  hipLaunchKernelGGL(probe_copy_kernel, dim3(blocks), dim3(256), 0, st, (const u32x4*)src,
                     (u32x4*)dst, bytes / 16);
  return hipGetLastError();
}

hipError_t launch_probe_compute(int kind, int blocks, int iters, void* sink, hipStream_t st) {
  const dim3 g(blocks), b(256);
  uint32_t* sk = (uint32_t*)sink;
  switch (kind) {
    case 0: hipLaunchKernelGGL(probe_compute_kernel<0>, g, b, 0, st, iters, sk); break;
    case 1: hipLaunchKernelGGL(probe_compute_kernel<1>, g, b, 0, st, iters, sk); break;
    case 2: hipLaunchKernelGGL(probe_compute_kernel<2>, g, b, 0, st, iters, sk); break;
    case 3: hipLaunchKernelGGL(probe_compute_kernel<3>, g, b, 0, st, iters, sk); break;
    default: hipLaunchKernelGGL(probe_compute_kernel<4>, g, b, 0, st, iters, sk); break;
  }
  return hipGetLastError();
}

}  // namespace sve
