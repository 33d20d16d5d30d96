// Device-side helpers shared by the gfx950 kernels of libsve.
// Wave64 throughout; MFMA operand types for v_mfma_f32_16x16x32_bf16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sve {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even float -> bf16 pair (hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// two floats to fp16 (round to nearest even), low half first
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 v;
  v[0] = (_Float16)lo;
  v[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D = A(16x32) * B(32x16) + C. Lane l supplies A row (l%16), B column (l%16),
// each with 8 consecutive contraction elements of block (l/16); lane l
// receives D rows 4*(l/16)+i, column l%16, i = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void store16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// Direct global-to-LDS loads (buffer_load ... lds, 16 bytes per lane)
// through raw buffer resources: LDS pointer type and word 3 of a resource
// (32-bit data format, no swizzle).
typedef __attribute__((address_space(3))) void lds_void;
constexpr int kBufWord3 = 0x00020000;

// Cache policy of a buffer store that writes through this XCD's L2 (the
// sc1 bit: device scope). Split partials leave this way: the kernel that
// adds them runs on every XCD and finds them in memory, instead of dirty in
// the writer's L2 until that kernel's end writes the L2 back.
constexpr int kStoreThrough = 16;

// wait until at most N vector-memory requests of this wave are outstanding
// (lgkm and export counters untouched)
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ float xor_shfl(float v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

// max over lanes l, l^16, l^32, l^48 with the gfx950 row-swap permutes:
// permlane32_swap(x, x) leaves (x[l % 32], x[l % 32 + 32]) in its two
// results and permlane16_swap(x, x) the two 16-lane rows of each half, so
// one max per step combines the partner lanes without going through LDS.
__device__ __forceinline__ float max4_rows(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

}  // namespace sve
