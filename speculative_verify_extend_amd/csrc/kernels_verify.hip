// Greedy acceptance of a speculative verify step on gfx950.
//
// thinkspread, "The economics of speculative decoding" (opening section): a
// draft head proposes k tokens, one pass over m = k + 1 rows checks them, and
// the runtime keeps the ones that were right. Row i of the verify logits
// predicts the token after input i (inputs: the last accepted token, then
// the k drafts); draft i+1 is kept while it equals row i's argmax, and the
// row after the last kept draft gives the next token. Argmax ties go to the
// lowest token id and a NaN counts as larger than any number.
//
// Two launches: per (row, 4096-entry chunk) a workgroup reduces its chunk to
// (largest value, its first index); then one wave per row reduces the row's
// chunk results and one lane runs the acceptance scan. The order (value descending, index
// ascending) is total, so the result does not depend on the reduction order.
#include <climits>
#include <mutex>

#include "common.h"
#include "launch.h"

namespace sve {

constexpr int kVerifyChunk = 4096;  // logits per first-pass workgroup
constexpr int kVerifyThreads = 256;

// (va, ia) comes before (vb, ib): NaN first, then larger values, then the
// lower index among equal values
__device__ __forceinline__ bool verify_before(float va, int ia, float vb, int ib) {
  const bool na = va != va, nb = vb != vb;
  if (na || nb) return na && (!nb || ia < ib);
  return va > vb || (va == vb && ia < ib);
}

__device__ __forceinline__ void verify_take(float& bv, int& bi, float v, int i) {
  if (verify_before(v, i, bv, bi)) {
    bv = v;
    bi = i;
  }
}

// wave-wide best of (bv, bi)
__device__ __forceinline__ void verify_wave_best(float& bv, int& bi) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(bv, o, kWave);
    const int oi = __shfl_xor(bi, o, kWave);
    verify_take(bv, bi, ov, oi);
  }
}

// grid (chunks, m), block 256: best entry of logits[row][chunk] into
// part_v / part_i [row][chunk]
__global__ __launch_bounds__(kVerifyThreads) void verify_argmax_partial_kernel(
    const float* __restrict__ logits, int V, int nchunk, int vec4, float* __restrict__ part_v,
    int* __restrict__ part_i) {
  const int row = blockIdx.y, c = blockIdx.x;
  const float* x = logits + (size_t)row * V;
  const int lo = c * kVerifyChunk, hi = min(V, lo + kVerifyChunk);
  float bv = -INFINITY;
  int bi = INT_MAX;  // any entry comes before this
  if (vec4) {
    // rows start 16-byte aligned and V % 4 == 0: one float4 per lane and step
    for (int j = lo + 4 * threadIdx.x; j < hi; j += 4 * kVerifyThreads) {
      const float4 v = *reinterpret_cast<const float4*>(x + j);
      verify_take(bv, bi, v.x, j);
      verify_take(bv, bi, v.y, j + 1);
      verify_take(bv, bi, v.z, j + 2);
      verify_take(bv, bi, v.w, j + 3);
    }
  } else {
    for (int j = lo + threadIdx.x; j < hi; j += kVerifyThreads) verify_take(bv, bi, x[j], j);
  }
  verify_wave_best(bv, bi);
  __shared__ float sv[kVerifyThreads / kWave];
  __shared__ int si[kVerifyThreads / kWave];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (lane == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kVerifyThreads / kWave; ++w) verify_take(bv, bi, sv[w], si[w]);
    part_v[(size_t)row * nchunk + c] = bv;
    part_i[(size_t)row * nchunk + c] = bi;
  }
}

// one wave per row: its argmax from the chunk results; then one lane runs the
// acceptance scan. result: [0] accepted drafts, [1] next token, [2 + i]
// argmax of row i.
__global__ __launch_bounds__(kWave * kVerifyMaxRows) void verify_accept_kernel(
    const float* __restrict__ part_v, const int* __restrict__ part_i, int m, int nchunk,
    const int32_t* __restrict__ draft, int32_t* __restrict__ result) {
  __shared__ int top[kVerifyMaxRows];
  const int row = threadIdx.x / kWave, lane = threadIdx.x % kWave;  // blockDim = 64 * m
  float bv = -INFINITY;
  int bi = INT_MAX;
  for (int c = lane; c < nchunk; c += kWave)
    verify_take(bv, bi, part_v[(size_t)row * nchunk + c], part_i[(size_t)row * nchunk + c]);
  verify_wave_best(bv, bi);
  if (lane == 0) {
    top[row] = bi;
    result[2 + row] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int a = 0;
    while (a < m - 1 && draft[a] == top[a]) ++a;
    result[0] = a;
    result[1] = top[a];
  }
}

size_t verify_workspace_bytes(int m, int V) {
  const size_t nchunk = ((size_t)V + kVerifyChunk - 1) / kVerifyChunk;
  const size_t half = ((size_t)m * nchunk * 4 + 255) / 256 * 256;
  return 2 * half;
}

// Scratch of the allocation-free entry point: the per-(row, chunk) partial
// results of up to kVerifyMaxRows rows of kVerifyNoAllocMaxV logits (the
// layout of verify_workspace_bytes). Every GPU the library runs on holds its
// own copy until the process ends; every call on that GPU shares it, so
// calls that overlap on one GPU race. Nothing in it has to start at zero:
// the first kernel writes every (row, chunk) entry the second one reads.
constexpr size_t kVerifyScratchBytes =
    2 * (((size_t)kVerifyMaxRows * (kVerifyNoAllocMaxV / kVerifyChunk) * 4 + 255) / 256 * 256);
static __device__ __align__(256) uint8_t scratch[kVerifyScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each GPU
}  // namespace

// Device address of this GPU's copy of `scratch`, looked up once per device
// (with that device current). In host code the array's name only stands in
// for the symbol: kernels get the looked-up address.
static hipError_t verify_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_verify_accept_noalloc(const float* logits, int m, int V, const int32_t* draft,
                                        int32_t* result, hipStream_t st) {
  if (verify_workspace_bytes(m, V) > kVerifyScratchBytes) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t e = verify_scratch(&ws);
  if (e != hipSuccess) return e;
  return launch_verify_accept(logits, m, V, draft, result, ws, st);
}

hipError_t launch_verify_accept(const float* logits, int m, int V, const int32_t* draft,
                                int32_t* result, void* workspace, hipStream_t st) {
  const int nchunk = (V + kVerifyChunk - 1) / kVerifyChunk;
  const size_t half = verify_workspace_bytes(m, V) / 2;
  float* part_v = (float*)workspace;
  int* part_i = (int*)((char*)workspace + half);
  const int vec4 = (V % 4 == 0) && ((uintptr_t)logits % 16 == 0);
  hipLaunchKernelGGL(verify_argmax_partial_kernel, dim3(nchunk, m), dim3(kVerifyThreads), 0, st,
                     logits, V, nchunk, vec4, part_v, part_i);
  hipLaunchKernelGGL(verify_accept_kernel, dim3(1), dim3(kWave * m), 0, st, part_v, part_i, m,
                     nchunk, draft, result);
  return hipGetLastError();
}

}  // namespace sve
