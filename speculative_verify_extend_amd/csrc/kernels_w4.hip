// int4 group-32 weights on gfx950: device layout, dequantisation and the
// m-row GEMV (dense and expert-routed).
//
// Logical format (what callers hold): nibbles uint8 [N][K/2], element k of
// row n in the low nibble of byte k/2 when k is even, the high nibble when
// odd; fp16 scales [N][K/32]; value = (code - 8) * scale. This is the plain
// group-32 / zero-point-8 block with one fp16 scale (thinkspread, "Models and
// quantizations", section "Quantizations": 32-element blocks used in place).
//
// Device format (written once by w4_pack, read by every GEMV): rows are cut
// into tiles of 16 and k into quads of 4 groups (128 k). Tile (t, q) is one
// 1024-byte nibble block followed, in a separate region, by a 128-byte scale
// block:
//   nibble block: lane l (0..63) owns bytes [16l, 16l+16); dword j (0..3)
//     holds group 4q+j, row 16t + l%16, elements 8*(l/16) .. +7 of the group;
//     inside the dword element e sits at bit 4*(e/2) for even e and at bit
//     16 + 4*(e/2) for odd e, so (dw >> 4s) & 0x000F000F yields the codes of
//     elements (2s, 2s+1) in the two 16-bit halves.
//   scale block: row r (0..15) owns 8 bytes: the fp16 scales of groups
//     4q..4q+3.
// One wave-wide 16-byte load of a nibble block is 1 KB contiguous and gives
// every lane exactly the B operand of four v_mfma_f32_16x16x32_bf16 (one per
// group). Rows past N and groups past K/32 are padded with code 8 and scale 0.
#include "common.h"
#include "launch.h"

namespace sve {

__device__ __forceinline__ int w4_code(const uint8_t* w, int K, int n, int k) {
  uint32_t byte = w[(size_t)n * (K / 2) + (k >> 1)];
  return (byte >> (4 * (k & 1))) & 0xF;
}

// grid: (n_tiles * quads), block 64: one thread per lane of a tile block.
__global__ __launch_bounds__(64) void w4_pack_kernel(const uint8_t* __restrict__ w,
                                                     const uint16_t* __restrict__ scales,
                                                     int N, int K, int Q,
                                                     uint8_t* __restrict__ out_nib,
                                                     uint8_t* __restrict__ out_scl) {
  const int blk = blockIdx.x;
  const int t = blk / Q, q = blk % Q;
  const int lane = threadIdx.x;
  const int n = 16 * t + (lane & 15);
  const int kb = lane >> 4;
  const int G = K / 32;
  u32x4 v;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int g = 4 * q + j;
    uint32_t dw = 0;
    for (int s = 0; s < 4; ++s) {
      int ce = 8, co = 8;
      if (n < N && g < G) {
        const int k = 32 * g + 8 * kb + 2 * s;
        ce = w4_code(w, K, n, k);
        co = w4_code(w, K, n, k + 1);
      }
      dw |= (uint32_t)ce << (4 * s);
      dw |= (uint32_t)co << (16 + 4 * s);
    }
    v[j] = dw;
  }
  store16(out_nib + (size_t)blk * 1024 + lane * 16, v);
  if (lane < 16) {
    uint16_t sc[4];
    for (int j = 0; j < 4; ++j) {
      const int g = 4 * q + j;
      sc[j] = (n < N && g < G) ? scales[(size_t)n * G + g] : (uint16_t)0;
    }
    u32x2 p;
    p[0] = (uint32_t)sc[0] | ((uint32_t)sc[1] << 16);
    p[1] = (uint32_t)sc[2] | ((uint32_t)sc[3] << 16);
    *reinterpret_cast<u32x2*>(out_scl + (size_t)blk * 128 + lane * 8) = p;
  }
}

// Decode the device format to fp32 [N][K]: (code - 8) * scale, exact in fp32.
__global__ __launch_bounds__(256) void w4_dequant_kernel(const uint8_t* __restrict__ nib,
                                                         const uint8_t* __restrict__ scl,
                                                         int N, int K, int Q,
                                                         float* __restrict__ out) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;  // one per 8 elements
  const int per_row = K / 8;
  if (idx >= (long long)N * per_row) return;
  const int n = (int)(idx / per_row);
  const int k0 = (int)(idx % per_row) * 8;
  const int t = n >> 4, q = k0 >> 7, j = (k0 >> 5) & 3, kb = (k0 >> 3) & 3;
  const int lane = 16 * kb + (n & 15);
  const size_t blk = (size_t)t * Q + q;
  const uint32_t dw = *reinterpret_cast<const uint32_t*>(nib + blk * 1024 + lane * 16 + j * 4);
  const uint16_t sbits = *reinterpret_cast<const uint16_t*>(scl + blk * 128 + (n & 15) * 8 + j * 2);
  const float s = f16_bits_to_f32(sbits);
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int shift = (e & 1) ? 16 + 4 * (e >> 1) : 4 * (e >> 1);
    r[e] = (float)((int)((dw >> shift) & 0xF) - 8) * s;
  }
  float* o = out + (size_t)n * K + k0;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = r[e];
}

// ---------------------------------------------------------------------------
// m-row GEMV core.
//
// The workgroup owns NT row tiles (16 output rows each) and all of K; its 4
// waves take contiguous quarters of the k quads. Per group the weights enter
// v_mfma_f32_16x16x32_bf16 as B = bf16(128 + code) (one v_and_or per element
// pair), the activations as A (row r of the MFMA tile = input row r, zero
// beyond the live rows), and the accumulator starts at C0 = -136 * sum(x) of
// the group (one extra MFMA per group against a constant -136 operand, shared
// by all row tiles), so D = sum x * (code - 8). D is then scaled by the
// group's fp16 scale into the fp32 accumulators. The 16-row MFMA is used as a
// multiply engine only: the kernel stays a single pass over the weight stream
// and costs the same for every m <= 16.
// ---------------------------------------------------------------------------

constexpr int kGemvWaves = 4;
constexpr int kGemvThreads = 64 * kGemvWaves;
// quads of weight loads issued together per wave: 8 KB of the weight stream
// in flight per wave whatever the number of row tiles
template <int NT>
struct GemvBatch {
  static constexpr int value = 8 / NT;
};

template <int NT>
struct GemvAcc {
  f32x4 v[NT];
};

// xrow: this lane's activation row (A row lane%16), or nullptr for a padded
// row. Weight tiles t0 .. t0+nt-1 (nt <= NT), quads [q0, q1).
template <int NT>
__device__ __forceinline__ void gemv_core(const uint16_t* __restrict__ xrow, int K,
                                          const uint8_t* __restrict__ nib,
                                          const uint8_t* __restrict__ scl, int Q, int t0, int nt,
                                          int q0, int q1, GemvAcc<NT>& acc) {
  constexpr int kGemvBatch = GemvBatch<NT>::value;
  const int lane = threadIdx.x & 63;
  const int kb = lane >> 4;
  u32x4 m136;
  m136[0] = m136[1] = m136[2] = m136[3] = 0xC308C308u;  // bf16(-136) x 8
  const bf16x8 neg136 = as_bf16x8(m136);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  auto load_x = [&](int q, u32x4 (&xa)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = 128 * q + 32 * j + 8 * kb;
      if (xrow != nullptr && k < K) {
        xa[j] = load16(xrow + k);
      } else {
        xa[j][0] = xa[j][1] = xa[j][2] = xa[j][3] = 0u;
      }
    }
  };

  u32x4 xnext[4];
  if (q0 < q1) load_x(q0, xnext);
  for (int qb = q0; qb < q1; qb += kGemvBatch) {
    const int nq = min(kGemvBatch, q1 - qb);
    u32x4 wv[kGemvBatch][NT];
    u32x2 sv[kGemvBatch][NT];
#pragma unroll
    for (int p = 0; p < kGemvBatch; ++p) {
      if (p < nq) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (t < nt) {
            const size_t blk = (size_t)(t0 + t) * Q + (qb + p);
            wv[p][t] = load16(nib + blk * 1024 + lane * 16);
            sv[p][t] = *reinterpret_cast<const u32x2*>(scl + blk * 128 + (lane & 15) * 8);
          }
        }
      }
    }
#pragma unroll
    for (int p = 0; p < kGemvBatch; ++p) {
      if (p < nq) {
        u32x4 xa[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) xa[j] = xnext[j];
        if (qb + p + 1 < q1) load_x(qb + p + 1, xnext);
        bf16x8 a[4];
        f32x4 c0[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a[j] = as_bf16x8(xa[j]);
          c0[j] = mfma16x16x32(a[j], neg136, zero4);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (t < nt) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint32_t dw = wv[p][t][j];
              u32x4 b;
              b[0] = (dw & 0x000F000Fu) | 0x43004300u;
              b[1] = ((dw >> 4) & 0x000F000Fu) | 0x43004300u;
              b[2] = ((dw >> 8) & 0x000F000Fu) | 0x43004300u;
              b[3] = ((dw >> 12) & 0x000F000Fu) | 0x43004300u;
              const f32x4 d = mfma16x16x32(a[j], as_bf16x8(b), c0[j]);
              const uint32_t sw = sv[p][t][j >> 1];
              const float s = f16_bits_to_f32((j & 1) ? (sw >> 16) : (sw & 0xFFFFu));
#pragma unroll
              for (int i = 0; i < 4; ++i) acc.v[t][i] = fmaf(s, d[i], acc.v[t][i]);
            }
          }
        }
      }
    }
  }
}

// Sum the four waves' accumulators in a fixed order and hand each output
// (tile t, MFMA row r, column c) to store(t, r, c, value).
template <int NT, class Store>
__device__ __forceinline__ void gemv_reduce(GemvAcc<NT>& acc, int nt, Store store) {
  __shared__ float red[kGemvWaves][NT][4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][t][i][lane] = acc.v[t][i];
  __syncthreads();
  // thread -> (i, lane) pair; each thread handles every tile
  const int i = threadIdx.x >> 6;  // 0..3
  const int l = threadIdx.x & 63;
  for (int t = 0; t < nt; ++t) {
    float s = red[0][t][i][l];
#pragma unroll
    for (int w = 1; w < kGemvWaves; ++w) s += red[w][t][i][l];
    store(t, 4 * (l >> 4) + i, l & 15, s);
  }
}

template <int NT>
__global__ __launch_bounds__(kGemvThreads) void w4_gemv_kernel(const uint16_t* __restrict__ x,
                                                               int m,
                                                               const uint8_t* __restrict__ nib,
                                                               const uint8_t* __restrict__ scl,
                                                               int N, int K, int Q, int n_tiles,
                                                               float* __restrict__ y) {
  const int t0 = blockIdx.x * NT;
  const int nt = min(NT, n_tiles - t0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const uint16_t* xrow = (r < m) ? x + (size_t)r * K : nullptr;
  const int per = (Q + kGemvWaves - 1) / kGemvWaves;
  const int q0 = min(Q, wave * per), q1 = min(Q, q0 + per);
  GemvAcc<NT> acc;
#pragma unroll
  for (int t = 0; t < NT; ++t) acc.v[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  gemv_core<NT>(xrow, K, nib, scl, Q, t0, nt, q0, q1, acc);
  gemv_reduce<NT>(acc, nt, [&](int t, int row, int col, float v) {
    const int n = 16 * (t0 + t) + col;
    if (row < m && n < N) y[(size_t)row * N + n] = v;
  });
}

// Expert-routed form. Block (pair slot ps, tile group): the expert of pair ps
// is handled by the first pair slot that names it, which gathers every pair
// routed to that expert (at most 16 per pass) into the rows of the MFMA tile,
// so each distinct expert's weights stream through the chip exactly once.
template <int NT>
__global__ __launch_bounds__(kGemvThreads) void w4_gemv_routed_kernel(
    const uint16_t* __restrict__ x, int x_per_slot, int m, const int32_t* __restrict__ ids,
    int topk, const uint8_t* __restrict__ packed_all, size_t expert_bytes, size_t scale_off,
    int E, int N, int K, int Q, int n_tiles, float* __restrict__ y) {
  const int ps = blockIdx.y;
  const int npairs = m * topk;
  const int e = ids[ps];
  for (int p = 0; p < ps; ++p)
    if (ids[p] == e) return;  // an earlier pair slot owns this expert
  const int t0 = blockIdx.x * NT;
  const int nt = min(NT, n_tiles - t0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int per = (Q + kGemvWaves - 1) / kGemvWaves;
  const int q0 = min(Q, wave * per), q1 = min(Q, q0 + per);
  const bool valid = (e >= 0 && e < E);
  const uint8_t* nib = packed_all + (valid ? (size_t)e * expert_bytes : 0);
  const uint8_t* scl = nib + scale_off;

  __shared__ int rows[16];
  int start = ps;  // pairs with this expert all sit at or after ps
  while (true) {
    // gather up to 16 pairs routed to e, starting at `start`
    __syncthreads();
    if (threadIdx.x == 0) {
      int c = 0, p = start;
      for (; p < npairs && c < 16; ++p)
        if (ids[p] == e) rows[c++] = p;
      for (int j = c; j < 16; ++j) rows[j] = -1;
    }
    __syncthreads();
    int next = npairs;
    {
      // first pair after the gathered ones (uniform)
      int last = -1;
      for (int j = 0; j < 16; ++j)
        if (rows[j] >= 0) last = rows[j];
      if (last >= 0)
        for (int p = last + 1; p < npairs; ++p)
          if (ids[p] == e) { next = p; break; }
    }
    if (!valid) {
      // out-of-range expert id: its outputs are NaN
      for (int j = 0; j < 16; ++j) {
        const int p = rows[j];
        if (p < 0) continue;
        for (int c = threadIdx.x; c < nt * 16; c += kGemvThreads) {
          const int n = 16 * t0 + c;
          if (n < N) y[(size_t)p * N + n] = __builtin_nanf("");
        }
      }
    } else {
      const int mr = lane & 15;
      const int pr = rows[mr];
      const uint16_t* xrow = nullptr;
      if (pr >= 0) {
        const int r = pr / topk;
        xrow = x_per_slot ? x + (size_t)pr * K : x + (size_t)r * K;
      }
      GemvAcc<NT> acc;
#pragma unroll
      for (int t = 0; t < NT; ++t) acc.v[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      gemv_core<NT>(xrow, K, nib, scl, Q, t0, nt, q0, q1, acc);
      gemv_reduce<NT>(acc, nt, [&](int t, int row, int col, float v) {
        const int p = rows[row];
        const int n = 16 * (t0 + t) + col;
        if (p >= 0 && n < N) y[(size_t)p * N + n] = v;
      });
    }
    if (next >= npairs) break;
    start = next;
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

size_t w4_packed_bytes(int N, int K) {
  const size_t nt = (size_t)(N + 15) / 16, q = (size_t)(K + 127) / 128;
  return nt * q * (1024 + 128);
}

hipError_t launch_w4_pack(const uint8_t* w, const uint16_t* s, int N, int K, void* packed,
                          hipStream_t st) {
  const int nt = (N + 15) / 16, Q = (K + 127) / 128;
  uint8_t* nib = (uint8_t*)packed;
  uint8_t* scl = nib + (size_t)nt * Q * 1024;
  hipLaunchKernelGGL(w4_pack_kernel, dim3(nt * Q), dim3(64), 0, st, w, s, N, K, Q, nib, scl);
  return hipGetLastError();
}

hipError_t launch_w4_dequant(const void* packed, int N, int K, float* out, hipStream_t st) {
  const int nt = (N + 15) / 16, Q = (K + 127) / 128;
  const uint8_t* nib = (const uint8_t*)packed;
  const uint8_t* scl = nib + (size_t)nt * Q * 1024;
  const long long total = (long long)N * (K / 8);
  const int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL(w4_dequant_kernel, dim3(blocks), dim3(256), 0, st, nib, scl, N, K, Q, out);
  return hipGetLastError();
}

// Row tiles per workgroup: enough workgroups to cover the 256 CUs at least
// twice before a workgroup takes more than one tile.
static int gemv_nt(int n_tiles, int groups) {
  const long long per_cu = 512;
  if ((long long)n_tiles * groups >= per_cu * 4) return 4;
  if ((long long)n_tiles * groups >= per_cu * 2) return 2;
  return 1;
}

hipError_t launch_w4_gemv(const void* x, int m, const void* packed, int N, int K, float* y,
                          hipStream_t st, int nt_override) {
  const int n_tiles = (N + 15) / 16, Q = (K + 127) / 128;
  const uint8_t* nib = (const uint8_t*)packed;
  const uint8_t* scl = nib + (size_t)n_tiles * Q * 1024;
  const int nt = nt_override > 0 ? nt_override : gemv_nt(n_tiles, 1);
  const dim3 block(kGemvThreads);
  const uint16_t* xp = (const uint16_t*)x;
  switch (nt) {
    case 4:
      hipLaunchKernelGGL(w4_gemv_kernel<4>, dim3((n_tiles + 3) / 4), block, 0, st, xp, m, nib, scl,
                         N, K, Q, n_tiles, y);
      break;
    case 2:
      hipLaunchKernelGGL(w4_gemv_kernel<2>, dim3((n_tiles + 1) / 2), block, 0, st, xp, m, nib, scl,
                         N, K, Q, n_tiles, y);
      break;
    default:
      hipLaunchKernelGGL(w4_gemv_kernel<1>, dim3(n_tiles), block, 0, st, xp, m, nib, scl, N, K, Q,
                         n_tiles, y);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_w4_gemv_routed(const void* x, int x_per_slot, int m, const int32_t* ids,
                                 int topk, const void* packed_all, int E, int N, int K, float* y,
                                 hipStream_t st) {
  const int n_tiles = (N + 15) / 16, Q = (K + 127) / 128;
  const size_t eb = w4_packed_bytes(N, K);
  const size_t scale_off = (size_t)n_tiles * Q * 1024;
  const dim3 grid(n_tiles, m * topk);
  hipLaunchKernelGGL(w4_gemv_routed_kernel<1>, grid, dim3(kGemvThreads), 0, st,
                     (const uint16_t*)x, x_per_slot, m, ids, topk, (const uint8_t*)packed_all, eb,
                     scale_off, E, N, K, Q, n_tiles, y);
  return hipGetLastError();
}

}  // namespace sve
