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
#include <algorithm>
#include <cstdlib>

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
// Workgroup = 8 waves. The k quads are cut into KS contiguous slices and the
// waves are laid out as (8/KS tile lanes) x (KS slices); a workgroup owns
// NT*(8/KS) row tiles of 16 output rows. Each wave streams its slice of its
// tiles through a ring of PD quads in flight (weights, scales and the
// activation operands together), so the loads of quad q+PD are issued as
// soon as quad q is consumed and the weight stream never drains.
//
// Per group the weights enter v_mfma_f32_16x16x32_bf16 as B = bf16(128 +
// code) (one v_and_or per element pair), the activations as A (row r of the
// MFMA tile = input row r, zero beyond the live rows), and the accumulator
// starts at C0 = -136 * sum(x) of the group (one extra MFMA per group against
// a constant -136 operand, shared by the NT tiles), so D = sum x * (code - 8).
// D is then scaled by the group's fp16 scale into fp32 accumulators. The
// 16-row MFMA is only the multiply engine: the kernel is a single pass over
// the weight stream and costs the same for every m <= 16. Partial sums of
// the KS slices are added in LDS in a fixed order.
// ---------------------------------------------------------------------------

constexpr int kGemvWaves = 8;
constexpr int kGemvThreads = 64 * kGemvWaves;
constexpr int kGemvPD = 4;  // quads in flight per wave

template <int NT>
struct GemvAcc {
  f32x4 v[NT];
};

template <int NT>
struct GemvSlot {
  u32x4 w[NT];
  u32x2 s[NT];
  u32x4 x[4];
};

// xrow: this lane's activation row (A row lane%16; padded rows pass a live
// row, whose MFMA output rows are never stored). Tiles t0 .. t0+nt-1
// (1 <= nt <= NT), quads [q0, q1). Every load is issued unconditionally from
// a valid address (tiles, quads and k clamped into range): a load under a
// divergent branch whose other side writes the same registers forces a full
// drain of the memory pipeline, which would serialise the stream. Groups past
// K carry zero scales, so whatever activations they meet contribute nothing.
template <int NT>
__device__ __forceinline__ void gemv_core(const uint16_t* __restrict__ xrow, bool xlive, int K,
                                          const uint8_t* __restrict__ nib,
                                          const uint8_t* __restrict__ scl, int Q, int t0, int nt,
                                          int q0, int q1, GemvAcc<NT>& acc) {
  const int lane = threadIdx.x & 63;
  const int kb = lane >> 4;
  u32x4 m136;
  m136[0] = m136[1] = m136[2] = m136[3] = 0xC308C308u;  // bf16(-136) x 8
  const bf16x8 neg136 = as_bf16x8(m136);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  if (q0 >= q1) return;

  auto issue = [&](int q, GemvSlot<NT>& sl) {
    q = min(q, q1 - 1);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const size_t blk = (size_t)(t0 + min(t, nt - 1)) * Q + q;
      sl.w[t] = load16(nib + blk * 1024 + lane * 16);
      sl.s[t] = *reinterpret_cast<const u32x2*>(scl + blk * 128 + (lane & 15) * 8);
    }
    if (xlive) {  // lanes of padded rows keep zeros (no write on the other side)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = min(128 * q + 32 * j + 8 * kb, K - 8);
        sl.x[j] = load16(xrow + k);
      }
    }
  };
  auto consume = [&](const GemvSlot<NT>& sl) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 a = as_bf16x8(sl.x[j]);
      const f32x4 c0 = mfma16x16x32(a, neg136, zero4);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t dw = sl.w[t][j];
        u32x4 b;
        b[0] = (dw & 0x000F000Fu) | 0x43004300u;
        b[1] = ((dw >> 4) & 0x000F000Fu) | 0x43004300u;
        b[2] = ((dw >> 8) & 0x000F000Fu) | 0x43004300u;
        b[3] = ((dw >> 12) & 0x000F000Fu) | 0x43004300u;
        const f32x4 d = mfma16x16x32(a, as_bf16x8(b), c0);
        const uint32_t sw = sl.s[t][j >> 1];
        const float sc = f16_bits_to_f32((j & 1) ? (sw >> 16) : (sw & 0xFFFFu));
#pragma unroll
        for (int i = 0; i < 4; ++i) acc.v[t][i] = fmaf(sc, d[i], acc.v[t][i]);
      }
    }
  };

  GemvSlot<NT> ring[kGemvPD];
#pragma unroll
  for (int p = 0; p < kGemvPD; ++p)
#pragma unroll
    for (int j = 0; j < 4; ++j) ring[p].x[j] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int p = 0; p < kGemvPD; ++p)
    if (q0 + p < q1) issue(q0 + p, ring[p]);  // wave-uniform
  for (int qb = q0; qb < q1; qb += kGemvPD) {
#pragma unroll
    for (int p = 0; p < kGemvPD; ++p) {
      const int q = qb + p;
      if (q < q1) {
        consume(ring[p]);
        if (q + kGemvPD < q1) issue(q + kGemvPD, ring[p]);  // wave-uniform
      }
    }
  }
}

// Sum the KS slices' accumulators in a fixed order and hand each output
// (tile, MFMA row r, column c) to store(tile, r, c, value). Tiles are
// numbered ts*NT + t for tile lane ts.
template <int NT, class Store>
__device__ __forceinline__ void gemv_reduce(GemvAcc<NT>& acc, int KS, int tiles, Store store) {
  __shared__ float red[kGemvWaves][NT][4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][t][i][lane] = acc.v[t][i];
  __syncthreads();
  const int TPW = kGemvWaves / KS;
  for (int idx = threadIdx.x; idx < TPW * NT * 256; idx += kGemvThreads) {
    const int l = idx & 63, i = (idx >> 6) & 3, tt = idx >> 8;
    const int ts = tt / NT, t = tt % NT;
    if (tt >= tiles) continue;
    float sum = red[ts * KS][t][i][l];
    for (int k = 1; k < KS; ++k) sum += red[ts * KS + k][t][i][l];
    store(tt, 4 * (l >> 4) + i, l & 15, sum);
  }
}

// Choose the k-slice count of the routed kernel: 8 slices when there are at
// least 8 quads, fewer (and more tile lanes per workgroup) for short K.
__host__ __device__ inline int gemv_ks(int Q) { return Q >= 8 ? 8 : Q >= 4 ? 4 : Q >= 2 ? 2 : 1; }

// ---------------------------------------------------------------------------
// Dense m-row GEMV.
//
// A workgroup of W waves (W <= 16) owns a contiguous run of 16-row output
// tiles; wave w owns a contiguous slice of the k quads and accumulates its
// slice's contribution to every tile of the run. The slices' partial sums
// are parked in LDS (one 1 KB slot per tile and wave, written without a
// barrier) and added in a fixed wave order once per batch of tiles, so the
// waves never wait for each other inside the weight stream and the result
// does not depend on the launch shape.
//
// Instruction budget per 32-element group and 16 output rows: one wave-wide
// 16-byte load per 4 groups, seven VALU ops to turn the group's nibble dword
// into the MFMA B operand (bf16 128 + code), one fp16->fp32 scale
// conversion, one v_mfma_f32_16x16x32_bf16 whose accumulator input is the
// precomputed C0 = -136 * sum(x) of the group (so D = sum x * (code - 8)),
// and four FMAs that apply the group scale. All addressing is wave-uniform
// (scalar registers) plus a fixed per-lane offset.
//
//  * short K (one slice of at most QPW quads per wave covers K): the wave's
//    activation operands and their C0 stay in registers for the whole run;
//    tile blocks are double buffered.
//  * long K: one tile per workgroup; each wave walks its slice two quads at
//    a time with weights, scales and activations double buffered, C0 being
//    computed per group.
// No load sits under a data-dependent branch: requests past the end of a
// run (or of a wave's slice) keep their instructions, reading either
// through a buffer resource of no bytes (zeros, no fetch) or, inside a
// slice, the last valid block; their results are discarded or add zero.
// ---------------------------------------------------------------------------

constexpr int kGemvMaxWaves = 16;
constexpr int kGemvPartSlots = 128;  // 1 KB LDS slots for parked partial sums

// B operand of one group: lane dword dw holds 8 codes (element e at bit
// 4*(e/2) for even e, 16 + 4*(e/2) for odd e); returns bf16 pairs 128+code.
// Each pair is a shift and one gfx950 three-input bit operation
// (v_bitop3_b32, truth table 0xEA = (src0 & src1) | src2).
__device__ __forceinline__ bf16x8 w4_bfrag(uint32_t dw) {
  constexpr uint32_t kMask = 0x000F000Fu, kExp = 0x43004300u;
  u32x4 b;
  b[0] = __builtin_amdgcn_bitop3_b32(dw, kMask, kExp, 0xEA);
  b[1] = __builtin_amdgcn_bitop3_b32(dw >> 4, kMask, kExp, 0xEA);
  b[2] = __builtin_amdgcn_bitop3_b32(dw >> 8, kMask, kExp, 0xEA);
  b[3] = __builtin_amdgcn_bitop3_b32(dw >> 12, kMask, kExp, 0xEA);
  return as_bf16x8(b);
}

__device__ __forceinline__ float scale_of(u32x2 sv, int j) {
  const uint32_t sw = sv[j >> 1];
  return f16_bits_to_f32((j & 1) ? (sw >> 16) : (sw & 0xFFFFu));
}

__device__ __forceinline__ bf16x8 neg136_operand() {
  u32x4 m136;
  m136[0] = m136[1] = m136[2] = m136[3] = 0xC308C308u;  // bf16(-136) x 8
  return as_bf16x8(m136);
}

// One group: acc += sc * (MFMA(a, B(dw)) + c0).
__device__ __forceinline__ void w4_group(bf16x8 a, f32x4 c0, uint32_t dw, float sc, f32x4& acc) {
  const f32x4 d = mfma16x16x32(a, w4_bfrag(dw), c0);
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = fmaf(sc, d[i], acc[i]);
}

// Park a wave's partial sums of one tile in LDS slot `slot`.
__device__ __forceinline__ void park(f32x4* part, int slot, const f32x4& acc) {
  part[slot * 64 + (threadIdx.x & 63)] = acc;
}

// Add the W parked partials of tiles [tile0, tile0 + nt) in wave order and
// store the live rows. Slot of (tile-in-batch tl, wave w) is tl * W + w.
__device__ __forceinline__ void flush_tiles(const f32x4* part, int W, int tile0, int nt, int m,
                                            int N, float* __restrict__ y, int ts = 1) {
  __syncthreads();
  const float* pf = reinterpret_cast<const float*>(part);
  for (int id = threadIdx.x; id < nt * 256; id += blockDim.x) {
    const int i = id & 3, l = (id >> 2) & 63, tl = id >> 8;
    const int row = 4 * (l >> 4) + i;
    const int n = 16 * (tile0 + tl * ts) + (l & 15);
    if (row >= m || n >= N) continue;
    float sum = 0.f;
    for (int w = 0; w < W; ++w) sum += pf[((tl * W + w) * 64 + l) * 4 + i];
    y[(size_t)row * N + n] = sum;
  }
  __syncthreads();
}

template <int QPW>
struct TileBuf {
  u32x4 w[QPW];
  u32x2 s[QPW];
};

// waves per workgroup the short kernel allows for QPW quads per wave (its
// register budget: activations and C0 of 4*QPW groups plus two tile buffers)
__host__ __device__ constexpr int short_max_waves(int qpw) { return qpw <= 2 ? 16 : 8; }

// HOIST: C0 of every group of the wave's slice is computed once and kept in
// registers (one MFMA per group in the stream); otherwise it is recomputed
// per group (two MFMAs per group, fewer registers).
template <int QPW, bool SINGLE, bool HOIST, int PD>
__global__ __launch_bounds__(64 * short_max_waves(QPW)) void w4_gemv_short_kernel(
    const uint16_t* __restrict__ x, int m, const uint8_t* __restrict__ nib,
    const uint8_t* __restrict__ scl, int N, int K, int Q, int n_tiles, int strided,
    float* __restrict__ y) {
  constexpr int SLOTS = SINGLE ? kGemvMaxWaves : kGemvPartSlots;
  __shared__ f32x4 part[SLOTS * 64];
  const int W = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kb = lane >> 4, r = lane & 15;
  const int G = K >> 5;
  // the workgroup's tiles are t0 + i*ts, i in [0, cnt): a contiguous run
  // (ts = 1), or every gridDim.x-th tile, so that the workgroups read
  // neighbouring tiles at any moment
  const int t0 = strided ? (int)blockIdx.x : (int)((long long)blockIdx.x * n_tiles / gridDim.x);
  const int ts = strided ? (int)gridDim.x : 1;
  const int cnt = strided ? (n_tiles - t0 + ts - 1) / ts
                          : (int)((long long)(blockIdx.x + 1) * n_tiles / gridDim.x) - t0;
  const int q0 = wave * QPW;
  const int nq = max(0, min(QPW, Q - q0));  // real quads of this wave (uniform)
  const int batch = SLOTS / W;              // tiles per LDS batch
  const bf16x8 neg136 = neg136_operand();
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  // activation operands (A row = input row r) and their C0 terms, once for
  // the whole run. Rows past m are never stored: their lanes read past the
  // end of a buffer resource over x, which returns zeros without fetching,
  // so only the m live rows cost address and cache bandwidth.
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x), (short)0, m * K * 2, kBufWord3);  // (m <= 16, K < 2^26)
  const uint32_t xoff = r < m ? (uint32_t)(r * K + 8 * kb) * 2u : 0x80000000u;
  bf16x8 xa[QPW][4];
  f32x4 c0[HOIST ? QPW : 1][4];
#pragma unroll
  for (int a = 0; a < QPW; ++a)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int g = min(4 * (q0 + a) + j, G - 1);
      xa[a][j] = as_bf16x8(__builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff + 64u * g, 0, 0)));
    }
  // quads past K (the last wave of an uneven split re-reads a real block
  // there) meet zero activations, so they add exactly zero
#pragma unroll
  for (int a = 0; a < QPW; ++a)
    if (a >= nq)
#pragma unroll
      for (int j = 0; j < 4; ++j) xa[a][j] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  // C0 terms: computed once the activations arrive, after the first weight
  // loads are in flight (the in-order load counter then waits for the
  // activations only)
  auto hoist_c0 = [&]() {
    if constexpr (HOIST) {
#pragma unroll
      for (int a = 0; a < QPW; ++a)
#pragma unroll
        for (int j = 0; j < 4; ++j) c0[a][j] = mfma16x16x32(xa[a][j], neg136, zero4);
    }
  };

  const uint32_t loff = lane * 16, soff = r * 8;
  // Requests through buffer resources over one tile's blocks. A request
  // past the run gets a resource of no bytes: every lane reads past its end
  // (zeros, no fetch), while the instructions and their count stay the
  // same (its sums are parked in slots the flush does not read). Re-reading
  // the run's last tile instead cost each workgroup two tiles of load
  // bandwidth at the end of a run of two.
  auto issue = [&](int i, TileBuf<QPW>& b) {
    const int t = t0 + min(i, cnt - 1) * ts;
    const bool live = i < cnt;  // (uniform)
    const __amdgpu_buffer_rsrc_t nrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(nib + (size_t)t * Q * 1024), (short)0, live ? Q * 1024 : 0, kBufWord3);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(scl + (size_t)t * Q * 128), (short)0, live ? Q * 128 : 0, kBufWord3);
#pragma unroll
    for (int a = 0; a < QPW; ++a) {
      const uint32_t q = min(q0 + a, Q - 1);
      b.w[a] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(nrs, q * 1024 + loff, 0, 0));
      if constexpr (QPW != 2)
        b.s[a] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(srs, q * 128 + soff, 0, 0));
    }
    if constexpr (QPW == 2) {
      // one scale load for both quads: lanes kb < 2 fetch quad 0's row,
      // lanes kb >= 2 quad 1's (spread to every lane when consumed)
      const uint32_t q = min(q0 + (kb >> 1), Q - 1);
      b.s[0] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(srs, q * 128 + soff, 0, 0));
    }
  };
  auto consume = [&](TileBuf<QPW> b) {
    if constexpr (QPW == 2) {
      const u32x2 own = b.s[0];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        b.s[0][e] = __shfl(own[e], r, 64);       // a lane with kb = 0
        b.s[1][e] = __shfl(own[e], r + 32, 64);  // a lane with kb = 2
      }
    }
    f32x4 acc = zero4;
#pragma unroll
    for (int a = 0; a < QPW; ++a)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float sc = scale_of(b.s[a], j);
        const f32x4 c = HOIST ? c0[HOIST ? a : 0][j] : mfma16x16x32(xa[a][j], neg136, zero4);
        w4_group(xa[a][j], c, b.w[a][j], sc, acc);
      }
    return acc;
  };

  if constexpr (SINGLE) {
    TileBuf<QPW> A;
    issue(0, A);
    hoist_c0();
    park(part, wave, consume(A));
    flush_tiles(part, W, t0, 1, m, N, y);
    return;
  }
  // walk over the run with PD tiles in flight; the fences keep each
  // buffer's loads contiguous in issue order so the wait before a consume
  // covers only it. Requests past the run fetch nothing (see issue), and
  // their sums are parked in slots the flush does not read (a flush comes before
  // a batch could hold more than `batch` tiles; a conditional park here
  // split the schedule and spilled).
  TileBuf<QPW> buf[PD];
#pragma unroll
  for (int u = 0; u < PD; ++u) {
    issue(u, buf[u]);
    __builtin_amdgcn_sched_barrier(0);
  }
  hoist_c0();
  int ib = 0;  // first tile (index into the workgroup's tiles) of the current LDS batch
  for (int i = 0; i < cnt; i += PD) {
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      const f32x4 acc = consume(buf[u]);
      __builtin_amdgcn_sched_barrier(0);
      issue(i + PD + u, buf[u]);
      __builtin_amdgcn_sched_barrier(0);
      park(part, (i + u - ib) * W + wave, acc);  // past the run: never flushed
    }
    const int done = min(i + PD, cnt) - ib;
    if (done + PD > batch || i + PD >= cnt) {  // batch full (or run ends): add and store
      flush_tiles(part, W, t0 + ib * ts, done, m, N, y, ts);
      ib += done;
    }
  }
}

constexpr int kLongChunk = 2;  // quads per pipeline step

constexpr int kLongStepK = 128 * kLongChunk;  // k per pipeline step

// Weights and scales of one step, plus the step's activations in compact
// form: m rows x kLongStepK elements, 16 bytes per lane and load (at most 8
// loads for m <= 16), instead of the MFMA operand layout (eight loads per
// step whatever m is).
struct LongBuf {
  u32x4 w[kLongChunk];
  u32x2 s[kLongChunk];
  u32x4 xc[8];
};

constexpr int kLongMaxWaves = 8;
constexpr int kLongDepth = 2;  // steps in flight per wave (3: 9.0 us, 4: 11.1 us against 8.8 at m = 1)

// NU = (m + 1) / 2 compact activation loads per step, a template argument:
// with a count known only at run time the compiler could not count the
// step's requests, and before each step's products it waited for the
// oldest requests of the next step as well (one step in flight, not two).
// (x, nib and scl are not declared __restrict__: with it the compiler may
// move their loads across the fences below.)
template <int NU>
__global__ __launch_bounds__(64 * kLongMaxWaves) void w4_gemv_long_kernel(
    const uint16_t* x, int m, const uint8_t* nib, const uint8_t* scl, int N, int K, int Q,
    int n_tiles, float* __restrict__ y) {
  __shared__ f32x4 part[kGemvMaxWaves * 64];
  // per wave: one step's activations, [row][kLongStepK] bf16 with rows
  // kXRow elements apart, rewritten every step (LDS operations of a wave
  // complete in order). The 16 extra bytes per row put the rows on
  // different banks: with 512-byte rows every row of an operand read hit
  // the same banks (8-way conflicts at m = 8).
  constexpr int kXRow = kLongStepK + 8;
  __shared__ __attribute__((aligned(16))) uint16_t xs[kLongMaxWaves][16 * kXRow];
  const int W = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kb = lane >> 4, r = lane & 15;
  const int tile = blockIdx.x;
  const int per = (Q + W - 1) / W;
  const int q0 = wave * per;
  const int nq = max(0, min(per, Q - q0));
  const int nchunks = (per + kLongChunk - 1) / kLongChunk;  // same for every wave
  // (m <= 16, K < 2^26: the activation byte offsets fit 32 bits)
  const bf16x8 neg136 = neg136_operand();
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const uint32_t loff = lane * 16, soff = r * 8;
  const size_t tbase = (size_t)tile * Q;
  const int xr = min(r, m - 1);  // operand row (rows past m repeat row m-1; never stored)
  uint16_t* xw = xs[wave];

  auto quad_of = [&](int c, int a) { return min(q0 + min(c * kLongChunk + a, max(nq - 1, 0)), Q - 1); };
  static_assert(kLongChunk == 2, "one scale load serves the two quads of a step");
  // A step past the wave's last one (the pipeline's tail) requests through
  // resources of no bytes: zeros, no fetch, the same instructions.
  auto issue = [&](int c, LongBuf& b) {
    const bool live = c < nchunks;  // (uniform)
    const __amdgpu_buffer_rsrc_t nrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(nib + tbase * 1024), (short)0, live ? Q * 1024 : 0, kBufWord3);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(scl + tbase * 128), (short)0, live ? Q * 128 : 0, kBufWord3);
    const __amdgpu_buffer_rsrc_t xcs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(x), (short)0, live ? m * K * 2 : 0, kBufWord3);
#pragma unroll
    for (int a = 0; a < kLongChunk; ++a)
      b.w[a] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             nrs, (uint32_t)quad_of(c, a) * 1024 + loff, 0, 0));
    // lanes kb < 2 fetch quad 0's scale row, lanes kb >= 2 quad 1's
    b.s[0] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                           srs, (uint32_t)quad_of(c, kb >> 1) * 128 + soff, 0, 0));
    // compact activations: lane slot e = lane + 64u holds row e / 32,
    // elements 8 * (e % 32) .. +7 of the step (quad (e % 32) / 16); a row
    // past m (the second row of the last load when m is odd) reads past the
    // buffer's end: zeros, no fetch, and the request count stays NU
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int e = lane + 64 * u, rr = e >> 5, kc = e & 31;
      const int k = min(128 * quad_of(c, kc >> 4) + 8 * (kc & 15), K - 8);
      b.xc[u] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     xcs, rr < m ? (uint32_t)(rr * K + k) * 2u : 0x80000000u, 0, 0));
    }
  };
  f32x4 acc = zero4;
  auto consume = [&](int c, LongBuf b) {
    const u32x2 own = b.s[0];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      b.s[0][e] = __shfl(own[e], r, 64);       // a lane with kb = 0
      b.s[1][e] = __shfl(own[e], r + 32, 64);  // a lane with kb = 2
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int e = lane + 64 * u;  // row e / 32, elements 8 * (e % 32) .. +7
      store16(xw + (e >> 5) * kXRow + 8 * (e & 31), b.xc[u]);
    }
#pragma unroll
    for (int a = 0; a < kLongChunk; ++a) {
      const bool real = c * kLongChunk + a < nq;  // uniform
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 xa =
            as_bf16x8(load16(xw + xr * kXRow + 128 * a + 32 * j + 8 * kb));
        const f32x4 c0 = mfma16x16x32(xa, neg136, zero4);
        const float sc = real ? scale_of(b.s[a], j) : 0.f;
        w4_group(xa, c0, b.w[a][j], sc, acc);
      }
    }
  };
  // kLongDepth steps in flight. The first round is peeled, so the loop is
  // entered with the request history of its own back edge (the prologue's
  // requests came out interleaved, and at a merged loop head the compiler
  // then waited for the next step's requests too). Steps past nchunks
  // request nothing (empty resources) and add zero.
  // (The fences also stop loads from being moved at the IR level, where a
  // scheduling barrier does not hold: an activation load sunk below the
  // next step's requests changed the order the waits count on.)
  auto fence = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  LongBuf buf[kLongDepth];
#pragma unroll
  for (int d = 0; d < kLongDepth; ++d) {
    issue(d, buf[d]);
    fence();
  }
  auto round = [&](int c) {
#pragma unroll
    for (int d = 0; d < kLongDepth; ++d) {
      consume(c + d, buf[d]);
      fence();
      issue(c + d + kLongDepth, buf[d]);
      fence();
    }
  };
  round(0);
  for (int c = kLongDepth; c < nchunks; c += kLongDepth) round(c);
  park(part, wave, acc);
  flush_tiles(part, W, tile, 1, m, N, y);
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
  const int KS = gemv_ks(Q), TPW = kGemvWaves / KS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ts = wave / KS, ks = wave % KS;
  const int wg_t0 = blockIdx.x * TPW * NT;
  const int wg_tiles = min(TPW * NT, n_tiles - wg_t0);
  const int t0 = wg_t0 + ts * NT;
  const int nt = max(0, min(NT, n_tiles - t0));
  const int per = (Q + KS - 1) / KS;
  const int q0 = min(Q, ks * per), q1 = min(Q, q0 + per);
  const bool valid = (e >= 0 && e < E);
  const uint8_t* nib = packed_all + (valid ? (size_t)e * expert_bytes : 0);
  const uint8_t* scl = nib + scale_off;

  __shared__ int rows[16];
  int start = ps;  // pairs with this expert all sit at or after ps
  while (true) {
    __syncthreads();
    if (threadIdx.x == 0) {
      int c = 0;
      for (int p = start; p < npairs && c < 16; ++p)
        if (ids[p] == e) rows[c++] = p;
      for (int j = c; j < 16; ++j) rows[j] = -1;
    }
    __syncthreads();
    int next = npairs;
    {
      int last = -1;
      for (int j = 0; j < 16; ++j)
        if (rows[j] >= 0) last = rows[j];
      if (last >= 0)
        for (int p = last + 1; p < npairs; ++p)
          if (ids[p] == e) {
            next = p;
            break;
          }
    }
    if (!valid) {
      // out-of-range expert id: its outputs are NaN
      for (int j = 0; j < 16; ++j) {
        const int p = rows[j];
        if (p < 0) continue;
        for (int c = threadIdx.x; c < wg_tiles * 16; c += kGemvThreads) {
          const int n = 16 * wg_t0 + c;
          if (n < N) y[(size_t)p * N + n] = __builtin_nanf("");
        }
      }
    } else {
      const int pr = max(rows[lane & 15], rows[0]);
      const bool xlive = rows[lane & 15] >= 0;
      const uint16_t* xrow = x_per_slot ? x + (size_t)pr * K : x + (size_t)(pr / topk) * K;
      GemvAcc<NT> acc;
#pragma unroll
      for (int t = 0; t < NT; ++t) acc.v[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (nt > 0) gemv_core<NT>(xrow, xlive, K, nib, scl, Q, t0, nt, q0, q1, acc);
      gemv_reduce<NT>(acc, KS, wg_tiles, [&](int tt, int row, int col, float v) {
        const int p = rows[row];
        const int n = 16 * (wg_t0 + tt) + col;
        if (p >= 0 && n < N) y[(size_t)p * N + n] = v;
      });
    }
    if (next >= npairs) break;
    start = next;
  }
}

// Expert-routed form on the dense short kernel's pipeline (K of at most 32
// quads). Workgroup (run of row tiles, pair slot ps): the expert of pair ps
// is handled by the first pair slot that names it; that workgroup gathers
// every pair routed to the expert (16 per pass) as the rows of the MFMA
// tile, keeps their activations (and C0) in registers, one k slice per
// wave, and walks its run of the expert's row tiles double buffered. Each
// distinct expert's weights therefore stream through the chip once, spread
// over many workgroups.
constexpr int kRoutedRun = 2;        // fewest row tiles per workgroup
constexpr int kRoutedMaxPairs = 256;  // m * topk (16 x 16)

template <int QPW>
__global__ __launch_bounds__(64 * short_max_waves(QPW)) void w4_gemv_routed_short_kernel(
    const uint16_t* __restrict__ x, int x_per_slot, int m, const int32_t* __restrict__ ids,
    int topk, const uint8_t* __restrict__ packed_all, size_t expert_bytes, size_t scale_off,
    int E, int N, int K, int Q, int n_tiles, int run, int batch, float* __restrict__ y) {
  // parked partial sums: `batch` tiles of W 1 KB slots (dynamic LDS, sized
  // by the launcher so that short-K shapes keep several workgroups per CU)
  extern __shared__ f32x4 part[];
  __shared__ int sid[kRoutedMaxPairs];  // the routing table, read once
  __shared__ int rows[16];
  __shared__ int s_next;
  const int ps = blockIdx.y;
  const int npairs = m * topk;
  const int W = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kb = lane >> 4, r = lane & 15;
  const int G = K >> 5;
  const int t0 = blockIdx.x * run, t1 = min(n_tiles, t0 + run);
  if (t0 >= t1) return;
  // Every wave reads the routing table into registers (pair lane + 64c)
  // and decides by itself, with no barrier, whether an earlier pair slot
  // names the same expert (then that slot owns it); every wave reaches the
  // same answer. The owner's first weight requests go out right after, so
  // the weight stream does not wait for the pair gathering below.
  const int e = ids[ps];
  int tid[kRoutedMaxPairs / 64];
  bool earlier = false;
#pragma unroll
  for (int c = 0; c < kRoutedMaxPairs / 64; ++c) {
    const int p = lane + 64 * c;
    tid[c] = p < npairs ? ids[p] : -1;
    earlier |= p < ps && tid[c] == e;
  }
  if (__ballot(earlier) != 0ull) return;  // (uniform)
  const int nt = t1 - t0;
  const bool valid = (e >= 0 && e < E);
  const uint8_t* nib = packed_all + (valid ? (size_t)e * expert_bytes : 0);
  const uint8_t* scl = nib + scale_off;
  const int q0 = wave * QPW;
  const int nq = max(0, min(QPW, Q - q0));
  const bf16x8 neg136 = neg136_operand();
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const uint32_t loff = lane * 16, soff = r * 8;
  // (a tile past the run requests through resources of no bytes: zeros,
  // no fetch, the same instructions)
  auto issue = [&](int t, TileBuf<QPW>& b) {
    const bool live = t < t1;  // (uniform)
    t = min(t, t1 - 1);
    const __amdgpu_buffer_rsrc_t nrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(nib + (size_t)t * Q * 1024), (short)0, live ? Q * 1024 : 0, kBufWord3);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(scl + (size_t)t * Q * 128), (short)0, live ? Q * 128 : 0, kBufWord3);
#pragma unroll
    for (int a = 0; a < QPW; ++a) {
      const uint32_t q = min(q0 + a, Q - 1);
      b.w[a] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(nrs, q * 1024 + loff, 0, 0));
      b.s[a] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(srs, q * 128 + soff, 0, 0));
    }
  };
  // the first pass's first two tiles (an invalid expert id reads expert 0's,
  // unused: its outputs are NaN)
  TileBuf<QPW> A, B;
  issue(t0, A);
  __builtin_amdgcn_sched_barrier(0);
  issue(t0 + 1, B);
  __builtin_amdgcn_sched_barrier(0);
  if (wave == 0)
#pragma unroll
    for (int c = 0; c < kRoutedMaxPairs / 64; ++c)
      if (lane + 64 * c < npairs) sid[lane + 64 * c] = tid[c];

  int start = ps;  // pairs with this expert all sit at or after ps
  while (true) {
    __syncthreads();
    if (wave == 0) {
      // the first 16 pairs at or after `start` routed to e, in pair order
      // (ballot compaction), and the one after them
      int c = 0, nxt = npairs;
      for (int c0 = 0; c0 < npairs; c0 += 64) {
        const int p = c0 + lane;
        const bool hit = p >= start && p < npairs && sid[p] == e;
        const unsigned long long mask = __ballot(hit);
        const int pos = c + __popcll(mask & ((1ull << lane) - 1));
        if (hit && pos < 16) rows[pos] = p;
        if (hit && pos == 16) nxt = p;
        c += __popcll(mask);
      }
      if (lane >= c && lane < 16) rows[lane] = -1;
      nxt = __reduce_min_sync(~0ull, nxt);
      if (lane == 0) s_next = nxt;
    }
    __syncthreads();
    const int cnt = min(16, __popcll(__ballot(lane < 16 && rows[lane] >= 0)));
    const int next = s_next;
    if (!valid) {
      // out-of-range expert id: its outputs are NaN
      for (int c = threadIdx.x; c < cnt * nt * 16; c += blockDim.x) {
        const int j = c / (nt * 16), n = 16 * t0 + c % (nt * 16);
        if (n < N) y[(size_t)rows[j] * N + n] = __builtin_nanf("");
      }
    } else {
      // activations of the gathered pairs; rows past cnt are never stored
      // and read past the end of a buffer resource over x (zeros, no
      // fetch); quads past K meet zero activations
      const int pr = rows[min(r, cnt - 1)];
      const size_t xrows = x_per_slot ? (size_t)npairs : (size_t)m;
      const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(x), (short)0, (int)(xrows * K * 2), kBufWord3);
      const uint32_t xoff =
          r < cnt ? (uint32_t)(((x_per_slot ? (size_t)pr : (size_t)(pr / topk)) * K + 8 * kb) * 2)
                  : 0x80000000u;
      // (unconditional loads, quads past K reading past the buffer's end:
      // a load under a condition made the compiler lose count of the
      // requests and wait for all of them in the tile loop)
      bf16x8 xa[QPW][4];
#pragma unroll
      for (int a = 0; a < QPW; ++a)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xa[a][j] = as_bf16x8(__builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                         xrs, a < nq ? xoff + 64u * min(4 * (q0 + a) + j, G - 1) : 0x80000000u,
                         0, 0)));
      auto consume = [&](const TileBuf<QPW>& b) {
        f32x4 acc = zero4;
#pragma unroll
        for (int a = 0; a < QPW; ++a)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            w4_group(xa[a][j], mfma16x16x32(xa[a][j], neg136, zero4), b.w[a][j], scale_of(b.s[a], j),
                     acc);
        return acc;
      };
      // add the waves' parked partial sums of tiles [tile0, tile0 + k) in
      // wave order and store the gathered rows
      auto flush = [&](int tile0, int k) {
        __syncthreads();
        const float* pf = reinterpret_cast<const float*>(part);
        for (int id = threadIdx.x; id < k * 256; id += blockDim.x) {
          const int i = id & 3, l = (id >> 2) & 63, tl = id >> 8;
          const int row = 4 * (l >> 4) + i;
          const int n = 16 * (tile0 + tl) + (l & 15);
          if (row >= cnt || n >= N) continue;
          float sum = 0.f;
          for (int w = 0; w < W; ++w) sum += pf[((tl * W + w) * 64 + l) * 4 + i];
          y[(size_t)rows[row] * N + n] = sum;
        }
        __syncthreads();
      };
      // double-buffered walk over the run (as in the dense short kernel);
      // tiles t0 and t0+1 are already requested. Everything requested so
      // far is awaited here (the activations were requested after both
      // tiles, so the first products need all of it anyway): the loop head
      // otherwise merges two different counts of loads in flight and the
      // compiler then waits for all of them in every step.
      wait_vmem<0>();
      int tb = t0;
      for (int t = t0; t < t1; t += 2) {
        const f32x4 acc0 = consume(A);
        __builtin_amdgcn_sched_barrier(0);
        issue(t + 2, A);
        __builtin_amdgcn_sched_barrier(0);
        park(part, (t - tb) * W + wave, acc0);
        const f32x4 acc1 = consume(B);
        __builtin_amdgcn_sched_barrier(0);
        issue(t + 3, B);
        __builtin_amdgcn_sched_barrier(0);
        // parked even past the run's end (an odd run): the slot is inside
        // the batch (t - tb + 2 <= batch, batch even) and never summed, and
        // a store under a condition let the compiler finish acc1 after the
        // next requests, which then waited for them
        park(part, (t + 1 - tb) * W + wave, acc1);
        const int done = min(t + 2, t1) - tb;
        if (done + 2 > batch || t + 2 >= t1) {
          flush(tb, done);
          tb += done;
        }
      }
      (void)nt;
    }
    if (next >= npairs) break;
    start = next;
    // the next pass walks the run again from its first tiles
    issue(t0, A);
    __builtin_amdgcn_sched_barrier(0);
    issue(t0 + 1, B);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// int4 GEMM for many rows (a prefill's m >= 16): y = x W^T on fp16 matrix
// cores. Unlike the GEMV, whose group scale costs one fp32 multiply-add per
// output and group (as many vector operations as the products themselves
// at this size), the GEMM dequantises each weight once per workgroup to
// fp16: w = (code - 8) * scale rounded once (relative error at most 2^-11),
// and x is converted to fp16 once by a first pass (exact for |x| < 65504).
// The products then accumulate in fp32 with no vector work per product.
// Workgroup = four waves over one 64-column tile and 256 rows; wave = 64
// rows x 64 columns (4 x 4 tiles of 16 x 16).
//   weights: nibble and scale blocks reach a ring of four LDS slots by
//     direct buffer-to-LDS loads, three quads ahead, each wave loading one
//     16-row tile (each slot its own LDS variable and the quad loop
//     unrolled by four, so a read waits only for its slot's loads). While
//     the products of quad q run, each wave dequantises its tile of quad
//     q+1 into the fp16 operand buffer of that quad's parity, which all four
//     waves read after the next barrier (one barrier per quad).
//   activations: the wave's own rows, packed by the first pass in operand
//     order (each A operand a contiguous 1 KB block), straight into
//     registers two groups ahead.
// The k range may be split over several workgroups (grid z); each split then
// writes its partial y to the workspace, and a second kernel adds the splits
// in split order.
// ---------------------------------------------------------------------------
constexpr int kGemmWaveRows = 64;
constexpr int kGemmCols = 64;
constexpr int kGemmGroupRows = 4 * kGemmWaveRows;
constexpr int kGemmMaxSplits = 16;
constexpr int kGemmWAhead = 3;  // weight quads requested ahead (ring of 4)
constexpr int kGemmXAhead = 2;  // activation groups requested ahead

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma16x16x32_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

struct GemmWSlot {
  uint8_t nib[4][1024];  // [tile][64 lanes x 16 bytes]
  uint8_t scl[4][128];   // [tile][16 rows x 8 bytes]
};

// fp16 B operand of one group from a lane's nibble dword: (code - 8) * s
__device__ __forceinline__ u32x4 w4_f16frag(uint32_t dw, f16x2 s2) {
  constexpr uint32_t kMask = 0x000F000Fu, kExp = 0x64006400u;  // fp16 1024 + code
  const f16x2 off = {(_Float16)-1032.f, (_Float16)-1032.f};
  u32x4 b;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t v = __builtin_amdgcn_bitop3_b32(dw >> (4 * p), kMask, kExp, 0xEA);
    f16x2 h = __builtin_bit_cast(f16x2, v) + off;  // code - 8, exact
    h = h * s2;                                      // one rounding
    b[p] = __builtin_bit_cast(uint32_t, h);
  }
  return b;
}

// x (bf16 [m][K]) to fp16 in MFMA operand order: block (row tile rt of 16
// rows, group g) is 1 KB at (rt * G + g) * 1024 bytes, lane (r, kb) of it
// holding row 16 rt + r, elements 32 g + 8 kb .. +7 (the A operand of one
// product); rows from m up to a multiple of 64 are zero. One 16-byte piece
// per thread.
__global__ __launch_bounds__(256) void w4_x_pack_kernel(const uint16_t* __restrict__ x, int m,
                                                        int K, long long pieces,
                                                        uint16_t* __restrict__ xp) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= pieces) return;
  const int G = K >> 5;
  const int lane = (int)(i & 63);
  const long long blk = i >> 6;
  const int g = (int)(blk % G), rt = (int)(blk / G);
  const int row = 16 * rt + (lane & 15);
  u32x4 h = {0u, 0u, 0u, 0u};
  if (row < m) {
    const u32x4 v = load16(x + (size_t)row * K + 32 * g + 8 * (lane >> 4));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f16x2 p;
      p[0] = (_Float16)__uint_as_float(v[e] << 16);
      p[1] = (_Float16)__uint_as_float(v[e] & 0xFFFF0000u);
      h[e] = __builtin_bit_cast(uint32_t, p);
    }
  }
  store16(xp + 8 * i, h);
}

__global__ __launch_bounds__(256, 2) void w4_gemm_kernel(const uint16_t* __restrict__ xh, int m,
                                                         const uint8_t* __restrict__ nib,
                                                         const uint8_t* __restrict__ scl, int N,
                                                         int K, int Q, int qps,
                                                         float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) GemmWSlot ws0, ws1, ws2, ws3;
  // fp16 B operands of a quad: [tile][group][64 lanes x 16 bytes], by parity
  __shared__ __attribute__((aligned(16))) uint8_t bq0[4][4][1024], bq1[4][4][1024];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kb = lane >> 4, r = lane & 15;
  const int m0 = blockIdx.y * kGemmGroupRows + wave * kGemmWaveRows;
  const bool live = m0 < m;  // (uniform) rows of this wave exist; it loads either way
  const int n_tiles = (N + 15) / 16, G = K >> 5;
  const int q0 = blockIdx.z * qps, q1 = min(Q, q0 + qps);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  // this wave's weight tile, the weight buffer resources
  const int tw = min(4 * (int)blockIdx.x + wave, n_tiles - 1);
  const __amdgpu_buffer_rsrc_t nrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(nib), (short)0, n_tiles * Q * 1024, kBufWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(scl), (short)0, n_tiles * Q * 128, kBufWord3);
  // quad q's blocks of tile tw into a slot (two requests; past the split a
  // real block, unused)
  auto issue_w = [&](GemmWSlot& sl, int q) {
    q = min(q, Q - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(nrs, (lds_void*)&sl.nib[wave][0], 16, lane * 16,
                                             (tw * Q + q) * 1024, 0, 0);
    if (lane < 8)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (lds_void*)&sl.scl[wave][0], 16, lane * 16,
                                               (tw * Q + q) * 128, 0, 0);
  };
  auto slot = [&](int u) -> GemmWSlot& { return u == 0 ? ws0 : u == 1 ? ws1 : u == 2 ? ws2 : ws3; };

  // A operands of group g for the wave's four 16-row tiles: four 1 KB
  // blocks of the packed x (rows past m are zero; groups past K read a real
  // group, whose weights are code 8 with scale 0) - four requests
  // (a wave with no rows loads the first wave's blocks, unused: its loads
  // keep the request counts the same)
  const uint8_t* xw = reinterpret_cast<const uint8_t*>(xh) +
                      (size_t)((live ? m0 : 0) / 16) * G * 1024 + lane * 16;
  auto load_x = [&](int g, f16x8* xa) {
    g = min(g, G - 1);
#pragma unroll
    for (int a = 0; a < 4; ++a)
      xa[a] = __builtin_bit_cast(f16x8, load16(xw + ((size_t)a * G + g) * 1024));
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[a][t] = zero4;

  // dequantise this wave's tile of the quad in slot sl into operand buffer bq
  auto dequant = [&](GemmWSlot& sl, uint8_t (*bq)[4][1024]) {
    const u32x4 wd = *reinterpret_cast<const u32x4*>(&sl.nib[wave][lane * 16]);
    const u32x2 sv = *reinterpret_cast<const u32x2*>(&sl.scl[wave][r * 8]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t sw = sv[j >> 1] >> (16 * (j & 1));
      const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)(sw & 0xFFFFu));
      const f16x2 s2 = {s, s};
      *reinterpret_cast<u32x4*>(&bq[wave][j][lane * 16]) = w4_f16frag(wd[j], s2);
    }
  };

  // prologue: weight quads q0 .. q0+2 into slots 0..2 and groups 4q0, 4q0+1
  // requested; quad q0 dequantised into operand buffer 0
  issue_w(ws0, q0);
  issue_w(ws1, q0 + 1);
  issue_w(ws2, q0 + 2);
  f16x8 xr[kGemmXAhead][4];  // activation groups in flight, oldest first
#pragma unroll
  for (int i = 0; i < kGemmXAhead; ++i) load_x(4 * q0 + i, xr[i]);
  wait_vmem<4 * kGemmXAhead>();  // the three weight quads are in
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  dequant(ws0, bq0);

  // Quad q: one barrier (every wave has finished quad q-1 and written the
  // operands of quad q; the weight blocks of quad q+1 are in); then the
  // products of quad q run beside the dequantisation of quad q+1 into the
  // other operand buffer (last read in quad q-1).
  for (int qb = q0; qb < q1; qb += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = qb + u;
      if (q >= q1) break;
      // weight quad q+1 (slot (u+1)%4, requested at the start of quad q-2)
      // is in for this wave: since then 16 activation requests per quad
      // and one weight pair. A bare s_barrier: a fenced one would also wait
      // for the quads still in flight, which are LDS writes.
      __builtin_amdgcn_sched_barrier(0);
      wait_vmem<32 + 2>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      issue_w(slot((u + 3) & 3), q + kGemmWAhead);
      uint8_t(*bq)[4][1024] = (u & 1) ? bq1 : bq0;
      uint8_t(*bn)[4][1024] = (u & 1) ? bq0 : bq1;
      dequant(slot((u + 1) & 3), bn);  // quad q+1 (past the split: unused)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f16x8 xa[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          xa[a] = xr[0][a];
#pragma unroll
          for (int i = 0; i + 1 < kGemmXAhead; ++i) xr[i][a] = xr[i + 1][a];
        }
        load_x(4 * q + j + kGemmXAhead, xr[kGemmXAhead - 1]);
        if (!live) continue;
        f16x8 bf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          bf[t] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(&bq[t][j][lane * 16]));
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int a = 0; a < 4; ++a) acc[a][t] = mfma16x16x32_f16(xa[a], bf[t], acc[a][t]);
      }
    }
  }
  wait_vmem<0>();  // no request may land in LDS after the workgroup ends
  if (!live) return;

  // lane holds rows m0 + 16a + 4kb + i of column 64 * tile + 16t + r
  float* o = out + (size_t)blockIdx.z * m * N;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int col = kGemmCols * blockIdx.x + 16 * t + r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + 16 * a + 4 * kb + i;
        if (row < m && col < N) o[(size_t)row * N + col] = acc[a][t][i];
      }
    }
}

// Wide form: workgroup = four waves over 64 rows and 256 columns; wave w
// owns columns 64w .. 64w+63 of the workgroup (4 x 4 tiles of 16 x 16, as
// above). The activation operands of a quad (4 row tiles x 4 groups, 16 KB
// of the packed x) reach a ring of three LDS slots by direct loads, two
// quads ahead, each wave loading one row tile; all four waves read them.
// Each wave loads its own weight tiles (nibbles and scales) straight into
// registers two quads ahead and dequantises them there, so no weight goes
// through LDS. Per 256 products a workgroup then fetches 34 KB (16 KB of
// activations + 4 x 4.5 KB of weights) where the form above fetches 68.5 KB
// (every wave its own 16 KB of activations), and the load return path is
// what that form saturates. The price is four times the dequantisation
// work (each wave dequantises the 64 columns it multiplies). 48 KB of LDS
// and at most 168 registers keep three workgroups on a CU, so 592
// workgroups (a 37888-column matrix at 254 rows) are resident at once.
// Slots are separate LDS variables and the quad loop is unrolled by six
// (three slots, two weight buffers), so every read names its slot and
// buffer (the compiler then waits only for their loads).
constexpr int kWideCols = 256;
constexpr int kWideRows = 64;

struct WideB {
  u32x4 w[4];  // nibble dwords of the wave's 4 column tiles
  u32x2 s[4];  // scale row (4 group scales) of each tile, lane r = row r
};

__global__ __launch_bounds__(256, 3) void w4_gemm_wide_kernel(
    const uint16_t* __restrict__ xh, int m, int rows_pad, const uint8_t* __restrict__ nib,
    const uint8_t* __restrict__ scl, int N, int K, int Q, int qps, int ncb, int nrb,
    float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t as0[4][4][1024], as1[4][4][1024],
      as2[4][4][1024];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kb = lane >> 4, r = lane & 15;
  // workgroups are dealt to the eight XCDs in turn (b % 8); the row blocks
  // of a column block take consecutive turns on one XCD, so its weights are
  // fetched into that XCD's L2 once and hit there for the other row blocks
  const int b = blockIdx.x, xcd = b & 7, turn = b >> 3;
  const int rb = turn % nrb, cb = (turn / nrb) * 8 + xcd;
  if (cb >= ncb) return;  // (whole workgroup, before any barrier)
  const int m0 = rb * kWideRows;
  const int n_tiles = (N + 15) / 16, G = K >> 5;
  const int q0 = blockIdx.z * qps, q1 = min(Q, q0 + qps);
  const int tile0 = cb * (kWideCols / 16) + wave * 4;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(xh), (short)0, rows_pad * K * 2, kBufWord3);
  const __amdgpu_buffer_rsrc_t nrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(nib), (short)0, n_tiles * Q * 1024, kBufWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(scl), (short)0, n_tiles * Q * 128, kBufWord3);
  // Requests for quads past the split (the loop runs a multiple of six)
  // take a lane offset past every buffer's end: they return zeros without
  // a fetch and keep the request counts uniform.
  constexpr uint32_t kPast = 0x80000000u;

  // this wave's row tile of quad q (groups 4q .. 4q+3, each clamped to a
  // real group: groups past K meet weights of scale 0) into a slot: four
  // requests
  const int xrt = m0 / 16 + wave;
  auto issue_a = [&](uint8_t (*sl)[4][1024], int q) {
    const uint32_t vo = q < q1 ? lane * 16u : kPast + lane * 16u;
    q = min(q, q1 - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int g = min(4 * q + j, G - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_void*)&sl[wave][j][0], 16, vo,
                                               (xrt * G + g) * 1024, 0, 0);
    }
  };
  // the wave's four weight tiles of quad q: eight requests (tiles past N
  // re-read the last tile; their columns are never stored)
  auto issue_b = [&](WideB& wb, int q) {
    const uint32_t vn = q < q1 ? lane * 16u : kPast + lane * 16u;
    const uint32_t vs = q < q1 ? r * 8u : kPast + r * 8u;
    q = min(q, q1 - 1);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int tt = min(tile0 + t, n_tiles - 1);
      wb.w[t] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(nrs, vn, (tt * Q + q) * 1024, 0));
      wb.s[t] = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(srs, vs, (tt * Q + q) * 128, 0));
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[a][t] = zero4;

  // products of one quad: activation slot sl, weights wb
  auto quad = [&](uint8_t (*sl)[4][1024], const WideB& wb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f16x8 xa[4], bf[4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
        xa[a] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(&sl[a][j][lane * 16]));
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t sw = wb.s[t][j >> 1] >> (16 * (j & 1));
        const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)(sw & 0xFFFFu));
        const f16x2 s2 = {sc, sc};
        bf[t] = __builtin_bit_cast(f16x8, w4_f16frag(wb.w[t][j], s2));
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int a = 0; a < 4; ++a) acc[a][t] = mfma16x16x32_f16(xa[a], bf[t], acc[a][t]);
    }
  };

  // Issue order, as in the loop (quad i requests A(i+2) at its start and
  // B(i+2) at its end): A(q0) B(q0) | A(q0+1) B(q0+1). At the start of
  // quad q the requests after B(q) are A(q+1) and B(q+1): 4 + 8.
  WideB B0, B1;
  issue_a(as0, q0);
  __builtin_amdgcn_sched_barrier(0);
  issue_b(B0, q0);
  __builtin_amdgcn_sched_barrier(0);
  issue_a(as1, q0 + 1);
  __builtin_amdgcn_sched_barrier(0);
  issue_b(B1, q0 + 1);
  // Quads past the split keep their (empty) requests and barriers but skip
  // the products. (With an early exit from the unrolled body, the loop head
  // was reachable with a different request history, and the compiler then
  // waited for every request before the first quad of each round.)
  for (int qb = q0; qb < q1; qb += 6) {
#pragma unroll
    for (int u = 0; u < 6; ++u) {
      const int q = qb + u;
      // A(q) of every wave is in and every wave is done with quad q-1's
      // slot, which A(q+2) now refills. A bare s_barrier after the
      // count-based wait: a fenced one would also wait for the LDS writes
      // of the quad still in flight.
      __builtin_amdgcn_sched_barrier(0);
      wait_vmem<12>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      uint8_t(*cur)[4][1024] = u % 3 == 0 ? as0 : u % 3 == 1 ? as1 : as2;
      uint8_t(*nxt)[4][1024] = u % 3 == 0 ? as2 : u % 3 == 1 ? as0 : as1;
      issue_a(nxt, q + 2);
      __builtin_amdgcn_sched_barrier(0);
      WideB& wb = (u & 1) ? B1 : B0;
      if (q < q1) quad(cur, wb);  // uniform
      __builtin_amdgcn_sched_barrier(0);
      issue_b(wb, q + 2);
    }
  }
  wait_vmem<0>();  // no request may land in LDS after the workgroup ends

  // lane holds rows m0 + 16a + 4kb + i of column 16 (tile0 + t) + r
  float* o = out + (size_t)blockIdx.z * m * N;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int col = 16 * (tile0 + t) + r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + 16 * a + 4 * kb + i;
        if (row < m && col < N) o[(size_t)row * N + col] = acc[a][t][i];
      }
    }
}

// y = sum of the splits' partial results, in split order
__global__ __launch_bounds__(256) void w4_gemm_reduce_kernel(const float* __restrict__ ws, int ks,
                                                             long long mn, float* __restrict__ y) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= mn) return;
  float s = ws[i];
  for (int k = 1; k < ks; ++k) s += ws[(size_t)k * mn + i];
  y[i] = s;
}

// k splits of the GEMM: enough workgroups for two per compute unit, at most
// kGemmMaxSplits and at most one per quad of 128 k
// Form of the GEMM: 0 = 256 rows x 64 columns per workgroup, 1 = wide (64
// rows x 256 columns). The wide form is chosen when padding the rows to 256
// would leave at least one wave of a workgroup without rows (m mod 256 in
// 1..192): at 134 rows of a 7B-like layer it took 172.8 us against 191.9
// (gate|up 67.4 against 84.7), at 254 rows 225.3 against 214.5, where the
// wide form's four-fold dequantisation (vector work about equal to the
// products' time) outweighs its halved operand traffic. SVE_GEMM_FORM=0|1
// overrides.
static int gemm_form(int m) {
  const char* v = getenv("SVE_GEMM_FORM");
  if (v && *v) return atoi(v) != 0;
  const int rows_narrow = (m + kGemmGroupRows - 1) / kGemmGroupRows * kGemmGroupRows;
  const int rows_wide = (m + kWideRows - 1) / kWideRows * kWideRows;
  return rows_narrow - rows_wide >= kGemmWaveRows;
}

// quads per k split: enough workgroups for two per compute unit, at most
// kGemmMaxSplits splits and at least one quad each; the wide form's quad
// loop runs in rounds of six, so its count is rounded up to a multiple of
// six (fewer, fuller splits instead of empty rounds)
static int gemm_qps(int m, int N, int K) {
  const int Q = (K + 127) / 128;
  const bool wide = gemm_form(m);
  const int base =
      wide ? ((N + kWideCols - 1) / kWideCols) * ((m + kWideRows - 1) / kWideRows)
           : ((N + kGemmCols - 1) / kGemmCols) * ((m + kGemmGroupRows - 1) / kGemmGroupRows);
  int ks = std::max(1, std::min({512 / std::max(base, 1), kGemmMaxSplits, Q}));
  const int forced = getenv("SVE_GEMM_SPLITS") ? atoi(getenv("SVE_GEMM_SPLITS")) : 0;
  if (forced > 0) ks = std::min({forced, kGemmMaxSplits, Q});
  int qps = (Q + ks - 1) / ks;
  if (wide && forced <= 0 && ks > 1) qps = std::min(Q, (qps + 5) / 6 * 6);
  return qps;
}

int w4_gemm_splits(int m, int N, int K) {
  const int Q = (K + 127) / 128, qps = gemm_qps(m, N, K);
  return (Q + qps - 1) / qps;
}

// workspace: x in fp16 in operand order (rows padded to a multiple of 64),
// then the splits' partial results ([splits][m][N] fp32) when k is split
static size_t gemm_xh_bytes(int m, int K) {
  return (size_t)((m + kGemmWaveRows - 1) / kGemmWaveRows) * kGemmWaveRows * K * 2;
}

size_t w4_gemm_workspace_bytes(int m, int N, int K) {
  const int ks = w4_gemm_splits(m, N, K);
  return gemm_xh_bytes(m, K) + (ks > 1 ? (size_t)ks * m * N * sizeof(float) : 0);
}

hipError_t launch_w4_gemm(const void* x, int m, const void* packed, int N, int K, float* y,
                          void* ws, hipStream_t st) {
  const int n_tiles = (N + 15) / 16, Q = (K + 127) / 128;
  const uint8_t* nib = (const uint8_t*)packed;
  const uint8_t* scl = nib + (size_t)n_tiles * Q * 1024;
  const int qps = gemm_qps(m, N, K);
  const int ks = (Q + qps - 1) / qps;
  // the kernel's buffer offsets are 32-bit
  if ((size_t)n_tiles * Q * 1024 >= (1u << 31) || gemm_xh_bytes(m, K) >= (1u << 31))
    return hipErrorInvalidValue;
  const dim3 grid((N + kGemmCols - 1) / kGemmCols, (m + kGemmGroupRows - 1) / kGemmGroupRows, ks);
  uint16_t* xh = (uint16_t*)ws;
  float* part = (float*)((uint8_t*)ws + gemm_xh_bytes(m, K));
  const long long pieces = (long long)gemm_xh_bytes(m, K) / 16;
  hipLaunchKernelGGL(w4_x_pack_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, st,
                     (const uint16_t*)x, m, K, pieces, xh);
  float* out = ks > 1 ? part : y;
  if (gemm_form(m)) {
    const int ncb = (N + kWideCols - 1) / kWideCols, nrb = (m + kWideRows - 1) / kWideRows;
    const int rows_pad = (int)(gemm_xh_bytes(m, K) / ((size_t)K * 2));
    const dim3 wgrid((unsigned)((ncb + 7) / 8 * 8 * nrb), 1, ks);
    hipLaunchKernelGGL(w4_gemm_wide_kernel, wgrid, dim3(256), 0, st, xh, m, rows_pad, nib, scl, N,
                       K, Q, qps, ncb, nrb, out);
  } else {
    hipLaunchKernelGGL(w4_gemm_kernel, grid, dim3(256), 0, st, xh, m, nib, scl, N, K, Q, qps, out);
  }
  if (ks > 1) {
    const long long mn = (long long)m * N;
    hipLaunchKernelGGL(w4_gemm_reduce_kernel, dim3((unsigned)((mn + 255) / 256)), dim3(256), 0, st,
                       part, ks, mn, y);
  }
  return hipGetLastError();
}

static int env_int_w4(const char* name, int dflt) {
  const char* v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

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

hipError_t launch_w4_gemv(const void* x, int m, const void* packed, int N, int K, float* y,
                          hipStream_t st, int wgs_per_cu) {
  const int n_tiles = (N + 15) / 16, Q = (K + 127) / 128;
  const uint8_t* nib = (const uint8_t*)packed;
  const uint8_t* scl = nib + (size_t)n_tiles * Q * 1024;
  const uint16_t* xp = (const uint16_t*)x;
  // short K: the fewest quads per wave (1, 2 or 4) whose slices cover K
  // within the kernel's wave limit
  int qpw = 0;
  for (int c : {1, 2, 4})
    if (qpw == 0 && (Q + c - 1) / c <= short_max_waves(c)) qpw = c;
  const int forced = env_int_w4("SVE_GEMV_QPW", 0);
  if (qpw > 0 && (forced == 1 || forced == 2 || forced == 4) &&
      (Q + forced - 1) / forced <= short_max_waves(forced))
    qpw = forced;
  if (qpw > 0) {
    const int W = (Q + qpw - 1) / qpw;
    // one tile per workgroup while that fits one round of the chip (one
    // workgroup per CU), else a grid of runs of at least two tiles
    const int per_cu = wgs_per_cu > 0 ? wgs_per_cu : 1;
    const bool single = wgs_per_cu <= 0 && n_tiles <= 256;
    const int grid = single ? n_tiles : std::max(1, std::min(n_tiles / 2, 256 * per_cu));
    // runs of tiles: every grid-th tile per workgroup (measured 0.5 us faster
    // than contiguous runs on a 24576x4096 matrix); SVE_GEMV_STRIDE=0 keeps
    // the contiguous runs
    const int strided = env_int_w4("SVE_GEMV_STRIDE", 1);
    // C0 terms once per wave: with one quad per wave, and for single tiles
    // (4096x4096 at m = 1 / 8: 5.28 / 5.96 us against 5.60 / 6.48 recomputed);
    // runs of two-quad waves recompute them (6144x4096 and 24576x4096 were
    // 0.1-0.7 us slower hoisted)
    const int hoist_env = env_int_w4("SVE_GEMV_HOIST", -1);
    const bool hoist = hoist_env >= 0 ? hoist_env != 0 : (qpw == 1 || single);
#define SVE_SHORT(Q_, S_, H_, D_)                                                              \
  hipLaunchKernelGGL((w4_gemv_short_kernel<Q_, S_, H_, D_>), dim3(grid), dim3(64 * W), 0, st, \
                     xp, m, nib, scl, N, K, Q, n_tiles, strided, y)
#define SVE_RUN(Q_, H_) SVE_SHORT(Q_, false, H_, 2)
    switch (qpw * 4 + (single ? 2 : 0) + (hoist ? 1 : 0)) {
      case 4: SVE_RUN(1, false); break;
      case 5: SVE_RUN(1, true); break;
      case 6: SVE_SHORT(1, true, false, 1); break;
      case 7: SVE_SHORT(1, true, true, 1); break;
      case 8: SVE_RUN(2, false); break;
      case 9: SVE_RUN(2, true); break;
      case 10: SVE_SHORT(2, true, false, 1); break;
      case 11: SVE_SHORT(2, true, true, 1); break;
      case 16: SVE_RUN(4, false); break;
      case 17: SVE_RUN(4, true); break;
      case 18: SVE_SHORT(4, true, false, 1); break;
      default: SVE_SHORT(4, true, true, 1); break;  // 19
    }
#undef SVE_RUN
#undef SVE_SHORT
  } else {
    const int W = kLongMaxWaves;
#define SVE_LONG(NU_)                                                                            \
  hipLaunchKernelGGL(w4_gemv_long_kernel<NU_>, dim3(n_tiles), dim3(64 * W), 0, st, xp, m, nib, scl, \
                     N, K, Q, n_tiles, y)
    switch ((m + 1) / 2) {
      case 1: SVE_LONG(1); break;
      case 2: SVE_LONG(2); break;
      case 3: SVE_LONG(3); break;
      case 4: SVE_LONG(4); break;
      case 5: SVE_LONG(5); break;
      case 6: SVE_LONG(6); break;
      case 7: SVE_LONG(7); break;
      default: SVE_LONG(8); break;
    }
#undef SVE_LONG
  }
  return hipGetLastError();
}

hipError_t launch_w4_gemv_routed(const void* x, int x_per_slot, int m, const int32_t* ids,
                                 int topk, const void* packed_all, int E, int N, int K, float* y,
                                 hipStream_t st) {
  const int n_tiles = (N + 15) / 16, Q = (K + 127) / 128;
  const size_t eb = w4_packed_bytes(N, K);
  const size_t scale_off = (size_t)n_tiles * Q * 1024;
  // (two quads per wave would exceed the 16-wave register budget here)
  int qpw = 0;
  for (int c : {1, 4})
    if (qpw == 0 && (Q + c - 1) / c <= short_max_waves(c)) qpw = c;
  if (qpw > 0) {
    const int W = (Q + qpw - 1) / qpw;
    // row tiles per workgroup: about 8192 waves in all if every pair slot
    // owned a distinct expert (two rounds of 16 waves per CU); an even
    // count, at least two
    const int npairs = m * topk;
    int run = (int)(((long long)n_tiles * npairs * W + 8191) / 8192);
    run = std::max(kRoutedRun, std::min((run + 1) / 2 * 2, n_tiles));
    // tiles per LDS batch: an even count, at most the run
    const int batch = std::max(2, std::min((run + 1) / 2 * 2, kGemvPartSlots / W / 2 * 2));
    const size_t lds = (size_t)batch * W * 64 * sizeof(float) * 4;
    const dim3 grid((n_tiles + run - 1) / run, npairs);
#define SVE_ROUTED(Q_)                                                                          \
  hipLaunchKernelGGL((w4_gemv_routed_short_kernel<Q_>), grid, dim3(64 * W), lds, st,             \
                     (const uint16_t*)x, x_per_slot, m, ids, topk, (const uint8_t*)packed_all, eb, \
                     scale_off, E, N, K, Q, n_tiles, run, batch, y)
    if (qpw == 1)
      SVE_ROUTED(1);
    else
      SVE_ROUTED(4);
#undef SVE_ROUTED
    return hipGetLastError();
  }
  // long K: the ring-pipelined form
  const int tpw = kGemvWaves / gemv_ks(Q);
  const dim3 grid((n_tiles + tpw - 1) / tpw, m * topk);
  hipLaunchKernelGGL(w4_gemv_routed_kernel<1>, grid, dim3(kGemvThreads), 0, st,
                     (const uint16_t*)x, x_per_slot, m, ids, topk, (const uint8_t*)packed_all, eb,
                     scale_off, E, N, K, Q, n_tiles, y);
  return hipGetLastError();
}

}  // namespace sve
