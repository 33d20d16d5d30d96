// Extend-prefill attention on gfx950.
//
// m new query rows (positions P .. P+m-1) attend causally to the P cached
// positions of a resident KV slot plus themselves: row i sees keys 0..P+i.
// (goinfer, "Turn nine in under half a second", sections "What goinfer does"
// and "How it works": the cache keeps one key and one value vector per token
// and layer, and only the tokens after the reused start are prefilled.)
// Scores are scaled by 1/sqrt(D); q head h reads KV head h / (Hq/Hkv).
//
// Store layout per (slot, layer): K [Hkv][cap][D] (row per position) and
// Vt [Hkv][D][cap] (V transposed, position fastest), bf16. cap is a multiple
// of 64. Grouped-query rows are packed: for KV head h the packed row index is
// pr = i*g + j (query row i, query head h*g + j), so one K/V tile serves all g
// heads of the group.
//
// Work is split over key ranges ("splits") aligned to absolute multiples of
// the split length; each split yields an unnormalised partial (O, running
// max, sum) merged afterwards in a fixed order.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace sve {

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// 2^x by the hardware exponential (v_exp_f32); results below the normal
// range flush to zero, which only ever affects probabilities that round to
// nothing next to the row maximum.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Split partials hold a split's normalised output o = O / l (a convex mix of
// value rows) in fp16, divided by 2^e: e = 0 unless the row's largest |o|
// reaches 2^15, so the stored values stay inside the fp16 range. fp16 keeps
// 11 significant bits, four more than the bf16 output.
__device__ __forceinline__ int partial_exp(float rowmax) {
  const int k = (int)((__float_as_uint(rowmax) >> 23) & 0xffu) - 127;  // floor(log2) of a normal
  return max(0, k - 14);
}

struct SegRef {
  int s, local;
};

__device__ __forceinline__ SegRef find_seg(const AttnParams& p, int L) {
  int s = 0;
#pragma unroll
  for (int j = 1; j < kMaxSeg; ++j)
    if (j < p.nseg && L >= p.seg[j].block_begin) s = j;
  return SegRef{s, L - p.seg[s].block_begin};
}

// Linear work index of this workgroup, arranged so that each of the 8 XCDs
// (workgroups are dealt to XCDs round robin) receives one contiguous range of
// work: neighbouring row blocks of a KV head then share that XCD's L2.
__device__ __forceinline__ int xcd_linear(int b, int nb) {
  const int xcd = b & 7, per = nb >> 3, rem = nb & 7;
  return xcd * per + min(xcd, rem) + (b >> 3);
}

// ---------------------------------------------------------------------------
// KV append: K rows copied, V rows transposed into Vt through LDS.
// grid (ceil(m/16), Hkv, nseg), block 256: 16 new rows of one KV head.
// ---------------------------------------------------------------------------
constexpr int kAppendRows = 16;

template <int D>
__global__ __launch_bounds__(256) void kv_append_kernel(AttnParams p) {
  const AttnSeg& sg = p.seg[blockIdx.z];
  // the attention kernel appends this piece, or nothing is appended
  if (sg.new_tile0 >= 0 || sg.no_append) return;
  const int i0 = blockIdx.x * kAppendRows;
  if (i0 >= sg.m) return;
  const int h = blockIdx.y, Hkv = p.Hkv, cap = p.cap;
  const int rows = min(kAppendRows, sg.m - i0);
  constexpr int CPR = D / 8;
  uint16_t* K = const_cast<uint16_t*>(sg.K) + (size_t)h * cap * D;
  uint16_t* Vt = const_cast<uint16_t*>(sg.Vt) + (size_t)h * D * cap;
  __shared__ uint16_t tile[D][kAppendRows + 2];
  for (int c = threadIdx.x; c < rows * CPR; c += 256) {
    const int r = c / CPR, col = c % CPR;
    const size_t src = ((size_t)(i0 + r) * Hkv + h) * D + col * 8;
    store16(K + (size_t)(sg.P + i0 + r) * D + col * 8, load16(sg.nk + src));
    const u32x4 v = load16(sg.nv + src);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[col * 8 + 2 * e][r] = (uint16_t)(v[e] & 0xFFFFu);
      tile[col * 8 + 2 * e + 1][r] = (uint16_t)(v[e] >> 16);
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < D * kAppendRows; c += 256) {
    const int d = c / kAppendRows, r = c % kAppendRows;
    if (r < rows) Vt[(size_t)d * cap + sg.P + i0 + r] = tile[d][r];
  }
  // Positions after the sequence up to the end of its last 64-key tile are
  // read by the attention kernels (with zero probability): keep them zero so
  // stale cache contents can never reach the value product.
  if (blockIdx.x == 0) {
    const int e0 = sg.P + sg.m, e1 = min(cap, (e0 + 63) / 64 * 64);
    for (int c = threadIdx.x; c < D * 64; c += 256) {
      const int d = c >> 6, pos = e0 + (c & 63);
      if (pos < e1) Vt[(size_t)d * cap + pos] = 0;
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA path. Workgroup = 8 waves in two key groups of 4. Both groups hold the
// same 64*RT packed rows of one KV head (each wave 16*RT rows); group G takes
// the 64-key tiles kstart + 64*(2j + G) of the workgroup's key split, so two
// waves share every SIMD and one's matrix work overlaps the other's softmax.
// Each group stages its tiles with direct global-to-LDS loads into its own
// double buffer (K [64][D] and Vt [D][64], dense with an XOR swizzle of the
// 16-byte chunks applied on the global side), requesting tile j+1 while
// computing tile j. At the end group 1 hands its (max, sum, O) to group 0
// through LDS and group 0 merges and writes.
//   S^T = K Q^T   (A = 16 keys x 32 d from LDS, B = Q^T held in registers)
//   O^T += Vt P^T (A = 16 d x 32 keys from LDS, B = P^T straight from the
//                  S^T accumulators, rounded to bf16)
// Within a 32-key chunk the 16-key MFMA sub-tiles take keys
// 8*(j/4) + 4*sub + j%4, so that lane (row, kb) ends up holding keys
// 8*kb .. 8*kb+7 of the chunk: exactly its B operand for the value product,
// and its Vt A operand is one 16-byte LDS read. Each lane owns one packed
// row (lane % 16): row statistics need two cross-lane steps only.
// ---------------------------------------------------------------------------
// swizzled 16-byte chunk position of chunk c in K-tile row `key` (D/8 chunks
// per row) and in Vt-tile row `d` (8 chunks per row)
template <int D>
__device__ __forceinline__ int kswz(int key, int c) {
  constexpr int CPR = D / 8;
  return c ^ (((key & (CPR - 1)) ^ (((key >> 4) & 1) << 2)) & (CPR - 1));
}
__device__ __forceinline__ int vswz(int d, int c) { return c ^ ((d >> 1) & 7); }

// row-block workgroups of the last split that append the call's rows
constexpr int kAppendBlocks = 4;

// dwords per staged partial row (D/2 fp16 pairs + 4 of padding against bank
// conflicts)
template <int D>
constexpr int kStageRow = D / 2 + 4;

// ONE: the call has a single piece (its fields load without first finding
// the piece, one scalar round trip less). QB: several questions about one
// state, so a new row also masks the new rows of the other questions (kept
// out of the ordinary variant: the band costs a calls' epilogue about a
// microsecond)
template <int D, int RT, bool ONE, bool QB>
__global__ __launch_bounds__(512) void attn_mfma_kernel(AttnParams prm) {
  constexpr int DC = D / 32;
  constexpr int DT = D / 16;
  constexpr int CPR = D / 8;            // 16-byte chunks per K row
  constexpr int TILE = 64 * D;          // bf16 elements per K (or Vt) tile
  constexpr int DMA_PER_WAVE = (TILE * 2) / 1024 / 4;  // 1 KB DMA steps per wave per tile part
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][2][TILE];  // [group][buf][K|Vt]

  const int L = xcd_linear(blockIdx.x, gridDim.x);
  const SegRef ref = ONE ? SegRef{0, L} : find_seg(prm, L);
  const AttnSeg& sg = prm.seg[ONE ? 0 : ref.s];
  const int g = prm.g, Hq = prm.Hq, cap = prm.cap;
  const int P = sg.P, m = sg.m, R = m * g;
  // split-major within a KV head: a split has a workgroup for each row block
  // from the first one whose last row sees a key of the split's tiles (the
  // first such block: g * X / (64 RT) for the split's first key P + X)
  const int kvh = ref.local / sg.head_blocks;
  int split = 0, rb = 0, t_lo = 0, t_hi = 0;
  {
    // (unrolled over the table so its entries load together)
    int j = ref.local - kvh * sg.head_blocks;
    bool found = false;
#pragma unroll
    for (int n = 0; n < kMaxSplits; ++n) {
      if (!found && n < sg.splits) {
        const int lo = sg.tile_bound[n];
        const int X = 64 * lo - P;
        const int rb0 = X > 0 ? (g * X) / (64 * RT) : 0;
        if (j < sg.row_blocks - rb0) {
          found = true;
          split = n;
          rb = rb0 + j;
          t_lo = lo;
          t_hi = sg.tile_bound[n + 1];
        }
        j -= sg.row_blocks - rb0;
      }
    }
  }

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2, gw = wave & 3;
  const int kb = lane >> 4, col = lane & 15;

  const int wg_row0 = rb * 64 * RT;
  const int wg_last = min(R - 1, wg_row0 + 64 * RT - 1);
  // 64-key tiles [64T, 64T+64); a split is a run of them [t_lo, t_hi). With
  // new_tile0 >= 0 the tiles from new_tile0 = P / 64 on go through the
  // epilogue, which reads keys at or past P from the call's rows; the others
  // come from the store through the staged loop.
  const int nt0 = sg.new_tile0;
  const bool fused = nt0 >= 0;
  const int t_rows = (P + wg_last / g) / 64 + 1;  // tiles any row of the block sees
  const int t_begin = t_lo;
  const int t_end = min(t_hi, t_rows);
  if (t_begin >= t_end) return;  // (not launched: no row of the block sees the split)
  const int wg_min_lim = P + wg_row0 / g;
  const int t_cend = fused ? max(t_begin, min(t_end, nt0)) : t_end;
  const int ntiles = t_cend - t_begin;  // staged loop
  const int nnew = t_end - t_cend;      // epilogue
  const int kstart = 64 * t_begin;

  // packed row of (lane, rt): query row qi, query head qh (recomputed where
  // needed rather than held through the key loop)
  auto prow = [&](int rt) { return wg_row0 + gw * 16 * RT + 16 * rt + col; };
  int lim[RT];
  bf16x8 qreg[RT][DC];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int pr = prow(rt);
    const bool valid = pr < R;
    const int i = valid ? pr / g : 0;
    const int qh = kvh * g + (valid ? pr % g : 0);
    lim[rt] = valid ? P + i : 0;
    // padded rows read a live query row; their outputs are never stored
    const uint16_t* qrow = sg.q + ((size_t)i * Hq + qh) * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) qreg[rt][dc] = as_bf16x8(load16(qrow + 32 * dc + 8 * kb));
  }

  f32x4 O[RT][DT];
  float mref[RT], lrun[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    mref[rt] = -INFINITY;
    lrun[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const uint16_t* Kg = sg.K + (size_t)kvh * cap * D;
  const uint16_t* Vg = sg.Vt + (size_t)kvh * D * cap;
  const float cs = prm.c;

  // Per-lane byte offsets of the direct loads. Step u of a wave covers tile
  // chunks (gw + 4u)*64 + lane: K rows 4096u bytes further on, with the
  // swizzle of step u & 1, and Vt rows 64u*cap bytes further on, with the
  // swizzle of step 0; the step terms are uniform and join the scalar base.
  uint32_t kloc[2], vloc;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int pos = (gw + 4 * u) * 64 + lane;
    const int key = pos / CPR;
    kloc[u] = (uint32_t)(key * D + kswz<D>(key, pos % CPR) * 8) * 2u - 4096u * u;
  }
  {
    const int pos = gw * 64 + lane, d = pos >> 3;
    vloc = (uint32_t)(d * cap + vswz(d, pos & 7) * 8) * 2u;
  }
  // Every row block walks its tiles in order (key group G takes tiles G,
  // G+2, ...): the workgroups' first requests then cover only the first
  // tiles of each split. (Starting each row block at a different tile
  // spread the L2 traffic but made the opening burst fetch nearly every tile
  // from HBM before any workgroup could start: 0.3 us slower at turn 9.)
  const int mytiles = (ntiles - grp + 1) / 2;  // tiles of this key group
  auto tile_kt = [&](int t) { return kstart + 64 * (2 * t + grp); };
  // direct loads of the K (or Vt) part of tile t into buffer t % 2, through
  // buffer resources over this KV head's K and Vt (the tile and step terms
  // are uniform offsets)
  const __amdgpu_buffer_rsrc_t krsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Kg), (short)0, cap * D * 2, kBufWord3);
  const __amdgpu_buffer_rsrc_t vrsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Vg), (short)0, D * cap * 2, kBufWord3);
  auto dma_k = [&](int t) {
    const int base = tile_kt(t) * D * 2;
#pragma unroll
    for (int u = 0; u < DMA_PER_WAVE; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc,
                                               (lds_void*)&lds[grp][t & 1][0][(gw + 4 * u) * 512],
                                               16, (int)kloc[u & 1], base + 4096 * u, 0, 0);
  };
  auto dma_v = [&](int t) {
    const int base = tile_kt(t) * 2;
#pragma unroll
    for (int u = 0; u < DMA_PER_WAVE; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrsrc,
                                               (lds_void*)&lds[grp][t & 1][1][(gw + 4 * u) * 512],
                                               16, (int)vloc, base + 64 * u * cap, 0, 0);
  };

  f32x4 S[RT][2][2];
  bf16x8 pb[RT][2];
  // online softmax of tile t: mask, running max, rescale, bf16 probabilities
  // lower end of the new keys a row sees (epilogue only): P + the start of
  // its question; P for an ordinary extend
  int blo[RT];
  auto softmax = [&](int kt, auto edge_tag, auto band_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    constexpr bool BAND = decltype(band_tag)::value;
    bool grow = false;
    float mcand[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float mx = -INFINITY;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = S[rt][c][sub][i];
            if constexpr (EDGE) {
              const int key = kt + 32 * c + 8 * kb + 4 * sub + i;
              // (bitwise, not short-circuit: no branch per element)
              bool vis = key <= lim[rt];
              if constexpr (BAND) vis = vis & ((key < P) | (key >= blo[rt]));
              v = vis ? v : -INFINITY;
              S[rt][c][sub][i] = v;
            }
            mx = fmaxf(mx, v);
          }
      mx = max4_rows(mx);
      mcand[rt] = mx * cs;
      // the reference max moves only when a row's max grows by more than 8
      // (log2 units): probabilities then stay below 2^8 and the running
      // output is rescaled rarely
      grow |= mcand[rt] > mref[rt] + 8.f;
    }
    if (__ballot(grow) != 0) {
      // only the rows that grew move their reference, so every row's
      // arithmetic depends on that row alone
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const bool up = mcand[rt] > mref[rt] + 8.f;
        const float alpha = up ? fast_exp2(mref[rt] - mcand[rt]) : 1.f;
        mref[rt] = up ? mcand[rt] : mref[rt];
        lrun[rt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) O[rt][dt][i] *= alpha;
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float muse = (mref[rt] == -INFINITY) ? 0.f : mref[rt];
      float psum = lrun[rt];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        u32x4 pk;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const float p0 = fast_exp2(fmaf(S[rt][c][sub][i], cs, -muse));
            const float p1 = fast_exp2(fmaf(S[rt][c][sub][i + 1], cs, -muse));
            const uint32_t w = pack_bf16x2(p0, p1);
            pk[2 * sub + (i >> 1)] = w;
            psum = dot2_bf16(w, 0x3F803F80u, psum);  // + both bf16 values exactly
          }
        pb[rt][c] = as_bf16x8(pk);
      }
      lrun[rt] = psum;
    }
  };
  // Matrix stage: PV(tpv) (O^T += Vt P^T from tile tpv's Vt part) and/or
  // QK(tqk) (S^T = K Q^T from tile tqk's K part) as one stream of 16-byte
  // LDS operand reads, each feeding the two row tiles' products, with the
  // read for step s+4 issued before the products of step s so that LDS
  // latency hides behind the matrix pipe. Step order keeps consecutive
  // products on different accumulators.
  auto mstage = [&](int tpv, int tqk, auto pv_tag, auto qk_tag) {
    constexpr bool DO_PV = decltype(pv_tag)::value, DO_QK = decltype(qk_tag)::value;
    constexpr int NPV = DO_PV ? 2 * DT : 0;  // V operands (c, dt), dt fastest
    constexpr int NQK = DO_QK ? 4 * DC : 0;  // K operands (dc, c, sub), (c, sub) fastest
    constexpr int N = NPV + NQK;
    constexpr int AHEAD = 4;
    const uint16_t* Vs = lds[grp][tpv & 1][1];
    const uint16_t* Ks = lds[grp][tqk & 1][0];
    auto operand = [&](int st) -> bf16x8 {
      if (st < NPV) {
        const int c = st / DT, dt = st % DT;
        const int d = 16 * dt + col;
        return as_bf16x8(load16(Vs + d * 64 + vswz(d, 4 * c + kb) * 8));
      }
      const int q = st - NPV;
      const int dc = q / 4, c = (q >> 1) & 1, sub = q & 1;
      const int kappa = 32 * c + 8 * (col >> 2) + 4 * sub + (col & 3);
      return as_bf16x8(load16(Ks + kappa * D + kswz<D>(kappa, 4 * dc + kb) * 8));
    };
    if constexpr (DO_QK) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) S[rt][c][sub] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    bf16x8 ring[AHEAD];
#pragma unroll
    for (int st = 0; st < AHEAD; ++st) ring[st] = operand(st);
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
    for (int st = 0; st < N; ++st) {
      const bf16x8 op = ring[st % AHEAD];
      if (st + AHEAD < N) ring[st % AHEAD] = operand(st + AHEAD);
      if (st < NPV) {
        const int c = st / DT, dt = st % DT;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) O[rt][dt] = mfma16x16x32(op, pb[rt][c], O[rt][dt]);
      } else {
        const int q = st - NPV;
        const int dc = q / 4, c = (q >> 1) & 1, sub = q & 1;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          S[rt][c][sub] = mfma16x16x32(op, qreg[rt][dc], S[rt][c][sub]);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, RT, 0);
      if (st + AHEAD < N) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  auto stage_end = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Staged schedule. A key group's stages are
  //   QK(0) | softmax(0) | PV(0) QK(1) | softmax(1) | ... | softmax(n-1) | PV(n-1)
  // and group 1 runs one stage behind group 0, so in every stage one wave of
  // each SIMD issues matrix products while its partner computes
  // exponentials. A workgroup barrier closes every stage. The K part of tile
  // j+2 and the Vt part of tile j+1 are requested at the start of
  // softmax(j) (their buffers were last read in the stage before); the end
  // of softmax(j) waits only for the requests made two stages earlier,
  // which are what the next stage reads.
  constexpr int NV = DMA_PER_WAVE;
  const int n = mytiles;
  if (n > 0) {
    dma_k(0);
    dma_v(0);
  }
  if (n > 1) dma_k(1);
  if (grp == 1) stage_end();  // group 1 starts one stage later
  if (n > 1)
    wait_vmem<2 * NV>();  // K(0) in; V(0), K(1) may be in flight
  else if (n == 1)
    wait_vmem<NV>();
  // (with no staged tile the query loads stay in flight into the epilogue,
  // beside its first tile requests)
  stage_end();
  int nbar = grp + 1;
  if (n > 0) {
    mstage(0, 0, std::false_type{}, std::true_type{});
    stage_end();
    for (int j = 0; j + 1 < n; ++j) {
      const bool k2 = j + 2 < n;
      if (k2) dma_k(j + 2);
      dma_v(j + 1);
      // Keys past a row's causal limit only occur in tiles that reach beyond
      // the smallest limit of the workgroup's rows; only those mask.
      if (tile_kt(j) + 63 > wg_min_lim)
        softmax(tile_kt(j), std::true_type{}, std::false_type{});
      else
        softmax(tile_kt(j), std::false_type{}, std::false_type{});
      if (k2)
        wait_vmem<2 * NV>();
      else
        wait_vmem<NV>();
      stage_end();
      mstage(j, j + 1, std::true_type{}, std::true_type{});
      stage_end();
    }
    if (tile_kt(n - 1) + 63 > wg_min_lim)
      softmax(tile_kt(n - 1), std::true_type{}, std::false_type{});
    else
      softmax(tile_kt(n - 1), std::false_type{}, std::false_type{});
    wait_vmem<0>();
    stage_end();
    mstage(n - 1, 0, std::true_type{}, std::false_type{});
    stage_end();
    nbar += 2 * n + 1;
  }
  // both groups pass the same number of barriers
  const int n0 = (ntiles + 1) / 2, n1 = ntiles / 2;
  const int total = max(2 * n0 + 2, 2 * n1 + 3);
  for (; nbar < total; ++nbar) stage_end();

  if (nnew > 0) {
    // Tiles holding new keys, two per round (group G takes tile 2r + G).
    // K: each 16-byte piece from the store below P and from the call's rows
    // at or past P, straight into LDS in the K-tile layout (round r uses
    // buffer r % 2's K part). V: the store's Vt pieces whose keys are below P
    // (only in the tile holding P) straight into buffer 1's V part (Vt-tile
    // layout); the call's V rows into buffer 0's V part (16-byte chunk c of
    // row key at chunk c ^ (key % CPR)), transposed from there into buffer
    // 1's V part (overwriting the store's values at or past P in the piece
    // holding P). Reads past row m-1 of the call return zeros. The requests
    // of round r+1 go out once round r's V rows are transposed, so they
    // overlap round r's products. No workgroup of the call reads the store
    // at positions P .. P+m-1 except as masked keys.
    const int Hkv = prm.Hkv;
    const int new_bytes = ((m - 1) * Hkv + 1) * D * 2;
    const __amdgpu_buffer_rsrc_t nkrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(sg.nk + (size_t)kvh * D), (short)0, new_bytes, kBufWord3);
    const __amdgpu_buffer_rsrc_t nvrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(sg.nv + (size_t)kvh * D), (short)0, new_bytes, kBufWord3);
    uint16_t* Kw = const_cast<uint16_t*>(Kg);
    uint16_t* Vw = const_cast<uint16_t*>(Vg);
    // the lane index taken afresh: offsets built from it here are not merged
    // with the prologue's, which would keep them live through the key loop
    const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) & 63;
    const int gt = gw * 64 + ln;  // thread within the key group
    // each row's question (several questions: rows of question j see the
    // prefix and the rows of question j only), from the fresh lane index;
    // only the questions variant has the band
    if constexpr (QB) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int i = min(wg_row0 + gw * 16 * RT + 16 * rt + (ln & 15), R - 1) / g;
        int s0 = 0;
#pragma unroll
        for (int j = 1; j < kMaxQuestions; ++j)
          if (j < sg.nq && i >= sg.qstart[j]) s0 = sg.qstart[j];
        blo[rt] = P + s0;
      }
    }
    const int wt = wave * 64 + ln;  // thread within the workgroup
    constexpr int ITEMS = CPR / 4;  // 16-byte pieces per thread per tile part
    uint16_t* Vr = lds[grp][0][1];  // the call's V rows as loaded
    uint16_t* Vs = lds[grp][1][1];  // Vt-tile layout
    auto new_tile_key0 = [&](int r) { return 64 * (t_cend + r + grp); };
    // requests of round r (this group's tile, if it has one)
    auto requests = [&](int r) {
      if (r + grp >= nnew) return;
      const int kt = new_tile_key0(r);
      uint16_t* Ks = lds[grp][(r >> 1) & 1][0];
#pragma unroll
      for (int u = 0; u < DMA_PER_WAVE; ++u) {
        const int pos = (gw + 4 * u) * 64 + ln;
        lds_void* dk = (lds_void*)&Ks[(gw + 4 * u) * 512];
        lds_void* dvr = (lds_void*)&Vr[(gw + 4 * u) * 512];
        lds_void* dvs = (lds_void*)&Vs[(gw + 4 * u) * 512];
        {  // K piece (key, slot): chunk kswz(key, slot) of key kt + key
          const int key = pos / CPR, slot = pos % CPR, k = kt + key;
          const int ch = kswz<D>(key, slot);
          if (k < P)  // the same piece as the key loop's direct loads
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, dk, 16, (int)kloc[u & 1],
                                                     kt * D * 2 + 4096 * u, 0, 0);
          else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                nkrsrc, dk, 16, ((k - P) * Hkv * D + ch * 8) * 2, 0, 0, 0);
          // V row piece of the same (key, slot) for keys at or past P
          if (k >= P)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                nvrsrc, dvr, 16, ((k - P) * Hkv * D + (slot ^ (key % CPR)) * 8) * 2, 0, 0, 0);
        }
        if (kt < P) {  // Vt piece (d, slot), when its first key is cached
          const int d = pos >> 3, k8 = kt + 8 * vswz(d, pos & 7);
          if (k8 < P)  // the same piece as the key loop's direct loads
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrsrc, dvs, 16, (int)vloc,
                                                     kt * 2 + 64 * u * cap, 0, 0);
        }
      }
    };
    // rounds use buffer (r / 2) % 2's K part: r counts tiles, two per round
    requests(0);
    for (int r0 = 0; r0 < nnew; r0 += 2) {
      const bool has = r0 + grp < nnew;
      const int kt = new_tile_key0(r0);
      const uint16_t* Ks = lds[grp][(r0 >> 1) & 1][0];
      wait_vmem<0>();
      __syncthreads();
      if (has) {
        // transpose the keys at or past P: lane = key, so the 2-byte writes
        // of one column are contiguous
#pragma unroll
        for (int u = 0; u < ITEMS; ++u) {
          const int item = gt + 256 * u, key = item & 63, c = item >> 6, k = kt + key;
          if (k >= P) {
            const u32x4 v = load16(Vr + key * D + (c ^ (key % CPR)) * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int d = 8 * c + e;
              const uint16_t x = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
              Vs[d * 64 + vswz(d, key >> 3) * 8 + (key & 7)] = x;
            }
          }
        }
      }
      __syncthreads();
      requests(r0 + 2);  // into the other K buffer and the now free row buffer
      if (has) {
        mstage(0, (r0 >> 1) & 1, std::false_type{}, std::true_type{});
        softmax(kt, std::true_type{}, std::bool_constant<QB>{});
        mstage(1, 0, std::true_type{}, std::false_type{});
      }
      __syncthreads();
    }

    // Append (unsplit pieces; a split piece's rows are appended by the
    // combine kernel): workgroup rb < A takes the 64-key tiles T0 + rb,
    // T0 + rb + A, ... of the new range. K rows are copied as they are; V rows go into
    // LDS as [key][D + 2] (odd dword stride: the column reads below meet
    // distinct banks) and leave as 16-byte pieces of 8 keys of one column,
    // key by key in the pieces holding P or P+m.
    const int A = min(sg.row_blocks, kAppendBlocks);
    if (sg.splits == 1 && !sg.no_append && rb < A) {
      constexpr int VST = D + 2;
      uint16_t* Va = &lds[0][0][0][0];  // [64][VST]
      const uint16_t* nkh = sg.nk + (size_t)kvh * D;
      const uint16_t* nvh = sg.nv + (size_t)kvh * D;
      const int T0 = P / 64, T1 = (P + m - 1) / 64;
      for (int T = T0 + rb; T <= T1; T += A) {
        for (int it = wt; it < 64 * CPR; it += 512) {
          const int key = it / CPR, c = it % CPR, k = 64 * T + key;
          if (k >= P && k < P + m) {
            const size_t src = (size_t)(k - P) * Hkv * D + c * 8;
            store16(Kw + (size_t)k * D + c * 8, load16(nkh + src));
            const u32x4 v = load16(nvh + src);
            uint32_t* row = reinterpret_cast<uint32_t*>(Va + key * VST + c * 8);
#pragma unroll
            for (int e = 0; e < 4; ++e) row[e] = v[e];
          }
        }
        __syncthreads();
        for (int it = wt; it < D * 8; it += 512) {
          const int j = it & 7, d = it >> 3, k8 = 64 * T + 8 * j;
          if (k8 + 8 <= P || k8 >= P + m) continue;
          uint16_t x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = Va[(8 * j + e) * VST + d];
          uint16_t* dst = Vw + (size_t)d * cap + k8;
          if (k8 >= P && k8 + 8 <= P + m) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (uint32_t)x[2 * e] | ((uint32_t)x[2 * e + 1] << 16);
            store16(dst, w);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (k8 + e >= P && k8 + e < P + m) dst[e] = x[e];
          }
        }
        __syncthreads();
      }
    }
  }

  // merge group 1 into group 0 (same lane = same rows and columns)
  f32x4* xo = reinterpret_cast<f32x4*>(&lds[0][0][0][0]);  // [RT*(DT+1)][256 lanes]
  const int gl = gw * 64 + lane;
  if (grp == 1) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      xo[(rt * (DT + 1)) * 256 + gl] = f32x4{mref[rt], lrun[rt], 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) xo[(rt * (DT + 1) + 1 + dt) * 256 + gl] = O[rt][dt];
    }
  }
  __syncthreads();
  if (grp == 1) return;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const f32x4 ml1 = xo[(rt * (DT + 1)) * 256 + gl];
    const float M = fmaxf(mref[rt], ml1[0]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    const float s0 = fast_exp2(mref[rt] - Mu), s1 = fast_exp2(ml1[0] - Mu);
    lrun[rt] = lrun[rt] * s0 + ml1[1] * s1;
    mref[rt] = M;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const f32x4 o1 = xo[(rt * (DT + 1) + 1 + dt) * 256 + gl];
#pragma unroll
      for (int i = 0; i < 4; ++i) O[rt][dt][i] = O[rt][dt][i] * s0 + o1[i] * s1;
    }
  }

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float l = lrun[rt];
    l += xor_shfl(l, 16);
    l += xor_shfl(l, 32);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    // largest |o| of the row (its D columns: this lane's tiles, then the
    // row's four lanes) for the partial's scale
    float mx = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(O[rt][dt][i]));
    mx *= inv;
    mx = fmaxf(mx, xor_shfl(mx, 16));
    mx = fmaxf(mx, xor_shfl(mx, 32));
    const int ex = partial_exp(mx);
    const int pr = prow(rt);
    if (pr >= R) continue;
    const int qi = pr / g, qh = kvh * g + pr % g;
    const size_t orow = ((size_t)qi * Hq + qh) * D;
    if (sg.splits == 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        u32x2 w;
        w[0] = pack_bf16x2(O[rt][dt][0] * inv, O[rt][dt][1] * inv);
        w[1] = pack_bf16x2(O[rt][dt][2] * inv, O[rt][dt][3] * inv);
        *reinterpret_cast<u32x2*>(sg.out + orow + 16 * dt + 4 * kb) = w;
      }
    } else {
      const float f = ldexpf(inv, -ex);
      // The row's fp16 partial goes through this wave's own LDS rows (group
      // 1's second buffer, unused after the merge; LDS operations of a wave
      // complete in order), so that each lane stores 16 contiguous bytes and
      // a row leaves as 64-byte runs rather than 8-byte pieces. The stores
      // write through the L2 (read once, by the combine kernel, from any
      // XCD). Buffer resources over this split's partials (the host keeps
      // one split's partials below 2 GiB).
      const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
          sg.ws_o + (size_t)split * m * Hq * D, (short)0, m * Hq * D * 2, kBufWord3);
      const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
          sg.ws_ml + (size_t)split * m * Hq * 4, (short)0, m * Hq * 16, kBufWord3);
      uint32_t* sr = reinterpret_cast<uint32_t*>(&lds[1][1][0][0]) + (gw * 16 + col) * kStageRow<D>;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        u32x2 w;
        w[0] = pack_f16x2(O[rt][dt][0] * f, O[rt][dt][1] * f);
        w[1] = pack_f16x2(O[rt][dt][2] * f, O[rt][dt][3] * f);
        *reinterpret_cast<u32x2*>(sr + 8 * dt + 2 * kb) = w;
      }
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
        __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(sr + 16 * c + 4 * kb),
                                               ors, (uint32_t)((orow + 32 * c + 8 * kb) * 2), 0,
                                               kStoreThrough);
      if (kb == 0)
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4, f32x4{mref[rt], l, ldexpf(1.f, ex), 0.f}), mrs,
            (uint32_t)(((size_t)qi * Hq + qh) * 16), 0, kStoreThrough);
    }
  }
}

// ---------------------------------------------------------------------------
// Decode path: few rows per KV head (m*g <= 64 packed rows), as in a
// speculative verify or a short question. Workgroup = (KV head, block of at
// most 32 packed rows, key split). The cached keys [0, P) are cut into
// splits of whole 128-key rounds; one more split holds exactly the call's
// m new keys [P, P+m). The 4 waves of a workgroup take its 32-key steps in
// turn (wave w: steps w, w+4, ...), NS steps per round, with every load of
// a round issued at once straight from global memory into MFMA operand
// registers: each workgroup has little work, so what keeps HBM busy is many
// workgroups with all their loads in flight.
//
// The new-key split reads its keys from the call's inputs: K rows directly,
// V rows transposed through LDS (zero past m). It also appends the new rows
// to the cache (K rows copied, V columns written into Vt); no other
// workgroup of the call reads those positions, so nothing waits for the
// stores. The 32-key steps use the same key order as the MFMA path (lane
// (row, kb) holds keys 8*kb .. 8*kb+7 of the step) and the four wave states
// are merged in LDS in a fixed order.
// ---------------------------------------------------------------------------
constexpr int kDecWaves = 4;
constexpr int kDecRowsPerBlock = 32;
constexpr int kDecMaxNew = 64;  // new keys per call on this path (m <= 64)

template <int D, int RT, int NS, bool ONE>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnParams prm) {
  constexpr int DC = D / 32, DT = D / 16, CPR = D / 8;
  constexpr int XO = kDecWaves * RT * (DT + 1) * 64;  // f32x4 slots: wave states
  static_assert(XO * 16 >= D * kDecMaxNew * 2, "new-row staging fits the merge area");
  __shared__ f32x4 xo[XO];

  const int L = xcd_linear(blockIdx.x, gridDim.x);
  const SegRef ref = ONE ? SegRef{0, L} : find_seg(prm, L);
  const AttnSeg& sg = prm.seg[ONE ? 0 : ref.s];
  const int S = sg.splits;
  const int split = ref.local % S;
  const int rest = ref.local / S;
  const int rb = rest % sg.row_blocks, kvh = rest / sg.row_blocks;
  const int g = prm.g, Hq = prm.Hq, Hkv = prm.Hkv, cap = prm.cap;
  const int P = sg.P, m = sg.m, R = m * g;
  const bool tail = split == S - 1;  // the new-key split (uniform)
  const int k0 = tail ? P : split * sg.split_keys;
  const int k1 = tail ? P + m : min(P, k0 + sg.split_keys);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kb = lane >> 4, col = lane & 15;
  uint16_t* Kg = const_cast<uint16_t*>(sg.K) + (size_t)kvh * cap * D;
  uint16_t* Vg = const_cast<uint16_t*>(sg.Vt) + (size_t)kvh * D * cap;
  const uint16_t* nkh = sg.nk + (size_t)kvh * D;  // new row r of this head: + r * Hkv * D
  const uint16_t* nvh = sg.nv + (size_t)kvh * D;
  const float cs = prm.c;

  // query operands (B of S^T = K Q^T): lane (col, kb) holds packed row
  // 32*rb + 16*rt + col, elements 32*dc + 8*kb .. +7
  int lim[RT], qi[RT], qh[RT];
  bool rvalid[RT];
  bf16x8 qop[RT][DC];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int pr = kDecRowsPerBlock * rb + 16 * rt + col;
    rvalid[rt] = pr < R;
    const int i = rvalid[rt] ? pr / g : 0;
    qi[rt] = i;
    qh[rt] = kvh * g + (rvalid[rt] ? pr % g : 0);
    lim[rt] = min(P + i, k1 - 1);  // last visible key of this split
    // padded rows read a live query row; their outputs are never stored
    const uint16_t* qrow = sg.q + ((size_t)i * Hq + qh[rt]) * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) qop[rt][dc] = as_bf16x8(load16(qrow + 32 * dc + 8 * kb));
  }

  // new-key split: V rows transposed into LDS (Vs[d][r], r < 64, zero past
  // m), then appended to the cache from there; K rows appended directly
  uint16_t* Vs = reinterpret_cast<uint16_t*>(xo);
  if (tail) {
    const int rows_used = (m + 31) / 32 * 32;  // the steps read up to here
    for (int c = threadIdx.x; c < rows_used * CPR; c += 256) {
      const int r = c / CPR, ch = c % CPR;
      const size_t src = (size_t)min(r, m - 1) * Hkv * D + ch * 8;
      const u32x4 v = load16(nvh + src);
      const u32x4 kr = load16(nkh + src);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Vs[(ch * 8 + 2 * e) * kDecMaxNew + r] = r < m ? (uint16_t)(v[e] & 0xFFFFu) : 0;
        Vs[(ch * 8 + 2 * e + 1) * kDecMaxNew + r] = r < m ? (uint16_t)(v[e] >> 16) : 0;
      }
      if (r < m) store16(Kg + (size_t)(P + r) * D + ch * 8, kr);
    }
    __syncthreads();
    for (int c = threadIdx.x; c < D * m; c += 256) {
      const int d = c / m, r = c % m;
      Vg[(size_t)d * cap + P + r] = Vs[d * kDecMaxNew + r];
    }
  }

  f32x4 O[RT][DT];
  float mref[RT], lrun[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    mref[rt] = -INFINITY;
    lrun[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int nsteps = (k1 - k0 + 31) / 32;
  for (int u0 = 0; wave + kDecWaves * u0 < nsteps; u0 += NS) {
    bf16x8 kop[NS][2][DC], vop[NS][DT];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      // steps past the range re-read the range's first step (discarded)
      const int st = wave + kDecWaves * (u0 + u);
      const int sst = st < nsteps ? st : 0;
      const int kbase = k0 + 32 * sst;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int key = kbase + 8 * (col >> 2) + 4 * sub + (col & 3);
        // cached keys read the store, new keys the call's rows; a key at or
        // past the split's end (the last 32-key step of the last cached
        // split when P % 32 != 0) reads the split's last row instead: its
        // score is masked, and the store at or past P is never read (the
        // new-key split writes there in this launch, and past P + m it
        // holds whatever an earlier, cut-back extend left)
        const uint16_t* krow = tail ? nkh + (size_t)min(key - P, m - 1) * Hkv * D
                                    : Kg + (size_t)min(key, k1 - 1) * D;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc)
          kop[u][sub][dc] = as_bf16x8(load16(krow + 32 * dc + 8 * kb));
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 16 * dt + col;
        if (tail) {
          vop[u][dt] = as_bf16x8(
              *reinterpret_cast<const u32x4*>(Vs + d * kDecMaxNew + 32 * sst + 8 * kb));
        } else {
          // the lane's 8 keys; value operands at or past the split's end are
          // zero (a masked key has probability 0, and 0 times a stale
          // non-finite value would still be NaN), and never read
          const int c0 = kbase + 8 * kb;
          const uint16_t* vrow = Vg + (size_t)d * cap;
          if (c0 + 8 <= k1) {
            vop[u][dt] = as_bf16x8(load16(vrow + c0));
          } else {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t lo = c0 + 2 * e < k1 ? vrow[c0 + 2 * e] : 0u;
              const uint32_t hi = c0 + 2 * e + 1 < k1 ? vrow[c0 + 2 * e + 1] : 0u;
              w[e] = lo | (hi << 16);
            }
            vop[u][dt] = as_bf16x8(w);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int st = wave + kDecWaves * (u0 + u);
      if (st >= nsteps) break;  // uniform
      const int kbase = k0 + 32 * st;
      f32x4 Sc[RT][2];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          Sc[rt][sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int dc = 0; dc < DC; ++dc)
            Sc[rt][sub] = mfma16x16x32(kop[u][sub][dc], qop[rt][dc], Sc[rt][sub]);
        }
      bool grow = false;
      float mcand[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float mx = -INFINITY;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kbase + 8 * kb + 4 * sub + i;
            const float v = (key <= lim[rt]) ? Sc[rt][sub][i] : -INFINITY;
            Sc[rt][sub][i] = v;
            mx = fmaxf(mx, v);
          }
        mx = max4_rows(mx);
        mcand[rt] = mx * cs;
        grow |= mcand[rt] > mref[rt] + 8.f;
      }
      if (__ballot(grow) != 0) {
        // only the rows that grew move their reference, so every row's
        // arithmetic depends on that row alone
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const bool up = mcand[rt] > mref[rt] + 8.f;
          const float alpha = up ? fast_exp2(mref[rt] - mcand[rt]) : 1.f;
          mref[rt] = up ? mcand[rt] : mref[rt];
          lrun[rt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) O[rt][dt][i] *= alpha;
        }
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float muse = (mref[rt] == -INFINITY) ? 0.f : mref[rt];
        float psum = lrun[rt];
        u32x4 pk;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const float p0 = fast_exp2(fmaf(Sc[rt][sub][i], cs, -muse));
            const float p1 = fast_exp2(fmaf(Sc[rt][sub][i + 1], cs, -muse));
            const uint32_t w = pack_bf16x2(p0, p1);
            pk[2 * sub + (i >> 1)] = w;
            psum = dot2_bf16(w, 0x3F803F80u, psum);  // + both bf16 values exactly
          }
        lrun[rt] = psum;
        const bf16x8 pb = as_bf16x8(pk);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) O[rt][dt] = mfma16x16x32(vop[u][dt], pb, O[rt][dt]);
      }
    }
  }

  // park the wave states (the staging area is reused: wait for every wave),
  // then merge them in wave order: wave w finishes d tiles w, w+4, ...
  if (tail) __syncthreads();
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float l = lrun[rt];
    l += xor_shfl(l, 16);
    l += xor_shfl(l, 32);
    const int base = (wave * RT + rt) * (DT + 1);
    xo[base * 64 + lane] = f32x4{mref[rt], l, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) xo[(base + 1 + dt) * 64 + lane] = O[rt][dt];
  }
  __syncthreads();
  // merged outputs of this wave's d tiles (wave w: tiles w, w+4, ...)
  constexpr int DPW = (DT + kDecWaves - 1) / kDecWaves;
  f32x4 ofin[RT][DPW];
  float Mr[RT], Lr[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float M = -INFINITY;
    float mw[kDecWaves], lw[kDecWaves];
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const f32x4 ml = xo[((w * RT + rt) * (DT + 1)) * 64 + lane];
      mw[w] = ml[0];
      lw[w] = ml[1];
      M = fmaxf(M, ml[0]);
    }
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float sw[kDecWaves], L = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      sw[w] = fast_exp2(mw[w] - Mu);
      L += sw[w] * lw[w];
    }
    Mr[rt] = M;
    Lr[rt] = L;
#pragma unroll
    for (int u = 0; u < DPW; ++u) {
      const int dt = wave + kDecWaves * u;
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
      if (dt < DT) {
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) {
          const f32x4 ow = xo[((w * RT + rt) * (DT + 1) + 1 + dt) * 64 + lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] += sw[w] * ow[i];
        }
      }
      ofin[rt][u] = o;
    }
  }
  if (S > 1) {
    // largest |o| of each row for the partial's scale: this wave's tiles,
    // the row's four lanes, then the four waves (through LDS)
    __shared__ float rmax[kDecWaves][RT][64];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float mx = 0.f;
#pragma unroll
      for (int u = 0; u < DPW; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(ofin[rt][u][i]));
      mx = fmaxf(mx, xor_shfl(mx, 16));
      mx = fmaxf(mx, xor_shfl(mx, 32));
      rmax[wave][rt][lane] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float mx = 0.f;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) mx = fmaxf(mx, rmax[w][rt][lane]);
      const float inv = Lr[rt] > 0.f ? 1.f / Lr[rt] : 0.f;
      const int ex = partial_exp(mx * inv);
      const float f = ldexpf(inv, -ex);
      if (!(rvalid[rt] && k0 <= lim[rt])) continue;
      const size_t orow = ((size_t)qi[rt] * Hq + qh[rt]) * D;
#pragma unroll
      for (int u = 0; u < DPW; ++u) {
        const int dt = wave + kDecWaves * u;
        if (dt >= DT) continue;
        u32x2 w2;
        w2[0] = pack_f16x2(ofin[rt][u][0] * f, ofin[rt][u][1] * f);
        w2[1] = pack_f16x2(ofin[rt][u][2] * f, ofin[rt][u][3] * f);
        *reinterpret_cast<u32x2*>(sg.ws_o + (size_t)split * m * Hq * D + orow + 16 * dt + 4 * kb) =
            w2;
      }
      if (wave == 0 && kb == 0)
        *reinterpret_cast<f32x4*>(sg.ws_ml + (((size_t)split * m + qi[rt]) * Hq + qh[rt]) * 4) =
            f32x4{Mr[rt], Lr[rt], ldexpf(1.f, ex), 0.f};
    }
  } else {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if (!(rvalid[rt] && k0 <= lim[rt])) continue;
      const size_t orow = ((size_t)qi[rt] * Hq + qh[rt]) * D;
      const float inv = 1.f / Lr[rt];
#pragma unroll
      for (int u = 0; u < DPW; ++u) {
        const int dt = wave + kDecWaves * u;
        if (dt >= DT) continue;
        u32x2 w2;
        w2[0] = pack_bf16x2(ofin[rt][u][0] * inv, ofin[rt][u][1] * inv);
        w2[1] = pack_bf16x2(ofin[rt][u][2] * inv, ofin[rt][u][3] * inv);
        *reinterpret_cast<u32x2*>(sg.out + orow + 16 * dt + 4 * kb) = w2;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// VALU path for short suffixes. Workgroup = (KV head, block of 16 packed rows,
// key split); its 4 waves take the 64-key tiles of the split in turn. For the
// scores a lane owns one key (dot products by v_dot2_f32_bf16 against q pairs
// broadcast from LDS); for the value product a lane owns D/64 columns of Vt
// (dot2 of bf16 probability pairs against key-adjacent V pairs). The four
// waves' partial states are merged in LDS in a fixed order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, xor_shfl(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += xor_shfl(v, o);
  return v;
}

constexpr int kValuRows = 16;

template <int D>
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnParams prm) {
  constexpr int DP = D / 2;   // bf16 pairs per row
  constexpr int DPL = D / 64; // Vt columns per lane
  __shared__ uint32_t qs[kValuRows][DP];                 // q rows, bf16 pairs
  __shared__ uint32_t ps[4][kValuRows][32];              // per wave: p pairs
  __shared__ float wm[4][kValuRows], wl[4][kValuRows];
  __shared__ float wo[4][kValuRows][D];
  __shared__ float fm[kValuRows], fl[kValuRows];  // merged (max, sum) per row

  const int L = xcd_linear(blockIdx.x, gridDim.x);
  const SegRef ref = find_seg(prm, L);
  const AttnSeg& sg = prm.seg[ref.s];
  const int split = ref.local % sg.splits;
  const int rest = ref.local / sg.splits;
  const int rb = rest % sg.row_blocks;
  const int kvh = rest / sg.row_blocks;
  const int g = prm.g, Hq = prm.Hq, cap = prm.cap;
  const int P = sg.P, m = sg.m, R = m * g;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  const int row0 = rb * kValuRows;
  const int nrows = min(kValuRows, R - row0);
  const int wg_last = row0 + nrows - 1;
  const int kstart = split * sg.split_keys;
  const int kend = min(P + wg_last / g + 1, kstart + sg.split_keys);
  if (kstart >= kend) return;

  for (int c = threadIdx.x; c < kValuRows * DP; c += 256) {
    const int r = c / DP, dp = c % DP;
    uint32_t v = 0;
    if (r < nrows) {
      const int pr = row0 + r;
      const int i = pr / g, h = kvh * g + pr % g;
      v = reinterpret_cast<const uint32_t*>(sg.q + ((size_t)i * Hq + h) * D)[dp];
    }
    qs[r][dp] = v;
  }
  __syncthreads();

  float mrun[kValuRows], lrun[kValuRows];
  float oacc[kValuRows][DPL];
#pragma unroll
  for (int r = 0; r < kValuRows; ++r) {
    mrun[r] = -INFINITY;
    lrun[r] = 0.f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) oacc[r][j] = 0.f;
  }

  const uint16_t* Kg = sg.K + (size_t)kvh * cap * D;
  const uint16_t* Vg = sg.Vt + (size_t)kvh * D * cap;
  const int kv_end = P + m;
  const float cs = prm.c;

  for (int kt = kstart + 64 * wave; kt < kend; kt += 256) {
    // scores: lane = key kt + lane
    const int key = kt + lane;
    uint32_t kr[DP];
    const uint16_t* krow = Kg + (size_t)key * D;  // key < cap always (kt + 64 <= cap)
#pragma unroll
    for (int c = 0; c < DP / 4; ++c) {
      const u32x4 v = load16(krow + 8 * c);
      kr[4 * c + 0] = v[0];
      kr[4 * c + 1] = v[1];
      kr[4 * c + 2] = v[2];
      kr[4 * c + 3] = v[3];
    }
    uint32_t vr[DPL][32];
#pragma unroll
    for (int j = 0; j < DPL; ++j) {
      const uint16_t* vrow = Vg + (size_t)(lane + 64 * j) * cap + kt;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        u32x4 v = load16(vrow + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k0 = kt + 8 * c + 2 * e;
          uint32_t w = v[e];
          if (k0 >= kv_end) w &= 0xFFFF0000u;
          if (k0 + 1 >= kv_end) w &= 0x0000FFFFu;
          vr[j][4 * c + e] = w;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kValuRows; ++r) {
      if (r < nrows) {
        float s = 0.f;
#pragma unroll
        for (int dp = 0; dp < DP; ++dp) s = dot2_bf16(kr[dp], qs[r][dp], s);
        const int pr = row0 + r;
        const int limr = P + pr / g;
        s = (key <= limr) ? s : -INFINITY;
        const float mx = wave_max(s);
        const float mnew = fmaxf(mrun[r], mx * cs);
        const float muse = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = fast_exp2(mrun[r] - muse);
        mrun[r] = mnew;
        const float p = fast_exp2(fmaf(s, cs, -muse));
        const uint32_t pw = pack_bf16x2(p, 0.f) & 0xFFFFu;
        lrun[r] = lrun[r] * alpha + bf16_to_f32(pw);
        // key-adjacent pairs of p: lane 2t holds the low half, 2t+1 the high
        const uint32_t nb = (uint32_t)__shfl_xor((int)pw, 1, 64);
        if ((lane & 1) == 0) ps[wave][r][lane >> 1] = pw | (nb << 16);
#pragma unroll
        for (int j = 0; j < DPL; ++j) oacc[r][j] *= alpha;
      }
    }
    // make this wave's p visible to all its lanes (wave-local LDS traffic)
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int r = 0; r < kValuRows; ++r) {
      if (r < nrows) {
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
          float o = oacc[r][j];
#pragma unroll
          for (int t = 0; t < 32; ++t) o = dot2_bf16(vr[j][t], ps[wave][r][t], o);
          oacc[r][j] = o;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // merge the four waves
#pragma unroll
  for (int r = 0; r < kValuRows; ++r) {
    const float l = wave_sum(lrun[r]);
    if (lane == 0) {
      wm[wave][r] = mrun[r];
      wl[wave][r] = l;
    }
#pragma unroll
    for (int j = 0; j < DPL; ++j) wo[wave][r][lane + 64 * j] = oacc[r][j];
  }
  __syncthreads();
  // merged o = O / l of each (row, column); kept in wo[0] for the partials
  for (int c = threadIdx.x; c < nrows * D; c += 256) {
    const int r = c / D, d = c % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][r]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = fast_exp2(wm[w][r] - Mu);
      o += sc * wo[w][r][d];
      l += sc * wl[w][r];
    }
    const int pr = row0 + r;
    const int i = pr / g, h = kvh * g + pr % g;
    if (sg.splits == 1) {
      reinterpret_cast<__bf16*>(sg.out)[((size_t)i * Hq + h) * D + d] = (__bf16)(o / l);
    } else {
      wo[0][r][d] = l > 0.f ? o / l : 0.f;  // only this thread reads (r, d)
      if (d == 0) {
        fm[r] = M;
        fl[r] = l;
      }
    }
  }
  if (sg.splits == 1) return;
  __syncthreads();
  // one wave per row: the row's largest |o| sets the partial's scale
  for (int r = wave; r < nrows; r += 4) {
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) mx = fmaxf(mx, fabsf(wo[0][r][lane + 64 * j]));
    mx = wave_max(mx);
    const int ex = partial_exp(mx);
    const int pr = row0 + r;
    const int i = pr / g, h = kvh * g + pr % g;
    const size_t base = (((size_t)split * m + i) * Hq + h) * D;
#pragma unroll
    for (int j = 0; j < DPL; ++j)
      sg.ws_o[base + lane + 64 * j] =
          __builtin_bit_cast(uint16_t, (_Float16)ldexpf(wo[0][r][lane + 64 * j], -ex));
    if (lane == 0)
      *reinterpret_cast<f32x4*>(sg.ws_ml + (((size_t)split * m + i) * Hq + h) * 4) =
          f32x4{fm[r], fl[r], ldexpf(1.f, ex), 0.f};
  }
}

// ---------------------------------------------------------------------------
// Split combine: out = sum_s 2^(m_s - M) l_s o_s / sum_s 2^(m_s - M) l_s over
// the splits that start at or before the row's last key (one that holds no
// key the row sees has l_s = 0 and weighs exactly 0), in split order,
// with o_s = O_s / l_s the split's normalised output (stored in fp16 times
// its scale s_s).
// grid over rows (i, h) of all pieces; 4 columns per thread.
// ---------------------------------------------------------------------------
// One wave per (row, q head), four per workgroup. Lane (chunk, part): D/4
// chunks of 4 columns times 256/D parts; part t merges splits t, t+P,
// t+2P, ... (P = 256/D), loading BATCH of them per round, and the parts are
// then merged in part order through lane shuffles. Every (row, head) is
// merged in the same fixed order whatever the launch shape.
//
// The first append_total workgroups instead append the new rows of split
// MFMA-path pieces to the store, D/32 per (KV head, 64-key tile of [P, P+m))
// (the attention kernel read them from the call's inputs, and no later work
// reads the store before this kernel ends). K rows are copied as they are;
// V columns are gathered 8 keys at a time with lanes along d (each of a
// wave's 8 loads reads 128 contiguous bytes) and leave as 16-byte Vt
// pieces, key by key in the pieces holding P or P+m.
template <int D>
__device__ void append_new_rows(const AttnParams& p, int a) {
  constexpr int CPR = D / 8, PARTS = D / 32;  // a tile's work in PARTS blocks
  int s = 0;
#pragma unroll
  for (int j = 1; j < kMaxSeg; ++j)
    if (j < p.nseg && p.seg[j].append_blocks > 0 && a >= p.seg[j].append_begin) s = j;
  const AttnSeg& sg = p.seg[s];
  a -= sg.append_begin;
  const int P = sg.P, m = sg.m, Hkv = p.Hkv, cap = p.cap;
  const int T0 = P / 64, nT = (P + m - 1) / 64 - T0 + 1;
  const int part = a % PARTS, tile = a / PARTS;
  const int kvh = tile / nT, k0 = 64 * (T0 + tile % nT);
  uint16_t* K = const_cast<uint16_t*>(sg.K) + (size_t)kvh * cap * D;
  uint16_t* Vt = const_cast<uint16_t*>(sg.Vt) + (size_t)kvh * D * cap;
  const uint16_t* nk = sg.nk + (size_t)kvh * D;
  const uint16_t* nv = sg.nv + (size_t)kvh * D;
  // one K piece and one 8-key V column piece per thread; every load first
  // and unconditionally (rows clamped into [P, P+m)), so all are in flight
  // together
  auto row = [&](int k) { return (size_t)(min(max(k, P), P + m - 1) - P) * Hkv * D; };
  const int it = threadIdx.x + 256 * part;
  const int kk = k0 + it / CPR, kc = it % CPR;
  const u32x4 kr = load16(nk + row(kk) + kc * 8);
  const int d = it % D, k8 = k0 + 8 * (it / D);
  uint32_t x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = nv[row(k8 + e) + d];
  if (kk >= P && kk < P + m) store16(K + (size_t)kk * D + kc * 8, kr);
  if (k8 + 8 <= P || k8 >= P + m) return;
  uint16_t* dst = Vt + (size_t)d * cap + k8;
  if (k8 >= P && k8 + 8 <= P + m) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = x[2 * e] | (x[2 * e + 1] << 16);
    store16(dst, w);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (k8 + e >= P && k8 + e < P + m) dst[e] = (uint16_t)x[e];
  }
}

template <int D, int BATCH, bool ONE>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnParams p) {
  constexpr int CH = D / 4, PARTS = 64 / CH;
  if ((int)blockIdx.x < p.append_total) {
    append_new_rows<D>(p, blockIdx.x);
    return;
  }
  // (grow, h): one per wave
  const int row = ((int)blockIdx.x - p.append_total) * 4 + (threadIdx.x >> 6);
  if (row >= p.total_rows * p.Hq) return;
  const int grow = row / p.Hq, h = row % p.Hq;
  int s = 0;
  if constexpr (!ONE) {
#pragma unroll
    for (int j = 1; j < kMaxSeg; ++j)
      if (j < p.nseg && grow >= p.seg[j].row_begin) s = j;
  }
  const AttnSeg& sg = p.seg[s];
  if (sg.splits == 1) return;
  const int lane = threadIdx.x & 63;
  const int c4 = (lane % CH) * 4, part = lane / CH;
  const int i = grow - sg.row_begin;
  // the splits that hold a key the row sees: the decode layout (cached
  // splits + one new-key split): all of them; otherwise those starting at or
  // before the row's last key
  int nvalid;
  if (sg.tail_split) {
    nvalid = sg.splits;
  } else if (sg.tiled) {
    // the splits whose first tile is at or before the row's last one
    const int lt = (sg.P + i) / 64;
    nvalid = 0;
#pragma unroll
    for (int n = 0; n < kMaxSplits; ++n) nvalid += (n < sg.splits) & (sg.tile_bound[n] <= lt);
  } else {
    nvalid = min(sg.splits, (sg.P + i) / sg.split_keys + 1);
  }
  const float* mlp = sg.ws_ml + ((size_t)i * p.Hq + h) * 4;
  const uint16_t* op = sg.ws_o + ((size_t)i * p.Hq + h) * D + c4;
  const size_t ml_stride = (size_t)sg.m * p.Hq * 4, o_stride = (size_t)sg.m * p.Hq * D;
  // running (max, sum, sum of weighted outputs); a split's weight is
  // 2^(m_s - M) l_s and its stored value o_s / s_s
  float M = -INFINITY, l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int b0 = 0; b0 * PARTS < nvalid; b0 += BATCH) {
    float ml[BATCH][3];  // (max, sum, scale); the fourth word is not read
    u32x2 o[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const size_t q = (size_t)min((b0 + u) * PARTS + part, nvalid - 1);
#pragma unroll
      for (int e = 0; e < 3; ++e) ml[u][e] = mlp[q * ml_stride + e];
      o[u] = *reinterpret_cast<const u32x2*>(op + q * o_stride);
    }
    // branch-free: a split past nvalid re-read the last valid one (finite
    // values) and weighs 0, so every load above is issued before any use
    float Mb = M;
#pragma unroll
    for (int u = 0; u < BATCH; ++u)
      Mb = (b0 + u) * PARTS + part < nvalid ? fmaxf(Mb, ml[u][0]) : Mb;
    const float r = (M == -INFINITY) ? 0.f : fast_exp2(M - Mb);
    l *= r;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= r;
    M = Mb;
    // a split with no key this row sees (several questions: a split inside
    // another question's rows) has max -inf and sum 0; with every split so
    // far like that, M is -inf too and the weight must still come out 0
    const float Mu = (M == -INFINITY) ? 0.f : M;
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const bool ok = (b0 + u) * PARTS + part < nvalid;
      const float sc = fast_exp2(ml[u][0] - Mu);
      const float wl = ok ? sc * ml[u][1] : 0.f;
      const float wo = ok ? wl * ml[u][2] : 0.f;
      l += wl;
      acc[0] += wo * f16_bits_to_f32(o[u][0] & 0xFFFFu);
      acc[1] += wo * f16_bits_to_f32(o[u][0] >> 16);
      acc[2] += wo * f16_bits_to_f32(o[u][1] & 0xFFFFu);
      acc[3] += wo * f16_bits_to_f32(o[u][1] >> 16);
    }
  }
  // merge the parts in order: part 0 absorbs parts 1 .. PARTS-1 (always
  // reading the other parts' own states, never a partly merged one)
  const float Mp = M, lp = l;
  const f32x4 ap = acc;
#pragma unroll
  for (int t = 1; t < PARTS; ++t) {
    const float Mt = __shfl(Mp, (lane % CH) + t * CH, 64);
    const float lt = __shfl(lp, (lane % CH) + t * CH, 64);
    f32x4 at;
#pragma unroll
    for (int e = 0; e < 4; ++e) at[e] = __shfl(ap[e], (lane % CH) + t * CH, 64);
    const float Mn = fmaxf(M, Mt);
    const float Mu = (Mn == -INFINITY) ? 0.f : Mn;
    const float r0 = fast_exp2(M - Mu), r1 = fast_exp2(Mt - Mu);
    l = l * r0 + lt * r1;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = acc[e] * r0 + at[e] * r1;
    M = Mn;
  }
  if (part != 0) return;
  const float inv = 1.f / l;
  u32x2 w;
  w[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  w[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<u32x2*>(sg.out + ((size_t)i * p.Hq + h) * D + c4) = w;
}

// KV read-back (test export): K rows and transposed-back V rows.
__global__ __launch_bounds__(256) void kv_read_kernel(const uint16_t* K, const uint16_t* Vt,
                                                      int Hkv, int D, int cap, int start, int len,
                                                      uint16_t* k_out, uint16_t* v_out) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)len * Hkv * D) return;
  const int d = (int)(t % D);
  const int h = (int)((t / D) % Hkv);
  const int i = (int)(t / ((long long)D * Hkv));
  k_out[t] = K[((size_t)h * cap + start + i) * D + d];
  v_out[t] = Vt[((size_t)h * D + d) * cap + start + i];
}

// ---------------------------------------------------------------------------
// Row-tile path: extends whose pieces have too few packed rows for 128-row
// blocks to fill the chip without key splits. Workgroup = (piece, KV head,
// block of 16*RT packed rows) over every key its rows see: no key split, no
// partials, no combine launch. Its 8 waves hold the same rows and take the
// 32-key tiles in turn (wave w: tiles w, w+8, ...), each wave with its own
// LDS part for the K rows (32 x D) and one for the Vt columns (D x 32), filled
// by direct loads (from L2 after the first workgroup of the XCD touched the
// tile): the next tile's K part is requested once this tile's scores are
// computed, its Vt part once this tile's value products are done. No
// barrier inside the key loop: the two waves of a SIMD drift freely, one's
// matrix products overlapping the other's softmax.
// Keys at or past P come from the call's rows: K rows by direct loads, V
// rows through registers, transposed into the Vt part (zero past m). The
// waves' (max, sum, output) states are merged through LDS in a fixed order,
// and the first row blocks of each KV head append the call's rows.
// ---------------------------------------------------------------------------
constexpr int kRowsWaves = 8;

// Vt part of a 32-key tile: row d holds four 16-byte chunks (8 keys each),
// chunk c at position c ^ ((d >> 2) & 3), so that one value operand read
// (16 consecutive rows, one chunk) meets 16 distinct bank groups.
__device__ __forceinline__ int vswz4(int d, int c) { return c ^ ((d >> 2) & 3); }

template <int D, int RT, bool ONE>
__global__ __launch_bounds__(512) void attn_rows_kernel(AttnParams prm) {

  constexpr int DC = D / 32;
  constexpr int DT = D / 16;
  constexpr int CPR = D / 8;          // 16-byte chunks per K row
  constexpr int ROWS = 16 * RT;
  constexpr int PART = 32 * D;        // bf16 elements of a K (or Vt) part
  constexpr int NK = PART * 2 / 1024; // 1 KB requests per part
  constexpr int KPS = 64 / CPR;       // keys per K request
  // K parts and Vt parts are separate arrays, so the compiler can tell a
  // read of one from a pending direct load into the other (with one array
  // indexed by the wave it waited for every request before the scores)
  __shared__ __attribute__((aligned(16))) uint16_t kpart[kRowsWaves][PART];
  __shared__ __attribute__((aligned(16))) uint16_t vpart[kRowsWaves][PART];
  __shared__ float wml[kRowsWaves][RT][2][64];                                // (max, sum)

  const int L = xcd_linear(blockIdx.x, gridDim.x);
  const SegRef ref = ONE ? SegRef{0, L} : find_seg(prm, L);
  const AttnSeg& sg = prm.seg[ONE ? 0 : ref.s];
  const int g = prm.g, Hq = prm.Hq, Hkv = prm.Hkv, cap = prm.cap;
  const int P = sg.P, m = sg.m, R = m * g;
  const int kvh = ref.local / sg.row_blocks;
  const int rb = ref.local - kvh * sg.row_blocks;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kb = lane >> 4, col = lane & 15;
  const int row0 = rb * ROWS;
  const int last = min(R - 1, row0 + ROWS - 1);
  const int kend = P + last / g + 1;   // the block's rows see keys [0, kend)
  const int min_lim = P + row0 / g;    // smallest last key of the block's rows
  // Keys [0, pc) come from the store in 32-key tiles from key 0 (the last one
  // cut at pc); keys [pc, kend) from the call's rows in 32-key tiles from pc.
  // pc = P, or kend when the rows were appended beforehand.
  const int pc = sg.new_tile0 >= 0 ? P : kend;
  const int ncached = (pc + 31) >> 5;
  const int ntiles = ncached + (kend > pc ? (kend - pc + 31) >> 5 : 0);
  auto tile_key = [&](int t) { return t < ncached ? 32 * t : pc + 32 * (t - ncached); };

  int lim[RT];
  bf16x8 qreg[RT][DC];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int pr = row0 + 16 * rt + col;
    lim[rt] = pr < R ? P + pr / g : 0;  // padded rows read a live query row; never stored
  }
  f32x4 O[RT][DT];
  float mref[RT], lrun[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    mref[rt] = -INFINITY;
    lrun[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const uint16_t* Kg = sg.K + (size_t)kvh * cap * D;
  const uint16_t* Vg = sg.Vt + (size_t)kvh * D * cap;
  const __amdgpu_buffer_rsrc_t krsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Kg), (short)0, cap * D * 2, kBufWord3);
  const __amdgpu_buffer_rsrc_t vrsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Vg), (short)0, D * cap * 2, kBufWord3);
  // the call's rows of this KV head (row r at r * Hkv * D); reads past row
  // m-1 return zeros
  const int new_bytes = ((m - 1) * Hkv + 1) * D * 2;
  const __amdgpu_buffer_rsrc_t nkrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(sg.nk + (size_t)kvh * D), (short)0, new_bytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t nvrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(sg.nv + (size_t)kvh * D), (short)0, new_bytes, kBufWord3);
  const float cs = prm.c;
  uint16_t* Ks = kpart[wave];
  uint16_t* Vs = vpart[wave];

  // K part of tile t: request u fills chunk positions 64u + lane (key
  // (64u + lane) / CPR of the tile, slot (64u + lane) % CPR) with the row's
  // chunk kswz(key, slot): from the store for a cached tile (stale rows past
  // pc are masked), from the call's rows for a new one (zeros past m). A
  // tile index past the last one requests nothing that lands (every offset
  // out of range), so that every tile issues the same NK requests.
  // (The swizzle is computed into a variable before each request: called
  // inside the builtin's argument list, the host compiler drops the kernel's
  // launch stub.)
  // Cached tiles and new tiles run in two loops of their own (a wave's
  // cached tiles all come first), each with one request pattern. In one
  // loop with a branch per kind, the new tiles' V registers and the cached
  // tiles' request offsets shared registers, and the compiler then waited
  // for the K requests before every cached Vt request.
  auto k_issue_store = [&](int t) {  // cached tile t, or nothing lands (t >= ncached)
    const bool live = t < ncached;
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const int pos = 64 * u + lane, key = pos / CPR, slot = pos % CPR;
      const int sw = kswz<D>(key, slot) * 8;  // (a variable: see the note above)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krsrc, (lds_void*)&Ks[512 * u], 16,
                                               live ? (key * D + sw) * 2 : (int)0x80000000,
                                               live ? 32 * t * D * 2 : 0, 0, 0);
    }
  };
  // (A new tile past the last re-reads the last one, unused: with an
  // out-of-range offset chosen per tile the compiler branched around each
  // request and lost count of them.)
  auto k_issue_new = [&](int t) {  // new tile t (clamped to the last)
    const int kt = tile_key(min(t, ntiles - 1));
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const int pos = 64 * u + lane, key = pos / CPR, slot = pos % CPR;
      const int sw = kswz<D>(key, slot) * 8;  // (a variable: see the note above)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(nkrsrc, (lds_void*)&Ks[512 * u], 16,
                                               ((kt + key - P) * Hkv * D + sw) * 2, 0, 0, 0);
    }
  };
  // (The call's V rows are taken key-major: item (key, c) = (item % 32,
  // item / 32), so that the transposed 2-byte writes of a column come from
  // adjacent lanes and meet adjacent bytes.)
  // Vt part of tile t. Cached tile: the store's 8-key chunks by direct loads
  // (request u: rows 16u .. 16u+15, lane -> row 16u + lane / 4, slot lane %
  // 4); chunks from pc on read as zeros (out of range), and the keys from pc
  // on inside the chunk holding pc are zeroed once it has landed. New tile:
  // the call's V rows into registers (vreg, zeros past m), transposed into
  // the part once they have landed. NK requests either way.
  u32x4 vreg[NK];
  const int vd = lane >> 2, vslot = lane & 3;
  const int vloc = (vd * cap + vswz4(vd, vslot) * 8) * 2;
  auto v_issue_store = [&](int t) {  // cached tile t, or nothing lands (t >= ncached)
    const bool live = t < ncached;
    const int kt = 32 * t;
    const int k8 = kt + 8 * vswz4(vd, vslot);
    const int voff = live && k8 < pc ? vloc : (int)0x80000000;
#pragma unroll
    for (int u = 0; u < NK; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrsrc, (lds_void*)&Vs[512 * u], 16, voff,
                                               live ? kt * 2 + 32 * u * cap : 0, 0, 0);
  };
  auto v_issue_new = [&](int t) {  // new tile t (clamped to the last)
    const int kt = tile_key(min(t, ntiles - 1));
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const int item = 64 * j + lane, key = item & 31, c = item >> 5;
      vreg[j] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     nvrsrc, ((kt + key - P) * Hkv * D + c * 8) * 2, 0, 0));
    }
  };
  auto v_transpose = [&]() {
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const int item = 64 * j + lane, key = item & 31, c = item >> 5;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * c + e;
        Vs[d * 32 + vswz4(d, key >> 3) * 8 + (key & 7)] =
            (uint16_t)(vreg[j][e >> 1] >> (16 * (e & 1)));
      }
    }
  };
  // the keys kt + key >= pc of the chunk holding pc (rows lane, lane + 64, ...)
  auto v_zero_tail = [&](int kt) {
    const int k0 = pc - kt;  // 1 .. 31: the tile's first key to clear
    if ((k0 & 7) == 0) return;  // (the chunk starting at pc read as zeros)
#pragma unroll
    for (int d = lane; d < D; d += 64)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e >= (k0 & 7)) Vs[d * 32 + vswz4(d, k0 >> 3) * 8 + e] = 0;
  };

  f32x4 S[RT][2];
  bf16x8 pb[RT];
  auto qk = [&]() {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) S[rt][sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 2 * DC; ++q) {
      const int dc = q >> 1, sub = q & 1;
      const int kappa = 8 * (col >> 2) + 4 * sub + (col & 3);
      const bf16x8 op = as_bf16x8(load16(Ks + kappa * D + kswz<D>(kappa, 4 * dc + kb) * 8));
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) S[rt][sub] = mfma16x16x32(op, qreg[rt][dc], S[rt][sub]);
    }
  };
  auto pv = [&]() {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = 16 * dt + col;
      const bf16x8 op = as_bf16x8(load16(Vs + d * 32 + vswz4(d, kb) * 8));
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) O[rt][dt] = mfma16x16x32(op, pb[rt], O[rt][dt]);
    }
  };
  // online softmax of a tile: mask (only tiles reaching past the smallest
  // limit), row maxima, a rescale when some row's max grew by more than 8
  // (log2 units; only the rows that grew move), bf16 probabilities
  auto softmax = [&](int kt, bool cached) {
    // a row sees keys up to its limit; a cached tile's keys stop at pc
    const int kcut = cached ? pc : 0x7FFFFFFF;
    if (kt + 31 > min_lim || kt + 31 >= kcut) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kt + 8 * kb + 4 * sub + i;
            S[rt][sub][i] = ((key <= lim[rt]) & (key < kcut)) ? S[rt][sub][i] : -INFINITY;
          }
    }
    float mcand[RT];
    bool grow = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float mx = -INFINITY;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, S[rt][sub][i]);
      mcand[rt] = max4_rows(mx) * cs;
      grow |= mcand[rt] > mref[rt] + 8.f;
    }
    if (__ballot(grow) != 0) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const bool up = mcand[rt] > mref[rt] + 8.f;
        const float alpha = up ? fast_exp2(mref[rt] - mcand[rt]) : 1.f;
        mref[rt] = up ? mcand[rt] : mref[rt];
        lrun[rt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) O[rt][dt][i] *= alpha;
      }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float muse = (mref[rt] == -INFINITY) ? 0.f : mref[rt];
      float psum = lrun[rt];
      u32x4 pk;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float p0 = fast_exp2(fmaf(S[rt][sub][i], cs, -muse));
          const float p1 = fast_exp2(fmaf(S[rt][sub][i + 1], cs, -muse));
          const uint32_t w = pack_bf16x2(p0, p1);
          pk[2 * sub + (i >> 1)] = w;
          psum = dot2_bf16(w, 0x3F803F80u, psum);  // + both bf16 values exactly
        }
      pb[rt] = as_bf16x8(pk);
      lrun[rt] = psum;
    }
  };

  const int nmine = ntiles > wave ? (ntiles - 1 - wave) / kRowsWaves + 1 : 0;
  const int nmine_c = ncached > wave ? (ncached - 1 - wave) / kRowsWaves + 1 : 0;
  // the first tile's K part (nothing lands for a wave with no tile) and the
  // queries
  if (nmine_c > 0)
    k_issue_store(wave);
  else if (nmine > 0)
    k_issue_new(wave);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int pr = row0 + 16 * rt + col;
    const bool valid = pr < R;
    const int i = valid ? pr / g : 0;
    const int qh = kvh * g + (valid ? pr % g : 0);
    const uint16_t* qrow = sg.q + ((size_t)i * Hq + qh) * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) qreg[rt][dc] = as_bf16x8(load16(qrow + 32 * dc + 8 * kb));
  }
  // the queries and the first K part in; from here on every tile issues NK
  // K requests after its scores and NK V requests after its products
  wait_vmem<0>();
  int j = 0;
  // cached tiles
  if (nmine_c > 0) {
    v_issue_store(wave);
    for (; j < nmine_c; ++j) {
      const int t = wave + kRowsWaves * j, kt = 32 * t;
      wait_vmem<NK>();  // K(t) in; Vt(t) may be in flight
      qk();
      // (every K operand read has returned before the part is refilled)
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_sched_barrier(0);
      k_issue_store(t + kRowsWaves);  // (nothing lands past the cached tiles)
      __builtin_amdgcn_sched_barrier(0);
      softmax(kt, true);
      wait_vmem<NK>();  // Vt(t) in; K(t+8) may be in flight
      if (kt + 31 >= pc) v_zero_tail(kt);
      pv();
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_sched_barrier(0);
      v_issue_store(t + kRowsWaves);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the requests past the last cached tile landed nothing; the first new
    // tile's K part follows
    wait_vmem<0>();
    if (j < nmine) k_issue_new(wave + kRowsWaves * j);
  }
  // new tiles (the call's rows)
  if (j < nmine) {
    v_issue_new(wave + kRowsWaves * j);
    for (; j < nmine; ++j) {
      const int t = wave + kRowsWaves * j, kt = tile_key(t);
      wait_vmem<NK>();  // K(t) in; V(t) may be in flight
      qk();
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_sched_barrier(0);
      k_issue_new(t + kRowsWaves);  // (past the last tile: the last re-read, unused)
      __builtin_amdgcn_sched_barrier(0);
      softmax(kt, false);
      wait_vmem<NK>();  // V(t) in; K(t+8) may be in flight
      v_transpose();
      pv();
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_sched_barrier(0);
      v_issue_new(t + kRowsWaves);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // the requests for the tile past the last one: nothing lands, but they
  // must have completed before LDS is reused
  wait_vmem<0>();

  // merge the 8 waves (same lane = same rows and columns): each hands over
  // (max, row sum) and O; wave w then finishes column tiles w, w + 8, ...
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float l = lrun[rt];
    l += xor_shfl(l, 16);
    l += xor_shfl(l, 32);
    lrun[rt] = l;
  }
  __syncthreads();  // every wave is done with its parts
  // wave w's O: [RT][DT][64 lanes] f32x4 in the K parts (w < 4) or the Vt
  // parts (w >= 4), RT * D * 64 bytes each (at most a quarter of an array)
  auto xo = [&](int w) {
    return reinterpret_cast<f32x4*>(w < kRowsWaves / 2 ? &kpart[0][0] : &vpart[0][0]) +
           (w % (kRowsWaves / 2)) * RT * DT * 64;
  };
  static_assert(kRowsWaves / 2 * RT * DT * 64 * 16 <= kRowsWaves * PART * 2, "merge area");
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    wml[wave][rt][0][lane] = mref[rt];
    wml[wave][rt][1][lane] = lrun[rt];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) xo(wave)[(rt * DT + dt) * 64 + lane] = O[rt][dt];
  }
  __syncthreads();
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int pr = row0 + 16 * rt + col;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kRowsWaves; ++w) M = fmaxf(M, wml[w][rt][0][lane]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float sw[kRowsWaves], Lt = 0.f;
#pragma unroll
    for (int w = 0; w < kRowsWaves; ++w) {
      sw[w] = fast_exp2(wml[w][rt][0][lane] - Mu);
      Lt += wml[w][rt][1][lane] * sw[w];
    }
    const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
    if (pr >= R) continue;
    const size_t orow = ((size_t)(pr / g) * Hq + kvh * g + pr % g) * D;
    for (int dt = wave; dt < DT; dt += kRowsWaves) {
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kRowsWaves; ++w) {
        const f32x4 ow = xo(w)[(rt * DT + dt) * 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] += sw[w] * ow[i];
      }
      u32x2 w2;
      w2[0] = pack_bf16x2(o[0] * inv, o[1] * inv);
      w2[1] = pack_bf16x2(o[2] * inv, o[3] * inv);
      *reinterpret_cast<u32x2*>(sg.out + orow + 16 * dt + 4 * kb) = w2;
    }
  }

  // Append the call's rows [P, P+m) of this KV head (row blocks rb < A take
  // the 64-key tiles T0 + rb, T0 + rb + A, ... of the range). K rows are
  // copied; V rows go through LDS as [key][D + 2] (odd dword stride: the
  // column reads below meet distinct banks) and leave as 16-byte pieces of 8
  // keys of one column, key by key in the pieces holding P or P+m. No
  // workgroup of the call reads these positions except inside the 8-key
  // chunk holding P, whose values at or past P it replaces in LDS.
  const int A = min(sg.row_blocks, kAppendBlocks);
  if (sg.new_tile0 >= 0 && !sg.no_append && rb < A) {
    constexpr int VST = D + 2;
    uint16_t* Va = &kpart[0][0];  // [64][VST]
    static_assert(64 * VST <= kRowsWaves * PART, "append staging area");
    uint16_t* Kw = const_cast<uint16_t*>(Kg);
    uint16_t* Vw = const_cast<uint16_t*>(Vg);
    const uint16_t* nkh = sg.nk + (size_t)kvh * D;
    const uint16_t* nvh = sg.nv + (size_t)kvh * D;
    const int wt = threadIdx.x;
    const int T0 = P / 64, T1 = (P + m - 1) / 64;
    __syncthreads();  // the merge's reads of LDS are done
    for (int T = T0 + rb; T <= T1; T += A) {
      for (int it = wt; it < 64 * CPR; it += 512) {
        const int key = it / CPR, c = it % CPR, k = 64 * T + key;
        if (k >= P && k < P + m) {
          const size_t src = (size_t)(k - P) * Hkv * D + c * 8;
          store16(Kw + (size_t)k * D + c * 8, load16(nkh + src));
          const u32x4 v = load16(nvh + src);
          uint32_t* row = reinterpret_cast<uint32_t*>(Va + key * VST + c * 8);
#pragma unroll
          for (int e = 0; e < 4; ++e) row[e] = v[e];
        }
      }
      __syncthreads();
      for (int it = wt; it < D * 8; it += 512) {
        const int j8 = it & 7, d = it >> 3, k8 = 64 * T + 8 * j8;
        if (k8 + 8 <= P || k8 >= P + m) continue;
        uint16_t x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = Va[(8 * j8 + e) * VST + d];
        uint16_t* dst = Vw + (size_t)d * cap + k8;
        if (k8 >= P && k8 + 8 <= P + m) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = (uint32_t)x[2 * e] | ((uint32_t)x[2 * e + 1] << 16);
          store16(dst, w);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (k8 + e >= P && k8 + e < P + m) dst[e] = x[e];
        }
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

int attn_rows_per_block(int path) {
  return path == kPathValu ? kValuRows : path == kPathDecode ? kDecRowsPerBlock : 64 * 2;
}

template <int D, bool ONE>
static void launch_rows(const AttnParams& p, hipStream_t st) {
  if (p.rows_rt == 1)
    hipLaunchKernelGGL((attn_rows_kernel<D, 1, ONE>), dim3(p.total_blocks), dim3(64 * kRowsWaves),
                       0, st, p);
  else
    hipLaunchKernelGGL((attn_rows_kernel<D, 2, ONE>), dim3(p.total_blocks), dim3(64 * kRowsWaves),
                       0, st, p);
}

hipError_t launch_kv_append(const AttnParams& p, hipStream_t st) {
  int maxm = 0;
  for (int s = 0; s < p.nseg; ++s) maxm = p.seg[s].m > maxm ? p.seg[s].m : maxm;
  if (maxm == 0) return hipSuccess;
  const dim3 grid((maxm + kAppendRows - 1) / kAppendRows, p.Hkv, p.nseg);
  if (p.D == 128)
    hipLaunchKernelGGL(kv_append_kernel<128>, grid, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(kv_append_kernel<64>, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

template <int D, bool ONE>
static void launch_decode(const AttnParams& p, int rt, int ns, hipStream_t st) {
  const dim3 grid(p.total_blocks), block(256);
  switch (rt * 2 + ns) {
    case 3: hipLaunchKernelGGL((attn_decode_kernel<D, 1, 1, ONE>), grid, block, 0, st, p); break;
    case 4: hipLaunchKernelGGL((attn_decode_kernel<D, 1, 2, ONE>), grid, block, 0, st, p); break;
    case 5: hipLaunchKernelGGL((attn_decode_kernel<D, 2, 1, ONE>), grid, block, 0, st, p); break;
    default: hipLaunchKernelGGL((attn_decode_kernel<D, 2, 2, ONE>), grid, block, 0, st, p); break;
  }
}

template <int D, bool ONE>
static void launch_mfma(const AttnParams& p, hipStream_t st) {
  // several questions about one state: the variant with the question band
  // (always a single piece list)
  if (ONE && p.seg[0].nq > 1)
    hipLaunchKernelGGL((attn_mfma_kernel<D, 2, true, true>), dim3(p.total_blocks), dim3(512), 0,
                       st, p);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<D, 2, ONE, false>), dim3(p.total_blocks), dim3(512), 0,
                       st, p);
}

template <int D, bool ONE>
static void launch_combine(const AttnParams& p, bool wide, hipStream_t st) {
  const int blocks = p.append_total + (p.total_rows * p.Hq + 3) / 4;
  if (wide)
    hipLaunchKernelGGL((attn_combine_kernel<D, 16, ONE>), dim3(blocks), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((attn_combine_kernel<D, 4, ONE>), dim3(blocks), dim3(256), 0, st, p);
}

hipError_t launch_attn(const AttnParams& p, int path, hipStream_t st) {
  if (p.total_blocks == 0) return hipSuccess;
  const dim3 grid(p.total_blocks), block(256);
  if (path == kPathDecode) {
    const bool one = p.nseg == 1;
    if (p.D == 128)
      one ? launch_decode<128, true>(p, p.dec_rt, p.dec_ns, st)
          : launch_decode<128, false>(p, p.dec_rt, p.dec_ns, st);
    else
      one ? launch_decode<64, true>(p, p.dec_rt, p.dec_ns, st)
          : launch_decode<64, false>(p, p.dec_rt, p.dec_ns, st);
  } else if (path == kPathValu) {
    if (p.D == 128)
      hipLaunchKernelGGL(attn_valu_kernel<128>, grid, block, 0, st, p);
    else
      hipLaunchKernelGGL(attn_valu_kernel<64>, grid, block, 0, st, p);
  } else if (path == kPathRows) {
    const bool one = p.nseg == 1;
    if (p.D == 128)
      one ? launch_rows<128, true>(p, st) : launch_rows<128, false>(p, st);
    else
      one ? launch_rows<64, true>(p, st) : launch_rows<64, false>(p, st);
  } else {
    const bool one = p.nseg == 1;
    if (p.D == 128)
      one ? launch_mfma<128, true>(p, st) : launch_mfma<128, false>(p, st);
    else
      one ? launch_mfma<64, true>(p, st) : launch_mfma<64, false>(p, st);
  }
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnParams& p, hipStream_t st) {
  bool any = false;
  for (int s = 0; s < p.nseg; ++s) any |= p.seg[s].splits > 1 && p.seg[s].m > 0;
  if (!any) return hipSuccess;
  int max_s = 0;
  for (int s = 0; s < p.nseg; ++s) max_s = p.seg[s].splits > max_s ? p.seg[s].splits : max_s;
  // splits loaded per part and round: few splits -> short rounds
  const bool wide = max_s > (p.D == 128 ? 8 : 16);
  const bool one = p.nseg == 1;
  if (p.D == 128)
    one ? launch_combine<128, true>(p, wide, st) : launch_combine<128, false>(p, wide, st);
  else
    one ? launch_combine<64, true>(p, wide, st) : launch_combine<64, false>(p, wide, st);
  return hipGetLastError();
}

hipError_t launch_kv_read(const uint16_t* K, const uint16_t* Vt, int Hkv, int D, int cap,
                          int start, int len, uint16_t* k_out, uint16_t* v_out, hipStream_t st) {
  const long long total = (long long)len * Hkv * D;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_read_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, K,
                     Vt, Hkv, D, cap, start, len, k_out, v_out);
  return hipGetLastError();
}

}  // namespace sve
