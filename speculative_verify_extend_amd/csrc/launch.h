// Host-side launchers of the gfx950 kernels (internal to libsve).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sve {

// ---- int4 weights -----------------------------------------------------------
size_t w4_packed_bytes(int N, int K);
hipError_t launch_w4_pack(const uint8_t* w, const uint16_t* s, int N, int K, void* packed,
                          hipStream_t st);
hipError_t launch_w4_dequant(const void* packed, int N, int K, float* out, hipStream_t st);
hipError_t launch_w4_gemv(const void* x, int m, const void* packed, int N, int K, float* y,
                          hipStream_t st, int wgs_per_cu);
// many-row GEMM: workspace of w4_gemm_workspace_bytes(m, N, K) bytes (0:
// unused) for the k splits' partial results
int w4_gemm_splits(int m, int N, int K);
size_t w4_gemm_workspace_bytes(int m, int N, int K);
hipError_t launch_w4_gemm(const void* x, int m, const void* packed, int N, int K, float* y,
                          void* ws, hipStream_t st);
hipError_t launch_w4_gemv_routed(const void* x, int x_per_slot, int m, const int32_t* ids,
                                 int topk, const void* packed_all, int E, int N, int K, float* y,
                                 hipStream_t st);

// ---- attention ------------------------------------------------------------------
constexpr int kMaxSeg = 4;
constexpr int kMaxSplits = 16;  // key splits per piece (workspace: kMaxSplits x max_rows rows)
constexpr int kMaxQuestions = 16;

// One (slot, layer) piece of an extend call. The KV store of a slot and layer
// is K [Hkv][cap][D] followed by Vt [Hkv][D][cap] (bf16).
struct AttnSeg {
  const uint16_t* K;
  const uint16_t* Vt;
  const uint16_t* q;   // [m][Hq][D]
  const uint16_t* nk;  // new rows [m][Hkv][D]
  const uint16_t* nv;
  uint16_t* out;       // [m][Hq][D]
  // split partials (this piece's part of the workspace): the split's
  // normalised output o = O / l in fp16, divided by the power of two s
  // (s = 1 unless the row's largest |o| reaches 2^15), and per (split, row,
  // head) the running max m (log2 units), the sum l and s
  uint16_t* ws_o;      // [splits][m][Hq][D] fp16
  float* ws_ml;        // [splits][m][Hq][4]: m, l, s, 0
  int P, m;
  int row_blocks;      // per KV head
  int splits, split_keys;
  int tail_split;      // decode layout: splits-1 cached splits of split_keys, then [P, P+m)
  // MFMA path (tiled = 1): head_blocks workgroups per KV head, split-major;
  // split s holds the 64-key tiles [tile_bound[s], tile_bound[s+1]) (key
  // [64t, 64t+64) is tile t), and a row block has a workgroup for a split
  // only when one of its rows sees a key there. tiled = 0 (other paths):
  // split s holds the keys [s, s+1) * split_keys.
  int head_blocks;
  int tiled;
  int tile_bound[kMaxSplits + 1];
  // MFMA path: first 64-key tile [64t, 64t+64) that holds new keys (P / 64).
  // With new_tile0 >= 0 the attention kernel reads keys at or past P from
  // nk/nv (tiles from new_tile0 on); the rows are appended by the combine
  // kernel's first append_blocks workgroups (D / 32 per KV head and 64-key
  // tile of [P, P+m)), or, for an unsplit piece (append_blocks 0), by the
  // attention kernel. -1: every key is in the store, appended beforehand.
  int new_tile0;
  int append_blocks, append_begin;
  // several questions on one prefix (MFMA path): the m rows are nq
  // questions starting at rows qstart[0] = 0 < qstart[1] < ...; a row sees
  // the prefix [0, P) and the rows of its own question up to itself, and
  // nothing is appended. nq <= 1: an ordinary extend.
  int nq;
  // 1: the call only reads the store (several questions, any nq): no kernel
  // appends the piece's rows, and every key at or past P comes from nk/nv
  int no_append;
  int qstart[kMaxQuestions];
  int block_begin;     // first linear workgroup of this piece
  int row_begin;       // first output row of this piece in a combined launch
};

struct AttnParams {
  AttnSeg seg[kMaxSeg];
  int nseg;
  int Hq, Hkv, g, D, cap;
  int total_blocks;
  int total_rows;      // sum of m over pieces
  int append_total;    // combine-kernel append workgroups (before the combine's own)
  float c;             // log2(e) / sqrt(D)
  int dec_rt, dec_ns;  // decode path: 16-row tiles per block (1, 2), steps per round (1, 2)
  int rows_rt;         // row-tile path: 16-row tiles per block (1, 2)
};

enum AttnPath { kPathValu = 0, kPathMfma = 1, kPathDecode = 2, kPathRows = 3 };

// rows of packed (query row, head-in-group) per workgroup for each path
int attn_rows_per_block(int path);
hipError_t launch_kv_append(const AttnParams& p, hipStream_t st);
hipError_t launch_attn(const AttnParams& p, int path, hipStream_t st);
hipError_t launch_attn_combine(const AttnParams& p, hipStream_t st);
// copy rows [start, start+len) of one slot/layer back to [len][Hkv][D] (test export)
hipError_t launch_kv_read(const uint16_t* K, const uint16_t* Vt, int Hkv, int D, int cap,
                          int start, int len, uint16_t* k_out, uint16_t* v_out, hipStream_t st);

// ---- speculative verify -------------------------------------------------------------
constexpr int kVerifyMaxRows = 16;
size_t verify_workspace_bytes(int m, int V);
hipError_t launch_verify_accept(const float* logits, int m, int V, const int32_t* draft,
                                int32_t* result, void* workspace, hipStream_t st);
// the same kernels over the library's static per-GPU scratch array (no
// allocation, no workspace argument); V <= kVerifyNoAllocMaxV
constexpr int kVerifyNoAllocMaxV = 1 << 20;
hipError_t launch_verify_accept_noalloc(const float* logits, int m, int V, const int32_t* draft,
                                        int32_t* result, hipStream_t st);

// ---- measurement probes ------------------------------------------------------------
// mode 0: plain loads, 1: nontemporal loads, 2: direct global-to-LDS loads
hipError_t launch_probe_read(const void* src, size_t bytes, int blocks, int threads, int unroll,
                             int mode, void* sink, hipStream_t st);
// kind 0: MFMA 16x16x32 bf16, 1: MFMA 32x32x16 bf16, 2: MFMA 16x16x32 f16,
// 3: v_exp_f32, 4: LDS reads of 16 bytes
hipError_t launch_probe_compute(int kind, int blocks, int iters, void* sink, hipStream_t st);
hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t st);

// ---- slot matcher ----------------------------------------------------------------
constexpr int kMaxLcpPairs = 16;
struct LcpArgs {
  const int32_t* a[kMaxLcpPairs];
  const int32_t* b[kMaxLcpPairs];
  int n[kMaxLcpPairs];
  int npairs;
  int32_t* out;
};
hipError_t launch_lcp(const LcpArgs& args, hipStream_t st);

}  // namespace sve
