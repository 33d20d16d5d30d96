// libsve host side: the C ABI declared in include/sve.h.
//
// The context owns only host metadata (cached lengths, selected prompts'
// lengths, LRU ticks). Device memory is the caller's arena:
//   [prompt tokens: cap int32][slot token mirrors: 4 x cap int32][LCP out]
//   [split workspace: partial o fp16, (max, sum, scale) fp32][slot 0][slot 1]...
// and each slot holds n_layers x { K [Hkv][cap][D], Vt [Hkv][D][cap] } bf16.
#include "sve.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "launch.h"

using namespace sve;

namespace {

constexpr int kMaxDecodeSplits = 64;
// the GEMVs address x through 32-bit buffer offsets: 256 rows of K bf16
constexpr int kMaxGemvK = 1 << 22;
static_assert(SVE_VERIFY_NOALLOC_MAX_V == kVerifyNoAllocMaxV, "header and kernels agree");
constexpr size_t kAlign = 256;
thread_local std::string g_err;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  int cap;
  size_t off_tok, off_slot_tok, off_lcp, off_ws_o, off_ws_ml, fixed, layer_bytes, slot_bytes;
};

bool config_ok(const sve_config* c, std::string* why) {
  if (!c) return *why = "null config", false;
  if (c->n_slots < 1 || c->n_slots > SVE_MAX_SLOTS) return *why = "n_slots must be 1..4", false;
  if (c->n_layers < 1) return *why = "n_layers must be >= 1", false;
  if (c->n_kv_heads < 1 || c->n_q_heads < 1 || c->n_q_heads % c->n_kv_heads)
    return *why = "n_q_heads must be a positive multiple of n_kv_heads", false;
  if (c->head_dim != 64 && c->head_dim != 128) return *why = "head_dim must be 64 or 128", false;
  if (c->capacity < 1 || c->capacity > (1 << 20)) return *why = "capacity out of range", false;
  if (c->max_rows < 1 || c->max_rows > SVE_MAX_SLOTS * c->capacity)
    return *why = "max_rows must be 1..4*capacity", false;
  if ((size_t)c->max_rows * c->n_q_heads * c->head_dim * 2 >= ((size_t)1 << 31))
    return *why = "max_rows * n_q_heads * head_dim * 2 must stay below 2 GiB", false;
  if (c->match_rule != 0 && c->match_rule != 1) return *why = "match_rule must be 0 or 1", false;
  return true;
}

Layout make_layout(const sve_config* c) {
  Layout L;
  L.cap = (c->capacity + 63) / 64 * 64;
  size_t off = 0;
  L.off_tok = off;
  off += align_up((size_t)L.cap * 4);
  L.off_slot_tok = off;
  off += align_up((size_t)SVE_MAX_SLOTS * L.cap * 4);
  L.off_lcp = off;
  off += align_up((size_t)kMaxLcpPairs * 4);
  L.off_ws_o = off;
  off += align_up((size_t)kMaxSplits * c->max_rows * c->n_q_heads * c->head_dim * 2);
  L.off_ws_ml = off;
  off += align_up((size_t)kMaxSplits * c->max_rows * c->n_q_heads * 4 * 4);
  L.fixed = off;
  L.layer_bytes = align_up((size_t)2 * c->n_kv_heads * L.cap * c->head_dim * 2);
  L.slot_bytes = (size_t)c->n_layers * L.layer_bytes;
  return L;
}

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  return atoi(v);
}

bool log_on() { return env_int("SVE_LOG", 0) != 0; }

}  // namespace

struct sve_ctx {
  sve_config cfg;
  Layout lay;
  int granted;
  hipStream_t stream;
  uint8_t* arena;
  size_t arena_bytes;
  std::vector<std::vector<int>> kv_len;  // [slot][layer]
  std::vector<int> committed;            // length of the prompt selected into the slot
  std::vector<long long> tick;
  long long clock;
  std::string err;
  // kernel timing: 4 events per timed extend call (before the KV append,
  // after it, after the attention kernel, after the combine kernel)
  std::vector<hipEvent_t> tev;
  // per timed call: bit k set when kernel k (append, attention, combine) ran
  std::vector<uint8_t> tran;
  int timed_max = 0, timed_used = 0;

  int32_t* tok() { return (int32_t*)(arena + lay.off_tok); }
  int32_t* slot_tok(int s) { return (int32_t*)(arena + lay.off_slot_tok) + (size_t)s * lay.cap; }
  int32_t* lcp_out() { return (int32_t*)(arena + lay.off_lcp); }
  uint16_t* ws_o() { return (uint16_t*)(arena + lay.off_ws_o); }
  float* ws_ml() { return (float*)(arena + lay.off_ws_ml); }
  uint16_t* kbase(int s, int l) {
    return (uint16_t*)(arena + lay.fixed + (size_t)s * lay.slot_bytes + (size_t)l * lay.layer_bytes);
  }
  uint16_t* vtbase(int s, int l) {
    return kbase(s, l) + (size_t)cfg.n_kv_heads * lay.cap * cfg.head_dim;
  }
  int resident(int s) const {
    int r = kv_len[s][0];
    for (int v : kv_len[s]) r = std::min(r, v);
    return r;
  }
};

namespace {

int fail(const sve_ctx* c, int code, const std::string& msg) {
  if (c)
    const_cast<sve_ctx*>(c)->err = msg;
  else
    g_err = msg;
  return code;
}

int hip_fail(const sve_ctx* c, hipError_t e, const char* what) {
  return fail(c, SVE_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define SVE_HIP(ctx, expr)                                 \
  do {                                                     \
    hipError_t e_ = (expr);                                \
    if (e_ != hipSuccess) return hip_fail(ctx, e_, #expr); \
  } while (0)

// MFMA path. A row block (128 packed rows) gets a workgroup for a split only
// when its last row sees a key there: for a split starting at key P + X the
// first such row block is g * X / 128 (row i sees keys up to P + i), so no
// workgroup is empty.
int mfma_first_block(int X, int g) { return X > 0 ? (int)(((long long)g * X) / 128) : 0; }

// tiles the rows of a piece see: keys [0, P + m)
int mfma_tiles(const AttnSeg& sg) { return sg.m > 0 ? (sg.P + sg.m - 1) / 64 + 1 : 0; }

// Workgroups per KV head of a piece whose split s holds tiles [b[s], b[s+1]).
int mfma_head_blocks(const AttnSeg& sg, int g, const int* b, int S) {
  int hb = 0;
  for (int s = 0; s < S; ++s) hb += sg.row_blocks - mfma_first_block(64 * b[s] - sg.P, g);
  return hb;
}

// Uniform layout: split s holds tiles [s, s+1) * tps. Returns the split count.
int bounds_uniform(const AttnSeg& sg, int tps, int* b) {
  const int T = mfma_tiles(sg), S = (T + tps - 1) / tps;
  for (int s = 0; s <= S; ++s) b[s] = std::min(s * tps, T);
  return S;
}

// Cached/new layout: S1 pieces cut the cached tiles [0, nt0) evenly, then
// pieces of tpn tiles hold the tiles from nt0 on (the new keys).
int bounds_cn(const AttnSeg& sg, int nt0, int S1, int tpn, int* b) {
  const int T = mfma_tiles(sg);
  nt0 = std::min(std::max(nt0, 0), T);
  S1 = nt0 > 0 ? std::max(1, std::min(S1, nt0)) : 0;
  int S = 0;
  for (int s = 0; s < S1; ++s) b[S++] = s * nt0 / S1;
  for (int t = nt0; t < T && S < kMaxSplits + 1; t += tpn) b[S++] = t;
  b[std::min(S, kMaxSplits)] = T;
  return S;
}

// Estimated time (us), from the kernel's start, of the slowest workgroup of
// a piece with `cached` tiles in the staged loop and `fresh` tiles in the
// new-key epilogue, fitted to per-workgroup timestamps of the replay's turn
// 9: arguments, query loads and the first tile, then 0.85 per tile (the two
// key groups share them), the epilogue's first round (which waits for the
// call's rows) and its later tiles, the merge and the partial stores. A
// piece of new tiles only skips the staged loop's first wait.
double mfma_piece_us(int cached, int fresh) {
  if (cached == 0) return 7.4 + 1.6 * fresh;
  return 8.9 + 0.85 * cached + (fresh > 0 ? 2.55 + 1.4 * (fresh - 1) : 0.0);
}

// cost of a piece of tiles [a, e) when tiles from nt0 on are new (nt0 < 0:
// every tile is in the store)
double mfma_span_us(int a, int e, int nt0) {
  const int cached = nt0 < 0 ? e - a : std::max(0, std::min(e, nt0) - a);
  return mfma_piece_us(cached, e - a - cached);
}

// Balanced layout: from the first tile on, each piece takes tiles while its
// estimated time stays within tau (at least one tile). Returns the split
// count, kMaxSplits + 1 if more pieces would be needed.
int bounds_balanced(const AttnSeg& sg, int nt0, double tau, int* b) {
  const int T = mfma_tiles(sg);
  int S = 0, t = 0;
  while (t < T) {
    if (S == kMaxSplits) return kMaxSplits + 1;
    b[S++] = t;
    int e = t + 1;
    while (e < T && mfma_span_us(t, e + 1, nt0) <= tau) ++e;
    t = e;
  }
  b[S] = T;
  return S;
}

int plan_mfma(sve_ctx* c, AttnParams& p) {
  constexpr int kTarget = 256;  // one workgroup per CU (128 KB of LDS each)
  const int g = p.g;
  // the attention kernel reads the new rows from the call's inputs; they
  // are appended by the combine kernel (split pieces) or by the attention
  // kernel itself (unsplit pieces)
  const bool fused = env_int("SVE_FUSED_APPEND", 1) != 0;
  const int forced = env_int("SVE_KV_SPLIT", 0);
  // SVE_ATTN_LAYOUT: 0 chooses (below), 1 the uniform layout, 2 the
  // cached/new one, 3 balanced pieces
  const int layout = forced > 0 ? 1 : env_int("SVE_ATTN_LAYOUT", 0);
  int nt0[kMaxSeg];
  for (int s = 0; s < p.nseg; ++s)  // questions read their rows from the inputs
    nt0[s] = (fused || p.seg[s].no_append) ? p.seg[s].P / 64 : -1;
  int bnd[kMaxSeg][kMaxSplits + 1];
  int S[kMaxSeg];
  auto blocks_of = [&]() {
    long long wg = 0;
    for (int s = 0; s < p.nseg; ++s) wg += (long long)p.Hkv * mfma_head_blocks(p.seg[s], g, bnd[s], S[s]);
    return wg;
  };
  auto worst_of = [&]() {
    double w = 0;
    for (int s = 0; s < p.nseg; ++s)
      for (int n = 0; n < S[s]; ++n) w = std::max(w, mfma_span_us(bnd[s][n], bnd[s][n + 1], nt0[s]));
    return w;
  };
  int tmax = 1;
  for (int s = 0; s < p.nseg; ++s) tmax = std::max(tmax, mfma_tiles(p.seg[s]));
  // uniform layout: the fewest tiles per split that keep the grid within
  // one round (one unsplit piece when even that needs more)
  int tps = std::max(1, (tmax + kMaxSplits - 1) / kMaxSplits);
  if (forced > 0) tps = std::max(tps, (tmax + forced - 1) / forced);
  for (;; ++tps) {
    for (int s = 0; s < p.nseg; ++s) S[s] = bounds_uniform(p.seg[s], tps, bnd[s]);
    if (forced > 0 || blocks_of() <= kTarget || tps >= tmax) break;
  }
  int max_splits = 0;
  for (int s = 0; s < p.nseg; ++s) max_splits = std::max(max_splits, S[s]);
  // Choice (measured on the replay's turns): balanced pieces where the
  // uniform split has long pieces (turn 9, 7 tiles: 0.5 us faster per call);
  // the uniform split where its pieces are short (turns 2-8, 2-4 tiles:
  // balanced pieces were 0.5-1.2 us slower, the piece model misjudging
  // them) and where one unsplit piece already fills a round (the 1668-row
  // prefill: no combine, 75 us against 79 us for split pieces + combine).
  constexpr int kBalancedMinTiles = 5;
  const bool balanced =
      layout == 3 || (layout == 0 && max_splits > 1 && tps >= kBalancedMinTiles);
  if (layout == 1 || (layout == 0 && !balanced)) {
    // (the uniform tables above)
  } else if (layout == 2) {
    // the (S1, tpn) with the least estimated time
    double best = 1e30;
    int bS1 = 1, btpn = 1;
    for (int a = 1; a < kMaxSplits; ++a)
      for (int tpn = 1; tpn <= tmax; ++tpn) {
        bool ok = true;
        for (int s = 0; s < p.nseg && ok; ++s) {
          S[s] = bounds_cn(p.seg[s], nt0[s] < 0 ? mfma_tiles(p.seg[s]) : nt0[s], a, tpn, bnd[s]);
          ok = S[s] <= kMaxSplits;
        }
        if (!ok) continue;
        const double est = worst_of() * (double)((blocks_of() + kTarget - 1) / kTarget);
        if (est < best - 1e-9) {
          best = est;
          bS1 = a;
          btpn = tpn;
        }
      }
    for (int s = 0; s < p.nseg; ++s)
      S[s] = bounds_cn(p.seg[s], nt0[s] < 0 ? mfma_tiles(p.seg[s]) : nt0[s], bS1, btpn, bnd[s]);
  } else {
    // Balanced pieces: for r rounds of workgroups, the smallest per-piece
    // time tau whose pieces fit r rounds (bisection: a larger tau makes
    // fewer, longer pieces); estimated time = the slowest piece x r.
    auto build = [&](double tau) {
      for (int s = 0; s < p.nseg; ++s) {
        S[s] = bounds_balanced(p.seg[s], nt0[s], tau, bnd[s]);
        if (S[s] > kMaxSplits) return false;
      }
      return true;
    };
    double hi = 0;
    for (int s = 0; s < p.nseg; ++s) hi = std::max(hi, mfma_span_us(0, mfma_tiles(p.seg[s]), nt0[s]));
    double best = 1e30, best_tau = hi;
    long long best_wg = 0;
    for (int r = 1; r <= 4; ++r) {
      auto fits = [&](double tau) { return build(tau) && blocks_of() <= (long long)r * kTarget; };
      if (!fits(hi)) continue;
      double lo = 0.0, h = hi;
      for (int it = 0; it < 30; ++it) {
        const double mid = 0.5 * (lo + h);
        if (fits(mid))
          h = mid;
        else
          lo = mid;
      }
      build(h);
      const long long wg = blocks_of();
      const double est = worst_of() * (double)((wg + kTarget - 1) / kTarget);
      if (est < best - 1e-9 || (est < best + 1e-9 && wg < best_wg)) {
        best = est;
        best_tau = h;
        best_wg = wg;
      }
    }
    if (!build(best_tau)) {  // (cannot happen: one piece per call always fits)
      for (int s = 0; s < p.nseg; ++s) S[s] = bounds_uniform(p.seg[s], tmax, bnd[s]);
    }
  }
  long long ws_rows = 0;
  int blocks = 0, rows = 0, app = 0;
  for (int s = 0; s < p.nseg; ++s) {
    AttnSeg& sg = p.seg[s];
    sg.new_tile0 = nt0[s];
    sg.tiled = 1;
    sg.splits = std::max(S[s], 1);
    for (int n = 0; n <= kMaxSplits; ++n)
      sg.tile_bound[n] = n <= S[s] ? bnd[s][n] : bnd[s][S[s]];
    if (S[s] == 0) sg.tile_bound[1] = 0;
    sg.head_blocks = mfma_head_blocks(sg, g, bnd[s], S[s]);
    sg.split_keys = 64;  // (the tile table holds the splits)
    sg.tail_split = 0;
    sg.append_begin = app;
    sg.append_blocks = fused && !sg.no_append && sg.splits > 1 && sg.m > 0
                           ? p.Hkv * ((sg.P + sg.m - 1) / 64 - sg.P / 64 + 1) * (p.D / 32)
                           : 0;
    app += sg.append_blocks;
    sg.block_begin = blocks;
    sg.row_begin = rows;
    sg.ws_o = c->ws_o() + (size_t)ws_rows * p.Hq * p.D;
    sg.ws_ml = c->ws_ml() + (size_t)ws_rows * p.Hq * 4;
    ws_rows += (long long)sg.splits * sg.m;
    blocks += p.Hkv * sg.head_blocks;
    rows += sg.m;
  }
  p.total_blocks = blocks;
  p.total_rows = rows;
  p.append_total = app;
  if (ws_rows > (long long)kMaxSplits * c->cfg.max_rows)
    return fail(c, SVE_E_CAPACITY, "split workspace too small for this call");
  if (log_on()) {
    fprintf(stderr, "[sve] extend: path=mfma pieces=%d blocks=%d layout=%s append=%d", p.nseg,
            blocks, layout == 2 ? "cached/new" : balanced ? "balanced" : "uniform", app);
    for (int s = 0; s < p.nseg; ++s) {
      fprintf(stderr, " (P=%d m=%d tiles", p.seg[s].P, p.seg[s].m);
      for (int n = 0; n <= S[s]; ++n) fprintf(stderr, " %d", bnd[s][n]);
      fprintf(stderr, ")");
    }
    fprintf(stderr, "\n");
  }
  return SVE_OK;
}

// Row-tile path for a call: when 32-row blocks leave the chip with fewer
// than 192 workgroups (mid-size extends, such as a ~135-row turn of a 7B-like
// layer: 16-row blocks, no key splits, no combine launch). Measured on the
// agent replay (graph replays, 32 layers): 13-24% less per layer than the
// split MFMA path at turns 2-7 (134-135 new rows over 727-1399 cached), even
// at turns 8-9; the split path stays far ahead for long prefills (turn 1,
// 727 rows) and is kept from 192 workgroups on.
bool rows_fits(const AttnParams& p) {
  long long blocks32 = 0;
  for (int s = 0; s < p.nseg; ++s) blocks32 += (long long)p.Hkv * ((p.seg[s].m * p.g + 31) / 32);
  return blocks32 < 192;
}

// Row-tile path: no key splits; a workgroup covers 16 * rt packed rows of
// one KV head and every key they see. rt = 2 unless that leaves the chip
// with fewer than 192 workgroups (then 16-row blocks).
int plan_rows(sve_ctx* c, AttnParams& p) {
  const bool fused = env_int("SVE_FUSED_APPEND", 1) != 0;
  long long packed = 0;
  for (int s = 0; s < p.nseg; ++s) packed += (long long)p.Hkv * ((p.seg[s].m * p.g + 31) / 32);
  int rt = env_int("SVE_ROWS_RT", 0);
  if (rt != 1 && rt != 2) rt = packed >= 192 ? 2 : 1;
  p.rows_rt = rt;
  int blocks = 0, rows = 0;
  for (int s = 0; s < p.nseg; ++s) {
    AttnSeg& sg = p.seg[s];
    sg.row_blocks = (sg.m * p.g + 16 * rt - 1) / (16 * rt);
    sg.head_blocks = sg.row_blocks;
    sg.splits = 1;
    sg.split_keys = sg.P + sg.m;
    sg.tiled = 0;
    sg.tail_split = 0;
    sg.new_tile0 = fused ? 0 : -1;  // >= 0: keys at or past P come from the call's rows
    sg.append_blocks = 0;
    sg.append_begin = 0;
    sg.block_begin = blocks;
    sg.row_begin = rows;
    blocks += p.Hkv * sg.row_blocks;
    rows += sg.m;
  }
  p.total_blocks = blocks;
  p.total_rows = rows;
  p.append_total = 0;
  if (log_on())
    fprintf(stderr, "[sve] extend: path=rows pieces=%d blocks=%d rows/block=%d fused=%d\n", p.nseg,
            blocks, 16 * rt, (int)fused);
  return SVE_OK;
}

// Choose the path, row blocks and key splits of every piece of a call.
//   decode: every piece has at most 64 packed rows (m*g) per KV head; a
//           workgroup covers 32 packed rows and a key split of whole
//           128-key rounds (4 waves x 32 keys)
//   mfma:   longer suffixes, 128 packed rows per workgroup, 64-key tiles
//   valu:   kept for comparison (SVE_MFMA_MIN_ROWS / SVE_ATTN_PATH select it)
// Splits: as many as keep the grid near one round of workgroups, within 64
// per piece and within the split workspace (16 x max_rows rows in total).
int plan_attention(sve_ctx* c, AttnParams& p, int& path) {
  const int g = p.g;
  int max_m = 0, max_r = 0;
  for (int s = 0; s < p.nseg; ++s) {
    max_m = std::max(max_m, p.seg[s].m);
    max_r = std::max(max_r, p.seg[s].m * g);
  }
  const char* want = getenv("SVE_ATTN_PATH");
  const int mfma_min = env_int("SVE_MFMA_MIN_ROWS", -1);
  if (want && !strcmp(want, "valu"))
    path = kPathValu;
  else if (want && !strcmp(want, "mfma"))
    path = kPathMfma;
  else if (want && !strcmp(want, "rows"))
    path = kPathRows;
  else if (want && !strcmp(want, "decode"))
    path = max_r <= 64 ? kPathDecode : kPathMfma;
  else if (mfma_min > 0)
    path = (max_m >= mfma_min) ? kPathMfma : kPathValu;
  else if (max_r <= 64)
    path = kPathDecode;
  else
    path = rows_fits(p) ? kPathRows : kPathMfma;
  if (path == kPathRows) return plan_rows(c, p);
  const int rpb = attn_rows_per_block(path);
  int base = 0;
  for (int s = 0; s < p.nseg; ++s) {
    p.seg[s].row_blocks = (p.seg[s].m * g + rpb - 1) / rpb;
    base += p.Hkv * p.seg[s].row_blocks;
  }
  if (path == kPathMfma) return plan_mfma(c, p);
  const int target = path == kPathValu ? 512 : 256;
  const int unit = path == kPathDecode ? 128 : 64;  // split length granule (keys)
  const int max_splits = path == kPathDecode ? kMaxDecodeSplits : kMaxSplits;
  const int forced = env_int("SVE_KV_SPLIT", 0);
  const long long ws_cap = (long long)kMaxSplits * c->cfg.max_rows;  // workspace rows
  const bool dec = path == kPathDecode;
  // fewest splits a piece can take: a decode piece with cached keys has at
  // least one cached split and the new-key split
  auto min_splits = [&](const AttnSeg& sg) { return dec && sg.P > 0 ? 2 : 1; };
  long long ws_rows = 0;
  int blocks = 0, rows = 0;
  for (int s = 0; s < p.nseg; ++s) {
    AttnSeg& sg = p.seg[s];
    // decode: the cached keys [0, P) are split, and one more split holds
    // the new keys; other paths split all P + m keys uniformly
    const int keys = dec ? sg.P : sg.P + sg.m;
    // (whole rounds of workgroups: at most `target` workgroups in flight)
    int S = forced > 0 ? forced : target / std::max(base, 1);
    S = std::max(1, std::min(S, max_splits));
    // the pieces after this one keep the workspace rows of their fewest
    // splits (the workspace holds kMaxSplits x max_rows rows, so the fewest
    // splits of every piece always fit together)
    long long later = 0;
    for (int t = s + 1; t < p.nseg; ++t) later += (long long)min_splits(p.seg[t]) * p.seg[t].m;
    const long long room = ws_cap - ws_rows - later;
    S = (int)std::max<long long>(min_splits(sg), std::min<long long>(S, room / std::max(sg.m, 1)));
    if (dec) S = std::max(S - 1, 1);  // cached splits
    S = std::min(S, (keys + unit - 1) / unit);
    int sk = 0;
    if (keys > 0) {
      sk = (keys + S - 1) / S;
      sk = (sk + unit - 1) / unit * unit;
      S = (keys + sk - 1) / sk;
    } else {
      S = 0;
      sk = unit;
    }
    if (dec) ++S;  // + the new-key split
    sg.splits = S;
    sg.split_keys = sk;
    sg.tail_split = dec ? 1 : 0;
    sg.new_tile0 = -1;
    sg.head_blocks = sg.row_blocks * S;
    sg.tiled = 0;  // splits of split_keys keys (the combine's range rule)
    sg.append_blocks = sg.append_begin = 0;
    sg.block_begin = blocks;
    sg.row_begin = rows;
    sg.ws_o = c->ws_o() + (size_t)ws_rows * p.Hq * p.D;
    sg.ws_ml = c->ws_ml() + (size_t)ws_rows * p.Hq * 4;
    ws_rows += (long long)S * sg.m;
    blocks += p.Hkv * sg.row_blocks * S;
    rows += sg.m;
  }
  p.total_blocks = blocks;
  p.total_rows = rows;
  if (ws_rows > ws_cap) return fail(c, SVE_E_CAPACITY, "split workspace too small for this call");
  if (path == kPathDecode) {
    int max_sk = 0;
    for (int s = 0; s < p.nseg; ++s) max_sk = std::max(max_sk, p.seg[s].split_keys);
    p.dec_rt = max_r <= 16 ? 1 : 2;
    p.dec_ns = max_sk >= 256 ? 2 : 1;
  }
  if (log_on()) {
    fprintf(stderr, "[sve] extend: path=%s pieces=%d blocks=%d",
            path == kPathMfma ? "mfma" : path == kPathDecode ? "decode" : "valu", p.nseg, blocks);
    for (int s = 0; s < p.nseg; ++s)
      fprintf(stderr, " (P=%d m=%d splits=%d x %d keys)", p.seg[s].P, p.seg[s].m, p.seg[s].splits,
              p.seg[s].split_keys);
    fprintf(stderr, "\n");
  }
  return SVE_OK;
}

int run_extend(sve_ctx* c, int n, const int32_t* slots, const int32_t* ms, int layer,
               const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out) {
  const sve_config& cf = c->cfg;
  if (n < 1 || n > kMaxSeg) return fail(c, SVE_E_ARG, "batched extend takes 1..4 slots");
  if (layer < 0 || layer >= cf.n_layers) return fail(c, SVE_E_SLOT, "layer out of range");
  int total = 0;
  for (int i = 0; i < n; ++i) {
    if (slots[i] < 0 || slots[i] >= c->granted) return fail(c, SVE_E_SLOT, "slot out of range");
    for (int j = 0; j < i; ++j)
      if (slots[j] == slots[i]) return fail(c, SVE_E_ARG, "a slot appears twice in one call");
    if (ms[i] < 0) return fail(c, SVE_E_ARG, "m must be >= 0");
    const int P = c->kv_len[slots[i]][layer];
    if (P + ms[i] > c->committed[slots[i]])
      return fail(c, SVE_E_STATE, "extend past the prompt committed by the last select");
    total += ms[i];
  }
  if (total > cf.max_rows) return fail(c, SVE_E_CAPACITY, "more rows than max_rows");
  if (total == 0) return SVE_OK;
  if (!q || !k || !v || !out) return fail(c, SVE_E_ARG, "null tensor pointer");

  AttnParams p;
  memset(&p, 0, sizeof(p));
  p.Hq = cf.n_q_heads;
  p.Hkv = cf.n_kv_heads;
  p.g = p.Hq / p.Hkv;
  p.D = cf.head_dim;
  p.cap = c->lay.cap;
  p.c = (float)(1.4426950408889634 / std::sqrt((double)p.D));
  int row = 0;
  for (int i = 0; i < n; ++i) {
    if (ms[i] == 0) continue;
    AttnSeg& sg = p.seg[p.nseg++];
    sg.K = c->kbase(slots[i], layer);
    sg.Vt = c->vtbase(slots[i], layer);
    sg.q = q + (size_t)row * p.Hq * p.D;
    sg.nk = k + (size_t)row * p.Hkv * p.D;
    sg.nv = v + (size_t)row * p.Hkv * p.D;
    sg.out = out + (size_t)row * p.Hq * p.D;
    sg.P = c->kv_len[slots[i]][layer];
    sg.m = ms[i];
    row += ms[i];
  }
  int path = kPathMfma;
  if (const int rc = plan_attention(c, p, path)) return rc;
  hipEvent_t* ev = nullptr;
  uint8_t* ran = nullptr;
  if (c->timed_used < c->timed_max) {
    ev = &c->tev[4 * (size_t)c->timed_used];
    ran = &c->tran[c->timed_used++];
  }
  if (ev) SVE_HIP(c, hipEventRecord(ev[0], c->stream));
  hipError_t e = hipSuccess;
  // the decode kernel, and the MFMA kernel with new tiles, append their rows
  bool need_append = false, need_combine = false;
  for (int s = 0; s < p.nseg; ++s) {
    need_append |= path != kPathDecode && p.seg[s].new_tile0 < 0;
    need_combine |= p.seg[s].splits > 1 && p.seg[s].m > 0;
  }
  if (ran) *ran = (uint8_t)((need_append ? 1 : 0) | 2 | (need_combine ? 4 : 0));
  if (need_append) {
    e = launch_kv_append(p, c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "kv_append launch");
  }
  if (ev) SVE_HIP(c, hipEventRecord(ev[1], c->stream));
  e = launch_attn(p, path, c->stream);
  if (e != hipSuccess) return hip_fail(c, e, "extend_attn launch");
  if (ev) SVE_HIP(c, hipEventRecord(ev[2], c->stream));
  if (need_combine) {
    e = launch_attn_combine(p, c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "combine launch");
  }
  if (ev) SVE_HIP(c, hipEventRecord(ev[3], c->stream));
  for (int i = 0; i < n; ++i) c->kv_len[slots[i]][layer] += ms[i];
  return SVE_OK;
}

// Several questions on one slot's resident prefix, one MFMA launch (plus the
// combine): nothing is appended and kv_len stays.
int run_questions(sve_ctx* c, int slot, int layer, int nq, const int32_t* ms,
                  const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out) {
  const sve_config& cf = c->cfg;
  if (slot < 0 || slot >= c->granted) return fail(c, SVE_E_SLOT, "slot out of range");
  if (layer < 0 || layer >= cf.n_layers) return fail(c, SVE_E_SLOT, "layer out of range");
  if (nq < 1 || nq > kMaxQuestions) return fail(c, SVE_E_ARG, "questions must be 1..16");
  if (!ms) return fail(c, SVE_E_ARG, "null question sizes");
  long long total = 0;
  for (int j = 0; j < nq; ++j) {
    if (ms[j] < 1) return fail(c, SVE_E_ARG, "every question needs at least one row");
    total += ms[j];
  }
  if (total > cf.max_rows) return fail(c, SVE_E_CAPACITY, "more rows than max_rows");
  if (!q || !k || !v || !out) return fail(c, SVE_E_ARG, "null tensor pointer");
  AttnParams p;
  memset(&p, 0, sizeof(p));
  p.Hq = cf.n_q_heads;
  p.Hkv = cf.n_kv_heads;
  p.g = p.Hq / p.Hkv;
  p.D = cf.head_dim;
  p.cap = c->lay.cap;
  p.c = (float)(1.4426950408889634 / std::sqrt((double)p.D));
  p.nseg = 1;
  AttnSeg& sg = p.seg[0];
  sg.K = c->kbase(slot, layer);
  sg.Vt = c->vtbase(slot, layer);
  sg.q = q;
  sg.nk = k;
  sg.nv = v;
  sg.out = out;
  sg.P = c->kv_len[slot][layer];
  sg.m = (int)total;
  sg.nq = nq;
  for (int j = 0, r = 0; j < nq; r += ms[j], ++j) sg.qstart[j] = r;
  sg.no_append = 1;  // the slot is only read, whatever the number of questions
  sg.row_blocks = (sg.m * p.g + attn_rows_per_block(kPathMfma) - 1) / attn_rows_per_block(kPathMfma);
  if (const int rc = plan_mfma(c, p)) return rc;
  hipError_t e = launch_attn(p, kPathMfma, c->stream);
  if (e != hipSuccess) return hip_fail(c, e, "questions attention launch");
  e = launch_attn_combine(p, c->stream);
  if (e != hipSuccess) return hip_fail(c, e, "questions combine launch");
  return SVE_OK;
}

}  // namespace

extern "C" {

size_t sve_arena_bytes(const sve_config* cfg, int32_t n_slots) {
  std::string why;
  if (!config_ok(cfg, &why) || n_slots < 1 || n_slots > SVE_MAX_SLOTS) return 0;
  const Layout L = make_layout(cfg);
  return L.fixed + (size_t)n_slots * L.slot_bytes;
}

int sve_create(const sve_config* cfg, void* arena, size_t arena_bytes, void* hip_stream,
               sve_ctx** out, int32_t* granted_slots) {
  std::string why;
  if (!config_ok(cfg, &why)) return fail(nullptr, SVE_E_ARG, why);
  if (!arena || !out || !granted_slots) return fail(nullptr, SVE_E_ARG, "null pointer");
  if ((uintptr_t)arena % kAlign) return fail(nullptr, SVE_E_ARG, "arena must be 256-byte aligned");
  const Layout L = make_layout(cfg);
  if (arena_bytes < L.fixed + L.slot_bytes)
    return fail(nullptr, SVE_E_CAPACITY, "arena too small for one slot");
  const int granted =
      (int)std::min<size_t>((size_t)cfg->n_slots, (arena_bytes - L.fixed) / L.slot_bytes);
  sve_ctx* c = new sve_ctx();
  c->cfg = *cfg;
  c->lay = L;
  c->granted = granted;
  c->stream = (hipStream_t)hip_stream;
  c->arena = (uint8_t*)arena;
  c->arena_bytes = arena_bytes;
  c->kv_len.assign(granted, std::vector<int>(cfg->n_layers, 0));
  c->committed.assign(granted, 0);
  c->tick.assign(granted, 0);
  c->clock = 0;
  hipError_t e = hipMemsetAsync(arena, 0, L.fixed + (size_t)granted * L.slot_bytes, c->stream);
  if (e != hipSuccess) {
    delete c;
    return hip_fail(nullptr, e, "hipMemsetAsync(arena)");
  }
  if (log_on())
    fprintf(stderr, "[sve] slots requested %d, granted %d (cap %d, %zu bytes per slot)\n",
            cfg->n_slots, granted, L.cap, L.slot_bytes);
  *out = c;
  *granted_slots = granted;
  return SVE_OK;
}

int sve_destroy(sve_ctx* ctx) {
  if (!ctx) return fail(nullptr, SVE_E_ARG, "null context");
  for (hipEvent_t e : ctx->tev) (void)hipEventDestroy(e);
  delete ctx;
  return SVE_OK;
}

int sve_timing_start(sve_ctx* c, int32_t n_calls) {
  if (!c) return fail(nullptr, SVE_E_ARG, "null context");
  if (n_calls < 1 || n_calls > 65536) return fail(c, SVE_E_ARG, "n_calls must be 1..65536");
  if (c->timed_max) return fail(c, SVE_E_STATE, "timing already started");
  c->tev.assign(4 * (size_t)n_calls, nullptr);
  c->tran.assign((size_t)n_calls, 0);
  for (size_t i = 0; i < c->tev.size(); ++i) {
    // no system-scope fence at the events: a cache write-back there would be
    // timed as part of the neighbouring kernels
    hipError_t e = hipEventCreateWithFlags(&c->tev[i], hipEventDisableSystemFence);
    if (e != hipSuccess) {
      for (size_t j = 0; j < i; ++j) (void)hipEventDestroy(c->tev[j]);
      c->tev.clear();
      return hip_fail(c, e, "hipEventCreate");
    }
  }
  c->timed_max = n_calls;
  c->timed_used = 0;
  return SVE_OK;
}

int sve_timing_read(sve_ctx* c, float* append_ms, float* attn_ms, float* combine_ms,
                    int32_t* calls) {
  if (!c) return fail(nullptr, SVE_E_ARG, "null context");
  if (!append_ms || !attn_ms || !combine_ms || !calls) return fail(c, SVE_E_ARG, "null pointer");
  if (!c->timed_max) return fail(c, SVE_E_STATE, "timing was not started");
  double acc[3] = {0, 0, 0};
  hipError_t err = hipSuccess;
  if (c->timed_used > 0) err = hipEventSynchronize(c->tev[4 * (size_t)c->timed_used - 1]);
  for (int i = 0; i < c->timed_used && err == hipSuccess; ++i)
    for (int k = 0; k < 3 && err == hipSuccess; ++k) {
      // a kernel the call did not launch counts as 0: an empty event bracket
      // still reads a few microseconds on an eager stream
      if (!(c->tran[i] >> k & 1)) continue;
      float ms = 0.f;
      err = hipEventElapsedTime(&ms, c->tev[4 * (size_t)i + k], c->tev[4 * (size_t)i + k + 1]);
      acc[k] += ms;
    }
  const int used = c->timed_used;
  for (hipEvent_t e : c->tev) (void)hipEventDestroy(e);
  c->tev.clear();
  c->tran.clear();
  c->timed_max = c->timed_used = 0;
  if (err != hipSuccess) return hip_fail(c, err, "reading timing events");
  *append_ms = (float)acc[0];
  *attn_ms = (float)acc[1];
  *combine_ms = (float)acc[2];
  *calls = used;
  return SVE_OK;
}

int sve_set_stream(sve_ctx* ctx, void* hip_stream) {
  if (!ctx) return fail(nullptr, SVE_E_ARG, "null context");
  ctx->stream = (hipStream_t)hip_stream;
  return SVE_OK;
}

int sve_info(const sve_ctx* ctx, int32_t* granted_slots, int32_t* capacity) {
  if (!ctx || !granted_slots || !capacity) return fail(ctx, SVE_E_ARG, "null pointer");
  *granted_slots = ctx->granted;
  *capacity = ctx->lay.cap;
  return SVE_OK;
}

int sve_kv_slot_select(sve_ctx* c, const int32_t* tokens, int32_t n, int32_t* slot,
                       int32_t* reused) {
  if (!c) return fail(nullptr, SVE_E_ARG, "null context");
  if (!tokens || !slot || !reused) return fail(c, SVE_E_ARG, "null pointer");
  if (n < 1) return fail(c, SVE_E_ARG, "empty prompt");
  if (n > c->lay.cap) return fail(c, SVE_E_CAPACITY, "prompt longer than the slot capacity");
  const int S = c->granted;
  std::vector<int> res(S);
  for (int s = 0; s < S; ++s) res[s] = c->resident(s);

  LcpArgs a;
  memset(&a, 0, sizeof(a));
  a.out = c->lcp_out();
  int idxL[SVE_MAX_SLOTS], idxO[SVE_MAX_SLOTS][SVE_MAX_SLOTS];
  for (int s = 0; s < S; ++s) {
    idxL[s] = -1;
    for (int t = 0; t < S; ++t) idxO[s][t] = -1;
  }
  for (int s = 0; s < S; ++s) {
    if (res[s] <= 0) continue;
    idxL[s] = a.npairs;
    a.a[a.npairs] = c->tok();
    a.b[a.npairs] = c->slot_tok(s);
    a.n[a.npairs++] = std::min(n, res[s]);
  }
  for (int s = 0; s < S; ++s)
    for (int t = s + 1; t < S; ++t) {
      if (res[s] <= 0 || res[t] <= 0) continue;
      idxO[s][t] = idxO[t][s] = a.npairs;
      a.a[a.npairs] = c->slot_tok(s);
      a.b[a.npairs] = c->slot_tok(t);
      a.n[a.npairs++] = std::min(res[s], res[t]);
    }
  SVE_HIP(c, hipMemcpyAsync(c->tok(), tokens, (size_t)n * 4, hipMemcpyHostToDevice, c->stream));
  int32_t lcp[kMaxLcpPairs] = {0};
  if (a.npairs > 0) {
    SVE_HIP(c, launch_lcp(a, c->stream));
    SVE_HIP(c, hipMemcpyAsync(lcp, c->lcp_out(), (size_t)a.npairs * 4, hipMemcpyDeviceToHost,
                              c->stream));
  }
  SVE_HIP(c, hipStreamSynchronize(c->stream));

  int Ls[SVE_MAX_SLOTS], Os[SVE_MAX_SLOTS];
  int n_occ = 0;
  for (int s = 0; s < S; ++s) n_occ += res[s] > 0;
  int chosen = -1, r = 0;
  for (int s = 0; s < S; ++s) {
    Ls[s] = idxL[s] >= 0 ? lcp[idxL[s]] : 0;
    Os[s] = 0;
    for (int t = 0; t < S; ++t)
      if (t != s && idxO[s][t] >= 0) Os[s] = std::max(Os[s], lcp[idxO[s][t]]);
  }
  for (int s = 0; s < S; ++s) {
    if (res[s] <= 0 || Ls[s] <= 0 || Ls[s] <= Os[s]) continue;
    const bool lone_ok = c->cfg.match_rule == 1 || Ls[s] == res[s] || n_occ > 1;
    if (!lone_ok) continue;
    chosen = s;  // at most one slot can qualify (common-prefix lengths are ultrametric)
    r = std::min(Ls[s], n - 1);
    break;
  }
  if (chosen < 0) {  // a slot is empty until a prompt has been selected into it
    for (int s = 0; s < S; ++s)
      if (c->committed[s] == 0) {
        chosen = s;
        r = 0;
        break;
      }
  }
  if (chosen < 0) {
    chosen = 0;
    for (int s = 1; s < S; ++s)
      if (c->tick[s] < c->tick[chosen]) chosen = s;
    r = std::min(Ls[chosen], n - 1);
  }
  if (!c->cfg.reuse) r = 0;

  SVE_HIP(c, hipMemcpyAsync(c->slot_tok(chosen), c->tok(), (size_t)n * 4,
                            hipMemcpyDeviceToDevice, c->stream));
  c->tick[chosen] = ++c->clock;
  for (int& v : c->kv_len[chosen]) v = r;
  c->committed[chosen] = n;
  if (log_on())
    fprintf(stderr, "[sve] select: n=%d -> slot %d, reused %d (occupied %d)\n", n, chosen, r, n_occ);
  *slot = chosen;
  *reused = r;
  return SVE_OK;
}

int sve_kv_truncate(sve_ctx* c, int32_t slot, int32_t len) {
  if (!c) return fail(nullptr, SVE_E_ARG, "null context");
  if (slot < 0 || slot >= c->granted) return fail(c, SVE_E_SLOT, "slot out of range");
  if (len < 0 || len > c->resident(slot)) return fail(c, SVE_E_ARG, "truncate can only shorten");
  for (int& v : c->kv_len[slot]) v = len;
  return SVE_OK;
}

int sve_kv_len(const sve_ctx* c, int32_t slot, int32_t layer, int32_t* len) {
  if (!c || !len) return fail(c, SVE_E_ARG, "null pointer");
  if (slot < 0 || slot >= c->granted) return fail(c, SVE_E_SLOT, "slot out of range");
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(c, SVE_E_SLOT, "layer out of range");
  *len = c->kv_len[slot][layer];
  return SVE_OK;
}

int sve_extend_attn(sve_ctx* c, int32_t slot, int32_t layer, const void* q, const void* new_k,
                    const void* new_v, int32_t m, void* out) {
  if (!c) return fail(nullptr, SVE_E_ARG, "null context");
  return run_extend(c, 1, &slot, &m, layer, (const uint16_t*)q, (const uint16_t*)new_k,
                    (const uint16_t*)new_v, (uint16_t*)out);
}

int sve_extend_attn_batched(sve_ctx* c, int32_t n, const int32_t* slots, const int32_t* ms,
                            int32_t layer, const void* q, const void* k, const void* v,
                            void* out) {
  if (!c) return fail(nullptr, SVE_E_ARG, "null context");
  if (!slots || !ms) return fail(c, SVE_E_ARG, "null pointer");
  return run_extend(c, n, slots, ms, layer, (const uint16_t*)q, (const uint16_t*)k,
                    (const uint16_t*)v, (uint16_t*)out);
}

int sve_extend_attn_questions(sve_ctx* ctx, int32_t slot, int32_t layer, int32_t n_questions,
                              const int32_t* m_host, const void* q, const void* new_k,
                              const void* new_v, void* out) {
  if (!ctx) return fail(nullptr, SVE_E_ARG, "null context");
  return run_questions(ctx, slot, layer, n_questions, m_host, (const uint16_t*)q,
                       (const uint16_t*)new_k, (const uint16_t*)new_v, (uint16_t*)out);
}

int sve_kv_read(sve_ctx* c, int32_t slot, int32_t layer, int32_t start, int32_t len, void* k_out,
                void* v_out) {
  if (!c) return fail(nullptr, SVE_E_ARG, "null context");
  if (slot < 0 || slot >= c->granted) return fail(c, SVE_E_SLOT, "slot out of range");
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(c, SVE_E_SLOT, "layer out of range");
  if (start < 0 || len < 0 || start + len > c->kv_len[slot][layer])
    return fail(c, SVE_E_ARG, "rows outside the cached range");
  if (len > 0 && (!k_out || !v_out)) return fail(c, SVE_E_ARG, "null pointer");
  SVE_HIP(c, launch_kv_read(c->kbase(slot, layer), c->vtbase(slot, layer), c->cfg.n_kv_heads,
                            c->cfg.head_dim, c->lay.cap, start, len, (uint16_t*)k_out,
                            (uint16_t*)v_out, c->stream));
  return SVE_OK;
}

size_t sve_w4_packed_bytes(int32_t N, int32_t K) {
  if (N < 1 || K < 32 || K % 32) return 0;
  return w4_packed_bytes(N, K);
}

int sve_w4_pack(const uint8_t* w, const uint16_t* scales, int32_t N, int32_t K, void* packed,
                void* hip_stream) {
  if (N < 1 || K < 32 || K % 32) return fail(nullptr, SVE_E_ARG, "need N >= 1 and K % 32 == 0");
  if (!w || !scales || !packed) return fail(nullptr, SVE_E_ARG, "null pointer");
  SVE_HIP(nullptr, launch_w4_pack(w, scales, N, K, packed, (hipStream_t)hip_stream));
  return SVE_OK;
}

int sve_w4_dequant(const void* packed, int32_t N, int32_t K, float* out, void* hip_stream) {
  if (N < 1 || K < 32 || K % 32) return fail(nullptr, SVE_E_ARG, "need N >= 1 and K % 32 == 0");
  if (!packed || !out) return fail(nullptr, SVE_E_ARG, "null pointer");
  SVE_HIP(nullptr, launch_w4_dequant(packed, N, K, out, (hipStream_t)hip_stream));
  return SVE_OK;
}

int sve_w4_gemv_m(const void* x, int32_t m, const void* packed, int32_t N, int32_t K, float* y,
                  void* hip_stream) {
  if (m < 1 || m > 16) return fail(nullptr, SVE_E_ARG, "m must be 1..16");
  if (N < 1 || K < 32 || K % 32 || K > kMaxGemvK)
    return fail(nullptr, SVE_E_ARG, "need N >= 1, K % 32 == 0 and K <= 4194304");
  if (!x || !packed || !y) return fail(nullptr, SVE_E_ARG, "null pointer");
  SVE_HIP(nullptr, launch_w4_gemv(x, m, packed, N, K, y, (hipStream_t)hip_stream,
                                  env_int("SVE_GEMV_WGS_PER_CU", 0)));
  return SVE_OK;
}

size_t sve_w4_gemm_workspace_bytes(int32_t m, int32_t N, int32_t K) {
  if (m < 1 || N < 1 || K < 32 || K % 32) return 0;
  return w4_gemm_workspace_bytes(m, N, K);
}

int sve_w4_gemm(const void* x, int32_t m, const void* packed, int32_t N, int32_t K, float* y,
                void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (m < 1 || N < 1 || K < 32 || K % 32)
    return fail(nullptr, SVE_E_ARG, "need m >= 1, N >= 1 and K % 32 == 0");
  if ((long long)m * N > (1LL << 40) / 4 || (long long)m * K * 2 >= (1LL << 31))
    return fail(nullptr, SVE_E_ARG, "m * N or m * K too large for one call");
  if (!x || !packed || !y) return fail(nullptr, SVE_E_ARG, "null pointer");
  const size_t need = w4_gemm_workspace_bytes(m, N, K);
  if (!workspace || workspace_bytes < need)
    return fail(nullptr, SVE_E_ARG, "workspace smaller than sve_w4_gemm_workspace_bytes");
  SVE_HIP(nullptr, launch_w4_gemm(x, m, packed, N, K, y, workspace, (hipStream_t)hip_stream));
  return SVE_OK;
}

int sve_w4_gemv_m_routed(const void* x, int32_t x_per_slot, int32_t m, const int32_t* ids,
                         int32_t topk, const void* packed_all, int32_t E, int32_t N, int32_t K,
                         float* y, void* hip_stream) {
  if (m < 1 || m > 16) return fail(nullptr, SVE_E_ARG, "m must be 1..16");
  if (topk < 1 || topk > 16) return fail(nullptr, SVE_E_ARG, "topk must be 1..16");
  if (x_per_slot != 0 && x_per_slot != 1) return fail(nullptr, SVE_E_ARG, "x_per_slot is 0 or 1");
  if (E < 1 || N < 1 || K < 32 || K % 32 || K > kMaxGemvK)
    return fail(nullptr, SVE_E_ARG, "bad E, N or K (K % 32 == 0, K <= 4194304)");
  if (!x || !ids || !packed_all || !y) return fail(nullptr, SVE_E_ARG, "null pointer");
  SVE_HIP(nullptr, launch_w4_gemv_routed(x, x_per_slot, m, ids, topk, packed_all, E, N, K, y,
                                         (hipStream_t)hip_stream));
  return SVE_OK;
}

int sve_ngram_draft(const int32_t* tokens, int32_t n, int32_t k, int32_t max_ngram,
                    int32_t min_ngram, int32_t* draft, int32_t* n_draft) {
  if (n < 0 || k < 0 || k > SVE_NGRAM_MAX_DRAFT) return fail(nullptr, SVE_E_ARG, "bad n or k");
  if (min_ngram < 1 || max_ngram < min_ngram || max_ngram > 64)
    return fail(nullptr, SVE_E_ARG, "need 1 <= min_ngram <= max_ngram <= 64");
  if (!n_draft || (n > 0 && !tokens) || (k > 0 && !draft))
    return fail(nullptr, SVE_E_ARG, "null pointer");
  *n_draft = 0;
  if (k == 0) return SVE_OK;
  // longest suffix first; for each length the latest earlier start
  for (int g = std::min(max_ngram, n - 1); g >= min_ngram; --g) {
    const int32_t* suffix = tokens + (n - g);
    for (int p = n - g - 1; p >= 0; --p) {
      if (tokens[p + g - 1] != suffix[g - 1] || tokens[p] != suffix[0]) continue;
      if (std::equal(tokens + p, tokens + p + g, suffix)) {
        const int cnt = std::min(k, n - (p + g));
        std::copy(tokens + p + g, tokens + p + g + cnt, draft);
        *n_draft = cnt;
        return SVE_OK;
      }
    }
  }
  return SVE_OK;
}

size_t sve_verify_workspace_bytes(int32_t m, int32_t V) {
  if (m < 1 || m > SVE_VERIFY_MAX_ROWS || V < 1) return 0;
  return verify_workspace_bytes(m, V);
}

int sve_verify_accept(const float* logits, int32_t m, int32_t V, const int32_t* draft,
                      int32_t* result, void* workspace, size_t workspace_bytes,
                      void* hip_stream) {
  if (m < 1 || m > SVE_VERIFY_MAX_ROWS) return fail(nullptr, SVE_E_ARG, "m must be 1..16");
  if (V < 1) return fail(nullptr, SVE_E_ARG, "V must be >= 1");
  if (!logits || !result || !workspace || (m > 1 && !draft))
    return fail(nullptr, SVE_E_ARG, "null pointer");
  if (workspace_bytes < verify_workspace_bytes(m, V))
    return fail(nullptr, SVE_E_ARG, "workspace smaller than sve_verify_workspace_bytes");
  SVE_HIP(nullptr, launch_verify_accept(logits, m, V, draft, result, workspace,
                                        (hipStream_t)hip_stream));
  return SVE_OK;
}

int sve_verify_accept_noalloc(const float* logits, int32_t m, int32_t V, const int32_t* draft,
                              int32_t* result, void* hip_stream) {
  if (m < 1 || m > SVE_VERIFY_MAX_ROWS) return fail(nullptr, SVE_E_ARG, "m must be 1..16");
  if (V < 1 || V > SVE_VERIFY_NOALLOC_MAX_V)
    return fail(nullptr, SVE_E_ARG, "V must be 1..SVE_VERIFY_NOALLOC_MAX_V (static scratch size)");
  if (!logits || !result || (m > 1 && !draft)) return fail(nullptr, SVE_E_ARG, "null pointer");
  SVE_HIP(nullptr, launch_verify_accept_noalloc(logits, m, V, draft, result,
                                                (hipStream_t)hip_stream));
  return SVE_OK;
}

int sve_spec_gate_init(sve_spec_gate* g, int32_t k, double min_accept, int32_t window) {
  if (!g) return fail(nullptr, SVE_E_ARG, "null gate");
  if (k < 0 || k > SVE_VERIFY_MAX_ROWS - 1) return fail(nullptr, SVE_E_ARG, "k must be 0..15");
  if (!(min_accept >= 0.0 && min_accept <= 1.0))
    return fail(nullptr, SVE_E_ARG, "min_accept must be in [0, 1]");
  if (window < 1 || window > SVE_GATE_MAX_WINDOW)
    return fail(nullptr, SVE_E_ARG, "window must be 1..64");
  memset(g, 0, sizeof(*g));
  g->k = k;
  g->window = window;
  g->min_accept = min_accept;
  return SVE_OK;
}

int sve_spec_gate_step(sve_spec_gate* g, int32_t accepted, int32_t* k_next) {
  if (!g || !k_next) return fail(nullptr, SVE_E_ARG, "null pointer");
  if (g->window < 1 || g->window > SVE_GATE_MAX_WINDOW || g->k < 0)
    return fail(nullptr, SVE_E_ARG, "gate not initialised");
  if (g->k > 0) {
    if (accepted < 0 || accepted > g->k) return fail(nullptr, SVE_E_ARG, "accepted must be 0..k");
    g->accepted[g->steps % g->window] = accepted;
    ++g->steps;
    const int n = std::min(g->steps, g->window);
    long long sum = 0;
    for (int i = 0; i < n; ++i) sum += g->accepted[i];
    // (sum of counts) / (k * steps), one rounding
    if ((double)sum / ((double)g->k * (double)n) < g->min_accept) g->k = 0;
  }
  *k_next = g->k;
  return SVE_OK;
}

double sve_spec_break_even(double a, double b, int32_t k) {
  if (!(a + b > 0.0) || !(b >= 0.0) || k < 0) return -1.0;
  if (k == 0) return 0.0;
  auto tokens = [k](double alpha) {
    double t = 0.0;
    for (int i = 0; i <= k; ++i) t += std::pow(alpha, i);
    return t;
  };
  const double need = (a + b * (k + 1)) / (a + b);
  if (tokens(1.0) < need) return 1.0;
  double lo = 0.0, hi = 1.0;
  for (int it = 0; it < 200; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (tokens(mid) < need)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

int sve_probe_read(const void* src, size_t bytes, int32_t blocks, int32_t threads,
                   int32_t unroll, int32_t mode, void* sink, void* hip_stream) {
  if (!src || !sink || bytes == 0 || bytes % 16) return fail(nullptr, SVE_E_ARG, "bad probe buffer");
  if (blocks < 1 || blocks > 65536) return fail(nullptr, SVE_E_ARG, "blocks must be 1..65536");
  if (threads < 64 || threads > 1024 || threads % 64)
    return fail(nullptr, SVE_E_ARG, "threads must be a multiple of 64 in 64..1024");
  if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8 && unroll != 16)
    return fail(nullptr, SVE_E_ARG, "unroll must be 1, 2, 4, 8 or 16");
  if (mode < 0 || mode > 3) return fail(nullptr, SVE_E_ARG, "mode must be 0..3");
  if (mode == 3 && (bytes % 32768 || bytes > 0x7FFFFFFFu || threads > 256))
    return fail(nullptr, SVE_E_ARG,
                "cache-resident LDS mode: bytes % 32768 == 0, < 2 GiB, at most 256 threads");
  if (mode == 2 && (bytes % 1024 || bytes > 0x7FFFFFFFu ||
                    (size_t)(threads / 64) * unroll * 1024 > 160 * 1024))
    return fail(nullptr, SVE_E_ARG, "LDS mode: bytes % 1024 == 0, < 2 GiB, ring within 160 KB");
  SVE_HIP(nullptr, launch_probe_read(src, bytes, blocks, threads, unroll, mode, sink,
                                     (hipStream_t)hip_stream));
  return SVE_OK;
}

int sve_probe_compute(int32_t kind, int32_t blocks, int32_t iters, void* sink, void* hip_stream) {
  if (kind < 0 || kind > 4) return fail(nullptr, SVE_E_ARG, "kind must be 0..4");
  if (blocks < 1 || blocks > 65536 || iters < 1) return fail(nullptr, SVE_E_ARG, "bad blocks or iters");
  if (!sink) return fail(nullptr, SVE_E_ARG, "null sink");
  SVE_HIP(nullptr, launch_probe_compute(kind, blocks, iters, sink, (hipStream_t)hip_stream));
  return SVE_OK;
}

int sve_probe_copy(const void* src, void* dst, size_t bytes, int32_t blocks, void* hip_stream) {
  if (!src || !dst || bytes == 0 || bytes % 16) return fail(nullptr, SVE_E_ARG, "bad probe buffer");
  if (blocks < 1 || blocks > 65536) return fail(nullptr, SVE_E_ARG, "blocks must be 1..65536");
  SVE_HIP(nullptr, launch_probe_copy(src, dst, bytes, blocks, (hipStream_t)hip_stream));
  return SVE_OK;
}

const char* sve_strerror(int code) {
  switch (code) {
    case SVE_OK: return "ok";
    case SVE_E_ARG: return "invalid argument";
    case SVE_E_SLOT: return "slot or layer out of range";
    case SVE_E_CAPACITY: return "capacity exceeded";
    case SVE_E_HIP: return "HIP runtime error";
    case SVE_E_STATE: return "call out of order";
    default: return "unknown status";
  }
}

const char* sve_last_error(const sve_ctx* ctx) {
  return ctx ? ctx->err.c_str() : g_err.c_str();
}

}  // extern "C"
