/*
 * sve.h — C ABI of libsve: extend-prefill attention over resident KV slots and
 * the m-row int4 GEMV, for AMD Instinct MI355X (gfx950).
 *
 * Conventions
 *   - Every function returns 0 (SVE_OK) or a negative SVE_E_* code and never
 *     throws. Arguments are checked on the host before anything is enqueued;
 *     on error nothing is enqueued and no state changes.
 *   - "device" pointers are HIP device memory owned by the caller (for example
 *     torch tensors); the library never allocates, frees or retains them
 *     beyond the call, except the arena handed to sve_create, which must stay
 *     allocated until sve_destroy.
 *   - "host" pointers are ordinary host memory, read during the call only.
 *   - hip_stream is a hipStream_t (NULL = the legacy default stream). Work is
 *     enqueued asynchronously on it unless a function says it synchronises.
 *   - bf16 and fp16 values are passed as their 16-bit patterns.
 *   - One context may be used by one host thread at a time.
 *
 * Source pages cited below:
 *   [goinfer]  goinfer, "Turn nine in under half a second"
 *   [spec]     thinkspread, "The economics of speculative decoding: +41% on
 *              9B, break-even on 35B"
 *   [quant]    thinkspread, "Models and quantizations"
 *   [openjev]  openjev-multimodal, "Latency"
 */
#ifndef SVE_H
#define SVE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SVE_OK = 0,
  SVE_E_ARG = -1,      /* null pointer, bad size or shape */
  SVE_E_SLOT = -2,     /* slot or layer index out of range */
  SVE_E_CAPACITY = -3, /* more tokens or rows than the context was built for */
  SVE_E_HIP = -4,      /* a HIP runtime call failed (text: sve_last_error) */
  SVE_E_STATE = -5     /* call out of order, e.g. extend past the selected prompt */
};

#define SVE_MAX_SLOTS 4

typedef struct sve_ctx sve_ctx;

/* Shape of a KV-slot store. [goinfer] "How it works": a GPU-resident model
 * keeps up to --kv-sessions KV slots, one conversation each; "Use it": the
 * default is 4 and 0 switches reuse off. */
typedef struct {
  int32_t n_slots;    /* requested slots, 1..SVE_MAX_SLOTS */
  int32_t n_layers;   /* KV layers held per slot, >= 1 */
  int32_t n_q_heads;  /* Hq, a multiple of n_kv_heads */
  int32_t n_kv_heads; /* Hkv */
  int32_t head_dim;   /* D: 64 or 128 */
  int32_t capacity;   /* max tokens per slot (rounded up to a multiple of 64) */
  int32_t max_rows;   /* max new rows per extend call (sum over a batched call),
                         1..4*capacity, and max_rows * n_q_heads * head_dim * 2
                         below 2 GiB (one key split's partials); sizes the
                         split workspace */
  int32_t reuse;      /* 0: select always reports 0 reused tokens */
  int32_t match_rule; /* 0: lone-slot clause on (default); 1: literal rule */
} sve_config;

/* Bytes of device memory a context needs for `n_slots` slots: the KV store,
 * the token mirrors, and the split-KV workspace. 0 if cfg is invalid. */
size_t sve_arena_bytes(const sve_config* cfg, int32_t n_slots);

/* Create a context over a caller-owned device arena of `arena_bytes` bytes
 * (256-byte aligned). As many of the requested slots as fit are granted
 * ([goinfer] "Use it": the memory check may grant fewer slots than asked,
 * and both numbers are reported); *granted_slots receives that number.
 * The arena is cleared on `hip_stream`. Errors: SVE_E_ARG (bad config, null
 * pointers, misaligned arena), SVE_E_CAPACITY (not even one slot fits),
 * SVE_E_HIP. */
int sve_create(const sve_config* cfg, void* arena, size_t arena_bytes, void* hip_stream,
               sve_ctx** out, int32_t* granted_slots);

/* Free the host-side context. The arena stays the caller's. */
int sve_destroy(sve_ctx* ctx);

/* Use another stream for later calls on this context. */
int sve_set_stream(sve_ctx* ctx, void* hip_stream);

/* Pick the slot for a new prompt and report how many of its leading tokens
 * are already cached ([goinfer] "How it works": longest common start, which
 * must beat what that slot shares with the other slots; a GPU request reuses
 * the slot holding the start of its prompt, else an empty slot, else the
 * least recently used one; the conversation is cut back to the shared point
 * and the reuse count reported to the caller).
 *   tokens_host: host int32 [n], 1 <= n <= capacity.
 *   *slot, *reused: the chosen slot and the reused prefix length r
 *     (r <= n-1, so the last prompt token always runs through the model).
 * Commits: the slot's prompt becomes `tokens`, every layer's cached length
 * becomes r, the slot becomes most recently used. Only tokens whose K/V rows
 * are cached in every layer take part in matching; a slot stays claimed (not
 * empty) from its first select on, even before its rows are prefilled, so
 * several prompts may be placed before one batched extend. A slot is eligible when
 * its common start with the prompt is > 0, exceeds its common start with
 * every other occupied slot, and either covers the whole slot or some other
 * slot is occupied (match_rule 1 drops this last clause).
 * SYNCHRONISES the context stream (one small device-to-host read).
 * Errors: SVE_E_ARG, SVE_E_CAPACITY (n > capacity), SVE_E_HIP. */
int sve_kv_slot_select(sve_ctx* ctx, const int32_t* tokens_host, int32_t n, int32_t* slot,
                       int32_t* reused);

/* Cut a slot back to `len` cached positions in every layer ([goinfer] "How it
 * works": cut back to the shared point). Metadata only; the selected prompt
 * is kept, so later extend calls may refill it. len must not exceed any
 * layer's cached length. Errors: SVE_E_SLOT, SVE_E_ARG. */
int sve_kv_truncate(sve_ctx* ctx, int32_t slot, int32_t len);

/* Cached length of (slot, layer). */
int sve_kv_len(const sve_ctx* ctx, int32_t slot, int32_t layer, int32_t* len);

/* Granted slot count and padded per-slot capacity. */
int sve_info(const sve_ctx* ctx, int32_t* granted_slots, int32_t* capacity);

/* Extend-prefill: append m new rows to (slot, layer) and attend.
 * With P the cached length, query row i (absolute position P+i) attends
 * causally to positions 0..P+i of that slot and layer, with scores scaled by
 * 1/sqrt(D) and q head h reading KV head h / (Hq/Hkv); q and k arrive
 * position-encoded. ([goinfer] "What goinfer does": only the tokens after the
 * reused start are prefilled against the kept KV cache; [spec] opening
 * section: the k+1 verify rows are one such pass.)
 *   q:     device bf16 [m][Hq][D]
 *   new_k: device bf16 [m][Hkv][D]   (stored at positions P..P+m-1)
 *   new_v: device bf16 [m][Hkv][D]
 *   out:   device bf16 [m][Hq][D]    (fp32 accumulation, rounded to nearest even)
 * m == 0 is a no-op. Asynchronous; the cached length becomes P+m.
 * The call enqueues kernel launches only (no memset or copy), so it can be
 * captured in a HIP graph. The checks, the launch plan and the cached length
 * are host work done when the call is made: a replay repeats the same
 * positions and inputs, so it is valid after the same cut back and select
 * as at capture.
 * Errors: SVE_E_SLOT, SVE_E_ARG, SVE_E_CAPACITY (m > max_rows),
 * SVE_E_STATE (P+m beyond the prompt committed by the last select), SVE_E_HIP. */
int sve_extend_attn(sve_ctx* ctx, int32_t slot, int32_t layer, const void* q, const void* new_k,
                    const void* new_v, int32_t m, void* out);

/* The same for n distinct slots in one launch (rows packed slot after slot:
 * q_packed [sum m][Hq][D], k_packed/v_packed [sum m][Hkv][D], out_packed
 * [sum m][Hq][D]). slots_host, m_host: host int32 [n], 1 <= n <= 4.
 * Errors as sve_extend_attn; SVE_E_ARG also for a repeated slot. */
int sve_extend_attn_batched(sve_ctx* ctx, int32_t n, const int32_t* slots_host,
                            const int32_t* m_host, int32_t layer, const void* q_packed,
                            const void* k_packed, const void* v_packed, void* out_packed);

/* Several questions about one resident state ([openjev] "What changed",
 * prefix priming: the shared prefix is evaluated once and each question
 * resumes from it, reading only its own text). With P the cached length of
 * (slot, layer), question j's rows i (0-based within the question) attend
 * to positions 0..P-1 of the slot and to rows 0..i of question j only;
 * scaling and GQA as sve_extend_attn. Nothing is appended: the cached
 * length stays P and the slot's rows are only read, so the state remains
 * the checkpoint for further questions.
 *   n_questions: 1..16; m_host: host int32 [n_questions], each >= 1, sum
 *   <= max_rows; q [sum m][Hq][D], new_k / new_v [sum m][Hkv][D] (the
 *   questions' own rows), out [sum m][Hq][D]: device bf16, rows packed
 *   question after question.
 * Asynchronous. Errors: SVE_E_SLOT, SVE_E_ARG, SVE_E_CAPACITY, SVE_E_HIP. */
int sve_extend_attn_questions(sve_ctx* ctx, int32_t slot, int32_t layer, int32_t n_questions,
                              const int32_t* m_host, const void* q, const void* new_k,
                              const void* new_v, void* out);

/* Copy cached rows [start, start+len) of (slot, layer) to k_out, v_out:
 * device bf16 [len][Hkv][D] each (test export). */
int sve_kv_read(sve_ctx* ctx, int32_t slot, int32_t layer, int32_t start, int32_t len,
                void* k_out, void* v_out);

/* ---- int4 group-32 weights ([quant] "Quantizations": 32-element blocks with
 * one scale, used in place) --------------------------------------------------
 * Logical format: w uint8 [N][K/2], element k in the low nibble of byte k/2
 * for even k and the high nibble for odd k; scales fp16 [N][K/32];
 * value = (code - 8) * scale. The GEMV reads a device layout written once by
 * sve_w4_pack (same byte count, rows padded to 16 and k to 128). */

/* Bytes of the device layout of an N x K weight. 0 if N < 1 or K % 32. */
size_t sve_w4_packed_bytes(int32_t N, int32_t K);

/* Convert a logical weight (device w, device scales) into the device layout
 * (device `packed`, sve_w4_packed_bytes(N, K) bytes). Errors: SVE_E_ARG, SVE_E_HIP. */
int sve_w4_pack(const uint8_t* w, const uint16_t* scales, int32_t N, int32_t K, void* packed,
                void* hip_stream);

/* Decode a packed weight to device fp32 [N][K]; (code-8)*scale is exact in
 * fp32 (test export). */
int sve_w4_dequant(const void* packed, int32_t N, int32_t K, float* out, void* hip_stream);

/* m-row GEMV: y[r][n] = sum_k x[r][k] * w[n][k], the weights read once for
 * all m rows ([spec] opening section: verify rows share one read of the
 * weights, so extra rows are nearly free).
 *   x: device bf16 [m][K]; packed: sve_w4_pack output; y: device fp32 [m][N].
 *   1 <= m <= 16, N >= 1, K % 32 == 0, K <= 4194304.
 * Errors: SVE_E_ARG, SVE_E_HIP. */
int sve_w4_gemv_m(const void* x, int32_t m, const void* packed, int32_t N, int32_t K, float* y,
                  void* hip_stream);

/* Many-row int4 GEMM for a prefill's new rows ([goinfer] "The problem": a
 * prefill runs every new prompt token through each weight matrix, so a turn
 * of m new tokens is an m-row product per matrix; [quant] "Quantizations":
 * the group-32 blocks are used in place). Same result definition as
 * sve_w4_gemv_m, for any number of rows: y[r][n] = sum_k x[r][k] * w[n][k],
 * w = (code - 8) * scale. It multiplies fp16 operands and accumulates in
 * fp32: each weight is (code - 8) * scale rounded once to fp16 and x is
 * converted from bf16 to fp16. Both conversions are exact or within a
 * relative 2^-11 in fp16's normal range (2^-14 <= |v| < 65504; a bf16 value
 * there is exact); below 2^-14 the error is at most half an fp16 subnormal
 * step (2^-25) and below 2^-25 values become 0; at 65520 and beyond they
 * become infinite.
 *   x: device bf16 [m][K]; packed: sve_w4_pack output; y: device fp32 [m][N];
 *   workspace: device memory of at least sve_w4_gemm_workspace_bytes(m, N,
 *   K) bytes, owned by the caller and used only during the call's kernels
 *   (x in fp16, and k-split partial results).
 *   m >= 1, N >= 1, K % 32 == 0. The result depends only on (x, w, m, N, K):
 *   repeated calls give identical bits.
 * Errors: SVE_E_ARG (shape, null pointer, workspace too small), SVE_E_HIP. */
size_t sve_w4_gemm_workspace_bytes(int32_t m, int32_t N, int32_t K);
int sve_w4_gemm(const void* x, int32_t m, const void* packed, int32_t N, int32_t K, float* y,
                void* workspace, size_t workspace_bytes, void* hip_stream);

/* Expert-routed GEMV for a mixture-of-experts layer ([spec] "Architecture
 * decides whether it pays": rows pick different experts, so expert weights
 * are not shared across rows). Pair (r, j) computes
 * y[r][j][:] = W_{ids[r][j]} x(r, j), where x(r, j) = x[r] (x_per_slot 0,
 * x device bf16 [m][K]) or x[r][j] (x_per_slot 1, x [m][topk][K]). Each
 * distinct expert's weights are read once for all pairs routed to it.
 *   expert_ids: device int32 [m][topk]; packed_all: E packed weights of
 *   sve_w4_packed_bytes(N, K) bytes each, back to back; y: device fp32
 *   [m][topk][N]. 1 <= m <= 16, 1 <= topk <= 16, K <= 4194304. An id outside 0..E-1
 *   yields NaN in that pair's output row.
 * Errors: SVE_E_ARG, SVE_E_HIP. */
int sve_w4_gemv_m_routed(const void* x, int32_t x_per_slot, int32_t m, const int32_t* expert_ids,
                         int32_t topk, const void* packed_all, int32_t E, int32_t N, int32_t K,
                         float* y, void* hip_stream);

/* ---- speculative verify: acceptance, rollback and gate --------------------
 * thinkspread, "The economics of speculative decoding: +41% on 9B, break-even
 * on 35B": a draft head proposes k tokens, one pass over m = k + 1 rows
 * checks them and the runtime keeps the ones that were right (opening
 * section); when the rolling acceptance drops under a threshold the runtime
 * falls back to ordinary decoding ("Gating: enable it only where it pays");
 * verify(m) = a + b*m prices whether it pays ("Closing the ledger"). */

#define SVE_VERIFY_MAX_ROWS 16
#define SVE_GATE_MAX_WINDOW 64

/* Device workspace bytes sve_verify_accept needs for m rows of V logits
 * (0 if m or V is out of range). */
size_t sve_verify_workspace_bytes(int32_t m, int32_t V);

/* Greedy acceptance of one verify step. Row i of `logits` holds the target
 * model's scores for the token after input i, where the inputs are the last
 * accepted token and the k = m - 1 drafts. Draft i+1 is kept while it equals
 * row i's argmax (ties: the lowest id; a NaN counts as larger than any
 * number); the row after the last kept draft gives the next token. The
 * caller then keeps P + accepted + 1 cached positions of the slot the m rows
 * were appended to (sve_kv_truncate), P being its length before the verify.
 *   logits: device fp32 [m][V], rows contiguous; 1 <= m <= SVE_VERIFY_MAX_ROWS,
 *           V >= 1.
 *   draft: device int32 [m-1] (may be NULL when m == 1).
 *   result: device int32 [2 + m]: accepted drafts (0..m-1), the next token,
 *           then the argmax of every row.
 *   workspace: caller-owned device memory of at least
 *              sve_verify_workspace_bytes(m, V) bytes.
 * ASYNC on hip_stream (two kernel launches). Errors: SVE_E_ARG, SVE_E_HIP. */
int sve_verify_accept(const float* logits, int32_t m, int32_t V, const int32_t* draft,
                      int32_t* result, void* workspace, size_t workspace_bytes,
                      void* hip_stream);

/* Allocation-free form of sve_verify_accept, for callers that cannot
 * allocate device memory or hand the library a workspace (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, result and kernels, without the workspace: the partial
 * results live in a static device array of the library (32 KB; every GPU it
 * runs on holds one copy until the process ends), whose address is looked
 * up once per GPU on the first call there with that GPU current (make that
 * first call outside graph capture). The call allocates nothing.
 *   1 <= m <= SVE_VERIFY_MAX_ROWS, 1 <= V <= SVE_VERIFY_NOALLOC_MAX_V; the
 *   stream must belong to the current device.
 * All calls on one GPU share the array and it keeps the last call's
 * contents (nothing in it needs to start cleared): calls that overlap on one
 * GPU, for instance on two streams, race and must be ordered by the caller.
 * ASYNC on hip_stream. Errors: SVE_E_ARG (also V beyond the maximum),
 * SVE_E_HIP. */
#define SVE_VERIFY_NOALLOC_MAX_V 1048576
int sve_verify_accept_noalloc(const float* logits, int32_t m, int32_t V, const int32_t* draft,
                              int32_t* result, void* hip_stream);

/* Rolling-acceptance gate of one request (host only). Each verify step
 * records its accepted count; the rolling acceptance is (sum of the last
 * `window` counts) / (k * those steps), fewer steps at the start; once it is
 * below min_accept the gate closes and the depth stays 0 for the request. */
typedef struct {
  int32_t k;          /* draft depth for the next step; 0 once closed */
  int32_t window;     /* 1..SVE_GATE_MAX_WINDOW */
  double min_accept;  /* e.g. 0.60 */
  int32_t steps;      /* steps recorded */
  int32_t accepted[SVE_GATE_MAX_WINDOW];  /* ring of the recent counts */
} sve_spec_gate;

/* 0 <= k <= SVE_VERIFY_MAX_ROWS - 1, 0 <= min_accept <= 1, window in range.
 * Errors: SVE_E_ARG. */
int sve_spec_gate_init(sve_spec_gate* gate, int32_t k, double min_accept, int32_t window);

/* Record a step that kept `accepted` (0..k) of k drafts; *k_next = the depth
 * for the next step. A closed gate ignores `accepted`. Errors: SVE_E_ARG. */
int sve_spec_gate_step(sve_spec_gate* gate, int32_t accepted, int32_t* k_next);

/* Break-even per-position acceptance of depth k under verify(m) = a + b*m:
 * the alpha in [0, 1] with (1 + alpha + ... + alpha^k) * (a + b) = a +
 * b*(k+1), the draft head's own cost left out; 0 for k = 0, 1 when even
 * alpha = 1 does not pay, -1 for a + b <= 0, b < 0 or k < 0. */
double sve_spec_break_even(double a, double b, int32_t k);

/* ---- measurement probes (not part of the computation) ---------------------
 * The achievable ceilings of the chip beside its published peaks, and a
 * kernel of known traffic that calibrates the hardware counters.
 *
 * Streaming read of `bytes` bytes of device memory at src (a multiple of
 * 16): `blocks` workgroups of `threads` threads (a multiple of 64, at most
 * 1024), grid-stride.
 *   mode 0: each thread keeps `unroll` 16-byte loads in flight (1, 2, 4, 8 or
 *           16) and folds them into one word: sink device uint32
 *           [blocks * threads].
 *   mode 1: the same with nontemporal loads.
 *   mode 2: direct global-to-LDS loads, each wave a ring of `unroll` 1 KB
 *           slots (bytes % 1024 == 0, bytes < 2 GiB, threads/64 * unroll KB
 *           of LDS at most 160 KB): sink device uint32 [blocks].
 *   mode 3: cache-resident direct-to-LDS fill: the region (bytes % 32768 ==
 *           0, < 2 GiB; small enough to stay in L2, e.g. 1 MB) is read over
 *           and over, every wave streaming 8 * `unroll` tiles of 32 KB
 *           (32 one-KB requests each, at most 32 KB in flight per wave, 32 KB
 *           of LDS per wave: at most 256 threads). Bytes moved = blocks *
 *           threads/64 * 8 * unroll * 32768. sink device uint32 [blocks].
 * Plain copy: src to dst, `bytes` each (a multiple of 16), 256-thread blocks.
 * Errors: SVE_E_ARG, SVE_E_HIP. */
int sve_probe_read(const void* src, size_t bytes, int32_t blocks, int32_t threads,
                   int32_t unroll, int32_t mode, void* sink, void* hip_stream);
int sve_probe_copy(const void* src, void* dst, size_t bytes, int32_t blocks, void* hip_stream);

/* Compute ceilings: `blocks` workgroups of 256 threads (4 waves) run `iters`
 * iterations each. Per wave and iteration:
 *   kind 0: 8 v_mfma_f32_16x16x32_bf16 (16384 flops each),
 *   kind 1: 8 v_mfma_f32_32x32x16_bf16 (32768 flops each),
 *   kind 2: 8 v_mfma_f32_16x16x32_f16  (16384 flops each),
 *   kind 3: 64 v_exp_f32 of 64 lanes (eight independent chains),
 *   kind 4: 8 LDS reads of 16 bytes per lane (1 KB per wave each).
 * sink: device uint32 [blocks * 256], written. The rate is the count above
 * times blocks * 4 * iters over the measured kernel time.
 * Errors: SVE_E_ARG, SVE_E_HIP. */
int sve_probe_compute(int32_t kind, int32_t blocks, int32_t iters, void* sink, void* hip_stream);

/* ---- kernel timing (measurement aid) -------------------------------------
 * sve_timing_start makes the next n_calls extend calls on ctx record HIP
 * timing events on the context stream around each of their three kernels
 * (KV append, attention, split combine); the events are created by the
 * library without a system-scope fence, so they add no cache write-back to
 * the timed kernels. sve_timing_read waits for the last recorded event, writes the
 * summed durations in milliseconds of each kernel over the timed calls and
 * their count, destroys the events and ends timing (a kernel that a call
 * does not launch counts as 0: the separate append on the paths whose
 * attention kernel appends its rows itself, the combine of an unsplit
 * call). Not for calls under graph capture.
 *   1 <= n_calls <= 65536. Errors: SVE_E_ARG, SVE_E_STATE (start while
 *   started, read while not started), SVE_E_HIP. */
int sve_timing_start(sve_ctx* ctx, int32_t n_calls);
int sve_timing_read(sve_ctx* ctx, float* append_ms, float* attn_ms, float* combine_ms,
                    int32_t* calls);

/* ---- prompt-lookup drafting ([goinfer] "What we got wrong": n-gram
 * speculation drafts by copying what followed an earlier occurrence of the
 * latest tokens in the prompt itself; one verify pass then accepts or rejects
 * the draft) -------------------------------------------------------------------
 * Host-only integer search. For suffix lengths g = min(max_ngram, n-1) down
 * to min_ngram, finds the latest earlier start p (p = n-g-1 down to 0;
 * overlapping the suffix is allowed) with tokens[p..p+g) equal to the last
 * g tokens, and writes the up to k tokens that followed it
 * (tokens[p+g .. p+g+k), fewer at the end of the history) to draft_host;
 * *n_draft = their count, 0 when no suffix of any length occurred before.
 *   tokens_host: host int32 [n], n >= 0; draft_host: host int32 [k];
 *   0 <= k <= SVE_NGRAM_MAX_DRAFT, 1 <= min_ngram <= max_ngram <= 64.
 * Errors: SVE_E_ARG. */
#define SVE_NGRAM_MAX_DRAFT 64
int sve_ngram_draft(const int32_t* tokens_host, int32_t n, int32_t k, int32_t max_ngram,
                    int32_t min_ngram, int32_t* draft_host, int32_t* n_draft);

/* Message for a status code. */
const char* sve_strerror(int code);

/* Text of the last error on this context, or of the calling thread's last
 * error from a context-free call when ctx is NULL. */
const char* sve_last_error(const sve_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* SVE_H */
