/*
 * ua.h -- C ABI of the Universal Attention (UA) layer library (libua.so).
 *
 * Universal Attention ("A Self-Pruning Transformer: Extreme KV-Cache
 * Compression with Universal Attention"; paperlayer.ai summary, sections 3-4.2,
 * and the ai4snews page, Figure 1 caption) is causal softmax attention over
 * RoPE'd queries and L2-normalised keys with an additive, content-dependent
 * decay bias.  Three decay terms -- query-aware, key-aware and
 * key-similarity -- are combined by a geometric mean, taken to log space and
 * accumulated causally; a low-rank sigmoid gate multiplies the output.  At
 * inference one scalar log-bias is kept per cached KV pair and a pair whose
 * effective mask exp(bias) falls below a threshold p is evicted, per KV head.
 *
 * Exact forms (the pages give none):
 *   k~ = round_cache(RoPE(k / max(|k|, 1e-12))),  q~ = RoPE(q), rotate-half,
 *        frequencies rope_base^(-2i/d), angles in fp64;
 *   per KV head h: lq = logsig(z[h]), lk = logsig(z[H_kv+h]),
 *        lb = logsig(z[2 H_kv+h]),  z = x W_dec + b_dec;
 *   pair term (j < t): s = <k~_t, k~_j>, lambda = mean over enabled terms of
 *        {lq_t, lk_j, lb_t + log min(s^2, 1)},  A_tj = log(1 - exp(lambda));
 *   bias: Lambda_ij = sum_{t=j+1..i} A_tj;   live iff Lambda >= log p;
 *   y = sigmoid((x W_dn) W_up + b_up) * softmax(sm_scale q~ k~^T + Lambda) V.
 *
 * Conventions shared by every entry point
 *   - All pointers inside the structs are DEVICE pointers (hipMalloc'd or
 *     torch CUDA tensors) unless stated otherwise; the struct itself lives on
 *     the host and is only read during the call.
 *   - The caller allocates and owns every buffer, including the workspace.
 *     The library never allocates, frees, or keeps pointers after returning.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *     the call returns without synchronising.  Segment lengths and positions
 *     stay on the device, so no call reads device memory on the host.
 *   - Host-side argument checks run before anything is enqueued; a non-zero
 *     return means nothing was enqueued.  Device-side conditions (a full
 *     segment) are reported through the sticky `status` word.
 *   - Calls that share a cache or workspace must be ordered on one stream.
 *   - No C++ exception crosses this interface; the library holds no mutable
 *     global state.
 */
#ifndef UA_H_
#define UA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define UA_ABI_VERSION 1

/* Return codes. */
typedef enum ua_status {
  UA_OK = 0,
  UA_ERR_INVALID_ARG = 1, /* null or misaligned pointer, bad shape, bad p  */
  UA_ERR_UNSUPPORTED = 2, /* head dim, group size, rank or dtype not built */
  UA_ERR_WORKSPACE = 3,   /* workspace smaller than ua_workspace_bytes()   */
  UA_ERR_HIP = 4          /* a HIP launch returned an error                */
} ua_status;

/* Element types. */
typedef enum ua_dtype { UA_F32 = 0, UA_BF16 = 1 } ua_dtype;

/* Decay terms (bitmask for ua_dims.terms).  paperlayer.ai section 4.1. */
enum { UA_TERM_Q = 1, UA_TERM_K = 2, UA_TERM_SIM = 4, UA_TERMS_ALL = 7 };

/* Sticky device status bits (ua_cache.status). */
/* bit 0: an append or a prefill found its segment full (that segment was left
 * unchanged); bit 1: a wait on another workgroup of the same call timed out
 * (never expected; the outputs and the cache contents are then undefined;
 * every such wait is on a workgroup that is already running, or, in a decode
 * step, on one of the first workgroups that fit on the GPU together, which
 * other work on the device can delay but not block);
 * bit 2: a decode step found a segment length above its capacity (a broken
 * cache table; the step changed nothing, and y is undefined). */
enum { UA_STATUS_SEGMENT_FULL = 1, UA_STATUS_WAIT_TIMEOUT = 2, UA_STATUS_BAD_LENGTH = 4 };

/*
 * Layer shape and numeric options.
 *   B         sequences per call
 *   H_q, H_kv query heads and KV heads; H_q % H_kv == 0, G = H_q / H_kv <= 8
 *   d_head    64 or 128
 *   d_model   width of x; a multiple of 8, at most 16384
 *   gate_rank rank r of the output gate, 1..64
 *   dtype     element type of q, k, v, x, W_dec, W_dn, W_up and cached K, V
 *   y_dtype   element type of the output y
 *   terms     enabled decay terms (UA_TERM_*), 0..7; 0 = plain causal softmax
 *   rope_base RoPE base theta (e.g. 10000)
 *   sm_scale  softmax scale; 0 selects 1/sqrt(d_head)
 */
typedef struct ua_dims {
  int32_t B;
  int32_t H_q;
  int32_t H_kv;
  int32_t d_head;
  int32_t d_model;
  int32_t gate_rank;
  int32_t dtype;
  int32_t y_dtype;
  int32_t terms;
  int32_t reserved0;
  double rope_base;
  float sm_scale;
  float reserved1;
} ua_dims;

/*
 * Layer weights (device, row-major, 16-byte aligned):
 *   W_dec [d_model, 3*H_kv]  gate projections; column m*H_kv + h feeds gate m
 *                            (0 query, 1 key, 2 similarity) of KV head h
 *   b_dec [3*H_kv]   fp32    gate biases
 *   W_dn  [d_model, r]       output-gate down projection
 *   W_up  [r, H_q*d_head]    output-gate up projection (column a*d + i)
 *   b_up  [H_q*d_head] fp32  output-gate bias, or NULL for zero
 */
typedef struct ua_params {
  const void* W_dec;
  const float* b_dec;
  const void* W_dn;
  const void* W_up;
  const float* b_up;
} ua_params;

/*
 * Per-call token inputs (device, contiguous, token-major, 16-byte aligned),
 * n = 1 for ua_decode_step and n = n_tokens for ua_prefill:
 *   q [B, n, H_q, d_head], k [B, n, H_kv, d_head], v [B, n, H_kv, d_head],
 *   x [B, n, d_model]
 * q/k/v are the layer's already-projected queries, keys and values.
 */
typedef struct ua_tokens {
  const void* q;
  const void* k;
  const void* v;
  const void* x;
} ua_tokens;

/*
 * The pruned KV cache of one layer.  Segment s = b*H_kv + h holds the entries
 * of sequence b, KV head h, contiguously and in insertion order in slots
 * [seg_off[s], seg_off[s] + seg_len[s]); its capacity is seg_cap[s] slots.
 *   K, V      [total_slots, d_head] in dims.dtype; K holds k~ (normalised,
 *             rotated, rounded to the cache type)
 *   logbias   [total_slots] fp32  Lambda_j, the entry's log effective mask
 *   kgate     [total_slots] fp32  lk_j, the key gate fixed at insertion
 *   seg_off   [B*H_kv] int64, read only; segments must not overlap
 *   seg_len   [B*H_kv] int32, updated by the library
 *   seg_cap   [B*H_kv] int32, read only
 *   next_pos  [B] int32, RoPE position of the next token; advanced by the
 *             library
 *   status    [1] int32, sticky bits (UA_STATUS_*); the library only sets bits
 *   total_slots  number of slots in K, V, logbias and kgate (host value)
 * K and V must be 16-byte aligned; seg_off[s] may be any slot index.
 */
typedef struct ua_cache {
  void* K;
  void* V;
  float* logbias;
  float* kgate;
  const int64_t* seg_off;
  int32_t* seg_len;
  const int32_t* seg_cap;
  int32_t* next_pos;
  int32_t* status;
  int64_t total_slots;
} ua_cache;

/*
 * Bytes of workspace the calls need for this shape: the maximum over
 * ua_decode_step, ua_prefill with up to max_tokens_per_call tokens, and
 * ua_compact, for a cache of total_slots slots whose largest segment has
 * max_seg_cap slots.  Returns 0 for invalid dims.  The workspace must be
 * 256-byte aligned.  Its first part holds counters and flags the kernels use
 * to coordinate workgroups: the whole workspace must be zero-filled once
 * before its first use (ua_workspace_init, or any zero fill), and every call
 * leaves that part zero again.  Calls that share a workspace must be ordered
 * on one stream; the rest of the workspace is scratch between calls.  A
 * workspace may be shared by calls whose dims have the same B and H_kv (the
 * layers of one model, say) on caches of different sizes: size it with the
 * largest total_slots, max_tokens_per_call and max_seg_cap among them.
 */
size_t ua_workspace_bytes(const ua_dims* dims, int32_t max_tokens_per_call, int64_t total_slots, int32_t max_seg_cap);

/*
 * Zero-fill ws_bytes bytes of a workspace on `stream` (a device kernel; no
 * memset node, so it may also be captured).  ws must be 256-byte aligned.
 */
ua_status ua_workspace_init(void* ws, size_t ws_bytes, void* stream);

/*
 * One decode step: one new token per sequence (paperlayer.ai section 4.2;
 * ai4snews Figure 1 caption).  For each sequence b, at position next_pos[b]:
 * forms q~, k~ and the gates; for every cached entry of its segments that is
 * still live (logbias >= log_p) adds the pair term A_tj to logbias; entries
 * that fall below log_p are left out of this step's softmax (they are removed
 * later by ua_compact); appends (k~, v, 0, lk) unless the segment is full
 * (then UA_STATUS_SEGMENT_FULL is set and the append skipped; the token still
 * attends to itself); writes y [B, H_q, d_head] in dims.y_dtype; advances
 * next_pos and seg_len.  Entries already below log_p on entry are skipped, so
 * results do not depend on how often ua_compact runs.
 *   log_p  log of the eviction threshold p in [0, 1): finite and <= 0, or
 *          -INFINITY for p = 0 (keep everything).  NaN or > 0 is invalid.
 *   y      device output, 16-byte aligned.
 */
ua_status ua_decode_step(const ua_dims* dims, const ua_params* params, const ua_cache* cache, const ua_tokens* in,
                         float log_p, void* y, void* ws, size_t ws_bytes, void* stream);

/*
 * One decode step followed, in the same pass over the cache, by the
 * compaction of every segment: the result equals ua_decode_step(log_p) then
 * ua_compact(log_p) on the same cache (paperlayer.ai section 4.2: evicted
 * entries never return; the new entry, when appended, lands after the
 * survivors).  kept_idx is as for ua_compact, with the new entry's index
 * given as the segment's length before the step.  The cached entries of a
 * segment are read once: the survivors move down from registers.
 */
ua_status ua_decode_compact_step(const ua_dims* dims, const ua_params* params, const ua_cache* cache,
                                 const ua_tokens* in, float log_p, void* y, int32_t* kept_idx, void* ws,
                                 size_t ws_bytes, void* stream);

/* Size of the library's own decode workspace (16 MiB per GPU). */
#define UA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step as ua_decode_compact_step, with the same arguments, results and status
 * words, but its workspace is a UA_NOALLOC_SCRATCH_BYTES array inside the
 * library, one per GPU, held from the first call on that GPU until the process
 * ends.  The call allocates and frees nothing.  Steps whose workspace
 * (ua_workspace_bytes with max_tokens_per_call = 1 bounds it from above) would
 * exceed the array return UA_ERR_WORKSPACE before anything is launched; the
 * decode step fits for caches of about two million slots at d_head = 64.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (several streams or host threads) race and must be serialised by the caller.
 * The first call on a GPU looks up the array's address (a host-side query,
 * made once, under a lock).
 */
ua_status ua_decode_compact_step_noalloc(const ua_dims* dims, const ua_params* params, const ua_cache* cache,
                                         const ua_tokens* in, float log_p, void* y, int32_t* kept_idx,
                                         void* stream);

/*
 * Chunked prefill: appends n_tokens tokens to every sequence and writes their
 * outputs y [B, n_tokens, H_q, d_head] (paperlayer.ai sections 4.2, 5 and
 * App. C: the bias is applied inside the softmax and the L x L bias matrix is
 * never stored).  Attention is dense inside the call: every cached entry and
 * every earlier token of the call is attended with its bias, whatever its
 * value.  Cached entries' logbias is advanced by the call's column sums; the
 * new entries' logbias ends at their final value, so after the last chunk the
 * cache's logbias is the final per-KV bias vector, ready for ua_compact.
 * Tokens get positions next_pos[b] + i.  Every segment must have room for
 * n_tokens more entries (checked on the device: if a segment lacks room,
 * UA_STATUS_SEGMENT_FULL is set and the call leaves that segment unchanged
 * and writes zeros to y for its heads).
 */
ua_status ua_prefill(const ua_dims* dims, const ua_params* params, const ua_cache* cache, const ua_tokens* in,
                     int32_t n_tokens, void* y, void* ws, size_t ws_bytes, void* stream);

/*
 * Pruned prefill (paperlayer.ai section 4.2: a KV pair whose effective mask
 * falls below p is evicted per head and never returns).  As ua_prefill, but
 * token i of the call attends a cached or earlier entry j only while its bias
 * Lambda_ij >= log_p (the token's own entry always), and the call ends with
 * ua_compact(log_p) on the whole cache.  Because a bias never increases, the
 * outputs and the surviving entries equal those of n_tokens calls of
 * ua_decode_compact_step at the same log_p, up to entries whose bias lies
 * within rounding of log_p.  kept_idx is as for ua_compact, indices counted in
 * the segment as it stands after the appends.  log_p as for ua_decode_step;
 * -INFINITY makes the call ua_prefill.  A segment without room for n_tokens
 * more entries is handled as by ua_prefill, then compacted.
 */
ua_status ua_prefill_pruned(const ua_dims* dims, const ua_params* params, const ua_cache* cache,
                            const ua_tokens* in, int32_t n_tokens, float log_p, void* y, int32_t* kept_idx,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Prefill with eviction at chunk boundaries (paperlayer.ai section 5: prefill
 * pruning in chunks of 128 tokens).  Tokens [c, c + chunk) of every sequence
 * go through ua_prefill, dense inside the chunk, and then ua_compact(log_p)
 * runs; c = 0, chunk, 2 chunk, ... up to n_tokens (the last chunk may be
 * shorter).  in and y hold all n_tokens tokens as for ua_prefill; the
 * workspace needs ua_prefill's for `chunk` tokens.
 */
ua_status ua_prefill_chunked(const ua_dims* dims, const ua_params* params, const ua_cache* cache,
                             const ua_tokens* in, int32_t n_tokens, int32_t chunk, float log_p, void* y, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * Variable-length prefill: ua_prefill for a batch whose sequences append
 * different numbers of tokens (paperlayer.ai section 4.2: the cache is kept
 * per sequence and KV head, so sequences are independent).  Sequence b
 * appends n_b = cu_seqlens[b + 1] - cu_seqlens[b] tokens; they are packed:
 * token t of sequence b is row cu_seqlens[b] + t of q [total_tokens, H_q, d],
 * k and v [total_tokens, H_kv, d], x [total_tokens, D] and y
 * [total_tokens, H_q, d].  cu_seqlens is a device int32 array [B + 1],
 * nondecreasing from 0 to total_tokens, with every n_b <= max_tokens (n_b = 0
 * is allowed).  The device reads it; the host checks only its pointer.  The
 * kernels clamp every row they touch into [0, total_tokens), so a malformed
 * array gives wrong results but no access outside the arrays.  Everything
 * else is as for ua_prefill with n_tokens = max_tokens, including the
 * workspace size; segments of sequence b need room for n_b entries, and
 * next_pos[b] advances by n_b.
 */
ua_status ua_prefill_varlen(const ua_dims* dims, const ua_params* params, const ua_cache* cache,
                            const ua_tokens* in, const int32_t* cu_seqlens, int32_t total_tokens, int32_t max_tokens,
                            void* y, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward pass of the decay-mask and attention kernels (paperlayer.ai summary,
 * section 4.2 and Appendix C: training pairs a decay-mask kernel with a fused
 * attention kernel; ai4snews Figure 1 caption: the three decays are combined
 * by a geometric mean, taken to log space and accumulated causally).  For a
 * training chunk of n_tokens tokens per sequence that starts from an empty
 * cache, with o [B, n, H_q, d] the attention output before the output gate,
 * ua_attention_backward turns dO = dL/do into the gradients of the
 * attention's inputs:
 *   q   [B, n, H_q, d]   rotated queries q~           (dims.dtype)
 *   k   [B, n, H_kv, d]  stored keys k~ (normalised, rotated, cache-rounded)
 *   v   [B, n, H_kv, d]  values                        (dims.dtype)
 *   lq, lk, lb [B, n, H_kv] fp32  log-gates (query, key, similarity)
 *   dO  [B, n, H_q, d] fp32
 * q, k, v and dO must be 16-byte aligned, the gates 4-byte aligned.
 * Outputs (fp32, device, 16-byte aligned, written in full): dq, dk, dv of the
 * shapes of q, k, v, and dlq, dlk, dlb of the gates'.  dk includes the
 * similarity term's share.  The gradient of min(s^2, 1) is taken as 0 where
 * the clamp holds.  The chain through RoPE, the key normalisation and the gate
 * projections is elementwise or a plain GEMM and stays with the caller.  The
 * workspace (ua_backward_workspace_bytes) holds the N x N bias and its
 * gradient per segment (2 N^2 fp32 per (sequence, KV head), 256-byte
 * aligned); it needs no zero fill, and ua_backward_workspace_bytes returns 0
 * for dims it rejects.  Errors: UA_ERR_INVALID_ARG (n_tokens < 1, a null or
 * misaligned pointer), UA_ERR_UNSUPPORTED (head dim other than 64 or 128),
 * UA_ERR_WORKSPACE (ws_bytes too small), UA_ERR_HIP (launch failure).  The
 * call is asynchronous on `stream`.
 */
typedef struct ua_grad_inputs {
  const void* q;
  const void* k;
  const void* v;
  const float* lq;
  const float* lk;
  const float* lb;
  const float* dO;
} ua_grad_inputs;

typedef struct ua_grads {
  float* dq;
  float* dk;
  float* dv;
  float* dlq;
  float* dlk;
  float* dlb;
} ua_grads;

size_t ua_backward_workspace_bytes(const ua_dims* dims, int32_t n_tokens);

ua_status ua_attention_backward(const ua_dims* dims, int32_t n_tokens, const ua_grad_inputs* in, const ua_grads* out,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * Qwen3-style normalised queries and keys (paperlayer.ai summary, Appendix E:
 * the UA ablation with normalised queries and keys), in place, before a
 * decode or prefill call takes q and k as its inputs.  Every head vector x of
 * q [B, n_tokens, H_q, d_head] and k [B, n_tokens, H_kv, d_head] (dims.dtype,
 * 16-byte aligned, device) becomes x / sqrt(mean(x^2) + eps) * w over the
 * head dimension, rounded to dims.dtype (nearest even for bf16).  w_q and w_k
 * are fp32 [d_head] device vectors shared by the heads; a NULL weight leaves
 * that tensor unchanged.  eps must be finite and >= 0 (1e-6 in Qwen3).
 */
ua_status ua_qk_norm(const ua_dims* dims, const float* w_q, const float* w_k, float eps, void* q, void* k,
                     int32_t n_tokens, void* stream);

/*
 * Stable in-place compaction (paperlayer.ai section 4.2: an entry whose
 * effective mask falls below p is evicted and never returns).  Per segment,
 * entries with logbias < log_p are removed and the survivors (K, V, logbias,
 * kgate) move down in order; seg_len becomes the survivor count.  If kept_idx
 * is not NULL (device int32 [total_slots]), slot seg_off[s] + i receives the
 * pre-compaction in-segment index of the i-th survivor of segment s, for
 * i < new seg_len[s]; other slots are left unchanged.
 */
ua_status ua_compact(const ua_dims* dims, const ua_cache* cache, float log_p, int32_t* kept_idx, void* ws,
                     size_t ws_bytes, void* stream);

/* Text for a return code (static storage). */
const char* ua_status_string(int32_t status);

/* UA_ABI_VERSION of the built library. */
int32_t ua_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* UA_H_ */
