/*
 * hsa_attn.h -- C ABI of the Hierarchical Sparse Attention (HSA) forward layer
 * for AMD MI355X (gfx950).  Library: libhsa_attn.so.
 *
 * What the layer computes (skill card "Every Token Counts 16m Context",
 * sections "Core Technique" and "Implementation"; abstract page "Every Token
 * Counts: Generalizing 16M Ultra-Long Context in Large Language Models"):
 * the keys are cut into chunks of S tokens, every chunk gets a landmark (the
 * mean of its keys), each query scores the landmarks of the complete chunks
 * before its own chunk with q.L/sqrt(D), keeps the k best (ties to the lower
 * chunk index), runs softmax attention inside every kept chunk, and fuses the
 * per-chunk outputs with a softmax over the kept scores.  A query with no
 * earlier complete chunk outputs zeros.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All tensors are dense, contiguous and head-major:
 *      prefill  Q [B, Hq, T, D]      K, V [B, Hkv, T, D]
 *      decode   Q [B, Hq, D]         K, V [B, Hkv, T, D]  (the caches)
 *      landmarks  [B, Hkv, floor(T/S), D]   (same storage dtype as K)
 *      out      fp32, shaped like Q
 *      sel_idx  int32 [..., k]  (-1 padding)   sel_score fp32 [..., k] (-inf padding)
 *    Query head h reads KV head floor(h * Hkv / Hq).
 *  - Q, K, V and landmarks are stored as bf16 or fp32 (hsa_attn_dims_t.dtype);
 *    arithmetic accumulates in fp32 (landmark sums in fp64); out is fp32.
 *  - Every pointer is a device pointer, owned by the caller, 16-byte aligned.
 *    The library allocates no memory and keeps no state between calls, apart
 *    from the fixed scratch array of hsa_forward_decode_noalloc.
 *  - Calls are asynchronous: they validate on the host, enqueue kernels on
 *    `stream` (a hipStream_t; NULL means the default stream) and return.
 *    HSA_ATTN_OK means "enqueued".  Validation happens before any HIP call,
 *    so a rejected call enqueues nothing.
 *  - Inputs must be finite; NaN or Inf inputs give undefined results.
 *  - Errors: HSA_ATTN_INVALID_ARGUMENT (null or misaligned pointer, bad
 *    sizes), HSA_ATTN_UNSUPPORTED (sizes outside the supported envelope:
 *    D in {64,128}, S == 64 for the forward calls, Hq/Hkv in {1,2,4,8},
 *    k <= 64 (the adaptive calls: base k <= 32; the prefill backward:
 *    k <= 32); prefill with more than 32 selection slots needs Hq/Hkv <= 4,
 *    and prefill also needs floor(T/S) <= 65536 and B*Hq*T*slots < 2^31),
 *    HSA_ATTN_WORKSPACE_TOO_SMALL,
 *    HSA_ATTN_HIP_ERROR (a launch failed).  hsa_attn_last_error() returns a
 *    thread-local message about the last failure.
 */
#ifndef HSA_ATTN_H_
#define HSA_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HSA_ATTN_OK = 0,
  HSA_ATTN_INVALID_ARGUMENT = 1,
  HSA_ATTN_UNSUPPORTED = 2,
  HSA_ATTN_WORKSPACE_TOO_SMALL = 3,
  HSA_ATTN_HIP_ERROR = 4
} hsa_attn_status_t;

typedef enum { HSA_ATTN_FP32 = 0, HSA_ATTN_BF16 = 1 } hsa_attn_dtype_t;

typedef struct {
  int32_t batch;        /* B */
  int32_t num_q_heads;  /* Hq */
  int32_t num_kv_heads; /* Hkv, divides Hq */
  int32_t head_dim;     /* D */
  int32_t chunk_size;   /* S */
  int32_t top_k;        /* k */
  int64_t seq_len;      /* prefill: T (queries = keys); decode: cache length T,
                           the query sits at position T */
  int32_t dtype;        /* hsa_attn_dtype_t: storage of Q, K, V, landmarks */
  int32_t reserved;     /* must be 0 */
} hsa_attn_dims_t;

/*
 * Landmark builder (card, "Implementation": a landmark per chunk from mean
 * pooling of the chunk's tokens; read as the plain mean of the keys).
 *
 * For every (b, g) and every chunk c in [chunk_begin, chunk_end):
 *   landmarks[b, g, c, :] = round_to_dtype( (sum_{t=cS}^{cS+S-1} K[b, g, t, :]) / S )
 * The sum is exact (fp64), the division is one fp64 operation and the result
 * is rounded once, to nearest even, to the storage dtype.  For bf16 keys the
 * result is bit-identical to the exact mean rounded to bf16.
 * k: K or K cache [B, Hkv, T, D]; landmarks: [B, Hkv, floor(T/S), D].
 * Requires 0 <= chunk_begin <= chunk_end <= floor(T/S) and S >= 1; only D in
 * {64, 128} is supported.  chunk_begin == chunk_end enqueues nothing (and then
 * k and landmarks may be NULL).
 */
hsa_attn_status_t hsa_build_landmarks(const hsa_attn_dims_t* d, const void* k, void* landmarks,
                                      int64_t chunk_begin, int64_t chunk_end, void* stream);

/*
 * Causal HSA forward over a whole sequence (card, "Core Technique" and
 * "Implementation").  Query row p of head h uses the complete chunks
 * c < min(floor(p/S), floor(T/S)) of KV head g(h).
 * q [B,Hq,T,D], k/v [B,Hkv,T,D], landmarks [B,Hkv,floor(T/S),D] (from
 * hsa_build_landmarks), out [B,Hq,T,D] fp32.  sel_idx / sel_score
 * [B,Hq,T,k] are optional outputs (NULL: kept in the workspace); slots are
 * ordered by score descending, then index ascending.  The selection ranks
 * the fp32 dot products q.L before the 1/sqrt(D) factor is applied; where
 * that factor rounds two different dot products to one stored score, the
 * larger dot product is the one kept at the cut.
 * T = 0 (no query rows) enqueues nothing and returns HSA_ATTN_OK without
 * looking at any pointer, so empty buffers may be NULL.
 * workspace: device scratch (never NULL when T > 0).  It holds, for the
 * whole call, the selection when sel_idx is NULL (8 bytes per slot), the
 * pair positions (4 bytes per slot), per-chunk bucket counts and a
 * transposed copy of V; and, for one slab of query rows at a time, the pairs
 * attended chunk-major (selected chunks before the query's aligned window
 * of 64 chunks, and window chunks that few rows of the query's 32-row block
 * selected) with one fp32 [D] attention output each, sized for the worst
 * case (every pair of the slab chunk-major: B*Hq*rows*k*(4*D + 4) bytes).
 * The call processes its rows in equal slabs of whole 64-row chunks, as
 * large as workspace_bytes allows (hsa_attn_prefill_slab_rows tells the
 * size); results do not depend on the slab size.  hsa_attn_workspace_size(d,
 * 0) returns the size for slabs whose worst case stays within about 16 GiB
 * (19.9 GB at B=1, Hq=32, T=2^18, k=16, D=128, bf16, in 4 slabs); the minimum is
 * the per-call part plus one slab of 64 rows, and less returns
 * HSA_ATTN_WORKSPACE_TOO_SMALL.
 */
hsa_attn_status_t hsa_forward_prefill(const hsa_attn_dims_t* d, const void* q, const void* k,
                                      const void* v, const void* landmarks, float* out,
                                      int32_t* sel_idx, float* sel_score, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * Query rows per slab that hsa_forward_prefill (adaptive = 0) or
 * hsa_forward_prefill_adaptive (adaptive != 0; d->top_k is the base k) uses
 * with a workspace of workspace_bytes, when the caller passes sel_idx and
 * sel_score (selection_given != 0) or not: a multiple of 64, or 0 when the
 * workspace is too small.  A planning query: it touches no device.
 */
hsa_attn_status_t hsa_attn_prefill_slab_rows(const hsa_attn_dims_t* d, int adaptive, int selection_given,
                                             size_t workspace_bytes, int64_t* slab_rows);

/*
 * Chunked prefill over a cached prefix (serving: new tokens appended to a
 * cache; card, "Core Technique"): the keys are the whole sequence,
 * k/v [B,Hkv,T,D] with d->seq_len = T, and landmarks [B,Hkv,floor(T/S),D]
 * (the prefix's and the new tokens' complete chunks); the queries are the
 * last T - q_offset positions only, q [B,Hq,T-q_offset,D], and out, sel_idx
 * and sel_score cover those rows ([B,Hq,T-q_offset,...]).  Query row r sits
 * at position q_offset + r and uses the complete chunks before its own, as
 * in hsa_forward_prefill; its results equal that call's row q_offset + r.
 * q_offset must be a multiple of S (the prefix is whole chunks).  The
 * workspace of hsa_forward_prefill for the same dims is sufficient.
 * q_offset = T (no new rows) enqueues nothing and returns HSA_ATTN_OK
 * without looking at any pointer.
 */
hsa_attn_status_t hsa_forward_prefill_cached(const hsa_attn_dims_t* d, int64_t q_offset, const void* q,
                                             const void* k, const void* v, const void* landmarks, float* out,
                                             int32_t* sel_idx, float* sel_score, void* workspace,
                                             size_t workspace_bytes, void* stream);

/*
 * Causal prefill with the near-tie adaptive budget (value-of-information
 * router abstract; the rule of hsa_forward_decode_adaptive applied to every
 * query row): row p of head h ranks its candidates as hsa_forward_prefill
 * does (k = d->top_k), and keeps its best min(2k, n_p) chunks when it has
 * more than k candidates and s_k - s_(k+1) < gap_threshold (fp32 scores with
 * the 1/sqrt(D) scale, the values written to sel_score), its best k
 * otherwise.  gap_threshold = 0 reproduces hsa_forward_prefill with top_k = k
 * and +inf with top_k = 2k, bit for bit.  gap_threshold must be >= 0 (+inf
 * allowed).  Requires k <= 32 (and Hq/Hkv <= 4 when k > 16).
 * sel_idx/sel_score [B,Hq,T,2k] optional, -1 /
 * -inf padding.  workspace: at least hsa_attn_workspace_size(d, 3) bytes.
 */
hsa_attn_status_t hsa_forward_prefill_adaptive(const hsa_attn_dims_t* d, float gap_threshold, const void* q,
                                               const void* k, const void* v, const void* landmarks, float* out,
                                               int32_t* sel_idx, float* sel_score, void* workspace,
                                               size_t workspace_bytes, void* stream);

/*
 * Backward pass of the causal prefill (training; the chain rule through the
 * steps of the card's "Core Technique" and "Implementation"): given the
 * forward's inputs, its output `out` [B,Hq,T,D] fp32, its selection sel_idx /
 * sel_score [B,Hq,T,k] (k = d->top_k slots, -1 / -inf padding, as written by
 * hsa_forward_prefill or hsa_forward_prefill_adaptive with k = its slot
 * count) and the upstream gradient dout [B,Hq,T,D] fp32, writes
 * dq [B,Hq,T,D] and dk, dv [B,Hkv,T,D] (fp32, every element).  The selection
 * is held fixed (it is piecewise constant in the inputs) and the landmark's
 * rounding to the storage dtype is taken as the identity, so each key of a
 * kept chunk receives 1/S of the chunk's landmark gradient.  Slots whose
 * index is not a candidate of the row (outside [0, floor(p/S))) are ignored.
 * Storage dtype bf16 only (HSA_ATTN_UNSUPPORTED otherwise); products run on
 * bf16 MFMA with fp32 accumulation: the gradients that feed dq are split
 * into a bf16 head and tail (relative error below 2^-15), the
 * probabilities and gradients that feed dk and dv are rounded to bf16
 * (2^-8).  dk and dv accumulate over pairs in an order that depends
 * on scheduling, so they are not bit-reproducible.
 * T = 0 enqueues nothing and returns HSA_ATTN_OK without looking at any
 * pointer.
 * workspace: at least hsa_attn_workspace_size(d, 4) bytes (about
 * B*Hq*T*k*(4*D + 12) bytes plus a transposed copy of K: 69 GB at B=1,
 * Hq=32, T=2^18, k=16, D=128).
 */
hsa_attn_status_t hsa_backward_prefill(const hsa_attn_dims_t* d, const void* q, const void* k, const void* v,
                                       const void* landmarks, const float* out, const float* dout,
                                       const int32_t* sel_idx, const float* sel_score, float* dq, float* dk, float* dv,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * HSA forward for B independent single-token queries, each after its own
 * cache of T tokens (card, "Core Technique": scoring is O(n/S) per query and
 * attention O(k*S)).  The query sits at position T, so its candidates are
 * all floor(T/S) complete chunks of its cache.
 * q [B,Hq,D], k_cache/v_cache [B,Hkv,T,D], landmarks [B,Hkv,floor(T/S),D],
 * out [B,Hq,D] fp32, sel_idx/sel_score [B,Hq,k] optional (NULL allowed).
 * Caches without a complete chunk (T < S, T = 0 included) are never read,
 * so k_cache, v_cache and landmarks may then be NULL; every query has no
 * candidate and its output is zero.
 * workspace: at least hsa_attn_workspace_size(d, 1) bytes.
 */
hsa_attn_status_t hsa_forward_decode(const hsa_attn_dims_t* d, const void* q, const void* k_cache,
                                     const void* v_cache, const void* landmarks, float* out,
                                     int32_t* sel_idx, float* sel_score, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * hsa_forward_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and results, bit for bit, without a
 * workspace argument.  The scratch memory lives in a fixed 64 MiB array of
 * the library, one copy per GPU, held until the process ends; its device
 * address is looked up once per device on the first call there (call with
 * the stream's device current).  Nothing is allocated, by the library or
 * anything it calls.  A shape whose workspace (hsa_attn_workspace_size(d, 1),
 * or less when sel_idx/sel_score are given) exceeds 64 MiB returns
 * HSA_ATTN_WORKSPACE_TOO_SMALL before any HIP call (both benchmark decodes,
 * 64 x 1M and 4 x 16M tokens, fit).  Every call on one GPU shares that
 * GPU's array: calls that overlap in time on one GPU (different streams or
 * threads without ordering) race and give undefined results.  No part of
 * the array needs to start at zero; it keeps the last call's contents.
 */
hsa_attn_status_t hsa_forward_decode_noalloc(const hsa_attn_dims_t* d, const void* q, const void* k_cache,
                                             const void* v_cache, const void* landmarks, float* out,
                                             int32_t* sel_idx, float* sel_score, void* stream);

/*
 * Decode over a batch of caches of different lengths (incremental decoding;
 * card, "Core Technique": per-query cost O(n/S) for scoring, O(k*S) for
 * attention, so a growing cache is served in place).  d->seq_len is the
 * capacity T_cap of every cache: k_cache/v_cache [B,Hkv,T_cap,D],
 * landmarks [B,Hkv,floor(T_cap/S),D].  cache_lens [B] (device int64,
 * 8-byte aligned) holds each cache's current length; sequence b's query sits
 * at position cache_lens[b] (values outside [0, T_cap] are clamped), so its
 * candidates are its floor(cache_lens[b]/S) complete chunks, whose landmarks
 * must be built.  Otherwise identical to hsa_forward_decode, including the
 * workspace (sized for the capacity) and the outputs.
 */
hsa_attn_status_t hsa_forward_decode_varlen(const hsa_attn_dims_t* d, const void* q, const void* k_cache,
                                            const void* v_cache, const void* landmarks, const int64_t* cache_lens,
                                            float* out, int32_t* sel_idx, float* sel_score, void* workspace,
                                            size_t workspace_bytes, void* stream);

/*
 * Decode with the near-tie adaptive budget (value-of-information router
 * abstract on the automata-index page: a doubled budget for the queries
 * whose k-th and (k+1)-th best scores are closest; read as a per-head
 * threshold on that gap).  Each query
 * head ranks its candidates as hsa_forward_decode does (k = d->top_k) and
 * computes gap = s_k - s_(k+1) from its fp32 scores (1/sqrt(D) included);
 * when it has more than k candidates and gap < gap_threshold it keeps its
 * best min(2k, n) chunks, otherwise its best k (all n if n <= k).
 * Attention and fusion then run over the kept chunks exactly as in
 * hsa_forward_decode, so gap_threshold = 0 reproduces hsa_forward_decode
 * with top_k = k and gap_threshold = +inf reproduces it with top_k = 2k,
 * bit for bit.  gap_threshold must be >= 0 (+inf allowed; NaN or negative:
 * HSA_ATTN_INVALID_ARGUMENT).  Requires k <= 32.
 * cache_lens: NULL (every cache holds d->seq_len tokens) or as in
 * hsa_forward_decode_varlen.  sel_idx/sel_score [B,Hq,2k] (optional): the
 * kept chunks in selection order, -1 / -inf padding (a head that did not
 * double has padding from slot k on).
 * workspace: at least hsa_attn_workspace_size(d, 2) bytes.
 */
hsa_attn_status_t hsa_forward_decode_adaptive(const hsa_attn_dims_t* d, float gap_threshold, const void* q,
                                              const void* k_cache, const void* v_cache, const void* landmarks,
                                              const int64_t* cache_lens, float* out, int32_t* sel_idx,
                                              float* sel_score, void* workspace, size_t workspace_bytes,
                                              void* stream);

/*
 * Append one token per sequence to the caches (card, "Implementation":
 * chunks and their mean-pooled landmarks): k_new/v_new [B,Hkv,D] are written
 * at position cache_lens[b] of k_cache/v_cache [B,Hkv,T_cap,D]
 * (d->seq_len = T_cap); if the token completes chunk c (cache_lens[b] + 1 a
 * multiple of S), landmarks[b,:,c,:] is built exactly as
 * hsa_build_landmarks would; then cache_lens[b] (device int64) advances by
 * one.  A sequence whose cache is full (cache_lens[b] >= T_cap) is left
 * unchanged.  Any chunk size S >= 1; D in {64, 128}.
 */
hsa_attn_status_t hsa_append_kv(const hsa_attn_dims_t* d, const void* k_new, const void* v_new, void* k_cache,
                                void* v_cache, void* landmarks, int64_t* cache_lens, void* stream);

/*
 * Diagnostics: per-launch timing.  After this call, every subsequent
 * forward, landmark or append call made on the calling thread records
 * events[2*i] (hipEvent_t, created by the caller) on its stream just before
 * its i-th kernel launch and events[2*i+1] just after it, for i < n_pairs;
 * the index restarts at 0 with each call.  Each recorded event adds a few
 * microseconds to the call's run on the device.
 * Launch order: landmarks: 1 kernel; prefill, cached and adaptive prefill (when T >= S): V transpose,
 * then per group of up to 64 slabs of query rows (hsa_attn_prefill_slab_rows)
 * zero, select, scan, scatter, then per slab of the group remote attention,
 * local attention (for T < S: select, then local attention per slab);
 * decode and varlen decode: scan, merge,
 * attention, fusion, for adaptive decode too (scan and attention are skipped when the cache capacity
 * holds no complete chunk); append: 1 kernel; backward: zero counts, row
 * preparation, scan, scatter, K transpose, chunk gradients, dq (zero counts,
 * scan, scatter, K transpose and chunk gradients only when T >= S), then zeros
 * for the tokens after the last complete chunk when T is not a multiple of S.  events == NULL or
 * n_pairs == 0 turns recording off.  The setting is thread-local; the events stay owned by the
 * caller and must outlive the calls that record them.
 */
hsa_attn_status_t hsa_attn_set_timing_events(void** events, int n_pairs);

/* Bytes of device workspace a call needs (is_decode: 0 prefill and cached
 * prefill, 1 decode and varlen decode, 2 adaptive-budget decode,
 * 3 adaptive-budget prefill, 4 prefill backward). */
hsa_attn_status_t hsa_attn_workspace_size(const hsa_attn_dims_t* d, int is_decode, size_t* bytes);

/* Static description of a status code. */
const char* hsa_attn_status_string(hsa_attn_status_t status);

/* Thread-local detail about the last failed call on this thread ("" if none). */
const char* hsa_attn_last_error(void);

/* ---------------------------------------------------------------------------
 * Debug build (libhsa_attn_debug.so: the same sources compiled with
 * HSA_ATTN_DEBUG=1).  Every call of the debug library first fills its
 * workspace and its outputs with the word 0x7FC00001 (a quiet NaN as fp32,
 * 2143289345 as int32), so a result that depends on memory the call did not
 * write shows up as NaN or as a failed check; and its kernels check every
 * index they read back from the workspace (chunk indices, pair positions,
 * bucket ranges, pair and row ids) before using it.  A failed check sets
 * its bit below in the call's flag word and the access is skipped (the
 * kernel does not trap).  The flag word is the first 256-byte block of the
 * workspace, which the debug library reserves: its hsa_attn_workspace_size
 * is 256 bytes larger than the release library's, and the calls use the
 * rest of the workspace as the release library uses all of it.  The
 * no-allocation decode keeps the flag word at the start of its scratch.
 * The fills and checks cost time; the release library has neither. */
#define HSA_ATTN_DEBUG_DECODE_ENTRIES   0x001u /* decode: a group's chunk count exceeds its slots */
#define HSA_ATTN_DEBUG_DECODE_CHUNK     0x002u /* decode: a listed chunk outside the cache */
#define HSA_ATTN_DEBUG_DECODE_SLOT      0x004u /* decode: a head's slot number beyond k */
#define HSA_ATTN_DEBUG_SCATTER_CHUNK    0x008u /* prefill bucketing: a selected chunk outside [0, Nc) */
#define HSA_ATTN_DEBUG_SCATTER_POS      0x010u /* prefill bucketing: a pair position beyond its slab's list */
#define HSA_ATTN_DEBUG_REMOTE_RANGE     0x020u /* prefill chunk-major: a bucket range outside its slab's list */
#define HSA_ATTN_DEBUG_REMOTE_ROW       0x040u /* prefill chunk-major: a listed query row out of range */
#define HSA_ATTN_DEBUG_LOCAL_CHUNK      0x080u /* prefill local: a window chunk outside the query's candidates */
#define HSA_ATTN_DEBUG_LOCAL_POS        0x100u /* prefill local: a chunk-major pair position beyond the list */
#define HSA_ATTN_DEBUG_BWD_SCATTER      0x200u /* backward bucketing: a pair position out of range */
#define HSA_ATTN_DEBUG_BWD_PAIR         0x400u /* backward chunks: a bucket range or pair id out of range */

/* Debug library: waits for the device to finish its work, then copies the
 * flag word of the calls that used `workspace` (NULL: the current device's
 * no-allocation decode scratch) into *flags (0: every check passed).  Each
 * call clears the word before its kernels run, so it reports the last call
 * that used the workspace.  The release library returns
 * HSA_ATTN_UNSUPPORTED and leaves *flags unchanged. */
hsa_attn_status_t hsa_attn_debug_flags(const void* workspace, uint32_t* flags);

#ifdef __cplusplus
}
#endif

#endif /* HSA_ATTN_H_ */
