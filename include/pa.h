/*
 * pa.h -- C ABI of libpa, the MI355X (gfx950) paged-KV attention step.
 *
 * One step of the method flattens every running request into a single
 * "super-sequence" of query tokens; each request attends causally to its own
 * tokens only, reading K/V from a cache held in fixed 16-token blocks that a
 * host-side allocator hands out per request (Inside vLLM summary, techfeed.io,
 * section "PagedAttentionの仕組み": block size 16, ceil(tokens/16) blocks per
 * request taken from the head of free_block_queue into req_to_blocks, and the
 * flattened super-sequence with positions and an attention mask).  Prefill
 * chunks and single-token decodes run in the same step (same page, section
 * "エンジンの中核：スケジューラとKVキャッシュ管理"; chunked prefill and prefix
 * caching in section "高度な機能群").
 *
 * Two device calls carry the step:
 *   pa_reshape_and_cache  -- writes the step's new K/V rows into their slots;
 *   pa_attention          -- attention of every query row over its sequence's
 *                            paged K/V, written as float32.
 * Around them: workspace sizing, a host metadata validator, the host block
 * allocator (pa_pool_*), options and a thread-local error string.
 *
 * Conventions shared by every call
 *   - Pointers are device pointers unless marked (host).  All tensors are
 *     dense, row-major, with the shapes given below.  The caller owns every
 *     buffer; the library never allocates or frees device memory and never
 *     synchronises a stream.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Device calls only
 *     enqueue work; the return value reports argument checks and launch
 *     errors.  A kernel fault shows up at the caller's next synchronisation.
 *   - dtype is PA_F32 or PA_BF16 and is the element type of q, k, v and both
 *     caches alike.  Outputs are always float32.
 *   - block_size must be 16; head_dim 64 or 128; num_q_heads a multiple of
 *     num_kv_heads with a group of 1, 2, 4 or 8; num_kv_heads < 2^15;
 *     num_blocks * 16 < 2^31.
 *   - Cache layout: [num_blocks, num_kv_heads, 16, head_dim]; the token at
 *     slot s lives in block s / 16 at offset s % 16, so one (block, kv head)
 *     page of 16 tokens is one contiguous 16*head_dim run.
 *   - Errors: negative pa_status; pa_last_error() then describes the first
 *     problem found, in this thread.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID = -1,      /* bad argument: null pointer, negative size, inconsistent dims */
  PA_ERR_UNSUPPORTED = -2,  /* valid but not built: dtype, head_dim, block_size, group */
  PA_ERR_HIP = -3,          /* the HIP runtime reported an error while launching */
  PA_ERR_WORKSPACE = -4,    /* workspace missing or smaller than pa_attention_workspace_size */
  PA_ERR_NO_BLOCKS = -5     /* allocator: not enough free blocks; nothing was changed */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/* Scatter the step's new K and V rows into the paged caches.
 *
 * The K/V of every token a request holds lives in the 16-token blocks it was
 * given, block by block in token order (Inside vLLM summary, techfeed.io,
 * section "PagedAttentionの仕組み": block size 16, blocks taken per request
 * into req_to_blocks); the step's new tokens are written into their slots
 * before attention reads them.  Slot s = block id * 16 + position % 16 is
 * this library's reading of that layout.
 *
 * For every token n < num_tokens with s = slot_mapping[n] >= 0 and every kv
 * head h:  k_cache[s/16][h][s%16][:] = k[n][h][:]  (and the same for v).
 * The copy is of raw element bits.  A negative slot skips the token.
 *
 *   k, v          [num_tokens, num_kv_heads, head_dim], dtype
 *   slot_mapping  [num_tokens] int32, slots in [0, num_blocks*16) or negative
 *   k_cache, v_cache  [num_blocks, num_kv_heads, 16, head_dim], dtype
 * Slots must be unique within a call (a repeated slot leaves either row).
 * k/v must not alias the caches.  num_tokens == 0 enqueues nothing.  A slot
 * at or past num_blocks*16 is skipped like a negative one; nothing else about
 * the slots is checked on the device (uniqueness needs a device->host copy):
 * use pa_validate_metadata on host copies for that.
 */
int pa_reshape_and_cache(const void* k, const void* v, const int32_t* slot_mapping,
                         void* k_cache, void* v_cache, int32_t num_tokens,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int64_t num_blocks, int32_t dtype, void* stream);

/* Bytes of device workspace pa_attention needs for a step of this shape
 * (work lists, partial results of split rows, counters).  Decoding reads the
 * whole cached context of every request and is bound by memory bandwidth
 * (Inside vLLM summary, section "エンジンの中核：スケジューラとKVキャッシュ管理"),
 * so pa_attention spreads each step's pages evenly over the whole GPU and
 * merges the pieces of rows it splits; the workspace holds those pieces.
 * The pool size does not enter (the pages are reached through block_tables);
 * the group size num_q_heads / num_kv_heads does.  Depends on the
 * arguments, the current device's compute-unit count and the options, so it
 * can be sized once for the largest step and reused.  Returns 0 if the
 * arguments are invalid. */
size_t pa_attention_workspace_size(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim,
                                   int32_t max_blocks_per_seq);

/* Attention of every query row of the step over its own sequence's paged K/V.
 *
 * All requests of a step are flattened into one super-sequence whose
 * positions and attention mask keep each request attending to its own tokens
 * only (Inside vLLM summary, techfeed.io, section "PagedAttentionの仕組み"),
 * and one step mixes prefill chunks with single-token decodes (section
 * "エンジンの中核：スケジューラとKVキャッシュ管理"; chunked prefill in section
 * "高度な機能群").  Causal alignment (a row at position p sees keys 0..p),
 * the GQA mapping and the scale's place before the maximum are this library's
 * readings where the pages are silent.
 *
 * Sequence i owns query rows [query_start_loc[i], query_start_loc[i+1]); its
 * row j sits at absolute position p = context_lens[i] + j and sees the keys at
 * positions 0..p (itself included), read through block_tables[i].  Query head
 * h reads kv head h / (num_q_heads / num_kv_heads).  For each row and head:
 *   out = sum_t softmax_t(scale * <q, K_t>) V_t,  t = 0..p      (float32)
 * for any finite scale (0 weighs every visible key equally; a non-finite
 * scale is PA_ERR_INVALID).
 *
 *   q                [num_tokens, num_q_heads, head_dim], dtype
 *   k_cache, v_cache [num_blocks, num_kv_heads, 16, head_dim], dtype
 *   block_tables     [num_seqs, max_blocks_per_seq] int32; entries past
 *                    ceil(seq_lens[i]/16) are never read (pad with -1)
 *   seq_lens         [num_seqs] int32, = context_lens[i] + query length
 *   query_start_loc  [num_seqs+1] int32, non-decreasing, last = num_tokens
 *   context_lens     [num_seqs] int32, cached tokens before this step
 *   out              [num_tokens, num_q_heads, head_dim] float32
 *   max_query_len    (host) the longest query of the step, as a scheduler
 *                    knows it.  <= 1 routes every row to the row-wise kernel
 *                    and skips the chunk kernel's launch; 2 .. 16 /
 *                    (q heads per kv head) on a bf16 step of at most 512
 *                    rows and sequences makes every sequence row-wise
 *                    records of up to that many rows (PA_OPT_VERIFY_ROWS
 *                    automatic) and skips the plan and chunk kernels; > 1 with
 *                    num_tokens == num_seqs * max_query_len (every sequence
 *                    that long) routes every row to the chunk kernel and skips
 *                    the row-wise kernels' launches.  A wrong value changes
 *                    which kernel computes a row, never the result; pass
 *                    num_tokens if unknown
 *   workspace        device buffer of at least
 *                    pa_attention_workspace_size(...) bytes, 256-B aligned
 * The new K/V of the step must already be in the caches (call
 * pa_reshape_and_cache on the same stream first).  out must not alias any
 * input.  Metadata contents are trusted (see pa_validate_metadata).  Rows of a
 * sequence with no query tokens do not exist; num_tokens == 0 enqueues nothing.
 */
int pa_attention(const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* seq_lens,
                 const int32_t* query_start_loc, const int32_t* context_lens, float scale,
                 float* out, int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                 int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_query_len,
                 int32_t dtype, void* workspace, size_t workspace_bytes, void* stream);

/* pa_attention for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, checks, kernels and results as pa_attention, without the
 * workspace: the library keeps one static device array of
 * PA_NOALLOC_WORKSPACE_MAX bytes per GPU it runs on (held until the process
 * ends) and uses it in place of the caller's buffer.  Calls nothing that
 * allocates.  A step whose pa_attention_workspace_size exceeds
 * PA_NOALLOC_WORKSPACE_MAX is rejected with PA_ERR_WORKSPACE before any launch.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (two streams or two threads at once) race and must be serialised by the
 * caller; calls on the same stream are ordered and safe. */
#define PA_NOALLOC_WORKSPACE_MAX (96u << 20)
int pa_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* seq_lens,
                         const int32_t* query_start_loc, const int32_t* context_lens, float scale,
                         float* out, int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_query_len,
                         int32_t dtype, void* stream);

/* Metadata the kernels had to clamp (a debug read-back).
 *
 * Metadata is trusted on the device, but no kernel indexes outside its
 * buffers even when it is wrong: a block id outside [0, num_blocks) is read
 * as the nearest valid block, and rows or a context inconsistent with
 * num_tokens and max_blocks_per_seq are clamped.  Such a step's outputs are
 * wrong.  Every kernel that clamps ORs a bit into a sticky flag word in the
 * workspace header (no kernel ever clears it):
 *   PA_FLAG_BLOCK_ID  a block id outside the pool was met;
 *   PA_FLAG_ROWS      a sequence's query_start_loc / context_lens entries were
 *                     inconsistent with the step (rows outside [0, num_tokens),
 *                     a negative count or context, more keys than its block-table
 *                     row holds) and were clamped.  seq_lens is not read on the
 *                     device; pa_validate_metadata checks it.
 * pa_attention_flags waits for `stream`, writes the word to *flags (host,
 * may be NULL) and, if clear != 0, zeroes it (enqueued on `stream`).  The
 * word is undefined in a fresh workspace: clear it once before the first step
 * whose flags will be read.  workspace NULL means the current device's
 * static workspace of pa_attention_noalloc (which starts at zero).  Not for
 * use under graph capture (it synchronises and enqueues a memset). */
enum { PA_FLAG_BLOCK_ID = 1, PA_FLAG_ROWS = 2 };
int pa_attention_flags(const void* workspace, int32_t* flags, int32_t clear, void* stream);

/* Check step metadata on host copies, O(num_tokens + num_seqs*max_blocks).
 *   seq_lens[i] == context_lens[i] + (query_start_loc[i+1]-query_start_loc[i]) >= 0,
 *   query_start_loc[0] == 0, non-decreasing, query_start_loc[num_seqs] == num_tokens,
 *   ceil(seq_lens[i]/16) <= max_blocks_per_seq, used block ids in [0, num_blocks),
 *   slot_mapping (may be NULL) in range or negative, and unique.
 * All pointers are (host).  Returns PA_OK or PA_ERR_INVALID with a message. */
int pa_validate_metadata(const int32_t* block_tables, const int32_t* seq_lens,
                         const int32_t* query_start_loc, const int32_t* context_lens,
                         const int32_t* slot_mapping, int32_t num_seqs, int32_t num_tokens,
                         int32_t max_blocks_per_seq, int64_t num_blocks, int32_t block_size);

/* Message of the last error raised in this thread ("" if none). */
const char* pa_last_error(void);

/* Tuning and debug options (process-wide).  Returns PA_OK or PA_ERR_INVALID. */
enum {
  PA_OPT_FORCE_ROWWISE = 1,  /* 1: every query row takes a row-wise kernel (the chunk kernel is off) */
  PA_OPT_SPLIT_TOKENS = 2,   /* >0: each decode wavefront range covers this many tokens' worth of
                                (row, kv head) pages (multiple of 16); 0: automatic, the step's
                                pages spread evenly over the resident wavefronts */
  PA_OPT_TARGET_ITEMS = 3,   /* >0: number of decode ranges in automatic mode; 0: one per
                                resident wavefront (VALU kernel) or per wavefront of one
                                workgroup per CU (MFMA kernel) */
  PA_OPT_DECODE_BUFFERS = 4, /* pages a decode wavefront holds at once (the page being scored
                                plus the ones in flight): VALU kernel 1 or 2, MFMA kernel 2..4
                                (a decode-only step the MFMA kernel plans itself always holds
                                2); 0 or a value the kernel does not take: automatic */
  PA_OPT_DECODE_KERNEL = 5,  /* row-wise rows of bf16 steps: 0 automatic (MFMA), 1 VALU kernel,
                                2 MFMA kernel; float32 steps always take the VALU kernel */
  PA_OPT_VERIFY_ROWS = 6,    /* bf16 steps with the MFMA row-wise kernel: a sequence with 2..n
                                query rows (a short query, e.g. speculative-decoding verification)
                                is one row-wise work item whose rows share every K/V page instead
                                of chunk tiles; n = this value capped at 16 / (q heads per kv
                                head); 1: off; 0 (automatic): n = 16 / (q heads per kv head) on
                                steps of at most 512 rows and sequences whose max_query_len is
                                at most that (the row-wise kernel plans them by itself, no chunk
                                kernel runs), off on other steps.  Values >= 2 change the
                                workspace size */
  PA_OPT_CHUNK_KERNEL = 7    /* bf16 chunk rows: 0 (automatic) and 1: the four-wavefront chunk
                                kernel; 2: the eight-wavefront kernel (two groups alternating
                                products and softmax) for every step with chunk rows, the plan
                                kernel then planning every step.  Both compute the same rows */
};
int pa_set_option(int32_t option, int64_t value);
int64_t pa_get_option(int32_t option);

/* Kernel timing for measurement (process-wide).  pa_profile_enable(mask)
 * turns on HIP-event timing of the kernel kinds whose bit (1 << kind) is set
 * in mask: each such launch made by pa_reshape_and_cache / pa_attention is
 * bracketed by two events recorded on the call's stream.  pa_profile_read
 * waits for the recorded events, writes per kind the number of timed launches
 * and their summed duration in milliseconds into counts / total_ms (host
 * arrays of PA_K_COUNT entries, either may be NULL) and clears the record.
 * mask 0 (the default) records nothing. */
enum { PA_K_RESHAPE = 0, PA_K_PLAN = 1, PA_K_CHUNK = 2, PA_K_DECODE = 3, PA_K_MERGE = 4, PA_K_COUNT = 5 };
int pa_profile_enable(int32_t mask);
int pa_profile_read(int64_t* counts, double* total_ms);

/* ---------------- host block allocator ----------------
 * The allocation procedure of the Inside vLLM summary, section
 * "PagedAttentionの仕組み": a request that will hold T tokens needs
 * ceil(T/block_size) blocks; the missing ones are taken from the head of the
 * free-block queue and appended to the request's block list.  If the queue
 * holds too few, the call fails with PA_ERR_NO_BLOCKS and changes nothing;
 * the caller chooses whom to preempt.  Releasing a request drops one reference
 * from each of its blocks (in list order) and appends blocks that reach zero
 * references to the tail of the queue.  Requests may share already allocated
 * blocks (a cached prompt prefix), which adds one reference per block.
 * Everything here is host-only and not thread-safe per pool.
 */
typedef struct pa_pool pa_pool;

/* initial_order (host, num_blocks entries, a permutation of 0..num_blocks-1)
 * is the starting order of the free queue; NULL means 0, 1, 2, ...
 * Returns NULL on bad arguments (see pa_last_error). */
pa_pool* pa_pool_create(int64_t num_blocks, int32_t block_size, const int32_t* initial_order);
void pa_pool_destroy(pa_pool* pool);

/* Grow request `req` to hold num_computed + num_new tokens.  The ids of the
 * blocks added (possibly none) are written to new_ids_out (host, capacity
 * `cap`, may be NULL when cap == 0 and the caller does not need them) and
 * their count to *n_out (host, may be NULL). */
int pa_allocate_slots(pa_pool* pool, int64_t req, int64_t num_computed, int64_t num_new,
                      int32_t* new_ids_out, int32_t cap, int32_t* n_out);
/* Append n allocated blocks (host ids) to request `req`, one reference each. */
int pa_share_prefix(pa_pool* pool, int64_t req, const int32_t* ids, int32_t n);
/* Release every block reference of `req` and forget it (unknown req: no-op). */
int pa_free(pa_pool* pool, int64_t req);
/* Prefix cache (Inside vLLM summary, section "高度な機能群", Prefix Caching: a
 * request that starts with the same prompt reuses the cached KV blocks; the
 * block pool holds the index).  A full block may be registered under a 64-bit
 * key the caller computes (e.g. a hash of its tokens chained with the previous
 * block's key).  A block released to zero references keeps its key and stays
 * findable until the free queue hands it out again, which drops the key.
 *
 * pa_prefix_match: for a request holding no blocks, append the blocks cached
 * under keys[0], keys[1], ... up to the first miss, one reference each (a
 * released block is taken out of the free queue); *n_hit (host) receives the
 * number of blocks reused.  keys: host, n entries.
 * pa_prefix_register: register the request's first n blocks under keys[0..n)
 * (host); a key already cached for another block keeps that block; a block
 * already cached under a different key is an error (PA_ERR_INVALID, nothing
 * changed).  pa_prefix_cached: blocks in the index (-1 for a null pool). */
int pa_prefix_match(pa_pool* pool, int64_t req, const uint64_t* keys, int32_t n, int32_t* n_hit);
int pa_prefix_register(pa_pool* pool, int64_t req, const uint64_t* keys, int32_t n);
int64_t pa_prefix_cached(const pa_pool* pool);
int64_t pa_num_free(const pa_pool* pool);
/* Number of blocks request `req` holds (0 if unknown). */
int32_t pa_num_req_blocks(const pa_pool* pool, int64_t req);
/* Reference count of one block (negative on a bad id). */
int32_t pa_refcount(const pa_pool* pool, int32_t block);
/* Write the request's block ids into out (host, `width` entries), padding the
 * rest with pad_value.  PA_ERR_INVALID if the request holds more than width. */
int pa_block_table_row(const pa_pool* pool, int64_t req, int32_t* out, int32_t width,
                       int32_t pad_value);
/* Slots of positions start_pos..start_pos+n-1 of `req` into out (host, n
 * entries): block_list[pos/block_size]*block_size + pos%block_size. */
int pa_slot_mapping(const pa_pool* pool, int64_t req, int64_t start_pos, int32_t n, int32_t* out);

#ifdef __cplusplus
}
#endif
#endif /* PA_H */
