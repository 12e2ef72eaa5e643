/*
 * kvc.h -- paged KV cache and split-K paged GQA decode attention for MI355X (gfx950).
 *
 * C ABI of libkvc.  Plain pointers and sizes only.  Device pointers are
 * borrowed: the library never allocates, frees or retains device memory that
 * is passed in, and the caller keeps it alive until the work queued on the
 * given stream has completed.  Host arrays are read (or written) before the
 * call returns.  Every call returns a kvc_status; on failure nothing has
 * changed (no allocator state, no queued device work) and kvc_last_error()
 * returns a message for the calling thread.
 *
 * The method (pages cited by title and section):
 *  - Decode: one new query token per sequence attends over that sequence's
 *    cached K/V plus its own appended row, softmax(q K^T * scale) V per query
 *    head ("LLM推理优化实战：从KV-Cache到Continuous Batching…" §1.1
 *    attention_step; "苦猿的大模型日记 · Day45 · 大模型推理加速" PART 02).
 *  - GQA: query head h reads KV head h / (num_heads / num_kv_heads)
 *    ("大模型推理加速核心KV Cache 复用机制与内存布局优化" §二; "大模型推理加速——KV Cache篇" §6.2).
 *  - Paging: fixed-size blocks of block_size tokens, reached through a
 *    per-sequence block table; the physical blocks need not be contiguous
 *    ("大模型推理加速核心KV Cache 复用机制与内存布局优化" §三 BlockTable;
 *    "LLM推理优化实战…" §2.2 PageAttentionBlock / RequestBlockTable;
 *    "大模型推理加速——KV Cache篇" §6.1).
 *  - Copy-on-write prefix sharing through refcounted fork (same passages).
 *  - Split-K over KV partitions with an exact merge of the per-partition
 *    (max, sum, acc) triples: the online-softmax recurrence of
 *    "LLM推理优化实战…" §3.2 and the "merge between blocks" a paged kernel needs
 *    ("大模型推理加速核心KV Cache 复用机制与内存布局优化" §四); decode is KV-read bound
 *    ("苦猿的大模型日记" PART 03, Flash-Decoding).
 *
 * ---------------------------------------------------------------------------
 * Pool layout (device memory the caller allocates; sizes from kvc_pool_bytes)
 * ---------------------------------------------------------------------------
 *  Let E = element bytes of the KV dtype (4 f32, 2 f16/bf16, 1 fp8) and
 *  x = 16 / E elements per 16-byte chunk.  A block id names the same block in
 *  every layer and in both pools.
 *    K pool: [num_layers][num_blocks][num_kv_heads][head_dim / x][block_size][x]
 *            (a (block, head) tile is head_dim/x rows of block_size 16-byte chunks)
 *    V pool: [num_layers][num_blocks][num_kv_heads][head_dim][block_size]
 *            (a (block, head) tile is V transposed: token index fastest)
 *    fp8 and int8 only: k_scale, v_scale float32 [num_layers][num_blocks][num_kv_heads];
 *            the value of a stored code c is e4m3(c) * scale.
 *  Token position p of a sequence lives in block table[p / block_size] at
 *  slot p % block_size.  The slots past a sequence's length in its last block
 *  may hold anything, never-written memory included (the pools need no
 *  clearing): the kernels read them but mask them out before they are used.
 *
 * fp8 (E4M3) storage: OCP E4M3 "FN" (bias 7, max 448, S.1111.111 = NaN).
 *  For each write of c new rows into one (layer, block, KV head) that already
 *  holds n0 rows with scale s: s_old = (n0 > 0 ? s : 0);
 *  s_new = max(s_old, amax(new rows) / 448) in IEEE float32; if s_new > s_old
 *  and n0 > 0 the held codes are re-encoded as enc((dec(c) * s_old) / s_new);
 *  new values are stored as enc(x / s_new) (enc(x) when s_new == 0).  enc is
 *  round-to-nearest-even with saturation at +-448.  The pages name E4M3 KV but
 *  give no scale rule; this is the plainest rule that never saturates a
 *  block's largest element.
 *
 * int8 storage: the same rule with 127 in place of 448 and enc(x) = x rounded
 *  to the nearest integer (ties to even), clamped to +-127, stored as a
 *  two's-complement byte; the value of code c is c * scale.  The pages list
 *  INT8 KV quantisation ("LLM推理优化实战…" §6.1, "LLM推理优化核心技术…" §1.2) but
 *  fix no scheme.
 */
#ifndef KVC_H_
#define KVC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t as an opaque pointer (0 = the default stream). */
typedef void* kvc_stream_t;
/* hipEvent_t as an opaque pointer. */
typedef void* kvc_event_t;

typedef enum kvc_status {
  KVC_OK = 0,
  KVC_E_INVALID = 1,      /* bad argument, shape or state; see kvc_last_error() */
  KVC_E_UNSUPPORTED = 2,  /* valid but not implemented (dtype combination, head_dim, block_size) */
  KVC_E_NO_BLOCKS = 3,    /* free list too short: nothing was taken (the caller may preempt and retry) */
  KVC_E_NO_SEQ = 4,       /* unknown sequence id */
  KVC_E_SEQ_EXISTS = 5,   /* sequence id already in use */
  KVC_E_HIP = 6,          /* a HIP runtime call failed */
  KVC_E_WORKSPACE = 7     /* device scratch or workspace smaller than required */
} kvc_status;

typedef enum kvc_dtype {
  KVC_F32 = 0,
  KVC_F16 = 1,
  KVC_BF16 = 2,
  KVC_FP8_E4M3 = 3,
  KVC_INT8 = 4      /* symmetric int8 codes with per-(block, KV head) scales (rule below) */
} kvc_dtype;

typedef struct kvc_config {
  int32_t num_layers;     /* >= 1 */
  int32_t num_kv_heads;   /* >= 1; one block of one layer, num_kv_heads x block_size x head_dim x dtype
                             bytes, below 4 GiB (else KVC_E_UNSUPPORTED) */
  int32_t head_dim;       /* 64 or 128 */
  int32_t block_size;     /* tokens per block; device work needs 16, bookkeeping accepts 1..256 */
  int32_t num_blocks;     /* physical blocks in the pool, >= 1 */
  kvc_dtype kv_dtype;     /* storage dtype of the pools */
  void* k_pool;           /* device, kvc_pool_bytes() bytes; may be NULL for bookkeeping-only use */
  void* v_pool;           /* device, same size as k_pool */
  float* k_scale;         /* device, fp8 and int8 only: kvc_scale_bytes() bytes */
  float* v_scale;         /* device, fp8 and int8 only */
  void* dev_scratch;      /* device, >= kvc_scratch_bytes(max batch, max tokens per append) bytes */
  size_t dev_scratch_bytes;
  const int32_t* free_order; /* host, optional: initial free list (a permutation of
                                0..num_blocks-1); blocks are taken from its END.
                                NULL = 0..num_blocks-1.  Copied at create. */
} kvc_config;

typedef struct kvc_stats_t {
  int64_t total_blocks;
  int64_t free_blocks;
  int64_t used_blocks;      /* blocks with refcount >= 1 */
  int64_t shared_blocks;    /* blocks with refcount >= 2 */
  int64_t peak_used_blocks;
  int64_t cow_copies;       /* block copies issued by copy-on-write */
  int64_t num_seqs;
} kvc_stats_t;

typedef struct kvc_cache kvc_cache;

/* ---- sizing (pure functions) ------------------------------------------- */

/* KV bytes per token: 2 x num_layers x num_kv_heads x head_dim x dtype bytes
 * ("苦猿的大模型日记 · Day45" PART 02).  fp8 scales are not included. */
size_t kvc_bytes_per_token(int32_t num_layers, int32_t num_kv_heads, int32_t head_dim, kvc_dtype dtype);
/* Bytes of ONE pool (K or V) for the layout above. */
size_t kvc_pool_bytes(int32_t num_layers, int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, kvc_dtype dtype);
/* Bytes of ONE fp8 scale array (K or V): 4 x layers x blocks x kv_heads. */
size_t kvc_scale_bytes(int32_t num_layers, int32_t num_blocks, int32_t num_kv_heads);
/* Device scratch an append of max_tokens new rows over max_batch sequences
 * that each receive at least one row needs (its write plan and copy-on-write
 * list); sequences listed with n_new = 0 do not count. */
size_t kvc_scratch_bytes(int32_t max_batch, int64_t max_tokens);

/* ---- handle --------------------------------------------------------------- */

/* Validates cfg and builds the host bookkeeping (free list, refcounts 0).
 * No device work.  *out is owned by the caller; release with kvc_destroy. */
kvc_status kvc_create(const kvc_config* cfg, kvc_cache** out);
void kvc_destroy(kvc_cache* cache);

/* Replace the device scratch kvc_append uses (for instance with a larger one).
 * The caller keeps the old buffer alive until work queued on it has finished. */
kvc_status kvc_set_scratch(kvc_cache* cache, void* dev_scratch, size_t dev_scratch_bytes);

/* ---- bookkeeping (host only, no device work) ------------------------------ */

/* Page 2 allocate: a new sequence with ceil(num_tokens / block_size) blocks
 * reserved (refcount 1 each) and length 0; appends fill reserved blocks first.
 * KVC_E_NO_BLOCKS takes nothing. */
kvc_status kvc_add_seq(kvc_cache* cache, int64_t seq_id, int32_t num_tokens);
/* Page 2 fork: child shares every block of parent (refcount + 1) and its length. */
kvc_status kvc_fork(kvc_cache* cache, int64_t parent_id, int64_t child_id);
/* Page 2 free: every block loses one reference; at 0 it returns to the free list. */
kvc_status kvc_free_seq(kvc_cache* cache, int64_t seq_id);
/* Drop tokens past num_tokens (<= length); blocks past ceil(num_tokens/bs) are
 * released last-first, so re-appending takes the same blocks back.
 * KVC_E_INVALID if the new end would fall inside a block kvc_evict released. */
kvc_status kvc_truncate(kvc_cache* cache, int64_t seq_id, int32_t num_tokens);
/* kvc_truncate of n sequences in one call: seq_ids[i] (host, n distinct ids)
 * to num_tokens[i] (host), applied from the last entry to the first, so that
 * rolling back an append of the same sequences in the same order returns the
 * blocks it took to the free list in the reverse of the order it took them,
 * and a repeat of that append takes the same blocks again.  Every entry is
 * checked first (as kvc_truncate checks it; a repeated id is KVC_E_INVALID);
 * on any failure nothing changes.  For rolling back a batch at once, as a verifier of draft
 * tokens does with the ones it rejects ("LLM推理优化实战…" §4.2: the target
 * model checks every draft token in one pass and keeps the accepted prefix). */
kvc_status kvc_truncate_many(kvc_cache* cache, int32_t n, const int64_t* seq_ids, const int32_t* num_tokens);
/* Sliding-window eviction ("苦猿的大模型日记 · Day45" PART 02: a fixed cache bound
 * paid for with the history that leaves the window).  Every block of the
 * sequence that holds only positions < keep_from (0 <= keep_from <= length)
 * loses this sequence's reference (freed at 0, in table order); its table
 * entry becomes -1, so logical indexing is unchanged and length stays.  With
 * a window w, keep_from = (position of the next query token) - w + 1 keeps
 * every row that token will see; attention calls must then pass that window
 * (a released block is never read inside it).  Forks share only the live
 * blocks; an append never lands in a released block. */
kvc_status kvc_evict(kvc_cache* cache, int64_t seq_id, int32_t keep_from);

/* Reserve slots for n_new[i] new tokens of seq_ids[i] (n_new NULL = 1 each)
 * without moving data: the bookkeeping half of kvc_append.  Sequences are
 * served in call order, positions ascending; a position past the table takes a
 * fresh block, a write into a block with refcount > 1 first takes a private
 * block (copy-on-write; a copy pair is reported when the sequence already has
 * rows in that block).  Ids must be distinct.  On KVC_E_NO_BLOCKS nothing is
 * taken.  slots_out (host, sum(n_new) entries, optional) receives
 * block * block_size + offset per new token in that order; cow_src / cow_dst
 * (host, optional, cow_capacity entries each) receive the copy pairs in the
 * order issued and *num_cow (optional) their count.  There is at most one pair
 * per block written, so batch + sum(n_new) / block_size + 1 entries always
 * suffice; with fewer, a call that needs more fails with KVC_E_INVALID and
 * takes nothing. */
kvc_status kvc_reserve_host(kvc_cache* cache, int32_t batch, const int64_t* seq_ids, const int32_t* n_new,
                            int32_t* slots_out, int32_t* cow_src, int32_t* cow_dst, int32_t cow_capacity,
                            int32_t* num_cow);

/* Host copy of one sequence's table: up to max_blocks ids into blocks_out
 * (-1 for a block kvc_evict released), *num_blocks = table length,
 * *length = tokens written. */
kvc_status kvc_get_table(const kvc_cache* cache, int64_t seq_id, int32_t* blocks_out, int32_t max_blocks,
                         int32_t* num_blocks, int32_t* length);
kvc_status kvc_stats(const kvc_cache* cache, kvc_stats_t* out);
/* The shared-prefix decode's preconditions (kvc_decode_opts.shared_prefix),
 * checked on the tables the handle owns: every one of the batch sequences
 * seq_ids (host, [batch]) exists, holds more than prefix_tokens tokens, and
 * starts with the same prefix_tokens / block_size physical blocks as
 * seq_ids[0] (as after kvc_fork of a prefix_tokens-token sequence, before any
 * write into those blocks), none of them released.  prefix_tokens must be a
 * positive multiple of block_size.  KVC_OK, KVC_E_NO_SEQ, or KVC_E_INVALID
 * naming the first sequence that breaks a condition.  Requests under one
 * system prompt share its physical blocks ("大模型推理加速核心KV Cache 复用机制与
 * 内存布局优化" §三). */
kvc_status kvc_check_shared_prefix(const kvc_cache* cache, int32_t batch, const int64_t* seq_ids,
                                   int32_t prefix_tokens);

/* ---- device work (asynchronous on `stream`) ------------------------------ */

/* Reserve (as kvc_reserve_host) and write: copies every copy-on-write block
 * (all layers, K and V, fp8 / int8 scales) then stores the new rows of every layer in
 * their slots.  With k_new and v_new both NULL (and at most one new token per
 * sequence) only the reservation and the copies are done: the rows are
 * written later, one layer at a time, by kvc_decode_attention (opts k_new /
 * v_new) -- the decode step with its append folded in.  k_new / v_new: device [num_layers][T][num_kv_heads][head_dim]
 * in in_dtype, T = sum(n_new), rows sequence by sequence in call order,
 * positions ascending.  in_dtype must equal kv_dtype, except that an fp8 or int8 cache
 * takes f32, f16 or bf16 rows and quantises them (rule above).  Requires
 * block_size 16, non-NULL pools (and scales for fp8 / int8) and dev_scratch of at
 * least kvc_scratch_bytes(batch, T).  Calls on one handle must use one stream
 * (or the caller orders them): the device scratch is reused call to call. */
kvc_status kvc_append(kvc_cache* cache, int32_t batch, const int64_t* seq_ids, const int32_t* n_new,
                      const void* k_new, const void* v_new, kvc_dtype in_dtype, kvc_stream_t stream);

/* Write the block-table rows and lengths of `batch` sequences into device
 * arrays: block_table [batch][max_blocks] int32 padded with -1, context_lens
 * [batch] int32 = tokens written (after an append, that count includes the
 * new token).  KVC_E_INVALID if a table is longer than max_blocks. */
kvc_status kvc_export_tables(kvc_cache* cache, int32_t batch, const int64_t* seq_ids, int32_t* block_table,
                             int32_t max_blocks, int32_t* context_lens, kvc_stream_t stream);

/* Decode options; pass NULL for the defaults. */
/* Work split of the decode.
 *  MFMA kernel: per KV head, the blocks of all sequences (in batch order) form
 *  one list that is cut into `work_items` equal runs, one wave each.  With
 *  pool_pieces > 0, the last 1/2^pool_shift of every run is further cut into
 *  pool_pieces pieces that the waves of that head take at run time, first come
 *  first served, so waves that progress faster take more of them (a wave's
 *  prefetch runs on into the pieces it takes; on MI355X the balance gains at
 *  most ~1% and costs fp8 caches ~5%, hence off by default).  Each chunk (a run's main part or a
 *  piece) yields one partial (max, sum, acc) per sequence it touches, or the
 *  final output when it holds a whole sequence, and a merge kernel combines
 *  the partials in list order.  Chunk bounds depend only on the lengths and
 *  these options, not on which wave takes a piece, so results are bit-for-bit
 *  reproducible for given options.
 *  FMA kernel: every sequence is cut into partitions of partition_tokens. */
typedef struct kvc_decode_opts {
  int32_t partition_tokens; /* FMA kernel: tokens per partition (multiple of 16, <= 1024); 0 = chosen from the shape */
  int32_t kernel;           /* 0 = auto, 1 = fp32 FMA (VALU) kernel, 2 = MFMA kernel (16-bit and fp8 KV) */
  int32_t work_items;       /* MFMA kernel: waves per KV head; 0 = max(1, W / num_kv_heads) with W = 1024
                               (16-bit and fp8 caches) or 2048 (int8) */
  int32_t pool_pieces;      /* MFMA kernel: pieces per run handed out at run time, <= 64; <= 0 = none
                               (static split, the default); unused when a piece would hold fewer than
                               two turns of the wave's prefetch ring (8 blocks for one-byte codes, 10
                               for 16-bit caches) */
  int32_t pool_shift;       /* MFMA kernel: the pool is the last 1/2^pool_shift of each run, 1..6; 0 = 3 */
  kvc_event_t split_start;  /* optional events recorded on `stream` around the split-K kernel */
  kvc_event_t split_end;
  int32_t window;           /* sliding window (both kernels, decode and several tokens): the token at
                               position p sees positions max(0, p - window + 1) .. p; 0 = all of them */
  int32_t tiles_per_wave;   /* several tokens: 16-column (token, head) tiles each wave holds, 1..4; 0 = auto */
  int32_t shared_prefix;    /* decode, MFMA kernel: 0, or P > 0, a multiple of block_size, when the first P
                               tokens of every sequence are one shared prefix (the same block ids in every
                               block table, as after kvc_fork of a P-token sequence) and every sequence
                               holds more than P tokens.  The prefix is then attended once for the whole
                               batch (its rows read by one pass, the batch's queries its columns, rows of
                               sequence 0's table) and each sequence's own rows apart, and the partials
                               are merged: a cascade split at the fork point, for requests that share one
                               system prompt's physical blocks ("大模型推理加速核心KV Cache 复用机制与内存
                               布局优化" §三; "苦猿的大模型日记 · Day45 · 大模型推理加速" PART 02).  Needs
                               window 0 and no pool; other fields as for decode.  A sequence whose table
                               does not start with sequence 0's P / block_size block ids, or that holds
                               no row past the prefix, gets NaN outputs (nothing faults); seq_ids below
                               turns such a batch into KVC_E_INVALID before any launch. */
  const int64_t* seq_ids;   /* host, optional, [batch]: the cache's ids of the batch's rows (the order of
                               kvc_export_tables).  With shared_prefix > 0 the decode first runs
                               kvc_check_shared_prefix on them and fails as it does; ignored otherwise. */
  const void* k_new;        /* decode only, optional (both or neither): this layer's new K and V rows,  */
  const void* v_new;        /* device [batch][num_kv_heads][head_dim] in q_dtype, written to position
                               context_lens[b] - 1 of every sequence before the attention reads it: the
                               append of a decode step whose slots kvc_append reserved without rows
                               ("苦猿的大模型日记 · Day45" PART 02: add the new token's K/V to the cache, then
                               attend).  With the matrix-core kernel, no pool and a 16-bit cache the walk
                               itself writes them (the wave that reads a sequence's last block writes its
                               newest row first); otherwise an append kernel (with the fp8 / int8 scale
                               rule) runs first.  A length or block id outside the arrays skips the write. */
} kvc_decode_opts;

/* Workspace bytes kvc_decode_attention needs for this shape (the split
 * kernel's partials).  With opts->kernel == 0 it is the larger of the two
 * kernels' needs. */
size_t kvc_decode_workspace_bytes(int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_context_len, const kvc_decode_opts* opts);

/* Decode attention for one layer.
 *  q:            device [batch][num_heads][head_dim], q_dtype (f32 for an f32 cache,
 *                f16 / bf16 for 16-bit caches of the same dtype, bf16 for fp8 and int8)
 *  block_table:  device int32 [batch][max_blocks_per_seq], physical block ids
 *  context_lens: device int32 [batch], tokens to attend per sequence, >= 1,
 *                including the appended token (what kvc_export_tables writes)
 *  max_context_len: host upper bound of context_lens (sizes the grid)
 *  scale:        softmax scale (normally 1/sqrt(head_dim)); finite and >= 0,
 *                else KVC_E_INVALID
 *  out:          device [batch][num_heads][head_dim], q_dtype (rounded to nearest even)
 *  workspace:    device, kvc_decode_workspace_bytes() bytes
 * Checks: num_heads % num_kv_heads == 0 and num_heads / num_kv_heads <= 16,
 * num_kv_heads / head_dim / block_size equal the cache's, block_size 16,
 * batch <= 8192, max_blocks_per_seq x block_size <= 2^31 - 1 and
 * batch x ceil(min(max_context_len, max_blocks_per_seq x block_size) / 16) < 2^30
 * (else KVC_E_UNSUPPORTED).
 * Device-side values are clamped so every access stays inside the arrays the
 * arguments describe: a length above max_context_len or max_blocks_per_seq *
 * block_size is cut to it, a block id outside [0, num_blocks) reads block 0
 * (the result for that sequence is then meaningless, but nothing faults). */
kvc_status kvc_decode_attention(kvc_cache* cache, int32_t layer, const void* q, kvc_dtype q_dtype,
                                const int32_t* block_table, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t max_context_len, int32_t batch,
                                int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                float scale, void* out, void* workspace, size_t workspace_bytes,
                                const kvc_decode_opts* opts, kvc_stream_t stream);

/* Bytes of the static decode workspace kvc_decode_attention_static uses. */
#define KVC_STATIC_SCRATCH_BYTES (32u << 20)

/* kvc_decode_attention without a caller workspace, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid allocation): the partials live in a static device
 * array of KVC_STATIC_SCRATCH_BYTES (32 MiB) that the library's code object
 * holds on each GPU it runs on until the process ends.  The call allocates
 * nothing (no hipMalloc, no hipFree, no allocating library routine); it
 * resolves the array's device address on its first call on a device.
 * Arguments, options, checks and results are those of kvc_decode_attention,
 * bit for bit; a shape whose kvc_decode_workspace_bytes exceeds
 * KVC_STATIC_SCRATCH_BYTES gives KVC_E_WORKSPACE and launches nothing.  Every
 * call on one GPU uses that GPU's one array: calls that overlap on one GPU
 * (two streams, two threads) race and give undefined results; order them.
 * Whatever a call needs zeroed (the pool's ticket counters) it zeroes itself
 * on its stream. */
kvc_status kvc_decode_attention_static(kvc_cache* cache, int32_t layer, const void* q, kvc_dtype q_dtype,
                                       const int32_t* block_table, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t max_context_len, int32_t batch,
                                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                       float scale, void* out, const kvc_decode_opts* opts, kvc_stream_t stream);

/* ---- several new query tokens per sequence --------------------------------- */

/* Attention of several new tokens per sequence over the paged cache: the
 * target model's pass over the draft tokens of speculative decoding (all
 * candidates verified in one forward pass, "LLM推理优化实战：从KV-Cache到Continuous
 * Batching…" §4.2) or one chunk of a chunked prefill (q_len > 1,
 * "苦猿的大模型日记 · Day45" PART 03).  The new tokens' K/V rows are appended first
 * (kvc_append with n_new = the tokens of each sequence); then query token i of
 * sequence b, which sits at position context_lens[b] - ql_b + i, attends
 * causally over rows 0 .. context_lens[b] - ql_b + i of that sequence (the
 * mask of "苦猿的大模型日记" PART 04's naive_attention, the lower triangle shifted
 * by kv_len - q_len).  With one token per sequence this is
 * kvc_decode_attention.
 *  q:            device [total_query][num_heads][head_dim], q_dtype (as for decode)
 *  query_start:  device int32 [batch + 1], non-decreasing, query_start[0] = 0,
 *                query_start[batch] = total_query: the query rows of sequence b
 *                are query_start[b] .. query_start[b + 1] - 1, oldest token first;
 *                ql_b = query_start[b + 1] - query_start[b] may be 0
 *  total_query:  rows of q and out (host)
 *  max_query_len: host upper bound of ql_b, 1..4096 (sizes the grid and the workspace)
 *  context_lens: device int32 [batch], rows cached per sequence including the
 *                ql_b new ones (what kvc_export_tables writes after the append);
 *                ql_b <= context_lens[b]
 *  out:          device [total_query][num_heads][head_dim], q_dtype
 *  workspace:    device, kvc_extend_workspace_bytes() bytes (may be NULL when
 *                that is 0)
 *  opts:         NULL, or kernel: 0 = auto (3 when max_query_len >= 64, else
 *                2); 2 = each KV head's rows split over waves, partials merged
 *                (needs the workspace; work_items = waves per KV head and
 *                column-tile group, tiles_per_wave = 16-column tiles per wave);
 *                3 = one wave per 32 (token, head) columns over every row they
 *                see, outputs written directly (no workspace: 0 bytes).  window
 *                applies to both; the other fields are ignored
 * Other arguments and checks as for kvc_decode_attention; an f32 cache gives
 * KVC_E_UNSUPPORTED (the kernel runs on matrix cores).  Device-side values are
 * clamped as for decode; ql_b is cut to min(max_query_len, context_lens[b]) and
 * rows outside [0, total_query) are neither read nor written, so a malformed
 * query_start gives meaningless rows but nothing faults. */
size_t kvc_extend_workspace_bytes(int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_query_len, int32_t max_context_len, const kvc_decode_opts* opts);
kvc_status kvc_extend_attention(kvc_cache* cache, int32_t layer, const void* q, kvc_dtype q_dtype,
                                const int32_t* query_start, int32_t total_query, int32_t max_query_len,
                                const int32_t* block_table, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t max_context_len, int32_t batch,
                                int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                float scale, void* out, void* workspace, size_t workspace_bytes,
                                const kvc_decode_opts* opts, kvc_stream_t stream);

/* ---- continuous-batching scheduler (host only) ------------------------------ */

/* Iteration-level scheduling of requests over one cache ("LLM推理优化实战…" §5.2:
 * every iteration keeps the unfinished running requests, tops the batch up
 * from the waiting queue, and frees a finished request's KV cache), with
 * recompute preemption when the pool cannot hold an iteration ("苦猿的大模型日记"
 * PART 05: wait, preempt, drop the cache and recompute rather than fail).
 * A request of P prompt tokens producing M tokens writes its K/V rows in
 * position order: the prompt in chunks of at most chunk_tokens, then the row
 * of each token it emitted.  An iteration that brings a request's cache up
 * to every known token (prompt + emitted) emits its next token; it finishes
 * after M (the last token's row is never written) and its blocks are freed.
 * Per iteration: every decoding request gets one row; prefill chunks follow
 * in admission order within max_tokens rows; if the running requests' new
 * blocks do not fit the free list, the most recently admitted one is
 * preempted (its blocks freed, its progress reset, requeued first: on
 * readmission it re-prefills prompt + emitted tokens); then waiting requests
 * are admitted in order while the batch (max_batch), the budget and the pool
 * allow -- the first that does not fit stops admission.  Request ids are the
 * cache's sequence ids.  The caller owns the cache and must not touch the
 * scheduler's sequences except through the plan. */
typedef struct kvc_sched kvc_sched;

typedef struct kvc_sched_config {
  int32_t max_batch;     /* sequences per iteration, >= 1 */
  int32_t chunk_tokens;  /* prefill rows per request per iteration, >= 1 */
  int32_t max_tokens;    /* rows per iteration (prefill chunks are cut to fit), >= 1 */
} kvc_sched_config;

typedef struct kvc_sched_stats {
  int64_t submitted, running, waiting, finished, preemptions, iterations, tokens_scheduled;
} kvc_sched_stats;

kvc_status kvc_sched_create(kvc_cache* cache, const kvc_sched_config* cfg, kvc_sched** out);
void kvc_sched_destroy(kvc_sched* sched);
/* Queue a request (prompt_len >= 1, max_new_tokens >= 1). */
kvc_status kvc_sched_submit(kvc_sched* sched, int64_t req_id, int32_t prompt_len, int32_t max_new_tokens);
/* Plan the next iteration (host arrays of at least max_batch entries):
 * seq_ids[i], n_new[i] rows to append, start[i] = position of the first
 * (optional), emits[i] = 1 if the iteration emits that request's next token
 * (optional); *batch = entries.  Preempted requests' ids go to preempted
 * (optional, up to preempt_capacity; *num_preempted counts all).  The caller
 * then appends the rows (kvc_append with these ids and n_new), runs the
 * attention and calls kvc_sched_commit.  KVC_E_NO_BLOCKS if the pool cannot
 * hold the next rows of even one request (the oldest running one is never
 * preempted to make room for itself; requests preempted on the way stay
 * preempted); KVC_E_INVALID if the previous plan was not committed. */
kvc_status kvc_sched_plan(kvc_sched* sched, int32_t capacity, int64_t* seq_ids, int32_t* n_new, int32_t* start,
                          int32_t* emits, int32_t* batch, int64_t* preempted, int32_t preempt_capacity,
                          int32_t* num_preempted);
/* Record the planned iteration as done (KVC_E_INVALID if the planned rows were
 * not appended); requests that emitted their last token are finished, their
 * blocks freed, their ids written to finished (optional, up to capacity). */
kvc_status kvc_sched_commit(kvc_sched* sched, int64_t* finished, int32_t capacity, int32_t* num_finished);
kvc_status kvc_sched_get_stats(const kvc_sched* sched, kvc_sched_stats* out);

/* ---- measurement helper ---------------------------------------------------- */

/* Streaming copy of `bytes` (multiple of 16) from src to dst on `stream`: a
 * plain copy kernel of known size, used to calibrate HBM byte counters and
 * achievable bandwidth.  Not part of the method. */
kvc_status kvc_stream_copy(void* dst, const void* src, size_t bytes, kvc_stream_t stream);
/* Streaming read of `bytes` (multiple of 16) from src on `stream`, every byte
 * once with non-temporal loads: the achievable HBM read rate that a decode's
 * KV read can be compared with.  Each wave stores the xor of what it read to
 * sink[(wave index) % sink_words] (device, sink_words >= 1 words), so the
 * reads cannot be dropped.  Not part of the method. */
kvc_status kvc_stream_read(const void* src, size_t bytes, uint32_t* sink, size_t sink_words, kvc_stream_t stream);

/* Message describing the last failure on the calling thread ("" if none). */
const char* kvc_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H_ */
