/*
 * pagedkv.h -- C ABI of libpagedkv: attention over a paged KV cache on AMD
 * Instinct MI355X (gfx950).
 *
 * The operation is the serving-engine step the pages describe:
 *   - "PyTorch LLM Serving Engine", section Loading: the new keys and values
 *     of a layer are stored in the cache first; the attention then visits the
 *     sequence's blocks in table order with an online softmax (a running
 *     maximum keeps every exponential bounded); section What is implemented:
 *     a pool of equal-sized blocks, a block-id table for each sequence,
 *     prefill in chunks.
 *   - "MicroGen: Modular, Hardware-Aware LLM Inference Engine", section Key
 *     Features: logical-to-physical block mapping, grouped-query attention
 *     (each KV head serves a group of query heads), dynamic per-vector INT8 KV
 *     quantisation, window-length eviction for long contexts.
 *   - "llminfer", section Paged KV Cache And Continuous Batching: 16-token pages.
 *
 * Conventions for every entry point
 *   - Tensor arguments are DEVICE pointers to dense row-major arrays; scalars
 *     are passed by value.  `stream` is a hipStream_t (NULL: the null stream).
 *   - Calls only enqueue work on `stream`; they never synchronise.  The caller
 *     owns every buffer and keeps it alive until that work has completed.
 *   - The library allocates no device memory and keeps no per-call state (the
 *     block allocator below is host state the caller creates and owns).
 *   - Return value: PKV_OK (0) or a pkv_status.  Host-visible arguments are
 *     validated before anything is enqueued; on failure nothing is enqueued
 *     and pkv_last_error() describes the problem.  No exception crosses the ABI.
 *   - Device-resident integers (slots, block ids, lengths) are read by the
 *     kernels: out-of-range slots and block ids are skipped rather than
 *     dereferenced, lengths are clamped to what a table row addresses,
 *     (max_blocks_per_seq + its table offset) * block_size.
 *     Setting the environment variable PKV_VALIDATE=1 makes every call copy
 *     them to the host first (synchronising) and reject bad values with
 *     PKV_EINVAL.
 *
 * Cache layout (one layer)
 *   K pool and V pool: [num_blocks][num_kv_heads][block_size][head_dim] of
 *   kv_dtype, so each (block, KV head) tile is one contiguous run.  The token
 *   at position p of sequence s lives in slot
 *       slot = block_tables[s][p / block_size] * block_size + p % block_size,
 *   i.e. in physical block slot / block_size at offset slot % block_size.
 *   INT8 pools add scale pools [num_blocks][num_kv_heads][block_size] of fp16
 *   bit patterns (one scale per token and KV head).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  Zero is deliberately not a valid type. */
typedef enum {
    PKV_F32 = 1,   /* IEEE binary32 */
    PKV_BF16 = 2,  /* bfloat16 */
    PKV_I8 = 4     /* signed 8-bit code with a per-vector fp16 scale (pools only) */
} pkv_dtype;

typedef enum {
    PKV_OK = 0,
    PKV_EINVAL = 1,       /* an argument is malformed (null pointer, negative size, ...) */
    PKV_EUNSUPPORTED = 2, /* well-formed but not implemented (dtype pair, head_dim, block_size) */
    PKV_EWORKSPACE = 3,   /* workspace missing or smaller than the query function's answer */
    PKV_EHIP = 4,         /* the HIP runtime reported an error (text in pkv_last_error) */
    PKV_ENOSPACE = 5      /* the block allocator has too few free blocks (nothing was changed) */
} pkv_status;

/* Shape and element type of one layer's cache. */
typedef struct {
    int32_t num_blocks;    /* physical blocks in each pool, > 0 */
    int32_t block_size;    /* tokens per block; 16 is supported */
    int32_t num_kv_heads;  /* KV heads, > 0 */
    int32_t head_dim;      /* 64 or 128 */
    int32_t kv_dtype;      /* PKV_F32, PKV_BF16 or PKV_I8 */
} pkv_cache_desc;

/*
 * kv_cache_write -- store new K/V vectors in their physical slots.
 * ("PyTorch LLM Serving Engine", Loading: new keys and values enter the cache
 * before attention reads them; "MicroGen", Key Features: dynamic per-vector
 * INT8.)
 *
 *   k, v          [num_tokens][num_kv_heads][head_dim] of in_dtype, consecutive
 *                 tokens token_stride elements apart (>= num_kv_heads*head_dim
 *                 for a packed array; a larger stride reads K/V in place out of
 *                 a fused QKV buffer).  16-byte aligned, token_stride * element
 *                 size a multiple of 16 bytes.
 *   slot_mapping  [num_tokens] int32; slot < 0 means "do not store".  Slots are
 *                 unique within one call (otherwise which write wins is
 *                 unspecified).
 *   k_pool/v_pool the pools of `cache`.
 *   k_scale/v_scale  fp16 scale pools; required iff cache->kv_dtype == PKV_I8,
 *                 NULL otherwise.
 * Type pairs: (F32 -> F32) and (BF16 -> BF16) copy the bits; (F32|BF16 -> I8)
 * quantises each (token, head) vector: a = max|x| (fp32), scale =
 * fp16_rne(a / 127) with an IEEE fp32 division, code = clamp(rne(x / scale),
 * -127, 127) with IEEE fp32 divisions (all codes 0 when the scale is 0).
 * num_tokens == 0 is a no-op.
 */
int kv_cache_write(const pkv_cache_desc* cache,
                   const void* k, const void* v, int32_t in_dtype, int64_t token_stride,
                   const int32_t* slot_mapping, int32_t num_tokens,
                   void* k_pool, void* v_pool, void* k_scale, void* v_scale,
                   void* stream);

/*
 * Bytes of workspace paged_attention_decode needs for these sizes.  Zero when
 * partition_size is 0 (single pass) or one partition covers every key a row
 * can address.  with_table_offsets: nonzero if the call passes table_offsets
 * (a row's keys may then straddle one more partition).  Returns 0 for invalid
 * sizes (the decode call then reports the error).
 */
size_t paged_attention_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                             int32_t head_dim, int32_t max_blocks_per_seq,
                                             int32_t block_size, int32_t partition_size,
                                             int32_t with_table_offsets);

/*
 * paged_attention_decode -- one query token per sequence.
 * ("PyTorch LLM Serving Engine", Loading and What is implemented: an online
 * softmax over the sequence's blocks in table order; "MicroGen", Key
 * Features: GQA by KV-head repetition, window-length limit.)
 *
 * For sequence s with L = context_lens[s] tokens (the current token, already
 * written by kv_cache_write, included) and query head h, with
 * G = num_q_heads / cache->num_kv_heads and g = h / G:
 *     p = L - 1;  keys j with 0 <= j <= p and, if sliding_window W > 0, j > p - W
 *     out[s][h] = sum_j softmax_j(softmax_scale * q[s][h] . K_s[j][g]) V_s[j][g]
 * where K_s[j] is the pool row at sequence position j.  A table entry that is
 * not a block of the pool (-1 after eviction or rollback, or an id outside
 * [0, num_blocks)) holds no keys: its positions take no part in the softmax.
 * L == 0, or no key left at all, gives a zero row.
 *
 *   q             [num_seqs][num_q_heads][head_dim]; BF16 for BF16 pools,
 *                 F32 for F32 pools, BF16 or F32 for INT8 pools.
 *   out           [num_seqs][num_q_heads][head_dim] of out_dtype (F32 or BF16).
 *   k_scale/v_scale  INT8 pools only, else NULL.
 *   block_tables  [num_seqs][max_blocks_per_seq] int32 physical block ids;
 *                 entries past ceil(L / block_size) are never used, and with a
 *                 window neither are entries wholly before it (they may be -1
 *                 after pkv_seq_evict_window).  Every entry of the array must
 *                 be readable: a single-pass call (no partitions) with no
 *                 window and no table_offsets reads a row's leading entries
 *                 before it knows L, and ignores those past it.
 *   table_offsets NULL, or [num_seqs] int32 >= 0: column c of row s holds
 *                 logical block c + table_offsets[s], so a windowed sequence's
 *                 row can drop its released blocks (pkv_seq_compact) and stay
 *                 max_blocks_per_seq wide however long the context grows.
 *                 Keys of blocks before the offset do not exist for the call:
 *                 the window must exclude them.  L is clamped to
 *                 (max_blocks_per_seq + offset) * block_size.
 *   context_lens  [num_seqs] int32.
 *   partition_size  0: each sequence in one pass.  Otherwise a positive
 *                 multiple of block_size: contexts are split into partitions
 *                 of that many keys, attended independently and merged by a
 *                 second kernel (log-sum-exp), which needs `workspace`.
 *   workspace     device scratch of at least
 *                 paged_attention_decode_workspace_size(...) bytes, 256-byte
 *                 aligned; may be NULL when that size is 0.  Its first 256
 *                 bytes hold a work counter that must be ZERO before the
 *                 first call that uses the workspace (allocate it zeroed);
 *                 every call leaves the counter at zero again when its work
 *                 completes, so a workspace can be reused call after call
 *                 with no clearing (and no extra launch, so the call can be
 *                 captured in a graph).  The rest holds split-K partial
 *                 results, not preserved between calls.  With
 *                 PKV_VALIDATE=1 a non-zero counter is rejected (PKV_EINVAL).
 *                 Two calls in flight at once must not share a workspace.
 * num_seqs == 0 is a no-op.  out must not alias any input or the workspace.
 */
int paged_attention_decode(const pkv_cache_desc* cache,
                           const void* q, int32_t q_dtype,
                           void* out, int32_t out_dtype,
                           int32_t num_seqs, int32_t num_q_heads,
                           const void* k_pool, const void* v_pool,
                           const void* k_scale, const void* v_scale,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* table_offsets,
                           const int32_t* context_lens,
                           float softmax_scale, int32_t sliding_window,
                           int32_t partition_size,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * paged_attention_decode_noalloc -- paged_attention_decode for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments and results as
 * paged_attention_decode (same kernels), without the workspace: the split-K
 * partial results and the work counter live in a fixed device array of the
 * library, of paged_attention_decode_noalloc_max_scratch() bytes (32 MiB),
 * one copy on each GPU it runs on, held until the process ends.  Nothing is
 * allocated or freed by the call.  A call whose workspace size
 * (paged_attention_decode_workspace_size) exceeds that maximum is rejected
 * with PKV_EWORKSPACE before anything is enqueued.  The first call on a GPU
 * looks the array up there and clears its work counter with a kernel on
 * `stream`; every call leaves the counter at zero.  All calls on one GPU
 * share the array: calls that overlap in time on one GPU (other streams,
 * other threads) race and give wrong results; serialise them.
 */
int paged_attention_decode_noalloc(const pkv_cache_desc* cache,
                                   const void* q, int32_t q_dtype,
                                   void* out, int32_t out_dtype,
                                   int32_t num_seqs, int32_t num_q_heads,
                                   const void* k_pool, const void* v_pool,
                                   const void* k_scale, const void* v_scale,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* table_offsets,
                                   const int32_t* context_lens,
                                   float softmax_scale, int32_t sliding_window,
                                   int32_t partition_size,
                                   void* stream);

/* Bytes of the fixed scratch paged_attention_decode_noalloc uses on each GPU. */
size_t paged_attention_decode_noalloc_max_scratch(void);

/*
 * paged_attention_prefill_chunk -- a chunk of new query tokens per sequence.
 * ("PyTorch LLM Serving Engine", What is implemented: chunked prefill sharing
 * the step with decode work; Loading: write, then attend over the block table.)
 *
 * Sequence s owns query rows [cu_q_lens[s], cu_q_lens[s+1]), C_s of them, and
 * has L_s = seq_lens[s] tokens in the cache, its C_s new ones included (they
 * were written by kv_cache_write first).  Row i sits at position
 * p = L_s - C_s + i and attends to keys j <= p (and j > p - W when
 * sliding_window W > 0), with the same formula as the decode call.
 *
 *   q             [total_rows][num_q_heads][head_dim] BF16 (total_rows =
 *                 cu_q_lens[num_seqs]).
 *   out           [total_rows][num_q_heads][head_dim] of out_dtype (F32 or BF16).
 *   cu_q_lens     [num_seqs + 1] int32 prefix sums, cu_q_lens[0] == 0.
 *   max_q_len     host-side upper bound of every C_s (sizes the grid); rows of
 *                 a longer chunk beyond max_q_len are not computed.
 *   seq_lens      [num_seqs] int32, L_s >= C_s.
 *   block_tables  as for decode; with a window, entries wholly before the
 *                 first row's window may be -1 (evicted): they hold no key
 *                 any row can see.
 *   table_offsets NULL, or per-sequence offsets as for decode.
 *   k_scale/v_scale  INT8 pools only (16-byte aligned), else NULL.
 * Pools are BF16 or INT8 ("MicroGen", Key Features: dynamic per-vector INT8
 * KV).  Q.K^T is exact in both (bf16 products, fp32 sums); P.V runs on fp16
 * matrix instructions with fp32 accumulation, which sets two range limits:
 *   - BF16 pools: V is converted to fp16 for P.V.  V values must satisfy
 *     |v| <= 65504 (a larger value becomes inf and the row's output is not
 *     finite).  Values with |v| < 2^-14 land on fp16's subnormal grid: each
 *     is off by at most 2^-25 in absolute terms (so the output's absolute
 *     error bound holds, but an output made only of such values can exceed
 *     the 1e-2 relative bound).  Values in between convert exactly.
 *   - INT8 pools: codes are exact in fp16; each V scale is folded into its
 *     key's softmax weight, carried in two fp16 parts (~22 significant
 *     bits).  Weights reach 256 before a rescale, so V scales must be <= 255
 *     (|values| <= 32385).
 * The decode call has neither limit (its products run in fp32).
 * A table entry that holds no block holds no keys, as for decode.
 * num_seqs == 0 or max_q_len == 0 is a no-op.
 */
int paged_attention_prefill_chunk(const pkv_cache_desc* cache,
                                  const void* q, int32_t q_dtype,
                                  void* out, int32_t out_dtype,
                                  const int32_t* cu_q_lens, int32_t num_seqs,
                                  int32_t max_q_len, int32_t num_q_heads,
                                  const void* k_pool, const void* v_pool,
                                  const void* k_scale, const void* v_scale,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* table_offsets,
                                  const int32_t* seq_lens,
                                  float softmax_scale, int32_t sliding_window,
                                  void* stream);

/*
 * pkv_build_slot_mapping -- the cache slot of every new row of a step, on the
 * device, from the block tables.
 * ("MicroGen", Key Features: logical blocks map to physical blocks through the
 * sequence's table; "PyTorch LLM Serving Engine", Loading: every new key/value
 * vector has a cache position of its own.)
 *
 * Sequence s owns rows [cu_q_lens[s], cu_q_lens[s+1]) (C_s of them: 1 for a
 * decode step, the chunk length for prefill) and holds L_s = seq_lens[s]
 * tokens once they are written, so row i sits at position p = L_s - C_s + i:
 *     slot_mapping[row] = block_tables[s][p / block_size - o_s] * block_size + p % block_size
 * with o_s = table_offsets[s] (0 when table_offsets is NULL), or -1
 * (kv_cache_write then skips the row) when p < 0, the column is outside
 * [0, max_blocks_per_seq), or the table entry is outside [0, num_blocks).
 *
 *   cu_q_lens     [num_seqs + 1] int32 prefix sums, cu_q_lens[0] == 0.
 *   seq_lens      [num_seqs] int32.
 *   block_tables  [num_seqs][max_blocks_per_seq] int32.
 *   slot_mapping  [total_rows] int32 output; rows at or past total_rows are
 *                 not written (total_rows is the array's length, normally
 *                 cu_q_lens[num_seqs]).
 * Only cache->num_blocks and cache->block_size are used.  num_seqs == 0 or
 * total_rows == 0 is a no-op.
 */
int pkv_build_slot_mapping(const pkv_cache_desc* cache, const int32_t* cu_q_lens, int32_t num_seqs,
                           const int32_t* seq_lens, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* table_offsets, int32_t* slot_mapping, int32_t total_rows,
                           void* stream);

/*
 * kv_cache_copy_blocks -- copy whole physical blocks: for each pair n, block
 * dst_blocks[n] of the K pool, the V pool and (INT8) both scale pools becomes
 * a copy of block src_blocks[n], every KV head and slot.  A sequence that
 * shares a partly filled block with another (a forked prefix, "MicroGen", Key
 * Features) copies it before writing into it; pkv_seq_append names the pairs.
 *
 *   src_blocks, dst_blocks  [num_pairs] int32 device arrays.  A pair naming a
 *                 block outside [0, num_blocks) is skipped.  Destinations must
 *                 be distinct and no destination may be the source of another
 *                 pair (otherwise the result is unspecified).
 *   k_scale/v_scale  INT8 pools only (4-byte aligned), else NULL.
 * num_pairs == 0 is a no-op.
 */
int kv_cache_copy_blocks(const pkv_cache_desc* cache, void* k_pool, void* v_pool, void* k_scale, void* v_scale,
                         const int32_t* src_blocks, const int32_t* dst_blocks, int32_t num_pairs, void* stream);

/*
 * Block allocator -- host-side owner of a pool's physical blocks ("PyTorch LLM
 * Serving Engine", What is implemented: the pool is cut into blocks of one
 * size, and each sequence lists its blocks in a table).  Free blocks are kept on a stack (O(1)
 * per block); every block carries a reference count so that sequences can
 * share blocks (a forked prefix) and a block is free again when its count
 * drops to zero.  The allocator touches no device memory: table rows are HOST
 * int32 arrays the caller owns and copies to the device for the kernels.
 * Entries that hold no block are -1.  Every call validates first and changes
 * nothing on failure.  One allocator must not be used by two threads at once.
 */
typedef struct pkv_block_allocator pkv_block_allocator;

/* New allocator for blocks 0 .. num_blocks-1, all free; *out is NULL on failure. */
int pkv_allocator_create(int32_t num_blocks, int32_t block_size, pkv_block_allocator** out);
/* Free the allocator (NULL is allowed). */
int pkv_allocator_destroy(pkv_block_allocator* a);
/* Number of free blocks (-1 for NULL). */
int32_t pkv_allocator_num_free(const pkv_block_allocator* a);
/* References held on `block` (0 = free; -1 for an id outside the pool). */
int32_t pkv_allocator_refcount(const pkv_block_allocator* a, int32_t block);
/* Take n free blocks into ids[0..n) (count 1 each); PKV_ENOSPACE if fewer are free. */
int pkv_allocator_alloc(pkv_block_allocator* a, int32_t n, int32_t* ids);
/* One more reference on each allocated block of ids (negative ids are skipped). */
int pkv_allocator_retain(pkv_block_allocator* a, const int32_t* ids, int32_t n);
/* Drop one reference on each block of ids (negative ids skipped); a block whose
 * count reaches 0 is free.  Releasing more references than held: PKV_EINVAL. */
int pkv_allocator_release(pkv_block_allocator* a, const int32_t* ids, int32_t n);

/*
 * pkv_seq_append -- make room for num_new tokens after the len tokens of a
 * sequence whose table row is table_row[0 .. max_blocks_per_seq).  Blocks are
 * allocated for the logical blocks that positions len .. len+num_new-1 start.
 * If position len falls inside a block that other sequences also hold (count
 * > 1), that entry is replaced by a fresh block and the pair (old, fresh) is
 * returned in copy_src[0], copy_dst[0] with *num_copies = 1 (else 0): the
 * caller copies it with kv_cache_copy_blocks before the cache write.  The slot
 * of each new token then follows from the table (pkv_build_slot_mapping).
 * copy_src and copy_dst hold at least one entry.  PKV_ENOSPACE if the pool
 * cannot supply every block needed.
 */
int pkv_seq_append(pkv_block_allocator* a, int32_t* table_row, int32_t max_blocks_per_seq, int32_t len,
                   int32_t num_new, int32_t* copy_src, int32_t* copy_dst, int32_t* num_copies);

/*
 * pkv_seq_fork -- a new sequence that shares the first len tokens of a parent
 * (prefix reuse, "MicroGen", Key Features): child_row receives the parent's
 * ceil(len / block_size) entries, each block gains a reference, and the rest
 * of child_row[0 .. max_blocks_per_seq) is set to -1.  No bytes are copied;
 * the attention kernels read shared blocks like private ones.
 */
int pkv_seq_fork(pkv_block_allocator* a, const int32_t* parent_row, int32_t len, int32_t* child_row,
                 int32_t max_blocks_per_seq);

/*
 * pkv_seq_truncate -- roll a sequence back from len to new_len tokens (rejected
 * draft tokens of speculative decoding, "MicroGen", Key Features): entries
 * from ceil(new_len / block_size) to ceil(len / block_size) are released and
 * set to -1.  Positions >= new_len inside the kept last block are simply
 * overwritten by the next append.  Also frees a whole sequence (new_len 0).
 * table_row must hold at least ceil(len / block_size) entries.
 */
int pkv_seq_truncate(pkv_block_allocator* a, int32_t* table_row, int32_t len, int32_t new_len);

/*
 * pkv_seq_evict_window -- window-length eviction ("MicroGen", Key Features):
 * once a sequence holds len tokens, every later query sits at position >= len
 * and, with sliding window W, sees only keys j > len - W.  The blocks wholly
 * before that, entries 0 .. floor((len - W + 1) / block_size) - 1, are
 * released and set to -1; *num_released (may be NULL) counts the entries
 * released by this call.  The attention calls never read an entry before the
 * window, and treat an entry of -1 as no keys, so their results are unchanged
 * as long as they run with the same window.  table_row must hold at least
 * ceil(len / block_size) entries.
 */
int pkv_seq_evict_window(pkv_block_allocator* a, int32_t* table_row, int32_t len, int32_t window,
                         int32_t* num_released);

/*
 * pkv_seq_compact -- drop the released (-1) entries at the start of a table row
 * and add their count to the row's offset (*table_offset; 0 for a row that
 * starts at logical block 0), so a windowed sequence keeps a row of bounded
 * width however long it grows; the attention calls and
 * pkv_build_slot_mapping take the offsets as table_offsets.  A row of only
 * -1 entries is left as it is.  The pkv_seq_* calls above work on an offset
 * row when given lengths minus offset * block_size (they address the row's
 * columns).  Host memory only; no allocator state is touched.
 */
int pkv_seq_compact(int32_t* table_row, int32_t max_blocks_per_seq, int32_t* table_offset);

/* Text for the last non-OK status returned on this thread ("" if none). */
const char* pkv_last_error(void);

/* Library version string. */
const char* pkv_version(void);

/*
 * Profiling aid: while `hip_event` (a hipEvent_t) is non-NULL, every decode
 * call on this thread that runs the merge kernel records the event on its
 * stream between the partition kernel and the merge kernel, so the partition
 * kernel can be timed alone.  Pass NULL to stop.  Always returns PKV_OK.
 */
int pkv_profile_set_decode_split_event(void* hip_event);

/*
 * Profiling aid: while `hip_event` is non-NULL, every decode call on this
 * thread records the event on its stream immediately before the partition
 * kernel (after the kernel that clears the work counter), so that with the
 * split event the partition kernel is timed alone.  Pass NULL to stop.
 * Always returns PKV_OK.
 */
int pkv_profile_set_decode_start_event(void* hip_event);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
