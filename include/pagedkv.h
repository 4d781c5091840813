/*
 * pagedkv.h -- C ABI of libpagedkv: attention over a paged KV cache on AMD
 * Instinct MI355X (gfx950).
 *
 * The operation is the serving-engine step the pages describe:
 *   - "PyTorch LLM Serving Engine", section Loading: each layer writes its new
 *     K/V vectors into physical cache slots, then attends with a numerically
 *     stable online softmax while walking the sequence's block table;
 *     section What is implemented: fixed-size physical blocks, per-sequence
 *     block tables, chunked prefill.
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
 *   - The library allocates no device memory and keeps no per-call state.
 *   - Return value: PKV_OK (0) or a pkv_status.  Host-visible arguments are
 *     validated before anything is enqueued; on failure nothing is enqueued
 *     and pkv_last_error() describes the problem.  No exception crosses the ABI.
 *   - Device-resident integers (slots, block ids, lengths) are read by the
 *     kernels: out-of-range slots and block ids are skipped rather than
 *     dereferenced, lengths are clamped to max_blocks_per_seq * block_size.
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
    PKV_EHIP = 4          /* the HIP runtime reported an error (text in pkv_last_error) */
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
 * ("PyTorch LLM Serving Engine", Loading: K/V are written to a physical cache
 * slot before attention; "MicroGen", Key Features: dynamic per-vector INT8.)
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
 * partition_size is 0 (single pass) or covers max_blocks_per_seq*block_size.
 * Returns 0 for invalid sizes (the decode call then reports the error).
 */
size_t paged_attention_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                             int32_t head_dim, int32_t max_blocks_per_seq,
                                             int32_t block_size, int32_t partition_size);

/*
 * paged_attention_decode -- one query token per sequence.
 * ("PyTorch LLM Serving Engine", Loading and What is implemented: online
 * softmax while walking the sequence's block table; "MicroGen", Key Features:
 * GQA by KV-head repetition, window-length limit.)
 *
 * For sequence s with L = context_lens[s] tokens (the current token, already
 * written by kv_cache_write, included) and query head h, with
 * G = num_q_heads / cache->num_kv_heads and g = h / G:
 *     p = L - 1;  keys j with 0 <= j <= p and, if sliding_window W > 0, j > p - W
 *     out[s][h] = sum_j softmax_j(softmax_scale * q[s][h] . K_s[j][g]) V_s[j][g]
 * where K_s[j] is the pool row at sequence position j.  L == 0 gives a zero row.
 *
 *   q             [num_seqs][num_q_heads][head_dim]; BF16 for BF16 pools,
 *                 F32 for F32 pools, BF16 or F32 for INT8 pools.
 *   out           [num_seqs][num_q_heads][head_dim] of out_dtype (F32 or BF16).
 *   k_scale/v_scale  INT8 pools only, else NULL.
 *   block_tables  [num_seqs][max_blocks_per_seq] int32 physical block ids;
 *                 entries past ceil(L / block_size) are never read.
 *   context_lens  [num_seqs] int32.
 *   partition_size  0: each sequence in one pass.  Otherwise a positive
 *                 multiple of block_size: contexts are split into partitions
 *                 of that many keys, attended independently and merged by a
 *                 second kernel (log-sum-exp), which needs `workspace`.
 *   workspace     device scratch of at least
 *                 paged_attention_decode_workspace_size(...) bytes, 256-byte
 *                 aligned; may be NULL when that size is 0.  Its contents need
 *                 no initialisation and are not preserved: the call clears its
 *                 work counter (first 256 bytes) with a kernel on `stream`
 *                 before use, so the call can be captured in a graph.  Two
 *                 calls in flight at once must not share a workspace.
 * num_seqs == 0 is a no-op.  out must not alias any input or the workspace.
 */
int paged_attention_decode(const pkv_cache_desc* cache,
                           const void* q, int32_t q_dtype,
                           void* out, int32_t out_dtype,
                           int32_t num_seqs, int32_t num_q_heads,
                           const void* k_pool, const void* v_pool,
                           const void* k_scale, const void* v_scale,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens,
                           float softmax_scale, int32_t sliding_window,
                           int32_t partition_size,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

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
 * Pools must be BF16.  num_seqs == 0 or max_q_len == 0 is a no-op.
 */
int paged_attention_prefill_chunk(const pkv_cache_desc* cache,
                                  const void* q, int32_t q_dtype,
                                  void* out, int32_t out_dtype,
                                  const int32_t* cu_q_lens, int32_t num_seqs,
                                  int32_t max_q_len, int32_t num_q_heads,
                                  const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* seq_lens,
                                  float softmax_scale, int32_t sliding_window,
                                  void* stream);

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
