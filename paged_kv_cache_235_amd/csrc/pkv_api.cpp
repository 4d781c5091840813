// pkv_api.cpp -- the C ABI of libpagedkv (declared in include/pagedkv.h):
// argument validation, error reporting and dispatch to the kernel launchers.
// Nothing is enqueued unless every host-visible argument is valid.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "pagedkv.h"
#include "pkv_internal.h"

namespace {

thread_local std::string g_error;
thread_local hipEvent_t g_split_event = nullptr;
thread_local hipEvent_t g_start_event = nullptr;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return status;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(PKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

const char* dtype_name(int32_t t) {
    switch (t) {
    case PKV_F32: return "F32";
    case PKV_BF16: return "BF16";
    case PKV_I8: return "I8";
    default: return "invalid";
    }
}

int check_cache(const pkv_cache_desc* c) {
    if (!c) return fail(PKV_EINVAL, "cache descriptor is NULL");
    if (c->num_blocks <= 0) return fail(PKV_EINVAL, "num_blocks must be > 0 (got %d)", c->num_blocks);
    if (c->num_kv_heads <= 0) return fail(PKV_EINVAL, "num_kv_heads must be > 0 (got %d)", c->num_kv_heads);
    if (c->block_size <= 0 || c->head_dim <= 0)
        return fail(PKV_EINVAL, "block_size and head_dim must be > 0");
    if (c->block_size != 16) return fail(PKV_EUNSUPPORTED, "block_size %d unsupported (16 only)", c->block_size);
    if (c->head_dim != 64 && c->head_dim != 128)
        return fail(PKV_EUNSUPPORTED, "head_dim %d unsupported (64 or 128)", c->head_dim);
    if (c->kv_dtype != PKV_F32 && c->kv_dtype != PKV_BF16 && c->kv_dtype != PKV_I8)
        return fail(PKV_EINVAL, "kv_dtype %d is not a pkv_dtype", c->kv_dtype);
    if ((int64_t)c->num_blocks * c->block_size > INT32_MAX)
        return fail(PKV_EUNSUPPORTED, "num_blocks * block_size exceeds the int32 slot range");
    return PKV_OK;
}

bool validate_env() {
    static const bool on = [] {
        const char* v = std::getenv("PKV_VALIDATE");
        return v && *v && std::strcmp(v, "0") != 0;
    }();
    return on;
}

template <typename T>
int copy_to_host(std::vector<T>& dst, const T* src, size_t n, hipStream_t stream) {
    dst.resize(n);
    if (n == 0) return PKV_OK;
    hipError_t e = hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    return e == hipSuccess ? PKV_OK : hip_fail(e, "PKV_VALIDATE copy");
}

// PKV_VALIDATE=1: check device-resident tables and lengths on the host.
// Entries wholly before the window of the call's first query may be -1 (evicted).
int validate_tables(const pkv_cache_desc* c, int32_t num_seqs, const int32_t* block_tables,
                    int32_t max_blocks, const int32_t* offsets, const int32_t* lens, const int32_t* cu,
                    int32_t window, hipStream_t stream) {
    std::vector<int32_t> L, T, CU, OFF;
    int rc = copy_to_host(L, lens, (size_t)num_seqs, stream);
    if (rc == PKV_OK) rc = copy_to_host(T, block_tables, (size_t)num_seqs * max_blocks, stream);
    if (rc == PKV_OK && cu) rc = copy_to_host(CU, cu, (size_t)num_seqs + 1, stream);
    if (rc == PKV_OK && offsets) rc = copy_to_host(OFF, offsets, (size_t)num_seqs, stream);
    if (rc != PKV_OK) return rc;
    if (cu && CU[0] != 0) return fail(PKV_EINVAL, "cu_q_lens[0] = %d, expected 0", CU[0]);
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int64_t off = offsets ? OFF[s] : 0;
        if (off < 0) return fail(PKV_EINVAL, "table_offsets[%d] = %lld is negative", s, (long long)off);
        const int64_t cap = ((int64_t)max_blocks + off) * c->block_size;
        if (L[s] < 0 || L[s] > cap)
            return fail(PKV_EINVAL, "length %d of sequence %d outside [0, %lld]", L[s], s, (long long)cap);
        if (cu) {
            const int32_t C = CU[s + 1] - CU[s];
            if (C < 0 || C > L[s]) return fail(PKV_EINVAL, "chunk length %d of sequence %d outside [0, %d]", C, s, L[s]);
        }
        const int32_t used = (L[s] + c->block_size - 1) / c->block_size;
        const int64_t first_query = cu ? (int64_t)L[s] - (CU[s + 1] - CU[s]) : (int64_t)L[s] - 1;
        const int64_t first_key = window > 0 ? std::max<int64_t>(0, first_query - window + 1) : 0;
        if (first_key / c->block_size < off)
            return fail(PKV_EINVAL, "sequence %d: keys from %lld are visible but its row starts at block %lld", s,
                        (long long)first_key, (long long)off);
        for (int32_t b = (int32_t)(first_key / c->block_size); b < used; ++b) {
            const int32_t id = T[(size_t)s * max_blocks + (b - off)];
            if (id < 0 || id >= c->num_blocks)
                return fail(PKV_EINVAL, "block_tables[%d][%lld] = %d outside [0, %d)", s, (long long)(b - off), id,
                            c->num_blocks);
        }
    }
    return PKV_OK;
}

}  // namespace

namespace pkv {
int report(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return status;
}

void clear_error() { g_error.clear(); }

int device_cu_count() {
    static thread_local int cached_dev = -1;
    static thread_local int cached_cus = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev != cached_dev) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cached_dev = dev;
        cached_cus = cus;
    }
    return cached_cus;
}
}  // namespace pkv

extern "C" {

const char* pkv_last_error(void) { return g_error.c_str(); }

const char* pkv_version(void) { return "libpagedkv 0.1 (gfx950)"; }

int pkv_profile_set_decode_split_event(void* hip_event) {
    g_split_event = static_cast<hipEvent_t>(hip_event);
    return PKV_OK;
}

int pkv_profile_set_decode_start_event(void* hip_event) {
    g_start_event = static_cast<hipEvent_t>(hip_event);
    return PKV_OK;
}

int kv_cache_write(const pkv_cache_desc* cache, const void* k, const void* v, int32_t in_dtype,
                   int64_t token_stride, const int32_t* slot_mapping, int32_t num_tokens,
                   void* k_pool, void* v_pool, void* k_scale, void* v_scale, void* stream) {
    g_error.clear();
    int rc = check_cache(cache);
    if (rc != PKV_OK) return rc;
    if (num_tokens < 0) return fail(PKV_EINVAL, "num_tokens must be >= 0 (got %d)", num_tokens);
    if (in_dtype != PKV_F32 && in_dtype != PKV_BF16)
        return fail(in_dtype == PKV_I8 ? PKV_EUNSUPPORTED : PKV_EINVAL, "input dtype %s unsupported (F32 or BF16)",
                    dtype_name(in_dtype));
    const bool quantise = cache->kv_dtype == PKV_I8;
    if (!quantise && cache->kv_dtype != in_dtype)
        return fail(PKV_EUNSUPPORTED, "writing %s vectors into a %s pool is unsupported", dtype_name(in_dtype),
                    dtype_name(cache->kv_dtype));
    if (quantise && (!k_scale || !v_scale)) return fail(PKV_EINVAL, "INT8 pools need k_scale and v_scale");
    if (!quantise && (k_scale || v_scale)) return fail(PKV_EINVAL, "k_scale/v_scale must be NULL for %s pools",
                                                       dtype_name(cache->kv_dtype));
    if (num_tokens == 0) return PKV_OK;
    if (!k || !v || !slot_mapping || !k_pool || !v_pool) return fail(PKV_EINVAL, "NULL tensor pointer");
    const int64_t esz = in_dtype == PKV_BF16 ? 2 : 4;
    const int64_t row = (int64_t)cache->num_kv_heads * cache->head_dim;
    if (token_stride < row) return fail(PKV_EINVAL, "token_stride %lld < num_kv_heads * head_dim = %lld",
                                        (long long)token_stride, (long long)row);
    if ((token_stride * esz) % 16 != 0) return fail(PKV_EINVAL, "token_stride * element size must be a multiple of 16 bytes");
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
        return fail(PKV_EINVAL, "k, v and the pools must be 16-byte aligned");
    if (quantise && (!aligned(k_scale, 2) || !aligned(v_scale, 2))) return fail(PKV_EINVAL, "scale pools must be 2-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (validate_env()) {
        std::vector<int32_t> slots;
        rc = copy_to_host(slots, slot_mapping, (size_t)num_tokens, st);
        if (rc != PKV_OK) return rc;
        const int64_t nslots = (int64_t)cache->num_blocks * cache->block_size;
        std::vector<char> seen((size_t)nslots, 0);
        for (int32_t t = 0; t < num_tokens; ++t) {
            if (slots[t] < 0) continue;
            if (slots[t] >= nslots) return fail(PKV_EINVAL, "slot_mapping[%d] = %d outside [0, %lld)", t, slots[t], (long long)nslots);
            if (seen[slots[t]]++) return fail(PKV_EINVAL, "slot %d written twice", slots[t]);
        }
    }
    pkv::KvWriteLaunch L;
    L.k = k;
    L.v = v;
    L.in_bf16 = in_dtype == PKV_BF16;
    L.quantise = quantise;
    L.token_stride = token_stride;
    L.slot_mapping = slot_mapping;
    L.num_tokens = num_tokens;
    L.num_blocks = cache->num_blocks;
    L.block_size = cache->block_size;
    L.num_kv_heads = cache->num_kv_heads;
    L.head_dim = cache->head_dim;
    L.k_pool = k_pool;
    L.v_pool = v_pool;
    L.k_scale = k_scale;
    L.v_scale = v_scale;
    const hipError_t e = pkv::launch_kv_write(L, st);
    return e == hipSuccess ? PKV_OK : hip_fail(e, "kv_cache_write launch");
}

size_t paged_attention_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                             int32_t max_blocks_per_seq, int32_t block_size,
                                             int32_t partition_size, int32_t with_table_offsets) {
    if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || max_blocks_per_seq <= 0 || block_size <= 0 ||
        partition_size < 0)
        return 0;
    const int32_t np = pkv::decode_max_partitions(max_blocks_per_seq, block_size, partition_size,
                                                  with_table_offsets != 0);
    return pkv::decode_workspace_bytes(num_seqs, num_q_heads, head_dim, np);
}

// Shared body of the two decode entry points.  fixed_scratch: the workspace is
// the library's fixed device array (looked up here), not the caller's.
static int decode_call(const pkv_cache_desc* cache, const void* q, int32_t q_dtype, void* out,
                       int32_t out_dtype, int32_t num_seqs, int32_t num_q_heads, const void* k_pool,
                       const void* v_pool, const void* k_scale, const void* v_scale,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* table_offsets, const int32_t* context_lens, float softmax_scale,
                       int32_t sliding_window, int32_t partition_size, void* workspace,
                       size_t workspace_bytes, bool fixed_scratch, void* stream) {
    g_error.clear();
    int rc = check_cache(cache);
    if (rc != PKV_OK) return rc;
    if (num_seqs < 0) return fail(PKV_EINVAL, "num_seqs must be >= 0 (got %d)", num_seqs);
    if (num_q_heads <= 0 || num_q_heads % cache->num_kv_heads != 0)
        return fail(PKV_EINVAL, "num_q_heads %d is not a positive multiple of num_kv_heads %d", num_q_heads,
                    cache->num_kv_heads);
    if (max_blocks_per_seq <= 0) return fail(PKV_EINVAL, "max_blocks_per_seq must be > 0");
    if ((int64_t)max_blocks_per_seq * cache->block_size > INT32_MAX)
        return fail(PKV_EUNSUPPORTED, "max_blocks_per_seq * block_size exceeds int32");
    if (sliding_window < 0) return fail(PKV_EINVAL, "sliding_window must be >= 0");
    if (!std::isfinite(softmax_scale) || softmax_scale < 0.0f)
        return fail(PKV_EINVAL, "softmax_scale must be finite and >= 0");
    if (partition_size < 0 || partition_size % cache->block_size != 0)
        return fail(PKV_EINVAL, "partition_size %d must be 0 or a positive multiple of block_size", partition_size);
    const int32_t kv = cache->kv_dtype;
    const bool q_ok = (kv == PKV_BF16 && q_dtype == PKV_BF16) || (kv == PKV_F32 && q_dtype == PKV_F32) ||
                      (kv == PKV_I8 && (q_dtype == PKV_BF16 || q_dtype == PKV_F32));
    if (q_dtype != PKV_F32 && q_dtype != PKV_BF16) return fail(PKV_EINVAL, "q_dtype %d is not F32 or BF16", q_dtype);
    if (!q_ok) return fail(PKV_EUNSUPPORTED, "q dtype %s with a %s pool is unsupported", dtype_name(q_dtype), dtype_name(kv));
    if (out_dtype != PKV_F32 && out_dtype != PKV_BF16) return fail(PKV_EUNSUPPORTED, "out_dtype must be F32 or BF16");
    if (kv == PKV_I8 && (!k_scale || !v_scale)) return fail(PKV_EINVAL, "INT8 pools need k_scale and v_scale");
    if (kv != PKV_I8 && (k_scale || v_scale)) return fail(PKV_EINVAL, "k_scale/v_scale must be NULL for %s pools", dtype_name(kv));
    if (num_seqs == 0) return PKV_OK;
    if (!q || !out || !k_pool || !v_pool || !block_tables || !context_lens) return fail(PKV_EINVAL, "NULL tensor pointer");
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
        return fail(PKV_EINVAL, "q, out and the pools must be 16-byte aligned");
    const size_t need = paged_attention_decode_workspace_size(num_seqs, num_q_heads, cache->head_dim,
                                                              max_blocks_per_seq, cache->block_size, partition_size,
                                                              table_offsets != nullptr);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (fixed_scratch && need > 0) {
        workspace_bytes = pkv::decode_fixed_scratch_bytes();
        if (need > workspace_bytes)
            return fail(PKV_EWORKSPACE, "this call needs %zu bytes of split-K scratch; the fixed scratch of "
                        "paged_attention_decode_noalloc holds %zu (use a larger partition_size, fewer sequences, "
                        "or paged_attention_decode with a workspace)", need, workspace_bytes);
        const hipError_t e = pkv::decode_fixed_scratch(&workspace, st);
        if (e != hipSuccess) return hip_fail(e, "fixed decode scratch");
    }
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(PKV_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace ? workspace_bytes : (size_t)0);
    if (need > 0 && !aligned(workspace, 256)) return fail(PKV_EINVAL, "workspace must be 256-byte aligned");
    if (validate_env()) {
        rc = validate_tables(cache, num_seqs, block_tables, max_blocks_per_seq, table_offsets, context_lens,
                             nullptr, sliding_window, st);
        if (rc != PKV_OK) return rc;
        if (need > 0) {
            // the work counter at the head of the workspace must be zero
            std::vector<uint32_t> head;
            rc = copy_to_host(head, static_cast<const uint32_t*>(workspace), 1, st);
            if (rc != PKV_OK) return rc;
            if (head[0] != 0)
                return fail(PKV_EINVAL, "workspace work counter is %u, expected 0 (zero the workspace before its "
                            "first use)", head[0]);
        }
    }
    pkv::DecodeLaunch L;
    L.q = q;
    L.q_bf16 = q_dtype == PKV_BF16;
    L.out = out;
    L.out_bf16 = out_dtype == PKV_BF16;
    L.num_seqs = num_seqs;
    L.num_q_heads = num_q_heads;
    L.num_kv_heads = cache->num_kv_heads;
    L.head_dim = cache->head_dim;
    L.block_size = cache->block_size;
    L.num_blocks = cache->num_blocks;
    L.kv = kv == PKV_F32 ? pkv::KV_F32 : kv == PKV_BF16 ? pkv::KV_BF16
                                          : (q_dtype == PKV_BF16 ? pkv::KV_I8Q : pkv::KV_I8);
    L.k_pool = k_pool;
    L.v_pool = v_pool;
    L.k_scale = static_cast<const uint16_t*>(k_scale);
    L.v_scale = static_cast<const uint16_t*>(v_scale);
    L.block_tables = block_tables;
    L.max_blocks_per_seq = max_blocks_per_seq;
    L.table_offsets = table_offsets;
    L.context_lens = context_lens;
    L.softmax_scale = softmax_scale;
    L.window = sliding_window;
    L.partition_size = partition_size;
    L.workspace = workspace;
    L.split_event = g_split_event;
    L.start_event = g_start_event;
    const hipError_t e = pkv::launch_decode(L, st);
    return e == hipSuccess ? PKV_OK : hip_fail(e, "paged_attention_decode launch");
}

int paged_attention_decode(const pkv_cache_desc* cache, const void* q, int32_t q_dtype, void* out,
                           int32_t out_dtype, int32_t num_seqs, int32_t num_q_heads, const void* k_pool,
                           const void* v_pool, const void* k_scale, const void* v_scale,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* table_offsets, const int32_t* context_lens, float softmax_scale,
                           int32_t sliding_window, int32_t partition_size, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return decode_call(cache, q, q_dtype, out, out_dtype, num_seqs, num_q_heads, k_pool, v_pool, k_scale, v_scale,
                       block_tables, max_blocks_per_seq, table_offsets, context_lens, softmax_scale, sliding_window,
                       partition_size, workspace, workspace_bytes, false, stream);
}

int paged_attention_decode_noalloc(const pkv_cache_desc* cache, const void* q, int32_t q_dtype, void* out,
                                   int32_t out_dtype, int32_t num_seqs, int32_t num_q_heads, const void* k_pool,
                                   const void* v_pool, const void* k_scale, const void* v_scale,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* table_offsets, const int32_t* context_lens,
                                   float softmax_scale, int32_t sliding_window, int32_t partition_size,
                                   void* stream) {
    return decode_call(cache, q, q_dtype, out, out_dtype, num_seqs, num_q_heads, k_pool, v_pool, k_scale, v_scale,
                       block_tables, max_blocks_per_seq, table_offsets, context_lens, softmax_scale, sliding_window,
                       partition_size, nullptr, 0, true, stream);
}

size_t paged_attention_decode_noalloc_max_scratch(void) { return pkv::decode_fixed_scratch_bytes(); }

int paged_attention_prefill_chunk(const pkv_cache_desc* cache, const void* q, int32_t q_dtype, void* out,
                                  int32_t out_dtype, const int32_t* cu_q_lens, int32_t num_seqs,
                                  int32_t max_q_len, int32_t num_q_heads, const void* k_pool,
                                  const void* v_pool, const void* k_scale, const void* v_scale,
                                  const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* table_offsets,
                                  const int32_t* seq_lens, float softmax_scale,
                                  int32_t sliding_window, void* stream) {
    g_error.clear();
    int rc = check_cache(cache);
    if (rc != PKV_OK) return rc;
    if (num_seqs < 0 || max_q_len < 0) return fail(PKV_EINVAL, "num_seqs and max_q_len must be >= 0");
    if (num_q_heads <= 0 || num_q_heads % cache->num_kv_heads != 0)
        return fail(PKV_EINVAL, "num_q_heads %d is not a positive multiple of num_kv_heads %d", num_q_heads,
                    cache->num_kv_heads);
    if (max_blocks_per_seq <= 0) return fail(PKV_EINVAL, "max_blocks_per_seq must be > 0");
    if ((int64_t)max_blocks_per_seq * cache->block_size > INT32_MAX)
        return fail(PKV_EUNSUPPORTED, "max_blocks_per_seq * block_size exceeds int32");
    if (sliding_window < 0) return fail(PKV_EINVAL, "sliding_window must be >= 0");
    if (!std::isfinite(softmax_scale) || softmax_scale < 0.0f)
        return fail(PKV_EINVAL, "softmax_scale must be finite and >= 0");
    if (q_dtype != PKV_BF16) return fail(q_dtype == PKV_F32 ? PKV_EUNSUPPORTED : PKV_EINVAL, "prefill needs BF16 q");
    const bool i8 = cache->kv_dtype == PKV_I8;
    if (cache->kv_dtype != PKV_BF16 && !i8)
        return fail(PKV_EUNSUPPORTED, "prefill needs a BF16 or INT8 pool (got %s)", dtype_name(cache->kv_dtype));
    if (i8 && (!k_scale || !v_scale)) return fail(PKV_EINVAL, "INT8 pools need k_scale and v_scale");
    if (!i8 && (k_scale || v_scale)) return fail(PKV_EINVAL, "k_scale/v_scale must be NULL for %s pools", dtype_name(cache->kv_dtype));
    if (i8 && (!aligned(k_scale, 16) || !aligned(v_scale, 16)))
        return fail(PKV_EINVAL, "INT8 scale pools must be 16-byte aligned for prefill");
    if (out_dtype != PKV_F32 && out_dtype != PKV_BF16) return fail(PKV_EUNSUPPORTED, "out_dtype must be F32 or BF16");
    if ((int64_t)max_q_len * (num_q_heads / cache->num_kv_heads) > INT32_MAX / 2)
        return fail(PKV_EUNSUPPORTED, "max_q_len too large");
    if (num_seqs == 0 || max_q_len == 0) return PKV_OK;
    if (!q || !out || !cu_q_lens || !k_pool || !v_pool || !block_tables || !seq_lens)
        return fail(PKV_EINVAL, "NULL tensor pointer");
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
        return fail(PKV_EINVAL, "q, out and the pools must be 16-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (validate_env()) {
        rc = validate_tables(cache, num_seqs, block_tables, max_blocks_per_seq, table_offsets, seq_lens,
                             cu_q_lens, sliding_window, st);
        if (rc != PKV_OK) return rc;
    }
    pkv::PrefillLaunch L;
    L.q = q;
    L.out = out;
    L.out_bf16 = out_dtype == PKV_BF16;
    L.cu_q_lens = cu_q_lens;
    L.num_seqs = num_seqs;
    L.max_q_len = max_q_len;
    L.num_q_heads = num_q_heads;
    L.num_kv_heads = cache->num_kv_heads;
    L.head_dim = cache->head_dim;
    L.block_size = cache->block_size;
    L.num_blocks = cache->num_blocks;
    L.k_pool = k_pool;
    L.v_pool = v_pool;
    L.int8 = i8;
    L.k_scale = static_cast<const uint16_t*>(k_scale);
    L.v_scale = static_cast<const uint16_t*>(v_scale);
    L.block_tables = block_tables;
    L.max_blocks_per_seq = max_blocks_per_seq;
    L.table_offsets = table_offsets;
    L.seq_lens = seq_lens;
    L.softmax_scale = softmax_scale;
    L.window = sliding_window;
    const hipError_t e = pkv::launch_prefill(L, st);
    return e == hipSuccess ? PKV_OK : hip_fail(e, "paged_attention_prefill_chunk launch");
}


int pkv_build_slot_mapping(const pkv_cache_desc* cache, const int32_t* cu_q_lens, int32_t num_seqs,
                           const int32_t* seq_lens, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* table_offsets, int32_t* slot_mapping, int32_t total_rows,
                           void* stream) {
    g_error.clear();
    int rc = check_cache(cache);
    if (rc != PKV_OK) return rc;
    if (num_seqs < 0 || total_rows < 0) return fail(PKV_EINVAL, "num_seqs and total_rows must be >= 0");
    if (max_blocks_per_seq <= 0) return fail(PKV_EINVAL, "max_blocks_per_seq must be > 0");
    if (num_seqs == 0 || total_rows == 0) return PKV_OK;
    if (num_seqs > 0x7fffffff / 2) return fail(PKV_EUNSUPPORTED, "num_seqs too large");
    if (!cu_q_lens || !seq_lens || !block_tables || !slot_mapping) return fail(PKV_EINVAL, "NULL tensor pointer");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (validate_env()) {
        std::vector<int32_t> CU;
        rc = copy_to_host(CU, cu_q_lens, (size_t)num_seqs + 1, st);
        if (rc != PKV_OK) return rc;
        if (CU[0] != 0) return fail(PKV_EINVAL, "cu_q_lens[0] = %d, expected 0", CU[0]);
        for (int32_t s = 0; s < num_seqs; ++s)
            if (CU[s + 1] < CU[s]) return fail(PKV_EINVAL, "cu_q_lens decreases at %d", s);
        if (CU[num_seqs] > total_rows)
            return fail(PKV_EINVAL, "cu_q_lens[num_seqs] = %d exceeds total_rows %d", CU[num_seqs], total_rows);
    }
    pkv::SlotMappingLaunch L;
    L.cu_q_lens = cu_q_lens;
    L.seq_lens = seq_lens;
    L.block_tables = block_tables;
    L.table_offsets = table_offsets;
    L.num_seqs = num_seqs;
    L.max_blocks_per_seq = max_blocks_per_seq;
    L.block_size = cache->block_size;
    L.num_blocks = cache->num_blocks;
    L.slot_mapping = slot_mapping;
    L.total_rows = total_rows;
    const hipError_t e = pkv::launch_slot_mapping(L, st);
    return e == hipSuccess ? PKV_OK : hip_fail(e, "pkv_build_slot_mapping launch");
}

int kv_cache_copy_blocks(const pkv_cache_desc* cache, void* k_pool, void* v_pool, void* k_scale, void* v_scale,
                         const int32_t* src_blocks, const int32_t* dst_blocks, int32_t num_pairs, void* stream) {
    g_error.clear();
    int rc = check_cache(cache);
    if (rc != PKV_OK) return rc;
    if (num_pairs < 0) return fail(PKV_EINVAL, "num_pairs must be >= 0 (got %d)", num_pairs);
    const bool i8 = cache->kv_dtype == PKV_I8;
    if (i8 && (!k_scale || !v_scale)) return fail(PKV_EINVAL, "INT8 pools need k_scale and v_scale");
    if (!i8 && (k_scale || v_scale))
        return fail(PKV_EINVAL, "k_scale/v_scale must be NULL for %s pools", dtype_name(cache->kv_dtype));
    if (num_pairs == 0) return PKV_OK;
    if (!k_pool || !v_pool || !src_blocks || !dst_blocks) return fail(PKV_EINVAL, "NULL tensor pointer");
    if (!aligned(k_pool, 16) || !aligned(v_pool, 16)) return fail(PKV_EINVAL, "the pools must be 16-byte aligned");
    if (i8 && (!aligned(k_scale, 4) || !aligned(v_scale, 4)))
        return fail(PKV_EINVAL, "scale pools must be 4-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (validate_env()) {
        std::vector<int32_t> S, D;
        rc = copy_to_host(S, src_blocks, (size_t)num_pairs, st);
        if (rc == PKV_OK) rc = copy_to_host(D, dst_blocks, (size_t)num_pairs, st);
        if (rc != PKV_OK) return rc;
        std::vector<char> role((size_t)cache->num_blocks, 0);   // bit 0: source, bit 1: destination
        for (int32_t n = 0; n < num_pairs; ++n) {
            if (S[n] < 0 || S[n] >= cache->num_blocks || D[n] < 0 || D[n] >= cache->num_blocks)
                return fail(PKV_EINVAL, "pair %d (%d -> %d) names a block outside [0, %d)", n, S[n], D[n],
                            cache->num_blocks);
            role[S[n]] |= 1;
        }
        for (int32_t n = 0; n < num_pairs; ++n) {
            if (role[D[n]] & 2) return fail(PKV_EINVAL, "block %d is the destination of two pairs", D[n]);
            if ((role[D[n]] & 1) && S[n] != D[n]) return fail(PKV_EINVAL, "block %d is both a source and a destination", D[n]);
            role[D[n]] |= 2;
        }
    }
    pkv::CopyBlocksLaunch L;
    L.k_pool = k_pool;
    L.v_pool = v_pool;
    L.k_scale = k_scale;
    L.v_scale = v_scale;
    L.src = src_blocks;
    L.dst = dst_blocks;
    L.num_pairs = num_pairs;
    L.num_blocks = cache->num_blocks;
    L.num_kv_heads = cache->num_kv_heads;
    L.block_size = cache->block_size;
    L.head_dim = cache->head_dim;
    L.elem_size = cache->kv_dtype == PKV_F32 ? 4 : cache->kv_dtype == PKV_BF16 ? 2 : 1;
    const hipError_t e = pkv::launch_copy_blocks(L, st);
    return e == hipSuccess ? PKV_OK : hip_fail(e, "kv_cache_copy_blocks launch");
}

}  // extern "C"
