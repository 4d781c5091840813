// block_allocator.cpp -- host-side owner of a pool's physical blocks and the
// table edits that allocation implies.
//
// "PyTorch LLM Serving Engine", What is implemented: the pool is cut into
// blocks of one size, and each sequence lists the blocks it holds in a table.  "MicroGen",
// Key Features: logical-to-physical block mapping, window-length eviction for
// long contexts, prefix sharing and KV rollback for speculative decoding.
//
// Free blocks sit on a stack, so allocating and freeing a block is O(1).  A
// block carries a reference count: a sequence forked from another shares its
// blocks (count + 1 each) instead of copying them, and a block returns to the
// stack when its count reaches zero.  Before a sequence appends into a shared,
// partly filled block, it gets a private copy (copy on write): the allocator
// names the (source, destination) pair and the caller moves the bytes with
// kv_cache_copy_blocks before writing.  Every call checks its arguments first
// and changes nothing when it fails.
#include <cstdint>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"
#include "pkv_internal.h"

struct pkv_block_allocator {
    int32_t num_blocks;
    int32_t block_size;
    std::vector<int32_t> free_ids;   // stack of free blocks (top = back)
    std::vector<int32_t> ref;        // references per block, 0 = free
};

namespace {

using pkv::report;

int32_t blocks_for(int64_t tokens, int32_t bs) { return (int32_t)((tokens + bs - 1) / bs); }

bool owned(const pkv_block_allocator* a, int32_t id) {
    return id >= 0 && id < a->num_blocks && a->ref[id] > 0;
}

int32_t pop(pkv_block_allocator* a) {
    const int32_t id = a->free_ids.back();
    a->free_ids.pop_back();
    a->ref[id] = 1;
    return id;
}

void drop(pkv_block_allocator* a, int32_t id) {
    if (--a->ref[id] == 0) a->free_ids.push_back(id);
}

// Each non-negative id must be a held block, and a block may appear at most
// as often as it is referenced.
int check_release(const pkv_block_allocator* a, const int32_t* ids, int32_t n) {
    std::unordered_map<int32_t, int32_t> uses;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t id = ids[i];
        if (id < 0) continue;
        if (id >= a->num_blocks) return report(PKV_EINVAL, "block %d outside [0, %d)", id, a->num_blocks);
        if (++uses[id] > a->ref[id])
            return report(PKV_EINVAL, "block %d released more often than it is held (%d)", id, a->ref[id]);
    }
    return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_allocator_create(int32_t num_blocks, int32_t block_size, pkv_block_allocator** out) {
    pkv::clear_error();
    if (!out) return report(PKV_EINVAL, "out is NULL");
    *out = nullptr;
    if (num_blocks <= 0 || block_size <= 0)
        return report(PKV_EINVAL, "num_blocks and block_size must be > 0 (got %d, %d)", num_blocks, block_size);
    pkv_block_allocator* a = new (std::nothrow) pkv_block_allocator;
    if (!a) return report(PKV_ENOSPACE, "out of host memory");
    a->num_blocks = num_blocks;
    a->block_size = block_size;
    a->ref.assign((size_t)num_blocks, 0);
    a->free_ids.resize((size_t)num_blocks);
    for (int32_t i = 0; i < num_blocks; ++i) a->free_ids[(size_t)i] = num_blocks - 1 - i;   // block 0 first
    *out = a;
    return PKV_OK;
}

int pkv_allocator_destroy(pkv_block_allocator* a) {
    delete a;
    return PKV_OK;
}

int32_t pkv_allocator_num_free(const pkv_block_allocator* a) {
    return a ? (int32_t)a->free_ids.size() : -1;
}

int32_t pkv_allocator_refcount(const pkv_block_allocator* a, int32_t block) {
    if (!a || block < 0 || block >= a->num_blocks) return -1;
    return a->ref[block];
}

int pkv_allocator_alloc(pkv_block_allocator* a, int32_t n, int32_t* ids) {
    pkv::clear_error();
    if (!a || n < 0 || (n > 0 && !ids)) return report(PKV_EINVAL, "bad allocator, count or output array");
    if ((size_t)n > a->free_ids.size())
        return report(PKV_ENOSPACE, "%d blocks requested, %zu free", n, a->free_ids.size());
    for (int32_t i = 0; i < n; ++i) ids[i] = pop(a);
    return PKV_OK;
}

int pkv_allocator_retain(pkv_block_allocator* a, const int32_t* ids, int32_t n) {
    pkv::clear_error();
    if (!a || n < 0 || (n > 0 && !ids)) return report(PKV_EINVAL, "bad allocator, count or id array");
    for (int32_t i = 0; i < n; ++i)
        if (ids[i] >= 0 && !owned(a, ids[i])) return report(PKV_EINVAL, "block %d is not allocated", ids[i]);
    for (int32_t i = 0; i < n; ++i)
        if (ids[i] >= 0) ++a->ref[ids[i]];
    return PKV_OK;
}

int pkv_allocator_release(pkv_block_allocator* a, const int32_t* ids, int32_t n) {
    pkv::clear_error();
    if (!a || n < 0 || (n > 0 && !ids)) return report(PKV_EINVAL, "bad allocator, count or id array");
    const int rc = check_release(a, ids, n);
    if (rc != PKV_OK) return rc;
    for (int32_t i = 0; i < n; ++i)
        if (ids[i] >= 0) drop(a, ids[i]);
    return PKV_OK;
}

int pkv_seq_append(pkv_block_allocator* a, int32_t* table_row, int32_t max_blocks_per_seq, int32_t len,
                   int32_t num_new, int32_t* copy_src, int32_t* copy_dst, int32_t* num_copies) {
    pkv::clear_error();
    if (!a || !table_row || !copy_src || !copy_dst || !num_copies) return report(PKV_EINVAL, "NULL argument");
    *num_copies = 0;
    if (len < 0 || num_new < 0) return report(PKV_EINVAL, "len and num_new must be >= 0");
    const int32_t bs = a->block_size;
    const int64_t new_len = (int64_t)len + num_new;
    if (blocks_for(new_len, bs) > max_blocks_per_seq)
        return report(PKV_EINVAL, "%lld tokens need more than %d blocks", (long long)new_len, max_blocks_per_seq);
    const int32_t have = blocks_for(len, bs);
    const int32_t fresh = blocks_for(new_len, bs) - have;
    const bool partial = num_new > 0 && len % bs != 0;
    if (partial && !owned(a, table_row[len / bs]))
        return report(PKV_EINVAL, "table entry %d (block %d) is not an allocated block", len / bs, table_row[len / bs]);
    const bool cow = partial && a->ref[table_row[len / bs]] > 1;
    const int32_t need = fresh + (cow ? 1 : 0);
    if ((size_t)need > a->free_ids.size())
        return report(PKV_ENOSPACE, "%d blocks needed, %zu free", need, a->free_ids.size());
    if (cow) {
        const int32_t old = table_row[len / bs];
        const int32_t mine = pop(a);
        drop(a, old);                       // still held by the other sequences
        copy_src[0] = old;
        copy_dst[0] = mine;
        *num_copies = 1;
        table_row[len / bs] = mine;
    }
    for (int32_t i = 0; i < fresh; ++i) table_row[have + i] = pop(a);
    return PKV_OK;
}

int pkv_seq_fork(pkv_block_allocator* a, const int32_t* parent_row, int32_t len, int32_t* child_row,
                 int32_t max_blocks_per_seq) {
    pkv::clear_error();
    if (!a || !parent_row || !child_row) return report(PKV_EINVAL, "NULL argument");
    if (len < 0) return report(PKV_EINVAL, "len must be >= 0");
    const int32_t n = blocks_for(len, a->block_size);
    if (n > max_blocks_per_seq) return report(PKV_EINVAL, "%d tokens need more than %d blocks", len, max_blocks_per_seq);
    for (int32_t i = 0; i < n; ++i)
        if (parent_row[i] >= 0 && !owned(a, parent_row[i]))
            return report(PKV_EINVAL, "parent entry %d (block %d) is not allocated", i, parent_row[i]);
    for (int32_t i = 0; i < n; ++i) {
        child_row[i] = parent_row[i];
        if (parent_row[i] >= 0) ++a->ref[parent_row[i]];
    }
    for (int32_t i = n; i < max_blocks_per_seq; ++i) child_row[i] = -1;
    return PKV_OK;
}

int pkv_seq_truncate(pkv_block_allocator* a, int32_t* table_row, int32_t len, int32_t new_len) {
    pkv::clear_error();
    if (!a || !table_row) return report(PKV_EINVAL, "NULL argument");
    if (new_len < 0 || new_len > len) return report(PKV_EINVAL, "new_len %d outside [0, %d]", new_len, len);
    const int32_t keep = blocks_for(new_len, a->block_size), have = blocks_for(len, a->block_size);
    int rc = check_release(a, table_row + keep, have - keep);
    if (rc != PKV_OK) return rc;
    for (int32_t i = keep; i < have; ++i) {
        if (table_row[i] >= 0) drop(a, table_row[i]);
        table_row[i] = -1;
    }
    return PKV_OK;
}

int pkv_seq_evict_window(pkv_block_allocator* a, int32_t* table_row, int32_t len, int32_t window,
                         int32_t* num_released) {
    pkv::clear_error();
    if (!a || !table_row) return report(PKV_EINVAL, "NULL argument");
    if (len < 0 || window <= 0) return report(PKV_EINVAL, "len must be >= 0 and window > 0");
    // a later query sits at position >= len and sees keys j > len - window: keys
    // 0 .. len - window are gone for good, and with them every block that ends there
    const int64_t dead_keys = (int64_t)len - window + 1;
    const int32_t dead = dead_keys > 0 ? (int32_t)(dead_keys / a->block_size) : 0;
    int rc = check_release(a, table_row, dead);
    if (rc != PKV_OK) return rc;
    int32_t n = 0;
    for (int32_t i = 0; i < dead; ++i) {
        if (table_row[i] >= 0) {
            drop(a, table_row[i]);
            ++n;
        }
        table_row[i] = -1;
    }
    if (num_released) *num_released = n;
    return PKV_OK;
}

int pkv_seq_compact(int32_t* table_row, int32_t max_blocks_per_seq, int32_t* table_offset) {
    pkv::clear_error();
    if (!table_row || !table_offset) return report(PKV_EINVAL, "NULL argument");
    if (max_blocks_per_seq < 0 || *table_offset < 0) return report(PKV_EINVAL, "negative size or offset");
    int32_t n = 0;
    while (n < max_blocks_per_seq && table_row[n] < 0) ++n;
    if (n == max_blocks_per_seq) return PKV_OK;        // nothing held: leave the row as it is
    if ((int64_t)*table_offset + n > INT32_MAX / 16) return report(PKV_EINVAL, "offset overflows");
    for (int32_t i = n; i < max_blocks_per_seq; ++i) table_row[i - n] = table_row[i];
    for (int32_t i = max_blocks_per_seq - n; i < max_blocks_per_seq; ++i) table_row[i] = -1;
    *table_offset += n;
    return PKV_OK;
}

}  // extern "C"
