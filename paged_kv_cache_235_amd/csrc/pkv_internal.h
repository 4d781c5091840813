// pkv_internal.h -- host-side interface between the C ABI (pkv_api.cpp) and
// the kernel launchers.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace pkv {

// Launch `kern` and return the runtime's status for this launch only.
template <typename... Params, typename... Args>
inline hipError_t launch(void (*kern)(Params...), dim3 grid, dim3 block, size_t shmem,
                         hipStream_t stream, Args... args) {
    static_assert(sizeof...(Params) == sizeof...(Args), "argument count");
    void* ptrs[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, ptrs, shmem, stream);
}

// Set this thread's pkv_last_error() text and return `status`.
int report(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Compute units and per-kernel occupancy of the current device (cached).
int device_cu_count();

struct KvWriteLaunch {
    const void* k;
    const void* v;
    bool in_bf16;              // else fp32
    bool quantise;             // INT8 pool
    int64_t token_stride;      // elements
    const int32_t* slot_mapping;
    int32_t num_tokens;
    int32_t num_blocks, block_size, num_kv_heads, head_dim;
    void* k_pool;
    void* v_pool;
    void* k_scale;
    void* v_scale;
};
hipError_t launch_kv_write(const KvWriteLaunch& L, hipStream_t stream);

// KV_I8Q: an INT8 pool read with a bf16 query (Q.K^T by bf16 dot products of the codes)
enum KvKind { KV_F32 = 0, KV_BF16 = 1, KV_I8 = 2, KV_I8Q = 3 };

struct DecodeLaunch {
    const void* q;
    bool q_bf16;
    void* out;
    bool out_bf16;
    int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks;
    KvKind kv;
    const void* k_pool;
    const void* v_pool;
    const uint16_t* k_scale;
    const uint16_t* v_scale;
    const int32_t* block_tables;
    int32_t max_blocks_per_seq;
    const int32_t* table_offsets;  // per sequence, or null
    const int32_t* context_lens;
    float softmax_scale;
    int32_t window;
    int32_t partition_size;    // 0: single pass
    void* workspace;
    hipEvent_t split_event;    // recorded between the two kernels when non-null
    hipEvent_t start_event;    // recorded right before the partition kernel when non-null
};
// Number of partition slots per (sequence, head) in the workspace (0 if no merge).
int32_t decode_max_partitions(int32_t max_blocks_per_seq, int32_t block_size, int32_t partition_size,
                              bool with_table_offsets);
size_t decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                              int32_t max_partitions);
hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream);
// The fixed device scratch of the allocation-free decode entry point: its size,
// and its address on the current device (looked up, and its work counter
// cleared by a kernel on `stream`, at the first call on each device).
size_t decode_fixed_scratch_bytes();
hipError_t decode_fixed_scratch(void** ptr, hipStream_t stream);

struct PrefillLaunch {
    const void* q;             // bf16 [rows][Hq][D]
    void* out;
    bool out_bf16;
    const int32_t* cu_q_lens;
    int32_t num_seqs, max_q_len, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks;
    const void* k_pool;        // bf16, or int8 codes
    const void* v_pool;
    bool int8;
    const uint16_t* k_scale;   // INT8 pools: fp16 scales, else null
    const uint16_t* v_scale;
    const int32_t* block_tables;
    int32_t max_blocks_per_seq;
    const int32_t* table_offsets;  // per sequence, or null
    const int32_t* seq_lens;
    float softmax_scale;
    int32_t window;
};
hipError_t launch_prefill(const PrefillLaunch& L, hipStream_t stream);

struct SlotMappingLaunch {
    const int32_t* cu_q_lens;
    const int32_t* seq_lens;
    const int32_t* block_tables;
    const int32_t* table_offsets;  // per sequence, or null
    int32_t num_seqs, max_blocks_per_seq, block_size, num_blocks;
    int32_t* slot_mapping;
    int32_t total_rows;
};
hipError_t launch_slot_mapping(const SlotMappingLaunch& L, hipStream_t stream);

struct CopyBlocksLaunch {
    void* k_pool;
    void* v_pool;
    void* k_scale;             // INT8 pools only, else null
    void* v_scale;
    const int32_t* src;
    const int32_t* dst;
    int32_t num_pairs, num_blocks, num_kv_heads, block_size, head_dim, elem_size;
};
hipError_t launch_copy_blocks(const CopyBlocksLaunch& L, hipStream_t stream);

}  // namespace pkv
