/*
 * pkv_oracle.h -- declarations of the reference implementation (test
 * infrastructure only; see pkv_oracle.c).  All buffers are host memory.
 */
#ifndef PKV_ORACLE_H
#define PKV_ORACLE_H

#include <stdint.h>

/* element types of Q, K/V inputs and pools */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_I8 = 3 };

double orc_bf16_to_f64(uint16_t b);
double orc_f16_to_f64(uint16_t h);
uint16_t orc_f32_to_f16(float x);
void orc_f32_to_f16_array(const float* x, int64_t n, uint16_t* out);
void orc_f16_to_f64_array(const uint16_t* h, int64_t n, double* out);

void orc_quantize_vector(const float* x, int32_t n, int8_t* q, uint16_t* scale);

int orc_kv_write(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                 int32_t kv_dtype, const void* k, const void* v, int32_t in_dtype,
                 int64_t token_stride, const int32_t* slot_mapping, int32_t num_tokens,
                 void* k_pool, void* v_pool, uint16_t* k_scale, uint16_t* v_scale);

int orc_slot_mapping(int32_t num_blocks, int32_t block_size, int32_t num_seqs,
                     const int32_t* cu_q_lens, const int32_t* seq_lens,
                     const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t* slots);

int orc_copy_blocks(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                    int32_t kv_dtype, void* k_pool, void* v_pool, uint16_t* k_scale,
                    uint16_t* v_scale, const int32_t* src, const int32_t* dst, int32_t num_pairs);

int orc_attention(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                  int32_t kv_dtype, const void* q, int32_t q_dtype, int32_t num_seqs,
                  int32_t num_q_heads, const int32_t* cu_q_lens, const int32_t* seq_lens,
                  const void* k_pool, const void* v_pool, const uint16_t* k_scale,
                  const uint16_t* v_scale, const int32_t* block_tables, int32_t max_blocks_per_seq,
                  float softmax_scale, int32_t window, double* out, double* weights,
                  int64_t weights_stride);

int orc_decode(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
               int32_t kv_dtype, const void* q, int32_t q_dtype, int32_t num_seqs,
               int32_t num_q_heads, const void* k_pool, const void* v_pool,
               const uint16_t* k_scale, const uint16_t* v_scale, const int32_t* block_tables,
               int32_t max_blocks_per_seq, const int32_t* context_lens, float softmax_scale,
               int32_t window, double* out, double* weights, int64_t weights_stride);

int orc_decode_split(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                     int32_t kv_dtype, const void* q, int32_t q_dtype, int32_t num_seqs,
                     int32_t num_q_heads, const void* k_pool, const void* v_pool,
                     const uint16_t* k_scale, const uint16_t* v_scale, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* context_lens, float softmax_scale,
                     int32_t window, int32_t partition_size, double* out);

#endif
