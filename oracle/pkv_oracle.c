/*
 * pkv_oracle.c -- reference implementation of attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the oracle the GPU library is checked
 * against.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg load it; the library never does.  It shares no code, header, table or
 * constant with the GPU path, and includes nothing from it.
 *
 * Plain single-threaded C99.  Attention is computed in binary64.  The INT8
 * quantiser works in binary32 on purpose: the method fixes that precision
 * (see quantize_vector), so the bytes it writes are the unique expected bytes.
 *
 * What is computed, and where the pages state it:
 *  - "PyTorch LLM Serving Engine", section Loading: in the serving path a
 *    layer stores the new keys and values in the cache first; its attention
 *    then visits the sequence's blocks in table order with an online softmax
 *    (a running maximum keeps the exponentials bounded).  Section What is
 *    implemented: a cache of equal-sized blocks, a table of block ids per
 *    sequence, prefill in chunks.
 *  - "MicroGen", section Key Features: logical-to-physical block mapping;
 *    grouped-query attention by repeating each KV head for its group of query
 *    heads; dynamic per-vector INT8 KV quantisation; window-length eviction.
 *  - "llminfer", section Paged KV Cache And Continuous Batching: 16-token pages.
 *
 * A block-wise online softmax reaches exactly (up to rounding order) the plain
 * softmax-attention result, so the oracle is that plain definition: gather the
 * sequence's blocks into contiguous fp64 K and V through the block table, then
 * a textbook two-pass softmax (maximum first, then normalised weights).
 *
 * Readings taken where the pages are silent (each one lives in one place):
 *  - pool layout [num_blocks][num_kv_heads][block_size][head_dim]; INT8 scale
 *    pools [num_blocks][num_kv_heads][block_size] of fp16 bit patterns;
 *  - slot = physical_block * block_size + offset; a negative slot is skipped;
 *  - query head h reads KV head h / (num_q_heads / num_kv_heads);
 *  - a sequence length counts the tokens written by the current step, and a
 *    query at position p sees key j iff j <= p and, with a window W > 0,
 *    j > p - W (W keys including itself);
 *  - INT8: see quantize_vector; an empty context gives a zero output row;
 *  - a table entry that is not a block of the pool (-1: released by window
 *    eviction or a rollback) holds no keys, and a query with no key left
 *    gets a zero output row, like an empty context.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "pkv_oracle.h"

/* ------------------------------------------------------------------ numbers */

/* Round a non-negative binary64 value to the nearest integer, ties to even. */
static double round_half_even(double r)
{
    double f = floor(r);
    double frac = r - f;
    if (frac > 0.5) return f + 1.0;
    if (frac < 0.5) return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

double orc_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;   /* bf16 is the top half of a binary32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double orc_f16_to_f64(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* binary32 -> binary16, round to nearest, ties to even; overflow gives inf. */
uint16_t orc_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs((double)x);
    if (isnan(x)) return (uint16_t)(sign | 0x7e00);
    /* 65520 is halfway between 65504 (largest finite, odd fraction) and 2^16:
       ties go to the even neighbour, which overflows. */
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: value = m * 2^-24, m in [0, 1024]; m == 1024 is the
           smallest normal number and has the same encoding 0x0400 */
        double m = round_half_even(a * ldexp(1.0, 24));
        return (uint16_t)(sign | (uint16_t)m);
    }
    int k;
    frexp(a, &k);               /* a = f * 2^k, f in [0.5, 1) */
    int E = k - 1;              /* a in [2^E, 2^(E+1)) */
    double m = round_half_even((a * ldexp(1.0, -E) - 1.0) * 1024.0);
    if (m == 1024.0) { m = 0.0; E += 1; }
    if (E + 15 >= 31) return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)m);
}

void orc_f32_to_f16_array(const float* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_f16(x[i]);
}

void orc_f16_to_f64_array(const uint16_t* h, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_to_f64(h[i]);
}

/* ------------------------------------------------------------- INT8 vectors */

/*
 * Dynamic per-vector INT8 quantisation ("MicroGen", Key Features: vector scale
 * dynamic quantisation of the KV cache), symmetric, one fp16 scale per
 * (token, KV head) vector:
 *   a   = max_d |x_d|                       (binary32, exact)
 *   s   = fp16_rne(a / 127)                 (one binary32 division)
 *   q_d = clamp(rne(x_d / float(s)), -127, 127)   (binary32 division)
 * The division uses the stored fp16 scale, so dequantising q_d * s reproduces
 * what was quantised against.  If s is zero (a == 0, or a / 127 rounds to zero
 * in fp16) every q_d is zero.  The operations are binary32 by design: doing
 * them in binary64 can move a byte at a .5 boundary.
 */
void orc_quantize_vector(const float* x, int32_t n, int8_t* q, uint16_t* scale)
{
    float a = 0.0f;
    for (int32_t i = 0; i < n; ++i) {
        float v = fabsf(x[i]);
        if (v > a) a = v;
    }
    volatile float ratio = a / 127.0f;
    uint16_t s = orc_f32_to_f16(ratio);
    float sf = (float)orc_f16_to_f64(s);   /* exact: every fp16 is a binary32 */
    *scale = s;
    for (int32_t i = 0; i < n; ++i) {
        if (sf == 0.0f) { q[i] = 0; continue; }
        volatile float t = x[i] / sf;
        double r = round_half_even(fabs((double)t));
        if (t < 0.0f) r = -r;
        if (r > 127.0) r = 127.0;
        if (r < -127.0) r = -127.0;
        q[i] = (int8_t)r;
    }
}

/* ------------------------------------------------------------- cache write */

static int elem_size(int32_t dtype)
{
    switch (dtype) {
    case ORC_F32: return 4;
    case ORC_BF16: return 2;
    case ORC_I8: return 1;
    default: return 0;
    }
}

static float input_as_float(const void* base, int32_t dtype, int64_t i)
{
    if (dtype == ORC_F32) return ((const float*)base)[i];
    return (float)orc_bf16_to_f64(((const uint16_t*)base)[i]);
}

/*
 * Write each token's K and V vectors into its physical slot ("PyTorch LLM
 * Serving Engine", Loading: new keys and values enter the cache before the
 * attention reads it).  Token t's vector for KV head h starts at element
 * t * token_stride + h * head_dim of k and v.  The destination of element d is
 *   pool[slot / block_size][h][slot % block_size][d].
 * Same input and pool type: a bit copy.  INT8 pool: quantize_vector per
 * (token, head) vector, with its scale at scale[slot / bs][h][slot % bs].
 */
int orc_kv_write(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                 int32_t kv_dtype, const void* k, const void* v, int32_t in_dtype,
                 int64_t token_stride, const int32_t* slot_mapping, int32_t num_tokens,
                 void* k_pool, void* v_pool, uint16_t* k_scale, uint16_t* v_scale)
{
    if (kv_dtype == ORC_I8) {
        if (in_dtype != ORC_F32 && in_dtype != ORC_BF16) return 1;
        if (!k_scale || !v_scale) return 1;
    } else if (kv_dtype != in_dtype || elem_size(kv_dtype) == 0) {
        return 1;
    }
    const int esz = elem_size(kv_dtype);
    const int in_esz = elem_size(in_dtype);
    float* xbuf = (float*)malloc(sizeof(float) * (size_t)head_dim);
    if (!xbuf) return 2;
    for (int32_t t = 0; t < num_tokens; ++t) {
        int32_t slot = slot_mapping[t];
        if (slot < 0) continue;
        int64_t blk = slot / block_size;
        int64_t off = slot % block_size;
        if (blk >= num_blocks) { free(xbuf); return 1; }
        for (int32_t h = 0; h < num_kv_heads; ++h) {
            int64_t src = (int64_t)t * token_stride + (int64_t)h * head_dim;
            int64_t vec = (blk * num_kv_heads + h) * block_size + off;   /* vector index */
            for (int which = 0; which < 2; ++which) {
                const void* in = which ? v : k;
                void* pool = which ? v_pool : k_pool;
                if (kv_dtype == ORC_I8) {
                    uint16_t* scales = which ? v_scale : k_scale;
                    for (int32_t d = 0; d < head_dim; ++d) xbuf[d] = input_as_float(in, in_dtype, src + d);
                    orc_quantize_vector(xbuf, head_dim, (int8_t*)pool + vec * head_dim, &scales[vec]);
                } else {
                    memcpy((char*)pool + vec * head_dim * esz, (const char*)in + src * in_esz,
                           (size_t)head_dim * esz);
                }
            }
        }
    }
    free(xbuf);
    return 0;
}

/* ------------------------------------------------------------ slot mapping */

/*
 * Slot of every new row of a step ("MicroGen", Key Features: logical blocks
 * map to physical blocks through the sequence's table; "PyTorch LLM Serving
 * Engine", Loading: every new key/value vector gets a cache position of its
 * own).  Sequence s owns
 * rows [cu_q_lens[s], cu_q_lens[s+1]), C_s of them, and holds L_s = seq_lens[s]
 * tokens once they are written, so its row i sits at position p = L_s - C_s + i
 * and goes to
 *     slot = block_tables[s][p / block_size] * block_size + p % block_size.
 * A row whose position is negative or past the table, or whose table entry is
 * not a block of the pool, gets -1 (the cache write skips it).
 */
int orc_slot_mapping(int32_t num_blocks, int32_t block_size, int32_t num_seqs,
                     const int32_t* cu_q_lens, const int32_t* seq_lens,
                     const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t* slots)
{
    if (block_size <= 0 || num_seqs < 0 || max_blocks_per_seq < 0) return 1;
    for (int32_t s = 0; s < num_seqs; ++s) {
        int32_t r0 = cu_q_lens[s], r1 = cu_q_lens[s + 1];
        for (int32_t r = r0; r < r1; ++r) {
            int64_t p = (int64_t)seq_lens[s] - (r1 - r0) + (r - r0);
            int32_t slot = -1;
            if (p >= 0 && p / block_size < max_blocks_per_seq) {
                int32_t blk = block_tables[(int64_t)s * max_blocks_per_seq + p / block_size];
                if (blk >= 0 && blk < num_blocks)
                    slot = (int32_t)((int64_t)blk * block_size + p % block_size);
            }
            slots[r] = slot;
        }
    }
    return 0;
}

/*
 * Copy whole physical blocks: for each pair n, block dst[n] of the K pool, the
 * V pool and (INT8) both scale pools becomes a copy of block src[n] -- every
 * KV head and every slot.  This is what sharing a block between sequences
 * needs before one of them writes into it.  All copies read the pools as they
 * were before the call (a block copied into is not a source of another pair);
 * pairs with an id outside [0, num_blocks) are skipped.
 */
int orc_copy_blocks(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                    int32_t kv_dtype, void* k_pool, void* v_pool, uint16_t* k_scale,
                    uint16_t* v_scale, const int32_t* src, const int32_t* dst, int32_t num_pairs)
{
    const int esz = elem_size(kv_dtype);
    if (esz == 0 || num_pairs < 0) return 1;
    if (kv_dtype == ORC_I8 && (!k_scale || !v_scale)) return 1;
    const size_t blk_bytes = (size_t)num_kv_heads * block_size * head_dim * esz;
    const size_t sc_bytes = (size_t)num_kv_heads * block_size * sizeof(uint16_t);
    char* snap = (char*)malloc(2 * (blk_bytes + sc_bytes) * (size_t)(num_pairs > 0 ? num_pairs : 1));
    if (!snap) return 2;
    /* read every source first, then write every destination */
    for (int pass = 0; pass < 2; ++pass) {
        for (int32_t n = 0; n < num_pairs; ++n) {
            if (src[n] < 0 || src[n] >= num_blocks || dst[n] < 0 || dst[n] >= num_blocks) continue;
            char* keep = snap + (size_t)n * 2 * (blk_bytes + sc_bytes);
            char* kp = (char*)k_pool;
            char* vp = (char*)v_pool;
            if (pass == 0) {
                memcpy(keep, kp + (size_t)src[n] * blk_bytes, blk_bytes);
                memcpy(keep + blk_bytes, vp + (size_t)src[n] * blk_bytes, blk_bytes);
                if (kv_dtype == ORC_I8) {
                    memcpy(keep + 2 * blk_bytes, (char*)k_scale + (size_t)src[n] * sc_bytes, sc_bytes);
                    memcpy(keep + 2 * blk_bytes + sc_bytes, (char*)v_scale + (size_t)src[n] * sc_bytes,
                           sc_bytes);
                }
            } else {
                memcpy(kp + (size_t)dst[n] * blk_bytes, keep, blk_bytes);
                memcpy(vp + (size_t)dst[n] * blk_bytes, keep + blk_bytes, blk_bytes);
                if (kv_dtype == ORC_I8) {
                    memcpy((char*)k_scale + (size_t)dst[n] * sc_bytes, keep + 2 * blk_bytes, sc_bytes);
                    memcpy((char*)v_scale + (size_t)dst[n] * sc_bytes, keep + 2 * blk_bytes + sc_bytes,
                           sc_bytes);
                }
            }
        }
    }
    free(snap);
    return 0;
}

/* ------------------------------------------------------------------ gather */

static double pool_value(const void* pool, const uint16_t* scale, int32_t kv_dtype,
                         int64_t vec, int32_t head_dim, int32_t d)
{
    int64_t i = vec * head_dim + d;
    switch (kv_dtype) {
    case ORC_F32: return (double)((const float*)pool)[i];
    case ORC_BF16: return orc_bf16_to_f64(((const uint16_t*)pool)[i]);
    default:      /* INT8: q * s, exact in binary64 */
        return (double)((const int8_t*)pool)[i] * orc_f16_to_f64(scale[vec]);
    }
}

/*
 * Contiguous K and V of sequence s, KV head g, tokens [0, len): dst[j][d].
 * Token j of the sequence lives in physical block block_table[j / bs] at
 * offset j % bs ("MicroGen", Key Features: logical-to-physical mapping).
 * A table entry that is not a block of the pool (-1 after window eviction or
 * a rollback) holds no keys: present[j] is 0 for its tokens (1 otherwise) and
 * their rows are left NaN, so any use of them would show.
 */
static void gather(const void* pool, const uint16_t* scale, int32_t kv_dtype, int32_t num_blocks,
                   int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                   const int32_t* table_row, int32_t g, int32_t len, double* dst,
                   unsigned char* present)
{
    for (int32_t j = 0; j < len; ++j) {
        int64_t blk = table_row[j / block_size];
        if (blk < 0 || blk >= num_blocks) {
            present[j] = 0;
            for (int32_t d = 0; d < head_dim; ++d) dst[(int64_t)j * head_dim + d] = NAN;
            continue;
        }
        present[j] = 1;
        int64_t vec = (blk * num_kv_heads + g) * block_size + j % block_size;
        for (int32_t d = 0; d < head_dim; ++d)
            dst[(int64_t)j * head_dim + d] = pool_value(pool, scale, kv_dtype, vec, head_dim, d);
    }
}

/* ---------------------------------------------------------------- attention */

/* Keys visible from position p: [lo, p], lo = 0, or p - W + 1 with a window. */
static int32_t first_visible(int32_t p, int32_t window)
{
    if (window > 0 && p - window + 1 > 0) return p - window + 1;
    return 0;
}

/*
 * Softmax attention of one query vector over the present keys of [lo, hi] of
 * contiguous K, V:
 *   score_j = scale * sum_d q_d K_jd
 *   out     = sum_j (exp(score_j - m) / Z) V_j,  m = max_j score_j,
 *                                                  Z = sum_j exp(score_j - m)
 * Two passes: the maximum first (numerical stability), then the weights.
 * Keys whose block is missing (present[j] == 0) take no part; no key at all
 * gives a zero vector.  weights (optional) gets each weight at its key index,
 * zero elsewhere in [0, wlen).
 */
static void attend(const double* qv, const double* K, const double* V, const unsigned char* present,
                   int32_t D, int32_t lo, int32_t hi, double scale, double* scores,
                   double* out, double* weights, int32_t wlen)
{
    for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
    if (weights)
        for (int32_t j = 0; j < wlen; ++j) weights[j] = 0.0;

    double m = -INFINITY;
    int32_t n = 0;
    for (int32_t j = lo; j <= hi; ++j) {
        if (!present[j]) continue;
        double dot = 0.0;
        for (int32_t d = 0; d < D; ++d) dot += qv[d] * K[(int64_t)j * D + d];
        scores[j] = scale * dot;
        if (n == 0 || scores[j] > m) m = scores[j];
        ++n;
    }
    if (n == 0) return;
    double Z = 0.0;
    for (int32_t j = lo; j <= hi; ++j)
        if (present[j]) Z += exp(scores[j] - m);
    for (int32_t j = lo; j <= hi; ++j) {
        if (!present[j]) continue;
        double w = exp(scores[j] - m) / Z;
        if (weights) weights[j] = w;
        for (int32_t d = 0; d < D; ++d) out[d] += w * V[(int64_t)j * D + d];
    }
}

static double q_value(const void* q, int32_t q_dtype, int64_t i)
{
    if (q_dtype == ORC_F32) return (double)((const float*)q)[i];
    return orc_bf16_to_f64(((const uint16_t*)q)[i]);
}

/*
 * Attention for every query row of every sequence.
 * Sequence s owns query rows [cu_q_lens[s], cu_q_lens[s+1]) (C_s rows) and has
 * seq_lens[s] = L_s tokens in the cache, its own C_s new ones included.  Row i
 * sits at position p = L_s - C_s + i.  Decode is the case C_s = 1 (p = L_s - 1).
 * q and out are [total_rows][num_q_heads][head_dim]; weights, if given, is
 * [total_rows][num_q_heads][weights_stride] with weights_stride >= max L_s.
 */
int orc_attention(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                  int32_t kv_dtype, const void* q, int32_t q_dtype, int32_t num_seqs,
                  int32_t num_q_heads, const int32_t* cu_q_lens, const int32_t* seq_lens,
                  const void* k_pool, const void* v_pool, const uint16_t* k_scale,
                  const uint16_t* v_scale, const int32_t* block_tables, int32_t max_blocks_per_seq,
                  float softmax_scale, int32_t window, double* out, double* weights,
                  int64_t weights_stride)
{
    (void)num_blocks;
    if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0) return 1;
    if (q_dtype != ORC_F32 && q_dtype != ORC_BF16) return 1;
    if (elem_size(kv_dtype) == 0) return 1;
    const int32_t G = num_q_heads / num_kv_heads;
    const int32_t D = head_dim;
    const double scale = (double)softmax_scale;

    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t L = seq_lens[s];
        const int32_t r0 = cu_q_lens[s], C = cu_q_lens[s + 1] - cu_q_lens[s];
        if (C < 0 || L < 0 || C > (L > 0 ? L : 1)) return 1;
        if (L > (int64_t)max_blocks_per_seq * block_size) return 1;
        const int32_t* table_row = block_tables + (int64_t)s * max_blocks_per_seq;

        double* K = (double*)malloc(sizeof(double) * ((size_t)L * D + 1));
        double* V = (double*)malloc(sizeof(double) * ((size_t)L * D + 1));
        double* scores = (double*)malloc(sizeof(double) * ((size_t)L + 1));
        double* qv = (double*)malloc(sizeof(double) * (size_t)D);
        unsigned char* present = (unsigned char*)malloc((size_t)L + 1);
        if (!K || !V || !scores || !qv || !present) {
            free(K); free(V); free(scores); free(qv); free(present);
            return 2;
        }

        for (int32_t g = 0; g < num_kv_heads; ++g) {
            gather(k_pool, k_scale, kv_dtype, num_blocks, block_size, num_kv_heads, D, table_row, g, L, K,
                   present);
            gather(v_pool, v_scale, kv_dtype, num_blocks, block_size, num_kv_heads, D, table_row, g, L, V,
                   present);
            for (int32_t i = 0; i < C; ++i) {
                const int64_t row = (int64_t)r0 + i;
                const int32_t p = L - C + i;
                const int32_t lo = first_visible(p, window);
                for (int32_t h = g * G; h < (g + 1) * G; ++h) {
                    for (int32_t d = 0; d < D; ++d)
                        qv[d] = q_value(q, q_dtype, (row * num_q_heads + h) * D + d);
                    double* o = out + (row * num_q_heads + h) * D;
                    double* w = weights ? weights + (row * num_q_heads + h) * weights_stride : NULL;
                    attend(qv, K, V, present, D, lo, p, scale, scores, o, w, L);
                }
            }
        }
        free(K); free(V); free(scores); free(qv); free(present);
    }
    return 0;
}

/*
 * Decode (one query per sequence, at position context_lens[s] - 1): the
 * C_s = 1 case of orc_attention.  q and out are [num_seqs][num_q_heads][D].
 */
int orc_decode(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
               int32_t kv_dtype, const void* q, int32_t q_dtype, int32_t num_seqs,
               int32_t num_q_heads, const void* k_pool, const void* v_pool,
               const uint16_t* k_scale, const uint16_t* v_scale, const int32_t* block_tables,
               int32_t max_blocks_per_seq, const int32_t* context_lens, float softmax_scale,
               int32_t window, double* out, double* weights, int64_t weights_stride)
{
    int rc = 0;
    for (int32_t s = 0; s < num_seqs && rc == 0; ++s) {
        if (context_lens[s] == 0) {
            /* no key at all: the row exists and is zero */
            for (int32_t h = 0; h < num_q_heads; ++h)
                for (int32_t d = 0; d < head_dim; ++d)
                    out[((int64_t)s * num_q_heads + h) * head_dim + d] = 0.0;
            if (weights)
                for (int32_t h = 0; h < num_q_heads; ++h)
                    for (int64_t j = 0; j < weights_stride; ++j)
                        weights[((int64_t)s * num_q_heads + h) * weights_stride + j] = 0.0;
            continue;
        }
        /* sequence s alone, as query row s */
        int32_t one_cu[2] = {s, s + 1};
        rc = orc_attention(num_blocks, block_size, num_kv_heads, head_dim, kv_dtype, q, q_dtype, 1,
                           num_q_heads, one_cu, context_lens + s, k_pool, v_pool, k_scale, v_scale,
                           block_tables + (int64_t)s * max_blocks_per_seq, max_blocks_per_seq,
                           softmax_scale, window, out, weights, weights_stride);
    }
    return rc;
}

/* ------------------------------------------------------------ split-K path */

/*
 * Decode computed per partition of partition_size keys and merged, as a
 * check of the merge algebra (CPU only).  For partition k with visible keys:
 *   m_k = max score, l_k = sum exp(score - m_k), o_k = sum exp(score - m_k) V_j;
 * merged with M = max_k m_k and w_k = exp(m_k - M):
 *   out = (sum_k w_k o_k) / (sum_k w_k l_k).
 * Partitions without a visible key (none in range, or all in missing blocks)
 * take no part; a row with none at all is zero.
 */
int orc_decode_split(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                     int32_t kv_dtype, const void* q, int32_t q_dtype, int32_t num_seqs,
                     int32_t num_q_heads, const void* k_pool, const void* v_pool,
                     const uint16_t* k_scale, const uint16_t* v_scale, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* context_lens, float softmax_scale,
                     int32_t window, int32_t partition_size, double* out)
{
    (void)num_blocks;
    if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || partition_size <= 0) return 1;
    const int32_t G = num_q_heads / num_kv_heads;
    const int32_t D = head_dim;
    const double scale = (double)softmax_scale;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t L = context_lens[s];
        const int32_t* table_row = block_tables + (int64_t)s * max_blocks_per_seq;
        double* K = (double*)malloc(sizeof(double) * ((size_t)L * D + 1));
        double* V = (double*)malloc(sizeof(double) * ((size_t)L * D + 1));
        double* qv = (double*)malloc(sizeof(double) * (size_t)D);
        double* acc = (double*)malloc(sizeof(double) * (size_t)D);
        double* ok = (double*)malloc(sizeof(double) * (size_t)D);
        unsigned char* present = (unsigned char*)malloc((size_t)L + 1);
        if (!K || !V || !qv || !acc || !ok || !present) {
            free(K); free(V); free(qv); free(acc); free(ok); free(present);
            return 2;
        }
        for (int32_t g = 0; g < num_kv_heads; ++g) {
            gather(k_pool, k_scale, kv_dtype, num_blocks, block_size, num_kv_heads, D, table_row, g, L, K,
                   present);
            gather(v_pool, v_scale, kv_dtype, num_blocks, block_size, num_kv_heads, D, table_row, g, L, V,
                   present);
            const int32_t p = L - 1;
            const int32_t lo = first_visible(p, window);
            for (int32_t h = g * G; h < (g + 1) * G; ++h) {
                for (int32_t d = 0; d < D; ++d) qv[d] = q_value(q, q_dtype, ((int64_t)s * num_q_heads + h) * D + d);
                double* o = out + ((int64_t)s * num_q_heads + h) * D;
                /* first pass over partitions: the global maximum of the partition maxima */
                double M = -INFINITY;
                for (int32_t k0 = 0; k0 < L; k0 += partition_size) {
                    int32_t a = k0 > lo ? k0 : lo, b = (k0 + partition_size - 1 < p) ? k0 + partition_size - 1 : p;
                    for (int32_t j = a; j <= b; ++j) {
                        if (!present[j]) continue;
                        double dot = 0.0;
                        for (int32_t d = 0; d < D; ++d) dot += qv[d] * K[(int64_t)j * D + d];
                        if (scale * dot > M) M = scale * dot;   /* max over all = max of partition maxima */
                    }
                }
                double num_l = 0.0;
                for (int32_t d = 0; d < D; ++d) acc[d] = 0.0;
                for (int32_t k0 = 0; k0 < L; k0 += partition_size) {
                    int32_t a = k0 > lo ? k0 : lo, b = (k0 + partition_size - 1 < p) ? k0 + partition_size - 1 : p;
                    double mk = -INFINITY, lk = 0.0;
                    int32_t n = 0;
                    for (int32_t j = a; j <= b; ++j) {
                        if (!present[j]) continue;
                        double dot = 0.0;
                        for (int32_t d = 0; d < D; ++d) dot += qv[d] * K[(int64_t)j * D + d];
                        if (n == 0 || scale * dot > mk) mk = scale * dot;
                        ++n;
                    }
                    if (n == 0) continue;
                    for (int32_t d = 0; d < D; ++d) ok[d] = 0.0;
                    for (int32_t j = a; j <= b; ++j) {
                        if (!present[j]) continue;
                        double dot = 0.0;
                        for (int32_t d = 0; d < D; ++d) dot += qv[d] * K[(int64_t)j * D + d];
                        double e = exp(scale * dot - mk);
                        lk += e;
                        for (int32_t d = 0; d < D; ++d) ok[d] += e * V[(int64_t)j * D + d];
                    }
                    double wk = exp(mk - M);
                    num_l += wk * lk;
                    for (int32_t d = 0; d < D; ++d) acc[d] += wk * ok[d];
                }
                for (int32_t d = 0; d < D; ++d) o[d] = (num_l > 0.0) ? acc[d] / num_l : 0.0;
            }
        }
        free(K); free(V); free(qv); free(acc); free(ok); free(present);
    }
    return 0;
}
