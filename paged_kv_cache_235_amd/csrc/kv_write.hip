// kv_write.hip -- store new K/V vectors at their slots in the block pool.
//
// "PyTorch LLM Serving Engine", Loading: the cache receives the new keys and
// values before attention runs.  "MicroGen", Key Features: dynamic per-vector INT8 KV.
//
// Copy path: one thread per 16-byte chunk of a (token, head) vector, K and V
// handled by the same thread; loads and stores are 16 B wide and a wave moves
// whole 1 KiB runs.  INT8 path: a group of head_dim/8 lanes owns one vector;
// the absmax is reduced inside the group and each lane quantises 8 elements.
#include "pkv_internal.h"
#include "pkv_device.h"

namespace pkv {

struct WriteArgs {
    const char* k;
    const char* v;
    const int32_t* slots;
    char* k_pool;
    char* v_pool;
    uint16_t* k_scale;
    uint16_t* v_scale;
    int64_t token_stride_bytes;
    int64_t num_slots;        // num_blocks * block_size
    int32_t num_tokens;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size;
};

// Byte offset of (slot, head) vector start inside a pool of element size esz.
__device__ __forceinline__ int64_t vec_index(int64_t slot, int h, const WriteArgs& a) {
    const int64_t blk = slot / a.block_size;
    const int64_t off = slot - blk * a.block_size;
    return (blk * a.num_kv_heads + h) * a.block_size + off;
}

// The same for 0 <= slot < 2^32.
__device__ __forceinline__ int64_t vec_index32(uint32_t slot, int h, const WriteArgs& a) {
    const uint32_t blk = slot / (uint32_t)a.block_size;
    const uint32_t off = slot - blk * (uint32_t)a.block_size;
    return ((int64_t)blk * a.num_kv_heads + h) * a.block_size + off;
}

__global__ __launch_bounds__(256) void kv_write_copy_kernel(WriteArgs a, int esz) {
    const int chunks = a.head_dim * esz / 16;            // 16-byte chunks per vector
    const int64_t per_token = (int64_t)a.num_kv_heads * chunks;
    const int64_t total = (int64_t)a.num_tokens * per_token;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = i / per_token;
        const int rem = (int)(i - t * per_token);
        const int h = rem / chunks;
        const int c = rem - h * chunks;
        const int64_t slot = a.slots[t];
        if (slot < 0 || slot >= a.num_slots) continue;
        const int64_t src = t * a.token_stride_bytes + ((int64_t)h * a.head_dim * esz) + c * 16;
        const int64_t dst = vec_index(slot, h, a) * a.head_dim * esz + c * 16;
        const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(a.k + src);
        const u32x4_t vv = *reinterpret_cast<const u32x4_t*>(a.v + src);
        // streaming stores: the pool is read back much later, in pieces (65,536
        // tokens: 112 -> 88 us against plain stores; streaming loads as well
        // measured slower, 110 us)
        __builtin_nontemporal_store(kv, reinterpret_cast<u32x4_t*>(a.k_pool + dst));
        __builtin_nontemporal_store(vv, reinterpret_cast<u32x4_t*>(a.v_pool + dst));
    }
}

// Quantise 8 values against the stored fp16 scale sf (0 -> all codes 0):
// code = clamp(rne(x / sf), -127, 127) with an IEEE fp32 division.
__device__ __forceinline__ u32x2_t quantise8(const float* x, float sf) {
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        int q = 0;
        if (sf != 0.0f) {
            float r = __builtin_rintf(__fdiv_rn(x[e], sf));
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            q = (int)r;
        }
        w[e >> 2] |= ((uint32_t)(q & 0xff)) << (8 * (e & 3));
    }
    u32x2_t out;
    out[0] = w[0];
    out[1] = w[1];
    return out;
}

// The same codes for bf16 inputs, with one multiplication by the scale's
// reciprocal in place of each division.  Why the result is the same: write
// x = mx 2^a (|mx| < 2^8, a bf16 value) and sf = ms 2^b (0 < ms < 2^11, a
// binary16 value).  For a half-integer h, x - h sf is a multiple of
// 2^min(a, b-1), so either x / sf = h exactly or |x / sf - h| >=
// min(2^(a-b) / ms, 1 / (2 ms)) >= 2^-12 (the first term is |x / sf| / |mx|,
// and h is only in reach once |x / sf| >= 1/4).  The product x * rcp(sf),
// with the reciprocal within 1 ulp and one rounding, is within 2^-22
// relative, i.e. < 2^-14 absolute for |x / sf| <= 191 (the largest ratio a
// binary16-rounded scale allows).  So when the product is at least 2^-13 from
// every half-integer, x / sf and its fp32 rounding lie on the same side of
// every half-integer as the product and all three round to the same integer.
// A lane with a product closer than that (exact ties among them) takes the
// IEEE divisions.  NaN, infinite and zero inputs give what the divisions give.
__device__ __forceinline__ u32x2_t quantise8_bf16(const float* x, float sf) {
    if (sf == 0.0f) return u32x2_t{0u, 0u};
    const float r = __builtin_amdgcn_rcpf(sf);
    float c[8];
    bool near = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float q = x[e] * r;
        c[e] = __builtin_rintf(q);
        near |= fabsf(q - c[e]) > 0.5f - 0x1p-13f;
    }
    if (near) return quantise8(x, sf);
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        // clamp by one median (c comes from rint, so it is never a signalling NaN)
        const int q = (int)__builtin_amdgcn_fmed3f(c[e], -127.0f, 127.0f);
        w[e >> 2] |= ((uint32_t)(q & 0xff)) << (8 * (e & 3));
    }
    u32x2_t out;
    out[0] = w[0];
    out[1] = w[1];
    return out;
}

// Max over an aligned group of W <= 16 lanes of values that are >= +0 and never
// NaN: their bit patterns order like the values, so an integer max does it
// without the NaN canonicalisation a float max needs.
template <int W>
__device__ __forceinline__ float group_max_nonneg(float x) {
    static_assert(W <= 16, "DPP exchanges within a row");
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    if constexpr (W >= 16) u = max(u, __builtin_bit_cast(uint32_t, xchg<8>(__builtin_bit_cast(float, u))));
    if constexpr (W >= 8) u = max(u, __builtin_bit_cast(uint32_t, xchg<4>(__builtin_bit_cast(float, u))));
    if constexpr (W >= 4) u = max(u, __builtin_bit_cast(uint32_t, xchg<2>(__builtin_bit_cast(float, u))));
    if constexpr (W >= 2) u = max(u, __builtin_bit_cast(uint32_t, xchg<1>(__builtin_bit_cast(float, u))));
    return __builtin_bit_cast(float, u);
}

template <bool IN_BF16, int D>
__global__ __launch_bounds__(256) void kv_write_int8_kernel(WriteArgs a) {
    constexpr int GL = D / 8;                        // lanes per vector
    const int64_t vecs = (int64_t)a.num_tokens * a.num_kv_heads;
    const int64_t gid = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / GL;
    const int part = threadIdx.x % GL;
    // 32-bit divisions where the sizes allow (a uniform branch)
    const bool narrow = vecs <= (int64_t)UINT32_MAX && a.num_slots <= (int64_t)UINT32_MAX;
    // every lane of a group takes the same trip count, so the group reductions stay converged
    for (int64_t vi = gid; vi < vecs; vi += (int64_t)gridDim.x * blockDim.x / GL) {
        int64_t t;
        if (narrow) t = (uint32_t)vi / (uint32_t)a.num_kv_heads;
        else t = vi / a.num_kv_heads;
        const int h = (int)(vi - t * a.num_kv_heads);
        const int64_t slot = a.slots[t];
        const bool store = slot >= 0 && slot < a.num_slots;
        const int64_t src = t * a.token_stride_bytes + (int64_t)h * D * (IN_BF16 ? 2 : 4);
        // bf16: both vectors' loads in flight before either is quantised
        u32x4_t wkv[2];
        if constexpr (IN_BF16) {
            wkv[0] = *reinterpret_cast<const u32x4_t*>(a.k + src + part * 16);
            wkv[1] = *reinterpret_cast<const u32x4_t*>(a.v + src + part * 16);
        }
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            const char* in = which ? a.v : a.k;
            float x[8];
            if constexpr (IN_BF16) {
                const u32x4_t w = wkv[which];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[2 * e] = bf16lo(w[e]);
                    x[2 * e + 1] = bf16hi(w[e]);
                }
            } else {
                const f32x4_t w0 = *reinterpret_cast<const f32x4_t*>(in + src + part * 32);
                const f32x4_t w1 = *reinterpret_cast<const f32x4_t*>(in + src + part * 32 + 16);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[e] = w0[e];
                    x[4 + e] = w1[e];
                }
            }
            float am = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(x[e]));
            am = group_max_nonneg<GL>(am);             // am >= +0, never NaN (fmaxf skips NaN)
            // binary16(fp32(am / 127)), RNE.  For bf16 inputs am is a bf16 value, and for
            // every one of those a multiplication by fp32(1/127) rounds to the same
            // binary16 value as the IEEE quotient (checked over all of them on the host)
            const _Float16 s16 = IN_BF16 ? (_Float16)(am * 0x1.020408p-7f) : (_Float16)__fdiv_rn(am, 127.0f);
            const float sf = (float)s16;
            u32x2_t codes;
            if constexpr (IN_BF16) codes = quantise8_bf16(x, sf);
            else codes = quantise8(x, sf);
            if (store) {
                const int64_t vec = narrow ? vec_index32((uint32_t)slot, h, a) : vec_index(slot, h, a);
                char* pool = which ? a.v_pool : a.k_pool;
                // streaming stores, as in the copy (65,536 tokens: 122 -> 110 us)
                __builtin_nontemporal_store(codes, reinterpret_cast<u32x2_t*>(pool + vec * D + part * 8));
                if (part == 0) (which ? a.v_scale : a.k_scale)[vec] = __builtin_bit_cast(uint16_t, s16);
            }
        }
    }
}

hipError_t launch_kv_write(const KvWriteLaunch& L, hipStream_t stream) {
    WriteArgs a;
    a.k = static_cast<const char*>(L.k);
    a.v = static_cast<const char*>(L.v);
    a.slots = L.slot_mapping;
    a.k_pool = static_cast<char*>(L.k_pool);
    a.v_pool = static_cast<char*>(L.v_pool);
    a.k_scale = static_cast<uint16_t*>(L.k_scale);
    a.v_scale = static_cast<uint16_t*>(L.v_scale);
    a.token_stride_bytes = L.token_stride * (L.in_bf16 ? 2 : 4);
    a.num_slots = (int64_t)L.num_blocks * L.block_size;
    a.num_tokens = L.num_tokens;
    a.num_kv_heads = L.num_kv_heads;
    a.head_dim = L.head_dim;
    a.block_size = L.block_size;

    const int threads = 256;
    if (!L.quantise) {
        const int esz = L.in_bf16 ? 2 : 4;
        const int64_t work = (int64_t)L.num_tokens * L.num_kv_heads * (L.head_dim * esz / 16);
        const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((work + threads - 1) / threads, 65536));
        return launch(kv_write_copy_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, a, esz);
    }
    const int gl = L.head_dim / 8;
    const int64_t work = (int64_t)L.num_tokens * L.num_kv_heads * gl;
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((work + threads - 1) / threads, 65536));
    auto kern = L.in_bf16 ? (L.head_dim == 64 ? kv_write_int8_kernel<true, 64> : kv_write_int8_kernel<true, 128>)
                          : (L.head_dim == 64 ? kv_write_int8_kernel<false, 64> : kv_write_int8_kernel<false, 128>);
    return launch(kern, dim3((unsigned)blocks), dim3(threads), 0, stream, a);
}

}  // namespace pkv
