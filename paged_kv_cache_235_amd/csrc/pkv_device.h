// pkv_device.h -- device helpers shared by the gfx950 kernels of libpagedkv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ---- bf16 <-> f32 ------------------------------------------------------------
// A bf16 value is the upper half of a binary32, so widening is a shift or mask.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __builtin_bit_cast(float, (uint32_t)h << 16); }

// Round to nearest even (the hardware conversion in the default rounding mode).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// Two fp32 values to a packed pair of binary16, round to nearest even.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    f16x2_t v;
    v[0] = (_Float16)lo;
    v[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// ---- cross-lane exchange -----------------------------------------------------
// DPP controls (gfx9 encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <- lane 7-i within each 8 lanes (flips bits 0..2)
constexpr int kDppRowRor8 = 0x128;      // lane i <- lane (i+8) mod 16 (flips bit 3)

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Value of lane (lane ^ MASK) for MASK = 1 and 2; for 4 and 8 the partner also
// differs in the lower bits (half mirror, rotate), which is all a butterfly that
// walks the bits from the highest down needs; 16 and 32 go through ds_swizzle /
// bpermute.
template <int MASK>
__device__ __forceinline__ float xchg(float x) {
    if constexpr (MASK == 1) return dpp_mov<kDppQuadXor1>(x);
    else if constexpr (MASK == 2) return dpp_mov<kDppQuadXor2>(x);
    else if constexpr (MASK == 4) return dpp_mov<kDppHalfMirror>(x);
    else if constexpr (MASK == 8) return dpp_mov<kDppRowRor8>(x);
    else return __shfl_xor(x, MASK, kWave);
}

// Sum / max over the lanes of aligned groups of W lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (W >= 64) x += __shfl_xor(x, 32, kWave);
    if constexpr (W >= 32) x += __shfl_xor(x, 16, kWave);
    if constexpr (W >= 16) x += xchg<8>(x);
    if constexpr (W >= 8) x += xchg<4>(x);
    if constexpr (W >= 4) x += xchg<2>(x);
    if constexpr (W >= 2) x += xchg<1>(x);
    return x;
}
template <int W>
__device__ __forceinline__ float group_max(float x) {
    if constexpr (W >= 64) x = fmaxf(x, __shfl_xor(x, 32, kWave));
    if constexpr (W >= 32) x = fmaxf(x, __shfl_xor(x, 16, kWave));
    if constexpr (W >= 16) x = fmaxf(x, xchg<8>(x));
    if constexpr (W >= 8) x = fmaxf(x, xchg<4>(x));
    if constexpr (W >= 4) x = fmaxf(x, xchg<2>(x));
    if constexpr (W >= 2) x = fmaxf(x, xchg<1>(x));
    return x;
}

// Transposed butterfly: v[0..N) hold this lane's partial sums of N quantities
// whose full sums run over the lanes of an aligned group (lane bits below
// 2*BIT).  Each step pairs lanes that differ in bit BIT; one keeps the lower
// half of the quantities, its partner the upper half (padded with a zero when
// the count is odd), and each adds the other's contribution for the half it
// keeps.  After the bits down to 1, lane holds the full sums of quantities
// [base, base + valid) in v[0..valid); the returned compile-time count bounds
// valid.  When N is smaller than the group, several lanes hold the same
// quantity.  Costs about N exchanges instead of N * log2(group).
template <int N, int BIT>
__device__ __forceinline__ int tbfly(float* v, int lane, int& base, int& valid) {
    if constexpr (BIT == 0) {
        return N;
    } else if constexpr (N >= 2) {
        constexpr int H = (N + 1) / 2;
        const bool up = (lane & BIT) != 0;
#pragma unroll
        for (int k = 0; k < H; ++k) {
            const float lo = v[k];
            const float hi = (H + k < N) ? v[H + k] : 0.0f;
            const float keep = up ? hi : lo;
            const float send = up ? lo : hi;
            v[k] = keep + xchg<BIT>(send);
        }
        base += up ? H : 0;
        valid = up ? (valid > H ? valid - H : 0) : (valid < H ? valid : H);
        return tbfly<H, BIT / 2>(v, lane, base, valid);
    } else {
        v[0] += xchg<BIT>(v[0]);
        return tbfly<1, BIT / 2>(v, lane, base, valid);
    }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pkv
