// peak_probe.hip -- the two measurement kernels of pkv_probe.h: a streaming read
// of a large buffer (achievable HBM read rate) and bf16 matrix-core chains with
// no memory traffic (achievable MFMA rate).  Built into a library of its own;
// nothing of the attention path uses it.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// chunk i (16 bytes) of the buffer is read by thread i % stride, once
__global__ __launch_bounds__(PKV_PROBE_THREADS) void stream_read_kernel(const u32x4* buf, int64_t chunks,
                                                                      uint32_t* sink) {
    const int64_t stride = (int64_t)gridDim.x * PKV_PROBE_THREADS;
    const int64_t t = (int64_t)blockIdx.x * PKV_PROBE_THREADS + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    int64_t i = t;
    for (; i + 3 * stride < chunks; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(buf + i);
        const u32x4 b = __builtin_nontemporal_load(buf + i + stride);
        const u32x4 c = __builtin_nontemporal_load(buf + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(buf + i + 3 * stride);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < chunks; i += stride) acc ^= __builtin_nontemporal_load(buf + i);
    sink[t] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// workgroup w reads chunks [w span, min((w + 1) span, chunks)) once, in order
__global__ __launch_bounds__(PKV_PROBE_THREADS) void stream_read_spans_kernel(const u32x4* buf, int64_t chunks,
                                                                            int64_t span, uint32_t* sink) {
    constexpr int T = PKV_PROBE_THREADS;
    const int64_t start = (int64_t)blockIdx.x * span;
    const int64_t end = start + span < chunks ? start + span : chunks;
    u32x4 acc = {0u, 0u, 0u, 0u};
    int64_t i = start + threadIdx.x;
    for (; i + 3 * T < end; i += 4 * T) {
        const u32x4 a = __builtin_nontemporal_load(buf + i);
        const u32x4 b = __builtin_nontemporal_load(buf + i + T);
        const u32x4 c = __builtin_nontemporal_load(buf + i + 2 * T);
        const u32x4 d = __builtin_nontemporal_load(buf + i + 3 * T);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < end; i += T) acc ^= __builtin_nontemporal_load(buf + i);
    sink[(int64_t)blockIdx.x * T + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}
__global__ __launch_bounds__(PKV_PROBE_THREADS) void mfma_bf16_kernel(float* sink, int32_t iters, uint32_t seed) {
    const int t = blockIdx.x * PKV_PROBE_THREADS + threadIdx.x;
    // operands from the thread id and a run-time seed, small enough that the
    // accumulators stay finite
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)((float)((seed + 7u * (uint32_t)t + (uint32_t)e) & 15u) * 0.0009765625f);
        b[e] = (__bf16)((float)((seed * 3u + (uint32_t)t + 5u * (uint32_t)e) & 15u) * 0.0009765625f);
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
    sink[t] = s;
}

}  // namespace

extern "C" int pkv_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t grid,
                                     hipStream_t stream) {
    if (!buf || !sink || bytes <= 0 || bytes % 16 != 0 || grid <= 0 ||
        reinterpret_cast<uintptr_t>(buf) % 16 != 0)
        return 1;
    stream_read_kernel<<<dim3(grid), dim3(PKV_PROBE_THREADS), 0, stream>>>(static_cast<const u32x4*>(buf),
                                                                          bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int pkv_probe_stream_read_spans(const void* buf, int64_t bytes, uint32_t* sink, int32_t grid,
                                           hipStream_t stream) {
    if (!buf || !sink || bytes <= 0 || bytes % 16 != 0 || grid <= 0 ||
        reinterpret_cast<uintptr_t>(buf) % 16 != 0)
        return 1;
    const int64_t chunks = bytes / 16;
    const int64_t span = (chunks + grid - 1) / grid;
    stream_read_spans_kernel<<<dim3(grid), dim3(PKV_PROBE_THREADS), 0, stream>>>(static_cast<const u32x4*>(buf),
                                                                                chunks, span, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
extern "C" int pkv_probe_mfma_bf16(float* sink, int32_t iters, int32_t grid, uint32_t seed, hipStream_t stream) {
    if (!sink || iters < 0 || grid <= 0) return 1;
    mfma_bf16_kernel<<<dim3(grid), dim3(PKV_PROBE_THREADS), 0, stream>>>(sink, iters, seed);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
