// prefill.hip -- paged attention for a chunk of new query tokens per sequence
// (chunked prefill) on bf16 MFMA.
//
// "PyTorch LLM Serving Engine", What is implemented: prefill is cut into
// chunks of a chosen size that run in the same engine step as decode rows;
// Loading: the chunk's keys and values are stored first, then its queries
// visit the block table with an online (running-maximum) softmax.  "MicroGen", Key
// Features: grouped-query heads, window-length limit.
//
// Many query rows make Q.K^T and P.V dense contractions, so they run on
// 32x32x16 MFMA with fp32 accumulation: Q.K^T in bf16 (the inputs' own
// type, exact), P.V in fp16.  The softmax weights P are rounded to fp16
// (11 significant bits) rather than bf16 (8): with few visible keys a bf16
// weight error of 2^-9 moves the output by up to ~2^-9 * max|v|.  V is
// converted from bf16 to fp16 as it is staged; that is exact for
// 2^-14 <= |v| <= 65504 (smaller values keep an absolute error below 2^-25;
// larger ones are outside what this path supports).
//  * A workgroup (8 waves, one per CU) owns 256 rows of one (sequence, KV
//    head): rows are (chunk token, query head of the group) pairs, so all G
//    heads of a group share every K/V tile the workgroup stages.  Each wave
//    owns 32 rows; its Q fragment stays in registers.
//  * Keys come in tiles of 64 (four 16-token blocks gathered through the
//    block table), staged through registers into two LDS buffers: K
//    row-major, V transposed.  Tiles wholly outside every row's
//    causal/window range are never visited; masks are applied only on edge
//    tiles, by selection.
//  * Each wave computes S^T = K Q^T, so one lane's accumulators hold one
//    query row's scores: the row max/sum are lane-local plus one exchange
//    with lane^32.  K rows are staged with bits 2 and 3 of the key index
//    swapped, which makes each lane's 8 consecutive accumulators 8
//    consecutive keys: converted to fp16 they are directly the B operand of
//    O^T += V^T P^T, and V^T is read with one 16-byte LDS load per operand.
//  * Software pipeline: while a wave exponentiates tile t, the MFMAs of tile
//    t + 1's S^T are already issued (same basic block), so the matrix cores
//    and the VALU work at once; tile t + 2 is in registers on its way to LDS.
//  * Online softmax in fp32 with exp2 (scale * log2 e folded in) and a lazy
//    rescale (the output is rescaled only when a row maximum grows by > 2^8).
//  * Workgroups of one (sequence, KV head) are placed on the same XCD so the
//    K/V tiles they all read stay in that XCD's L2; the (sequence, KV head)
//    units are dealt to the XCDs round-robin, so each gets the same mix.
//
// INT8 pools ("MicroGen", Key Features: dynamic per-vector INT8 KV): K codes
// are staged as bf16 (integers up to 127 are exact), so Q.K^T of the codes is
// the same MFMA, and each score column is then multiplied by its key's scale
// (times softmax scale * log2 e, staged per tile in LDS): the dequantised
// logit without rounding K.  V codes are staged as exact fp16 integers and
// each key's V scale goes into its weight: w = p * scale (fp32) is carried as
// an fp16 value plus its fp16 remainder, and P.V takes one MFMA for each, so
// the weights keep ~22 significant bits (one fp16 rounding of w moves the
// output by up to ~2^-12 |v|, which the 1% x8 outliers make visible); the row
// sum adds the fp32 p.  Weights and P.V go one 16-key k-step at a time so the
// remainders add little to the registers live at once.
#include <type_traits>

#include "pkv_internal.h"
#include "pkv_device.h"

namespace pkv {

namespace {

constexpr int kKeys = 64;               // keys per tile
constexpr int kBlk = 16;
constexpr int kVtStride = kKeys + 8;    // halfwords per V^T row (16-byte aligned)
constexpr int kXcds = 8;
#ifndef PKV_RING_WAVES
#define PKV_RING_WAVES 8
#endif
constexpr int kRingWaves = PKV_RING_WAVES;  // waves per workgroup of the bf16 head_dim-128 kernel

struct PrefillArgs {
    const uint16_t* q;
    void* out;
    const void* k_pool;         // bf16, or int8 codes
    const void* v_pool;
    const uint16_t* k_scale;    // INT8 pools: fp16 scales [blocks][heads][16]
    const uint16_t* v_scale;
    const int32_t* block_tables;
    const int32_t* table_offsets;   // per sequence: logical block of column 0 (null: all 0)
    const int32_t* seq_lens;
    const int32_t* cu_q_lens;
    int32_t num_seqs, num_q_heads, num_kv_heads, group, num_blocks, max_blocks;
    int32_t m_tiles;          // row tiles per (sequence, KV head)
    int32_t total;            // num_seqs * num_kv_heads * m_tiles
    int32_t window;
    float scale_log2;
    int32_t out_bf16;
};

__device__ __forceinline__ int swap23(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ f16x8_t as_f16x8(const u32x4_t& v) { return __builtin_bit_cast(f16x8_t, v); }

// Vt (V transposed, fp16) row d (72 halfwords apart) holds 8 groups of 8
// keys; group g sits at position g ^ ((d >> 4) & 7).  On gfx950's LDS (64
// banks, a 16-byte access served 16 lanes per pass) this keeps both the
// staging writes (rows 4q + e of 16 consecutive q) and the MFMA operand reads
// (rows d..d+15 of one group) at one pass per 16 lanes.
__device__ __forceinline__ int vt_col(int d, int g) { return ((g ^ ((d >> 4) & 7)) << 3); }

// W waves (32 query rows each) share double-buffered K/V tiles; each wave
// issues the next tile's S^T = K Q^T MFMAs with this tile's softmax.
template <int D, int W, bool ZS, bool I8>
__global__ __launch_bounds__(64 * W) void prefill_pipe_kernel(PrefillArgs a) {
    using KT = typename std::conditional<I8, int8_t, uint16_t>::type;   // pool element
    constexpr int NTH = 64 * W;                 // threads
    constexpr int ROWS = 32 * W;                // query rows per workgroup
    constexpr int KS = D + 8;                   // halfwords per K row in LDS
    constexpr int DK = D / 16;                  // k-steps of Q.K^T
    constexpr int NT = D / 32;                  // 32-wide d tiles of the output
    constexpr int KCH = kKeys * (D / 8) / NTH;  // 16-byte K chunks staged per thread
    constexpr int KPB = kBlk * (D / 8);         // K chunks per block
    constexpr int VPIECES = 8 * (D / 2);        // (8-key group, 2 dims) pieces of V per tile
    constexpr float kRescale = 8.0f;            // rescale O only when a row max grows by > 2^8
    static_assert(KCH >= 1 && NTH % KPB == 0 && VPIECES <= NTH, "staging shape");
    __shared__ __attribute__((aligned(16))) uint16_t s_k[2][kKeys * KS];
    __shared__ __attribute__((aligned(16))) uint16_t s_vt[2][D * kVtStride];   // V^T as fp16
    __shared__ __attribute__((aligned(16))) float s_ksc[I8 ? 2 : 1][I8 ? kKeys : 4];  // K scale * scale_log2
    __shared__ __attribute__((aligned(16))) float s_vsc[I8 ? 2 : 1][I8 ? kKeys : 4];  // V scale

    // ---- work item: workgroup i runs on XCD i % 8.  (sequence, KV head) units are
    // dealt round-robin to the XCDs: the row tiles of a unit stay on one XCD and
    // share its K/V tiles through that XCD's L2, and every XCD gets the same mix
    // of short and long sequences
    const int units = a.total / a.m_tiles;
    const int xcd = blockIdx.x % kXcds;
    const int j = blockIdx.x / kXcds;                       // position on that XCD
    const int unit = (j / a.m_tiles) * kXcds + xcd;
    if (unit >= units) return;
    const int mt = j % a.m_tiles;
    const int w_idx = unit * a.m_tiles + mt;
    const int g = (w_idx / a.m_tiles) % a.num_kv_heads;
    const int s = w_idx / (a.m_tiles * a.num_kv_heads);
    const int G = a.group;
    const int q0 = a.cu_q_lens[s];
    const int C = a.cu_q_lens[s + 1] - q0;
    // column c of the sequence's row holds logical block c + off (blocks before it released)
    const int off = a.table_offsets ? max(0, a.table_offsets[s]) : 0;
    const int L = (int)min((int64_t)a.seq_lens[s], ((int64_t)a.max_blocks + off) * kBlk);
    const int nrows = C * G;
    const int r0 = mt * ROWS;
    if (r0 >= nrows || C <= 0 || C > L) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;                    // lane half
    const int base_pos = L - C;                 // position of chunk token 0
    const int p_min = base_pos + r0 / G;
    const int p_max = base_pos + (min(nrows, r0 + ROWS) - 1) / G;

    // ---- this lane's query row and its Q fragment (B operand of S^T = K Q^T)
    const int row = r0 + wave * 32 + (lane & 31);
    const bool row_ok = row < nrows;
    const int tok = row_ok ? row / G : 0;
    const int jh = row_ok ? row - tok * G : 0;
    const int p_row = row_ok ? base_pos + tok : p_max;
    bf16x8_t qf[DK];
    {
        const uint16_t* qp = a.q + ((int64_t)(q0 + tok) * a.num_q_heads + g * G + jh) * D + 8 * h;
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) {
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (row_ok) v = *reinterpret_cast<const u32x4_t*>(qp + 16 * ks);
            qf[ks] = as_bf16x8(v);
        }
    }

    f32x16_t o[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[nt][v] = 0.0f;
    float m_used = -INFINITY;    // max the weights are taken against (log2 units)
    float l_run = 0.0f;          // this lane's share of the row sum

    const int k_lo = (a.window > 0) ? max(0, p_min - a.window + 1) : 0;
    // tiles of 64 keys from a 64-key boundary, but never before the row's first
    // block (tiles need only block alignment), so every table read is in the row
    const int kt_first = max((k_lo / kKeys) * kKeys, off * kBlk);
    const int n_tiles = kt_first <= p_max ? (p_max - kt_first) / kKeys + 1 : 0;
    const int last_blk = (L - 1) / kBlk;        // last logical block with keys
    // read-only during the kernel: through the constant address space its reads stay
    // scalar loads whatever else the kernel does
    const __attribute__((address_space(4))) int32_t* table =
        (const __attribute__((address_space(4))) int32_t*)(a.block_tables + (int64_t)s * a.max_blocks - off);
    const int64_t head_stride = (int64_t)kBlk * D;          // elements per (block, head) tile
    const int64_t blk_stride = (int64_t)a.num_kv_heads * head_stride;

    // ---- staging roles: KCH 16-byte K chunks and (if any) one V piece per thread
    //  K chunk c = tid + NTH i: key c / (D/8), dims (c % (D/8)) * 8 .. +8
    //  V piece t = tid: dims 2 (t % (D/2)), +1 of keys 8 (t / (D/2)) .. +8
    const bool v_task = tid < VPIECES;
    const int v_dp = tid % (D / 2);
    const int v_kg = (tid / (D / 2)) & 7;
    const int k_off = ((tid / (D / 8)) % kBlk) * D + (tid % (D / 8)) * 8;
    const int v_off = ((8 * v_kg) % kBlk) * D + 2 * v_dp;
    u32x4_t kreg[I8 ? 1 : KCH];          // bf16: 8 elements per chunk
    u32x2_t kreg8[I8 ? KCH : 1];         // INT8: 8 codes per chunk
    uint32_t vreg[I8 ? 4 : 8];           // bf16: 2 elements of key i; INT8: 2 codes of keys 2i, 2i + 1
    uint32_t ksreg = 0, vsreg = 0;      // INT8: fp16 K and V scales of key tid (wave 0)
    int id0 = 0, id1 = 0, id2 = 0, id3 = 0;     // physical blocks of the staged tile (0 when invalid)

    auto kt_of = [&](int t) { return kt_first + kKeys * t; };
    auto tile_ids = [&](int kt) {               // block ids of a tile (wave-uniform): bit b = block b valid
        int m = 0;
        int got[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int lb = kt / kBlk + b;
            const int id = lb <= last_blk ? table[lb] : -1;   // lb >= off: kt_first
            const bool ok = id >= 0 && id < a.num_blocks;
            got[b] = ok ? id : 0;               // an invalid block reads block 0 and is masked
            m |= (ok ? 1 : 0) << b;
        }
        id0 = got[0]; id1 = got[1]; id2 = got[2]; id3 = got[3];
        return m;
    };
    auto sel = [&](int b) { return b == 0 ? id0 : (b == 1 ? id1 : (b == 2 ? id2 : id3)); };
    auto blk_base = [&](const void* pool, int id) {
        return static_cast<const KT*>(pool) + (int64_t)id * blk_stride + g * head_stride;
    };
    // INT8 scale of (block id, this head, offset)
    auto scale_at = [&](const uint16_t* sc, int id, int off) {
        return sc + ((int64_t)id * a.num_kv_heads + g) * kBlk + off;
    };
    auto load_tile = [&]() {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int id = sel((NTH * i) / KPB + tid / KPB);
            if constexpr (I8) {
                kreg8[i] = *reinterpret_cast<const u32x2_t*>(blk_base(a.k_pool, id) + k_off);
            } else {
                kreg[i] = *reinterpret_cast<const u32x4_t*>(blk_base(a.k_pool, id) + k_off);
            }
        }
        if (v_task) {
            const KT* vp = blk_base(a.v_pool, sel(v_kg / 2)) + v_off;
            if constexpr (I8) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    vreg[i] = (uint32_t)*reinterpret_cast<const uint16_t*>(vp + 2 * i * D) |
                              ((uint32_t)*reinterpret_cast<const uint16_t*>(vp + (2 * i + 1) * D) << 16);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) vreg[i] = *reinterpret_cast<const uint32_t*>(vp + i * D);
            }
        }
        if constexpr (I8) {
            if (tid < kKeys) {
                ksreg = *scale_at(a.k_scale, sel(tid / kBlk), tid % kBlk);
                vsreg = *scale_at(a.v_scale, sel(tid / kBlk), tid % kBlk);
            }
        }
    };
    auto store_tile = [&](int buf, int kt, int m) {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int c = tid + NTH * i;
            const int key = c / (D / 8), dc = c % (D / 8);
            u32x4_t kv;
            if constexpr (I8) {
                // 8 codes -> 8 bf16 integers (exact): the top half of each code's fp32
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t word = kreg8[i][w >> 1] >> (16 * (w & 1));
                    const float lo = (float)(int8_t)(word & 0xffu);
                    const float hi = (float)(int8_t)((word >> 8) & 0xffu);
                    kv[w] = (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xffff0000u);
                }
            } else {
                kv = kreg[i];
            }
            *reinterpret_cast<u32x4_t*>(&s_k[buf][swap23(key) * KS + dc * 8]) = kv;
        }
        if constexpr (I8) {
            if (tid < kKeys) {
                // keys past the sequence or in a missing block may hold NaN scales: 0
                const bool live = ((m >> (tid / kBlk)) & 1) && kt + tid < L;
                const float ks = (float)__builtin_bit_cast(_Float16, (uint16_t)ksreg);
                const float vs = (float)__builtin_bit_cast(_Float16, (uint16_t)vsreg);
                s_ksc[buf][tid] = live ? ks * a.scale_log2 : 0.0f;
                s_vsc[buf][tid] = live ? vs : 0.0f;
            }
            if (v_task) {
                // 8 keys x 2 dims -> 2 rows of 8 keys, the codes as exact fp16
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    u32x4_t r;
#pragma unroll
                    for (int mm = 0; mm < 4; ++mm)
                        r[mm] = pack_f16x2((float)(int8_t)((vreg[mm] >> (8 * e)) & 0xffu),
                                           (float)(int8_t)((vreg[mm] >> (16 + 8 * e)) & 0xffu));
                    const int d = 2 * v_dp + e;
                    *reinterpret_cast<u32x4_t*>(&s_vt[buf][d * kVtStride + vt_col(d, v_kg)]) = r;
                }
            }
        } else if (v_task) {
            uint32_t* w = vreg;
            if (m != 15 || kt + kKeys > L) {    // edge tile (uniform branch): zero dead keys, they may hold NaN
                const bool blk_live = (m >> (v_kg / 2)) & 1;
#pragma unroll
                for (int i = 0; i < 8; ++i) w[i] = (blk_live && kt + 8 * v_kg + i < L) ? w[i] : 0u;
            }
            // 8 keys x 2 dims -> 2 rows of 8 keys, bf16 -> fp16
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                u32x4_t r;
#pragma unroll
                for (int mm = 0; mm < 4; ++mm)
                    r[mm] = e ? pack_f16x2(bf16hi(w[2 * mm]), bf16hi(w[2 * mm + 1]))
                              : pack_f16x2(bf16lo(w[2 * mm]), bf16lo(w[2 * mm + 1]));
                const int d = 2 * v_dp + e;
                *reinterpret_cast<u32x4_t*>(&s_vt[buf][d * kVtStride + vt_col(d, v_kg)]) = r;
            }
        }
    };

    // S^T of a staged tile for the wave's 32 rows: two 32-key halves, their MFMA
    // chains interleaved and the K operands read a k-step ahead
    auto compute_s = [&](f32x16_t* S, int buf) {
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int v = 0; v < 16; ++v) S[T][v] = 0.0f;
        const uint16_t* kr0 = &s_k[buf][(lane & 31) * KS + 8 * h];
        const uint16_t* kr1 = kr0 + 32 * KS;
        u32x4_t k0 = *reinterpret_cast<const u32x4_t*>(kr0);
        u32x4_t k1 = *reinterpret_cast<const u32x4_t*>(kr1);
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) {
            u32x4_t n0 = k0, n1 = k1;
            if (ks + 1 < DK) {
                n0 = *reinterpret_cast<const u32x4_t*>(kr0 + 16 * (ks + 1));
                n1 = *reinterpret_cast<const u32x4_t*>(kr1 + 16 * (ks + 1));
            }
            S[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(k0), qf[ks], S[0], 0, 0, 0);
            S[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(k1), qf[ks], S[1], 0, 0, 0);
            k0 = n0;
            k1 = n1;
        }
    };

    // masks, online softmax and O^T += V^T P^T for tile t (scores in S, V in buf);
    // the next tile's S^T MFMAs (into S_nxt, from buffer buf ^ 1) are issued in
    // the same basic block as the exp2 work so the two overlap.  On the last
    // tile that buffer holds stale data: the MFMAs still read in-bounds LDS and
    // their result is never used.
    // the factor that turns an accumulated score into log2 units (INT8: the
    // per-key factor is already applied)
    const float sl2 = I8 ? 1.0f : a.scale_log2;
    const int xaddr = (lane ^ 32) << 2;        // ds_bpermute address of lane ^ 32
    float msub = 0.0f;                         // m_used, or 0 while it is -inf
    auto finish_tile = [&](f32x16_t* S, f32x16_t* S_nxt, int buf, int kt, int tmask) {
        if constexpr (I8) {
            // score of key j times scale_j * softmax scale * log2 e (before masking: a
            // dead key's NaN scale is then selected away)
            const float* kp = &s_ksc[buf][8 * h];
#pragma unroll
            for (int T = 0; T < 2; ++T)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const f32x4_t f0 = *reinterpret_cast<const f32x4_t*>(kp + 32 * T + 16 * u);
                    const f32x4_t f1 = *reinterpret_cast<const f32x4_t*>(kp + 32 * T + 16 * u + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        S[T][8 * u + e] *= f0[e];
                        S[T][8 * u + 4 + e] *= f1[e];
                    }
                }
        }
        // masks (edge tiles only): key of accumulator v = kt + 32T + 16(v/8) + 8h + v%8
        const bool full = tmask == 15 && kt + kKeys - 1 <= p_min && (a.window <= 0 || kt >= p_max - a.window + 1);
        if (!full) {
#pragma unroll
            for (int T = 0; T < 2; ++T)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int key = kt + 32 * T + 16 * (v / 8) + 8 * h + (v % 8);
                    const bool vis = ((tmask >> ((key - kt) / kBlk)) & 1) && key <= p_row &&
                                     (a.window <= 0 || key > p_row - a.window);
                    S[T][v] = vis ? S[T][v] : -INFINITY;
                }
        }
        // online softmax for the row (lane-local + lane^32), lazy rescale
        float mt_ = -INFINITY;
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int v = 0; v < 16; ++v) mt_ = fmaxf(mt_, S[T][v]);
        mt_ = fmaxf(mt_, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(xaddr, __builtin_bit_cast(int, mt_))));
        // with a positive scale, m_used + 8 stays -inf until the row's first visible
        // key, so the comparison alone starts the running maximum, and 2^(m_used -
        // m_new) is then 2^-inf = 0 (a zero scale keeps the explicit guards)
        const float m_tile = (ZS && mt_ == -INFINITY) ? -INFINITY : mt_ * sl2;
        const bool grow = ZS ? (m_tile > m_used + kRescale || (m_used == -INFINITY && m_tile != -INFINITY))
                             : m_tile > m_used + kRescale;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float m_new = grow ? m_tile : m_used;
            const float alpha = (ZS && m_used == -INFINITY) ? 0.0f : fast_exp2(m_used - m_new);
            m_used = m_new;
            msub = (m_used == -INFINITY) ? 0.0f : m_used;
            const float f = grow ? alpha : 1.0f;
            l_run *= f;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int v = 0; v < 16; ++v) o[nt][v] *= f;
        }
        compute_s(S_nxt, buf ^ 1);
        // V^T row d = 32 nt + (lane & 31), key group 2 ks + h, at one base + constants
        const uint16_t* vt_base = &s_vt[buf][(lane & 31) * kVtStride + 8 * (h ^ ((lane >> 4) & 1))];
        if constexpr (I8) {
            // w = p * V scale as fp16 + fp16 remainder; O^T += V^T W^T for each part.
            // One k-step (16 keys) at a time: its weights, then its MFMAs.
            const float* vsp = &s_vsc[buf][8 * h];
            float ls = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int T = ks >> 1, u = ks & 1;
                const f32x4_t f0 = *reinterpret_cast<const f32x4_t*>(vsp + 32 * T + 16 * u);
                const f32x4_t f1 = *reinterpret_cast<const f32x4_t*>(vsp + 32 * T + 16 * u + 4);
                u32x4_t pb, pr;
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float x0 = S[T][8 * u + e], x1 = S[T][8 * u + e + 1];
                    float p0, p1;
                    if constexpr (ZS) {
                        p0 = (x0 == -INFINITY) ? 0.0f : fast_exp2(x0 - msub);
                        p1 = (x1 == -INFINITY) ? 0.0f : fast_exp2(x1 - msub);
                    } else {
                        p0 = fast_exp2(x0 - msub);
                        p1 = fast_exp2(x1 - msub);
                    }
                    ls += p0 + p1;
                    const float w0 = p0 * (e < 4 ? f0[e] : f1[e - 4]);
                    const float w1 = p1 * (e < 4 ? f0[e + 1] : f1[e - 3]);
                    const float h0 = (float)(_Float16)w0, h1 = (float)(_Float16)w1;
                    pb[e / 2] = pack_f16x2(h0, h1);
                    pr[e / 2] = pack_f16x2(w0 - h0, w1 - h1);
                }
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const u32x4_t vv = *reinterpret_cast<const u32x4_t*>(
                        vt_base + 32 * nt * kVtStride + 16 * ((ks ^ nt) & 7));
                    o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(vv), as_f16x8(pb), o[nt], 0, 0, 0);
                    o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(vv), as_f16x8(pr), o[nt], 0, 0, 0);
                }
            }
            l_run += ls;
        } else {
            uint32_t pw[2][8];                       // P^T as fp16 pairs: [T][4u + word]
            if constexpr (!ZS) {
                // a masked score (-inf) scales to -inf and exp2 gives 0 by itself
#pragma unroll
                for (int T = 0; T < 2; ++T)
#pragma unroll
                    for (int v = 0; v < 16; v += 2)
                        pw[T][v / 2] = pack_f16x2(fast_exp2(fmaf(S[T][v], sl2, -msub)),
                                                  fast_exp2(fmaf(S[T][v + 1], sl2, -msub)));
            } else {
                // scale 0: -inf * 0 would be NaN, so masked scores are selected away
#pragma unroll
                for (int T = 0; T < 2; ++T)
#pragma unroll
                    for (int v = 0; v < 16; v += 2) {
                        const float x0 = S[T][v], x1 = S[T][v + 1];
                        const float p0 = (x0 == -INFINITY) ? 0.0f : fast_exp2(fmaf(x0, sl2, -msub));
                        const float p1 = (x1 == -INFINITY) ? 0.0f : fast_exp2(fmaf(x1, sl2, -msub));
                        pw[T][v / 2] = pack_f16x2(p0, p1);
                    }
            }
            // row sum of the fp16 weights -- the values P.V multiplies -- two per dot2
            {
                const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
                float ls0 = 0.0f, ls1 = 0.0f;
#pragma unroll
                for (int w = 0; w < 8; ++w) {
                    ls0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pw[0][w]), one, ls0, false);
                    ls1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pw[1][w]), one, ls1, false);
                }
                l_run += ls0 + ls1;
            }
            // O^T += V^T P^T: k-step ks covers keys 16ks..16ks+15 (tile T = ks/2, u = ks%2)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int T = ks >> 1, u = ks & 1;
                u32x4_t pb;
                pb[0] = pw[T][4 * u + 0]; pb[1] = pw[T][4 * u + 1];
                pb[2] = pw[T][4 * u + 2]; pb[3] = pw[T][4 * u + 3];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const int off = 32 * nt * kVtStride + 16 * ((ks ^ nt) & 7);
                    const u32x4_t vv = *reinterpret_cast<const u32x4_t*>(vt_base + off);
                    o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(vv), as_f16x8(pb), o[nt], 0, 0, 0);
                }
            }
        }
    };

    // ---- prologue: tiles 0 and 1 staged (buffers 0 and 1), S of tile 0, tile 2 in registers
    int mk0 = 0, mk1 = 0, mk2 = 0;              // masks of tiles t, t + 1, t + 2 (t + 2: in registers)
    f32x16_t sa[2], sb[2];
    if (n_tiles > 0) {
        mk0 = tile_ids(kt_of(0));
        load_tile();
        store_tile(0, kt_of(0), mk0);
    }
    if (n_tiles > 1) {
        mk1 = tile_ids(kt_of(1));
        load_tile();
    }
    __syncthreads();                            // tile 0 visible
    // unconditional (with no tile it reads stale LDS and the result is unused): Q's
    // first use is then on every path into the loop, so the wait the compiler puts
    // on Q's loads stays out of the loop, where it would also cover the tile loads
    // just issued and expose their latency every tile
    compute_s(sa, 0);
    if (n_tiles > 1) store_tile(1, kt_of(1), mk1);
    if (n_tiles > 2) {
        mk2 = tile_ids(kt_of(2));
        load_tile();
    }
    __syncthreads();                            // tile 1 visible

    // ---- steady state: tile t in buffer t & 1 with its S in hand; tile t + 1 in
    // the other buffer; tile t + 2 in registers
    auto step = [&](f32x16_t* s_cur, f32x16_t* s_nxt, int t) {
        const int buf = t & 1;
        finish_tile(s_cur, s_nxt, buf, kt_of(t), mk0);
        __syncthreads();                        // every wave is done with buffer buf
        if (t + 2 < n_tiles) store_tile(buf, kt_of(t + 2), mk2);
        __syncthreads();                        // tile t + 2 visible
        mk0 = mk1;
        mk1 = mk2;
        if (t + 3 < n_tiles) {                  // fetch tile t + 3 while t + 1 is used
            mk2 = tile_ids(kt_of(t + 3));
            load_tile();
        }
    };
    for (int t = 0; t < n_tiles; t += 2) {
        step(sa, sb, t);
        if (t + 1 < n_tiles) step(sb, sa, t + 1);
    }

    // ---- normalise and store: lane holds d = 32nt + 8(v/4) + 4h + v%4 of its row
    const float l_row = l_run + __shfl_xor(l_run, 32, kWave);
    if (!row_ok) return;
    const float inv = l_row > 0.0f ? 1.0f / l_row : 0.0f;
    const int64_t obase = ((int64_t)(q0 + tok) * a.num_q_heads + g * G + jh) * D;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            const int d = 32 * nt + 8 * v4 + 4 * h;
            const float r0_ = o[nt][4 * v4 + 0] * inv, r1_ = o[nt][4 * v4 + 1] * inv;
            const float r2_ = o[nt][4 * v4 + 2] * inv, r3_ = o[nt][4 * v4 + 3] * inv;
            if (a.out_bf16) {
                u32x2_t pk;
                pk[0] = pack_bf16x2(r0_, r1_);
                pk[1] = pack_bf16x2(r2_, r3_);
                *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(a.out) + obase + d) = pk;
            } else {
                f32x4_t fv = {r0_, r1_, r2_, r3_};
                *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.out) + obase + d) = fv;
            }
        }
}

// ---------------------------------------------------------------- bf16 pools, head_dim 128
// The same work decomposition, online softmax and MFMA layouts as
// prefill_pipe_kernel, with the K tiles copied from the pool straight into LDS
// (no registers, no VALU, no LDS store instructions) and one barrier per tile:
//  * K: each wave copies 8 of a tile's 64 rows, one 256-byte row per
//    global_load_lds_dword (lane l's 4 bytes land at the row's LDS address +
//    4 l), so each row keeps its 16-byte pad and the MFMA operand reads stay
//    conflict-free.  LDS row R holds key swap23(R); rows 8w .. 8w+7 of wave w
//    all lie in block w / 2 of the tile.
//  * V: staged through registers as before (converted to fp16 and transposed).
//  * Two K slots and two V slots.  Iteration t: store V(t+1) (loaded during
//    iteration t-1) into its slot, start copying K(t+2) and loading V(t+2),
//    then the softmax of tile t with tile t+1's S^T MFMAs, then P.V of tile t;
//    then wait for this wave's loads and copies and pass the one barrier.
//    Each slot is overwritten only after the barrier that follows its last
//    reader.
// The copies are issued with inline asm (the compiler would otherwise wait for
// every outstanding load before each LDS read, which defeats the prefetch);
// the waits for them are explicit, and M0 is saved and restored around each.

// Eight 256-byte K rows of one (block, KV head) run, at keys {0, 1, 2, 3, 8, 9,
// 10, 11} from `src`, to eight consecutive padded LDS rows (272 bytes apart)
// from LDS address `lds`: lane l's 4 bytes of each row from row + 4 l to the
// LDS row + 4 l.  A global_load_lds writes LDS address M0 + offset + 4 lane,
// where the instruction's immediate offset moves the global address too, so
// the offsets stay 0: the rows' global offsets come in `voff` (lane l: 4 l +
// 256 k for keys k = 0..3, keys 8..11 from a second base 2048 bytes on), and
// M0 steps by one padded row.  One asm block: M0 is saved and restored,
// `s_nop 4` first (a VMEM read of an SGPR that a VALU op has just written
// needs 5 wait states), `s_nop 0` after each M0 write (an LDS copy reading M0
// right after a SALU write of it needs 1).
__device__ __forceinline__ void lds_copy_k8(uint32_t lds, const uint16_t* src, const uint32_t (&voff)[4]) {
    const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
    const uint64_t gp = (uint64_t)(uintptr_t)src;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)gp);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(gp >> 32));
    const uint64_t g0 = ((uint64_t)hi << 32) | lo;
    const uint64_t g1 = g0 + 2048;
    uint32_t saved;
    asm volatile(
        "s_nop 4\n\t"
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %2, %6\n\t"
        "s_add_u32 m0, m0, 0x110\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %3, %6\n\t"
        "s_add_u32 m0, m0, 0x110\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %4, %6\n\t"
        "s_add_u32 m0, m0, 0x110\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %5, %6\n\t"
        "s_add_u32 m0, m0, 0x110\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %2, %7\n\t"
        "s_add_u32 m0, m0, 0x110\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %3, %7\n\t"
        "s_add_u32 m0, m0, 0x110\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %4, %7\n\t"
        "s_add_u32 m0, m0, 0x110\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %5, %7\n\t"
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0"
        : "=&s"(saved)
        : "s"(m), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(g0), "s"(g1)
        : "memory", "scc");
}

// Wait for every load and LDS copy this wave has issued, and for its LDS
// stores, then the workgroup barrier.
__device__ __forceinline__ void wait_all_and_barrier() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// W waves per workgroup (4 or 8), two waves per SIMD either way: with W = 4
// two workgroups share a CU, so the two waves of a SIMD belong to different
// workgroups and do not meet at the same barriers.
template <int W, bool ZS>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_ring_kernel(PrefillArgs a) {
    constexpr int D = 128;
    constexpr int NTH = 64 * W;
    constexpr int ROWS = 32 * W;                // query rows per workgroup
    constexpr int KROWS = kKeys / W;            // K rows of a tile each wave copies (8 or 16)
    constexpr int NVP = 8 * (D / 2) / NTH;      // V pieces each thread stages (1 or 2)
    static_assert(KROWS % 8 == 0 && NVP >= 1, "staging shape");
    constexpr int KS = D + 8;                   // halfwords per K row in LDS (272 bytes)
    constexpr int DK = D / 16;                  // k-steps of Q.K^T
    constexpr int NT = D / 32;                  // 32-wide d tiles of the output
    constexpr float kRescale = 8.0f;            // rescale O only when a row max grows by > 2^8
    __shared__ __attribute__((aligned(16))) uint16_t s_k[2][kKeys * KS];
    __shared__ __attribute__((aligned(16))) uint16_t s_vt[2][D * kVtStride];   // V^T as fp16

    // ---- work item (as in prefill_pipe_kernel)
    const int units = a.total / a.m_tiles;
    const int xcd = blockIdx.x % kXcds;
    const int j = blockIdx.x / kXcds;
    const int unit = (j / a.m_tiles) * kXcds + xcd;
    if (unit >= units) return;
    const int mt = j % a.m_tiles;
    const int w_idx = unit * a.m_tiles + mt;
    const int g = (w_idx / a.m_tiles) % a.num_kv_heads;
    const int s = w_idx / (a.m_tiles * a.num_kv_heads);
    const int G = a.group;
    const int q0 = a.cu_q_lens[s];
    const int C = a.cu_q_lens[s + 1] - q0;
    const int off = a.table_offsets ? max(0, a.table_offsets[s]) : 0;
    const int L = (int)min((int64_t)a.seq_lens[s], ((int64_t)a.max_blocks + off) * kBlk);
    const int nrows = C * G;
    const int r0 = mt * ROWS;
    if (r0 >= nrows || C <= 0 || C > L) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;
    const int base_pos = L - C;
    const int p_min = base_pos + r0 / G;
    const int p_max = base_pos + (min(nrows, r0 + ROWS) - 1) / G;

    const int row = r0 + wave * 32 + (lane & 31);
    const bool row_ok = row < nrows;
    const int tok = row_ok ? row / G : 0;
    const int jh = row_ok ? row - tok * G : 0;
    const int p_row = row_ok ? base_pos + tok : p_max;
    bf16x8_t qf[DK];
    {
        const uint16_t* qp = a.q + ((int64_t)(q0 + tok) * a.num_q_heads + g * G + jh) * D + 8 * h;
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) {
            u32x4_t v = {0u, 0u, 0u, 0u};
            if (row_ok) v = *reinterpret_cast<const u32x4_t*>(qp + 16 * ks);
            qf[ks] = as_bf16x8(v);
        }
    }

    f32x16_t o[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[nt][v] = 0.0f;
    float m_used = -INFINITY;
    float l_run = 0.0f;

    const int k_lo = (a.window > 0) ? max(0, p_min - a.window + 1) : 0;
    const int kt_first = max((k_lo / kKeys) * kKeys, off * kBlk);
    const int n_tiles = kt_first <= p_max ? (p_max - kt_first) / kKeys + 1 : 0;
    const int last_blk = (L - 1) / kBlk;
    const __attribute__((address_space(4))) int32_t* table =
        (const __attribute__((address_space(4))) int32_t*)(a.block_tables + (int64_t)s * a.max_blocks - off);
    const int64_t head_stride = (int64_t)kBlk * D;
    const int64_t blk_stride = (int64_t)a.num_kv_heads * head_stride;
    const uint16_t* k_pool = static_cast<const uint16_t*>(a.k_pool);
    const uint16_t* v_pool = static_cast<const uint16_t*>(a.v_pool);

    auto kt_of = [&](int t) { return kt_first + kKeys * t; };
    // physical block of block b of the tile at kt (block 0 when the entry is not a
    // block of the pool: those keys are masked), and the tile's validity mask
    auto block_id = [&](int kt, int b, bool& ok) {
        const int lb = kt / kBlk + b;
        const int id = lb <= last_blk ? table[lb] : -1;
        ok = id >= 0 && id < a.num_blocks;
        return ok ? id : 0;
    };
    auto tile_mask = [&](int kt) {
        int m = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            bool ok;
            (void)block_id(kt, b, ok);
            m |= (ok ? 1 : 0) << b;
        }
        return m;
    };

    // ---- this wave's K rows: groups of 8 rows R0 + i (R0 = KROWS wave + 8 c), in
    // block R0 / 16 of the tile, row R holding key swap23(R) = key0 + {0, 1, 2,
    // 3, 8, 9, 10, 11}[i] of that block, key0 = 4 when R0 is 8 past a block start
    static_assert(KS * 2 == 0x110 && D * 2 == 256, "row strides assumed by lds_copy_k8");
    const uint32_t k_voff[4] = {(uint32_t)lane * 4u, (uint32_t)lane * 4u + 256u, (uint32_t)lane * 4u + 512u,
                                (uint32_t)lane * 4u + 768u};
    auto copy_k = [&](int slot, int kt) {
#pragma unroll
        for (int c = 0; c < KROWS / 8; ++c) {
            const int r0 = KROWS * wave + 8 * c;
            bool ok;
            const int id = block_id(kt, r0 / kBlk, ok);
            const uint16_t* src = k_pool + (int64_t)id * blk_stride + g * head_stride + ((r0 / 8) & 1) * 4 * D;
            lds_copy_k8((uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)&s_k[slot][r0 * KS], src,
                        k_voff);
        }
    };

    // ---- V: piece (v_kg, v_dp) = dims 2 v_dp, +1 of keys 8 v_kg .. +8 (block
    // v_kg / 2); thread tid stages pieces v_kg = wave + W n, v_dp = tid % 64
    const int v_dp = tid % (D / 2);
    uint32_t vreg[NVP][8];
    auto load_v = [&](int kt) {
#pragma unroll
        for (int n = 0; n < NVP; ++n) {
            const int v_kg = wave + W * n;
            bool ok;
            const int id = block_id(kt, v_kg / 2, ok);
            const uint16_t* vp = v_pool + (int64_t)id * blk_stride + g * head_stride +
                                 ((8 * v_kg) % kBlk) * D + 2 * v_dp;
#pragma unroll
            for (int i = 0; i < 8; ++i) vreg[n][i] = *reinterpret_cast<const uint32_t*>(vp + i * D);
        }
    };
    auto store_v = [&](int slot, int kt, int m) {
#pragma unroll
        for (int n = 0; n < NVP; ++n) {
            const int v_kg = wave + W * n;
            uint32_t* w = vreg[n];
            if (m != 15 || kt + kKeys > L) {    // edge tile (uniform branch): zero dead keys, they may hold NaN
                const bool blk_live = (m >> (v_kg / 2)) & 1;
#pragma unroll
                for (int i = 0; i < 8; ++i) w[i] = (blk_live && kt + 8 * v_kg + i < L) ? w[i] : 0u;
            }
            // 8 keys x 2 dims -> 2 rows of 8 keys, bf16 -> fp16
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                u32x4_t r;
#pragma unroll
                for (int mm = 0; mm < 4; ++mm)
                    r[mm] = e ? pack_f16x2(bf16hi(w[2 * mm]), bf16hi(w[2 * mm + 1]))
                              : pack_f16x2(bf16lo(w[2 * mm]), bf16lo(w[2 * mm + 1]));
                const int d = 2 * v_dp + e;
                *reinterpret_cast<u32x4_t*>(&s_vt[slot][d * kVtStride + vt_col(d, v_kg)]) = r;
            }
        }
    };

    // S^T of a staged tile for the wave's 32 rows (as in prefill_pipe_kernel)
    auto compute_s = [&](f32x16_t* S, int slot) {
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int v = 0; v < 16; ++v) S[T][v] = 0.0f;
        const uint16_t* kr0 = &s_k[slot][(lane & 31) * KS + 8 * h];
        const uint16_t* kr1 = kr0 + 32 * KS;
        u32x4_t k0 = *reinterpret_cast<const u32x4_t*>(kr0);
        u32x4_t k1 = *reinterpret_cast<const u32x4_t*>(kr1);
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) {
            u32x4_t n0 = k0, n1 = k1;
            if (ks + 1 < DK) {
                n0 = *reinterpret_cast<const u32x4_t*>(kr0 + 16 * (ks + 1));
                n1 = *reinterpret_cast<const u32x4_t*>(kr1 + 16 * (ks + 1));
            }
            S[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(k0), qf[ks], S[0], 0, 0, 0);
            S[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(k1), qf[ks], S[1], 0, 0, 0);
            k0 = n0;
            k1 = n1;
        }
    };

    const int xaddr = (lane ^ 32) << 2;        // ds_bpermute address of lane ^ 32
    float msub = 0.0f;                         // m_used, or 0 while it is -inf
    // masks, online softmax and O^T += V^T P^T for tile t (scores in S, V in slot);
    // the next tile's S^T MFMAs (from K slot slot ^ 1) go out in the same basic
    // block as the exp2 work.  On the last tile that slot holds stale data: the
    // MFMAs read in-bounds LDS and the result is never used.
    const float sl2 = a.scale_log2;
    auto finish_tile = [&](f32x16_t* S, f32x16_t* S_nxt, int slot, int kt, int tmask) {
        const bool full = tmask == 15 && kt + kKeys - 1 <= p_min && (a.window <= 0 || kt >= p_max - a.window + 1);
        if (!full) {
#pragma unroll
            for (int T = 0; T < 2; ++T)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int key = kt + 32 * T + 16 * (v / 8) + 8 * h + (v % 8);
                    const bool vis = ((tmask >> ((key - kt) / kBlk)) & 1) && key <= p_row &&
                                     (a.window <= 0 || key > p_row - a.window);
                    S[T][v] = vis ? S[T][v] : -INFINITY;
                }
        }
        float mt_ = -INFINITY;
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int v = 0; v < 16; ++v) mt_ = fmaxf(mt_, S[T][v]);
        mt_ = fmaxf(mt_, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(xaddr, __builtin_bit_cast(int, mt_))));
        // with a positive scale, m_used + 8 stays -inf until the row's first visible
        // key, so the comparison alone starts the running maximum, and 2^(m_used -
        // m_new) is then 2^-inf = 0 (a zero scale keeps the explicit guards)
        const float m_tile = (ZS && mt_ == -INFINITY) ? -INFINITY : mt_ * sl2;
        const bool grow = ZS ? (m_tile > m_used + kRescale || (m_used == -INFINITY && m_tile != -INFINITY))
                             : m_tile > m_used + kRescale;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float m_new = grow ? m_tile : m_used;
            const float alpha = (ZS && m_used == -INFINITY) ? 0.0f : fast_exp2(m_used - m_new);
            m_used = m_new;
            msub = (m_used == -INFINITY) ? 0.0f : m_used;
            const float f = grow ? alpha : 1.0f;
            l_run *= f;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int v = 0; v < 16; ++v) o[nt][v] *= f;
        }
        compute_s(S_nxt, slot ^ 1);
        const uint16_t* vt_base = &s_vt[slot][(lane & 31) * kVtStride + 8 * (h ^ ((lane >> 4) & 1))];
        uint32_t pw[2][8];                       // P^T as fp16 pairs: [T][4u + word]
        if constexpr (!ZS) {
#pragma unroll
            for (int T = 0; T < 2; ++T)
#pragma unroll
                for (int v = 0; v < 16; v += 2)
                    pw[T][v / 2] = pack_f16x2(fast_exp2(fmaf(S[T][v], sl2, -msub)),
                                              fast_exp2(fmaf(S[T][v + 1], sl2, -msub)));
        } else {
#pragma unroll
            for (int T = 0; T < 2; ++T)
#pragma unroll
                for (int v = 0; v < 16; v += 2) {
                    const float x0 = S[T][v], x1 = S[T][v + 1];
                    const float p0 = (x0 == -INFINITY) ? 0.0f : fast_exp2(fmaf(x0, sl2, -msub));
                    const float p1 = (x1 == -INFINITY) ? 0.0f : fast_exp2(fmaf(x1, sl2, -msub));
                    pw[T][v / 2] = pack_f16x2(p0, p1);
                }
        }
        {
            const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
            float ls0 = 0.0f, ls1 = 0.0f;
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                ls0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pw[0][w]), one, ls0, false);
                ls1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pw[1][w]), one, ls1, false);
            }
            l_run += ls0 + ls1;
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int T = ks >> 1, u = ks & 1;
            u32x4_t pb;
            pb[0] = pw[T][4 * u + 0]; pb[1] = pw[T][4 * u + 1];
            pb[2] = pw[T][4 * u + 2]; pb[3] = pw[T][4 * u + 3];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int vo = 32 * nt * kVtStride + 16 * ((ks ^ nt) & 7);
                const u32x4_t vv = *reinterpret_cast<const u32x4_t*>(vt_base + vo);
                o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(vv), as_f16x8(pb), o[nt], 0, 0, 0);
            }
        }
    };

    // ---- prologue: K(0), K(1) copied, V(0) staged, S^T(0), V(1) in registers
    int mk0 = 0, mk1 = 0;                       // validity masks of tiles t and t + 1
    f32x16_t sa[2], sb[2];
    if (n_tiles > 0) {
        mk0 = tile_mask(kt_of(0));
        copy_k(0, kt_of(0));
        load_v(kt_of(0));
    }
    if (n_tiles > 1) {
        mk1 = tile_mask(kt_of(1));
        copy_k(1, kt_of(1));
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (n_tiles > 0) store_v(0, kt_of(0), mk0);
    if (n_tiles > 1) load_v(kt_of(1));
    wait_all_and_barrier();                     // K(0), K(1), V(0) in LDS
    // unconditional, so Q's first use is on every path into the loop
    compute_s(sa, 0);
    wait_all_and_barrier();                     // every wave is done reading K slot 0

    auto step = [&](f32x16_t* s_cur, f32x16_t* s_nxt, int t) {
        const int slot = t & 1;
        if (t + 1 < n_tiles) store_v(slot ^ 1, kt_of(t + 1), mk1);
        int mk2 = 0;
        if (t + 2 < n_tiles) {
            mk2 = tile_mask(kt_of(t + 2));
            copy_k(slot, kt_of(t + 2));
            load_v(kt_of(t + 2));
        }
        finish_tile(s_cur, s_nxt, slot, kt_of(t), mk0);
        wait_all_and_barrier();
        mk0 = mk1;
        mk1 = mk2;
    };
    for (int t = 0; t < n_tiles; t += 2) {
        step(sa, sb, t);
        if (t + 1 < n_tiles) step(sb, sa, t + 1);
    }

    // ---- normalise and store
    const float l_row = l_run + __shfl_xor(l_run, 32, kWave);
    if (!row_ok) return;
    const float inv = l_row > 0.0f ? 1.0f / l_row : 0.0f;
    const int64_t obase = ((int64_t)(q0 + tok) * a.num_q_heads + g * G + jh) * D;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            const int d = 32 * nt + 8 * v4 + 4 * h;
            const float r0_ = o[nt][4 * v4 + 0] * inv, r1_ = o[nt][4 * v4 + 1] * inv;
            const float r2_ = o[nt][4 * v4 + 2] * inv, r3_ = o[nt][4 * v4 + 3] * inv;
            if (a.out_bf16) {
                u32x2_t pk;
                pk[0] = pack_bf16x2(r0_, r1_);
                pk[1] = pack_bf16x2(r2_, r3_);
                *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(a.out) + obase + d) = pk;
            } else {
                f32x4_t fv = {r0_, r1_, r2_, r3_};
                *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.out) + obase + d) = fv;
            }
        }
}

}  // namespace

hipError_t launch_prefill(const PrefillLaunch& L, hipStream_t stream) {
    PrefillArgs a;
    a.q = static_cast<const uint16_t*>(L.q);
    a.out = L.out;
    a.k_pool = L.k_pool;
    a.v_pool = L.v_pool;
    a.k_scale = L.k_scale;
    a.v_scale = L.v_scale;
    a.block_tables = L.block_tables;
    a.table_offsets = L.table_offsets;
    a.seq_lens = L.seq_lens;
    a.cu_q_lens = L.cu_q_lens;
    a.num_seqs = L.num_seqs;
    a.num_q_heads = L.num_q_heads;
    a.num_kv_heads = L.num_kv_heads;
    a.group = L.num_q_heads / L.num_kv_heads;
    a.num_blocks = L.num_blocks;
    a.max_blocks = L.max_blocks_per_seq;
    constexpr int kPipeWaves = 8;
    constexpr int kPipeRows = 32 * kPipeWaves;
    const int64_t rows = (int64_t)L.max_q_len * a.group;
    a.m_tiles = (int32_t)((rows + kPipeRows - 1) / kPipeRows);
    const int64_t total = (int64_t)L.num_seqs * L.num_kv_heads * a.m_tiles;
    if (total > INT32_MAX / 2) return hipErrorInvalidValue;
    a.total = (int32_t)total;
    a.window = L.window;
    a.scale_log2 = L.softmax_scale * kLog2e;
    a.out_bf16 = L.out_bf16;
    const int64_t units = (int64_t)L.num_seqs * L.num_kv_heads;
    const int64_t grid = ((units + kXcds - 1) / kXcds) * a.m_tiles * kXcds;
    const dim3 g3((unsigned)grid), b3(64 * kPipeWaves);
    const bool zs = !(a.scale_log2 > 0.0f);
    if (L.int8) {
        if (L.head_dim == 64)
            return zs ? launch(prefill_pipe_kernel<64, kPipeWaves, true, true>, g3, b3, 0, stream, a)
                      : launch(prefill_pipe_kernel<64, kPipeWaves, false, true>, g3, b3, 0, stream, a);
        return zs ? launch(prefill_pipe_kernel<128, kPipeWaves, true, true>, g3, b3, 0, stream, a)
                  : launch(prefill_pipe_kernel<128, kPipeWaves, false, true>, g3, b3, 0, stream, a);
    }
    if (L.head_dim == 64)
        return zs ? launch(prefill_pipe_kernel<64, kPipeWaves, true, false>, g3, b3, 0, stream, a)
                  : launch(prefill_pipe_kernel<64, kPipeWaves, false, false>, g3, b3, 0, stream, a);
    // bf16, head_dim 128: the ring kernel, kRingWaves waves (32 rows each) per workgroup
    PrefillArgs r = a;
    r.m_tiles = (int32_t)((rows + 32 * kRingWaves - 1) / (32 * kRingWaves));
    const int64_t rtotal = (int64_t)L.num_seqs * L.num_kv_heads * r.m_tiles;
    if (rtotal > INT32_MAX / 2) return hipErrorInvalidValue;
    r.total = (int32_t)rtotal;
    const dim3 rg((unsigned)(((units + kXcds - 1) / kXcds) * r.m_tiles * kXcds)), rb(64 * kRingWaves);
    return zs ? launch(prefill_ring_kernel<kRingWaves, true>, rg, rb, 0, stream, r)
              : launch(prefill_ring_kernel<kRingWaves, false>, rg, rb, 0, stream, r);
}

}  // namespace pkv
