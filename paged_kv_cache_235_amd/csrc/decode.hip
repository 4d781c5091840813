// decode.hip -- paged attention for one query token per sequence.
//
// "PyTorch LLM Serving Engine", Loading and What is implemented: the query
// visits the sequence's cache blocks in table order and keeps a running
// maximum, so the softmax (an online one) never overflows.  "MicroGen", Key Features: grouped-query attention (every KV head
// serves G query heads), dynamic INT8 KV, window-length limit.
//
// Work decomposition (gfx950, wave64):
//  * A work item is (sequence, partition of the context, KV head, chunk of at
//    most 8 of its query heads).  The kernel is persistent: each workgroup
//    first turns the context lengths into a prefix of per-sequence partition
//    counts in LDS; items 0 .. grid-1 go to the workgroups in order, later ones
//    are claimed from a counter in the workspace (balanced, and the items in
//    flight stay neighbours).  No host knowledge of the lengths is needed.  A
//    batch whose every possible item has a workgroup needs no counter.  The
//    counter clears itself: every workgroup stops at its first claim past the
//    last item, so exactly `total` claims are made, and the workgroup whose
//    claim returns total - 1 (the last claim of the launch) stores 0 back.
//  * Inside an item the 4 waves take the blocks round-robin.  Each wave streams
//    its blocks' K and V tiles -- whole (block, KV head) runs, read with
//    coalesced 16-byte loads -- as one sequence K0 V0 K1 V1 ..., each tile
//    buffer reloaded as soon as its step is done, and the stream runs on
//    across items, so the memory pipe never drains.  A K step forms all the
//    query heads' dot products from the same registers (one K read serves the
//    whole group), reduces the per-lane partial sums with a transposed DPP
//    butterfly and updates an online softmax: the running maximum only moves
//    (with a rescale of what was accumulated) when a logit passes it by more
//    than 2^8, which after the first tile is rare.  The probabilities go
//    through LDS to the V step, which accumulates p * v (INT8 pools at
//    head_dim 128, and bf16 pools with more than 4 heads per item: Q.K^T and
//    P.V on the matrix cores, see the steps).  At the end of the item the 4
//    waves' (m, l, acc) are combined through LDS.
//  * Nothing in the stream waits for more than the tile it is about to use:
//    values derived from a load (scales, query sums, the work counter's claim)
//    are formed where they are used, and the ids and lengths an item needs
//    before its first load are read through the scalar cache.
//  * Keys outside the sequence, its window or a valid block are removed by
//    selection (logit -inf, V row zeroed), never by multiplying by zero, so
//    poisoned (NaN) tail slots cannot leak.
//  * With more than one partition per sequence the items write unnormalised
//    partial results (m, l, o) with device-scope stores and a second kernel
//    merges them (log-sum-exp).
#include <mutex>

#include "pkv_internal.h"
#include "pkv_device.h"

namespace pkv {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kBatchKeys = 64 * 4 * 16; // keys per batch of block ids (64 blocks per wave)
constexpr float kRescale = 8.0f;       // lazy rescale threshold (log2 units)
constexpr int kBlk = 16;               // tokens per cache block
constexpr int kMaxSeqs = 2048;         // sequences per launch (LDS prefix)
constexpr int kMaxGroup = 8;           // query heads per item
constexpr size_t kTicketBytes = 256;   // workspace head: the item counter

struct DecodeArgs {
    const void* q;
    void* out;
    float* part_ml;          // [num_seqs][max_parts][Hq][2]  running max (log2 units), sum
    float* part_o;           // [num_seqs][Hq][max_parts][D]  unnormalised outputs
    unsigned* ticket;        // item counter (zero at launch, zero again when the launch ends), or null: items by stride
    const char* k_pool;
    const char* v_pool;
    const uint16_t* k_scale;
    const uint16_t* v_scale;
    const int32_t* block_tables;
    const int32_t* table_offsets;   // per sequence: logical block of column 0 (null: all 0)
    const int32_t* context_lens;
    int32_t num_seqs, num_q_heads, num_kv_heads, group, head_chunks, num_blocks, max_blocks;
    int32_t window, part_tokens, max_parts;
    float scale_log2;        // softmax_scale * log2(e)
    int32_t q_bf16, out_bf16;
};

template <int KV> struct KvT;
template <> struct KvT<KV_F32> { static constexpr int ESZ = 4, LW = 16; };
template <> struct KvT<KV_BF16> { static constexpr int ESZ = 2, LW = 16; };
template <> struct KvT<KV_I8> { static constexpr int ESZ = 1, LW = 8; };
template <> struct KvT<KV_I8Q> { static constexpr int ESZ = 1, LW = 8; };
constexpr bool is_i8(int kv) { return kv == KV_I8 || kv == KV_I8Q; }

template <int KV, int D, int GT>
struct Cfg {
    static constexpr int ESZ = KvT<KV>::ESZ;
    static constexpr int LW = KvT<KV>::LW;       // bytes per lane per load
    static constexpr int WORDS = LW / 4;
    static constexpr int EPL = LW / ESZ;         // row elements per lane
    static constexpr int LPR = D / EPL;          // lanes sharing one row
    static constexpr int RPL = kWave / LPR;      // rows per load instruction
    static constexpr int NLOAD = kBlk / RPL;     // load instructions per tile
    static constexpr int ROW_BYTES = D * ESZ;
    static constexpr int TILE_BYTES = kBlk * ROW_BYTES;
    static constexpr int GTP = GT <= 4 ? 4 : 8;  // LDS stride of one token's logits
    static constexpr int NV = NLOAD * GT;        // partial dot products per lane per tile
    static_assert(LPR >= 1 && LPR <= kWave && NLOAD >= 1, "tile shape");
};

// Number of partitions of sequence s that contain a visible key (1 for an
// empty context: an item that writes the zero row).
__device__ __forceinline__ int seq_off(const DecodeArgs& a, int s) {
    return a.table_offsets ? max(0, a.table_offsets[s]) : 0;
}
// The same for a wave-uniform s, through the scalar cache (a vector load here
// would make the wave wait for every load it has in flight).
__device__ __forceinline__ int seq_off_uniform(const DecodeArgs& a, int s) {
    if (!a.table_offsets) return 0;
    const __attribute__((address_space(4))) int32_t* t =
        (const __attribute__((address_space(4))) int32_t*)a.table_offsets;
    return max(0, t[s]);
}
// the context length, clamped to what the table row can address
__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int L, int off) {
    const int64_t cap = ((int64_t)a.max_blocks + off) * kBlk;
    return L < 0 ? 0 : (L > cap ? (int)cap : L);
}
__device__ __forceinline__ int seq_len(const DecodeArgs& a, int s) {
    return clamp_len(a, a.context_lens[s], seq_off(a, s));
}
__device__ __forceinline__ int seq_len_uniform(const DecodeArgs& a, int s) {
    const __attribute__((address_space(4))) int32_t* t =
        (const __attribute__((address_space(4))) int32_t*)a.context_lens;
    return clamp_len(a, t[s], seq_off_uniform(a, s));
}
// First visible key: the window's start, and never before the row's first
// block (keys of released blocks do not exist for the kernels), so the keys of
// a sequence span at most max_blocks * 16 positions.
__device__ __forceinline__ int first_key(const DecodeArgs& a, int L, int off) {
    const int lo = (a.window > 0 && L > a.window) ? L - a.window : 0;
    return max(lo, off * kBlk);
}
__device__ __forceinline__ int num_parts(const DecodeArgs& a, int s) {
    const int L = seq_len(a, s);
    if (L == 0 || a.part_tokens == 0) return 1;
    const int lo = first_key(a, L, seq_off(a, s));
    if (lo >= L) return 1;                      // no key left: one item writes the zero row
    return (L - 1) / a.part_tokens - lo / a.part_tokens + 1;
}

template <int WORDS>
struct Words {
    uint32_t w[WORDS];
};

template <int WORDS>
__device__ __forceinline__ Words<WORDS> load_words(const char* p) {
    Words<WORDS> r;
    if constexpr (WORDS == 4) {
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
        r.w[0] = v[0]; r.w[1] = v[1]; r.w[2] = v[2]; r.w[3] = v[3];
    } else {
        const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
        r.w[0] = v[0]; r.w[1] = v[1];
    }
    return r;
}

// Row elements of one load as fp32 (INT8: the biased code u = q8 + 128).
template <int KV, int WORDS>
__device__ __forceinline__ void widen(const Words<WORDS>& t, float* x) {
    if constexpr (KV == KV_F32) {
#pragma unroll
        for (int i = 0; i < WORDS; ++i) x[i] = __builtin_bit_cast(float, t.w[i]);
    } else if constexpr (KV == KV_BF16) {
#pragma unroll
        for (int i = 0; i < WORDS; ++i) {
            x[2 * i] = bf16lo(t.w[i]);
            x[2 * i + 1] = bf16hi(t.w[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < WORDS; ++i) {
            const uint32_t u = t.w[i] ^ 0x80808080u;
            x[4 * i + 0] = (float)((u >> 0) & 0xffu);
            x[4 * i + 1] = (float)((u >> 8) & 0xffu);
            x[4 * i + 2] = (float)((u >> 16) & 0xffu);
            x[4 * i + 3] = (float)((u >> 24) & 0xffu);
        }
    }
}

// One (block, KV head) tile as this lane holds it: NLOAD 16- or 8-byte pieces
// (rows i * RPL + lane / LPR), plus the rows' INT8 scales.
// The scales stay binary16 until a step uses them: converted next to their
// load, they would make the wave wait there for every load issued before them.
template <int KV, int D, int GT>
struct Tile {
    Words<Cfg<KV, D, GT>::WORDS> w[Cfg<KV, D, GT>::NLOAD];
    _Float16 sc[Cfg<KV, D, GT>::NLOAD];
};

template <int KV, int D, int GT>
__device__ __forceinline__ void load_tile(Tile<KV, D, GT>& t, const char* pool, const uint16_t* scales,
                                          int64_t tile, int lane) {
    using C = Cfg<KV, D, GT>;
    const char* p = pool + tile * C::TILE_BYTES;
#pragma unroll
    for (int i = 0; i < C::NLOAD; ++i) t.w[i] = load_words<C::WORDS>(p + (i * kWave + lane) * C::LW);
    if constexpr (is_i8(KV)) {
#pragma unroll
        for (int i = 0; i < C::NLOAD; ++i)
            t.sc[i] = __builtin_bit_cast(_Float16, scales[tile * kBlk + i * C::RPL + lane / C::LPR]);
    }
}

// A K tile (bf16 or INT8, head_dim 128) laid out for Q.K^T on 4x4x4 MFMAs:
// load i holds keys 4i .. 4i+3, lane l the 8 elements of key 4i + (l & 3) at
// columns 8 (l >> 2) .. +7 (each load still reads one contiguous run of four
// rows), so the four lanes of an MFMA block hold four keys at the same
// columns; INT8: sc[0] is the scale of key l >> 2, the key whose logit the
// lane ends up with.
template <int KV, int D, int GT>
__device__ __forceinline__ void load_tile_keys_by_lane(Tile<KV, D, GT>& t, const char* pool,
                                                       const uint16_t* scales, int64_t tile, int lane) {
    using C = Cfg<KV, D, GT>;
    const char* p = pool + tile * C::TILE_BYTES + (lane & 3) * C::ROW_BYTES + (lane >> 2) * C::LW;
#pragma unroll
    for (int i = 0; i < C::NLOAD; ++i) t.w[i] = load_words<C::WORDS>(p + i * 4 * C::ROW_BYTES);
    if constexpr (is_i8(KV)) t.sc[0] = __builtin_bit_cast(_Float16, scales[tile * kBlk + (lane >> 2)]);
}

// The key whose logit lane l holds after the INT8 wide-load Q.K^T: key bits
// 0-1 are lane bits 2-3, key bit 2 is lane bit 5, key bit 3 is lane bit 4.
__device__ __forceinline__ int wide_key(int lane) {
    return ((lane >> 2) & 3) | ((lane >> 3) & 4) | ((lane >> 1) & 8);
}

// Stores of the split-K partials, which the merge kernel (possibly on another
// XCD) reads next: device-scope stores (SC1), written through to the level
// the XCDs share.  Through the cache they measured ~4% of the call slower on
// the large batch, as streaming stores ~1% (and the merge reading them 1.2 us
// slower).  `base` is the start of the run written (n bytes); offsets stay
// small, so the buffer's 32-bit range suffices.
constexpr int kCpolDeviceScope = 16;   // SC1: device scope
__device__ __forceinline__ void store_partial4(float* base, int n, int byte_off, f32x4_t v) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, n, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, byte_off, 0, kCpolDeviceScope);
}
__device__ __forceinline__ void store_partial1(float* base, int n, int byte_off, float v) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, n, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, byte_off, 0, kCpolDeviceScope);
}

// An INT8 K tile (head_dim 128) for Q.K^T on 4x4x4 MFMAs with 16-byte loads:
// load i holds keys 8i .. 8i+7 (one contiguous 1 KiB run), lane l the 16 codes
// of key 8i + 4 (l >> 5) + (l & 3) at columns 16 ((l >> 2) & 7) .. +15, in
// w[2i] (columns +0..7) and w[2i+1] (+8..15); so the four lanes of an MFMA
// block hold four keys at the same columns.  sc[0] is the scale of key
// wide_key(l), the key whose logit the lane ends up with.  Rows reached by
// lanes in four different 128-byte rows per quad cost less at 16 bytes per
// lane than at 8.
template <int KV, int D, int GT>
__device__ __forceinline__ void load_tile_keys_wide(Tile<KV, D, GT>& t, const char* pool,
                                                    const uint16_t* scales, int64_t tile, int lane) {
    using C = Cfg<KV, D, GT>;
    static_assert(KV == KV_I8Q && D == 128 && C::NLOAD == 4 && C::WORDS == 2, "INT8 rows of 128 codes");
    const char* p = pool + tile * C::TILE_BYTES + (4 * (lane >> 5) + (lane & 3)) * C::ROW_BYTES +
                    16 * ((lane >> 2) & 7);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + i * 8 * C::ROW_BYTES));
        t.w[2 * i].w[0] = v[0];
        t.w[2 * i].w[1] = v[1];
        t.w[2 * i + 1].w[0] = v[2];
        t.w[2 * i + 1].w[1] = v[3];
    }
    t.sc[0] = __builtin_bit_cast(_Float16, scales[tile * kBlk + wide_key(lane)]);
}

// Exchange with lane ^ MASK exactly (every lane bit kept but MASK).
template <int MASK>
__device__ __forceinline__ float xchg_exact(float x) {
    if constexpr (MASK == 8) return dpp_mov<kDppRowRor8>(x);       // (i + 8) mod 16 == i ^ 8
    else return __shfl_xor(x, MASK, kWave);
}

// One step of a transposed butterfly across lane bit 16 or 32 in one
// instruction: lo holds quantities the lanes without the bit keep, hi those the
// lanes with it keep.  v_permlane16_swap exchanges the odd 16-lane rows of its
// first operand with the even rows of its second (v_permlane32_swap: the upper
// half of the first with the lower half of the second), after which lo + hi is
// the kept quantity plus the partner lane's copy of it, in every lane.  (Inline
// asm: the compiler's builtin for these swaps returns the first register twice.)
template <int BIT>
__device__ __forceinline__ float swap_add(float lo, float hi) {
    static_assert(BIT == 16 || BIT == 32, "lane bit of a permlane swap");
    if constexpr (BIT == 16)
        asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
    else
        asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
    return lo + hi;
}

// Transposed butterfly over lane bits BIT, BIT/2, .., 4 (the 16 groups of 4
// lanes): v[0..N) are this lane's partial sums of N quantities; afterwards v[0]
// holds the full sum of quantity lane >> 2 (N = 16).
template <int N, int BIT>
__device__ __forceinline__ void tbfly_blocks(float* v, int lane) {
    if constexpr (BIT >= 16) {
        constexpr int H = N / 2;
#pragma unroll
        for (int k = 0; k < H; ++k) v[k] = swap_add<BIT>(v[k], v[H + k]);
        tbfly_blocks<H, BIT / 2>(v, lane);
    } else if constexpr (BIT >= 4) {
        constexpr int H = N / 2;
        const bool up = (lane & BIT) != 0;
#pragma unroll
        for (int k = 0; k < H; ++k) {
            const float keep = up ? v[H + k] : v[k];
            const float send = up ? v[k] : v[H + k];
            v[k] = keep + xchg_exact<BIT>(send);
        }
        tbfly_blocks<H, BIT / 2>(v, lane);
    }
}

// Values per lane left by tbfly<N, BIT>, and the lane bits across which the
// lanes hold copies of the same quantity (the steps that had one value left).
constexpr int tb_count(int n, int bit) { return bit == 0 ? n : (n >= 2 ? tb_count((n + 1) / 2, bit / 2) : 1); }
constexpr int tb_dup(int n, int bit) {
    return bit == 0 ? 0 : (n >= 2 ? tb_dup((n + 1) / 2, bit / 2) : (bit | tb_dup(1, bit / 2)));
}

// DIRECT: a single-pass call (no partitions) with no window and no table
// offsets; the host launches this variant only then.
template <int KV, int D, int GT, bool DIRECT>
__global__ __launch_bounds__(kThreads) void decode_partition_kernel(DecodeArgs a) {
    using C = Cfg<KV, D, GT>;
    constexpr int NT = tb_count(C::NV, C::LPR / 2);   // logits per lane after the butterfly
    constexpr int DUP = tb_dup(C::NV, C::LPR / 2);
    __shared__ int s_prefix[kMaxSeqs + 1];
    __shared__ int s_len[kMaxSeqs];              // visible context length of each sequence
    // per-wave probabilities of the tile in hand: [key][GTP]
    __shared__ __attribute__((aligned(16))) float s_p[kWaves][kBlk * C::GTP];
    // per-wave partial outputs and (m, l) of an item, double-buffered by item parity
    __shared__ __attribute__((aligned(16))) float s_comb[2][kWaves][GT * D];
    __shared__ float s_ml[2][kWaves][2][C::GTP];
    __shared__ int s_next[2];                    // next items, by item parity
    static_assert(kThreads <= 2 * kWaves * GT * D, "prefix scan scratch");

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    // wave-uniform in a scalar register, so per-wave loop bounds are scalar branches
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int B = a.num_seqs;

    // Single-pass calls with no window and no table offsets (DIRECT): every
    // sequence is one item per (KV head, head chunk) and its keys start at 0, so
    // an item's sequence and first table columns are known from its index
    // alone -- no prefix, and the context length and the table ids are read at
    // the same time instead of one after the other.
    constexpr bool direct = DIRECT;

    // ---- prefix of partition counts (each thread owns up to 8 consecutive sequences)
    if constexpr (!direct) {
        const int per = (B + kThreads - 1) / kThreads;
        int cnt[8];
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int s = tid * per + i;
            // partitions before the last one (the last ones are items of their own
            // at the end of the order)
            cnt[i] = (i < per && s < B) ? num_parts(a, s) - 1 : 0;
            sum += cnt[i];
        }
        // inclusive prefix of the per-thread sums: inside each wave by shuffles,
        // then the waves' totals through LDS (one barrier)
        int incl = sum;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int up = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += up;
        }
        int* wtot = reinterpret_cast<int*>(&s_comb[0][0][0]);
        if (lane == kWave - 1) wtot[wave] = incl;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kWaves; ++w) incl += w < wave ? wtot[w] : 0;
        int run = incl - sum;        // exclusive prefix
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int s = tid * per + i;
            if (i < per && s < B) {
                s_prefix[s] = run;
                s_len[s] = seq_len(a, s);
            }
            run += cnt[i];
        }
        if (tid == kThreads - 1) s_prefix[B] = incl;
        __syncthreads();
    }

    const int HC = a.num_kv_heads * a.head_chunks;
    // Items in claim order: first every partition but each sequence's last
    // (s_prefix counts them), then the last partition of every sequence, one
    // per sequence -- usually the short ones, so the launch ends on short items
    // (a last-claimed full partition leaves its workgroup's neighbours idle for
    // up to an item's time).
    const int nfull = direct ? 0 : s_prefix[B];
    const int total = direct ? B * HC : (nfull + B) * HC;
    const int row_lane = lane / C::LPR;          // row of this lane inside each load
    const int col = (lane % C::LPR) * C::EPL;    // first column of this lane

    // work item -> (sequence, partition, KV head, query-head chunk) and its key range
    struct Item {
        int s, nparts, k, kr, t0, t1, g, h0, nh, off;   // kr: k - the first partition with keys
    };
    auto item_info = [&](int item) {
        Item I;
        const int gp = item / HC;
        const int hc = item - gp * HC;
        I.g = hc / a.head_chunks;
        const int hchunk = hc - I.g * a.head_chunks;
        // LDS values are the same in every lane: keep them in scalar registers
        auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
        int ps, L;
        if constexpr (direct) {
            // one item per (sequence, KV head, head chunk), keys from 0 to L
            I.s = gp;
            L = seq_len_uniform(a, I.s);
            I.nparts = 1;
            I.k = I.kr = 0;
            I.off = 0;
            I.t0 = 0;
            I.t1 = L;
            I.h0 = I.g * a.group + hchunk * GT;
            I.nh = min(GT, a.group - hchunk * GT);
            return I;
        } else {
            if (gp < nfull) {
                int lo_s = 0, hi_s = B - 1;             // largest s with s_prefix[s] <= gp
                while (lo_s < hi_s) {
                    const int mid = (lo_s + hi_s + 1) >> 1;
                    if (uni(s_prefix[mid]) <= gp) lo_s = mid; else hi_s = mid - 1;
                }
                I.s = lo_s;
                ps = uni(s_prefix[I.s]);
            } else {
                // the last partition of sequence gp - nfull: as if its index
                // were counted after the sequence's others
                I.s = gp - nfull;
                ps = gp - (uni(s_prefix[I.s + 1]) - uni(s_prefix[I.s]));   // kr = the count before it
            }
            I.nparts = uni(s_prefix[I.s + 1]) - uni(s_prefix[I.s]) + 1;
            L = uni(s_len[I.s]);
        }
        const int off = seq_off_uniform(a, I.s);
        const int lo = min(first_key(a, L, off), L);
        const int P = a.part_tokens;
        I.k = (P > 0 ? lo / P : 0) + (gp - ps);
        I.kr = gp - ps;
        I.off = off;
        I.t0 = P > 0 ? max(lo, I.k * P) : lo;
        I.t1 = P > 0 ? min(L, (I.k + 1) * P) : L;
        I.h0 = I.g * a.group + hchunk * GT;         // first query head of the item
        I.nh = min(GT, a.group - hchunk * GT);
        return I;
    };

    // query fragment: this lane's columns of each head
    uint32_t qw[GT][C::WORDS];      // bf16 pairs (bf16 pools)
    uint32_t qb[GT][C::EPL / 2];    // bf16 pairs (INT8 pools with a bf16 query)
    // keys-by-lane Q.K^T: head 4 nq + (lane & 3) at columns 8 (lane >> 2) .. +7
    // (two MFMA B operands), and -128 x that head's query sum (the codes' bias)
    constexpr bool MKQ = (KV == KV_I8Q || (KV == KV_BF16 && GT > 4)) && D == 128;
    constexpr int NHQQ = (GT + 3) / 4;
    // INT8 pools with a bf16 query, head_dim 128: K tiles come with 16-byte
    // loads (load_tile_keys_wide), and the query fragment is head 4 nq +
    // (lane & 3) at columns 16 ((lane >> 2) & 7) .. +15 (four B operands)
    constexpr bool KW = KV == KV_I8Q && D == 128;
    uint32_t qk[MKQ ? NHQQ : 1][KW ? 8 : 4];
    float qkb[MKQ ? NHQQ : 1];
    float qf[GT][C::EPL];           // fp32 (fp32 pools, INT8 pools with an fp32 query)
    float qsum[GT];
    // The query's loads are issued during the previous item's last batch; what
    // is derived from them (the sums that remove the INT8 codes' bias) waits
    // for finish_q at the top of the item, where the loads of the item's first
    // tiles, issued after the query's, may still be in flight.
    auto load_q = [&](const Item& I) {
        if constexpr (KW) {
#pragma unroll
            for (int nq = 0; nq < NHQQ; ++nq) {
                const int j = 4 * nq + (lane & 3);
                u32x4_t v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
                if (j < I.nh) {
                    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(
                        static_cast<const uint16_t*>(a.q) + ((int64_t)I.s * a.num_q_heads + I.h0 + j) * D +
                        16 * ((lane >> 2) & 7));
                    v0 = qp[0];
                    v1 = qp[1];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    qk[nq][i] = v0[i];
                    qk[nq][4 + i] = v1[i];
                }
            }
            return;
        } else if constexpr (MKQ) {
#pragma unroll
            for (int nq = 0; nq < NHQQ; ++nq) {
                const int j = 4 * nq + (lane & 3);
                u32x4_t v = {0u, 0u, 0u, 0u};
                if (j < I.nh)
                    v = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.q) +
                                                          ((int64_t)I.s * a.num_q_heads + I.h0 + j) * D +
                                                          8 * (lane >> 2));
#pragma unroll
                for (int i = 0; i < 4; ++i) qk[nq][i] = v[i];
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < GT; ++j) {
            const int64_t qoff = ((int64_t)I.s * a.num_q_heads + I.h0 + j) * D + col;
            if constexpr (KV == KV_BF16) {
                Words<4> t{};
                if (j < I.nh) {
                    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.q) + qoff);
                    t.w[0] = v[0]; t.w[1] = v[1]; t.w[2] = v[2]; t.w[3] = v[3];
                }
#pragma unroll
                for (int i = 0; i < C::WORDS; ++i) qw[j][i] = t.w[i];
            } else if constexpr (KV == KV_I8Q) {
                u32x4_t v = {0u, 0u, 0u, 0u};
                if (j < I.nh) v = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.q) + qoff);
#pragma unroll
                for (int i = 0; i < 4; ++i) qb[j][i] = v[i];
            } else {
#pragma unroll
                for (int e = 0; e < C::EPL; ++e) {
                    float x = 0.0f;
                    if (j < I.nh)
                        x = a.q_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(a.q)[qoff + e])
                                     : static_cast<const float*>(a.q)[qoff + e];
                    qf[j][e] = x;
                }
            }
        }
    };
    auto finish_q = [&]() {
        if constexpr (KW) {
#pragma unroll
            for (int nq = 0; nq < NHQQ; ++nq) {
                float t = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) t += bf16lo(qk[nq][i]) + bf16hi(qk[nq][i]);
                // sum over the 8 column chunks (lane bits 2-4; bit 5 holds copies)
                t += __shfl_xor(t, 4, kWave);
                t += xchg_exact<8>(t);
                t += __shfl_xor(t, 16, kWave);
                qkb[nq] = -128.0f * t;
            }
        } else if constexpr (MKQ) {
#pragma unroll
            for (int nq = 0; nq < NHQQ; ++nq) {
                if constexpr (KV == KV_I8Q) {
                    float t = 0.0f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) t += bf16lo(qk[nq][i]) + bf16hi(qk[nq][i]);
                    // sum over the 16 column blocks (lanes of the same head)
                    t += __shfl_xor(t, 4, kWave);
                    t += xchg_exact<8>(t);
                    t += __shfl_xor(t, 16, kWave);
                    t += __shfl_xor(t, 32, kWave);
                    qkb[nq] = -128.0f * t;
                } else {
                    qkb[nq] = 0.0f;
                }
            }
        } else if constexpr (is_i8(KV)) {
#pragma unroll
            for (int j = 0; j < GT; ++j) {
                float t = 0.0f;
                if constexpr (KV == KV_I8Q) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) t += bf16lo(qb[j][i]) + bf16hi(qb[j][i]);
                } else {
#pragma unroll
                    for (int e = 0; e < C::EPL; ++e) t += qf[j][e];
                }
                qsum[j] = t;
            }
        }
    };

    // Block ids of a batch of up to 64 blocks per wave: this wave takes blocks
    // wave, wave + 4, ...; lane j holds the id of its j-th one.  ids_of issues
    // the load (the id, or -1 for lanes past the wave's blocks); install makes
    // them current, invalid ids reading block 0 under a cleared mask bit.
    int lid = 0;
    uint64_t okmask = 0;
    auto ids_of = [&](const Item& I, int c0, int nbw) {
        int id = -1;
        // column of the lane's block in the sequence's row (blocks before the row's
        // offset have been released: no id)
        const int col = c0 / kBlk + wave + kWaves * lane - I.off;
        if constexpr (direct) {
            // read before the wave's block count is known (it needs the context
            // length); entries past the sequence are never used
            if (col < a.max_blocks) id = a.block_tables[(int64_t)I.s * a.max_blocks + col];
        } else if (lane < nbw && col >= 0 && col < a.max_blocks) {
            id = a.block_tables[(int64_t)I.s * a.max_blocks + col];
        }
        return id;
    };
    auto valid_id = [&](int id) { return id >= 0 && id < a.num_blocks; };
    // the block tables through the constant address space: wave-uniform reads
    // become scalar loads
    const __attribute__((address_space(4))) int32_t* s_table =
        (const __attribute__((address_space(4))) int32_t*)a.block_tables;
    auto install = [&](int id) {
        const bool ok = valid_id(id);
        lid = ok ? id : 0;
        okmask = __builtin_amdgcn_ballot_w64(ok);
    };
    auto tile_of = [&](int i, int g) {
        return (int64_t)__builtin_amdgcn_readlane(lid, i) * a.num_kv_heads + g;
    };
    auto batch_end = [](int c0, int t1) { return min(t1, (c0 / kBatchKeys + 1) * kBatchKeys); };
    auto blocks_of_wave = [&](int c0, int c1) {
        if (c1 <= c0) return 0;
        const int nblk = (c1 - 1) / kBlk - c0 / kBlk + 1;
        return wave < nblk ? (nblk - 1 - wave) / kWaves + 1 : 0;
    };

    // Items 0 .. grid-1 go to the workgroups in order; after that each workgroup
    // takes the next unclaimed item from the counter, so the work stays balanced
    // and the items in flight at any time are neighbours (adjacent KV heads of
    // the same blocks).  The item after the current one is known an item ahead
    // (s_next), so its loads can start before the current item is combined.
    const bool dyn = a.ticket != nullptr;
    // one claim on the counter.  The claim that returns total - 1 is the last
    // one of the launch (each workgroup claims until it passes the last item, so
    // claims 0 .. total - 1 are made), and whoever holds it stores 0 back
    // (settle) for the next launch that uses this workspace.  Inside the item
    // loop the claim's value is first looked at when the item ends: a look at
    // once would make the wave wait for every load it has in flight.
    auto claim = [&]() { return (int)atomicAdd(a.ticket, 1u); };
    auto settle = [&](int c) {
        if ((unsigned)c == (unsigned)total - 1u) atomicExch(a.ticket, 0u);
    };
    if (dyn) {
        if (tid == 0 && (int)blockIdx.x < total) {
            const int c = claim();
            settle(c);
            s_next[1] = (int)gridDim.x + c;
        } else if (tid == 0) {
            s_next[1] = total;
        }
        __syncthreads();
    }

    // The wave's tiles form one stream K0 V0 K1 V1 ... across blocks, batches
    // and items.  tk holds K tiles and tv V tiles; each is reloaded with the
    // next tile of its kind as soon as its step is done (sched_barrier keeps the
    // compiler from sinking the load), so one to two tiles are always in flight
    // and there is no softmax phase to stall the stream: the softmax is online.
    Tile<KV, D, GT> tk, tv;
    auto load_k = [&](Tile<KV, D, GT>& t, int64_t tile) {
        if constexpr (KW)
            load_tile_keys_wide<KV, D, GT>(t, a.k_pool, a.k_scale, tile, lane);
        else if constexpr (MKQ)
            load_tile_keys_by_lane<KV, D, GT>(t, a.k_pool, a.k_scale, tile, lane);
        else load_tile<KV, D, GT>(t, a.k_pool, a.k_scale, tile, lane);
    };
    float* lp = s_p[wave];
    int parity = 0;              // combine buffer of the current item
    Item I = item_info(blockIdx.x < total ? blockIdx.x : 0);
    if ((int)blockIdx.x < total) {
        load_q(I);
        const int nbw0 = blocks_of_wave(I.t0, batch_end(I.t0, I.t1));
        install(ids_of(I, I.t0, nbw0));
        if (nbw0 > 0) {
            load_k(tk, tile_of(0, I.g));
            load_tile<KV, D, GT>(tv, a.v_pool, a.v_scale, tile_of(0, I.g), lane);
        }
    }
    // this lane's logits after the butterfly: quantity base + kk is head
    // (base + kk) % GT of key row ((base + kk) / GT) * RPL + row_lane
    int tb_base = 0, tb_valid = C::NV;
    {
        float dummy[C::NV];
#pragma unroll
        for (int v = 0; v < C::NV; ++v) dummy[v] = 0.0f;
        tbfly<C::NV, C::LPR / 2>(dummy, lane, tb_base, tb_valid);
    }
    const bool owner = (lane & DUP) == 0;        // one lane per distinct quantity

    // INT8 pools, head_dim 128: P.V on the matrix cores.  A lane's four loads of a
    // tile hold keys 4t + q (t = 0..3, q = lane / 16) at its 8 columns, which is
    // the B operand of v_mfma_f32_4x4x4bf16_1k (16 blocks of 4 lanes; lane 4b + r
    // supplies row r of A and column r of B over k = t, and receives column r of
    // D, rows t): B = the biased codes of one of the lane's columns (exact in
    // bf16), A = the weights p * v_scale of head 4 nq + (lane & 3) at the same 4
    // keys, as a bf16 value plus its bf16 remainder (two MFMAs, 16 bits of the
    // weight), D = that column's partial output for 4 heads.  The keys of the
    // other row groups are added in the combine, as for the FMA form.
    // bf16 pools take the MFMA forms only with more than 4 heads per item: at 4
    // (the HBM-bound large batches) the MFMA-and-butterfly chain measured ~0.5%
    // slower than the FMA form, at 6 (latency-bound small batches) 3-5% faster
    constexpr bool MV = (is_i8(KV) || (KV == KV_BF16 && GT > 4)) && D == 128;
    constexpr int NHQ = (GT + 3) / 4;            // groups of 4 heads
    const int hr = lane & 3;                     // this lane's head within a group
    // INT8 pools with a bf16 query and bf16 pools with more than 4 heads per
    // item, head_dim 128: Q.K^T on the matrix cores too.  The K tile comes
    // keys-by-lane, so that in an MFMA block A = K (row r: one of four keys
    // over 4 columns), B = Q^T (column r: head 4 nq + r at the same columns),
    // D = the 4 x 4 partial logits over the block's columns; a transposed
    // butterfly across the blocks that hold the same keys then leaves each lane
    // one logit per head group, of head 4 nq + hr.  bf16
    // (load_tile_keys_by_lane): 4 loads of keys 4i .. 4i+3, 8 columns per
    // lane, butterfly over 16 blocks, key lane >> 2.  INT8
    // (load_tile_keys_wide): 2 loads of keys 8i .. 8i+7, 16 columns per lane,
    // butterfly over 8 column chunks, key wide_key(lane).
    constexpr bool MK = (KV == KV_I8Q || (KV == KV_BF16 && GT > 4)) && D == 128;
    constexpr int NS = MK ? NHQ : NT;            // logit slots per lane

    for (int item = blockIdx.x, following; item < total; item = following) {
        following = dyn ? __builtin_amdgcn_readfirstlane(s_next[parity ^ 1]) : item + (int)gridDim.x;
        int claimed = 0;
        if (dyn && wave == 0 && lane == 0 && following < total) claimed = claim();
        const bool have_next = following < total;
        const Item NI = item_info(have_next ? following : item);
        const int s = I.s, g = I.g, h0 = I.h0, nh = I.nh, k = I.kr, nparts = I.nparts;
        finish_q();

        // running softmax state of this wave's keys: m per head (uniform), the
        // same m per logit slot of this lane, l per logit slot, acc per column
        float m_run[GT], m_lane[NS], l_lane[NS], acc[GT][C::EPL], psum[GT];
        f32x4_t accv[MV ? NHQ : 1][MV ? C::EPL : 1];  // MV: [head group][column] -> 4 heads
        float psl[MV ? NHQ : 1];                     // MV: weight sum of head 4 nq + hr, this lane's keys
#pragma unroll
        for (int j = 0; j < GT; ++j) {
            m_run[j] = -INFINITY;
            psum[j] = 0.0f;
#pragma unroll
            for (int e = 0; e < C::EPL; ++e) acc[j][e] = 0.0f;
        }
        if constexpr (MV) {
#pragma unroll
            for (int nq = 0; nq < NHQ; ++nq) {
                psl[nq] = 0.0f;
#pragma unroll
                for (int e = 0; e < C::EPL; ++e) accv[nq][e] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
#pragma unroll
        for (int kk = 0; kk < NS; ++kk) {
            m_lane[kk] = -INFINITY;
            l_lane[kk] = 0.0f;
        }

        // one pass per batch of block ids; an empty item still makes one pass,
        // which hands the stream over to the next item
        int c0 = I.t0;
        do {
            const int c1 = batch_end(c0, I.t1);
            const int tbase = (c0 / kBlk) * kBlk;   // first token of the batch's first block
            const int nbw = blocks_of_wave(c0, c1);
            // the batch after this one: the next of this item, else the first of the next item
            const bool more = c1 < I.t1;
            const bool any_next = more || have_next;
            const Item& J = more ? I : NI;
            const int jc0 = more ? c1 : NI.t0;
            const int nbw_n = any_next ? blocks_of_wave(jc0, batch_end(jc0, J.t1)) : 0;
            const int id_n = ids_of(J, jc0, nbw_n);
            const int g_n = J.g;

            // MFMA Q.K^T: this lane's logits x[nq] (key r, head 4 nq + hr) into
            // the online softmax (rescale only when one passes the running
            // maximum by more than 2^kRescale), probabilities to LDS
            auto softmax_update = [&](const float* x, bool over, int r) {
                if constexpr (MK) {
                    if (__builtin_amdgcn_ballot_w64(over) != 0) {
#pragma unroll
                        for (int j = 0; j < GT; ++j) {
                            float v = -INFINITY;
#pragma unroll
                            for (int nq = 0; nq < NHQ; ++nq)
                                if (4 * nq + hr == j) v = fmaxf(v, x[nq]);
                            const float m_new = fmaxf(m_run[j], group_max<kWave>(v));
                            const float alpha = (m_run[j] == -INFINITY) ? 0.0f : fast_exp2(m_run[j] - m_new);
                            m_run[j] = m_new;
#pragma unroll
                            for (int e = 0; e < C::EPL; ++e) accv[j >> 2][e][j & 3] *= alpha;
                            if constexpr (is_i8(KV)) psl[j >> 2] *= hr == (j & 3) ? alpha : 1.0f;
#pragma unroll
                            for (int nq = 0; nq < NHQ; ++nq)
                                if (4 * nq + hr == j) {
                                    l_lane[nq] *= alpha;
                                    m_lane[nq] = m_new;
                                }
                        }
                    }
#pragma unroll
                    for (int nq = 0; nq < NHQ; ++nq) {
                        const float p = (x[nq] == -INFINITY) ? 0.0f : fast_exp2(x[nq] - m_lane[nq]);
                        l_lane[nq] += p;
                        lp[r * C::GTP + 4 * nq + hr] = p;
                    }
                }
            };

            // ---- K tile -> logits of its 16 keys for every head, online softmax
            // update (rescale only when a logit passes the running maximum by
            // more than 2^kRescale), probabilities to LDS
            auto k_step = [&](const Tile<KV, D, GT>& t, int it) {
                const int b = wave + kWaves * it;
                const bool blk_ok = (okmask >> it) & 1;
                if constexpr (KW) {
                    // INT8, 16-byte K loads: per load i, four MFMAs (one per 4
                    // columns of the lane's 16) give keys 8i + 4 (lane >> 5) + r'
                    // x heads 4 nq + r over the lane's column chunk
                    f32x4_t dk[NHQ][2];
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
#pragma unroll
                        for (int nq = 0; nq < NHQ; ++nq) dk[nq][i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            // four biased codes u = q8 + 128 as bf16 (exact)
                            const uint32_t u = t.w[2 * i + (m >> 1)].w[m & 1] ^ 0x80808080u;
                            const float f0 = (float)(u & 0xffu), f1 = (float)((u >> 8) & 0xffu);
                            const float f2 = (float)((u >> 16) & 0xffu), f3 = (float)(u >> 24);
                            const uint32_t c01 = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f1),
                                                                       __builtin_bit_cast(uint32_t, f0), 0x07060302u);
                            const uint32_t c23 = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f3),
                                                                       __builtin_bit_cast(uint32_t, f2), 0x07060302u);
                            const bf16x4_t am = __builtin_bit_cast(bf16x4_t, u32x2_t{c01, c23});
#pragma unroll
                            for (int nq = 0; nq < NHQ; ++nq) {
                                const bf16x4_t bm =
                                    __builtin_bit_cast(bf16x4_t, u32x2_t{qk[nq][2 * m], qk[nq][2 * m + 1]});
                                dk[nq][i] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(am, bm, dk[nq][i], 0, 0, 0);
                            }
                        }
                    }
                    const int r = wide_key(lane);
                    const int tok = tbase + b * kBlk + r;
                    const bool key_ok = blk_ok && tok >= c0 && tok < c1;
                    float x[NHQ];
                    bool over = false;
#pragma unroll
                    for (int nq = 0; nq < NHQ; ++nq) {
                        float v[8];
#pragma unroll
                        for (int i = 0; i < 2; ++i)
#pragma unroll
                            for (int k2 = 0; k2 < 4; ++k2) v[4 * i + k2] = dk[nq][i][k2];
                        tbfly_blocks<8, 16>(v, lane);
                        const bool ok = key_ok && 4 * nq + hr < GT;
                        x[nq] = ok ? (v[0] + qkb[nq]) * (float)t.sc[0] * a.scale_log2 : -INFINITY;
                        over |= x[nq] > m_lane[nq] + kRescale;
                    }
                    softmax_update(x, over, r);
                    return;
                }
                if constexpr (MK) {
                    f32x4_t dk[NHQ][4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        // bf16 pools: the row's 8 elements as they are; INT8: the
                        // 8 biased codes u = q8 + 128 as bf16 (exact)
                        uint32_t cw[4];
                        if constexpr (KV == KV_BF16) {
#pragma unroll
                            for (int w = 0; w < 4; ++w) cw[w] = t.w[i].w[w];
                        } else
#pragma unroll
                        for (int w = 0; w < 2; ++w) {
                            const uint32_t u = t.w[i].w[w] ^ 0x80808080u;
                            const float f0 = (float)(u & 0xffu), f1 = (float)((u >> 8) & 0xffu);
                            const float f2 = (float)((u >> 16) & 0xffu), f3 = (float)(u >> 24);
                            cw[2 * w] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f1),
                                                              __builtin_bit_cast(uint32_t, f0), 0x07060302u);
                            cw[2 * w + 1] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f3),
                                                                  __builtin_bit_cast(uint32_t, f2), 0x07060302u);
                        }
                        const bf16x4_t a0 = __builtin_bit_cast(bf16x4_t, u32x2_t{cw[0], cw[1]});
                        const bf16x4_t a1 = __builtin_bit_cast(bf16x4_t, u32x2_t{cw[2], cw[3]});
#pragma unroll
                        for (int nq = 0; nq < NHQ; ++nq) {
                            const bf16x4_t b0 = __builtin_bit_cast(bf16x4_t, u32x2_t{qk[nq][0], qk[nq][1]});
                            const bf16x4_t b1 = __builtin_bit_cast(bf16x4_t, u32x2_t{qk[nq][2], qk[nq][3]});
                            dk[nq][i] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a0, b0, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f},
                                                                               0, 0, 0);
                            dk[nq][i] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a1, b1, dk[nq][i], 0, 0, 0);
                        }
                    }
                    // the lane's key and its visibility
                    const int r = lane >> 2;
                    const int tok = tbase + b * kBlk + r;
                    const bool key_ok = blk_ok && tok >= c0 && tok < c1;
                    float x[NHQ];
                    bool over = false;
#pragma unroll
                    for (int nq = 0; nq < NHQ; ++nq) {
                        float v[16];
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int k2 = 0; k2 < 4; ++k2) v[4 * i + k2] = dk[nq][i][k2];
                        tbfly_blocks<16, 32>(v, lane);
                        const bool ok = key_ok && 4 * nq + hr < GT;
                        const float sc = is_i8(KV) ? (float)t.sc[0] : 1.0f;
                        x[nq] = ok ? (v[0] + qkb[nq]) * sc * a.scale_log2 : -INFINITY;
                        over |= x[nq] > m_lane[nq] + kRescale;
                    }
                    softmax_update(x, over, r);
                    return;
                }
                float part[C::NV];
#pragma unroll
                for (int i = 0; i < C::NLOAD; ++i) {
                    if constexpr (KV == KV_BF16) {
#pragma unroll
                        for (int j = 0; j < GT; ++j) {
                            float d = 0.0f;
#pragma unroll
                            for (int w = 0; w < C::WORDS; ++w)
                                d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, t.w[i].w[w]),
                                                                    __builtin_bit_cast(bf16x2_t, qw[j][w]), d, false);
                            part[i * GT + j] = d;
                        }
                    } else if constexpr (KV == KV_I8Q) {
                        // the 8 biased codes u = q8 + 128 as 4 bf16 pairs (small
                        // integers: exact), then the bf16 path's dot2 products
                        uint32_t cw[4];
#pragma unroll
                        for (int w = 0; w < 2; ++w) {
                            const uint32_t u = t.w[i].w[w] ^ 0x80808080u;
                            const float f0 = (float)(u & 0xffu), f1 = (float)((u >> 8) & 0xffu);
                            const float f2 = (float)((u >> 16) & 0xffu), f3 = (float)(u >> 24);
                            cw[2 * w] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f1),
                                                              __builtin_bit_cast(uint32_t, f0), 0x07060302u);
                            cw[2 * w + 1] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f3),
                                                                  __builtin_bit_cast(uint32_t, f2), 0x07060302u);
                        }
#pragma unroll
                        for (int j = 0; j < GT; ++j) {
                            float d = 0.0f;
#pragma unroll
                            for (int w = 0; w < 4; ++w)
                                d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, cw[w]),
                                                                    __builtin_bit_cast(bf16x2_t, qb[j][w]), d, false);
                            part[i * GT + j] = (d - 128.0f * qsum[j]) * (float)t.sc[i];
                        }
                    } else {
                        float x[C::EPL];
                        widen<KV, C::WORDS>(t.w[i], x);
#pragma unroll
                        for (int j = 0; j < GT; ++j) {
                            float d = 0.0f;
#pragma unroll
                            for (int e = 0; e < C::EPL; ++e) d = fmaf(qf[j][e], x[e], d);
                            if constexpr (KV == KV_I8) d = (d - 128.0f * qsum[j]) * (float)t.sc[i];
                            part[i * GT + j] = d;
                        }
                    }
                }
                int base = 0, valid = C::NV;
                tbfly<C::NV, C::LPR / 2>(part, lane, base, valid);
                float x[NT];
                bool over = false;
#pragma unroll
                for (int kk = 0; kk < NT; ++kk) {
                    const int idx = base + kk;
                    const int r = (idx / GT) * C::RPL + row_lane;
                    const int tok = tbase + b * kBlk + r;
                    const bool ok = kk < valid && blk_ok && tok >= c0 && tok < c1;
                    x[kk] = ok ? part[kk] * a.scale_log2 : -INFINITY;
                    over |= x[kk] > m_lane[kk] + kRescale;
                }
                if (__builtin_amdgcn_ballot_w64(over) != 0) {
                    // new maxima: the tile's maximum per head, then rescale what
                    // has been accumulated with the old ones
#pragma unroll
                    for (int j = 0; j < GT; ++j) {
                        float v = -INFINITY;
#pragma unroll
                        for (int kk = 0; kk < NT; ++kk)
                            if ((base + kk) % GT == j) v = fmaxf(v, x[kk]);
                        const float m_new = fmaxf(m_run[j], group_max<kWave>(v));
                        const float alpha = (m_run[j] == -INFINITY) ? 0.0f : fast_exp2(m_run[j] - m_new);
                        m_run[j] = m_new;
                        if constexpr (MV) {
#pragma unroll
                            for (int e = 0; e < C::EPL; ++e) accv[j >> 2][e][j & 3] *= alpha;
                            if constexpr (is_i8(KV)) psl[j >> 2] *= hr == (j & 3) ? alpha : 1.0f;
                        } else {
                            psum[j] *= alpha;
#pragma unroll
                            for (int e = 0; e < C::EPL; ++e) acc[j][e] *= alpha;
                        }
#pragma unroll
                        for (int kk = 0; kk < NT; ++kk)
                            if ((base + kk) % GT == j) {
                                l_lane[kk] *= alpha;
                                m_lane[kk] = m_new;
                            }
                    }
                }
#pragma unroll
                for (int kk = 0; kk < NT; ++kk) {
                    if (kk < valid) {
                        const int idx = base + kk;
                        const int j = idx % GT;
                        const int r = (idx / GT) * C::RPL + row_lane;
                        const float p = (x[kk] == -INFINITY) ? 0.0f : fast_exp2(x[kk] - m_lane[kk]);
                        if (owner) l_lane[kk] += p;
                        lp[r * C::GTP + j] = p;
                    }
                }
            };

            // ---- V tile: acc += p * v over its 16 keys
            auto v_step = [&](const Tile<KV, D, GT>& t, int it) {
                const int b = wave + kWaves * it;
                const bool blk_ok = (okmask >> it) & 1;
                const bool full = blk_ok && tbase + b * kBlk >= c0 && tbase + (b + 1) * kBlk <= c1;
                if constexpr (MV) {
                    // A: weights of head 4 nq + hr at keys 4t + q, hi and remainder
                    bf16x4_t a_hi[NHQ], a_lo[NHQ];
#pragma unroll
                    for (int nq = 0; nq < NHQ; ++nq) {
                        const int j = 4 * nq + hr;
                        float w[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int r = i * C::RPL + row_lane;
                            const int tok = tbase + b * kBlk + r;
                            const bool row_ok = full || (blk_ok && tok >= c0 && tok < c1);
                            const float pj = lp[r * C::GTP + (j < GT ? j : 0)];
                            if constexpr (is_i8(KV)) {
                                w[i] = (row_ok && j < GT) ? pj * (float)t.sc[i] : 0.0f;
                                psl[nq] += w[i];
                            } else {
                                w[i] = (row_ok && j < GT) ? pj : 0.0f;
                            }
                        }
                        const uint32_t h01 = pack_bf16x2(w[0], w[1]), h23 = pack_bf16x2(w[2], w[3]);
                        const uint32_t l01 = pack_bf16x2(w[0] - bf16lo(h01), w[1] - bf16hi(h01));
                        const uint32_t l23 = pack_bf16x2(w[2] - bf16lo(h23), w[3] - bf16hi(h23));
                        a_hi[nq] = __builtin_bit_cast(bf16x4_t, u32x2_t{h01, h23});
                        a_lo[nq] = __builtin_bit_cast(bf16x4_t, u32x2_t{l01, l23});
                    }
                    if constexpr (KV == KV_BF16) {
                        // B: column e of keys 4t + q; rows past the keys zeroed on an
                        // edge tile (they may hold NaN, and 0 x NaN is NaN)
                        uint32_t vw[4][4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int r = i * C::RPL + row_lane;
                            const int tok = tbase + b * kBlk + r;
                            const bool row_ok = full || (blk_ok && tok >= c0 && tok < c1);
#pragma unroll
                            for (int wd = 0; wd < 4; ++wd) vw[i][wd] = (full || row_ok) ? t.w[i].w[wd] : 0u;
                        }
#pragma unroll
                        for (int e = 0; e < C::EPL; ++e) {
                            const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                            const uint32_t b01 = __builtin_amdgcn_perm(vw[1][e >> 1], vw[0][e >> 1], sel);
                            const uint32_t b23 = __builtin_amdgcn_perm(vw[3][e >> 1], vw[2][e >> 1], sel);
                            const bf16x4_t bv = __builtin_bit_cast(bf16x4_t, u32x2_t{b01, b23});
#pragma unroll
                            for (int nq = 0; nq < NHQ; ++nq)
                                accv[nq][e] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a_hi[nq], bv, accv[nq][e], 0, 0, 0);
#pragma unroll
                            for (int nq = 0; nq < NHQ; ++nq)
                                accv[nq][e] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a_lo[nq], bv, accv[nq][e], 0, 0, 0);
                        }
                        return;
                    }
                    // B: column e's biased codes u = q8 + 128 at keys 4t + q, as bf16
                    uint32_t u[4][2];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int wd = 0; wd < 2; ++wd) u[i][wd] = t.w[i].w[wd] ^ 0x80808080u;
#pragma unroll
                    for (int e = 0; e < C::EPL; ++e) {
                        float f[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) f[i] = (float)((u[i][e >> 2] >> (8 * (e & 3))) & 0xffu);
                        const uint32_t b01 = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f[1]),
                                                                   __builtin_bit_cast(uint32_t, f[0]), 0x07060302u);
                        const uint32_t b23 = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f[3]),
                                                                   __builtin_bit_cast(uint32_t, f[2]), 0x07060302u);
                        const bf16x4_t bv = __builtin_bit_cast(bf16x4_t, u32x2_t{b01, b23});
#pragma unroll
                        for (int nq = 0; nq < NHQ; ++nq)
                            accv[nq][e] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a_hi[nq], bv, accv[nq][e], 0, 0, 0);
#pragma unroll
                        for (int nq = 0; nq < NHQ; ++nq)
                            accv[nq][e] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a_lo[nq], bv, accv[nq][e], 0, 0, 0);
                    }
                    return;
                }
#pragma unroll
                for (int i = 0; i < C::NLOAD; ++i) {
                    Words<C::WORDS> wv = t.w[i];
                    const int r = i * C::RPL + row_lane;
                    const int tok = tbase + b * kBlk + r;
                    const bool row_ok = full || (blk_ok && tok >= c0 && tok < c1);
                    if (!full) {
#pragma unroll
                        for (int w = 0; w < C::WORDS; ++w) wv.w[w] = row_ok ? wv.w[w] : 0u;
                    }
                    const float* pp = &lp[r * C::GTP];
                    float p[C::GTP];
                    const f32x4_t p0 = *reinterpret_cast<const f32x4_t*>(pp);
                    p[0] = p0[0]; p[1] = p0[1]; p[2] = p0[2]; p[3] = p0[3];
                    if constexpr (C::GTP == 8) {
                        const f32x4_t p1 = *reinterpret_cast<const f32x4_t*>(pp + 4);
                        p[4] = p1[0]; p[5] = p1[1]; p[6] = p1[2]; p[7] = p1[3];
                    }
                    if constexpr (is_i8(KV)) {
#pragma unroll
                        for (int j = 0; j < GT; ++j) {
                            p[j] = row_ok ? p[j] * (float)t.sc[i] : 0.0f;
                            psum[j] += p[j];
                        }
                    }
                    float x[C::EPL];
                    widen<KV, C::WORDS>(wv, x);
#pragma unroll
                    for (int j = 0; j < GT; ++j)
#pragma unroll
                        for (int e = 0; e < C::EPL; ++e) acc[j][e] = fmaf(p[j], x[e], acc[j][e]);
                }
            };

            int it = 0;
            for (; it + 1 < nbw; ++it) {
                k_step(tk, it);
                load_k(tk, tile_of(it + 1, g));
                __builtin_amdgcn_sched_barrier(0);
                v_step(tv, it);
                load_tile<KV, D, GT>(tv, a.v_pool, a.v_scale, tile_of(it + 1, g), lane);
                __builtin_amdgcn_sched_barrier(0);
            }
            // the last block of the batch: the stream continues with the first
            // block of the next batch or item (and that item's Q, which this
            // item no longer needs once its last K step is done).  Both loads
            // are unconditional (block 0 when there is no next block): with a
            // condition on each, the compiler would allow for a K load not
            // followed by a V load and wait for every load at the next K step.
            if (nbw > 0) k_step(tk, it);
            if (!more && have_next) load_q(NI);
            // the wave's first block of that batch, read again through the scalar
            // cache: a use of id_n here would wait for every load in flight (the
            // loads of this batch may number zero, so the compiler cannot count
            // them), the V tile of this step included
            int id0 = -1;
            {
                const int col0 = jc0 / kBlk + wave - J.off;
                if (nbw_n > 0 && col0 >= 0 && col0 < a.max_blocks) id0 = s_table[(int64_t)J.s * a.max_blocks + col0];
            }
            const int64_t t_n = (int64_t)(valid_id(id0) ? id0 : 0) * a.num_kv_heads + g_n;
            load_k(tk, t_n);
            __builtin_amdgcn_sched_barrier(0);
            if (nbw > 0) v_step(tv, it);
            load_tile<KV, D, GT>(tv, a.v_pool, a.v_scale, t_n, lane);
            __builtin_amdgcn_sched_barrier(0);
            if (any_next) install(id_n);
            c0 = c1;
        } while (c0 < I.t1);

        // ---- combine: the lanes of each column, then the waves, each wave's
        // state rescaled to the common maximum
        float l_run[GT];
#pragma unroll
        for (int j = 0; j < GT; ++j) {
            float v = 0.0f;
            if constexpr (MK) {
#pragma unroll
                for (int nq = 0; nq < NHQ; ++nq)
                    if (4 * nq + hr == j) v += l_lane[nq];
            } else {
#pragma unroll
                for (int kk = 0; kk < NT; ++kk)
                    if (kk < tb_valid && (tb_base + kk) % GT == j) v += l_lane[kk];
            }
            l_run[j] = group_sum<kWave>(v);
        }
        if constexpr (MV) {
            // INT8: heads' weight sums for this lane's keys: lane (lane & ~3) +
            // (j & 3) holds head j's
            if constexpr (is_i8(KV)) {
#pragma unroll
                for (int j = 0; j < GT; ++j) psum[j] = __shfl(psl[j >> 2], (lane & ~3) | (j & 3), kWave);
            }
#pragma unroll
            for (int j = 0; j < GT; ++j)
#pragma unroll
                for (int e = 0; e < C::EPL; ++e) acc[j][e] = accv[j >> 2][e][j & 3];
        }
        if constexpr (is_i8(KV)) {
#pragma unroll
            for (int j = 0; j < GT; ++j)
#pragma unroll
                for (int e = 0; e < C::EPL; ++e) acc[j][e] -= 128.0f * psum[j];
        }
        float* cb = s_comb[parity][wave];
        if constexpr (C::LPR == 16 && (GT * C::EPL) % 4 == 0) {
            // the lanes of a column are lane bits 4 and 5 apart: a transposed
            // reduction over those bits by lane swaps leaves each lane a quarter
            // of the GT x EPL sums, the ones of rows base .. base + N/4 - 1
            constexpr int N = GT * C::EPL, H = N / 2, Q = N / 4;
            float v[N];
#pragma unroll
            for (int j = 0; j < GT; ++j)
#pragma unroll
                for (int e = 0; e < C::EPL; ++e) v[j * C::EPL + e] = acc[j][e];
#pragma unroll
            for (int q = 0; q < H; ++q) v[q] = swap_add<32>(v[q], v[H + q]);
#pragma unroll
            for (int q = 0; q < Q; ++q) v[q] = swap_add<16>(v[q], v[Q + q]);
            const int base = ((lane >> 5) & 1) * H + ((lane >> 4) & 1) * Q;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int idx = base + q;
                cb[(idx / C::EPL) * D + col + idx % C::EPL] = v[q];
            }
        } else {
#pragma unroll
            for (int j = 0; j < GT; ++j)
#pragma unroll
                for (int e = 0; e < C::EPL; ++e) {
                    float v = acc[j][e];
#pragma unroll
                    for (int off = C::LPR; off < kWave; off <<= 1) v += __shfl_xor(v, off, kWave);
                    acc[j][e] = v;
                }
            if (lane < C::LPR) {
#pragma unroll
                for (int j = 0; j < GT; ++j)
#pragma unroll
                    for (int e = 0; e < C::EPL; ++e) cb[j * D + col + e] = acc[j][e];
            }
        }
        if (lane == 0) {
#pragma unroll
            for (int j = 0; j < GT; ++j) {
                s_ml[parity][wave][0][j] = m_run[j];
                s_ml[parity][wave][1][j] = l_run[j];
            }
            // the item after the following one; every wave read this slot
            // before the previous item's barrier
            if (dyn && wave == 0) {
                if (following < total) settle(claimed);
                s_next[parity] = following < total ? (int)gridDim.x + claimed : total;
            }
        }
        // One barrier per item: the buffers alternate, so a wave that runs ahead
        // writes the other buffer, and it can only come back to this one after
        // every wave has passed the next item's barrier, i.e. finished reading.
        // The barrier waits for LDS only; the next item's loads stay in flight.
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        // The waves' partial rows, rescaled to the common maximum and summed,
        // four adjacent columns per thread (one 16-byte LDS read per wave and
        // one 16-byte store): every round's reads and arithmetic first (chunks
        // past GT rows read row GT - 1, in bounds, and are not stored), so the
        // rounds overlap, then the stores.
        constexpr int NCH = GT * D / 4;
        constexpr int R = (NCH + kThreads - 1) / kThreads;
        f32x4_t ov[R];
        float lv[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int c = tid + r * kThreads;
            const int j = min(c / (D / 4), GT - 1), d0 = (c % (D / 4)) * 4;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_ml[parity][w][0][j]);
            f32x4_t o = {0.0f, 0.0f, 0.0f, 0.0f};
            float l = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float mw = s_ml[parity][w][0][j];
                const float f = (mw == -INFINITY) ? 0.0f : fast_exp2(mw - M);
                const f32x4_t x = *reinterpret_cast<const f32x4_t*>(&s_comb[parity][w][j * D + d0]);
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = fmaf(f, x[e], o[e]);
                l = fmaf(f, s_ml[parity][w][1][j], l);
            }
            ov[r] = o;
            lv[r] = l;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int c = tid + r * kThreads;
            const int j = c / (D / 4), d0 = (c % (D / 4)) * 4;
            if (c >= NCH || j >= nh) continue;
            const int h = h0 + j;
            if (nparts == 1) {
                const int64_t oi = ((int64_t)s * a.num_q_heads + h) * D + d0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float q = lv[r] > 0.0f ? ov[r][e] / lv[r] : 0.0f;
                    if (a.out_bf16) static_cast<uint16_t*>(a.out)[oi + e] = f32_to_bf16(q);
                    else static_cast<float*>(a.out)[oi + e] = q;
                }
            } else {
                // rows of the item's heads are max_parts * D floats apart; the
                // base (the first head's row) is the same for the whole wave
                const int64_t p0 = ((int64_t)s * a.num_q_heads + h0) * a.max_parts + k;
                const int hstride = a.max_parts * D;
                store_partial4(&a.part_o[p0 * D], ((nh - 1) * hstride + D) * 4, (j * hstride + d0) * 4, ov[r]);
            }
        }
        // the item's (m, l) pairs: adjacent lanes of wave 0 write the run of
        // 2 nh floats in one store (written one pair per head, 4-byte stores to
        // scattered addresses measured ~2.5% of the call)
        if (nparts > 1 && wave == 0 && lane < 2 * nh) {
            const int j = lane >> 1;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_ml[parity][w][0][j]);
            float l = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float mw = s_ml[parity][w][0][j];
                l = fmaf((mw == -INFINITY) ? 0.0f : fast_exp2(mw - M), s_ml[parity][w][1][j], l);
            }
            const int64_t mi = (((int64_t)s * a.max_parts + k) * a.num_q_heads + h0) * 2;
            store_partial1(&a.part_ml[mi], 2 * nh * 4, lane * 4, (lane & 1) ? l : M);
        }
        parity ^= 1;
        I = NI;
    }
}

// Merge the partitions of every (sequence, head) with more than one:
// out = sum_k 2^(m_k - M) o_k / sum_k 2^(m_k - M) l_k, M = max_k m_k; a
// partition without keys (m_k = -inf) has weight 0, and a row with no key in
// any partition is zero.  One wave per (sequence, head): lane k owns partition
// k's weight (64 at a time), broadcast with readlane; the D-wide partial rows
// are read kMergeBatch partitions at a time.  The first batch's loads do not
// depend on the weights, so they are issued together with the loads of the
// maxima: a row of up to kMergeBatch partitions (most rows) waits for memory
// once.
constexpr int kMergeBatch = 16;

template <int D>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(DecodeArgs a) {
    constexpr int E = D / kWave;                 // output elements per lane
    const int lane = threadIdx.x & (kWave - 1);
    const int pair = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (pair >= a.num_seqs * a.num_q_heads) return;
    const int s = pair / a.num_q_heads;
    const int n = num_parts(a, s);
    if (n <= 1) return;
    // partials are stored from the sequence's first partition with visible keys
    const int h = pair - s * a.num_q_heads;
    // (m, l) of partition k: ml[k * mstride], ml[k * mstride + 1]
    const float* ml = a.part_ml + ((int64_t)s * a.max_parts * a.num_q_heads + h) * 2;
    const int64_t mstride = (int64_t)a.num_q_heads * 2;
    const float* po = a.part_o + (int64_t)pair * a.max_parts * D + lane * E;

    float v[kMergeBatch][E];
    auto load_batch = [&](int k0) {
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e) v[u][e] = (k0 + u < n) ? po[(int64_t)(k0 + u) * D + e] : 0.0f;
    };
    load_batch(0);
    float mk0 = -INFINITY, lk0 = 0.0f;           // this lane's partition of the first 64
    if (lane < n) {
        mk0 = ml[lane * mstride];
        lk0 = ml[lane * mstride + 1];
    }
    float M = mk0;
    for (int k = lane + kWave; k < n; k += kWave) M = fmaxf(M, ml[k * mstride]);
    M = group_max<kWave>(M);
    float den = 0.0f;
    float o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = 0.0f;
    for (int kb = 0; kb < n; kb += kWave) {
        const int k = kb + lane;
        float w = 0.0f;
        if (k < n) {
            const float mk = kb == 0 ? mk0 : ml[k * mstride];
            const float lk = kb == 0 ? lk0 : ml[k * mstride + 1];
            w = (mk == -INFINITY) ? 0.0f : fast_exp2(mk - M);
            den += w * lk;
        }
        const int cnt = min(kWave, n - kb);
        for (int j = 0; j < cnt; j += kMergeBatch) {
            if (kb + j > 0) load_batch(kb + j);
#pragma unroll
            for (int u = 0; u < kMergeBatch; ++u) {
                const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w),
                                                                                      (j + u) & (kWave - 1)));
#pragma unroll
                for (int e = 0; e < E; ++e) o[e] = fmaf(wu, v[u][e], o[e]);
            }
        }
    }
    den = group_sum<kWave>(den);
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int64_t oi = (int64_t)pair * D + lane * E + e;
        const float r = o[e] * inv;
        if (a.out_bf16) static_cast<uint16_t*>(a.out)[oi] = f32_to_bf16(r);
        else static_cast<float*>(a.out)[oi] = r;
    }
}

// ------------------------------------------------- fixed scratch (no allocation)
// Scratch of paged_attention_decode_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: kernels get the address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device at the first call there.  Its first 256 bytes are the work counter,
// which every call leaves at zero.
constexpr size_t kFixedScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kFixedScratchBytes];

__global__ void decode_clear_counter_kernel(unsigned* counter) {
    if (threadIdx.x == 0) *counter = 0u;
}

size_t decode_fixed_scratch_bytes() { return kFixedScratchBytes; }

hipError_t decode_fixed_scratch(void** ptr, hipStream_t stream) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        // set-up on this device: the counter starts at zero (a kernel, so a
        // first call made under graph capture records no memset)
        e = launch(decode_clear_counter_kernel, dim3(1), dim3(kWave), 0, stream, static_cast<unsigned*>(p));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

// ---------------------------------------------------------------- host side
using PartKernel = void (*)(DecodeArgs);

template <int KV, int D, bool DIRECT>
static PartKernel pick_gt(int gt) {
    switch (gt) {
    case 1: return decode_partition_kernel<KV, D, 1, DIRECT>;
    case 2: return decode_partition_kernel<KV, D, 2, DIRECT>;
    case 3: return decode_partition_kernel<KV, D, 3, DIRECT>;
    case 4: return decode_partition_kernel<KV, D, 4, DIRECT>;
    case 5: return decode_partition_kernel<KV, D, 5, DIRECT>;
    case 6: return decode_partition_kernel<KV, D, 6, DIRECT>;
    case 7: return decode_partition_kernel<KV, D, 7, DIRECT>;
    default: return decode_partition_kernel<KV, D, 8, DIRECT>;
    }
}

template <bool DIRECT>
static PartKernel pick_kv(KvKind kv, int D, int gt) {
    if (kv == KV_F32) return D == 64 ? pick_gt<KV_F32, 64, DIRECT>(gt) : pick_gt<KV_F32, 128, DIRECT>(gt);
    if (kv == KV_BF16) return D == 64 ? pick_gt<KV_BF16, 64, DIRECT>(gt) : pick_gt<KV_BF16, 128, DIRECT>(gt);
    if (kv == KV_I8Q) return D == 64 ? pick_gt<KV_I8Q, 64, DIRECT>(gt) : pick_gt<KV_I8Q, 128, DIRECT>(gt);
    return D == 64 ? pick_gt<KV_I8, 64, DIRECT>(gt) : pick_gt<KV_I8, 128, DIRECT>(gt);
}

static PartKernel pick(KvKind kv, int D, int gt, bool direct) {
    return direct ? pick_kv<true>(kv, D, gt) : pick_kv<false>(kv, D, gt);
}

int32_t decode_max_partitions(int32_t max_blocks_per_seq, int32_t block_size, int32_t partition_size,
                              bool with_table_offsets) {
    if (partition_size <= 0) return 0;
    const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
    // with offset rows the keys a row addresses need not start on a partition
    // boundary, so they can straddle one more partition
    const int64_t n = (cap + partition_size - 1) / partition_size + (with_table_offsets ? 1 : 0);
    return n <= 1 ? 0 : (int32_t)n;
}

size_t decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                              int32_t max_partitions) {
    if (max_partitions <= 0) return 0;
    const size_t slots = (size_t)num_seqs * num_q_heads * max_partitions;
    const size_t ml = (slots * 2 * sizeof(float) + 255) & ~(size_t)255;
    return kTicketBytes + ml + slots * head_dim * sizeof(float);
}

hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream) {
    const int G = L.num_q_heads / L.num_kv_heads;
    const int chunks = (G + kMaxGroup - 1) / kMaxGroup;
    const int gt = (G + chunks - 1) / chunks;
    const int max_parts = decode_max_partitions(L.max_blocks_per_seq, L.block_size, L.partition_size,
                                                L.table_offsets != nullptr);
    const bool merge = max_parts > 1;

    DecodeArgs a;
    a.q = L.q;
    a.out = L.out;
    a.k_pool = static_cast<const char*>(L.k_pool);
    a.v_pool = static_cast<const char*>(L.v_pool);
    a.k_scale = L.k_scale;
    a.v_scale = L.v_scale;
    a.num_q_heads = L.num_q_heads;
    a.num_kv_heads = L.num_kv_heads;
    a.group = G;
    a.head_chunks = chunks;
    a.num_blocks = L.num_blocks;
    a.max_blocks = L.max_blocks_per_seq;
    a.table_offsets = nullptr;          // set per launch below
    a.window = L.window;
    a.part_tokens = merge ? L.partition_size : 0;
    a.max_parts = merge ? max_parts : 1;
    a.scale_log2 = L.softmax_scale * kLog2e;
    a.q_bf16 = L.q_bf16;
    a.out_bf16 = L.out_bf16;

    // single pass, no window, no table offsets: the variant that maps items to
    // sequences directly
    const bool direct = !merge && L.window <= 0 && L.table_offsets == nullptr;
    PartKernel kern = pick(L.kv, L.head_dim, gt, direct);
    static thread_local PartKernel occ_kern = nullptr;
    static thread_local int occ = 0;
    if (occ_kern != kern) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(kern), kThreads, 0) != hipSuccess || n < 1) n = 1;
        occ = n;
        occ_kern = kern;
    }
    const int64_t resident = (int64_t)device_cu_count() * occ;
    const int64_t per_seq_items = (int64_t)(merge ? max_parts : 1) * L.num_kv_heads * chunks;

    const size_t slots_total = (size_t)L.num_seqs * L.num_q_heads * (merge ? max_parts : 0);
    unsigned* ticket = merge ? static_cast<unsigned*>(L.workspace) : nullptr;
    char* ws = merge ? static_cast<char*>(L.workspace) + kTicketBytes : nullptr;
    float* ml_base = reinterpret_cast<float*>(ws);
    float* o_base = merge ? reinterpret_cast<float*>(ws + ((slots_total * 2 * sizeof(float) + 255) & ~(size_t)255))
                          : nullptr;

    for (int32_t s0 = 0; s0 < L.num_seqs; s0 += kMaxSeqs) {
        const int32_t n = std::min<int32_t>(kMaxSeqs, L.num_seqs - s0);
        DecodeArgs b = a;
        b.num_seqs = n;
        const int64_t qoff = (int64_t)s0 * L.num_q_heads * L.head_dim;
        b.q = static_cast<const char*>(L.q) + qoff * (L.q_bf16 ? 2 : 4);
        b.out = static_cast<char*>(L.out) + qoff * (L.out_bf16 ? 2 : 4);
        b.block_tables = L.block_tables + (int64_t)s0 * L.max_blocks_per_seq;
        b.table_offsets = L.table_offsets ? L.table_offsets + s0 : nullptr;
        b.context_lens = L.context_lens + s0;
        b.part_ml = merge ? ml_base + (int64_t)s0 * L.num_q_heads * max_parts * 2 : nullptr;
        b.part_o = merge ? o_base + (int64_t)s0 * L.num_q_heads * max_parts * L.head_dim : nullptr;
        // when every possible item has a workgroup of its own (a small batch), items
        // go by stride and the counter -- and the launch that clears it -- is not needed
        const bool claim = ticket && (int64_t)n * per_seq_items > resident;
        b.ticket = claim ? ticket : nullptr;
        const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(resident, (int64_t)n * per_seq_items));
        hipError_t e = hipSuccess;
        if (L.start_event) {
            e = hipEventRecord(L.start_event, stream);
            if (e != hipSuccess) return e;
        }
        e = launch(kern, dim3((unsigned)grid), dim3(kThreads), 0, stream, b);
        if (e != hipSuccess) return e;
        if (merge) {
            if (L.split_event) {
                e = hipEventRecord(L.split_event, stream);
                if (e != hipSuccess) return e;
            }
            const int64_t pairs = (int64_t)n * L.num_q_heads;
            const unsigned mg = (unsigned)((pairs + kWaves - 1) / kWaves);
            e = L.head_dim == 64 ? launch(decode_merge_kernel<64>, dim3(mg), dim3(kThreads), 0, stream, b)
                                 : launch(decode_merge_kernel<128>, dim3(mg), dim3(kThreads), 0, stream, b);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace pkv
