// Paged decode attention: one query token per sequence against its whole cached context.
//
// Operation ("Nano-vLLM Field Guide", Step 10.3, decode with flash_attn_with_kvcache; Step
// 07.6 for context_lens): out[b, h] = softmax(scale * q[b, h] . K_b^T) V_b over the
// context_lens[b] keys of sequence b, read through its block table. Query head h reads kv head
// h / G (G = num_heads / num_kv_heads). A row with no keys (a padding row) outputs zeros.
//
// gfx950 design. Decode reads every K/V byte of the context once and does ~1 FMA per byte: it
// is bound by HBM bandwidth, so the kernel is built around keeping enough bytes in flight and
// spending few instructions per byte.
//  - Work item = (sequence b, kv head g, split s of the key range). The G query heads of the
//    group share every K/V load. The split's slice of the block table is staged in LDS once,
//    so no K/V address waits on a table load.
//  - Each of the 4 waves of a workgroup walks its own chunks of 16 keys (chunks w, w+4, ...)
//    with an online softmax. K and V of the next chunk are loaded while the current one is
//    processed (two register buffers), 16 KiB per wave in flight.
//  - Lane layout: 16 lanes x 16 B cover one 256-byte key (or value) row of the kv head, a wave
//    covers 4 rows per load instruction. K . q is v_dot2_f32_bf16 (bf16 pairs, fp32 sum)
//    followed by a DPP sum over the 16 lanes of the row; P.V takes two keys at a time as
//    v_dot2_f32_bf16 of (p_i, p_i+1) with (v_i, v_i+1), 8 output dims per lane, and the row
//    sum adds the same bf16 probabilities. When a chunk lies inside one block, one table
//    lookup gives a scalar base and each lane adds a fixed offset. The 8B shape (G = 4) was
//    instruction-bound before these cuts (now about 360 VALU instructions per 16-key chunk,
//    the VALU busy half the time); they pay as long as the kernel keeps 3 waves per SIMD.
//    (Scores by a 16x16x32 bf16 MFMA with the query heads as columns were measured slower:
//    the extra registers halve the waves per SIMD.)
//  - The running max may lag by a bounded slack, so the output rescale is rare.
//  - With G <= 4 the 16 lanes of a key row would all compute the same 4 G probabilities;
//    instead each lane computes one, pairs it with the next row's (DPP rotate), and the bf16
//    pairs are broadcast back to the row (DPP row_newbcast): one exp per lane and chunk.
//  - At the end the 4 waves' (max, sum, output) are merged through LDS. A split's result is
//    final when it is the sequence's only split; otherwise it goes to the workspace and a
//    second kernel merges the splits with the log-sum-exp rule:
//    out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, M = max_s m_s.
//    When no row can have a second split the merge kernel is not launched; rows without keys
//    get their zeros from the split kernel.
//  - Splits are as long as possible (up to 8192 keys) while the launch keeps >= 4096 work
//    items, e.g. the Qwen3-8B step (512 sequences x 8 kv heads, contexts <= 4096) runs
//    unsplit and the Qwen3-0.6B decode of 256 sequences in two 2048-key splits.
//  - Scores are kept in log2 units (scale * log2(e) folded in; exp2 is the hardware exp).
//  - Grid order (XCD-aware): the hardware deals consecutive workgroup ids round-robin to the
//    8 XCDs. A unit of gcd(Hkv, G) consecutive kv heads of one (sequence, split) runs as
//    consecutive workgroups on one XCD, and consecutive units go to different XCDs, so each
//    XCD reads contiguous 256*G-byte stretches of the same pool rows at the same time.
//    Measured +2% (Qwen3-0.6B, 256 sequences) and +4% (Qwen3-8B step) over the kv-head-
//    fastest 3D grid, which gave each XCD one head's 256-byte slice of every row; that order
//    was itself +9% on the 8B decode over split-major order. (Sequence, split) pairs are
//    numbered sequence fastest when the grid is larger than the chip holds at once (every
//    first split is dispatched before any second one, and each split index spreads over all
//    XCDs: numbered split fastest, the first splits sat on a fixed half of the XCDs), and
//    split fastest when it runs in one go (a sequence's splits start together, which the
//    in-kernel merge of small steps prefers). Larger grids also take the sequences longest
//    first, from a counting sort of the context lengths written just before the launch: the
//    long rows start in the first wave of workgroups instead of leaving a tail (+3.5-6% on
//    the 8B, 0.6B and tensor-parallel share decodes).
//  - One-launch store + decode (nv_paged_attn_decode_store, a decode step's two calls): the
//    workgroup holding a row's new token loads that key's row from the step's new K/V rows and
//    writes it to the pools; with arrival counters the last workgroup of a split row to finish
//    merges the partials itself (coherent relaxed-atomic partials, no cache-wide fence), so
//    neither a store kernel nor a merge kernel runs.
// The split size depends only on host-known launch parameters: no device round trip.
#include <atomic>
#include <mutex>
#include <numeric>

#include "nv_common.h"

// Build-time knobs (defaults are the measured best on MI355X).
#ifndef NV_DECODE_NT
#define NV_DECODE_NT 1          // non-temporal K/V loads
#endif
#ifndef NV_DECODE_CHUNK
#define NV_DECODE_CHUNK 16      // keys per wave iteration (16 or 32)
#endif
#ifndef NV_DECODE_MAX_SPLIT
#define NV_DECODE_MAX_SPLIT 8192     // longest split (keys)
#endif
#ifndef NV_DECODE_TARGET_ITEMS
#define NV_DECODE_TARGET_ITEMS 4096  // work items the split size aims for
#endif
#ifndef NV_DECODE_PV_DOT2
#define NV_DECODE_PV_DOT2 1     // P.V as bf16-pair dot products over two keys at a time
#endif
#ifndef NV_DECODE_EXPDEDUP
#define NV_DECODE_EXPDEDUP 1    // G <= 4: one exp per lane, bf16 pairs broadcast back to the row
#endif
#ifndef NV_DECODE_SLACK
#define NV_DECODE_SLACK 8.0f    // rescale only when a running max grows by more (log2 units)
#endif
#ifndef NV_DECODE_HEAD_MAJOR
// Grid order: 0 split index fastest, 1 kv head fastest (3D grid), 2 XCD-grouped (1D grid).
#define NV_DECODE_HEAD_MAJOR 2
#endif
#ifndef NV_DECODE_XCD_HEADS
#define NV_DECODE_XCD_HEADS 0   // order 2: kv heads kept together per XCD (0: the group size G)
#endif
#ifndef NV_DECODE_ONE_GO_GROUPS
#define NV_DECODE_ONE_GO_GROUPS 768  // grids up to this many workgroups keep splits together
#endif
#ifndef NV_DECODE_MIN_WAVES
#define NV_DECODE_MIN_WAVES 1   // occupancy hint: waves per SIMD the register budget must allow
#endif

namespace nvp {
namespace {

static_assert(NV_DECODE_CHUNK == 16 || NV_DECODE_CHUNK == 32, "chunk of 16 or 32 keys");
static_assert(NV_DECODE_CHUNK % 8 == 0, "P.V pairs rows of a chunk");
constexpr int kChunk = NV_DECODE_CHUNK;  // keys per wave iteration
constexpr int kRowLoads = kChunk / 4;    // 16-byte loads per lane per chunk, per tensor
constexpr int kMaxSplitKeys = NV_DECODE_MAX_SPLIT;
#ifndef NV_DECODE_MIN_SPLIT
#define NV_DECODE_MIN_SPLIT 128
#endif
constexpr int kMinSplitKeys = NV_DECODE_MIN_SPLIT;
constexpr int kTableSlots = 264;    // block ids of one split staged in LDS

struct DecodeArgs {
    const uint16_t *q;
    const uint16_t *k_cache;
    const uint16_t *v_cache;
    const int32_t *context_lens;
    const int32_t *block_tables;
    float *ws_ml;  // [B, Hq, max_splits, 2]  (max, sum) in log2 units
    float *ws_o;   // [B, Hq, max_splits, 128] unnormalised partial outputs
    uint16_t *out;
    int32_t bt_width;
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t block_size;
    int32_t bs_shift;  // log2(block_size) if a power of two, else -1
    int32_t split_keys;
    int32_t max_splits;
    int32_t n_pairs;  // batch * max_splits
    int32_t batch;
    int32_t splits_together;  // 1: a sequence's splits are consecutive pairs (small grids)
    const int32_t *perm;      // large grids: sequences longest first (decode_order_kernel)
    int32_t xcd_heads;  // kv heads of one pair kept together on one XCD (divides num_kv_heads)
    float scale_log2;  // softmax_scale * log2(e)
    float rescale_slack;  // raw-score growth of a running max tolerated without a rescale
    // Fused store (decode rows' new K/V): row b's key and value rows, its slot, and the pools
    // to write; unused by the plain decode.
    const uint16_t *new_k;
    const uint16_t *new_v;
    int64_t new_k_stride;
    int64_t new_v_stride;
    const int32_t *slot_mapping;
    uint16_t *k_pool;
    uint16_t *v_pool;
    // Arrival counters of the in-kernel merge, [B * Hkv] (null: the merge kernel runs). Zero
    // before the launch; the workgroup that merges a row returns its counter to zero.
    uint32_t *counters;
};

struct Chunk {
    u32x4 k[kRowLoads];
    u32x4 v[kRowLoads];
};

// Streaming 16-byte load of K/V (non-temporal by default: each byte is read once).
#if NV_DECODE_NT
#define NV_LOAD_STREAM(ptr) __builtin_nontemporal_load(ptr)
#else
#define NV_LOAD_STREAM(ptr) (*(ptr))
#endif

// DPP within each 16-lane row: the value of lane kSrc in every lane (row_newbcast), and the
// value of lane l - kBy (mod 16) in lane l (row_ror: a rotation towards higher lanes).
template <int kSrc>
__device__ __forceinline__ uint32_t row_bcast(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x150 + kSrc, 0xf, 0xf, false);
}
template <int kBy>
__device__ __forceinline__ float row_ror(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + kBy, 0xf,
                                                      0xf, false));
}
template <int G, int J, int H>
__device__ __forceinline__ void bcast_pairs(uint32_t pk, uint32_t (&pp)[2][G]) {
    if constexpr (J < 2) {
        if constexpr (H < G) {
            pp[J][H] = row_bcast<2 * J * G + H>(pk);
            bcast_pairs<G, J, H + 1>(pk, pp);
        } else {
            bcast_pairs<G, J + 1, 0>(pk, pp);
        }
    }
}

template <int G>
struct DecodeSmem {
    int32_t table[kTableSlots];
    float o[4][G][kHeadDim];
    float ml[4][G][2];
    int32_t merges;  // in-kernel merge: this workgroup arrived last for its row
};

// Partials of the in-kernel merge are written and read as relaxed agent-scope atomics: on
// gfx950 those bypass the caches that are not coherent across XCDs (sc1), so they need no
// cache-wide write-back or invalidate, which a device-scope fence would do in every workgroup.
template <bool kCoherent>
__device__ __forceinline__ float ld_part(const float *p) {
    if constexpr (kCoherent) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else return *p;
}
template <bool kCoherent>
__device__ __forceinline__ void st_part(float *p, float v) {
    if constexpr (kCoherent) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
}

// Log-sum-exp merge of the nsplit partials of row bh at dim e, in split order; the merge
// kernel and the in-kernel merge share it, so both give the same bits.
template <bool kCoherent = false>
__device__ __forceinline__ float merge_splits(const DecodeArgs &a, int64_t bh, int nsplit,
                                              int e) {
    const float *ml = a.ws_ml + bh * a.max_splits * 2;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ld_part<kCoherent>(ml + 2 * s));
    float num = 0.f, den = 0.f;
    for (int s = 0; s < nsplit; ++s) {
        const float w = fast_exp2(ld_part<kCoherent>(ml + 2 * s) - M);
        den = fmaf(w, ld_part<kCoherent>(ml + 2 * s + 1), den);
        num = fmaf(w, ld_part<kCoherent>(a.ws_o + (bh * a.max_splits + s) * kHeadDim + e), num);
    }
    return num / den;
}

// Up to G = 4 the kernel fits 3 waves per SIMD (168 VGPRs) without spilling; the hint makes the
// compiler hold that budget.
//
// kFused: the call also stores each row's new K/V (the store of this step's decode rows). The
// workgroup of kv head g that holds a row's last key (key L - 1, the new token) writes head g's
// key and value rows into the pools at the row's slot and reads that key from the new rows
// rather than from the pool, so no store kernel has to run first. Rows without keys store from
// their split-0 workgroups. No other workgroup reads those bytes.
template <int G, bool kFused>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 3 : NV_DECODE_MIN_WAVES))) void decode_split_kernel(DecodeArgs a) {
    __shared__ DecodeSmem<G> sm;

#if NV_DECODE_HEAD_MAJOR == 2
    // 1D grid; workgroup i runs on XCD i % 8. A unit is xcd_heads consecutive kv heads of one
    // (sequence, split) pair; a unit's heads are consecutive workgroups of one XCD, and
    // consecutive units go to different XCDs.
    const int hg = a.xcd_heads;
    const int local = blockIdx.x >> 3;
    const int unit = (local / hg) * 8 + (blockIdx.x & 7);
    const int per_pair = a.num_kv_heads / hg;
    if (unit >= a.n_pairs * per_pair) return;
    const int g = (unit % per_pair) * hg + local % hg;
    // Pair numbering. A grid that runs in one go numbers a sequence's splits consecutively
    // (they start together, which matters when the last one merges). A larger grid numbers
    // sequences fastest: every sequence's first (longest) split is dispatched before any
    // second one, and each split index spreads over all XCDs.
    // Large grids also take the sequences longest first (a permutation written just before),
    // so the longest rows do not start last and leave a tail.
    const int pair = unit / per_pair;
    const int bi = a.splits_together ? pair / a.max_splits : pair % a.batch;
    const int s = a.splits_together ? pair % a.max_splits : pair / a.batch;
    const int b = a.perm ? a.perm[bi] : bi;
#elif NV_DECODE_HEAD_MAJOR
    const int g = blockIdx.x, s = blockIdx.y, b = blockIdx.z;
#else
    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
#endif
    const int L = a.context_lens[b];
    const int k0 = s * a.split_keys;
    // Fused store for a row without keys (no chunk to carry it): head g's 256-byte key and
    // value rows of row b, 16 lanes x 16 bytes each.
    auto store_new = [&]() {
        const int32_t slot = a.slot_mapping[b];
        if (slot < 0 || threadIdx.x >= 32) return;
        const int dcs = threadIdx.x & 15;
        const int64_t dst = ((int64_t)slot * a.num_kv_heads + g) * kHeadDim + 8 * dcs;
        if (threadIdx.x < 16)
            *reinterpret_cast<u32x4 *>(a.k_pool + dst) = *reinterpret_cast<const u32x4 *>(
                a.new_k + (int64_t)b * a.new_k_stride + g * kHeadDim + 8 * dcs);
        else
            *reinterpret_cast<u32x4 *>(a.v_pool + dst) = *reinterpret_cast<const u32x4 *>(
                a.new_v + (int64_t)b * a.new_v_stride + g * kHeadDim + 8 * dcs);
    };
    if (k0 >= L) {  // past this sequence's context, or a padding row
        if (L <= 0 && s == 0) {  // a row without keys outputs zeros
            for (int idx = threadIdx.x; idx < G * kHeadDim; idx += 256)
                a.out[((int64_t)b * a.num_heads + g * G) * kHeadDim + idx] = 0;
            if (kFused) store_new();
        }
        return;
    }
    const int n = min(a.split_keys, L - k0);
    const int nsplit = (L + a.split_keys - 1) / a.split_keys;
    const bool holds_new = kFused && s == nsplit - 1;  // this split ends with key L - 1

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int bs = a.block_size;
    const int lb0 = a.bs_shift >= 0 ? (k0 >> a.bs_shift) : k0 / bs;
    {
        const int lb1 = a.bs_shift >= 0 ? ((k0 + n - 1) >> a.bs_shift) : (k0 + n - 1) / bs;
        const int32_t *table = a.block_tables + (int64_t)b * a.bt_width;
        for (int i = tid; i <= lb1 - lb0; i += 256) sm.table[i] = table[lb0 + i];
    }
    // Pool row of key k0 + jl.
    auto row_of = [&](int jl) -> int64_t {
        const int j = k0 + jl;
        int lb, off;
        if (a.bs_shift >= 0) {
            lb = j >> a.bs_shift;
            off = j & (bs - 1);
        } else {
            lb = j / bs;
            off = j - lb * bs;
        }
        return (int64_t)sm.table[lb - lb0] * bs + off;
    };

    const int64_t rs = (int64_t)a.num_kv_heads * kHeadDim;  // pool row stride (elements)
    const uint16_t *kbase = a.k_cache + (int64_t)g * kHeadDim;
    const uint16_t *vbase = a.v_cache + (int64_t)g * kHeadDim;
    const uint16_t *qbase = a.q + ((int64_t)b * a.num_heads + g * G) * kHeadDim;
    const int sub = lane >> 4;  // key slot of the 16-lane row
    const int dc = lane & 15;   // dims [8 dc, 8 dc + 8) in the row layout

    // This lane's 8 dims of every query head of the group, as bf16 pairs.
    uint32_t qp[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(qbase + h * kHeadDim + 8 * dc);
#pragma unroll
        for (int i = 0; i < 4; ++i) qp[h][i] = v[i];
    }
    __syncthreads();  // table slice visible

    // Chunks inside one block (block size a multiple of the chunk, split aligned to it): one
    // table lookup per chunk gives a scalar base, each lane adds a fixed 32-bit offset.
    const bool chunk_in_block = (bs % kChunk) == 0 && (k0 % kChunk) == 0;
    uint32_t lane_off[kRowLoads];
#pragma unroll
    for (int i = 0; i < kRowLoads; ++i)
        lane_off[i] = (uint32_t)(((4 * i + sub) * rs + 8 * dc) * 2);
    // Fused store: the chunk that holds split key n - 1 (the new token) loads that key's
    // row from the new rows rather than from the pool (an address choice, so the loads stay
    // in flight like any other). The lanes that loaded it write it to the pools as the chunk
    // is processed, when its loads are waited for anyway.
    const uint16_t *new_k_row = kFused ? a.new_k + (int64_t)b * a.new_k_stride + g * kHeadDim
                                       : nullptr;
    const uint16_t *new_v_row = kFused ? a.new_v + (int64_t)b * a.new_v_stride + g * kHeadDim
                                       : nullptr;
    auto put_new = [&](const Chunk &buf, int kc) {
        const int r = n - 1 - kc;
        if (r >= kChunk || sub != (r & 3)) return;
        const int32_t slot = a.slot_mapping[b];
        if (slot < 0) return;
        const int64_t dst = ((int64_t)slot * a.num_kv_heads + g) * kHeadDim + 8 * dc;
        // Register selects (a store per candidate row would be merged into one store indexed
        // at run time, which puts the chunk in scratch memory).
        u32x4 kn = buf.k[0], vn = buf.v[0];
#pragma unroll
        for (int i = 1; i < kRowLoads; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kn[e] = i == (r >> 2) ? buf.k[i][e] : kn[e];
                vn[e] = i == (r >> 2) ? buf.v[i][e] : vn[e];
            }
        *reinterpret_cast<u32x4 *>(a.k_pool + dst) = kn;
        *reinterpret_cast<u32x4 *>(a.v_pool + dst) = vn;
    };
    auto load_chunk = [&](Chunk &buf, int ch) {
        const int kc = ch * kChunk;
        const bool tail_new = holds_new && n - kc <= kChunk;  // wave-uniform
        if (chunk_in_block && kc + kChunk <= n && !tail_new) {
            const int j = k0 + kc;
            int lb, off;
            if (a.bs_shift >= 0) {
                lb = j >> a.bs_shift;
                off = j & (bs - 1);
            } else {
                lb = j / bs;
                off = j - lb * bs;
            }
            const int blk = __builtin_amdgcn_readfirstlane(sm.table[lb - lb0]);
            const int64_t row0 = (int64_t)blk * bs + off;
            const char *kp = reinterpret_cast<const char *>(kbase + row0 * rs);
            const char *vp = reinterpret_cast<const char *>(vbase + row0 * rs);
#pragma unroll
            for (int i = 0; i < kRowLoads; ++i) {
                buf.k[i] = NV_LOAD_STREAM(reinterpret_cast<const u32x4 *>(kp + lane_off[i]));
                buf.v[i] = NV_LOAD_STREAM(reinterpret_cast<const u32x4 *>(vp + lane_off[i]));
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < kRowLoads; ++i) {
            const int jl = kc + 4 * i + sub;
            const bool ok = jl < n;
            const int64_t off = (ok ? row_of(jl) : 0) * rs + 8 * dc;
            const uint16_t *kr = kbase + off, *vr = vbase + off;
            if (kFused && tail_new && jl == n - 1) {
                // Formed here, not hoisted: two more 64-bit addresses live through the loop
                // would spill at G = 4.
                uint32_t lo = 16 * dc;
                asm volatile("" : "+v"(lo));
                kr = reinterpret_cast<const uint16_t *>(
                    reinterpret_cast<const char *>(new_k_row) + lo);
                vr = reinterpret_cast<const uint16_t *>(
                    reinterpret_cast<const char *>(new_v_row) + lo);
            }
            buf.k[i] = ok ? NV_LOAD_STREAM(reinterpret_cast<const u32x4 *>(kr))
                          : u32x4{0, 0, 0, 0};
            buf.v[i] = ok ? NV_LOAD_STREAM(reinterpret_cast<const u32x4 *>(vr))
                          : u32x4{0, 0, 0, 0};
        }
    };

    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    // Running max (log2 units) and this lane's share of the sum, per head.
    float m_run[G], l_run[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
    }

    // One chunk: raw scores q.k, online softmax (max kept in raw units, probabilities as
    // exp2(scale * log2(e) * (s - max))), then P.V into the accumulators.
    auto process = [&](const Chunk &buf, int ch) {
        const int kc = ch * kChunk;
        const bool full = kc + kChunk <= n;  // wave-uniform: only the tail chunk masks
        float sv[kRowLoads][G];
#pragma unroll
        for (int i = 0; i < kRowLoads; ++i) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t kw = buf.k[i][e];
                    d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kw), as_bf16x2(qp[h][e]), d,
                                                        false);
                }
                sv[i][h] = row16_sum(d);
            }
        }
        if (!full) {  // only a split's last chunk has keys past its end
            asm volatile("");  // keeps the masking a real branch (not if-converted)
#pragma unroll
            for (int i = 0; i < kRowLoads; ++i)
#pragma unroll
                for (int h = 0; h < G; ++h)
                    if (kc + 4 * i + sub >= n) sv[i][h] = -INFINITY;
        }
        // The running max may lag the true one by a bounded slack (probabilities up to
        // 2^slack, far from overflow); the max cancels between numerator and sum, so the
        // result is the same. The output rescale runs only when some head's max grows past
        // the slack, typically a few times per split instead of on most chunks; the first
        // chunk always rescales (m_run = -inf).
        float cm[G];
        bool grow = false;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            cm[h] = sv[0][h];
#pragma unroll
            for (int i = 1; i < kRowLoads; ++i) cm[h] = fmaxf(cm[h], sv[i][h]);
            cm[h] = fmaxf(cm[h], __shfl_xor(cm[h], 16));
            cm[h] = fmaxf(cm[h], __shfl_xor(cm[h], 32));
            grow |= cm[h] > m_run[h] + a.rescale_slack;
        }
        if (__any(grow)) {
            asm volatile("");  // keeps the rescale a real branch (not if-converted)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float m_new = fmaxf(m_run[h], cm[h]);
                const float alpha = fast_exp2((m_run[h] - m_new) * a.scale_log2);
                m_run[h] = m_new;
                l_run[h] *= alpha;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
            }
        }
        // With G <= 4 the 16 lanes of a key row hold the same 4 G scores: lane dc computes
        // only value dc = i G + h (row i, head h), pairs it with row i + 1 of the same head
        // (lane dc + G) as bf16, and the pairs of even rows are broadcast back to the row.
        constexpr bool kDedup = NV_DECODE_EXPDEDUP && NV_DECODE_PV_DOT2 && G <= 4 &&
                                kRowLoads == 4;
        if constexpr (kDedup) {
            float sel = sv[0][0], msel = m_run[0];
#pragma unroll
            for (int i = 0; i < kRowLoads; ++i)
#pragma unroll
                for (int h = 0; h < G; ++h)
                    if (i * G + h != 0) sel = dc == i * G + h ? sv[i][h] : sel;
#pragma unroll
            for (int h = 1; h < G; ++h) msel = dc % G == h ? m_run[h] : msel;
            const float p = fast_exp2(fmaf(sel, a.scale_log2, -msel * a.scale_log2));
            const uint32_t pk = pack_bf16(p, row_ror<16 - G>(p));  // with lane dc + G's value
            uint32_t pp[2][G];
            bcast_pairs<G, 0, 0>(pk, pp);
            const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int h = 0; h < G; ++h)
                    l_run[h] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pp[j][h]), ones,
                                                               l_run[h], false);
#pragma unroll
                for (int wd = 0; wd < 4; ++wd) {
                    const uint32_t x = buf.v[2 * j][wd], y = buf.v[2 * j + 1][wd];
                    const uint32_t lo = __builtin_amdgcn_perm(y, x, 0x05040100u);  // dim 2 wd
                    const uint32_t hi = __builtin_amdgcn_perm(y, x, 0x07060302u);  // dim 2 wd + 1
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        acc[h][2 * wd] = __builtin_amdgcn_fdot2_f32_bf16(
                            as_bf16x2(lo), as_bf16x2(pp[j][h]), acc[h][2 * wd], false);
                        acc[h][2 * wd + 1] = __builtin_amdgcn_fdot2_f32_bf16(
                            as_bf16x2(hi), as_bf16x2(pp[j][h]), acc[h][2 * wd + 1], false);
                    }
                }
            }
            return;
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float msc = m_run[h] * a.scale_log2;
            float ps = 0.f;
#pragma unroll
            for (int i = 0; i < kRowLoads; ++i) {
                sv[i][h] = fast_exp2(fmaf(sv[i][h], a.scale_log2, -msc));
                if constexpr (!NV_DECODE_PV_DOT2) ps += sv[i][h];
            }
            if constexpr (!NV_DECODE_PV_DOT2) l_run[h] += ps;
        }
        if constexpr (NV_DECODE_PV_DOT2) {
            const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
            // Two keys at a time: pack (v_i[e], v_{i+1}[e]) and (p_i, p_{i+1}) as bf16 pairs
            // and accumulate their dot product in fp32 (p rounded to bf16, as for the MFMA
            // P.V of prefill).
#pragma unroll
            for (int i = 0; i < kRowLoads; i += 2) {
                uint32_t pp[G];
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    pp[h] = pack_bf16(sv[i][h], sv[i + 1][h]);
                    // the sum takes exactly the bf16 probabilities that multiply V
                    l_run[h] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pp[h]), ones, l_run[h],
                                                               false);
                }
#pragma unroll
                for (int wd = 0; wd < 4; ++wd) {
                    const uint32_t x = buf.v[i][wd], y = buf.v[i + 1][wd];
                    const uint32_t lo = (x & 0xffffu) | (y << 16);          // dim 2 wd
                    const uint32_t hi = (x >> 16) | (y & 0xffff0000u);      // dim 2 wd + 1
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        acc[h][2 * wd] = __builtin_amdgcn_fdot2_f32_bf16(
                            as_bf16x2(lo), as_bf16x2(pp[h]), acc[h][2 * wd], false);
                        acc[h][2 * wd + 1] = __builtin_amdgcn_fdot2_f32_bf16(
                            as_bf16x2(hi), as_bf16x2(pp[h]), acc[h][2 * wd + 1], false);
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < kRowLoads; ++i) {
                float vf[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vf[2 * e] = bf16lo(buf.v[i][e]);
                    vf[2 * e + 1] = bf16hi(buf.v[i][e]);
                }
#pragma unroll
                for (int h = 0; h < G; ++h)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(sv[i][h], vf[e], acc[h][e]);
            }
        }
    };

    // Two register buffers: the next chunk is in flight while the current one is processed.
    const int nch = (n + kChunk - 1) / kChunk;
    Chunk A, B;
    int ch = w;
    if (ch < nch) load_chunk(A, ch);
    while (ch < nch) {
        if (ch + 4 < nch) load_chunk(B, ch + 4);
        if (holds_new) put_new(A, ch * kChunk);
        process(A, ch);
        ch += 4;
        if (ch >= nch) break;
        if (ch + 4 < nch) load_chunk(A, ch + 4);
        if (holds_new) put_new(B, ch * kChunk);
        process(B, ch);
        ch += 4;
    }

    // Merge: within the wave (sum over the 4 key slots), then across the 4 waves.
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = acc[h][e];
            x += __shfl_xor(x, 16);
            x += __shfl_xor(x, 32);
            acc[h][e] = x;
        }
    if (sub == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.o[w][h][8 * dc + e] = acc[h][e];
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float l = l_run[h];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if (lane == 0) {
            sm.ml[w][h][0] = m_run[h] * a.scale_log2;  // -inf for a wave without keys
            sm.ml[w][h][1] = l;
        }
    }
    __syncthreads();

    for (int idx = tid; idx < G * kHeadDim; idx += 256) {
        const int h = idx / kHeadDim, e = idx % kHeadDim;
        float M = sm.ml[0][h][0];
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, sm.ml[ww][h][0]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            const float f = fast_exp2(sm.ml[ww][h][0] - M);  // 0 for a wave without keys
            num = fmaf(f, sm.o[ww][h][e], num);
            den = fmaf(f, sm.ml[ww][h][1], den);
        }
        const int64_t bh = (int64_t)b * a.num_heads + g * G + h;
        if (nsplit == 1) {
            a.out[bh * kHeadDim + e] = __builtin_bit_cast(uint16_t, (__bf16)(num / den));
        } else if (kFused && a.counters) {
            st_part<true>(a.ws_o + (bh * a.max_splits + s) * kHeadDim + e, num);
            if (e == 0) {
                st_part<true>(a.ws_ml + (bh * a.max_splits + s) * 2, M);
                st_part<true>(a.ws_ml + (bh * a.max_splits + s) * 2 + 1, den);
            }
        } else {
            a.ws_o[(bh * a.max_splits + s) * kHeadDim + e] = num;
            if (e == 0) {
                a.ws_ml[(bh * a.max_splits + s) * 2] = M;
                a.ws_ml[(bh * a.max_splits + s) * 2 + 1] = den;
            }
        }
    }
    if (!kFused || nsplit == 1 || a.counters == nullptr) return;

    // In-kernel merge: the last of the row's nsplit workgroups to finish merges all partials.
    // Every wave waits until its (coherent) partial stores have completed, the workgroup
    // meets, and one lane counts the arrival; the workgroup that brings the count to nsplit
    // reads the partials with coherent loads, issued only after the count returned. Nothing
    // waits on another workgroup, so any dispatch order completes.
    // Ordering, per the AMDGPU memory model's code sequences for gfx942-class targets (LLVM's
    // AMDGPU backend user guide, "Memory Model GFX942"; the ISA here matches them): an
    // agent-scope relaxed atomic store/load is a global store/load with sc1, performed at the
    // device coherence point rather than in this XCD's L2; an agent-scope release is
    // buffer_wbl2 sc1 + s_waitcnt vmcnt(0) and an acquire s_waitcnt vmcnt(0) + buffer_inv sc1,
    // where the write-back and invalidate only serve non-atomic data. The partials are sc1
    // atomics, so the wait below is the whole release they need: when the fetch_add is
    // performed they are complete at the coherence point. The merger's sc1 loads depend on the
    // fetch_add's result (barrier and branch), so they are issued after it returns and read
    // the coherence point; no cache-wide write-back or invalidate is needed.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    uint32_t *cnt = a.counters + (int64_t)b * a.num_kv_heads + g;
    if (tid == 0)
        sm.merges = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                    (uint32_t)(nsplit - 1);
    __syncthreads();
    if (!sm.merges) return;
    if (tid == 0)  // ready for the next call
        __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int idx = tid; idx < G * kHeadDim; idx += 256) {
        const int h = idx / kHeadDim, e = idx % kHeadDim;
        const int64_t bh = (int64_t)b * a.num_heads + g * G + h;
        a.out[bh * kHeadDim + e] =
            __builtin_bit_cast(uint16_t, (__bf16)merge_splits<true>(a, bh, nsplit, e));
    }
}

// Merges the splits of each (sequence, head); writes zeros for rows without keys.
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeArgs a) {
    const int h = blockIdx.x, b = blockIdx.y, e = threadIdx.x;
    const int L = a.context_lens[b];
    const int64_t bh = (int64_t)b * a.num_heads + h;
    if (L <= 0) {
        a.out[bh * kHeadDim + e] = 0;
        return;
    }
    const int nsplit = (L + a.split_keys - 1) / a.split_keys;
    if (nsplit == 1) return;  // the split kernel wrote the final row
    a.out[bh * kHeadDim + e] = __builtin_bit_cast(uint16_t, (__bf16)merge_splits(a, bh, nsplit, e));
}

// Sequences longest first, for the dispatch order of large decode grids: a counting sort of
// context lengths into 1024 buckets (one workgroup, histogram and offsets in LDS). Rows of one
// bucket land in any order; each row's result does not depend on the order.
constexpr int kOrderThreads = 1024;
__global__ __launch_bounds__(kOrderThreads) void decode_order_kernel(const int32_t *lens,
                                                                     int32_t batch,
                                                                     int64_t max_ctx,
                                                                     int32_t *perm) {
    __shared__ int32_t next[kOrderThreads];
    __shared__ int32_t scan[kOrderThreads];
    const int t = threadIdx.x;
    auto key_of = [&](int32_t L) -> int {  // longer rows get smaller keys
        const int64_t l = L < 0 ? 0 : (L > max_ctx ? max_ctx : L);
        return kOrderThreads - 1 - (int)(l * kOrderThreads / (max_ctx + 1));
    };
    next[t] = 0;
    __syncthreads();
    for (int b = t; b < batch; b += kOrderThreads) atomicAdd(&next[key_of(lens[b])], 1);
    __syncthreads();
    const int count = next[t];
    scan[t] = count;
    __syncthreads();
    for (int off = 1; off < kOrderThreads; off <<= 1) {  // inclusive prefix sum
        const int x = t >= off ? scan[t - off] : 0;
        __syncthreads();
        scan[t] += x;
        __syncthreads();
    }
    next[t] = scan[t] - count;  // first position of bucket t
    __syncthreads();
    for (int b = t; b < batch; b += kOrderThreads) perm[atomicAdd(&next[key_of(lens[b])], 1)] = b;
}

template <int G, bool kFused>
nv_status launch_decode(const DecodeArgs &a, int batch, hipStream_t stream) {
#if NV_DECODE_HEAD_MAJOR == 2
    if (a.perm) {
        const nv_status st = launch(decode_order_kernel, dim3(1), dim3(kOrderThreads), 0, stream,
                                    a.context_lens, (int32_t)batch,
                                    (int64_t)a.bt_width * a.block_size,
                                    const_cast<int32_t *>(a.perm));
        if (st != NV_OK) return st;
    }
    const int64_t units = (int64_t)a.n_pairs * (a.num_kv_heads / a.xcd_heads);
    const dim3 grid((uint32_t)(8 * ((units + 7) / 8) * a.xcd_heads));
#elif NV_DECODE_HEAD_MAJOR
    const dim3 grid(a.num_kv_heads, a.max_splits, batch);
#else
    const dim3 grid(a.max_splits, a.num_kv_heads, batch);
#endif
    nv_status st = launch(decode_split_kernel<G, kFused>, grid, dim3(256), 0, stream, a);
    // One split: every row is final already. With counters the split kernel merged.
    if (st != NV_OK || a.max_splits == 1 || (kFused && a.counters)) return st;
    return launch(decode_combine_kernel, dim3(a.num_heads, batch), dim3(kHeadDim), 0, stream, a);
}

int64_t max_context(int32_t max_blocks_per_seq, int32_t block_size) {
    return (int64_t)max_blocks_per_seq * block_size;
}

int32_t split_keys_for(int32_t batch, int32_t num_kv_heads, int32_t max_blocks_per_seq,
                       int32_t block_size) {
    // Largest split (fewest partials) that still yields enough work items over the padded
    // context, so every CU gets work; capped so that one split's table slice fits in LDS.
    const int64_t ctx = max_context(max_blocks_per_seq, block_size);
    const int64_t cap = (int64_t)(kTableSlots - 2) * (block_size > 0 ? block_size : 1);
    int32_t S = kMaxSplitKeys;
    while (S > kMinSplitKeys &&
           (S > cap || (int64_t)batch * num_kv_heads * ((ctx + S - 1) / S) < NV_DECODE_TARGET_ITEMS))
        S /= 2;
    return S;
}

// The launch shape and workspace layout of one decode call; the workspace size query and the
// call itself both derive them here so they agree. Workspace: ml [B, Hq, splits, 2] (256-byte
// padded), o [B, Hq, splits, head_dim], then the longest-first sequence order [B] (large grids
// with more than one sequence only), 256-byte padded.
struct DecodePlan {
    int32_t split_keys = 0;
    int64_t splits = 0;
    int32_t xcd_heads = 1;
    bool splits_together = true;
    bool ordered = false;
    size_t ml_bytes = 0, o_bytes = 0, perm_bytes = 0;
    size_t total() const { return ml_bytes + o_bytes + perm_bytes; }
};

DecodePlan plan_decode(int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t max_blocks_per_seq, int32_t block_size) {
    DecodePlan p;
    p.split_keys = split_keys_for(batch, num_kv_heads, max_blocks_per_seq, block_size);
    p.splits = (max_context(max_blocks_per_seq, block_size) + p.split_keys - 1) / p.split_keys;
    p.xcd_heads = std::gcd(num_kv_heads, NV_DECODE_XCD_HEADS > 0 ? (int32_t)NV_DECODE_XCD_HEADS
                                                                  : num_heads / num_kv_heads);
    // Workgroups of the 1D grid; up to 3 per CU (the register budget of G <= 4) it runs in one
    // go on the 256 CUs. Larger grids run in waves, where the dispatch order matters.
    const int64_t units = (int64_t)batch * p.splits * (num_kv_heads / p.xcd_heads);
    p.splits_together = 8 * ((units + 7) / 8) * p.xcd_heads <= NV_DECODE_ONE_GO_GROUPS;
    p.ordered = !p.splits_together && batch > 1;
    if (p.splits > 1) {
        const size_t rows = (size_t)batch * num_heads * p.splits;
        p.ml_bytes = (rows * 2 * sizeof(float) + 255) / 256 * 256;
        p.o_bytes = (rows * head_dim * sizeof(float) + 255) / 256 * 256;
    }
    if (p.ordered) p.perm_bytes = ((size_t)batch * sizeof(int32_t) + 255) / 256 * 256;
    return p;
}

}  // namespace
}  // namespace nvp

extern "C" int32_t nv_paged_attn_decode_split_keys(int32_t batch, int32_t num_kv_heads,
                                                   int32_t max_blocks_per_seq,
                                                   int32_t block_size) {
    return nvp::split_keys_for(batch, num_kv_heads, max_blocks_per_seq, block_size);
}

extern "C" size_t nv_paged_attn_decode_workspace_size(int32_t batch, int32_t num_heads,
                                                      int32_t num_kv_heads, int32_t head_dim,
                                                      int32_t max_blocks_per_seq,
                                                      int32_t block_size) {
    if (batch <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        max_blocks_per_seq <= 0 || block_size <= 0 || num_heads % num_kv_heads != 0)
        return 0;
    return nvp::plan_decode(batch, num_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                            block_size)
        .total();
}

namespace nvp {
namespace {

// The decode rows' new K/V for the fused call (null for the plain decode).
struct FusedStore {
    const uint16_t *key;
    int64_t key_row_stride;
    const uint16_t *value;
    int64_t value_row_stride;
    const int32_t *slot_mapping;
    uint32_t *counters;  // in-kernel merge counters [B * Hkv], or null
};

nv_status decode_impl(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *context_lens, const int32_t *block_tables,
                      int32_t max_blocks_per_seq, int32_t batch, int32_t num_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      float softmax_scale, void *workspace, size_t workspace_bytes, void *out,
                      hipStream_t stream, const FusedStore *fs);

}  // namespace
}  // namespace nvp

extern "C" nv_status nv_paged_attn_decode(const void *q, const void *k_cache,
                                          const void *v_cache, const int32_t *context_lens,
                                          const int32_t *block_tables,
                                          int32_t max_blocks_per_seq, int32_t batch,
                                          int32_t num_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t block_size,
                                          float softmax_scale, void *workspace,
                                          size_t workspace_bytes, void *out,
                                          hipStream_t stream) {
    return nvp::decode_impl(q, k_cache, v_cache, context_lens, block_tables, max_blocks_per_seq,
                            batch, num_heads, num_kv_heads, head_dim, block_size, softmax_scale,
                            workspace, workspace_bytes, out, stream, nullptr);
}

extern "C" nv_status nv_paged_attn_decode_store(
    const void *q, const void *key, int64_t key_row_stride, const void *value,
    int64_t value_row_stride, const int32_t *slot_mapping, void *k_cache, void *v_cache,
    int64_t num_slots, const int32_t *context_lens, const int32_t *block_tables,
    int32_t max_blocks_per_seq, int32_t batch, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, float softmax_scale, void *workspace,
    size_t workspace_bytes, uint32_t *counters, int64_t num_counters, void *out,
    hipStream_t stream) {
    using namespace nvp;
    if (batch < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_slots < 0)
        return NV_ERR_INVALID_ARG;
    if (counters && (num_counters < (int64_t)batch * num_kv_heads ||
                     reinterpret_cast<uintptr_t>(counters) % 4 != 0))
        return NV_ERR_INVALID_ARG;
    const int64_t D = (int64_t)num_kv_heads * head_dim;
    if (key_row_stride < D || value_row_stride < D) return NV_ERR_INVALID_ARG;
    if (batch > 0 && (!key || !value || !slot_mapping || !k_cache || !v_cache))
        return NV_ERR_INVALID_ARG;
    // One launch needs whole 16-byte lanes; otherwise (or with no key slots at all) the store
    // and the decode run one after the other, with the same result.
    const auto a16 = [](const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
    const bool fusable = key_row_stride % 8 == 0 && value_row_stride % 8 == 0 && a16(key) &&
                         a16(value) && a16(k_cache) && a16(v_cache) && max_blocks_per_seq > 0;
    if (!fusable) {
        const nv_status st = nv_store_kvcache(key, key_row_stride, value, value_row_stride,
                                              k_cache, v_cache, slot_mapping, batch,
                                              num_kv_heads, head_dim, num_slots, stream);
        if (st != NV_OK) return st;
        return nv_paged_attn_decode(q, k_cache, v_cache, context_lens, block_tables,
                                    max_blocks_per_seq, batch, num_heads, num_kv_heads, head_dim,
                                    block_size, softmax_scale, workspace, workspace_bytes, out,
                                    stream);
    }
    const FusedStore fs{static_cast<const uint16_t *>(key), key_row_stride,
                        static_cast<const uint16_t *>(value), value_row_stride, slot_mapping,
                        counters};
    return decode_impl(q, k_cache, v_cache, context_lens, block_tables, max_blocks_per_seq, batch,
                       num_heads, num_kv_heads, head_dim, block_size, softmax_scale, workspace,
                       workspace_bytes, out, stream, &fs);
}

namespace nvp {
namespace {

nv_status decode_impl(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *context_lens, const int32_t *block_tables,
                      int32_t max_blocks_per_seq, int32_t batch, int32_t num_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      float softmax_scale, void *workspace, size_t workspace_bytes, void *out,
                      hipStream_t stream, const FusedStore *fs) {
    if (batch < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        max_blocks_per_seq < 0)
        return NV_ERR_INVALID_ARG;
    if (num_heads % num_kv_heads != 0) return NV_ERR_INVALID_ARG;
    if (!(softmax_scale > 0.f) || softmax_scale == INFINITY) return NV_ERR_INVALID_ARG;
    if (head_dim != kHeadDim) return NV_ERR_UNSUPPORTED;
    const int G = num_heads / num_kv_heads;
    if (G > 8) return NV_ERR_UNSUPPORTED;
    if (batch == 0) return NV_OK;
    if (!q || !k_cache || !v_cache || !context_lens || !out) return NV_ERR_INVALID_ARG;
    if (batch > 65535 || num_kv_heads > 65535) return NV_ERR_UNSUPPORTED;
    if (max_blocks_per_seq == 0) {
        // No sequence can hold a key: every row is a padding row; only the zeros are written.
        DecodeArgs z{};
        z.context_lens = context_lens;
        z.out = static_cast<uint16_t *>(out);
        z.num_heads = num_heads;
        z.split_keys = kMaxSplitKeys;
        z.max_splits = 1;
        return launch(decode_combine_kernel, dim3(num_heads, batch), dim3(kHeadDim), 0, stream, z);
    }
    if (!block_tables) return NV_ERR_INVALID_ARG;
    const DecodePlan p = plan_decode(batch, num_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                                     block_size);
    const size_t need = p.total();
    if (need > 0 && (!workspace || workspace_bytes < need ||
                     reinterpret_cast<uintptr_t>(workspace) % 256 != 0))
        return NV_ERR_WORKSPACE;
    DecodeArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k_cache = static_cast<const uint16_t *>(k_cache);
    a.v_cache = static_cast<const uint16_t *>(v_cache);
    a.context_lens = context_lens;
    a.block_tables = block_tables;
    a.out = static_cast<uint16_t *>(out);
    a.bt_width = max_blocks_per_seq;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.block_size = block_size;
    a.bs_shift = (block_size & (block_size - 1)) == 0 ? __builtin_ctz((unsigned)block_size) : -1;
    a.split_keys = p.split_keys;
    if (p.splits > 65535) return NV_ERR_UNSUPPORTED;
    a.max_splits = (int32_t)p.splits;
    if ((int64_t)batch * p.splits * num_kv_heads + 8 * (int64_t)num_kv_heads > INT32_MAX)
        return NV_ERR_UNSUPPORTED;  // grid size
    a.n_pairs = (int32_t)(batch * p.splits);
    a.batch = batch;
    a.xcd_heads = p.xcd_heads;
    a.splits_together = p.splits_together;
    char *ws = static_cast<char *>(workspace);
    a.ws_ml = p.ml_bytes ? reinterpret_cast<float *>(ws) : nullptr;
    a.ws_o = p.o_bytes ? reinterpret_cast<float *>(ws + p.ml_bytes) : nullptr;
    a.perm = p.ordered ? reinterpret_cast<int32_t *>(ws + p.ml_bytes + p.o_bytes) : nullptr;
    a.scale_log2 = softmax_scale * kLog2e;
    a.rescale_slack = NV_DECODE_SLACK / a.scale_log2;
    a.new_k = fs ? fs->key : nullptr;
    a.new_v = fs ? fs->value : nullptr;
    a.new_k_stride = fs ? fs->key_row_stride : 0;
    a.new_v_stride = fs ? fs->value_row_stride : 0;
    a.slot_mapping = fs ? fs->slot_mapping : nullptr;
    a.k_pool = fs ? static_cast<uint16_t *>(const_cast<void *>(k_cache)) : nullptr;
    a.v_pool = fs ? static_cast<uint16_t *>(const_cast<void *>(v_cache)) : nullptr;
    a.counters = fs ? fs->counters : nullptr;
    if (fs) {
        switch (G) {
            case 1: return launch_decode<1, true>(a, batch, stream);
            case 2: return launch_decode<2, true>(a, batch, stream);
            case 3: return launch_decode<3, true>(a, batch, stream);
            case 4: return launch_decode<4, true>(a, batch, stream);
            case 5: return launch_decode<5, true>(a, batch, stream);
            case 6: return launch_decode<6, true>(a, batch, stream);
            case 7: return launch_decode<7, true>(a, batch, stream);
            default: return launch_decode<8, true>(a, batch, stream);
        }
    }
    switch (G) {
        case 1: return launch_decode<1, false>(a, batch, stream);
        case 2: return launch_decode<2, false>(a, batch, stream);
        case 3: return launch_decode<3, false>(a, batch, stream);
        case 4: return launch_decode<4, false>(a, batch, stream);
        case 5: return launch_decode<5, false>(a, batch, stream);
        case 6: return launch_decode<6, false>(a, batch, stream);
        case 7: return launch_decode<7, false>(a, batch, stream);
        default: return launch_decode<8, false>(a, batch, stream);
    }
}

}  // namespace
}  // namespace nvp

// ---- Decode without a caller workspace (callers that cannot allocate) ----
//
// The workspace of nv_paged_attn_decode_noalloc: one static device array; every GPU the
// library runs on holds its own copy until the process ends. In host code `scratch` names a
// host-side stand-in, not device memory: the device address comes from hipGetSymbolAddress,
// once per device with that device current, and only that address reaches a kernel.
static __device__ __align__(256) unsigned char scratch[NV_DECODE_SCRATCH_BYTES];

namespace nvp {
namespace {

constexpr int kMaxScratchDevices = 256;
std::atomic<void *> g_scratch_addr[kMaxScratchDevices];
std::mutex g_scratch_lookup;

// Device address of the current device's scratch array.
nv_status device_scratch(void **addr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
        return NV_ERR_LAUNCH;
    void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_lookup);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
                return NV_ERR_LAUNCH;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *addr = p;
    return NV_OK;
}

}  // namespace
}  // namespace nvp

extern "C" nv_status nv_paged_attn_decode_noalloc(const void *q, const void *k_cache,
                                                  const void *v_cache,
                                                  const int32_t *context_lens,
                                                  const int32_t *block_tables,
                                                  int32_t max_blocks_per_seq, int32_t batch,
                                                  int32_t num_heads, int32_t num_kv_heads,
                                                  int32_t head_dim, int32_t block_size,
                                                  float softmax_scale, void *out,
                                                  hipStream_t stream) {
    using namespace nvp;
    // The size is known on the host before anything runs (0 also for arguments the decode
    // itself rejects); nothing is launched when it exceeds the array.
    const size_t need = nv_paged_attn_decode_workspace_size(batch, num_heads, num_kv_heads,
                                                            head_dim, max_blocks_per_seq,
                                                            block_size);
    if (need > NV_DECODE_SCRATCH_BYTES) return NV_ERR_SCRATCH;
    void *ws = nullptr;
    if (need > 0) {
        const nv_status st = device_scratch(&ws);
        if (st != NV_OK) return st;
    }
    return decode_impl(q, k_cache, v_cache, context_lens, block_tables, max_blocks_per_seq,
                       batch, num_heads, num_kv_heads, head_dim, block_size, softmax_scale, ws,
                       ws ? NV_DECODE_SCRATCH_BYTES : 0, out, stream, nullptr);
}
