// Paged prefill attention: causal varlen attention of each sequence's new rows against its
// cached prefix plus its new keys, all read through its block table.
//
// Operation ("Nano-vLLM Field Guide", Step 10.3, prefill with block_table; Step 07.5 for the
// packing): sequence b has Lq new rows and Lk keys; new row i sees keys 0 .. (Lk - Lq) + i
// (the causal mask aligned to the bottom-right corner). out = softmax(scale q K^T) V per query
// head; query head h reads kv head h / G.
//
// gfx950 design (bf16 MFMA, fp32 accumulation, online softmax):
//  - A workgroup of W waves owns one kv head g, HPW query heads of its group (4 when the group
//    size allows, else 2 or 1) and a tile of M = 32 W / HPW new rows; W is 8 with four heads
//    or when the context is long next to the new tokens, else 4. Each wave
//    owns 32 rows of one head. Every K/V tile staged in LDS is therefore shared by all query
//    heads and rows the workgroup holds.
//  - K/V are walked in tiles of 64 keys, copied from HBM straight into LDS with
//    global_load_lds (16 bytes per lane, no staging registers) into two LDS stages: the next
//    tile streams in while the current one is multiplied; one barrier per tile. When the block
//    size is a multiple of 64 a full tile lies inside one block: one table lookup per tile
//    gives a scalar base address and each lane adds a fixed offset. Otherwise (and for the
//    last, partial tile) each lane looks up its own key's block, so any block size works;
//    padding entries are never read, and keys past the end re-read the last valid key (a
//    stale row could hold NaN, which 0 x NaN would carry into O) before being masked.
//  - LDS rows are 256 bytes, unpadded; bank conflicts are avoided by XOR-swizzling the 16-byte
//    chunks of a row (K: chunk ^ (row % 16); V: chunk ^ 6 (row % 2) ^ 12 (row / 2 % 2)),
//    applied on the global side since the copy places lane i's 16 bytes at 16 i.
//  - Scores are computed transposed, S^T[key, row] = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    K (A operand) is read from LDS, Q^T (B operand) stays in registers for the whole loop. In
//    the 32x32 accumulator a lane holds one query row and 16 of its keys, so the softmax row
//    max is an in-register max plus one swap with the lane 32 away, and the row sum is kept
//    per lane and merged once at the end.
//  - O^T[dim, row] += V^T P^T. The probabilities never leave registers: the accumulator of S^T
//    already is the B operand layout once converted to bf16, with the key order inside each
//    16-key MFMA step chosen to match it. The V^T operand is read from row-major V in LDS
//    with ds_read_b64_tr_b16 (each 16-lane group turns 4 keys x 16 dims into one dim x 4
//    keys per lane), two reads per MFMA.
//  - Softmax in log2 units with the scale folded into one FMA before exp2; masking only on
//    tiles the causal diagonal or the key end cuts. The running max used for the exponent may
//    lag the true one by a bounded slack (probabilities up to 2^slack), so the 64-register
//    output rescale runs only when some row's max grows past it, typically once per row
//    block instead of on most tiles; the max cancels between O and l, so the result is the
//    same. Row sums are dot products of the packed bf16 probabilities with ones, i.e. the
//    sums of exactly the values that multiply V.
//  - Work is dealt to the 8 XCDs by (head subgroup, sequence, kv head) group, round-robin with
//    the kv head fastest: with a multiple of 8 kv heads every workgroup reading one kv head's
//    K/V shares an L2, and every XCD gets a share of every sequence (balanced under mixed
//    prompt lengths). Within an XCD the q tiles that see the most keys start first.
#include "nv_common.h"

#include <type_traits>

#ifndef NV_PREFILL_WAVES
#define NV_PREFILL_WAVES 2  // register budget for this many waves per SIMD
#endif
#ifndef NV_PREFILL_FASTCOPY
#define NV_PREFILL_FASTCOPY 1  // whole-block tiles: scalar base address + fixed lane offsets
#endif
#ifndef NV_PREFILL_KPF
#define NV_PREFILL_KPF 4       // K fragments read this many dim-steps ahead of their products
#endif
// Scheduling-group pins for the K read / score product interleave: off, since the iterative
// ILP scheduler this file is built with orders the loop better unpinned.
#ifndef NV_PREFILL_SGB
#define NV_PREFILL_SGB 0
#endif
#ifndef NV_PREFILL_VPF
#define NV_PREFILL_VPF 1       // read the first P.V step's V fragments before the softmax
#endif
#ifndef NV_PREFILL_SLACK
#define NV_PREFILL_SLACK 8.0f  // rescale only when a row max grows by more than this (log2 units)
#endif


namespace nvp {
namespace {

constexpr int kTileKeys = 64;
constexpr int kTableSlots = 2048;  // block-table entries staged in LDS (caps max_seqlen_k / block_size)
constexpr int kRowBytes = kHeadDim * 2;           // one key row of one kv head in LDS
constexpr int kTileBytes = kTileKeys * kRowBytes;  // 16 KiB

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4v;
#define NV_LDS __attribute__((address_space(3)))

// Asynchronous copy of 16 bytes per lane from global memory into LDS: lane i's bytes land at
// lds_base + 16 i (lds_base wave-uniform). Issued through inline assembly so that the
// compiler's wait insertion does not treat the in-flight copy as aliasing every LDS read
// (it would drain the copy before each one); completion is waited for explicitly
// (s_waitcnt vmcnt) before the barrier that publishes a tile.
//
// M0 carries the LDS address of the copy. The compiler reports the m0 clobber as ignored (M0 is
// a reserved register) but never uses M0 itself in these kernels: in their ISA every write of
// M0 is one of these two helpers, each immediately followed by its copy. The clobber stays as
// documentation and that one diagnostic is muted here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(const void *src, void *lds_base) {
    const uint32_t base = (uint32_t)(uintptr_t)lds_base;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(base)), "v"(src)
                 : "memory", "m0");
}

// Same copy with a wave-uniform 64-bit base address in SGPRs and a 32-bit per-lane byte
// offset: no per-lane address arithmetic.
__device__ __forceinline__ void copy16_to_lds_sbase(const void *sbase, uint32_t voff,
                                                    void *lds_base) {
    const uint32_t base = (uint32_t)(uintptr_t)lds_base;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(base)), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Waits until at most N of this wave's memory loads are outstanding and all its LDS accesses
// are done (loads complete in order, so the older tile's copies have landed), then meets the
// workgroup at a barrier. Unlike __syncthreads this does not drain the younger copies.
template <int N>
__device__ __forceinline__ void wait_copies_and_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Waits until at most N of this wave's memory loads are outstanding (no LDS wait, no barrier).
template <int N>
__device__ __forceinline__ void wait_copies() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0xf << 8) | (0x7 << 4));
    asm volatile("" ::: "memory");
}

// max / sum of x over lanes l and l ^ 32, in every lane: v_permlane32_swap trades the two
// 32-lane halves of two registers in the VALU (a lane shuffle would go through LDS). With x in
// both, the results hold [x(0..31), x(0..31)] and [x(32..63), x(32..63)].
__device__ __forceinline__ float halves_max(float x) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// 16-byte chunk position of logical chunk c of tile row r in LDS.
__device__ __forceinline__ int k_chunk_pos(int r, int c) { return c ^ (r & 15); }
// V rows are read four at a time by 16-lane groups (32 bytes of each row) and two such groups
// (the other 32 bytes) are served together: the XOR pattern below gives the 4 rows x 4 chunks
// 16 distinct chunk positions, and each group's 4 rows x 2 chunks 8 distinct positions modulo
// 8, so neither read width hits a bank twice.
__device__ __forceinline__ int v_chunk_pos(int r, int c) {
    return c ^ ((r & 1) * 6) ^ (((r >> 1) & 1) * 12);
}

struct PrefillArgs {
    const uint16_t *q;
    const uint16_t *k_cache;
    const uint16_t *v_cache;
    const int32_t *cu_q;
    const int32_t *cu_k;
    const int32_t *block_tables;
    uint16_t *out;
    int32_t bt_width;
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t group;       // G
    int32_t block_size;
    int32_t bs_shift;
    int32_t batch;
    int32_t n_groups;        // head subgroups x sequences x kv heads
    int32_t groups_per_xcd;
    int32_t tile_in_block;  // block_size % 64 == 0: a 64-key tile never straddles two blocks
    int64_t k_row_stride;   // elements between consecutive K rows (pool rows or packed rows)
    int64_t v_row_stride;
    float scale_log2;
    float rescale_slack;    // raw-score growth of a row max tolerated without a rescale
};

template <int HPW, int kWaves>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(NV_PREFILL_WAVES))) void prefill_kernel(PrefillArgs a) {
    constexpr int kWavesPerHead = kWaves / HPW;
    constexpr int M = 32 * kWavesPerHead;  // rows per workgroup
    // Two stages each of K and V tiles (row-major, swizzled), 16 KiB per tile.
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds[2][kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds[2][kTileBytes];
    __shared__ int32_t tbl[kTableSlots];  // the sequence's first block ids, staged once
    // Query rows pass through LDS once, 8 KiB per wave: waves 0-3 use the second K/V stage
    // (free until the second tile's copies, issued after everyone has read its queries),
    // waves 4-7 a buffer of their own.
    constexpr int kQWaveBytes = 32 * kRowBytes;
    __shared__ __attribute__((aligned(1024))) uint8_t q_lds_hi[kWaves == 8 ? 4 * kQWaveBytes : 16];

    // Work decomposition. A group is one (head subgroup, sequence, kv head), numbered with the
    // kv head fastest; group q runs on XCD q % 8 (the hardware deals consecutive workgroup ids
    // round-robin to the 8 XCDs). Within an XCD the q tiles are issued by rank from the end of
    // their sequence: the last tiles, which see the most keys, start first.
    const int bid = blockIdx.x;
    const int slot = bid >> 3;
    const int rank = slot / a.groups_per_xcd;
    const int grp = (bid & 7) + 8 * (slot - rank * a.groups_per_xcd);
    if (grp >= a.n_groups) return;
    const int g = grp % a.num_kv_heads;
    const int b = (grp / a.num_kv_heads) % a.batch;
    const int hs = grp / (a.num_kv_heads * a.batch);

    const int q0 = a.cu_q[b];
    const int Lq = a.cu_q[b + 1] - q0;
    const int n_tiles_q = (Lq + M - 1) / M;
    if (rank >= n_tiles_q) return;
    const int qt = n_tiles_q - 1 - rank;
    const int Lk = a.cu_k[b + 1] - a.cu_k[b];
    const int P = Lk - Lq;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in SGPRs
    const int col = lane & 31;  // query row within the wave's 32
    const int hg = lane >> 5;   // lane half
    const int h = g * a.group + hs * HPW + w / kWavesPerHead;
    const int r0 = qt * M + (w % kWavesPerHead) * 32;  // first row of this wave
    const int my_row = r0 + col;
    const int rows_hi = min(qt * M + M, Lq);
    const int kv_end = min(Lk, P + rows_hi);  // keys any row of this workgroup can see
    const int n_tiles = (kv_end + kTileKeys - 1) / kTileKeys;
    // Packed mode (no block table): key j of sequence b is row cu_seqlens_k[b] + j of the
    // packed K/V tensors.
    const bool packed = a.block_tables == nullptr;
    const int32_t *table = packed ? nullptr : a.block_tables + (int64_t)b * a.bt_width;

    // This wave's 32 query rows of head h, copied HBM -> LDS 4 rows per instruction (lane i:
    // row 4j + i/16, chunk position i%16, K's swizzle), so every load covers whole rows. Rows
    // past the sequence's end repeat its last row (their outputs are not stored).
    uint8_t *q_slot = w < 2 ? k_lds[1] + w * kQWaveBytes
                    : w < 4 ? v_lds[1] + (w - 2) * kQWaveBytes
                            : q_lds_hi + (w - 4) * kQWaveBytes;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = 4 * j + (lane >> 4);
        const int row = min(r0 + r, Lq - 1);
        const uint16_t *src = a.q + ((int64_t)(q0 + row) * a.num_heads + h) * kHeadDim +
                              8 * k_chunk_pos(r, lane & 15);
        copy16_to_lds(src, q_slot + 4 * j * kRowBytes);
    }
    bf16x8 qreg[8];  // Q^T fragments, read from q_slot once the copies have landed

    // Block ids of the keys this workgroup reads, staged in LDS so that no copy address waits
    // on a global load (the host guarantees they fit: ceil(max_seqlen_k / block_size) <=
    // kTableSlots).
    const int k_first = a.cu_k[b];
    if (!packed) {
        const int n_blocks = a.bs_shift >= 0 ? (kv_end + a.block_size - 1) >> a.bs_shift
                                             : (kv_end + a.block_size - 1) / a.block_size;
        for (int i = tid; i < n_blocks; i += kWaves * 64) tbl[i] = table[i];
    }
    auto key_row_staged = [&](int j) -> int64_t {
        if (packed) return (int64_t)k_first + j;
        int lb, off;
        if (a.bs_shift >= 0) {
            lb = j >> a.bs_shift;
            off = j & (a.block_size - 1);
        } else {
            lb = j / a.block_size;
            off = j - lb * a.block_size;
        }
        return (int64_t)tbl[lb] * a.block_size + off;
    };
    __syncthreads();

    // ---- HBM -> LDS copy of the tile at key0 into stage st ----
    // Wave w, instruction j moves tile rows 16w + 4j .. +3 (1 KiB, contiguous in LDS); lane i
    // lands at 16 i: row 16w + 4j + i/16, chunk position i%16, i.e. logical chunk
    // position ^ swizzle(row) of that row.
    constexpr int kRowsPerWave = kTileKeys / kWaves;
    constexpr int kCopyGroups = kRowsPerWave / 4;
    // Whole-block tiles: lane byte offsets from the tile's first pool row, fixed for the loop.
    uint32_t koff[kCopyGroups], voff[kCopyGroups];
#pragma unroll
    for (int j = 0; j < kCopyGroups; ++j) {
        const int r = kRowsPerWave * w + 4 * j + (lane >> 4);
        koff[j] = (uint32_t)(r * a.k_row_stride * 2) + 16 * k_chunk_pos(r, lane & 15);
        voff[j] = (uint32_t)(r * a.v_row_stride * 2) + 16 * v_chunk_pos(r, lane & 15);
    }
    // Whole-block tiles (a multiple-of-64 block size, or packed rows) that end inside the keys
    // take the fast copy: one block id per tile gives the tile's first pool row, and each lane
    // adds its fixed offset. The block id comes from the LDS table one tile ahead (read while
    // the current tile is computed), so the copy issue never waits on an LDS round trip; K and
    // V share it.
    auto fast_tile = [&](int key0) {
        return NV_PREFILL_FASTCOPY && (packed || a.tile_in_block) && key0 + kTileKeys <= kv_end;
    };
    auto tile_block = [&](int key0) -> int {  // block id of a tile's first key (paged mode)
        if (packed) return 0;
        return tbl[a.bs_shift >= 0 ? key0 >> a.bs_shift : key0 / a.block_size];
    };
    auto copy_fast = [&](int64_t row0, uint8_t *dst, const uint16_t *pool, const uint32_t *offs,
                         int64_t row_stride) {
        const uint16_t *base = pool + row0 * row_stride + (int64_t)g * kHeadDim;
#pragma unroll
        for (int j = 0; j < kCopyGroups; ++j)
            copy16_to_lds_sbase(base, offs[j], dst + (kRowsPerWave * w + 4 * j) * kRowBytes);
    };
    // Any other tile: each lane looks up its own key's row; keys past the end re-read the last
    // valid key (masked later).
    auto copy_rows = [&](int key0, uint8_t *dst, const uint16_t *pool, bool is_v) {
        const int64_t row_stride = is_v ? a.v_row_stride : a.k_row_stride;
        const int pos = lane & 15;
#pragma unroll
        for (int j = 0; j < kCopyGroups; ++j) {
            const int r = kRowsPerWave * w + 4 * j + (lane >> 4);
            const int key = min(key0 + r, kv_end - 1);
            const uint16_t *src = pool + key_row_staged(key) * row_stride + g * kHeadDim;
            const int c = is_v ? v_chunk_pos(r, pos) : k_chunk_pos(r, pos);
            copy16_to_lds(src + 8 * c, dst + (kRowsPerWave * w + 4 * j) * kRowBytes);
        }
    };
    // K and V of tile t into stage st; blk: the tile's block id (fast tiles, paged mode).
    auto copy_tile = [&](int t, int st, int blk) {
        const int key0 = t * kTileKeys;
        uint8_t *kd = k_lds[st];
        uint8_t *vd = v_lds[st];
        if (fast_tile(key0)) {
            int64_t row0;
            if (packed) {
                row0 = (int64_t)k_first + key0;
            } else {
                const int off0 = a.bs_shift >= 0 ? (key0 & (a.block_size - 1))
                                                 : key0 - (key0 / a.block_size) * a.block_size;
                row0 = (int64_t)__builtin_amdgcn_readfirstlane(blk) * a.block_size + off0;
            }
            copy_fast(row0, kd, a.k_cache, koff, a.k_row_stride);
            copy_fast(row0, vd, a.v_cache, voff, a.v_row_stride);
            return;
        }
        copy_rows(key0, kd, a.k_cache, false);
        copy_rows(key0, vd, a.v_cache, true);
    };

    // ---- S^T = K Q^T for the tile in LDS at Ks: two 32-key blocks ----
    auto scores = [&](const uint8_t *Ks, f32x16 (&sc)[2]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) sc[kb][i] = 0.f;
        // K fragments are read NV_PREFILL_KPF dim-steps ahead of the products that use them.
        bf16x8 kf[8][2];
        auto load_k = [&](int kt) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int r = kb * 32 + col;
                kf[kt][kb] = *reinterpret_cast<const bf16x8 *>(
                    Ks + r * kRowBytes + 16 * k_chunk_pos(r, 2 * kt + hg));
            }
        };
#pragma unroll
        for (int kt = 0; kt < NV_PREFILL_KPF; ++kt) load_k(kt);
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) {
            if (kt + NV_PREFILL_KPF < 8) load_k(kt + NV_PREFILL_KPF);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kt][kb], qreg[kt], sc[kb], 0,
                                                                 0, 0);
        }
#if NV_PREFILL_SGB
        // Keep that order in the instruction schedule: the first reads, then two products and
        // the next two reads per dim-step, then the last products.
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * NV_PREFILL_KPF, 0);
#pragma unroll
        for (int i = 0; i < 8 - NV_PREFILL_KPF; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * NV_PREFILL_KPF, 0);
#endif
    };

    f32x16 o[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
    float m_run = -INFINITY;  // running max of this lane's row (raw score units), may lag
    float l_part = 0.f;       // this lane's share of the row sum

    // ---- mask (only tiles the diagonal or the key end cuts), row max, rare rescale ----
    // Row i of the wave sees keys < P + r0 + i + 1; the whole tile is visible to every row of
    // the wave when its last key is <= P + r0 (and below Lk).
    auto mask_and_max = [&](int t, f32x16 (&sc)[2]) {
        const int key0 = t * kTileKeys;
        if (key0 + kTileKeys - 1 > P + r0 || key0 + kTileKeys > Lk) {
            const int vis_end = min(Lk, P + my_row + 1);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int j = key0 + kb * 32 + 8 * (i >> 2) + 4 * hg + (i & 3);
                    if (j >= vis_end) sc[kb][i] = -INFINITY;
                }
        }
        float tmax = sc[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sc[kb][i]);
        tmax = halves_max(tmax);
        // Rescale only when some row's max grew by more than the slack: until then the stale
        // max keeps every probability below 2^slack, far from fp32/bf16 overflow, and the
        // result is unchanged because the max cancels between O and l. The first tile always
        // rescales (m_run = -inf; key 0 is visible to every row, so tmax is finite).
        if (__any(tmax > m_run + a.rescale_slack)) {
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = fast_exp2((m_run - m_new) * a.scale_log2);  // 0 on the first tile
            l_part *= alpha;
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[d][i] *= alpha;
            m_run = m_new;
        }
    };

    // ---- P = exp2(scale (S - m)) in bf16; word 4u + e holds keys of P.V step u ----
    auto probs = [&](f32x16 (&sc)[2], uint32_t (&pw)[16]) {
        const float msc = m_run * a.scale_log2;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int kb = u >> 1, i = 8 * (u & 1) + 2 * e;
                pw[4 * u + e] = pack_bf16(fast_exp2(fmaf(sc[kb][i], a.scale_log2, -msc)),
                                          fast_exp2(fmaf(sc[kb][i + 1], a.scale_log2, -msc)));
            }
    };

    // ---- O^T += V^T P^T for the tile in LDS at Vs, 16 keys per MFMA step; row sums ----
    // V^T operand of lane (group vj, lane vt): dim 32 d + 16 (vj & 1) + vt, keys
    // 16u + 4hg + {0..3} (first read) and 16u + 8 + 4hg + {0..3} (second read); the read
    // address of lane vt is row 16u + 4hg + vt/4 (+8), dims 16 (vj & 1) + 4 (vt%4) .. +3.
    const int vt = lane & 15, vj = lane >> 4;
    // V^T fragments of P.V step u for the four 32-dim blocks.
    auto load_v = [&](const uint8_t *Vs, int u, bf16x8 (&vf)[4]) {
        const int ra = 16 * u + 4 * hg + (vt >> 2), rb = ra + 8;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int dim = 32 * d + 16 * (vj & 1) + 4 * (vt & 3);
            const int ca = v_chunk_pos(ra, dim >> 3), cb = v_chunk_pos(rb, dim >> 3);
            const bf16x4v va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (NV_LDS bf16x4v *)(Vs + ra * kRowBytes + 16 * ca + 2 * (dim & 7)));
            const bf16x4v vb = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (NV_LDS bf16x4v *)(Vs + rb * kRowBytes + 16 * cb + 2 * (dim & 7)));
            vf[d] = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };
    // vf0: the fragments of step 0, read by the caller ahead of time.
    auto pv = [&](const uint8_t *Vs, const uint32_t (&pw)[16], bf16x8 (&vf0)[4]) {
        bf16x8 vf[4][4];
#pragma unroll
        for (int d = 0; d < 4; ++d) vf[0][d] = vf0[d];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (u + 1 < 4) load_v(Vs, u + 1, vf[u + 1]);
            const u32x4 pu = {pw[4 * u], pw[4 * u + 1], pw[4 * u + 2], pw[4 * u + 3]};
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pu);
#pragma unroll
            for (int d = 0; d < 4; ++d)
                o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[u][d], pb, o[d], 0, 0, 0);
        }
        // Row sums of exactly the bf16 probabilities that multiplied V, in four independent
        // chains (one dependent chain of 16 would expose its latency on every tile).
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 16; ++e)
            ps[e & 3] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pw[e]), ones, ps[e & 3], false);
        l_part += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    };

    f32x16 sc[2];
    // One tile per step: wait for its copies and publish it with a barrier (which also
    // retires the other stage), start copying the next tile into the other stage, then
    // scores, softmax and P.V of this one. The block id of the tile after next is read from
    // the LDS table during this step, so no copy waits on an LDS round trip.
    copy_tile(0, 0, fast_tile(0) ? tile_block(0) : 0);
    int blk_next = n_tiles > 1 && fast_tile(kTileKeys) ? tile_block(kTileKeys) : 0;
    // Q^T as the B operand: lane holds query row `col`, dims 16t + 8hg .. +8 for step t. The
    // query copies are this wave's oldest loads: wait until only the first tile's remain.
    wait_copies<2 * kCopyGroups>();
#pragma unroll
    for (int t = 0; t < 8; ++t)
        qreg[t] = *reinterpret_cast<const bf16x8 *>(q_slot + col * kRowBytes +
                                                    16 * k_chunk_pos(col, 2 * t + hg));
    auto step = [&](int t, auto stage) {
        constexpr int st = decltype(stage)::value;
        wait_copies_and_barrier<0>();
        if (t + 1 < n_tiles) {
            copy_tile(t + 1, st ^ 1, blk_next);
            if (t + 2 < n_tiles && fast_tile((t + 2) * kTileKeys))
                blk_next = tile_block((t + 2) * kTileKeys);
        }
        scores(k_lds[st], sc);
        bf16x8 vf0[4];
        if (NV_PREFILL_VPF) load_v(v_lds[st], 0, vf0);
        mask_and_max(t, sc);
        uint32_t pw[16];
        probs(sc, pw);
        if (!NV_PREFILL_VPF) load_v(v_lds[st], 0, vf0);
        pv(v_lds[st], pw, vf0);
    };
    for (int t = 0; t < n_tiles; t += 2) {
        step(t, std::integral_constant<int, 0>{});
        if (t + 1 < n_tiles) step(t + 1, std::integral_constant<int, 1>{});
    }

    // ---- normalise and store: lane holds row `col`, dims 32d + 8(i/4) + 4hg + (i%4) ----
    // Lanes l and l + 32 hold the two 4-dim halves of the same 8-dim groups. One
    // v_permlane32_swap per word trades halves so that lane l ends with whole groups
    // 8 (2rp + 1) .. +7 and lane l + 32 with groups 8 (2rp) .. +7 (rp = 0, 1): 16-byte stores
    // instead of 8-byte ones.
    const float l_tot = halves_sum(l_part);
    const float inv = 1.f / l_tot;
    uint16_t *op = a.out + ((int64_t)(q0 + my_row) * a.num_heads + h) * kHeadDim;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int rp = 0; rp < 2; ++rp) {
            const int ra = 2 * rp, rb = 2 * rp + 1;
            const uint32_t a0 = pack_bf16(o[d][4 * ra] * inv, o[d][4 * ra + 1] * inv);
            const uint32_t a1 = pack_bf16(o[d][4 * ra + 2] * inv, o[d][4 * ra + 3] * inv);
            const uint32_t b0 = pack_bf16(o[d][4 * rb] * inv, o[d][4 * rb + 1] * inv);
            const uint32_t b1 = pack_bf16(o[d][4 * rb + 2] * inv, o[d][4 * rb + 3] * inv);
            // first result: lanes 0-31 keep b, lanes 32-63 get lanes 0-31's a;
            // second result: lanes 0-31 get lanes 32-63's b, lanes 32-63 keep a
            const auto s0 = __builtin_amdgcn_permlane32_swap(b0, a0, false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(b1, a1, false, false);
            const u32x4 pk = {s0[0], s1[0], s0[1], s1[1]};
            if (my_row < Lq)
                *reinterpret_cast<u32x4 *>(op + 32 * d + 8 * (hg ? ra : rb)) = pk;
        }
}

template <int HPW, int kWaves>
nv_status launch_prefill(PrefillArgs a, int batch, int max_seqlen_q, hipStream_t stream) {
    constexpr int M = 32 * kWaves / HPW;
    const int64_t n_qtiles = (max_seqlen_q + M - 1) / M;
    const int64_t groups = (int64_t)batch * a.num_kv_heads * (a.group / HPW);
    const int64_t groups_per_xcd = (groups + 7) / 8;
    const int64_t blocks = 8 * groups_per_xcd * n_qtiles;
    if (blocks == 0) return NV_OK;
    if (blocks > (int64_t)INT32_MAX) return NV_ERR_UNSUPPORTED;
    a.batch = batch;
    a.n_groups = (int32_t)groups;
    a.groups_per_xcd = (int32_t)groups_per_xcd;
    return launch(prefill_kernel<HPW, kWaves>, dim3((uint32_t)blocks), dim3(64 * kWaves), 0,
                  stream, a);
}

// 8-wave workgroups (twice the query rows per K/V tile) pay off when each row sees a long
// context: chunked or prefix-cached prefill. With two heads per workgroup, fresh prompts keep 4
// waves (more workgroups); with four heads, 8 waves hold only 64 rows per head, so they are
// taken for every prompt.
template <int HPW>
nv_status launch_prefill_sized(PrefillArgs a, int batch, int max_seqlen_q, int max_seqlen_k,
                               hipStream_t stream) {
    if (HPW == 4 || max_seqlen_k >= 2 * max_seqlen_q)
        return launch_prefill<HPW, 8>(a, batch, max_seqlen_q, stream);
    return launch_prefill<HPW, 4>(a, batch, max_seqlen_q, stream);
}

}  // namespace
}  // namespace nvp

namespace nvp {
namespace {

// Checks shared by the paged and packed entry points, then the launch.
nv_status prefill_checked(PrefillArgs a, int32_t max_seqlen_q, int32_t max_seqlen_k,
                          int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                          int32_t head_dim, float softmax_scale, hipStream_t stream) {
    if (batch < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_seqlen_q < 0 ||
        max_seqlen_k < 0)
        return NV_ERR_INVALID_ARG;
    if (num_heads % num_kv_heads != 0) return NV_ERR_INVALID_ARG;
    if (!(softmax_scale > 0.f) || softmax_scale == INFINITY) return NV_ERR_INVALID_ARG;
    if (max_seqlen_q > max_seqlen_k) return NV_ERR_INVALID_ARG;
    if (head_dim != kHeadDim) return NV_ERR_UNSUPPORTED;
    const int G = num_heads / num_kv_heads;
    if (G > 8) return NV_ERR_UNSUPPORTED;
    if (num_kv_heads > 65536) return NV_ERR_UNSUPPORTED;  // 32-bit in-tile byte offsets
    const int64_t min_stride = (int64_t)num_kv_heads * kHeadDim;
    if (a.k_row_stride < min_stride || a.v_row_stride < min_stride) return NV_ERR_INVALID_ARG;
    if (a.k_row_stride % 8 != 0 || a.v_row_stride % 8 != 0) return NV_ERR_INVALID_ARG;
    if ((int64_t)kTileKeys * (a.k_row_stride > a.v_row_stride ? a.k_row_stride : a.v_row_stride) *
            2 > (int64_t)UINT32_MAX)
        return NV_ERR_UNSUPPORTED;  // in-tile byte offsets are 32-bit
    if (batch == 0 || max_seqlen_q == 0) return NV_OK;
    if (!a.q || !a.k_cache || !a.v_cache || !a.cu_q || !a.cu_k || !a.out)
        return NV_ERR_INVALID_ARG;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = G;
    a.scale_log2 = softmax_scale * kLog2e;
    a.rescale_slack = NV_PREFILL_SLACK / a.scale_log2;
    a.batch = a.n_groups = a.groups_per_xcd = 0;
    if (G % 4 == 0) return launch_prefill_sized<4>(a, batch, max_seqlen_q, max_seqlen_k, stream);
    if (G % 2 == 0) return launch_prefill_sized<2>(a, batch, max_seqlen_q, max_seqlen_k, stream);
    return launch_prefill_sized<1>(a, batch, max_seqlen_q, max_seqlen_k, stream);
}

}  // namespace
}  // namespace nvp

extern "C" nv_status nv_attn_prefill_packed(const void *q, const void *k, int64_t k_row_stride,
                                            const void *v, int64_t v_row_stride,
                                            const int32_t *cu_seqlens_q,
                                            const int32_t *cu_seqlens_k, int32_t max_seqlen_q,
                                            int32_t max_seqlen_k, int32_t batch,
                                            int32_t num_heads, int32_t num_kv_heads,
                                            int32_t head_dim, float softmax_scale, void *out,
                                            hipStream_t stream) {
    using namespace nvp;
    PrefillArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.k_cache = static_cast<const uint16_t *>(k);
    a.v_cache = static_cast<const uint16_t *>(v);
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.block_tables = nullptr;
    a.out = static_cast<uint16_t *>(out);
    a.bs_shift = -1;
    a.k_row_stride = k_row_stride;
    a.v_row_stride = v_row_stride;
    return prefill_checked(a, max_seqlen_q, max_seqlen_k, batch, num_heads, num_kv_heads,
                           head_dim, softmax_scale, stream);
}

extern "C" nv_status nv_paged_attn_prefill(const void *q, const void *k_cache,
                                           const void *v_cache, const int32_t *cu_seqlens_q,
                                           const int32_t *cu_seqlens_k, int32_t max_seqlen_q,
                                           int32_t max_seqlen_k, const int32_t *block_tables,
                                           int32_t max_blocks_per_seq, int32_t batch,
                                           int32_t num_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           float softmax_scale, void *out, hipStream_t stream) {
    using namespace nvp;
    if (num_kv_heads <= 0 || head_dim <= 0) return NV_ERR_INVALID_ARG;
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    if (!block_tables)  // the engine's fresh-prompt path: contiguous packed K/V
        return nv_attn_prefill_packed(q, k_cache, row, v_cache, row, cu_seqlens_q, cu_seqlens_k,
                                      max_seqlen_q, max_seqlen_k, batch, num_heads,
                                      num_kv_heads, head_dim, softmax_scale, out, stream);
    if (block_size <= 0 || max_blocks_per_seq < 0 || max_seqlen_k < 0) return NV_ERR_INVALID_ARG;
    if ((int64_t)max_seqlen_k > (int64_t)max_blocks_per_seq * block_size)
        return NV_ERR_INVALID_ARG;
    if (((int64_t)max_seqlen_k + block_size - 1) / block_size > kTableSlots)
        return NV_ERR_UNSUPPORTED;  // the block-table prefix must fit the LDS staging area
    PrefillArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.k_cache = static_cast<const uint16_t *>(k_cache);
    a.v_cache = static_cast<const uint16_t *>(v_cache);
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.block_tables = block_tables;
    a.out = static_cast<uint16_t *>(out);
    a.bt_width = max_blocks_per_seq;
    a.block_size = block_size;
    a.bs_shift = (block_size & (block_size - 1)) == 0 ? __builtin_ctz((unsigned)block_size) : -1;
    a.tile_in_block = block_size % kTileKeys == 0;
    a.k_row_stride = a.v_row_stride = row;
    return prefill_checked(a, max_seqlen_q, max_seqlen_k, batch, num_heads, num_kv_heads,
                           head_dim, softmax_scale, stream);
}
