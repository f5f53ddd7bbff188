// Paged prefill attention: causal varlen attention of each sequence's new rows against its
// cached prefix plus its new keys, all read through its block table.
//
// Operation ("Nano-vLLM Field Guide", Step 10.3, prefill with block_table; Step 07.5 for the
// packing): sequence b has Lq new rows and Lk keys; new row i sees keys 0 .. (Lk - Lq) + i
// (the causal mask aligned to the bottom-right corner). out = softmax(scale q K^T) V per query
// head; query head h reads kv head h / G.
//
// gfx950 design (bf16 MFMA, fp32 accumulation, online softmax):
//  - A workgroup of 4 waves owns one kv head g, HPW query heads of its group and a tile of
//    M = 128 / HPW new rows; each wave owns 32 rows of one head. Every K/V tile staged in LDS
//    is therefore shared by all query heads the workgroup holds.
//  - K/V are walked in tiles of 64 keys, copied from HBM straight into LDS with
//    global_load_lds (16 bytes per lane, no staging registers) into two LDS stages: the next
//    tile streams in while the current one is multiplied; one barrier per tile. Each thread
//    looks up its own key's block in the table, so any block size works and padding entries
//    are never read (keys past the tile's end re-read the last valid key, then get masked).
//  - LDS rows are 256 bytes, unpadded; bank conflicts are avoided by XOR-swizzling the 16-byte
//    chunks of a row (K: chunk ^ (row % 16); V: chunk ^ 2 (row % 4)), applied on the global
//    side since the copy places lane i's 16 bytes at 16 i.
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
//    tiles the causal diagonal or the key end cuts; the output rescale is skipped when no row
//    max moved.
//  - Work items are ordered (sequence, kv head, head subgroup, q tile from last to first) and
//    remapped so consecutive items land on the same XCD: workgroups that read the same K/V
//    share that XCD's L2.
#include "nv_common.h"

#ifndef NV_PREFILL_WAVES
#define NV_PREFILL_WAVES 2  // register budget for this many waves per SIMD
#endif

namespace nvp {
namespace {

constexpr int kTileKeys = 64;
constexpr int kRowBytes = kHeadDim * 2;           // one key row of one kv head in LDS
constexpr int kTileBytes = kTileKeys * kRowBytes;  // 16 KiB

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4v;
#define NV_LDS __attribute__((address_space(3)))

// 16-byte chunk position of logical chunk c of tile row r in LDS.
__device__ __forceinline__ int k_chunk_pos(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int v_chunk_pos(int r, int c) { return c ^ ((r & 3) << 1); }

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
    int32_t n_qtiles;
    int32_t items;
    int32_t items_per_xcd;
    float scale_log2;
};

template <int HPW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NV_PREFILL_WAVES))) void prefill_kernel(PrefillArgs a) {
    constexpr int kWavesPerHead = 4 / HPW;
    constexpr int M = 32 * kWavesPerHead;  // rows per workgroup
    // Two stages of K and V tiles (row-major, swizzled): 64 KiB.
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2][2][kTileBytes];

    // XCD-aware remap: hardware hands consecutive workgroup ids to different XCDs; give each
    // XCD a contiguous range of work items.
    const int bid = blockIdx.x;
    const int item = (bid & 7) * a.items_per_xcd + (bid >> 3);
    if (item >= a.items) return;
    const int hsub_count = a.group / HPW;
    const int qt = a.n_qtiles - 1 - item % a.n_qtiles;
    int rest = item / a.n_qtiles;
    const int hs = rest % hsub_count;
    rest /= hsub_count;
    const int g = rest % a.num_kv_heads;
    const int b = rest / a.num_kv_heads;

    const int q0 = a.cu_q[b];
    const int Lq = a.cu_q[b + 1] - q0;
    if (qt * M >= Lq) return;
    const int Lk = a.cu_k[b + 1] - a.cu_k[b];
    const int P = Lk - Lq;

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int col = lane & 31;  // query row within the wave's 32
    const int hg = lane >> 5;   // lane half
    const int h = g * a.group + hs * HPW + w / kWavesPerHead;
    const int r0 = qt * M + (w % kWavesPerHead) * 32;  // first row of this wave
    const int my_row = r0 + col;
    const int rows_hi = min(qt * M + M, Lq);
    const int kv_end = min(Lk, P + rows_hi);  // keys any row of this workgroup can see
    const int n_tiles = (kv_end + kTileKeys - 1) / kTileKeys;
    const int32_t *table = a.block_tables + (int64_t)b * a.bt_width;
    const int64_t kv_row_stride = (int64_t)a.num_kv_heads * kHeadDim;

    // Q^T as the B operand: lane holds query row `col`, dims 16t + 8hg .. +8 for step t.
    bf16x8 qreg[8];
    {
        const uint16_t *qp = a.q + ((int64_t)(q0 + my_row) * a.num_heads + h) * kHeadDim + 8 * hg;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            u32x4 v = u32x4{0, 0, 0, 0};
            if (my_row < Lq) v = *reinterpret_cast<const u32x4 *>(qp + 16 * t);
            qreg[t] = __builtin_bit_cast(bf16x8, v);
        }
    }

    // ---- HBM -> LDS copy of the tile at key0 into stage st ----
    // Wave w, instruction j moves tile rows 16w + 4j .. +3 (1 KiB, contiguous in LDS); lane i
    // lands at 16 i: row 16w + 4j + i/16, chunk position i%16, i.e. logical chunk
    // position ^ swizzle(row) of that row.
    auto copy_tile = [&](int key0, int st) {
        const int pos = lane & 15;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * w + 4 * j + (lane >> 4);
            const int key = min(key0 + r, kv_end - 1);  // past the end: a valid row, masked later
            const int64_t row = key_row(table, key, a.block_size, a.bs_shift);
            const uint16_t *kg = a.k_cache + row * kv_row_stride + g * kHeadDim;
            const uint16_t *vg = a.v_cache + row * kv_row_stride + g * kHeadDim;
            NV_LDS void *kd = (NV_LDS void *)&lds[st][0][(16 * w + 4 * j) * kRowBytes];
            NV_LDS void *vd = (NV_LDS void *)&lds[st][1][(16 * w + 4 * j) * kRowBytes];
            __builtin_amdgcn_global_load_lds(kg + 8 * (pos ^ (r & 15)), kd, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(vg + 8 * (pos ^ ((r & 3) << 1)), vd, 16, 0, 0);
        }
    };

    f32x16 o[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
    float m_run = -INFINITY;  // running max of this lane's row, raw score units
    float l_part = 0.f;       // this lane's share of the row sum

    copy_tile(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    const int vt = lane & 15, vj = lane >> 4;  // lane in its 16-lane group, group index
    for (int t = 0; t < n_tiles; ++t) {
        const int st = t & 1;
        const int key0 = t * kTileKeys;
        if (t + 1 < n_tiles) copy_tile(key0 + kTileKeys, st ^ 1);  // streams in meanwhile
        const uint8_t *Ks = lds[st][0];
        const uint8_t *Vs = lds[st][1];

        // ---- S^T = K Q^T for two 32-key blocks ----
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
            const int r = kb * 32 + col;
#pragma unroll
            for (int kt = 0; kt < 8; ++kt) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(
                    Ks + r * kRowBytes + 16 * k_chunk_pos(r, 2 * kt + hg));
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[kt], s[kb], 0, 0, 0);
            }
        }

        // ---- mask (only tiles the diagonal or the key end cuts), online softmax ----
        // Row i of the wave sees keys < P + r0 + i + 1; the whole tile is visible to every
        // row of the wave when its last key is <= P + r0 (and below Lk).
        if (key0 + kTileKeys - 1 > P + r0 || key0 + kTileKeys > Lk) {
            const int vis_end = min(Lk, P + my_row + 1);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int j = key0 + kb * 32 + 8 * (i >> 2) + 4 * hg + (i & 3);
                    if (j >= vis_end) s[kb][i] = -INFINITY;
                }
        }
        float tmax = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[kb][i]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);  // finite: key 0 is visible to every row
        if (__any(m_new != m_run)) {  // rescale only when some row's max moved
            const float alpha = fast_exp2((m_run - m_new) * a.scale_log2);  // 0 on the first tile
            l_part *= alpha;
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[d][i] *= alpha;
            m_run = m_new;
        }
        const float msc = m_run * a.scale_log2;
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = fast_exp2(fmaf(s[kb][i], a.scale_log2, -msc));
                s[kb][i] = p;
                psum += p;
            }
        l_part += psum;

        // ---- O^T += V^T P^T, 16 keys per MFMA step ----
        // V^T operand of lane (group vj, lane vt): dim 32 d + 16 (vj & 1) + vt, keys
        // 16u + 4hg + {0..3} (first read) and 16u + 8 + 4hg + {0..3} (second read); the read
        // address of lane vt is row 16u + 4hg + vt/4 (+8), dims 16 (vj & 1) + 4 (vt%4) .. +3.
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int kb = u >> 1, ib = 8 * (u & 1);
            u32x4 pw;
#pragma unroll
            for (int e = 0; e < 4; ++e) pw[e] = pack_bf16(s[kb][ib + 2 * e], s[kb][ib + 2 * e + 1]);
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
            const int ra = 16 * u + 4 * hg + (vt >> 2), rb = ra + 8;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int dim = 32 * d + 16 * (vj & 1) + 4 * (vt & 3);
                const int ca = v_chunk_pos(ra, dim >> 3), cb = v_chunk_pos(rb, dim >> 3);
                const bf16x4v va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (NV_LDS bf16x4v *)(Vs + ra * kRowBytes + 16 * ca + 2 * (dim & 7)));
                const bf16x4v vb = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (NV_LDS bf16x4v *)(Vs + rb * kRowBytes + 16 * cb + 2 * (dim & 7)));
                const bf16x8 vw = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
                o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vw, pb, o[d], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);  // this thread's copies of the next tile have landed
        __syncthreads();
    }

    // ---- normalise and store: lane holds row `col`, dims 32d + 8(i/4) + 4hg + (i%4) ----
    const float l_tot = l_part + __shfl_xor(l_part, 32);
    if (my_row < Lq) {
        const float inv = 1.f / l_tot;
        uint16_t *op = a.out + ((int64_t)(q0 + my_row) * a.num_heads + h) * kHeadDim + 4 * hg;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                u32x2 pk;
                pk[0] = pack_bf16(o[d][4 * r] * inv, o[d][4 * r + 1] * inv);
                pk[1] = pack_bf16(o[d][4 * r + 2] * inv, o[d][4 * r + 3] * inv);
                *reinterpret_cast<u32x2 *>(op + 32 * d + 8 * r) = pk;
            }
    }
}

template <int HPW>
nv_status launch_prefill(PrefillArgs a, int batch, int max_seqlen_q, hipStream_t stream) {
    constexpr int M = 128 / HPW;
    a.n_qtiles = (max_seqlen_q + M - 1) / M;
    const int64_t items = (int64_t)batch * a.num_kv_heads * (a.group / HPW) * a.n_qtiles;
    if (items == 0) return NV_OK;
    if (items > (int64_t)INT32_MAX / 2) return NV_ERR_UNSUPPORTED;
    a.items = (int32_t)items;
    a.items_per_xcd = (int32_t)((items + 7) / 8);
    return launch(prefill_kernel<HPW>, dim3(8 * a.items_per_xcd), dim3(256), 0, stream, a);
}

}  // namespace
}  // namespace nvp

extern "C" nv_status nv_paged_attn_prefill(const void *q, const void *k_cache,
                                           const void *v_cache, const int32_t *cu_seqlens_q,
                                           const int32_t *cu_seqlens_k, int32_t max_seqlen_q,
                                           int32_t max_seqlen_k, const int32_t *block_tables,
                                           int32_t max_blocks_per_seq, int32_t batch,
                                           int32_t num_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           float softmax_scale, void *out, hipStream_t stream) {
    using namespace nvp;
    if (batch < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        max_seqlen_q < 0 || max_seqlen_k < 0 || max_blocks_per_seq < 0)
        return NV_ERR_INVALID_ARG;
    if (num_heads % num_kv_heads != 0) return NV_ERR_INVALID_ARG;
    if (!(softmax_scale > 0.f) || softmax_scale == INFINITY) return NV_ERR_INVALID_ARG;
    if (max_seqlen_q > max_seqlen_k) return NV_ERR_INVALID_ARG;
    if ((int64_t)max_seqlen_k > (int64_t)max_blocks_per_seq * block_size)
        return NV_ERR_INVALID_ARG;
    if (head_dim != kHeadDim) return NV_ERR_UNSUPPORTED;
    const int G = num_heads / num_kv_heads;
    if (G > 8) return NV_ERR_UNSUPPORTED;
    if (batch == 0 || max_seqlen_q == 0) return NV_OK;
    if (!block_tables) return NV_ERR_UNSUPPORTED;  // packed fresh-K/V mode not built
    if (!q || !k_cache || !v_cache || !cu_seqlens_q || !cu_seqlens_k || !out)
        return NV_ERR_INVALID_ARG;
    PrefillArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k_cache = static_cast<const uint16_t *>(k_cache);
    a.v_cache = static_cast<const uint16_t *>(v_cache);
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.block_tables = block_tables;
    a.out = static_cast<uint16_t *>(out);
    a.bt_width = max_blocks_per_seq;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = G;
    a.block_size = block_size;
    a.bs_shift = (block_size & (block_size - 1)) == 0 ? __builtin_ctz((unsigned)block_size) : -1;
    a.scale_log2 = softmax_scale * kLog2e;
    a.n_qtiles = a.items = a.items_per_xcd = 0;
    if (G % 2 == 0) return launch_prefill<2>(a, batch, max_seqlen_q, stream);
    return launch_prefill<1>(a, batch, max_seqlen_q, stream);
}
