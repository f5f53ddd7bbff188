// Paged decode attention: one query token per sequence against its whole cached context.
//
// Operation ("Nano-vLLM Field Guide", Step 10.3, decode with flash_attn_with_kvcache; Step
// 07.6 for context_lens): out[b, h] = softmax(scale * q[b, h] . K_b^T) V_b over the
// context_lens[b] keys of sequence b, read through its block table. Query head h reads kv head
// h / G (G = num_heads / num_kv_heads). A row with no keys (a padding row) outputs zeros.
//
// gfx950 design. Decode reads every K/V byte of the context once and does ~1 FMA per byte, so
// it is bound by HBM bandwidth. Work item = (sequence b, kv head g, split s of the key range);
// the G query heads of the group share every K/V load. A workgroup of 4 waves
//   1) streams the split's keys of kv head g: 16 lanes x 16 B cover one 256-byte key row, a
//      wave covers 4 keys per load; partial dot products are summed across the 16 lanes with
//      DPP row rotations and the scores (already in log2 units) go to LDS;
//   2) takes the exact max and sum of exp2 over the split's scores (no running rescale);
//   3) streams the same keys' values, each lane accumulating 8 output dims for all G heads,
//      then reduces over keys with two cross-lane swaps and an LDS sum over the 4 waves.
// A split's result is final when it is the sequence's only split; otherwise (max, sum,
// unnormalised output) goes to the workspace and a second kernel merges the splits with the
// log-sum-exp rule: out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, M = max_s m_s.
// The split size depends only on host-known launch parameters, so there is no device round
// trip.
#include "nv_common.h"

namespace nvp {
namespace {

constexpr int kMaxSplitKeys = 512;
constexpr int kMinSplitKeys = 64;
constexpr int kUnroll = 8;  // 16-byte loads in flight per lane per phase

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
    float scale_log2;  // softmax_scale * log2(e)
};

template <int G>
__global__ __launch_bounds__(256) void decode_partial_kernel(DecodeArgs a) {
    __shared__ float sc[G][kMaxSplitKeys];
    __shared__ float red[4][G][kHeadDim];
    __shared__ float stat[4][G];

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int L = a.context_lens[b];
    const int k0 = s * a.split_keys;
    if (k0 >= L) return;  // past this sequence's context (or a padding row)
    const int n = min(a.split_keys, L - k0);
    const int nsplit = (L + a.split_keys - 1) / a.split_keys;

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int sub = lane >> 4;  // which of the wave's 4 keys
    const int c = lane & 15;    // dims [8c, 8c + 8)
    const int Hkv = a.num_kv_heads;
    const int32_t *table = a.block_tables + (int64_t)b * a.bt_width;

    // q of the G heads, 8 dims per lane, pre-scaled into log2 units.
    float qf[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(
            a.q + ((int64_t)b * a.num_heads + g * G + h) * kHeadDim + 8 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qf[h][2 * i] = bf16lo(v[i]) * a.scale_log2;
            qf[h][2 * i + 1] = bf16hi(v[i]) * a.scale_log2;
        }
    }

    const uint16_t *kbase = a.k_cache + (int64_t)g * kHeadDim + 8 * c;
    const uint16_t *vbase = a.v_cache + (int64_t)g * kHeadDim + 8 * c;
    const int64_t row_stride = (int64_t)Hkv * kHeadDim;

    // Phase 1: scores.
    for (int base = 0; base < n; base += 16 * kUnroll) {
        u32x4 kv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int kk = base + 16 * u + 4 * w + sub;
            if (kk < n) {
                const int64_t row = key_row(table, k0 + kk, a.block_size, a.bs_shift);
                kv[u] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4 *>(kbase + row * row_stride));
            } else {
                kv[u] = u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int kk = base + 16 * u + 4 * w + sub;
            float kf[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                kf[2 * i] = bf16lo(kv[u][i]);
                kf[2 * i + 1] = bf16hi(kv[u][i]);
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float d = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) d = fmaf(qf[h][i], kf[i], d);
                d = row16_sum(d);
                if (c == 0 && kk < n) sc[h][kk] = d;
            }
        }
    }
    __syncthreads();

    // Phase 2: exact max and sum of exp2 over the split, per head.
    float mx[G], sm[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float m = -INFINITY;
        for (int i = tid; i < n; i += 256) m = fmaxf(m, sc[h][i]);
        m = wave_max(m);
        if (lane == 0) stat[w][h] = m;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h)
        mx[h] = fmaxf(fmaxf(stat[0][h], stat[1][h]), fmaxf(stat[2][h], stat[3][h]));
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float l = 0.f;
        for (int i = tid; i < n; i += 256) {
            const float p = fast_exp2(sc[h][i] - mx[h]);
            sc[h][i] = p;
            l += p;
        }
        l = wave_sum(l);
        if (lane == 0) stat[w][h] = l;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) sm[h] = (stat[0][h] + stat[1][h]) + (stat[2][h] + stat[3][h]);

    // Phase 3: weighted values.
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
    for (int base = 0; base < n; base += 16 * kUnroll) {
        u32x4 vv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int kk = base + 16 * u + 4 * w + sub;
            if (kk < n) {
                const int64_t row = key_row(table, k0 + kk, a.block_size, a.bs_shift);
                vv[u] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4 *>(vbase + row * row_stride));
            } else {
                vv[u] = u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int kk = base + 16 * u + 4 * w + sub;
            if (kk < n) {
                float vf[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    vf[2 * i] = bf16lo(vv[u][i]);
                    vf[2 * i + 1] = bf16hi(vv[u][i]);
                }
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float p = sc[h][kk];
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[h][i] = fmaf(p, vf[i], acc[h][i]);
                }
            }
        }
    }
    // Sum over the wave's 4 key slots (lanes c, c+16, c+32, c+48 hold the same dims).
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float x = acc[h][i];
            x += __shfl_xor(x, 16);
            x += __shfl_xor(x, 32);
            acc[h][i] = x;
        }
    if (sub == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int i = 0; i < 8; ++i) red[w][h][8 * c + i] = acc[h][i];
    }
    __syncthreads();

    for (int idx = tid; idx < G * kHeadDim; idx += 256) {
        const int h = idx / kHeadDim, e = idx % kHeadDim;
        const float o = (red[0][h][e] + red[1][h][e]) + (red[2][h][e] + red[3][h][e]);
        const int64_t bh = (int64_t)b * a.num_heads + g * G + h;
        if (nsplit == 1) {
            const float r = o / sm[h];
            a.out[bh * kHeadDim + e] = __builtin_bit_cast(uint16_t, (__bf16)r);
        } else {
            a.ws_o[(bh * a.max_splits + s) * kHeadDim + e] = o;
            if (e == 0) {
                a.ws_ml[(bh * a.max_splits + s) * 2] = mx[h];
                a.ws_ml[(bh * a.max_splits + s) * 2 + 1] = sm[h];
            }
        }
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
    if (nsplit == 1) return;  // the partial kernel wrote the final row
    const float *ml = a.ws_ml + bh * a.max_splits * 2;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[2 * s]);
    float num = 0.f, den = 0.f;
    for (int s = 0; s < nsplit; ++s) {
        const float w = fast_exp2(ml[2 * s] - M);
        den = fmaf(w, ml[2 * s + 1], den);
        num = fmaf(w, a.ws_o[(bh * a.max_splits + s) * kHeadDim + e], num);
    }
    a.out[bh * kHeadDim + e] = __builtin_bit_cast(uint16_t, (__bf16)(num / den));
}

template <int G>
nv_status launch_decode(const DecodeArgs &a, int batch, hipStream_t stream) {
    nv_status st = launch(decode_partial_kernel<G>,
                          dim3(a.max_splits, a.num_kv_heads, batch), dim3(256), 0, stream, a);
    if (st != NV_OK) return st;
    return launch(decode_combine_kernel, dim3(a.num_heads, batch), dim3(kHeadDim), 0, stream, a);
}

int64_t max_context(int32_t max_blocks_per_seq, int32_t block_size) {
    return (int64_t)max_blocks_per_seq * block_size;
}

}  // namespace
}  // namespace nvp

extern "C" int32_t nv_paged_attn_decode_split_keys(int32_t batch, int32_t num_kv_heads,
                                                   int32_t max_blocks_per_seq,
                                                   int32_t block_size) {
    using namespace nvp;
    // Largest split (fewest partials) that still yields >= 2048 work items over the padded
    // context, so small batches spread over all 256 CUs.
    const int64_t ctx = max_context(max_blocks_per_seq, block_size);
    int32_t S = kMaxSplitKeys;
    while (S > kMinSplitKeys &&
           (int64_t)batch * num_kv_heads * ((ctx + S - 1) / S) < 2048)
        S /= 2;
    return S;
}

extern "C" size_t nv_paged_attn_decode_workspace_size(int32_t batch, int32_t num_heads,
                                                      int32_t num_kv_heads, int32_t head_dim,
                                                      int32_t max_blocks_per_seq,
                                                      int32_t block_size) {
    using namespace nvp;
    if (batch <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        max_blocks_per_seq <= 0 || block_size <= 0)
        return 0;
    const int32_t S = nv_paged_attn_decode_split_keys(batch, num_kv_heads, max_blocks_per_seq,
                                                      block_size);
    const int64_t splits = (max_context(max_blocks_per_seq, block_size) + S - 1) / S;
    if (splits <= 1) return 0;
    const size_t rows = (size_t)batch * num_heads * splits;
    const size_t ml = (rows * 2 * sizeof(float) + 255) / 256 * 256;
    return ml + rows * head_dim * sizeof(float);
}

extern "C" nv_status nv_paged_attn_decode(const void *q, const void *k_cache,
                                          const void *v_cache, const int32_t *context_lens,
                                          const int32_t *block_tables,
                                          int32_t max_blocks_per_seq, int32_t batch,
                                          int32_t num_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t block_size,
                                          float softmax_scale, void *workspace,
                                          size_t workspace_bytes, void *out,
                                          hipStream_t stream) {
    using namespace nvp;
    if (batch < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        max_blocks_per_seq < 0)
        return NV_ERR_INVALID_ARG;
    if (num_heads % num_kv_heads != 0) return NV_ERR_INVALID_ARG;
    if (head_dim != kHeadDim) return NV_ERR_UNSUPPORTED;
    const int G = num_heads / num_kv_heads;
    if (G > 8) return NV_ERR_UNSUPPORTED;
    if (batch == 0) return NV_OK;
    if (!q || !k_cache || !v_cache || !context_lens || !out) return NV_ERR_INVALID_ARG;
    if (max_blocks_per_seq == 0) {
        // No sequence can hold a key: every row is a padding row; only the zeros are written.
        DecodeArgs z{};
        z.context_lens = context_lens;
        z.out = static_cast<uint16_t *>(out);
        z.num_heads = num_heads;
        z.split_keys = kMaxSplitKeys;
        z.max_splits = 1;
        if (batch > 65535) return NV_ERR_UNSUPPORTED;
        return launch(decode_combine_kernel, dim3(num_heads, batch), dim3(kHeadDim), 0, stream, z);
    }
    if (!block_tables) return NV_ERR_INVALID_ARG;
    const size_t need = nv_paged_attn_decode_workspace_size(batch, num_heads, num_kv_heads,
                                                            head_dim, max_blocks_per_seq,
                                                            block_size);
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
    a.split_keys = nv_paged_attn_decode_split_keys(batch, num_kv_heads, max_blocks_per_seq,
                                                   block_size);
    const int64_t splits = (max_context(max_blocks_per_seq, block_size) + a.split_keys - 1) /
                           a.split_keys;
    if (splits > 65535 || batch > 65535 || num_kv_heads > 65535) return NV_ERR_UNSUPPORTED;
    a.max_splits = (int32_t)splits;
    const size_t rows = (size_t)batch * num_heads * splits;
    const size_t ml_bytes = (rows * 2 * sizeof(float) + 255) / 256 * 256;
    a.ws_ml = need ? static_cast<float *>(workspace) : nullptr;
    a.ws_o = need ? reinterpret_cast<float *>(static_cast<char *>(workspace) + ml_bytes)
                  : nullptr;
    a.scale_log2 = softmax_scale * kLog2e;
    switch (G) {
        case 1: return launch_decode<1>(a, batch, stream);
        case 2: return launch_decode<2>(a, batch, stream);
        case 3: return launch_decode<3>(a, batch, stream);
        case 4: return launch_decode<4>(a, batch, stream);
        case 5: return launch_decode<5>(a, batch, stream);
        case 6: return launch_decode<6>(a, batch, stream);
        case 7: return launch_decode<7>(a, batch, stream);
        default: return launch_decode<8>(a, batch, stream);
    }
}
