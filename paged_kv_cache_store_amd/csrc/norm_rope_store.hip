// Fused per-head RMSNorm + rotary embedding of q and k, and the K/V store.
//
// Operation ("Nano-vLLM Field Guide", Step 9.5, Qwen3Attention.forward: q_norm and k_norm on
// every head of the fused projection output, rotary_emb on q and k at each token's position,
// then store_kvcache; Step 10.4, layernorm.py, and Step 10.5, rotary_embedding.py, for the two
// formulas; Step 10.3 for the store and its -1 slots):
//   RMSNorm of a head x (d = 128 values): n = bf16(x * rsqrt(mean(x^2) + eps)),
//                                         y = bf16(n * w)
//   rotary embedding, halves y1 = y[0:64], y2 = y[64:128], frequency i < 64 at position p:
//                                         z1 = bf16(y1 cos - y2 sin), z2 = bf16(y2 cos + y1 sin)
//   with cos/sin read from the caller's fp32 table row p (cos of the 64 frequencies, then sin).
// q heads go to q_out; k heads to k_out (optional) and to the K pool at the token's slot; v
// heads are copied to the V pool unchanged. A slot of -1 stores nothing.
//
// gfx950 design: the op streams each projection row once and writes it once (HBM-bound). One
// 16-lane group owns one (token, head) item and 8 consecutive dims per lane (16-byte loads and
// stores); the head's sum of squares is a DPP sum over the group's 16 lanes, and the rotation
// partner of dims 8j .. 8j+7 (first half) is lane j+8 of the same group (second half), reached
// with one DPP rotate of the 16-lane row. Products and sums of the rotation are rounded one by
// one (no fused multiply-add), as the formula is written.
#include "nv_common.h"

namespace nvp {
namespace {

struct NormRopeArgs {
    const uint16_t *qkv;
    int64_t qkv_row_stride;
    const int64_t *positions;
    const uint16_t *q_w;
    const uint16_t *k_w;
    const float *cos_sin;
    int64_t max_position;
    float eps;
    uint16_t *q_out;
    uint16_t *k_out;
    uint16_t *k_cache;
    uint16_t *v_cache;
    const int32_t *slot_mapping;
    int64_t num_tokens;
    int32_t num_heads;
    int32_t num_kv_heads;
    int64_t items;  // num_tokens * (num_heads + 2 num_kv_heads)
};

__device__ __forceinline__ float dpp_ror8(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
}

__device__ __forceinline__ float round_bf16f(float x) { return (float)(__bf16)x; }

__global__ __launch_bounds__(256) void norm_rope_store_kernel(NormRopeArgs a) {
#pragma clang fp contract(off)  // products and sums rounded one by one, as written
    const int lane = threadIdx.x & 15;              // lane in the 16-lane group
    const int64_t item = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    if (item >= a.items) return;                    // whole 16-lane groups leave together
    const int heads = a.num_heads + 2 * a.num_kv_heads;
    const int64_t t = item / heads;
    const int h = (int)(item - t * heads);
    const int32_t slot = a.slot_mapping[t];
    const int64_t row_kv = (int64_t)a.num_kv_heads * kHeadDim;
    const uint16_t *src = a.qkv + t * a.qkv_row_stride + (int64_t)h * kHeadDim + 8 * lane;
    const u32x4 raw = *reinterpret_cast<const u32x4 *>(src);

    if (h >= a.num_heads + a.num_kv_heads) {        // v head: bit copy to the V pool
        if (slot >= 0) {
            const int vh = h - a.num_heads - a.num_kv_heads;
            *reinterpret_cast<u32x4 *>(a.v_cache + (int64_t)slot * row_kv + vh * kHeadDim +
                                       8 * lane) = raw;
        }
        return;
    }
    const bool is_q = h < a.num_heads;
    const u32x4 wraw =
        *reinterpret_cast<const u32x4 *>((is_q ? a.q_w : a.k_w) + 8 * lane);

    float x[8], w[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf16lo(raw[e]);
        x[2 * e + 1] = bf16hi(raw[e]);
        w[2 * e] = bf16lo(wraw[e]);
        w[2 * e + 1] = bf16hi(wraw[e]);
    }
    // RMSNorm over the head's 128 values (16 lanes x 8).
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    ss = row16_sum(ss);
    const float var = ss * (1.0f / kHeadDim);
    const float r = __fdiv_rn(1.0f, __fsqrt_rn(var + a.eps));
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = round_bf16f(round_bf16f(x[e] * r) * w[e]);

    // Rotary embedding: lane j < 8 holds first-half dims 8j.., lane j + 8 the matching
    // second-half dims; positions outside the table are clamped into it (a precondition
    // violation that must not read out of bounds).
    int64_t p = a.positions[t];
    p = p < 0 ? 0 : (p >= a.max_position ? a.max_position - 1 : p);
    const int i0 = 8 * (lane & 7);                  // first frequency of this lane
    const float *cs = a.cos_sin + p * kHeadDim;
    const f32x4 c0 = *reinterpret_cast<const f32x4 *>(cs + i0);
    const f32x4 c1 = *reinterpret_cast<const f32x4 *>(cs + i0 + 4);
    const f32x4 s0 = *reinterpret_cast<const f32x4 *>(cs + kHeadDim / 2 + i0);
    const f32x4 s1 = *reinterpret_cast<const f32x4 *>(cs + kHeadDim / 2 + i0 + 4);
    const bool first = lane < 8;
    uint32_t out[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        float z[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int k = e + u;
            const float c = k < 4 ? c0[k] : c1[k - 4];
            const float s = k < 4 ? s0[k] : s1[k - 4];
            const float other = dpp_ror8(y[k]);     // the partner half's value
            const float yc = y[k] * c, os = other * s;
            z[u] = first ? yc - os : yc + os;
        }
        out[e / 2] = pack_bf16(z[0], z[1]);
    }
    const u32x4 ov = {out[0], out[1], out[2], out[3]};
    if (is_q) {
        *reinterpret_cast<u32x4 *>(a.q_out + (t * a.num_heads + h) * kHeadDim + 8 * lane) = ov;
        return;
    }
    const int kh = h - a.num_heads;
    if (a.k_out)
        *reinterpret_cast<u32x4 *>(a.k_out + (t * a.num_kv_heads + kh) * kHeadDim + 8 * lane) =
            ov;
    if (slot >= 0)
        *reinterpret_cast<u32x4 *>(a.k_cache + (int64_t)slot * row_kv + kh * kHeadDim +
                                   8 * lane) = ov;
}

}  // namespace
}  // namespace nvp

extern "C" nv_status nv_qk_norm_rope_store(const void *qkv, int64_t qkv_row_stride,
                                           const int64_t *positions, const void *q_norm_weight,
                                           const void *k_norm_weight, const float *cos_sin_cache,
                                           int64_t max_position, float eps, void *q_out,
                                           void *k_out, void *k_cache, void *v_cache,
                                           const int32_t *slot_mapping, int64_t num_tokens,
                                           int32_t num_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int64_t num_slots,
                                           hipStream_t stream) {
    using namespace nvp;
    if (num_tokens < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        max_position <= 0 || num_slots < 0)
        return NV_ERR_INVALID_ARG;
    if (num_heads % num_kv_heads != 0) return NV_ERR_INVALID_ARG;
    if (head_dim != kHeadDim) return NV_ERR_UNSUPPORTED;
    if (!(eps >= 0.f) || eps == INFINITY) return NV_ERR_INVALID_ARG;
    const int64_t heads = (int64_t)num_heads + 2 * num_kv_heads;
    if (qkv_row_stride < heads * head_dim || qkv_row_stride % 8 != 0) return NV_ERR_INVALID_ARG;
    if (num_tokens == 0) return NV_OK;
    if (!qkv || !positions || !q_norm_weight || !k_norm_weight || !cos_sin_cache || !q_out ||
        !k_cache || !v_cache || !slot_mapping)
        return NV_ERR_INVALID_ARG;
    // Every lane moves whole 16-byte vectors of these buffers (rows are 256-byte head slices,
    // the table rows 512 bytes): their bases must be 16-byte aligned.
    const auto a16 = [](const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
    if (!a16(qkv) || !a16(q_norm_weight) || !a16(k_norm_weight) || !a16(cos_sin_cache) ||
        !a16(q_out) || (k_out && !a16(k_out)) || !a16(k_cache) || !a16(v_cache))
        return NV_ERR_INVALID_ARG;
    NormRopeArgs a;
    a.qkv = static_cast<const uint16_t *>(qkv);
    a.qkv_row_stride = qkv_row_stride;
    a.positions = positions;
    a.q_w = static_cast<const uint16_t *>(q_norm_weight);
    a.k_w = static_cast<const uint16_t *>(k_norm_weight);
    a.cos_sin = cos_sin_cache;
    a.max_position = max_position;
    a.eps = eps;
    a.q_out = static_cast<uint16_t *>(q_out);
    a.k_out = static_cast<uint16_t *>(k_out);
    a.k_cache = static_cast<uint16_t *>(k_cache);
    a.v_cache = static_cast<uint16_t *>(v_cache);
    a.slot_mapping = slot_mapping;
    a.num_tokens = num_tokens;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.items = num_tokens * heads;
    const int64_t blocks = (a.items + 15) / 16;
    if (blocks > (int64_t)INT32_MAX) return NV_ERR_UNSUPPORTED;
    return launch(norm_rope_store_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, a);
}
