// K/V store: scatter this step's new key and value rows into the block-paged pools.
//
// Operation ("Nano-vLLM Field Guide", Step 10.3, the store kernel and its wrapper): row i of
// key and of value is copied bit for bit into row slot_mapping[i] of the flattened key pool and
// value pool; a slot of -1 (a padding row) writes nothing.
//
// gfx950 mapping: one 64-lane wave per token row, so the slot is read once per wave and the
// -1 test is a wave-uniform branch. Each lane moves 16-byte vectors; a row of D bf16 values is
// D / 8 vectors, so the wave's accesses to one row are contiguous and fully coalesced. Four
// waves per workgroup. Unaligned strides fall back to 4- or 2-byte vectors.
#include "nv_common.h"

namespace nvp {
namespace {

template <typename Vec>
__global__ __launch_bounds__(256) void store_kvcache_kernel(
    const Vec *__restrict__ key, int64_t key_stride_vec, const Vec *__restrict__ value,
    int64_t value_stride_vec, Vec *__restrict__ k_cache, Vec *__restrict__ v_cache,
    const int32_t *__restrict__ slot_mapping, int64_t num_tokens, int32_t row_vecs) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= num_tokens) return;
    const int lane = threadIdx.x & 63;
    const int64_t slot = __builtin_amdgcn_readfirstlane(slot_mapping[row]);
    if (slot == -1) return;
    const Vec *ks = key + row * key_stride_vec;
    const Vec *vs = value + row * value_stride_vec;
    Vec *kd = k_cache + slot * row_vecs;
    Vec *vd = v_cache + slot * row_vecs;
    for (int c = lane; c < row_vecs; c += 64) {
        const Vec kv = __builtin_nontemporal_load(ks + c);
        const Vec vv = __builtin_nontemporal_load(vs + c);
        kd[c] = kv;
        vd[c] = vv;
    }
}

template <typename Vec>
nv_status launch_store(const void *key, int64_t key_row_stride, const void *value,
                       int64_t value_row_stride, void *k_cache, void *v_cache,
                       const int32_t *slot_mapping, int64_t num_tokens, int64_t row_elems,
                       hipStream_t stream) {
    constexpr int64_t per = sizeof(Vec) / 2;  // bf16 values per vector
    const int64_t blocks = (num_tokens + 3) / 4;
    if (blocks > INT32_MAX) return NV_ERR_INVALID_ARG;
    return launch(store_kvcache_kernel<Vec>, dim3((uint32_t)blocks), dim3(256), 0, stream,
                  static_cast<const Vec *>(key), key_row_stride / per,
                  static_cast<const Vec *>(value), value_row_stride / per,
                  static_cast<Vec *>(k_cache), static_cast<Vec *>(v_cache), slot_mapping,
                  num_tokens, (int32_t)(row_elems / per));
}

bool aligned(const void *p, int64_t stride_elems, int64_t bytes) {
    return (reinterpret_cast<uintptr_t>(p) % bytes) == 0 && ((stride_elems * 2) % bytes) == 0;
}

}  // namespace
}  // namespace nvp

extern "C" nv_status nv_store_kvcache(const void *key, int64_t key_row_stride,
                                      const void *value, int64_t value_row_stride,
                                      void *k_cache, void *v_cache,
                                      const int32_t *slot_mapping, int64_t num_tokens,
                                      int32_t num_kv_heads, int32_t head_dim, int64_t num_slots,
                                      hipStream_t stream) {
    using namespace nvp;
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_slots < 0)
        return NV_ERR_INVALID_ARG;
    const int64_t D = (int64_t)num_kv_heads * head_dim;
    if (key_row_stride < D || value_row_stride < D) return NV_ERR_INVALID_ARG;
    if (num_tokens == 0) return NV_OK;
    if (!key || !value || !k_cache || !v_cache || !slot_mapping) return NV_ERR_INVALID_ARG;
    if (D / 8 > INT32_MAX) return NV_ERR_UNSUPPORTED;
    const bool v16 = D % 8 == 0 && aligned(key, key_row_stride, 16) &&
                     aligned(value, value_row_stride, 16) && aligned(k_cache, D, 16) &&
                     aligned(v_cache, D, 16);
    if (v16)
        return launch_store<u32x4>(key, key_row_stride, value, value_row_stride, k_cache,
                                   v_cache, slot_mapping, num_tokens, D, stream);
    const bool v4 = D % 2 == 0 && aligned(key, key_row_stride, 4) &&
                    aligned(value, value_row_stride, 4) && aligned(k_cache, D, 4) &&
                    aligned(v_cache, D, 4);
    if (v4)
        return launch_store<uint32_t>(key, key_row_stride, value, value_row_stride, k_cache,
                                      v_cache, slot_mapping, num_tokens, D, stream);
    return launch_store<uint16_t>(key, key_row_stride, value, value_row_stride, k_cache, v_cache,
                                  slot_mapping, num_tokens, D, stream);
}
