// Host side of the library: status names, the index metadata a runner builds before each
// forward ("Nano-vLLM Field Guide", Steps 07.5-07.7) and a debug check of index preconditions.
#include <stdint.h>
#include <string.h>

#include <vector>

#include "nv_paged.h"

extern "C" const char *nv_status_string(nv_status status) {
    switch (status) {
        case NV_OK: return "NV_OK";
        case NV_ERR_INVALID_ARG: return "NV_ERR_INVALID_ARG: invalid argument";
        case NV_ERR_UNSUPPORTED: return "NV_ERR_UNSUPPORTED: shape not implemented by this library";
        case NV_ERR_LAUNCH: return "NV_ERR_LAUNCH: kernel launch failed";
        case NV_ERR_WORKSPACE: return "NV_ERR_WORKSPACE: decode workspace missing or too small";
        case NV_ERR_SCRATCH:
            return "NV_ERR_SCRATCH: the call needs more workspace than the library's static "
                   "scratch (NV_DECODE_SCRATCH_BYTES) holds";
    }
    return "unknown nv_status";
}

namespace {

// Writes one table row padded with -1 to `width` entries.
bool write_table_row(const int32_t *ids, int32_t n, int32_t width, int32_t *dst) {
    if (n > width) return false;
    for (int32_t j = 0; j < n; ++j) dst[j] = ids[j];
    for (int32_t j = n; j < width; ++j) dst[j] = -1;
    return true;
}

bool offsets_ok(const int32_t *off, int32_t batch) {
    if (off[0] != 0) return false;
    for (int32_t b = 0; b < batch; ++b)
        if (off[b + 1] < off[b]) return false;
    return true;
}

}  // namespace

extern "C" nv_status nv_prepare_prefill(const int32_t *num_cached, const int32_t *num_new,
                                        const int32_t *table_offsets, const int32_t *block_ids,
                                        int32_t batch, int32_t block_size, int32_t *slot_mapping,
                                        int32_t *cu_seqlens_q, int32_t *cu_seqlens_k,
                                        int32_t *max_seqlen_q, int32_t *max_seqlen_k,
                                        int32_t *block_tables, int32_t bt_width,
                                        int32_t *has_cached_context) {
    if (batch < 0 || block_size <= 0 || bt_width < 0) return NV_ERR_INVALID_ARG;
    if (batch > 0 && (!num_cached || !num_new || !table_offsets || !cu_seqlens_q ||
                      !cu_seqlens_k))
        return NV_ERR_INVALID_ARG;
    if (!cu_seqlens_q || !cu_seqlens_k) return NV_ERR_INVALID_ARG;
    if (batch > 0 && !offsets_ok(table_offsets, batch)) return NV_ERR_INVALID_ARG;
    if (batch > 0 && table_offsets[batch] > 0 && !block_ids) return NV_ERR_INVALID_ARG;
    int64_t cq = 0, ck = 0;
    int32_t mq = 0, mk = 0;
    cu_seqlens_q[0] = 0;
    cu_seqlens_k[0] = 0;
    int64_t row = 0;
    for (int32_t b = 0; b < batch; ++b) {
        const int32_t start = num_cached[b], n = num_new[b];
        if (start < 0 || n < 0) return NV_ERR_INVALID_ARG;
        const int64_t end = (int64_t)start + n;
        const int32_t *table = block_ids + table_offsets[b];
        const int32_t tlen = table_offsets[b + 1] - table_offsets[b];
        if (end > (int64_t)tlen * block_size) return NV_ERR_INVALID_ARG;
        if (n > 0 && !slot_mapping) return NV_ERR_INVALID_ARG;
        // Walk the new positions block by block: one table lookup per touched block.
        for (int64_t p = start; p < end;) {
            const int64_t lb = p / block_size;
            const int64_t base = (int64_t)table[lb] * block_size;
            const int64_t stop = (lb + 1) * block_size < end ? (lb + 1) * block_size : end;
            for (; p < stop; ++p) slot_mapping[row++] = (int32_t)(base + p % block_size);
        }
        cq += n;
        ck += end;
        if (cq > INT32_MAX || ck > INT32_MAX) return NV_ERR_INVALID_ARG;
        cu_seqlens_q[b + 1] = (int32_t)cq;
        cu_seqlens_k[b + 1] = (int32_t)ck;
        if (n > mq) mq = n;
        if (end > mk) mk = (int32_t)end;
        if (block_tables && !write_table_row(table, tlen, bt_width, block_tables + (int64_t)b * bt_width))
            return NV_ERR_INVALID_ARG;
    }
    if (max_seqlen_q) *max_seqlen_q = mq;
    if (max_seqlen_k) *max_seqlen_k = mk;
    if (has_cached_context) *has_cached_context = ck > cq ? 1 : 0;
    return NV_OK;
}

extern "C" nv_status nv_prepare_decode(const int32_t *num_cached, const int32_t *num_new,
                                       const int32_t *table_offsets, const int32_t *block_ids,
                                       int32_t batch, int32_t block_size, int32_t *slot_mapping,
                                       int32_t *context_lens, int32_t *block_tables,
                                       int32_t bt_width) {
    if (batch < 0 || block_size <= 0 || bt_width < 0) return NV_ERR_INVALID_ARG;
    if (batch == 0) return NV_OK;
    if (!num_cached || !num_new || !table_offsets || !slot_mapping || !context_lens)
        return NV_ERR_INVALID_ARG;
    if (!offsets_ok(table_offsets, batch)) return NV_ERR_INVALID_ARG;
    if (table_offsets[batch] > 0 && !block_ids) return NV_ERR_INVALID_ARG;
    for (int32_t b = 0; b < batch; ++b) {
        const int32_t *table = block_ids + table_offsets[b];
        const int32_t tlen = table_offsets[b + 1] - table_offsets[b];
        if (num_new[b] == 0 && num_cached[b] == 0) {  // padding row of a captured batch
            slot_mapping[b] = -1;
            context_lens[b] = 0;
        } else {
            if (num_new[b] != 1 || num_cached[b] < 0) return NV_ERR_INVALID_ARG;
            const int64_t len = (int64_t)num_cached[b] + 1;
            if (len > (int64_t)tlen * block_size || len > INT32_MAX) return NV_ERR_INVALID_ARG;
            // The last block holds len - (tlen - 1) * block_size tokens; the new token is the last.
            const int64_t fill = len - (int64_t)(tlen - 1) * block_size;
            if (fill <= 0) return NV_ERR_INVALID_ARG;  // table longer than the sequence needs
            slot_mapping[b] = (int32_t)((int64_t)table[tlen - 1] * block_size + fill - 1);
            context_lens[b] = (int32_t)len;
        }
        if (block_tables && !write_table_row(table, tlen, bt_width, block_tables + (int64_t)b * bt_width))
            return NV_ERR_INVALID_ARG;
    }
    return NV_OK;
}

extern "C" nv_status nv_check_indices(const int32_t *slot_mapping, int64_t num_tokens,
                                      int64_t num_slots, const int32_t *block_tables,
                                      const int32_t *lens, int32_t batch,
                                      int32_t max_blocks_per_seq, int32_t block_size,
                                      int64_t num_blocks, int64_t *bad_index) {
    if (num_tokens < 0 || num_slots < 0 || batch < 0 || block_size <= 0 ||
        max_blocks_per_seq < 0 || num_blocks < 0)
        return NV_ERR_INVALID_ARG;
    if ((num_tokens > 0 && !slot_mapping) || (batch > 0 && (!block_tables || !lens)))
        return NV_ERR_INVALID_ARG;
    if (num_tokens > 0) {
        std::vector<uint8_t> seen((size_t)num_slots, 0);
        for (int64_t i = 0; i < num_tokens; ++i) {
            const int64_t s = slot_mapping[i];
            if (s == -1) continue;
            if (s < 0 || s >= num_slots || seen[(size_t)s]) {
                if (bad_index) *bad_index = i;
                return NV_ERR_INVALID_ARG;
            }
            seen[(size_t)s] = 1;
        }
    }
    for (int32_t b = 0; b < batch; ++b) {
        const int64_t need = ((int64_t)lens[b] + block_size - 1) / block_size;
        if (lens[b] < 0 || need > max_blocks_per_seq) {
            if (bad_index) *bad_index = (int64_t)b * max_blocks_per_seq;
            return NV_ERR_INVALID_ARG;
        }
        for (int64_t j = 0; j < need; ++j) {
            const int64_t id = block_tables[(int64_t)b * max_blocks_per_seq + j];
            if (id < 0 || id >= num_blocks) {
                if (bad_index) *bad_index = (int64_t)b * max_blocks_per_seq + j;
                return NV_ERR_INVALID_ARG;
            }
        }
    }
    return NV_OK;
}
