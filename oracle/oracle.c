/*
 * Oracle for the paged-KV hot path. TEST INFRASTRUCTURE ONLY: only tests/, the smoke check
 * and the benchmark's CPU-baseline leg may load this library. The product path never calls it.
 *
 * It computes what the method computes by its plain definition, slowly and in double
 * precision, with no tiling, no online softmax and no split of the key range:
 *
 *  - store: each token row whose slot is not -1 is copied bit for bit into row `slot` of the
 *    flattened key and value pools ("Nano-vLLM Field Guide", Step 10.3, the Triton store
 *    kernel and its wrapper; the slot formula is in Step 05.1).
 *  - gather: logical key j of a sequence lives in pool row
 *    block_table[j / block_size] * block_size + j % block_size (Step 05.1); within that row,
 *    kv head g occupies values [g * head_dim, (g + 1) * head_dim) (Step 07.4, the per-layer
 *    pool view [num_blocks, block_size, kv_heads, head_dim]).
 *  - attention: softmax(scale * q K^T) V over the visible keys. Query head h reads kv head
 *    h / (num_heads / num_kv_heads). In prefill, new row i of a sequence with Lq new tokens and
 *    Lk keys sees keys 0 .. (Lk - Lq) + i, the bottom-right causal alignment that Step 10.3
 *    describes for cached context. In decode a sequence sees all context_lens[b] keys, which
 *    include the token stored in the same step (Step 07.6); a row with context 0 attends to
 *    nothing and its output is defined here as zeros.
 *
 * bf16 inputs are widened exactly to double; sums run in increasing index order; the softmax
 * subtracts the row maximum before exp(). Outputs are double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_to_double(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Store: k_cache[slot] <- key[i], v_cache[slot] <- value[i] for every i with slot != -1.
 * key/value rows are `row_elems` contiguous 16-bit values at the given row strides
 * (in elements). Returns the number of rows written. */
int64_t oracle_store_kvcache(const uint16_t *key, int64_t key_row_stride,
                             const uint16_t *value, int64_t value_row_stride,
                             uint16_t *k_cache, uint16_t *v_cache,
                             const int32_t *slot_mapping, int64_t num_tokens,
                             int64_t row_elems) {
    int64_t written = 0;
    for (int64_t i = 0; i < num_tokens; ++i) {
        int64_t slot = slot_mapping[i];
        if (slot == -1) continue;
        memcpy(k_cache + slot * row_elems, key + i * key_row_stride,
               (size_t)row_elems * sizeof(uint16_t));
        memcpy(v_cache + slot * row_elems, value + i * value_row_stride,
               (size_t)row_elems * sizeof(uint16_t));
        ++written;
    }
    return written;
}

/* Gather keys 0..n-1 of one sequence and one kv head into contiguous [n, head_dim] doubles. */
static void gather(const uint16_t *cache, const int32_t *table, int64_t n, int64_t kv_head,
                   int64_t num_kv_heads, int64_t head_dim, int64_t block_size, double *dst) {
    for (int64_t j = 0; j < n; ++j) {
        int64_t row = (int64_t)table[j / block_size] * block_size + j % block_size;
        const uint16_t *src = cache + (row * num_kv_heads + kv_head) * head_dim;
        for (int64_t e = 0; e < head_dim; ++e) dst[j * head_dim + e] = bf16_to_double(src[e]);
    }
}

/* Softmax attention of one query vector over n contiguous keys/values.
 * out[head_dim] = sum_j w_j V_j with w = softmax(scale * K q). If `weights` is not NULL the
 * n normalised weights are written there. n == 0 gives zeros. */
void oracle_attend_row(const double *q, const double *K, const double *V, int64_t n,
                       int64_t head_dim, double scale, double *out, double *weights) {
    for (int64_t e = 0; e < head_dim; ++e) out[e] = 0.0;
    if (n <= 0) return;
    double *s = (double *)malloc((size_t)n * sizeof(double));
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int64_t e = 0; e < head_dim; ++e) dot += q[e] * K[j * head_dim + e];
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int64_t j = 0; j < n; ++j) {
        double w = s[j] / l;
        if (weights) weights[j] = w;
        for (int64_t e = 0; e < head_dim; ++e) out[e] += w * V[j * head_dim + e];
    }
    free(s);
}

/* Prefill over a packed batch. q: [total_q, num_heads, head_dim] bf16; out the same shape in
 * double. Sequence b has Lq = cu_q[b+1] - cu_q[b] new rows starting at packed row cu_q[b] and
 * Lk = cu_k[b+1] - cu_k[b] keys, read from the pools through row b of block_tables
 * ([batch, bt_width]). */
void oracle_attn_prefill(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                         const int32_t *cu_q, const int32_t *cu_k, const int32_t *block_tables,
                         int64_t bt_width, int64_t batch, int64_t num_heads, int64_t num_kv_heads,
                         int64_t head_dim, int64_t block_size, double scale, double *out) {
    const int64_t group = num_heads / num_kv_heads;
    for (int64_t b = 0; b < batch; ++b) {
        const int64_t q0 = cu_q[b], Lq = cu_q[b + 1] - cu_q[b];
        const int64_t Lk = cu_k[b + 1] - cu_k[b];
        const int64_t P = Lk - Lq;
        const int32_t *table = block_tables + b * bt_width;
        double *K = (double *)malloc((size_t)(Lk > 0 ? Lk : 1) * head_dim * sizeof(double));
        double *V = (double *)malloc((size_t)(Lk > 0 ? Lk : 1) * head_dim * sizeof(double));
        for (int64_t g = 0; g < num_kv_heads; ++g) {
            gather(k_cache, table, Lk, g, num_kv_heads, head_dim, block_size, K);
            gather(v_cache, table, Lk, g, num_kv_heads, head_dim, block_size, V);
            const int64_t items = group * Lq;
#pragma omp parallel for schedule(dynamic, 4)
            for (int64_t it = 0; it < items; ++it) {
                const int64_t h = g * group + it / Lq;
                const int64_t i = it % Lq;
                double qv[512];
                const uint16_t *qr = q + ((q0 + i) * num_heads + h) * head_dim;
                for (int64_t e = 0; e < head_dim; ++e) qv[e] = bf16_to_double(qr[e]);
                oracle_attend_row(qv, K, V, P + i + 1, head_dim, scale,
                                  out + ((q0 + i) * num_heads + h) * head_dim, NULL);
            }
        }
        free(K);
        free(V);
    }
}

/* Decode: one query row per sequence. q: [batch, num_heads, head_dim] bf16; sequence b reads
 * context_lens[b] keys through row b of block_tables. */
void oracle_attn_decode(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                        const int32_t *context_lens, const int32_t *block_tables,
                        int64_t bt_width, int64_t batch, int64_t num_heads, int64_t num_kv_heads,
                        int64_t head_dim, int64_t block_size, double scale, double *out) {
    const int64_t group = num_heads / num_kv_heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t it = 0; it < batch * num_kv_heads; ++it) {
        const int64_t b = it / num_kv_heads, g = it % num_kv_heads;
        const int64_t Lk = context_lens[b];
        const int32_t *table = block_tables + b * bt_width;
        double *K = (double *)malloc((size_t)(Lk > 0 ? Lk : 1) * head_dim * sizeof(double));
        double *V = (double *)malloc((size_t)(Lk > 0 ? Lk : 1) * head_dim * sizeof(double));
        gather(k_cache, table, Lk, g, num_kv_heads, head_dim, block_size, K);
        gather(v_cache, table, Lk, g, num_kv_heads, head_dim, block_size, V);
        for (int64_t h = g * group; h < (g + 1) * group; ++h) {
            double qv[512];
            const uint16_t *qr = q + (b * num_heads + h) * head_dim;
            for (int64_t e = 0; e < head_dim; ++e) qv[e] = bf16_to_double(qr[e]);
            oracle_attend_row(qv, K, V, Lk, head_dim, scale, out + (b * num_heads + h) * head_dim,
                              NULL);
        }
        free(K);
        free(V);
    }
}
