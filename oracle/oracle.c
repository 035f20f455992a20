/*
 * oracle.c -- plain fp64 CPU reference for paged grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the HIP library.  It shares no code,
 * header or table with the GPU path.
 *
 * What it computes, and where the pages define it:
 *   - Attention(Q,K,V) = softmax(Q K^T / sqrt(d)) V: "Modern LLM Inference --
 *     Workloads, Bottlenecks, and Optimization Techniques" (gozhiyuan.github.io,
 *     stanford-llm-11), subsection "Why Cross-Layer Attention Shares K/V but Not
 *     Q", the attention equation.  The scale is passed in explicitly (the
 *     caller passes 1/sqrt(d)) and widened to double.
 *   - Grouped-query attention: Hq query heads share Hkv KV heads, each KV head
 *     serving a contiguous group of G = Hq/Hkv query heads, and Hq % Hkv == 0.
 *     Same notes, section 4.1 "Grouped-Query Attention (GQA)"; "The Ultimate
 *     Guide to LLM Inference Optimization- Part 2" (wpnews.pro), section
 *     "Grouped Query Attention" (the divisibility rule); itinai.com/?p=48087,
 *     second paragraph (the 5-D [batch, seq, groups, heads-per-group, dim]
 *     query view whose flattening makes query head qh use KV head qh / G).
 *   - Paged KV cache: fixed-size blocks placed anywhere in a pool, found
 *     through a per-sequence block table.  "Advanced Optimizations: MQA, GQA,
 *     and PagedAttention" (tryclaro.ai), section "PagedAttention: The OS
 *     Analogy"; the Ultimate Guide, section "Paged Attention"; the lecture
 *     notes, section 8.2 "Paged Attention", item 1 "Non-Contiguous KV Blocks".
 *   - Decode attends to every earlier token of the sequence through the cache:
 *     the Ultimate Guide, introduction (decode phase and KV caching).
 *   - Packed variable-length batches with a block-diagonal, optionally causal
 *     bias built from the true lengths: itinai.com/?p=48087, first paragraph;
 *     the lecture notes, section 8.1 (lengths 3, 9, 5 flattened to 17 tokens).
 *   - Softmax is exact (no approximation): the lecture notes, "Linear Attention
 *     vs. FlashAttention (Online Softmax)".  So this file is the plain
 *     definition: every score, then the max, the exponentials, their sum, the
 *     weights, and the weighted sum of values -- two passes in fp64, no tiling,
 *     no partitions, no online rescaling.
 *
 * Threading: OpenMP over independent (sequence, query head) or (row, query head)
 * units, for timing only.  Each unit's arithmetic is serial in a fixed order,
 * so results do not depend on the thread count.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Exact widening of one element to double. */
static double elem(const void* base, int64_t idx, int32_t dtype) {
    if (dtype == ORACLE_BF16) {
        uint32_t u = (uint32_t)((const uint16_t*)base)[idx] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    if (dtype == ORACLE_F64) return ((const double*)base)[idx];
    return (double)((const float*)base)[idx];
}

static int elem_size(int32_t dtype) { return dtype == ORACLE_BF16 ? 2 : (dtype == ORACLE_F64 ? 8 : 4); }

static int dtype_ok(int32_t dtype) { return dtype == ORACLE_F32 || dtype == ORACLE_BF16 || dtype == ORACLE_F64; }

/*
 * FP8 E4M3 in the OCP 8-bit floating point layout ("E4M3FN"): bit 7 sign, bits
 * 6..3 exponent (bias 7), bits 2..0 mantissa.  Exponent field e > 0 gives
 * (1 + m/8) * 2^(e-7); e = 0 gives the subnormals (m/8) * 2^-6; the codes
 * S.1111.111 are NaN, and there is no infinity, so the largest finite
 * magnitude is 1.75 * 2^8 = 448 (code 0x7E).
 */
static double e4m3_value(uint8_t code) {
    const int sign = code >> 7, e = (code >> 3) & 0xF, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    const double mag = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* Values of the 127 non-negative finite codes 0x00 .. 0x7E, which increase
 * with the code (filled once, before any parallel region). */
static double e4m3_table[0x7F];
static int e4m3_table_ready = 0;

static void e4m3_init(void) {
    if (e4m3_table_ready) return;
    for (int c = 0; c <= 0x7E; ++c) e4m3_table[c] = e4m3_value((uint8_t)c);
    e4m3_table_ready = 1;
}

/* Nearest E4M3 code to x (|x| <= 448), ties to the code with an even mantissa:
 * lo = the largest code whose value is <= |x| (binary search in the increasing
 * table), then the nearer of lo and lo + 1. */
static uint8_t e4m3_encode(float x) {
    const double a = fabs((double)x);
    int lo = 0, hi = 0x7E;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (e4m3_table[mid] <= a) lo = mid;
        else hi = mid - 1;
    }
    int best = lo;
    if (lo < 0x7E) {
        const double dl = a - e4m3_table[lo], du = e4m3_table[lo + 1] - a;
        if (du < dl || (du == dl && ((lo + 1) & 1) == 0)) best = lo + 1;
    }
    return (uint8_t)(best | ((x < 0.0f || (x == 0.0f && signbit(x))) ? 0x80 : 0));
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int pick_threads(int32_t num_threads) {
    if (num_threads > 0) return num_threads;
    return oracle_max_threads();
}

/* Physical block holding logical position pos of sequence b, or -1 when the
 * position is past the table or the entry is outside the pool. */
static int64_t block_of(const int32_t* block_table, int32_t max_blocks_per_seq, int32_t num_blocks,
                        int32_t b, int64_t pos, int32_t block_size) {
    int64_t page = pos / block_size;
    if (page >= max_blocks_per_seq) return -1;
    int64_t blk = block_table[(int64_t)b * max_blocks_per_seq + page];
    if (blk < 0 || blk >= num_blocks) return -1;
    return blk;
}

/* Element offset of (blk, head, slot, 0) in a [num_blocks, Hkv, bs, d] pool. */
static int64_t page_offset(int64_t blk, int32_t head, int64_t slot, int32_t num_kv_heads,
                           int32_t block_size, int32_t head_dim) {
    return ((blk * num_kv_heads + head) * block_size + slot) * head_dim;
}

int oracle_paged_kv_write(const void* k, const void* v, const int32_t* cu_seqlens,
                          const int32_t* start_pos, const int32_t* block_table,
                          int32_t max_blocks_per_seq, void* k_cache, void* v_cache,
                          int32_t batch, int32_t num_blocks, int32_t block_size,
                          int32_t num_kv_heads, int32_t head_dim, int32_t dtype) {
    if (!k || !v || !cu_seqlens || !start_pos || !block_table || !k_cache || !v_cache) return ORACLE_EINVAL;
    if (batch < 0 || num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0) return ORACLE_EINVAL;
    if (!dtype_ok(dtype)) return ORACLE_EINVAL;
    const int es = elem_size(dtype);
    const size_t row_bytes = (size_t)head_dim * es;
    for (int32_t b = 0; b < batch; ++b) {
        if (cu_seqlens[b + 1] < cu_seqlens[b] || start_pos[b] < 0) return ORACLE_ERANGE;
        for (int64_t t = cu_seqlens[b]; t < cu_seqlens[b + 1]; ++t) {
            const int64_t pos = (int64_t)start_pos[b] + (t - cu_seqlens[b]);
            const int64_t blk = block_of(block_table, max_blocks_per_seq, num_blocks, b, pos, block_size);
            if (blk < 0) return ORACLE_ERANGE;
            const int64_t slot = pos % block_size;
            for (int32_t h = 0; h < num_kv_heads; ++h) {
                const int64_t src = (t * num_kv_heads + h) * (int64_t)head_dim;
                const int64_t dst = page_offset(blk, h, slot, num_kv_heads, block_size, head_dim);
                memcpy((char*)k_cache + dst * es, (const char*)k + src * es, row_bytes);
                memcpy((char*)v_cache + dst * es, (const char*)v + src * es, row_bytes);
            }
        }
    }
    return ORACLE_OK;
}

int oracle_paged_kv_gather(const void* k_cache, const void* v_cache, const int32_t* block_table,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           void* k_out, void* v_out, int32_t batch, int32_t num_blocks,
                           int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                           int32_t dtype) {
    if (!k_cache || !v_cache || !block_table || !context_lens || !k_out || !v_out) return ORACLE_EINVAL;
    if (batch < 0 || num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0) return ORACLE_EINVAL;
    if (!dtype_ok(dtype)) return ORACLE_EINVAL;
    const int es = elem_size(dtype);
    const size_t row_bytes = (size_t)head_dim * es;
    int64_t t = 0;
    for (int32_t b = 0; b < batch; ++b) {
        if (context_lens[b] < 0) return ORACLE_ERANGE;
        for (int64_t pos = 0; pos < context_lens[b]; ++pos, ++t) {
            const int64_t blk = block_of(block_table, max_blocks_per_seq, num_blocks, b, pos, block_size);
            if (blk < 0) return ORACLE_ERANGE;
            const int64_t slot = pos % block_size;
            for (int32_t h = 0; h < num_kv_heads; ++h) {
                const int64_t src = page_offset(blk, h, slot, num_kv_heads, block_size, head_dim);
                const int64_t dst = (t * num_kv_heads + h) * (int64_t)head_dim;
                memcpy((char*)k_out + dst * es, (const char*)k_cache + src * es, row_bytes);
                memcpy((char*)v_out + dst * es, (const char*)v_cache + src * es, row_bytes);
            }
        }
    }
    return ORACLE_OK;
}

int oracle_paged_kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst,
                                int32_t num_pairs, int32_t num_blocks, int32_t block_size,
                                int32_t num_kv_heads, int32_t head_dim, int32_t dtype) {
    if (!k_cache || !v_cache || (num_pairs > 0 && (!src || !dst))) return ORACLE_EINVAL;
    if (num_pairs < 0 || num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0)
        return ORACLE_EINVAL;
    if (!dtype_ok(dtype)) return ORACLE_EINVAL;
    for (int32_t i = 0; i < num_pairs; ++i)
        if (src[i] < 0 || src[i] >= num_blocks || dst[i] < 0 || dst[i] >= num_blocks) return ORACLE_ERANGE;
    const int es = elem_size(dtype);
    const size_t row_bytes = (size_t)head_dim * es;
    for (int32_t i = 0; i < num_pairs; ++i)
        for (int32_t h = 0; h < num_kv_heads; ++h)
            for (int32_t slot = 0; slot < block_size; ++slot) {
                const int64_t from = page_offset(src[i], h, slot, num_kv_heads, block_size, head_dim);
                const int64_t to = page_offset(dst[i], h, slot, num_kv_heads, block_size, head_dim);
                memmove((char*)k_cache + to * es, (const char*)k_cache + from * es, row_bytes);
                memmove((char*)v_cache + to * es, (const char*)v_cache + from * es, row_bytes);
            }
    return ORACLE_OK;
}

int oracle_fp8_e4m3_decode(const uint8_t* codes, int64_t n, double* out) {
    if (n < 0 || (n > 0 && (!codes || !out))) return ORACLE_EINVAL;
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_value(codes[i]);
    return ORACLE_OK;
}

int oracle_fp8_e4m3_encode(const float* x, int64_t n, uint8_t* codes) {
    if (n < 0 || (n > 0 && (!x || !codes))) return ORACLE_EINVAL;
    e4m3_init();
    for (int64_t i = 0; i < n; ++i) {
        if (!(fabsf(x[i]) <= 448.0f)) return ORACLE_ERANGE;
        codes[i] = e4m3_encode(x[i]);
    }
    return ORACLE_OK;
}

int oracle_paged_kv_write_fp8(const void* k, const void* v, const int32_t* cu_seqlens,
                              const int32_t* start_pos, const int32_t* block_table,
                              int32_t max_blocks_per_seq, uint8_t* k_cache, uint8_t* v_cache,
                              float* k_scale, float* v_scale, int32_t batch, int32_t num_blocks,
                              int32_t block_size, int32_t num_kv_heads, int32_t head_dim, int32_t dtype) {
    if (!k || !v || !cu_seqlens || !start_pos || !block_table || !k_cache || !v_cache || !k_scale || !v_scale)
        return ORACLE_EINVAL;
    if (batch < 0 || num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0) return ORACLE_EINVAL;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return ORACLE_EINVAL;
    e4m3_init();
    /* Contract check first (serial), so the parallel part cannot fail. */
    for (int32_t b = 0; b < batch; ++b) {
        if (cu_seqlens[b + 1] < cu_seqlens[b] || start_pos[b] < 0) return ORACLE_ERANGE;
        for (int64_t t = cu_seqlens[b]; t < cu_seqlens[b + 1]; ++t)
            if (block_of(block_table, max_blocks_per_seq, num_blocks, b, (int64_t)start_pos[b] + (t - cu_seqlens[b]),
                         block_size) < 0)
                return ORACLE_ERANGE;
    }
    /* Rows are independent (a written slot belongs to one token). */
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t b = 0; b < batch; ++b) {
        for (int64_t t = cu_seqlens[b]; t < cu_seqlens[b + 1]; ++t) {
            const int64_t pos = (int64_t)start_pos[b] + (t - cu_seqlens[b]);
            const int64_t blk = block_of(block_table, max_blocks_per_seq, num_blocks, b, pos, block_size);
            const int64_t slot = pos % block_size;
            for (int32_t h = 0; h < num_kv_heads; ++h) {
                const int64_t src = (t * num_kv_heads + h) * (int64_t)head_dim;
                const int64_t dst = page_offset(blk, h, slot, num_kv_heads, block_size, head_dim);
                const int64_t srow = (blk * num_kv_heads + h) * block_size + slot;
                for (int pool = 0; pool < 2; ++pool) {
                    const void* x = pool ? v : k;
                    uint8_t* codes = pool ? v_cache : k_cache;
                    /* The row's scale maps its largest magnitude onto 448; both
                     * the scale and x / scale are single-precision operations,
                     * the precision the codes are decided in. */
                    float amax = 0.0f;
                    for (int32_t i = 0; i < head_dim; ++i) {
                        const float a = fabsf((float)elem(x, src + i, dtype));
                        if (a > amax) amax = a;
                    }
                    const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
                    for (int32_t i = 0; i < head_dim; ++i) {
                        float y = (float)elem(x, src + i, dtype) / sc;
                        if (y > 448.0f) y = 448.0f;
                        if (y < -448.0f) y = -448.0f;
                        codes[dst + i] = e4m3_encode(y);
                    }
                    (pool ? v_scale : k_scale)[srow] = sc;
                }
            }
        }
    }
    return ORACLE_OK;
}

int oracle_dequantize_fp8(const uint8_t* codes, const float* scales, int64_t rows, int32_t head_dim, double* out) {
    if (rows < 0 || head_dim <= 0 || (rows > 0 && (!codes || !scales || !out))) return ORACLE_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t i = 0; i < head_dim; ++i)
            out[r * head_dim + i] = e4m3_value(codes[r * head_dim + i]) * (double)scales[r];
    return ORACLE_OK;
}

/*
 * softmax(scores) . values for one query row, in fp64, two passes:
 *   m = max_j s_j;  w_j = exp(s_j - m);  Z = sum_j w_j;  p_j = w_j / Z;
 *   out[x] = sum_j p_j * value_j[x]
 * s holds the n scaled scores; value_ptrs[j] is the element offset of value row j
 * inside `values`.  p (length n) receives the weights.
 */
static void softmax_weighted_sum(const double* s, int64_t n, const void* values,
                                 const int64_t* value_offs, int32_t head_dim, int32_t dtype,
                                 double* p, double* out) {
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j)
        if (s[j] > m) m = s[j];
    double z = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        p[j] = exp(s[j] - m);
        z += p[j];
    }
    for (int64_t j = 0; j < n; ++j) p[j] = p[j] / z;
    for (int32_t x = 0; x < head_dim; ++x) {
        double acc = 0.0;
        for (int64_t j = 0; j < n; ++j) acc += p[j] * elem(values, value_offs[j] + x, dtype);
        out[x] = acc;
    }
}

/* Scaled dot product of query row (element offset qo in q) and key row (offset ko in keys). */
static double scaled_dot(const void* q, int64_t qo, const void* keys, int64_t ko, int32_t head_dim,
                         double scale, int32_t dtype) {
    double acc = 0.0;
    for (int32_t x = 0; x < head_dim; ++x) acc += elem(q, qo + x, dtype) * elem(keys, ko + x, dtype);
    return scale * acc;
}

int oracle_gqa_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, double scale, int32_t window, int32_t dtype, double* out,
                            double* probs, int32_t probs_stride, int32_t num_threads) {
    if (!q || !k_cache || !v_cache || !block_table || !context_lens || !out) return ORACLE_EINVAL;
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
        return ORACLE_EINVAL;
    if (num_q_heads % num_kv_heads != 0 || !dtype_ok(dtype)) return ORACLE_EINVAL;
    const int32_t group = num_q_heads / num_kv_heads;

    /* Contract check first (serial), so the parallel part cannot fail. */
    int64_t max_ctx = 0;
    for (int32_t b = 0; b < batch; ++b) {
        if (context_lens[b] < 0) return ORACLE_ERANGE;
        if (probs && context_lens[b] > probs_stride) return ORACLE_EINVAL;
        for (int64_t j = 0; j < context_lens[b]; ++j)
            if (block_of(block_table, max_blocks_per_seq, num_blocks, b, j, block_size) < 0) return ORACLE_ERANGE;
        if (context_lens[b] > max_ctx) max_ctx = context_lens[b];
    }

    const int64_t units = (int64_t)batch * num_q_heads;
    int failed = 0;
#pragma omp parallel num_threads(pick_threads(num_threads))
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(max_ctx > 0 ? max_ctx : 1));
        double* p = (double*)malloc(sizeof(double) * (size_t)(max_ctx > 0 ? max_ctx : 1));
        int64_t* voff = (int64_t*)malloc(sizeof(int64_t) * (size_t)(max_ctx > 0 ? max_ctx : 1));
        if (!s || !p || !voff) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            if (!s || !p || !voff) continue;
            const int32_t b = (int32_t)(u / num_q_heads);
            const int32_t qh = (int32_t)(u % num_q_heads);
            const int32_t h = qh / group;
            const int64_t n = context_lens[b];
            double* o = out + u * head_dim;
            if (n == 0) {
                for (int32_t x = 0; x < head_dim; ++x) o[x] = 0.0;
                continue;
            }
            /* Local attention: only the newest `window` positions (the query's
             * own included) are attended to. */
            const int64_t lo = (window > 0 && n > window) ? n - window : 0;
            const int64_t qo = u * head_dim;
            for (int64_t j = lo; j < n; ++j) {
                const int64_t blk = block_of(block_table, max_blocks_per_seq, num_blocks, b, j, block_size);
                const int64_t slot = j % block_size;
                const int64_t ko = page_offset(blk, h, slot, num_kv_heads, block_size, head_dim);
                s[j - lo] = scaled_dot(q, qo, k_cache, ko, head_dim, scale, dtype);
                voff[j - lo] = ko;
            }
            softmax_weighted_sum(s, n - lo, v_cache, voff, head_dim, dtype, p, o);
            if (probs)
                for (int64_t j = 0; j < n; ++j) probs[u * probs_stride + j] = j < lo ? 0.0 : p[j - lo];
        }
        free(s);
        free(p);
        free(voff);
    }
    return failed ? ORACLE_EINVAL : ORACLE_OK;
}

int oracle_gqa_varlen_prefill(const void* q, const void* k, const void* v,
                              const int32_t* cu_seqlens, int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, double scale,
                              int32_t causal, int32_t window, int32_t dtype, const int32_t* rows,
                              int32_t num_rows, double* out, int32_t num_threads) {
    if (!q || !k || !v || !cu_seqlens || !out) return ORACLE_EINVAL;
    if (window > 0 && !causal) return ORACLE_EINVAL;
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0) return ORACLE_EINVAL;
    if (num_q_heads % num_kv_heads != 0 || !dtype_ok(dtype)) return ORACLE_EINVAL;
    const int32_t group = num_q_heads / num_kv_heads;
    if (cu_seqlens[0] != 0) return ORACLE_ERANGE;
    for (int32_t s = 0; s < batch; ++s)
        if (cu_seqlens[s + 1] < cu_seqlens[s]) return ORACLE_ERANGE;
    const int64_t total = cu_seqlens[batch];
    if (!rows) num_rows = (int32_t)total;
    if (num_rows < 0) return ORACLE_EINVAL;
    for (int32_t r = 0; rows && r < num_rows; ++r)
        if (rows[r] < 0 || rows[r] >= total) return ORACLE_ERANGE;

    const int64_t units = (int64_t)num_rows * num_q_heads;
    /* Per-thread scratch is sized for the whole packed batch, not just the
     * longest sequence, so any key range inside [0, T) fits. */
    const size_t scratch = (size_t)(total > 0 ? total : 1);
    int failed = 0;
#pragma omp parallel num_threads(pick_threads(num_threads))
    {
        double* s = (double*)malloc(sizeof(double) * scratch);
        double* p = (double*)malloc(sizeof(double) * scratch);
        int64_t* voff = (int64_t*)malloc(sizeof(int64_t) * scratch);
        if (!s || !p || !voff) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t u = 0; u < units; ++u) {
            if (!s || !p || !voff) continue;
            const int64_t r = u / num_q_heads;
            const int32_t qh = (int32_t)(u % num_q_heads);
            const int32_t h = qh / group;
            const int64_t i = rows ? rows[r] : r;
            /* The sequence that owns row i: the block-diagonal bias keeps every
             * row inside its own sequence. */
            int32_t seq = 0;
            while (cu_seqlens[seq + 1] <= i) ++seq;
            int64_t first = cu_seqlens[seq];
            const int64_t last = causal ? i : (int64_t)cu_seqlens[seq + 1] - 1;
            if (window > 0 && i - window + 1 > first) first = i - window + 1;   /* newest `window` keys */
            const int64_t n = last - first + 1;
            const int64_t qo = (i * num_q_heads + qh) * (int64_t)head_dim;
            for (int64_t j = 0; j < n; ++j) {
                const int64_t ko = ((first + j) * num_kv_heads + h) * (int64_t)head_dim;
                s[j] = scaled_dot(q, qo, k, ko, head_dim, scale, dtype);
                voff[j] = ko;
            }
            softmax_weighted_sum(s, n, v, voff, head_dim, dtype, p, out + u * head_dim);
        }
        free(s);
        free(p);
        free(voff);
    }
    return failed ? ORACLE_EINVAL : ORACLE_OK;
}

int oracle_gqa_paged_extend(const void* q, const int32_t* cu_q, const void* k_cache,
                            const void* v_cache, const int32_t* block_table,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            double scale, int32_t window, int32_t dtype, const int32_t* rows,
                            int32_t num_rows, double* out, int32_t num_threads) {
    if (!q || !cu_q || !k_cache || !v_cache || !block_table || !context_lens || !out) return ORACLE_EINVAL;
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
        return ORACLE_EINVAL;
    if (num_q_heads % num_kv_heads != 0 || !dtype_ok(dtype)) return ORACLE_EINVAL;
    const int32_t group = num_q_heads / num_kv_heads;

    /* Contract check first (serial), so the parallel part cannot fail. */
    if (cu_q[0] != 0) return ORACLE_ERANGE;
    int64_t max_ctx = 0;
    for (int32_t b = 0; b < batch; ++b) {
        if (cu_q[b + 1] < cu_q[b] || context_lens[b] < 0) return ORACLE_ERANGE;
        for (int64_t j = 0; j < context_lens[b]; ++j)
            if (block_of(block_table, max_blocks_per_seq, num_blocks, b, j, block_size) < 0) return ORACLE_ERANGE;
        if (context_lens[b] > max_ctx) max_ctx = context_lens[b];
    }

    const int64_t total = cu_q[batch];
    if (!rows) num_rows = (int32_t)total;
    if (num_rows < 0) return ORACLE_EINVAL;
    for (int32_t x = 0; rows && x < num_rows; ++x)
        if (rows[x] < 0 || rows[x] >= total) return ORACLE_ERANGE;

    const int64_t units = (int64_t)num_rows * num_q_heads;
    int failed = 0;
#pragma omp parallel num_threads(pick_threads(num_threads))
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(max_ctx > 0 ? max_ctx : 1));
        double* p = (double*)malloc(sizeof(double) * (size_t)(max_ctx > 0 ? max_ctx : 1));
        int64_t* voff = (int64_t*)malloc(sizeof(int64_t) * (size_t)(max_ctx > 0 ? max_ctx : 1));
        if (!s || !p || !voff) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t u = 0; u < units; ++u) {
            if (!s || !p || !voff) continue;
            const int64_t r = rows ? rows[u / num_q_heads] : u / num_q_heads;
            const int32_t qh = (int32_t)(u % num_q_heads);
            const int32_t h = qh / group;
            int32_t b = 0;
            while (cu_q[b + 1] <= r) ++b;
            const int64_t q_len = (int64_t)cu_q[b + 1] - cu_q[b];
            const int64_t i = r - cu_q[b];
            /* The query's own position: its sequence's q_len tokens are the last
             * positions of the context. */
            const int64_t pos = (int64_t)context_lens[b] - q_len + i;
            const int64_t n = pos + 1;   /* keys 0 .. pos */
            double* o = out + u * head_dim;
            if (n <= 0) {
                for (int32_t x = 0; x < head_dim; ++x) o[x] = 0.0;
                continue;
            }
            const int64_t lo = (window > 0 && n > window) ? n - window : 0;   /* newest `window` keys */
            const int64_t qo = (r * num_q_heads + qh) * head_dim;
            for (int64_t j = lo; j < n; ++j) {
                const int64_t blk = block_of(block_table, max_blocks_per_seq, num_blocks, b, j, block_size);
                const int64_t ko = page_offset(blk, h, j % block_size, num_kv_heads, block_size, head_dim);
                s[j - lo] = scaled_dot(q, qo, k_cache, ko, head_dim, scale, dtype);
                voff[j - lo] = ko;
            }
            softmax_weighted_sum(s, n - lo, v_cache, voff, head_dim, dtype, p, o);
        }
        free(s);
        free(p);
        free(voff);
    }
    return failed ? ORACLE_EINVAL : ORACLE_OK;
}
