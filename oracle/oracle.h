/*
 * oracle.h -- plain, slow, fp64 CPU reference for paged grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The HIP library never
 * links, includes or calls it, and this file shares no code with it.
 *
 * All pointers are HOST pointers owned by the caller.  Element data is fp32
 * (dtype ORACLE_F32), raw bf16 bit patterns (ORACLE_BF16, uint16 per element)
 * or fp64 (ORACLE_F64, for pools dequantised from fp8); every value is widened
 * exactly to double before any arithmetic.
 *
 * Layouts (row-major, innermost last):
 *   packed K/V        [T, Hkv, d]        T = total tokens, sequences concatenated
 *   decode Q          [B, Hq, d]         one query token per sequence
 *   prefill Q         [T, Hq, d]
 *   KV page pool      [num_blocks, Hkv, block_size, d]   (separate K and V pools)
 *   block_table       int32 [B, max_blocks_per_seq]      logical page -> physical block
 *   cu_seqlens        int32 [B+1]                        prefix sums of lengths
 *
 * Return value: ORACLE_OK, or ORACLE_EINVAL for a bad argument, or
 * ORACLE_ERANGE when the data breaks the caller's contract (a block id
 * outside the pool, a position past the block table, decreasing cu_seqlens).
 */
#ifndef PGQA_ORACLE_H
#define PGQA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };
enum { ORACLE_OK = 0, ORACLE_EINVAL = 1, ORACLE_ERANGE = 2 };

/* Scatter packed K/V of each sequence's new tokens into the page pools.
 * Token t of sequence b sits at logical position start_pos[b] + (t - cu_seqlens[b]);
 * position p lives in block block_table[b][p / block_size], slot p % block_size.
 * Element bytes are copied unchanged. */
int oracle_paged_kv_write(const void* k, const void* v, const int32_t* cu_seqlens,
                          const int32_t* start_pos, const int32_t* block_table,
                          int32_t max_blocks_per_seq, void* k_cache, void* v_cache,
                          int32_t batch, int32_t num_blocks, int32_t block_size,
                          int32_t num_kv_heads, int32_t head_dim, int32_t dtype);

/* Inverse of the write: copy positions [0, context_lens[b]) of every sequence
 * out of the pools into packed [sum(context_lens), Hkv, d] arrays. */
int oracle_paged_kv_gather(const void* k_cache, const void* v_cache, const int32_t* block_table,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           void* k_out, void* v_out, int32_t batch, int32_t num_blocks,
                           int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                           int32_t dtype);

/* Low-precision KV pages (the Ultimate Guide, section "KV Cache Compression":
 * KV memory shrinks with fewer bits per value; the pages give the motivation and
 * byte sizes only, so the format here is a reading): codes are FP8 E4M3 in the
 * OCP layout (bias 7, largest finite 448, no infinity) and every (token, KV
 * head) row of d values has its own fp32 scale, stored in a scale pool laid out
 * like the pages, [num_blocks, Hkv, block_size].  Quantising a row: amax =
 * max |x|, scale = amax / 448 (1 for an all-zero row), code = the nearest E4M3
 * value to x / scale (ties to even), the division and the scale in single
 * precision.  The row's values are then code * scale.
 *
 * oracle_fp8_e4m3_decode / _encode: the value of each code (NaN for the NaN
 * codes) and the nearest code of each value (|x| <= 448, else ORACLE_ERANGE).
 * oracle_paged_kv_write_fp8: paged_kv_write that quantises (K/V input fp32 or
 * bf16), writing codes into the uint8 pools and the row scales.
 * oracle_dequantize_fp8: out[r][i] = value(codes[r][i]) * scales[r] in fp64 for
 * rows flattened row-major (e.g. a whole pool and its scale pool); attention
 * over fp8 pages is attention over these fp64 pools (dtype ORACLE_F64). */
int oracle_fp8_e4m3_decode(const uint8_t* codes, int64_t n, double* out);
int oracle_fp8_e4m3_encode(const float* x, int64_t n, uint8_t* codes);
int oracle_paged_kv_write_fp8(const void* k, const void* v, const int32_t* cu_seqlens,
                              const int32_t* start_pos, const int32_t* block_table,
                              int32_t max_blocks_per_seq, uint8_t* k_cache, uint8_t* v_cache,
                              float* k_scale, float* v_scale, int32_t batch, int32_t num_blocks,
                              int32_t block_size, int32_t num_kv_heads, int32_t head_dim, int32_t dtype);
int oracle_dequantize_fp8(const uint8_t* codes, const float* scales, int64_t rows, int32_t head_dim, double* out);

/* Copy-on-write block copy (the lecture notes, section 8.2 "Prefix Sharing": when
 * sequences diverge only the modified block is copied).  For i = 0 .. num_pairs-1
 * in order, every KV head's block_size slots of block src[i] are copied, bytes
 * unchanged, onto block dst[i], in the K pool and in the V pool. */
int oracle_paged_kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst,
                                int32_t num_pairs, int32_t num_blocks, int32_t block_size,
                                int32_t num_kv_heads, int32_t head_dim, int32_t dtype);

/* Local attention (the lecture notes, section 4.4): with window > 0 every
 * query attends only to the newest `window` positions up to its own (its own
 * included), i.e. keys p - window + 1 .. p for a query at position p; window
 * <= 0 means no window.  The three attention calls below take it.
 *
 * Decode: one query token per sequence attends to every cached position
 * [0, context_lens[b]) of its sequence (the query sits at context_lens[b] - 1).
 * Query head qh reads KV head qh / (Hq / Hkv).  out is fp64 [B, Hq, d]; a
 * sequence with no context gets 0.  probs (may be NULL) receives the softmax
 * weights, fp64 [B, Hq, probs_stride] (0 for positions outside the window),
 * entries past the context left untouched.  num_threads <= 0 uses the default. */
int oracle_gqa_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, double scale, int32_t window, int32_t dtype, double* out,
                            double* probs, int32_t probs_stride, int32_t num_threads);

/* Packed variable-length prefill with a block-diagonal (optionally causal) mask.
 * Row i of sequence s (cu_seqlens[s] <= i < cu_seqlens[s+1]) attends to keys j of
 * the same sequence with j <= i when causal, else to all of that sequence
 * (a window needs causal).  rows (may be NULL) lists the packed row indices to evaluate; NULL means every
 * row 0..T-1 with num_rows = T.  out is fp64 [num_rows, Hq, d]. */
int oracle_gqa_varlen_prefill(const void* q, const void* k, const void* v,
                              const int32_t* cu_seqlens, int32_t batch, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, double scale,
                              int32_t causal, int32_t window, int32_t dtype, const int32_t* rows,
                              int32_t num_rows, double* out, int32_t num_threads);

/* Several query tokens per sequence over its paged cache: chunked prefill on
 * top of a cached prefix, or verification of draft tokens.  Sequence b has
 * q_len_b = cu_q[b+1] - cu_q[b] query tokens, the LAST q_len_b positions of
 * its context [0, context_lens[b]) (their K/V are already in the pages).
 * Query row r = cu_q[b] + i sits at position p = context_lens[b] - q_len_b + i
 * and attends to the cached keys j <= p (causal mask aligned to the end of the
 * context).  Query head qh reads KV head qh / (Hq / Hkv).  q is
 * [cu_q[batch], Hq, d].  A row with no key (p < 0, i.e. q_len_b >
 * context_lens[b]) gets 0.  rows (may be NULL) lists the query rows to
 * evaluate; NULL means every row 0..cu_q[batch]-1 with num_rows = cu_q[batch].
 * out is fp64 [num_rows, Hq, d]. */
int oracle_gqa_paged_extend(const void* q, const int32_t* cu_q, const void* k_cache,
                            const void* v_cache, const int32_t* block_table,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            double scale, int32_t window, int32_t dtype, const int32_t* rows,
                            int32_t num_rows, double* out, int32_t num_threads);

/* Number of OpenMP threads a parallel region would use (for reporting). */
int oracle_max_threads(void);

#ifdef __cplusplus
}
#endif

#endif /* PGQA_ORACLE_H */
