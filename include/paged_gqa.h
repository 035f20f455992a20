/*
 * paged_gqa.h -- C ABI of libpaged_gqa.so: grouped-query attention read through
 * a paged KV cache, for AMD Instinct MI355X (gfx950).
 *
 * Problem statement these calls implement (the pages are cited by title and
 * section; no call depends on anything beyond them):
 *   - Attention(Q, K, V) = softmax(Q K^T * scale) V with scale = 1/sqrt(d):
 *     "Modern LLM Inference -- Workloads, Bottlenecks, and Optimization
 *     Techniques" (gozhiyuan.github.io, stanford-llm-11), subsection "Why
 *     Cross-Layer Attention Shares K/V but Not Q", attention equation.
 *   - Grouped-query attention: Hq query heads share Hkv KV heads, query head
 *     qh reads KV head qh / (Hq / Hkv), and Hq must be a multiple of Hkv:
 *     same notes, section 4.1; "The Ultimate Guide to LLM Inference
 *     Optimization- Part 2" (wpnews.pro), section "Grouped Query Attention";
 *     itinai.com/?p=48087, second paragraph (5-D grouped query layout).
 *   - Paged KV cache: each sequence's K/V live in fixed-size blocks anywhere
 *     in a pool, located through a per-sequence block table: "Advanced
 *     Optimizations: MQA, GQA, and PagedAttention" (tryclaro.ai), sections
 *     "PagedAttention: The OS Analogy" and "Optimizing Block Size"; the
 *     Ultimate Guide, section "Paged Attention"; the lecture notes, section 8.2.
 *   - Packed variable-length batches with a block-diagonal, optionally causal
 *     mask built from the true lengths (cu_seqlens): itinai.com/?p=48087, first
 *     paragraph; the lecture notes, section 8.1 (selective batching).
 *   - Prefill (whole prompt, compute-bound) and decode (one new token per
 *     sequence, memory-bound) are separate phases: the lecture notes, section 2;
 *     the Ultimate Guide, introduction.
 *
 * Local attention (the lecture notes, section 4.4): a token may attend only to
 * the most recent positions.  The attention calls take `window`: 0 means full
 * (causal) attention; window > 0 keeps, for a query at position p, the keys
 * p - window + 1 .. p (the newest `window` positions, its own included).
 * Negative windows are PGQA_EINVAL.  Pages wholly before every query's window
 * are never read, so a caller may release them (their table entries may then
 * hold any value).
 *
 * Conventions shared by every call (the pgqa_bm_* block manager below is
 * host-only and documented on its own)
 *   - Every array argument is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or keeps device memory (the one
 *     exception, gqa_paged_decode_noalloc's scratch, is documented with it) and
 *     never synchronises.  Its only state between calls is a per-device cache of
 *     launch facts read from the HIP runtime (compute units, LDS per compute
 *     unit, kernel occupancy), guarded by a lock, so the calls are thread-safe.
 *   - `scale` (the attention calls) may be any finite float: the result is
 *     softmax(scale * q.k) for that value, a zero scale giving every visible
 *     key the same weight.  NaN or infinite scales are PGQA_EINVAL.
 *   - Element arrays hold PGQA_F32 (float) or PGQA_BF16 (bfloat16 bit
 *     patterns, 2 bytes each); out has the dtype of q.  Index arrays are int32.
 *   - Element pointers and the workspace must be 16-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on it and returns.
 *   - Return value: PGQA_OK, or an error code.  Arguments are checked on the
 *     host before any HIP call; a failed check returns PGQA_EINVAL,
 *     PGQA_ENOTSUP or PGQA_ENOSPC and enqueues nothing.  PGQA_EHIP reports a
 *     failed launch.  No exception or abort crosses this boundary.
 *   - Device-side contents are the caller's promise and are not checked on
 *     the host: block ids in [0, num_blocks) for every used page, context
 *     lengths in [0, max_context_len], cu_seqlens non-decreasing.  Kernels
 *     clamp every index they read, so a broken promise gives unspecified
 *     numbers but never an access outside the caller's buffers; the KV write
 *     skips tokens whose block id is outside the pool.
 *
 * Layouts (row-major, innermost last)
 *   packed K/V            [T, Hkv, d]          T = total tokens of the batch
 *   decode q / out        [B, Hq, d]           one query token per sequence
 *   prefill q / out       [T, Hq, d]
 *   k_cache, v_cache      [num_blocks, Hkv, block_size, d]
 *   block_table           [B, max_blocks_per_seq]  logical page -> physical block
 *   cu_seqlens            [B + 1], cu_seqlens[0] = 0, cu_seqlens[B] = T
 *   extend q / out        [total_q, Hq, d], rows of sequence b at cu_q[b] ..
 */
#ifndef PAGED_GQA_H
#define PAGED_GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PGQA_F32 = 0, PGQA_BF16 = 1 } pgqa_dtype;

enum {
    PGQA_OK = 0,
    PGQA_EINVAL = 1,  /* invalid argument: null or misaligned pointer, negative size,
                         Hq % Hkv != 0, max_context_len beyond the block table, ... */
    PGQA_ENOTSUP = 2, /* valid but not built: head_dim, block_size, group size or dtype */
    PGQA_ENOSPC = 3,  /* decode workspace smaller than gqa_paged_decode_workspace_size() */
    PGQA_EHIP = 4     /* a HIP launch failed */
};

/* Flags of pgqa_check_contents (status[0]). */
enum {
    PGQA_CHECK_BLOCK_ID = 1,      /* a page the call would touch has a block id outside [0, num_blocks) */
    PGQA_CHECK_CONTEXT = 2,       /* a context length outside [0, max_context_len] (or a write past the table row) */
    PGQA_CHECK_ROWS = 4,          /* row offsets not starting at 0, decreasing, not ending at the row
                                     count, or a sequence with more rows than max_rows */
    PGQA_CHECK_SHORT_CONTEXT = 8  /* fewer cached positions than new query rows */
};

/* Supported shapes: head_dim in {16, 32, 64, 128}; block_size a power of two in
 * [1, 256]; Hq / Hkv in {1, 2, 4, 8, 16, 32, 64}. */

/*
 * paged_kv_write -- scatter packed new K/V rows into the page pools.
 * Defined by the paging passages above: token t of sequence b (cu_seqlens[b] <= t
 * < cu_seqlens[b+1]) is logical position pos = start_pos[b] + (t - cu_seqlens[b]);
 * it goes to block block_table[b][pos / block_size], slot pos % block_size, for
 * every KV head h:  k_cache[blk][h][slot][:] = k[t][h][:]  (same for v).
 * Bytes are copied unchanged (bit-exact).  Tokens whose page lies past the
 * table row or whose block id is outside [0, num_blocks) are skipped.
 *   k, v         [total_tokens, Hkv, d] packed new rows (read)
 *   cu_seqlens   [batch + 1] token offsets of each sequence in k / v
 *   start_pos    [batch] logical position of each sequence's first new token
 *   block_table  [batch, max_blocks_per_seq]
 *   k_cache, v_cache [num_blocks, Hkv, block_size, d] (written in place)
 */
int paged_kv_write(const void* k, const void* v,
                   const int32_t* cu_seqlens, const int32_t* start_pos,
                   const int32_t* block_table, int32_t max_blocks_per_seq,
                   void* k_cache, void* v_cache,
                   int32_t batch, int32_t total_tokens, int32_t num_blocks,
                   int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                   pgqa_dtype dtype, void* stream);

/*
 * paged_kv_gather -- the exact inverse of paged_kv_write: reads position
 * start_pos[b] + (t - cu_seqlens[b]) of sequence b out of the pools into packed
 * row t of k_out / v_out (bit-exact copy).  With start_pos = 0 and cu_seqlens
 * the prefix sums of the context lengths it unpacks every cached token.  Rows
 * whose page is past the table row or outside the pool are left untouched.
 * Exported so that the write can be checked on the device.
 */
int paged_kv_gather(const void* k_cache, const void* v_cache,
                    const int32_t* cu_seqlens, const int32_t* start_pos,
                    const int32_t* block_table, int32_t max_blocks_per_seq,
                    void* k_out, void* v_out,
                    int32_t batch, int32_t total_tokens, int32_t num_blocks,
                    int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                    pgqa_dtype dtype, void* stream);

/*
 * Bytes of device workspace gqa_paged_decode needs for these sizes: fp32
 * split-KV partials (running max, sum and unnormalised output per query head)
 * for at most (num_splits + batch * Hkv) pieces, and the per-sequence tile
 * counts the merge step reads (batch + 1 int32).  num_splits = 0 sizes it for
 * the library's own choice.  Returns 0 for invalid sizes.  Its contents need no
 * initialisation; two calls that may run at the same time must not share it.
 */
size_t gqa_paged_decode_workspace_size(int32_t batch, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       int32_t num_splits);

/*
 * gqa_paged_decode -- one query token per sequence attends to every cached
 * position [0, context_lens[b]) of its sequence (the decode phase reads the
 * whole KV cache of earlier tokens: the Ultimate Guide, introduction; the
 * lecture notes, section 2).  For query head qh, with h = qh / (Hq / Hkv):
 *   s_j = scale * dot(q[b][qh], K_j),  K_j = k_cache[block_table[b][j / bs]][h][j % bs]
 *   out[b][qh] = sum_j softmax(s)_j * V_j        (exact softmax; fp32 accumulation)
 * A sequence with context length 0 gets an all-zero output.
 * Work is split into num_splits equal shares of all (sequence, KV head) tiles
 * (0 = library choice, which fills the GPU); the partials of a sequence cut
 * across shares are merged exactly (log-sum-exp, in share order) by a second
 * kernel.  The result is deterministic for a given num_splits.  With
 * num_splits = 0 and max_context_len within two of the kernel's tiles (tiles of
 * 16 tokens for bf16 at head_dim 128, 32 at head_dim 64, 8 for fp32 at head_dim
 * 128, 64 at head_dim 16; FP8 pages twice the bf16 length), each (sequence, KV
 * head) gets one workgroup that writes its outputs directly and no merge kernel
 * runs.
 * With one KV head and Hq a multiple of 32 (bf16, head_dim 64 or 128, block_size
 * >= 8 for d 64 / >= 4 for d 128, window 0, num_splits 0), the call runs on the
 * matrix cores instead: the Hq query heads of a token are the rows of the MFMA
 * tile (Hq = 32: one tile of 16-row waves), the batch's key blocks are cut into
 * equal stream-K shares whose partials are merged by log-sum-exp (or, past 4,096
 * sequences or with a smaller workspace, into chunks of 20 blocks of 64 keys);
 * partials use the same workspace and the result is deterministic as well.
 *   q            [batch, Hq, d]
 *   k_cache, v_cache [num_blocks, Hkv, block_size, d]
 *   block_table  [batch, max_blocks_per_seq]; entries past ceil(ctx/bs) never read
 *   context_lens [batch]
 *   max_context_len  host-side upper bound of context_lens;
 *                    must be <= max_blocks_per_seq * block_size
 *   scale        softmax scale, normally 1/sqrt(head_dim); any finite value
 *   window       0, or > 0 for local attention: only positions
 *                [ctx - window, ctx) are attended to (see "Local attention" above);
 *                tiles wholly before the window are not read
 *   out          [batch, Hq, d] (written)
 *   workspace    >= gqa_paged_decode_workspace_size(batch, Hq, Hkv, d, num_splits) bytes
 * Errors: PGQA_EINVAL, PGQA_ENOTSUP, PGQA_ENOSPC (workspace too small), PGQA_EHIP.
 */
int gqa_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_table, int32_t max_blocks_per_seq,
                     const int32_t* context_lens,
                     int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t num_blocks,
                     int32_t max_context_len, float scale, int32_t window, pgqa_dtype dtype,
                     void* out, int32_t num_splits,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * gqa_paged_decode_noalloc -- gqa_paged_decode for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, result and errors
 * as gqa_paged_decode (bit-identical output for the same num_splits) without
 * the workspace: the split-KV partials go to a scratch array of 128 MiB that the
 * library holds on each GPU it runs on until the process ends (its device address
 * is looked up once per device, at the first call there).  The call allocates
 * nothing.  Sizes whose workspace, gqa_paged_decode_workspace_size(batch, Hq,
 * Hkv, head_dim, num_splits), exceeds 128 MiB return PGQA_ENOSPC (from about
 * 7,560 sequences with Hq 32, Hkv 8, head_dim 128).  The scratch needs no
 * initialisation, and every call on one GPU shares it: calls that may overlap on
 * one GPU (different streams, or host threads) race and give wrong results; the
 * caller serialises them.  PGQA_EHIP if the scratch cannot be located.
 */
int gqa_paged_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, int32_t max_blocks_per_seq,
                             const int32_t* context_lens,
                             int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t num_blocks,
                             int32_t max_context_len, float scale, int32_t window, pgqa_dtype dtype,
                             void* out, int32_t num_splits, void* stream);

/*
 * gqa_varlen_prefill -- packed variable-length prefill with a block-diagonal
 * mask (itinai.com/?p=48087, first paragraph; the lecture notes, section 8.1).
 * Row i of sequence s (cu_seqlens[s] <= i < cu_seqlens[s+1]), query head qh,
 * KV head h = qh / (Hq / Hkv):
 *   out[i][qh] = sum_j softmax_j(scale * dot(q[i][qh], k[j][h])) * v[j][h]
 * over keys j of the same sequence with j <= i (causal != 0) or all of them;
 * with window > 0 (causal only, else PGQA_EINVAL) also j > i - window.
 * QK^T and PV run on bf16 MFMA with fp32 accumulation; P is rounded to bf16
 * for the PV product.  bf16 only.
 *   q [total_tokens, Hq, d], k / v [total_tokens, Hkv, d], out [total_tokens, Hq, d]
 *   cu_seqlens [batch + 1]; max_seqlen = host-side upper bound of the lengths
 * Errors: PGQA_EINVAL (bad sizes or pointers, or a problem whose workgroup
 * count would pass 2^31: about (max_seqlen/32) * batch * Hq), PGQA_ENOTSUP
 * (fp32, head_dim other than 64 / 128, group size not 1, 2 or a multiple of 4
 * up to 64), PGQA_EHIP.
 */
int gqa_varlen_prefill(const void* q, const void* k, const void* v,
                       const int32_t* cu_seqlens, int32_t batch, int32_t total_tokens,
                       int32_t max_seqlen, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, float scale, int32_t causal, int32_t window,
                       pgqa_dtype dtype, void* out, void* stream);

/*
 * gqa_paged_extend -- q_len >= 1 new query tokens per sequence attend to the
 * sequence's paged cache: a chunk of a prompt prefilled on top of an already
 * cached (possibly shared) prefix (the lecture notes, section 8.2, "Prefix
 * Sharing"; the Ultimate Guide, section "Paged Attention"), or k draft tokens
 * that the target model checks in one parallel pass (the lecture notes,
 * section 7.1, speculative decoding).  The new
 * tokens' own K/V must already be in the pages (paged_kv_write), so the cache
 * holds ctx = context_lens[b] positions of which the last q_len are the new
 * ones.  Query row i of sequence b (0 <= i < q_len = cu_q[b+1] - cu_q[b]) sits
 * at position p = ctx - q_len + i and, like any causal row (the lecture notes,
 * section 2: a token depends on the tokens before it), sees
 * keys 0 .. p of the sequence (bottom-right aligned causal mask; with
 * window > 0 only keys p - window + 1 .. p, blocks before them are not read); with
 * q_len = 1 this is gqa_paged_decode, with ctx = q_len it is a causal prefill.
 * For query head qh, h = qh / (Hq / Hkv), K_j read through the block table as
 * in gqa_paged_decode:
 *   out[cu_q[b] + i][qh] = sum_{j <= p} softmax_j(scale * dot(q[cu_q[b] + i][qh], K_j)) V_j
 * A row with p < 0 (ctx < q_len, a broken promise) gets an all-zero output.
 * QK^T and PV run on bf16 MFMA with fp32 accumulation; P is rounded to bf16
 * for the PV product.  bf16 only.
 *   q, out       [total_q, Hq, d] packed new tokens
 *   cu_q         [batch + 1] query-row offsets, cu_q[0] = 0, cu_q[batch] = total_q
 *   k_cache, v_cache [num_blocks, Hkv, block_size, d]
 *   block_table  [batch, max_blocks_per_seq]
 *   context_lens [batch] cached positions per sequence, new tokens included
 *   max_q_len    host-side upper bound of the q_len of every sequence
 *   max_context_len  host-side upper bound of context_lens;
 *                    must be <= max_blocks_per_seq * block_size
 *   workspace    NULL, or device memory (16-byte aligned) of workspace_bytes for
 *                the key split (gqa_paged_extend_workspace_size); its contents
 *                need no initialisation; calls that may run at once must not share it
 * Errors: PGQA_EINVAL (bad sizes or pointers, or a grid past 2^31 workgroups),
 * PGQA_ENOTSUP (fp32; head_dim other than 64 / 128; group size not 1, 2 or a
 * multiple of 4 up to 64; block_size below 4 for head_dim 128 or below 8 for
 * head_dim 64, the rows one 1 KB load of the kernel covers), PGQA_EHIP.
 */
int gqa_paged_extend(const void* q, const int32_t* cu_q, const void* k_cache, const void* v_cache,
                     const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens,
                     int32_t batch, int32_t total_q, int32_t max_q_len,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int32_t num_blocks, int32_t max_context_len,
                     float scale, int32_t window, pgqa_dtype dtype, void* out,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace gqa_paged_extend can use for these sizes (0 when it
 * would not split).  Two ways of splitting write fp32 partials (running max, sum
 * and unnormalised output per row and query head) that a second kernel merges
 * exactly (log-sum-exp in key order; deterministic):
 *   - key chunks: when the call has too few (query tile, sequence, KV head)
 *     pieces to balance the GPU, long key ranges are cut into chunks handled by
 *     separate workgroups;
 *   - stream-K shares: when every sequence's query tokens times the group fit
 *     one 32-row tile (q_len * Hq / Hkv <= 32, e.g. a few draft tokens) and the
 *     call has at most 4,096 (sequence, KV head) pairs, all pairs' key blocks
 *     are cut into one equal share per workgroup slot of the GPU (about 17 MB
 *     at head_dim 128 on 256 CUs, whatever the lengths).
 * A smaller (or NULL) workspace only means fewer chunks, key chunks instead of
 * shares, or no split.  The size depends on the GPU's CU count (the current
 * device's).  Returns 0 for invalid sizes.
 */
size_t gqa_paged_extend_workspace_size(int32_t batch, int32_t total_q, int32_t max_q_len, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len);

/*
 * Low-precision KV pages.  The pages give only the byte sizes (bf16 2 bytes,
 * int8 1 byte: the lecture notes, section 6) and the motivation (a smaller KV
 * cache: the Ultimate Guide, section "KV Cache Compression"); the format is
 * this library's choice: FP8 E4M3 codes (OCP layout: bias 7, largest finite
 * 448, no infinity), one byte per value, in code pools laid out like the bf16
 * pools, [num_blocks, Hkv, block_size, d] uint8, and one fp32 scale per
 * (token, KV head) row in scale pools [num_blocks, Hkv, block_size].  A row x
 * is stored as codes c = nearest-even E4M3(x / s), s = max|x| / 448 (1 for an
 * all-zero row), both single-precision operations, and stands for c * s.  A
 * token's scale is fixed when it is written, so appending tokens never
 * re-quantises a page.
 *
 * paged_kv_write_fp8 -- paged_kv_write that quantises bf16 K/V rows into code
 * and scale pools (same positions, same skipping rules).  Errors as for
 * paged_kv_write; PGQA_ENOTSUP for an input dtype other than bf16.
 *
 * gqa_paged_decode_fp8 -- gqa_paged_decode over FP8 pages: the same result as
 * gqa_paged_decode over the values code * scale (bf16 q and out, fp32
 * accumulation; the K scale multiplies each score and the V scale each weight,
 * the codes are converted to bf16 exactly).  Same arguments, workspace
 * (gqa_paged_decode_workspace_size) and window as gqa_paged_decode, plus the
 * scale pools.  PGQA_ENOTSUP unless head_dim is 64 or 128 and block_size >= 16.
 */
int paged_kv_write_fp8(const void* k, const void* v, const int32_t* cu_seqlens, const int32_t* start_pos,
                       const int32_t* block_table, int32_t max_blocks_per_seq, void* k_cache, void* v_cache,
                       float* k_scale, float* v_scale, int32_t batch, int32_t total_tokens, int32_t num_blocks,
                       int32_t block_size, int32_t num_kv_heads, int32_t head_dim, pgqa_dtype dtype,
                       void* stream);

int gqa_paged_decode_fp8(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                         const float* v_scale, const int32_t* block_table, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_context_len,
                         float scale, int32_t window, void* out, int32_t num_splits, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * gqa_paged_extend_fp8 -- gqa_paged_extend over FP8 pages: the same result as
 * gqa_paged_extend over the values code * scale (bf16 q and out, fp32
 * accumulation; each tile of codes is converted to bf16 exactly in LDS and the
 * MFMA products are the bf16 ones; the K scale multiplies each score, the V
 * scale each weight before its bf16 rounding, and the row sum adds the
 * unrounded weights).  Same arguments, mask, window and workspace
 * (gqa_paged_extend_workspace_size) as gqa_paged_extend, plus the scale pools
 * [num_blocks, Hkv, block_size] fp32 (k_scale, v_scale, both non-NULL).
 * Errors as for gqa_paged_extend; PGQA_ENOTSUP also for block_size below
 * 1024 / head_dim (8 for head_dim 128, 16 for 64: the rows one 1 KB load of
 * codes covers); PGQA_EINVAL also for scale pools of 4 GiB or more.
 */
int gqa_paged_extend_fp8(const void* q, const int32_t* cu_q, const void* k_cache, const void* v_cache,
                         const float* k_scale, const float* v_scale, const int32_t* block_table,
                         int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch, int32_t total_q,
                         int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, int32_t max_context_len, float scale,
                         int32_t window, void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_kv_copy_blocks -- the device half of copy-on-write (the lecture notes,
 * section 8.2, "Prefix Sharing (Copy-on-Write)": when sequences sharing prefix
 * blocks diverge, only the block being modified is copied).  For every pair p,
 * the whole of block src_blocks[p] (all KV heads, all block_size slots) is
 * copied bit for bit onto block dst_blocks[p], in the K pool and in the V pool.
 * Pairs run concurrently: no dst may equal another pair's src or dst (the
 * caller's promise; pgqa_bm_append never produces such pairs within one step).
 * Pairs with an id outside [0, num_blocks) are skipped.
 *   k_cache, v_cache  [num_blocks, Hkv, block_size, d] (modified in place)
 *   src_blocks, dst_blocks  [num_pairs] device int32 arrays
 * Errors: PGQA_EINVAL, PGQA_ENOTSUP (head_dim, block_size or dtype), PGQA_EHIP.
 */
int paged_kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_blocks, const int32_t* dst_blocks,
                         int32_t num_pairs, int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                         int32_t head_dim, pgqa_dtype dtype, void* stream);

/*
 * Block manager -- host-side bookkeeping of refcounted KV blocks with
 * copy-on-write, the block tables the calls above read.  Pages: a sequence's
 * cache is a list of fixed-size blocks taken from the pool only when a token
 * needs one and given back when the request ends (the Ultimate Guide, section
 * "Paged Attention"); blocks carry a reference counter, several sequences may
 * point at the same prefix blocks, and when they diverge only the modified
 * block is copied (the lecture notes, section 8.2, "Prefix Sharing").
 *
 * Unlike every call above, these are HOST-only calls on a host object: pointer
 * arguments are host memory, nothing touches the GPU, and a manager must not be
 * used by two threads at once.  Policy: new blocks are the lowest-numbered free
 * ones; new sequences get the lowest unused id (>= 0).
 *
 *   pgqa_bm_create(num_blocks, block_size)  NULL for sizes <= 0 or no memory.
 *   pgqa_bm_new_sequence(bm, &seq)          an empty sequence.
 *   pgqa_bm_fork(bm, parent, &child)        child shares all of parent's blocks
 *                                           (one more reference each) and its length.
 *   pgqa_bm_append(bm, seq, n, &src, &dst)  room for n more tokens (positions
 *       len .. len+n-1).  If the last block is partly filled and shared, it is
 *       replaced by a fresh block and (src, dst) = (old, new) is returned: copy
 *       that block on the device (paged_kv_copy_blocks) before writing the new
 *       tokens; otherwise src = dst = -1.  Pages past the old end get fresh
 *       blocks.  PGQA_ENOSPC when the pool lacks free blocks (nothing changes);
 *       PGQA_EINVAL for an unknown sequence or n < 0.
 *   pgqa_bm_free_sequence(bm, seq)          drops one reference to each of its
 *                                           blocks; blocks at zero become free.
 *   pgqa_bm_sequence_length / pgqa_bm_refcount / pgqa_bm_num_free_blocks
 *                                           -1 for an unknown sequence / block.
 *   pgqa_bm_block_table(bm, seq, pages, capacity)  writes up to capacity block
 *       ids of the sequence's pages (logical order) to host memory; returns its
 *       page count (-1 for an unknown sequence).
 */
typedef struct pgqa_block_manager pgqa_block_manager;

pgqa_block_manager* pgqa_bm_create(int32_t num_blocks, int32_t block_size);
void pgqa_bm_destroy(pgqa_block_manager* bm);
int pgqa_bm_new_sequence(pgqa_block_manager* bm, int32_t* seq);
int pgqa_bm_fork(pgqa_block_manager* bm, int32_t parent, int32_t* child);
int pgqa_bm_append(pgqa_block_manager* bm, int32_t seq, int32_t num_tokens, int32_t* copy_src,
                   int32_t* copy_dst);
int pgqa_bm_free_sequence(pgqa_block_manager* bm, int32_t seq);
int32_t pgqa_bm_sequence_length(const pgqa_block_manager* bm, int32_t seq);
int32_t pgqa_bm_block_table(const pgqa_block_manager* bm, int32_t seq, int32_t* pages, int32_t capacity);
int32_t pgqa_bm_refcount(const pgqa_block_manager* bm, int32_t block);
int32_t pgqa_bm_num_free_blocks(const pgqa_block_manager* bm);

/* Static, human-readable text of a status code. */
const char* pgqa_status_string(int status);

/*
 * pgqa_check_contents -- debugging aid: checks on the device the promises the
 * calls above take on trust about device array contents (the conventions
 * section: block ids of every used page inside the pool, which the paging
 * passages require of a block table; context lengths within the host bound;
 * row offsets non-decreasing from 0 to the row count, as a packed batch's
 * offsets are by construction, itinai.com/?p=48087, first paragraph).  It
 * reads and reports, nothing else; the hot path never runs it.  Pass the
 * arrays of the call to be checked:
 *   decode:   block_table, context_lens (cu_rows = start_pos = NULL); with
 *             window > 0 only pages from ctx - window on are checked
 *   extend:   block_table, context_lens, cu_rows = cu_q, total_rows = total_q,
 *             max_rows = max_q_len (pages from the first row's window edge on)
 *   prefill:  cu_rows = cu_seqlens, total_rows, max_rows = max_seqlen
 *   KV write: block_table, cu_rows = cu_seqlens, start_pos (the pages of the
 *             written positions, which the write skips when their id is bad)
 * NULL arrays are not checked; max_rows < 0 leaves the per-sequence row count
 * unchecked.  The kernels read only inside the caller's arrays whatever the
 * contents (a length past the table row is cut to it).
 *   status   device int32[4], written in stream order: [0] PGQA_CHECK_* flags
 *            (0: every promise kept), [1] the lowest sequence with a
 *            violation (INT32_MAX if none), [2] the number of bad block-table
 *            entries, [3] the number of sequences with a violation.
 * Errors: PGQA_EINVAL (null or misaligned status, negative sizes, start_pos
 * without cu_rows, a block table without num_blocks / max_blocks_per_seq > 0),
 * PGQA_ENOTSUP (block_size not a power of two up to 256), PGQA_EHIP.
 */
int pgqa_check_contents(const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens,
                        const int32_t* cu_rows, const int32_t* start_pos, int32_t batch, int32_t total_rows,
                        int32_t max_rows, int32_t num_blocks, int32_t block_size, int32_t max_context_len,
                        int32_t window, int32_t* status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_GQA_H */
