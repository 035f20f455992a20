// api.cpp -- the C ABI of libpaged_gqa.so (declared in include/paged_gqa.h):
// host-side argument checks, then launches on the caller's stream.  Every check
// runs before any HIP call, so a rejected call enqueues nothing.
#include "paged_gqa.h"

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "launch.hpp"

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool pow2_log2(int32_t x, int32_t* lg) {
    if (x <= 0 || (x & (x - 1))) return false;
    int32_t l = 0;
    while ((1 << l) < x) ++l;
    *lg = l;
    return true;
}

bool head_dim_ok(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

int elem_bytes(pgqa_dtype dt) { return dt == PGQA_BF16 ? 2 : (dt == PGQA_F32 ? 4 : 0); }

constexpr int32_t kMaxDecodeBatch = 8192;

int check_elem_ptr(const void* p) { return (p && aligned(p, 16)) ? PGQA_OK : PGQA_EINVAL; }
int check_index_ptr(const void* p) { return (p && aligned(p, 4)) ? PGQA_OK : PGQA_EINVAL; }

int check_copy_args(const void* a, const void* b, const int32_t* cu, const int32_t* sp, const int32_t* bt,
                    int32_t max_blocks_per_seq, void* c, void* d, int32_t batch, int32_t total_tokens,
                    int32_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                    pgqa_dtype dtype, int32_t* bs_log2) {
    if (batch < 0 || total_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0)
        return PGQA_EINVAL;
    if (elem_bytes(dtype) == 0) return PGQA_ENOTSUP;
    if (!head_dim_ok(head_dim)) return PGQA_ENOTSUP;
    if (!pow2_log2(block_size, bs_log2) || block_size > 256) return PGQA_ENOTSUP;
    if ((int64_t)batch * max_blocks_per_seq > INT32_MAX) return PGQA_EINVAL;
    if (check_elem_ptr(a) || check_elem_ptr(b) || check_elem_ptr(c) || check_elem_ptr(d)) return PGQA_EINVAL;
    if (check_index_ptr(cu) || check_index_ptr(sp) || check_index_ptr(bt)) return PGQA_EINVAL;
    return PGQA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? PGQA_OK : PGQA_EHIP; }

}  // namespace

extern "C" {

const char* pgqa_status_string(int status) {
    switch (status) {
        case PGQA_OK: return "ok";
        case PGQA_EINVAL: return "invalid argument";
        case PGQA_ENOTSUP: return "unsupported shape or dtype";
        case PGQA_ENOSPC: return "decode workspace too small";
        case PGQA_EHIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

int paged_kv_write(const void* k, const void* v, const int32_t* cu_seqlens, const int32_t* start_pos,
                   const int32_t* block_table, int32_t max_blocks_per_seq, void* k_cache, void* v_cache,
                   int32_t batch, int32_t total_tokens, int32_t num_blocks, int32_t block_size,
                   int32_t num_kv_heads, int32_t head_dim, pgqa_dtype dtype, void* stream) {
    int32_t lg = 0;
    const int rc = check_copy_args(k, v, cu_seqlens, start_pos, block_table, max_blocks_per_seq, k_cache, v_cache,
                                   batch, total_tokens, num_blocks, block_size, num_kv_heads, head_dim, dtype, &lg);
    if (rc != PGQA_OK) return rc;
    if (batch == 0 || total_tokens == 0) return PGQA_OK;
    pgqa::KvCopyLaunch L{k, v, k_cache, v_cache, cu_seqlens, start_pos, block_table, max_blocks_per_seq,
                         batch, total_tokens, num_blocks, lg, num_kv_heads, head_dim, elem_bytes(dtype)};
    return hip_status(pgqa::launch_kv_copy(L, true, (hipStream_t)stream));
}

int paged_kv_gather(const void* k_cache, const void* v_cache, const int32_t* cu_seqlens, const int32_t* start_pos,
                    const int32_t* block_table, int32_t max_blocks_per_seq, void* k_out, void* v_out,
                    int32_t batch, int32_t total_tokens, int32_t num_blocks, int32_t block_size,
                    int32_t num_kv_heads, int32_t head_dim, pgqa_dtype dtype, void* stream) {
    int32_t lg = 0;
    const int rc = check_copy_args(k_cache, v_cache, cu_seqlens, start_pos, block_table, max_blocks_per_seq, k_out,
                                   v_out, batch, total_tokens, num_blocks, block_size, num_kv_heads, head_dim,
                                   dtype, &lg);
    if (rc != PGQA_OK) return rc;
    if (batch == 0 || total_tokens == 0) return PGQA_OK;
    pgqa::KvCopyLaunch L{k_cache, v_cache, k_out, v_out, cu_seqlens, start_pos, block_table, max_blocks_per_seq,
                         batch, total_tokens, num_blocks, lg, num_kv_heads, head_dim, elem_bytes(dtype)};
    return hip_status(pgqa::launch_kv_copy(L, false, (hipStream_t)stream));
}

int paged_kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_blocks, const int32_t* dst_blocks,
                         int32_t num_pairs, int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                         int32_t head_dim, pgqa_dtype dtype, void* stream) {
    if (num_pairs < 0 || num_blocks <= 0 || num_kv_heads <= 0) return PGQA_EINVAL;
    if (elem_bytes(dtype) == 0 || !head_dim_ok(head_dim)) return PGQA_ENOTSUP;
    int32_t lg = 0;
    if (!pow2_log2(block_size, &lg) || block_size > 256) return PGQA_ENOTSUP;
    if (check_elem_ptr(k_cache) || check_elem_ptr(v_cache)) return PGQA_EINVAL;
    if (check_index_ptr(src_blocks) || check_index_ptr(dst_blocks)) return PGQA_EINVAL;
    if (num_pairs == 0) return PGQA_OK;
    pgqa::BlockCopyLaunch L{k_cache, v_cache, src_blocks, dst_blocks, num_pairs, num_blocks, block_size,
                            num_kv_heads, head_dim, elem_bytes(dtype)};
    return hip_status(pgqa::launch_block_copy(L, (hipStream_t)stream));
}

size_t gqa_paged_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t num_splits) {
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || num_splits < 0) return 0;
    if (num_q_heads % num_kv_heads) return 0;
    return pgqa::decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, num_splits);
}

// Host-side checks of gqa_paged_decode's arguments other than the workspace;
// block_size's log2 in *lg.
static int check_decode_args(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                             int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t max_context_len, float scale, int32_t window,
                             pgqa_dtype dtype, const void* out, int32_t num_splits, int32_t* lg) {
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 ||
        max_context_len < 0 || num_splits < 0 || window < 0)
        return PGQA_EINVAL;
    if (num_q_heads % num_kv_heads) return PGQA_EINVAL;
    const int es = elem_bytes(dtype);
    if (es == 0 || !head_dim_ok(head_dim)) return PGQA_ENOTSUP;
    if (!pow2_log2(block_size, lg) || block_size > 256) return PGQA_ENOTSUP;
    if (!pgqa::decode_supported(es, head_dim, num_q_heads / num_kv_heads)) return PGQA_ENOTSUP;
    if (batch > kMaxDecodeBatch) return PGQA_ENOTSUP;
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PGQA_EINVAL;
    if ((int64_t)batch * max_blocks_per_seq > INT32_MAX) return PGQA_EINVAL;
    if ((int64_t)batch * num_kv_heads * (int64_t)max_context_len > INT32_MAX) return PGQA_EINVAL;
    if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff()) return PGQA_EINVAL;
    if (check_elem_ptr(q) || check_elem_ptr(k_cache) || check_elem_ptr(v_cache) || check_elem_ptr(out))
        return PGQA_EINVAL;
    if (check_index_ptr(block_table) || check_index_ptr(context_lens)) return PGQA_EINVAL;
    return PGQA_OK;
}

int gqa_paged_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                     int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                     int32_t max_context_len, float scale, int32_t window, pgqa_dtype dtype, void* out,
                     int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream) {
    int32_t lg = 0;
    const int rc = check_decode_args(q, k_cache, v_cache, block_table, max_blocks_per_seq, context_lens, batch,
                                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_context_len,
                                     scale, window, dtype, out, num_splits, &lg);
    if (rc != PGQA_OK) return rc;
    if (batch == 0) return PGQA_OK;
    const size_t need = gqa_paged_decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, num_splits);
    if (!workspace || !aligned(workspace, 16)) return workspace_bytes < need ? PGQA_ENOSPC : PGQA_EINVAL;
    if (workspace_bytes < need) return PGQA_ENOSPC;
    pgqa::DecodeLaunch L{q, k_cache, v_cache, block_table, context_lens, out, workspace, max_blocks_per_seq,
                         batch, num_q_heads, num_kv_heads, head_dim, lg, num_blocks, max_context_len,
                         num_splits, dtype == PGQA_BF16 ? 1 : 0, scale, window, nullptr, nullptr};
    return hip_status(pgqa::launch_decode(L, (hipStream_t)stream));
}

int gqa_paged_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                             int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t max_context_len, float scale, int32_t window,
                             pgqa_dtype dtype, void* out, int32_t num_splits, void* stream) {
    int32_t lg = 0;
    const int rc = check_decode_args(q, k_cache, v_cache, block_table, max_blocks_per_seq, context_lens, batch,
                                     num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_context_len,
                                     scale, window, dtype, out, num_splits, &lg);
    if (rc != PGQA_OK) return rc;
    if (batch == 0) return PGQA_OK;
    // The same partials gqa_paged_decode would need, in the library's own scratch.
    const size_t need = gqa_paged_decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, num_splits);
    if (need > pgqa::kDecodeScratchBytes) return PGQA_ENOSPC;
    void* scratch = pgqa::decode_scratch();
    if (!scratch) return PGQA_EHIP;
    pgqa::DecodeLaunch L{q, k_cache, v_cache, block_table, context_lens, out, scratch, max_blocks_per_seq,
                         batch, num_q_heads, num_kv_heads, head_dim, lg, num_blocks, max_context_len,
                         num_splits, dtype == PGQA_BF16 ? 1 : 0, scale, window, nullptr, nullptr};
    return hip_status(pgqa::launch_decode(L, (hipStream_t)stream));
}

size_t gqa_paged_extend_workspace_size(int32_t batch, int32_t total_q, int32_t max_q_len, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len) {
    if (batch <= 0 || total_q <= 0 || max_q_len <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0)
        return 0;
    if (num_q_heads % num_kv_heads) return 0;
    return pgqa::extend_workspace_bytes(batch, total_q, max_q_len, num_q_heads, num_kv_heads, head_dim,
                                        max_context_len);
}

int paged_kv_write_fp8(const void* k, const void* v, const int32_t* cu_seqlens, const int32_t* start_pos,
                       const int32_t* block_table, int32_t max_blocks_per_seq, void* k_cache, void* v_cache,
                       float* k_scale, float* v_scale, int32_t batch, int32_t total_tokens, int32_t num_blocks,
                       int32_t block_size, int32_t num_kv_heads, int32_t head_dim, pgqa_dtype dtype, void* stream) {
    int32_t lg = 0;
    const int rc = check_copy_args(k, v, cu_seqlens, start_pos, block_table, max_blocks_per_seq, k_cache, v_cache,
                                   batch, total_tokens, num_blocks, block_size, num_kv_heads, head_dim, dtype, &lg);
    if (rc != PGQA_OK) return rc;
    if (dtype != PGQA_BF16) return PGQA_ENOTSUP;
    if (check_index_ptr(k_scale) || check_index_ptr(v_scale)) return PGQA_EINVAL;
    if (batch == 0 || total_tokens == 0) return PGQA_OK;
    pgqa::KvCopyLaunch L{k, v, k_cache, v_cache, cu_seqlens, start_pos, block_table, max_blocks_per_seq,
                         batch, total_tokens, num_blocks, lg, num_kv_heads, head_dim, 2};
    return hip_status(pgqa::launch_kv_write_fp8(L, k_scale, v_scale, (hipStream_t)stream));
}

int gqa_paged_decode_fp8(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                         const float* v_scale, const int32_t* block_table, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_context_len,
                         float scale, int32_t window, void* out, int32_t num_splits, void* workspace,
                         size_t workspace_bytes, void* stream) {
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 ||
        max_context_len < 0 || num_splits < 0 || window < 0)
        return PGQA_EINVAL;
    if (num_q_heads % num_kv_heads) return PGQA_EINVAL;
    int32_t lg = 0;
    if (!pow2_log2(block_size, &lg) || block_size > 256) return PGQA_ENOTSUP;
    if (!pgqa::decode_fp8_supported(head_dim, num_q_heads / num_kv_heads, block_size)) return PGQA_ENOTSUP;
    if (batch > kMaxDecodeBatch) return PGQA_ENOTSUP;
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PGQA_EINVAL;
    if ((int64_t)batch * max_blocks_per_seq > INT32_MAX) return PGQA_EINVAL;
    if ((int64_t)batch * num_kv_heads * (int64_t)max_context_len > INT32_MAX) return PGQA_EINVAL;
    if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff()) return PGQA_EINVAL;
    if (check_elem_ptr(q) || check_elem_ptr(k_cache) || check_elem_ptr(v_cache) || check_elem_ptr(out))
        return PGQA_EINVAL;
    if (check_index_ptr(k_scale) || check_index_ptr(v_scale) || check_index_ptr(block_table) ||
        check_index_ptr(context_lens))
        return PGQA_EINVAL;
    if (batch == 0) return PGQA_OK;
    const size_t need = gqa_paged_decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, num_splits);
    if (!workspace || !aligned(workspace, 16)) return workspace_bytes < need ? PGQA_ENOSPC : PGQA_EINVAL;
    if (workspace_bytes < need) return PGQA_ENOSPC;
    pgqa::DecodeLaunch L{q, k_cache, v_cache, block_table, context_lens, out, workspace, max_blocks_per_seq,
                         batch, num_q_heads, num_kv_heads, head_dim, lg, num_blocks, max_context_len,
                         num_splits, 1, scale, window, k_scale, v_scale};
    return hip_status(pgqa::launch_decode(L, (hipStream_t)stream));
}

int gqa_varlen_prefill(const void* q, const void* k, const void* v, const int32_t* cu_seqlens, int32_t batch,
                       int32_t total_tokens, int32_t max_seqlen, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, float scale, int32_t causal, int32_t window, pgqa_dtype dtype,
                       void* out, void* stream) {
    if (batch < 0 || total_tokens < 0 || max_seqlen < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || window < 0)
        return PGQA_EINVAL;
    if (window > 0 && !causal) return PGQA_EINVAL;
    if (num_q_heads % num_kv_heads) return PGQA_EINVAL;
    if (dtype != PGQA_BF16 && dtype != PGQA_F32) return PGQA_ENOTSUP;
    if (dtype != PGQA_BF16) return PGQA_ENOTSUP;
    if (!pgqa::prefill_supported(head_dim, num_q_heads / num_kv_heads)) return PGQA_ENOTSUP;
    if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff()) return PGQA_EINVAL;
    if ((int64_t)total_tokens * num_q_heads * head_dim > ((int64_t)1 << 40)) return PGQA_EINVAL;
    // Grid size (one workgroup per 32-row query tile, head group and sequence)
    // and 32-bit K/V offsets inside a 64-key block.
    if ((int64_t)(max_seqlen / 32 + 1) * ((int64_t)batch * num_kv_heads + 7) * (num_q_heads / num_kv_heads) >
        INT32_MAX)
        return PGQA_EINVAL;
    if ((int64_t)num_kv_heads * head_dim * 2 * 64 > INT32_MAX) return PGQA_EINVAL;
    if (check_elem_ptr(q) || check_elem_ptr(k) || check_elem_ptr(v) || check_elem_ptr(out)) return PGQA_EINVAL;
    if (check_index_ptr(cu_seqlens)) return PGQA_EINVAL;
    if (batch == 0 || total_tokens == 0 || max_seqlen == 0) return PGQA_OK;
    pgqa::PrefillLaunch L{q, k, v, cu_seqlens, out, batch, total_tokens, max_seqlen, num_q_heads, num_kv_heads,
                          head_dim, causal ? 1 : 0, scale, window};
    return hip_status(pgqa::launch_prefill(L, (hipStream_t)stream));
}

// Shared checks and launch of gqa_paged_extend and gqa_paged_extend_fp8
// (k_scale / v_scale null: bf16 pages).
static int extend_call(const void* q, const int32_t* cu_q, const void* k_cache, const void* v_cache,
                       const float* k_scale, const float* v_scale, const int32_t* block_table,
                       int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch, int32_t total_q,
                       int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks, int32_t max_context_len, float scale, int32_t window,
                       pgqa_dtype dtype, void* out, void* workspace, size_t workspace_bytes, void* stream) {
    const bool fp8 = k_scale != nullptr || v_scale != nullptr;
    if (batch < 0 || total_q < 0 || max_q_len < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
        max_blocks_per_seq <= 0 || max_context_len < 0 || window < 0)
        return PGQA_EINVAL;
    if (num_q_heads % num_kv_heads) return PGQA_EINVAL;
    if (dtype != PGQA_BF16) return PGQA_ENOTSUP;
    int32_t lg = 0;
    if (!pow2_log2(block_size, &lg) || block_size > 256) return PGQA_ENOTSUP;
    if (fp8 ? !pgqa::extend_supported_fp8(head_dim, num_q_heads / num_kv_heads, block_size)
            : !pgqa::extend_supported(head_dim, num_q_heads / num_kv_heads, block_size))
        return PGQA_ENOTSUP;
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PGQA_EINVAL;
    // The kernel addresses a scale pool with 32-bit byte offsets.
    if (fp8 && (int64_t)num_blocks * num_kv_heads * block_size * 4 > UINT32_MAX) return PGQA_EINVAL;
    if (fp8 && (check_index_ptr(k_scale) || check_index_ptr(v_scale))) return PGQA_EINVAL;
    if ((int64_t)batch * max_blocks_per_seq > INT32_MAX) return PGQA_EINVAL;
    if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff()) return PGQA_EINVAL;
    if ((int64_t)total_q * num_q_heads * head_dim > ((int64_t)1 << 40)) return PGQA_EINVAL;
    // Grid size: one workgroup per 32-row query tile, head group and sequence.
    if ((int64_t)(max_q_len / 32 + 1) * ((int64_t)batch * num_kv_heads + 7) * (num_q_heads / num_kv_heads) >
        INT32_MAX)
        return PGQA_EINVAL;
    if (check_elem_ptr(q) || check_elem_ptr(k_cache) || check_elem_ptr(v_cache) || check_elem_ptr(out))
        return PGQA_EINVAL;
    if (check_index_ptr(cu_q) || check_index_ptr(block_table) || check_index_ptr(context_lens)) return PGQA_EINVAL;
    if (workspace && !aligned(workspace, 16)) return PGQA_EINVAL;
    if (batch == 0 || total_q == 0 || max_q_len == 0) return PGQA_OK;
    pgqa::ExtendLaunch L{q, k_cache, v_cache, cu_q, block_table, context_lens, out, batch, total_q, max_q_len,
                         max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, lg, num_blocks,
                         max_context_len, scale, window, workspace, workspace ? workspace_bytes : 0};
    L.k_scale = k_scale;
    L.v_scale = v_scale;
    return hip_status(pgqa::launch_extend(L, (hipStream_t)stream));
}

int gqa_paged_extend(const void* q, const int32_t* cu_q, const void* k_cache, const void* v_cache,
                     const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens,
                     int32_t batch, int32_t total_q, int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_context_len, float scale,
                     int32_t window, pgqa_dtype dtype, void* out, void* workspace, size_t workspace_bytes,
                     void* stream) {
    return extend_call(q, cu_q, k_cache, v_cache, nullptr, nullptr, block_table, max_blocks_per_seq, context_lens,
                       batch, total_q, max_q_len, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_context_len, scale, window, dtype, out, workspace, workspace_bytes, stream);
}

int gqa_paged_extend_fp8(const void* q, const int32_t* cu_q, const void* k_cache, const void* v_cache,
                         const float* k_scale, const float* v_scale, const int32_t* block_table,
                         int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch, int32_t total_q,
                         int32_t max_q_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, int32_t max_context_len, float scale,
                         int32_t window, void* out, void* workspace, size_t workspace_bytes, void* stream) {
    if (!k_scale || !v_scale) return PGQA_EINVAL;
    return extend_call(q, cu_q, k_cache, v_cache, k_scale, v_scale, block_table, max_blocks_per_seq, context_lens,
                       batch, total_q, max_q_len, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_context_len, scale, window, PGQA_BF16, out, workspace, workspace_bytes, stream);
}

int pgqa_check_contents(const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens,
                        const int32_t* cu_rows, const int32_t* start_pos, int32_t batch, int32_t total_rows,
                        int32_t max_rows, int32_t num_blocks, int32_t block_size, int32_t max_context_len,
                        int32_t window, int32_t* status, void* stream) {
    if (check_index_ptr(status) || batch < 0 || total_rows < 0 || max_context_len < 0 || window < 0)
        return PGQA_EINVAL;
    if (start_pos && !cu_rows) return PGQA_EINVAL;
    int32_t lg = 0;
    if (block_table) {
        if (max_blocks_per_seq <= 0 || num_blocks <= 0) return PGQA_EINVAL;
        if (!pow2_log2(block_size, &lg) || block_size > 256) return PGQA_ENOTSUP;
        if ((int64_t)batch * max_blocks_per_seq > INT32_MAX) return PGQA_EINVAL;
    }
    if ((block_table && check_index_ptr(block_table)) || (context_lens && check_index_ptr(context_lens)) ||
        (cu_rows && check_index_ptr(cu_rows)) || (start_pos && check_index_ptr(start_pos)))
        return PGQA_EINVAL;
    pgqa::CheckLaunch L{block_table, context_lens, cu_rows, start_pos, status, max_blocks_per_seq, batch,
                        total_rows, max_rows, num_blocks, lg, max_context_len, window};
    return hip_status(pgqa::launch_check(L, (hipStream_t)stream));
}

}  // extern "C"
