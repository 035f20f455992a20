// launch.hpp -- internal host-side launch descriptors of libpaged_gqa.so.
// Validation happens in api.cpp; these launchers assume valid arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "paged_gqa.h"

namespace pgqa {

// The softmax scale as the attention kernels apply it.  They take the running
// maximum of the raw dot products and fold the scale into the exponent,
// exp2(s * cs - m * cs), which needs cs > 0.  Any finite scale is reduced to that
// case exactly: s * scale = (sign(scale) q) . k * |scale|, and the kernels apply
// the sign to the query bits when they load them (q_and clears, q_xor flips the
// sign bit of every element; a zero scale zeroes the query, so every visible key
// gets the same weight).  cs = |scale| * log2(e) (log2(e) for a zero scale).
struct ScaleFold {
    float cs;
    uint32_t q_and;
    uint32_t q_xor;
};

inline ScaleFold fold_scale(float scale, bool bf16) {
    const double log2e = 1.4426950408889634;
    const uint32_t sign = bf16 ? 0x80008000u : 0x80000000u;
    if (scale > 0.0f) return {(float)((double)scale * log2e), 0xffffffffu, 0u};
    if (scale < 0.0f) return {(float)(-(double)scale * log2e), 0xffffffffu, sign};
    return {(float)log2e, 0u, 0u};
}

struct KvCopyLaunch {
    const void* src_k;
    const void* src_v;
    void* dst_k;
    void* dst_v;
    const int32_t* cu_seqlens;
    const int32_t* start_pos;
    const int32_t* block_table;
    int32_t max_blocks_per_seq;
    int32_t batch;
    int32_t total_tokens;
    int32_t num_blocks;
    int32_t block_size_log2;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t elem_bytes;
};

// to_pages = true: packed -> pages; false: pages -> packed.
hipError_t launch_kv_copy(const KvCopyLaunch& L, bool to_pages, hipStream_t stream);

// Quantising write of bf16 rows into FP8 E4M3 code pools (dst_k / dst_v) and fp32
// row-scale pools [num_blocks, Hkv, block_size]; head_dim in {16, 32, 64, 128}.
hipError_t launch_kv_write_fp8(const KvCopyLaunch& L, void* k_scale, void* v_scale, hipStream_t stream);

struct BlockCopyLaunch {
    void* k_cache;
    void* v_cache;
    const int32_t* src;
    const int32_t* dst;
    int32_t num_pairs;
    int32_t num_blocks;
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t elem_bytes;
};

hipError_t launch_block_copy(const BlockCopyLaunch& L, hipStream_t stream);

struct DecodeLaunch {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_table;
    const int32_t* context_lens;
    void* out;
    void* workspace;
    int32_t max_blocks_per_seq;
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size_log2;
    int32_t num_blocks;
    int32_t max_context_len;
    int32_t num_splits;   // 0 = choose
    int32_t is_bf16;
    float scale;
    int32_t window;       // 0: none; > 0: the newest `window` positions only
    const void* k_scale;  // non-null: FP8 E4M3 pages with fp32 row scales (bf16 q / out)
    const void* v_scale;
};

// Largest number of splits (workgroups of the split-KV kernel) the library picks itself.
constexpr int32_t kDecodeMaxSplits = 4096;

// Tokens per tile of the decode kernel for this element size and head_dim.
int32_t decode_tile_tokens(int32_t elem_bytes, int32_t head_dim);

// Is there a decode kernel for this (dtype, head_dim, group size)?
bool decode_supported(int32_t elem_bytes, int32_t head_dim, int32_t group);

// ... for FP8 pages with bf16 queries?
bool decode_fp8_supported(int32_t head_dim, int32_t group, int32_t block_size);

hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream);

// Decode workspace: fp32 partials for (splits + batch * Hkv) pieces x G heads x (head_dim + 2), then
// (batch + 1) int32 tile prefix sums.
size_t decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t num_splits);

// Size of the library's own device scratch, which takes the place of the
// caller's workspace in the allocation-free decode entry point.
constexpr size_t kDecodeScratchBytes = (size_t)128 << 20;

// Device address of that scratch on the current device (looked up once per
// device); null if the lookup fails.
void* decode_scratch();

struct PrefillLaunch {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* cu_seqlens;
    void* out;
    int32_t batch;
    int32_t total_tokens;
    int32_t max_seqlen;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t causal;
    float scale;
    int32_t window;   // 0: none; > 0: keys i - window + 1 .. i (causal only)
};

bool prefill_supported(int32_t head_dim, int32_t group);

hipError_t launch_prefill(const PrefillLaunch& L, hipStream_t stream);

struct ExtendLaunch {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* cu_q;
    const int32_t* block_table;
    const int32_t* context_lens;
    void* out;
    int32_t batch;
    int32_t total_q;
    int32_t max_q_len;
    int32_t max_blocks_per_seq;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t block_size_log2;
    int32_t num_blocks;
    int32_t max_context_len;
    float scale;
    int32_t window;   // 0: none; > 0: keys p - window + 1 .. p for a row at position p
    void* workspace;  // key-split partials (may be null: no split)
    size_t workspace_bytes;
    int32_t non_causal;  // 1: every row sees all keys [0, ctx) (rows = query heads of one token)
    int32_t fixed_qlen;  // > 0: sequence s holds rows [s * fixed_qlen, (s + 1) * fixed_qlen); cu_q unused
    int32_t chunk_blocks;  // > 0: key chunks of this many 64-key blocks (0: the library's choice)
    // FP8 pages: k_cache / v_cache hold E4M3 codes and these the fp32 row scales
    // [num_blocks, Hkv, block_size]; null for bf16 pages.
    const float* k_scale;
    const float* v_scale;
};

// Workspace bytes for the library's key split of a paged multi-token call (0: none).
size_t extend_workspace_bytes(int32_t batch, int32_t total_q, int32_t max_q_len, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len);

// Is there a paged multi-token kernel for this (head_dim, group size, block size)?
bool extend_supported(int32_t head_dim, int32_t group, int32_t block_size);
bool extend_supported_fp8(int32_t head_dim, int32_t group, int32_t block_size);

hipError_t launch_extend(const ExtendLaunch& L, hipStream_t stream);

// PGQA_LOG=1 in the environment: every attention launch prints its route,
// grid and key split to stderr.
bool log_enabled();
void log_line(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

// Debug check of device array contents (pgqa_check_contents).
struct CheckLaunch {
    const int32_t* block_table;
    const int32_t* context_lens;
    const int32_t* cu;
    const int32_t* start_pos;
    int32_t* status;
    int32_t max_blocks_per_seq;
    int32_t batch;
    int32_t total_rows;
    int32_t max_rows;
    int32_t num_blocks;
    int32_t block_size_log2;
    int32_t max_context_len;
    int32_t window;
};

hipError_t launch_check(const CheckLaunch& L, hipStream_t stream);

}  // namespace pgqa
