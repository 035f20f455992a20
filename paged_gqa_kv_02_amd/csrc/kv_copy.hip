// kv_copy.hip -- paged K/V write (packed rows -> pages) and its inverse gather.
//
// Token t of sequence b is logical position start_pos[b] + (t - cu_seqlens[b]);
// that position lives in block block_table[b][pos / bs], slot pos % bs (paging
// through a block table: "Advanced Optimizations: MQA, GQA, and PagedAttention",
// section "PagedAttention: The OS Analogy"; "The Ultimate Guide to LLM
// Inference Optimization- Part 2", section "Paged Attention").
//
// Pure HBM copy work.  One thread moves one 16-byte chunk of one (token, head)
// row of K and the same chunk of V; consecutive threads walk a row, so both the
// packed side and the page side are read and written in whole 256-byte rows
// (bf16, d = 128).  Element bytes are never interpreted, so the copy is
// bit-exact for any dtype.
#include "device_common.hpp"
#include "launch.hpp"

namespace pgqa {

namespace {

struct CopyArgs {
    const char* src_k;
    const char* src_v;
    char* dst_k;
    char* dst_v;
    const int32_t* cu_seqlens;
    const int32_t* start_pos;
    const int32_t* block_table;
    int64_t total_chunks;       // total_tokens * Hkv * chunks_per_row
    int32_t batch;
    int32_t total_tokens;
    int32_t max_blocks_per_seq;
    int32_t num_blocks;
    int32_t block_size_log2;
    int32_t num_kv_heads;
    int32_t chunks_per_row;     // head_dim * elem_bytes / 16
};

// Sequence owning packed token t: the last b with cu_seqlens[b] <= t.
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ cu, int batch, int t) {
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// TO_PAGES = true: packed -> pages (write); false: pages -> packed (gather).
template <bool TO_PAGES>
__global__ __launch_bounds__(256) void kv_copy_kernel(CopyArgs a) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.total_chunks; i += stride) {
        const int c = (int)(i % a.chunks_per_row);
        const int64_t row = i / a.chunks_per_row;          // t * Hkv + h
        const int h = (int)(row % a.num_kv_heads);
        const int t = (int)(row / a.num_kv_heads);
        const int b = find_seq(a.cu_seqlens, a.batch, t);
        const int64_t pos = (int64_t)a.start_pos[b] + (t - a.cu_seqlens[b]);
        const int64_t page = pos >> a.block_size_log2;
        if (pos < 0 || page >= a.max_blocks_per_seq) continue;
        const int blk = a.block_table[(int64_t)b * a.max_blocks_per_seq + page];
        if (blk < 0 || blk >= a.num_blocks) continue;
        const int64_t slot = pos & ((1 << a.block_size_log2) - 1);
        const int64_t page_row = (((int64_t)blk * a.num_kv_heads + h) << a.block_size_log2) + slot;
        const int64_t packed_off = (row * a.chunks_per_row + c) * 16;
        const int64_t page_off = (page_row * a.chunks_per_row + c) * 16;
        const int64_t s_off = TO_PAGES ? packed_off : page_off;
        const int64_t d_off = TO_PAGES ? page_off : packed_off;
        const u32x4 kx = *(const u32x4*)(a.src_k + s_off);
        const u32x4 vx = *(const u32x4*)(a.src_v + s_off);
        *(u32x4*)(a.dst_k + d_off) = kx;
        *(u32x4*)(a.dst_v + d_off) = vx;
    }
}

// Copy-on-write block copy.  A block is one contiguous run of Hkv * bs * d
// elements in each pool, so pair p copies that run of K and of V from block
// src[p] onto block dst[p]; thread i moves 16-byte chunk i of the flattened
// (pair, pool, chunk) space.  Pairs whose ids fall outside the pool are skipped.
struct BlockCopyArgs {
    char* k;
    char* v;
    const int32_t* src;
    const int32_t* dst;
    int64_t total_chunks;       // num_pairs * 2 * chunks_per_block
    int64_t chunks_per_block;   // Hkv * bs * d * elem_bytes / 16
    int32_t num_blocks;
};

__global__ __launch_bounds__(256) void kv_block_copy_kernel(BlockCopyArgs a) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.total_chunks; i += stride) {
        const int64_t c = i % a.chunks_per_block;
        const int64_t pp = i / a.chunks_per_block;      // 2 * pair + pool
        const int64_t pair = pp >> 1;
        char* pool = (pp & 1) ? a.v : a.k;
        const int s = a.src[pair];
        const int d = a.dst[pair];
        if (s < 0 || s >= a.num_blocks || d < 0 || d >= a.num_blocks) continue;
        const u32x4 x = *(const u32x4*)(pool + ((int64_t)s * a.chunks_per_block + c) * 16);
        *(u32x4*)(pool + ((int64_t)d * a.chunks_per_block + c) * 16) = x;
    }
}

// Quantising paged write (FP8 E4M3 pages, one fp32 scale per (token, KV head)
// row).  LPR = d / 8 consecutive lanes hold one bf16 row, 8 values (16 bytes)
// each: the row's largest magnitude comes from an xor-shuffle max over those
// lanes, scale = amax / 448 (1 for an all-zero row), and every value is divided
// by the scale (correctly rounded, single precision), clamped to +-448 and
// converted to the nearest E4M3 code (ties to even) two at a time.  Each lane
// stores its 8 codes; the row's first lane stores the scale.
struct QuantArgs {
    const char* k;
    const char* v;
    uint8_t* k_cache;
    uint8_t* v_cache;
    float* k_scale;
    float* v_scale;
    const int32_t* cu_seqlens;
    const int32_t* start_pos;
    const int32_t* block_table;
    int64_t total_lanes;        // total_tokens * Hkv * LPR
    int32_t batch;
    int32_t max_blocks_per_seq;
    int32_t num_blocks;
    int32_t block_size_log2;
    int32_t num_kv_heads;
    int32_t lpr;                // lanes per row: head_dim / 8 (a power of two <= 16)
};

__device__ __forceinline__ uint32_t fp8x4(const float* y) {
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
}

__global__ __launch_bounds__(256) void kv_write_fp8_kernel(QuantArgs a) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;   // a multiple of 64: rows never straddle waves
    for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x; i0 < a.total_lanes; i0 += stride) {
        const int64_t i = i0 + threadIdx.x;
        const bool live = i < a.total_lanes;
        const int c = (int)(i % a.lpr);
        const int64_t row = i / a.lpr;                    // t * Hkv + h
        const int h = (int)(row % a.num_kv_heads);
        const int t = (int)(row / a.num_kv_heads);
        int64_t dst_row = -1;
        if (live) {
            const int b = find_seq(a.cu_seqlens, a.batch, t);
            const int64_t pos = (int64_t)a.start_pos[b] + (t - a.cu_seqlens[b]);
            const int64_t page = pos >> a.block_size_log2;
            if (pos >= 0 && page < a.max_blocks_per_seq) {
                const int blk = a.block_table[(int64_t)b * a.max_blocks_per_seq + page];
                if (blk >= 0 && blk < a.num_blocks)
                    dst_row = ((((int64_t)blk * a.num_kv_heads + h) << a.block_size_log2) +
                               (pos & ((1 << a.block_size_log2) - 1)));
            }
        }
#pragma unroll
        for (int pool = 0; pool < 2; ++pool) {
            float x[8];
            if (live) {
                const u32x4 w = *(const u32x4*)((pool ? a.v : a.k) + (row * a.lpr + c) * 16);
                x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
                x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = 0.0f;
            }
            float amax = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
            for (int m = 1; m < a.lpr; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
            const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = fminf(fmaxf(x[e] / sc, -448.0f), 448.0f);
            if (dst_row >= 0) {
                uint8_t* codes = pool ? a.v_cache : a.k_cache;
                *(u32x2*)(codes + dst_row * (int64_t)a.lpr * 8 + c * 8) = u32x2{fp8x4(y), fp8x4(y + 4)};
                if (c == 0) (pool ? a.v_scale : a.k_scale)[dst_row] = sc;
            }
        }
    }
}

}  // namespace

hipError_t launch_kv_write_fp8(const KvCopyLaunch& L, void* k_scale, void* v_scale, hipStream_t stream) {
    QuantArgs a;
    a.k = (const char*)L.src_k;
    a.v = (const char*)L.src_v;
    a.k_cache = (uint8_t*)L.dst_k;
    a.v_cache = (uint8_t*)L.dst_v;
    a.k_scale = (float*)k_scale;
    a.v_scale = (float*)v_scale;
    a.cu_seqlens = L.cu_seqlens;
    a.start_pos = L.start_pos;
    a.block_table = L.block_table;
    a.batch = L.batch;
    a.max_blocks_per_seq = L.max_blocks_per_seq;
    a.num_blocks = L.num_blocks;
    a.block_size_log2 = L.block_size_log2;
    a.num_kv_heads = L.num_kv_heads;
    a.lpr = L.head_dim / 8;
    a.total_lanes = (int64_t)L.total_tokens * L.num_kv_heads * a.lpr;
    if (a.total_lanes == 0 || L.batch == 0) return hipSuccess;
    const int threads = 256;
    int64_t blocks = (a.total_lanes + threads - 1) / threads;
    if (blocks > 65536) blocks = 65536;  // grid-stride beyond this
    hipLaunchKernelGGL(kv_write_fp8_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_block_copy(const BlockCopyLaunch& L, hipStream_t stream) {
    BlockCopyArgs a;
    a.k = (char*)L.k_cache;
    a.v = (char*)L.v_cache;
    a.src = L.src;
    a.dst = L.dst;
    a.num_blocks = L.num_blocks;
    a.chunks_per_block = (int64_t)L.num_kv_heads * L.block_size * L.head_dim * L.elem_bytes / 16;
    a.total_chunks = (int64_t)L.num_pairs * 2 * a.chunks_per_block;
    if (a.total_chunks == 0) return hipSuccess;
    const int threads = 256;
    int64_t blocks = (a.total_chunks + threads - 1) / threads;
    if (blocks > 65536) blocks = 65536;  // grid-stride beyond this
    hipLaunchKernelGGL(kv_block_copy_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_kv_copy(const KvCopyLaunch& L, bool to_pages, hipStream_t stream) {
    CopyArgs a;
    a.src_k = (const char*)L.src_k;
    a.src_v = (const char*)L.src_v;
    a.dst_k = (char*)L.dst_k;
    a.dst_v = (char*)L.dst_v;
    a.cu_seqlens = L.cu_seqlens;
    a.start_pos = L.start_pos;
    a.block_table = L.block_table;
    a.batch = L.batch;
    a.total_tokens = L.total_tokens;
    a.max_blocks_per_seq = L.max_blocks_per_seq;
    a.num_blocks = L.num_blocks;
    a.block_size_log2 = L.block_size_log2;
    a.num_kv_heads = L.num_kv_heads;
    a.chunks_per_row = L.head_dim * L.elem_bytes / 16;
    a.total_chunks = (int64_t)L.total_tokens * L.num_kv_heads * a.chunks_per_row;
    if (a.total_chunks == 0 || L.batch == 0) return hipSuccess;
    const int threads = 256;
    int64_t blocks = (a.total_chunks + threads - 1) / threads;
    if (blocks > 65536) blocks = 65536;  // grid-stride beyond this
    if (to_pages)
        hipLaunchKernelGGL(kv_copy_kernel<true>, dim3((unsigned)blocks), dim3(threads), 0, stream, a);
    else
        hipLaunchKernelGGL(kv_copy_kernel<false>, dim3((unsigned)blocks), dim3(threads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pgqa
