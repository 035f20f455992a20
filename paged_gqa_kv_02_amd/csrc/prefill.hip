// prefill.hip -- packed variable-length prefill, block-diagonal (optionally causal)
// grouped-query attention on bf16 MFMA.
//
// What it computes: row i of sequence s (cu_seqlens[s] <= i < cu_seqlens[s+1]),
// query head qh, KV head h = qh / G:
//   out[i][qh] = sum_j softmax_j(scale * q[i][qh] . k[j][h]) v[j][h],
// keys j of the same sequence only (block-diagonal bias built from the true
// lengths: itinai.com/?p=48087, first paragraph), j <= i when causal.  Prefill
// is the compute-bound phase ("Modern LLM Inference", section 2), so both
// products run on the matrix cores.
//
// Design for gfx950 (v_mfma_f32_32x32x16_bf16, wave64):
//  * A workgroup of 4 waves owns one (sequence, KV head, query tile); the 4
//    waves are 4 query heads of the KV head's group (or, for G < 4, G heads x
//    4/G consecutive 32-token blocks), so every K/V tile staged in LDS serves
//    128 query rows: GQA reuse of K/V across the group.
//  * K and V tiles of 64 keys stream through two 2-slot LDS rings (K, V) with
//    global->LDS DMA (global_load_lds_dwordx4, 16 B per lane, 1 KB per
//    instruction).  Rows are XOR-swizzled by 16-byte chunk (chunk c of key row r
//    lands in chunk c ^ f(r), f a per-row bijection); the swizzle is chosen
//    through each lane's source address, so the global reads stay whole rows,
//    and makes both LDS read patterns below bank-conflict-free.
//  * Each wave computes S^T = K Q^T for 64 keys x its 32 query rows.  In the
//    32x32 accumulator layout a lane then holds 32 keys of ONE query row, so the
//    row max / sum need a single cross-lane step (lane ^ 32).
//  * O^T += V^T P^T: the B operand (P^T) is the lane's own S^T values rounded to
//    bf16, taken in the key order the accumulator layout gives; the A operand
//    (V^T) comes straight from the row-major V tile with ds_read_b64_tr_b16,
//    the transposing LDS read (two reads give the 8 keys of one dim per lane,
//    in exactly the B operand's key order).
//  * Online softmax in log2 units with the scale folded into the exponent and a
//    lazy rescale (only when a row max grows by more than 8), exact because the
//    final O / l uses the same reference.  The row sum l adds the bf16-rounded
//    weights (v_dot2 with (1, 1)), i.e. exactly the weights the PV product used.
//  * Masks select -inf (never multiply) and only on the diagonal block (causal)
//    and the ragged last block; key rows past the sequence are clamped to its
//    last row (in bounds, masked).
//  * Tiles of one (sequence, KV head) pair share an XCD (and its L2); each XCD
//    works through its pairs one at a time, a pair's tiles heaviest-first, so
//    K/V is fetched from HBM about once.
//  * The softmax of key block k overlaps the MFMAs of block k+1's scores
//    (software pipeline within the wave: two score buffers, separate K and V
//    rings so K(k+1) and V(k) are resident together).
//  * The output tile is staged through LDS and written as whole rows.
//
// The same kernel, instantiated with PAGED = true, serves queries that extend
// a cached sequence (chunked prefill on top of a cached prefix, or checking k
// draft tokens): K/V come from the page pools through the block table
// ("PagedAttention: The OS Analogy", tryclaro.ai; the Ultimate Guide, section
// "Paged Attention"), and the q_len new rows of a sequence with ctx cached
// positions (the new ones included) sit at positions ctx - q_len .. ctx - 1, so
// the causal diagonal is shifted by ctx - q_len (bottom-right alignment).  Each
// 1 KB wave-load covers 4 (d = 128) or 8 (d = 64) consecutive rows of one
// page, so its source is one scalar base (block id from a scalar load of the
// block-table row, issued before the block's DMA wait and barrier) plus the
// lane's offset, exactly as for packed K/V.
#include <algorithm>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace pgqa {

namespace {

struct PrefillArgs {
    const char* q;
    const char* k;
    const char* v;
    const int32_t* cu_seqlens;
    char* out;
    int32_t total_tokens;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t causal;
    float scale_log2;        // |scale| * log2(e)
    u32 q_and;               // the scale's sign, applied to the query bits as they are loaded
    u32 q_xor;
    int32_t batch;
    int32_t nqt;             // query-tile levels (tiles of the longest sequence)
    int32_t pairs_per_xcd;   // ceil(batch * num_kv_heads / 8)
    int32_t dense;           // 1: each XCD's list holds only existing query tiles (pairs_per_xcd <= 64)
    int32_t fixed_qlen;      // > 0: sequence s holds rows [s * fixed_qlen, +fixed_qlen) (cu_seqlens unused)
    int32_t chunk_lpt;       // 1: dense lists of key chunks, full chunks first (one query tile and head group per pair)
    int32_t kv_nt;           // 1: K/V read by one workgroup only (one query tile and head group per pair): non-temporal loads
    int32_t pack;            // host side: the packed-rows kernel was chosen
    int32_t sk_nw;           // > 0 (packed rows): stream-K shares, one per workgroup
    int32_t sk_pair_units;   // work units charged per pair on top of its key blocks (its piece's start-up)
    int32_t* sk_cut;         // [sk_nw][4]: per share, the pair cut at its end (or -1), its units, the total
    // Paged K/V only (k, v are then the pools [num_blocks, Hkv, block_size, d]).
    const int32_t* block_table;
    const int32_t* context_lens;
    int32_t max_blocks_per_seq;
    int32_t num_blocks;
    int32_t bs_log2;
    int32_t ctx_cap;         // host-side bound of context_lens
    int32_t window;          // > 0: row i sees only its newest `window` keys (local attention)
    // Key split (paged only): a pair's key range is cut into chunks of kchunk
    // blocks, nchunk per pair at most; a sequence whose keys span more than one
    // chunk gets fp32 partials per (row, head, chunk), merged afterwards.
    int32_t nchunk;          // 1 = no split
    int32_t kchunk;          // key blocks per chunk
    float* part_o;           // [total_tokens, Hq, nchunk, D]  (stream-K: [2 * sk_nw, 32, D])
    float* part_ml;          // [total_tokens, Hq, nchunk, 2]  (m in log2 units, l; stream-K: [2 * sk_nw, 32, 2])
    // FP8 pages only (k, v are then code pools [num_blocks, Hkv, block_size, d] uint8).
    const float* k_scale;    // row scales [num_blocks, Hkv, block_size]
    const float* v_scale;
};

#ifndef PGQA_KREADS_AHEAD
#define PGQA_KREADS_AHEAD 2
#endif

// Block-table rows are read through the constant address space, which makes
// the compiler fetch a uniform entry with a scalar load (the table is never
// written while a kernel runs).
typedef const __attribute__((address_space(4))) int32_t* ConstI32Ptr;

typedef short __attribute__((ext_vector_type(4))) i16x4;

constexpr int BQ = 32;   // query rows per wave
constexpr int BN = 64;   // keys per block

template <int D>
struct PGeo {
    static constexpr int ROWB = D * 2;            // bytes per K/V row
    static constexpr int CPR = D / 8;             // 16-byte chunks per row
    static constexpr int RPL = 64 / CPR;          // rows per 1 KB wave-load
    static constexpr int TILEB = BN * ROWB;       // K (or V) tile bytes
    static constexpr int LOADS = TILEB / 1024;    // wave-loads per K (or V) tile
    static constexpr int STAGEB = 2 * TILEB;      // K + V tile
    static constexpr int KSTEPS = D / 16;         // k-steps of S^T over head_dim
    static constexpr int DBLK = D / 32;           // 32-row blocks of O^T over head_dim
    static_assert((2 * LOADS) % 4 == 0, "loads split over 4 waves");
};

// The lane's index, produced afresh where it is needed.  The kernel re-derives
// its lane values after the prologue instead of keeping them live across the
// key loop, where every register is taken (kept, they are spilled to scratch).
__device__ __forceinline__ int lane_now() {
    int x;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
    return x;
}

// Row r's swizzle key.  LDS has 64 banks of 4 bytes; a 16-byte-per-lane read
// is served 16 lanes at a time and an 8-byte transposed read 32 lanes at a
// time, so a read is conflict-free when every lane of a phase hits its own
// 16-byte bank group.  The K operand read (one chunk from each of 16
// consecutive rows) needs the key to be a permutation on every aligned run of
// 16 rows; the transposed V read (chunks 4b .. 4b+3 of 4 consecutive rows)
// needs the keys of an aligned run of 4 rows to differ in bits 2..3.  For 64-dim
// rows (two rows per 256-byte bank line) the same holds per row parity.
template <int D>
__device__ __forceinline__ int swz_key(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Byte offset of 16-byte chunk c of key row r inside a swizzled tile.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
    using P = PGeo<D>;
    return r * P::ROWB + ((c ^ swz_key<D>(r)) << 4);
}

// DMA of key block kb into ring slot `slot`.  Waves 0 and 1 fetch the K tile,
// waves 2 and 3 the V tile, NPW 1 KB wave-loads each.  `soff` holds the lane's
// source offsets relative to the block's first key row (row * row stride +
// swizzled chunk); a block that runs past the sequence end clamps its rows to
// the last key instead (those keys are masked out of the scores).
template <int D>
struct DmaLane {
    static constexpr int NPW = 2 * PGeo<D>::LOADS / 4;
    // Loads j and j + JP are 16 rows apart, which keeps the swizzle key, so
    // they differ by 16 rows of source only (added to the uniform base).
    static constexpr int JP = 16 / PGeo<D>::RPL;
    uint32_t soff[JP];
};

template <int D>
__device__ __forceinline__ void dma_lane_init(DmaLane<D>& dl, int wave, int lane, int64_t kvstride) {
    using P = PGeo<D>;
#pragma unroll
    for (int j = 0; j < DmaLane<D>::JP; ++j) {
        const int r = ((wave & 1) * DmaLane<D>::NPW + j) * P::RPL + lane / P::CPR;
        const int c = (lane % P::CPR) ^ swz_key<D>(r);
        dl.soff[j] = (uint32_t)(r * kvstride + c * 16);
    }
}


// DMA of one tile of key block kb: waves 0 and 1 fetch K(kb) into K slot par,
// waves 2 and 3 fetch V(kb) into V slot par (LDS: K slots, then V slots; par is
// the parity of the block's index in the workgroup's stream).
template <int D>
__device__ __forceinline__ void issue_tile(const PrefillArgs& a, const DmaLane<D>& dl, uint32_t ring, int kb,
                                           int par, int seq0, int L, int kvh, int wave, int lane,
                                           int64_t kvstride) {
    using P = PGeo<D>;
    constexpr int NPW = DmaLane<D>::NPW;
    const bool isv = wave >= 2;
    const char* base = (isv ? a.v : a.k) + (int64_t)(seq0 + kb * BN) * kvstride + (int64_t)kvh * P::ROWB;
    const uint32_t dst = ring + (isv ? 2 * P::TILEB : 0) + par * P::TILEB + (wave & 1) * NPW * 1024;
    if (kb * BN + BN <= L) {
        constexpr int JP = DmaLane<D>::JP;
#pragma unroll
        for (int j = 0; j < NPW; ++j) dma16(base + (j / JP) * 16 * kvstride, dl.soff[j % JP], dst + j * 1024, a.kv_nt);
    } else {
        const int last = L - 1 - kb * BN;
#pragma unroll
        for (int j = 0; j < NPW; ++j) {
            const int r = ((wave & 1) * NPW + j) * P::RPL + lane / P::CPR;
            const int c = (lane % P::CPR) ^ swz_key<D>(r);
            dma16(base, (uint32_t)(min(r, last) * kvstride + c * 16), dst + j * 1024, a.kv_nt);
        }
    }
}

// FP8 pages (E4M3 codes, one fp32 scale per key row).  LDS holds one bf16 K
// tile and one bf16 V tile (swizzled as above), then two stages of K codes and
// two of V codes (BN rows of D bytes each, plain order), so the ring's size is
// unchanged.  A tile's codes are DMA'd 1 KB (RPL8 rows of one page) per
// wave-load, K waves and V waves NPW8 loads each; once they land, every thread
// converts its share into the bf16 tile (exact), so the MFMA code is the bf16
// one.  The tile's row scales go to a small LDS area by one 4-byte-per-lane
// DMA per pool (wave 1: K, wave 3: V).
template <int D>
struct Q8Geo {
    static constexpr int CODEB = BN * D;          // code bytes per tile and pool
    static constexpr int LOADS = CODEB / 1024;    // 1 KB wave-loads per tile and pool
    static constexpr int NPW8 = LOADS / 2;        // per DMA wave
    static constexpr int RPL8 = 1024 / D;         // rows per wave-load
    static constexpr int NG = BN / RPL8;          // wave-loads (row groups) per tile
    static constexpr int CPT = CODEB / 16 / 256;  // 16-byte code chunks per thread in the conversion
    static_assert(CPT >= 1 && NG <= 8, "FP8 tile geometry");
};

// LDS of the row scales: K scales in three slots (a tile's K scales are used one
// block after its codes, when its scores are scaled), V scales in two; 64 floats each.
constexpr int kScaleSlotB = BN * 4;
constexpr int kScaleB = 5 * kScaleSlotB;

// Paged K/V: the lane's offset inside wave-load j, relative to that load's
// first row (the swizzle key only depends on the row modulo 16, and loads j and
// j + JP are 16 rows apart).
template <int D>
__device__ __forceinline__ void dma_lane_init_paged(DmaLane<D>& dl, int lane) {
    using P = PGeo<D>;
#pragma unroll
    for (int j = 0; j < DmaLane<D>::JP; ++j) {
        const int r = lane / P::CPR;
        const int c = (lane % P::CPR) ^ swz_key<D>(j * P::RPL + r);
        dl.soff[j] = (uint32_t)(r * P::ROWB + c * 16);
    }
}

// Paged source of one wave: its pool (K for waves 0-1, V for waves 2-3, NPW
// wave-loads each from wave-load j0 = (wave & 1) * NPW on), the sequence's
// block-table row and the block ids of the next tile it will fetch (one per
// wave-load, loaded before the DMA wait and barrier that precede the tile's
// issue and clamped only at the issue, so their latency hides behind those).
template <int D>
struct PagedSrc {
    static constexpr int NPW = DmaLane<D>::NPW;
    ConstI32Ptr bt;
    const char* pool;
    int64_t head_off;    // kvh * block_size * row bytes
    int64_t blk_bytes;   // Hkv * block_size * row bytes
    int lbs;
    int last;            // last key row of the sequence (ctx - 1)
    int lo;              // first key row the workgroup needs (its first row's window edge, or 0)
    int nb;
    bool nt;             // non-temporal loads
    bool isv;            // this wave fetches V (else K)
    int j0;              // first wave-load of the tile this wave issues
    int id[NPW];
};

// First key row (relative to the sequence) of wave-load j of tile kb.
template <int D, bool Q8 = false>
__device__ __forceinline__ int paged_row0(int kb, int j) {
    return kb * BN + j * (Q8 ? Q8Geo<D>::RPL8 : PGeo<D>::RPL);
}

template <int D, bool Q8 = false>
__device__ __forceinline__ void paged_load_ids(PagedSrc<D>& ps, int kb) {
    if constexpr (Q8) {
        // FP8 pages: the ids of every row group of the tile (the scale loads need them all).
#pragma unroll
        for (int g = 0; g < Q8Geo<D>::NG; ++g)
            ps.id[g] = ps.bt[min(max(paged_row0<D, true>(kb, g), ps.lo), ps.last) >> ps.lbs];
    } else {
#pragma unroll
        for (int j = 0; j < PagedSrc<D>::NPW; ++j)
            ps.id[j] = ps.bt[min(max(paged_row0<D>(kb, ps.j0 + j), ps.lo), ps.last) >> ps.lbs];
    }
}

// DMA of tile kb from the pages (same LDS placement as issue_tile).  A load's
// rows lie in one page (block_size >= rows per load), so its source is a
// uniform base plus the lane offset; rows past the sequence end re-read its
// last row, and rows below the first key the workgroup needs (under a window:
// rows of pages the caller may have released) re-read that key's row (in bounds
// and written; those keys are masked, and their values are finite, so a zero
// weight cannot meet a NaN in P.V).
template <int D>
__device__ __forceinline__ void issue_tile_paged(const PagedSrc<D>& ps, const DmaLane<D>& dl, uint32_t ring,
                                                 int kb, int par, int lane) {
    using P = PGeo<D>;
    constexpr int NPW = DmaLane<D>::NPW;
    constexpr int JP = DmaLane<D>::JP;
    const uint32_t dst = ring + (ps.isv ? 2 * P::TILEB : 0) + par * P::TILEB + ps.j0 * 1024;
    const int bs_mask = (1 << ps.lbs) - 1;
    auto base_of = [&](int j, int rb) {
        return ps.pool + (int64_t)clampi(ps.id[j], 0, ps.nb - 1) * ps.blk_bytes + ps.head_off +
               (int64_t)(rb & bs_mask) * P::ROWB;
    };
    if (kb * BN >= ps.lo && kb * BN + BN <= ps.last + 1) {
#pragma unroll
        for (int j = 0; j < NPW; ++j) {
            const int row0 = paged_row0<D>(kb, ps.j0 + j);
            dma16(base_of(j, row0), dl.soff[j % JP], dst + j * 1024, ps.nt);
        }
    } else {
        const int r = lane / P::CPR;
#pragma unroll
        for (int j = 0; j < NPW; ++j) {
            const int row0 = paged_row0<D>(kb, ps.j0 + j);
            const int rb = min(max(row0, ps.lo), ps.last);
            const int rc = min(max(row0 + r, ps.lo), ps.last);
            const int c = (lane % P::CPR) ^ swz_key<D>((j % JP) * P::RPL + r);
            dma16(base_of(j, rb), (uint32_t)((rc - rb) * P::ROWB + c * 16), dst + j * 1024, ps.nt);
        }
    }
}

// DMA of tile kb of FP8 pages: codes into code stage `par` of the wave's pool
// (rows in plain order, D bytes each), and, from wave 1 (K) and wave 3 (V), the
// tile's 64 row scales into scale slot `ssl`.  Rows outside [lo, last] re-read
// the nearest of the two (as in issue_tile_paged).
template <int D>
__device__ __forceinline__ void issue_tile_paged_q8(const PagedSrc<D>& ps, const float* scale_pool, uint32_t ring,
                                                    uint32_t scales, int kb, int par, int ssl, int wave, int lane,
                                                    int kvh, int hkv) {
    using P = PGeo<D>;
    using Q = Q8Geo<D>;
    const uint32_t dst = ring + 2 * P::TILEB + ((ps.isv ? 2 : 0) + par) * Q::CODEB;
    const int bs_mask = (1 << ps.lbs) - 1;
    const int64_t row_b = D;                                    // code bytes per row
    const int64_t blk_b = ((int64_t)hkv << ps.lbs) * row_b;     // code bytes per block
    const int64_t head_b = ((int64_t)kvh << ps.lbs) * row_b;
    // (Ids are picked with constant indexes: a runtime index would put the array in scratch.)
    auto base_of = [&](int id, int rb) {
        return ps.pool + (int64_t)clampi(id, 0, ps.nb - 1) * blk_b + head_b + (int64_t)(rb & bs_mask) * row_b;
    };
    const bool full = kb * BN >= ps.lo && kb * BN + BN <= ps.last + 1;
    const int r = lane / (D / 16);
    const int col = (lane % (D / 16)) * 16;
#pragma unroll
    for (int j = 0; j < Q::NPW8; ++j) {
        const int g = (wave & 1) * Q::NPW8 + j;
        const int id = (wave & 1) ? ps.id[Q::NPW8 + j] : ps.id[j];
        const int row0 = paged_row0<D, true>(kb, g);
        if (full) {
            dma16(base_of(id, row0), (uint32_t)(lane * 16), dst + g * 1024, ps.nt);
        } else {
            const int rb = min(max(row0, ps.lo), ps.last);
            const int rc = min(max(row0 + r, ps.lo), ps.last);
            dma16(base_of(id, rb), (uint32_t)((rc - rb) * row_b + col), dst + g * 1024, ps.nt);
        }
    }
    if (wave & 1) {
        // Row scale of key kb*BN + lane (clamped like the codes): its row group's
        // block id, picked from the wave's uniform ids.
        const int key = min(max(kb * BN + lane, ps.lo), ps.last);
        const int g = (key - kb * BN) / Q::RPL8;
        int id = ps.id[0];
#pragma unroll
        for (int gg = 1; gg < Q::NG; ++gg) id = g == gg ? ps.id[gg] : id;
        id = clampi(id, 0, ps.nb - 1);
        const uint32_t off = (uint32_t)((((int64_t)id * hkv + kvh) << ps.lbs) + (key & bs_mask)) * 4u;
        dma4((const char*)scale_pool, off, scales + ssl * kScaleSlotB, ps.nt);
    }
}

// Conversion of landed FP8 code tiles into the bf16 tiles: the K codes of
// stage kpar (kpar < 0: none) and the V codes of stage vpar (vpar < 0: none).
// Every thread converts its own code chunks into bf16 rows (swizzled like
// DMA'd bf16 tiles); a barrier then publishes them.
template <int D>
__device__ __forceinline__ void convert_q8(PGQA_LDS char* ring, int kpar, int vpar) {
    using P = PGeo<D>;
    using Q = Q8Geo<D>;
    const int t = threadIdx.x;
    u32x4 kc[Q::CPT], vc[Q::CPT];
    const PGQA_LDS char* codes = ring + 2 * P::TILEB;
#pragma unroll
    for (int i = 0; i < Q::CPT; ++i) {
        const int c = t + 256 * i;
        if (kpar >= 0) kc[i] = lds_read_16(codes + kpar * Q::CODEB + c * 16);
        if (vpar >= 0) vc[i] = lds_read_16(codes + (2 + vpar) * Q::CODEB + c * 16);
    }
#pragma unroll
    for (int i = 0; i < Q::CPT; ++i) {
        const int c = t + 256 * i;
        const int row = c / (D / 16);
        const int c16 = c % (D / 16);
        const int o0 = row * P::ROWB + (((2 * c16) ^ swz_key<D>(row)) << 4);
        const int o1 = row * P::ROWB + (((2 * c16 + 1) ^ swz_key<D>(row)) << 4);
        if (kpar >= 0) {
            PGQA_LDS char* kt = ring;
            *(PGQA_LDS u32x4*)(kt + o0) = fp8x8_to_bf16(u32x2{kc[i].x, kc[i].y});
            *(PGQA_LDS u32x4*)(kt + o1) = fp8x8_to_bf16(u32x2{kc[i].z, kc[i].w});
        }
        if (vpar >= 0) {
            PGQA_LDS char* vt = ring + P::TILEB;
            *(PGQA_LDS u32x4*)(vt + o0) = fp8x8_to_bf16(u32x2{vc[i].x, vc[i].y});
            *(PGQA_LDS u32x4*)(vt + o1) = fp8x8_to_bf16(u32x2{vc[i].z, vc[i].w});
        }
    }
    __syncthreads();
}

// PACK (paged calls with at most 32 query rows per KV head and sequence: q_len
// x G <= 32, e.g. decode of many heads on one KV head, or draft verification):
// the rows of a workgroup are the (token, head) pairs of one sequence and KV
// head, row r = token r / G, head r % G of the KV head's group, so a few tokens
// fill one 32-row MFMA tile instead of G mostly empty ones.  Waves 0 and 1 then
// share every key block, each taking one 32-key half with its own running max,
// sum and output, merged through LDS at the end; waves 2 and 3 only fetch V.
template <int D, int HG, bool PAGED, bool Q8 = false, bool PACK = false, bool P16 = false>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillArgs a) {
    static_assert(PAGED || !Q8, "FP8 K/V only from pages");
    static_assert(!PACK || (PAGED && HG == 1), "packed rows: paged, one workgroup per KV head");
    static_assert(!P16 || (PACK && !Q8), "16-row waves: packed rows over bf16 pages");
    using P = PGeo<D>;
    constexpr int NH = PACK ? 1 : 2;          // 32-key halves of a block each wave computes
    constexpr int TB = 4 / HG;               // 32-row token blocks per workgroup
    constexpr int KSTEPS = P::KSTEPS, DBLK = P::DBLK;
    constexpr int NPW = DmaLane<D>::NPW;   // wave-loads per tile and DMA wave (normal roles)

    extern __shared__ __attribute__((aligned(16))) char smem[];
    PGQA_LDS char* ring = (PGQA_LDS char*)smem;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int G = a.num_q_heads / a.num_kv_heads;
    const int groups = PACK ? 1 : G / HG;

    // One tile: query tile `qtile` of head group `grp` of pair (s, kvh) (rows
    // seq0 .. seq0 + Lq - 1 of the packed q / out, Lk keys), over the key blocks
    // [c_lo, c_hi) cut to those the tile reads.  Its output goes to `out`, or
    // (split) as partials: of key chunk `chunk`, or in stream-K slot `slot` >= 0.
    // Query row i sits at key position koff + i (packed prefill: the sequence's
    // own rows, koff = 0; paged: the cached context, koff = ctx - q_len) and,
    // when causal, sees keys 0 .. koff + i.
    auto tile = [&](const int s, const int kvh, const int grp, const int qtile, const int seq0, const int Lq,
                    const int Lk, const int c_lo, const int c_hi, const bool split, const int chunk,
                    const int slot) __attribute__((always_inline)) {
        const int koff = PAGED ? Lk - Lq : 0;
        const int tok0 = qtile * TB * BQ;
        const int head = kvh * G + grp * HG + (wave % HG);
        // This wave's first query row (sequence-local); packed: token 0 for waves 0, 1.
        const int i0 = PACK ? (P16 || wave < 2 ? 0 : 1 << 30) : tok0 + (wave / HG) * BQ;
        const int hoff = PACK ? (wave & 1) : 0;          // packed: the wave's key half
        const int prows = PACK ? Lq * G : 0;             // packed rows (<= 32)

        const int wg_rows_end = min(Lq, tok0 + TB * BQ);
        const int keys = a.causal ? min(Lk, koff + wg_rows_end) : Lk;   // keys the workgroup reads
        const int nkb = keys > 0 ? (keys + BN - 1) / BN : 0;
        const bool active = i0 < Lq;
        const int last_key = a.causal ? min(Lk, koff + min(i0 + BQ, Lq)) - 1 : Lk - 1;
        const int last_kb = last_key >= 0 ? last_key / BN : -1;
        // Local attention (window > 0, causal only): row i also drops keys below
        // koff + i - window + 1.  The workgroup streams key blocks kb0 .. nkb-1, kb0
        // set by its first row; every wave computes from kb0 (the blocks before its
        // own rows' windows are fully masked) to its last block.  Ring slots and the
        // block loop run on the index relative to kb0.
        const int win = a.window;
        const int kbw = (win > 0 && nkb > 0) ? max(0, koff + tok0 - win + 1) / BN : 0;
        // This workgroup's key blocks: the window's range cut to its chunk (or piece).
        const int kb0 = max(kbw, c_lo);
        const int kb1 = min(nkb, c_hi);
        const int nrel = max(0, kb1 - kb0);
        const float cs = a.scale_log2;

        const int64_t qstride = (int64_t)a.num_q_heads * D * 2;   // bytes per packed Q row
        const int64_t kvstride = (int64_t)a.num_kv_heads * P::ROWB;

        // Prologue: K(0), V(0) and K(1) in flight while Q is read.
        DmaLane<D> dl;
        PagedSrc<D> ps;
        const uint32_t ring_addr = (uint32_t)(uintptr_t)ring;
        // FP8 row scales: K scales of relative tile t in slot t % 3, V scales in slot 3 + t % 2.
        const uint32_t scale_addr = ring_addr + 4 * P::TILEB;
        const PGQA_LDS float* scale_lds = (const PGQA_LDS float*)(ring + 4 * P::TILEB);
        // DMA of relative tile t (key block kb0 + t) of this wave's pool.
        auto issue_paged = [&](int t, int ln) {
            if constexpr (Q8)
                issue_tile_paged_q8<D>(ps, ps.isv ? a.v_scale : a.k_scale, ring_addr, scale_addr, kb0 + t, t & 1,
                                       ps.isv ? 3 + (t & 1) : t % 3, wave, ln, kvh, a.num_kv_heads);
            else
                issue_tile_paged<D>(ps, dl, ring_addr, kb0 + t, t & 1, ln);
        };
        if constexpr (PAGED) {
            dma_lane_init_paged<D>(dl, lane);
            ps.bt = (ConstI32Ptr)(a.block_table + (int64_t)s * a.max_blocks_per_seq);
            ps.isv = wave >= 2;
            ps.j0 = (wave & 1) * NPW;
            ps.pool = ps.isv ? a.v : a.k;
            ps.lbs = a.bs_log2;
            ps.head_off = ((int64_t)kvh << a.bs_log2) * P::ROWB;
            ps.blk_bytes = ((int64_t)a.num_kv_heads << a.bs_log2) * P::ROWB;
            ps.last = Lk - 1;
            ps.lo = win > 0 ? min(max(0, koff + tok0 - win + 1), Lk - 1) : 0;
            ps.nb = a.num_blocks;
            ps.nt = a.kv_nt != 0;
            if (nrel > 0) {
                paged_load_ids<D, Q8>(ps, kb0);
                issue_paged(0, lane);
                if (!ps.isv && nrel > 1) {
                    paged_load_ids<D, Q8>(ps, kb0 + 1);
                    issue_paged(1, lane);
                }
            }
        } else {
            dma_lane_init<D>(dl, wave, lane, kvstride);
            issue_tile<D>(a, dl, ring_addr, kb0, 0, seq0, Lk, kvh, wave, lane, kvstride);
            if (wave < 2 && nrel > 1) issue_tile<D>(a, dl, ring_addr, kb0 + 1, 1, seq0, Lk, kvh, wave, lane, kvstride);
        }

        // Q^T operand: lane holds row (i0 + l32), d = 16*kk + 8*half .. +8.
        u32x4 qreg[KSTEPS];
        if constexpr (!P16) {
            const int row = min(i0 + l32, Lq - 1);
            const char* qp = a.q + (int64_t)(seq0 + row) * qstride + (int64_t)head * D * 2 + half * 16;
            if constexpr (PACK) {
                const int r = min(l32, prows - 1);
                qp = a.q + (int64_t)(seq0 + r / G) * qstride + (int64_t)(kvh * G + r % G) * D * 2 + half * 16;
            }
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) qreg[kk] = (*(const u32x4*)(qp + kk * 32) & a.q_and) ^ a.q_xor;
        }

        float m = kMaxInit, lsum = 0.0f;
        f32x16 o[DBLK];
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] = 0.0f;

        // V^T operand addressing (ds_read_b64_tr_b16): in each 16-lane group, lane j
        // supplies row (key0 + j/4), dims d0 + 4*(j%4) .. +3 of the V tile; lane i
        // of the group then receives dims d0 + i of keys key0 .. key0+3.
        const int gl = lane & 15;
        const int vrow = gl >> 2;                          // + key0
        const int vdim = 16 * ((lane >> 4) & 1) + 4 * (gl & 3);   // + 32*db
        // Per-lane LDS offsets, fixed for the whole key loop.  K operand, step kk:
        // row l32 (+32 per key half, which keeps the swizzle key), chunk 2*kk + half,
        // i.e. kx ^ (kk << 5).  V operand, dim block db, keys +8h: rows
        // 4*half + vrow + 8h (+16 per key step, same key), chunk 4*db + vdim/8; the
        // key of row r + 8 is key(r) ^ 2, so this is (vx ^ (db << 6) ^ (h << 5)) +
        // 8h rows.  The XORs only touch the chunk field of the offset.
        const int kx = swz<D>(l32, half);
        const int vx = swz<D>(4 * half + vrow, vdim >> 3) + ((vdim & 7) << 1);
        const u32 ones_bf16x2 = 0x3F803F80u;   // (1.0, 1.0) in bf16

        // S^T = K Q^T for key block kb (K slot kb % 2): per 32-key half kb2, lane
        // (l32, half) gets row l32, keys 32*kb2 + 8*(i/4) + 4*half + i%4.
        auto scores = [&](f32x16 (&st)[2], auto slot) {
            // (FP8 pages: the one bf16 K tile.)
            const PGQA_LDS char* kt = ring + (Q8 ? 0 : decltype(slot)::value * P::TILEB);
#pragma unroll
            for (int kb2 = 0; kb2 < NH; ++kb2) {
#pragma unroll
                for (int i = 0; i < 16; ++i) st[kb2][i] = 0.0f;
#pragma unroll
                for (int kk = 0; kk < KSTEPS; ++kk)
                    st[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, lds_read_16(kt + 32 * (kb2 + hoff) * P::ROWB + (kx ^ (kk << 5)))),
                        __builtin_bit_cast(bf16x8, qreg[kk]), st[kb2], 0, 0, 0);
            }
        };

        // One key block: softmax of the block's scores `cur`, overlapped with the
        // next block's scores into `nxt` (when HAS_NEXT), then O^T += V^T P^T.
        auto step = [&](f32x16 (&cur)[2], f32x16 (&nxt)[2], int kr, auto par, auto has_next) {
            constexpr int PAR = decltype(par)::value;   // kr % 2
            const int j0 = (kb0 + kr) * BN;
            // FP8 pages: scores times the keys' row scales (key offsets as in the masking below).
            if constexpr (Q8) {
                const PGQA_LDS float* ks = scale_lds + (kr % 3) * BN + 32 * hoff + 4 * (lane_now() >> 5);
#pragma unroll
                for (int g = 0; g < 4 * NH; ++g) {
                    const f32x4 k4 = *(const PGQA_LDS f32x4*)(ks + 8 * g);
#pragma unroll
                    for (int t = 0; t < 4; ++t) cur[g >> 2][4 * (g & 3) + t] *= k4[t];
                }
            }
            // Masking (last block of the sequence, a block crossing the diagonal,
            // or one crossing the window's lower edge): key j0 + off is kept iff
            // llim <= off <= lim, with off = 32*kb2 + 8*(i/4) + i%4 and the lane's
            // 4*half folded into both bounds.
            if ((j0 + BN > Lk) || (a.causal && j0 + BN - 1 > koff + i0) || (win > 0 && j0 < koff + i0 + BQ - win)) {
                const int ln = lane_now();
                // The lane's row position (packed: its row's token).
                const int lrow = koff + (PACK ? (ln & 31) / G : i0 + (ln & 31));
                const int lim = (a.causal ? min(lrow, Lk - 1) : Lk - 1) - j0 - 4 * (ln >> 5) - 32 * hoff;
                if (win > 0) {
                    const int llim = lrow - win + 1 - j0 - 4 * (ln >> 5) - 32 * hoff;
#pragma unroll
                    for (int kb2 = 0; kb2 < NH; ++kb2)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int off = 32 * kb2 + 8 * (i >> 2) + (i & 3);
                            cur[kb2][i] = (off <= lim && off >= llim) ? cur[kb2][i] : -INFINITY;
                        }
                } else {
                    // (No window: one comparison per score.)
#pragma unroll
                    for (int kb2 = 0; kb2 < NH; ++kb2)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int off = 32 * kb2 + 8 * (i >> 2) + (i & 3);
                            cur[kb2][i] = off <= lim ? cur[kb2][i] : -INFINITY;
                        }
                }
            }
            float mt = cur[0][0];
#pragma unroll
            for (int kb2 = 0; kb2 < NH; ++kb2)
#pragma unroll
                for (int i = 0; i < 16; ++i) mt = fmaxf(mt, cur[kb2][i]);
            mt = max_xor32(mt) * cs;
            const bool need = mt > m + 8.0f;
            if (__builtin_expect(__any(need), 0)) {
                if (need) {
                    const float alpha = __builtin_amdgcn_exp2f(m - mt);
                    m = mt;
                    lsum *= alpha;
#pragma unroll
                    for (int db = 0; db < DBLK; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
                }
            }
            // The MFMA + softmax interleave runs at raised wave priority, so of the
            // two workgroups sharing a SIMD the one in this phase issues first and
            // the other's P.V products fill the matrix pipe around it.
            __builtin_amdgcn_s_setprio(3);
            if constexpr (decltype(has_next)::value) scores(nxt, std::integral_constant<int, 1 - PAR>{});
            // P^T operand for 16-key step kk: keys 16kk + 8*(jj/4) + 4*half + jj%4,
            // i.e. accumulator entries 8*(kk%2) .. +7 of half kk/2.  The row sum
            // adds the bf16-rounded weights, the same ones the PV product uses.
            u32x4 pb[2 * NH];
#pragma unroll
            for (int kk = 0; kk < 2 * NH; ++kk) {
                float p[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(fmaf(cur[kk >> 1][8 * (kk & 1) + j], cs, -m));
                if constexpr (Q8) {
                    // Weights times the values' row scales (accumulator entry 8*(kk%2) + j
                    // of half kk/2 is key 16*kk + 8*(j/4) + 4*half + j%4); the row sum
                    // takes the plain weights.
                    const PGQA_LDS float* vs = scale_lds + (3 + PAR) * BN + 16 * (kk + 2 * hoff) + 4 * (lane_now() >> 5);
                    const f32x4 v0 = *(const PGQA_LDS f32x4*)vs;
                    const f32x4 v1 = *(const PGQA_LDS f32x4*)(vs + 8);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        lsum += p[2 * j] + p[2 * j + 1];
                        const f32x4& vv = j < 2 ? v0 : v1;
                        pb[kk][j] = pack_bf16x2_rne_hw(p[2 * j] * vv[(2 * j) & 3], p[2 * j + 1] * vv[(2 * j + 1) & 3]);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        pb[kk][j] = pack_bf16x2_rne_hw(p[2 * j], p[2 * j + 1]);
                        lsum = dot2_bf16(pb[kk][j], ones_bf16x2, lsum);
                    }
                }
            }
            if constexpr (decltype(has_next)::value) {
                // Interleave: per next-block MFMA one K read and a slice of the
                // softmax arithmetic, so the VALU work hides under the matrix pipe
                // and only a few K fragments are live at a time.
                __builtin_amdgcn_sched_group_barrier(0x100, PGQA_KREADS_AHEAD, 0);   // K reads ahead
#pragma unroll
                for (int i = 0; i < NH * KSTEPS; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    if (i + PGQA_KREADS_AHEAD < NH * KSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // K read
                    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // VALU
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
            // O^T += V^T P^T: A = V^T for dims 32*db + l32, keys {16kk + 4*half + 0..3, +8 ..}.
            const PGQA_LDS char* vt = ring + (Q8 ? 1 : 2 + PAR) * P::TILEB;
#pragma unroll
            for (int db = 0; db < DBLK; ++db) {
                u32x4 va[2 * NH];
#pragma unroll
                for (int kk = 0; kk < 2 * NH; ++kk) {
                    const PGQA_LDS char* vk = vt + 16 * (kk + 2 * hoff) * P::ROWB;
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PGQA_LDS i16x4*)(vk + (vx ^ (db << 6))));
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PGQA_LDS i16x4*)(vk + 8 * P::ROWB + (vx ^ (db << 6) ^ 32)));
                    va[kk] = u32x4{__builtin_bit_cast(u32x2, lo).x, __builtin_bit_cast(u32x2, lo).y,
                                   __builtin_bit_cast(u32x2, hi).x, __builtin_bit_cast(u32x2, hi).y};
                }
#pragma unroll
                for (int kk = 0; kk < 2 * NH; ++kk)
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va[kk]),
                                                                    __builtin_bit_cast(bf16x8, pb[kk]), o[db], 0, 0, 0);
            }
        };

        // Top of block kb: every wave's DMA has landed (K(kb+1), V(kb)) and every
        // wave is done with K(kb) and V(kb-1), so their slots are refilled with
        // K(kb+2) and V(kb+1).
        auto top = [&](int kr) {
            const int tb = (PAGED ? !ps.isv : wave < 2) ? kr + 2 : kr + 1;
            // The block ids of the tile issued below are loaded before the DMA wait
            // and the barrier, which cover their latency; no scalar load is then in
            // flight during the block's LDS reads (whose waits would otherwise also
            // wait for it, scalar loads returning out of order).
            if constexpr (PAGED)
                if (tb < nrel) paged_load_ids<D, Q8>(ps, kb0 + tb);
            wait_vmcnt<0>();
            __syncthreads();
            if (tb < nrel) {
                if constexpr (PAGED) {
                    issue_paged(tb, lane_now());
                } else {
                    issue_tile<D>(a, dl, ring_addr, kb0 + tb, tb & 1, seq0, Lk, kvh, wave, lane_now(), kvstride);
                }
            }
            // FP8 pages: the codes of K(kr+1) and V(kr) have landed; into the bf16
            // tiles, which every wave is done with (the codes just issued go to the
            // other stages).
            if constexpr (Q8) convert_q8<D>(ring, kr + 1 < nrel ? (kr + 1) & 1 : -1, kr & 1);
        };
        if constexpr (P16) {
            // 16-row waves (packed rows, more than 16 of them): wave (rh, hoff)
            // takes rows 16 rh .. +15 of the packed tile and keys 32 hoff .. +31 of
            // every block, so all four waves compute (two per SIMD with two
            // workgroups per CU) on v_mfma_f32_16x16x32_bf16, whose lane l holds
            // A[l % 16][8 (l / 16) + j], B[8 (l / 16) + j][l % 16] and
            // D[4 (l / 16) + i][l % 16].  S^T = K Q^T per 16-key group g: lane
            // (n = l % 16, q = l / 16) gets row 16 rh + n, keys 16 g + 4 q + i of the
            // half.  O^T += V^T P^T over the half's 32 keys in the order
            // k = 8 q + 4 g + i <-> key 16 g + 4 q + i, so the lane's B operand is its
            // own 8 weights and its A operand two transposed reads of 4 keys.  The two
            // key halves of a row half merge through LDS at the end.
            constexpr int KS = D / 32;    // k-steps of S^T
            constexpr int DB = D / 16;    // 16-dim blocks of O^T
            const int rh = wave >> 1;
            const int ln0 = lane_now();
            const int n16 = ln0 & 15;
            const int q4 = ln0 >> 4;
            u32x4 qv[KS];
            {
                const int r = min(16 * rh + n16, prows - 1);
                const char* qp = a.q + (int64_t)(seq0 + r / G) * qstride + (int64_t)(kvh * G + r % G) * D * 2 + q4 * 16;
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) qv[kk] = (*(const u32x4*)(qp + kk * 64) & a.q_and) ^ a.q_xor;
            }
            // K operand: row n16 (+16 g + 32 hoff: the swizzle key depends on row % 16),
            // chunk q4 + 4 kk, i.e. kx16 ^ (kk << 6).  V operand (transposed read,
            // dims 16 db + 4 (n16 % 4) .. +3 of key row 4 q4 + n16 / 4, +16 for the
            // second read): chunk 2 db + (n16 % 4) / 2, i.e. vx16 ^ (db << 5).
            const int kx16 = swz<D>(n16, q4);
            const int vx16 = swz<D>(4 * q4 + (n16 >> 2), (n16 & 3) >> 1) + ((n16 & 1) << 3);
            auto scores16 = [&](f32x4 (&st)[2], auto slot) {
                const PGQA_LDS char* kt = ring + decltype(slot)::value * P::TILEB + 32 * hoff * P::ROWB;
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    st[g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk)
                        st[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, lds_read_16(kt + 16 * g * P::ROWB + (kx16 ^ (kk << 6)))),
                            __builtin_bit_cast(bf16x8, qv[kk]), st[g], 0, 0, 0);
                }
            };
            float m16 = kMaxInit, l16 = 0.0f;   // l16: this lane's share of the row sum
            f32x4 o16[DB];
#pragma unroll
            for (int db = 0; db < DB; ++db) o16[db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            // The row's token (packed: row / G) for the causal and window limits.
            const int lrow16 = koff + min(16 * rh + n16, prows - 1) / G;
            auto step16 = [&](f32x4 (&cur)[2], f32x4 (&nxt)[2], int kr, auto par, auto has_next) {
                constexpr int PAR = decltype(par)::value;
                const int j0 = (kb0 + kr) * BN;
                if ((j0 + BN > Lk) || (a.causal && j0 + BN - 1 > koff) || win > 0) {
                    // Key 16 g + i of the lane's 4-key run (offset 32 hoff + 4 q4 in the block).
                    const int base = j0 + 32 * hoff + 4 * q4;
                    const int lim = (a.causal ? min(lrow16, Lk - 1) : Lk - 1) - base;
                    const int llim = win > 0 ? lrow16 - win + 1 - base : -(1 << 30);
#pragma unroll
                    for (int g = 0; g < 2; ++g)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int off = 16 * g + i;
                            cur[g][i] = (off <= lim && off >= llim) ? cur[g][i] : -INFINITY;
                        }
                }
                float mt = fmaxf(fmaxf(fmaxf(cur[0][0], cur[0][1]), fmaxf(cur[0][2], cur[0][3])),
                                 fmaxf(fmaxf(cur[1][0], cur[1][1]), fmaxf(cur[1][2], cur[1][3])));
                mt = fmaxf(mt, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(mt), 0x401F)));   // lane ^ 16
                mt = max_xor32(mt) * cs;
                const bool need = mt > m16 + 8.0f;
                if (__builtin_expect(__any(need), 0)) {
                    if (need) {
                        const float alpha = __builtin_amdgcn_exp2f(m16 - mt);
                        m16 = mt;
                        l16 *= alpha;
#pragma unroll
                        for (int db = 0; db < DB; ++db)
#pragma unroll
                            for (int i = 0; i < 4; ++i) o16[db][i] *= alpha;
                    }
                }
                if constexpr (decltype(has_next)::value) scores16(nxt, std::integral_constant<int, 1 - PAR>{});
                u32x4 pb;
                {
                    float p[8];
#pragma unroll
                    for (int g = 0; g < 2; ++g)
#pragma unroll
                        for (int i = 0; i < 4; ++i) p[4 * g + i] = __builtin_amdgcn_exp2f(fmaf(cur[g][i], cs, -m16));
                    pb = u32x4{pack_bf16x2_rne_hw(p[0], p[1]), pack_bf16x2_rne_hw(p[2], p[3]),
                               pack_bf16x2_rne_hw(p[4], p[5]), pack_bf16x2_rne_hw(p[6], p[7])};
                    // The row sum adds the bf16-rounded weights the product uses.
                    l16 = dot2_bf16(pb.x, ones_bf16x2, l16);
                    l16 = dot2_bf16(pb.y, ones_bf16x2, l16);
                    l16 = dot2_bf16(pb.z, ones_bf16x2, l16);
                    l16 = dot2_bf16(pb.w, ones_bf16x2, l16);
                }
                const PGQA_LDS char* vt = ring + (2 + PAR) * P::TILEB + 32 * hoff * P::ROWB;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PGQA_LDS i16x4*)(vt + (vx16 ^ (db << 5))));
                    const i16x4 hi =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((PGQA_LDS i16x4*)(vt + 16 * P::ROWB + (vx16 ^ (db << 5))));
                    const u32x4 va = u32x4{__builtin_bit_cast(u32x2, lo).x, __builtin_bit_cast(u32x2, lo).y,
                                           __builtin_bit_cast(u32x2, hi).x, __builtin_bit_cast(u32x2, hi).y};
                    o16[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va),
                                                                      __builtin_bit_cast(bf16x8, pb), o16[db], 0, 0, 0);
                }
            };
            using J0 = std::integral_constant<int, 0>;
            using J1 = std::integral_constant<int, 1>;
            f32x4 sa16[2], sb16[2];
            wait_vmcnt<0>();
            __syncthreads();
            const int kend16 = Lq > 0 && last_kb >= 0 ? min(last_kb, kb1 - 1) - kb0 : -1;
            if (kend16 >= 0) scores16(sa16, J0{});
            int kb = 0;
            for (; kb + 2 <= kend16; kb += 2) {
                top(kb);
                step16(sa16, sb16, kb, J0{}, std::true_type{});
                top(kb + 1);
                step16(sb16, sa16, kb + 1, J1{}, std::true_type{});
            }
            if (kb + 1 == kend16) {
                top(kb);
                step16(sa16, sb16, kb, J0{}, std::true_type{});
                top(kb + 1);
                step16(sb16, sa16, kb + 1, J1{}, std::false_type{});
                kb += 2;
            } else if (kb == kend16) {
                top(kb);
                step16(sa16, sb16, kb, J0{}, std::false_type{});
                kb += 1;
            }
            for (; kb < nrel; ++kb) top(kb);

            // Key halves: wave (rh, 1) hands its running max, sum and output to
            // wave (rh, 0) through the idle ring (value-major, lane-minor).
            __syncthreads();
            PGQA_LDS float* xs = (PGQA_LDS float*)ring + rh * (4 * DB + 2) * 64;
            const int ln = lane_now();
            if (hoff == 1) {
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int i = 0; i < 4; ++i) xs[(4 * db + i) * 64 + ln] = o16[db][i];
                xs[4 * DB * 64 + ln] = m16;
                xs[(4 * DB + 1) * 64 + ln] = l16;
            }
            __syncthreads();
            if (hoff == 1 || Lq <= 0) return;
            {
                const float m1 = xs[4 * DB * 64 + ln];
                const float l1 = xs[(4 * DB + 1) * 64 + ln];
                const float mx = fmaxf(m16, m1);
                const float a0 = __builtin_amdgcn_exp2f(m16 - mx);
                const float a1 = __builtin_amdgcn_exp2f(m1 - mx);
                m16 = mx;
                l16 = l16 * a0 + l1 * a1;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int i = 0; i < 4; ++i) o16[db][i] = o16[db][i] * a0 + xs[(4 * db + i) * 64 + ln] * a1;
            }
            // The row sum over the four lanes of the row (lanes n, n+16, n+32, n+48).
            l16 += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(l16), 0x401F));
            l16 += shfl_xor_f32(l16, 32);
            const int r = 16 * rh + (ln & 15);
            const int qe = ln >> 4;
            if (r >= prows) return;
            const int tok = r / G;
            const int hq = kvh * G + r % G;
            if (split) {
                // Partial rows as the 32-row path writes them: O (dims 16 db + 4 qe ..
                // +3 from this lane), then (m, l) from the row's first lane.
                const int64_t prow = slot >= 0 ? (int64_t)slot * BQ + r
                                               : ((int64_t)(seq0 + tok) * a.num_q_heads + hq) * a.nchunk + chunk;
                float* po = a.part_o + prow * D + 4 * qe;
#pragma unroll
                for (int db = 0; db < DB; ++db) *(f32x4*)(po + 16 * db) = o16[db];
                if (qe == 0) *(float2*)(a.part_ml + prow * 2) = make_float2(m16, l16);
                return;
            }
            const float inv = l16 > 0.0f ? 1.0f / l16 : 0.0f;
            char* op = a.out + (int64_t)(seq0 + tok) * qstride + (int64_t)hq * D * 2 + 8 * qe;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                u32x2 w;
                w.x = pack_bf16x2_rne_hw(o16[db][0] * inv, o16[db][1] * inv);
                w.y = pack_bf16x2_rne_hw(o16[db][2] * inv, o16[db][3] * inv);
                *(u32x2*)(op + 32 * db) = w;
            }
            return;
        } else {
        // Blocks kb0 .. kb0 + kend are computed (kend = last_kb - kb0, or -1 for a
        // wave with no rows or no keys); each but the last overlaps the next block's
        // scores.  The two score
        // buffers alternate, so the loop runs two blocks per trip and every block
        // fully rewrites the buffer it fills; the ring parity is a compile-time
        // constant in each copy.  Waves past their last block keep the workgroup's
        // barriers and DMA going to the end.
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        f32x16 sa[2], sb[2];
        wait_vmcnt<0>();
        __syncthreads();
        if constexpr (Q8)
            if (nrel > 0) convert_q8<D>(ring, 0, -1);
        const int kend = active && last_kb >= 0 ? min(last_kb, kb1 - 1) - kb0 : -1;
        if (kend >= 0) scores(sa, I0{});
        int kb = 0;
        for (; kb + 2 <= kend; kb += 2) {
            top(kb);
            step(sa, sb, kb, I0{}, std::true_type{});
            top(kb + 1);
            step(sb, sa, kb + 1, I1{}, std::true_type{});
        }
        if (kb + 1 == kend) {
            top(kb);
            step(sa, sb, kb, I0{}, std::true_type{});
            top(kb + 1);
            step(sb, sa, kb + 1, I1{}, std::false_type{});
            kb += 2;
        } else if (kb == kend) {
            top(kb);
            step(sa, sb, kb, I0{}, std::false_type{});
            kb += 1;
        }
        for (; kb < nrel; ++kb) top(kb);

        // Epilogue: O / l rounded to bf16, staged through the idle ring so that
        // each output row is written whole.  The wave's 32 x D tile goes to LDS
        // (swizzled like the K/V tiles), then each lane writes one 16-byte chunk of
        // one row, CPR consecutive lanes per row.
        __syncthreads();   // every wave is done with the ring
        if constexpr (PACK) {
            // The two key halves of the same rows: wave 1's running max, sum and
            // output go through LDS (value-major, lane-minor: conflict-free) to wave 0,
            // which rescales both to the larger max and adds them.
            PGQA_LDS float* xs = (PGQA_LDS float*)(ring + 2 * BQ * P::ROWB);
            const int ln = lane_now();
            if (wave == 1 && active) {
#pragma unroll
                for (int db = 0; db < DBLK; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) xs[(16 * db + i) * 64 + ln] = o[db][i];
                xs[16 * DBLK * 64 + ln] = m;
                xs[(16 * DBLK + 1) * 64 + ln] = lsum;
            }
            __syncthreads();
            if (wave != 0) return;
            const float m1 = xs[16 * DBLK * 64 + ln];
            const float l1 = xs[(16 * DBLK + 1) * 64 + ln];
            const float mx = fmaxf(m, m1);
            const float a0 = __builtin_amdgcn_exp2f(m - mx);
            const float a1 = __builtin_amdgcn_exp2f(m1 - mx);
            m = mx;
            lsum = lsum * a0 + l1 * a1;
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][i] = o[db][i] * a0 + xs[(16 * db + i) * 64 + ln] * a1;
        }
        if (!active) return;
        const int lane_e = lane_now();
        const int half_e = lane_e >> 5;
        const int l32_e = lane_e & 31;
        lsum += shfl_xor_f32(lsum, 32);
        // Output row of the lane's row l32_e: token and query head (packed: the
        // row's token and head; else row i0 + l32_e of the wave's head).
        auto out_row = [&](int r, int& tok, int& hq) {
            if constexpr (PACK) {
                tok = r / G;
                hq = kvh * G + r % G;
            } else {
                tok = i0 + r;
                hq = head;
            }
        };
        const int rows_here = PACK ? prows : Lq - i0;   // valid rows of the wave's tile
        if (split) {
            // Partial of this key chunk (or of this piece of a stream-K share, in
            // its slot): unnormalised O, running max m and sum l (both halves of the
            // wave hold the row's m); a row with no key in the range leaves O = 0,
            // l = 0.
            if (l32_e < rows_here) {
                int tok, hq;
                out_row(l32_e, tok, hq);
                const int64_t prow = slot >= 0 ? (int64_t)slot * BQ + l32_e
                                               : ((int64_t)(seq0 + tok) * a.num_q_heads + hq) * a.nchunk + chunk;
                float* po = a.part_o + prow * D + 4 * half_e;
#pragma unroll
                for (int db = 0; db < DBLK; ++db)
#pragma unroll
                    for (int qd = 0; qd < 4; ++qd)
                        *(f32x4*)(po + 32 * db + 8 * qd) = f32x4{o[db][4 * qd], o[db][4 * qd + 1], o[db][4 * qd + 2],
                                                                o[db][4 * qd + 3]};
                if (half_e == 0) *(float2*)(a.part_ml + prow * 2) = make_float2(m, lsum);
            }
            return;
        }
        const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
        PGQA_LDS char* ot = ring + wave * (BQ * P::ROWB);
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                // dims 32*db + 8*qd + 4*half_e .. +3 of row l32_e: chunk 4*db + qd, byte 8*half_e
                u32x2 w;
                w.x = pack_bf16x2_rne_hw(o[db][4 * qd + 0] * inv, o[db][4 * qd + 1] * inv);
                w.y = pack_bf16x2_rne_hw(o[db][4 * qd + 2] * inv, o[db][4 * qd + 3] * inv);
                *(PGQA_LDS u32x2*)(ot + swz<D>(l32_e, 4 * db + qd) + 8 * half_e) = w;
            }
        const int c = lane_e % P::CPR;
#pragma unroll
        for (int t = 0; t < BQ / P::RPL; ++t) {
            const int r = t * P::RPL + lane_e / P::CPR;
            const u32x4 val = lds_read_16(ot + swz<D>(r, c));
            if (r < rows_here) {
                int tok, hq;
                out_row(r, tok, hq);
                *(u32x4*)(a.out + (int64_t)(seq0 + tok) * qstride + (int64_t)hq * D * 2 + c * 16) = val;
            }
        }
        }   // !P16
    };

    if constexpr (PACK) {
        if (a.sk_nw > 0) {
            // Stream-K shares.  A pair's work is counted in units: sk_pair_units
            // for the start-up of its piece (Q and the first tiles' latency, about
            // that of a few blocks), then one per key block (those of its window,
            // as the tile computes them; at least one unit in all, so a pair whose
            // rows have no key gets the piece that writes its zero rows).  A
            // piece's blocks are its units past the start-up ones.  The pairs'
            // units, concatenated in pair order, are cut into
            // sk_nw equal shares and workgroup w runs the pieces of share w: whole
            // pairs straight to the output, a pair cut by a share edge as partials
            // in slot 2w (the share's first piece) or 2w + 1 (its last), which
            // sk_merge_kernel combines.  Shares are equal in bytes whatever the
            // context lengths, and share w runs on XCD w % 8, so the XCDs and
            // workgroups finish together.
            const int npairs = a.batch * a.num_kv_heads;
            const int per = (npairs + 255) / 256;              // pairs per thread in the scan
            const int t = threadIdx.x;
            auto units = [&](int p, int& b0, int& lq, int& lk, int& kbw) {
                const int sq = p / a.num_kv_heads;
                if (a.fixed_qlen > 0) {
                    b0 = min(sq * a.fixed_qlen, a.total_tokens);
                    lq = min(b0 + a.fixed_qlen, a.total_tokens) - b0;
                } else {
                    b0 = clampi(a.cu_seqlens[sq], 0, a.total_tokens);
                    lq = clampi(a.cu_seqlens[sq + 1], b0, a.total_tokens) - b0;
                }
                lk = clampi(a.context_lens[sq], 0, a.ctx_cap);
                // Every packed row's keys end at the sequence's last key; a window
                // starts the reads at the first row's edge.
                const int nkb = (lk + BN - 1) / BN;
                kbw = (a.window > 0 && nkb > 0) ? max(0, lk - lq - a.window + 1) / BN : 0;
                return lq > 0 ? max(1, a.sk_pair_units + nkb - kbw) : 0;
            };
            // Block-wide exclusive scan of the per-thread sums (thread t: pairs
            // t * per .. t * per + per - 1).
            int sum = 0;
            for (int i = 0; i < per; ++i) {
                const int p = t * per + i;
                int b0, lq, lk, kbw;
                if (p < npairs) sum += units(p, b0, lq, lk, kbw);
            }
            int inc = sum;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(inc, off);
                if (lane >= off) inc += y;
            }
            PGQA_LDS int* sh = (PGQA_LDS int*)ring;
            if (lane == 63) sh[wave] = inc;
            __syncthreads();
            const int wsum0 = sh[0], wsum1 = sh[1], wsum2 = sh[2], wsum3 = sh[3];
            const int total = wsum0 + wsum1 + wsum2 + wsum3;
            const int excl = (wave > 0 ? wsum0 : 0) + (wave > 1 ? wsum1 : 0) + (wave > 2 ? wsum2 : 0) + inc - sum;
            const int w = blockIdx.x;
            const int lo = (int)((int64_t)w * total / a.sk_nw);
            const int hi = (int)((int64_t)(w + 1) * total / a.sk_nw);
            // The pair holding unit lo, found by the thread whose range holds it.
            if (lo < hi && lo >= excl && lo < excl + sum) {
                int u0 = excl;
                for (int i = 0; i < per; ++i) {
                    const int p = t * per + i;
                    int b0, lq, lk, kbw;
                    const int u = p < npairs ? units(p, b0, lq, lk, kbw) : 0;
                    if (lo < u0 + u) {
                        sh[4] = p;
                        sh[5] = u0;
                        break;
                    }
                    u0 += u;
                }
            }
            __syncthreads();
            int cut_p = -1, cut_u0 = 0, cut_u1 = 0;
            if (lo < hi) {
                int p = __builtin_amdgcn_readfirstlane(sh[4]);
                int U = __builtin_amdgcn_readfirstlane(sh[5]);
                while (U < hi && p < npairs) {
                    int b0, lq, lk, kbw;
                    const int u = __builtin_amdgcn_readfirstlane(units(p, b0, lq, lk, kbw));
                    if (u > 0) {
                        b0 = __builtin_amdgcn_readfirstlane(b0);
                        lq = __builtin_amdgcn_readfirstlane(lq);
                        lk = __builtin_amdgcn_readfirstlane(lk);
                        kbw = __builtin_amdgcn_readfirstlane(kbw);
                        const int plo = max(lo, U) - U;
                        const int phi = min(hi, U + u) - U;
                        const bool whole = plo == 0 && phi == u;
                        const int slot = whole ? -1 : 2 * w + (U <= lo ? 0 : 1);
                        if (U >= lo && U + u > hi) {   // begins here, ends in a later share
                            cut_p = p;
                            cut_u0 = U;
                            cut_u1 = U + u;
                        }
                        const int sq = p / a.num_kv_heads;
                        // Every wave is done with the ring (the scan's words, the
                        // previous piece's tiles) before this piece's DMA.
                        __syncthreads();
                        const int c0 = a.sk_pair_units;
                        tile(sq, p - sq * a.num_kv_heads, 0, 0, b0, lq, lk, kbw + max(0, plo - c0), kbw + max(0, phi - c0),
                             !whole, 0, slot);
                    }
                    U += u;
                    ++p;
                }
            }
            // For the merge: the pair that begins in this share and is cut at its end.
            if (t == 0) *(int4*)(a.sk_cut + 4 * w) = make_int4(cut_p, cut_u0, cut_u1, total);
            return;
        }
    }

    // Work mapping.  Workgroups are dealt to the 8 XCDs round-robin by linear
    // id and every XCD has its own L2, so all tiles of one (sequence, KV head)
    // pair stay on one XCD: pair p = seq * Hkv + kvh lives on XCD p % 8.  Each
    // XCD runs its pairs one after another (so the K/V being read at any time
    // is that of one or two pairs, which its L2 holds), and a pair's tiles
    // heaviest-first (query tiles from the last), the head groups sharing the
    // pair's K/V side by side.
    //
    // Dense lists (up to 64 pairs per XCD): XCD x's list holds, pair after
    // pair, only the query tiles that exist (ceil(Lq / rows) per pair, found by
    // a wave-wide scan of the pairs' lengths), so no workgroup is launched for
    // the tiles short sequences lack.  Otherwise every pair gets nqt levels
    // (the longest sequence's tile count) and levels past a sequence's end exit.
    const int id = blockIdx.x;
    const int per_tile = groups * a.nchunk;
    int kq, r3, ntiles;
    int d_seq0 = 0, d_lq = 0, d_lk = 0;   // the chosen pair's rows and keys, from the scan's loads
    if (a.dense) {
        const int j = id >> 3;
        const int p = (id & 7) + 8 * lane;
        int nt = 0, b0 = 0, lq = 0, lk = 0;
        if (lane < a.pairs_per_xcd && p < a.batch * a.num_kv_heads) {
            const int sq = p / a.num_kv_heads;
            if (a.fixed_qlen > 0) {
                b0 = min(sq * a.fixed_qlen, a.total_tokens);
                lq = min(b0 + a.fixed_qlen, a.total_tokens) - b0;
            } else {
                b0 = clampi(a.cu_seqlens[sq], 0, a.total_tokens);
                lq = clampi(a.cu_seqlens[sq + 1], b0, a.total_tokens) - b0;
            }
            if constexpr (PAGED) lk = clampi(a.context_lens[sq], 0, a.ctx_cap);
            nt = (lq + TB * BQ - 1) / (TB * BQ);
        }
        if (a.chunk_lpt) {
            // Key chunks longest first: every pair's full chunks (pair after
            // pair), then every pair's last, shorter chunk.  A batch whose chunks
            // outnumber the workgroup slots then leaves short chunks, not full
            // ones, for the second round.  Only the chunks that exist are listed
            // (a pair with no keys keeps one chunk, which writes its zero rows).
            const int ck = a.kchunk * BN;
            const int fa = nt > 0 ? lk / ck : 0;
            const int tb = (nt > 0 && (lk == 0 || lk % ck != 0)) ? 1 : 0;
            int pa = fa, pb = tb;                        // inclusive scans
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int ya = __shfl_up(pa, off);
                const int yb = __shfl_up(pb, off);
                if (lane >= off) {
                    pa += ya;
                    pb += yb;
                }
            }
            const int tot_a = __builtin_amdgcn_readfirstlane(__shfl(pa, 63));
            if (j < tot_a) {
                kq = __builtin_amdgcn_readfirstlane(__popcll(__ballot(pa <= j)));
                if (kq >= a.pairs_per_xcd) return;
                r3 = j - (kq > 0 ? __builtin_amdgcn_readfirstlane(__shfl(pa, kq - 1)) : 0);
            } else {
                kq = __builtin_amdgcn_readfirstlane(__popcll(__ballot(pb <= j - tot_a)));
                if (kq >= a.pairs_per_xcd) return;
                r3 = __builtin_amdgcn_readfirstlane(__shfl(fa, kq));   // the last chunk's index
            }
        } else {
            int pre = nt * per_tile;                      // inclusive scan of the list lengths
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(pre, off);
                if (lane >= off) pre += y;
            }
            // Pairs whose list ends at or before j come first (pre is non-decreasing).
            kq = __builtin_amdgcn_readfirstlane(__popcll(__ballot(pre <= j)));
            if (kq >= a.pairs_per_xcd) return;
            r3 = j - (kq > 0 ? __builtin_amdgcn_readfirstlane(__shfl(pre, kq - 1)) : 0);
        }
        ntiles = __builtin_amdgcn_readfirstlane(__shfl(nt, kq));
        d_seq0 = __builtin_amdgcn_readfirstlane(__shfl(b0, kq));
        d_lq = __builtin_amdgcn_readfirstlane(__shfl(lq, kq));
        if constexpr (PAGED) d_lk = __builtin_amdgcn_readfirstlane(__shfl(lk, kq));
    } else {
        const int per_pair = a.nqt * per_tile;
        kq = (id >> 3) / per_pair;                       // the XCD's kq-th pair
        r3 = (id >> 3) - kq * per_pair;
        ntiles = a.nqt;
    }
    const int r2 = r3 / a.nchunk;
    const int chunk = r3 - r2 * a.nchunk;                // key chunk (0 without a split)
    const int level = r2 / groups;
    const int grp = r2 - level * groups;
    const int pair = (id & 7) + 8 * kq;
    if (pair >= a.batch * a.num_kv_heads) return;
    const int s = pair / a.num_kv_heads;
    const int kvh = pair - s * a.num_kv_heads;
    // The pair's query rows and keys.
    // (Loaded values count as divergent for the compiler: readfirstlane keeps
    // the sizes, and every branch on them, scalar.)
    // (With dense lists these come from the scan's loads: no second round trip.)
    const int seq0 = a.dense ? d_seq0
                     : a.fixed_qlen > 0 ? min(s * a.fixed_qlen, a.total_tokens)
                     : __builtin_amdgcn_readfirstlane(clampi(a.cu_seqlens[s], 0, a.total_tokens));
    const int Lq = a.dense ? d_lq
                   : a.fixed_qlen > 0 ? min(seq0 + a.fixed_qlen, a.total_tokens) - seq0
                   : __builtin_amdgcn_readfirstlane(clampi(a.cu_seqlens[s + 1], seq0, a.total_tokens)) - seq0;
    const int Lk = PAGED ? (a.dense ? d_lk : __builtin_amdgcn_readfirstlane(clampi(a.context_lens[s], 0, a.ctx_cap)))
                         : Lq;
    const int qtile = ntiles - 1 - level;
    const int tok0 = qtile * TB * BQ;
    if (tok0 >= Lq) return;
    // Chunks past the sequence's keys do not exist (chunk 0 always does).
    const int ckeys = a.kchunk * BN;
    if (chunk > 0 && chunk * ckeys >= Lk) return;
    const bool split = Lk > ckeys;                       // partials instead of the output
    tile(s, kvh, grp, qtile, seq0, Lq, Lk, chunk * a.kchunk, chunk * a.kchunk + a.kchunk, split, chunk, -1);
}

// Merge of the key-chunk partials of split sequences: a query row's Hq x D
// outputs go to one thread each, a 256-thread workgroup taking 256 / (Hq x D)
// rows when a row has fewer outputs than that (one wave or more per row, so
// each wave belongs to one row and finds its sequence once), else
// (Hq x D) / 256 workgroups sharing one row.  Log-sum-exp of the chunks in chunk order with a
// running maximum (deterministic; the loads of successive chunks do not wait on
// one another).  A chunk in which a row sees no key holds m = -1e30 (finite),
// l = 0, O = 0 and so adds nothing.  Rows of sequences that fit one chunk were
// written by the attention kernel.
// Merge workgroups of the whole call (a row's outputs, Hq x D, are a multiple
// of 64; a row with more than 256 of them takes (Hq x D + 255) / 256 workgroups).
template <int D>
int64_t merge_grid(int total_rows, int num_q_heads) {
    const int per = num_q_heads * D;
    if (per >= 256) return (int64_t)total_rows * ((per + 255) / 256);
    const int rpw = 256 / per;
    return ((int64_t)total_rows + rpw - 1) / rpw;
}

template <int D>
__global__ __launch_bounds__(256) void extend_merge_kernel(PrefillArgs a) {
    const int per = a.num_q_heads * D;
    const int rpw = per >= 256 ? 1 : 256 / per;
    const int wpr = per > 256 ? (per + 255) / 256 : 1;     // workgroups per row
    const int sub = rpw > 1 ? (int)threadIdx.x / per : 0;
    if (sub >= rpw) return;                                 // threads past the last whole row
    const int row = wpr > 1 ? (int)(blockIdx.x / wpr) : (int)blockIdx.x * rpw + sub;
    if (row >= a.total_tokens) return;
    int lo = 0, hi = a.batch - 1;                          // the sequence holding the row
    if (a.fixed_qlen > 0) {
        lo = min(row / a.fixed_qlen, hi);
    } else {
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (__builtin_amdgcn_readfirstlane(a.cu_seqlens[mid]) <= row) lo = mid;
            else hi = mid - 1;
        }
    }
    const int Lk = __builtin_amdgcn_readfirstlane(clampi(a.context_lens[lo], 0, a.ctx_cap));
    const int ckeys = a.kchunk * BN;
    const int nc = Lk > ckeys ? (Lk + ckeys - 1) / ckeys : 1;
    if (nc <= 1) return;
    const int e0 = rpw > 1 ? (int)threadIdx.x - sub * per : (int)(blockIdx.x % wpr) * 256 + (int)threadIdx.x;
    for (int e = e0; e < per; e += 256 * wpr) {
        const int64_t rh = (int64_t)row * a.num_q_heads + e / D;
        const float* ml = a.part_ml + rh * a.nchunk * 2;
        const float* po = a.part_o + rh * a.nchunk * D + e % D;
        float M = -INFINITY, acc = 0.0f, L = 0.0f;
#pragma unroll 4
        for (int c = 0; c < nc; ++c) {
            const float mc = ml[2 * c];
            const float lc = ml[2 * c + 1];
            const float oc = po[(int64_t)c * D];
            const float mn = fmaxf(M, mc);
            const float sa = __builtin_amdgcn_exp2f(M - mn);
            const float sb = __builtin_amdgcn_exp2f(mc - mn);
            acc = acc * sa + oc * sb;
            L = L * sa + lc * sb;
            M = mn;
        }
        const float r = L > 0.0f ? acc / L : 0.0f;
        *(uint16_t*)(a.out + (rh * D + e % D) * 2) = (uint16_t)f32_to_bf16_bits(r);
    }
}

// Merge of the stream-K partials (packed rows): workgroup w merges the pair that
// begins in share w and is cut at its end, if any (each cut pair has exactly one
// such share).  Its pieces lie in shares w .. wl: slot 2w + 1 (or 2w when the
// pair begins at the share's start) and slot 2v for each later share v (the
// piece that opens share v).  Log-sum-exp over the pieces in key order with a
// running maximum, as extend_merge_kernel does over key chunks.  Workgroup
// (w, g) takes rows g * RPP .. of share w's pair, each thread 4 dims of one row.
template <int D>
constexpr int sk_merge_groups() { return BQ / (256 / (D / 4)); }

template <int D>
__global__ __launch_bounds__(256) void sk_merge_kernel(PrefillArgs a) {
    const int w = blockIdx.x / sk_merge_groups<D>();
    const int g = blockIdx.x % sk_merge_groups<D>();
    const int4 cut = *(const int4*)(a.sk_cut + 4 * w);
    const int p = __builtin_amdgcn_readfirstlane(cut.x);
    if (p < 0) return;
    const int u0 = __builtin_amdgcn_readfirstlane(cut.y);
    const int u1 = __builtin_amdgcn_readfirstlane(cut.z);
    const int total = __builtin_amdgcn_readfirstlane(cut.w);
    const int nw = a.sk_nw;
    const int lo = (int)((int64_t)w * total / nw);
    const int wl = (int)(((int64_t)u1 * nw - 1) / total);   // share holding unit u1 - 1
    const int sq = p / a.num_kv_heads;
    const int kvh = p - sq * a.num_kv_heads;
    const int G = a.num_q_heads / a.num_kv_heads;
    int b0, lq;
    if (a.fixed_qlen > 0) {
        b0 = min(sq * a.fixed_qlen, a.total_tokens);
        lq = min(b0 + a.fixed_qlen, a.total_tokens) - b0;
    } else {
        b0 = __builtin_amdgcn_readfirstlane(clampi(a.cu_seqlens[sq], 0, a.total_tokens));
        lq = __builtin_amdgcn_readfirstlane(clampi(a.cu_seqlens[sq + 1], b0, a.total_tokens)) - b0;
    }
    const int rows = min(lq * G, BQ);
    constexpr int TPR = D / 4;          // threads per row
    constexpr int RPP = 256 / TPR;      // rows per pass
    const int c4 = (int)threadIdx.x % TPR;
    const int r = g * RPP + (int)threadIdx.x / TPR;
    if (r < rows) {
        float M = -INFINITY, L = 0.0f;
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        // Four pieces per trip, their loads issued together (share w's piece
        // comes first, so M is finite after it; a share past wl or an empty one
        // adds nothing).
        for (int v0 = w; v0 <= wl; v0 += 4) {
            float2 ml[4];
            f32x4 oc[4];
            bool ok[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int v = v0 + j;
                ok[j] = v <= wl && (int)((int64_t)v * total / nw) < (int)((int64_t)(v + 1) * total / nw);
                const int slot = ok[j] ? 2 * v + ((v == w && u0 > lo) ? 1 : 0) : 2 * w;
                const int64_t row = (int64_t)slot * BQ + r;
                ml[j] = *(const float2*)(a.part_ml + row * 2);
                oc[j] = *(const f32x4*)(a.part_o + row * D + 4 * c4);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (!ok[j]) continue;
                const float mn = fmaxf(M, ml[j].x);
                const float sa = __builtin_amdgcn_exp2f(M - mn);
                const float sb = __builtin_amdgcn_exp2f(ml[j].x - mn);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = acc[i] * sa + oc[j][i] * sb;
                L = L * sa + ml[j].y * sb;
                M = mn;
            }
        }
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        const int tok = r / G;
        const int hq = kvh * G + r % G;
        u32x2 o;
        o.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
        o.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
        *(u32x2*)(a.out + (((int64_t)(b0 + tok) * a.num_q_heads + hq) * D + 4 * c4) * 2) = o;
    }
}

typedef void (*PrefillFn)(PrefillArgs);

template <int D, bool PAGED, bool Q8>
PrefillFn pick_hg(int h, bool pack, bool p16 = false) {
    if constexpr (!PAGED) {
        return Q8 || pack ? nullptr
                          : (h == 4 ? prefill_kernel<D, 4, false> : (h == 2 ? prefill_kernel<D, 2, false>
                                                                               : prefill_kernel<D, 1, false>));
    } else {
        if constexpr (!Q8)
            if (pack && p16) return prefill_kernel<D, 1, true, false, true, true>;
        if (pack) return prefill_kernel<D, 1, true, Q8, true>;
        return h == 4 ? prefill_kernel<D, 4, PAGED, Q8>
                      : (h == 2 ? prefill_kernel<D, 2, PAGED, Q8> : prefill_kernel<D, 1, PAGED, Q8>);
    }
}

#ifndef PGQA_EXT_PACK
#define PGQA_EXT_PACK 1
#endif

// Packed rows (paged calls): every sequence's query tokens times the group fit
// one 32-row tile.
bool use_pack(int group, int max_q_len) {
    return PGQA_EXT_PACK && max_q_len > 0 && group <= BQ && (int64_t)max_q_len * group <= BQ;
}

#ifndef PGQA_PACK16
#define PGQA_PACK16 1
#endif

// Packed rows in 16-row waves (bf16 pages, more than 16 rows: both row halves of
// the tile are used, so all four waves compute).
bool use_pack16(int group, int max_q_len, bool q8) {
    return PGQA_PACK16 && !q8 && use_pack(group, max_q_len) && (int64_t)max_q_len * group > 16;
}

#ifndef PGQA_EXT_SK
#define PGQA_EXT_SK 1
#endif

#ifndef PGQA_SK_PAIR_UNITS
#define PGQA_SK_PAIR_UNITS 3
#endif

constexpr int kSkMaxPairs = 4096;   // every share's workgroup scans all pairs: 16 per thread at most

int cu_count();

// Stream-K shares of a packed-rows call: one per workgroup slot (two per CU, the
// kernel's occupancy), but no more than the call has work units (an upper bound
// from the host-side sizes), or 0 when the pairs are too many for the
// per-workgroup scan.
int sk_shares(int64_t npairs, int max_context_len, int window, int max_q_len) {
    if (!PGQA_EXT_SK || npairs <= 0 || npairs > kSkMaxPairs) return 0;
    int64_t blocks = ((int64_t)max_context_len + BN - 1) / BN;
    if (window > 0) blocks = std::min<int64_t>(blocks, ((int64_t)window + max_q_len + 2 * BN - 2) / BN);
    const int64_t units = npairs * (std::max<int64_t>(blocks, 1) + PGQA_SK_PAIR_UNITS);
    return (int)std::min<int64_t>((int64_t)2 * cu_count(), units);
}

// Workspace of nw shares: the per-share cut records, then two partial slots of
// 32 rows per share (output rows, then (m, l)).
size_t sk_workspace_bytes(int nw, int head_dim) {
    return (size_t)nw * 16 + (size_t)2 * nw * BQ * (head_dim + 2) * 4;
}

// Kernel for a head_dim and group size; hg = heads per workgroup (packed: the
// whole group, one workgroup per KV head).
template <bool PAGED>
bool pick(int head_dim, int group, PrefillFn* fn, int* hg, bool q8 = false, bool pack = false, bool p16 = false) {
    const int h = group >= 4 ? 4 : group;
    if (group != 1 && group != 2 && group % 4 != 0) return false;
    if (group > 64) return false;
    if ((q8 || pack) && !PAGED) return false;
    *hg = pack ? group : h;
    if (head_dim == 128) {
        *fn = q8 ? pick_hg<128, PAGED, true>(h, pack) : pick_hg<128, PAGED, false>(h, pack, p16);
        return true;
    }
    if (head_dim == 64) {
        *fn = q8 ? pick_hg<64, PAGED, true>(h, pack) : pick_hg<64, PAGED, false>(h, pack, p16);
        return true;
    }
    return false;
}

// Ring (two K and two V tiles), plus the row-scale slots with FP8 pages.
size_t lds_bytes(int head_dim, bool q8) {
    return (head_dim == 128 ? 4 * PGeo<128>::TILEB : 4 * PGeo<64>::TILEB) + (q8 ? kScaleB : 0);
}

int rows_per_load(int head_dim) { return head_dim == 128 ? PGeo<128>::RPL : PGeo<64>::RPL; }

int cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return 256;
    return n;
}

constexpr int kNoSplit = 1 << 24;   // key blocks per chunk when nothing is split

// Key split of a paged multi-token call.  Without it there is one workgroup per
// (query tile, head group, sequence, KV head); when that grid cannot even fill
// the GPU's workgroup slots (two per CU) the long contexts run on a few CUs, so
// key ranges are cut into chunks (at least 4 blocks) for about two workgroups
// per slot.  (A grid that fills the slots once is left alone: shorter chunks
// cost more in per-workgroup start-up than they recover in balance.)
// max_chunks (from the caller's workspace) caps the count.
void extend_split(int64_t wgs_unsplit, int max_context_len, int64_t max_chunks, int* nchunk, int* kchunk) {
    *nchunk = 1;
    *kchunk = kNoSplit;
    const int64_t slots = 2 * (int64_t)cu_count();
    const int blocks = (max_context_len + BN - 1) / BN;
    if (wgs_unsplit >= slots || blocks < 8 || max_chunks < 2) return;
    int64_t nc = (2 * slots + wgs_unsplit - 1) / wgs_unsplit;
    if (nc > max_chunks) nc = max_chunks;
    int kc = (int)((blocks + nc - 1) / nc);
    if (kc < 4) kc = 4;
    nc = (blocks + kc - 1) / kc;
    if (nc <= 1) return;
    *nchunk = (int)nc;
    *kchunk = kc;
}

// Query tokens per workgroup: (4 / hg) tiles of 32 rows; packed, 32 / group
// tokens (every sequence has at most that many).
int tokens_per_wg(const PrefillArgs& a, int hg, int group) { return a.pack ? max(1, BQ / group) : (4 / hg) * BQ; }

// Tile levels, XCD packing and grid size shared by both entry points.
void grid_dims(PrefillArgs& a, int hg, int group, int max_q_rows) {
    const int rows_per_wg = tokens_per_wg(a, hg, group);
    a.nqt = a.pack ? 1 : (max_q_rows + rows_per_wg - 1) / rows_per_wg;
    a.pairs_per_xcd = (int)(((int64_t)a.batch * a.num_kv_heads + 7) / 8);
    (void)group;
}

int64_t grid_size(const PrefillArgs& a, int hg, int group) {
    return 8 * (int64_t)a.nqt * a.pairs_per_xcd * (group / hg) * a.nchunk;
}

// Launched grid: with dense lists, 8 x the longest XCD list, bounded by the
// rows: an XCD holds at most ceil(Hkv / 8) pairs of any one sequence, so its
// list has at most ceil(Hkv/8) * T / rows + pairs_per_xcd tiles per head group
// and chunk (T = packed query rows).  Workgroups past their XCD's list exit.
int64_t launch_grid(PrefillArgs& a, int hg, int group, int64_t total_rows) {
    const int rows_per_wg = tokens_per_wg(a, hg, group);
    a.dense = a.pairs_per_xcd <= 64 ? 1 : 0;
    if (!a.dense) return grid_size(a, hg, group);
    const int64_t per_kv = ((int64_t)a.num_kv_heads + 7) / 8;
    const int64_t tiles = min((int64_t)a.nqt * a.pairs_per_xcd, per_kv * total_rows / rows_per_wg + a.pairs_per_xcd);
    return 8 * tiles * (group / hg) * a.nchunk;
}

hipError_t launch(PrefillFn fn, PrefillArgs& a, int hg, int group, int head_dim, hipStream_t stream) {
    const int64_t wgs = a.sk_nw > 0 ? a.sk_nw : launch_grid(a, hg, group, a.total_tokens);
    if (wgs > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (log_enabled() && a.sk_nw > 0)
        log_line("extend B=%d rows=%d Hq=%d Hkv=%d d=%d%s window=%d: packed rows%s, %d stream-K shares, %s K/V loads",
                 a.batch, a.total_tokens, a.num_q_heads, a.num_kv_heads, head_dim, a.k_scale ? " fp8" : "",
                 a.window, a.pack == 2 ? " in 16-row waves" : "", a.sk_nw, a.kv_nt ? "non-temporal" : "cached");
    else if (log_enabled())
        log_line("%s B=%d rows=%d Hq=%d Hkv=%d d=%d%s window=%d: %lld workgroups (%s tile lists, %d query-tile "
                 "levels, %d pairs per XCD, %d head(s) per wave group%s), key chunks %d x %d blocks%s, %s K/V loads",
                 a.block_table ? "extend" : "prefill", a.batch, a.total_tokens, a.num_q_heads, a.num_kv_heads,
                 head_dim, a.k_scale ? " fp8" : "", a.window, (long long)wgs, a.dense ? "dense" : "full", a.nqt,
                 a.pairs_per_xcd, hg, a.pack == 2 ? ", 16-row waves" : "", a.nchunk, a.nchunk > 1 ? a.kchunk : 0,
                 a.chunk_lpt ? " (longest first)" : "", a.kv_nt ? "non-temporal" : "cached");
    hipLaunchKernelGGL(fn, dim3((unsigned)wgs), dim3(256), lds_bytes(head_dim, a.k_scale != nullptr), stream, a);
    return hipGetLastError();
}

}  // namespace

bool prefill_supported(int32_t head_dim, int32_t group) {
    PrefillFn fn;
    int hg;
    return pick<false>(head_dim, group, &fn, &hg);
}

bool extend_supported(int32_t head_dim, int32_t group, int32_t block_size) {
    PrefillFn fn;
    int hg;
    return pick<true>(head_dim, group, &fn, &hg) && block_size >= rows_per_load(head_dim) && block_size <= 256;
}

bool extend_supported_fp8(int32_t head_dim, int32_t group, int32_t block_size) {
    PrefillFn fn;
    int hg;
    // A 1 KB wave-load of codes (1024 / head_dim rows) must lie in one page.
    return pick<true>(head_dim, group, &fn, &hg, true) && block_size >= 1024 / head_dim && block_size <= 256;
}

hipError_t launch_prefill(const PrefillLaunch& L, hipStream_t stream) {
    const int group = L.num_q_heads / L.num_kv_heads;
    PrefillFn fn;
    int hg;
    if (!pick<false>(L.head_dim, group, &fn, &hg)) return hipErrorInvalidValue;
    PrefillArgs a = {};
    a.q = (const char*)L.q;
    a.k = (const char*)L.k;
    a.v = (const char*)L.v;
    a.cu_seqlens = L.cu_seqlens;
    a.out = (char*)L.out;
    a.total_tokens = L.total_tokens;
    a.num_q_heads = L.num_q_heads;
    a.num_kv_heads = L.num_kv_heads;
    a.causal = L.causal;
    const ScaleFold sf = fold_scale(L.scale, true);
    a.scale_log2 = sf.cs;
    a.q_and = sf.q_and;
    a.q_xor = sf.q_xor;
    a.batch = L.batch;
    a.window = L.window;
    a.nchunk = 1;
    a.kchunk = kNoSplit;
    grid_dims(a, hg, group, L.max_seqlen);
    a.kv_nt = (group == hg && a.nqt == 1) ? 1 : 0;
    return launch(fn, a, hg, group, L.head_dim, stream);
}

hipError_t launch_extend(const ExtendLaunch& L, hipStream_t stream) {
    const int group = L.num_q_heads / L.num_kv_heads;
    PrefillFn fn;
    int hg;
    const bool q8 = L.k_scale != nullptr;
    if (q8 ? !extend_supported_fp8(L.head_dim, group, 1 << L.block_size_log2)
           : !extend_supported(L.head_dim, group, 1 << L.block_size_log2))
        return hipErrorInvalidValue;
    const bool pack = use_pack(group, L.max_q_len);
    const bool p16 = use_pack16(group, L.max_q_len, q8);
    pick<true>(L.head_dim, group, &fn, &hg, q8, pack, p16);
    PrefillArgs a = {};
    a.pack = pack ? (p16 ? 2 : 1) : 0;   // 2: 16-row waves
    a.k_scale = L.k_scale;
    a.v_scale = L.v_scale;
    a.q = (const char*)L.q;
    a.k = (const char*)L.k_cache;
    a.v = (const char*)L.v_cache;
    a.cu_seqlens = L.cu_q;
    a.out = (char*)L.out;
    a.total_tokens = L.total_q;
    a.num_q_heads = L.num_q_heads;
    a.num_kv_heads = L.num_kv_heads;
    a.causal = L.non_causal ? 0 : 1;
    a.fixed_qlen = L.fixed_qlen;
    const ScaleFold sf = fold_scale(L.scale, true);
    a.scale_log2 = sf.cs;
    a.q_and = sf.q_and;
    a.q_xor = sf.q_xor;
    a.batch = L.batch;
    a.block_table = L.block_table;
    a.context_lens = L.context_lens;
    a.max_blocks_per_seq = L.max_blocks_per_seq;
    a.num_blocks = L.num_blocks;
    a.bs_log2 = L.block_size_log2;
    a.ctx_cap = L.max_context_len;
    a.window = L.window;
    grid_dims(a, hg, group, L.max_q_len);
    a.nchunk = 1;
    if (pack) {
        // Packed rows: stream-K shares when the workspace holds their partials.
        const int nw = sk_shares((int64_t)L.batch * L.num_kv_heads, L.max_context_len, L.window, L.max_q_len);
        if (nw > 0 && L.workspace && L.workspace_bytes >= sk_workspace_bytes(nw, L.head_dim)) {
            a.sk_nw = nw;
            a.sk_pair_units = PGQA_SK_PAIR_UNITS;
            a.kchunk = kNoSplit;
            a.kv_nt = 1;   // each K/V byte goes to one workgroup
            a.sk_cut = (int32_t*)L.workspace;
            a.part_o = (float*)((char*)L.workspace + (size_t)nw * 16);
            a.part_ml = a.part_o + (int64_t)2 * nw * BQ * L.head_dim;
            hipError_t err = launch(fn, a, hg, group, L.head_dim, stream);
            if (err != hipSuccess) return err;
            if (L.head_dim == 128)
                hipLaunchKernelGGL(sk_merge_kernel<128>, dim3((unsigned)nw * sk_merge_groups<128>()), dim3(256), 0,
                                   stream, a);
            else
                hipLaunchKernelGGL(sk_merge_kernel<64>, dim3((unsigned)nw * sk_merge_groups<64>()), dim3(256), 0,
                                   stream, a);
            return hipGetLastError();
        }
    }
    const int64_t per_chunk = (int64_t)L.total_q * L.num_q_heads * (L.head_dim + 2) * 4;
    const int64_t max_chunks = (L.workspace && per_chunk > 0) ? (int64_t)(L.workspace_bytes / per_chunk) : 0;
    a.kchunk = kNoSplit;
    if (L.chunk_blocks > 0) {
        // Caller-chosen chunk length (few query rows per sequence: every
        // workgroup is bound by its ring's one-block-ahead DMA latency, so many
        // short chunks beat a few long ones), capped by the workspace.
        const int blocks = (L.max_context_len + BN - 1) / BN;
        int kc = L.chunk_blocks;
        int64_t nc = (blocks + kc - 1) / kc;
        if (nc > max_chunks) {
            nc = max_chunks > 0 ? max_chunks : 1;
            kc = (int)((blocks + nc - 1) / nc);
            nc = (blocks + kc - 1) / kc;
        }
        if (nc > 1) {
            a.nchunk = (int)nc;
            a.kchunk = kc;
        }
    } else {
        extend_split(grid_size(a, hg, group), L.max_context_len, max_chunks, &a.nchunk, &a.kchunk);
    }
    // One query tile and one head group per pair: list the key chunks longest
    // first (the kernel does so with dense lists).
    a.chunk_lpt = (a.nchunk > 1 && group == hg && a.nqt == 1) ? 1 : 0;
    // One query tile and one head group per pair: each K/V byte goes to one workgroup.
    a.kv_nt = (group == hg && a.nqt == 1) ? 1 : 0;
    a.part_o = (float*)L.workspace;
    a.part_ml = a.part_o + (int64_t)L.total_q * L.num_q_heads * a.nchunk * L.head_dim;
    hipError_t err = launch(fn, a, hg, group, L.head_dim, stream);
    if (err != hipSuccess || a.nchunk == 1) return err;
    const int64_t mg = L.head_dim == 128 ? merge_grid<128>(L.total_q, L.num_q_heads)
                                         : merge_grid<64>(L.total_q, L.num_q_heads);
    if (mg > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (L.head_dim == 128)
        hipLaunchKernelGGL(extend_merge_kernel<128>, dim3((unsigned)mg), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(extend_merge_kernel<64>, dim3((unsigned)mg), dim3(256), 0, stream, a);
    return hipGetLastError();
}

size_t extend_workspace_bytes(int32_t batch, int32_t total_q, int32_t max_q_len, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len) {
    const int group = num_q_heads / num_kv_heads;
    PrefillFn fn;
    int hg;
    const bool pack = use_pack(group, max_q_len);
    if (!pick<true>(head_dim, group, &fn, &hg, false, pack)) return 0;
    PrefillArgs a = {};
    a.pack = pack ? 1 : 0;
    a.batch = batch;
    a.num_kv_heads = num_kv_heads;
    a.nchunk = 1;
    grid_dims(a, hg, group, max_q_len);
    int nc = 1, kc = kNoSplit;
    extend_split(grid_size(a, hg, group), max_context_len, 1 << 20, &nc, &kc);
    const size_t chunks = nc > 1 ? (size_t)total_q * num_q_heads * nc * (head_dim + 2) * 4 : 0;
    // (The window is not an argument here: the bound without one covers it.)
    const int nw = pack ? sk_shares((int64_t)batch * num_kv_heads, max_context_len, 0, max_q_len) : 0;
    return std::max(chunks, nw > 0 ? sk_workspace_bytes(nw, head_dim) : (size_t)0);
}

}  // namespace pgqa
