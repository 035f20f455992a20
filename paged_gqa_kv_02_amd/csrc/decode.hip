// decode.hip -- grouped-query attention decode over a paged KV cache.
//
// What it computes (one new query token per sequence, attending to every cached
// position of its sequence): for query head qh and its KV head h = qh / G,
//   out[b][qh] = softmax_j(scale * q[b][qh] . K_j) . V_j,  j in [0, ctx_b),
// with K_j / V_j found through the block table (paged KV cache: "Advanced
// Optimizations: MQA, GQA, and PagedAttention", "PagedAttention: The OS
// Analogy"; attention equation: "Modern LLM Inference", "Why Cross-Layer
// Attention Shares K/V but Not Q"; GQA grouping: same notes, section 4.1).
// The softmax is exact and computed online, FlashAttention-style; the split of
// long contexts across workgroups merged by a log-sum-exp reduce is the
// FlashDecoding idea named in the lecture notes, section 8.3, with the details
// chosen here.  Decode is bound by HBM reads of K/V (lecture notes, section 2).
//
// Design for gfx950:
//  * Work split ("stream-K"): the K/V of all (sequence, KV head) segments are
//    cut into tiles of TT tokens; the tiles are laid end to end and every
//    workgroup takes an equal contiguous share.  Ragged context lengths
//    therefore balance across the 256 CUs.  A share that covers a whole
//    segment writes the output; a segment cut across shares writes fp32
//    partials (running max m, sum l, unnormalised o) merged by decode_merge.
//    (Merging inside the split kernel by the last-arriving share needs
//    device-scope release fences, which write back every XCD's L2 and cost far
//    more than the second launch.)
//  * Streaming: a tile is DRPT 1 KB rows of K plus DRPT rows of V, moved with
//    16-byte-per-lane global->LDS DMA (global_load_lds_dwordx4) into a ring of
//    kStages tiles, so loads for later tiles are in flight while the current
//    one is computed and no VGPRs are tied up by the prefetch.
//  * Lane mapping: LPT = d*elem/16 lanes cover one token row (16 lanes for
//    bf16 d = 128), so one wave row holds TPR = 64/LPT tokens.  Each lane keeps
//    its 16-byte slice of the G query rows in registers; every K row is read
//    once from LDS and used for all G query heads of the group.
//  * Scores: v_dot2_f32_bf16 partial dot products, then a reduce-scatter
//    butterfly of DPP exchanges over the LPT lanes of the row: each exchange
//    both adds and halves the heads a lane keeps, so a lane ends with the full
//    score of one head (5 DPP adds instead of 16 for 4 heads, and one exp per
//    lane instead of 4).  Each lane holds its query heads in a lane-dependent
//    register order, so every exchange is a plain add (no per-lane select).
//    The weights are then broadcast back across the row (DPP row_newbcast)
//    for the P.V accumulation in fp32.
//  * Online softmax in log2 units with the scale folded into the exponent,
//    p = exp2(s * scale*log2e - m) (a negative or zero scale is applied as the
//    sign of the query bits, so the folded factor is always positive), each
//    weight rounded to bf16 once and the same rounded weight added to the sum
//    and used in P.V (bf16 pages), and a lazy rescale: o and l are rescaled
//    only when a running max grows by more than 8, which keeps every weight
//    <= 256 and is exact because the final o / l uses the same reference max.
//  * Masking selects (never multiplies) and only on the ragged last tile of a
//    sequence (and, under a local-attention window, its first tile): scores
//    outside [lo, ctx) become -inf and those V rows are zeroed, so NaN in
//    unused slots (or in pages dropped before the window) cannot leak.
//  * Low-precision pages (FP8 E4M3 codes, one fp32 scale per token and KV head
//    row): the same kernel with KES = 1.  A tile moves the 8 KB of a bf16
//    tile's K and V as codes (twice the tokens), plus the tile's row scales by
//    4-byte-per-lane DMA.  A lane converts its 8 K codes of a row to bf16 right
//    before the dot products (one instruction per pair, exact); for P.V it
//    interleaves the bytes of two token rows first, so each conversion yields
//    the two rows' values of one dim, the pair v_dot2 takes.  Scores and P.V are
//    the bf16 path's; the K scale multiplies a token's score and the V scale
//    its weight.
//  * Large groups (G >= 16) use G/8 waves per workgroup sharing one ring; each
//    wave owns 8 query heads.
#include "device_common.hpp"
#include "launch.hpp"

#include <math.h>

#include <algorithm>
#include <mutex>

#ifndef PGQA_DECODE_STAGES
#define PGQA_DECODE_STAGES 2
#endif
#ifndef PGQA_DECODE_RPT
#define PGQA_DECODE_RPT 4
#endif
#ifndef PGQA_MQA_PACK
#define PGQA_MQA_PACK 1
#endif
#ifndef PGQA_MQA_CHUNK
#define PGQA_MQA_CHUNK 20  // 64-key blocks per key chunk on the matrix-core MQA route
#endif
#ifndef PGQA_DECODE_RPT8
#define PGQA_DECODE_RPT8 8
#endif
#ifndef PGQA_DECODE_LDS_DIV
#define PGQA_DECODE_LDS_DIV 4   // one-wave workgroups per CU on bf16 / fp32 pages (one per SIMD)
#endif
#ifndef PGQA_DECODE_LDS_DIV8
#define PGQA_DECODE_LDS_DIV8 8  // one-wave workgroups per CU on FP8 pages (two per SIMD)
#endif

namespace pgqa {

namespace {

struct DecodeArgs {
    const char* q;
    const char* k_cache;
    const char* v_cache;
    const int32_t* block_table;
    const int32_t* context_lens;
    char* out;
    float* part_o;       // [slots][G][D]   slots = num_splits + batch * Hkv
    float* part_ml;      // [slots][G][2]   (m, l) in log2 units
    int32_t* tile_pref;  // [batch + 1] tiles of the sequences before b (written by the split kernel's first share)
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t max_blocks_per_seq;
    int32_t num_blocks;
    int32_t bs_log2;
    int32_t ctx_cap;     // max_context_len: device context lengths are clamped to it
    int32_t num_splits;  // requested shares == gridDim.x of the split kernel
    float scale_log2;    // |scale| * log2(e): scores live in log2 units, weights use exp2
    u32 q_and;           // the scale's sign, applied to the query bits as they are loaded
    u32 q_xor;
    int32_t window;      // > 0: only the newest `window` positions are attended to
    const float* k_scale;   // FP8 pages: row scales [num_blocks, Hkv, block_size]
    const float* v_scale;
    int32_t seg_mode;       // 1: one workgroup per (sequence, KV head) segment, whole (no partials, no merge)
};

constexpr int kStages = PGQA_DECODE_STAGES;   // ring depth (tiles) of the split kernel
constexpr int kSegModeTiles = 2;              // segments this short take one workgroup each, no merge
constexpr int kRows = PGQA_DECODE_RPT;        // 1 KB wave rows per tile, for K and for V
constexpr int kRows8 = PGQA_DECODE_RPT8;      // compute rows per tile over FP8 pages
static_assert(kStages >= 2 && kStages <= 6, "ring depth");
static_assert(kRows == 1 || kRows == 2 || kRows == 4 || kRows == 8 || kRows == 16, "rows per tile");

// Tile geometry.  ES = bytes of a q / compute element (4 fp32, 2 bf16); KES =
// bytes of a cached K/V element (= ES, or 1 for FP8 pages, whose codes are
// converted to bf16 right after the LDS read, so the compute side is the bf16
// one).  A compute row is 64 lanes x 16 bytes of compute elements: TPR tokens,
// LPT lanes per token.  K/V move in 1 KB DMA rows of TPRD tokens; an FP8 tile
// has twice the compute rows of a bf16 one so that it moves the same bytes.
template <int ES, int D, int KES = ES>
struct Geo {
    static constexpr int EPL = 16 / ES;            // compute elements per lane
    static constexpr int LPT = D / EPL;            // lanes per token
    static constexpr int TPR = kWave / LPT;        // tokens per compute row
    static constexpr int RPT = KES == ES ? kRows : kRows8;   // compute rows per tile
    static constexpr int TT = RPT * TPR;           // tokens per tile
    static constexpr int ROWB = 1024;              // bytes per DMA row
    static constexpr int CROWB = TPR * D * KES;    // LDS bytes of one compute row (per pool)
    static constexpr int LB = CROWB / kWave;       // LDS bytes a lane reads per compute row
    static constexpr int TPRD = ROWB / (D * KES);  // tokens per DMA row
    static constexpr int LPTD = kWave / TPRD;      // lanes per token in a DMA row
    static constexpr int DRPT = RPT * CROWB / ROWB;   // DMA rows per tile, per pool
    static constexpr int KVB = DRPT * ROWB;        // bytes of K (or V) per tile
    static constexpr int NSL = KES == ES ? 0 : 2 * TT / kWave;   // 4-byte-per-lane loads of K then V row scales
    static constexpr int NL = 2 * DRPT + NSL;      // loads per tile
    static constexpr int TILEB = 2 * KVB + NSL * kWave * 4;
    static_assert(LPT >= 2 && LPT <= 32 && TPR * LPT == kWave, "unsupported head_dim / dtype");
    static_assert(DRPT * ROWB == RPT * CROWB && TPRD * LPTD == kWave, "unsupported head_dim / KV dtype");
    static_assert(KES == ES || NSL * kWave == 2 * TT, "scale loads cover K and V scales of the tile");
};

constexpr int ilog2c(int x) { return x <= 1 ? 0 : 1 + ilog2c(x / 2); }

// Reduce-scatter of GW per-lane partial dot products over the LPT lanes of a
// token row.  Split step s (partner distance LPT >> (s+1)) halves the values a
// lane keeps; after NSPLIT steps each lane holds VPL full sums, for heads
// head_off(lane) .. +VPL, and the remaining steps only add.  So that every step
// is one add with no per-lane select, register slot j of a lane holds head
// j ^ head_off(lane) (the query slices are loaded in that order): each step then
// keeps the lower half of the live slots and sends the upper half, and the
// partner's upper half holds the same heads as this lane's lower half.  Bit s
// of head_off (value GW >> (s+1)) is the lane's distance bit of step s; the
// distance-4 exchange (row_half_mirror) pairs lane l with l ^ 7, so when it
// splits, the bits of the later split steps are taken relative to bit 2, which
// that partner flips with them.
template <int LPT, int GW>
struct Scatter {
    static constexpr int NSPLIT = ilog2c(GW) < ilog2c(LPT) ? ilog2c(GW) : ilog2c(LPT);
    static constexpr int VPL = GW >> NSPLIT;
    static constexpr bool MIRROR = LPT >= 8 && ilog2c(LPT) - 3 < NSPLIT;   // the distance-4 step splits

    __device__ static int head_off(int lane) {
        int off = 0;
#pragma unroll
        for (int s = 0; s < NSPLIT; ++s) {
            const int d = LPT >> (s + 1);
            int bit = (lane & d) != 0;
            if (MIRROR && d < 4) bit ^= (lane >> 2) & 1;
            if (bit) off += GW >> (s + 1);
        }
        return off;
    }
    // Lane (within the token group) that holds head g, and which of its values.
    static constexpr int owner(int g) {
        int lane = 0;
        for (int s = 0; s < NSPLIT; ++s) {
            const int d = LPT >> (s + 1);
            int bit = (g & (GW >> (s + 1))) != 0;
            if (MIRROR && d < 4) bit ^= (lane >> 2) & 1;
            if (bit) lane |= d;
        }
        return lane;
    }
    static constexpr int slot(int g) { return g & (VPL - 1); }
};

// Exchange with a partner at distance DLT inside an aligned group of 2*DLT lanes
// (the partner has bit DLT flipped; row_half_mirror also flips the bits below,
// which the later steps sum over).
template <int DLT>
__device__ __forceinline__ float xchg(float x) {
    if constexpr (DLT == 16) return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
    else if constexpr (DLT == 8) return dpp_f32<0x128>(x);   // row_ror:8 == lane ^ 8 within 16
    else if constexpr (DLT == 4) return dpp_f32<0x141>(x);   // row_half_mirror
    else if constexpr (DLT == 2) return dpp_f32<0x4E>(x);    // quad_perm [2,3,0,1]
    else return dpp_f32<0xB1>(x);                              // quad_perm [1,0,3,2]
}

// v holds the GW values in the lane's head order (slot j = head j ^ head_off).
template <int DLT, int N>
__device__ __forceinline__ void scatter_steps(float* v) {
    if constexpr (DLT >= 1) {
        if constexpr (N > 1) {
#pragma unroll
            for (int k = 0; k < N / 2; ++k) v[k] += xchg<DLT>(v[N / 2 + k]);
            scatter_steps<DLT / 2, N / 2>(v);
        } else {
            v[0] += xchg<DLT>(v[0]);
            scatter_steps<DLT / 2, 1>(v);
        }
    }
}

// Value of lane OWNER of this lane's token group, broadcast to the whole group.
template <int LPT, int OWNER>
__device__ __forceinline__ float group_bcast(float x, int lane) {
    // Every lane reads a valid source lane, so the DPP move needs no old value
    // (update_dpp with a zero old value costs a v_mov of zero per broadcast).
    if constexpr (LPT == 16) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + OWNER, 0xF, 0xF, false));
    } else if constexpr (LPT == 4) {
        constexpr int ctrl = OWNER | (OWNER << 2) | (OWNER << 4) | (OWNER << 6);
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xF, 0xF, false));
    } else if constexpr (LPT == 2) {
        constexpr int ctrl = OWNER | (OWNER << 2) | ((2 + OWNER) << 4) | ((2 + OWNER) << 6);
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xF, 0xF, false));
    } else {
        const int src = (lane & ~(LPT - 1)) | OWNER;
        return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
    }
}

// A sequence's segment covers positions [lo, ctx) with lo = ctx - window under
// local attention ("Modern LLM Inference", section 4.4: a token attends only to
// the most recent positions) and lo = 0 otherwise; its tiles are the TT-token
// tiles from the one holding lo to the one holding ctx - 1, so pages wholly
// before the window are never read.
__device__ __forceinline__ int window_lo(int ctx, int window) { return (window > 0 && ctx > window) ? ctx - window : 0; }

__device__ __forceinline__ int tiles_of(int ctx, int cap, int tt, int window) {
    ctx = clampi(ctx, 0, cap);
    return ctx > 0 ? (ctx + tt - 1) / tt - window_lo(ctx, window) / tt : 0;
}

// a.b over one bf16 pair with no accumulator.  Written as the three-operand
// v_dot2_f32_bf16 with an inline zero: the builtin with a 0.0f accumulator is
// emitted as a v_mov of zero plus the tied-accumulator v_dot2c form, one extra
// VALU instruction per dot product.  Plain register arithmetic, no memory access.
__device__ __forceinline__ float dot2_bf16_first(u32 a, u32 b) {
    float r;
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// q . k for one lane's 16-byte slices (fp32 accumulation).
template <int ES>
__device__ __forceinline__ float slice_dot(const u32x4& q, const u32x4& k) {
    if constexpr (ES == 2) {
        float acc = dot2_bf16_first(q.x, k.x);
        acc = dot2_bf16(q.y, k.y, acc);
        acc = dot2_bf16(q.z, k.z, acc);
        return dot2_bf16(q.w, k.w, acc);
    } else {
        float acc = __uint_as_float(q.x) * __uint_as_float(k.x);
        acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
        acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
        return fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
    }
}

template <int ES>
__device__ __forceinline__ void unpack16(const u32x4& x, float* f) {
    if constexpr (ES == 2) {
        f[0] = bf16_lo(x.x); f[1] = bf16_hi(x.x);
        f[2] = bf16_lo(x.y); f[3] = bf16_hi(x.y);
        f[4] = bf16_lo(x.z); f[5] = bf16_hi(x.z);
        f[6] = bf16_lo(x.w); f[7] = bf16_hi(x.w);
    } else {
        f[0] = __uint_as_float(x.x); f[1] = __uint_as_float(x.y);
        f[2] = __uint_as_float(x.z); f[3] = __uint_as_float(x.w);
    }
}

template <int ES>
__device__ __forceinline__ void store_out16(char* dst, const float* f, float inv) {
    if constexpr (ES == 2) {
        u32x4 w;
        w.x = pack_bf16x2(f[0] * inv, f[1] * inv);
        w.y = pack_bf16x2(f[2] * inv, f[3] * inv);
        w.z = pack_bf16x2(f[4] * inv, f[5] * inv);
        w.w = pack_bf16x2(f[6] * inv, f[7] * inv);
        *(u32x4*)dst = w;
    } else {
        f32x4 w = {f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv};
        *(f32x4*)dst = w;
    }
}

// The block-table entries of the pages a piece streams, one per lane: lane k
// holds the block of page base + k.  A tile's block ids are then read with
// v_readlane (no memory access on the issue path); the window moves forward
// (one vector load) when a page is 64 or more past its base.  Entries are
// clamped to the sequence's last page and to the pool, so every read is in range.
struct PageWin {
    const int32_t* bt_row;
    int last_page;
    int num_blocks;
    int base;
    int reg;

    __device__ __forceinline__ void load(int first, int lane) {
        base = first;
        reg = clampi(bt_row[min(first + lane, last_page)], 0, num_blocks - 1);
    }
    __device__ __forceinline__ int get(int page, int lane) {
        if (page - base >= kWave) load(page, lane);
        return __builtin_amdgcn_readlane(reg, page - base);
    }
    // Make pages first .. last (last - first < 64) readable by every lane.
    __device__ __forceinline__ void cover(int first, int last, int lane) {
        if (first < base || last - base >= kWave) load(first, lane);
    }
};

// Issue the global->LDS loads of one tile (DMA rows of K, then of V, then for
// FP8 pages the row scales of K and of V) into ring slot `slot`.  Wave `wave`
// issues the loads li with li % W == wave (the wait counts rely on the per-wave
// count being fixed).
template <int ES, int D, int W, int KES>
__device__ __forceinline__ void issue_tile(const DecodeArgs& a, PGQA_LDS char* ring, int slot, int tile,
                                           int h, int ctx, PageWin& win, int wave, int lane) {
    using Gm = Geo<ES, D, KES>;
    constexpr int DRPT = Gm::DRPT, TPRD = Gm::TPRD;
    const int tg = lane / Gm::LPTD;
    const int bs_mask = (1 << a.bs_log2) - 1;
    const int tile_tok = tile * Gm::TT;
    PGQA_LDS char* dst = ring + slot * Gm::TILEB;
    if constexpr (Gm::NSL > 0) {
        // Every block id the scale loads need must sit in the window (at most
        // TT / block_size + 1 pages; FP8 pages are at least 16 tokens).
        win.cover(tile_tok >> a.bs_log2, min(tile_tok + Gm::TT - 1, ctx - 1) >> a.bs_log2, lane);
    }
    if (TPRD <= (1 << a.bs_log2)) {
        // Every 1 KB row (TPRD tokens) lies in one page, so row r is one
        // contiguous run of that page.  Row starts are clamped to the last row
        // holding a context token (TPRD-aligned): rows past the context re-read
        // that row (in bounds) and are masked in compute.
        const int last_row_tok = (ctx - 1) & ~(TPRD - 1);
        int64_t run[DRPT];
        if (Gm::TT <= (1 << a.bs_log2)) {
            // The whole tile is in one page (it starts before the context end).
            const int bid = win.get(tile_tok >> a.bs_log2, lane);
            const int64_t base = ((((int64_t)bid * a.num_kv_heads + h) << a.bs_log2) + (tile_tok & bs_mask)) * (D * KES);
#pragma unroll
            for (int r = 0; r < DRPT; ++r) run[r] = base + r * Gm::ROWB + lane * 16;
        } else {
#pragma unroll
            for (int r = 0; r < DRPT; ++r) {
                const int tok = min(tile_tok + r * TPRD, last_row_tok);
                const int bid = win.get(tok >> a.bs_log2, lane);
                run[r] = ((((int64_t)bid * a.num_kv_heads + h) << a.bs_log2) + (tok & bs_mask)) * (D * KES) + lane * 16;
            }
        }
#pragma unroll
        for (int li = 0; li < 2 * DRPT; ++li) {
            if (li % W != wave) continue;
            const int r = li % DRPT;
            const bool isv = li >= DRPT;
            load_lds_16((isv ? a.v_cache : a.k_cache) + run[r], dst + li * Gm::ROWB);
        }
    } else {
        // Pages smaller than a row: each lane looks up its own token's page
        // (positions clamped to the context so every table read is in range).
        const int c = lane % Gm::LPTD;
        int blk[DRPT];
        int tok[DRPT];
#pragma unroll
        for (int r = 0; r < DRPT; ++r) {
            tok[r] = min(tile_tok + r * TPRD + tg, ctx - 1);
            blk[r] = clampi(win.bt_row[tok[r] >> a.bs_log2], 0, a.num_blocks - 1);
        }
#pragma unroll
        for (int li = 0; li < 2 * DRPT; ++li) {
            if (li % W != wave) continue;
            const int r = li % DRPT;
            const bool isv = li >= DRPT;
            const int64_t prow = (((int64_t)blk[r] * a.num_kv_heads + h) << a.bs_log2) + (tok[r] & bs_mask);
            const char* src = (isv ? a.v_cache : a.k_cache) + prow * (D * KES) + c * 16;
            load_lds_16(src, dst + li * Gm::ROWB);
        }
    }
    if constexpr (Gm::NSL > 0) {
        // Row scales, 4 bytes per lane, K scales then V scales: entry p = 64 j + l
        // of load j is pool p / TT, position q = p % TT, the scale of the token
        // that compute lane group g = q / RPT meets in compute row r = q % RPT,
        // so each group's RPT scales are contiguous in LDS.  Tokens past the
        // context re-read the last one (masked).
        constexpr int RPT = Gm::RPT, TT = Gm::TT;
#pragma unroll
        for (int j = 0; j < Gm::NSL; ++j) {
            const int li = 2 * DRPT + j;
            if (li % W != wave) continue;
            const int p = j * kWave + lane;
            const int qq = p % TT;
            const int tok = min(tile_tok + (qq % RPT) * Gm::TPR + qq / RPT, ctx - 1);
            const int blk = __builtin_amdgcn_ds_bpermute(((tok >> a.bs_log2) - win.base) << 2, win.reg);
            const int64_t srow = (((int64_t)blk * a.num_kv_heads + h) << a.bs_log2) + (tok & bs_mask);
            __builtin_amdgcn_global_load_lds((p >= TT ? a.v_scale : a.k_scale) + srow,
                                             dst + 2 * Gm::KVB + j * kWave * 4, 4, 0, PGQA_KV_CPOL);
        }
    }
}

template <int LPT, int OWNER>
__device__ __forceinline__ u32 group_bcast_u32(u32 x, int lane) {
    return __float_as_uint(group_bcast<LPT, OWNER>(__uint_as_float(x), lane));
}

template <int LPT, int GW, int G0 = 0>
__device__ __forceinline__ void bcast_heads_u32(const u32* vals, u32* out, int lane) {
    if constexpr (G0 < GW) {
        using S = Scatter<LPT, GW>;
        out[G0] = group_bcast_u32<LPT, S::owner(G0)>(vals[S::slot(G0)], lane);
        bcast_heads_u32<LPT, GW, G0 + 1>(vals, out, lane);
    }
}

// Broadcast each head's owned value (vals[slot(g)] at lane owner(g)) to every
// lane of the token group: out[g] for g < GW.
template <int LPT, int GW, int G0 = 0>
__device__ __forceinline__ void bcast_heads(const float* vals, float* out, int lane) {
    if constexpr (G0 < GW) {
        using S = Scatter<LPT, GW>;
        out[G0] = group_bcast<LPT, S::owner(G0)>(vals[S::slot(G0)], lane);
        bcast_heads<LPT, GW, G0 + 1>(vals, out, lane);
    }
}

// This lane's slice of compute row r of a K or V tile (bf16 / fp32 as stored,
// or FP8 codes converted to bf16).
template <int ES, int D, int KES>
__device__ __forceinline__ u32x4 kv_slice(const PGQA_LDS char* base, int r) {
    using Gm = Geo<ES, D, KES>;
    if constexpr (KES == ES) return lds_read_16(base + r * Gm::CROWB);
    else return fp8x8_to_bf16(lds_read_8(base + r * Gm::CROWB));
}

// One tile: scores, online-softmax update and P.V for this wave's GW heads.
// FULL: every token of the tile is inside [lo, ctx) (no masking needed).
// PF: all K and V slices of the tile are read from LDS up front, so their
// latency is paid once per tile instead of once per row pair (off where the
// extra registers would spill: 8-wave groups and head_dim 16).
// tb is the tile's ring slot.  FP8 pages: the row scale of K multiplies the
// token's score, that of V its weight in P.V (the softmax sum keeps the plain
// weight), so the codes are used as they are.
template <bool FULL, int ES, int D, int GW, int KES, bool PF>
__device__ __forceinline__ void tile_compute(const PGQA_LDS char* tb, const u32x4* qv, float* m, float* l,
                                             float (*o)[16 / ES], int tok0, int ctx, int lo, float c, int lane) {
    using Gm = Geo<ES, D, KES>;
    using S = Scatter<Gm::LPT, GW>;
    constexpr int EPL = Gm::EPL, RPT = Gm::RPT, TPR = Gm::TPR, VPL = S::VPL;
    constexpr bool Q8 = KES != ES;
    const PGQA_LDS char* kb = tb + lane * Gm::LB;
    const PGQA_LDS char* vb = kb + Gm::KVB;
    // Row scales of this lane's tokens (FP8): group g's RPT scales are contiguous.
    const PGQA_LDS float* ksc = (const PGQA_LDS float*)(tb + 2 * Gm::KVB) + (lane / Gm::LPT) * RPT;
    const PGQA_LDS float* vsc = ksc + Gm::TT;

    // FP8 pages prefetch the raw codes (8 bytes a row): K rows are converted
    // right before their dot products, V rows pairwise inside P.V.
    u32x4 kxs[PF && !Q8 ? RPT : 1], vxs[PF && !Q8 ? RPT : 1];
    u32x2 kcs[PF && Q8 ? RPT : 1], vcs[PF && Q8 ? RPT : 1];
    if constexpr (PF) {
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            if constexpr (Q8) kcs[r] = lds_read_8(kb + r * Gm::CROWB);
            else kxs[r] = kv_slice<ES, D, KES>(kb, r);
        }
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            if constexpr (Q8) vcs[r] = lds_read_8(vb + r * Gm::CROWB);
            else vxs[r] = kv_slice<ES, D, KES>(vb, r);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the arithmetic
    }
    float s[RPT][VPL];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        u32x4 kx;
        if constexpr (PF && Q8) kx = fp8x8_to_bf16(kcs[r]);
        else kx = PF ? kxs[PF ? r : 0] : kv_slice<ES, D, KES>(kb, r);
        float v[GW];
#pragma unroll
        for (int g = 0; g < GW; ++g) v[g] = slice_dot<ES>(qv[g], kx);
        scatter_steps<Gm::LPT / 2, GW>(v);
        const bool valid = FULL || (tok0 + r * TPR < ctx && tok0 + r * TPR >= lo);
        if constexpr (Q8) {
            const float ks = ksc[r];
#pragma unroll
            for (int k = 0; k < VPL; ++k) v[k] *= ks;
        }
#pragma unroll
        for (int k = 0; k < VPL; ++k) s[r][k] = valid ? v[k] : -INFINITY;
    }
    bool need = false;
    float mt[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        float x = s[0][k];
#pragma unroll
        for (int r = 1; r < RPT; ++r) x = fmaxf(x, s[r][k]);
        mt[k] = x * c;
        need |= mt[k] > m[k] + 8.0f;
    }
    if (__builtin_expect(__any(need), 0)) {
        float alpha[VPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            alpha[k] = 1.0f;
            if (mt[k] > m[k] + 8.0f) {
                alpha[k] = __builtin_amdgcn_exp2f(m[k] - mt[k]);
                m[k] = mt[k];
                l[k] *= alpha[k];
            }
        }
        float ag[GW];
        bcast_heads<Gm::LPT, GW>(alpha, ag, lane);
#pragma unroll
        for (int g = 0; g < GW; ++g)
#pragma unroll
            for (int x = 0; x < EPL; ++x) o[g][x] *= ag[g];
    }
    if constexpr (ES == 2) {
        // P.V on v_dot2_f32_bf16 over pairs of token rows (r, r+1): the two rows'
        // values of one dim are packed into one register (v_perm_b32), each
        // owned weight pair is rounded to bf16 once (v_cvt_pk_bf16_f32) and
        // broadcast as one packed word per head; accumulation stays in fp32.
        static_assert(RPT % 2 == 0, "bf16 P.V pairs token rows");
#pragma unroll
        for (int r = 0; r < RPT; r += 2) {
            const bool ok0 = FULL || (tok0 + r * TPR < ctx && tok0 + r * TPR >= lo);
            const bool ok1 = FULL || (tok0 + (r + 1) * TPR < ctx && tok0 + (r + 1) * TPR >= lo);
            float vs0 = 1.0f, vs1 = 1.0f;
            if constexpr (Q8) {
                vs0 = ok0 ? vsc[r] : 0.0f;
                vs1 = ok1 ? vsc[r + 1] : 0.0f;
            }
            u32 pk[VPL];
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s[r][k], c, -m[k]));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s[r + 1][k], c, -m[k]));
                if constexpr (Q8) {
                    l[k] += p0 + p1;
                    pk[k] = pack_bf16x2_rne_hw(p0 * vs0, p1 * vs1);
                } else {
                    // The sum adds the bf16-rounded weights, exactly the ones P.V uses.
                    pk[k] = pack_bf16x2_rne_hw(p0, p1);
                    l[k] = dot2_bf16(pk[k], 0x3F803F80u, l[k]);
                }
            }
            u32 pg[GW];
            bcast_heads_u32<Gm::LPT, GW>(pk, pg, lane);
            u32 vp[EPL];
            if constexpr (Q8) {
                // Codes of rows r and r+1 (8 dims each): interleave the bytes of
                // the two rows, then each conversion of a byte pair yields the
                // (row r, row r+1) bf16 pair of one dim.  A zero code is +0.
                u32x2 c0 = PF ? vcs[PF ? r : 0] : lds_read_8(vb + r * Gm::CROWB);
                u32x2 c1 = PF ? vcs[PF ? r + 1 : 0] : lds_read_8(vb + (r + 1) * Gm::CROWB);
                if (!FULL) {
                    if (!ok0) c0 = u32x2{0, 0};
                    if (!ok1) c1 = u32x2{0, 0};
                }
                const u32 a[2] = {c0.x, c0.y};
                const u32 b[2] = {c1.x, c1.y};
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const u32 lo = __builtin_amdgcn_perm(b[i], a[i], 0x05010400u);   // dims 4i, 4i+1
                    const u32 hi = __builtin_amdgcn_perm(b[i], a[i], 0x07030602u);   // dims 4i+2, 4i+3
                    vp[4 * i] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
                    vp[4 * i + 1] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
                    vp[4 * i + 2] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
                    vp[4 * i + 3] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
                }
            } else {
                u32x4 v0 = PF ? vxs[PF ? r : 0] : kv_slice<ES, D, KES>(vb, r);
                u32x4 v1 = PF ? vxs[PF ? r + 1 : 0] : kv_slice<ES, D, KES>(vb, r + 1);
                if (!FULL) {
                    if (!ok0) v0 = u32x4{0, 0, 0, 0};
                    if (!ok1) v1 = u32x4{0, 0, 0, 0};
                }
                const u32 w0[4] = {v0.x, v0.y, v0.z, v0.w};
                const u32 w1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    vp[2 * i] = __builtin_amdgcn_perm(w1[i], w0[i], 0x05040100u);      // (row r, row r+1) of dim 2i
                    vp[2 * i + 1] = __builtin_amdgcn_perm(w1[i], w0[i], 0x07060302u);  // ... of dim 2i+1
                }
            }
#pragma unroll
            for (int g = 0; g < GW; ++g)
#pragma unroll
                for (int x = 0; x < EPL; ++x) o[g][x] = dot2_bf16(pg[g], vp[x], o[g][x]);
        }
    } else {
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            float p[VPL];
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                p[k] = __builtin_amdgcn_exp2f(fmaf(s[r][k], c, -m[k]));
                l[k] += p[k];
            }
            float pg[GW];
            bcast_heads<Gm::LPT, GW>(p, pg, lane);
            const u32x4 vx = PF ? vxs[PF ? r : 0] : kv_slice<ES, D, KES>(vb, r);
            float vf[EPL];
            unpack16<ES>(vx, vf);
            if (!FULL && (tok0 + r * TPR >= ctx || tok0 + r * TPR < lo)) {
#pragma unroll
                for (int x = 0; x < EPL; ++x) vf[x] = 0.0f;
            }
#pragma unroll
            for (int g = 0; g < GW; ++g)
#pragma unroll
                for (int x = 0; x < EPL; ++x) o[g][x] = fmaf(pg[g], vf[x], o[g][x]);
        }
    }
}

// Share (workgroup) of the split kernel that holds global tile X, with
// share w covering tiles [w*total/nw, (w+1)*total/nw).
__device__ __forceinline__ int64_t share_of(int64_t X, int64_t total, int64_t nw) {
    return ((X + 1) * nw - 1) / total;
}

template <int ES, int D, int GW, int W, int KES>
__global__ __launch_bounds__(64 * W) void decode_split_kernel(DecodeArgs a) {
    using Gm = Geo<ES, D, KES>;
    using S = Scatter<Gm::LPT, GW>;
    constexpr int EPL = Gm::EPL, LPT = Gm::LPT, TT = Gm::TT, VPL = S::VPL;
    constexpr int G = GW * W;
    constexpr bool kPF = W <= 4 && D >= 32;   // read a tile's K/V slices up front
    // Loads per tile: NL, wave w issues loads li with li % W == w.
    constexpr int LPW_MAX = (Gm::NL + W - 1) / W;

    extern __shared__ __attribute__((aligned(16))) char smem[];
    PGQA_LDS char* ring = (PGQA_LDS char*)smem;
    int* pref = (int*)(smem + kStages * Gm::TILEB);   // [batch + 1] tile prefix sums

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int B = a.batch;
    const int Hkv = a.num_kv_heads;

    // ---- tiles per sequence, prefix-summed in LDS ------------------------
    if (wave == 0) {
        int carry = 0;
        for (int base = 0; base < B; base += 64) {
            const int b = base + lane;
            int x = b < B ? tiles_of(a.context_lens[b], a.ctx_cap, TT, a.window) : 0;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(x, off);
                if (lane >= off) x += y;
            }
            if (b < B) pref[b + 1] = carry + x;
            carry += __shfl(x, 63);
        }
        if (lane == 0) pref[0] = 0;
    }
    __syncthreads();
    // The merge kernel reads the same prefix sums (no rescan of every context there).
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i <= B; i += 64 * W) a.tile_pref[i] = pref[i];

    // Shares: min(num_splits, total) so that no share is empty and every share
    // of a cut segment writes the partial the merge reads.
    const int64_t total = (int64_t)Hkv * pref[B];
    const int64_t NW = min((int64_t)a.num_splits, total);
    const int64_t w = blockIdx.x;
    // Sequences with no context get zeros (no share visits them).
    for (int bb = blockIdx.x; bb < B; bb += gridDim.x) {
        if (pref[bb + 1] != pref[bb]) continue;
        for (int e = threadIdx.x; e < a.num_q_heads * D; e += 64 * W) {
            char* dst = a.out + ((int64_t)bb * a.num_q_heads * D + e) * ES;
            if constexpr (ES == 2) *(uint16_t*)dst = 0;
            else *(float*)dst = 0.0f;
        }
    }
    int64_t X, X1;
    int b, h, t0, tiles_b;
    if (a.seg_mode) {
        // One workgroup per segment: workgroup w runs all tiles of segment
        // (w / Hkv, w % Hkv) as one whole piece (empty ones are zero-filled above).
        b = blockIdx.x / Hkv;
        h = blockIdx.x % Hkv;
        if (b >= B) return;
        tiles_b = pref[b + 1] - pref[b];
        if (tiles_b == 0) return;
        t0 = 0;
        X = (int64_t)Hkv * pref[b] + (int64_t)h * tiles_b;
        X1 = X + tiles_b;
    } else {
        if (w >= NW) return;
        X = w * total / NW;
        X1 = (w + 1) * total / NW;
        // Segment (b, h) and tile t of the first tile of this share.
        {
            int lo = 0, hi = B - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if ((int64_t)Hkv * pref[mid] <= X) lo = mid;
                else hi = mid - 1;
            }
            b = lo;
        }
        tiles_b = pref[b + 1] - pref[b];
        const int64_t rem = X - (int64_t)Hkv * pref[b];
        h = (int)(rem / tiles_b);
        t0 = (int)(rem % tiles_b);
    }

    const int c = lane % LPT;
    const int tg = lane / LPT;
    const float cs = a.scale_log2;
    const int lpw = wave < Gm::NL ? (Gm::NL - wave + W - 1) / W : 0;   // this wave's loads per tile

    while (X < X1) {
        const int n = (int)min((int64_t)(tiles_b - t0), X1 - X);   // tiles in this piece
        const bool whole = (t0 == 0) && (n == tiles_b);
        const int ctx = clampi(a.context_lens[b], 0, a.ctx_cap);
        const int lo = window_lo(ctx, a.window);
        const int tf = lo / TT + t0;   // sequence tile index of the piece's first tile
        const int qh0 = h * G + wave * GW;
        PageWin win;
        win.bt_row = a.block_table + (int64_t)b * a.max_blocks_per_seq;
        win.last_page = (ctx - 1) >> a.bs_log2;
        win.num_blocks = a.num_blocks;
        if (Gm::TPRD <= (1 << a.bs_log2)) win.load((tf * TT) >> a.bs_log2, lane);

        // This wave's query slices: GW heads x 16 bytes, slot g holding head
        // g ^ head_off (the reduce-scatter's order).
        u32x4 qv[GW];
        const int hoff = S::head_off(lane);
#pragma unroll
        for (int g = 0; g < GW; ++g)
            qv[g] = (*(const u32x4*)(a.q + ((int64_t)(b * a.num_q_heads + qh0 + (g ^ hoff)) * D + c * EPL) * ES) &
                     a.q_and) ^ a.q_xor;

        // Running max / sum of the heads this lane owns; o for all GW heads.
        float m[VPL], l[VPL], o[GW][EPL];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            m[k] = kMaxInit;
            l[k] = 0.0f;
        }
#pragma unroll
        for (int g = 0; g < GW; ++g)
#pragma unroll
            for (int x = 0; x < EPL; ++x) o[g][x] = 0.0f;

        // Prologue: fill the first kStages-1 ring slots.
#pragma unroll
        for (int i = 0; i < kStages - 1; ++i)
            if (i < n) issue_tile<ES, D, W, KES>(a, ring, i, tf + i, h, ctx, win, wave, lane);

        // Tiles of the piece: every tile but a segment's first (under a window)
        // and last is full, so the loop body is one path and those two are
        // peeled off with the masked path if they need it.
        auto step = [&](int it) {
            const int slot = it % kStages;
            // This wave's loads issued after this tile's: at most kStages-2 tiles of lpw each.
            wait_vmcnt_dyn<(kStages - 2) * LPW_MAX>(lpw * min(kStages - 2, n - 1 - it));
            if constexpr (W > 1) __syncthreads();
            if (it + kStages - 1 < n)
                issue_tile<ES, D, W, KES>(a, ring, (it + kStages - 1) % kStages, tf + it + kStages - 1, h, ctx,
                                          win, wave, lane);
            return ring + slot * Gm::TILEB;
        };
        int it0 = 0;
        if (n > 1 && tf * TT < lo) {
            const PGQA_LDS char* kb = step(0);
            tile_compute<false, ES, D, GW, KES, kPF>(kb, qv, m, l, o, tf * TT + tg, ctx, lo, cs, lane);
            it0 = 1;
        }
        for (int it = it0; it < n - 1; ++it) {
            const PGQA_LDS char* kb = step(it);
            tile_compute<true, ES, D, GW, KES, kPF>(kb, qv, m, l, o, (tf + it) * TT + tg, ctx, lo, cs, lane);
        }
        {
            const int it = n - 1;
            const PGQA_LDS char* kb = step(it);
            const int tile = tf + it;
            if (tile * TT >= lo && (tile + 1) * TT <= ctx)
                tile_compute<true, ES, D, GW, KES, kPF>(kb, qv, m, l, o, tile * TT + tg, ctx, lo, cs, lane);
            else
                tile_compute<false, ES, D, GW, KES, kPF>(kb, qv, m, l, o, tile * TT + tg, ctx, lo, cs, lane);
        }

        // ---- per-head (m, l) to every lane, then merge the TPR token groups ----
        float mh[GW], lh[GW];
        bcast_heads<LPT, GW>(m, mh, lane);
        bcast_heads<LPT, GW>(l, lh, lane);
#pragma unroll
        for (int mask = LPT; mask < kWave; mask <<= 1) {
#pragma unroll
            for (int g = 0; g < GW; ++g) {
                const float mo = shfl_xor_f32(mh[g], mask);
                const float lo = shfl_xor_f32(lh[g], mask);
                const float mx = fmaxf(mh[g], mo);
                const float a0 = __builtin_amdgcn_exp2f(mh[g] - mx);
                const float a1 = __builtin_amdgcn_exp2f(mo - mx);
                lh[g] = lh[g] * a0 + lo * a1;
#pragma unroll
                for (int x = 0; x < EPL; ++x) {
                    const float oo = shfl_xor_f32(o[g][x], mask);
                    o[g][x] = o[g][x] * a0 + oo * a1;
                }
                mh[g] = mx;
            }
        }

        if (whole) {
            if (tg == 0) {
#pragma unroll
                for (int g = 0; g < GW; ++g) {
                    const float inv = lh[g] > 0.0f ? 1.0f / lh[g] : 0.0f;
                    store_out16<ES>(a.out + ((int64_t)(b * a.num_q_heads + qh0 + g) * D + c * EPL) * ES, o[g], inv);
                }
            }
        } else {
            const int64_t seg = (int64_t)b * Hkv + h;
            if (tg == 0) {
#pragma unroll
                for (int g = 0; g < GW; ++g) {
                    const int64_t row = (w + seg) * G + wave * GW + g;
                    float* po = a.part_o + row * D + c * EPL;
#pragma unroll
                    for (int x = 0; x < EPL; x += 4) {
                        f32x4 v4 = {o[g][x], o[g][x + 1], o[g][x + 2], o[g][x + 3]};
                        *(f32x4*)(po + x) = v4;
                    }
                    if (c == 0) {
                        a.part_ml[row * 2 + 0] = mh[g];
                        a.part_ml[row * 2 + 1] = lh[g];
                    }
                }
            }
        }

        // ---- next piece ----------------------------------------------------------
        X += n;
        t0 += n;
        if (t0 == tiles_b) {
            t0 = 0;
            if (++h == Hkv) {
                h = 0;
                do {
                    ++b;
                } while (b < B && pref[b + 1] == pref[b]);
            }
            if (b < B) tiles_b = pref[b + 1] - pref[b];
        }
        if constexpr (W > 1) __syncthreads();   // ring slots are reused by the next piece
    }
}

// kMergeSlices 256-thread workgroups per (sequence, KV head) segment, each
// owning 256 of its G x D outputs: nothing when one share covered the whole
// segment (or it is empty), else the log-sum-exp merge of the segment's partials
// in share order (deterministic).  The loads of successive shares are
// independent.
// Shares merged per trip of the merge loop, their loads issued together (a 4,096-
// token window over 32K contexts cuts each segment into ~16 shares: 8 took its merge
// about 1 µs below 4).
#ifndef PGQA_MERGE_UNROLL
#define PGQA_MERGE_UNROLL 8
#endif

template <int G, int D>
constexpr int merge_slices() { return (G * D + 255) / 256; }

template <int ES, int D, int G>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
    constexpr int NS = merge_slices<G, D>();
    const int tid = threadIdx.x;
    const int Hkv = a.num_kv_heads;
    const int seg = blockIdx.x / NS;
    const int e = (blockIdx.x % NS) * 256 + tid;
    const int b = seg / Hkv;
    const int h = seg % Hkv;

    // Tiles of the sequences before b, of b, and of all: the split kernel's prefix sums.
    const int before = __builtin_amdgcn_readfirstlane(a.tile_pref[b]);
    const int tiles_b = __builtin_amdgcn_readfirstlane(a.tile_pref[b + 1]) - before;
    const int all = __builtin_amdgcn_readfirstlane(a.tile_pref[a.batch]);
    if (tiles_b == 0) return;   // zero-filled by the split kernel
    const int64_t total = (int64_t)Hkv * all;
    const int64_t nw = min((int64_t)a.num_splits, total);
    const int64_t xs = (int64_t)Hkv * before + (int64_t)h * tiles_b;
    const int64_t w0 = share_of(xs, total, nw);
    const int64_t w1 = share_of(xs + tiles_b - 1, total, nw);
    if (w0 == w1) return;

    if (e < G * D) {
        const int g = e / D;
        const int x = e % D;
        float M = -INFINITY, L = 0.0f, acc = 0.0f;
#pragma unroll PGQA_MERGE_UNROLL
        for (int64_t w = w0; w <= w1; ++w) {
            const int64_t row = (w + seg) * G + g;
            const float mw = a.part_ml[row * 2];
            const float lw = a.part_ml[row * 2 + 1];
            const float ow = a.part_o[row * D + x];
            const float mn = fmaxf(M, mw);
            const float sa = __builtin_amdgcn_exp2f(M - mn);
            const float sb = __builtin_amdgcn_exp2f(mw - mn);
            acc = acc * sa + ow * sb;
            L = L * sa + lw * sb;
            M = mn;
        }
        const float r = L > 0.0f ? acc / L : 0.0f;
        char* dst = a.out + ((int64_t)(b * a.num_q_heads + h * G) * D + e) * ES;
        if constexpr (ES == 2) *(uint16_t*)dst = (uint16_t)f32_to_bf16_bits(r);
        else *(float*)dst = r;
    }
}

// ---- dispatch ------------------------------------------------------------------

typedef void (*SplitFn)(DecodeArgs);
typedef void (*MergeFn)(DecodeArgs);

struct Entry {
    SplitFn split;
    MergeFn merge;
    int waves;
    int tile_bytes;
    int tt;
    int merge_slices;
};

template <int ES, int D, int G, int KES>
Entry make_entry() {
    constexpr int GW = G <= 8 ? G : 8;
    constexpr int W = G / GW;
    Entry e;
    e.split = decode_split_kernel<ES, D, GW, W, KES>;
    e.merge = decode_merge_kernel<ES, D, G>;
    e.waves = W;
    e.tile_bytes = Geo<ES, D, KES>::TILEB;
    e.tt = Geo<ES, D, KES>::TT;
    e.merge_slices = merge_slices<G, D>();
    return e;
}

template <int ES, int D, int KES = ES>
bool pick_g(int group, Entry* e) {
    switch (group) {
        case 1: *e = make_entry<ES, D, 1, KES>(); return true;
        case 2: *e = make_entry<ES, D, 2, KES>(); return true;
        case 4: *e = make_entry<ES, D, 4, KES>(); return true;
        case 8: *e = make_entry<ES, D, 8, KES>(); return true;
        case 16: *e = make_entry<ES, D, 16, KES>(); return true;
        case 32: *e = make_entry<ES, D, 32, KES>(); return true;
        case 64: *e = make_entry<ES, D, 64, KES>(); return true;
        default: return false;
    }
}

template <int ES>
bool pick_d(int head_dim, int group, Entry* e) {
    switch (head_dim) {
        case 16: return pick_g<ES, 16>(group, e);
        case 32: return pick_g<ES, 32>(group, e);
        case 64: return pick_g<ES, 64>(group, e);
        case 128: return pick_g<ES, 128>(group, e);
        default: return false;
    }
}

// FP8 pages with bf16 queries: head_dim 64 or 128.
bool pick_fp8(int head_dim, int group, Entry* e) {
    switch (head_dim) {
        case 64: return pick_g<2, 64, 1>(group, e);
        case 128: return pick_g<2, 128, 1>(group, e);
        default: return false;
    }
}

bool pick(int elem_bytes, int head_dim, int group, Entry* e) {
    if (elem_bytes == 2) return pick_d<2>(head_dim, group, e);
    if (elem_bytes == 4) return pick_d<4>(head_dim, group, e);
    return false;
}

// Concurrent workgroups per CU of a split kernel (cached per kernel and LDS size).
int occupancy(SplitFn fn, int threads, size_t lds) {
    static std::mutex mu;
    static struct { SplitFn fn; size_t lds; int occ; } cache[64];
    static int used = 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
        if (cache[i].fn == fn && cache[i].lds == lds) return cache[i].occ;
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void*)fn, threads, lds) != hipSuccess || occ < 1)
        occ = 1;
    if (used < 64) cache[used++] = {fn, lds, occ};
    return occ;
}

// LDS bytes per CU of the current device (cached per device).
size_t lds_per_cu() {
    static std::mutex mu;
    static size_t bytes[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    const int slot = dev < 64 ? dev : 63;
    std::lock_guard<std::mutex> lock(mu);
    if (bytes[slot] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess || n < 1)
            n = 160 * 1024;
        bytes[slot] = (size_t)n;
    }
    return bytes[slot];
}

int cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return 256;
    return n;
}

}  // namespace

int32_t decode_tile_tokens(int32_t elem_bytes, int32_t head_dim) {
    if (elem_bytes <= 0 || head_dim <= 0) return 0;
    const int epl = 16 / elem_bytes;
    const int lpt = head_dim / epl;
    if (lpt <= 0 || 64 % lpt) return 0;
    return kRows * (64 / lpt);
}

bool decode_supported(int32_t elem_bytes, int32_t head_dim, int32_t group) {
    Entry e;
    return pick(elem_bytes, head_dim, group, &e);
}

bool decode_fp8_supported(int32_t head_dim, int32_t group, int32_t block_size) {
    Entry e;
    return pick_fp8(head_dim, group, &e) && block_size >= 16 && block_size <= 256;
}

hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream) {
    const int es = L.is_bf16 ? 2 : 4;
    const int group = L.num_q_heads / L.num_kv_heads;
    Entry e;
    if (L.k_scale ? !pick_fp8(L.head_dim, group, &e) : !pick(es, L.head_dim, group, &e)) return hipErrorInvalidValue;
    if (L.batch == 0) return hipSuccess;

    // Many query heads on one KV head (MQA, G a multiple of 32): the G heads of a
    // token are rows of the matrix-core kernel (G = 32: the packed rows of one
    // tile, two waves sharing every key block; larger G: q [B, G, d] read as B
    // sequences of G tokens with one head, the same bytes), every row seeing
    // all keys [0, ctx) of the sequence's pages; the kernel's key split spreads
    // the long contexts.  At ~32 FLOP per K/V byte this shape outruns the VALU
    // dot products of the split kernel (bf16 only; no window; library-chosen
    // splits, so an explicit split count keeps the split-KV path).
    if (L.num_kv_heads == 1 && group % 32 == 0 && L.is_bf16 && !L.k_scale && L.window == 0 && L.num_splits == 0 &&
        (L.head_dim == 64 || L.head_dim == 128) && extend_supported(L.head_dim, 1, 1 << L.block_size_log2) &&
        (int64_t)L.batch * group <= 0x7fffffff) {
        ExtendLaunch x{};
        x.q = L.q;
        x.k_cache = L.k_cache;
        x.v_cache = L.v_cache;
        x.cu_q = nullptr;
        x.block_table = L.block_table;
        x.context_lens = L.context_lens;
        x.out = L.out;
        x.batch = L.batch;
        // G = 32: one token per sequence whose 32 heads are the packed rows of
        // one tile (its position ctx - 1 sees every key).  Otherwise the G heads
        // are read as G tokens of one head, all seeing every key.
        const bool packed = PGQA_MQA_PACK && group == 32;
        x.total_q = packed ? L.batch : L.batch * group;
        x.max_q_len = packed ? 1 : group;
        x.num_q_heads = packed ? group : 1;
        x.max_blocks_per_seq = L.max_blocks_per_seq;
        x.num_kv_heads = 1;
        x.head_dim = L.head_dim;
        x.block_size_log2 = L.block_size_log2;
        x.num_blocks = L.num_blocks;
        x.max_context_len = L.max_context_len;
        x.scale = L.scale;
        x.window = 0;
        x.workspace = L.workspace;
        x.workspace_bytes = decode_workspace_bytes(L.batch, L.num_q_heads, L.num_kv_heads, L.head_dim, 0);
        x.non_causal = packed ? 0 : 1;
        x.fixed_qlen = packed ? 1 : group;
        x.chunk_blocks = PGQA_MQA_CHUNK;
        if (log_enabled())
            log_line("decode B=%d Hq=%d Hkv=1 d=%d: %d query heads of a token as rows of the matrix-core kernel",
                     L.batch, L.num_q_heads, L.head_dim, group);
        return launch_extend(x, stream);
    }

    DecodeArgs a;
    a.q = (const char*)L.q;
    a.k_cache = (const char*)L.k_cache;
    a.v_cache = (const char*)L.v_cache;
    a.block_table = L.block_table;
    a.context_lens = L.context_lens;
    a.out = (char*)L.out;
    a.batch = L.batch;
    a.num_q_heads = L.num_q_heads;
    a.num_kv_heads = L.num_kv_heads;
    a.max_blocks_per_seq = L.max_blocks_per_seq;
    a.num_blocks = L.num_blocks;
    a.bs_log2 = L.block_size_log2;
    a.ctx_cap = L.max_context_len;
    const ScaleFold sf = fold_scale(L.scale, L.is_bf16 || L.k_scale);
    a.scale_log2 = sf.cs;
    a.q_and = sf.q_and;
    a.q_xor = sf.q_xor;
    a.window = L.window;
    a.k_scale = (const float*)L.k_scale;
    a.v_scale = (const float*)L.v_scale;

    const int threads = 64 * e.waves;
    // ring + tile prefix sums [batch + 1]
    size_t lds = (size_t)kStages * e.tile_bytes + (((size_t)L.batch + 1) * 4 + 15) / 16 * 16;
    // One-wave workgroups: ask for a quarter of the CU's LDS so that exactly one
    // runs per SIMD (bf16 / fp32 pages), or an eighth for exactly two (FP8
    // pages, whose code conversion makes the tile arithmetic the bound, so a
    // second wave per SIMD hides its latencies).  An uneven count (a second
    // wave on some SIMDs only) leaves those SIMDs twice as long on the same
    // shares: on the Llama-3-8B-shaped batch, 5 per CU ran 177 us against
    // 128 us for 4 (32-token tiles), the 16-token tiles 126-129 us at the 9 per
    // CU their LDS allows against 122 us at 4, and FP8 pages 78-86 us at 8 per
    // CU (8-row tiles) against 87-93 us at 4 (16-row tiles).
    if (e.waves == 1) lds = std::max(lds, lds_per_cu() / (L.k_scale ? PGQA_DECODE_LDS_DIV8 : PGQA_DECODE_LDS_DIV));
    int nw = L.num_splits;
    // Latency-bound calls (every segment at most kSegModeTiles tiles, no split
    // count asked for): one workgroup per segment writes its outputs directly,
    // so the merge kernel is not launched.  (At most kDecodeMaxSplits segments:
    // the workspace of a call without a split count is laid out for that many
    // shares.)
    const int64_t segs = (int64_t)L.batch * L.num_kv_heads;
    a.seg_mode = (nw <= 0 && segs <= kDecodeMaxSplits &&
                  ((int64_t)L.max_context_len + e.tt - 1) / e.tt <= kSegModeTiles) ? 1 : 0;
    if (a.seg_mode) {
        nw = (int)segs;
    } else if (nw <= 0) {
        nw = occupancy(e.split, threads, lds) * cu_count();
        if (nw > kDecodeMaxSplits) nw = kDecodeMaxSplits;
    }
    a.num_splits = nw;
    const int64_t slots = (int64_t)nw + (int64_t)L.batch * L.num_kv_heads;
    a.part_o = (float*)L.workspace;
    a.part_ml = a.part_o + slots * (L.num_q_heads / L.num_kv_heads) * L.head_dim;
    a.tile_pref = (int32_t*)(a.part_ml + slots * (L.num_q_heads / L.num_kv_heads) * 2);

    if (log_enabled() && a.seg_mode)
        log_line("decode B=%d Hq=%d Hkv=%d d=%d bs=%d%s window=%d: split-KV kernel, one workgroup per segment "
                 "(%d x %d waves), LDS %zu B; no merge",
                 L.batch, L.num_q_heads, L.num_kv_heads, L.head_dim, 1 << L.block_size_log2,
                 L.k_scale ? " fp8" : (L.is_bf16 ? " bf16" : " f32"), L.window, nw, e.waves, lds);
    else if (log_enabled())
        log_line("decode B=%d Hq=%d Hkv=%d d=%d bs=%d%s window=%d: split-KV kernel, %d workgroups x %d waves "
                 "(%s splits), LDS %zu B; merge %d workgroups",
                 L.batch, L.num_q_heads, L.num_kv_heads, L.head_dim, 1 << L.block_size_log2,
                 L.k_scale ? " fp8" : (L.is_bf16 ? " bf16" : " f32"), L.window, nw, e.waves,
                 L.num_splits > 0 ? "caller's" : "occupancy", lds, L.batch * L.num_kv_heads * e.merge_slices);
    hipLaunchKernelGGL(e.split, dim3(nw), dim3(threads), lds, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.seg_mode) return err;
    hipLaunchKernelGGL(e.merge, dim3(L.batch * L.num_kv_heads * e.merge_slices), dim3(256), 0, stream, a);
    return hipGetLastError();
}

// Scratch of the allocation-free decode entry point: a file-scope device array,
// one copy per GPU (held until the process ends).  Host code never passes the
// array's name to a kernel (on the host that name is only a stand-in for the
// symbol); it looks up the device address on each device once and passes that.
// Every call on one GPU shares the array: calls that may overlap on that GPU race.
static __device__ __attribute__((aligned(256))) char scratch[kDecodeScratchBytes];

void* decode_scratch() {
    static std::mutex mu;
    static void* addr[64] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        addr[dev] = p;
    }
    return addr[dev];
}

size_t decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t num_splits) {
    const int64_t splits = num_splits > 0 ? num_splits : kDecodeMaxSplits;
    const int64_t slots = splits + (int64_t)batch * num_kv_heads;
    const int64_t group = num_q_heads / num_kv_heads;
    return (size_t)(slots * group * (head_dim + 2) * 4 + ((int64_t)batch + 1) * 4);
}

}  // namespace pgqa
