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
//  * Streaming: each tile is 4 KB of K plus 4 KB of V (bf16, d = 128), moved
//    with 16-byte-per-lane global->LDS DMA (global_load_lds_dwordx4) into a
//    ring of NSTAGE tiles, so loads for later tiles are in flight while the
//    current one is computed and no VGPRs are tied up by the prefetch.
//  * Lane mapping: LPT = d*elem/16 lanes cover one token row (16 lanes for
//    bf16 d = 128), so one wave row holds TPR = 64/LPT tokens.  Each lane keeps
//    its 16-byte slice of the G query rows in registers; every K row is read
//    once from LDS and used for all G query heads of the group.
//  * Dot products: v_dot2_f32_bf16 (fp32 accumulate) then a DPP butterfly over
//    the LPT lanes of the row.  Softmax state (m, l, o) is kept per lane and
//    merged across the TPR token groups with shuffles once per share.
//  * Online softmax with a lazy rescale: o and l are rescaled only when the
//    running max grows by more than 8 (log2 units), which keeps every weight
//    <= 256 and is exact because the final o / l uses the same reference max.
//  * Masking selects (never multiplies): scores past the context become -inf
//    and V rows past the context are zeroed, so NaN in unused slots cannot leak.
//  * Large groups (G >= 16) use G/8 waves per workgroup sharing one ring; each
//    wave owns 8 query heads.
#include "device_common.hpp"
#include "launch.hpp"

#include <math.h>
#include <mutex>

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
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t max_blocks_per_seq;
    int32_t num_blocks;
    int32_t bs_log2;
    int32_t ctx_cap;     // max_context_len: device context lengths are clamped to it
    int32_t num_splits;  // number of shares == gridDim.x of the split kernel
    float scale_log2;    // scale * log2(e): scores live in log2 units, weights use exp2
};

template <int ES, int D>
struct Geo {
    static constexpr int EPL = 16 / ES;          // elements per lane per 16-byte load
    static constexpr int LPT = D / EPL;          // lanes per token row
    static constexpr int TPR = kWave / LPT;      // tokens per 1 KB wave row
    static constexpr int RPT = 4;                // wave rows per tile, for K and for V
    static constexpr int TT = RPT * TPR;         // tokens per tile
    static constexpr int ROWB = 1024;
    static constexpr int TILEB = 2 * RPT * ROWB; // bytes of K + V per tile
    static_assert(LPT >= 1 && LPT <= 32 && TPR * LPT == kWave, "unsupported head_dim / dtype");
};

constexpr int kStages = 3;   // ring depth (tiles) of the split kernel

__device__ __forceinline__ int tiles_of(int ctx, int cap, int tt) {
    ctx = clampi(ctx, 0, cap);
    return (ctx + tt - 1) / tt;
}

// q . k for one lane's 16-byte slices (fp32 accumulation).
template <int ES>
__device__ __forceinline__ float slice_dot(const u32x4& q, const u32x4& k) {
    if constexpr (ES == 2) {
        float acc = dot2_bf16(q.x, k.x, 0.0f);
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

// Issue the global->LDS loads of one tile (token rows of K, then of V) into
// ring slot `slot`.  Wave `wave` issues the loads li with li % W == wave, so each
// wave issues exactly 2*RPT/W loads per tile (the wait counts rely on it).
template <int ES, int D, int W>
__device__ __forceinline__ void issue_tile(const DecodeArgs& a, PGQA_LDS char* ring, int slot, int tile,
                                           int h, int ctx, const int32_t* __restrict__ bt_row,
                                           int wave, int lane) {
    using Gm = Geo<ES, D>;
    const int tg = lane / Gm::LPT;
    const int bs_mask = (1 << a.bs_log2) - 1;
    const int tile_tok = tile * Gm::TT;
    PGQA_LDS char* dst = ring + slot * Gm::TILEB;
    if (Gm::TT <= (1 << a.bs_log2)) {
        // The tile lies inside one page (the page is allocated because the tile
        // starts before the context end), and its K rows are one contiguous
        // 4 KB run of that page: row r of the tile is bytes [1024 r, 1024 r + 1024).
        // Slots past the context are read (in bounds) and masked in compute.
        const int bid = clampi(bt_row[tile_tok >> a.bs_log2], 0, a.num_blocks - 1);
        const int64_t run = ((((int64_t)bid * a.num_kv_heads + h) << a.bs_log2) + (tile_tok & bs_mask)) * (D * ES);
        const char* kp = a.k_cache + run + lane * 16;
        const char* vp = a.v_cache + run + lane * 16;
#pragma unroll
        for (int li = 0; li < 2 * Gm::RPT; ++li) {
            if (li % W != wave) continue;
            const int r = li % Gm::RPT;
            const bool isv = li >= Gm::RPT;
            load_lds_16((isv ? vp : kp) + r * Gm::ROWB, dst + li * Gm::ROWB);
        }
    } else {
        // Pages smaller than a tile: each lane looks up its own token's page
        // (positions clamped to the context so every table read is in range).
        const int c = lane % Gm::LPT;
        int blk[Gm::RPT];
        int tok[Gm::RPT];
#pragma unroll
        for (int r = 0; r < Gm::RPT; ++r) {
            tok[r] = min(tile_tok + r * Gm::TPR + tg, ctx - 1);
            blk[r] = clampi(bt_row[tok[r] >> a.bs_log2], 0, a.num_blocks - 1);
        }
#pragma unroll
        for (int li = 0; li < 2 * Gm::RPT; ++li) {
            if (li % W != wave) continue;
            const int r = li % Gm::RPT;
            const bool isv = li >= Gm::RPT;
            const int64_t prow = (((int64_t)blk[r] * a.num_kv_heads + h) << a.bs_log2) + (tok[r] & bs_mask);
            const char* src = (isv ? a.v_cache : a.k_cache) + prow * (D * ES) + c * 16;
            load_lds_16(src, dst + li * Gm::ROWB);
        }
    }
}

template <int ES, int D, int GW, int W>
__global__ __launch_bounds__(64 * W) void decode_split_kernel(DecodeArgs a) {
    using Gm = Geo<ES, D>;
    constexpr int EPL = Gm::EPL, LPT = Gm::LPT, TPR = Gm::TPR, RPT = Gm::RPT, TT = Gm::TT;
    constexpr int G = GW * W;
    constexpr int LPW = 2 * RPT / W;   // loads per wave per tile
    static_assert((2 * RPT) % W == 0, "loads must split evenly across waves");

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
            int x = b < B ? tiles_of(a.context_lens[b], a.ctx_cap, TT) : 0;
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

    // Shares: min(num_splits, total) so that no share is empty and every share
    // of a cut segment writes the partial the merge reads.
    const int64_t total = (int64_t)Hkv * pref[B];
    const int64_t NW = min((int64_t)a.num_splits, total);
    const int64_t w = blockIdx.x;
    if (w >= NW) return;
    int64_t X = w * total / NW;
    const int64_t X1 = (w + 1) * total / NW;

    // Segment (b, h) and tile t of the first tile of this share.
    int b;
    {
        int lo = 0, hi = B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((int64_t)Hkv * pref[mid] <= X) lo = mid;
            else hi = mid - 1;
        }
        b = lo;
    }
    int tiles_b = pref[b + 1] - pref[b];
    int64_t rem = X - (int64_t)Hkv * pref[b];
    int h = (int)(rem / tiles_b);
    int t0 = (int)(rem % tiles_b);

    const int c = lane % LPT;
    const int tg = lane / LPT;

    while (X < X1) {
        const int n = (int)min((int64_t)(tiles_b - t0), X1 - X);   // tiles in this piece
        const bool whole = (t0 == 0) && (n == tiles_b);
        const int ctx = clampi(a.context_lens[b], 0, a.ctx_cap);
        const int32_t* bt_row = a.block_table + (int64_t)b * a.max_blocks_per_seq;
        const int qh0 = h * G + wave * GW;

        // This wave's query slices: GW heads x 16 bytes.
        u32x4 qv[GW];
#pragma unroll
        for (int g = 0; g < GW; ++g)
            qv[g] = *(const u32x4*)(a.q + ((int64_t)(b * a.num_q_heads + qh0 + g) * D + c * EPL) * ES);

        float m[GW], l[GW], o[GW][EPL];
#pragma unroll
        for (int g = 0; g < GW; ++g) {
            m[g] = kMaxInit;
            l[g] = 0.0f;
#pragma unroll
            for (int x = 0; x < EPL; ++x) o[g][x] = 0.0f;
        }

        // Prologue: fill the first kStages-1 ring slots.
#pragma unroll
        for (int i = 0; i < kStages - 1; ++i)
            if (i < n) issue_tile<ES, D, W>(a, ring, i, t0 + i, h, ctx, bt_row, wave, lane);

        for (int it = 0; it < n; ++it) {
            const int tile = t0 + it;
            const int slot = it % kStages;
            // Loads issued after this tile's: at most kStages-2 tiles of LPW loads each.
            wait_vmcnt_dyn<(kStages - 2) * LPW>(LPW * min(kStages - 2, n - 1 - it));
            if constexpr (W > 1) __syncthreads();
            if (it + kStages - 1 < n)
                issue_tile<ES, D, W>(a, ring, (it + kStages - 1) % kStages, tile + kStages - 1, h, ctx,
                                     bt_row, wave, lane);

            // ---- compute tile ------------------------------------------------
            const PGQA_LDS char* kb = ring + (slot * 2) * RPT * Gm::ROWB + lane * 16;
            const PGQA_LDS char* vb = kb + RPT * Gm::ROWB;
            const int tok0 = tile * TT + tg;
            const bool full = (tile + 1) * TT <= ctx;

            float s[RPT][GW];
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const u32x4 kx = lds_read_16(kb + r * Gm::ROWB);
                const bool valid = tok0 + r * TPR < ctx;
#pragma unroll
                for (int g = 0; g < GW; ++g) {
                    const float sc = group_sum<LPT>(slice_dot<ES>(qv[g], kx));
                    s[r][g] = valid ? sc * a.scale_log2 : -INFINITY;
                }
            }
            bool need = false;
            float mt[GW];
#pragma unroll
            for (int g = 0; g < GW; ++g) {
                mt[g] = s[0][g];
#pragma unroll
                for (int r = 1; r < RPT; ++r) mt[g] = fmaxf(mt[g], s[r][g]);
                need |= mt[g] > m[g] + 8.0f;
            }
            if (__any(need)) {
#pragma unroll
                for (int g = 0; g < GW; ++g) {
                    if (mt[g] > m[g] + 8.0f) {
                        const float alpha = __builtin_amdgcn_exp2f(m[g] - mt[g]);
                        m[g] = mt[g];
                        l[g] *= alpha;
#pragma unroll
                        for (int x = 0; x < EPL; ++x) o[g][x] *= alpha;
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < RPT; ++r)
#pragma unroll
                for (int g = 0; g < GW; ++g) {
                    s[r][g] = __builtin_amdgcn_exp2f(s[r][g] - m[g]);
                    l[g] += s[r][g];
                }
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const u32x4 vx = lds_read_16(vb + r * Gm::ROWB);
                float vf[EPL];
                unpack16<ES>(vx, vf);
                if (!full && tok0 + r * TPR >= ctx) {
#pragma unroll
                    for (int x = 0; x < EPL; ++x) vf[x] = 0.0f;
                }
#pragma unroll
                for (int g = 0; g < GW; ++g)
#pragma unroll
                    for (int x = 0; x < EPL; ++x) o[g][x] = fmaf(s[r][g], vf[x], o[g][x]);
            }
        }

        // ---- merge the TPR token groups of the wave ----------------------------
#pragma unroll
        for (int mask = LPT; mask < kWave; mask <<= 1) {
#pragma unroll
            for (int g = 0; g < GW; ++g) {
                const float mo = shfl_xor_f32(m[g], mask);
                const float lo = shfl_xor_f32(l[g], mask);
                const float mx = fmaxf(m[g], mo);
                const float a0 = __builtin_amdgcn_exp2f(m[g] - mx);
                const float a1 = __builtin_amdgcn_exp2f(mo - mx);
                l[g] = l[g] * a0 + lo * a1;
#pragma unroll
                for (int x = 0; x < EPL; ++x) {
                    const float oo = shfl_xor_f32(o[g][x], mask);
                    o[g][x] = o[g][x] * a0 + oo * a1;
                }
                m[g] = mx;
            }
        }

        if (tg == 0) {
            if (whole) {
#pragma unroll
                for (int g = 0; g < GW; ++g) {
                    const float inv = l[g] > 0.0f ? 1.0f / l[g] : 0.0f;
                    store_out16<ES>(a.out + ((int64_t)(b * a.num_q_heads + qh0 + g) * D + c * EPL) * ES, o[g], inv);
                }
            } else {
                const int64_t slot_id = w + (int64_t)b * Hkv + h;
#pragma unroll
                for (int g = 0; g < GW; ++g) {
                    const int64_t row = slot_id * G + wave * GW + g;
                    float* po = a.part_o + row * D + c * EPL;
#pragma unroll
                    for (int x = 0; x < EPL; x += 4) {
                        f32x4 v4 = {o[g][x], o[g][x + 1], o[g][x + 2], o[g][x + 3]};
                        *(f32x4*)(po + x) = v4;
                    }
                    if (c == 0) {
                        a.part_ml[row * 2 + 0] = m[g];
                        a.part_ml[row * 2 + 1] = l[g];
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

// Share (workgroup) of the split kernel that holds global tile X.
__device__ __forceinline__ int64_t share_of(int64_t X, int64_t total, int64_t nw) {
    return ((X + 1) * nw - 1) / total;
}

// One wave per (sequence, KV head) segment: writes zeros for an empty context,
// nothing when one share covered the whole segment, else the log-sum-exp merge
// of the segment's partials in share order (deterministic).
template <int ES, int D, int G>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a, int tt) {
    const int lane = threadIdx.x;
    const int Hkv = a.num_kv_heads;
    const int seg = blockIdx.x;
    const int b = seg / Hkv;
    const int h = seg % Hkv;

    int before = 0, all = 0;
    for (int i = lane; i < a.batch; i += 64) {
        const int t = tiles_of(a.context_lens[i], a.ctx_cap, tt);
        all += t;
        if (i < b) before += t;
    }
    for (int mk = 32; mk >= 1; mk >>= 1) {
        before += __shfl_xor(before, mk);
        all += __shfl_xor(all, mk);
    }
    const int tiles_b = tiles_of(a.context_lens[b], a.ctx_cap, tt);
    if (tiles_b == 0) {
        for (int g = 0; g < G; ++g)
            for (int x = lane; x < D; x += 64) {
                char* dst = a.out + ((int64_t)(b * a.num_q_heads + h * G + g) * D + x) * ES;
                if constexpr (ES == 2) *(uint16_t*)dst = 0;
                else *(float*)dst = 0.0f;
            }
        return;
    }
    const int64_t total = (int64_t)Hkv * all;
    const int64_t nw = min((int64_t)a.num_splits, total);
    const int64_t xs = (int64_t)Hkv * before + (int64_t)h * tiles_b;
    const int64_t xe = xs + tiles_b - 1;
    const int64_t w0 = share_of(xs, total, nw);
    const int64_t w1 = share_of(xe, total, nw);
    if (w0 == w1) return;

    for (int g = 0; g < G; ++g) {
        float mx = -INFINITY;
        for (int64_t w = w0; w <= w1; ++w) mx = fmaxf(mx, a.part_ml[((w + seg) * G + g) * 2]);
        float L = 0.0f;
        for (int64_t w = w0; w <= w1; ++w) {
            const float* ml = a.part_ml + ((w + seg) * G + g) * 2;
            L += __builtin_amdgcn_exp2f(ml[0] - mx) * ml[1];
        }
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        for (int x = lane; x < D; x += 64) {
            float acc = 0.0f;
            for (int64_t w = w0; w <= w1; ++w) {
                const int64_t row = (w + seg) * G + g;
                acc += __builtin_amdgcn_exp2f(a.part_ml[row * 2] - mx) * a.part_o[row * D + x];
            }
            const float r = acc * inv;
            char* dst = a.out + ((int64_t)(b * a.num_q_heads + h * G + g) * D + x) * ES;
            if constexpr (ES == 2) *(uint16_t*)dst = (uint16_t)f32_to_bf16_bits(r);
            else *(float*)dst = r;
        }
    }
}

// ---- dispatch ------------------------------------------------------------------

typedef void (*SplitFn)(DecodeArgs);
typedef void (*MergeFn)(DecodeArgs, int);

struct Entry {
    SplitFn split;
    MergeFn merge;
    int waves;
    int tile_bytes;
    int tt;
};

template <int ES, int D, int G>
Entry make_entry() {
    constexpr int GW = G <= 8 ? G : 8;
    constexpr int W = G / GW;
    Entry e;
    e.split = decode_split_kernel<ES, D, GW, W>;
    e.merge = decode_merge_kernel<ES, D, G>;
    e.waves = W;
    e.tile_bytes = Geo<ES, D>::TILEB;
    e.tt = Geo<ES, D>::TT;
    return e;
}

template <int ES, int D>
bool pick_g(int group, Entry* e) {
    switch (group) {
        case 1: *e = make_entry<ES, D, 1>(); return true;
        case 2: *e = make_entry<ES, D, 2>(); return true;
        case 4: *e = make_entry<ES, D, 4>(); return true;
        case 8: *e = make_entry<ES, D, 8>(); return true;
        case 16: *e = make_entry<ES, D, 16>(); return true;
        case 32: *e = make_entry<ES, D, 32>(); return true;
        case 64: *e = make_entry<ES, D, 64>(); return true;
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
    return 4 * (64 / lpt);
}

bool decode_supported(int32_t elem_bytes, int32_t head_dim, int32_t group) {
    Entry e;
    return pick(elem_bytes, head_dim, group, &e);
}

hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream) {
    const int es = L.is_bf16 ? 2 : 4;
    const int group = L.num_q_heads / L.num_kv_heads;
    Entry e;
    if (!pick(es, L.head_dim, group, &e)) return hipErrorInvalidValue;
    if (L.batch == 0) return hipSuccess;

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
    a.scale_log2 = (float)((double)L.scale * 1.4426950408889634);

    const int threads = 64 * e.waves;
    const size_t lds = (size_t)kStages * e.tile_bytes + (((size_t)L.batch + 1) * 4 + 15) / 16 * 16;
    int nw = L.num_splits;
    if (nw <= 0) {
        nw = occupancy(e.split, threads, lds) * cu_count();
        if (nw > kDecodeMaxSplits) nw = kDecodeMaxSplits;
    }
    a.num_splits = nw;
    const int64_t slots = (int64_t)nw + (int64_t)L.batch * L.num_kv_heads;
    a.part_o = (float*)L.workspace;
    a.part_ml = a.part_o + slots * L.num_q_heads / L.num_kv_heads * L.head_dim;

    hipLaunchKernelGGL(e.split, dim3(nw), dim3(threads), lds, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(e.merge, dim3(L.batch * L.num_kv_heads), dim3(64), 0, stream, a, e.tt);
    return hipGetLastError();
}

}  // namespace pgqa
