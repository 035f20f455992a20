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
//  * Each wave computes S^T = K Q^T for 32 keys x its 32 query rows.  In the
//    32x32 accumulator layout a lane then holds 16 keys of ONE query row, so the
//    row max / sum need a single cross-lane step (lane ^ 32).
//  * O^T += V^T P^T: the B operand (P^T) is exactly the lane's own S^T values
//    rounded to bf16, taken in the key order the accumulator layout gives; the
//    A operand is V^T read from LDS, where V is stored transposed while staged.
//  * Online softmax in log2 units with a lazy rescale (only when a row max grows
//    by more than 8), exact because the final O / l uses the same reference.
//  * Masks select -inf (never multiply); keys past the sequence are staged as
//    zeros.  Only the diagonal block (causal) and the ragged last block mask.
//  * Query tiles are launched heaviest-first (reverse order) to shorten the tail.
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
    float scale_log2;
};

constexpr int BQ = 32;   // query rows per wave
constexpr int BN = 32;   // keys per block

template <int D, int HG>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
    constexpr int TB = 4 / HG;               // 32-row token blocks per workgroup
    constexpr int KSTEPS = D / 16;           // k-steps of S^T over head_dim
    constexpr int DBLK = D / 32;             // 32-row blocks of O^T over head_dim
    constexpr int KROW = D * 2 + 16;         // padded K row in LDS (bytes)
    constexpr int VROW = BN * 2 + 8;         // padded V^T row in LDS (bytes)
    constexpr int CPR = D / 8;               // 16-byte chunks per K/V row
    constexpr int CHUNKS = BN * CPR;         // chunks per K (or V) block
    constexpr int PER_T = (CHUNKS + 255) / 256;
    static_assert(CHUNKS % 256 == 0, "K/V block must split evenly over 256 threads");

    __shared__ __attribute__((aligned(16))) char k_lds[BN * KROW];
    __shared__ __attribute__((aligned(16))) char vt_lds[D * VROW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int G = a.num_q_heads / a.num_kv_heads;
    const int groups = G / HG;

    const int s = blockIdx.z;
    const int seq0 = clampi(a.cu_seqlens[s], 0, a.total_tokens);
    const int L = clampi(a.cu_seqlens[s + 1], seq0, a.total_tokens) - seq0;
    const int qtile = gridDim.x - 1 - blockIdx.x;
    const int tok0 = qtile * TB * BQ;
    if (tok0 >= L) return;
    const int kvh = blockIdx.y / groups;
    const int head = kvh * G + (blockIdx.y % groups) * HG + (wave % HG);
    const int i0 = tok0 + (wave / HG) * BQ;          // this wave's first query row (sequence-local)

    const int wg_rows_end = min(L, tok0 + TB * BQ);
    const int nkb = a.causal ? (wg_rows_end + BN - 1) / BN : (L + BN - 1) / BN;
    const bool active = i0 < L;
    const int last_kb = a.causal ? min(nkb - 1, (i0 + BQ - 1) / BN) : nkb - 1;

    const int64_t qstride = (int64_t)a.num_q_heads * D * 2;    // bytes per packed Q row
    const int64_t kvstride = (int64_t)a.num_kv_heads * D * 2;  // bytes per packed K/V row

    // Q^T operand: lane holds row (i0 + l32), d = 16*kk + 8*half .. +8.
    u32x4 qreg[KSTEPS];
    {
        const int row = min(i0 + l32, L - 1);
        const char* qp = a.q + (int64_t)(seq0 + row) * qstride + (int64_t)head * D * 2 + half * 16;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) qreg[kk] = *(const u32x4*)(qp + kk * 32);
    }

    float m = kMaxInit, lsum = 0.0f;
    f32x16 o[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.0f;

    // Register prefetch of one K/V block: thread chunk c -> key c / CPR, 16-byte column c % CPR.
    u32x4 kpre[PER_T], vpre[PER_T];
    auto fetch = [&](int kb) {
#pragma unroll
        for (int e = 0; e < PER_T; ++e) {
            const int ch = tid + e * 256;
            const int key = kb * BN + ch / CPR;
            const int col = ch % CPR;
            if (key < L) {
                const int64_t off = (int64_t)(seq0 + key) * kvstride + (int64_t)kvh * D * 2 + col * 16;
                kpre[e] = *(const u32x4*)(a.k + off);
                vpre[e] = *(const u32x4*)(a.v + off);
            } else {
                kpre[e] = u32x4{0, 0, 0, 0};
                vpre[e] = u32x4{0, 0, 0, 0};
            }
        }
    };

    fetch(0);
    for (int kb = 0; kb < nkb; ++kb) {
        __syncthreads();   // every wave is done reading the previous block
#pragma unroll
        for (int e = 0; e < PER_T; ++e) {
            const int ch = tid + e * 256;
            const int key = ch / CPR;
            const int col = ch % CPR;
            *(u32x4*)(k_lds + key * KROW + col * 16) = kpre[e];
            const u32 w[4] = {vpre[e].x, vpre[e].y, vpre[e].z, vpre[e].w};
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                *(uint16_t*)(vt_lds + (col * 8 + 2 * x) * VROW + key * 2) = (uint16_t)(w[x] & 0xffffu);
                *(uint16_t*)(vt_lds + (col * 8 + 2 * x + 1) * VROW + key * 2) = (uint16_t)(w[x] >> 16);
            }
        }
        __syncthreads();
        if (kb + 1 < nkb) fetch(kb + 1);

        if (active && kb <= last_kb) {
            const int j0 = kb * BN;
            // S^T = K Q^T: lane (l32, half) gets rows l32, keys 8*(i/4) + 4*half + i%4.
            f32x16 st;
#pragma unroll
            for (int i = 0; i < 16; ++i) st[i] = 0.0f;
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                const u32x4 ka = *(const u32x4*)(k_lds + l32 * KROW + kk * 32 + half * 16);
                st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka),
                                                             __builtin_bit_cast(bf16x8, qreg[kk]), st, 0, 0, 0);
            }
            const int row = i0 + l32;
            const bool edge = (j0 + BN > L) || (a.causal && j0 + BN - 1 > i0);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = j0 + 8 * (i >> 2) + 4 * half + (i & 3);
                const bool ok = !edge || (key < L && (!a.causal || key <= row));
                st[i] = ok ? st[i] * a.scale_log2 : -INFINITY;
            }
            float mt = st[0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mt = fmaxf(mt, st[i]);
            mt = fmaxf(mt, shfl_xor_f32(mt, 32));
            const bool need = mt > m + 8.0f;
            if (__any(need)) {
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
            u32x4 pb[2];
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                float p[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    p[j] = __builtin_amdgcn_exp2f(st[8 * k2 + j] - m);
                    lsum += p[j];
                }
                pb[k2] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                               pack_bf16x2(p[6], p[7])};
            }
            // O^T += V^T P^T: A = V^T rows d, keys {16*k2 + 4*half + 0..3, 16*k2 + 8 + 4*half + 0..3}.
#pragma unroll
            for (int db = 0; db < DBLK; ++db) {
                const char* vrow = vt_lds + (db * 32 + l32) * VROW + half * 8;
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) {
                    const u32x2 lo = *(const u32x2*)(vrow + k2 * 32);
                    const u32x2 hi = *(const u32x2*)(vrow + k2 * 32 + 16);
                    const u32x4 va = {lo.x, lo.y, hi.x, hi.y};
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va),
                                                                    __builtin_bit_cast(bf16x8, pb[k2]), o[db], 0, 0,
                                                                    0);
                }
            }
        }
    }

    if (!active) return;
    lsum += shfl_xor_f32(lsum, 32);
    const int row = i0 + l32;
    if (row >= L) return;
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
    char* op = a.out + (int64_t)(seq0 + row) * qstride + (int64_t)head * D * 2;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const int d = db * 32 + 8 * qd + 4 * half;
            u32x2 w;
            w.x = pack_bf16x2(o[db][4 * qd + 0] * inv, o[db][4 * qd + 1] * inv);
            w.y = pack_bf16x2(o[db][4 * qd + 2] * inv, o[db][4 * qd + 3] * inv);
            *(u32x2*)(op + d * 2) = w;
        }
}

typedef void (*PrefillFn)(PrefillArgs);

bool pick(int head_dim, int group, PrefillFn* fn, int* hg) {
    const int h = group >= 4 ? 4 : group;
    if (group != 1 && group != 2 && group % 4 != 0) return false;
    if (group > 64) return false;
    *hg = h;
    if (head_dim == 128) {
        *fn = h == 4 ? prefill_kernel<128, 4> : (h == 2 ? prefill_kernel<128, 2> : prefill_kernel<128, 1>);
        return true;
    }
    if (head_dim == 64) {
        *fn = h == 4 ? prefill_kernel<64, 4> : (h == 2 ? prefill_kernel<64, 2> : prefill_kernel<64, 1>);
        return true;
    }
    return false;
}

}  // namespace

bool prefill_supported(int32_t head_dim, int32_t group) {
    PrefillFn fn;
    int hg;
    return pick(head_dim, group, &fn, &hg);
}

hipError_t launch_prefill(const PrefillLaunch& L, hipStream_t stream) {
    const int group = L.num_q_heads / L.num_kv_heads;
    PrefillFn fn;
    int hg;
    if (!pick(L.head_dim, group, &fn, &hg)) return hipErrorInvalidValue;
    PrefillArgs a;
    a.q = (const char*)L.q;
    a.k = (const char*)L.k;
    a.v = (const char*)L.v;
    a.cu_seqlens = L.cu_seqlens;
    a.out = (char*)L.out;
    a.total_tokens = L.total_tokens;
    a.num_q_heads = L.num_q_heads;
    a.num_kv_heads = L.num_kv_heads;
    a.causal = L.causal;
    a.scale_log2 = (float)((double)L.scale * 1.4426950408889634);
    const int rows_per_wg = (4 / hg) * BQ;
    const int nqt = (L.max_seqlen + rows_per_wg - 1) / rows_per_wg;
    dim3 grid(nqt, L.num_kv_heads * (group / hg), L.batch);
    hipLaunchKernelGGL(fn, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pgqa
