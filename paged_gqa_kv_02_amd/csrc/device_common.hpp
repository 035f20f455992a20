// device_common.hpp -- small gfx950 device helpers shared by the kernels of
// libpaged_gqa.so: bf16 packing, DPP lane reductions, LDS-DMA loads and
// explicit wait counters.  Wave64 throughout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pgqa {

#define PGQA_LDS __attribute__((address_space(3)))

typedef uint32_t u32;
typedef __attribute__((ext_vector_type(4))) u32 u32x4;
typedef __attribute__((ext_vector_type(2))) u32 u32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;

constexpr int kWave = 64;

// Finite stand-in for -inf as the initial running max: keeps every exp2 argument
// finite, so an empty token group yields weight 0 instead of NaN.
constexpr float kMaxInit = -1.0e30f;

// ---- bf16 <-> fp32 -------------------------------------------------------
__device__ __forceinline__ float bf16_lo(u32 w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(u32 w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ u32 f32_to_bf16_bits(float f) {
    u32 u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ u32 pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Two fp32 -> packed bf16 pair (lo, hi) with the hardware's round-to-nearest-even.
__device__ __forceinline__ u32 pack_bf16x2_rne_hw(float lo, float hi) {
    typedef __attribute__((ext_vector_type(2))) float f32x2_t;
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(u32, __builtin_convertvector(v, bf16x2));
}

// bf16 pair dot product accumulated in fp32: acc + a.lo*b.lo + a.hi*b.hi
__device__ __forceinline__ float dot2_bf16(u32 a, u32 b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                           acc, false);
}

// 8 FP8 E4M3 codes (little-endian bytes of w) -> 8 bf16 values in the same
// order, as a bf16 row slice (exact: every E4M3 value is a bf16 value).
__device__ __forceinline__ u32x4 fp8x8_to_bf16(u32x2 w) {
    return u32x4{__builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false)),
                 __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true)),
                 __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false)),
                 __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true))};
}

// ---- cross-lane ---------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of LANES lanes (LANES in {1, 2, 4, 8, 16, 32}); every
// lane of a group ends with the same bits (each step adds a commutative pair).
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(LANES == 1 || LANES == 2 || LANES == 4 || LANES == 8 || LANES == 16 || LANES == 32, "");
    if constexpr (LANES >= 2) x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (LANES >= 4) x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (LANES >= 8) x += dpp_f32<0x141>(x);  // row_half_mirror: quad 0 <-> quad 1
    if constexpr (LANES >= 16) x += dpp_f32<0x140>(x); // row_mirror: half-row 0 <-> 1
    if constexpr (LANES >= 32)                          // ds_swizzle xor 16 within 32 lanes
        x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
    return x;
}

__device__ __forceinline__ float shfl_xor_f32(float x, int mask) {
    const int lane = __lane_id();
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(x)));
}

// max(x of this lane, x of lane ^ 32) with gfx950's half-wave swap
// (v_permlane32_swap: a VALU operation, no LDS round trip).  Swapping the upper
// half of one copy with the lower half of another leaves the lower halves in the
// first result and the upper halves in the second, each duplicated over the wave.
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_max(float x) {
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, shfl_xor_f32(x, m));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
    for (int m = 32; m >= 1; m >>= 1) x += shfl_xor_f32(x, m);
    return x;
}

// ---- memory ---------------------------------------------------------------
// Cache policy of the K/V streaming loads.  Where a K/V byte is read once per
// call (decode; multi-token calls whose pairs have one query tile), it is loaded
// non-temporal (the gfx950 "nt" bit, cache-policy value 2), so its lines are not
// kept for reuse in L2 / Infinity Cache.  On randomly placed 4 KB page runs
// through an LDS-DMA ring this raised the sustained read rate of a plain
// streaming probe from ~5.65 to ~6.0 TB/s (one wave per SIMD) and from ~5.7 to
// ~6.4 TB/s (two per SIMD).  Where several workgroups of one XCD read the same
// K/V (the query tiles of a prefill pair), the default policy keeps it in L2.
#ifndef PGQA_KV_CPOL
#define PGQA_KV_CPOL 2
#endif

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land at
// lds_row + 16 * l (lds_row must be wave-uniform and 16-byte aligned).
__device__ __forceinline__ void load_lds_16(const void* gsrc, PGQA_LDS void* lds_row) {
    __builtin_amdgcn_global_load_lds(gsrc, lds_row, 16, 0, PGQA_KV_CPOL);
}

// Global->LDS DMA of 16 bytes per lane (global_load_lds_dwordx4): lane l
// copies 16 bytes from sbase + voff into LDS at lds + 16*l (M0 holds the
// wave's LDS base).  Written as inline assembly so that the compiler does not
// track the load: its own tracking makes later LDS reads wait for every DMA in
// flight, including the next tile's.  Callers wait for the DMA explicitly
// (s_waitcnt vmcnt); M0 is used for nothing else in the kernels that call it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Source sbase + voff (wave-uniform 64-bit base, 32-bit per-lane offset).  The
// base and LDS address are read from the first lane, which makes them scalar
// operands even where the compiler cannot prove them uniform.
// nt: non-temporal load (wave-uniform).
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, uint32_t lds, bool nt) {
    // readfirstlane returns a signed int: widen each half through uint32_t so
    // the low half is not sign-extended into the high one.
    const uint64_t p = (uint64_t)(uintptr_t)sbase;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint64_t s = ((uint64_t)hi << 32) | (uint64_t)lo;
    if (nt)
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"((const char*)s),
                     "s"(__builtin_amdgcn_readfirstlane(lds))
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"((const char*)s),
                     "s"(__builtin_amdgcn_readfirstlane(lds))
                     : "memory", "m0");
}
// 4 bytes per lane: lane l copies 4 bytes from sbase + voff into LDS at lds + 4*l.
__device__ __forceinline__ void dma4(const char* sbase, uint32_t voff, uint32_t lds, bool nt) {
    const uint64_t p = (uint64_t)(uintptr_t)sbase;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint64_t s = ((uint64_t)hi << 32) | (uint64_t)lo;
    if (nt)
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1 nt" ::"v"(voff), "s"((const char*)s),
                     "s"(__builtin_amdgcn_readfirstlane(lds))
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"((const char*)s),
                     "s"(__builtin_amdgcn_readfirstlane(lds))
                     : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N), leaving the other counters unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Runtime count in [0, MAXN]: branches to the constant-immediate wait.
template <int MAXN>
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
    if constexpr (MAXN <= 0) {
        wait_vmcnt<0>();
    } else {
        if (n >= MAXN) wait_vmcnt<MAXN>();
        else wait_vmcnt_dyn<MAXN - 1>(n);
    }
}

__device__ __forceinline__ u32x4 lds_read_16(const PGQA_LDS void* p) {
    return *(const PGQA_LDS u32x4*)p;
}

__device__ __forceinline__ u32x2 lds_read_8(const PGQA_LDS void* p) {
    return *(const PGQA_LDS u32x2*)p;
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

}  // namespace pgqa
