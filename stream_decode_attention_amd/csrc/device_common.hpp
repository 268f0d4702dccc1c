// Device helpers shared by the libdecattn kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace decattn {

constexpr float kNegInf = -__builtin_inff();

// bf16 holds the upper 16 bits of a binary32, so widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ void bf16x8_to_f32(const uint4 r, float f[8]) {
    f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x);
    f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
    f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z);
    f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
}

// Round binary32 to the nearest bf16, ties to even: add half an output step
// (minus one when the kept low bit is 0) and truncate. NaN maps to a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// One DPP lane move inside a 16-lane row, all rows and banks written. Every
// pattern used here (quad permutes, mirrors, rotations) gives each lane a
// source inside its row. dpp_move feeds an add, which the compiler fuses into
// one v_add_f32_dpp; dpp_copy is a bare move (v_mov_b32_dpp, no "old" value).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ float dpp_copy(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_copy_i(int x) {
    return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, false);
}

constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within each 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within each 16 lanes
constexpr int kDppRor8 = 0x128;       // lane i <- lane (i+8) mod 16

// Sum over aligned groups of N (8 or 16) lanes; every lane of a group ends with
// the same bits (each step adds a pair in both orders, and + commutes).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
    x += dpp_move<kDppXor1>(x);
    x += dpp_move<kDppXor2>(x);
    x += dpp_move<kDppHalfMirror>(x);
    if constexpr (N == 16) x += dpp_move<kDppMirror>(x);
    return x;
}

// Lane moves by XOR inside 32-lane halves (ds_swizzle bitmask mode: LDS
// crossbar, no LDS memory and no VALU slot).
template <int XOR>
__device__ __forceinline__ float swizzle_xor(float x) {
    static_assert(XOR > 0 && XOR < 32, "xor inside 32 lanes");
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x1F | (XOR << 10)));
}
template <int XOR>
__device__ __forceinline__ int swizzle_xor_i(int x) {
    return __builtin_amdgcn_ds_swizzle(x, 0x1F | (XOR << 10));
}

// gfx950 VALU lane swaps (no LDS traffic), as measured on the GPU:
// swap16(a, b) returns {[a.r0, b.r0, a.r2, b.r2], [a.r1, b.r1, a.r3, b.r3]}
// and swap32(a, b) returns {[a.lo, b.lo], [a.hi, b.hi]}, where r0..r3 are the
// 16-lane rows of a register and lo/hi its 32-lane halves. Adding the two
// results of swap16(a, b) gives rows 0/2 the pair sums of a's rows (0+1, 2+3)
// and rows 1/3 those of b; adding those of swap32(a, b) gives the lower half
// a.lo + a.hi and the upper half b.lo + b.hi.
struct f32x2 {
    float x, y;
};
__device__ __forceinline__ f32x2 swap16(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ f32x2 swap32(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Reduce across the 64/N lane groups of a wave (lanes with equal index inside
// their group), result in every lane. N = 8 or 16. The order of the additions
// is ((g0 + g1) + (g2 + g3)) over the 16-lane rows for every lane.
template <int N>
__device__ __forceinline__ float across_groups_sum(float x) {
    if constexpr (N == 8) x += dpp_move<kDppRor8>(x);
    const f32x2 a = swap16(x, x);
    x = a.x + a.y;
    const f32x2 b = swap32(x, x);
    return b.x + b.y;
}

template <int N>
__device__ __forceinline__ float across_groups_max(float x) {
    if constexpr (N == 8) x = fmaxf(x, dpp_move<kDppRor8>(x));
    const f32x2 a = swap16(x, x);
    x = fmaxf(a.x, a.y);
    const f32x2 b = swap32(x, x);
    return fmaxf(b.x, b.y);
}

// Reduce-scatter of M values (M a multiple of 4) across the 64/N lane groups:
// on return, every lane of 16-lane row q holds in out[m] the sum over all
// groups of v[4m + q], added in the same order as across_groups_sum.
template <int N, int M>
__device__ __forceinline__ void across_groups_sum_scatter(float (&v)[M], float (&out)[M / 4]) {
    static_assert(M % 4 == 0, "values come in fours");
    if constexpr (N == 8) {
#pragma unroll
        for (int j = 0; j < M; ++j) v[j] += dpp_move<kDppRor8>(v[j]);
    }
    float w[M / 2];
#pragma unroll
    for (int j = 0; j < M / 2; ++j) {       // rows 0,2: v[2j] pair sums; rows 1,3: v[2j+1]
        const f32x2 a = swap16(v[2 * j], v[2 * j + 1]);
        w[j] = a.x + a.y;
    }
#pragma unroll
    for (int m = 0; m < M / 4; ++m) {       // lower half: w[2m] halves summed, upper: w[2m+1]
        const f32x2 b = swap32(w[2 * m], w[2 * m + 1]);
        out[m] = b.x + b.y;
    }
}

// Sum of an int over the 64 lanes of a wave, in every lane: DPP moves inside
// each 16-lane row, then the row swaps (no LDS round trips, unlike a
// shuffle-based reduction).
__device__ __forceinline__ int wave_sum_i(int x) {
    x += dpp_copy_i<kDppXor1>(x);
    x += dpp_copy_i<kDppXor2>(x);
    x += dpp_copy_i<kDppHalfMirror>(x);
    x += dpp_copy_i<kDppMirror>(x);
    const auto a = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
    x = (int)(a[0] + a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
    return (int)(b[0] + b[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// acc + a.lo*b.lo + a.hi*b.hi on two packed bf16 pairs (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Raw buffer resource over [base, base + bytes): 16-byte loads at offsets at
// or past `bytes` return zeros, so rows past a length need no exec masking.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Cache-policy bits of a gfx950 buffer load: "nt" marks streaming data that
// is read once. On MI355X it lifts a pure streaming read from about 6.3 to
// about 7.1 TB/s (measured).
constexpr int kLoadStream = 2;

template <int POLICY>
__device__ __forceinline__ uint4 buffer_load16_policy(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POLICY);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return buffer_load16_policy<kLoadStream>(r, off);
}

__device__ __forceinline__ int clamp_len(int n, int s_max) {
    return n < 0 ? 0 : (n > s_max ? s_max : n);
}

// clamp(len + add, 0, s_max) with the sum taken in 64 bits: a device length
// near INT_MAX plus a token offset must clamp to s_max, not wrap negative.
__device__ __forceinline__ int clamp_len_add(int len, int add, int s_max) {
    const long long n = (long long)len + add;
    return n < 0 ? 0 : (n > s_max ? s_max : (int)n);
}

}  // namespace decattn
