// The step before attention: rotary position embedding of a step's new
// tokens, and the write of their K/V into the static cache.
//
// tinydecode README ("What's in here": an in-place rope kernel; "how the
// decode step is put together": positions come from the device-resident
// lengths and the K/V write is an indexed store at those positions) and
// llm-decode-cuda's per-layer step list (rotation and cache write as one step).
//
// Token i of row b sits at position p = clamp(pos0[b], 0, S_max) + i. Pair j
// of a head (j < D/2) turns by the angle p * f_j, f_j = theta^(-2j/D), with
// the llama3 frequency scaling applied when asked; a pair (a, b) becomes
// (a cos - b sin, a sin + b cos). "half" pairs are (x_j, x_{j+D/2}),
// "adjacent" pairs (x_{2j}, x_{2j+1}). q is rotated into q_out (which may be
// q_in itself); k is rotated into the cache slot of its position and v copied
// there unchanged; a token at p >= S_max has no slot and writes no K/V.
//
// Angles and rotations are computed in fp64 (an angle p * f at p ~ 3e4 would
// carry ~2e-3 rad of error in fp32) and each result is rounded once to the
// nearest-even bf16. One workgroup per token: it computes the D/2 cos/sin
// pairs once into LDS, then its threads each rotate 8 pairs of one head (two
// 16-byte loads and stores) or copy 16 bytes of v.
#pragma once

#include "device_common.hpp"

namespace decattn {

struct RopeParams {
    const uint16_t* q_in;      // [B][T][Hq][D]
    const uint16_t* k_in;      // [B][T][Hkv][D]
    const uint16_t* v_in;      // [B][T][Hkv][D]
    const int32_t* pos0;       // [B]
    uint16_t* q_out;           // [B][T][Hq][D], may equal q_in
    uint16_t* k_cache;         // [B][Hkv][S_max][D]
    uint16_t* v_cache;         // [B][Hkv][S_max][D]
    int T, Hq, Hkv, S_max;
    int llama3;                // 1: apply the llama3 frequency scaling
    double theta;
    double factor, low_freq_factor, high_freq_factor, original_max_position;
};

constexpr int kRopeThreads = 256;
constexpr double kTwoPi = 6.283185307179586;   // 2 pi rounded to fp64

// Nearest-even bf16 of an fp64 value, rounded once: the binary32 conversion is
// made round-to-odd (truncate, then set the last bit when inexact), which
// keeps every bit the second rounding needs, and that binary32 is then
// rounded to nearest-even bf16.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double d) {
    const float f = (float)d;
    uint32_t u = __float_as_uint(f);
    const double back = (double)f;
    if (back != d && (u & 0x7F800000u) != 0x7F800000u) {
        if (fabs(back) > fabs(d)) u -= 1u;       // rounded away from zero: step back to the truncation
        u |= 1u;
    }
    return f32_to_bf16_rne(__uint_as_float(u));
}

// Frequency of pair j: theta^(-2j/D), then the llama3 scaling if asked (the
// wavelength 2 pi / f decides: below L / high_freq_factor kept, above
// L / low_freq_factor divided by the factor, in between a linear blend whose
// weight on the unscaled frequency grows with L / wavelength).
__device__ __forceinline__ double rope_frequency(const RopeParams& p, int j, int D) {
    double f = pow(p.theta, -(2.0 * j) / (double)D);
    if (p.llama3) {
        const double L = p.original_max_position;
        const double wavelen = kTwoPi / f;
        if (wavelen < L / p.high_freq_factor) {
            // high frequency: unchanged
        } else if (wavelen > L / p.low_freq_factor) {
            f = f / p.factor;
        } else {
            const double s = (L / wavelen - p.low_freq_factor) / (p.high_freq_factor - p.low_freq_factor);
            f = (1.0 - s) * f / p.factor + s * f;
        }
    }
    return f;
}

// ADJ selects the pairing: false = half, true = adjacent.
//
// Latency, not bandwidth, sets the time of this kernel (a decode step moves
// ~200 KB), so nothing waits on anything it does not need: the row's length,
// each thread's first two units of q/k/v and the pair frequencies (which do
// not depend on the position) are all in flight or in progress together, and
// only the sines and cosines wait for the length.
template <int D, bool ADJ>
__global__ void __launch_bounds__(kRopeThreads)
rope_kv_write_kernel(const RopeParams p) {
    static_assert(D % 16 == 0, "8 pairs per thread");
    constexpr int NP = D / 2;          // pairs per head
    constexpr int UPH = D / 16;        // rotation units (8 pairs) per head
    constexpr int VPH = D / 8;         // 16-byte pieces per head
    static_assert(NP <= kRopeThreads, "one thread per pair frequency");
    __shared__ double s_cos[NP];
    __shared__ double s_sin[NP];

    const int tok = blockIdx.x;        // b * T + i
    const int b = tok / p.T;
    const int i = tok - b * p.T;
    const int tid = threadIdx.x;

    const int nq = p.Hq * UPH;
    const int nk = p.Hkv * UPH;
    const int nv = p.Hkv * VPH;
    const int total = nq + nk + nv;

    // unit u: a q or k rotation unit (pairs 8t..8t+7 of one head: two 16-byte
    // pieces at element offsets o0, o1; half pairing takes 8 of the first half
    // and the 8 facing them, adjacent takes 16 in a row), or 16 bytes of v
    auto src_of = [&](int u, int& o0, int& o1) -> const uint16_t* {
        if (u >= nq + nk) {
            const int w = u - nq - nk;
            const int h = w / VPH;
            o0 = (w - h * VPH) * 8;
            o1 = o0;
            return p.v_in + ((size_t)tok * p.Hkv + h) * D;
        }
        const bool is_q = u < nq;
        const int w = is_q ? u : u - nq;
        const int h = w / UPH;
        const int t = w - h * UPH;
        o0 = ADJ ? 16 * t : 8 * t;
        o1 = ADJ ? 16 * t + 8 : NP + 8 * t;
        return is_q ? p.q_in + ((size_t)tok * p.Hq + h) * D : p.k_in + ((size_t)tok * p.Hkv + h) * D;
    };
    auto load_unit = [&](int u, uint4& x0, uint4& x1) {
        int o0, o1;
        const uint16_t* src = src_of(u, o0, o1);
        x0 = *reinterpret_cast<const uint4*>(src + o0);
        x1 = *reinterpret_cast<const uint4*>(src + o1);     // v: the same piece again (cache hit)
    };
    auto finish_unit = [&](int u, const uint4& x0, const uint4& x1, int pos, bool has_slot) {
        if (u >= nq + nk) {                                  // v: stored unchanged
            if (!has_slot) return;
            const int w = u - nq - nk;
            const int h = w / VPH;
            *reinterpret_cast<uint4*>(p.v_cache + (((size_t)b * p.Hkv + h) * p.S_max + pos) * D +
                                      (w - h * VPH) * 8) = x0;
            return;
        }
        const bool is_q = u < nq;
        if (!is_q && !has_slot) return;
        const int w = is_q ? u : u - nq;
        const int h = w / UPH;
        const int t = w - h * UPH;
        const int o0 = ADJ ? 16 * t : 8 * t;
        const int o1 = ADJ ? 16 * t + 8 : NP + 8 * t;
        uint16_t* dst = is_q ? p.q_out + ((size_t)tok * p.Hq + h) * D
                             : p.k_cache + (((size_t)b * p.Hkv + h) * p.S_max + pos) * D;
        float e[16];
        bf16x8_to_f32(x0, e);
        bf16x8_to_f32(x1, e + 8);
        uint16_t r[16];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            // pair 8t + m: (a, b) at (e[m], e[8 + m]) or (e[2m], e[2m + 1])
            const int ia = ADJ ? 2 * m : m;
            const int ib = ADJ ? 2 * m + 1 : 8 + m;
            const double a = e[ia], bb = e[ib];
            const double c = s_cos[8 * t + m], sn = s_sin[8 * t + m];
            r[ia] = f64_to_bf16_rne(a * c - bb * sn);
            r[ib] = f64_to_bf16_rne(a * sn + bb * c);
        }
        uint4 y0, y1;
        y0.x = r[0] | ((uint32_t)r[1] << 16);   y0.y = r[2] | ((uint32_t)r[3] << 16);
        y0.z = r[4] | ((uint32_t)r[5] << 16);   y0.w = r[6] | ((uint32_t)r[7] << 16);
        y1.x = r[8] | ((uint32_t)r[9] << 16);   y1.y = r[10] | ((uint32_t)r[11] << 16);
        y1.z = r[12] | ((uint32_t)r[13] << 16); y1.w = r[14] | ((uint32_t)r[15] << 16);
        *reinterpret_cast<uint4*>(dst + o0) = y0;
        *reinterpret_cast<uint4*>(dst + o1) = y1;
    };

    // first two units of this thread: loads in flight with the length's
    const int ua = tid, ub = tid + (int)blockDim.x;
    uint4 a0 = make_uint4(0, 0, 0, 0), a1 = a0, b0 = a0, b1 = a0;
    if (ua < total) load_unit(ua, a0, a1);
    if (ub < total) load_unit(ub, b0, b1);
    // the row's length as a vector load too: a scalar load would be waited
    // for on its own before the address arithmetic of the loads above
    const int len = (int)__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(p.pos0, (uint32_t)(b + 1) * 4u),
                                                               b * 4, 0, 0);
    const double f = tid < NP ? rope_frequency(p, tid, D) : 0.0;

    const int pos = clamp_len(len, p.S_max) + i;
    const bool has_slot = pos < p.S_max;
    if (tid < NP) {
        double sn, cs;
        sincos((double)pos * f, &sn, &cs);
        s_cos[tid] = cs;
        s_sin[tid] = sn;
    }
    __syncthreads();

    if (ua < total) finish_unit(ua, a0, a1, pos, has_slot);
    if (ub < total) finish_unit(ub, b0, b1, pos, has_slot);
    for (int u = tid + 2 * (int)blockDim.x; u < total; u += blockDim.x) {
        uint4 x0, x1;
        load_unit(u, x0, x1);
        finish_unit(u, x0, x1, pos, has_slot);
    }
}

}  // namespace decattn
