// Log-sum-exp merge of the split-KV partial state: one workgroup per output row.
//
// For an output row with n attended keys, the first NA = ceil(n / chunk)
// tiles hold its partial state (m_c in log2 units, l_c, acc_c). The tiles are
// combined by rescaling each to a common maximum (the log-sum-exp merge of
// llm-decode-cuda's attention section):
//     M = max_c m_c,  w_c = 2^(m_c - M),
//     out = sum_c w_c acc_c / sum_c w_c l_c  (as a product with 1 / sum),
// then stored as fp32 or rounded to bf16. Rows with n = 0 store zeros.
//
// The partial state was written by another kernel; the loads of a batch of
// tiles are issued together (one round trip per batch), and the first batch
// before the row's length arrives. The code stays short and free of branches
// up to the first wait (a tile index past the workspace is clamped into it
// and its values dropped by a select), so the waves start their loads after
// few instruction fetches.
// Thread (cl, q4) owns 4 dims (one 16-byte load) of the tiles c = cl,
// cl + 8, ...; it folds them into a running (m, l, acc) with the same rule;
// the tile lanes of a wave are joined by lane swaps and the waves (2 or 4)
// through LDS, each in a fixed order, so the result does not depend on
// scheduling.
#pragma once

#include <type_traits>

#include "device_common.hpp"

namespace decattn {

// Arguments the first loads depend on come first, as scalars, so that they
// can be preloaded into SGPRs at wave launch; the rest arrive by a scalar load
// from the kernel-argument segment while the first loads are in flight.
struct MergeParams {
    void* out;              // [B][T][Hq][D]
    int out_bf16;
    int T, S_max, chunk, causal;
};

// Threads per row: 256, tile lanes of D / 4 threads (16 lanes at D = 64, 8
// at D = 128), each loading up to 8 tiles per batch. Measured on MI355X: at
// D = 128 this is about 0.2 us faster per call than 512 threads of 4 tiles
// (fewer waves to start and to join through LDS) and than 128 threads of 8;
// at D = 64 it is 0.08 us faster than 128 threads on 64-tile rows.
// One wave of 16 tiles per thread (no LDS join) took 0.4 us longer on short
// calls and 1.5 us longer on a 32-tile row: its 48 loads issue one after
// another from one wave.
__host__ __device__ constexpr int merge_threads(int) { return 256; }
constexpr int kMergeUnroll = 8;

// ws_ml [B][Hkv][NC][RT][2], ws_acc [B][Hkv][NC][RT][D], lens [B]; one
// workgroup per output row, grid (Hkv, T * G, B). NU0: slots of the first batch,
// ceil(NC / tile lanes) rounded up to 1, 2, 4 or 8 by the host (a slot past
// every row's tiles loads a clamped duplicate that the select drops), so that
// the first batch is straight-line code. NWT: waves per row, 4, or one
// when one wave's tile lanes (64 / (D / 4)) hold every tile slot; it then
// needs no join through LDS and no barrier.
template <int D, int NU0, int NWT>
__global__ void __launch_bounds__(64 * NWT)
lse_merge(const float* ws_ml_, const float* ws_acc_, const int32_t* lens, int G, int Hkv, int NC, int RT,
          uint32_t g_recip, const MergeParams p) {
    constexpr int QPR = D / 4;                    // float4 quads per row
    constexpr int kMergeThreads = 64 * NWT;
    constexpr int NCL = kMergeThreads / QPR;      // tile lanes working in parallel
    __shared__ float4 s_acc[kMergeThreads / 64][QPR];
    __shared__ float s_m[kMergeThreads / 64];
    __shared__ float s_l[kMergeThreads / 64];

    // the kv head is the fastest grid dimension, as in the one-round partial
    // grids, so a row is merged on the XCD that wrote its tiles when Hkv is
    // a multiple of 8
    const int kvh = blockIdx.x, r = blockIdx.y, b = blockIdx.z;

    const size_t head0 = (size_t)(b * Hkv + kvh) * NC * RT;   // tile 0, row 0
    const float* ml = ws_ml_ + head0 * 2;
    const float* accp = ws_acc_ + head0 * D;
    const int tid = threadIdx.x;
    const int q4 = tid % QPR;
    const int cl = tid / QPR;

    // tiles c0, c0 + NCL, ...: every load lands inside the workspace (tile
    // index clamped to NC - 1); which of them count is decided by a select
    // once the row's tile count is known
    float mv[kMergeUnroll], lv[kMergeUnroll];
    float4 av[kMergeUnroll];
    // slots u < nu are loaded (nu is uniform); the others stay empty
    auto fetch = [&](int c0, int nu) {
#pragma unroll
        for (int u = 0; u < kMergeUnroll; ++u) {
            if (u < nu) {
                const int c = min(c0 + u * NCL, NC - 1);
                const size_t tr = (size_t)c * RT + r;
                const float2 x = *reinterpret_cast<const float2*>(ml + tr * 2);
                mv[u] = x.x;
                lv[u] = x.y;
                av[u] = *reinterpret_cast<const float4*>(accp + tr * D + q4 * 4);
            } else {
                mv[u] = kNegInf;
                lv[u] = 0.f;
                av[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    };
    // the first batch: only slots that can hold a tile of the workspace (a
    // slot u past ceil(NC / NCL) lies past every row's tiles)
    static_assert(NU0 >= 1 && NU0 <= kMergeUnroll, "first-batch slots");
    fetch(cl, NU0);
    // keep those loads ahead of the length's: without this the compiler
    // moves the exit test for an empty row (and the length's round trip)
    // above them
    asm volatile("" ::: "memory");

    const int len = lens[b];
    // query token i = r / G as a multiply-high by g_recip = ceil(2^32 / G)
    // (exact for r < 2^28, G <= 8); for G = 1 the host passes 0 and the
    // select adds r
    const int i = (int)__umulhi((uint32_t)r, g_recip) + (g_recip == 0u ? r : 0);
    const int h = kvh * G + (r - i * G);
    const int n = clamp_len_add(len, p.causal ? i + 1 : 0, p.S_max);
    int na = (n + p.chunk - 1) >> __builtin_ctz(p.chunk);   // chunk is a power of two
    na = na < NC ? na : NC;
    const size_t row = ((size_t)b * p.T + i) * (size_t)(Hkv * G) + h;   // (b, i, h) flattened

    if (na == 0) {
#pragma unroll
        for (int d = tid; d < D; d += kMergeThreads) {
            if (p.out_bf16) reinterpret_cast<uint16_t*>(p.out)[row * D + d] = 0;
            else reinterpret_cast<float*>(p.out)[row * D + d] = 0.f;
        }
        return;
    }

    float m_t = kNegInf, l_t = 0.f;
    float4 a_t = make_float4(0.f, 0.f, 0.f, 0.f);
    // fold slots u < NU of the batch at c0 into (m_t, l_t, a_t)
    auto fold = [&](int c0, auto nu_tag) {
        constexpr int NU = decltype(nu_tag)::value;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            if (c0 + u * NCL >= na) {       // not this row's tile: drop (select, no arithmetic)
                mv[u] = kNegInf;
                lv[u] = 0.f;
                av[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        float mb = mv[0];
#pragma unroll
        for (int u = 1; u < NU; ++u) mb = fmaxf(mb, mv[u]);
        // An empty tile state (m = -inf, l = 0, acc = 0) adds nothing: while this
        // lane has seen only such tiles its maximum stays -inf and the weights
        // are taken against 0, which makes them all 0 (never 2^(-inf + inf)).
        const float m_new = fmaxf(m_t, mb);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float sc = fast_exp2(m_t - m_use);
        l_t *= sc;
        a_t.x *= sc; a_t.y *= sc; a_t.z *= sc; a_t.w *= sc;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const float wt = fast_exp2(mv[u] - m_use);
            l_t = __builtin_fmaf(wt, lv[u], l_t);
            a_t.x = __builtin_fmaf(wt, av[u].x, a_t.x);
            a_t.y = __builtin_fmaf(wt, av[u].y, a_t.y);
            a_t.z = __builtin_fmaf(wt, av[u].z, a_t.z);
            a_t.w = __builtin_fmaf(wt, av[u].w, a_t.w);
        }
        m_t = m_new;
    };
    if constexpr (NU0 < kMergeUnroll) {
        // NU0 * NCL slots cover the workspace's NC tiles: one batch, NU0 slots
        fold(cl, std::integral_constant<int, NU0>{});
    } else {
        for (int c0 = cl; c0 < na; c0 += NCL * kMergeUnroll) {
            if (c0 != cl) fetch(c0, kMergeUnroll);
            fold(c0, std::integral_constant<int, kMergeUnroll>{});
        }
    }
    // Tile lanes of one wave (4 at D = 64 in its 16-lane rows, 2 at D = 128 in
    // its halves) are joined with lane swaps, in the same order for every
    // lane; then the waves' states are joined through LDS in wave order.
    auto join = [&](const f32x2& mm, const f32x2& ll, const f32x2& ax, const f32x2& ay, const f32x2& az,
                    const f32x2& aw) {
        // the two states (m, l, acc) in .x and .y; an empty state (m = -inf)
        // adds nothing, and two empty states stay empty
        const float M = fmaxf(mm.x, mm.y);
        const float mu = (M == kNegInf) ? 0.f : M;
        const float w0 = fast_exp2(mm.x - mu), w1 = fast_exp2(mm.y - mu);
        m_t = M;
        l_t = __builtin_fmaf(w1, ll.y, w0 * ll.x);
        a_t.x = __builtin_fmaf(w1, ax.y, w0 * ax.x);
        a_t.y = __builtin_fmaf(w1, ay.y, w0 * ay.x);
        a_t.z = __builtin_fmaf(w1, az.y, w0 * az.x);
        a_t.w = __builtin_fmaf(w1, aw.y, w0 * aw.x);
    };
    if constexpr (QPR == 16) {              // rows r and r ^ 1 of the wave
        join(swap16(m_t, m_t), swap16(l_t, l_t), swap16(a_t.x, a_t.x), swap16(a_t.y, a_t.y),
             swap16(a_t.z, a_t.z), swap16(a_t.w, a_t.w));
    }
    join(swap32(m_t, m_t), swap32(l_t, l_t), swap32(a_t.x, a_t.x), swap32(a_t.y, a_t.y), swap32(a_t.z, a_t.z),
         swap32(a_t.w, a_t.w));
    constexpr int NW = kMergeThreads / 64;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    if constexpr (NW == 1) {
        // every lane holds the row's state: lanes < QPR store their 4 dims
        if (tid < QPR) {
            const float inv = 1.f / l_t;
            const float o0 = a_t.x * inv, o1 = a_t.y * inv, o2 = a_t.z * inv, o3 = a_t.w * inv;
            const size_t o = row * D + tid * 4;
            if (p.out_bf16) {
                uint16_t* ob = reinterpret_cast<uint16_t*>(p.out) + o;
                const uint2 packed = make_uint2(
                    (uint32_t)f32_to_bf16_rne(o0) | ((uint32_t)f32_to_bf16_rne(o1) << 16),
                    (uint32_t)f32_to_bf16_rne(o2) | ((uint32_t)f32_to_bf16_rne(o3) << 16));
                *reinterpret_cast<uint2*>(ob) = packed;
            } else {
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + o) = make_float4(o0, o1, o2, o3);
            }
        }
        return;
    }
    if (lane < QPR) {
        s_acc[wave][lane] = a_t;
        if (lane == 0) {
            s_m[wave] = m_t;
            s_l[wave] = l_t;
        }
    }
    __syncthreads();

    if (tid < QPR) {
        float M = s_m[0];
#pragma unroll
        for (int k = 1; k < NW; ++k) M = fmaxf(M, s_m[k]);
        float L = 0.f;
        float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int k = 0; k < NW; ++k) {
            const float wt = fast_exp2(s_m[k] - M);    // waves with no tile: 2^-inf = 0
            const float4 u = s_acc[k][tid];
            L = __builtin_fmaf(wt, s_l[k], L);
            t.x = __builtin_fmaf(wt, u.x, t.x);
            t.y = __builtin_fmaf(wt, u.y, t.y);
            t.z = __builtin_fmaf(wt, u.z, t.z);
            t.w = __builtin_fmaf(wt, u.w, t.w);
        }
        // one correctly rounded reciprocal and four products (one more
        // rounding than four divisions, far inside the fp32 tolerance; about
        // 0.08 us less per call than four IEEE divisions)
        const float inv = 1.f / L;
        const float o0 = t.x * inv, o1 = t.y * inv, o2 = t.z * inv, o3 = t.w * inv;
        const size_t o = row * D + tid * 4;
        if (p.out_bf16) {
            uint16_t* ob = reinterpret_cast<uint16_t*>(p.out) + o;
            const uint2 packed = make_uint2(
                (uint32_t)f32_to_bf16_rne(o0) | ((uint32_t)f32_to_bf16_rne(o1) << 16),
                (uint32_t)f32_to_bf16_rne(o2) | ((uint32_t)f32_to_bf16_rne(o3) << 16));
            *reinterpret_cast<uint2*>(ob) = packed;
        } else {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + o) = make_float4(o0, o1, o2, o3);
        }
    }
}

}  // namespace decattn
