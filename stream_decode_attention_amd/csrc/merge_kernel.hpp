// Log-sum-exp merge of the split-KV partial state: one workgroup per output row.
//
// For an output row with n attended keys, the first NA = ceil(n / chunk)
// tiles hold its partial state (m_c in log2 units, l_c, acc_c). The merge
// (llm-decode-cuda, attention section: "merges the chunks with the log-sum-exp
// trick") is
//     M = max_c m_c,  w_c = 2^(m_c - M),
//     out = sum_c w_c acc_c / sum_c w_c l_c,
// then stored as fp32 or rounded to bf16. Rows with n = 0 store zeros.
//
// 256 threads: each handles 4 consecutive dims (one 16-byte load of acc) of a
// strided subset of the tiles; the per-thread sums are then added in a fixed
// order through LDS, so the result does not depend on scheduling.
#pragma once

#include "device_common.hpp"

namespace decattn {

struct MergeParams {
    const float* ws_ml;     // [B][Hkv][NC][RT][2]
    const float* ws_acc;    // [B][Hkv][NC][RT][D]
    const int32_t* lens;    // [B]
    void* out;              // [B][T][Hq][D]
    int out_bf16;
    int T, Hq, Hkv, G, S_max, chunk, NC, RT, causal;
};

constexpr int kMergeThreads = 256;

template <int D>
__global__ void __launch_bounds__(kMergeThreads)
lse_merge(const MergeParams p) {
    constexpr int QPR = D / 4;                    // float4 quads per row
    constexpr int NCL = kMergeThreads / QPR;      // tile lanes working in parallel
    __shared__ float s_red[kMergeThreads / 64];
    __shared__ float4 s_acc[NCL][QPR];
    __shared__ float s_l[NCL];

    const int row = blockIdx.x;                   // (b, i, h) flattened
    const int b = row / (p.T * p.Hq);
    const int rem = row - b * p.T * p.Hq;
    const int i = rem / p.Hq;
    const int h = rem - i * p.Hq;
    const int kvh = h / p.G;
    const int r = i * p.G + (h - kvh * p.G);

    const int len = p.lens[b];
    const int n = clamp_len(p.causal ? len + i + 1 : len, p.S_max);
    int na = (n + p.chunk - 1) / p.chunk;
    na = na < p.NC ? na : p.NC;

    const int tid = threadIdx.x;
    if (na == 0) {
        if (tid < D) {
            if (p.out_bf16) reinterpret_cast<uint16_t*>(p.out)[(size_t)row * D + tid] = 0;
            else reinterpret_cast<float*>(p.out)[(size_t)row * D + tid] = 0.f;
        }
        return;
    }

    const size_t head0 = (size_t)(b * p.Hkv + kvh) * p.NC * p.RT;   // tile 0, row 0
    const float* ml = p.ws_ml + head0 * 2;
    const float* accp = p.ws_acc + head0 * D;

    // pass 1: M = max over the row's tiles
    float mx = kNegInf;
    for (int c = tid; c < na; c += kMergeThreads) mx = fmaxf(mx, ml[((size_t)c * p.RT + r) * 2]);
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    mx = fmaxf(mx, __shfl_xor(mx, 4));
    mx = fmaxf(mx, __shfl_xor(mx, 8));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if ((tid & 63) == 0) s_red[tid >> 6] = mx;
    __syncthreads();
    float M = s_red[0];
#pragma unroll
    for (int w = 1; w < kMergeThreads / 64; ++w) M = fmaxf(M, s_red[w]);

    // pass 2: weighted sums
    const int q4 = tid % QPR;
    const int cl = tid / QPR;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    float l = 0.f;
    for (int c = cl; c < na; c += NCL) {
        const size_t tr = (size_t)c * p.RT + r;
        const float wt = fast_exp2(ml[tr * 2] - M);
        l = __builtin_fmaf(wt, ml[tr * 2 + 1], l);
        const float4 x = *reinterpret_cast<const float4*>(accp + tr * D + q4 * 4);
        a.x = __builtin_fmaf(wt, x.x, a.x);
        a.y = __builtin_fmaf(wt, x.y, a.y);
        a.z = __builtin_fmaf(wt, x.z, a.z);
        a.w = __builtin_fmaf(wt, x.w, a.w);
    }
    s_acc[cl][q4] = a;
    if (q4 == 0) s_l[cl] = l;
    __syncthreads();

    if (cl == 0) {
        float4 t = s_acc[0][q4];
        float L = s_l[0];
#pragma unroll
        for (int k = 1; k < NCL; ++k) {
            const float4 u = s_acc[k][q4];
            t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
            L += s_l[k];
        }
        const float o0 = t.x / L, o1 = t.y / L, o2 = t.z / L, o3 = t.w / L;
        const size_t o = (size_t)row * D + q4 * 4;
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
