// Speculative decoding's accept/reject step with the rollback of the cache
// lengths, on the device (tinydecode README, "speculative decoding": keep a
// draft with probability min(1, p_t / p_d), take the extra token from the
// residual (p_t - p_d)+ at the first rejection or from the bonus row, greedy
// keeps drafts while they equal the argmax, rollback only moves the length;
// FlashSpec page, correctness paragraph: Leviathan et al. 2023, Algorithm 1,
// the test taken in log space).
//
// Launches, no host sync:
//   spec_stats_kernel   one workgroup per (row b, position i, vocabulary
//                       chunk): the chunk's max logit and sum of
//                       exp2((l - max) * log2(e) / tau), or for greedy its
//                       largest logit and first index of it;
//   spec_finish_kernel  per (row b, chunk): every workgroup merges the chunk
//                       statistics of all positions of its row (the same
//                       instructions on the same data, so every workgroup of
//                       the row reaches the same bits) and takes the accept
//                       decisions; it then sums the residual weights of its
//                       chunk for the first rejected position (or p of the
//                       bonus row). Greedy needs no residual, so its finish is
//                       one workgroup per row and writes the result itself;
//   spec_select_kernel  (sampling) one workgroup per row: scans the chunk sums
//                       in index order, rescans the one chunk that holds the
//                       draw, and writes the accept count, the token and the
//                       new length.
// Each kernel only reads what earlier launches wrote, so the kernel
// boundaries order every exchange: no atomics, fences or counters.
#pragma once

#include <climits>

#include "device_common.hpp"

namespace decattn {

constexpr int kSpecThreads = 256;
constexpr int kSpecWaves = kSpecThreads / 64;
constexpr int kSpecSeg = kSpecThreads * 4;    // elements per segment: one float4 per thread
constexpr int kSpecMaxT = 32;                 // gamma + 1 positions: one ballot decides them all
constexpr int kSpecStage = 4096;              // chunk statistics staged in LDS at once (float2)


struct SpecParams {
    const float* logits;      // [B][T][V]
    const float* q;           // [B][T-1][V]  (sampling only)
    const int32_t* drafts;    // [B][T-1]
    const float* u;           // [B][T-1]     (sampling only)
    const float* r;           // [B]          (sampling only)
    int32_t* lens;            // [B] in: length before the verify pass; out: after the rollback
    int32_t* result;          // [B][2]: accepted drafts, next token
    float2* stats;            // [B][T][NC]
    float2* parts;            // [B][NC]
    float4* rowinfo;          // [B]: max and 1/sum of the drawing position's softmax, accept count
    float4* dinfo;            // [B][T-1]: each draft's target logit, q and u, and its id (sampling)
    float c2;                 // log2(e) / tau
    int T, V, NC, S_max;
};

// Chunk element (j, e) of thread t has vocabulary index c0 + j*kSpecSeg + 4t + e:
// each segment j is one coalesced float4 read by the workgroup. Indices at or
// past V read as `fill`.
template <int U, bool VEC>
__device__ __forceinline__ void spec_load(const float* __restrict__ row, int V, int c0, float fill,
                                          float (&x)[4 * U]) {
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const int e0 = c0 + j * kSpecSeg + 4 * t;
        if constexpr (VEC) {
            float4 v = make_float4(fill, fill, fill, fill);
            if (e0 < V) v = *reinterpret_cast<const float4*>(row + e0);     // V % 4 == 0 here
            x[4 * j] = v.x; x[4 * j + 1] = v.y; x[4 * j + 2] = v.z; x[4 * j + 3] = v.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * j + e] = e0 + e < V ? row[e0 + e] : fill;
        }
    }
}

// (v, i) beats (bv, bi): larger value, or the same value at a smaller index.
// INT_MAX marks "no element yet", which anything in range beats.
__device__ __forceinline__ bool spec_better(float v, int i, float bv, int bi) {
    return bi == INT_MAX ? i != INT_MAX : (v > bv || (v == bv && i < bi));
}

__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (spec_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

// Butterfly sum: every lane ends with the same bits.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// Inclusive prefix sum over the wave. Shuffles read the source lane's
// register only while that lane is active, so every lane must execute them.
__device__ __forceinline__ float wave_incl_scan(float x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_up(x, d);
        if (lane >= d) x += o;
    }
    return x;
}

// Rescale a partial sum s taken relative to max m onto the max M >= m.
__device__ __forceinline__ float spec_rescale(float s, float m, float M, float c2) {
    return m == kNegInf ? 0.f : s * fast_exp2((m - M) * c2);
}

// The weight of one vocabulary entry in the final draw: the residual
// max(0, p - q), or p itself (bonus row, or a residual with no positive mass).
__device__ __forceinline__ float spec_weight(float l, float qv, float M, float c2, float inv_s, bool use_p) {
    const float pk = fast_exp2((l - M) * c2) * inv_s;
    return use_p ? pk : fmaxf(pk - qv, 0.f);
}

template <int U, bool VEC, bool GREEDY>
__global__ __launch_bounds__(kSpecThreads) void spec_stats_kernel(const SpecParams p) {
    const int c = blockIdx.x % p.NC;
    const int row = blockIdx.x / p.NC;               // b * T + i
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int c0 = c * (U * kSpecSeg);
    float x[4 * U];
    spec_load<U, VEC>(p.logits + (size_t)row * p.V, p.V, c0, kNegInf, x);
    __shared__ float sh_v[kSpecWaves], sh_s[kSpecWaves];
    __shared__ int sh_i[kSpecWaves];
    if constexpr (GREEDY) {
        float bv = kNegInf;
        int bi = INT_MAX;
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int idx = c0 + j * kSpecSeg + 4 * t + e;
                if (idx < p.V && (bi == INT_MAX || x[4 * j + e] > bv)) { bv = x[4 * j + e]; bi = idx; }
            }
        wave_argmax(bv, bi);
        if (lane == 0) { sh_v[w] = bv; sh_i[w] = bi; }
        __syncthreads();
        if (t == 0) {
            bv = sh_v[0]; bi = sh_i[0];
            for (int k = 1; k < kSpecWaves; ++k)
                if (spec_better(sh_v[k], sh_i[k], bv, bi)) { bv = sh_v[k]; bi = sh_i[k]; }
            p.stats[(size_t)row * p.NC + c] = make_float2(bv, __int_as_float(bi));
        }
    } else {
        float m = kNegInf;
#pragma unroll
        for (int k = 0; k < 4 * U; ++k) m = fmaxf(m, x[k]);
        float s = 0.f;
        if (m != kNegInf) {
#pragma unroll
            for (int k = 0; k < 4 * U; ++k) s += fast_exp2((x[k] - m) * p.c2);
        }
        // the workgroup whose chunk holds draft i's token records that token's
        // logit, q and u for the decision (row 0 of the chunk holds the id of
        // a draft outside the vocabulary)
        const int gamma = p.T - 1, i = row % p.T, b = row / p.T;
        if (i < gamma) {
            const int d = p.drafts[(size_t)b * gamma + i];
            const int li = d - c0;
            if (d >= 0 && d < p.V && li < U * kSpecSeg && li >= 0 && (li % kSpecSeg) / 4 == t) {
                float ld = 0.f;
#pragma unroll
                for (int k = 0; k < 4 * U; ++k)
                    if (k == 4 * (li / kSpecSeg) + li % 4) ld = x[k];
                const size_t di = (size_t)b * gamma + i;
                p.dinfo[di] = make_float4(ld, p.q[di * p.V + d], p.u[di], __int_as_float(d));
            } else if ((d < 0 || d >= p.V) && c == 0 && t == 0) {
                p.dinfo[(size_t)b * gamma + i] = make_float4(0.f, 0.f, 0.f, __int_as_float(d));
            }
        }
        const float M = wave_max(m);
        s = wave_sum(spec_rescale(s, m, M, p.c2));
        if (lane == 0) { sh_v[w] = M; sh_s[w] = s; }
        __syncthreads();
        if (t == 0) {
            float Mb = sh_v[0];
            for (int k = 1; k < kSpecWaves; ++k) Mb = fmaxf(Mb, sh_v[k]);
            float Sb = 0.f;
            for (int k = 0; k < kSpecWaves; ++k) Sb += spec_rescale(sh_s[k], sh_v[k], Mb, p.c2);
            p.stats[(size_t)row * p.NC + c] = make_float2(Mb, Sb);
        }
    }
}

__device__ __forceinline__ int spec_new_len(int ctx, int n, int s_max) {
    const long long v = (long long)clamp_len(ctx, s_max) + n + 1;
    return v > s_max ? s_max : (int)v;
}

template <int U, bool VEC, bool GREEDY>
__global__ __launch_bounds__(kSpecThreads) void spec_finish_kernel(const SpecParams p) {
    constexpr int CH = U * kSpecSeg;
    const int NCB = GREEDY ? 1 : p.NC;
    const int c = blockIdx.x % NCB, b = blockIdx.x / NCB;
    const int T = p.T, gamma = T - 1, V = p.V;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    __shared__ float row_m[kSpecMaxT], row_s[kSpecMaxT];
    __shared__ int row_i[kSpecMaxT];
    __shared__ int sh_n;

    // the draft side of each position (threads t < gamma, all in wave 0):
    // its token id and, for sampling, the target logit, q and u at that id
    // as the first kernel recorded them
    int d = -1;
    float ld = 0.f, qd = 0.f, ud = 0.f;
    if (t < gamma) {
        if constexpr (GREEDY) {
            d = p.drafts[(size_t)b * gamma + t];
        } else {
            const float4 di = p.dinfo[(size_t)b * gamma + t];
            ld = di.x; qd = di.y; ud = di.z;
            d = __float_as_int(di.w);
        }
    }

    // merge the chunk statistics of every position: stage tiles of whole
    // positions in LDS (one batch of loads), then one wave per position
    __shared__ float2 st_lds[kSpecStage];
    const int NC = p.NC;
    const int rpt = kSpecStage / NC;                  // NC <= kSpecStage / 2
    for (int i0 = 0; i0 < T; i0 += rpt) {
        const int nr = T - i0 < rpt ? T - i0 : rpt;
        const float2* src = p.stats + ((size_t)b * T + i0) * NC;
#pragma unroll 4
        for (int e = t; e < nr * NC; e += kSpecThreads) st_lds[e] = src[e];
        __syncthreads();
        for (int i = i0 + w; i < i0 + nr; i += kSpecWaves) {
            const float2* st = st_lds + (size_t)(i - i0) * NC;
            if constexpr (GREEDY) {
                float bv = kNegInf;
                int bi = INT_MAX;
                for (int k = lane; k < NC; k += 64) {
                    const float2 v = st[k];
                    const int vi = __float_as_int(v.y);
                    if (spec_better(v.x, vi, bv, bi)) { bv = v.x; bi = vi; }
                }
                wave_argmax(bv, bi);
                if (lane == 0) row_i[i] = bi;
            } else {
                float m = kNegInf, s = 0.f;
                for (int k = lane; k < NC; k += 64) {
                    const float2 v = st[k];
                    const float M2 = fmaxf(m, v.x);
                    s = spec_rescale(s, m, M2, p.c2) + spec_rescale(v.y, v.x, M2, p.c2);
                    m = M2;
                }
                const float M = wave_max(m);
                s = wave_sum(spec_rescale(s, m, M, p.c2));
                if (lane == 0) { row_m[i] = M; row_s[i] = s; }
            }
        }
        __syncthreads();
    }

    // keep draft i iff log2 u_i < log2 p_i(d_i) - log2 q_i(d_i) (greedy: d_i is
    // the argmax); n = the first position not kept, or gamma
    if (w == 0) {
        bool keep = false;
        if (lane < gamma && d >= 0 && d < V) {
            if constexpr (GREEDY) {
                keep = d == row_i[lane];
            } else {
                const float lp = (ld - row_m[lane]) * p.c2 - log2f(row_s[lane]);
                keep = log2f(ud) < lp - log2f(qd);
            }
        }
        const unsigned long long rej = __ballot(lane < gamma && !keep);
        if (lane == 0) sh_n = rej ? __ffsll(rej) - 1 : gamma;
    }
    __syncthreads();
    const int n = sh_n;

    if constexpr (GREEDY) {
        if (t == 0) {
            p.result[2 * (size_t)b] = n;
            p.result[2 * (size_t)b + 1] = row_i[n];
            p.lens[b] = spec_new_len(p.lens[b], n, p.S_max);
        }
        return;
    } else {
        const float M = row_m[n];
        const float inv_s = 1.0f / row_s[n];
        const bool bonus = n == gamma;
        const float* lrow = p.logits + ((size_t)b * T + n) * V;
        const float* qrow = bonus ? nullptr : p.q + ((size_t)b * gamma + n) * V;

        // this chunk's residual mass and p mass, summed in a fixed order
        {
            float x[4 * U], y[4 * U];
            spec_load<U, VEC>(lrow, V, c * CH, kNegInf, x);
            if (bonus) {
#pragma unroll
                for (int k = 0; k < 4 * U; ++k) y[k] = 0.f;
            } else {
                spec_load<U, VEC>(qrow, V, c * CH, 0.f, y);
            }
            float ws = 0.f, ps = 0.f;
#pragma unroll
            for (int k = 0; k < 4 * U; ++k) {
                ws += spec_weight(x[k], y[k], M, p.c2, inv_s, bonus);
                ps += spec_weight(x[k], 0.f, M, p.c2, inv_s, true);
            }
            ws = wave_sum(ws);
            ps = wave_sum(ps);
            __shared__ float sh_w[kSpecWaves], sh_p[kSpecWaves];
            if (lane == 0) { sh_w[w] = ws; sh_p[w] = ps; }
            __syncthreads();
            if (t == 0) {
                float a = 0.f, e = 0.f;
                for (int k = 0; k < kSpecWaves; ++k) { a += sh_w[k]; e += sh_p[k]; }
                p.parts[(size_t)b * p.NC + c] = make_float2(a, e);
            }
        }

        if (c == 0 && t == 0) p.rowinfo[b] = make_float4(M, inv_s, __int_as_float(n), 0.f);
    }
}

template <int U, bool VEC>
__global__ __launch_bounds__(kSpecThreads) void spec_select_kernel(const SpecParams p) {
    constexpr int CH = U * kSpecSeg;
    const int b = blockIdx.x;
    const int T = p.T, gamma = T - 1, V = p.V;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const float4 info = p.rowinfo[b];
    const float M = info.x, inv_s = info.y;
    const int n = __float_as_int(info.z);
    const bool bonus = n == gamma;
    const float* lrow = p.logits + ((size_t)b * T + n) * V;
    const float* qrow = bonus ? nullptr : p.q + ((size_t)b * gamma + n) * V;

    // which chunk holds the draw: running sums over chunks in index order,
    // from the chunk sums staged in LDS
    __shared__ int sh_c, sh_mode, sh_use_p;
    __shared__ float sh_t, sh_base;
    __shared__ float2 pr[kSpecStage / 2];
    {
        const float2* src = p.parts + (size_t)b * p.NC;
#pragma unroll 4
        for (int e = t; e < p.NC; e += kSpecThreads) pr[e] = src[e];
    }
    __syncthreads();
    if (w == 0) {
        float tw = 0.f, tp = 0.f;                     // totals, by the same scan as below
        for (int k0 = 0; k0 < p.NC; k0 += 64) {
            const int k = k0 + lane;
            const float2 v = k < p.NC ? pr[k] : make_float2(0.f, 0.f);
            tw += __shfl(wave_incl_scan(v.x), 63);
            tp += __shfl(wave_incl_scan(v.y), 63);
        }
        const bool use_p = bonus || !(tw > 0.f);
        const float total = use_p ? tp : tw;
        const float thr = p.r[b] * total;
        int found = -1, last_pos = -1;
        float base = 0.f, carry = 0.f;
        for (int k0 = 0; k0 < p.NC; k0 += 64) {
            const int k = k0 + lane;
            const float2 v2 = k < p.NC ? pr[k] : make_float2(0.f, 0.f);
            const float v = use_p ? v2.y : v2.x;
            const float inc = wave_incl_scan(v);
            const float cum = carry + inc;
            const float up = __shfl_up(inc, 1);          // every lane takes part in the shuffle
            const float excl = carry + (lane ? up : 0.f);
            const unsigned long long hit = __ballot(k < p.NC && v > 0.f && cum > thr);
            if (hit) {
                const int L = __ffsll(hit) - 1;
                found = k0 + L;
                base = __shfl(excl, L);
                break;
            }
            const unsigned long long pos = __ballot(k < p.NC && v > 0.f);
            if (pos) last_pos = k0 + 63 - __clzll(pos);
            carry += __shfl(inc, 63);
        }
        if (lane == 0) {
            sh_use_p = use_p;
            sh_t = thr;
            sh_base = base;
            // 0: first entry whose running sum passes thr; 1: rounding left
            // thr at or past the total, take the last positive entry;
            // 2: no positive weight at all (rows that break the input rules)
            sh_mode = found >= 0 ? 0 : (last_pos >= 0 ? 1 : 2);
            sh_c = found >= 0 ? found : (last_pos >= 0 ? last_pos : 0);
        }
    }
    __syncthreads();

    // rescan the chosen chunk: its weights into LDS in index order; thread t
    // then owns the run of R consecutive entries [tR, tR + R), adds the
    // running sum of the runs before it to the chunk's base, and walks its
    // run; the first entry (smallest index) whose running sum passes thr wins
    constexpr int R = CH / kSpecThreads;
    __shared__ __attribute__((aligned(16))) float wbuf[CH];
    __shared__ int sh_lastpos, sh_pick;
    __shared__ float sh_wtot[kSpecWaves];
    if (t == 0) { sh_lastpos = -1; sh_pick = INT_MAX; }
    __syncthreads();
    const int cs = sh_c, mode = sh_mode;
    const bool use_p = sh_use_p;
    {
        float x[4 * U], y[4 * U];
        spec_load<U, VEC>(lrow, V, cs * CH, kNegInf, x);
        if (bonus) {
#pragma unroll
            for (int k = 0; k < 4 * U; ++k) y[k] = 0.f;
        } else {
            spec_load<U, VEC>(qrow, V, cs * CH, 0.f, y);
        }
        int lp = -1;
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int li = j * kSpecSeg + 4 * t + e;
                const float wk = spec_weight(x[4 * j + e], y[4 * j + e], M, p.c2, inv_s, use_p);
                wbuf[li] = wk;
                if (wk > 0.f) lp = li > lp ? li : lp;
            }
        if (lp >= 0) atomicMax(&sh_lastpos, lp);
    }
    __syncthreads();
    float run[R];
#pragma unroll
    for (int k = 0; k < R; k += 4) {
        const float4 v = *reinterpret_cast<const float4*>(&wbuf[t * R + k]);
        run[k] = v.x; run[k + 1] = v.y; run[k + 2] = v.z; run[k + 3] = v.w;
    }
    float rs = 0.f;
#pragma unroll
    for (int k = 0; k < R; ++k) rs += run[k];
    const float inc = wave_incl_scan(rs);
    const float up = __shfl_up(inc, 1);
    if (lane == 63) sh_wtot[w] = inc;
    __syncthreads();
    if (mode == 0) {
        float c = sh_base;
        for (int k = 0; k < w; ++k) c += sh_wtot[k];
        c += lane ? up : 0.f;
        const float thr = sh_t;
        int cand = INT_MAX;
#pragma unroll
        for (int k = 0; k < R; ++k) {
            c += run[k];
            if (cand == INT_MAX && run[k] > 0.f && c > thr) cand = t * R + k;
        }
        if (cand != INT_MAX) atomicMin(&sh_pick, cand);
    }
    __syncthreads();
    if (t == 0) {
        // no entry passed thr (rounding in the last chunk, or modes 1 and 2):
        // the chunk's last positive entry
        int pick = sh_pick != INT_MAX ? sh_pick : (mode == 2 ? 0 : sh_lastpos);
        if (pick < 0) pick = 0;
        p.result[2 * (size_t)b] = n;
        p.result[2 * (size_t)b + 1] = cs * CH + pick;
        p.lens[b] = spec_new_len(p.lens[b], n, p.S_max);
    }
}

}  // namespace decattn
