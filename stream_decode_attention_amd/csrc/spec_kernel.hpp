// Speculative decoding's accept/reject step with the rollback of the cache
// lengths, on the device. The rule (tinydecode README, "speculative
// decoding"; FlashSpec page, correctness paragraph, after Leviathan et al.
// 2023, Algorithm 1): a draft survives when a uniform falls under the ratio of
// target to draft probability (compared here as logarithms); at the first
// draft that fails, the step's extra token is sampled from the positive part
// of target minus draft, and when all survive, from the target's last row; at
// temperature 0 the survivors are the drafts that match the target's argmax;
// rolling back is only a change of the length.
//
// Launches (no host sync):
//   spec_stats_kernel   one workgroup per (row b, position i, vocabulary
//                       chunk): the chunk's max logit and sum of
//                       exp2((l - max) * log2(e) / tau), or for greedy its
//                       largest logit and first index of it; the workgroup
//                       whose chunk holds a draft's token also records that
//                       token's logit, q and u;
//   spec_greedy_kernel  (tau = 0) one workgroup per row: merges the chunk
//                       statistics of every position, takes the decisions and
//                       writes the accept count, the argmax and the length;
//   spec_resid_kernel   (sampling) one workgroup per (row, chunk): the same
//                       merge and decisions (the same instructions on the same
//                       data, so every workgroup of a row reaches the same
//                       bits), then the chunk's mass of the draw weights;
//   spec_select_kernel  (sampling) one workgroup per row: finds the chunk
//                       holding the draw, rescans it, writes the results.
// Each launch reads only what earlier launches wrote, so the kernel
// boundaries order every exchange: no atomics, fences or counters (a
// last-arriving-workgroup scheme would need an L2 write-back per workgroup
// to publish its chunk sum across the chip's eight L2s, which costs more
// than the extra launch).
#pragma once

#include <climits>

#include "device_common.hpp"

namespace decattn {

constexpr int kSpecThreads = 256;
constexpr int kSpecWaves = kSpecThreads / 64;
constexpr int kSpecSeg = kSpecThreads * 4;    // elements per segment: one float4 per thread
constexpr int kSpecMaxT = 32;                 // gamma + 1 positions: one ballot decides them all
constexpr int kSpecStage = 4096;              // chunk statistics staged in LDS at once (float2)
constexpr int kSpecMaxNC = kSpecStage / 2;    // chunks per position: two positions fit the stage


struct SpecParams {
    const float* logits;      // [B][T][V]
    const float* q;           // [B][T-1][V]  (sampling only)
    const int32_t* drafts;    // [B][T-1]
    const float* u;           // [B][T-1]     (sampling only)
    const float* r;           // [B]          (sampling only)
    int32_t* lens;            // [B] in: length before the verify pass; out: after the rollback
    int32_t* result;          // [B][2]: accepted drafts, next token
    float2* stats;            // [B][T][NC]
    float2* parts;            // [B][NC2]: each draw chunk's residual mass and p mass (sampling)
    float4* rowinfo;          // [B]: max and 1/sum of p_n, and n (sampling)
    float4* dinfo;            // [B][T-1]: each draft's target logit, q and u, and its id (sampling)
    float c2;                 // log2(e) / tau
    int T, V, NC, S_max;
    int NC2;                  // chunks of the draw (sampling), 1024 * U2 entries each
    int stage_n;              // float2 entries of LDS the decision stages: min(T * NC, kSpecStage)
};

// Chunk element (j, e) of thread t has vocabulary index c0 + j*kSpecSeg + 4t + e:
// each segment j is one coalesced float4 read by the workgroup. Indices at or
// past V read as `fill`.
// STREAM marks data read once (the statistics pass over every position):
// non-temporal loads, which keep it from displacing what is read again.
#ifndef DECATTN_SPEC_NT
#define DECATTN_SPEC_NT 1
#endif
typedef float spec_f4 __attribute__((ext_vector_type(4)));

template <int U, bool VEC, bool STREAM = false>
__device__ __forceinline__ void spec_load(const float* __restrict__ row, int V, int c0, float fill,
                                          float (&x)[4 * U]) {
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const int e0 = c0 + j * kSpecSeg + 4 * t;
        if constexpr (VEC) {
            spec_f4 v = {fill, fill, fill, fill};
            if (e0 < V) {                                                   // V % 4 == 0 here
                const spec_f4* src = reinterpret_cast<const spec_f4*>(row + e0);
                v = (STREAM && DECATTN_SPEC_NT) ? __builtin_nontemporal_load(src) : *src;
            }
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

// Wave-wide reductions and scans on DPP lane moves inside 16-lane rows and
// the gfx950 lane swaps across rows (no LDS traffic). Every lane of a
// reduction ends with the same bits.
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& bv, int& bi) {
    const float ov = dpp_copy<CTRL>(bv);
    const int oi = dpp_copy_i<CTRL>(bi);
    if (spec_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
}

__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
    argmax_step<kDppXor1>(bv, bi);
    argmax_step<kDppXor2>(bv, bi);
    argmax_step<kDppHalfMirror>(bv, bi);
    argmax_step<kDppMirror>(bv, bi);
    // rows (0, 1) and (2, 3), then the two halves: every lane compares the
    // same pair in the same order
    const f32x2 v1 = swap16(bv, bv), i1 = swap16(__int_as_float(bi), __int_as_float(bi));
    bv = v1.x; bi = __float_as_int(i1.x);
    if (spec_better(v1.y, __float_as_int(i1.y), bv, bi)) { bv = v1.y; bi = __float_as_int(i1.y); }
    const f32x2 v2 = swap32(bv, bv), i2 = swap32(__int_as_float(bi), __int_as_float(bi));
    bv = v2.x; bi = __float_as_int(i2.x);
    if (spec_better(v2.y, __float_as_int(i2.y), bv, bi)) { bv = v2.y; bi = __float_as_int(i2.y); }
}

__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_copy<kDppXor1>(x));
    x = fmaxf(x, dpp_copy<kDppXor2>(x));
    x = fmaxf(x, dpp_copy<kDppHalfMirror>(x));
    x = fmaxf(x, dpp_copy<kDppMirror>(x));
    return across_groups_max<16>(x);
}

__device__ __forceinline__ float wave_sum(float x) {
    return across_groups_sum<16>(group_sum<16>(x));
}

// Inclusive prefix sum over the wave in lane order: a shift-and-add scan
// inside each 16-lane row (lanes shifted in from outside the row read 0),
// then each row adds the totals of the rows before it.
__device__ __forceinline__ float wave_incl_scan(float x) {
    x += dpp_move<0x111>(x);          // row_shr:1
    x += dpp_move<0x112>(x);          // row_shr:2
    x += dpp_move<0x114>(x);          // row_shr:4
    x += dpp_move<0x118>(x);          // row_shr:8
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47));
    const float o2 = r0 + r1, o3 = o2 + r2;
    const int row = (threadIdx.x & 63) >> 4;
    return row == 0 ? x : x + (row == 1 ? r0 : (row == 2 ? o2 : o3));
}

// Runs of consecutive entries are laid out by lane in index order, so the
// first candidate of a wave is the lowest lane's and the last positive entry
// the highest lane's: one LDS atomic per wave instead of one per lane (those
// on one word serialize).
__device__ __forceinline__ void wave_first_min(int* dst, int v, bool has) {
    const unsigned long long m = __ballot(has);
    if (m) {
        const int L = __ffsll(m) - 1;
        const int x = __shfl(v, L);
        if ((threadIdx.x & 63) == 0) atomicMin(dst, x);
    }
}

__device__ __forceinline__ void wave_last_max(int* dst, int v, bool has) {
    const unsigned long long m = __ballot(has);
    if (m) {
        const int L = 63 - __clzll((long long)m);
        const int x = __shfl(v, L);
        if ((threadIdx.x & 63) == 0) atomicMax(dst, x);
    }
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
    spec_load<U, VEC, true>(p.logits + (size_t)row * p.V, p.V, c0, kNegInf, x);
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


// Merge the chunk statistics of every position of row b and take the accept
// decisions; returns n, the number of drafts kept, in every thread. Fills
// row_m/row_s (sampling: max logit and sum of exp2((l - max) * c2)) or row_i
// (greedy: first index of the largest logit). `stage` holds p.stage_n
// float2 (dynamic LDS). Whole positions are staged in LDS with one batch of
// loads, then one wave merges each position.
template <int WAVES, bool GREEDY>
__device__ __forceinline__ int spec_decide(const SpecParams& p, int b, float2* stage, float* row_m, float* row_s,
                                           int* row_i, int* sh_n) {
    const int T = p.T, gamma = T - 1, V = p.V, NC = p.NC;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;

    // the draft side of each position (threads t < gamma, all in wave 0):
    // its token id and, for sampling, the target logit, q and u at that id
    // as the statistics kernel recorded them
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

    const int rpt = p.stage_n / NC;                   // >= 1: stage_n >= min(T, 2) * NC
    for (int i0 = 0; i0 < T; i0 += rpt) {
        const int nr = T - i0 < rpt ? T - i0 : rpt;
        const float2* src = p.stats + ((size_t)b * T + i0) * NC;
#pragma unroll 4
        for (int e = t; e < nr * NC; e += WAVES * 64) stage[e] = src[e];
        __syncthreads();
        for (int i = i0 + w; i < i0 + nr; i += WAVES) {
            const float2* st = stage + (size_t)(i - i0) * NC;
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
        if (lane == 0) *sh_n = rej ? __ffsll(rej) - 1 : gamma;
    }
    __syncthreads();
    return *sh_n;
}

// Greedy finish: one workgroup per row writes n, the argmax of position n and
// the new length.
__global__ __launch_bounds__(kSpecThreads) void spec_greedy_kernel(const SpecParams p) {
    extern __shared__ float2 stage[];
    __shared__ float row_m[kSpecMaxT], row_s[kSpecMaxT];
    __shared__ int row_i[kSpecMaxT], sh_n;
    const int b = blockIdx.x;
    const int ctx = p.lens[b];
    const int n = spec_decide<kSpecWaves, true>(p, b, stage, row_m, row_s, row_i, &sh_n);
    if (threadIdx.x == 0) {
        p.result[2 * (size_t)b] = n;
        p.result[2 * (size_t)b + 1] = row_i[n];
        p.lens[b] = spec_new_len(ctx, n, p.S_max);
    }
}

// Sampling, second launch: per (row b, chunk c of the draw's own chunking),
// the decision, then the chunk's mass of the draw weights: the residual
// max(0, p_n - q_n) of the first rejected position n (and p_n, for a
// residual with no positive mass), or p of the bonus row. Chunk 0 also
// records n, the max and 1 / sum of p_n.

template <int U, bool VEC>
__global__ __launch_bounds__(kSpecThreads) void spec_resid_kernel(const SpecParams p) {
    constexpr int CH = U * kSpecSeg;
    extern __shared__ float2 stage[];
    __shared__ float row_m[kSpecMaxT], row_s[kSpecMaxT];
    __shared__ int row_i[kSpecMaxT], sh_n;
    __shared__ float sh_w[kSpecWaves], sh_p[kSpecWaves];
    const int c = blockIdx.x % p.NC2, b = blockIdx.x / p.NC2;
    const int T = p.T, gamma = T - 1, V = p.V;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const float* lrows = p.logits + (size_t)b * T * V;
    const float* qrows = p.q + (size_t)b * gamma * V;
    const int n = spec_decide<kSpecWaves, false>(p, b, stage, row_m, row_s, row_i, &sh_n);
    float x[4 * U], y[4 * U];
    spec_load<U, VEC>(lrows + (size_t)n * V, V, c * CH, kNegInf, x);
    if (n < gamma) spec_load<U, VEC>(qrows + (size_t)n * V, V, c * CH, 0.f, y);
    const float M = row_m[n];
    const float inv_s = 1.0f / row_s[n];
    const bool bonus = n == gamma;
    float ws = 0.f, ps = 0.f;
#pragma unroll
    for (int k = 0; k < 4 * U; ++k) {
        ws += spec_weight(x[k], bonus ? 0.f : y[k], M, p.c2, inv_s, bonus);
        ps += spec_weight(x[k], 0.f, M, p.c2, inv_s, true);
    }
    ws = wave_sum(ws);
    ps = wave_sum(ps);
    if (lane == 0) { sh_w[w] = ws; sh_p[w] = ps; }
    __syncthreads();
    if (t == 0) {
        float a = 0.f, e = 0.f;
        for (int k = 0; k < kSpecWaves; ++k) { a += sh_w[k]; e += sh_p[k]; }
        p.parts[(size_t)b * p.NC2 + c] = make_float2(a, e);
        if (c == 0) p.rowinfo[b] = make_float4(M, inv_s, __int_as_float(n), 0.f);
    }
}

// Sampling, third launch: one workgroup per row draws the token. Thread t
// takes the chunks [t*RC, t*RC + RC) in index order; a block-wide running
// sum over those runs finds the first chunk whose running mass passes
// r * total, which is then rescanned entry by entry the same way.
template <int U, bool VEC>
__global__ __launch_bounds__(kSpecThreads) void spec_select_kernel(const SpecParams p) {
    constexpr int CH = U * kSpecSeg;
    constexpr int R = CH / kSpecThreads;
    extern __shared__ float2 pr[];                      // p.NC2 entries
    __shared__ __attribute__((aligned(16))) float wbuf[CH];
    __shared__ float sh_tw[kSpecWaves], sh_tp[kSpecWaves], sh_base;
    __shared__ int sh_pick, sh_last;
    const int b = blockIdx.x;
    const int T = p.T, gamma = T - 1, V = p.V, NC = p.NC2;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;

    // everything read here was written by earlier launches or is an input:
    // one batch of loads
    const float4 info = p.rowinfo[b];
    const float rb = p.r[b];
    const int ctx = p.lens[b];
    {
        const float2* src = p.parts + (size_t)b * NC;
#pragma unroll 4
        for (int e = t; e < NC; e += kSpecThreads) pr[e] = src[e];
    }
    if (t == 0) { sh_pick = INT_MAX; sh_last = -1; }
    __syncthreads();
    const float M = info.x, inv_s = info.y;
    const int n = __float_as_int(info.z);
    const bool bonus = n == gamma;

    // the chunk: per-thread masses, block running sum, each thread walks its run
    const int RC = (NC + kSpecThreads - 1) / kSpecThreads;
    const int k0 = t * RC < NC ? t * RC : NC, k1 = k0 + RC < NC ? k0 + RC : NC;
    float aw = 0.f, ap = 0.f;
    for (int k = k0; k < k1; ++k) { aw += pr[k].x; ap += pr[k].y; }
    const float iw = wave_incl_scan(aw), ip = wave_incl_scan(ap);
    const float uw = __shfl_up(iw, 1), up = __shfl_up(ip, 1);
    if (lane == 63) { sh_tw[w] = iw; sh_tp[w] = ip; }
    __syncthreads();
    float tw = 0.f, tp = 0.f;
    for (int k = 0; k < kSpecWaves; ++k) { tw += sh_tw[k]; tp += sh_tp[k]; }
    // a residual with no positive mass (only through rounding): draw from p
    const bool use_p = bonus || !(tw > 0.f);
    const float thr = rb * (use_p ? tp : tw);
    float run = 0.f;
    for (int k = 0; k < w; ++k) run += use_p ? sh_tp[k] : sh_tw[k];
    run += lane ? (use_p ? up : uw) : 0.f;
    int cand = INT_MAX, lastp = -1;
    float cbase = 0.f;
    for (int k = k0; k < k1; ++k) {
        const float v = use_p ? pr[k].y : pr[k].x;
        if (v > 0.f) {
            lastp = k;
            if (cand == INT_MAX && run + v > thr) { cand = k; cbase = run; }
        }
        run += v;
    }
    wave_first_min(&sh_pick, cand, cand != INT_MAX);
    wave_last_max(&sh_last, lastp, lastp >= 0);
    __syncthreads();
    if (cand != INT_MAX && cand == sh_pick) sh_base = cbase;
    // 0: first chunk whose running mass passes thr; 1: rounding left thr at
    // or past the total, take the last positive entry; 2: no positive weight
    // at all (rows that break the input rules)
    const int mode = sh_pick != INT_MAX ? 0 : (sh_last >= 0 ? 1 : 2);
    const int cs = mode == 0 ? sh_pick : (mode == 1 ? sh_last : 0);
    __syncthreads();

    // the chunk's weights into LDS in index order; thread t walks [tR, tR + R)
    {
        float x[4 * U], y[4 * U];
        spec_load<U, VEC>(p.logits + ((size_t)b * T + n) * V, V, cs * CH, kNegInf, x);
        if (bonus) {
#pragma unroll
            for (int k = 0; k < 4 * U; ++k) y[k] = 0.f;
        } else {
            spec_load<U, VEC>(p.q + ((size_t)b * gamma + n) * V, V, cs * CH, 0.f, y);
        }
#pragma unroll
        for (int j = 0; j < U; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                wbuf[j * kSpecSeg + 4 * t + e] = spec_weight(x[4 * j + e], y[4 * j + e], M, p.c2, inv_s, use_p);
    }
    if (t == 0) { sh_pick = INT_MAX; sh_last = -1; }
    __syncthreads();
    float rw[R];
#pragma unroll
    for (int k = 0; k < R; k += 4) {
        const float4 v = *reinterpret_cast<const float4*>(&wbuf[t * R + k]);
        rw[k] = v.x; rw[k + 1] = v.y; rw[k + 2] = v.z; rw[k + 3] = v.w;
    }
    float rs = 0.f;
#pragma unroll
    for (int k = 0; k < R; ++k) rs += rw[k];
    const float inc = wave_incl_scan(rs);
    const float upe = __shfl_up(inc, 1);
    if (lane == 63) sh_tw[w] = inc;
    __syncthreads();
    float c2 = sh_base;
    for (int k = 0; k < w; ++k) c2 += sh_tw[k];
    c2 += lane ? upe : 0.f;
    int pick = INT_MAX, lp = -1;
#pragma unroll
    for (int k = 0; k < R; ++k) {
        c2 += rw[k];
        if (rw[k] > 0.f) {
            lp = t * R + k;
            if (mode == 0 && pick == INT_MAX && c2 > thr) pick = t * R + k;
        }
    }
    wave_first_min(&sh_pick, pick, pick != INT_MAX);
    wave_last_max(&sh_last, lp, lp >= 0);
    __syncthreads();
    if (t == 0) {
        // no entry passed thr (rounding in the last chunk, or modes 1 and 2):
        // the chunk's last positive entry
        int k = sh_pick != INT_MAX ? sh_pick : (mode == 2 ? 0 : sh_last);
        if (k < 0) k = 0;
        p.result[2 * (size_t)b] = n;
        p.result[2 * (size_t)b + 1] = cs * CH + k;
        p.lens[b] = spec_new_len(ctx, n, p.S_max);
    }
}

}  // namespace decattn
