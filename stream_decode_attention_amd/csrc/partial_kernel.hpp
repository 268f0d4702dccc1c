// Split-KV partial attention: one workgroup per (batch, kv head, key tile).
//
// The method (tinydecode README, "how the decode step is put together";
// llm-decode-cuda, attention section): each block takes one chunk of the
// cache, computes scores, softmax statistics and p.V for every query head that
// shares the tile's kv head, and writes partial state (m, l, acc); a second
// kernel merges the chunks. Tiles at or past a row's length exit at once.
//
// Work split inside a tile (gfx950, wave64):
//  * A wave owns R query rows and walks "sub-tiles" of KPW = 32 keys. A key row
//    of D bf16 (128 or 256 bytes) is spread over LPK = D/8 lanes, 16 bytes per
//    lane, so one wave-wide 16-byte load covers 64/LPK whole keys: fully
//    coalesced, no lane reads a byte another lane reads.
//  * q.k: each lane multiplies its 8 dims by the row's query slice (pre-scaled
//    by scale*log2(e), kept in VGPRs) and the LPK lanes of a key sum with DPP
//    moves inside their 16-lane row.
//  * softmax: an online (running max) softmax over the wave's sub-tiles in the
//    log2 domain; each lane keeps partial l and acc for the keys of its lane
//    group, summed across groups once at the end.
//  * Up to NWK "key waves" split the tile's keys (sub-tile s of wave w covers
//    keys t0 + (s*NWK + w)*KPW ...); their states are combined once through LDS.
//  * Waves of the same workgroup may also hold different row groups (the chunk
//    path has T*G rows per kv head); every row group reads the same K/V tile.
//
// Every row is computed with the same sequence of floating-point operations
// whatever R is and whatever other rows share its wave, so a verify-chunk row
// is bit-identical to the decode call with the same key limit.
#pragma once

#include "device_common.hpp"

namespace decattn {

constexpr int kKeysPerWave = 32;   // keys a wave handles per sub-tile (KPW)

struct PartialParams {
    const uint16_t* q;      // bf16 [B][T][Hq][D]
    const uint16_t* k;      // bf16 [B][Hkv][S_max][D]
    const uint16_t* v;
    const int32_t* lens;    // [B]: seq_lens (decode) or ctx_lens (causal)
    float* ws_ml;           // [B][Hkv][NC][RT][2]  (m in log2 units, l)
    float* ws_acc;          // [B][Hkv][NC][RT][D]
    int T, Hq, Hkv, G, S_max, chunk, NC, RT, causal;
    int nwk;                // key waves per workgroup
    int rg_per_block;       // row groups per workgroup
    int n_row_blocks;       // workgroups per tile along the row axis
    float qscale;           // scale * log2(e)
};

template <int D, int R>
__global__ void __launch_bounds__(512)
split_kv_partial(const PartialParams p) {
    constexpr int LPK = D / 8;              // lanes per key row
    constexpr int KPL = 64 / LPK;           // keys per wave-wide load
    constexpr int NSTEP = kKeysPerWave / KPL;
    static_assert(D == 64 || D == 128, "head dim 64 or 128");

    extern __shared__ float smem[];

    const int c = blockIdx.x;
    const int kvh = blockIdx.y / p.n_row_blocks;
    const int rblk = blockIdx.y - kvh * p.n_row_blocks;
    const int b = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kw = wave % p.nwk;
    const int rgl = wave / p.nwk;
    const int rg = rblk * p.rg_per_block + rgl;

    const int len = p.lens[b];
    const int t0 = c * p.chunk;
    const int t1 = min(t0 + p.chunk, p.S_max);
    const int lim_tile = clamp_len(p.causal ? len + p.T : len, p.S_max);
    if (t0 >= lim_tile) return;             // whole workgroup: nothing to attend
    const int lim_all = min(lim_tile, t1);

    const int kk = lane / LPK;              // key slot inside one load
    const int db = lane % LPK;              // 8-dim block of this lane

    // ---- stage this wave's query rows (fp32, pre-scaled) and key limits
    float qf[R][8];
    int row_lim[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int r = rg * R + j;
        if (r < p.RT) {
            const int i = r / p.G;
            const int h = kvh * p.G + (r - i * p.G);
            const int n = clamp_len(p.causal ? len + i + 1 : len, p.S_max);
            row_lim[j] = min(n, t1);
            const uint4 raw = *reinterpret_cast<const uint4*>(
                p.q + ((size_t)(b * p.T + i) * p.Hq + h) * D + db * 8);
            float f[8];
            bf16x8_to_f32(raw, f);
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[j][e] = f[e] * p.qscale;
        } else {
            row_lim[j] = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[j][e] = 0.f;
        }
    }

    float m_run[R], l_run[R], acc[R][8];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        m_run[j] = kNegInf;
        l_run[j] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
    }

    const size_t head_base = (size_t)(b * p.Hkv + kvh) * p.S_max * D + db * 8;
    const uint16_t* kbase = p.k + head_base;
    const uint16_t* vbase = p.v + head_base;
    const int sub_stride = p.nwk * kKeysPerWave;

    for (int base = t0 + kw * kKeysPerWave; base < lim_all; base += sub_stride) {
        uint4 kr[NSTEP], vr[NSTEP];
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            const int j = base + st * KPL + kk;
            if (j < lim_all) {
                kr[st] = *reinterpret_cast<const uint4*>(kbase + (size_t)j * D);
                vr[st] = *reinterpret_cast<const uint4*>(vbase + (size_t)j * D);
            } else {
                kr[st] = make_uint4(0, 0, 0, 0);
                vr[st] = make_uint4(0, 0, 0, 0);
            }
        }

        // scores in log2 units; keys at or past a row's limit get -inf
        float s[NSTEP][R];
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            float kf[8];
            bf16x8_to_f32(kr[st], kf);
            const int j = base + st * KPL + kk;
#pragma unroll
            for (int jr = 0; jr < R; ++jr) {
                float part = qf[jr][0] * kf[0];
#pragma unroll
                for (int e = 1; e < 8; ++e) part = __builtin_fmaf(qf[jr][e], kf[e], part);
                part = group_sum<LPK>(part);
                s[st][jr] = (j < row_lim[jr]) ? part : kNegInf;
            }
        }

        float vf[NSTEP][8];
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) bf16x8_to_f32(vr[st], vf[st]);

#pragma unroll
        for (int jr = 0; jr < R; ++jr) {
            float mx = s[0][jr];
#pragma unroll
            for (int st = 1; st < NSTEP; ++st) mx = fmaxf(mx, s[st][jr]);
            mx = across_groups_max<LPK>(mx);
            const float m_new = fmaxf(m_run[jr], mx);
            const float m_use = (m_new == kNegInf) ? 0.f : m_new;
            const float alpha = fast_exp2(m_run[jr] - m_use);
            m_run[jr] = m_new;
            float l = l_run[jr] * alpha;
            float a[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = acc[jr][e] * alpha;
#pragma unroll
            for (int st = 0; st < NSTEP; ++st) {
                const float pj = fast_exp2(s[st][jr] - m_use);
                l += pj;
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] = __builtin_fmaf(pj, vf[st][e], a[e]);
            }
            l_run[jr] = l;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[jr][e] = a[e];
        }
    }

    // ---- sum the lane groups of the wave, then combine the key waves in LDS
#pragma unroll
    for (int jr = 0; jr < R; ++jr) {
        l_run[jr] = across_groups_sum<LPK>(l_run[jr]);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[jr][e] = across_groups_sum<LPK>(acc[jr][e]);
    }

    // LDS: [rg_per_block][nwk][R] x (D acc floats), then [rg_per_block][nwk][R] x (m, l)
    float* s_acc = smem;
    float* s_ml = smem + (size_t)p.rg_per_block * p.nwk * R * D;
    const int slot = (rgl * p.nwk + kw) * R;
    if (kk == 0) {
#pragma unroll
        for (int jr = 0; jr < R; ++jr) {
#pragma unroll
            for (int e = 0; e < 8; ++e) s_acc[(size_t)(slot + jr) * D + db * 8 + e] = acc[jr][e];
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int jr = 0; jr < R; ++jr) {
            s_ml[(slot + jr) * 2 + 0] = m_run[jr];
            s_ml[(slot + jr) * 2 + 1] = l_run[jr];
        }
    }
    __syncthreads();

    const int total = p.rg_per_block * R * D;
    const size_t tile_row0 = ((size_t)(b * p.Hkv + kvh) * p.NC + c) * p.RT;
    for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
        const int rg2 = idx / (R * D);
        const int rem = idx - rg2 * (R * D);
        const int jr = rem / D;
        const int d = rem - jr * D;
        const int r = (rblk * p.rg_per_block + rg2) * R + jr;
        if (r >= p.RT) continue;
        const int base_slot = rg2 * p.nwk * R + jr;     // slot of key wave 0 for this row
        float M = kNegInf;
        for (int w = 0; w < p.nwk; ++w) M = fmaxf(M, s_ml[(base_slot + w * R) * 2]);
        float A = 0.f, L = 0.f;
        if (M != kNegInf) {
            for (int w = 0; w < p.nwk; ++w) {
                const int sl = base_slot + w * R;
                const float wt = fast_exp2(s_ml[sl * 2] - M);
                A = __builtin_fmaf(wt, s_acc[(size_t)sl * D + d], A);
                L = __builtin_fmaf(wt, s_ml[sl * 2 + 1], L);
            }
        }
        p.ws_acc[(tile_row0 + r) * D + d] = A;
        if (d == 0) {
            p.ws_ml[(tile_row0 + r) * 2 + 0] = M;
            p.ws_ml[(tile_row0 + r) * 2 + 1] = L;
        }
    }
}

}  // namespace decattn
