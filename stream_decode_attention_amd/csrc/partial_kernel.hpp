// Split-KV partial attention: one workgroup per (batch, kv head, key tile).
//
// The method (tinydecode README, "how the decode step is put together";
// llm-decode-cuda, attention section): each block takes one chunk of the
// cache, computes scores, softmax statistics and p.V for every query head that
// shares the tile's kv head, and writes partial state (m, l, acc); a second
// kernel merges the chunks. Tiles at or past a row's length exit at once.
//
// Work split inside a tile (gfx950, wave64):
//  * A wave owns R query rows (padded to RP, a power of two) and walks
//    "sub-tiles" of KPW keys. A key row of D bf16 (128 or 256 bytes) is spread
//    over a group of LPK = D/8 lanes, 16 bytes per lane, so one wave-wide
//    16-byte load covers 64/LPK whole keys: fully coalesced, no byte read
//    twice. Loads go through a range-checked buffer resource that ends at the
//    tile's last attended key, so keys past a length read as zeros and are
//    never touched in memory.
//  * While a sub-tile is computed, the next NBUF-1 are already being loaded
//    into other register sets (software pipeline): at full load the HBM
//    latency is several microseconds, so each compute unit needs on the order
//    of 128 KB in flight to stream at the roofline.
//  * q.k: v_dot2c_f32_bf16 on the raw bf16 pairs of q and k gives each lane a
//    partial dot product over its 8 dims for every row; a butterfly
//    reduce-scatter over the lane group (DPP moves, halving the rows held at
//    each stage) leaves each lane with the complete score of ONE row (its
//    "own" row), so the mask, the exponential and the row sum run once per
//    lane instead of once per row. p of the other rows is gathered back from
//    the lanes that own them (DPP row rotations, or ds_swizzle for 8-lane
//    groups) into "slots": slot k of a lane holds row slot_row[k].
//  * softmax: online (running-max) softmax over the wave's sub-tiles in log2
//    units; accumulators are rescaled only when some row's maximum grew.
//  * Up to NWK "key waves" split the tile (sub-tile s of wave w covers keys
//    t0 + (s*NWK + w)*KPW ...); their states are combined once through LDS.
//  * Waves of the same workgroup may hold different row groups (the verify
//    chunk has T*G rows per kv head); all row groups share the tile's K/V.
//  * Work distribution, two modes. Persistent: a grid of the resident
//    workgroups stages the lengths, counts the attended tiles and walks them
//    (tiles past a length are never scheduled; a workgroup may take several,
//    with the next item's loads in flight while one is finished). One round
//    (ONE_ROUND, when every possible tile up to S_max fits on the device at
//    once and a tile is at most kNumBuf sub-tiles per wave): one workgroup
//    per possible tile, which knows its tile from its index, reads only its
//    own row's length (no staging, counting or barrier) and exits if the
//    tile lies past it.
//
// Every row is computed with the same sequence of floating-point operations
// whatever R is and whatever other rows share its wave (the butterfly pairs
// lanes in the same fixed order for every row count, and a rescale by an
// unchanged maximum multiplies by exactly 1), so a verify-chunk row computed
// here is bit-identical to the decode call with the same key limit.
#pragma once

#include "device_common.hpp"

#ifndef DECATTN_KEYS_PER_WAVE
#define DECATTN_KEYS_PER_WAVE 16
#endif
#ifndef DECATTN_PREFETCH_FENCE
#define DECATTN_PREFETCH_FENCE 1
#endif
#ifndef DECATTN_NBUF
#define DECATTN_NBUF 2
#endif
#ifndef DECATTN_WAVES_PER_EU
#define DECATTN_WAVES_PER_EU 1
#endif

namespace decattn {

constexpr int kKeysPerWave = DECATTN_KEYS_PER_WAVE;   // keys a wave handles per sub-tile (KPW)
constexpr int kNumBuf = DECATTN_NBUF;                 // sub-tiles in registers: 1 computed + (NBUF-1) in flight
#ifndef DECATTN_MAX_KEY_WAVES
#define DECATTN_MAX_KEY_WAVES 4
#endif
constexpr int kMaxKeyWaves = DECATTN_MAX_KEY_WAVES;   // waves splitting one tile's keys (nwk <= this)
static_assert((kMaxKeyWaves & (kMaxKeyWaves - 1)) == 0, "the partial kernel splits its waves by shifts");
static_assert((kKeysPerWave & (kKeysPerWave - 1)) == 0, "keys per wave is a power of two");

// Key waves per tile for a tile of `chunk` keys (a power of two): one per
// kKeysPerWave keys, at least one and at most kMaxKeyWaves. The host sizes the
// workgroup with it and the kernel derives its wave layout from it.
__host__ __device__ constexpr int key_waves_for(int chunk) {
    return chunk / kKeysPerWave < 1 ? 1 : (chunk / kKeysPerWave > kMaxKeyWaves ? kMaxKeyWaves : chunk / kKeysPerWave);
}
static_assert(kNumBuf >= 2, "the load pointer must run ahead of the compute pointer");

// ceil(2^16 / G) for 1 <= G <= 8: r / G = (r * g_magic) >> 16 exactly for
// every r < 8192 (a select chain, no division)
__host__ __device__ constexpr int g_magic_for(int G) {
    return G <= 4 ? (G <= 2 ? (G == 1 ? 65536 : 32768) : (G == 3 ? 21846 : 16384))
                  : (G <= 6 ? (G == 5 ? 13108 : 10923) : (G == 7 ? 9363 : 8192));
}

// What the partial kernels read after their first loads (the pointers and
// shapes those loads need come as leading scalar arguments, preloaded into
// SGPRs). The host also carries the inputs and the causal flag here, which
// it passes on as leading arguments.
struct PartialParams {
    const uint16_t* q;      // bf16 [B][T][Hq][D]            (host side)
    const uint16_t* k;      // bf16 [B][Hkv][S_max][D]       (host side)
    const uint16_t* v;      //                                (host side)
    const int32_t* lens;    // [B]: seq_lens (decode) or ctx_lens (causal)   (host side)
    float* ws_ml;           // [B][Hkv][NC][RT][2]  (m in log2 units, l)
    float* ws_acc;          // [B][Hkv][NC][RT][D]
    int NC;                 // tiles per row (slots in the workspace)
    int causal;             // (host side) 1: causal chunk, 0: decode
    int rg_per_block;       // row groups per workgroup
    int n_row_blocks;       // workgroups per tile along the row axis
    float qscale;           // scale * log2(e); magnitude at least FLT_MIN, sign of scale
    int B;                  // batch rows (lengths staged in LDS)
    int lds_main;           // bytes of dynamic LDS before the staged lengths (verify kernel)
};

constexpr int pad_rows(int r) { return r <= 1 ? 1 : r <= 2 ? 2 : r <= 4 ? 4 : 8; }
constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

// One butterfly stage over bit BIT of the lane's index in its group: holding
// H rows, a lane keeps the upper H/2 rows if its bit is set (else the lower
// half) and adds its partner's partial sums of the rows it keeps; with one row
// left it just adds the partner's value. Partners: BIT 3 row_mirror (l, 15-l),
// BIT 2 row_half_mirror (l, 7-l), BIT 1 and 0 quad permutes (l^2, l^1).
template <int BIT, int H>
__device__ __forceinline__ void butterfly_stage(float (&x)[8], int db) {
    constexpr int CTRL = BIT == 3 ? kDppMirror : BIT == 2 ? kDppHalfMirror : BIT == 1 ? kDppXor2 : kDppXor1;
    if constexpr (H > 1) {
        const bool up = (db >> BIT) & 1;
#pragma unroll
        for (int i = 0; i < H / 2; ++i) {
            const float lo = x[i], hi = x[i + H / 2];
            const float send = up ? lo : hi;
            const float keep = up ? hi : lo;
            x[i] = keep + dpp_move<CTRL>(send);
        }
    } else {
        x[0] = x[0] + dpp_move<CTRL>(x[0]);
    }
}

// Reduce-scatter of RP row partials over a group of LPK lanes: returns the
// full sum of the lane's own row, whose index is the top log2(RP) bits of db.
template <int LPK, int RP>
__device__ __forceinline__ float reduce_scatter(float (&x)[8], int db) {
    constexpr int H2 = LPK == 16 ? (RP > 1 ? RP / 2 : 1) : RP;   // rows held entering bit 2
    constexpr int H1 = H2 > 1 ? H2 / 2 : 1;
    constexpr int H0 = H1 > 1 ? H1 / 2 : 1;
    if constexpr (LPK == 16) butterfly_stage<3, RP>(x, db);
    butterfly_stage<2, H2>(x, db);
    butterfly_stage<1, H1>(x, db);
    butterfly_stage<0, H0>(x, db);
    return x[0];
}

// Value of slot K: the same quantity held by the lanes owning row slot_row[K].
// 16-lane groups rotate inside the DPP row by K row-sets; 8-lane groups swap
// row-sets by XOR with ds_swizzle.
template <int LPK, int RP, int K>
__device__ __forceinline__ float gather_slot(float x) {
    constexpr int SET = LPK / RP;                       // lanes per row-set
    if constexpr (K == 0) return x;
    else if constexpr (LPK == 16) return dpp_copy<0x120 + K * SET>(x);   // row_ror
    else return swizzle_xor<K * SET>(x);
}
template <int LPK, int RP, int K>
__device__ __forceinline__ int gather_slot_i(int x) {
    constexpr int SET = LPK / RP;
    if constexpr (K == 0) return x;
    else if constexpr (LPK == 16) return dpp_copy_i<0x120 + K * SET>(x);
    else return swizzle_xor_i<K * SET>(x);
}

template <int LPK, int RP, int K = 0>
__device__ __forceinline__ void gather_all(float x, float (&out)[8]) {
    if constexpr (K < RP) {
        out[K] = gather_slot<LPK, RP, K>(x);
        gather_all<LPK, RP, K + 1>(x, out);
    }
}
template <int LPK, int RP, int K = 0>
__device__ __forceinline__ void gather_all_i(int x, int (&out)[8]) {
    if constexpr (K < RP) {
        out[K] = gather_slot_i<LPK, RP, K>(x);
        gather_all_i<LPK, RP, K + 1>(x, out);
    }
}

// ONE_ROUND: every possible work item has a workgroup of its own (the host
// launches a grid of (kv head, tile, sequence) when they all fit on the
// device at once and one row block holds every row), so a workgroup knows its
// tile from its index alone, with no division. Its
// first K/V loads are written over the whole tile (keys up to t1 lie inside
// the cache) so that they need no length; keys past the length are masked by
// select (scores to -inf, V to 0), never by a multiply, since stale slots may
// hold any bits. The length's load leaves first and the length is not used
// before those loads are issued.
// The pointers and shapes the first loads depend on are leading scalar
// arguments (preloaded into SGPRs at wave launch): lens, K, V, q, S_max,
// chunk, Hkv, gm_or_B, G, and tok_add (T for a causal chunk of T tokens, 0
// for a decode call, whose T is 1). gm_or_B is g_magic = ceil(2^16 / G) for
// the one-round launch (row / G as a multiply-shift before its first loads;
// it never needs the batch size) and the batch size B for the persistent walk
// (which stages every length first and derives g_magic from G off that path):
// the 14 dwords are all that the hardware preloads.
template <int D, int R, bool ONE_ROUND>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(DECATTN_WAVES_PER_EU)))
split_kv_partial(const int32_t* lens, const uint16_t* kc, const uint16_t* vc, const uint16_t* qp, int S_max,
                 int chunk, int Hkv, int gm_or_B, int G, int tok_add, const PartialParams p) {
    constexpr int LPK = D / 8;              // lanes per key row
    constexpr int KPL = 64 / LPK;           // keys per wave-wide load
    constexpr int NSTEP = kKeysPerWave / KPL;
    constexpr int RP = pad_rows(R);         // rows per wave, padded
    constexpr int SET_BITS = ilog2(LPK) - ilog2(RP);
    static_assert(D == 64 || D == 128, "head dim 64 or 128");
    static_assert(R >= 1 && R <= 8, "1..8 rows per wave");
    static_assert(NSTEP >= 1 && NSTEP * KPL == kKeysPerWave, "keys per wave must be a multiple of keys per load");

    extern __shared__ float smem[];
    __shared__ int s_count[16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // the shape, from preloaded arguments only: tok_add = T for a causal chunk
    // of T tokens, 0 for a decode call (T = 1)
    const int T = tok_add > 0 ? tok_add : 1;
    const int RT = T * G;                   // rows per kv head
    const int Hq = G * Hkv;
    const bool causal = tok_add != 0;
    const int g_magic = ONE_ROUND ? gm_or_B : g_magic_for(G);   // r / G = (r * g_magic) >> 16
    const int B = ONE_ROUND ? 0 : gm_or_B;  // batch rows (persistent walk only)
    const int nwk = key_waves_for(chunk);   // a power of two
    const int kw = wave & (nwk - 1);
    const int rgl = wave >> __builtin_ctz(nwk);
    const int kk = lane / LPK;              // key slot inside one load
    const int db = lane % LPK;              // 8-dim block of this lane
    const int own = db >> SET_BITS;         // the row this lane completes
    int slot_row[8];
    gather_all_i<LPK, RP>(own, slot_row);

    // ---- lengths into LDS; count the tiles that hold attended keys
    float* s_acc = smem;                                    // [rgb][nwk][R][D]
    float* s_ml = smem + (size_t)p.rg_per_block * nwk * R * D;   // [rgb][nwk][R][2]
    int* s_len = reinterpret_cast<int*>(s_ml + (size_t)p.rg_per_block * nwk * R * 2);   // [B]
    const int per_tile = Hkv * p.n_row_blocks;              // work items per (b, tile)
    int n_items = 0;
    if constexpr (!ONE_ROUND) {
        int my_tiles = 0;
        auto count_len = [&](int i, int len) {
            s_len[i] = len;
            const int lim = clamp_len_add(len, tok_add, S_max);
            my_tiles += (lim + chunk - 1) >> __builtin_ctz(chunk);   // chunk is a power of two
        };
        // Each thread's first length is loaded before anything waits (B is
        // preloaded); the fields of p and the workgroup size the walk needs
        // are used right after it, so their scalar loads return under the
        // length's round trip instead of one after another ahead of it.
        const int len0 = tid < B ? lens[tid] : 0;
        asm volatile("" :: "s"(p.rg_per_block), "s"(p.n_row_blocks), "s"((int)blockDim.x));
        if (tid < B) count_len(tid, len0);
        for (int i = tid + (int)blockDim.x; i < B; i += blockDim.x) count_len(i, lens[i]);
        my_tiles = wave_sum_i(my_tiles);
        if (lane == 0) s_count[wave] = my_tiles;
        __syncthreads();
        int n_tiles = 0;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) n_tiles += s_count[w];
        n_items = n_tiles * per_tile;
    }

    // Work item t enumerates (b, kvh, row block, tile c) over attended tiles
    // only, b-major; workgroup w takes items w, w + P, w + 2P, ... (P = grid),
    // so every workgroup gets the same number of items to within one. The
    // walk over b only moves forward.
    int b_cur = 0, pre_cur = 0;
    auto tiles_of = [&](int b) {
        const int len = s_len[b];
        return (clamp_len_add(len, tok_add, S_max) + chunk - 1) >> __builtin_ctz(chunk);
    };

    struct Tile {
        int b, kvh, rblk, c, len, t0, t1, lim_all;
    };
    auto locate = [&](int t) {
        while (t >= pre_cur + tiles_of(b_cur) * per_tile) {
            pre_cur += tiles_of(b_cur) * per_tile;
            ++b_cur;
        }
        Tile tl;
        const int na = tiles_of(b_cur);
        const int u = t - pre_cur;
        tl.b = b_cur;
        tl.c = u % na;
        const int rest = u / na;
        tl.rblk = rest % p.n_row_blocks;
        tl.kvh = rest / p.n_row_blocks;
        tl.len = s_len[b_cur];
        tl.t0 = tl.c * chunk;
        tl.t1 = min(tl.t0 + chunk, S_max);
        tl.lim_all = min(clamp_len_add(tl.len, tok_add, S_max), tl.t1);
        return tl;
    };

    // this wave's query rows of a tile (raw bf16 pairs) and its own row's key
    // limit. Every slot loads a valid row, with no branch: slots past the
    // wave's rows take row 0 of the item; their scores land only in lanes whose
    // own row is one of them, which have a key limit of 0. Nothing here waits
    // for the loads, so entering the next item does not drain the K/V loads in
    // flight (vector memory completes in order).
    auto load_q = [&](const Tile& tl, uint4 (&qraw)[RP], int& my_lim) {
        const int rg = tl.rblk * p.rg_per_block + rgl;
        my_lim = 0;
#pragma unroll
        for (int j = 0; j < RP; ++j) {
            const int r0 = rg * R + j;
            const bool ok = j < R && r0 < RT;
            const int r = ok ? r0 : 0;
            const int i = (r * g_magic) >> 16;      // r / G
            const int h = tl.kvh * G + (r - i * G);
            if (j == own && ok) my_lim = min(clamp_len_add(tl.len, causal ? i + 1 : 0, S_max), tl.t1);
            qraw[j] = *reinterpret_cast<const uint4*>(qp + ((size_t)(tl.b * T + i) * Hq + h) * D + db * 8);
        }
    };

    const uint32_t lane_off = (uint32_t)(kk * D + db * 8) * 2;
    const int sub_stride = nwk * kKeysPerWave;
    const float qs = p.qscale;

    // K/V of a tile's (b, kvh): rows [0, lim_all) are in range, the rest read as 0
    struct Rsrc {
        __amdgpu_buffer_rsrc_t k, v;
    };
    auto make_tile_rsrc = [&](const Tile& tl) {
        const size_t head_base = (size_t)(tl.b * Hkv + tl.kvh) * S_max * D;
        const uint32_t range = (uint32_t)tl.lim_all * D * 2;
        return Rsrc{make_rsrc(kc + head_base, range), make_rsrc(vc + head_base, range)};
    };

    auto load = [&](const Rsrc& rs, uint4 (&kb)[NSTEP], uint4 (&vb)[NSTEP], int base) {
        // keys at or past lim_all (including a whole sub-tile past the tile)
        // are outside the resource and load zeros; base < S_max + chunk keeps
        // the byte offset far below 2^32
        const uint32_t off = (uint32_t)base * (D * 2) + lane_off;
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            kb[st] = buffer_load16(rs.k, off + st * KPL * D * 2);
            vb[st] = buffer_load16(rs.v, off + st * KPL * D * 2);
        }
    };

    float m_run, l_run;                     // own row
    float acc[RP][8];                       // slot k, this lane's 8 dims

    auto compute = [&](const uint4 (&qraw)[RP], int my_lim, const uint4 (&kb)[NSTEP],
                       const uint4 (&vb)[NSTEP], int base, int v_lim) {
        // own-row scores in log2 units, -inf past the row's limit
        float dm[NSTEP];
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            float x[8];
#pragma unroll
            for (int j = 0; j < RP; ++j) {
                float d = dot2_bf16(qraw[j].x, kb[st].x, 0.f);
                d = dot2_bf16(qraw[j].y, kb[st].y, d);
                d = dot2_bf16(qraw[j].z, kb[st].z, d);
                x[j] = dot2_bf16(qraw[j].w, kb[st].w, d);
            }
            const float d = reduce_scatter<LPK, RP>(x, db);
            const int j = base + st * KPL + kk;
            // the score is rounded once here and the maximum is taken over the
            // same values, so the largest key gets 2^0 = 1 exactly
            dm[st] = (j < my_lim) ? d * qs : kNegInf;
        }
        float mx = dm[0];
#pragma unroll
        for (int st = 1; st < NSTEP; ++st) mx = fmaxf(mx, dm[st]);
        mx = across_groups_max<LPK>(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        if (__any(m_run != kNegInf && m_new > m_run)) {   // some row's maximum grew
            const float alpha = fast_exp2(m_run - m_use);
            l_run *= alpha;
            float al[8];
            gather_all<LPK, RP>(alpha, al);
#pragma unroll
            for (int k = 0; k < RP; ++k)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[k][e] *= al[k];
        }
        m_run = m_new;
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            const float pj = fast_exp2(dm[st] - m_use);
            l_run += pj;
            float ps[8];
            gather_all<LPK, RP>(pj, ps);
            float vf[8];
            bf16x8_to_f32(vb[st], vf);
            if (base + kKeysPerWave > v_lim) {     // wave-uniform: keys past v_lim were loaded
                const bool in = base + st * KPL + kk < v_lim;
#pragma unroll
                for (int e = 0; e < 8; ++e) vf[e] = in ? vf[e] : 0.f;
            }
#pragma unroll
            for (int k = 0; k < RP; ++k)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[k][e] = __builtin_fmaf(ps[k], vf[e], acc[k][e]);
        }
    };

    auto reset_state = [&]() {
        m_run = kNegInf;
        l_run = 0.f;
#pragma unroll
        for (int k = 0; k < RP; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[k][e] = 0.f;
    };

    // Sum the lane groups of the wave, combine the key waves of the workgroup
    // in LDS and write the tile's partial state. Every wave calls this once per
    // work item, in the same order (a workgroup barrier, and a second one when
    // another item follows: `more`, uniform).
    auto finish = [&](const Tile& tl, bool more) {
        l_run = across_groups_sum<LPK>(l_run);
        // acc summed over the key groups and scattered over the four 16-lane
        // rows: row q ends with dims db*8 + q and db*8 + 4 + q of every slot
        // (for D = 64 both 8-lane halves of a row hold the same sums)
        float flat[RP * 8];
#pragma unroll
        for (int k = 0; k < RP; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e) flat[k * 8 + e] = acc[k][e];
        float red[RP * 2];
        across_groups_sum_scatter<LPK>(flat, red);

        const int slot = (rgl * nwk + kw) * R;
        const int q = lane >> 4;
        if (LPK == 16 || (kk & 1) == 0) {
#pragma unroll
            for (int k = 0; k < RP; ++k) {
                const int row = slot_row[k];
                if (row < R) {
                    float* dst = s_acc + (size_t)(slot + row) * D + db * 8 + q;
                    dst[0] = red[2 * k];
                    dst[4] = red[2 * k + 1];
                }
            }
        }
        if (kk == 0 && (db & ((1 << SET_BITS) - 1)) == 0 && own < R) {
            s_ml[(slot + own) * 2 + 0] = m_run;
            s_ml[(slot + own) * 2 + 1] = l_run;
        }
        __syncthreads();

        // four dims per thread, the key waves folded in a fixed order
        constexpr int Q4 = D / 4;
        const int total = p.rg_per_block * R * Q4;
        const size_t tile_row0 = ((size_t)(tl.b * Hkv + tl.kvh) * p.NC + tl.c) * RT;
        for (int idx = tid; idx < total; idx += blockDim.x) {
            const int rg2 = idx / (R * Q4);
            const int rem = idx - rg2 * (R * Q4);
            const int jr = rem / Q4;
            const int d = (rem - jr * Q4) * 4;
            const int r = (tl.rblk * p.rg_per_block + rg2) * R + jr;
            if (r >= RT) continue;
            const int base_slot = rg2 * nwk * R + jr;     // slot of key wave 0 for this row
            // all key waves' state read at once: waves w >= nwk read wave
            // nwk - 1's slot again (same maximum) and get weight 0, which adds
            // exactly nothing, so the sums are those of the nwk waves in order
            float mw[kMaxKeyWaves], lw[kMaxKeyWaves];
            float4 aw[kMaxKeyWaves];
#pragma unroll
            for (int w = 0; w < kMaxKeyWaves; ++w) {
                const int sl = base_slot + min(w, nwk - 1) * R;
                const float2 ml = *reinterpret_cast<const float2*>(s_ml + sl * 2);
                mw[w] = ml.x;
                lw[w] = ml.y;
                aw[w] = *reinterpret_cast<const float4*>(s_acc + (size_t)sl * D + d);
            }
            float M = mw[0];
#pragma unroll
            for (int w = 1; w < kMaxKeyWaves; ++w) M = fmaxf(M, mw[w]);
            // no key in any wave: weights against 0 are 2^-inf = 0
            const float Mu = (M == kNegInf) ? 0.f : M;
            float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
            float L = 0.f;
#pragma unroll
            for (int w = 0; w < kMaxKeyWaves; ++w) {
                const float wt = w < nwk ? fast_exp2(mw[w] - Mu) : 0.f;
                A.x = __builtin_fmaf(wt, aw[w].x, A.x);
                A.y = __builtin_fmaf(wt, aw[w].y, A.y);
                A.z = __builtin_fmaf(wt, aw[w].z, A.z);
                A.w = __builtin_fmaf(wt, aw[w].w, A.w);
                L = __builtin_fmaf(wt, lw[w], L);
            }
            *reinterpret_cast<float4*>(p.ws_acc + (tile_row0 + r) * D + d) = A;
            if (d == 0) {
                p.ws_ml[(tile_row0 + r) * 2 + 0] = M;
                p.ws_ml[(tile_row0 + r) * 2 + 1] = L;
            }
        }
        if (more) __syncthreads();          // LDS is rewritten by the next item's combine (uniform)
    };

    // ---- one stream of sub-tiles across this workgroup's work items
    // Work items of this workgroup: blockIdx.x, +P, +2P, ... Each item gives a
    // wave SPT slots (sub-tile s at t0 + kw*KPW + s*stride), SPT rounded up to
    // a multiple of kNumBuf; slots at or past the item's last key read nothing
    // (outside the buffer resource) and are not computed. A ring of kNumBuf
    // register slots holds loaded sub-tiles and the load pointer runs
    // kNumBuf-1 slots ahead of the compute pointer, across item boundaries,
    // so the memory pipe stays full from one item to the next; since an item
    // has at least kNumBuf slots, the load pointer is at most one item ahead
    // (one spare set of query registers), and every item ends at the end of a
    // ring cycle, where it is combined.
    if constexpr (ONE_ROUND) {
        // grid (Hkv, NC, B), one row block: the work item is the block index
        Tile tl;
        tl.kvh = blockIdx.x;
        tl.c = blockIdx.y;
        tl.b = blockIdx.z;
        tl.rblk = 0;
        tl.t0 = tl.c * chunk;
        tl.t1 = min(tl.t0 + chunk, S_max);
        int len = lens[tl.b];
        asm volatile("" ::: "memory");      // the length's load leaves first
        const int spt_real = (chunk + sub_stride - 1) >> __builtin_ctz(sub_stride);   // both powers of two
        const int spt = (spt_real + kNumBuf - 1) / kNumBuf * kNumBuf;
        uint4 qc[RP];
        int limc;
        tl.len = 0;
        tl.lim_all = tl.t1;
        load_q(tl, qc, limc);               // the limit is recomputed once the length is known
        // the first kNumBuf sub-tiles are requested over the whole tile (keys
        // up to t1 all lie inside the cache); later ones only up to the
        // attended keys
        Rsrc rs = make_tile_rsrc(tl);
        uint4 kb[kNumBuf][NSTEP], vb[kNumBuf][NSTEP];
        auto slot_base = [&](int s, int lim) {
            return min(s < spt_real ? tl.t0 + kw * kKeysPerWave + s * sub_stride : lim, lim);
        };
#pragma unroll
        for (int u = 0; u < kNumBuf; ++u) load(rs, kb[u], vb[u], slot_base(u, tl.t1));
        // keep those loads ahead of the length's first use: the length passes
        // through here, so nothing computed from it (the exit test for a tile
        // past the length, and the wait for its round trip) moves above them
        asm volatile("" : "+s"(len) : : "memory");

        tl.len = len;
        tl.lim_all = min(clamp_len_add(len, tok_add, S_max), tl.t1);
        if (tl.t0 >= tl.lim_all) return;    // workgroup-uniform: a tile past the length
        {
            const int rg = tl.rblk * p.rg_per_block + rgl;
            const int r0 = rg * R + own;
            const int i = ((r0 < RT ? r0 : 0) * g_magic) >> 16;   // r0 / G
            limc = (own < R && r0 < RT) ? min(clamp_len_add(len, causal ? i + 1 : 0, S_max), tl.t1) : 0;
        }
        rs = make_tile_rsrc(tl);
        reset_state();
        for (int s0 = 0; s0 < spt; s0 += kNumBuf) {
#pragma unroll
            for (int u = 0; u < kNumBuf; ++u) {
                const int base = tl.t0 + kw * kKeysPerWave + (s0 + u) * sub_stride;
                if (s0 + u < spt_real && base < tl.lim_all) compute(qc, limc, kb[u], vb[u], base, tl.lim_all);
                if (s0 + u + kNumBuf < spt) load(rs, kb[u], vb[u], slot_base(s0 + u + kNumBuf, tl.lim_all));
                // the reload stays ahead of the next sub-tile's compute
                if (DECATTN_PREFETCH_FENCE) __builtin_amdgcn_sched_barrier(0);
            }
        }
        finish(tl, false);
        return;
    }

    int c_item = blockIdx.x;
    if (c_item >= n_items) return;          // workgroup-uniform
    const int P = (int)gridDim.x;
    const int spt_real = (chunk + sub_stride - 1) >> __builtin_ctz(sub_stride);   // both powers of two
    const int spt = (spt_real + kNumBuf - 1) / kNumBuf * kNumBuf;

    uint4 kb[kNumBuf][NSTEP], vb[kNumBuf][NSTEP];
    uint4 qc[RP], qn[RP];
    int limc, limn = 0;

    Tile ct = locate(c_item);
    load_q(ct, qc, limc);
    int l_item = c_item;                    // work item of the load pointer
    int l_s = 0;                            // its next slot
    Tile lt = ct;
    Rsrc lrs = make_tile_rsrc(lt);

    auto issue = [&](uint4 (&kd)[NSTEP], uint4 (&vd)[NSTEP]) {
        if (l_s == spt) {                   // the load pointer enters the next item
            l_s = 0;
            l_item += P;
            if (l_item < n_items) {
                lt = locate(l_item);
                lrs = make_tile_rsrc(lt);
                load_q(lt, qn, limn);
            }
        }
        // past the last item, or past the item's keys: reads nothing
        const int base = (l_item < n_items && l_s < spt_real) ? lt.t0 + kw * kKeysPerWave + l_s * sub_stride
                                                              : lt.lim_all;
        load(lrs, kd, vd, min(base, lt.lim_all));
        ++l_s;
    };

    reset_state();
#pragma unroll
    for (int u = 0; u < kNumBuf - 1; ++u) issue(kb[u], vb[u]);

    for (;;) {
        for (int s0 = 0; s0 < spt; s0 += kNumBuf) {
#pragma unroll
            for (int u = 0; u < kNumBuf; ++u) {
                const int nu = (u + kNumBuf - 1) % kNumBuf;     // constant after unrolling
                issue(kb[nu], vb[nu]);
                if (DECATTN_PREFETCH_FENCE) __builtin_amdgcn_sched_barrier(0);
                const int base = ct.t0 + kw * kKeysPerWave + (s0 + u) * sub_stride;
                if (s0 + u < spt_real && base < ct.lim_all) compute(qc, limc, kb[u], vb[u], base, 0x7FFFFFFF);
            }
        }
        finish(ct, c_item + P < n_items);
        c_item += P;
        if (c_item >= n_items) break;
        ct = lt;                            // the load pointer is already in this item
#pragma unroll
        for (int j = 0; j < RP; ++j) qc[j] = qn[j];
        limc = limn;
        reset_state();
    }
}

}  // namespace decattn
