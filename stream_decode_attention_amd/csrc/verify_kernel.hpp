// Verify-chunk partial attention on the matrix cores (gfx950 MFMA).
//
// The verify pass of speculative decoding (tinydecode README, "speculative
// decoding") attends T query tokens, each over the cache plus the tokens
// before it, for all G query heads of a kv head: T*G rows share every key and
// value row, so scores and p.V are genuine matrix products (18 rows x 128 dims
// per key at the Llama-3.2-3B shape: about 18 flop per byte read, above what
// the vector ALUs sustain at HBM speed). This kernel computes the same partial
// state (m, l, acc) per tile as split_kv_partial, for up to 32 rows per kv
// head, with v_mfma_f32_32x32x16_bf16:
//
//  * scores as S^T = K Q^T: the A operand of a lane is 16 contiguous bytes of
//    one key row (key = lane % 32, dims 8*(lane/32)..+7 of a 16-dim step), the
//    B operand the same slice of one query row; no transpose of K. Lane l ends
//    with 16 keys of row l % 32 per 32-key block (the other 16 sit in l ^ 32).
//  * softmax on that layout: the mask (key < row limit) and exp2 per element,
//    row maxima and sums joined across the two lane halves by one shuffle;
//    online across sub-tiles, rescaling only when a row maximum grew.
//  * O^T = V^T P^T: V is loaded coalesced and stored row-major in LDS with
//    16-byte writes; the A operand (V^T) is read back with the gfx950
//    transposing LDS load (ds_read_b64_tr_b16), which hands each lane four
//    consecutive keys at one dim, in the key order the S^T registers give P,
//    so the B operand (P) is packed from registers as is. Precision follows
//    the output (SPLIT): for fp32 output P is split into bf16 hi + lo parts
//    (two MFMAs), so the product keeps about 16 bits of P (error below 1e-4),
//    V being exact in bf16; for bf16 output P is rounded once to bf16 (one
//    MFMA; each weight within 2^-9 of itself, under the output's own
//    rounding step).
//  * the four waves of a workgroup split each sub-tile's keys (32 each);
//    sub-tiles stream through a ring of two register buffers, and the waves
//    are combined through LDS into the tile's partial state, written in the
//    decode layout.
//
// Work distribution, lengths and buffer-resource loads as split_kv_partial
// (persistent grid over attended tiles, keys past a limit read as zeros).
//
// Decode mode (causal = 0): every row attends j < seq_len. Decode calls with
// eight or more query heads per kv head run here, where the dot-product
// kernel's vector work per key (G rows x D dims of scores and p.V) would
// outlast the data it waits for.
#pragma once

#include "partial_kernel.hpp"

namespace decattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// K is read in the MFMA operand layout: each load instruction touches 32 bytes
// of 32 key rows, and four instructions share every cache line, so K keeps
// the default cache policy (the line stays in L1 for the other three); V is
// read in whole rows, streamed (non-temporal).
#ifndef DECATTN_VERIFY_K_POLICY
#define DECATTN_VERIFY_K_POLICY 0
#endif

constexpr int kVerifyWaves = 4;
constexpr int kVerifyMaxRows = 32;

// LDS of the cross-wave combine, in floats: per wave RT rows of D + 4 floats
// (the pad staggers the rows over the banks), then (m, l) per wave and row.
__host__ __device__ constexpr int verify_comb_floats(int RT, int D) {
    return kVerifyWaves * RT * (D + 4) + kVerifyWaves * RT * 2;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2v_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Bytes per key row of a wave's V tile in LDS: D bf16 plus 64 bytes, so that
// the eight rows one transposing load touches fall on distinct bank groups.
__host__ __device__ constexpr int verify_vrow(int D) { return D * 2 + 64; }

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 at LDS address p (8-byte aligned). Within each group of 16
// lanes, lane i receives element i%4 of the 8 bytes addressed by lanes
// 4r + i/4, r = 0..3 (checked on gfx950 against four address patterns).
// With lanes 4r..4r+3 pointing at key K+r, dims d0+4q..+3 (q = lane%4), lane i
// gets keys K..K+3 at dim d0+i.
__device__ __forceinline__ uint2 lds_read_tr16_b64(const char* p) {
    const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16_t*)(__attribute__((address_space(3))) char*)p);
    return __builtin_bit_cast(uint2, r);
}

// Leading scalar arguments as for split_kv_partial (preloaded into SGPRs;
// r / G = (r * g_magic) >> 16), then what the query addresses and key limits
// need, also preloaded: G query heads per kv head, and tok_add = T for a
// causal chunk of T tokens (row i attends j < len + i + 1) or 0 for a decode
// call (T = 1, every row attends j < len). These 14 dwords are all the
// hardware preloads, so nothing before the first loads waits for the
// kernel-argument segment.
template <int D, int KB, bool ONE_ROUND, bool SPLIT>
__global__ void __launch_bounds__(256)
verify_partial_mfma(const int32_t* lens, const uint16_t* kc, const uint16_t* vc, const uint16_t* qp, int S_max,
                    int chunk, int Hkv, int g_magic, int G, int tok_add, const PartialParams p) {
    constexpr int KS = D / 16;              // 16-dim steps of the score product
    constexpr int DB = D / 32;              // 32-dim blocks of the output
    constexpr int WK = 32 * KB;             // keys per wave per sub-tile
    constexpr int SUB = kVerifyWaves * WK;  // keys per workgroup sub-tile
    constexpr int LPK = D / 8;              // lanes per key row (coalesced V load)
    constexpr int KPL = 64 / LPK;           // keys per V load
    constexpr int VSTEP = WK / KPL;         // V loads per wave per sub-tile
    constexpr int VROW = verify_vrow(D);    // bytes per key row of a wave's V tile
    static_assert(D == 64 || D == 128, "head dim 64 or 128");
    static_assert(KB == 1 || KB == 2, "32 or 64 keys per wave");

    extern __shared__ float smem[];
    __shared__ int s_count[2 * kVerifyWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = lane & 31;                // row (B/D operand) or key (A operand) index
    const int h = lane >> 5;                // lane half
    char* vt = reinterpret_cast<char*>(smem) + (size_t)wave * WK * VROW;
    // this lane's byte offsets in the V tile: its 16-byte store (key lane/LPK
    // of a load, dims 8*(lane%LPK)..+7) and its transposing-read address
    // (group g = lane/16, i = lane%16: key 4*(lane/32) + i/4, dims
    // 16*(g%2) + 4*(i%4)..+3; the step, block and 8-key half add constants)
    const int v_st_off = (lane / LPK) * VROW + (lane % LPK) * 16;
    const int v_tr_off = (4 * h + ((lane & 15) >> 2)) * VROW + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
    const int T = tok_add > 0 ? tok_add : 1;                     // query tokens
    const int RT = T * G;                                        // rows per kv head
    constexpr int CST = D + 4;                                   // combine row stride (floats)
    // the combine area follows the V tiles (no aliasing), so a wave stores its
    // state as soon as its own last sub-tile is done, with no barrier first
    float* c_acc = smem + (size_t)kVerifyWaves * WK * VROW / sizeof(float);   // [waves][RT][CST]
    float* c_ml = c_acc + (size_t)kVerifyWaves * RT * CST;     // [waves][RT][2]
    int* s_len = reinterpret_cast<int*>(reinterpret_cast<char*>(smem) + p.lds_main);

    // One work item per attended tile (keys j < ctx + T) of every (b, kvh);
    // when that leaves a few items for a second round of workgroups and
    // taking every short last tile (at most a quarter chunk) with the tile
    // before it does not, those tiles are folded: the item before computes
    // them too (one more sub-tile, already in flight by then) and writes an
    // empty state (m = -inf, l = 0, acc = 0) into the folded tile's slot, so
    // the merge still reads, for every row, slots that partition exactly the
    // keys that row attends.
    const int csh = __builtin_ctz(chunk);     // chunk is a power of two
    const bool causal = tok_add != 0;         // a causal chunk (tok_add = T >= 1) or a decode call (0)
    // keys a row may attend: j < ctx + i + 1 for a causal chunk (row i), j < len
    // for a decode call (and a non-causal chunk)
    auto tiles_raw = [&](int len) { return (clamp_len_add(len, tok_add, S_max) + chunk - 1) >> csh; };
    auto short_tail = [&](int len) {
        const int lim = clamp_len_add(len, tok_add, S_max);
        const int na = (lim + chunk - 1) >> csh;
        return na >= 2 && 4 * (lim - ((na - 1) << csh)) <= chunk;
    };

    // This lane's row (n) and its query slice for the B operand. Lanes past
    // the last row load row 0 (all loads issue back to back with no branch)
    // and are masked by a key limit of 0.
    const bool row_ok = n < RT;
    const int nr = row_ok ? n : 0;
    const int i = (nr * g_magic) >> 16;   // nr / G
    const float qs = p.qscale;
    auto load_q = [&](int b, int kvh, uint4 (&qv)[KS]) {
        const uint16_t* qrow = qp + ((size_t)(b * T + i) * (G * Hkv) + kvh * G + (nr - i * G)) * D + h * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qv[ks] = *reinterpret_cast<const uint4*>(qrow + ks * 16);
    };

    // One work item: tile c of (b, kvh), which holds at least one attended
    // key; a folded item also takes the tile after it. `more`: the workgroup
    // has another item, whose combine rewrites the LDS.
    auto process = [&](int b, int kvh, int c, int len, bool folded, const uint4 (&qv)[KS], bool more) {
        const int lim_head = clamp_len_add(len, tok_add, S_max);
        const int t0 = c << csh;
        const int t1 = folded ? lim_head : min(t0 + chunk, S_max);
        const int lim_all = min(lim_head, t1);
        const int lim_n = row_ok ? min(clamp_len_add(len, causal ? i + 1 : 0, S_max), t1) : 0;
        const int lim_min = min(clamp_len_add(len, causal ? 1 : 0, S_max), t1);   // row i = 0 attends the fewest

        const size_t head_base = (size_t)(b * Hkv + kvh) * S_max * D;
        const uint32_t range = (uint32_t)lim_all * D * 2;
        const __amdgpu_buffer_rsrc_t krs = make_rsrc(kc + head_base, range);
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vc + head_base, range);

        float m_run = kNegInf, l_run = 0.f;
        f32x16_t acc[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

        // Sub-tiles of SUB keys (WK per wave) stream through a ring of two
        // register buffers: the next sub-tile's loads are in flight while the
        // current one is computed.
        uint4 vr[2][VSTEP];
        uint4 kr[2][KB][KS];
        auto load = [&](uint4 (&vd)[VSTEP], uint4 (&kd)[KB][KS], int sub) {
            const int kbase = sub + wave * WK;
            // V first (coalesced, 16 bytes per lane), then K in the A-operand layout
#pragma unroll
            for (int st = 0; st < VSTEP; ++st)
                vd[st] = buffer_load16(vrs, (uint32_t)(kbase + st * KPL + lane / LPK) * (D * 2) + (lane % LPK) * 16);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    kd[kb][ks] = buffer_load16_policy<DECATTN_VERIFY_K_POLICY>(krs, (uint32_t)(kbase + kb * 32 + n) * (D * 2) + ks * 32 + h * 16);
            __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the compute that follows
        };
        auto compute = [&](const uint4 (&vr)[VSTEP], const uint4 (&kr)[KB][KS], int sub) {
            const int kbase = sub + wave * WK;
            // V into this wave's LDS tile, row-major
#pragma unroll
            for (int st = 0; st < VSTEP; ++st)
                *reinterpret_cast<uint4*>(vt + v_st_off + st * KPL * VROW) = vr[st];

            // scores S^T = K Q^T, scaled to log2 units and masked per row
            float s[KB][16];
            float mx = kNegInf;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                f32x16_t st16;
#pragma unroll
                for (int r = 0; r < 16; ++r) st16[r] = 0.f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    st16 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kr[kb][ks]), as_bf16x8(qv[ks]), st16, 0, 0, 0);
                if (kbase + WK <= lim_min) {        // wave-uniform: every row attends every key here
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        s[kb][r] = st16[r] * qs;
                        mx = fmaxf(mx, s[kb][r]);
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kbase + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                        s[kb][r] = key < lim_n ? st16[r] * qs : kNegInf;
                        mx = fmaxf(mx, s[kb][r]);
                    }
                }
            }
            {
                const f32x2 sw = swap32(mx, mx);    // the other lane half's maximum, in VALU
                mx = fmaxf(sw.x, sw.y);
            }
            const float m_new = fmaxf(m_run, mx);
            const float m_use = (m_new == kNegInf) ? 0.f : m_new;
            if (__any(m_run != kNegInf && m_new > m_run)) {
                const float alpha = fast_exp2(m_run - m_use);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
            }
            m_run = m_new;

            // P = 2^(s - m) as bf16 (hi), plus the rounding remainder as bf16
            // (lo) when SPLIT, packed as B operands
            uint4 bhi[KB][2], blo[KB][2];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                float pv[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    pv[r] = fast_exp2(s[kb][r] - m_use);
                    l_run += pv[r];
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    uint32_t hw[4], lw[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float a0 = pv[8 * j + 2 * e], a1 = pv[8 * j + 2 * e + 1];
                        hw[e] = pack_bf16x2(a0, a1);
                        if constexpr (SPLIT)
                            lw[e] = pack_bf16x2(a0 - __uint_as_float(hw[e] << 16),
                                                a1 - __uint_as_float(hw[e] & 0xFFFF0000u));
                    }
                    bhi[kb][j] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
                    if constexpr (SPLIT) blo[kb][j] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
                }
            }

            // O^T += V^T P^T (transposing reads of this wave's own LDS tile, after its writes)
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int db = 0; db < DB; ++db) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        // keys 16j + 4h + 0..3 and 16j + 8 + 4h + 0..3 of block kb at
                        // dim 32db + lane%32: the order P has in registers
                        const char* ap = vt + v_tr_off + (kb * 32 + j * 16) * VROW + db * 64;
                        const uint2 a0 = lds_read_tr16_b64(ap);
                        const uint2 a1 = lds_read_tr16_b64(ap + 8 * VROW);
                        const uint4 a = make_uint4(a0.x, a0.y, a1.x, a1.y);
                        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(bhi[kb][j]), acc[db], 0, 0, 0);
                        if constexpr (SPLIT)
                            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(blo[kb][j]), acc[db], 0, 0, 0);
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();     // the next sub-tile rewrites the V tile
        };

        // The loads are issued without a condition (keys at or past lim_all
        // are outside the buffer resource and read nothing): a load skipped on
        // one path would leave the compiler unable to count the loads still
        // in flight, and it would then wait for the next sub-tile's as well.
        load(vr[0], kr[0], t0);                 // t0 < lim_all: the item holds an attended key
        for (int sub = t0; sub < lim_all; sub += 2 * SUB) {
            load(vr[1], kr[1], sub + SUB);
            compute(vr[0], kr[0], sub);
            if (sub + SUB >= lim_all) break;
            load(vr[0], kr[0], sub + 2 * SUB);
            compute(vr[1], kr[1], sub + SUB);
        }

        // ---- combine the waves
        {
            const f32x2 sw = swap32(l_run, l_run);
            l_run = sw.x + sw.y;
        }
        if (row_ok) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int dim = db * 32 + 8 * g4 + 4 * h;
                    *reinterpret_cast<float4*>(c_acc + ((size_t)wave * RT + n) * CST + dim) =
                        make_float4(acc[db][4 * g4], acc[db][4 * g4 + 1], acc[db][4 * g4 + 2], acc[db][4 * g4 + 3]);
                }
            if (h == 0) {
                c_ml[(wave * RT + n) * 2 + 0] = m_run;
                c_ml[(wave * RT + n) * 2 + 1] = l_run;
            }
        }
        __syncthreads();
        const size_t tile_row0 = ((size_t)(b * Hkv + kvh) * p.NC + c) * RT;
        // each thread takes four dims of one row and joins the waves itself:
        // their common maximum, weights and summed l come from the row's
        // (m, l) in LDS (recomputed per thread, so no further barrier); the
        // thread holding a row's first dims writes the row's (M, L)
        for (int idx = tid; idx < RT * (D / 4); idx += blockDim.x) {
            const int r = idx / (D / 4);
            const int d = (idx - r * (D / 4)) * 4;
            float M = kNegInf;
#pragma unroll
            for (int w = 0; w < kVerifyWaves; ++w) M = fmaxf(M, c_ml[(w * RT + r) * 2]);
            float L = 0.f;
            float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int w = 0; w < kVerifyWaves; ++w) {
                const float wt = M == kNegInf ? 0.f : fast_exp2(c_ml[(w * RT + r) * 2] - M);
                const float4 a = *reinterpret_cast<const float4*>(c_acc + ((size_t)w * RT + r) * CST + d);
                L = __builtin_fmaf(wt, c_ml[(w * RT + r) * 2 + 1], L);
                A.x = __builtin_fmaf(wt, a.x, A.x);
                A.y = __builtin_fmaf(wt, a.y, A.y);
                A.z = __builtin_fmaf(wt, a.z, A.z);
                A.w = __builtin_fmaf(wt, a.w, A.w);
            }
            *reinterpret_cast<float4*>(p.ws_acc + (tile_row0 + r) * D + d) = A;
            if (d == 0) {
                p.ws_ml[(tile_row0 + r) * 2 + 0] = M;
                p.ws_ml[(tile_row0 + r) * 2 + 1] = L;
                if (folded) {               // the folded tile's slot: an empty state
                    p.ws_ml[(tile_row0 + RT + r) * 2 + 0] = kNegInf;
                    p.ws_ml[(tile_row0 + RT + r) * 2 + 1] = 0.f;
                }
            }
        }
        if (folded)
            for (int idx = tid; idx < RT * (D / 4); idx += blockDim.x)
                *reinterpret_cast<float4*>(p.ws_acc + (tile_row0 + RT) * D + idx * 4) = make_float4(0.f, 0.f, 0.f, 0.f);
        if (more) __syncthreads();       // LDS is rewritten by the next item (uniform test)
    };

    if constexpr (ONE_ROUND) {
        // grid (Hkv, NC, B), every possible tile at once: the work item is the
        // block index (no lengths staged, no counting, no folding). The
        // length's load and the query loads (whose addresses need only the
        // preloaded leading arguments) are issued together at wave start.
        const int kvh = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
        const int len = lens[b];
        uint4 qv[KS];
        load_q(b, kvh, qv);
        asm volatile("" ::: "memory");   // both loads before the length's first use
        if ((c << csh) >= clamp_len_add(len, tok_add, S_max)) return;   // workgroup-uniform: past the length
        process(b, kvh, c, len, false, qv, false);
        return;
    }

    // ---- lengths into LDS; count attended tiles, with and without folding
    int my_raw = 0, my_short = 0;
    for (int i = tid; i < p.B; i += blockDim.x) {
        const int len = lens[i];
        s_len[i] = len;
        my_raw += tiles_raw(len);
        my_short += short_tail(len) ? 1 : 0;
    }
    my_raw = wave_sum_i(my_raw);
    my_short = wave_sum_i(my_short);
    if (lane == 0) {
        s_count[wave] = my_raw;
        s_count[kVerifyWaves + wave] = my_short;
    }
    __syncthreads();
    int n_raw = 0, n_short = 0;
#pragma unroll
    for (int w = 0; w < kVerifyWaves; ++w) {
        n_raw += s_count[w];
        n_short += s_count[kVerifyWaves + w];
    }
    const int P = (int)gridDim.x;
    const bool fold = (n_raw * Hkv + P - 1) / P > ((n_raw - n_short) * Hkv + P - 1) / P;
    const int n_items = (fold ? n_raw - n_short : n_raw) * Hkv;
    auto tiles_of = [&](int b) { return tiles_raw(s_len[b]) - (fold && short_tail(s_len[b]) ? 1 : 0); };
    int b_cur = 0, pre_cur = 0;

    for (int item = blockIdx.x; item < n_items; item += P) {
        // locate (b, kvh, tile); items are b-major, the walk only moves forward
        while (item >= pre_cur + tiles_of(b_cur) * Hkv) {
            pre_cur += tiles_of(b_cur) * Hkv;
            ++b_cur;
        }
        const int b = b_cur;
        const int na = tiles_of(b);
        const int u = item - pre_cur;
        const int c = u % na;
        const int kvh = u / na;
        const int len = s_len[b];
        const bool folded = c == na - 1 && fold && short_tail(len);   // also takes the tile after it
        uint4 qv[KS];
        load_q(b, kvh, qv);
        process(b, kvh, c, len, folded, qv, item + P < n_items);
    }
}

}  // namespace decattn
