// Causal attention of many query tokens at once (prefill, or a long chunk of
// it) on the matrix cores: the chunk computation of tinydecode's README
// ("speculative decoding": k+1 tokens on top of the context, read in one
// pass) generalised to T in the thousands, the tiled causal attention
// llm-decode-cuda names as its next step.
//
// Row (b, i, h), i < T, attends keys j < min(ctx_b + i + 1, S_max): the same
// operation as chunk_attn, so its results are checked against the same
// oracle. Unlike the decode and verify kernels there is no split over keys:
// T supplies the parallelism, and each workgroup runs whole rows to the end
// with an online softmax, so no partial state or merge is needed.
//
// A workgroup takes one (b, kv head) and 4*PW consecutive positions; each of
// its four waves owns 32 rows = PW positions x G heads (PW = floor(32 / G)),
// so every key and value row read from LDS feeds up to 32 query rows. Per
// tile of 64 keys:
//  * the workgroup loads K and V (16-byte coalesced loads, keys past the
//    workgroup's last limit read as zeros through the buffer range) into the
//    other of two LDS buffers while the waves compute on this one;
//  * scores S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = 16 bytes of one
//    key row from LDS, B = the lane's query row slice held in registers);
//  * per-row mask (only on tiles that cross a row's limit), online softmax in
//    log2 units, row max and sum joined across the two lane halves;
//  * O^T += V^T P^T: V^T read with the transposing LDS load in the key order
//    P has in registers; P as bf16 (bf16 output) or as bf16 hi + lo parts
//    (fp32 output, about 16 bits of P; V is exact in bf16).
// Position blocks are launched heaviest (latest) first, and the blocks of one
// (b, kv head) get block indices congruent modulo B*Hkv, which keeps them on
// one XCD (and its L2) when B*Hkv is a multiple of 8.
#pragma once

#include "verify_kernel.hpp"

namespace decattn {

struct PrefillParams {
    const uint16_t* q;       // [B][T][Hq][D]
    const uint16_t* k;       // [B][Hkv][S_max][D]
    const uint16_t* v;       // [B][Hkv][S_max][D]
    const int32_t* ctx;      // [B]
    void* out;               // [B][T][Hq][D], fp32 or bf16
    int out_bf16;
    int B, T, Hq, Hkv, G, S_max;
    int PW;                  // positions per wave: floor(32 / G)
    int NQB;                 // position blocks per (b, kv head)
    float qscale;            // scale * log2(e), signed
};

// Two shapes of workgroup: 4 waves on 64-key tiles, or 8 waves (256 query
// rows sharing every K/V tile, half the tile traffic) on 128-key tiles, the
// latter when it still gives 512 workgroups. Measured on MI355X (TFLOP/s,
// bf16 output, 4 x 64 / 8 x 128): Llama-3-8B T = 4096 756 / 817, a 2048-token
// chunk after 8192 923 / 992, TinyLlama T = 4096 743 / 787, SmolLM2-360M
// T = 4096 (260 workgroups of 8 waves) 485 / 430.
constexpr int kPrefillMaxKeys = 128;

// LDS row strides in bytes: K rows padded by 16 bytes (the A-operand reads of
// 32 lanes hit 32 rows at one column), V rows by 64 (as the verify kernel's,
// for the transposing reads).
__host__ __device__ constexpr int prefill_krow(int D) { return D * 2 + 16; }
__host__ __device__ constexpr int prefill_vrow(int D) { return D * 2 + 64; }
__host__ __device__ constexpr int prefill_tile_bytes(int D, int KT) {
    return KT * (prefill_krow(D) + prefill_vrow(D));
}
__host__ __device__ constexpr int prefill_lds_bytes(int D, int KT) { return 2 * prefill_tile_bytes(D, KT); }

// A pointer every lane holds the same value of, moved to scalar registers.
__device__ __forceinline__ const uint16_t* uniform_ptr(const uint16_t* ptr) {
    const uint64_t u = reinterpret_cast<uint64_t>(ptr);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
    return reinterpret_cast<const uint16_t*>(((uint64_t)hi << 32) | lo);
}

#ifndef DECATTN_PREFILL_WPE
#define DECATTN_PREFILL_WPE 2
#endif

template <int D, bool SPLIT, int WAVES, int KT>
__global__ void __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(DECATTN_PREFILL_WPE)))
prefill_attn_mfma(const PrefillParams p) {
    constexpr int kPrefillWaves = WAVES;
    constexpr int kPrefillThreads = 64 * WAVES;
    constexpr int KS = D / 16;              // 16-dim steps of the score product
    constexpr int DB = D / 32;              // 32-dim blocks of the output
    constexpr int KBLK = KT / 32;           // 32-key blocks per tile
    constexpr int KROW = prefill_krow(D);
    constexpr int VROW = prefill_vrow(D);
    constexpr int LPR = D / 8;              // 16-byte pieces per key row
    constexpr int PPT = KT * LPR / kPrefillThreads;   // pieces per thread per tensor per tile
    static_assert(D == 64 || D == 128, "head dim 64 or 128");
    static_assert(PPT * kPrefillThreads == KT * LPR, "whole pieces per thread");

    extern __shared__ __align__(16) char lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = lane & 31;                // this lane's query row (B operand / output column)
    const int h = lane >> 5;                // lane half

    const int BH = p.B * p.Hkv;
    const int bh = (int)(blockIdx.x % (unsigned)BH);
    const int qb = p.NQB - 1 - (int)(blockIdx.x / (unsigned)BH);
    const int b = bh / p.Hkv;
    const int kvh = bh - b * p.Hkv;

    const long long craw = p.ctx[b];
    auto lim_of = [&](int i) -> int {
        const long long x = craw + i + 1;
        return x < 0 ? 0 : (x > p.S_max ? p.S_max : (int)x);
    };
    const int pos0 = qb * kPrefillWaves * p.PW;        // < T
    const int wpos0 = pos0 + wave * p.PW;
    const int RW = p.PW * p.G;
    const int ipos = wpos0 + n / p.G;
    const int g = n - (n / p.G) * p.G;
    const bool row_ok = n < RW && ipos < p.T;
    const int lim_n = row_ok ? lim_of(ipos) : 0;
    const bool wave_has = wpos0 < p.T;
    const int lim_wmin = wave_has ? lim_of(wpos0) : 0;                       // fewest keys of the wave's rows
    const int lim_wmax = wave_has ? lim_of(min(wpos0 + p.PW, p.T) - 1) : 0;  // most keys
    // most keys of the workgroup; uniform, and said so: the buffer resources
    // below must sit in scalar registers (a value the compiler takes for
    // divergent would put every K/V load in a waterfall loop)
    const int lim_all = __builtin_amdgcn_readfirstlane(lim_of(min(pos0 + kPrefillWaves * p.PW, p.T) - 1));

    // query slice of this lane's row (idle lanes read the workgroup's first row)
    const int qpos = row_ok ? ipos : pos0;
    const int qhead = kvh * p.G + (row_ok ? g : 0);
    const uint16_t* qrow = p.q + ((size_t)(b * p.T + qpos) * p.Hq + qhead) * D + h * 8;
    uint4 qv[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qv[ks] = *reinterpret_cast<const uint4*>(qrow + ks * 16);

    const size_t head_base = (size_t)bh * p.S_max * D;
    const uint32_t range = (uint32_t)lim_all * D * 2;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(uniform_ptr(p.k + head_base), range);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(uniform_ptr(p.v + head_base), range);

    // this thread's pieces of a tile: key pc / LPR, 16-byte column pc % LPR.
    // LDS holds two K buffers, then two V buffers.
    char* const kbase_lds = lds;
    char* const vbase_lds = lds + 2 * KT * KROW;
    uint4 kst[PPT], vst[PPT];
    auto gload_k = [&](int t) {
#pragma unroll
        for (int r = 0; r < PPT; ++r) {
            const int pc = tid + kPrefillThreads * r;
            kst[r] = buffer_load16_policy<0>(krs, (uint32_t)(t * KT + pc / LPR) * (D * 2) + (pc % LPR) * 16);
        }
    };
    auto gload_v = [&](int t) {
#pragma unroll
        for (int r = 0; r < PPT; ++r) {
            const int pc = tid + kPrefillThreads * r;
            vst[r] = buffer_load16_policy<0>(vrs, (uint32_t)(t * KT + pc / LPR) * (D * 2) + (pc % LPR) * 16);
        }
    };
    auto lstore_k = [&](int buf) {
        char* kt = kbase_lds + buf * (KT * KROW);
#pragma unroll
        for (int r = 0; r < PPT; ++r) {
            const int pc = tid + kPrefillThreads * r;
            *reinterpret_cast<uint4*>(kt + (pc / LPR) * KROW + (pc % LPR) * 16) = kst[r];
        }
    };
    auto lstore_v = [&](int buf) {
        char* vt = vbase_lds + buf * (KT * VROW);
#pragma unroll
        for (int r = 0; r < PPT; ++r) {
            const int pc = tid + kPrefillThreads * r;
            *reinterpret_cast<uint4*>(vt + (pc / LPR) * VROW + (pc % LPR) * 16) = vst[r];
        }
    };

    // transposing-read address of this lane in a V tile (see the verify kernel:
    // lanes 4r..4r+3 of a 16-lane group point at key 4h + r, dims 16*(group%2) + 4*(lane%4))
    const int v_tr_off = (4 * h + ((lane & 15) >> 2)) * VROW + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
    // A negative scale is moved into q: flipping the sign bits of q negates
    // every product and sum exactly, and the exponent argument then takes
    // |scale*log2(e)|. This also makes the q loads complete before the tile
    // loop, so no wait inside it is charged to them.
    const float qs = fabsf(p.qscale);
    const uint32_t qflip = p.qscale < 0.f ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        qv[ks].x ^= qflip; qv[ks].y ^= qflip; qv[ks].z ^= qflip; qv[ks].w ^= qflip;
    }

    // m_run is the row maximum (log2 units) the weights are taken against; it
    // is moved only when a tile's maximum exceeds it by more than kSlack, so
    // weights reach 2^kSlack at most and rescaling is rare. acc and l share
    // the same m_run, so the quotient is unchanged (the online-softmax
    // identity holds for any reference value, not only the running maximum).
    constexpr float kSlack = 8.f;
    float m_run = kNegInf, l_run = 0.f;
    f32x16_t acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

    // raw scores S^T = K Q^T of the K tile in buffer kbuf: the KBLK
    // accumulation chains interleaved
    auto qk = [&](f32x16_t (&st)[KBLK], int kbuf) {
        const char* kt = kbase_lds + kbuf * (KT * KROW);
#pragma unroll
        for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) st[kb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 a[KBLK];
#pragma unroll
            for (int kb = 0; kb < KBLK; ++kb)
                a[kb] = *reinterpret_cast<const uint4*>(kt + (kb * 32 + n) * KROW + (ks * 16 + h * 8) * 2);
#pragma unroll
            for (int kb = 0; kb < KBLK; ++kb)
                st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[kb]), as_bf16x8(qv[ks]), st[kb], 0, 0, 0);
        }
    };

    // softmax of the raw scores of the tile at key k0, then O^T += V^T P^T
    // with the V tile in buffer vbuf
    auto softmax_pv = [&](f32x16_t (&st)[KBLK], int k0, int vbuf) {
        const char* vt = vbase_lds + vbuf * (KT * VROW);
        // keys at or past a row's limit: -inf (only on tiles that cross the
        // smallest limit of the wave's rows; wave-uniform test)
        if (k0 + KT > lim_wmin) {
#pragma unroll
            for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                    st[kb][r] = key < lim_n ? st[kb][r] : kNegInf;
                }
        }
        float mx = st[0][0];
#pragma unroll
        for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
            for (int r = (kb == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, st[kb][r]);
        {
            const f32x2 sw = swap32(mx, mx);
            mx = fmaxf(sw.x, sw.y);
        }
        const float m_tile = mx * qs;                      // -inf stays -inf (qs > 0)
        if (__any(m_tile > m_run + kSlack)) {
            const float m_new = fmaxf(m_run, m_tile);
            const float m_to = (m_new == kNegInf) ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_to);   // 0 while the row had no key
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
            m_run = m_new;
        }
        const float neg_m = (m_run == kNegInf) ? 0.f : -m_run;

        // P = 2^(s*qs - m) as B operands: uint4 j of block kb holds keys
        // 16j + 4h + 0..3 and 16j + 8 + 4h + 0..3 of that block
        uint4 bhi[KBLK][2], blo[KBLK][2];
#pragma unroll
        for (int kb = 0; kb < KBLK; ++kb) {
            float pv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                pv[r] = fast_exp2(__builtin_fmaf(st[kb][r], qs, neg_m));
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

        // O^T += V^T P^T: the DB accumulation chains interleaved
#pragma unroll
        for (int kb = 0; kb < KBLK; ++kb) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                uint4 a[DB];
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const char* ap = vt + v_tr_off + (kb * 32 + j * 16) * VROW + db * 64;
                    const uint2 a0 = lds_read_tr16_b64(ap);
                    const uint2 a1 = lds_read_tr16_b64(ap + 8 * VROW);
                    a[db] = make_uint4(a0.x, a0.y, a1.x, a1.y);
                }
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[db]), as_bf16x8(bhi[kb][j]), acc[db], 0, 0, 0);
                if constexpr (SPLIT) {
#pragma unroll
                    for (int db = 0; db < DB; ++db)
                        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[db]), as_bf16x8(blo[kb][j]), acc[db], 0, 0, 0);
                }
            }
        }
    };

    const int ntiles = (lim_all + KT - 1) / KT;
    // Two buffers each of K and V: tile t+1 is loaded into registers while
    // tile t is computed, then stored into the other buffers; one barrier per
    // tile. The load and store of tile t+1 are issued on every iteration (past
    // the last tile they read zeros and fill buffers nobody reads): a
    // conditional load would leave the compiler unsure how many loads are in
    // flight, and it would then wait for them before the score products.
    gload_k(0);
    gload_v(0);
    lstore_k(0);
    lstore_v(0);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        gload_k(t + 1);
        gload_v(t + 1);
        if (t * KT < lim_wmax) {                             // wave-uniform
            f32x16_t st[KBLK];
            qk(st, t & 1);
            softmax_pv(st, t * KT, t & 1);
        }
        lstore_k((t + 1) & 1);
        lstore_v((t + 1) & 1);
        __syncthreads();
    }

    // rows: join the two halves' sums, normalise, store 4 dims per group
    {
        const f32x2 sw = swap32(l_run, l_run);
        l_run = sw.x + sw.y;
    }
    if (!row_ok) return;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const size_t obase = ((size_t)(b * p.T + ipos) * p.Hq + kvh * p.G + g) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const int dim = db * 32 + 8 * qq + 4 * h;
            const float o0 = acc[db][4 * qq] * inv, o1 = acc[db][4 * qq + 1] * inv;
            const float o2 = acc[db][4 * qq + 2] * inv, o3 = acc[db][4 * qq + 3] * inv;
            if (p.out_bf16) {
                const uint2 packed = make_uint2(
                    (uint32_t)f32_to_bf16_rne(o0) | ((uint32_t)f32_to_bf16_rne(o1) << 16),
                    (uint32_t)f32_to_bf16_rne(o2) | ((uint32_t)f32_to_bf16_rne(o3) << 16));
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + obase + dim) = packed;
            } else {
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + obase + dim) = make_float4(o0, o1, o2, o3);
            }
        }
    }
}

}  // namespace decattn
