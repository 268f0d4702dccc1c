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

constexpr int kPrefillWaves = 4;
constexpr int kPrefillKeys = 64;         // keys per tile

// LDS row strides in bytes: K rows padded by 16 bytes (the A-operand reads of
// 32 lanes hit 32 rows at one column), V rows by 64 (as the verify kernel's,
// for the transposing reads).
__host__ __device__ constexpr int prefill_krow(int D) { return D * 2 + 16; }
__host__ __device__ constexpr int prefill_vrow(int D) { return D * 2 + 64; }
__host__ __device__ constexpr int prefill_tile_bytes(int D) {
    return kPrefillKeys * (prefill_krow(D) + prefill_vrow(D));
}
__host__ __device__ constexpr int prefill_lds_bytes(int D) { return 2 * prefill_tile_bytes(D); }

template <int D, bool SPLIT>
__global__ void __launch_bounds__(256)
prefill_attn_mfma(const PrefillParams p) {
    constexpr int KS = D / 16;              // 16-dim steps of the score product
    constexpr int DB = D / 32;              // 32-dim blocks of the output
    constexpr int KT = kPrefillKeys;
    constexpr int KBLK = KT / 32;           // 32-key blocks per tile
    constexpr int KROW = prefill_krow(D);
    constexpr int VROW = prefill_vrow(D);
    constexpr int TILE = prefill_tile_bytes(D);
    constexpr int LPR = D / 8;              // 16-byte pieces per key row
    constexpr int PPT = KT * LPR / 256;     // pieces per thread per tensor per tile
    static_assert(D == 64 || D == 128, "head dim 64 or 128");
    static_assert(PPT * 256 == KT * LPR, "whole pieces per thread");

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
    const int lim_all = lim_of(min(pos0 + kPrefillWaves * p.PW, p.T) - 1);   // most keys of the workgroup

    // query slice of this lane's row (idle lanes read the workgroup's first row)
    const int qpos = row_ok ? ipos : pos0;
    const int qhead = kvh * p.G + (row_ok ? g : 0);
    const uint16_t* qrow = p.q + ((size_t)(b * p.T + qpos) * p.Hq + qhead) * D + h * 8;
    uint4 qv[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qv[ks] = *reinterpret_cast<const uint4*>(qrow + ks * 16);

    const size_t head_base = (size_t)(b * p.Hkv + kvh) * p.S_max * D;
    const uint32_t range = (uint32_t)lim_all * D * 2;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k + head_base, range);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v + head_base, range);

    // this thread's pieces of a tile: key pc / LPR, 16-byte column pc % LPR
    uint4 kst[PPT], vst[PPT];
    auto gload = [&](int t) {
#pragma unroll
        for (int r = 0; r < PPT; ++r) {
            const int pc = tid + 256 * r;
            const uint32_t off = (uint32_t)(t * KT + pc / LPR) * (D * 2) + (pc % LPR) * 16;
            kst[r] = buffer_load16_policy<0>(krs, off);
            vst[r] = buffer_load16_policy<0>(vrs, off);
        }
    };
    auto lstore = [&](int buf) {
        char* kt = lds + buf * TILE;
        char* vt = kt + KT * KROW;
#pragma unroll
        for (int r = 0; r < PPT; ++r) {
            const int pc = tid + 256 * r;
            *reinterpret_cast<uint4*>(kt + (pc / LPR) * KROW + (pc % LPR) * 16) = kst[r];
            *reinterpret_cast<uint4*>(vt + (pc / LPR) * VROW + (pc % LPR) * 16) = vst[r];
        }
    };

    // transposing-read address of this lane in a V tile (see the verify kernel:
    // lanes 4r..4r+3 of a 16-lane group point at key 4h + r, dims 16*(group%2) + 4*(lane%4))
    const int v_tr_off = (4 * h + ((lane & 15) >> 2)) * VROW + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
    const float qs = p.qscale;

    float m_run = kNegInf, l_run = 0.f;
    f32x16_t acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

    auto compute = [&](int buf, int k0) {
        const char* kt = lds + buf * TILE;
        const char* vt = kt + KT * KROW;
        float s[KBLK][16];
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < KBLK; ++kb) {
            f32x16_t st;
#pragma unroll
            for (int r = 0; r < 16; ++r) st[r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const uint4 a = *reinterpret_cast<const uint4*>(kt + (kb * 32 + n) * KROW + (ks * 16 + h * 8) * 2);
                st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qv[ks]), st, 0, 0, 0);
            }
            const int kbase = k0 + kb * 32;
            if (kbase + 32 <= lim_wmin) {           // wave-uniform: every row of the wave attends every key
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    s[kb][r] = st[r] * qs;
                    mx = fmaxf(mx, s[kb][r]);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kbase + 8 * (r >> 2) + 4 * h + (r & 3);
                    s[kb][r] = key < lim_n ? st[r] * qs : kNegInf;
                    mx = fmaxf(mx, s[kb][r]);
                }
            }
        }
        {
            const f32x2 sw = swap32(mx, mx);
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

        // P = 2^(s - m) as B operands: uint4 j of block kb holds keys
        // 16j + 4h + 0..3 and 16j + 8 + 4h + 0..3 of that block
        uint4 bhi[KBLK][2], blo[KBLK][2];
#pragma unroll
        for (int kb = 0; kb < KBLK; ++kb) {
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

        // O^T += V^T P^T
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int kb = 0; kb < KBLK; ++kb) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
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
    };

    // two LDS buffers: tile t+1 is loaded into registers while tile t is
    // computed, then stored into the other buffer; one barrier per tile
    const int ntiles = (lim_all + KT - 1) / KT;
    if (ntiles > 0) {
        gload(0);
        lstore(0);
    }
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        if (t + 1 < ntiles) gload(t + 1);
        if (t * KT < lim_wmax) compute(t & 1, t * KT);      // wave-uniform
        if (t + 1 < ntiles) lstore((t + 1) & 1);
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
