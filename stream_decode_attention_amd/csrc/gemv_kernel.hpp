// The weight products of a decode step: y[b, n] = sum_k W[n, k] x[b, k] for
// a few activation vectors (B <= 8), W row-major [N][K] in bf16 or as INT8
// with one fp32 scale per output row (llm-decode-cuda: roofline paragraph,
// GEMV table and INT8 section). Every weight is read once per call and used
// for 2*B flops, so the kernel is bound by HBM bytes.
//
// A group of LPR lanes (16, 32 or 64, chosen from K) owns one output row at a
// time; each lane reads 16-byte chunks c = lane_in_group + LPR*i of the row
// (8 bf16 or 16 INT8 weights), eight chunks in flight before any is used. The
// activations are staged once per workgroup in LDS (zero-padded to whole
// chunk rounds, so the tail needs no branch) and read back as 16-byte pieces
// that line up with the lane's chunks. Products accumulate in fp32 with
// v_dot2c_f32_bf16; INT8 weights are widened once per chunk to bf16 pairs
// (exact for |q| <= 127) and reused for all B vectors, so a larger batch adds
// only the dot products (the fix the INT8 section names for its batch-4
// slowdown). Row sums are joined across the group with DPP and lane swaps;
// the group's first lane applies the row scale and stores y. The grid is
// persistent: every wave walks row groups wave, wave + all waves, ...
//
// By default this dot-product kernel serves one vector (bf16 matrices of
// 16384 rows or more excepted) and the matrix-core kernel further down every
// B from 2; the kernel itself takes up to 8 vectors (raising
// DECATTN_GEMV_MFMA_MIN_B_* hands them to it, the setting the rows-per-group
// rule below was measured in).
#pragma once

#include "device_common.hpp"

namespace decattn {

struct GemvParams {
    const void* W;            // bf16 [N][K] or int8 [N][K]
    const float* scale;       // [N], INT8 weights only
    const uint16_t* x;        // bf16 [B][K]
    void* y;                  // [B][N], fp32 or bf16
    int out_bf16;
    int N, K;
    int KC;                   // 16-byte chunks per weight row
    int KCP;                  // chunks per row padded to a multiple of LPR
    int xrow;                 // bf16 elements per staged activation row in LDS
};

constexpr int kGemvThreads = 512;
constexpr int kGemvUnroll = 8;        // chunks per lane in flight

template <int LPR>
__device__ __forceinline__ float gemv_group_sum(float v) {
    static_assert(LPR == 16 || LPR == 32 || LPR == 64, "16, 32 or 64 lanes per row");
    v = group_sum<16>(v);
    if constexpr (LPR >= 32) {
        const f32x2 a = swap16(v, v);           // [r0, r0, r2, r2] and [r1, r1, r3, r3]
        v = a.x + a.y;
    }
    if constexpr (LPR == 64) {
        const f32x2 a = swap32(v, v);
        v = a.x + a.y;
    }
    return v;
}

// INT8 weights: 16 codes in a uint4 -> eight packed bf16 pairs (exact:
// |q| <= 127 has at most 7 significant bits). Each code is one conversion
// reading its byte sign-extended in place (SDWA); one byte permute then keeps
// the upper halves of the two floats, the pair's bf16 bits.
__device__ __forceinline__ uint32_t int8x2_to_bf16x2(uint32_t w, int shift) {
    const float lo = (float)(int)(int8_t)(w >> shift);
    const float hi = (float)(int)(int8_t)(w >> (shift + 8));
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Rows each lane group works on at once, so that every activation piece read
// from LDS serves RB weight rows. Measured on MI355X over one Llama-3-8B
// layer: two rows at B = 2 (both types) and for INT8 at B >= 3 (+18% at
// B = 4 and 8 against one row); bf16 at B >= 3 keeps one row (two or four
// rows cost registers, hence waves, and ran 0-25% slower). Weight loads are
// non-temporal: +11% on bf16 against the default policy.
#ifndef DECATTN_GEMV_RB_BF16
#define DECATTN_GEMV_RB_BF16 1
#endif
#ifndef DECATTN_GEMV_RB_INT8
#define DECATTN_GEMV_RB_INT8 2
#endif
#ifndef DECATTN_GEMV_POLICY
#define DECATTN_GEMV_POLICY 2
#endif
template <int B, bool INT8>
__host__ __device__ constexpr int gemv_rows_per_group() {
    return B == 1 ? 1 : (B == 2 ? 2 : (INT8 ? DECATTN_GEMV_RB_INT8 : DECATTN_GEMV_RB_BF16));
}

template <int LPR, int B, bool INT8>
__global__ void __launch_bounds__(kGemvThreads)
gemv_kernel(const GemvParams p) {
    constexpr int RB = gemv_rows_per_group<B, INT8>();
    // one vector: four independent accumulation chains per row (the dot
    // products of a chunk alternate between them), so a lane's products do
    // not wait on each other; several vectors already give several chains
    constexpr int NCH = B == 1 ? 4 : 1;
    constexpr int U = kGemvUnroll / RB;             // chunk rounds in flight per row
    constexpr int RPW = 64 / LPR;                   // lane groups per wave
    constexpr int EPC = INT8 ? 16 : 8;              // weights per chunk
    extern __shared__ __align__(16) uint16_t xs[];  // [B][xrow]

    // stage x (zero-padded to KCP chunks)
    const int xelems = p.KCP * EPC;
    for (int b = 0; b < B; ++b) {
        for (int e = threadIdx.x * 8; e < xelems; e += kGemvThreads * 8) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (e < p.K) v = *reinterpret_cast<const uint4*>(p.x + (size_t)b * p.K + e);
            *reinterpret_cast<uint4*>(xs + b * p.xrow + e) = v;
        }
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int sub = lane % LPR;
    const int grp = lane / LPR;
    const int waves_total = (int)gridDim.x * (kGemvThreads / 64);
    const int wave_id = (int)blockIdx.x * (kGemvThreads / 64) + (int)(threadIdx.x >> 6);
    const int rows_per_wave = RPW * RB;
    const int groups = (p.N + rows_per_wave - 1) / rows_per_wave;
    const uint32_t row_bytes = (uint32_t)p.KC * 16;
    // weights are read once: streamed (non-temporal) through one buffer
    // resource over all of W, whose range also zero-fills reads past the end
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(p.W, (uint32_t)((size_t)p.N * row_bytes));

    for (int g = wave_id; g < groups; g += waves_total) {
        // lane group grp owns rows base + grp + RPW * r, r < RB
        const int base = g * rows_per_wave;
        float acc[RB][B][NCH];
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int b = 0; b < B; ++b)
#pragma unroll
                for (int h = 0; h < NCH; ++h) acc[r][b][h] = 0.f;

        for (int c0 = 0; c0 < p.KCP; c0 += LPR * U) {
            uint4 w[RB][U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                // rounds past the padded row are not loaded (uniform test):
                // they would read the next rows again
                if (c0 + u * LPR >= p.KCP) break;
                const int c = c0 + u * LPR + sub;
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    const int row = base + grp + RPW * r;
                    // rows past N read past the buffer's end: zeros
                    w[r][u] = buffer_load16_policy<DECATTN_GEMV_POLICY>(wrs, (uint32_t)row * row_bytes + (uint32_t)c * 16);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (c0 + u * LPR >= p.KCP) break;           // uniform: past the padded row
                const int c = c0 + u * LPR + sub;
                const bool in_row = c < p.KC;               // padded tail: the next row's bytes
                if constexpr (!INT8) {
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const uint4 xv = *reinterpret_cast<const uint4*>(xs + b * p.xrow + c * 8);
#pragma unroll
                        for (int r = 0; r < RB; ++r) {
                            // the padded tail holds the next row's bf16 weights, which
                            // may be non-finite: zeroed, not multiplied by x = 0
                            const uint4 wv = in_row ? w[r][u] : make_uint4(0, 0, 0, 0);
                            float* a = acc[r][b];
                            a[0] = dot2_bf16(wv.x, xv.x, a[0]);
                            a[1 % NCH] = dot2_bf16(wv.y, xv.y, a[1 % NCH]);
                            a[2 % NCH] = dot2_bf16(wv.z, xv.z, a[2 % NCH]);
                            a[3 % NCH] = dot2_bf16(wv.w, xv.w, a[3 % NCH]);
                        }
                    }
                } else {
                    uint32_t wb[RB][8];
                    (void)in_row;   // the padded tail's codes are finite and meet x = 0 (staged as zeros)
#pragma unroll
                    for (int r = 0; r < RB; ++r) {
                        const uint4 wv = w[r][u];
                        const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            wb[r][2 * i] = int8x2_to_bf16x2(wd[i], 0);
                            wb[r][2 * i + 1] = int8x2_to_bf16x2(wd[i], 16);
                        }
                    }
#pragma unroll
                    for (int b = 0; b < B; ++b) {
                        const uint4 x0 = *reinterpret_cast<const uint4*>(xs + b * p.xrow + c * 16);
                        const uint4 x1 = *reinterpret_cast<const uint4*>(xs + b * p.xrow + c * 16 + 8);
#pragma unroll
                        for (int r = 0; r < RB; ++r) {
                            float* a = acc[r][b];
                            a[0] = dot2_bf16(wb[r][0], x0.x, a[0]);
                            a[1 % NCH] = dot2_bf16(wb[r][1], x0.y, a[1 % NCH]);
                            a[2 % NCH] = dot2_bf16(wb[r][2], x0.z, a[2 % NCH]);
                            a[3 % NCH] = dot2_bf16(wb[r][3], x0.w, a[3 % NCH]);
                            a[0] = dot2_bf16(wb[r][4], x1.x, a[0]);
                            a[1 % NCH] = dot2_bf16(wb[r][5], x1.y, a[1 % NCH]);
                            a[2 % NCH] = dot2_bf16(wb[r][6], x1.z, a[2 % NCH]);
                            a[3 % NCH] = dot2_bf16(wb[r][7], x1.w, a[3 % NCH]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
#pragma unroll
            for (int b = 0; b < B; ++b) {
                float t = acc[r][b][0];
                if constexpr (NCH == 4) t = (acc[r][b][0] + acc[r][b][1]) + (acc[r][b][2] + acc[r][b][3]);
                acc[r][b][0] = gemv_group_sum<LPR>(t);
            }
            const int row = base + grp + RPW * r;
            if (sub == 0 && row < p.N) {
                const float sc = INT8 ? p.scale[row] : 1.f;
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const float v = INT8 ? acc[r][b][0] * sc : acc[r][b][0];
                    const size_t o = (size_t)b * p.N + row;
                    if (p.out_bf16) reinterpret_cast<uint16_t*>(p.y)[o] = f32_to_bf16_rne(v);
                    else reinterpret_cast<float*>(p.y)[o] = v;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Matrix-core path for two or more vectors: y^T = W x^T as
// 16 x 16 x 32 bf16 products (v_mfma_f32_16x16x32_bf16): 16 weight rows by
// 32 k times 32 k by 16 vectors (columns past B are zero). Each activation
// fragment then serves 16 weight rows, where the dot-product path reads it
// once per row and is bound by those reads from B = 2; the multiplies cost
// nothing next to the weight stream.
//
// A workgroup of 8 waves owns 16 * RT rows (RT = 1 or 2 tiles of 16 rows);
// the waves split K into 8 ranges of 128-byte blocks, and the 8 partial
// 16 x 16 results are summed in a fixed order through LDS. Activation
// fragments (vector lane % 16, 8 k per lane) come straight from L2. Masked lanes (k past K, vectors past B,
// blocks past the wave's range) read at the end of a buffer resource's
// range, which returns zeros (the host keeps every range and offset + 16
// below 2^32): every load is issued without a branch. INT8 codes are widened
// to exact bf16 as the fragments are read.
typedef __bf16 gemv_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float gemv_f32x4_t __attribute__((ext_vector_type(4)));

// Measured on MI355X over one Llama-3-8B layer (us per layer, dot-product
// path / matrix cores): bf16 B = 2 80.6 / 75.4, B = 4 90.8 / 76.1, B = 8
// 100.8 / 79.7; INT8 B = 2 54.8 / 53.8, B = 4 67.0 / 54.9. At B = 1 the
// dot products win on matrices of fewer rows (Llama-3-8B's 6144 x 4096:
// 10.8 / 13.0; the matrix-core grid is N / 16 workgroups, 1.5 per CU there).
#ifndef DECATTN_GEMV_MFMA_MIN_B_BF16
#define DECATTN_GEMV_MFMA_MIN_B_BF16 2
#endif
// bf16 matrices of this many rows take the matrix cores at B = 1 too: over
// one Llama-3-8B layer (four products, the 28672-row gate/up the only one
// this large) 80.0 -> 74.4 us; from 4096 or 6144 rows 76.1 / 76.8 us, the
// 6144 x 4096 product alone 10.7 -> 13.0 us.
#ifndef DECATTN_GEMV_MFMA_B1_MIN_N
#define DECATTN_GEMV_MFMA_B1_MIN_N 16384
#endif
#ifndef DECATTN_GEMV_MFMA_MIN_B_INT8
#define DECATTN_GEMV_MFMA_MIN_B_INT8 2
#endif
// INT8 rows from N = 8192 up take two 16-row tiles per workgroup (RT = 2),
// which halves the activation-fragment loads per weight byte: B = 8 on
// MI355X, 28672 x 4096 34.6 -> 29.2 us, 14336 x 4096 19.0 -> 16.8 us,
// 8192 x 8192 20.4 -> 18.3 us; below 8192 rows the halved grid loses what
// that gains. bf16 keeps one tile: two cost registers (104, 4 waves per
// SIMD instead of 7) and ran 19% slower on 28672 x 4096.
#ifndef DECATTN_GEMV_MFMA_RT2_MIN_N_INT8
#define DECATTN_GEMV_MFMA_RT2_MIN_N_INT8 8192
#endif
#ifndef DECATTN_GEMV_MFMA_WAVES
#define DECATTN_GEMV_MFMA_WAVES 8
#endif
constexpr int kGemvMfmaWaves = DECATTN_GEMV_MFMA_WAVES;
constexpr int kGemvMfmaThreads = 64 * kGemvMfmaWaves;

struct GemvMfmaParams {
    const void* W;            // bf16 [N][K] or int8 [N][K]
    const float* scale;       // [N], INT8 weights only
    const uint16_t* x;        // bf16 [B][K]
    void* y;                  // [B][N], fp32 or bf16
    int out_bf16;
    int B, N, K;
    uint32_t row_bytes;       // K * 2 (bf16) or K (int8)
};

__device__ __forceinline__ gemv_bf16x8_t gemv_frag(uint4 v) { return __builtin_bit_cast(gemv_bf16x8_t, v); }

// Weight rows go through LDS: each wave loads blocks of 128 bytes of each
// of its rows (64 k bf16, 128 k INT8; 8 rows of one whole 128-byte line per
// instruction) with the block's activation fragments, the next block's
// loads in flight while the current one is stored to the wave's own LDS
// tile and read back as MFMA fragments (16 rows x 64 or 32 bytes per read).
// Small blocks keep the kernel at 68 (bf16) / 76 (INT8) registers, 7 or 6
// waves per SIMD; 512- and 256-byte blocks (194 registers) took 26% longer
// at B = 8, 64-byte blocks slower again.
#ifndef DECATTN_GEMV_MFMA_BLK_BF16
#define DECATTN_GEMV_MFMA_BLK_BF16 128
#endif
#ifndef DECATTN_GEMV_MFMA_BLK_INT8
#define DECATTN_GEMV_MFMA_BLK_INT8 128
#endif
constexpr int gemv_mfma_blk(bool int8) { return int8 ? DECATTN_GEMV_MFMA_BLK_INT8 : DECATTN_GEMV_MFMA_BLK_BF16; }
// LDS row pitch: the block plus 16 bytes, so that the 16 rows of a fragment
// read start on different banks
constexpr int gemv_mfma_pitch(bool int8) { return gemv_mfma_blk(int8) + 16; }

template <int RT, bool INT8>
__global__ void __launch_bounds__(kGemvMfmaThreads)
gemv_mfma_kernel(const GemvMfmaParams p) {
    constexpr int ESZ = INT8 ? 1 : 2;              // bytes per weight
    constexpr int BLK = gemv_mfma_blk(INT8);       // bytes of a row per block
    constexpr int BLK_K = BLK / ESZ;               // k per block
    constexpr int LPRW = BLK / 16;                 // lanes per row in a load
    constexpr int RPL = 64 / LPRW;                 // rows per load instruction
    constexpr int NLD = 16 * RT / RPL;             // 16-byte weight loads per lane per block
    constexpr int STEPS = BLK_K / 32;              // MFMA k-steps per block
    constexpr int PITCH = gemv_mfma_pitch(INT8);
    extern __shared__ __align__(16) char gemv_lds[];            // [waves][16 RT][PITCH]
    __shared__ float red[kGemvMfmaWaves][RT][16][16];           // [wave][tile][vector][row]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = lane & 15, g = lane >> 4;
    char* tile = gemv_lds + (size_t)wave * 16 * RT * PITCH;
    const int row0 = (int)blockIdx.x * 16 * RT;
    const int nblk = (p.K + BLK_K - 1) / BLK_K;
    const int b0 = (int)((long long)wave * nblk / kGemvMfmaWaves);
    const int b1 = (int)((long long)(wave + 1) * nblk / kGemvMfmaWaves);
    const uint32_t w_end = (uint32_t)((size_t)p.N * p.row_bytes), x_end = (uint32_t)((size_t)p.B * p.K * 2);
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(p.W, w_end);
    const __amdgpu_buffer_rsrc_t xrs = make_rsrc(p.x, x_end);
    const bool xl = i < p.B;
    // load lane layout: load j covers rows RPL j .. RPL j + RPL - 1 of the
    // block, this lane's 16 bytes at column 16 * (lane % LPRW)
    const int lrow = lane / LPRW, lcol = (lane % LPRW) * 16;

    gemv_f32x4_t acc[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[r] = (gemv_f32x4_t){0.f, 0.f, 0.f, 0.f};

    // a block's weights and activation fragments, all issued together
    auto load = [&](uint4 (&w)[NLD], uint4 (&xv)[STEPS], int blk) {
        const int kb = blk * BLK + lcol;           // byte offset in the row
        const bool in = blk < b1 && kb < (int)p.row_bytes;
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const uint32_t off = (uint32_t)(row0 + RPL * j + lrow) * p.row_bytes + (uint32_t)kb;
            w[j] = buffer_load16_policy<DECATTN_GEMV_POLICY>(wrs, in ? off : w_end);
        }
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
            const int k = blk * BLK_K + 32 * t + 8 * g;
            xv[t] = buffer_load16_policy<0>(xrs, blk < b1 && xl && k < p.K ? (uint32_t)(i * p.K + k) * 2 : x_end);
        }
    };
    auto block = [&](const uint4 (&w)[NLD], const uint4 (&xv)[STEPS]) {
#pragma unroll
        for (int j = 0; j < NLD; ++j)
            *reinterpret_cast<uint4*>(tile + (RPL * j + lrow) * PITCH + lcol) = w[j];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const char* src = tile + (16 * r + i) * PITCH + (32 * t + 8 * g) * ESZ;
                uint4 a;
                if constexpr (INT8) {
                    const uint2 c = *reinterpret_cast<const uint2*>(src);
                    a = make_uint4(int8x2_to_bf16x2(c.x, 0), int8x2_to_bf16x2(c.x, 16),
                                   int8x2_to_bf16x2(c.y, 0), int8x2_to_bf16x2(c.y, 16));
                } else {
                    a = *reinterpret_cast<const uint4*>(src);
                }
                acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gemv_frag(a), gemv_frag(xv[t]), acc[r], 0, 0, 0);
            }
        }
        __builtin_amdgcn_wave_barrier();           // the next block rewrites the tile
    };
    uint4 wa[NLD], wb[NLD], xa[STEPS], xb[STEPS];
    load(wa, xa, b0);
    for (int blk = b0; blk < b1; blk += 2) {
        load(wb, xb, blk + 1);
        block(wa, xa);
        if (blk + 1 >= b1) break;
        load(wa, xa, blk + 2);
        block(wb, xb);
    }
    // lane (i, g) holds rows 4g .. 4g + 3 of vector i; sum the waves in order
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[wave][r][i][4 * g + j] = acc[r][j];
    __syncthreads();
    for (int t = threadIdx.x; t < RT * 16 * p.B; t += kGemvMfmaThreads) {
        const int r = t / (16 * p.B);
        const int b = (t / 16) % p.B;
        const int rr = t % 16;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kGemvMfmaWaves; ++w) v += red[w][r][b][rr];
        const int row = row0 + 16 * r + rr;
        if (row < p.N) {
            if constexpr (INT8) v *= p.scale[row];
            const size_t o = (size_t)b * p.N + row;
            if (p.out_bf16) reinterpret_cast<uint16_t*>(p.y)[o] = f32_to_bf16_rne(v);
            else reinterpret_cast<float*>(p.y)[o] = v;
        }
    }
}

// Per-output-row symmetric INT8 quantization, in fp32: a = max |w|,
// s = a / 127, q = round-half-even(w / s) kept in [-127, 127]; a row of zeros
// gets s = 0 and q = 0 (llm-decode-cuda, INT8 section: one fp32 scale per
// output channel, symmetric, quantized when the weights are loaded). One
// wave per row, two passes over it.
constexpr int kQuantThreads = 256;

__global__ void __launch_bounds__(kQuantThreads)
quantize_rows_int8_kernel(const uint16_t* __restrict__ W, int N, int K, int8_t* __restrict__ Wq,
                          float* __restrict__ scale) {
    const int lane = threadIdx.x & 63;
    const int row = (int)blockIdx.x * (kQuantThreads / 64) + (int)(threadIdx.x >> 6);
    if (row >= N) return;
    const uint16_t* w = W + (size_t)row * K;
    float a = 0.f;
    for (int e = lane * 8; e < K; e += 64 * 8) {
        float f[8];
        bf16x8_to_f32(*reinterpret_cast<const uint4*>(w + e), f);
#pragma unroll
        for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(f[i]));
    }
    // max is exact in any order
    a = fmaxf(a, dpp_move<kDppXor1>(a));
    a = fmaxf(a, dpp_move<kDppXor2>(a));
    a = fmaxf(a, dpp_move<kDppHalfMirror>(a));
    a = fmaxf(a, dpp_move<kDppMirror>(a));
    a = across_groups_max<16>(a);
    const float s = a / 127.f;                       // correctly rounded fp32 division
    if (lane == 0) scale[row] = a > 0.f ? s : 0.f;
    int8_t* q = Wq + (size_t)row * K;
    for (int e = lane * 8; e < K; e += 64 * 8) {
        float f[8];
        bf16x8_to_f32(*reinterpret_cast<const uint4*>(w + e), f);
        uint32_t packed[2] = {0u, 0u};
        if (a > 0.f) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float r = rintf(f[i] / s);              // fp32 quotient, ties to even
                r = fminf(fmaxf(r, -127.f), 127.f);
                packed[i >> 2] |= ((uint32_t)(int)r & 0xFFu) << (8 * (i & 3));
            }
        }
        *reinterpret_cast<uint2*>(q + e) = make_uint2(packed[0], packed[1]);
    }
}

}  // namespace decattn
