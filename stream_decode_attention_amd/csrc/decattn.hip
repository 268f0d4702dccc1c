// libdecattn host side: argument checks, launch shapes and the C ABI.
//
// The C ABI is declared in include/decattn.h. Nothing here allocates device
// memory or synchronizes, so every entry point can be captured in a hipGraph;
// all checks happen before the first launch. The only state is a host-side
// cache of per-device occupancy figures.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "../../include/decattn.h"
#include "gemv_kernel.hpp"
#include "merge_kernel.hpp"
#include "partial_kernel.hpp"
#include "prefill_kernel.hpp"
#include "probe_kernel.hpp"
#include "rope_kernel.hpp"
#include "spec_kernel.hpp"
#include "verify_kernel.hpp"

// The scratch of decode_attn_noalloc (its use is described there).
static __device__ __align__(256) unsigned char scratch[DECATTN_NOALLOC_SCRATCH_BYTES];

namespace decattn {
namespace {

constexpr int kMaxG = 8;
constexpr int kMaxT = 16;
constexpr int kMaxHq = 1 << 24;            // the merge divides head indices by G with a 32-bit multiply-high
constexpr int kMaxB = 4096;                // lengths are staged in LDS
constexpr int kMaxRowsPerWave = 8;
constexpr int kMaxWavesPerBlock = 8;       // matches __launch_bounds__(512)
constexpr size_t kMaxLdsBytes = 64 * 1024;
constexpr int kMinChunk = 16;
// Decode calls (T = 1) with at least this many query heads per kv head run on
// the matrix-core kernel when the tile is a multiple of 128 keys. Measured per
// call on MI355X: TinyLlama layers (G = 8, D = 64, one sequence of 1k-8k keys)
// 8.2-9.0 us against 8.8-9.9 on the dot-product kernel; eight sequences with
// G = 8, D = 128 at the headline lengths 83.7 against 91.9 us. With G = 3 or 4
// (SmolLM2-360M layers, the Llama-3-8B batch) the matrix cores were slower:
// 8.1 against 8.0 us and 83.0 against 79.1 us.
constexpr int kMfmaDecodeMinG = 8;
constexpr int kMaxChunk = 1 << 20;
constexpr size_t kAlign = 256;
constexpr int kKeyMargin = 512;            // keys a kernel may address past S_max (reading zeros)

bool is_pow2(long long x) { return x > 0 && (x & (x - 1)) == 0; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Plan {
    int B, T, Hq, Hkv, G, D, S_max, chunk, NC, RT;
    int R, NR, nwk, rg_per_block, n_row_blocks;
    size_t ml_bytes, acc_bytes, total_bytes, lds_bytes;
    bool mfma;              // verify chunk on the matrix cores
    int mfma_kb;            // 32-key blocks per wave in the matrix-core kernel
    size_t mfma_lds_main, mfma_lds_bytes;
};

int resident_blocks(const void* kernel, int threads, size_t lds);

// Dynamic LDS of the matrix-core kernel: the four waves' V tiles, the
// cross-wave combine area after them (not aliased: a wave stores its state
// without waiting for the others' last V reads; at most 108 KB at D = 128
// and 32 rows), then the B staged lengths (at most 16 KB).
size_t verify_lds_bytes(int D, int RT, int B, size_t* main_bytes = nullptr) {
    const size_t vt = (size_t)kVerifyWaves * 32 * verify_vrow(D);
    const size_t comb = (size_t)verify_comb_floats(RT, D) * sizeof(float);
    const size_t main = vt + comb;
    if (main_bytes) *main_bytes = main;
    return main + (size_t)B * sizeof(int);
}

int pick_default_chunk(int B, int T, int G, int Hkv, int D, int S_max) {
    // verify chunks that fit the matrix-core kernel: 256-key tiles (two
    // pipelined sub-tiles per workgroup; measured fastest per call at the
    // Llama-3.2-3B verify shape among calls that take the persistent walk),
    // or 512 when every 512-key tile fits on the current device at once and
    // not every 256-key tile does: the one-round launch then replaces the
    // walk (no length staging or counting pass). Measured on MI355X at the
    // Llama-3.2-3B verify shape (T = 6, 8 kv heads, 8192 keys of context:
    // 264 tiles of 256 keys against 256 resident workgroups): 14.9 us per
    // call against 16.1. Without a device to ask, 256.
    if (T > 1 && T * G <= kVerifyMaxRows) {
        const long long rows = (long long)B * Hkv;
        const long long n256 = rows * ((S_max + 255) / 256), n512 = rows * ((S_max + 511) / 512);
        const void* fn = D == 64 ? reinterpret_cast<const void*>(&verify_partial_mfma<64, 1, true, true>)
                                 : reinterpret_cast<const void*>(&verify_partial_mfma<128, 1, true, true>);
        const long long cap = resident_blocks(fn, 64 * kVerifyWaves, verify_lds_bytes(D, T * G, B));
        return (n256 > cap && n512 <= cap) ? 512 : 256;
    }
    // Decode: the largest tile (128 to 2048 keys) that still leaves at least
    // 1024 tiles over B*Hkv rows at S_max, the only length the host knows.
    // Larger tiles cut partial-state traffic (about G*(D+2)*4 bytes per tile
    // against 4*D bytes per key) and per-tile work; fewer than about 1024
    // tiles leave compute units idle once ragged rows skip theirs. Measured
    // per call on MI355X over B = 2..64 rows of 2k-32k keys, this rule lands
    // within about 7% of the best power of two in every case, and on 128 keys
    // for single-sequence calls of a few MB, where small tiles win.
    int c = 2048;
    while (c > 128 && (long long)B * Hkv * ((S_max + c - 1) / c) < 1024) c >>= 1;
    return c;
}

// Fills `pl` for the given shapes; returns a status. No pointer is touched.
int make_plan(int B, int T, int Hq, int Hkv, int D, int S_max, int chunk, Plan* pl) {
    if (B <= 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || S_max <= 0) return DECATTN_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return DECATTN_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return DECATTN_ERR_UNSUPPORTED;
    const int G = Hq / Hkv;
    if (G > kMaxG || T > kMaxT || Hq > kMaxHq) return DECATTN_ERR_UNSUPPORTED;
    if (chunk == 0) chunk = pick_default_chunk(B, T, G, Hkv, D, S_max);
    // a chunk >= S_max gives one tile per row
    if (chunk < kMinChunk || chunk > kMaxChunk || !is_pow2(chunk)) return DECATTN_ERR_UNSUPPORTED;
    const long long nc = ((long long)S_max + chunk - 1) / chunk;
    if ((long long)B * Hkv * S_max * (long long)D > (1LL << 46)) return DECATTN_ERR_UNSUPPORTED;
    // the kernels address one kv head's cache through a buffer resource with a
    // 32-bit byte range and 32-bit offsets; loads run up to a few sub-tiles
    // (under kKeyMargin keys) past the last attended key
    if (((long long)S_max + kKeyMargin) * D * 2 > 0xFFFFFFFFLL) return DECATTN_ERR_UNSUPPORTED;
    if (B > kMaxB || nc > 0x7FFFFFFF || (long long)B * T * Hq > 0x7FFFFFFF) return DECATTN_ERR_UNSUPPORTED;

    Plan p{};
    p.B = B; p.T = T; p.Hq = Hq; p.Hkv = Hkv; p.G = G; p.D = D; p.S_max = S_max;
    p.chunk = chunk; p.NC = (int)nc; p.RT = T * G;
    p.NR = (p.RT + kMaxRowsPerWave - 1) / kMaxRowsPerWave;
    p.R = (p.RT + p.NR - 1) / p.NR;
    p.nwk = key_waves_for(chunk);       // the partial kernel derives the same count
    const size_t lds_per_rg = (size_t)p.nwk * p.R * (D + 2) * sizeof(float);
    const size_t lds_lens = (size_t)B * sizeof(int);
    int rgb = kMaxWavesPerBlock / p.nwk;
    if ((size_t)rgb * lds_per_rg + lds_lens > kMaxLdsBytes) rgb = (int)((kMaxLdsBytes - lds_lens) / lds_per_rg);
    if (rgb > p.NR) rgb = p.NR;
    if (rgb < 1) return DECATTN_ERR_UNSUPPORTED;
    p.rg_per_block = rgb;
    p.n_row_blocks = (p.NR + rgb - 1) / rgb;
    // work items (b, kvh, row block, tile) must fit the kernel's int counters
    if ((long long)B * Hkv * p.n_row_blocks * nc > 0x7FFFFFFF) return DECATTN_ERR_UNSUPPORTED;
    p.lds_bytes = (size_t)rgb * lds_per_rg + lds_lens;

    // verify chunks (and decode calls with kMfmaDecodeMinG or more query heads
    // per kv head) of at most 32 rows per kv head on tiles of a multiple of 128
    // keys run on the matrix cores (scores and p.V are dense products there)
    p.mfma = (T > 1 || G >= kMfmaDecodeMinG) && p.RT <= kVerifyMaxRows && chunk % 128 == 0;
    // one 32-key block per wave: a 128-key sub-tile per workgroup, and room
    // in registers for the next sub-tile's loads while one is computed
    p.mfma_kb = 1;
    p.mfma_lds_bytes = verify_lds_bytes(D, p.RT, B, &p.mfma_lds_main);

    const size_t tiles_rows = (size_t)B * Hkv * p.NC * p.RT;
    p.ml_bytes = round_up(tiles_rows * 2 * sizeof(float), kAlign);
    p.acc_bytes = round_up(tiles_rows * (size_t)D * sizeof(float), kAlign);
    p.total_bytes = p.ml_bytes + p.acc_bytes;
    *pl = p;
    return DECATTN_OK;
}

// Workgroups of `kernel` that fit on the current device at once (all compute
// units times the per-unit occupancy), cached per device and launch shape.
// Host-side queries only: nothing is enqueued, so this is safe under capture.
int resident_blocks(const void* kernel, int threads, size_t lds) {
    struct Key {
        int dev;
        const void* fn;
        int threads;
        size_t lds;
    };
    static std::mutex mu;
    static std::vector<std::pair<Key, int>> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (const auto& e : cache)
            if (e.first.dev == dev && e.first.fn == kernel && e.first.threads == threads && e.first.lds == lds)
                return e.second;
    }
    int cus = 0, per_cu = 0;
    if (lds > 64 * 1024 &&
        hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds) != hipSuccess) return 0;
    const int n = cus * (per_cu > 0 ? per_cu : 1);
    std::lock_guard<std::mutex> lock(mu);
    // the key includes the dynamic LDS size, which some kernels size from the
    // call's shapes: keep the linear search short for callers that cycle
    // through many shapes (entries are recomputed on demand)
    if (cache.size() >= 512) cache.clear();
    cache.push_back({Key{dev, kernel, threads, lds}, n});
    return n;
}

template <int D, int R>
hipError_t launch_partial_dr(const Plan& pl, const PartialParams& pp, hipStream_t s) {
    const int threads = 64 * pl.nwk * pl.rg_per_block;
    const long long items = (long long)pl.B * pl.Hkv * pl.n_row_blocks * pl.NC;   // every possible tile
    const int tok_add = pp.causal ? pl.T : 0;          // keys past the context a causal chunk adds (T = 1 if 0)
    // one workgroup per possible work item when they all fit on the device at
    // once: each knows its tile from its index (grid Hkv x NC x B, one row
    // block) and reads only its own row's length (no staging, counting or
    // barrier; tiles past the length exit); measured 0.6-0.7 us faster per
    // call than the persistent walk on the single-sequence decode layers
    const void* fn1 = reinterpret_cast<const void*>(&split_kv_partial<D, R, true>);
    const long long res1 = resident_blocks(fn1, threads, pl.lds_bytes);
    if (res1 <= 0) return hipErrorInvalidDeviceFunction;
    // (only for tiles of at most kNumBuf sub-tiles per wave, the shape it was
    // measured on: a one-tile-per-row call on this loop ran 1.7x slower than
    // on the persistent walk)
    if (items <= res1 && pl.n_row_blocks == 1 && pl.chunk <= kNumBuf * pl.nwk * kKeysPerWave) {
        hipLaunchKernelGGL((split_kv_partial<D, R, true>), dim3((unsigned)pl.Hkv, (unsigned)pl.NC, (unsigned)pl.B),
                           dim3(threads), pl.lds_bytes, s, pp.lens, pp.k, pp.v, pp.q, pl.S_max, pl.chunk, pl.Hkv,
                           g_magic_for(pl.G), pl.G, tok_add, pp);
        return hipGetLastError();
    }
    // persistent: one wave of resident workgroups walks all attended tiles
    const void* fn = reinterpret_cast<const void*>(&split_kv_partial<D, R, false>);
    long long grid = resident_blocks(fn, threads, pl.lds_bytes);
    if (grid <= 0) return hipErrorInvalidDeviceFunction;
    if (grid > items) grid = items;
    hipLaunchKernelGGL((split_kv_partial<D, R, false>), dim3((unsigned)grid), dim3(threads), pl.lds_bytes, s, pp.lens,
                       pp.k, pp.v, pp.q, pl.S_max, pl.chunk, pl.Hkv, pl.B, pl.G, tok_add, pp);
    return hipGetLastError();
}

template <int D, int KB, bool SPLIT>
hipError_t launch_verify_dk(const Plan& pl, const PartialParams& pp, hipStream_t s) {
    const long long items = (long long)pl.B * pl.Hkv * pl.NC;   // every possible tile
    const int g_magic = g_magic_for(pl.G);             // r / G = (r * g_magic) >> 16 for r < 8192
    const int tok_add = pp.causal ? pl.T : 0;          // keys past the context a causal chunk adds (T = 1 if 0)
    // one workgroup per possible tile when they all fit on the device at once
    // (grid Hkv x NC x B; tiles past the length exit at once): no lengths
    // staged, no counting pass; the persistent walk would give every
    // workgroup one item and fold nothing there either, so both compute the
    // same tiles in the same way
    const void* fn1 = reinterpret_cast<const void*>(&verify_partial_mfma<D, KB, true, SPLIT>);
    const long long res1 = resident_blocks(fn1, 64 * kVerifyWaves, pl.mfma_lds_bytes);
    if (res1 <= 0) return hipErrorInvalidDeviceFunction;
    if (items <= res1) {
        hipLaunchKernelGGL((verify_partial_mfma<D, KB, true, SPLIT>), dim3((unsigned)pl.Hkv, (unsigned)pl.NC, (unsigned)pl.B),
                           dim3(64 * kVerifyWaves), pl.mfma_lds_bytes, s, pp.lens, pp.k, pp.v, pp.q, pl.S_max,
                           pl.chunk, pl.Hkv, g_magic, pl.G, tok_add, pp);
        return hipGetLastError();
    }
    const void* fn = reinterpret_cast<const void*>(&verify_partial_mfma<D, KB, false, SPLIT>);
    long long grid = resident_blocks(fn, 64 * kVerifyWaves, pl.mfma_lds_bytes);
    if (grid <= 0) return hipErrorInvalidDeviceFunction;
    if (grid > items) grid = items;
    hipLaunchKernelGGL((verify_partial_mfma<D, KB, false, SPLIT>), dim3((unsigned)grid), dim3(64 * kVerifyWaves),
                       pl.mfma_lds_bytes, s, pp.lens, pp.k, pp.v, pp.q, pl.S_max, pl.chunk, pl.Hkv, g_magic, pl.G,
                       tok_add, pp);
    return hipGetLastError();
}

template <int D>
hipError_t launch_partial_d(const Plan& pl, const PartialParams& pp, bool split_p, hipStream_t s) {
    if (pl.mfma)
        return split_p ? launch_verify_dk<D, 1, true>(pl, pp, s) : launch_verify_dk<D, 1, false>(pl, pp, s);
    switch (pl.R) {
        case 1: return launch_partial_dr<D, 1>(pl, pp, s);
        case 2: return launch_partial_dr<D, 2>(pl, pp, s);
        case 3: return launch_partial_dr<D, 3>(pl, pp, s);
        case 4: return launch_partial_dr<D, 4>(pl, pp, s);
        case 5: return launch_partial_dr<D, 5>(pl, pp, s);
        case 6: return launch_partial_dr<D, 6>(pl, pp, s);
        case 7: return launch_partial_dr<D, 7>(pl, pp, s);
        case 8: return launch_partial_dr<D, 8>(pl, pp, s);
        default: return hipErrorInvalidValue;
    }
}

// ---- the allocation-free decode entry point's scratch ----------------------
//
// decode_attn_noalloc keeps its partial state in this file-scope device array
// instead of a caller's workspace. Every GPU the library runs on holds its own
// copy, at its own address, until the process ends. In host code the array's
// name is only a host-side stand-in: kernels must be handed the device address
// that hipGetSymbolAddress returns for the current device, never `scratch`.
constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept; nullptr when the lookup fails.
void* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

// Scores are taken in log2 units (softmax on exp2): the kernels multiply q.k
// by scale*log2(e), rounded once to fp32; a zero scale becomes the smallest
// normal float, whose scores all round to 2^0.
float log2_scale(float scale) {
    const double qs = std::fabs((double)scale) * 1.4426950408889634;
    const float qmag = qs < (double)FLT_MIN ? FLT_MIN : (float)qs;
    return scale < 0.f ? -qmag : qmag;
}

// split_p: the matrix-core kernel carries the softmax weights as bf16 hi + lo
// parts in p.V (fp32 output, and the partial state of attn_partial, whose
// output type is not known yet) or as bf16 (bf16 output)
int run_partial(const Plan& pl, const void* q, const void* k, const void* v, const int32_t* lens,
                float scale, int causal, void* ws, bool split_p, hipStream_t s) {
    PartialParams pp{};
    pp.q = static_cast<const uint16_t*>(q);
    pp.k = static_cast<const uint16_t*>(k);
    pp.v = static_cast<const uint16_t*>(v);
    pp.lens = lens;
    pp.ws_ml = static_cast<float*>(ws);
    pp.ws_acc = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.ml_bytes);
    pp.NC = pl.NC; pp.causal = causal;
    pp.rg_per_block = pl.rg_per_block; pp.n_row_blocks = pl.n_row_blocks;
    pp.B = pl.B;
    pp.lds_main = (int)pl.mfma_lds_main;
    pp.qscale = log2_scale(scale);
    const hipError_t e = pl.D == 64 ? launch_partial_d<64>(pl, pp, split_p, s) : launch_partial_d<128>(pl, pp, split_p, s);
    return e == hipSuccess ? DECATTN_OK : DECATTN_ERR_HIP;
}

int run_merge(const Plan& pl, const int32_t* lens, int causal, void* out, int out_dtype, void* ws,
              hipStream_t s) {
    MergeParams mp{};
    const float* ws_ml = static_cast<const float*>(ws);
    const float* ws_acc = reinterpret_cast<const float*>(static_cast<const char*>(ws) + pl.ml_bytes);
    mp.out = out;
    mp.out_bf16 = out_dtype == DECATTN_OUT_BF16;
    mp.T = pl.T; mp.S_max = pl.S_max; mp.chunk = pl.chunk; mp.causal = causal;
    const dim3 grid(pl.Hkv, pl.RT, pl.B);
    // ceil(2^32 / G) (G >= 2; unused at G = 1): r / G = mulhi(r, g_recip) for r < 2^28
    const uint32_t g_recip = pl.G == 1 ? 0u : (uint32_t)(((1ull << 32) + pl.G - 1) / pl.G);
    // slots of the merge's first batch: ceil(NC / tile lanes), rounded up to
    // a power of two, at most kMergeUnroll
    const int ncl = merge_threads(pl.D) / (pl.D / 4);   // tile lanes of a workgroup
    const int need = (pl.NC + ncl - 1) / ncl;
    const int nu0 = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;
    auto launch = [&](auto d_tag, auto nu_tag) {
        constexpr int DD = decltype(d_tag)::value, NU = decltype(nu_tag)::value;
        hipLaunchKernelGGL((lse_merge<DD, NU, merge_threads(DD) / 64>), grid, dim3(merge_threads(DD)), 0, s, ws_ml,
                           ws_acc, lens, pl.G, pl.Hkv, pl.NC, pl.RT, g_recip, mp);
    };
    auto by_nu = [&](auto d_tag) {
        constexpr int DD = decltype(d_tag)::value;
        if (pl.NC * (DD / 4) <= 64) {
            // one wave's tile lanes hold every tile slot: one wave per row
            hipLaunchKernelGGL((lse_merge<DD, 1, 1>), grid, dim3(64), 0, s, ws_ml, ws_acc, lens, pl.G, pl.Hkv,
                               pl.NC, pl.RT, g_recip, mp);
            return;
        }
        switch (nu0) {
            case 1: launch(d_tag, std::integral_constant<int, 1>{}); break;
            case 2: launch(d_tag, std::integral_constant<int, 2>{}); break;
            case 4: launch(d_tag, std::integral_constant<int, 4>{}); break;
            default: launch(d_tag, std::integral_constant<int, 8>{}); break;
        }
    };
    if (pl.D == 64) by_nu(std::integral_constant<int, 64>{});
    else by_nu(std::integral_constant<int, 128>{});
    return hipGetLastError() == hipSuccess ? DECATTN_OK : DECATTN_ERR_HIP;
}

int check_inputs(const void* q, const void* k, const void* v, const int32_t* lens, float scale) {
    if (!q || !k || !v || !lens) return DECATTN_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (reinterpret_cast<uintptr_t>(lens) & 3u))
        return DECATTN_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return DECATTN_ERR_INVALID_ARG;
    return DECATTN_OK;
}

int check_common(const void* q, const void* k, const void* v, const int32_t* lens, float scale,
                 void* ws, size_t ws_bytes, const Plan& pl) {
    const int st = check_inputs(q, k, v, lens, scale);
    if (st != DECATTN_OK) return st;
    if (!ws || !aligned16(ws)) return DECATTN_ERR_INVALID_ARG;
    if (ws_bytes < pl.total_bytes) return DECATTN_ERR_WORKSPACE;
    return DECATTN_OK;
}

int check_out(void* out, int out_dtype) {
    if (!out || !aligned16(out)) return DECATTN_ERR_INVALID_ARG;
    if (out_dtype != DECATTN_OUT_BF16 && out_dtype != DECATTN_OUT_F32) return DECATTN_ERR_INVALID_ARG;
    return DECATTN_OK;
}

int attention(const void* q, const void* k, const void* v, const int32_t* lens, int B, int T, int Hq,
              int Hkv, int D, int S_max, float scale, int causal, void* out, int out_dtype, void* ws,
              size_t ws_bytes, int chunk, void* stream) {
    Plan pl;
    int st = make_plan(B, T, Hq, Hkv, D, S_max, chunk, &pl);
    if (st != DECATTN_OK) return st;
    if ((st = check_common(q, k, v, lens, scale, ws, ws_bytes, pl)) != DECATTN_OK) return st;
    if ((st = check_out(out, out_dtype)) != DECATTN_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = run_partial(pl, q, k, v, lens, scale, causal, ws, out_dtype != DECATTN_OUT_BF16, s)) != DECATTN_OK)
        return st;
    return run_merge(pl, lens, causal, out, out_dtype, ws, s);
}

// True when [a, a + na) and [b, b + nb) share a byte.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

bool positive_finite(double x) { return std::isfinite(x) && x > 0.0; }

int check_rope(const decattn_rope* r) {
    if (!r) return DECATTN_ERR_INVALID_ARG;
    if (r->pairing != DECATTN_ROPE_HALF && r->pairing != DECATTN_ROPE_ADJACENT) return DECATTN_ERR_INVALID_ARG;
    if (!positive_finite(r->theta)) return DECATTN_ERR_INVALID_ARG;
    if (r->llama3_scaling != 0 && r->llama3_scaling != 1) return DECATTN_ERR_INVALID_ARG;
    if (r->llama3_scaling) {
        if (!positive_finite(r->factor) || !positive_finite(r->low_freq_factor) ||
            !positive_finite(r->high_freq_factor) || !positive_finite(r->original_max_position))
            return DECATTN_ERR_INVALID_ARG;
        if (!(r->high_freq_factor > r->low_freq_factor)) return DECATTN_ERR_INVALID_ARG;
    }
    return DECATTN_OK;
}

// ---- weight products (GEMV) ------------------------------------------------

constexpr size_t kGemvLdsBudget = 144 * 1024;   // staged activations per workgroup
constexpr int kGemvMaxB = 8;

template <int LPR, int B, bool INT8>
int launch_gemv_b(const GemvParams& gp, size_t lds, hipStream_t s) {
    // batches from the matrix-core threshold up never reach the dot products
    if constexpr (B >= (INT8 ? DECATTN_GEMV_MFMA_MIN_B_INT8 : DECATTN_GEMV_MFMA_MIN_B_BF16)) {
        return DECATTN_ERR_UNSUPPORTED;
    } else {
        const void* fn = reinterpret_cast<const void*>(&gemv_kernel<LPR, B, INT8>);
        long long grid = resident_blocks(fn, kGemvThreads, lds);
        if (grid <= 0) return DECATTN_ERR_HIP;
        const long long rows_per_wave = (64 / LPR) * gemv_rows_per_group<B, INT8>();
        const long long groups = ((long long)gp.N + rows_per_wave - 1) / rows_per_wave;
        const long long need = (groups + kGemvThreads / 64 - 1) / (kGemvThreads / 64);
        if (grid > need) grid = need;
        hipLaunchKernelGGL((gemv_kernel<LPR, B, INT8>), dim3((unsigned)grid), dim3(kGemvThreads), lds, s, gp);
        return hipGetLastError() == hipSuccess ? DECATTN_OK : DECATTN_ERR_HIP;
    }
}

template <int LPR, bool INT8>
int launch_gemv_lpr(const GemvParams& gp, int B, size_t lds, hipStream_t s) {
    switch (B) {
        case 1: return launch_gemv_b<LPR, 1, INT8>(gp, lds, s);
        case 2: return launch_gemv_b<LPR, 2, INT8>(gp, lds, s);
        case 3: return launch_gemv_b<LPR, 3, INT8>(gp, lds, s);
        case 4: return launch_gemv_b<LPR, 4, INT8>(gp, lds, s);
        case 5: return launch_gemv_b<LPR, 5, INT8>(gp, lds, s);
        case 6: return launch_gemv_b<LPR, 6, INT8>(gp, lds, s);
        case 7: return launch_gemv_b<LPR, 7, INT8>(gp, lds, s);
        case 8: return launch_gemv_b<LPR, 8, INT8>(gp, lds, s);
        default: return DECATTN_ERR_UNSUPPORTED;
    }
}

template <int RT, bool INT8>
int launch_gemv_mfma(const GemvMfmaParams& mp, hipStream_t s) {
    const unsigned grid = (unsigned)((mp.N + 16 * RT - 1) / (16 * RT));
    const size_t lds = (size_t)kGemvMfmaWaves * 16 * RT * gemv_mfma_pitch(INT8);
    // sets the dynamic-LDS limit of this kernel on the current device (cached)
    if (resident_blocks(reinterpret_cast<const void*>(&gemv_mfma_kernel<RT, INT8>), kGemvMfmaThreads, lds) <= 0)
        return DECATTN_ERR_HIP;
    hipLaunchKernelGGL((gemv_mfma_kernel<RT, INT8>), dim3(grid), dim3(kGemvMfmaThreads), lds, s, mp);
    return hipGetLastError() == hipSuccess ? DECATTN_OK : DECATTN_ERR_HIP;
}

// y = x W^T for B vectors, in launches of as many vectors as the LDS budget
// holds (each launch reads the weights once).
int gemv_common(const void* W, const float* scale, const void* x, int B, int N, int K, void* y, int out_dtype,
                bool int8, void* stream) {
    if (!W || !x || !y || (int8 && !scale)) return DECATTN_ERR_INVALID_ARG;
    if (B <= 0 || N <= 0 || K <= 0) return DECATTN_ERR_INVALID_ARG;
    if (B > kGemvMaxB) return DECATTN_ERR_UNSUPPORTED;
    const int epc = int8 ? 16 : 8;
    if (K % epc != 0) return DECATTN_ERR_UNSUPPORTED;
    if (!aligned16(W) || !aligned16(x) || (int8 && (reinterpret_cast<uintptr_t>(scale) & 3u)))
        return DECATTN_ERR_INVALID_ARG;
    int st = check_out(y, out_dtype);
    if (st != DECATTN_OK) return st;
    // one buffer resource spans W: its bytes, plus the rows of the last
    // group past N, must stay below 2^32
    if ((long long)(N + 64) * K * (int8 ? 1 : 2) >= (1LL << 32)) return DECATTN_ERR_UNSUPPORTED;
    GemvParams gp{};
    gp.W = W;
    gp.scale = scale;
    gp.N = N;
    gp.K = K;
    gp.KC = K / epc;
    const int lpr = gp.KC >= 256 ? 64 : (gp.KC >= 128 ? 32 : 16);
    gp.KCP = (gp.KC + lpr - 1) / lpr * lpr;
    gp.xrow = gp.KCP * epc;
    const size_t per_vec = (size_t)gp.xrow * 2;
    const int bmax = (int)(kGemvLdsBudget / per_vec);
    if (bmax < 1) return DECATTN_ERR_UNSUPPORTED;          // one activation row does not fit in LDS
    gp.out_bf16 = out_dtype == DECATTN_OUT_BF16;
    const size_t osz = gp.out_bf16 ? 2 : 4;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (B >= (int8 ? DECATTN_GEMV_MFMA_MIN_B_INT8 : DECATTN_GEMV_MFMA_MIN_B_BF16) ||
        (!int8 && N >= DECATTN_GEMV_MFMA_B1_MIN_N)) {
        // the matrix cores: every vector in one pass over the weights
        if ((size_t)B * K * 2 + 16 >= (1ull << 32)) return DECATTN_ERR_UNSUPPORTED;
        GemvMfmaParams mp{};
        mp.W = W;
        mp.scale = scale;
        mp.x = static_cast<const uint16_t*>(x);
        mp.y = y;
        mp.out_bf16 = gp.out_bf16;
        mp.B = B;
        mp.N = N;
        mp.K = K;
        mp.row_bytes = (uint32_t)K * (int8 ? 1 : 2);
        if (int8)
            return N >= DECATTN_GEMV_MFMA_RT2_MIN_N_INT8 ? launch_gemv_mfma<2, true>(mp, s)
                                                         : launch_gemv_mfma<1, true>(mp, s);
        return launch_gemv_mfma<1, false>(mp, s);
    }
    for (int b0 = 0; b0 < B; b0 += bmax) {
        const int nb = B - b0 < bmax ? B - b0 : bmax;
        gp.x = static_cast<const uint16_t*>(x) + (size_t)b0 * K;
        gp.y = static_cast<char*>(y) + (size_t)b0 * N * osz;
        const size_t lds = (size_t)nb * per_vec;
        if (lpr == 64) st = int8 ? launch_gemv_lpr<64, true>(gp, nb, lds, s) : launch_gemv_lpr<64, false>(gp, nb, lds, s);
        else if (lpr == 32) st = int8 ? launch_gemv_lpr<32, true>(gp, nb, lds, s) : launch_gemv_lpr<32, false>(gp, nb, lds, s);
        else st = int8 ? launch_gemv_lpr<16, true>(gp, nb, lds, s) : launch_gemv_lpr<16, false>(gp, nb, lds, s);
        if (st != DECATTN_OK) return st;
    }
    return DECATTN_OK;
}

// ---- speculative accept/reject ----------------------------------------------

constexpr int kSpecMaxV = 1 << 24;
#ifndef DECATTN_SPEC_TARGET_BLOCKS
#define DECATTN_SPEC_TARGET_BLOCKS 2048
#endif

struct SpecPlan {
    int U, NC, U2, NC2;
    size_t stats_bytes, parts_bytes, rowinfo_bytes, total_bytes;
};

// Chunks of 1024*U vocabulary entries for the statistics kernel, U in
// {1, 2, 4, 8}: the largest U that still leaves DECATTN_SPEC_TARGET_BLOCKS
// workgroups over the B*T rows (small batches want many short chunks, since
// each workgroup's latency dominates; big ones want long chunks), and at most
// kSpecMaxNC chunks; U only grows while that cuts the chunk count. The draw
// (sampling) uses the same chunks (U2 = U): its second launch repeats the
// decision in every workgroup, so it wants few of them at large batch, and
// the final rescan of one chunk is cheap at any size. The workspace holds the
// chunk statistics [B][T][NC], the draw chunks' masses [B][NC2], one float4
// per row and one per draft.
int spec_plan(int B, int T, int V, SpecPlan* sp) {
    if (B <= 0 || T <= 0 || V <= 0) return DECATTN_ERR_INVALID_ARG;
    if (T > kSpecMaxT || V > kSpecMaxV) return DECATTN_ERR_UNSUPPORTED;
    auto nc = [V](int u) { return (V + u * kSpecSeg - 1) / (u * kSpecSeg); };
    int U = 1;
    while (U < 8 && nc(2 * U) < nc(U) &&
           ((long long)B * T * nc(2 * U) >= DECATTN_SPEC_TARGET_BLOCKS || nc(U) > kSpecMaxNC))
        U *= 2;
    const int NC = nc(U);
    if (NC > kSpecMaxNC || (long long)B * T * NC > 0x7FFFFFFF) return DECATTN_ERR_UNSUPPORTED;
    sp->U = U;
    sp->NC = NC;
    sp->U2 = U;
    sp->NC2 = NC;
    sp->stats_bytes = round_up((size_t)B * T * NC * sizeof(float2), kAlign);
    sp->parts_bytes = round_up((size_t)B * sp->NC2 * sizeof(float2), kAlign);
    sp->rowinfo_bytes = round_up((size_t)B * sizeof(float4), kAlign);
    sp->total_bytes = sp->stats_bytes + sp->parts_bytes + sp->rowinfo_bytes +
                      round_up((size_t)B * (T > 1 ? T - 1 : 1) * sizeof(float4), kAlign);
    return DECATTN_OK;
}

template <int U, bool VEC, bool GREEDY>
void spec_launch_stats(const SpecParams& sp, int B, hipStream_t s) {
    hipLaunchKernelGGL((spec_stats_kernel<U, VEC, GREEDY>), dim3((unsigned)(B * sp.T * sp.NC)), dim3(kSpecThreads), 0,
                       s, sp);
}

template <int U, bool VEC>
void spec_launch_draw(const SpecParams& sp, int B, hipStream_t s) {
    hipLaunchKernelGGL((spec_resid_kernel<U, VEC>), dim3((unsigned)(B * sp.NC2)), dim3(kSpecThreads),
                       (size_t)sp.stage_n * sizeof(float2), s, sp);
    hipLaunchKernelGGL((spec_select_kernel<U, VEC>), dim3((unsigned)B), dim3(kSpecThreads),
                       (size_t)sp.NC2 * sizeof(float2), s, sp);
}

template <int U>
void spec_launch_u(const SpecParams& sp, int B, bool vec, bool greedy, hipStream_t s) {
    if (vec) greedy ? spec_launch_stats<U, true, true>(sp, B, s) : spec_launch_stats<U, true, false>(sp, B, s);
    else greedy ? spec_launch_stats<U, false, true>(sp, B, s) : spec_launch_stats<U, false, false>(sp, B, s);
}

template <int U>
void spec_launch_draw_u(const SpecParams& sp, int B, bool vec, hipStream_t s) {
    if (vec) spec_launch_draw<U, true>(sp, B, s);
    else spec_launch_draw<U, false>(sp, B, s);
}

}  // namespace
}  // namespace decattn

using namespace decattn;

// ---- causal prefill attention ------------------------------------------------

template <int D, bool SPLIT, int WAVES, int KT>
int launch_prefill(const PrefillParams& pp, long long grid, hipStream_t s) {
    const size_t lds = (size_t)prefill_lds_bytes(D, KT);
    // sets the dynamic-LDS limit of this kernel on the current device (cached)
    if (resident_blocks(reinterpret_cast<const void*>(&prefill_attn_mfma<D, SPLIT, WAVES, KT>), 64 * WAVES, lds) <= 0)
        return DECATTN_ERR_HIP;
    hipLaunchKernelGGL((prefill_attn_mfma<D, SPLIT, WAVES, KT>), dim3((unsigned)grid), dim3(64 * WAVES), lds, s, pp);
    return hipGetLastError() == hipSuccess ? DECATTN_OK : DECATTN_ERR_HIP;
}

extern "C" {

int decattn_abi_version(void) { return DECATTN_ABI_VERSION; }

const char* decattn_status_str(int status) {
    switch (status) {
        case DECATTN_OK: return "ok";
        case DECATTN_ERR_INVALID_ARG: return "invalid argument";
        case DECATTN_ERR_UNSUPPORTED: return "unsupported shape or chunk size";
        case DECATTN_ERR_WORKSPACE: return "workspace too small";
        case DECATTN_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

int decattn_default_chunk(int B, int T, int Hq, int Hkv, int D, int S_max) {
    Plan pl;
    return make_plan(B, T, Hq, Hkv, D, S_max, 0, &pl) == DECATTN_OK ? pl.chunk : 0;
}

size_t decattn_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int S_max, int chunk) {
    Plan pl;
    return make_plan(B, T, Hq, Hkv, D, S_max, chunk, &pl) == DECATTN_OK ? pl.total_bytes : 0;
}

int decode_attn(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens, int B,
                int Hq, int Hkv, int D, int S_max, float scale, void* out, int out_dtype, void* workspace,
                size_t workspace_bytes, int chunk, void* stream) {
    return attention(q, k_cache, v_cache, seq_lens, B, 1, Hq, Hkv, D, S_max, scale, 0, out, out_dtype,
                     workspace, workspace_bytes, chunk, stream);
}

int decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                        int B, int Hq, int Hkv, int D, int S_max, float scale, void* out, int out_dtype,
                        int chunk, void* stream) {
    Plan pl;
    int st = make_plan(B, 1, Hq, Hkv, D, S_max, chunk, &pl);
    if (st != DECATTN_OK) return st;
    if ((st = check_inputs(q, k_cache, v_cache, seq_lens, scale)) != DECATTN_OK) return st;
    if ((st = check_out(out, out_dtype)) != DECATTN_OK) return st;
    if (pl.total_bytes > DECATTN_NOALLOC_SCRATCH_BYTES) return DECATTN_ERR_WORKSPACE;
    void* ws = scratch_for_current_device();    // the device address, never `scratch` itself
    if (!ws) return DECATTN_ERR_HIP;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = run_partial(pl, q, k_cache, v_cache, seq_lens, scale, 0, ws, out_dtype != DECATTN_OUT_BF16, s)) !=
        DECATTN_OK)
        return st;
    return run_merge(pl, seq_lens, 0, out, out_dtype, ws, s);
}

int chunk_attn(const void* q, const void* k_cache, const void* v_cache, const int32_t* ctx_lens, int B,
               int T, int Hq, int Hkv, int D, int S_max, float scale, void* out, int out_dtype,
               void* workspace, size_t workspace_bytes, int chunk, void* stream) {
    return attention(q, k_cache, v_cache, ctx_lens, B, T, Hq, Hkv, D, S_max, scale, 1, out, out_dtype,
                     workspace, workspace_bytes, chunk, stream);
}

int attn_partial(const void* q, const void* k_cache, const void* v_cache, const int32_t* lens, int B, int T,
                 int Hq, int Hkv, int D, int S_max, float scale, int causal, void* workspace,
                 size_t workspace_bytes, int chunk, void* stream) {
    if (causal != 0 && causal != 1) return DECATTN_ERR_INVALID_ARG;
    if (!causal && T != 1) return DECATTN_ERR_INVALID_ARG;
    Plan pl;
    int st = make_plan(B, T, Hq, Hkv, D, S_max, chunk, &pl);
    if (st != DECATTN_OK) return st;
    if ((st = check_common(q, k_cache, v_cache, lens, scale, workspace, workspace_bytes, pl)) != DECATTN_OK)
        return st;
    return run_partial(pl, q, k_cache, v_cache, lens, scale, causal, workspace, true,
                       static_cast<hipStream_t>(stream));
}

int attn_merge(const int32_t* lens, int B, int T, int Hq, int Hkv, int D, int S_max, int causal, void* out,
               int out_dtype, void* workspace, size_t workspace_bytes, int chunk, void* stream) {
    if (causal != 0 && causal != 1) return DECATTN_ERR_INVALID_ARG;
    if (!causal && T != 1) return DECATTN_ERR_INVALID_ARG;
    Plan pl;
    int st = make_plan(B, T, Hq, Hkv, D, S_max, chunk, &pl);
    if (st != DECATTN_OK) return st;
    if (!lens || !workspace || !aligned16(workspace) || (reinterpret_cast<uintptr_t>(lens) & 3u))
        return DECATTN_ERR_INVALID_ARG;
    if (workspace_bytes < pl.total_bytes) return DECATTN_ERR_WORKSPACE;
    if ((st = check_out(out, out_dtype)) != DECATTN_OK) return st;
    return run_merge(pl, lens, causal, out, out_dtype, workspace, static_cast<hipStream_t>(stream));
}

int prefill_attn(const void* q, const void* k_cache, const void* v_cache, const int32_t* ctx_lens, int B,
                 int T, int Hq, int Hkv, int D, int S_max, float scale, void* out, int out_dtype, void* stream) {
    if (!q || !k_cache || !v_cache || !ctx_lens || !out) return DECATTN_ERR_INVALID_ARG;
    if (B <= 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || S_max <= 0) return DECATTN_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return DECATTN_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return DECATTN_ERR_UNSUPPORTED;
    const int G = Hq / Hkv;
    if (G > kMaxG) return DECATTN_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || (reinterpret_cast<uintptr_t>(ctx_lens) & 3u))
        return DECATTN_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return DECATTN_ERR_INVALID_ARG;
    int st = check_out(out, out_dtype);
    if (st != DECATTN_OK) return st;
    // one kv head's cache must be addressable by a 32-bit buffer offset
    if ((long long)(S_max + 4 * kPrefillMaxKeys) * D * 2 > 0xFFFFFFFFLL) return DECATTN_ERR_UNSUPPORTED;
    if ((long long)B * T * Hq > 0x7FFFFFFF) return DECATTN_ERR_UNSUPPORTED;
    PrefillParams pp{};
    pp.q = static_cast<const uint16_t*>(q);
    pp.k = static_cast<const uint16_t*>(k_cache);
    pp.v = static_cast<const uint16_t*>(v_cache);
    pp.ctx = ctx_lens;
    pp.out = out;
    pp.out_bf16 = out_dtype == DECATTN_OUT_BF16;
    pp.B = B; pp.T = T; pp.Hq = Hq; pp.Hkv = Hkv; pp.G = G; pp.S_max = S_max;
    pp.PW = 32 / G;
    pp.qscale = log2_scale(scale);
    // 8 waves on 128-key tiles when that still gives 512 workgroups, else 4
    // waves on 64-key tiles
    const long long nqb8 = (T + 8LL * pp.PW - 1) / (8LL * pp.PW);
    const bool wide = (long long)B * Hkv * nqb8 >= 512;
    const int waves = wide ? 8 : 4;
    pp.NQB = (T + waves * pp.PW - 1) / (waves * pp.PW);
    const long long grid = (long long)B * Hkv * pp.NQB;
    if (grid > 0x7FFFFFFF) return DECATTN_ERR_UNSUPPORTED;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (wide) {
        if (D == 64) return pp.out_bf16 ? launch_prefill<64, false, 8, 128>(pp, grid, s)
                                        : launch_prefill<64, true, 8, 128>(pp, grid, s);
        return pp.out_bf16 ? launch_prefill<128, false, 8, 128>(pp, grid, s)
                           : launch_prefill<128, true, 8, 128>(pp, grid, s);
    }
    if (D == 64) return pp.out_bf16 ? launch_prefill<64, false, 4, 64>(pp, grid, s)
                                    : launch_prefill<64, true, 4, 64>(pp, grid, s);
    return pp.out_bf16 ? launch_prefill<128, false, 4, 64>(pp, grid, s)
                       : launch_prefill<128, true, 4, 64>(pp, grid, s);
}

int rope_kv_write(const void* q_in, const void* k_in, const void* v_in, const int32_t* pos0, int B, int T,
                  int Hq, int Hkv, int D, int S_max, const decattn_rope* rope, void* q_out, void* k_cache,
                  void* v_cache, void* stream) {
    if (!q_in || !k_in || !v_in || !pos0 || !q_out || !k_cache || !v_cache) return DECATTN_ERR_INVALID_ARG;
    if (B <= 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || S_max <= 0) return DECATTN_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return DECATTN_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return DECATTN_ERR_UNSUPPORTED;
    if ((long long)B * T > 0x7FFFFFFF || (long long)S_max + T > 0x7FFFFFFF) return DECATTN_ERR_UNSUPPORTED;
    int st = check_rope(rope);
    if (st != DECATTN_OK) return st;
    if (!aligned16(q_in) || !aligned16(k_in) || !aligned16(v_in) || !aligned16(q_out) || !aligned16(k_cache) ||
        !aligned16(v_cache) || (reinterpret_cast<uintptr_t>(pos0) & 3u))
        return DECATTN_ERR_INVALID_ARG;
    // q_out is q_in itself or apart from every other buffer; the new k/v rows
    // and the two caches do not overlap each other
    const size_t qb = (size_t)B * T * Hq * D * 2, kb = (size_t)B * T * Hkv * D * 2;
    const size_t cb = (size_t)B * Hkv * S_max * D * 2;
    if (q_out != q_in && overlaps(q_out, qb, q_in, qb)) return DECATTN_ERR_INVALID_ARG;
    const void* bufs[5] = {k_in, v_in, k_cache, v_cache, pos0};
    const size_t sizes[5] = {kb, kb, cb, cb, (size_t)B * 4};
    for (int a = 0; a < 5; ++a) {
        if (overlaps(q_out, qb, bufs[a], sizes[a])) return DECATTN_ERR_INVALID_ARG;
        for (int c = a + 1; c < 5; ++c)
            if (overlaps(bufs[a], sizes[a], bufs[c], sizes[c])) return DECATTN_ERR_INVALID_ARG;
    }
    RopeParams rp{};
    rp.q_in = static_cast<const uint16_t*>(q_in);
    rp.k_in = static_cast<const uint16_t*>(k_in);
    rp.v_in = static_cast<const uint16_t*>(v_in);
    rp.pos0 = pos0;
    rp.q_out = static_cast<uint16_t*>(q_out);
    rp.k_cache = static_cast<uint16_t*>(k_cache);
    rp.v_cache = static_cast<uint16_t*>(v_cache);
    rp.T = T; rp.Hq = Hq; rp.Hkv = Hkv; rp.S_max = S_max;
    rp.llama3 = rope->llama3_scaling;
    rp.theta = rope->theta;
    rp.factor = rope->factor;
    rp.low_freq_factor = rope->low_freq_factor;
    rp.high_freq_factor = rope->high_freq_factor;
    rp.original_max_position = rope->original_max_position;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)(B * T)), block(kRopeThreads);
    const bool adj = rope->pairing == DECATTN_ROPE_ADJACENT;
    if (D == 64) {
        if (adj) hipLaunchKernelGGL((rope_kv_write_kernel<64, true>), grid, block, 0, s, rp);
        else hipLaunchKernelGGL((rope_kv_write_kernel<64, false>), grid, block, 0, s, rp);
    } else {
        if (adj) hipLaunchKernelGGL((rope_kv_write_kernel<128, true>), grid, block, 0, s, rp);
        else hipLaunchKernelGGL((rope_kv_write_kernel<128, false>), grid, block, 0, s, rp);
    }
    return hipGetLastError() == hipSuccess ? DECATTN_OK : DECATTN_ERR_HIP;
}

int gemv_bf16(const void* W, const void* x, int B, int N, int K, void* y, int out_dtype, void* stream) {
    return gemv_common(W, nullptr, x, B, N, K, y, out_dtype, false, stream);
}

int gemv_int8(const void* Wq, const float* scale, const void* x, int B, int N, int K, void* y, int out_dtype,
              void* stream) {
    return gemv_common(Wq, scale, x, B, N, K, y, out_dtype, true, stream);
}

int quantize_rows_int8(const void* W, int N, int K, void* Wq, float* scale, void* stream) {
    if (!W || !Wq || !scale) return DECATTN_ERR_INVALID_ARG;
    if (N <= 0 || K <= 0) return DECATTN_ERR_INVALID_ARG;
    if (K % 16 != 0) return DECATTN_ERR_UNSUPPORTED;
    if (!aligned16(W) || !aligned16(Wq) || (reinterpret_cast<uintptr_t>(scale) & 3u)) return DECATTN_ERR_INVALID_ARG;
    const size_t wb = (size_t)N * K * 2, qb = (size_t)N * K, sb = (size_t)N * 4;
    if (overlaps(W, wb, Wq, qb) || overlaps(W, wb, scale, sb) || overlaps(Wq, qb, scale, sb))
        return DECATTN_ERR_INVALID_ARG;
    const long long blocks = ((long long)N + kQuantThreads / 64 - 1) / (kQuantThreads / 64);
    if (blocks > 0x7FFFFFFF) return DECATTN_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(quantize_rows_int8_kernel, dim3((unsigned)blocks), dim3(kQuantThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(W), N, K,
                       static_cast<int8_t*>(Wq), scale);
    return hipGetLastError() == hipSuccess ? DECATTN_OK : DECATTN_ERR_HIP;
}

size_t spec_accept_workspace_bytes(int B, int T, int V) {
    SpecPlan sp;
    return spec_plan(B, T, V, &sp) == DECATTN_OK ? sp.total_bytes : 0;
}

int spec_accept(const float* logits, const float* q, const int32_t* drafts, const float* u, const float* r,
                float tau, int B, int T, int V, int S_max, int32_t* lens, int32_t* result, void* workspace,
                size_t workspace_bytes, void* stream) {
    SpecPlan plan;
    int st = spec_plan(B, T, V, &plan);
    if (st != DECATTN_OK) return st;
    if (S_max <= 0 || !std::isfinite(tau) || !(tau >= 0.f)) return DECATTN_ERR_INVALID_ARG;
    const bool greedy = tau == 0.f;
    float c2 = 0.f;
    if (!greedy) {
        const double c = 1.4426950408889634 / (double)tau;     // log2(e) / tau
        if (!(c <= (double)FLT_MAX)) return DECATTN_ERR_INVALID_ARG;
        c2 = (float)c;
    }
    const int gamma = T - 1;
    if (!logits || !lens || !result || !workspace) return DECATTN_ERR_INVALID_ARG;
    if (gamma > 0 && !drafts) return DECATTN_ERR_INVALID_ARG;
    if (!greedy && (!r || (gamma > 0 && (!q || !u)))) return DECATTN_ERR_INVALID_ARG;
    const void* word_ptrs[7] = {logits, q, drafts, u, r, lens, result};
    for (const void* ptr : word_ptrs)
        if (reinterpret_cast<uintptr_t>(ptr) & 3u) return DECATTN_ERR_INVALID_ARG;
    if (!aligned16(workspace)) return DECATTN_ERR_INVALID_ARG;
    if (workspace_bytes < plan.total_bytes) return DECATTN_ERR_WORKSPACE;
    // what the call writes (lengths, results, workspace) must not overlap
    // anything else it reads or writes; lens itself is read and written
    const size_t lb = (size_t)B * T * V * 4, qb = (size_t)B * gamma * V * 4, db = (size_t)B * gamma * 4;
    const void* ins[5] = {logits, greedy ? nullptr : q, drafts, greedy ? nullptr : u, greedy ? nullptr : r};
    const size_t in_sz[5] = {lb, qb, db, db, (size_t)B * 4};
    const void* outs[3] = {lens, result, workspace};
    const size_t out_sz[3] = {(size_t)B * 4, (size_t)B * 8, plan.total_bytes};
    for (int a = 0; a < 3; ++a) {
        for (int c = 0; c < 5; ++c)
            if (ins[c] && in_sz[c] && overlaps(outs[a], out_sz[a], ins[c], in_sz[c])) return DECATTN_ERR_INVALID_ARG;
        for (int c = a + 1; c < 3; ++c)
            if (overlaps(outs[a], out_sz[a], outs[c], out_sz[c])) return DECATTN_ERR_INVALID_ARG;
    }
    SpecParams sp{};
    sp.logits = logits;
    sp.q = q;
    sp.drafts = drafts;
    sp.u = u;
    sp.r = r;
    sp.lens = lens;
    sp.result = result;
    char* ws = static_cast<char*>(workspace);
    sp.stats = reinterpret_cast<float2*>(ws);
    sp.parts = reinterpret_cast<float2*>(ws + plan.stats_bytes);
    sp.rowinfo = reinterpret_cast<float4*>(ws + plan.stats_bytes + plan.parts_bytes);
    sp.dinfo = reinterpret_cast<float4*>(ws + plan.stats_bytes + plan.parts_bytes + plan.rowinfo_bytes);
    sp.c2 = c2;
    sp.T = T;
    sp.V = V;
    sp.NC = plan.NC;
    sp.NC2 = plan.NC2;
    sp.stage_n = T * plan.NC < kSpecStage ? T * plan.NC : kSpecStage;
    sp.S_max = S_max;
    const bool vec = V % 4 == 0 && aligned16(logits) && (greedy || gamma == 0 || aligned16(q));
    const hipStream_t s = static_cast<hipStream_t>(stream);
    switch (plan.U) {
        case 1: spec_launch_u<1>(sp, B, vec, greedy, s); break;
        case 2: spec_launch_u<2>(sp, B, vec, greedy, s); break;
        case 4: spec_launch_u<4>(sp, B, vec, greedy, s); break;
        default: spec_launch_u<8>(sp, B, vec, greedy, s); break;
    }
    if (greedy) {
        hipLaunchKernelGGL(spec_greedy_kernel, dim3((unsigned)B), dim3(kSpecThreads),
                           (size_t)sp.stage_n * sizeof(float2), s, sp);
    } else {
        switch (plan.U2) {
            case 1: spec_launch_draw_u<1>(sp, B, vec, s); break;
            case 2: spec_launch_draw_u<2>(sp, B, vec, s); break;
            case 4: spec_launch_draw_u<4>(sp, B, vec, s); break;
            default: spec_launch_draw_u<8>(sp, B, vec, s); break;
        }
    }
    return hipGetLastError() == hipSuccess ? DECATTN_OK : DECATTN_ERR_HIP;
}

int decattn_probe_read(const void* buf, size_t bytes, void* sink, void* stream) {
    if (!buf || !sink || !aligned16(buf) || (bytes & 15u) || bytes == 0) return DECATTN_ERR_INVALID_ARG;
    const size_t n16 = bytes / 16;
    const size_t blocks = (n16 + kProbeBlockWords - 1) / kProbeBlockWords;
    if (blocks > 0x7FFFFFFF) return DECATTN_ERR_INVALID_ARG;
    hipLaunchKernelGGL(probe_read, dim3((unsigned)blocks), dim3(kProbeThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf), n16,
                       static_cast<uint32_t*>(sink));
    return hipGetLastError() == hipSuccess ? DECATTN_OK : DECATTN_ERR_HIP;
}

int decattn_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (!dst || !src || !aligned16(dst) || !aligned16(src) || (bytes & 15u) || bytes == 0)
        return DECATTN_ERR_INVALID_ARG;
    const size_t n16 = bytes / 16;
    size_t blocks = (n16 + kProbeThreads - 1) / kProbeThreads;
    if (blocks > 256 * 16) blocks = 256 * 16;
    hipLaunchKernelGGL(probe_copy, dim3((unsigned)blocks), dim3(kProbeThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<uint4*>(dst),
                       static_cast<const uint4*>(src), n16);
    return hipGetLastError() == hipSuccess ? DECATTN_OK : DECATTN_ERR_HIP;
}

}  // extern "C"
