/*
 * libdecattn — split-KV single-query decode attention ("flash-decoding") for
 * AMD Instinct MI355X (gfx950), as a plain C ABI.
 *
 * The operation (tinydecode README, "how the decode step is put together"):
 * for every batch row b and query head h, with G = Hq / Hkv query heads per kv
 * head and kvh = h / G,
 *
 *     out[b,h,:] = sum_{j < n_b} softmax_j(scale * <q[b,h,:], K[b,kvh,j,:]>) V[b,kvh,j,:]
 *
 * where n_b = seq_lens[b] is read on the device. The work is split over tiles
 * of `chunk` keys: each workgroup takes one (b, kvh, chunk) tile, serves all G
 * query heads of that kv head and writes partial softmax state (m, l, acc);
 * a second kernel merges the tiles with the log-sum-exp rule (llm-decode-cuda,
 * attention section). The grid depends only on S_max, never on seq_lens, and
 * tiles past a row's length exit at once, so a call can be captured in a
 * hipGraph and replayed after seq_lens changes on the device.
 *
 * Conventions shared by every entry point
 *  - Pointers are DEVICE pointers owned by the caller (q, caches, lengths,
 *    out, workspace), except where a comment says otherwise. The library
 *    allocates nothing, keeps no device state and never synchronizes; every
 *    launch is asynchronous on `stream` (a hipStream_t; NULL = null stream).
 *  - bf16 tensors are raw bf16 bit patterns (uint16), contiguous row-major,
 *    16-byte aligned. The KV cache of one layer is [B][Hkv][S_max][D] (one
 *    layer's slice of the [layer][sequence][kv_head][position][dim] layout of
 *    llm-decode-cuda's design notes).
 *  - Arguments are checked on the host before anything is launched; a failed
 *    check returns a status and launches nothing. Device-resident lengths are
 *    not validated (that would need a host sync): the kernels clamp them to
 *    [0, S_max], and a row with no keys outputs zeros.
 *  - Supported: D in {64, 128}; G = Hq / Hkv in 1..8; Hq <= 2^24; T in 1..16; chunk 0
 *    (library default) or a power of two in [16, 2^20] (a chunk >= S_max
 *    means one tile per row); B <= 4096; one kv head's cache, plus 512 keys
 *    of slack, within a 32-bit byte range: (S_max + 512) * D * 2 < 2^32, i.e.
 *    S_max <= 16776703 at D = 128 and <= 33553919 at D = 64. Shapes outside
 *    this set give DECATTN_ERR_UNSUPPORTED, and decattn_workspace_bytes /
 *    decattn_default_chunk return 0 for them.
 *  - Lengths and the token offsets added to them (ctx + i + 1) are summed in
 *    64 bits before the clamp, so any int32 length is safe.
 *  - Errors are returned, never thrown; no C++ exception crosses this ABI.
 */
#ifndef DECATTN_H
#define DECATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DECATTN_ABI_VERSION 1

typedef enum {
    DECATTN_OK = 0,
    DECATTN_ERR_INVALID_ARG = 1,   /* null pointer, bad dimension, misalignment, Hq % Hkv != 0 */
    DECATTN_ERR_UNSUPPORTED = 2,   /* D, G, T or chunk outside the supported set */
    DECATTN_ERR_WORKSPACE = 3,     /* workspace smaller than decattn_workspace_bytes() */
    DECATTN_ERR_HIP = 4            /* the HIP runtime rejected a launch */
} decattn_status;

typedef enum {
    DECATTN_OUT_BF16 = 0,          /* fp32 result rounded to nearest-even bf16 */
    DECATTN_OUT_F32 = 1
} decattn_out_dtype;

/* DECATTN_ABI_VERSION of the built library. */
int decattn_abi_version(void);

/* Static, NUL-terminated description of a status code (unknown codes included). */
const char* decattn_status_str(int status);

/* Keys per tile the library picks when `chunk` is 0, for these shapes on the
 * current device: a verify chunk takes 512-key tiles when all of them, but not
 * all 256-key tiles, fit on the device at once (256 otherwise, and 256 with no
 * device). Returns 0 when the shapes are invalid or unsupported. */
int decattn_default_chunk(int B, int T, int Hq, int Hkv, int D, int S_max);

/* Bytes of device workspace a call with these shapes needs (T = 1 for decode):
 * the partial state of every tile, B*T*Hq*ceil(S_max/chunk)*(D+2)*4 bytes plus
 * alignment. Returns 0 when the shapes are invalid or unsupported. */
size_t decattn_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int S_max, int chunk);

/* Single-query decode attention (the flash-decoding step of tinydecode's
 * README and llm-decode-cuda's attention section).
 *   q          bf16 [B][Hq][D]
 *   k_cache    bf16 [B][Hkv][S_max][D]
 *   v_cache    bf16 [B][Hkv][S_max][D]
 *   seq_lens   int32 [B], device; row b attends keys j < seq_lens[b]
 *   scale      softmax scale (typically 1/sqrt(D)), applied to q.k
 *   out        [B][Hq][D], bf16 or fp32 per out_dtype
 *   workspace  >= decattn_workspace_bytes(B, 1, Hq, Hkv, D, S_max, chunk) bytes,
 *              16-byte aligned; overwritten, may be reused between calls on the
 *              same stream
 *   chunk      keys per split tile; 0 = decattn_default_chunk()
 * Launches two kernels (partial tiles, then the merge) on `stream`.
 * Precision: fp32 scores, softmax statistics and accumulation. The vector
 * kernel weights V with fp32 softmax weights; the matrix-core kernel (see
 * chunk_attn) carries them as bf16 hi + lo parts (about 16 bits) for fp32
 * output and as bf16 (each within 2^-9 of itself, below the output's own
 * rounding step) for bf16 output. */
int decode_attn(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* seq_lens,
                int B, int Hq, int Hkv, int D, int S_max, float scale,
                void* out, int out_dtype,
                void* workspace, size_t workspace_bytes, int chunk,
                void* stream);

/* decode_attn for callers that cannot allocate device memory: code under
 * hipGraph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels and results as decode_attn (bit for bit, same
 * chunk), with no workspace argument: the partial state goes to a static
 * device array of DECATTN_NOALLOC_SCRATCH_BYTES inside the library, one per
 * GPU, held until the process ends. The call allocates nothing and calls no
 * allocating routine. Limits and behaviour:
 *  - shapes whose workspace (decattn_workspace_bytes with T = 1) exceeds
 *    DECATTN_NOALLOC_SCRATCH_BYTES are refused with DECATTN_ERR_WORKSPACE
 *    before anything is launched (pass a larger chunk, or use decode_attn);
 *  - every call on one GPU shares that GPU's array: calls that may overlap in
 *    time on one GPU (two streams, two threads) race and must be ordered by
 *    the caller, e.g. kept on one stream; the partial kernel writes every slot
 *    the merge reads, so no clearing is needed between calls;
 *  - the first call on each device looks up the array's device address
 *    (hipGetSymbolAddress, host side only) and keeps it; make that first call
 *    outside graph capture. A failed lookup returns DECATTN_ERR_HIP. */
#define DECATTN_NOALLOC_SCRATCH_BYTES (8u << 20)
int decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seq_lens,
                        int B, int Hq, int Hkv, int D, int S_max, float scale,
                        void* out, int out_dtype, int chunk, void* stream);

/* Causal multi-query "chunk" attention for verifying T speculative tokens
 * (tinydecode README, "speculative decoding": the verify pass runs k+1 tokens
 * on top of the existing context, reading the cache once for all of them).
 *   q          bf16 [B][T][Hq][D]
 *   ctx_lens   int32 [B], device; query token i of row b attends keys
 *              j < ctx_lens[b] + i + 1 (the T tokens' own K/V must already be
 *              at positions ctx .. ctx+T-1; the caller keeps ctx + T <= S_max,
 *              and the kernels clamp every limit to S_max)
 *   out        [B][T][Hq][D]
 *   workspace  >= decattn_workspace_bytes(B, T, Hq, Hkv, D, S_max, chunk)
 * Other arguments as decode_attn. Row (i, h) equals decode_attn on the same
 * cache with seq_lens = ctx + i + 1, the same chunk and output type: bit for
 * bit when both calls run on the same kernel, and otherwise to fp32 rounding
 * (|diff| <= 1e-4 of O(1) fp32 outputs; bf16 outputs within the bf16
 * tolerance of the exact result), since the two kernels sum q.k in different
 * orders and weight V at the precisions decode_attn states. The
 * matrix-core kernel runs a chunk call when T*G <= 32 rows per kv head and
 * chunk is a multiple of 128 (the default chunk is), and a decode call when
 * G >= 8 and chunk is a multiple of 128; the vector kernel runs the others. */
int chunk_attn(const void* q, const void* k_cache, const void* v_cache,
               const int32_t* ctx_lens,
               int B, int T, int Hq, int Hkv, int D, int S_max, float scale,
               void* out, int out_dtype,
               void* workspace, size_t workspace_bytes, int chunk,
               void* stream);

/* Causal attention of many query tokens (prefill, or a long chunk of it) on
 * the matrix cores: the chunk_attn operation for any T (query token i of row
 * b attends keys j < ctx_lens[b] + i + 1, clamped to S_max; the T tokens' K/V
 * already sit at positions ctx .. ctx+T-1), read with the tiled online
 * softmax that tinydecode's verify pass and llm-decode-cuda's next step call
 * for, with no split over keys and so no workspace.
 *   q          bf16 [B][T][Hq][D];  out [B][T][Hq][D], bf16 or fp32
 *   k_cache, v_cache, ctx_lens, scale as chunk_attn
 * bf16 output uses bf16 softmax weights in p.V; fp32 output carries them as
 * bf16 hi + lo parts (about 16 bits), which keeps |out - exact| within 1e-4.
 * One launch, no host sync, capturable. D in {64, 128}; G = Hq/Hkv in 1..8;
 * (S_max + 512) * D * 2 < 2^32. Rows with no key (ctx + i + 1 <= 0) output 0. */
int prefill_attn(const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* ctx_lens,
                 int B, int T, int Hq, int Hkv, int D, int S_max, float scale,
                 void* out, int out_dtype, void* stream);

/* The weight products of a decode step (llm-decode-cuda: roofline paragraph,
 * GEMV table, INT8 section): y[b][n] = sum_k W[n][k] x[b][k] for B <= 8
 * activation vectors. Each weight is read once per call (bytes-bound).
 *   W        bf16 [N][K] row-major (gemv_bf16), or
 *   Wq,scale int8 [N][K] row-major with one fp32 scale per row (gemv_int8):
 *            the weight is q * scale[n]
 *   x        bf16 [B][K];  y [B][N], fp32 or bf16 per out_dtype
 * Products accumulate in fp32. K must be a multiple of 8 (bf16) or 16 (int8);
 * B in 1..8, K up to 73728 (one staged vector fits 144 KB of LDS; larger K
 * gives DECATTN_ERR_UNSUPPORTED). One vector runs as dot products on the
 * vector units, with the vector in LDS (bf16 matrices of 16384 rows or more:
 * on the matrix cores); 2 to 8 run on the matrix cores in one launch
 * (16 x 16 x 32 bf16 products, INT8 codes widened to bf16 exactly). No host sync, capturable. W, Wq, x, y 16-byte aligned; scale
 * 4-byte aligned; (N + 64) * K weight bytes and B * K * 2 activation bytes
 * below 2^32. */
int gemv_bf16(const void* W, const void* x, int B, int N, int K,
              void* y, int out_dtype, void* stream);
int gemv_int8(const void* Wq, const float* scale, const void* x, int B, int N, int K,
              void* y, int out_dtype, void* stream);

/* Per-output-row symmetric INT8 quantization, done once when weights are
 * loaded (llm-decode-cuda, INT8 section), in fp32: a = max_k |W[n][k]|,
 * scale[n] = a / 127, Wq[n][k] = round-half-even(W[n][k] / scale[n]) in
 * [-127, 127]; a row of zeros gets scale 0 and codes 0.
 *   W bf16 [N][K] (K a multiple of 16) -> Wq int8 [N][K], scale fp32 [N];
 * the three buffers must not overlap. */
int quantize_rows_int8(const void* W, int N, int K, void* Wq, float* scale, void* stream);

/* The accept/reject step of speculative decoding after the verify pass, with
 * the rollback of the cache lengths, on the device (tinydecode README,
 * "speculative decoding"; the FlashSpec page's correctness paragraph, which
 * restates Leviathan et al. 2023, Algorithm 1). Per row b, gamma = T - 1:
 *   p_i = softmax(logits[b][i] / tau) for the T verified positions (position
 *   i scores the token after draft i-1; position gamma is the bonus row);
 *   draft i is kept while log u_i < log p_i(d_i) - log q_i(d_i) (log 0 = -inf,
 *   so u_i = 0 or q_i(d_i) = 0 keeps it; an id outside [0, V) is rejected);
 *   n = the number kept before the first rejection;
 *   the next token is drawn with r[b] by inverse CDF in vocabulary order from
 *   max(0, p_n - q_n) (n < gamma; from p_n if that has no positive mass) or
 *   from p_gamma (n = gamma): the first index k with positive weight whose
 *   running sum exceeds r * total (the last positive index if rounding leaves
 *   none);
 *   tau == 0 is greedy: draft i is kept while it equals argmax logits[b][i]
 *   (first index on ties) and the next token is argmax logits[b][n];
 *   lens[b] <- min(clamp(lens[b], 0, S_max) + n + 1, S_max): the pending token
 *   and the kept drafts stay in the cache, entries past the new length are
 *   stale and never read; the next token is the next pending one.
 *   logits   fp32 [B][T][V], finite or -inf, at least one finite per row
 *   q        fp32 [B][T-1][V]: the draft distributions the drafts came from
 *            (sampling only; NULL allowed when tau == 0 or T == 1)
 *   drafts   int32 [B][T-1] (NULL allowed when T == 1)
 *   u        fp32 [B][T-1] uniforms in [0, 1); r fp32 [B] uniforms in [0, 1)
 *            (sampling only; NULL allowed when tau == 0, u also when T == 1)
 *   tau      0 (greedy) or a positive temperature with log2(e)/tau finite
 *   lens     int32 [B], device, read and written: the length before the verify
 *            pass (ctx_lens of chunk_attn)
 *   result   int32 [B][2]: {n, next token}, one device-to-host read per step
 *   workspace >= spec_accept_workspace_bytes(B, T, V) bytes, 16-byte aligned;
 *            overwritten; calls that share it must be ordered on one stream
 * T in 1..32, V in 1..2^24. lens, result and workspace must not overlap each
 * other or the inputs (checked). Three launches on `stream` (two when
 * tau == 0), no host sync, capturable. */
size_t spec_accept_workspace_bytes(int B, int T, int V);
int spec_accept(const float* logits, const float* q, const int32_t* drafts, const float* u, const float* r,
                float tau, int B, int T, int V, int S_max, int32_t* lens, int32_t* result,
                void* workspace, size_t workspace_bytes, void* stream);

/* The two phases of decode_attn / chunk_attn as separate launches, for callers
 * that time them apart or merge partial state produced elsewhere.
 * `causal` = 0 gives decode (T must be 1, lens = seq_lens); 1 gives chunk
 * (lens = ctx_lens). attn_partial writes the workspace; attn_merge reads it and
 * must be given the same shapes, lens, causal flag and chunk. attn_partial
 * does not know the output type, so it keeps the fp32-output precision (on
 * the matrix cores, softmax weights as bf16 hi + lo): the pair equals
 * decode_attn / chunk_attn bit for bit for fp32 output, and for bf16 output
 * wherever the vector kernel runs. */
int attn_partial(const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* lens,
                 int B, int T, int Hq, int Hkv, int D, int S_max, float scale, int causal,
                 void* workspace, size_t workspace_bytes, int chunk,
                 void* stream);

int attn_merge(const int32_t* lens,
               int B, int T, int Hq, int Hkv, int D, int S_max, int causal,
               void* out, int out_dtype,
               void* workspace, size_t workspace_bytes, int chunk,
               void* stream);

/* The step before attention: rotary position embedding of a step's new
 * tokens and the write of their K/V into the static cache (tinydecode README,
 * "What's in here": in-place rope; "how the decode step is put together":
 * positions come from the device-resident lengths and the K/V write is an
 * indexed store at those positions; llm-decode-cuda's per-layer step list,
 * which puts the rotation and the cache write in one step; the llama3 flavour
 * of rope scaling as the only one, tinydecode README, "not done / known gaps").
 *
 * Token i of row b sits at position p = clamp(pos0[b], 0, S_max) + i. Pair j
 * of every head (j < D/2) turns by the angle p * f_j, f_j = theta^(-2j/D)
 * (llama3-scaled when asked): a pair (a, b) becomes (a cos - b sin,
 * a sin + b cos), computed in fp64 and rounded once to nearest-even bf16.
 *   q_in       bf16 [B][T][Hq][D]; q_out bf16 [B][T][Hq][D] receives the
 *              rotated q; q_out == q_in rotates in place (any other overlap
 *              with q_in is rejected)
 *   k_in, v_in bf16 [B][T][Hkv][D]: the new tokens' keys (unrotated) and values
 *   pos0       int32 [B], device: each row's length before the step (seq_lens
 *              for decode, ctx_lens for a verify chunk)
 *   k_cache, v_cache  bf16 [B][Hkv][S_max][D]: slot p of row b, head h gets
 *              the rotated k and the unchanged v of token i; a token with
 *              p >= S_max has no slot and writes no K/V (its q is still
 *              rotated at p); every other slot is left as it was
 *   rope       HOST pointer to the frequency description
 * The caller keeps pos0 + T <= S_max in normal use and advances its lengths
 * afterwards (for decode: attention over j < pos0 + 1, e.g. chunk_attn with
 * T = 1 and ctx_lens = pos0). k_in, v_in, the caches, pos0 and q_out must
 * not overlap (checked on the host). One launch of B*T workgroups; D in
 * {64, 128}; Hq % Hkv == 0. */
typedef enum {
    DECATTN_ROPE_HALF = 0,         /* pairs (x_j, x_{j+D/2}): the Hugging Face Llama layout */
    DECATTN_ROPE_ADJACENT = 1      /* pairs (x_{2j}, x_{2j+1}): the RoFormer paper's layout */
} decattn_rope_pairing;

typedef struct {
    double theta;                  /* frequency base, > 0 */
    int pairing;                   /* decattn_rope_pairing */
    int llama3_scaling;            /* 0: none; 1: llama3 frequency scaling with the fields below */
    double factor;                 /* low frequencies are divided by this */
    double low_freq_factor;        /* wavelengths above original_max_position / low_freq_factor: divided */
    double high_freq_factor;       /* wavelengths below original_max_position / high_freq_factor: kept */
    double original_max_position;  /* in between: linear blend in original_max_position / wavelength */
} decattn_rope;

int rope_kv_write(const void* q_in, const void* k_in, const void* v_in, const int32_t* pos0,
                  int B, int T, int Hq, int Hkv, int D, int S_max, const decattn_rope* rope,
                  void* q_out, void* k_cache, void* v_cache, void* stream);

/* Measurement helpers (the streaming-read probe of llm-decode-cuda's roofline
 * section). decattn_probe_read reads `bytes` (a multiple of 16) from `buf`
 * with 16-byte loads and writes at most 4 bytes to `sink`; decattn_probe_copy
 * copies `bytes` (a multiple of 16) from src to dst. Both 16-byte aligned. */
int decattn_probe_read(const void* buf, size_t bytes, void* sink, void* stream);
int decattn_probe_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DECATTN_H */
