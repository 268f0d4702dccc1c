"""HIP path vs the fp64 oracle on the same seeded bytes, through the C ABI.

Tolerances: max-abs 1e-4 for fp32 output and 1e-2 for bf16 output (bf16
elements beyond 1e-2 must be adjacent to the exact value); masks, indices,
early exits and batch/head isolation are checked bit-exactly.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import stream_decode_attention_amd as sda
import workloads
from workloads import BF16_NAN
from tests.gpu_util import (assert_bf16_close, assert_f32_close, bits_of, dev_bits, dev_lens,
                            run_chunk, run_decode, workspace)

pytestmark = pytest.mark.gpu


def _both_modes(c, ref, **kw):
    out32 = run_decode(c, out_dtype=torch.float32, **kw)
    assert_f32_close(out32, ref)
    out16 = run_decode(c, out_dtype=torch.bfloat16, **kw)
    assert_bf16_close(out16, ref)
    return out32, out16


# ------------------------------------------------------------- the five workloads

def test_workload1_single_call_both_modes():
    c = workloads.make_config(1)
    ref = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    _both_modes(c, ref, chunk=32)


@pytest.mark.parametrize("n", [64, 1024, 2048, 4096])
def test_workload2_smollm_layer(n):
    c = workloads.make_config(2, layer=n % 7, n=n)
    ref = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    _both_modes(c, ref)


@pytest.mark.parametrize("n", [1024, 4096, 8192])
def test_workload3_tinyllama_outlier_keys(n):
    c = workloads.make_config(3, layer=1, n=n)
    ref = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    _both_modes(c, ref)


def test_workload4_batched_ragged_full_size_every_row():
    """The headline call at full size (B=8, Hq=32, S_max=32768, ragged lengths):
    all 256 output rows against the oracle, in both output modes."""
    c = workloads.make_config(4)
    ref = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    tensors = (dev_bits(c["q"]), dev_bits(c["k"]), dev_bits(c["v"]))
    out32 = run_decode(c, tensors=tensors)
    assert_f32_close(out32, ref)
    out16 = run_decode(c, tensors=tensors, out_dtype=torch.bfloat16)
    assert_bf16_close(out16, ref)
    # the bf16 output is the fp32 output rounded to nearest even
    rne = out32.to(torch.bfloat16)
    assert torch.equal(rne.view(torch.int16), out16.view(torch.int16))


@pytest.mark.parametrize("chunk", [None, 256])
def test_workload5_verify_chunk_vs_oracle_and_sequential_decodes(chunk):
    """The default tile (512 keys on MI355X: every tile in one round of
    workgroups) and 256-key tiles (264 tiles on 256 resident workgroups: the
    persistent walk, which folds the short last tiles)."""
    c = workloads.make_config(5)
    ref = oracle.chunk_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    tensors = (dev_bits(c["q"]), dev_bits(c["k"]), dev_bits(c["v"]))
    kw = {} if chunk is None else {"chunk": chunk}
    out32 = run_chunk(c, tensors=tensors, **kw)
    assert_f32_close(out32, ref)
    out16 = run_chunk(c, tensors=tensors, out_dtype=torch.bfloat16, **kw)
    assert_bf16_close(out16, ref)
    # six sequential decode calls: token i with seq_len = ctx + i + 1. The
    # verify chunk runs on the matrix cores, the decode calls on the vector
    # path: equal to the fp32 tolerance (each within it of the oracle)
    T = c["q"].shape[1]
    for i in range(T):
        ci = dict(c, q=np.ascontiguousarray(c["q"][:, i]), lens=c["lens"] + i + 1)
        dec = run_decode(ci, tensors=(dev_bits(ci["q"]), tensors[1], tensors[2]))
        d = (dec - out32[:, i]).abs().max().item()
        assert d <= 1e-4, f"token {i}: chunk row and its decode call differ by {d}"


def test_verify_default_chunk_follows_one_round_capacity():
    """The default verify tile is 512 keys exactly when every 512-key tile, but
    not every 256-key tile, fits in one round of workgroups (one matrix-core
    workgroup per compute unit at D = 128)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    Hkv = 8
    for S in (4096 + 6, 8192 + 6, 16384 + 6, 65536):
        n256, n512 = Hkv * -(-S // 256), Hkv * -(-S // 512)
        expect = 512 if (n256 > cus and n512 <= cus) else 256
        assert sda.default_chunk(1, 6, 3 * Hkv, Hkv, 128, S) == expect, S


@pytest.mark.parametrize("T,G,chunk", [(6, 3, 64), (16, 3, 256), (4, 8, 32)])
def test_vector_chunk_path_bit_identical_to_sequential_decodes(T, G, chunk):
    # chunks below 128 keys, or more than 32 rows per kv head, take the vector
    # path, whose rows run exactly the decode operation sequence
    Hkv = 2
    c = workloads.make_case(1, G * Hkv, Hkv, 128, 1024, [700], T=T, seed=T * 10 + G)
    out = run_chunk(c, chunk=chunk)
    ref = oracle.chunk_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    assert_f32_close(out, ref)
    kt, vt = dev_bits(c["k"]), dev_bits(c["v"])
    for i in range(T):
        ci = dict(c, q=np.ascontiguousarray(c["q"][:, i]), lens=c["lens"] + i + 1)
        dec = run_decode(ci, chunk=chunk, tensors=(dev_bits(ci["q"]), kt, vt))
        assert torch.equal(dec, out[:, i]), f"token {i}: chunk row differs from its decode call"


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T,G,chunk", [(6, 3, 256), (2, 8, 128), (5, 6, 512), (1, 4, 256), (16, 2, 1024)])
def test_matrix_core_chunk_path_vs_oracle(D, T, G, chunk):
    Hkv = 3
    c = workloads.make_case(2, G * Hkv, Hkv, D, 1500, [1200, 90], T=T, seed=D + T * 7 + G + chunk)
    if T == 1:
        c["q"] = c["q"].reshape(2, 1, G * Hkv, D)
    ref = oracle.chunk_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    assert_f32_close(run_chunk(c, chunk=chunk), ref)
    assert_bf16_close(run_chunk(c, chunk=chunk, out_dtype=torch.bfloat16), ref)


@pytest.mark.parametrize("chunk", [128, 256])
def test_matrix_core_context_just_past_a_tile_boundary(chunk):
    """Sequence 0's keys end 4 into a new tile, so its first two query rows read
    one tile fewer than the other four; sequence 1 ends 46 keys into its last
    tile. The workspace starts as NaN everywhere."""
    c = workloads.make_case(2, 9, 3, 128, 4 * chunk + 64, [3 * chunk - 2, 2 * chunk + 40], T=6,
                            seed=77 + chunk)
    ref = oracle.chunk_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    assert_f32_close(run_chunk(c, chunk=chunk), ref)
    assert_bf16_close(run_chunk(c, chunk=chunk, out_dtype=torch.bfloat16), ref)


# ------------------------------------- batched decode on the persistent walk

# Shapes with more possible tiles than the device holds at once (the
# persistent tile walk): rows far shorter than a tile next to full ones, many
# sequences of random lengths, rows ending off tile boundaries.

@pytest.mark.parametrize("B,Hkv,G,D,S,lens", [
    # short rows (0, 1, 15, 17 keys) next to long ones
    (8, 8, 4, 128, 8192, [0, 1, 15, 17, 300, 8192, 5000, 2]),
    # 64 sequences of random lengths, every fifth under 40 keys
    (64, 2, 3, 64, 4096, None),
    # long rows ending off tile boundaries
    (4, 8, 4, 128, 32768, [30001, 29999, 32768, 31000]),
])
def test_persistent_walk_ragged_batches_vs_oracle(B, Hkv, G, D, S, lens):
    if lens is None:
        lens = np.random.default_rng(71).integers(0, S + 1, size=B)
        lens[::5] = np.random.default_rng(72).integers(0, 40, size=len(lens[::5]))
    c = workloads.make_case(B, G * Hkv, Hkv, D, S, lens, seed=70 + B)
    ref = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    tensors = (dev_bits(c["q"]), dev_bits(c["k"]), dev_bits(c["v"]))
    assert_f32_close(run_decode(c, tensors=tensors), ref)
    assert_bf16_close(run_decode(c, tensors=tensors, out_dtype=torch.bfloat16), ref)


def test_persistent_walk_nan_poison_past_length_is_never_read():
    lens = [1, 4095, 20, 2048, 0, 4096, 333, 17]
    c = workloads.make_case(8, 32, 8, 128, 4096, lens, seed=73)
    poisoned = dict(c, k=c["k"].copy(), v=c["v"].copy())
    for b, n in enumerate(lens):
        poisoned["k"][b, :, n:] = BF16_NAN
        poisoned["v"][b, :, n:] = BF16_NAN
    for dt in (torch.float32, torch.bfloat16):
        a = run_decode(c, out_dtype=dt)
        p = run_decode(poisoned, out_dtype=dt)
        assert torch.equal(a.view(torch.int16), p.view(torch.int16))
        assert not torch.isnan(p.float()).any()


def test_persistent_walk_graph_replay_follows_device_lengths():
    """The attended-tile list depends on the lengths, which change on the
    device between replays of one captured call."""
    c = workloads.make_case(8, 32, 8, 128, 8192, [8192] * 8, seed=74)
    q, k, v = dev_bits(c["q"]), dev_bits(c["k"]), dev_bits(c["v"])
    lens = dev_lens([8192] * 8)
    ws = workspace(8, 1, 32, 8, 128, 8192, 0, poison=True)
    out = torch.zeros((8, 32, 128), device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sda.decode_attn(q, k, v, lens, c["scale"], out, ws)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sda.decode_attn(q, k, v, lens, c["scale"], out, ws)
    rng = np.random.default_rng(75)
    for trial in range(4):
        n = rng.integers(0, 8193, size=8).astype(np.int32)
        if trial == 3:
            n[:] = 0
        lens.copy_(torch.from_numpy(n))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref = oracle.decode_attention(c["q"], c["k"], c["v"], n, c["scale"])
        assert_f32_close(got, ref)
        assert torch.equal(got, run_decode(c, lens=n, tensors=(q, k, v))), f"replay {trial} differs from eager"


# ------------------------------------------------------------- size extremes

def test_row_with_more_tiles_than_one_merge_batch():
    """1250 tiles in one row: the merge folds them in batches of 64 (8 tile
    lanes of eight slots at D = 128), 20 rounds."""
    c = workloads.make_case(2, 4, 1, 128, 40000, [40000, 17000], seed=41)
    ref = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    assert_f32_close(run_decode(c, chunk=32), ref)
    assert_bf16_close(run_decode(c, chunk=32, out_dtype=torch.bfloat16), ref)


def test_row_with_more_tiles_than_one_merge_batch_d64():
    """D = 64: 1000 tiles in the first row (8 batches of 128, the last one
    partial), 129 in the second (one tile into the second batch), and a row of
    0 keys."""
    c = workloads.make_case(3, 6, 2, 64, 16000, [16000, 2064, 0], seed=42)
    ref = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    assert_f32_close(run_decode(c, chunk=16), ref)
    assert_bf16_close(run_decode(c, chunk=16, out_dtype=torch.bfloat16), ref)


@pytest.mark.parametrize("D", [64, 128])
def test_tile_counts_around_one_merge_batch(D):
    """The merge takes 64 tiles per round trip at D = 128 and 128 at D = 64:
    rows of 63, 64 and 65 tiles (the 65th holding one key), 127, 128 and 129,
    next to an empty row."""
    lens = [63 * 16 - 5, 64 * 16, 64 * 16 + 1, 127 * 16 - 3, 128 * 16, 128 * 16 + 1, 0]
    c = workloads.make_case(len(lens), 4, 2, D, 2064, lens, seed=43 + D)
    ref = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    assert_f32_close(run_decode(c, chunk=16), ref)
    assert_bf16_close(run_decode(c, chunk=16, out_dtype=torch.bfloat16), ref)


@pytest.mark.parametrize("D", [64, 128])
def test_one_wave_merge_with_an_empty_row(D):
    """Two or four tile slots per row (S_max = 64, 32-key tiles at D = 128;
    S_max = 128 at D = 64): the merge runs one wave per row, whose zero fill of
    an empty row takes two passes at D = 128."""
    S = 64 if D == 128 else 128
    lens = [0, 1, 40, S]
    c = workloads.make_case(len(lens), 6, 2, D, S, lens, seed=44 + D)
    ref = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    out32, out16 = _both_modes(c, ref, chunk=32)
    assert torch.count_nonzero(out32[0]) == 0 and torch.count_nonzero(out16[0].float()) == 0


def test_largest_batch():
    """B = 4096 (the most lengths the kernels stage in LDS), lengths 0..16."""
    B = 4096
    rng = np.random.default_rng(42)
    lens = rng.integers(0, 17, size=B).astype(np.int32)
    c = workloads.make_case(B, 2, 1, 64, 16, lens, seed=42)
    ref = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    out = run_decode(c, chunk=16)
    assert_f32_close(out, ref)
    assert torch.all(out[torch.from_numpy(lens == 0).to(out.device)] == 0), "rows with no key must be zero"


def test_vector_chunk_path_at_most_tokens_and_group():
    """T = 16 tokens, G = 8: 128 query rows per kv head in 16 row groups."""
    c = workloads.make_case(2, 16, 2, 64, 700, [500, 33], T=16, seed=43)
    ref = oracle.chunk_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    assert_f32_close(run_chunk(c, chunk=64), ref)
    assert_f32_close(run_chunk(c), ref)


# ----------------------------------------------------------- shapes and chunking

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("chunk", [16, 32, 64, 128, 256, 2048])
def test_multi_tile_ragged_lengths_all_chunk_sizes(D, chunk):
    c = workloads.make_case(3, 8, 2, D, 1000, [1, 333, 1000], seed=D + chunk)
    ref = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    assert_f32_close(run_decode(c, chunk=chunk), ref)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 6, 7, 8])
def test_every_group_size(D, G):
    Hkv = 3
    c = workloads.make_case(2, G * Hkv, Hkv, D, 300, [300, 129], seed=10 * G + D)
    ref = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    _both_modes(c, ref, chunk=64)


@pytest.mark.parametrize("T,G,D,chunk", [(1, 2, 64, 64), (1, 8, 64, 64), (3, 2, 128, 64), (6, 3, 128, 128),
                                         (6, 3, 128, 64)])
def test_one_round_grids_with_many_kv_heads_and_sequences(T, G, D, chunk):
    """The one-round grids (kv head, tile, sequence) and the merge grid (kv head,
    group row, sequence): 12 kv heads (not a multiple of 8) over 3 sequences of
    ragged lengths, decode and chunk calls, vector and matrix-core kernels (the
    last case has more possible tiles than the matrix-core kernel's resident
    workgroups: the persistent walk beside the same merge grid)."""
    Hkv, S = 12, 512
    lens = [S - T, 1, 300] if T > 1 else [S, 1, 300]
    c = workloads.make_case(3, G * Hkv, Hkv, D, S, lens, T=T, seed=7 * G + T + D)
    if T == 1:
        ref = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
        _both_modes(c, ref, chunk=chunk)
    else:
        ref = oracle.chunk_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
        assert_f32_close(run_chunk(c, chunk=chunk), ref)
        assert_bf16_close(run_chunk(c, chunk=chunk, out_dtype=torch.bfloat16), ref)


@pytest.mark.parametrize("n", [1, 31, 32, 33, 63, 64, 65, 255, 256])
def test_length_boundaries(n):
    c = workloads.make_case(1, 6, 2, 64, 256, [n], seed=n)
    ref = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    for chunk in (32, 64):
        assert_f32_close(run_decode(c, chunk=chunk), ref)


def test_empty_negative_and_oversized_lengths():
    c = workloads.make_case(4, 8, 2, 128, 96, [0, -7, 500, 96], seed=5)
    clamped = np.array([0, 0, 96, 96], np.int32)
    ref = oracle.decode_attention(c["q"], c["k"], c["v"], clamped, c["scale"])
    for dt in (torch.float32, torch.bfloat16):
        out = run_decode(c, out_dtype=dt, chunk=32)
        o = out.view(torch.int16).cpu().numpy() if dt == torch.bfloat16 else out.cpu().numpy()
        assert np.all(o[0] == 0) and np.all(o[1] == 0)
        # a length beyond S_max behaves exactly as S_max
        same = run_decode(c, out_dtype=dt, chunk=32, lens=clamped)
        assert torch.equal(out.view(torch.int16), same.view(torch.int16))
    assert_f32_close(run_decode(c, chunk=32), ref)


@pytest.mark.parametrize("D", [64, 128])
def test_single_key_returns_v0_bit_exactly(D):
    c = workloads.make_case(2, 8, 4, D, 64, [1, 1], seed=6)
    v0 = c["v"][:, :, 0, :]                              # [B, Hkv, D] bf16 bits
    expect = np.repeat(v0, 2, axis=1)                    # G = 2
    out16 = run_decode(c, out_dtype=torch.bfloat16)
    assert np.array_equal(bits_of(out16), expect)
    out32 = run_decode(c, out_dtype=torch.float32)
    assert np.array_equal(out32.cpu().numpy(), oracle.bf16_bits_to_f64(expect).astype(np.float32))


# ------------------------------------------------------------ never-read slots

@pytest.mark.parametrize("D,chunk", [(64, 32), (128, 64), (128, 256)])
def test_nan_poison_past_length_is_never_read(D, chunk):
    lens = [1, 37, 64, 200]
    c = workloads.make_case(4, 8, 2, D, 256, lens, seed=7 + D)
    poisoned = dict(c, k=c["k"].copy(), v=c["v"].copy())
    for b, n in enumerate(lens):
        poisoned["k"][b, :, n:] = BF16_NAN
        poisoned["v"][b, :, n:] = BF16_NAN
    for dt in (torch.float32, torch.bfloat16):
        a = run_decode(c, chunk=chunk, out_dtype=dt)
        p = run_decode(poisoned, chunk=chunk, out_dtype=dt)
        assert torch.equal(a.view(torch.int16), p.view(torch.int16))
        assert not torch.isnan(p.float()).any()


def test_chunk_nan_poison_past_context_plus_t():
    c = workloads.make_case(2, 6, 2, 128, 300, [100, 257], T=5, seed=8)
    poisoned = dict(c, k=c["k"].copy(), v=c["v"].copy())
    for b, ctx in enumerate(c["lens"]):
        poisoned["k"][b, :, ctx + 5:] = BF16_NAN
        poisoned["v"][b, :, ctx + 5:] = BF16_NAN
    a = run_chunk(c, chunk=64)
    p = run_chunk(poisoned, chunk=64)
    assert torch.equal(a, p) and not torch.isnan(p).any()


@pytest.mark.parametrize("chunk", [128, 256])
def test_matrix_core_chunk_nan_poison_past_context_plus_t(chunk):
    c = workloads.make_case(2, 24, 8, 128, 700, [300, 517], T=6, seed=18 + chunk)
    poisoned = dict(c, k=c["k"].copy(), v=c["v"].copy())
    for b, ctx in enumerate(c["lens"]):
        poisoned["k"][b, :, ctx + 6:] = BF16_NAN
        poisoned["v"][b, :, ctx + 6:] = BF16_NAN
    a = run_chunk(c, chunk=chunk)
    p = run_chunk(poisoned, chunk=chunk)
    assert torch.equal(a, p) and not torch.isnan(p).any()


def test_rollback_shrinking_length_ignores_stale_tail():
    c = workloads.make_case(1, 8, 2, 128, 512, [512], seed=9)
    full = run_decode(c, chunk=64)
    short = run_decode(c, chunk=64, lens=np.array([300], np.int32))
    ref = oracle.decode_attention(c["q"], c["k"], c["v"], [300], c["scale"])
    assert_f32_close(short, ref)
    assert not torch.equal(full, short)


# ------------------------------------------------------- isolation, bit-exact

def test_gqa_perturbing_one_kv_head_changes_only_its_group():
    G, Hkv = 4, 4
    c = workloads.make_case(2, G * Hkv, Hkv, 128, 200, [200, 150], seed=10)
    base = run_decode(c, chunk=64)
    for kp in range(Hkv):
        pert = dict(c, v=c["v"].copy())
        pert["v"][1, kp, :150] ^= np.uint16(0x0040)          # flip a mantissa bit of every value
        out = run_decode(pert, chunk=64)
        changed = (out != base).any(-1).cpu().numpy()        # [B, Hq]
        expect = np.zeros_like(changed)
        expect[1, kp * G:(kp + 1) * G] = True
        assert np.array_equal(changed, expect)


def test_batch_rows_bit_identical_to_batch_one_calls():
    lens = [700, 5, 1024, 333]
    c = workloads.make_case(4, 16, 4, 64, 1024, lens, seed=11)
    full = run_decode(c, chunk=128)
    for b in range(4):
        cb = dict(c, q=c["q"][b:b + 1], k=c["k"][b:b + 1], v=c["v"][b:b + 1], lens=c["lens"][b:b + 1])
        one = run_decode(cb, chunk=128)
        assert torch.equal(one[0], full[b])


def test_chunk_row_unchanged_by_later_key():
    c = workloads.make_case(1, 6, 2, 128, 200, [120], T=4, seed=12)
    a = run_chunk(c, chunk=64)
    pert = dict(c, k=c["k"].copy())
    pert["k"][0, :, 122] ^= np.uint16(0x0100)                # key ctx+2: seen by tokens 2, 3
    b = run_chunk(pert, chunk=64)
    assert torch.equal(a[0, :2], b[0, :2])
    assert (a[0, 2:] != b[0, 2:]).any(-1).all()


@pytest.mark.parametrize("T,ctx", [(1, [50]), (3, [0]), (6, [8192]), (9, [300]), (16, [40])])
def test_chunk_shapes_vs_oracle(T, ctx):
    S = 8192 + 16 if ctx == [8192] else 512
    c = workloads.make_case(1, 24, 8, 128, S, ctx, T=T, seed=13 + T)
    c["q"] = c["q"].reshape(1, T, 24, 128)
    ref = oracle.chunk_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    assert_f32_close(run_chunk(c), ref)


@pytest.mark.parametrize("path", ["decode", "chunk_vector", "chunk_matrix_core"])
@pytest.mark.parametrize("scale_kind", ["negative", "zero", "large"])
def test_scale_sign_and_magnitude(path, scale_kind):
    D = 128 if path == "chunk_matrix_core" else 64
    if path == "decode":
        c = workloads.make_case(2, 12, 4, D, 700, [700, 65], seed=91)
        chunk = 64
    else:
        T, G = (6, 3) if path == "chunk_matrix_core" else (16, 3)     # 18 or 48 rows per kv head
        c = workloads.make_case(2, 3 * G, 3, D, 900, [600, 5], T=T, seed=92 + T)
        chunk = 256 if path == "chunk_matrix_core" else 64
    c["scale"] = {"negative": -1.0 / np.sqrt(D), "zero": 0.0, "large": 0.9}[scale_kind]
    if path == "decode":
        ref = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
        out = run_decode(c, chunk=chunk)
    else:
        ref = oracle.chunk_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
        out = run_chunk(c, chunk=chunk)
    assert_f32_close(out, ref)


@pytest.mark.parametrize("chunk", [64, 256])      # the vector path, then the matrix cores
def test_chunk_context_near_int_max_clamps_to_s_max(chunk):
    """ctx + i + 1 is summed in 64 bits before the clamp: a context near INT_MAX
    gives every row the whole cache, exactly as ctx = S_max does (a 32-bit sum
    would wrap negative and the partial and merge kernels would disagree on the
    row's tile count)."""
    S = 700
    c = workloads.make_case(2, 24, 8, 128, S, [2**31 - 3, 2**31 - 1], T=6, seed=61 + chunk)
    at_s = dict(c, lens=np.array([S, S], np.int32))
    ref = oracle.chunk_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    ref_s = oracle.chunk_attention(at_s["q"], at_s["k"], at_s["v"], at_s["lens"], at_s["scale"])
    assert np.array_equal(ref, ref_s)
    tensors = (dev_bits(c["q"]), dev_bits(c["k"]), dev_bits(c["v"]))
    for dt in (torch.float32, torch.bfloat16):
        big = run_chunk(c, chunk=chunk, out_dtype=dt, tensors=tensors)
        same = run_chunk(at_s, chunk=chunk, out_dtype=dt, tensors=tensors)
        assert torch.equal(big.view(torch.int16), same.view(torch.int16))
    assert_f32_close(run_chunk(c, chunk=chunk, tensors=tensors), ref)


def test_decode_length_int_max_clamps_to_s_max():
    c = workloads.make_case(2, 8, 2, 64, 300, [2**31 - 1, 300], seed=62)
    ref = oracle.decode_attention(c["q"], c["k"], c["v"], [300, 300], c["scale"])
    out = run_decode(c, chunk=64)
    assert_f32_close(out, ref)
    same = run_decode(c, chunk=64, lens=np.array([300, 300], np.int32))
    assert torch.equal(out, same)


def test_chunk_context_reaching_s_max_clamps():
    c = workloads.make_case(2, 8, 4, 64, 128, [125, 128], T=6, seed=14)
    ref = oracle.chunk_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    assert_f32_close(run_chunk(c, chunk=32), ref)


def test_phases_separately_equal_decode_attn():
    c = workloads.make_case(2, 32, 8, 128, 2048, [2048, 999], seed=15)
    q, k, v = dev_bits(c["q"]), dev_bits(c["k"]), dev_bits(c["v"])
    lens = dev_lens(c["lens"])
    ws = workspace(2, 1, 32, 8, 128, 2048, 128)
    out = torch.empty((2, 32, 128), device="cuda")
    sda.attn_partial(q, k, v, lens, c["scale"], ws, chunk=128)
    sda.attn_merge(lens, out, ws, T=1, Hq=32, Hkv=8, S_max=2048, chunk=128)
    torch.cuda.synchronize()
    assert torch.equal(out, run_decode(c, chunk=128, tensors=(q, k, v)))


# ------------------------------------------------------------------ hipGraph

def test_graph_replay_follows_device_lengths():
    c = workloads.make_case(1, 15, 5, 64, 4096, [4096], seed=16)
    q, k, v = dev_bits(c["q"]), dev_bits(c["k"]), dev_bits(c["v"])
    lens = dev_lens([64])
    ws = workspace(1, 1, 15, 5, 64, 4096, 0, poison=False)
    out = torch.zeros((1, 15, 64), device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            sda.decode_attn(q, k, v, lens, c["scale"], out, ws)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sda.decode_attn(q, k, v, lens, c["scale"], out, ws)
    for n in (64, 1024, 2048, 4096, 1, 3000, 64):
        lens.copy_(torch.tensor([n], dtype=torch.int32))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = run_decode(c, lens=np.array([n], np.int32), tensors=(q, k, v))
        assert torch.equal(got, eager), f"replay at n={n} differs from eager"
        ref = oracle.decode_attention(c["q"], c["k"], c["v"], [n], c["scale"])
        assert_f32_close(got, ref)


# ------------------------------------------------------------------- probes

def test_probe_copy_and_read():
    src = torch.randint(-2**31, 2**31 - 1, (1 << 20,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    sda.probe_copy(dst, src)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    sda.probe_read(src, sink)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
