"""Decode calls with eight or more query heads per kv head, on tiles of a
multiple of 128 keys, run on the matrix-core kernel in its decode mode (every
row attends j < seq_len). The same edge cases as the vector path: against the
fp64 oracle at the fp32 / bf16 tolerances, and bit-exactly where the method
fixes the result (a single key, keys past the length never read, kv-head and
batch-row isolation, a one-token causal chunk equal to its decode call)."""
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

G = 8


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("chunk", [128, 256])
def test_ragged_lengths_both_modes(D, chunk):
    # empty, one key, both sides of a tile edge, and the full cache
    lens = [0, 1, 127, 128, 129, 600, 1000]
    c = workloads.make_case(len(lens), G * 2, 2, D, 1000, lens, seed=300 + D + chunk)
    ref = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    out32 = run_decode(c, chunk=chunk)
    assert_f32_close(out32, ref)
    assert torch.count_nonzero(out32[0]) == 0
    assert_bf16_close(run_decode(c, chunk=chunk, out_dtype=torch.bfloat16), ref)


def test_tile_counts_around_one_merge_batch():
    """128-key tiles on the matrix cores: rows of 64 and 65 tiles (the last
    holding one key) around the merge's 64 tiles per round trip."""
    lens = [64 * 128, 64 * 128 + 1, 3000]
    c = workloads.make_case(len(lens), G, 1, 128, 64 * 128 + 128, lens, seed=305)
    ref = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    assert_f32_close(run_decode(c, chunk=128), ref)
    assert_bf16_close(run_decode(c, chunk=128, out_dtype=torch.bfloat16), ref)


@pytest.mark.parametrize("D", [64, 128])
def test_single_key_returns_v0_bit_exactly(D):
    c = workloads.make_case(2, G * 2, 2, D, 256, [1, 1], seed=310 + D)
    expect = np.repeat(c["v"][:, :, 0, :], G, axis=1)     # [B, Hq, D] bf16 bits
    assert np.array_equal(bits_of(run_decode(c, chunk=128, out_dtype=torch.bfloat16)), expect)
    out32 = run_decode(c, chunk=128)
    assert np.array_equal(out32.cpu().numpy(), oracle.bf16_bits_to_f64(expect).astype(np.float32))


@pytest.mark.parametrize("D,chunk", [(64, 128), (128, 128), (128, 256)])
def test_nan_poison_past_length_is_never_read(D, chunk):
    lens = [1, 37, 128, 200, 511]
    c = workloads.make_case(len(lens), G * 2, 2, D, 512, lens, seed=320 + D + chunk)
    poisoned = dict(c, k=c["k"].copy(), v=c["v"].copy())
    for b, n in enumerate(lens):
        poisoned["k"][b, :, n:] = BF16_NAN
        poisoned["v"][b, :, n:] = BF16_NAN
    for dt in (torch.float32, torch.bfloat16):
        a = run_decode(c, chunk=chunk, out_dtype=dt)
        p = run_decode(poisoned, chunk=chunk, out_dtype=dt)
        assert torch.equal(a.view(torch.int16), p.view(torch.int16))
        assert not torch.isnan(p.float()).any()


def test_gqa_perturbing_one_kv_head_changes_only_its_group():
    Hkv = 3
    c = workloads.make_case(2, G * Hkv, Hkv, 128, 512, [512, 300], seed=330)
    base = run_decode(c, chunk=128)
    for kp in range(Hkv):
        pert = dict(c, v=c["v"].copy())
        pert["v"][1, kp, :300] ^= np.uint16(0x0040)        # flip a mantissa bit of every value
        changed = (run_decode(pert, chunk=128) != base).any(-1).cpu().numpy()
        expect = np.zeros_like(changed)
        expect[1, kp * G:(kp + 1) * G] = True
        assert np.array_equal(changed, expect)


def test_batch_rows_bit_identical_to_batch_one_calls():
    # no row ends in a tile at most a quarter full, so no tile is folded into
    # the one before it and every row's tiles are the same in both calls
    lens = [700, 5, 1000, 333]
    c = workloads.make_case(4, G * 2, 2, 64, 1024, lens, seed=340)
    full = run_decode(c, chunk=128)
    for b, n in enumerate(lens):
        cb = dict(c, q=c["q"][b:b + 1].copy(), k=c["k"][b:b + 1].copy(), v=c["v"][b:b + 1].copy(),
                  lens=np.array([n], np.int32))
        assert torch.equal(run_decode(cb, chunk=128), full[b:b + 1])


@pytest.mark.parametrize("D", [64, 128])
def test_one_token_causal_chunk_equals_decode(D):
    """chunk_attn with T = 1 at context n - 1 attends the same keys as decode_attn
    at length n, on the same kernel: bit-identical."""
    lens = np.array([1, 300, 999], np.int32)
    c = workloads.make_case(3, G * 2, 2, D, 1000, lens, seed=350 + D)
    dec = run_decode(c, chunk=128)
    cc = dict(c, q=c["q"].reshape(3, 1, G * 2, D), lens=lens - 1)
    ch = run_chunk(cc, chunk=128)
    assert torch.equal(ch[:, 0], dec)


def test_graph_replay_follows_device_lengths():
    B, Hkv, D, S = 4, 2, 128, 2048
    c = workloads.make_case(B, G * Hkv, Hkv, D, S, [S] * B, seed=360)
    q, k, v = dev_bits(c["q"]), dev_bits(c["k"]), dev_bits(c["v"])
    lens = dev_lens([S] * B)
    ws = workspace(B, 1, G * Hkv, Hkv, D, S, 128, poison=True)
    out = torch.zeros((B, G * Hkv, D), device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sda.decode_attn(q, k, v, lens, c["scale"], out, ws, 128)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sda.decode_attn(q, k, v, lens, c["scale"], out, ws, 128)
    rng = np.random.default_rng(361)
    for trial in range(4):
        n = rng.integers(0, S + 1, size=B).astype(np.int32)
        if trial == 3:
            n[:] = 0
        lens.copy_(torch.from_numpy(n))
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        assert_f32_close(got, oracle.decode_attention(c["q"], c["k"], c["v"], n, c["scale"]))
        assert torch.equal(got, run_decode(c, chunk=128, lens=n, tensors=(q, k, v))), f"replay {trial}"


def test_phases_separately_keep_the_fp32_output_precision():
    """attn_partial does not know the output type, so on the matrix cores it
    keeps the softmax weights as bf16 hi + lo: the pair equals decode_attn bit
    for bit with fp32 output and stays within the bf16 tolerance with bf16."""
    c = workloads.make_case(2, G * 2, 2, 128, 1024, [1024, 500], seed=340)
    q, k, v = dev_bits(c["q"]), dev_bits(c["k"]), dev_bits(c["v"])
    lens = dev_lens(c["lens"])
    ref = oracle.decode_attention(c["q"], c["k"], c["v"], c["lens"], c["scale"])
    ws = workspace(2, 1, G * 2, 2, 128, 1024, 128)
    for dt in (torch.float32, torch.bfloat16):
        out = torch.empty((2, G * 2, 128), dtype=dt, device="cuda")
        sda.attn_partial(q, k, v, lens, c["scale"], ws, chunk=128)
        sda.attn_merge(lens, out, ws, T=1, Hq=G * 2, Hkv=2, S_max=1024, chunk=128)
        torch.cuda.synchronize()
        if dt == torch.float32:
            assert torch.equal(out, run_decode(c, chunk=128, tensors=(q, k, v)))
        else:
            assert_bf16_close(out, ref)
