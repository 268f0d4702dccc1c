"""HIP GEMV (bf16 and INT8 weight-only) and the INT8 quantizer vs the fp64
oracle on the same seeded bytes, through the C ABI.

Two checks for each product:
  * small-integer data (weights and activations in {-3..3}, codes in
    {-127..127} with power-of-two scales): every product and partial sum is
    an integer the fp32 accumulator holds exactly, so the GPU must equal the
    oracle bit for bit -- a dropped, repeated or misplaced term cannot hide;
  * N(0,1) data: |y_gpu - y| <= a worst-case fp32 bound derived from the
    kernels' summation (vector units: per lane at most 8 * ceil(K / 8 / 16)
    roundings in its chains of dot2 steps -- at B = 1 four chains, each a
    quarter of that, then two more additions --, the 16/32/64-lane tree, the row
    scale; matrix cores: per wave a chain of at most ceil(K / 256) + 4
    products of 32 terms, each a few roundings, then 8 waves and the row
    scale -- fewer): (8 * ceil(K / 128) + 8) * 2^-24 * sum_k |W x|, and for bf16
    output the result rounded to one of the bf16 values bracketing that
    interval.
The quantizer is compared bit for bit (codes and scales), both sides taking
the integer decisions in fp32.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import stream_decode_attention_amd as sda
import workloads
from oracle.bf16 import bf16_bracket
from tests.gpu_util import bits_of, dev_bits

pytestmark = pytest.mark.gpu


def _f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _small_int_bits(shape, seed, lo=-3, hi=3):
    v = np.random.default_rng(seed).integers(lo, hi + 1, size=shape).astype(np.float32)
    return (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _bound(Wf, xf):
    K = Wf.shape[1]
    steps = 8 * -(-K // 128) + 8
    return steps * 2.0 ** -24 * (np.abs(xf.astype(np.float64)) @ np.abs(Wf.astype(np.float64)).T)


def _check_f32(out, ref, bound):
    got = out.cpu().double().numpy()
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got))
    assert np.all(err <= bound), f"max err {err.max():.3e}, worst ratio {(err / np.maximum(bound, 1e-300)).max():.2f}"


def _check_bf16(out, ref, bound):
    bits = bits_of(out)
    lo, _ = bf16_bracket(ref - bound)
    _, hi = bf16_bracket(ref + bound)
    got = _f32(bits).astype(np.float64)
    assert np.all((got >= _f32(lo)) & (got <= _f32(hi)))


SHAPES = [
    # B, N, K   (vector units, B = 1 below 16384 rows: lanes per row from K/8
    # chunks, >= 256 -> 64, >= 128 -> 32, else 16; matrix cores, B >= 2 and
    # B = 1 from 16384 rows: 16-row tiles, 64-k blocks split over 8 waves)
    (1, 1600, 960),       # SmolLM2-360M fused q/k/v, 16 lanes per row
    (1, 960, 2560),       # SmolLM2 down projection, 64 lanes
    (1, 77, 1024),        # 32 lanes, ragged row count
    (1, 5, 968),          # 121 chunks: a partial round of the 16-lane group
    (1, 1, 64),
    (1, 77, 968),         # the last batch on the vector units
    (2, 77, 968),         # the first on the matrix cores: ragged rows, a partial 64-k block
    (3, 960, 2560),       # 40 blocks: 5 per wave
    (8, 77, 1024),
    (2, 5, 968),          # one partial 16-row tile
    (8, 256, 14336),      # Llama-3-8B down-projection width (224 blocks of 64 k)
    (7, 1, 64),           # one row, one block: seven waves with no work
    (8, 33, 200),         # 4 blocks for 8 waves, the last holding 8 k
    (8, 1600, 960),       # SmolLM2-360M q/k/v at B = 8: 15 blocks over 8 waves
    (1, 16383, 256),      # one row short of the matrix cores at B = 1 (bf16)
    (1, 16390, 200),      # the matrix cores at B = 1: ragged rows, a partial block
    (1, 2047, 2048),      # few long rows (64 lanes each), an odd row count
    (1, 4095, 14336),     # Llama-3-8B down-projection width at B = 1: two rounds of loads per row
]


@pytest.mark.parametrize("B,N,K", SHAPES)
def test_gemv_bf16_integer_data_is_exact(B, N, K):
    W = _small_int_bits((N, K), 700 + K)
    x = _small_int_bits((B, K), 701 + N)
    ref = oracle.gemv(W, x)
    y = torch.empty((B, N), dtype=torch.float32, device="cuda")
    sda.gemv_bf16(dev_bits(W), dev_bits(x), y)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().double().numpy(), ref)


@pytest.mark.parametrize("B,N,K", SHAPES)
def test_gemv_bf16_random_data_within_bound(B, N, K):
    W = workloads.bf16_randn((N, K), 710 + K)
    x = workloads.bf16_randn((B, K), 711 + N)
    ref = oracle.gemv(W, x)
    bound = _bound(_f32(W), _f32(x))
    dW, dx = dev_bits(W), dev_bits(x)
    y32 = torch.empty((B, N), dtype=torch.float32, device="cuda")
    y16 = torch.empty((B, N), dtype=torch.bfloat16, device="cuda")
    sda.gemv_bf16(dW, dx, y32)
    sda.gemv_bf16(dW, dx, y16)
    torch.cuda.synchronize()
    _check_f32(y32, ref, bound)
    _check_bf16(y16, ref, bound)


@pytest.mark.parametrize("N,K", [(1600, 960), (960, 2560), (33, 4096), (4, 16)])
def test_quantize_rows_matches_oracle_bit_for_bit(N, K):
    W = workloads.bf16_randn((N, K), 720 + K)
    W[min(2, N - 1)] = 0                                   # a row of zeros
    if N > 3:
        W[3] = 0
        W[3, K // 2] = 0xBF80                              # a row with a single -1.0
    q_ref, s_ref = oracle.quantize_rows_int8(W)
    dq = torch.empty((N, K), dtype=torch.int8, device="cuda")
    ds = torch.empty((N,), dtype=torch.float32, device="cuda")
    sda.quantize_rows_int8(dev_bits(W), dq, ds)
    torch.cuda.synchronize()
    assert np.array_equal(dq.cpu().numpy(), q_ref)
    assert np.array_equal(ds.cpu().numpy(), s_ref)


def _codes(shape, seed):
    return np.random.default_rng(seed).integers(-127, 128, size=shape).astype(np.int8)


@pytest.mark.parametrize("B,N,K", [(1, 1600, 960), (1, 960, 2560), (1, 77, 1024), (1, 3, 16), (1, 77, 976),
                                   (2, 77, 976), (4, 960, 2560), (8, 77, 1024), (8, 64, 14336), (2, 3, 16),
                                   (3, 77, 976), (5, 3, 16), (8, 33, 208),
                                   (3, 8200, 208), (8, 8193, 16),    # two 16-row tiles per workgroup from N = 8192
                                   (8, 1600, 960),                   # 7.5 blocks of 128 k over 8 waves
                                   (1, 1001, 4096), (1, 4095, 14336)])   # few long rows, odd counts
def test_gemv_int8_integer_data_is_exact(B, N, K):
    q = _codes((N, K), 730 + K)
    s = (2.0 ** np.random.default_rng(731).integers(-8, 1, size=N)).astype(np.float32)
    x = _small_int_bits((B, K), 732 + N)
    ref = oracle.gemv_int8(q, s, x)
    y = torch.empty((B, N), dtype=torch.float32, device="cuda")
    sda.gemv_int8(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(), dev_bits(x), y)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().double().numpy(), ref)


@pytest.mark.parametrize("B,N,K", [(1, 1600, 960), (4, 960, 2560), (8, 256, 14336), (8, 8208, 1024)])
def test_quantize_then_gemv_int8_random_data(B, N, K):
    """The load-time quantizer feeding the INT8 product, as a model would use
    them: codes and scales from the GPU (equal to the oracle's), product
    within the fp32 bound of the oracle's INT8 product."""
    W = workloads.bf16_randn((N, K), 740 + K)
    x = workloads.bf16_randn((B, K), 741 + N)
    dq = torch.empty((N, K), dtype=torch.int8, device="cuda")
    ds = torch.empty((N,), dtype=torch.float32, device="cuda")
    sda.quantize_rows_int8(dev_bits(W), dq, ds)
    y32 = torch.empty((B, N), dtype=torch.float32, device="cuda")
    y16 = torch.empty((B, N), dtype=torch.bfloat16, device="cuda")
    dx = dev_bits(x)
    sda.gemv_int8(dq, ds, dx, y32)
    sda.gemv_int8(dq, ds, dx, y16)
    torch.cuda.synchronize()
    q, s = oracle.quantize_rows_int8(W)
    assert np.array_equal(dq.cpu().numpy(), q) and np.array_equal(ds.cpu().numpy(), s)
    ref = oracle.gemv_int8(q, s, x)
    bound = _bound(q.astype(np.float32) * s[:, None], _f32(x))
    _check_f32(y32, ref, bound)
    _check_bf16(y16, ref, bound)


@pytest.mark.parametrize("B", [1, 2, 8])
def test_gemv_at_the_largest_k(B):
    """K = 73728, the largest K whose staged vector fits the 144 KB LDS budget
    of the dot-product path (B = 1); B = 2 and 8 run on the matrix cores at
    the same K (1152 blocks of 64 k over 8 waves). Integer data: exact."""
    N, K = 37, 73728
    W = _small_int_bits((N, K), 790 + B)
    x = _small_int_bits((B, K), 791 + B)
    y = torch.empty((B, N), dtype=torch.float32, device="cuda")
    sda.gemv_bf16(dev_bits(W), dev_bits(x), y)
    # codes within +-15 keep every partial sum an integer below 2^24
    q = np.random.default_rng(792 + B).integers(-15, 16, size=(N, K)).astype(np.int8)
    s = (2.0 ** np.random.default_rng(793).integers(-8, 1, size=N)).astype(np.float32)
    y8 = torch.empty((B, N), dtype=torch.float32, device="cuda")
    sda.gemv_int8(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(), dev_bits(x), y8)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().double().numpy(), oracle.gemv(W, x))
    assert np.array_equal(y8.cpu().double().numpy(), oracle.gemv_int8(q, s, x))


@pytest.mark.parametrize("N,K", [(6144, 4096), (4096, 4096), (28672, 4096), (4096, 14336)])
def test_gemv_llama3_8b_matrices_sampled_rows(N, K):
    """One Llama-3-8B layer's four products at full size, as the benchmark
    times them (seeded N(0,1) weights drawn on the device, bf16 and INT8,
    B = 1 and 8): the quantizer's codes and scales on 96 sampled rows (tile
    edges, the last rows, random ones) equal the oracle's bit for bit, and
    the products on those rows are within the fp32 bound of the oracle's."""
    g = torch.Generator(device="cuda")
    g.manual_seed(880 + N + K)
    W = torch.randn((N, K), generator=g, device="cuda").to(torch.bfloat16)
    Wq = torch.empty((N, K), dtype=torch.int8, device="cuda")
    sc = torch.empty((N,), dtype=torch.float32, device="cuda")
    sda.quantize_rows_int8(W, Wq, sc)
    edges = [0, 1, 15, 16, 31, 32, 33, N - 33, N - 32, N - 17, N - 16, N - 1]
    rows = sorted(set(edges) | set(np.random.default_rng(N + K).integers(0, N, 96 - len(edges)).tolist()))
    ridx = torch.tensor(rows, dtype=torch.long, device="cuda")
    W_rows = bits_of(W[ridx].contiguous())
    q_ref, s_ref = oracle.quantize_rows_int8(W_rows)           # per row: the sampled rows stand alone
    assert np.array_equal(Wq[ridx].cpu().numpy(), q_ref)
    assert np.array_equal(sc[ridx].cpu().numpy(), s_ref)
    for B in (1, 8):
        x = torch.randn((B, K), generator=g, device="cuda").to(torch.bfloat16)
        x_bits = bits_of(x)
        y32 = torch.empty((B, N), dtype=torch.float32, device="cuda")
        y16 = torch.empty((B, N), dtype=torch.bfloat16, device="cuda")
        y8 = torch.empty((B, N), dtype=torch.float32, device="cuda")
        sda.gemv_bf16(W, x, y32)
        sda.gemv_bf16(W, x, y16)
        sda.gemv_int8(Wq, sc, x, y8)
        torch.cuda.synchronize()
        ref = oracle.gemv(W_rows, x_bits)
        bound = _bound(_f32(W_rows), _f32(x_bits))
        _check_f32(y32[:, ridx], ref, bound)
        _check_bf16(y16[:, ridx].contiguous(), ref, bound)
        ref8 = oracle.gemv_int8(q_ref, s_ref, x_bits)
        _check_f32(y8[:, ridx], ref8, _bound(q_ref.astype(np.float32) * s_ref[:, None], _f32(x_bits)))


def test_gemv_graph_replay_with_new_activations():
    N, K, B = 512, 2048, 4
    W = workloads.bf16_randn((N, K), 750)
    dW = dev_bits(W)
    x = torch.empty((B, K), dtype=torch.int16, device="cuda")
    y = torch.empty((B, N), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        x.copy_(dev_bits(workloads.bf16_randn((B, K), 751)))
        sda.gemv_bf16(dW, x, y, stream=s)
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            sda.gemv_bf16(dW, x, y, stream=s)
    for t in range(3):
        xt = workloads.bf16_randn((B, K), 760 + t)
        with torch.cuda.stream(s):
            x.copy_(dev_bits(xt))
            g.replay()
        s.synchronize()
        _check_f32(y, oracle.gemv(W, xt), _bound(_f32(W), _f32(xt)))
