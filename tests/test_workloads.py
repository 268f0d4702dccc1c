"""The seeded input generators: determinism and the shapes/structure of the five workloads."""
import numpy as np

import workloads
from oracle import bf16_bits_to_f64


def test_generator_is_deterministic():
    a = workloads.bf16_randn((3, 5, 7), seed=99)
    b = workloads.bf16_randn((3, 5, 7), seed=99)
    c = workloads.bf16_randn((3, 5, 7), seed=100)
    assert a.dtype == np.uint16 and np.array_equal(a, b) and not np.array_equal(a, c)


def test_values_look_standard_normal():
    x = bf16_bits_to_f64(workloads.bf16_randn((200000,), seed=5))
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01


def test_config_shapes_small():
    c1 = workloads.make_config(1)
    w = c1["workload"]
    assert c1["q"].shape == (1, 15, 64)
    assert c1["k"].shape == (1, 5, 128, 64) and c1["v"].shape == (1, 5, 128, 64)
    assert list(c1["lens"]) == [64] and w.chunk == 32 and c1["scale"] == 0.125
    c5 = workloads.CONFIGS[5]
    assert (c5.T, c5.Hq, c5.Hkv, c5.D, c5.S_max, c5.G) == (6, 24, 8, 128, 16384, 3)


def test_outlier_keys_are_scaled_by_eight():
    c = workloads.make_case(1, 8, 4, 64, 4000, [4000], seed=3)
    o = workloads.make_case(1, 8, 4, 64, 4000, [4000], seed=3, outlier_frac=0.05)
    a, b = bf16_bits_to_f64(c["k"]), bf16_bits_to_f64(o["k"])
    ratio_rows = np.all((b == a) | (b == 8 * a), axis=-1)
    assert ratio_rows.all()
    scaled = np.any(b != a, axis=-1).mean()
    assert 0.04 < scaled < 0.06


def test_ragged_lengths_in_range():
    lens = workloads.ragged_lens(4, 8, 32768)
    assert lens.dtype == np.int32 and lens.shape == (8,)
    assert lens.min() >= 1 and lens.max() <= 32768
    assert np.array_equal(lens, workloads.ragged_lens(4, 8, 32768))


def test_spec_sampling_case_shapes_and_ranges():
    c = workloads.spec_sampling_case(3, 5, 1000, seed=1)
    assert c["logits"].shape == (3, 5, 1000) and c["logits"].dtype == np.float32
    assert c["q"].shape == (3, 4, 1000) and c["q"].dtype == np.float32
    assert np.allclose(c["q"].astype(np.float64).sum(-1), 1.0, atol=1e-5) and np.all(c["q"] >= 0)
    assert c["drafts"].shape == (3, 4) and np.all((c["drafts"] >= 0) & (c["drafts"] < 1000))
    assert np.all((c["u"] >= 0) & (c["u"] < 1)) and np.all((c["r"] >= 0) & (c["r"] < 1))
    assert c["tau"] == float(np.float32(c["tau"]))
    d = workloads.spec_sampling_case(3, 5, 1000, seed=1)
    assert all(np.array_equal(c[k], d[k]) for k in ("logits", "q", "drafts", "u", "r", "ctx"))


def test_spec_greedy_case_plants_the_top_tokens():
    c = workloads.spec_greedy_case(6, 5, 300, seed=2)
    for b in range(6):
        for i in range(5):
            row = c["logits"][b, i]
            assert int(np.flatnonzero(row == row.max())[0]) == c["top"][b, i]
        m = c["m"][b]
        assert list(c["drafts"][b, :m]) == list(c["top"][b, :m])
        if m < 4:
            assert c["drafts"][b, m] != c["top"][b, m]
