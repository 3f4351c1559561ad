"""Seeded generators: determinism, distributions, margin filter, Zipf calibration."""
import json
import os

import numpy as np

import workloads
from tests.margin import MIN_MARGIN, filtered_small

HERE = os.path.dirname(os.path.abspath(__file__))


def test_draws_are_deterministic_and_seed_dependent():
    a = workloads.make_host("tiny_fp32", seed=0)
    b = workloads.make_host("tiny_fp32", seed=0)
    c = workloads.make_host("tiny_fp32", seed=1)
    for key in ("x", "norm_w", "router_w", "corr_bias", "gate_up", "down", "shared_gate"):
        assert np.array_equal(a[key], b[key]), key
        assert not np.array_equal(a[key], c[key]), key


def test_distributions_and_shapes():
    cfg = workloads.config("tiny_fp32")
    a = workloads.make_host(cfg, seed=0)
    assert a["gate_up"].shape == (8, 256, 256) and a["down"].shape == (8, 128, 256)
    assert a["shared_gate"].shape == (128, 256) and a["shared_down"].shape == (256, 128)
    assert abs(a["gate_up"].std() - 0.02) < 1e-3
    assert abs(a["router_w"].std() - 0.02) < 2e-3
    assert abs(a["norm_w"].mean() - 1.0) < 0.03 and abs(a["norm_w"].std() - 0.1) < 0.02
    assert np.all(np.abs(a["corr_bias"]) <= 0.01)
    assert abs(a["x"].std() - 1.0) < 0.02


def test_bf16_storage_is_round_to_nearest_even():
    v = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.14159265], np.float32)
    bits = workloads.f32_to_bf16_bits(v)
    back = workloads.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins
    assert back.tolist()[:4] == [1.0, 1.0, 1.015625, -2.5]
    assert abs(back[4] - 3.140625) == 0


def test_margin_filter_tiny_and_glm5_decode():
    for name in ("tiny_fp32", "glm5_decode"):
        small, r, n = filtered_small(name, seed=0)
        assert np.all(r["margin"] >= MIN_MARGIN), name
        again, r2, _ = filtered_small(name, seed=0)
        assert np.array_equal(again["x"], small["x"])


def test_zipf_beta_matches_calibration_record():
    rec = json.load(open(os.path.join(HERE, "golden", "zipf_beta.json")))
    assert workloads.ZIPF_BETA == rec["beta"]
    assert abs(rec["slope"] + 1.1) < 0.05
    # "thousands of tokens" on the hottest expert; some experts with fewer than 10 or none
    assert rec["max_load"] >= 2000
    assert rec["experts_below_10"] >= 10
    assert sum(rec["sorted_loads"]) == 16384 * 8
