"""Pins of the CPU oracle against what the pages and the mathematics fix.

Runs on the CPU only.  Each test names what it pins:
  * closed forms printed on the pages (parameter accounting);
  * the library RMSNorm (torch.nn.functional.rms_norm) and hand-computed values;
  * special cases that reduce to a library routine (one expert, k = 1: a dense
    SwiGLU MLP through torch.nn.functional.linear on HF-oriented weights);
  * brute force (every expert evaluated densely, stable argsort selection);
  * invariants and metamorphic relations.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads
from tests.bruteforce import dense_forward
from tests.conftest import read_golden
from workloads import bf16_bits_to_f32, f32_to_bf16_bits


def _rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# ----------------------------------------------------------------------------- shapes
def test_glm5_parameter_accounting_matches_page():
    """Page "GLM-5 · MoE transformer block", Parameters table: the MoE sublayer of
    one block holds 9,702,998,272 parameters including one correction-bias value per
    expert; with the MLA and the two RMSNorms the block holds 9,877,404,672."""
    g = read_golden("glm5_moe_block_params.txt")
    cfg = workloads.config("glm5_decode")
    assert cfg.d == g["hidden_size"]
    assert workloads.param_count(cfg) == g["moe_params"]
    # router biases: 256 per block x 75 blocks
    assert cfg.E * g["moe_blocks"] == g["correction_bias_values_all_blocks"]
    block = g["attention_rmsnorm_params"] + g["mla_params"] + g["moe_rmsnorm_params"] + g["moe_params"]
    assert block == g["block_params"]
    assert block * g["moe_blocks"] == g["model_moe_block_params"]
    assert g["moe_rmsnorm_params"] == cfg.d
    # bf16 bytes of the MoE weights: 18.1 GiB; two RMSNorms: 24 KiB
    moe_bytes = 2 * g["moe_params"]
    assert round(moe_bytes / 2**30, 1) == g["moe_weight_gib_bf16"]
    assert round(2 * block / 2**30, 1) == g["block_weight_gib_bf16"]
    assert 2 * (g["attention_rmsnorm_params"] + g["moe_rmsnorm_params"]) / 1024 == g["two_rmsnorms_kib_bf16"]
    assert round(100 * g["moe_params"] / block, 1) == g["moe_share_percent"]
    # the only (E, I) with I a multiple of 64 and E*I + Is = 257*2048, Is = I, E = 256
    solved = (g["moe_params"] - cfg.E - cfg.E * cfg.d) // (3 * cfg.d)
    assert solved == cfg.E * cfg.I + cfg.Is == 257 * 2048


def test_glm5_mid_and_tiny_shapes_are_consistent():
    for name, cfg in workloads.CONFIGS.items():
        assert cfg.d % 64 == 0 and cfg.I % 64 == 0, name
        assert 1 <= cfg.k <= cfg.E
    assert workloads.config("mid_prefill").I == 11 * 128


# ----------------------------------------------------------------------------- RMSNorm
def test_rmsnorm_hand_computed():
    """x = (3, 4): mean of squares 12.5; h = x / sqrt(12.5 + 1e-6)."""
    x = np.array([[3.0, 4.0]], np.float32)
    w = np.ones(2, np.float32)
    h = oracle.rmsnorm(x, w, oracle.F32, 1e-6)
    ref = np.array([3.0, 4.0]) / math.sqrt(12.5 + 1e-6)
    np.testing.assert_allclose(h[0], ref, rtol=2e-7)


def test_rmsnorm_constant_row_and_zero_row():
    x = np.array([[0.5] * 64, [0.0] * 64], np.float32)
    h = oracle.rmsnorm(x, np.ones(64, np.float32), oracle.F32, 1e-6)
    np.testing.assert_allclose(h[0], 0.5 / math.sqrt(0.25 + 1e-6), rtol=2e-7)
    assert np.all(h[1] == 0.0)


def test_rmsnorm_matches_torch_library_fp32():
    """torch.nn.functional.rms_norm is an independent implementation of the same map."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((33, 384)).astype(np.float32) * 3
    w = (1 + 0.1 * rng.standard_normal(384)).astype(np.float32)
    h = oracle.rmsnorm(x, w, oracle.F32, 1e-6)
    ref = F.rms_norm(torch.from_numpy(x).double(), (384,), torch.from_numpy(w).double(), 1e-6)
    np.testing.assert_allclose(h, ref.numpy(), rtol=5e-7, atol=1e-7)


def test_rmsnorm_bf16_two_roundings():
    """bf16: the normalised value is cast back to bf16 before the gain multiply, then
    the product is rounded to bf16 again (page "GLM-5 · Input features", RMSNorm)."""
    rng = np.random.default_rng(2)
    x32 = rng.standard_normal((16, 256)).astype(np.float32)
    w32 = (1 + 0.1 * rng.standard_normal(256)).astype(np.float32)
    xb, wb = f32_to_bf16_bits(x32), f32_to_bf16_bits(w32)
    h = oracle.rmsnorm(xb, wb, oracle.BF16, 1e-6)
    # h holds bf16 values
    assert np.array_equal(bf16_bits_to_f32(f32_to_bf16_bits(h)), h)
    # against a float64 library norm of the same bf16 inputs: two roundings to bf16
    # (8 significant bits) each add at most 2^-8 relative error
    xv, wv = bf16_bits_to_f32(xb).astype(np.float64), bf16_bits_to_f32(wb).astype(np.float64)
    ref = F.rms_norm(torch.from_numpy(xv), (256,), torch.from_numpy(wv), 1e-6).numpy()
    assert np.max(np.abs(h - ref) / np.maximum(np.abs(ref), 1e-3)) <= (1 + 2.0**-8) ** 2 - 1 + 1e-6


def test_rmsnorm_scale_invariance_and_unit_gain_energy():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, 512)).astype(np.float32)
    one = np.ones(512, np.float32)
    h1 = oracle.rmsnorm(x, one, oracle.F32, 1e-6)
    h4 = oracle.rmsnorm(4 * x, one, oracle.F32, 1e-6)
    # invariant up to the epsilon term (relative eps / (2 ms) ~ 5e-7) and a few fp32 roundings
    np.testing.assert_allclose(h1, h4, rtol=1e-6, atol=1e-7)
    ms = np.mean(x.astype(np.float64) ** 2, axis=1)
    np.testing.assert_allclose(np.mean(h1.astype(np.float64) ** 2, axis=1), ms / (ms + 1e-6), rtol=1e-6)


# ----------------------------------------------------------------------------- router
def test_zero_gain_routes_by_bias_and_leaves_x_unchanged():
    """norm_w = 0 => h = 0 => every score is sigmoid(0) = 1/2: the selection is the
    top-k of the correction bias (ties to the lower index), every weight is rs/k, and
    every expert output is silu(0)*0 = 0, so out == x exactly."""
    inp = workloads.make_host("tiny_fp32", seed=5)
    inp["norm_w"] = np.zeros_like(inp["norm_w"])
    inp["corr_bias"] = np.array([0.3, -0.1, 0.5, 0.5, 0.0, -0.2, 0.3, 0.1], np.float32)
    r = oracle.forward(inp)
    assert np.all(r["scores"] == 0.5)
    assert np.all(r["idx"] == np.array([2, 3]))  # 0.5 twice: expert 2 before 3
    np.testing.assert_allclose(r["w"], inp["routed_scale"] / inp["top_k"], rtol=1e-15)
    assert np.array_equal(r["out"], inp["x"])
    assert np.all(r["delta"] == 0.0)


def test_tie_break_prefers_lower_index():
    scores = np.full((1, 6), 0.25, np.float32)
    bias = np.array([0.0, 0.1, 0.1, 0.0, 0.1, 0.0], np.float32)
    idx, w, margin = oracle.select(scores, bias, 3, 1.0)
    assert idx.tolist() == [[1, 2, 4]]
    idx, w, margin = oracle.select(scores, bias, 2, 1.0)
    assert idx.tolist() == [[1, 2]] and margin[0] == 0.0


def test_selection_uses_biased_key_but_unbiased_weights():
    scores = np.array([[0.9, 0.8, 0.2, 0.1]], np.float32)
    bias = np.array([0.0, 0.0, 0.75, 0.0], np.float32)
    idx, w, margin = oracle.select(scores, bias, 2, 2.5)
    assert idx.tolist() == [[2, 0]]  # keys 0.95 > 0.9 > 0.8
    np.testing.assert_allclose(w[0], 2.5 * np.array([0.2, 0.9]) / np.float64(np.float32(0.2) + np.float32(0.9)),
                               rtol=1e-7)
    np.testing.assert_allclose(margin[0], np.float32(0.9) - np.float64(np.float32(0.8)), rtol=1e-6)


def test_sigmoid_scores_closed_form():
    h = np.array([[1.0, 0.0], [0.0, -2.0]], np.float32)
    rw = np.array([[1.0, 0.0], [0.0, 1.0], [3.0, 0.0]], np.float32)
    logits, scores = oracle.router_scores(h, rw, oracle.F32)
    np.testing.assert_array_equal(logits, [[1, 0, 3], [0, -2, 0]])
    np.testing.assert_allclose(scores, 1 / (1 + np.exp(-logits.astype(np.float64))), rtol=1e-7)


def test_weights_sum_to_routed_scale_and_indices_distinct():
    inp = workloads.make_host("tiny_fp32", seed=0)
    r = oracle.forward(inp)
    np.testing.assert_allclose(r["w"].sum(1), inp["routed_scale"], rtol=1e-14)
    assert all(len(set(row)) == inp["top_k"] for row in r["idx"].tolist())
    cnt, off = r["counts"], r["offsets"]
    assert cnt.sum() == r["idx"].size
    assert np.array_equal(cnt, np.bincount(r["idx"].ravel(), minlength=len(cnt)))
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(cnt)]))


# ----------------------------------------------------------------------------- SwiGLU
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_expert_reduces_to_dense_swiglu_mlp(dtype):
    """E = 1, k = 1, rs = 1: out = x + S(h) + M(h), with M and S the dense SwiGLU MLP
    down(silu(gate h) * up h) evaluated by torch.nn.functional.linear on nn.Linear-shaped
    weights.  The grouped expert is converted to HF orientation per the adapter's
    layout: gate_proj.weight = gate_and_up[0][:, :I]^T, up_proj.weight =
    gate_and_up[0][:, I:]^T, down_proj.weight = down[0]^T."""
    cfg = workloads.config("tiny_fp32", E=1, k=1, T=17, dtype=dtype)
    inp = workloads.make_host(cfg, seed=11)
    r = oracle.forward(inp)
    assert np.all(r["idx"] == 0)
    np.testing.assert_allclose(r["w"], 1.0, rtol=1e-15)

    def val(a):
        return torch.from_numpy(bf16_bits_to_f32(a) if dtype == "bf16" else a).double()

    h = torch.from_numpy(r["h"]).double()
    I = cfg.I
    gu, dn = val(inp["gate_up"][0]), val(inp["down"][0])
    gate_w, up_w, down_w = gu[:, :I].T, gu[:, I:].T, dn.T      # HF [out, in]
    M = F.linear(F.silu(F.linear(h, gate_w)) * F.linear(h, up_w), down_w)
    S = F.linear(F.silu(F.linear(h, val(inp["shared_gate"]))) * F.linear(h, val(inp["shared_up"])),
                 val(inp["shared_down"]))
    np.testing.assert_allclose(r["delta"], (M + S).numpy(), rtol=1e-10, atol=1e-12)


def test_soft_moe_k_equals_E():
    """k = E: every expert contributes, weighted by its renormalised score."""
    cfg = workloads.config("tiny_fp32", k=8, T=9)
    inp = workloads.make_host(cfg, seed=4)
    r = oracle.forward(inp, debug=True)
    assert np.all(np.isinf(r["margin"]))
    s = r["scores"].astype(np.float64)
    np.testing.assert_allclose(np.sort(r["w"], 1),
                               np.sort(cfg.routed_scale * s / s.sum(1, keepdims=True), 1), rtol=1e-12)


# ----------------------------------------------------------------------------- brute force
@pytest.mark.parametrize("name,overrides,seed", [
    ("tiny_fp32", {}, 0),
    ("tiny_fp32", dict(dtype="bf16"), 0),
    ("tiny_fp32", dict(E=16, k=1, T=40, d=128, I=64, Is=64), 3),
    ("tiny_fp32", dict(E=5, k=5, T=12, d=64, I=64, Is=0), 7),
    ("tiny_fp32", dict(E=12, k=3, T=30, d=192, I=64, Is=128, dtype="bf16", routed_scale=2.5), 9),
])
def test_oracle_matches_dense_bruteforce(name, overrides, seed):
    cfg = workloads.config(name, **overrides)
    inp = workloads.make_host(cfg, seed=seed)
    if cfg.Is == 0:
        inp["shared_gate"] = inp["shared_up"] = inp["shared_down"] = None
    r = oracle.forward(inp, debug=True)
    b = dense_forward(inp)
    # h is bit-identical except where the fp64 sum of squares rounds differently (never here)
    np.testing.assert_array_equal(r["h"], b["h"].astype(np.float32))
    np.testing.assert_allclose(r["logits"], b["logits"], rtol=1e-6, atol=1e-7)
    assert np.array_equal(np.sort(r["idx"], 1), np.sort(b["idx"], 1))
    assert np.array_equal(r["idx"], b["idx"])  # same order: key desc, index asc
    np.testing.assert_allclose(r["w"], b["w"], rtol=1e-6)
    np.testing.assert_allclose(r["delta"], b["delta"], rtol=1e-6, atol=1e-9)
    # per-assignment expert outputs against the dense evaluation
    Yd = np.take_along_axis(b["Y"], b["idx"][:, :, None], axis=1)
    np.testing.assert_allclose(r["debug"]["y"], Yd, rtol=1e-9, atol=1e-12)
    Ad = np.take_along_axis(b["act"], b["idx"][:, :, None], axis=1)
    np.testing.assert_allclose(r["debug"]["act"], Ad, rtol=1e-9, atol=1e-12)
    if cfg.Is > 0:
        # the shared expert's activation and output (debug outputs the GPU tests use)
        np.testing.assert_allclose(r["debug"]["act_s"], b["act_s"], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(r["debug"]["s"], b["shared"], rtol=1e-9, atol=1e-12)
    assert np.array_equal(r["out"], b["out"])


# ----------------------------------------------------------------------------- metamorphic
def test_down_weight_scaling_is_linear():
    inp = workloads.make_host("tiny_fp32", seed=1)
    r1 = oracle.forward(inp)
    inp2 = dict(inp, down=inp["down"] * 2, shared_down=inp["shared_down"] * 2)
    r2 = oracle.forward(inp2)
    assert np.array_equal(r2["idx"], r1["idx"])
    np.testing.assert_array_equal(r2["delta"], 2 * r1["delta"])


def test_token_permutation_equivariance_and_batch_invariance():
    inp = workloads.make_host("tiny_fp32", seed=2)
    r = oracle.forward(inp)
    perm = np.random.default_rng(0).permutation(inp["x"].shape[0])
    rp = oracle.forward(dict(inp, x=inp["x"][perm]))
    np.testing.assert_array_equal(rp["out"], r["out"][perm])
    np.testing.assert_array_equal(rp["idx"], r["idx"][perm])
    one = oracle.forward(dict(inp, x=inp["x"][13:14]))
    np.testing.assert_array_equal(one["out"][0], r["out"][13])


def test_expert_relabelling_invariance():
    inp = workloads.make_host("tiny_fp32", seed=3)
    r = oracle.forward(inp)
    p = np.random.default_rng(1).permutation(8)  # new expert q holds old expert p[q]
    inp2 = dict(inp, gate_up=inp["gate_up"][p], down=inp["down"][p], router_w=inp["router_w"][p],
                corr_bias=inp["corr_bias"][p])
    r2 = oracle.forward(inp2)
    np.testing.assert_array_equal(p[r2["idx"]], r["idx"])
    np.testing.assert_array_equal(r2["out"], r["out"])


def test_subset_of_tokens_equals_full_batch_rows():
    inp = workloads.make_host("tiny_fp32", seed=6)
    r = oracle.forward(inp)
    sub = np.array([5, 0, 63, 17])
    rs = oracle.forward(inp, tokens=sub)
    np.testing.assert_array_equal(rs["out"], r["out"][sub])
    np.testing.assert_array_equal(rs["delta"], r["delta"][sub])


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.select(np.zeros((2, 4), np.float32), np.zeros(4, np.float32), 5, 1.0)
    with pytest.raises(ValueError):
        oracle.select(np.zeros((2, 4), np.float32), np.zeros(4, np.float32), 0, 1.0)
    with pytest.raises(TypeError):
        oracle.rmsnorm(np.zeros((2, 4), np.float32), np.zeros(4, np.float32), oracle.BF16)


# ----------------------------------------------------------------------------- dense block
def _dense_inputs(T, d, Id, dtype, seed):
    x, norm_w = workloads.draw_norm(T, d, d, dtype, seed=seed)
    w = workloads.draw_dense(d, Id, dtype, seed=seed)
    return x, norm_w, w


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dense_block_matches_torch_library(dtype):
    """The page's GlmMoeDsaMLP.forward is down_proj(act_fn(gate_proj(x)) * up_proj(x)) with
    bias-free nn.Linear maps: evaluated here by torch.nn.functional in fp64 on the oracle's
    (separately pinned) RMSNorm output, the dense-MLP oracle must agree to rounding."""
    T, d, Id = 13, 256, 192
    x, norm_w, w = _dense_inputs(T, d, Id, dtype, seed=5)
    dt = oracle.DTYPES[dtype]
    r = oracle.dense_block(x, norm_w, w["gate"], w["up"], w["down"], dt, debug=True)

    def val(a):
        return torch.from_numpy(bf16_bits_to_f32(a) if dtype == "bf16" else a).double()

    h = torch.from_numpy(r["h"]).double()
    act = F.silu(F.linear(h, val(w["gate"]))) * F.linear(h, val(w["up"]))
    ref = F.linear(act, val(w["down"]))
    np.testing.assert_allclose(r["act"], act.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["delta"], ref.numpy(), rtol=1e-10, atol=1e-12)
    # out = x + delta rounded once (to fp32, then to D)
    exact = (val(x) + ref).numpy()
    tol = 2.0 ** -7 if dtype == "bf16" else 2.0 ** -22
    np.testing.assert_allclose(r["out"], exact, rtol=tol, atol=tol * 1e-3)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dense_block_equals_single_expert_moe_block(dtype):
    """A dense block is the MoE block with one routed expert taken with weight 1 and no
    shared expert: E = 1, k = 1, routed_scale = 1, gate_and_up[0] = [gate^T | up^T],
    down[0] = down^T (the adapter's grouped orientation).  The two oracle paths must give
    the same delta and out."""
    T, d, Id = 9, 128, 64
    x, norm_w, w = _dense_inputs(T, d, Id, dtype, seed=8)
    dt = oracle.DTYPES[dtype]
    r = oracle.dense_block(x, norm_w, w["gate"], w["up"], w["down"], dt)
    gate_up = np.ascontiguousarray(np.concatenate([w["gate"].T, w["up"].T], axis=1))[None]
    down = np.ascontiguousarray(w["down"].T)[None]
    router_w = np.zeros((1, d), x.dtype)
    inp = dict(x=x, norm_w=norm_w, router_w=router_w, corr_bias=np.zeros(1, np.float32),
               gate_up=[gate_up[0]], down=[down[0]], shared_gate=None, shared_up=None,
               shared_down=None, dtype=dtype, top_k=1, routed_scale=1.0, eps=1e-6)
    m = oracle.forward(inp)
    np.testing.assert_allclose(m["delta"], r["delta"], rtol=1e-13, atol=1e-15)
    assert np.array_equal(m["out"], r["out"])


def test_dense_block_zero_down_is_identity_and_linear_in_down():
    T, d, Id = 7, 64, 64
    x, norm_w, w = _dense_inputs(T, d, Id, "f32", seed=2)
    r0 = oracle.dense_block(x, norm_w, w["gate"], w["up"], np.zeros_like(w["down"]), 0)
    assert np.array_equal(r0["out"], x) and np.all(r0["delta"] == 0)
    r1 = oracle.dense_block(x, norm_w, w["gate"], w["up"], w["down"], 0)
    r3 = oracle.dense_block(x, norm_w, w["gate"], w["up"], 4 * w["down"], 0)  # exact scaling
    np.testing.assert_allclose(r3["delta"], 4 * r1["delta"], rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------- layout packing
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_packed_hf_weights_give_the_hf_mlp(dtype):
    """HF per-expert weights packed into the grouped layout, run through the MoE oracle
    (E = 1, k = 1, rs = 1, no shared expert), equal the page's SwiGLU MLP evaluated by
    torch.nn.functional.linear directly on the HF [out, in] weights: this pins the packing
    orientation (gate columns first, transposes) independently of the oracle's own code."""
    T, d, I = 11, 128, 64
    x, norm_w = workloads.draw_block_input(T, d, dtype, seed=4)
    w = workloads.draw_dense(d, I, dtype, seed=4)      # stands in for one HF expert
    gate_up, down = oracle.pack_expert(w["gate"], w["up"], w["down"])
    assert gate_up.shape == (d, 2 * I) and down.shape == (I, d)
    inp = dict(x=x, norm_w=norm_w, router_w=np.zeros((1, d), x.dtype),
               corr_bias=np.zeros(1, np.float32), gate_up=[gate_up], down=[down],
               shared_gate=None, shared_up=None, shared_down=None, dtype=dtype, top_k=1,
               routed_scale=1.0, eps=1e-6)
    r = oracle.forward(inp)

    def val(a):
        return torch.from_numpy(bf16_bits_to_f32(a) if dtype == "bf16" else a).double()

    h = torch.from_numpy(r["h"]).double()
    ref = F.linear(F.silu(F.linear(h, val(w["gate"]))) * F.linear(h, val(w["up"])), val(w["down"]))
    np.testing.assert_allclose(r["delta"], ref.numpy(), rtol=1e-10, atol=1e-12)


def test_pack_unpack_round_trip_and_element_map():
    d, I = 24, 8
    gate = np.arange(I * d, dtype=np.float32).reshape(I, d)
    up = 1000 + np.arange(I * d, dtype=np.float32).reshape(I, d)
    down = 5000 + np.arange(d * I, dtype=np.float32).reshape(d, I)
    gu, dn = oracle.pack_expert(gate, up, down)
    # element map written out by hand: gu[i][n] = gate[n][i], gu[i][I+n] = up[n][i], dn[n][m] = down[m][n]
    for i in (0, 5, d - 1):
        for n in (0, 3, I - 1):
            assert gu[i, n] == gate[n, i] and gu[i, I + n] == up[n, i]
    for n in (0, I - 1):
        for m in (0, 7, d - 1):
            assert dn[n, m] == down[m, n]
    g2, u2, d2 = oracle.unpack_expert(gu, dn)
    assert np.array_equal(g2, gate) and np.array_equal(u2, up) and np.array_equal(d2, down)
