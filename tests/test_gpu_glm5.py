"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (one plan per workload, max_tokens = T, MOE_PATH_AUTO unless
stated).  Routing (selected sets, per-expert counts) is checked on every token;
outputs (out, delta) and the intermediates act and y of every (token, expert)
pair on every token for the decode batch, and on a seeded, stratified sample of
512 tokens (computed one by one by the oracle) for the prefill batches: every
256-row M-tile of the hottest expert, the last M-tile of the 8 busiest, the
rarest non-empty experts, the first and last token, the rest uniform.  For the
4096-token prefill, out and delta are checked on every token as well.  Plans sized
for more tokens than a call passes are checked too, with a guard region after
the workspace that must stay untouched."""
import numpy as np
import pytest
import torch

import mixture_experts_transformer_rmsnorm_amd as moe
import oracle
import workloads
from tests.gpu_harness import (assert_guard, check_intermediate, check_outputs, check_permutation,
                               check_routing, guard_workspace, make_block, read_all, run_gpu, say,
                               values)
from tests.margin import filtered_small

pytestmark = pytest.mark.gpu

N_SAMPLE = 512
M_TILE = 256  # rows per M-tile of the grouped kernels


class Weights:
    """Device weights of one shape family, drawn once, with a host cache of experts."""

    def __init__(self, cfg):
        say("drawing device weights for %s" % cfg.name)
        self.tin = workloads.make_torch(cfg, 0, device="cuda", weights="device")
        torch.cuda.synchronize()
        self.host = {}
        self.shared = None

    def host_experts(self, cfg, experts):
        for e in experts:
            if e not in self.host:
                self.host[e] = (workloads.torch_to_host(self.tin["gate_up"][e]),
                                workloads.torch_to_host(self.tin["down"][e]))
        if self.shared is None:
            self.shared = [workloads.torch_to_host(self.tin[n])
                           for n in ("shared_gate", "shared_up", "shared_down")]
        gu = [self.host[e][0] if e in self.host else None for e in range(cfg.E)]
        dn = [self.host[e][1] if e in self.host else None for e in range(cfg.E)]
        return gu, dn, self.shared


@pytest.fixture(scope="module")
def glm5_weights():
    w = Weights(workloads.config("glm5_decode"))
    yield w
    del w.tin
    torch.cuda.empty_cache()


def _inputs(cfg, weights):
    small, route, n_red = filtered_small(cfg, 0)
    say("%s: %d rows redrawn for the routing margin" % (cfg.name, n_red))
    tin = dict(weights.tin)
    for key in ("x", "norm_w", "router_w"):
        tin[key] = workloads.host_to_torch(small[key], cfg.dtype, "cuda")
    tin["corr_bias"] = torch.from_numpy(small["corr_bias"]).cuda()
    return small, route, tin


def _sample_tokens(cfg, route, n, seed=0):
    """Stratified token sample.  An expert's segment holds its tokens in token order,
    so its i-th token sits in M-tile i // 256."""
    rng = np.random.default_rng(seed)
    cnt = np.bincount(route["idx"].ravel(), minlength=cfg.E)
    order = np.argsort(-cnt, kind="stable")
    picks = {0, cfg.T - 1}

    def tokens_of(e):
        return np.nonzero(np.any(route["idx"] == e, 1))[0]

    hot = tokens_of(order[0])
    for m0 in range(0, len(hot), M_TILE):  # every M-tile of the hottest expert
        picks.add(int(rng.choice(hot[m0:m0 + M_TILE])))
    for e in order[:8]:  # the last M-tile (and last row) of the 8 busiest experts
        toks = tokens_of(e)
        picks.add(int(rng.choice(toks[(len(toks) - 1) // M_TILE * M_TILE:])))
        picks.add(int(toks[-1]))
    for e in [e for e in np.argsort(cnt, kind="stable") if cnt[e] > 0][:8]:  # rarest
        picks.add(int(tokens_of(e)[0]))
    for t in rng.permutation(cfg.T):
        if len(picks) >= n:
            break
        picks.add(int(t))
    return np.array(sorted(picks), np.int64)


def _check_intermediates(cfg, g, tokens, dbg):
    """act and y of every (token, expert) pair of the listed tokens, read through row_of."""
    rows = g["row_of"][tokens].ravel()
    check_intermediate(values(g["act"][rows], cfg.dtype), dbg["act"].reshape(-1, cfg.I),
                       cfg.dtype, "act")
    check_intermediate(values(g["y"][rows], cfg.dtype), dbg["y"].reshape(-1, cfg.d), cfg.dtype,
                       "y")


def _check(cfg, weights, path=moe.MOE_PATH_AUTO, n_sample=None, all_outputs=False):
    small, route, tin = _inputs(cfg, weights)
    say("%s: forward on the GPU (path %d)" % (cfg.name, path))
    block, out = run_gpu(cfg, tin, path)
    g = read_all(block, cfg, cfg.T)
    if cfg.dtype == "bf16":
        mism = int(np.sum(g["h"] != workloads.f32_to_bf16_bits(route["h"])))
        say("  h mismatches vs oracle: %d of %d" % (mism, g["h"].size))
        assert mism == 0
    check_routing(g, route, cfg)
    say("  routing exact on all %d tokens; active experts %d; max load %d" % (
        cfg.T, int(np.sum(g["counts"] > 0)), int(g["counts"].max())))
    check_permutation(g, cfg, cfg.T)
    tokens = np.arange(cfg.T) if n_sample is None else _sample_tokens(cfg, route, n_sample)
    experts = np.unique(route["idx"][tokens])
    say("  oracle on %d tokens (%d experts)" % (len(tokens), len(experts)))
    gu, dn, sh = weights.host_experts(cfg, experts)
    delta, out_ref, dbg = oracle.experts(tokens, small["x"], route["h"], route["idx"], route["w"],
                                         gu, dn, sh[0], sh[1], sh[2], oracle.DTYPES[cfg.dtype],
                                         debug=True)
    _check_intermediates(cfg, g, tokens, dbg)
    host_out = workloads.torch_to_host(out)
    check_outputs(cfg, small, host_out[tokens], delta, out_ref, tokens)
    if all_outputs and n_sample is not None:
        # out and delta of every token (no intermediates: they would not fit in memory)
        every = np.arange(cfg.T)
        gu, dn, sh = weights.host_experts(cfg, np.unique(route["idx"]))
        say("  oracle on all %d tokens (outputs only)" % cfg.T)
        delta, out_ref = oracle.experts(every, small["x"], route["h"], route["idx"], route["w"], gu,
                                        dn, sh[0], sh[1], sh[2], oracle.DTYPES[cfg.dtype])
        check_outputs(cfg, small, host_out, delta, out_ref, every)
    if moe.moe_plan_path(block.plan, cfg.T, cfg.k) == moe.MOE_PATH_FUSED:
        assert block.fused_error(cfg.T) == 0
    del block
    return g


def test_glm5_decode_stream(glm5_weights):
    cfg = workloads.config("glm5_decode")
    _check(cfg, glm5_weights, path=moe.MOE_PATH_STREAM)


@pytest.mark.parametrize("T", [1, 2, 8, 32])
def test_glm5_decode_small_batches(glm5_weights, T):
    """1 to 32 tokens: at most as many (expert, pass) items as resident blocks, so the
    streaming kernels split each item's columns over J blocks (J = 32, 16, 4 and 1
    here) and sum each block's row groups in LDS; no partial sums, no fixup."""
    cfg = workloads.config("glm5_decode", T=T)
    _check(cfg, glm5_weights, path=moe.MOE_PATH_AUTO)


def test_glm5_stream_split_items(glm5_weights):
    """256 tokens on the streaming path: more (expert, pass) items than resident
    blocks, so the balanced launch splits items between blocks and the fixup
    kernel finishes them."""
    cfg = workloads.config("glm5_decode", T=256)
    _check(cfg, glm5_weights, path=moe.MOE_PATH_STREAM)


def _fewer_tokens_than_planned(cfg, weights, path, max_tokens, calls):
    """One plan for max_tokens, called with each T in `calls` (smaller): every token's
    output against the oracle, and nothing written past the workspace."""
    small, route, tin = _inputs(cfg, weights)
    block = make_block(cfg, tin, path, max_tokens=max_tokens)
    guard = guard_workspace(block)
    for T in calls:
        say("%s: plan for %d tokens, call with %d (path %d)" % (cfg.name, max_tokens, T,
                                                                moe.moe_plan_path(block.plan, T, cfg.k)))
        _, out = run_gpu(cfg, tin, path, T=T, block=block)
        assert_guard(guard)
        g = read_all(block, cfg, T)
        sub = dict(route, idx=route["idx"][:T], w=route["w"][:T], margin=route["margin"][:T])
        check_routing(g, sub, cfg)
        tokens = np.arange(T)
        experts = np.unique(route["idx"][tokens])
        gu, dn, sh = weights.host_experts(cfg, experts)
        delta, out_ref, dbg = oracle.experts(tokens, small["x"], route["h"], route["idx"],
                                             route["w"], gu, dn, sh[0], sh[1], sh[2],
                                             oracle.DTYPES[cfg.dtype], debug=True)
        _check_intermediates(cfg, g, tokens, dbg)
        check_outputs(cfg, small, workloads.torch_to_host(out)[tokens], delta, out_ref, tokens)
        if moe.moe_plan_path(block.plan, T, cfg.k) == moe.MOE_PATH_FUSED:
            assert block.fused_error(T) == 0
    block.close()


def test_glm5_plan_for_8_tokens_called_with_fewer(glm5_weights):
    """The shared expert's 64-row products pick their K split from the row count, not
    monotonically: a plan for 8 tokens called with 1..7 (GLM-5 shared-expert sizes)."""
    cfg = workloads.config("glm5_decode", T=8)
    _fewer_tokens_than_planned(cfg, glm5_weights, moe.MOE_PATH_AUTO, 8, range(1, 8))


@pytest.mark.parametrize("path,max_tokens,calls", [
    (moe.MOE_PATH_STREAM, 16, (7, 3)),
    (moe.MOE_PATH_STREAM, 64, (49,)),
    (moe.MOE_PATH_MFMA, 64, (49, 7)),
    (moe.MOE_PATH_MFMA, 300, (257, 130)),
])
def test_glm5_plan_larger_than_call(glm5_weights, path, max_tokens, calls):
    cfg = workloads.config("glm5_decode", T=max_tokens)
    _fewer_tokens_than_planned(cfg, glm5_weights, path, max_tokens, calls)


@pytest.mark.parametrize("T", [64, 1])
def test_glm5_decode_fused(glm5_weights, T):
    cfg = workloads.config("glm5_decode", T=T)
    _check(cfg, glm5_weights, path=moe.MOE_PATH_FUSED)


def test_glm5_fused_plan_for_8_tokens_called_with_fewer(glm5_weights):
    cfg = workloads.config("glm5_decode", T=8)
    _fewer_tokens_than_planned(cfg, glm5_weights, moe.MOE_PATH_FUSED, 8, (3, 8))


def test_glm5_decode_mfma(glm5_weights):
    cfg = workloads.config("glm5_decode")
    _check(cfg, glm5_weights, path=moe.MOE_PATH_MFMA)


def test_glm5_prefill(glm5_weights):
    """4096 tokens: intermediates on the stratified sample, out and delta on every token."""
    _check(workloads.config("glm5_prefill"), glm5_weights, n_sample=N_SAMPLE, all_outputs=True)


def test_glm5_prefill_zipf(glm5_weights):
    g = _check(workloads.config("glm5_prefill_zipf"), glm5_weights, n_sample=N_SAMPLE)
    assert g["counts"].max() >= 2000 and np.sum(g["counts"] < 10) >= 10


def test_mid_prefill():
    cfg = workloads.config("mid_prefill")
    w = Weights(cfg)
    _check(cfg, w, n_sample=N_SAMPLE)
    # plans sized for more tokens than the call, on both kernel families
    for path in (moe.MOE_PATH_STREAM, moe.MOE_PATH_MFMA):
        _fewer_tokens_than_planned(workloads.config(cfg, T=64), w, path, 64, (49,))
    del w
    torch.cuda.empty_cache()
