"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (one plan per workload, max_tokens = T, MOE_PATH_AUTO unless
stated).  Routing (selected sets, per-expert counts) is checked on every token;
outputs on every token for the decode batch and on a seeded, stratified sample
of tokens (computed one by one by the oracle) for the prefill batches."""
import numpy as np
import pytest
import torch

import mixture_experts_transformer_rmsnorm_amd as moe
import oracle
import workloads
from tests.gpu_harness import (check_close, check_outputs, check_permutation, check_routing,
                               read_all, run_gpu, say, values)
from tests.margin import filtered_small

pytestmark = pytest.mark.gpu

N_SAMPLE = 24


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
    rng = np.random.default_rng(seed)
    picks = set(rng.choice(cfg.T, size=min(n, cfg.T), replace=False).tolist())
    cnt = np.bincount(route["idx"].ravel(), minlength=cfg.E)
    # stratify: tokens of the hottest expert and of the rarest non-empty experts
    hot = int(np.argmax(cnt))
    picks.update(np.nonzero(np.any(route["idx"] == hot, 1))[0][:4].tolist())
    rare = [e for e in np.argsort(cnt) if cnt[e] > 0][:4]
    for e in rare:
        picks.update(np.nonzero(np.any(route["idx"] == e, 1))[0][:1].tolist())
    picks.add(cfg.T - 1)
    return np.array(sorted(picks), np.int64)


def _check(cfg, weights, path=moe.MOE_PATH_AUTO, n_sample=None):
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
    delta, out_ref = oracle.experts(tokens, small["x"], route["h"], route["idx"], route["w"], gu,
                                    dn, sh[0], sh[1], sh[2], oracle.DTYPES[cfg.dtype])
    got = workloads.torch_to_host(out)[tokens]
    check_outputs(cfg, small, got, delta, out_ref, tokens)
    if moe.moe_plan_path(block.plan, cfg.T, cfg.k) == moe.MOE_PATH_FUSED:
        assert block.fused_error(cfg.T) == 0
    del block
    return g


def test_glm5_decode_stream(glm5_weights):
    cfg = workloads.config("glm5_decode")
    _check(cfg, glm5_weights, path=moe.MOE_PATH_STREAM)


@pytest.mark.parametrize("T", [1, 8])
def test_glm5_decode_small_batches(glm5_weights, T):
    """1 and 8 tokens: fewer (expert, pass) items than half the resident blocks, so
    the streaming kernels split every item over several blocks (equal ranges) and
    the fixup kernel finishes them all."""
    cfg = workloads.config("glm5_decode", T=T)
    _check(cfg, glm5_weights, path=moe.MOE_PATH_AUTO)


def test_glm5_stream_split_items(glm5_weights):
    """256 tokens on the streaming path: more (expert, pass) items than resident
    blocks, so the balanced launch splits items between blocks and the fixup
    kernel finishes them."""
    cfg = workloads.config("glm5_decode", T=256)
    _check(cfg, glm5_weights, path=moe.MOE_PATH_STREAM, n_sample=N_SAMPLE)


@pytest.mark.skip(reason="the fused decode kernel is switched off: its first GPU run did not "
                         "finish and the cause has not been established")
def test_glm5_decode_fused(glm5_weights):
    cfg = workloads.config("glm5_decode")
    _check(cfg, glm5_weights, path=moe.MOE_PATH_FUSED)


def test_glm5_decode_mfma(glm5_weights):
    cfg = workloads.config("glm5_decode")
    _check(cfg, glm5_weights, path=moe.MOE_PATH_MFMA, n_sample=16)


def test_glm5_prefill(glm5_weights):
    _check(workloads.config("glm5_prefill"), glm5_weights, n_sample=N_SAMPLE)


def test_glm5_prefill_zipf(glm5_weights):
    g = _check(workloads.config("glm5_prefill_zipf"), glm5_weights, n_sample=N_SAMPLE)
    assert g["counts"].max() >= 2000 and np.sum(g["counts"] < 10) >= 10


def test_mid_prefill():
    cfg = workloads.config("mid_prefill")
    w = Weights(cfg)
    _check(cfg, w, n_sample=N_SAMPLE)
    del w
    torch.cuda.empty_cache()
