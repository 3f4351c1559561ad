"""The allocation-free entry point moe_block_forward_static (its workspace is the
library's static buffer on the GPU) against moe_block_forward with a caller-owned
workspace: two calls in a row, the second with fewer tokens, on both kernel
families at a small shape and on the GLM-5 decode shape.  The same kernels run on
the same inputs, so the outputs must be identical."""
import numpy as np
import pytest
import torch

import mixture_experts_transformer_rmsnorm_amd as moe
import workloads
from tests.gpu_harness import check_close, make_block, prepare, say

pytestmark = pytest.mark.gpu


def _static(block, tin, T, out):
    w = block.weights
    moe.moe_block_forward_static(block.plan, None, T, tin["x"][:T], w["norm_w"], w["router_w"],
                                 w["corr_bias"], w["gate_up"], w["down"], w.get("shared_gate"),
                                 w.get("shared_up"), w.get("shared_down"), block.top_k,
                                 block.routed_scale, out)


def _compare(cfg, tin, path, calls):
    block = make_block(cfg, tin, path, max_tokens=max(calls))
    assert block.workspace_bytes <= moe.STATIC_WORKSPACE_BYTES
    refs = {}
    for T in calls:
        refs[T] = block.forward(tin["x"][:T]).clone()
    outs = {}
    for T in calls:  # the static calls in a row, the second smaller than the first
        say("static workspace: %s, %d tokens, path %d" % (cfg.name, T, path))
        outs[T] = torch.empty_like(refs[T])
        _static(block, tin, T, outs[T])
    torch.cuda.synchronize()
    for T in calls:
        check_close(outs[T].float().cpu().numpy(), refs[T].float().cpu().numpy(), cfg.dtype,
                    "static-vs-workspace T=%d" % T)
        assert torch.equal(outs[T], refs[T]), "T=%d: outputs differ" % T
    block.close()


@pytest.mark.parametrize("path", [moe.MOE_PATH_STREAM, moe.MOE_PATH_MFMA])
def test_static_matches_workspace_small(path):
    cfg = workloads.config("tiny_fp32", dtype="bf16", T=96, d=512, E=16, I=256, Is=256, k=4)
    cfg, small, route, tin = prepare(cfg, seed=29)
    _compare(cfg, tin, path, (96, 37))


def test_static_matches_workspace_glm5_decode():
    cfg = workloads.config("glm5_decode")
    tin = workloads.make_torch(cfg, 0, device="cuda", weights="device")
    torch.cuda.synchronize()
    _compare(cfg, tin, moe.MOE_PATH_AUTO, (64, 8))
    del tin
    torch.cuda.empty_cache()
