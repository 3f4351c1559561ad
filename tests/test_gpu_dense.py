"""Dense block (moe_dense_block_forward: RMSNorm + SwiGLU MLP + residual) against the
oracle's dense block, with the bars of the MoE block: h bit-exact; the MLP activation
within one rounding to D plus accumulation noise; out against the oracle's exact
x + delta, and delta beyond the one rounding of out."""
import types

import numpy as np
import pytest

import oracle
import workloads
import mixture_experts_transformer_rmsnorm_amd as moe
from tests.gpu_harness import check_intermediate, check_outputs, say

pytestmark = pytest.mark.gpu


def _run(case, T, seed, weights):
    import torch
    tin, host = workloads.make_dense_torch(case, seed, "cuda", weights=weights, T=T)
    blk = moe.DenseBlock({k: tin[k] for k in ("norm_w", "gate", "up", "down")}, max_tokens=T,
                         eps=case.eps)
    out = blk.forward(tin["x"])
    torch.cuda.synchronize()
    es_np = np.uint16 if case.dtype == "bf16" else np.float32
    g = dict(out=workloads.torch_to_host(out),
             h=blk.buffer(moe.MOE_BUF_H, T).cpu().numpy().view(es_np).reshape(T, case.d),
             act=blk.buffer(moe.MOE_BUF_SHARED_ACT, T).cpu().numpy().view(es_np).reshape(T, case.Id))
    return blk, tin, host, g


def _check(case, tin, host, g, tokens):
    dt = oracle.DTYPES[case.dtype]
    tokens = np.asarray(tokens, np.int64)
    xs = host["x"][tokens]
    h = oracle.rmsnorm(xs, host["norm_w"], dt, case.eps)
    ref_h = workloads.f32_to_bf16_bits(h) if case.dtype == "bf16" else h
    assert np.array_equal(g["h"][tokens], ref_h), "h differs from the oracle's RMSNorm"
    w = {k: workloads.torch_to_host(tin[k]) for k in ("gate", "up", "down")}
    delta, out_ref, act = oracle.dense_mlp(xs, h, w["gate"], w["up"], w["down"], dt, debug=True)
    vals = workloads.bf16_bits_to_f32 if case.dtype == "bf16" else (lambda a: a)
    check_intermediate(vals(g["act"][tokens]).astype(np.float64), act, case.dtype, "act")
    cfg = types.SimpleNamespace(dtype=case.dtype)
    check_outputs(cfg, dict(x=host["x"]), g["out"][tokens], delta, out_ref, tokens)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,d,Id", [(1, 256, 192), (37, 256, 320), (63, 512, 704), (64, 512, 704),
                                    (260, 256, 320), (300, 512, 1024)])
def test_small_dense_blocks(T, d, Id, dtype):
    case = workloads.DenseCase("small", T, d, Id, dtype)
    say("dense %s T %d d %d Id %d" % (dtype, T, d, Id))
    _, tin, host, g = _run(case, T, seed=T, weights="host")
    _check(case, tin, host, g, np.arange(T))


def test_dense_fused_swiglu_ragged_width():
    """Enough 256 x 128 tiles that the gate/up product runs unsplit with its SwiGLU
    epilogue fused, at an MLP width (1088 = 8.5 x 128) that leaves the last act
    tile half full and a token count (8000 = 31.25 x 256) that leaves the last
    row tile a quarter full; sampled tokens (and the last one) against the oracle."""
    case = workloads.DenseCase("fused_ragged", 8000, 256, 1088, "bf16")
    say("dense bf16 T %d d %d Id %d (fused SwiGLU, sampled tokens)" % (case.T, case.d, case.Id))
    _, tin, host, g = _run(case, case.T, seed=11, weights="host")
    rng = np.random.default_rng(3)
    tokens = np.sort(np.concatenate([rng.choice(case.T - 1, size=24, replace=False), [case.T - 1]]))
    _check(case, tin, host, g, tokens)


@pytest.mark.parametrize("name", ["glm5_dense_decode", "glm5_dense_prefill"])
def test_glm5_dense_block_sampled(name):
    case = workloads.DENSE_CASES[name]
    say("dense %s T %d d %d Id %d (sampled tokens)" % (name, case.T, case.d, case.Id))
    _, tin, host, g = _run(case, case.T, seed=0, weights="device")
    rng = np.random.default_rng(7)
    tokens = np.sort(rng.choice(case.T, size=min(case.T, 24), replace=False))
    _check(case, tin, host, g, tokens)


def test_zero_tokens_and_plan_mismatch():
    import torch
    say("dense: zero tokens; MoE entry on a dense plan")
    case = workloads.DenseCase("small", 8, 256, 192)
    tin, _ = workloads.make_dense_torch(case, 1, "cuda", weights="host")
    blk = moe.DenseBlock({k: tin[k] for k in ("norm_w", "gate", "up", "down")}, max_tokens=8)
    moe.moe_dense_block_forward(blk.plan, blk.workspace, blk.workspace_bytes, None, 0, None, None,
                                None, None, None, None)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_block_forward(blk.plan, blk.workspace, blk.workspace_bytes, None, 8, tin["x"],
                              tin["norm_w"], tin["gate"], None, tin["gate"], tin["down"], None, None,
                              None, 1, 1.0, tin["x"])
    assert ei.value.status == moe.MOE_ERROR_NOT_SUPPORTED
    out = blk.forward(tin["x"], out=tin["x"])  # in place
    torch.cuda.synchronize()
    assert out.data_ptr() == tin["x"].data_ptr()
