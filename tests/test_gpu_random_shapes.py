"""GPU parity on seeded random shapes within the library's documented limits (hidden
size and widths multiples of 64, top-k at most 8): every token's routing, permutation,
intermediates and output against the oracle, on the kernel path drawn for the case
(the fused path runs calls of at most 64 tokens and hands larger ones to the
streaming kernels).
The draws are fixed by the seed, so every run checks the same cases."""
import numpy as np
import pytest

import mixture_experts_transformer_rmsnorm_amd as moe
import workloads
from tests.gpu_harness import prepare, say
from tests.test_gpu_parity import _full_check

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=2024, tmax=700):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = "f32" if i % 5 == 4 else "bf16"
        d = 64 * int(rng.integers(2, 17))          # 128 .. 1024
        I = 64 * int(rng.integers(1, 9))           # 64 .. 512
        Is = 64 * int(rng.integers(0, 9))          # 0 (no shared expert) .. 512
        E = int(rng.integers(1, 301))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(1, tmax))
        paths = [moe.MOE_PATH_AUTO, moe.MOE_PATH_STREAM] + (
            [moe.MOE_PATH_MFMA, moe.MOE_PATH_FUSED] if dtype == "bf16" else [])
        path = paths[int(rng.integers(0, len(paths)))]
        rs = float(rng.choice([1.0, 2.5]))
        out.append((i, dict(dtype=dtype, d=d, I=I, Is=Is, E=E, k=k, T=T, routed_scale=rs), path))
    return out


@pytest.mark.parametrize("i,shape,path", _cases(), ids=lambda v: str(v) if isinstance(v, int) else None)
def test_random_shape(i, shape, path):
    cfg = workloads.config("tiny_fp32", **shape)
    say("random case %d: %s path %d" % (i, shape, path))
    cfg, small, route, tin = prepare(cfg, seed=100 + i)
    block, _ = _full_check(cfg, small, route, tin, path)
    if moe.moe_plan_path(block.plan, cfg.T, cfg.k) == moe.MOE_PATH_FUSED:
        assert block.fused_error(cfg.T) == 0
    block.close()


@pytest.mark.parametrize("i,shape,path", _cases(n=16, seed=4048, tmax=9),
                         ids=lambda v: str(v) if isinstance(v, int) else None)
def test_random_shape_few_tokens(i, shape, path):
    """1-8 tokens: the smallest batches' column and row-range splits of the weight
    streams and the shared expert beside the routing launches."""
    cfg = workloads.config("tiny_fp32", **shape)
    say("few-token random case %d: %s path %d" % (i, shape, path))
    cfg, small, route, tin = prepare(cfg, seed=300 + i)
    block, _ = _full_check(cfg, small, route, tin, path)
    if moe.moe_plan_path(block.plan, cfg.T, cfg.k) == moe.MOE_PATH_FUSED:
        assert block.fused_error(cfg.T) == 0
    block.close()
