"""Expert layout conversion (moe_pack_expert / moe_unpack_expert) against the oracle's
packing: bit-exact, on random bit patterns (the kernels move bits and do no
arithmetic), at small shapes with several tiles and at the GLM-5 expert shape; and
packed HF weights driving the MoE block."""
import numpy as np
import pytest

import oracle
import workloads
import mixture_experts_transformer_rmsnorm_amd as moe
from tests.gpu_harness import say

pytestmark = pytest.mark.gpu

DT = {"bf16": moe.MOE_DTYPE_BF16, "f32": moe.MOE_DTYPE_F32}


def _bits(shape, dtype, rng):
    if dtype == "bf16":
        return rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    return rng.integers(0, 1 << 32, size=shape, dtype=np.uint32).view(np.float32)


def _dev(a):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).cuda()
    return torch.from_numpy(a.view(np.int32).copy()).cuda()


def _host(t, like):
    return t.cpu().numpy().view(like.dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d,I", [(64, 64), (256, 128), (192, 320), (6144, 2048)])
def test_pack_unpack_bit_exact(d, I, dtype):
    import torch
    say("pack %s d %d I %d" % (dtype, d, I))
    rng = np.random.default_rng(d * 7 + I)
    gate, up, down = _bits((I, d), dtype, rng), _bits((I, d), dtype, rng), _bits((d, I), dtype, rng)
    g, u, dn = _dev(gate), _dev(up), _dev(down)
    gu = torch.empty((d, 2 * I), dtype=g.dtype, device="cuda")
    dp = torch.empty((I, d), dtype=g.dtype, device="cuda")
    moe.moe_pack_expert(None, DT[dtype], d, I, g, u, dn, gu, dp)
    ref_gu, ref_dp = oracle.pack_expert(gate, up, down)
    got_gu, got_dp = _host(gu, gate), _host(dp, gate)
    assert np.array_equal(got_gu.view(np.uint8), ref_gu.view(np.uint8))
    assert np.array_equal(got_dp.view(np.uint8), ref_dp.view(np.uint8))
    g2, u2, d2 = torch.empty_like(g), torch.empty_like(u), torch.empty_like(dn)
    moe.moe_unpack_expert(None, DT[dtype], d, I, gu, dp, g2, u2, d2)
    for got, ref in ((g2, gate), (u2, up), (d2, down)):
        assert np.array_equal(_host(got, ref).view(np.uint8), ref.view(np.uint8))


def test_packed_hf_experts_drive_the_block():
    """HF-layout experts packed on the device give the same grouped tensors as the
    oracle's packing, and the block run on them matches the oracle's forward."""
    import torch
    from tests.gpu_harness import check_outputs, oracle_outputs, prepare, run_gpu
    cfg, small, route, tin = prepare(workloads.config("tiny_fp32", dtype="bf16", T=48, E=8, k=2),
                                     seed=21)
    say("packed experts drive the block: T %d E %d k %d" % (cfg.T, cfg.E, cfg.k))
    host_gu = workloads.torch_to_host(tin["gate_up"])
    host_dn = workloads.torch_to_host(tin["down"])
    # unpack the grouped experts into HF tensors with the oracle, then pack them on the GPU
    hf = [oracle.unpack_expert(host_gu[e], host_dn[e]) for e in range(cfg.E)]
    gates = [_dev(h[0]).view(torch.bfloat16) for h in hf]
    ups = [_dev(h[1]).view(torch.bfloat16) for h in hf]
    downs = [_dev(h[2]).view(torch.bfloat16) for h in hf]
    gu, dn = moe.pack_experts(gates, ups, downs)
    torch.cuda.synchronize()
    assert np.array_equal(workloads.torch_to_host(gu), host_gu)
    assert np.array_equal(workloads.torch_to_host(dn), host_dn)
    tin = dict(tin, gate_up=gu, down=dn)
    block, res = run_gpu(cfg, tin)
    tokens = np.arange(cfg.T)
    delta, out_ref = oracle_outputs(cfg, small, route, tin, tokens)
    check_outputs(cfg, small, workloads.torch_to_host(res), delta, out_ref, tokens)
