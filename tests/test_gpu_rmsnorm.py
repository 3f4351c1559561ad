"""Standalone RMSNorm entry point (moe_rmsnorm) against the oracle's RMSNorm, at the
widths of the block's other norms: hidden size, query latent, key-value latent
(strided rows), per-head query/key width, and narrow / ragged edge cases.

Both sides round the fp64 mean of squares once to fp32 and take the IEEE fp32 sqrt
and divide, then round x*r and the gain product to the storage dtype, so the
results are compared bit for bit."""
import numpy as np
import pytest

import oracle
import workloads
import mixture_experts_transformer_rmsnorm_amd as moe
from tests.gpu_harness import say

pytestmark = pytest.mark.gpu

DT = {"bf16": 1, "f32": 0}


def _run(x_host, gain_host, rows, width, stride, dtype, out_stride=None, in_place=False):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = workloads.host_to_torch(x_host, dtype, "cuda")
    g = workloads.host_to_torch(gain_host, dtype, "cuda")
    if in_place:
        out, ost = x, stride
    else:
        ost = out_stride or width
        out = torch.full((rows, ost), 7.0, dtype=tdt, device="cuda")
    moe.moe_rmsnorm(None, DT[dtype], rows, width, 1e-6, x, stride, g, out, ost)
    torch.cuda.synchronize()
    return workloads.torch_to_host(out)


def _check(got, x_host, gain_host, rows, width, dtype, filler=None):
    ref = oracle.rmsnorm(np.ascontiguousarray(x_host[:, :width]), gain_host, DT[dtype], 1e-6)
    ref_bits = workloads.f32_to_bf16_bits(ref) if dtype == "bf16" else ref
    g = got[:, :width]
    mism = int(np.sum(g != ref_bits))
    say("  rows %d width %d %s: %d mismatches" % (rows, width, dtype, mism))
    assert mism == 0
    if filler is not None:  # columns past width are not written
        assert np.array_equal(got[:, width:], filler)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", ["input_norm", "q_latent_norm", "kv_latent_norm", "qk_head_norm"])
def test_block_norm_widths(case, dtype):
    c = workloads.NORM_CASES[case]
    rows = 1000 if c.width >= 2048 else 3001  # several blocks and a ragged last block
    say("case %s %s rows %d width %d stride %d" % (case, dtype, rows, c.width, c.stride))
    x, g = workloads.draw_norm(rows, c.width, c.stride, dtype, seed=3)
    got = _run(x, g, rows, c.width, c.stride, dtype, out_stride=c.stride)
    fill = np.full((rows, c.stride - c.width), 7.0, np.float32)
    fill = workloads.f32_to_bf16_bits(fill) if dtype == "bf16" else fill
    _check(got, x, g, rows, c.width, dtype, filler=fill if c.stride > c.width else None)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("width", [8, 64, 136, 1000, 2056, 8192])
def test_edge_widths_and_single_row(width, dtype):
    if dtype == "bf16" and width % 8:
        pytest.skip("bf16 rows are whole 16-byte vectors")
    for rows in (1, 2, 67):
        say("width %d %s rows %d" % (width, dtype, rows))
        x, g = workloads.draw_norm(rows, width, width, dtype, seed=rows)
        _check(_run(x, g, rows, width, width, dtype), x, g, rows, width, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_in_place_strided(dtype):
    rows, width, stride = 513, 512, 576
    say("in place %s rows %d width %d stride %d" % (dtype, rows, width, stride))
    x, g = workloads.draw_norm(rows, width, stride, dtype, seed=11)
    got = _run(x, g, rows, width, stride, dtype, in_place=True)
    _check(got, x, g, rows, width, dtype, filler=x[:, width:])


def test_zero_rows_and_python_wrapper():
    import torch
    say("zero rows; torch-facing wrapper")
    moe.moe_rmsnorm(None, 1, 0, 128, 1e-6, None, 128, None, None, 128)
    x, g = workloads.draw_norm(64, 256, 256, "bf16", seed=5)
    xt = workloads.host_to_torch(x, "bf16", "cuda").reshape(4, 16, 256)  # [tokens, heads, width]
    gt = workloads.host_to_torch(g, "bf16", "cuda")
    out = moe.rmsnorm(xt, gt)
    torch.cuda.synchronize()
    _check(workloads.torch_to_host(out.reshape(64, 256)), x, g, 64, 256, "bf16")
