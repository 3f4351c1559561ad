"""GPU parity of the HIP path (through the C ABI) against the CPU oracle at
small shapes that span several tiles and ragged tails, both kernel families,
and the degenerate cases."""
import numpy as np
import pytest
import torch

import mixture_experts_transformer_rmsnorm_amd as moe
import oracle
import workloads
from tests.gpu_harness import (assert_guard, check_close, check_intermediate, check_outputs,
                               check_permutation, check_routing, guard_workspace, make_block,
                               oracle_outputs, prepare, read_all, run_gpu, say, values)

pytestmark = pytest.mark.gpu

STREAM, MFMA, FUSED = moe.MOE_PATH_STREAM, moe.MOE_PATH_MFMA, moe.MOE_PATH_FUSED


def _full_check(cfg, small, route, tin, path, check_stages=True):
    say("case %s T=%d d=%d E=%d I=%d Is=%d k=%d %s path=%d" % (
        cfg.name, cfg.T, cfg.d, cfg.E, cfg.I, cfg.Is, cfg.k, cfg.dtype, path))
    block, out = run_gpu(cfg, tin, path)
    g = read_all(block, cfg, cfg.T)
    # RMSNorm output: same fp32 steps on both sides, bit-exact
    h_ref = route["h"]
    if cfg.dtype == "bf16":
        assert np.array_equal(g["h"], workloads.f32_to_bf16_bits(h_ref))
    else:
        assert np.array_equal(g["h"], h_ref)
    check_routing(g, route, cfg)
    check_permutation(g, cfg, cfg.T)
    tokens = np.arange(cfg.T)
    delta, out_ref, dbg = oracle_outputs(cfg, small, route, tin, tokens, debug=True)
    if check_stages:
        # per-stage intermediates: act and y of each (t, j) through row_of
        rows = g["row_of"].ravel()
        check_intermediate(values(g["act"][rows], cfg.dtype), dbg["act"].reshape(-1, cfg.I),
                           cfg.dtype, "act")
        check_intermediate(values(g["y"][rows], cfg.dtype), dbg["y"].reshape(-1, cfg.d),
                           cfg.dtype, "y")
    check_outputs(cfg, small, workloads.torch_to_host(out), delta, out_ref, tokens)
    return block, out


def test_tiny_fp32_config():
    """The tiny fp32 workload in full (streaming kernels)."""
    cfg, small, route, tin = prepare("tiny_fp32")
    _full_check(cfg, small, route, tin, moe.MOE_PATH_AUTO)


@pytest.mark.parametrize("path", [STREAM, MFMA])
@pytest.mark.parametrize("shape", [
    dict(T=300, d=256, E=16, I=192, Is=128, k=4),         # ragged M tiles, partial slices
    dict(T=77, d=384, E=8, I=64, Is=192, k=2),             # one 64-wide N tile, odd T
    dict(T=520, d=512, E=32, I=320, Is=0, k=6, routed_scale=2.5),  # no shared expert
])
def test_small_bf16_both_paths(shape, path):
    cfg = workloads.config("tiny_fp32", dtype="bf16", **shape)
    cfg, small, route, tin = prepare(cfg, seed=3)
    _full_check(cfg, small, route, tin, path)


@pytest.mark.parametrize("shape", [
    dict(d=192, Is=64, I=128, E=16, k=4),      # rows of 24 vectors, most extra blocks idle
    dict(d=640, Is=576, I=192, E=12, k=3),     # 2-3 act_s columns per block
    dict(d=1024, Is=2048, I=256, E=32, k=8),   # 8-9 columns per block, 4 KiB down rows
])
@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_shared_expert_beside_small_routing(shape, T):
    """Up to 4 bf16 tokens on the streaming path: the shared expert runs in extra
    blocks of the router, selection and permutation launches (act_s columns split
    between the first two).  act_s element-wise against the oracle, then the whole
    output."""
    cfg = workloads.config("tiny_fp32", dtype="bf16", T=T, **shape)
    cfg, small, route, tin = prepare(cfg, seed=11 + T)
    block, _ = _full_check(cfg, small, route, tin, STREAM)
    act_s = block.buffer(moe.MOE_BUF_SHARED_ACT, T).cpu().numpy().view(np.uint16)
    _, _, dbg = oracle_outputs(cfg, small, route, tin, np.arange(T), debug=True)
    check_intermediate(values(act_s.reshape(T, cfg.Is), "bf16"), dbg["act_s"], "bf16", "act_s")
    block.close()


@pytest.mark.parametrize("T", [1, 2, 5])
def test_fp32_smallest_batches(T):
    """fp32 at 1, 2 and 5 tokens on the streaming path: the gate_up splits its
    weight rows into ranges whose sums the down launch adds (1 and 2 tokens), and
    the side-stream shared expert (fp32 plans keep it there)."""
    cfg = workloads.config("tiny_fp32", T=T)
    cfg, small, route, tin = prepare(cfg, seed=21 + T)
    block, _ = _full_check(cfg, small, route, tin, STREAM)
    block.close()


@pytest.mark.parametrize("path", [STREAM, MFMA])
def test_top1_and_all_experts(path):
    for k, E in ((1, 8), (8, 8)):
        cfg = workloads.config("tiny_fp32", dtype="bf16", T=96, E=E, k=k, d=256, I=128, Is=64)
        cfg, small, route, tin = prepare(cfg, seed=5)
        _full_check(cfg, small, route, tin, path)


@pytest.mark.parametrize("path", [STREAM, MFMA])
def test_empty_experts_and_single_token(path):
    # 3 tokens x top-2 over 64 experts: most experts get no token
    for T in (1, 3):
        cfg = workloads.config("tiny_fp32", dtype="bf16", T=T, E=64, k=2, d=256, I=128, Is=128)
        cfg, small, route, tin = prepare(cfg, seed=7)
        _full_check(cfg, small, route, tin, path)


def test_zero_tokens_is_a_noop():
    cfg, small, route, tin = prepare(workloads.config("tiny_fp32", dtype="bf16", T=16))
    block, _ = run_gpu(cfg, tin, moe.MOE_PATH_AUTO)
    sentinel = torch.full((1, cfg.d), 7.0, dtype=torch.bfloat16, device="cuda")
    block.forward(tin["x"][:0], out=sentinel[:0])
    torch.cuda.synchronize()
    assert torch.all(sentinel == 7.0)


@pytest.mark.parametrize("T", [200, 1])
def test_out_aliases_x_and_repeatability(T):
    """Bitwise repeatability and in-place calls; at 1 token on the streaming path the
    shared expert's row sums and the gate_up's row-range sums take part."""
    cfg, small, route, tin = prepare(workloads.config("tiny_fp32", dtype="bf16", T=T, E=16,
                                                      k=4, d=256, I=128, Is=128))
    for path in (STREAM, MFMA):
        block, out1 = run_gpu(cfg, tin, path)
        _, out2 = run_gpu(cfg, tin, path, block=block)
        assert torch.equal(out1, out2), "bitwise repeatability"
        xin = tin["x"].clone()
        block.forward(xin, out=xin)  # in place
        torch.cuda.synchronize()
        assert torch.equal(xin, out1)
    # both kernel families agree closely
    b1, o1 = run_gpu(cfg, tin, STREAM)
    b2, o2 = run_gpu(cfg, tin, MFMA)
    check_close(o1.float().cpu().numpy(), o2.float().cpu().numpy(), "bf16", "stream-vs-mfma")


def test_stream_split_items_repeatable():
    """Streaming path with more (expert, pass) items than resident blocks (items
    split between blocks, finished by the fixup kernel): parity and bitwise
    repeatability."""
    cfg = workloads.config("tiny_fp32", dtype="bf16", T=520, E=32, k=6, d=256, I=320, Is=128)
    cfg, small, route, tin = prepare(cfg, seed=11)
    cnt = np.bincount(route["idx"].ravel(), minlength=cfg.E)
    assert int(np.sum((cnt + 7) // 8)) > 256  # more passes than blocks
    block, out1 = _full_check(cfg, small, route, tin, STREAM)
    _, out2 = run_gpu(cfg, tin, STREAM, block=block)
    assert torch.equal(out1, out2), "bitwise repeatability"


def test_smaller_call_after_larger_reuses_workspace():
    cfg, small, route, tin = prepare(workloads.config("tiny_fp32", dtype="bf16", T=256, E=16,
                                                      k=4, d=256, I=128, Is=128))
    block, _ = run_gpu(cfg, tin, MFMA)
    T2 = 37
    _, out = run_gpu(cfg, tin, MFMA, T=T2, block=block)
    g = read_all(block, cfg, T2)
    sub = dict(route, idx=route["idx"][:T2], w=route["w"][:T2], h=route["h"][:T2])
    cnt = np.bincount(sub["idx"].ravel(), minlength=cfg.E)
    assert np.array_equal(g["counts"], cnt)
    delta, out_ref = oracle_outputs(cfg, small, route, tin, np.arange(T2))
    check_outputs(cfg, small, workloads.torch_to_host(out), delta, out_ref, np.arange(T2))


@pytest.mark.parametrize("path", [STREAM, MFMA])
@pytest.mark.parametrize("max_tokens,calls", [(8, (3, 7)), (16, (7,)), (64, (49, 1)), (300, (129,))])
def test_plan_for_more_tokens_than_the_call(path, max_tokens, calls):
    """The serving case: a plan sized for the largest batch, called with fewer tokens.
    At d 2048 with a shared expert of 1024 the 64-row products' split-K counts vary
    with the row count; a guard region after the workspace must stay untouched."""
    cfg = workloads.config("tiny_fp32", dtype="bf16", T=max_tokens, d=2048, E=16, I=256,
                           Is=1024, k=4)
    cfg, small, route, tin = prepare(cfg, seed=19)
    block = make_block(cfg, tin, path, max_tokens=max_tokens)
    guard = guard_workspace(block)
    for T in calls:
        say("plan for %d tokens, call with %d, path %d" % (max_tokens, T, path))
        _, out = run_gpu(cfg, tin, path, T=T, block=block)
        assert_guard(guard)
        g = read_all(block, cfg, T)
        sub = dict(route, idx=route["idx"][:T], w=route["w"][:T], margin=route["margin"][:T])
        check_routing(g, sub, cfg)
        check_permutation(g, cfg, T)
        delta, out_ref, dbg = oracle_outputs(cfg, small, route, tin, np.arange(T), debug=True)
        rows = g["row_of"].ravel()
        check_intermediate(values(g["act"][rows], cfg.dtype), dbg["act"].reshape(-1, cfg.I),
                           cfg.dtype, "act")
        check_intermediate(values(g["y"][rows], cfg.dtype), dbg["y"].reshape(-1, cfg.d),
                           cfg.dtype, "y")
        check_outputs(cfg, small, workloads.torch_to_host(out), delta, out_ref, np.arange(T))
    block.close()


@pytest.mark.parametrize("path,T", [(STREAM, 64), (MFMA, 64), (STREAM, 1), (STREAM, 3)])
def test_first_call_captured_in_a_graph(path, T):
    """A forward call creates no HIP object (the side stream of the shared expert and
    its events come from plan creation), so even a plan's first call can be captured
    into a graph.  Each replay, with eager calls and synchronisations between them,
    must equal an uncaptured call bit for bit.  At 1 and 3 tokens the shared expert
    runs inside the routing launches and (at 1) the gate_up splits K."""
    cfg = workloads.config("tiny_fp32", dtype="bf16", T=T, d=512, E=16, I=256, Is=256, k=4)
    cfg, small, route, tin = prepare(cfg, seed=23)
    ref_block, ref = run_gpu(cfg, tin, path)
    block = make_block(cfg, tin, path)
    x = tin["x"]
    out = torch.empty_like(x)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        block.forward(x, out=out)
    for rep in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "replay %d differs from the eager call" % rep
        _, again = run_gpu(cfg, tin, path, block=ref_block)  # eager work between replays
        assert torch.equal(again, ref)
    block.close()
    ref_block.close()


# ----------------------------------------------------------------------------- fused decode
@pytest.mark.parametrize("shape", [
    dict(T=64, d=256, E=16, I=192, Is=128, k=4),           # several slices per expert
    dict(T=37, d=384, E=8, I=64, Is=192, k=2),              # odd T: a partial chunk
    dict(T=50, d=512, E=32, I=320, Is=0, k=6, routed_scale=2.5),  # no shared expert
    dict(T=64, d=256, E=8, I=128, Is=64, k=8),              # every expert selected
    dict(T=40, d=256, E=300, I=128, Is=128, k=8),           # E not a multiple of 64
    dict(T=1, d=256, E=64, I=128, Is=128, k=2),             # one token, most experts empty
])
def test_fused_decode(shape):
    cfg = workloads.config("tiny_fp32", dtype="bf16", **shape)
    cfg, small, route, tin = prepare(cfg, seed=13)
    block, _ = _full_check(cfg, small, route, tin, FUSED)
    assert moe.moe_plan_path(block.plan, cfg.T, cfg.k) == FUSED
    assert block.fused_error(cfg.T) == 0


def test_fused_repeatability_in_place_and_workspace_reuse():
    cfg, small, route, tin = prepare(workloads.config("tiny_fp32", dtype="bf16", T=64, E=16,
                                                      k=4, d=256, I=128, Is=128), seed=17)
    block, out1 = run_gpu(cfg, tin, FUSED)
    _, out2 = run_gpu(cfg, tin, FUSED, block=block)
    assert torch.equal(out1, out2), "bitwise repeatability"
    xin = tin["x"].clone()
    block.forward(xin, out=xin)  # in place
    torch.cuda.synchronize()
    assert torch.equal(xin, out1)
    # the fused and the multi-kernel streaming paths compute the same thing
    _, o_stream = run_gpu(cfg, tin, STREAM)
    check_close(out1.float().cpu().numpy(), o_stream.float().cpu().numpy(), "bf16", "fused-vs-stream")
    # a smaller call after a larger one on the same workspace
    T2 = 23
    _, out = run_gpu(cfg, tin, FUSED, T=T2, block=block)
    assert block.fused_error(T2) == 0
    delta, out_ref = oracle_outputs(cfg, small, route, tin, np.arange(T2))
    check_outputs(cfg, small, workloads.torch_to_host(out), delta, out_ref, np.arange(T2))


def test_debug_sync_gives_the_same_result(monkeypatch):
    """MOE_DEBUG_SYNC=1 synchronises after every stage (streaming path, with its side
    stream, and the MFMA path); the results are those of a normal call, bit for bit."""
    for path in (STREAM, MFMA):
        cfg = workloads.config("tiny_fp32", dtype="bf16", T=40, d=256, E=16, I=128, Is=128, k=4)
        cfg, small, route, tin = prepare(cfg, seed=29)
        monkeypatch.delenv("MOE_DEBUG_SYNC", raising=False)
        block, ref = run_gpu(cfg, tin, path)
        monkeypatch.setenv("MOE_DEBUG_SYNC", "1")
        _, got = run_gpu(cfg, tin, path, block=block)
        monkeypatch.delenv("MOE_DEBUG_SYNC")
        assert torch.equal(got, ref)
        block.close()
