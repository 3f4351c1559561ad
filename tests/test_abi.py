"""The C-ABI library loads, exports every symbol include/moe.h declares, and
validates its arguments on the host (no device work is enqueued by any call
made here)."""
import ctypes
import os
import re

import pytest

import mixture_experts_transformer_rmsnorm_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", src)))


def test_header_declarations_are_exported():
    names = _declared()
    assert "moe_block_forward" in names and "moe_plan_create" in names
    lib = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(moe.EXPORTS) == names


def test_abi_version_and_strings():
    assert moe.moe_abi_version() == moe.ABI_VERSION
    assert moe.moe_status_string(moe.MOE_ERROR_WORKSPACE_TOO_SMALL) == "workspace too small"
    assert moe.moe_stage_name(0) == "rmsnorm" and moe.moe_stage_name(99) is None
    assert ctypes.sizeof(moe.moe_config_t) == 48


def _cfg(**kw):
    base = dict(dim=6144, max_tokens=64, n_experts=256, moe_inter=2048, shared_inter=2048,
                max_top_k=8, dtype="bf16")
    base.update(kw)
    return moe.make_config(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(dim=100), moe.MOE_ERROR_NOT_SUPPORTED),
    (dict(moe_inter=96), moe.MOE_ERROR_NOT_SUPPORTED),
    (dict(shared_inter=32), moe.MOE_ERROR_NOT_SUPPORTED),
    (dict(max_top_k=17, n_experts=32), moe.MOE_ERROR_NOT_SUPPORTED),
    (dict(n_experts=2048), moe.MOE_ERROR_NOT_SUPPORTED),
    (dict(max_top_k=0), moe.MOE_ERROR_INVALID_VALUE),
    (dict(max_top_k=9, n_experts=8), moe.MOE_ERROR_INVALID_VALUE),
    (dict(max_tokens=-1), moe.MOE_ERROR_INVALID_VALUE),
    (dict(eps=0.0), moe.MOE_ERROR_INVALID_VALUE),
    (dict(dtype=7), moe.MOE_ERROR_NOT_SUPPORTED),
    (dict(dtype="f32", path=moe.MOE_PATH_MFMA), moe.MOE_ERROR_NOT_SUPPORTED),
    (dict(path=5), moe.MOE_ERROR_INVALID_VALUE),
    (dict(dtype="f32", path=moe.MOE_PATH_FUSED), moe.MOE_ERROR_NOT_SUPPORTED),
    (dict(flags=1), moe.MOE_ERROR_INVALID_VALUE),
])
def test_plan_validation(kw, status):
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_plan_create(_cfg(**kw))
    assert ei.value.status == status


def test_plan_struct_size_checked():
    cfg = _cfg()
    cfg.struct_size = 40
    with pytest.raises(moe.MoEError):
        moe.moe_plan_create(cfg)


def test_fused_plan_path():
    plan, _ = moe.moe_plan_create(_cfg(path=moe.MOE_PATH_FUSED, max_tokens=128))
    try:
        assert moe.moe_plan_path(plan, 64, 8) == moe.MOE_PATH_FUSED
        assert moe.moe_plan_path(plan, 1, 8) == moe.MOE_PATH_FUSED
        assert moe.moe_plan_path(plan, 65, 8) == moe.MOE_PATH_STREAM  # past the fused batch limit
    finally:
        moe.moe_plan_destroy(plan)


def test_workspace_sizing_and_path_choice():
    plan, ws = moe.moe_plan_create(_cfg(max_tokens=16384))
    try:
        assert moe.moe_plan_path(plan, 64, 8) == moe.MOE_PATH_STREAM     # decode: stream weights
        assert moe.moe_plan_path(plan, 4096, 8) == moe.MOE_PATH_MFMA     # prefill: matrix cores
        A = 16384 * 8
        # act [A, I] + y [A, d] in bf16 dominate the workspace
        assert ws >= 2 * A * (2048 + 6144)
        assert moe.moe_buffer_bytes(plan, 100, 8, moe.MOE_BUF_Y) == 100 * 8 * 6144 * 2
        assert moe.moe_buffer_bytes(plan, 100, 9, moe.MOE_BUF_Y) == 0
    finally:
        moe.moe_plan_destroy(plan)
    plan, ws32 = moe.moe_plan_create(_cfg(dtype="f32", dim=256, n_experts=8, moe_inter=128,
                                          shared_inter=0, max_top_k=2))
    assert moe.moe_plan_path(plan, 64, 2) == moe.MOE_PATH_STREAM
    moe.moe_plan_destroy(plan)


FAKE = 1 << 20  # aligned, never dereferenced: every call below fails validation


def _fwd(plan, ws, **kw):
    args = dict(plan=plan, workspace=FAKE, workspace_bytes=ws, stream=0, num_tokens=8, x=FAKE,
                norm_w=FAKE, router_w=FAKE, corr_bias=FAKE, gate_up=FAKE, down=FAKE,
                shared_gate=FAKE, shared_up=FAKE, shared_down=FAKE, top_k=8, routed_scale=2.5,
                out=FAKE)
    args.update(kw)
    moe.moe_block_forward(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(num_tokens=65), moe.MOE_ERROR_INVALID_VALUE),
    (dict(num_tokens=-1), moe.MOE_ERROR_INVALID_VALUE),
    (dict(top_k=0), moe.MOE_ERROR_INVALID_VALUE),
    (dict(top_k=9), moe.MOE_ERROR_INVALID_VALUE),
    (dict(routed_scale=float("inf")), moe.MOE_ERROR_INVALID_VALUE),
    (dict(routed_scale=float("nan")), moe.MOE_ERROR_INVALID_VALUE),
    (dict(x=None), moe.MOE_ERROR_INVALID_VALUE),
    (dict(shared_down=None), moe.MOE_ERROR_INVALID_VALUE),
    (dict(workspace=None), moe.MOE_ERROR_INVALID_VALUE),
    (dict(gate_up=FAKE + 8), moe.MOE_ERROR_MISALIGNED),
    (dict(out=FAKE + 2), moe.MOE_ERROR_MISALIGNED),
    (dict(workspace_bytes=1024), moe.MOE_ERROR_WORKSPACE_TOO_SMALL),
])
def test_forward_validation(kw, status):
    plan, ws = moe.moe_plan_create(_cfg())
    try:
        with pytest.raises(moe.MoEError) as ei:
            _fwd(plan, ws, **kw)
        assert ei.value.status == status
    finally:
        moe.moe_plan_destroy(plan)


def test_zero_tokens_succeeds_without_device_work():
    plan, ws = moe.moe_plan_create(_cfg())
    try:
        _fwd(plan, ws, num_tokens=0)
    finally:
        moe.moe_plan_destroy(plan)


def test_reader_validation():
    plan, ws = moe.moe_plan_create(_cfg())
    try:
        with pytest.raises(moe.MoEError):
            moe.moe_read_buffer(plan, FAKE, 0, 8, 8, 99, FAKE, 1 << 30)
        with pytest.raises(moe.MoEError):
            moe.moe_read_buffer(plan, FAKE, 0, 8, 8, moe.MOE_BUF_Y, FAKE, 16)
        with pytest.raises(moe.MoEError):
            moe.moe_read_routing(plan, FAKE, 0, 65, 8)
    finally:
        moe.moe_plan_destroy(plan)


# moe_rmsnorm: every case below is rejected (or is the rows == 0 no-op) before any
# device work, so fake, never dereferenced addresses are enough.
_X, _W, _O = 0x100000, 0x200000, 0x300000


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), moe.MOE_ERROR_NOT_SUPPORTED),
    (dict(rows=-1), moe.MOE_ERROR_INVALID_VALUE),
    (dict(width=0), moe.MOE_ERROR_INVALID_VALUE),
    (dict(width=100), moe.MOE_ERROR_INVALID_VALUE),            # bf16 rows need multiples of 8
    (dict(x_stride=64), moe.MOE_ERROR_INVALID_VALUE),          # stride below width
    (dict(out_stride=132), moe.MOE_ERROR_INVALID_VALUE),       # not a multiple of 8
    (dict(eps=0.0), moe.MOE_ERROR_INVALID_VALUE),
    (dict(eps=float("inf")), moe.MOE_ERROR_INVALID_VALUE),
    (dict(x=None), moe.MOE_ERROR_INVALID_VALUE),
    (dict(weight=None), moe.MOE_ERROR_INVALID_VALUE),
    (dict(out=_O + 2), moe.MOE_ERROR_MISALIGNED),
    (dict(out=_X + 16), moe.MOE_ERROR_INVALID_VALUE),          # overlaps x, not x itself
    (dict(out=_X, out_stride=136), moe.MOE_ERROR_INVALID_VALUE),  # in place needs equal strides
    (dict(rows=0, x=None, weight=None, out=None), moe.MOE_SUCCESS),
])
def test_rmsnorm_validation(kw, status):
    args = dict(dtype=moe.MOE_DTYPE_BF16, rows=4, width=128, eps=1e-6, x=_X, x_stride=128,
                weight=_W, out=_O, out_stride=128)
    args.update(kw)
    got = moe.load().moe_rmsnorm(0, args["dtype"], args["rows"], args["width"], args["eps"],
                                 args["x"], args["x_stride"], args["weight"], args["out"],
                                 args["out_stride"])
    assert got == status


def _dense_cfg(**kw):
    base = dict(dim=6144, max_tokens=64, n_experts=0, moe_inter=0, shared_inter=12288,
                max_top_k=0, dtype="bf16")
    base.update(kw)
    return moe.make_config(**base)


@pytest.mark.parametrize("kw", [dict(moe_inter=64), dict(max_top_k=1), dict(shared_inter=0),
                                dict(n_experts=-1)])
def test_dense_plan_validation(kw):
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_plan_create(_dense_cfg(**kw))
    assert ei.value.status == moe.MOE_ERROR_INVALID_VALUE


def test_dense_plan_entry_points_and_buffers():
    plan, ws = moe.moe_plan_create(_dense_cfg(max_tokens=4096))
    moe_plan, _ = moe.moe_plan_create(_cfg())
    lib = moe.load()
    try:
        assert ws >= 4096 * 12288 * 2  # the MLP activation in bf16
        assert moe.moe_plan_path(plan, 64, 0) == moe.MOE_PATH_MFMA
        assert moe.moe_buffer_bytes(plan, 10, 0, moe.MOE_BUF_H) == 10 * 6144 * 2
        assert moe.moe_buffer_bytes(plan, 10, 0, moe.MOE_BUF_SHARED_ACT) == 10 * 12288 * 2
        assert moe.moe_buffer_bytes(plan, 10, 1, moe.MOE_BUF_H) == 0
        assert moe.moe_buffer_bytes(plan, 10, 0, moe.MOE_BUF_Y) == 0
        X = 0x100000
        # wrong plan kind, either way round
        assert lib.moe_block_forward(plan, X, ws, 0, 4, X, X, X, X, X, X, X, X, X, 1, 1.0, X) == \
            moe.MOE_ERROR_NOT_SUPPORTED
        assert lib.moe_dense_block_forward(moe_plan, X, ws, 0, 4, X, X, X, X, X, X) == \
            moe.MOE_ERROR_NOT_SUPPORTED
        assert lib.moe_read_routing(plan, X, 0, 4, 1, X, X, X) == moe.MOE_ERROR_NOT_SUPPORTED
        # argument checks before any device work
        assert lib.moe_dense_block_forward(plan, X, ws, 0, 4097, X, X, X, X, X, X) == \
            moe.MOE_ERROR_INVALID_VALUE
        assert lib.moe_dense_block_forward(plan, X, ws, 0, 4, X, X, None, X, X, X) == \
            moe.MOE_ERROR_INVALID_VALUE
        assert lib.moe_dense_block_forward(plan, X, ws, 0, 4, X, X, X, X + 8, X, X) == \
            moe.MOE_ERROR_MISALIGNED
        assert lib.moe_dense_block_forward(plan, X, ws - 1, 0, 4, X, X, X, X, X, X) == \
            moe.MOE_ERROR_WORKSPACE_TOO_SMALL
        assert lib.moe_dense_block_forward(plan, None, 0, 0, 0, None, None, None, None, None,
                                           None) == moe.MOE_SUCCESS
        assert lib.moe_read_buffer(plan, X, 0, 4, 0, moe.MOE_BUF_Y, X, 1 << 20) == \
            moe.MOE_ERROR_INVALID_VALUE
    finally:
        moe.moe_plan_destroy(plan)
        moe.moe_plan_destroy(moe_plan)


@pytest.mark.parametrize("args,status", [
    (dict(dtype=5), moe.MOE_ERROR_NOT_SUPPORTED),
    (dict(dim=100), moe.MOE_ERROR_NOT_SUPPORTED),
    (dict(inter=0), moe.MOE_ERROR_INVALID_VALUE),
    (dict(gate=None), moe.MOE_ERROR_INVALID_VALUE),
    (dict(gate=0x100008), moe.MOE_ERROR_MISALIGNED),
    (dict(gate_up=0x100000 + 4096), moe.MOE_ERROR_INVALID_VALUE),  # output overlaps input gate
    (dict(down_packed=0x600000 + 16), moe.MOE_ERROR_INVALID_VALUE),  # outputs overlap
])
def test_pack_validation(args, status):
    a = dict(dtype=moe.MOE_DTYPE_BF16, dim=256, inter=128, gate=0x100000, up=0x200000,
             down=0x300000, gate_up=0x600000, down_packed=0x700000)
    a.update(args)
    got = moe.load().moe_pack_expert(0, a["dtype"], a["dim"], a["inter"], a["gate"], a["up"],
                                     a["down"], a["gate_up"], a["down_packed"])
    assert got == status
    if "gate_up" not in args and "down_packed" not in args:
        # shape, dtype and pointer checks are the same in the inverse direction
        got = moe.load().moe_unpack_expert(0, a["dtype"], a["dim"], a["inter"], a["gate_up"],
                                           a["down_packed"], a["gate"], a["up"], a["down"])
        assert got == status


def test_unpack_rejects_outputs_overlapping_inputs():
    lib = moe.load()
    # output `up` inside the input gate_up
    assert lib.moe_unpack_expert(0, moe.MOE_DTYPE_BF16, 256, 128, 0x600000, 0x700000, 0x100000,
                                 0x600000 + 1024, 0x300000) == moe.MOE_ERROR_INVALID_VALUE


@pytest.mark.parametrize("kw", [
    dict(max_tokens=8), dict(max_tokens=16), dict(max_tokens=64), dict(max_tokens=300),
    dict(max_tokens=8, path=moe.MOE_PATH_MFMA),
    dict(dim=4096, n_experts=128, moe_inter=1408, shared_inter=1408, max_tokens=64),
    dict(dim=2048, moe_inter=1024, shared_inter=1024, max_tokens=40),
    dict(dtype="f32", dim=256, n_experts=8, moe_inter=128, shared_inter=128, max_top_k=2,
         max_tokens=100),
])
def test_split_partials_fit_every_token_count(kw):
    """The split-K partial sums of every call size up to max_tokens fit the regions the
    plan sized (the 64-row kernel's split count is not monotone in the row count, so a
    plan for 8 tokens called with 7 needs more partial sums than at 8)."""
    plan, _ = moe.moe_plan_create(_cfg(**kw))
    try:
        k = kw.get("max_top_k", 8)
        for T in range(0, kw["max_tokens"] + 1):
            # the path (and with it the shared expert's split) depends on T * top_k
            for kk in sorted({1, max(1, k // 2), k}):
                moe.moe_plan_check(plan, T, kk)
        with pytest.raises(moe.MoEError) as ei:
            moe.moe_plan_check(plan, kw["max_tokens"] + 1, k)
        assert ei.value.status == moe.MOE_ERROR_INVALID_VALUE
        with pytest.raises(moe.MoEError):
            moe.moe_plan_check(plan, 1, k + 1)
    finally:
        moe.moe_plan_destroy(plan)


@pytest.mark.parametrize("max_tokens", [8, 64, 513])
def test_dense_split_partials_fit_every_token_count(max_tokens):
    plan, _ = moe.moe_plan_create(_dense_cfg(max_tokens=max_tokens))
    try:
        for T in range(0, max_tokens + 1):
            moe.moe_plan_check(plan, T, 0)
        with pytest.raises(moe.MoEError):
            moe.moe_plan_check(plan, 4, 1)
    finally:
        moe.moe_plan_destroy(plan)


def test_static_entry_point_limit():
    """moe_block_forward_static takes the plans whose workspace fits its static buffer
    (the GLM-5 decode plan for 64 tokens does) and rejects larger ones before any
    device work."""
    lib = moe.load()
    plan, ws = moe.moe_plan_create(_cfg(max_tokens=64))
    try:
        assert ws <= moe.STATIC_WORKSPACE_BYTES
    finally:
        moe.moe_plan_destroy(plan)
    plan, ws = moe.moe_plan_create(_cfg(max_tokens=4096))
    try:
        assert ws > moe.STATIC_WORKSPACE_BYTES
        X = 0x100000
        assert lib.moe_block_forward_static(plan, 0, 8, X, X, X, X, X, X, X, X, X, 8, 2.5, X) == \
            moe.MOE_ERROR_WORKSPACE_TOO_SMALL
    finally:
        moe.moe_plan_destroy(plan)
    assert lib.moe_block_forward_static(None, 0, 8, X, X, X, X, X, X, X, X, X, 8, 2.5, X) == \
        moe.MOE_ERROR_INVALID_VALUE
