"""MI355X (gfx950) MoE feed-forward sublayer: thin Python binding of ``include/moe.h``.

Every step of the sublayer runs in the HIP kernels of ``libmoe_mi355x.so``; this
module only marshals arguments (device pointers from torch tensors, the current
HIP stream) and turns status codes into exceptions.  There is no fallback: if the
library is missing, ``load()`` raises.

Functions keep the C names: ``moe_plan_create``, ``moe_plan_destroy``,
``moe_block_forward``, ``moe_read_routing``, ``moe_read_buffer``,
``moe_buffer_bytes``, ``moe_plan_path``, ``moe_set_stage_timing``,
``moe_stage_times``, ``moe_stage_name``, ``moe_status_string``,
``moe_abi_version``.  ``MoEBlock`` bundles a plan, its workspace and the weights.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_SUCCESS = 0
MOE_ERROR_INVALID_VALUE = 1
MOE_ERROR_NOT_SUPPORTED = 2
MOE_ERROR_WORKSPACE_TOO_SMALL = 3
MOE_ERROR_MISALIGNED = 4
MOE_ERROR_HIP = 5
MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
MOE_PATH_AUTO, MOE_PATH_STREAM, MOE_PATH_MFMA, MOE_PATH_FUSED = 0, 1, 2, 3
(MOE_BUF_H, MOE_BUF_OFFSETS, MOE_BUF_PERM_TOKEN, MOE_BUF_ROW_OF, MOE_BUF_ACT, MOE_BUF_Y,
 MOE_BUF_SHARED_ACT, MOE_BUF_FUSED_ERROR) = range(8)
MOE_MAX_STAGES = 16
ABI_VERSION = 1

EXPORTS = ("moe_plan_create", "moe_plan_destroy", "moe_block_forward", "moe_read_routing",
           "moe_read_buffer", "moe_buffer_bytes", "moe_plan_path", "moe_set_stage_timing",
           "moe_stage_times", "moe_stage_name", "moe_status_string", "moe_abi_version",
           "moe_rmsnorm", "moe_dense_block_forward", "moe_pack_expert", "moe_unpack_expert",
           "moe_plan_check", "moe_block_forward_static", "moe_calib_hbm_read",
           "moe_calib_mfma")
STATIC_WORKSPACE_BYTES = 128 << 20


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__("%s: %s (status %d)" % (what or "moe", moe_status_string(status), status))


class moe_config_t(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dim", ctypes.c_int32),
                ("max_tokens", ctypes.c_int64), ("n_experts", ctypes.c_int32),
                ("moe_inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
                ("max_top_k", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("path", ctypes.c_int32), ("eps", ctypes.c_float), ("flags", ctypes.c_uint32)]


_lib = None
_lock = threading.Lock()


def load(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise ImportError("libmoe_mi355x.so not found at %s; build it with "
                              "mixture_experts_transformer_rmsnorm_amd/build.py" % path)
        # torch ships its own HIP runtime under the same soname; loading torch first
        # makes the library bind to that one, so both share one runtime (streams,
        # device pointers).  Loading the library first would bring in a second copy.
        import torch  # noqa: F401
        lib = ctypes.CDLL(path)
        P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        lib.moe_plan_create.argtypes = [ctypes.POINTER(moe_config_t), ctypes.POINTER(P),
                                        ctypes.POINTER(ctypes.c_size_t)]
        lib.moe_plan_destroy.argtypes = [P]
        lib.moe_block_forward.argtypes = [P, P, ctypes.c_size_t, P, i64, P, P, P, P, P, P, P, P, P,
                                          i32, ctypes.c_float, P]
        lib.moe_block_forward_static.argtypes = [P, P, i64, P, P, P, P, P, P, P, P, P, i32,
                                                 ctypes.c_float, P]
        lib.moe_calib_hbm_read.argtypes = [P, P, ctypes.c_size_t, i32, P]
        lib.moe_calib_mfma.argtypes = [P, i32, i32, P, ctypes.POINTER(ctypes.c_double)]
        lib.moe_read_routing.argtypes = [P, P, P, i64, i32, P, P, P]
        lib.moe_read_buffer.argtypes = [P, P, P, i64, i32, i32, P, ctypes.c_size_t]
        lib.moe_buffer_bytes.argtypes = [P, i64, i32, i32]
        lib.moe_buffer_bytes.restype = ctypes.c_size_t
        lib.moe_plan_check.argtypes = [P, i64, i32]
        lib.moe_plan_path.argtypes = [P, i64, i32]
        lib.moe_plan_path.restype = i32
        lib.moe_set_stage_timing.argtypes = [P, i32]
        lib.moe_stage_times.argtypes = [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
        lib.moe_stage_name.argtypes = [i32]
        lib.moe_stage_name.restype = ctypes.c_char_p
        lib.moe_status_string.argtypes = [i32]
        lib.moe_status_string.restype = ctypes.c_char_p
        lib.moe_rmsnorm.argtypes = [P, i32, i64, i32, ctypes.c_float, P, i64, P, P, i64]
        lib.moe_dense_block_forward.argtypes = [P, P, ctypes.c_size_t, P, i64, P, P, P, P, P, P]
        lib.moe_pack_expert.argtypes = [P, i32, i32, i32, P, P, P, P, P]
        lib.moe_unpack_expert.argtypes = [P, i32, i32, i32, P, P, P, P, P]
        lib.moe_abi_version.argtypes = []
        lib.moe_abi_version.restype = i32
        for fn in ("moe_plan_create", "moe_plan_destroy", "moe_block_forward", "moe_read_routing",
                   "moe_read_buffer", "moe_set_stage_timing", "moe_stage_times", "moe_rmsnorm",
                   "moe_dense_block_forward", "moe_pack_expert", "moe_unpack_expert",
                   "moe_plan_check", "moe_block_forward_static", "moe_calib_hbm_read",
           "moe_calib_mfma"):
            getattr(lib, fn).restype = i32
        if lib.moe_abi_version() != ABI_VERSION:
            raise ImportError("libmoe_mi355x.so ABI %d != binding ABI %d"
                              % (lib.moe_abi_version(), ABI_VERSION))
        _lib = lib
        return lib


def _ptr(t):
    """Device pointer of a tensor (or an int / None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, what):
    if status != MOE_SUCCESS:
        raise MoEError(status, what)


# ----------------------------------------------------------------------------- C names
def moe_status_string(status: int) -> str:
    s = load().moe_status_string(status)
    return s.decode() if s else "unknown status"


def moe_abi_version() -> int:
    return load().moe_abi_version()


def moe_stage_name(stage: int):
    s = load().moe_stage_name(stage)
    return s.decode() if s else None


def make_config(dim, max_tokens, n_experts, moe_inter, shared_inter, max_top_k, dtype="bf16",
                path=MOE_PATH_AUTO, eps=1e-6, flags=0) -> moe_config_t:
    dt = {"f32": MOE_DTYPE_F32, "bf16": MOE_DTYPE_BF16}.get(dtype, dtype)
    return moe_config_t(ctypes.sizeof(moe_config_t), dim, max_tokens, n_experts, moe_inter,
                        shared_inter, max_top_k, dt, path, eps, flags)


def moe_plan_create(cfg: moe_config_t):
    """Returns (plan handle, workspace bytes)."""
    plan = ctypes.c_void_p()
    ws = ctypes.c_size_t()
    _check(load().moe_plan_create(ctypes.byref(cfg), ctypes.byref(plan), ctypes.byref(ws)),
           "moe_plan_create")
    return plan.value, ws.value


def moe_plan_destroy(plan) -> None:
    _check(load().moe_plan_destroy(plan), "moe_plan_destroy")


def moe_block_forward(plan, workspace, workspace_bytes, stream, num_tokens, x, norm_w, router_w,
                      corr_bias, gate_up, down, shared_gate, shared_up, shared_down, top_k,
                      routed_scale, out) -> None:
    _check(load().moe_block_forward(
        plan, _ptr(workspace), workspace_bytes, _stream(stream), num_tokens, _ptr(x),
        _ptr(norm_w), _ptr(router_w), _ptr(corr_bias), _ptr(gate_up), _ptr(down),
        _ptr(shared_gate), _ptr(shared_up), _ptr(shared_down), top_k, routed_scale, _ptr(out)),
        "moe_block_forward")


def moe_block_forward_static(plan, stream, num_tokens, x, norm_w, router_w, corr_bias, gate_up,
                             down, shared_gate, shared_up, shared_down, top_k, routed_scale,
                             out) -> None:
    _check(load().moe_block_forward_static(
        plan, _stream(stream), num_tokens, _ptr(x), _ptr(norm_w), _ptr(router_w), _ptr(corr_bias),
        _ptr(gate_up), _ptr(down), _ptr(shared_gate), _ptr(shared_up), _ptr(shared_down), top_k,
        routed_scale, _ptr(out)), "moe_block_forward_static")


def moe_calib_hbm_read(stream, src, nbytes, blocks, sink) -> None:
    _check(load().moe_calib_hbm_read(_stream(stream), _ptr(src), nbytes, blocks, _ptr(sink)),
           "moe_calib_hbm_read")


def moe_calib_mfma(stream, iters, blocks, sink) -> float:
    """Enqueues the MFMA loop; returns the FLOPs it performs."""
    flops = ctypes.c_double()
    _check(load().moe_calib_mfma(_stream(stream), iters, blocks, _ptr(sink), ctypes.byref(flops)),
           "moe_calib_mfma")
    return flops.value


def moe_rmsnorm(stream, dtype, rows, width, eps, x, x_stride, weight, out, out_stride) -> None:
    _check(load().moe_rmsnorm(_stream(stream), dtype, rows, width, eps, _ptr(x), x_stride,
                              _ptr(weight), _ptr(out), out_stride), "moe_rmsnorm")


def rmsnorm(x, weight, eps=1e-6, out=None, stream=None):
    """RMSNorm over the last dimension of x ([..., width] or a 2-D view whose rows
    are strided, e.g. the leading columns of wider rows); returns out (new, or the
    given tensor, which may be x itself)."""
    import torch
    width = x.shape[-1]
    x2 = x.reshape(-1, width) if x.dim() != 2 else x
    if x2.stride(-1) != 1:
        raise ValueError("rmsnorm: the last dimension must be contiguous")
    if out is None:
        out = torch.empty(x.shape, dtype=x.dtype, device=x.device)
    o2 = out.reshape(-1, width) if out.dim() != 2 else out
    if o2.stride(-1) != 1 or o2.shape != x2.shape:
        raise ValueError("rmsnorm: out must match x with a contiguous last dimension")
    dt = {torch.bfloat16: MOE_DTYPE_BF16, torch.float32: MOE_DTYPE_F32}[x.dtype]
    moe_rmsnorm(stream, dt, x2.shape[0], width, eps, x2, x2.stride(0) if x2.shape[0] > 1 else width,
                weight, o2, o2.stride(0) if o2.shape[0] > 1 else width)
    return out


def moe_dense_block_forward(plan, workspace, workspace_bytes, stream, num_tokens, x, norm_w, gate,
                            up, down, out) -> None:
    _check(load().moe_dense_block_forward(plan, _ptr(workspace), workspace_bytes, _stream(stream),
                                          num_tokens, _ptr(x), _ptr(norm_w), _ptr(gate), _ptr(up),
                                          _ptr(down), _ptr(out)), "moe_dense_block_forward")


def moe_pack_expert(stream, dtype, dim, inter, gate, up, down, gate_up, down_packed) -> None:
    _check(load().moe_pack_expert(_stream(stream), dtype, dim, inter, _ptr(gate), _ptr(up),
                                  _ptr(down), _ptr(gate_up), _ptr(down_packed)), "moe_pack_expert")


def moe_unpack_expert(stream, dtype, dim, inter, gate_up, down_packed, gate, up, down) -> None:
    _check(load().moe_unpack_expert(_stream(stream), dtype, dim, inter, _ptr(gate_up),
                                    _ptr(down_packed), _ptr(gate), _ptr(up), _ptr(down)),
           "moe_unpack_expert")


def pack_experts(gates, ups, downs, gate_up=None, down=None, stream=None):
    """HF per-expert weights (sequences of torch tensors: gate/up [I, d], down [d, I]) ->
    grouped gate_and_up [E, d, 2I] and down [E, I, d] (allocated unless given)."""
    import torch
    E = len(gates)
    I, d = gates[0].shape
    dt = {torch.bfloat16: MOE_DTYPE_BF16, torch.float32: MOE_DTYPE_F32}[gates[0].dtype]
    if gate_up is None:
        gate_up = torch.empty((E, d, 2 * I), dtype=gates[0].dtype, device=gates[0].device)
    if down is None:
        down = torch.empty((E, I, d), dtype=gates[0].dtype, device=gates[0].device)
    for e in range(E):
        moe_pack_expert(stream, dt, d, I, gates[e], ups[e], downs[e], gate_up[e], down[e])
    return gate_up, down


def moe_read_routing(plan, workspace, stream, num_tokens, top_k, topk_idx=None, topk_w=None,
                     counts=None) -> None:
    _check(load().moe_read_routing(plan, _ptr(workspace), _stream(stream), num_tokens, top_k,
                                   _ptr(topk_idx), _ptr(topk_w), _ptr(counts)),
           "moe_read_routing")


def moe_buffer_bytes(plan, num_tokens, top_k, which) -> int:
    return load().moe_buffer_bytes(plan, num_tokens, top_k, which)


def moe_read_buffer(plan, workspace, stream, num_tokens, top_k, which, dst, dst_bytes) -> None:
    _check(load().moe_read_buffer(plan, _ptr(workspace), _stream(stream), num_tokens, top_k,
                                  which, _ptr(dst), dst_bytes), "moe_read_buffer")


def moe_plan_check(plan, num_tokens, top_k) -> None:
    """Raises MoEError unless a forward call with these sizes fits the plan."""
    _check(load().moe_plan_check(plan, num_tokens, top_k), "moe_plan_check")


def moe_plan_path(plan, num_tokens, top_k) -> int:
    return load().moe_plan_path(plan, num_tokens, top_k)


def moe_set_stage_timing(plan, stage_mask: int) -> None:
    """Time the stages whose bit is set in stage_mask (0 disables)."""
    _check(load().moe_set_stage_timing(plan, int(stage_mask)), "moe_set_stage_timing")


def stage_mask(*names) -> int:
    """Bit mask of the named stages (all stages when no name is given)."""
    mask = 0
    for i in range(MOE_MAX_STAGES):
        n = moe_stage_name(i)
        if n is not None and (not names or n in names):
            mask |= 1 << i
    return mask


def moe_stage_times(plan):
    """Returns ({stage name: total ms}, calls) accumulated since the last read."""
    ms = (ctypes.c_double * MOE_MAX_STAGES)()
    calls = ctypes.c_int64()
    _check(load().moe_stage_times(plan, ms, ctypes.byref(calls)), "moe_stage_times")
    out = {}
    for i in range(MOE_MAX_STAGES):
        name = moe_stage_name(i)
        if name is not None:
            out[name] = ms[i]
    return out, calls.value


# ----------------------------------------------------------------------------- convenience
def _io_tensors(x, out, dim, dtype, device):
    """x as [T, dim] and out (new, or the caller's) checked against the plan: both
    contiguous, of the plan's dtype, on the workspace's device, of the same shape."""
    import torch
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    if x.shape[-1] != dim:
        raise ValueError("x: last dimension %d, the plan's is %d" % (x.shape[-1], dim))
    if x.dtype != tdt or x.device != device:
        raise ValueError("x: %s on %s, the plan needs %s on %s" % (x.dtype, x.device, tdt, device))
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    x2 = x.reshape(-1, dim)
    if out is None:
        return x2, torch.empty_like(x2)
    if out.dtype != tdt or out.device != device or not out.is_contiguous() or \
            out.numel() != x2.numel():
        raise ValueError("out must be a contiguous %s tensor on %s with x's %d elements" % (
            tdt, device, x2.numel()))
    return x2, out


def _check_weights(weights, shapes, dtype, device):
    """Every named weight present, contiguous, of its shape, dtype and device."""
    import torch
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    for name, shape in shapes.items():
        t = weights.get(name)
        want_dt = torch.float32 if name == "corr_bias" else tdt
        if t is None or tuple(t.shape) != tuple(shape) or t.dtype != want_dt or \
                t.device != device or not t.is_contiguous():
            raise ValueError("weight %s: need a contiguous %s tensor of shape %s on %s, got %s" % (
                name, want_dt, tuple(shape), device,
                None if t is None else "%s %s on %s" % (t.dtype, tuple(t.shape), t.device)))


class MoEBlock:
    """A plan, its device workspace and the sublayer's weights (torch tensors).

    weights: dict with norm_w, router_w, corr_bias, gate_up, down and, when
    shared_inter > 0, shared_gate, shared_up, shared_down, in the layouts of
    ``include/moe.h``.
    """

    def __init__(self, weights: dict, max_tokens: int, top_k: int, routed_scale: float,
                 eps: float = 1e-6, path: int = MOE_PATH_AUTO, device=None):
        import torch
        gu = weights["gate_up"]
        E, d, I2 = gu.shape
        sg = weights.get("shared_gate")
        Is = 0 if sg is None else sg.shape[0]
        self.dtype = {torch.bfloat16: "bf16", torch.float32: "f32"}[gu.dtype]
        self.weights = weights
        self.top_k, self.routed_scale = top_k, routed_scale
        self.dim, self.n_experts, self.moe_inter, self.shared_inter = d, E, I2 // 2, Is
        shapes = {"norm_w": (d,), "router_w": (E, d), "corr_bias": (E,), "gate_up": (E, d, I2),
                  "down": (E, I2 // 2, d)}
        if Is:
            shapes.update(shared_gate=(Is, d), shared_up=(Is, d), shared_down=(d, Is))
        _check_weights(weights, shapes, self.dtype, gu.device)
        self.cfg = make_config(d, max_tokens, E, I2 // 2, Is, top_k, self.dtype, path, eps)
        self.plan, self.workspace_bytes = moe_plan_create(self.cfg)
        self.workspace = torch.empty(max(self.workspace_bytes, 1), dtype=torch.uint8,
                                     device=device or gu.device)

    def close(self):
        if self.plan:
            moe_plan_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def forward(self, x, out=None, stream=None):
        """x: [..., d] tensor; returns out of the same shape (may be x itself)."""
        shape = x.shape
        x2, out = _io_tensors(x, out, self.dim, self.dtype, self.workspace.device)
        w = self.weights
        moe_block_forward(self.plan, self.workspace, self.workspace_bytes, stream, x2.shape[0], x2,
                          w["norm_w"], w["router_w"], w["corr_bias"], w["gate_up"], w["down"],
                          w.get("shared_gate"), w.get("shared_up"), w.get("shared_down"),
                          self.top_k, self.routed_scale, out)
        return out.reshape(shape)

    __call__ = forward

    def routing(self, num_tokens, stream=None):
        """(topk_idx int32 [T, k], topk_w fp32 [T, k], counts int32 [E]) of the last call."""
        import torch
        dev = self.workspace.device
        idx = torch.empty((num_tokens, self.top_k), dtype=torch.int32, device=dev)
        wts = torch.empty((num_tokens, self.top_k), dtype=torch.float32, device=dev)
        cnt = torch.empty((self.n_experts,), dtype=torch.int32, device=dev)
        moe_read_routing(self.plan, self.workspace, stream, num_tokens, self.top_k, idx, wts, cnt)
        return idx, wts, cnt

    def fused_error(self, num_tokens, stream=None) -> int:
        """The fused decode kernel's error word of the last call (0 = every wait completed)."""
        import numpy as np
        return int(self.buffer(MOE_BUF_FUSED_ERROR, num_tokens, stream).cpu().numpy().view(np.uint32)[0])

    def buffer(self, which, num_tokens, stream=None):
        """Intermediate buffer `which` (MOE_BUF_*) of the last call as a flat uint8 tensor."""
        import torch
        n = moe_buffer_bytes(self.plan, num_tokens, self.top_k, which)
        dst = torch.empty(max(n, 1), dtype=torch.uint8, device=self.workspace.device)
        moe_read_buffer(self.plan, self.workspace, stream, num_tokens, self.top_k, which, dst, n)
        return dst[:n]


class DenseBlock:
    """A dense block (RMSNorm + SwiGLU MLP + residual): a dense-block plan, its device
    workspace and the weights (torch tensors): norm_w [d], gate [Id, d], up [Id, d],
    down [d, Id], as in ``include/moe.h``."""

    def __init__(self, weights: dict, max_tokens: int, eps: float = 1e-6, device=None):
        import torch
        g = weights["gate"]
        Id, d = g.shape
        self.dtype = {torch.bfloat16: "bf16", torch.float32: "f32"}[g.dtype]
        self.weights = weights
        self.dim, self.width = d, Id
        _check_weights(weights, {"norm_w": (d,), "gate": (Id, d), "up": (Id, d), "down": (d, Id)},
                       self.dtype, g.device)
        self.cfg = make_config(d, max_tokens, 0, 0, Id, 0, self.dtype, MOE_PATH_AUTO, eps)
        self.plan, self.workspace_bytes = moe_plan_create(self.cfg)
        self.workspace = torch.empty(max(self.workspace_bytes, 1), dtype=torch.uint8,
                                     device=device or g.device)

    def close(self):
        if self.plan:
            moe_plan_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def forward(self, x, out=None, stream=None):
        """x: [..., d] tensor; returns out of the same shape (may be x itself)."""
        shape = x.shape
        x2, out = _io_tensors(x, out, self.dim, self.dtype, self.workspace.device)
        w = self.weights
        moe_dense_block_forward(self.plan, self.workspace, self.workspace_bytes, stream, x2.shape[0],
                                x2, w["norm_w"], w["gate"], w["up"], w["down"], out)
        return out.reshape(shape)

    __call__ = forward

    def buffer(self, which, num_tokens, stream=None):
        """MOE_BUF_H or MOE_BUF_SHARED_ACT of the last call as a flat uint8 tensor."""
        import torch
        n = moe_buffer_bytes(self.plan, num_tokens, 0, which)
        dst = torch.empty(max(n, 1), dtype=torch.uint8, device=self.workspace.device)
        moe_read_buffer(self.plan, self.workspace, stream, num_tokens, 0, which, dst, n)
        return dst[:n]
