"""CPU oracle for the MoE feed-forward sublayer (RMSNorm -> router -> routed and
shared SwiGLU experts -> combine + residual).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this package.  It shares no code with
the GPU library (``mixture_experts_transformer_rmsnorm_amd``) and must never be
used as a fallback for it.

The arithmetic lives in ``moe_oracle.c`` (plain C loops, fp64 accumulation,
OpenMP over tokens / experts); this module only marshals NumPy arrays.  Each
wrapper names the step of the method it computes; the C file cites the page
passages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16 = 0, 1
DTYPES = {"f32": F32, "bf16": BF16}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no FP contraction, IEEE math)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            i64, i32, f32, f64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_double
            lib.oracle_round_to_dtype.argtypes = [i64, P, P, i32]
            lib.oracle_rmsnorm.argtypes = [i64, i32, i32, f32, P, P, P]
            lib.oracle_router_scores.argtypes = [i64, i32, i32, i32, P, P, P, P]
            lib.oracle_select.argtypes = [i64, i32, i32, P, P, f64, P, P, P]
            lib.oracle_counts.argtypes = [i64, i32, i32, P, P, P]
            lib.oracle_experts.argtypes = [i64, P, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P,
                                           P, P, P, P, P, P, P, P, P]
            lib.oracle_dense_mlp.argtypes = [i64, i32, i32, i32, P, P, P, P, P, P, P, P]
            lib.oracle_num_threads.argtypes = []
            lib.oracle_set_num_threads.argtypes = [i32]
            for fn in ("oracle_num_threads", "oracle_set_num_threads", "oracle_round_to_dtype", "oracle_rmsnorm", "oracle_router_scores",
                       "oracle_select", "oracle_counts", "oracle_experts", "oracle_dense_mlp"):
                getattr(lib, fn).restype = ctypes.c_int
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _storage(a, dtype):
    """Contiguous storage array for a D-typed tensor: float32, or uint16 bf16 bits."""
    if dtype == BF16:
        a = np.ascontiguousarray(a)
        if a.dtype != np.uint16:
            raise TypeError("bf16 tensors are passed to the oracle as uint16 bit patterns")
        return a
    return np.ascontiguousarray(a, dtype=np.float32)


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments (rc=%d)" % (what, rc))


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads for the oracle's next calls on this thread (timing only)."""
    _check(_load().oracle_set_num_threads(int(n)), "set_num_threads")


def round_to_dtype(a, dtype):
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty_like(a)
    _check(_load().oracle_round_to_dtype(a.size, _ptr(a), _ptr(out), dtype), "round")
    return out


def rmsnorm(x, w, dtype, eps=1e-6):
    """Step O1: RMSNorm of each row of x [T, d]; returns h as float32 holding D values."""
    x = _storage(x, dtype)
    w = _storage(w, dtype)
    T, d = x.shape
    h = np.empty((T, d), np.float32)
    _check(_load().oracle_rmsnorm(T, d, dtype, eps, _ptr(x), _ptr(w), _ptr(h)), "rmsnorm")
    return h


def router_scores(h, router_w, dtype):
    """Step O2: fp32 logits and sigmoid scores [T, E]."""
    h = np.ascontiguousarray(h, np.float32)
    rw = _storage(router_w, dtype)
    T, d = h.shape
    E = rw.shape[0]
    logits = np.empty((T, E), np.float32)
    scores = np.empty((T, E), np.float32)
    _check(_load().oracle_router_scores(T, d, E, dtype, _ptr(h), _ptr(rw), _ptr(logits),
                                        _ptr(scores)), "router_scores")
    return logits, scores


def select(scores, corr_bias, k, routed_scale):
    """Steps O3-O4: top-k indices (key desc, index asc), fp64 weights, selection margin."""
    scores = np.ascontiguousarray(scores, np.float32)
    bias = np.ascontiguousarray(corr_bias, np.float32)
    T, E = scores.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    margin = np.empty((T,), np.float64)
    _check(_load().oracle_select(T, E, k, _ptr(scores), _ptr(bias), float(routed_scale),
                                 _ptr(idx), _ptr(w), _ptr(margin)), "select")
    return idx, w, margin


def counts(idx, E):
    """Step O5: per-expert counts and segment offsets."""
    idx = np.ascontiguousarray(idx, np.int32)
    T, k = idx.shape
    cnt = np.empty((E,), np.int32)
    off = np.empty((E + 1,), np.int64)
    _check(_load().oracle_counts(T, E, k, _ptr(idx), _ptr(cnt), _ptr(off)), "counts")
    return cnt, off


def experts(tokens, x, h, idx, w, gate_up, down, shared_gate, shared_up, shared_down, dtype,
            debug=False):
    """Steps O6-O8 for the listed tokens.

    gate_up / down: either full arrays [E, d, 2I] / [E, I, d] or lists of E per-expert
    arrays (entries for experts no listed token uses may be None).
    Returns (delta fp64 [n, d], out float32 [n, d] holding D values[, debug dict]).
    """
    tokens = np.ascontiguousarray(tokens, np.int64)
    x = _storage(x, dtype)
    h = np.ascontiguousarray(h, np.float32)
    idx = np.ascontiguousarray(idx, np.int32)
    w = np.ascontiguousarray(w, np.float64)
    T, d = x.shape
    k = idx.shape[1]
    E = len(gate_up)
    gu_list = [None if g is None else _storage(g, dtype) for g in gate_up]
    dn_list = [None if g is None else _storage(g, dtype) for g in down]
    I = next(g for g in dn_list if g is not None).shape[0]
    gu_ptrs = (ctypes.c_void_p * E)(*[None if g is None else g.ctypes.data for g in gu_list])
    dn_ptrs = (ctypes.c_void_p * E)(*[None if g is None else g.ctypes.data for g in dn_list])
    if shared_gate is not None:
        sg, su, sd = (_storage(a, dtype) for a in (shared_gate, shared_up, shared_down))
        Is = sg.shape[0]
    else:
        sg = su = sd = None
        Is = 0
    n = tokens.shape[0]
    delta = np.empty((n, d), np.float64)
    out = np.empty((n, d), np.float32)
    dbg = None
    if debug:
        dbg = dict(act=np.zeros((n, k, I)), y=np.zeros((n, k, d)),
                   act_s=np.zeros((n, max(Is, 1))), s=np.zeros((n, d)))
    rc = _load().oracle_experts(
        n, _ptr(tokens), d, E, I, Is, k, dtype, _ptr(x), _ptr(h), _ptr(idx), _ptr(w),
        ctypes.cast(gu_ptrs, ctypes.c_void_p), ctypes.cast(dn_ptrs, ctypes.c_void_p),
        _ptr(sg), _ptr(su), _ptr(sd), _ptr(delta), _ptr(out),
        _ptr(dbg["act"]) if dbg else None, _ptr(dbg["y"]) if dbg else None,
        _ptr(dbg["act_s"]) if dbg else None, _ptr(dbg["s"]) if dbg else None)
    _check(rc, "experts")
    if debug:
        return delta, out, dbg
    return delta, out


def route(x, norm_w, router_w, corr_bias, k, routed_scale, dtype, eps=1e-6):
    """Steps O1-O4 on every token: returns dict(h, logits, scores, idx, w, margin)."""
    h = rmsnorm(x, norm_w, dtype, eps)
    logits, scores = router_scores(h, router_w, dtype)
    idx, w, margin = select(scores, corr_bias, k, routed_scale)
    return dict(h=h, logits=logits, scores=scores, idx=idx, w=w, margin=margin)


def forward(inp, tokens=None, debug=False):
    """Whole sublayer (O1-O8) on a dict of host arrays as produced by ``workloads``.

    ``tokens``: optional subset of token rows to evaluate through the experts
    (routing is always computed for every token).
    """
    dt = DTYPES[inp["dtype"]]
    r = route(inp["x"], inp["norm_w"], inp["router_w"], inp["corr_bias"], inp["top_k"],
              inp["routed_scale"], dt, inp.get("eps", 1e-6))
    T = r["idx"].shape[0]
    if tokens is None:
        tokens = np.arange(T, dtype=np.int64)
    res = experts(tokens, inp["x"], r["h"], r["idx"], r["w"], inp["gate_up"], inp["down"],
                  inp.get("shared_gate"), inp.get("shared_up"), inp.get("shared_down"), dt,
                  debug=debug)
    r["tokens"] = np.asarray(tokens, np.int64)
    if debug:
        r["delta"], r["out"], r["debug"] = res
    else:
        r["delta"], r["out"] = res
    r["counts"], r["offsets"] = counts(r["idx"], len(inp["gate_up"]))
    return r


def dense_mlp(x, h, gate, up, down, dtype, debug=False):
    """Step O9: dense SwiGLU MLP block on h (the RMSNorm of x): returns (delta fp64 [T, d],
    out [T, d] float32 holding D values[, act fp64 [T, Id]])."""
    x = _storage(x, dtype)
    h = np.ascontiguousarray(h, np.float32)
    gate, up, down = (_storage(a, dtype) for a in (gate, up, down))
    T, d = x.shape
    Id = gate.shape[0]
    if gate.shape != (Id, d) or up.shape != (Id, d) or down.shape != (d, Id) or h.shape != (T, d):
        raise ValueError("dense_mlp: shapes x %s h %s gate %s up %s down %s" % (
            x.shape, h.shape, gate.shape, up.shape, down.shape))
    delta = np.empty((T, d), np.float64)
    out = np.empty((T, d), np.float32)
    act = np.empty((T, Id), np.float64) if debug else None
    _check(_load().oracle_dense_mlp(T, d, Id, dtype, _ptr(x), _ptr(h), _ptr(gate), _ptr(up),
                                    _ptr(down), _ptr(delta), _ptr(out), _ptr(act)), "dense_mlp")
    return (delta, out, act) if debug else (delta, out)


def dense_block(x, norm_w, gate, up, down, dtype, eps=1e-6, debug=False):
    """Steps O1 + O9: out = x + mlp(rmsnorm(x)) for a dense block; returns a dict with
    h, delta, out (and act when debug)."""
    h = rmsnorm(x, norm_w, dtype, eps)
    r = dense_mlp(x, h, gate, up, down, dtype, debug)
    res = dict(h=h, delta=r[0], out=r[1])
    if debug:
        res["act"] = r[2]
    return res


def pack_expert(gate, up, down):
    """Step O10: one expert's weights from the HF checkpoint layout (nn.Linear [out, in]:
    gate_proj.weight [I, d], up_proj.weight [I, d], down_proj.weight [d, I]) to the grouped
    native layout of class Glm4MoeStateDictAdapter (page
    "nemo_automodel.components.models.glm4_moe.state_dict_adapter"): its slice of
    gate_and_up_projs [d, 2I] (gate columns first, then up) and of down_projs [I, d].  Storage arrays of any dtype; the
    result holds the same elements, moved."""
    gate, up, down = (np.asarray(a) for a in (gate, up, down))
    I, d = gate.shape
    if up.shape != (I, d) or down.shape != (d, I):
        raise ValueError("pack_expert: gate %s up %s down %s" % (gate.shape, up.shape, down.shape))
    gate_up = np.ascontiguousarray(np.concatenate([gate.T, up.T], axis=1))
    return gate_up, np.ascontiguousarray(down.T)


def unpack_expert(gate_up, down):
    """Inverse of pack_expert: ([d, 2I], [I, d]) -> (gate [I, d], up [I, d], down [d, I])."""
    gate_up, down = np.asarray(gate_up), np.asarray(down)
    d, I2 = gate_up.shape
    I = I2 // 2
    if I2 != 2 * I or down.shape != (I, d):
        raise ValueError("unpack_expert: gate_up %s down %s" % (gate_up.shape, down.shape))
    return (np.ascontiguousarray(gate_up[:, :I].T), np.ascontiguousarray(gate_up[:, I:].T),
            np.ascontiguousarray(down.T))
