"""Seeded synthetic workloads for the MoE feed-forward sublayer.

This module only draws random inputs; it holds none of the method's arithmetic.
It serves both the GPU library's tests / benchmark and the CPU oracle.

Shapes follow the GLM-5 MoE block (hidden size 6144, 256 routed experts with
moe_inter 2048, one shared expert of the same width; "GLM-5 · MoE transformer
block", Parameters table) in the grouped-experts layout that page
"nemo_automodel.components.models.glm4_moe.state_dict_adapter" documents for class
Glm4MoeStateDictAdapter (gate_and_up_projs [E, d, 2I], down_projs [E, I, d];
shared expert as nn.Linear [out, in] weights).

Random streams: NumPy ``Generator(PCG64)`` seeded by ``SeedSequence(seed,
spawn_key=(tensor_id, ...))``.  Tensor ids: x 0, norm_w 1, router_w 2,
corr_bias 3, gate_up 4, down 5, shared_gate 6, shared_up 7, shared_down 8,
zipf rank permutation 9, row redraws 10; standalone RMSNorm inputs 11 (x), 12
(per-feature scales), 13 (gain); dense MLP weights 14 (gate), 15 (up), 16 (down).  Values are drawn in fp32 and rounded
to bfloat16 (round to nearest even) for bf16 workloads.

Expert weights of the GLM-5-sized workloads (19.4 GB in bf16) can instead be
drawn directly in device memory with torch's generator, seeded per
(tensor id, expert) from the same SeedSequence; consumers that need them on the
host copy them back.
"""
from __future__ import annotations

import dataclasses
import math
import os
from typing import Optional

import numpy as np

TID_X, TID_NORM, TID_ROUTER, TID_BIAS, TID_GATE_UP, TID_DOWN = 0, 1, 2, 3, 4, 5
TID_SH_GATE, TID_SH_UP, TID_SH_DOWN, TID_ZIPF, TID_REDRAW = 6, 7, 8, 9, 10
TID_NORM_X, TID_NORM_SCALE, TID_NORM_GAIN = 11, 12, 13
TID_DENSE_GATE, TID_DENSE_UP, TID_DENSE_DOWN = 14, 15, 16

# Strength of the Zipf-shaped correction bias of the skewed workload.  Written by
# tests/golden/calibrate_zipf.py (output tests/golden/zipf_beta.json): the value
# for which the fitted log-log slope of expert load against load rank, over
# ranks 2..128, is -1.1 on the seed-0 inputs.
ZIPF_BETA = 0.0615


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int            # tokens (batch x positions, flattened)
    d: int            # hidden size
    E: int            # routed experts
    I: int            # moe_inter (routed expert width)
    Is: int           # shared expert width (0: none)
    k: int            # experts per token
    dtype: str        # "f32" | "bf16"
    routed_scale: float
    eps: float = 1e-6
    routing: str = "balanced"   # "balanced" | "zipf"
    zipf_s: float = 1.1

    @property
    def A(self) -> int:
        return self.T * self.k


CONFIGS = {
    # Tiny fp32 block: the oracle finishes in well under a second.
    "tiny_fp32": MoEConfig("tiny_fp32", T=64, d=256, E=8, I=128, Is=128, k=2, dtype="f32",
                           routed_scale=1.0),
    # GLM-5 shape, decode batch: 64 sequences x 1 new position.
    "glm5_decode": MoEConfig("glm5_decode", T=64, d=6144, E=256, I=2048, Is=2048, k=8,
                             dtype="bf16", routed_scale=2.5),
    # GLM-5 shape, prefill of 4096 positions, balanced routing.
    "glm5_prefill": MoEConfig("glm5_prefill", T=4096, d=6144, E=256, I=2048, Is=2048, k=8,
                              dtype="bf16", routed_scale=2.5),
    # GLM-5 shape, prefill of 16384 positions with Zipf(1.1)-skewed expert popularity.
    "glm5_prefill_zipf": MoEConfig("glm5_prefill_zipf", T=16384, d=6144, E=256, I=2048,
                                   Is=2048, k=8, dtype="bf16", routed_scale=2.5,
                                   routing="zipf"),
    # Mid-size block with a non-power-of-two expert width (1408 = 11 x 128).
    "mid_prefill": MoEConfig("mid_prefill", T=8192, d=4096, E=128, I=1408, Is=1408, k=8,
                             dtype="bf16", routed_scale=1.0),
}


def config(name_or_cfg, **overrides) -> MoEConfig:
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    if overrides:
        cfg = dataclasses.replace(cfg, **overrides)
    return cfg


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def _torch_seed(seed: int, *key: int) -> int:
    s = np.random.SeedSequence(seed, spawn_key=key).generate_state(2, np.uint32)
    return int(s[0]) | (int(s[1] & 0x7FFFFFFF) << 32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a) if dtype == "bf16" else np.ascontiguousarray(a, np.float32)


def zipf_ranks(cfg: MoEConfig, seed: int) -> np.ndarray:
    """Popularity rank (1 = hottest) of each expert for the skewed workload."""
    return _rng(seed, TID_ZIPF).permutation(cfg.E).astype(np.int64) + 1


def draw_small(cfg: MoEConfig, seed: int = 0, zipf_beta: Optional[float] = None) -> dict:
    """x, norm_w, router_w (storage dtype) and corr_bias (fp32) as host arrays."""
    x = _rng(seed, TID_X).standard_normal((cfg.T, cfg.d), dtype=np.float32)
    norm_w = (1.0 + 0.1 * _rng(seed, TID_NORM).standard_normal(cfg.d)).astype(np.float32)
    router_w = (0.02 * _rng(seed, TID_ROUTER).standard_normal((cfg.E, cfg.d))).astype(np.float32)
    bias = _rng(seed, TID_BIAS).uniform(-0.01, 0.01, cfg.E).astype(np.float32)
    if cfg.routing == "zipf":
        beta = ZIPF_BETA if zipf_beta is None else zipf_beta
        ranks = zipf_ranks(cfg, seed)
        bias = (bias - beta * cfg.zipf_s * np.log(ranks)).astype(np.float32)
    return dict(x=_store(x, cfg.dtype), norm_w=_store(norm_w, cfg.dtype),
                router_w=_store(router_w, cfg.dtype), corr_bias=bias)


def redraw_rows(cfg: MoEConfig, seed: int, rows, attempt: int) -> np.ndarray:
    """Fresh N(0,1) rows of x for the given token indices (stream (10, t, attempt))."""
    out = np.empty((len(rows), cfg.d), np.float32)
    for i, t in enumerate(rows):
        out[i] = _rng(seed, TID_REDRAW, int(t), int(attempt)).standard_normal(cfg.d,
                                                                                dtype=np.float32)
    return _store(out, cfg.dtype)


def draw_expert_host(cfg: MoEConfig, seed: int, e: int):
    """(gate_up[e] [d, 2I], down[e] [I, d]) of one routed expert as host arrays."""
    gu = 0.02 * _rng(seed, TID_GATE_UP, e).standard_normal((cfg.d, 2 * cfg.I), dtype=np.float32)
    dn = 0.02 * _rng(seed, TID_DOWN, e).standard_normal((cfg.I, cfg.d), dtype=np.float32)
    return _store(gu, cfg.dtype), _store(dn, cfg.dtype)


def draw_shared_host(cfg: MoEConfig, seed: int):
    """(shared_gate [Is, d], shared_up [Is, d], shared_down [d, Is]) as host arrays."""
    if cfg.Is == 0:
        return None, None, None
    sg = 0.02 * _rng(seed, TID_SH_GATE).standard_normal((cfg.Is, cfg.d), dtype=np.float32)
    su = 0.02 * _rng(seed, TID_SH_UP).standard_normal((cfg.Is, cfg.d), dtype=np.float32)
    sd = 0.02 * _rng(seed, TID_SH_DOWN).standard_normal((cfg.d, cfg.Is), dtype=np.float32)
    return _store(sg, cfg.dtype), _store(su, cfg.dtype), _store(sd, cfg.dtype)


def make_host(cfg, seed: int = 0, zipf_beta: Optional[float] = None) -> dict:
    """Every input as host arrays (bf16 as uint16 bits).  Small workloads only."""
    cfg = config(cfg)
    inp = draw_small(cfg, seed, zipf_beta)
    gus, dns = zip(*(draw_expert_host(cfg, seed, e) for e in range(cfg.E)))
    inp["gate_up"] = np.stack(gus)
    inp["down"] = np.stack(dns)
    inp["shared_gate"], inp["shared_up"], inp["shared_down"] = draw_shared_host(cfg, seed)
    inp.update(meta(cfg))
    return inp


def meta(cfg: MoEConfig) -> dict:
    return dict(dtype=cfg.dtype, top_k=cfg.k, routed_scale=cfg.routed_scale, eps=cfg.eps,
                config=cfg.name)


# ----------------------------------------------------------------------------- torch side
def _torch():
    import torch
    return torch


def torch_dtype(cfg: MoEConfig):
    torch = _torch()
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def host_to_torch(a: np.ndarray, dtype: str, device):
    """Host storage array -> torch tensor of the storage dtype on ``device``."""
    torch = _torch()
    if a is None:
        return None
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    elif a.dtype == np.float32:
        t = torch.from_numpy(np.ascontiguousarray(a))
    else:
        raise TypeError(a.dtype)
    return t.to(device)


def torch_to_host(t) -> np.ndarray:
    """Torch tensor -> host storage array (bf16 as uint16 bits)."""
    torch = _torch()
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _device_normal(shape, std, seed_int, dtype, device):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed_int)
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, 1.0, generator=g)
    t.mul_(std)
    return t.to(dtype)


def make_torch(cfg, seed: int = 0, device="cuda", weights="device",
               small: Optional[dict] = None, zipf_beta: Optional[float] = None) -> dict:
    """Every input as torch tensors on ``device``.

    weights="host": expert weights drawn with NumPy (identical to ``make_host``);
    weights="device": drawn in device memory with torch's generator (fast at GLM-5
    size; the values differ from the host draw but are fixed by the seed).
    ``small``: optional pre-drawn host dict from ``draw_small`` (e.g. after row redraws).
    """
    torch = _torch()
    cfg = config(cfg)
    dt = torch_dtype(cfg)
    sm = draw_small(cfg, seed, zipf_beta) if small is None else small
    out = {key: host_to_torch(sm[key], cfg.dtype, device) for key in ("x", "norm_w", "router_w")}
    out["corr_bias"] = torch.from_numpy(np.ascontiguousarray(sm["corr_bias"], np.float32)).to(device)
    if weights == "host":
        gus, dns = zip(*(draw_expert_host(cfg, seed, e) for e in range(cfg.E)))
        out["gate_up"] = host_to_torch(np.stack(gus), cfg.dtype, device)
        out["down"] = host_to_torch(np.stack(dns), cfg.dtype, device)
        sg, su, sd = draw_shared_host(cfg, seed)
        out["shared_gate"] = host_to_torch(sg, cfg.dtype, device)
        out["shared_up"] = host_to_torch(su, cfg.dtype, device)
        out["shared_down"] = host_to_torch(sd, cfg.dtype, device)
    else:
        gate_up = torch.empty((cfg.E, cfg.d, 2 * cfg.I), dtype=dt, device=device)
        down = torch.empty((cfg.E, cfg.I, cfg.d), dtype=dt, device=device)
        for e in range(cfg.E):
            gate_up[e] = _device_normal((cfg.d, 2 * cfg.I), 0.02, _torch_seed(seed, TID_GATE_UP, e),
                                        dt, device)
            down[e] = _device_normal((cfg.I, cfg.d), 0.02, _torch_seed(seed, TID_DOWN, e), dt,
                                     device)
        out["gate_up"], out["down"] = gate_up, down
        if cfg.Is:
            out["shared_gate"] = _device_normal((cfg.Is, cfg.d), 0.02,
                                                _torch_seed(seed, TID_SH_GATE), dt, device)
            out["shared_up"] = _device_normal((cfg.Is, cfg.d), 0.02, _torch_seed(seed, TID_SH_UP),
                                              dt, device)
            out["shared_down"] = _device_normal((cfg.d, cfg.Is), 0.02,
                                                _torch_seed(seed, TID_SH_DOWN), dt, device)
        else:
            out["shared_gate"] = out["shared_up"] = out["shared_down"] = None
    out.update(meta(cfg))
    return out


def weight_bytes(cfg: MoEConfig) -> int:
    b = 2 if cfg.dtype == "bf16" else 4
    return b * (cfg.E * 3 * cfg.d * cfg.I + 3 * cfg.d * cfg.Is + cfg.E * cfg.d + cfg.d) + 4 * cfg.E


def param_count(cfg: MoEConfig) -> int:
    """Learned parameters of the MoE sublayer plus the router's correction-bias buffer."""
    return cfg.E * 3 * cfg.d * cfg.I + 3 * cfg.d * cfg.Is + cfg.E * cfg.d + cfg.E


# ----------------------------------------------------------------------------- RMSNorm cases
@dataclasses.dataclass(frozen=True)
class NormCase:
    """A standalone RMSNorm of the block: rows x width, rows `stride` elements apart."""
    name: str
    rows: int
    width: int
    stride: int
    dtype: str = "bf16"
    eps: float = 1e-6
    note: str = ""


# The widths of the block's other norms.  The input norm runs at the hidden size and
# the query-latent norm at 2048 ("GLM-5 · Query latent": q latent 2048; "GLM-5 ·
# Input features", excerpt block).  The key-value latent width is not printed: 512
# latent features in rows of 576 (with 64 rotary features after them) is synthetic.
# The per-head query/key norm runs over the query-key head width, 256 (the softmax
# scale printed on "GLM-5 · Query latent" is 1/sqrt(256)); rows = tokens x heads,
# with 64 heads as a synthetic head count.
NORM_CASES = {
    "input_norm": NormCase("input_norm", 4096, 6144, 6144, note="hidden size"),
    "q_latent_norm": NormCase("q_latent_norm", 4096, 2048, 2048, note="query latent"),
    "kv_latent_norm": NormCase("kv_latent_norm", 4096, 512, 576,
                               note="key-value latent (synthetic width), strided rows"),
    "qk_head_norm": NormCase("qk_head_norm", 4096 * 64, 256, 256,
                             note="per-head query/key norm (synthetic head count)"),
}


def draw_norm(rows: int, width: int, stride: int, dtype: str, seed: int = 0):
    """x [rows, stride] (only the first `width` columns are the norm's input; the rest
    is filler that must come through untouched) and gain [width], storage dtype.
    x = N(0, 1) times a per-feature log-normal scale (activations with uneven feature
    magnitudes); gain = 1 + 0.1 N(0, 1)."""
    scale = np.exp(0.5 * _rng(seed, TID_NORM_SCALE).standard_normal(stride)).astype(np.float32)
    x = _rng(seed, TID_NORM_X).standard_normal((rows, stride), dtype=np.float32) * scale
    gain = (1.0 + 0.1 * _rng(seed, TID_NORM_GAIN).standard_normal(width)).astype(np.float32)
    return _store(x, dtype), _store(gain, dtype)


# ----------------------------------------------------------------------------- dense MLP blocks
@dataclasses.dataclass(frozen=True)
class DenseCase:
    """A dense block (RMSNorm + SwiGLU MLP + residual): T tokens, hidden d, MLP width Id."""
    name: str
    T: int
    d: int
    Id: int
    dtype: str = "bf16"
    eps: float = 1e-6


# The blocks before the first MoE block use a dense SwiGLU MLP ("GLM-5 · Input
# features", excerpt block: the first first_k_dense_replace blocks).  Its width
# (intermediate_size) is not printed: 12288 (twice the hidden size) is synthetic.
DENSE_CASES = {
    "glm5_dense_decode": DenseCase("glm5_dense_decode", 64, 6144, 12288),
    "glm5_dense_prefill": DenseCase("glm5_dense_prefill", 4096, 6144, 12288),
}


def draw_dense(d: int, Id: int, dtype: str, seed: int = 0) -> dict:
    """Dense MLP weights in nn.Linear [out, in] layout: gate [Id, d], up [Id, d],
    down [d, Id], each N(0, 0.02^2), storage dtype."""
    gate = 0.02 * _rng(seed, TID_DENSE_GATE).standard_normal((Id, d), dtype=np.float32)
    up = 0.02 * _rng(seed, TID_DENSE_UP).standard_normal((Id, d), dtype=np.float32)
    down = 0.02 * _rng(seed, TID_DENSE_DOWN).standard_normal((d, Id), dtype=np.float32)
    return dict(gate=_store(gate, dtype), up=_store(up, dtype), down=_store(down, dtype))


def draw_block_input(T: int, d: int, dtype: str, seed: int = 0):
    """x [T, d] ~ N(0, 1) and norm_w = 1 + 0.1 N(0, 1): the residual-stream input of a
    block, drawn from the same streams (and so equal to) ``draw_small``'s x and norm_w."""
    x = _rng(seed, TID_X).standard_normal((T, d), dtype=np.float32)
    norm_w = (1.0 + 0.1 * _rng(seed, TID_NORM).standard_normal(d)).astype(np.float32)
    return _store(x, dtype), _store(norm_w, dtype)


def make_dense_torch(case, seed: int = 0, device="cuda", weights="device", T: Optional[int] = None):
    """Inputs of a dense block as torch tensors plus the host x / norm_w: x and norm_w from
    ``draw_block_input`` (the recipe of the MoE block's input); weights drawn on the
    device with torch's generator (seeded per tensor) or, with weights="host", by
    ``draw_dense``."""
    torch = _torch()
    T = case.T if T is None else T
    dt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    x, norm_w = draw_block_input(T, case.d, case.dtype, seed)
    out = dict(x=host_to_torch(x, case.dtype, device), norm_w=host_to_torch(norm_w, case.dtype, device))
    if weights == "host":
        w = draw_dense(case.d, case.Id, case.dtype, seed)
        for key in ("gate", "up", "down"):
            out[key] = host_to_torch(w[key], case.dtype, device)
    else:
        out["gate"] = _device_normal((case.Id, case.d), 0.02, _torch_seed(seed, TID_DENSE_GATE), dt, device)
        out["up"] = _device_normal((case.Id, case.d), 0.02, _torch_seed(seed, TID_DENSE_UP), dt, device)
        out["down"] = _device_normal((case.d, case.Id), 0.02, _torch_seed(seed, TID_DENSE_DOWN), dt, device)
    return out, dict(x=x, norm_w=norm_w)
