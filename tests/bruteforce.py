"""Brute-force twin of the oracle for tiny shapes (NumPy, float64).

Written independently of ``oracle/``: every routed expert is evaluated densely on
every token, the top-k selection is a full stable argsort, and the result is the
masked, weighted sum.  Used only to pin the oracle.
"""
import numpy as np

from workloads import bf16_bits_to_f32, f32_to_bf16_bits


def _val(a, dtype):
    """Storage array -> float64 values."""
    if a is None:
        return None
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, np.float32).astype(np.float64)


def _rnd(a32, dtype):
    """Round float32 values to the storage dtype, keep as float32."""
    a32 = np.asarray(a32, np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(a32))
    return a32


def dense_forward(inp):
    dt = inp["dtype"]
    k, rs, eps = inp["top_k"], inp["routed_scale"], np.float32(inp.get("eps", 1e-6))
    x = _val(inp["x"], dt)
    T, d = x.shape
    # norm: fp32 steps of the page's RMSNorm, the mean of squares rounded once to fp32
    x32 = x.astype(np.float32)
    ms = (np.einsum("td,td->t", x, x) / d).astype(np.float32)
    r = (np.float32(1.0) / np.sqrt(ms + eps)).astype(np.float32)
    nrm = _rnd(x32 * r[:, None], dt)
    h = _rnd(_val(inp["norm_w"], dt).astype(np.float32)[None, :] * nrm, dt).astype(np.float64)

    # router: every expert's sigmoid score, key = score + bias in fp32
    logits = (h @ _val(inp["router_w"], dt).T).astype(np.float32)
    s = (1.0 / (1.0 + np.exp(-logits.astype(np.float64)))).astype(np.float32)
    key = s + np.asarray(inp["corr_bias"], np.float32)[None, :]
    order = np.argsort(-key, axis=1, kind="stable")
    idx = order[:, :k]
    s_sel = np.take_along_axis(s, idx, axis=1).astype(np.float64)
    w = rs * s_sel / s_sel.sum(axis=1, keepdims=True)

    # every expert on every token
    gu = _val(inp["gate_up"], dt)            # [E, d, 2I]
    dn = _val(inp["down"], dt)               # [E, I, d]
    E, _, I2 = gu.shape
    I = I2 // 2
    z = np.einsum("td,edn->ten", h, gu)      # [T, E, 2I]
    g, u = z[..., :I], z[..., I:]
    a = g / (1.0 + np.exp(-g)) * u
    Y = np.einsum("tei,eid->ted", a, dn)     # [T, E, d]
    mask = np.zeros((T, E))
    np.put_along_axis(mask, idx, w, axis=1)
    routed = np.einsum("te,ted->td", mask, Y)

    shared = np.zeros_like(x)
    act_s = None
    if inp.get("shared_gate") is not None:
        sg, su, sd = (_val(inp[n], dt) for n in ("shared_gate", "shared_up", "shared_down"))
        gs, us = h @ sg.T, h @ su.T
        act_s = gs / (1.0 + np.exp(-gs)) * us
        shared = act_s @ sd.T
    delta = shared + routed
    out = _rnd((x + delta).astype(np.float32), dt)
    return dict(h=h, logits=logits, scores=s, key=key, idx=idx, w=w, delta=delta, out=out,
                Y=Y, act=a, act_s=act_s, shared=shared)
