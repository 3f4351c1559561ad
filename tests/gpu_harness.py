"""Helpers for the GPU parity tests: run the HIP library through its C ABI,
read back routing and intermediates, and compare with the CPU oracle.

Parity bars:
  * selected experts (as per-token sets) and per-expert counts: bit-exact;
  * bf16 outputs: relative L2 <= 1e-2 and max-abs <= 2e-2 * RMS(reference), on
    both out and delta = out - x;
  * fp32 outputs: delta relative L2 <= 1e-4 and max-abs <= 1e-3 * RMS(reference).
"""
import numpy as np
import torch

import mixture_experts_transformer_rmsnorm_amd as moe
import oracle
import workloads
from tests.margin import filtered_small

BF16_REL_L2, BF16_MAXABS = 1e-2, 2e-2
F32_REL_L2, F32_MAXABS = 1e-4, 1e-3


def say(*a):
    print(*a, flush=True)


def prepare(cfg, seed=0, weights="host"):
    """Margin-filtered inputs on the GPU plus the oracle's routing of every token."""
    cfg = workloads.config(cfg)
    small, route, n_redrawn = filtered_small(cfg, seed)
    tin = workloads.make_torch(cfg, seed, device="cuda", weights=weights, small=small)
    torch.cuda.synchronize()
    return cfg, small, route, tin


GUARD_BYTES = 1 << 20
GUARD_BYTE = 0xA5


def guard_workspace(block):
    """Re-seat the block's workspace at the front of a larger buffer whose tail (the
    guard) holds a fixed byte pattern; returns the guard."""
    big = torch.full((block.workspace_bytes + GUARD_BYTES,), GUARD_BYTE, dtype=torch.uint8,
                     device=block.workspace.device)
    block.workspace = big[:block.workspace_bytes]
    return big[block.workspace_bytes:]


def assert_guard(guard):
    torch.cuda.synchronize()
    bad = int((guard != GUARD_BYTE).sum())
    assert bad == 0, "%d bytes past the workspace were written" % bad


def make_block(cfg, tin, path=moe.MOE_PATH_AUTO, max_tokens=None):
    return moe.MoEBlock({k: tin[k] for k in ("norm_w", "router_w", "corr_bias", "gate_up", "down",
                                             "shared_gate", "shared_up", "shared_down")
                         if tin.get(k) is not None},
                        max_tokens=max(cfg.T if max_tokens is None else max_tokens, 1),
                        top_k=cfg.k, routed_scale=cfg.routed_scale, eps=cfg.eps, path=path)


def run_gpu(cfg, tin, path=moe.MOE_PATH_AUTO, T=None, out=None, x=None, block=None):
    """One forward through moe_block_forward; returns (block, out tensor)."""
    T = cfg.T if T is None else T
    if block is None:
        block = make_block(cfg, tin, path, max_tokens=T)
    x = tin["x"][:T] if x is None else x
    res = block.forward(x, out=out)
    torch.cuda.synchronize()
    return block, res


def read_all(block, cfg, T):
    """Routing and intermediates of the block's last call as host arrays."""
    idx, w, cnt = block.routing(T)
    es = 2 if cfg.dtype == "bf16" else 4
    bufs = {}
    for name, which in (("h", moe.MOE_BUF_H), ("offsets", moe.MOE_BUF_OFFSETS),
                        ("perm_token", moe.MOE_BUF_PERM_TOKEN), ("row_of", moe.MOE_BUF_ROW_OF),
                        ("act", moe.MOE_BUF_ACT), ("y", moe.MOE_BUF_Y)):
        bufs[name] = block.buffer(which, T).cpu().numpy()
    torch.cuda.synchronize()
    r = dict(idx=idx.cpu().numpy(), w=w.cpu().numpy(), counts=cnt.cpu().numpy())
    for name in ("offsets", "perm_token", "row_of"):
        r[name] = bufs[name].view(np.int32)
    r["row_of"] = r["row_of"].reshape(T, cfg.k)
    dt_np = np.uint16 if es == 2 else np.float32
    r["h"] = bufs["h"].view(dt_np).reshape(T, cfg.d)
    r["act"] = bufs["act"].view(dt_np).reshape(T * cfg.k, cfg.I)
    r["y"] = bufs["y"].view(dt_np).reshape(T * cfg.k, cfg.d)
    return r


def values(a, dtype):
    """Storage array (uint16 bf16 bits or float32) -> float64 values."""
    if dtype == "bf16":
        return workloads.bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, np.float64)


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_close(got, ref, dtype, what):
    """The parity bar for floating-point outputs; returns (rel_l2, maxabs/rms)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    rl = rel_l2(got, ref)
    ma = float(np.max(np.abs(got - ref))) / max(rms, 1e-300)
    lim_l2, lim_ma = (BF16_REL_L2, BF16_MAXABS) if dtype == "bf16" else (F32_REL_L2, F32_MAXABS)
    say("  %-14s rel_l2=%.3e  maxabs/rms=%.3e  (rms %.3e)" % (what, rl, ma, rms))
    assert rl <= lim_l2, "%s: relative L2 %.3e > %.1e" % (what, rl, lim_l2)
    assert ma <= lim_ma, "%s: max-abs/RMS %.3e > %.1e" % (what, ma, lim_ma)
    return rl, ma


def check_intermediate(got, ref, dtype, what):
    """Bar for intermediates rounded to D (act, y): relative L2 as for outputs, and
    per element one rounding to D (2^-8 relative for bf16) plus accumulation-order
    noise (2e-2 * RMS for bf16, 1e-3 * RMS for fp32)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    rl = rel_l2(got, ref)
    if dtype == "bf16":
        rel_elem, abs_elem, lim_l2 = 2.0 ** -8, BF16_MAXABS * rms, BF16_REL_L2
    else:
        rel_elem, abs_elem, lim_l2 = 2.0 ** -20, F32_MAXABS * rms, F32_REL_L2
    excess = np.abs(got - ref) - (rel_elem * np.abs(ref) + abs_elem)
    say("  %-14s rel_l2=%.3e  worst elem excess=%.3e  (rms %.3e)" % (what, rl, excess.max(), rms))
    assert rl <= lim_l2, "%s: relative L2 %.3e > %.1e" % (what, rl, lim_l2)
    assert excess.max() <= 0, "%s: element beyond one rounding + noise" % what


def check_routing(g, route, cfg, tokens=None):
    """Selected expert sets and counts bit-exact; weights close (aligned by expert)."""
    oi = route["idx"]
    gi = g["idx"]
    if tokens is not None:
        oi, gi = oi[tokens], gi[tokens]
    bad = np.nonzero(np.any(np.sort(gi, 1) != np.sort(oi, 1), axis=1))[0]
    if len(bad):
        say("  routing mismatch on %d tokens, e.g. %s; oracle margins %s" % (
            len(bad), bad[:5].tolist(), route["margin"][bad[:5]].tolist()))
    assert len(bad) == 0
    cnt_ref = np.bincount(route["idx"].ravel(), minlength=cfg.E)
    assert np.array_equal(g["counts"], cnt_ref), "per-expert counts differ"
    og = np.argsort(oi, 1, kind="stable")
    gg = np.argsort(gi, 1, kind="stable")
    ow = np.take_along_axis(route["w"] if tokens is None else route["w"][tokens], og, 1)
    gw = np.take_along_axis(g["w"] if tokens is None else g["w"][tokens], gg, 1)
    np.testing.assert_allclose(gw, ow, rtol=2e-5, atol=1e-7)


def check_permutation(g, cfg, T):
    """Offsets are the exclusive scan of the counts; every expert's segment holds
    exactly the tokens that chose it, in token order; row_of inverts the permutation."""
    cnt = g["counts"]
    off = g["offsets"]
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32))
    perm = g["perm_token"][: T * cfg.k]
    for e in np.nonzero(cnt)[0]:
        seg = perm[off[e]:off[e + 1]]
        expect = np.nonzero(np.any(g["idx"] == e, axis=1))[0]
        assert np.array_equal(seg, expect), "segment of expert %d" % e
    rows = g["row_of"]
    assert np.array_equal(perm[rows], np.repeat(np.arange(T)[:, None], cfg.k, 1))
    for j in range(cfg.k):
        e = g["idx"][:, j]
        assert np.all((rows[:, j] >= off[e]) & (rows[:, j] < off[e + 1]))


def host_weights(tin, cfg, experts):
    """Host copies of the listed experts (others None) and of the shared expert."""
    gu = [None] * cfg.E
    dn = [None] * cfg.E
    for e in experts:
        gu[e] = workloads.torch_to_host(tin["gate_up"][e])
        dn[e] = workloads.torch_to_host(tin["down"][e])
    sh = [None if tin.get(n) is None else workloads.torch_to_host(tin[n])
          for n in ("shared_gate", "shared_up", "shared_down")]
    return gu, dn, sh


def oracle_outputs(cfg, small, route, tin, tokens, debug=False):
    """Oracle delta/out for the listed tokens (routing of every token given)."""
    tokens = np.asarray(tokens, np.int64)
    experts = np.unique(route["idx"][tokens])
    gu, dn, sh = host_weights(tin, cfg, experts)
    return oracle.experts(tokens, small["x"], route["h"], route["idx"], route["w"], gu, dn,
                          sh[0], sh[1], sh[2], oracle.DTYPES[cfg.dtype], debug=debug)


def half_ulp(v, dtype):
    """Half a unit in the last place of D at |v| (the bound of one rounding to D)."""
    mant = 8 if dtype == "bf16" else 24
    e = np.floor(np.log2(np.maximum(np.abs(v), 1e-30)))
    return np.exp2(e - mant)


def check_delta(got_out, x, delta_ref, dtype):
    """The sublayer's contribution delta = out - x, beyond the one rounding of out
    to D: per element |out - (x + delta_ref)| - half_ulp(x + delta_ref) must stay
    within the output bar relative to RMS(delta_ref), in L2 and in max-abs.  (At
    small hidden sizes delta is small against x, and the rounding of out alone can
    exceed 1% of delta.)"""
    ref_out = x + delta_ref
    err = np.abs(got_out - ref_out)
    excess = np.maximum(err - half_ulp(ref_out, dtype), 0.0)
    rms = float(np.sqrt(np.mean(delta_ref ** 2)))
    rl = float(np.sqrt(np.mean(excess ** 2))) / max(rms, 1e-300)
    ma = float(excess.max()) / max(rms, 1e-300)
    lim_l2, lim_ma = (BF16_REL_L2, BF16_MAXABS) if dtype == "bf16" else (F32_REL_L2, F32_MAXABS)
    say("  %-14s rel_l2=%.3e  maxabs/rms=%.3e  (rms %.3e, beyond one rounding of out)" % (
        "delta", rl, ma, rms))
    assert rl <= lim_l2, "delta: relative L2 %.3e > %.1e" % (rl, lim_l2)
    assert ma <= lim_ma, "delta: max-abs/RMS %.3e > %.1e" % (ma, lim_ma)


def check_outputs(cfg, small, g_out, delta_ref, out_ref, tokens):
    """out against the oracle's exact x + delta (before its own rounding to D, so
    the two sides' independent roundings are not compared with each other), and
    delta beyond the one rounding of out.  How often the GPU's out differs from the
    oracle's own rounded out, and by how many units in the last place, is printed
    as a diagnostic only (near zero an ulp is far below the bar)."""
    x = values(small["x"][tokens], cfg.dtype)
    got = values(g_out, cfg.dtype)
    delta_ref = np.asarray(delta_ref, np.float64)
    check_close(got, x + delta_ref, cfg.dtype, "out")
    check_delta(got, x, delta_ref, cfg.dtype)
    ro = values(out_ref, "f32")
    ulps = np.abs(got - ro) / (2 * half_ulp(np.maximum(np.abs(got), np.abs(ro)), cfg.dtype))
    say("  out vs oracle's rounded out: %.2f%% of elements differ; 99.99th pct %.2f ulp" % (
        100 * np.mean(ulps > 0), np.percentile(ulps, 99.99)))
