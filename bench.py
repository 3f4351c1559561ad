#!/usr/bin/env python3
"""Benchmark of the MoE feed-forward sublayer on one MI355X.

One step = one moe_block_forward over one batch (RMSNorm, router top-k,
permutation, routed + shared SwiGLU experts, combine + residual) with every
input resident in HBM.  The headline line is the GLM-5-shaped decode batch
(64 tokens, d 6144, 256 experts of width 2048, top-8, one shared expert, bf16);
the same line carries the GLM-5 prefill batch (4096 tokens) as a secondary
measurement.  Inputs are seeded synthetic tensors (weights N(0, 0.02), x N(0,1),
gain 1 + N(0, 0.1), correction bias U(-0.01, 0.01)).

Output: one JSON line on stdout.  Progress goes to stderr.
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-block tokens/s at GLM-5 shape (T=64 decode, T=4096 prefill); % roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
DOMINANT = "expert_gate_up"    # the gate_and_up grouped kernel: 2/3 of bytes and FLOPs


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(workload, stage):
    """HBM-side bytes per launch of `stage` on `workload` from profiles/traffic.txt (rocprofv3
    counts of the L2's read and write requests to the memory fabric, by request size), or
    None when no record exists or the kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        wl, st, files, sha, fetch, write, _alg = line.split()
        if wl != workload or st != stage:
            continue
        h = hashlib.sha256()
        for f in files.split(","):
            h.update(open(os.path.join(ROOT, "mixture_experts_transformer_rmsnorm_amd", "csrc", f),
                          "rb").read())
        if h.hexdigest()[:16] != sha:
            return None
        return int(fetch) + int(write)
    return None


def algorithmic(cfg, counts):
    """Algorithmic HBM bytes and FLOPs of one step and of one gate_up launch."""
    b = 2 if cfg.dtype == "bf16" else 4
    n_active = int((counts > 0).sum())
    A = cfg.T * cfg.k
    step_bytes = (n_active * 3 * cfg.d * cfg.I * b + 3 * cfg.d * cfg.Is * b + cfg.E * cfg.d * b
                  + 4 * cfg.E + cfg.d * b + 2 * cfg.T * cfg.d * b)
    step_flops = 2 * cfg.T * cfg.E * cfg.d + 6 * A * cfg.d * cfg.I + 6 * cfg.T * cfg.d * cfg.Is
    # gate_up kernel: per active expert its [d, 2I] weights; plus h rows in, act rows out
    gu_unit_bytes = cfg.d * 2 * cfg.I * b
    gu_bytes = n_active * gu_unit_bytes + cfg.T * cfg.d * b + A * cfg.I * b
    gu_flops = 4 * A * cfg.d * cfg.I
    return dict(n_active=n_active, step_bytes=step_bytes, step_flops=step_flops,
                gu_unit_bytes=gu_unit_bytes, gu_bytes=gu_bytes, gu_flops=gu_flops)


ATTAINABLE = {}  # measured peaks of this GPU: "hbm" GB/s (read stream), "mfma" TFLOP/s (bf16)


def measure_peaks(launches=10):
    """The attainable HBM read rate and bf16 MFMA rate of this GPU, from the library's
    measurement kernels (moe_calib_hbm_read over 4 GiB on 256 blocks of 1024 lanes;
    moe_calib_mfma on 512 blocks of 8 waves), timed with HIP events."""
    import torch
    import mixture_experts_transformer_rmsnorm_amd as moe
    nbytes = 4 << 30
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        moe.moe_calib_hbm_read(None, buf, nbytes, 256, sink)
    e0.record()
    for _ in range(launches):
        moe.moe_calib_hbm_read(None, buf, nbytes, 256, sink)
    e1.record()
    torch.cuda.synchronize()
    hbm = nbytes * launches / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf
    iters, blocks = 4096, 512
    for _ in range(2):
        moe.moe_calib_mfma(None, iters, blocks, sink)
    e0.record()
    flops = 0.0
    for _ in range(launches):
        flops += moe.moe_calib_mfma(None, iters, blocks, sink)
    e1.record()
    torch.cuda.synchronize()
    mfma = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    ATTAINABLE.update(hbm=hbm, mfma=mfma)
    log("attainable peaks: HBM read %.1f GB/s, bf16 MFMA %.1f TFLOP/s" % (hbm, mfma))
    return {"hbm_read_GB_per_s": round(hbm, 1), "mfma_bf16_TFLOP_per_s": round(mfma, 1),
            "hbm_read_frac_of_published": round(hbm / HBM_PEAK_GBS, 4),
            "mfma_frac_of_published": round(mfma / BF16_PEAK_TFLOPS, 4),
            "how": "moe_calib_hbm_read: 4 GiB, 256 blocks x 1024 lanes, 16-byte nontemporal "
                   "loads; moe_calib_mfma: 512 blocks x 8 waves x 4096 rounds of 4 "
                   "independent v_mfma_f32_32x32x16_bf16; HIP events over %d launches" % launches}


def run_workload(cfg, tin, steps, warmup, path=None):
    import torch
    import mixture_experts_transformer_rmsnorm_amd as moe

    weights = {k: tin[k] for k in ("norm_w", "router_w", "corr_bias", "gate_up", "down",
                                   "shared_gate", "shared_up", "shared_down")}
    block = moe.MoEBlock(weights, max_tokens=cfg.T, top_k=cfg.k, routed_scale=cfg.routed_scale,
                         eps=cfg.eps, path=moe.MOE_PATH_AUTO if path is None else path)
    x = tin["x"]
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        block.forward(x, out=out)
    torch.cuda.synchronize()
    _, _, cnt = block.routing(cfg.T)
    counts = cnt.cpu().numpy()
    path = moe.moe_plan_path(block.plan, cfg.T, cfg.k)

    # timed region: K steps; HIP events on the forward's stream around the dominant kernel
    # (the fused decode kernel runs every stage in its one launch)
    dominant = "fused_decode" if path == moe.MOE_PATH_FUSED else DOMINANT
    moe.moe_set_stage_timing(block.plan, moe.stage_mask(dominant))
    moe.moe_stage_times(block.plan)  # reset
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        block.forward(x, out=out, stream=stream)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    stage_ms, calls = moe.moe_stage_times(block.plan)
    moe.moe_set_stage_timing(block.plan, 0)

    # one more pass with every stage timed, for the per-stage breakdown (not the headline)
    moe.moe_set_stage_timing(block.plan, moe.stage_mask())
    for _ in range(min(steps, 10)):
        block.forward(x, out=out, stream=stream)
    torch.cuda.synchronize()
    all_ms, all_calls = moe.moe_stage_times(block.plan)
    moe.moe_set_stage_timing(block.plan, 0)
    block.close()

    elapsed = t1 - t0
    ms_step = 1e3 * elapsed / steps
    alg = algorithmic(cfg, counts)
    gu_ms = stage_ms[dominant] / max(calls, 1)
    gu_s = gu_ms * 1e-3
    hbm_t = alg["gu_bytes"] / (HBM_PEAK_GBS * 1e9)
    mfma_t = alg["gu_flops"] / (BF16_PEAK_TFLOPS * 1e12)
    if hbm_t >= mfma_t:
        achieved = alg["gu_bytes"] / gu_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        achieved = alg["gu_flops"] / gu_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None}
    roof["traffic"] = measured_traffic(cfg.name, DOMINANT)
    if ATTAINABLE:
        att = ATTAINABLE["hbm"] if roof["bound"] == "hbm" else ATTAINABLE["mfma"]
        roof["attainable"] = round(att, 1)
        roof["frac_of_attainable"] = round(achieved / att, 4)
    roof.update(kernel=dominant, kernel_ms=round(gu_ms, 4), algorithmic_bytes=alg["gu_bytes"],
                algorithmic_flops=alg["gu_flops"], active_experts=alg["n_active"])
    if roof["traffic"]:
        roof["traffic_over_algorithmic"] = round(roof["traffic"] / alg["gu_bytes"], 4)
    step_s = ms_step * 1e-3
    hbm_frac = alg["step_bytes"] / step_s / (HBM_PEAK_GBS * 1e9)
    mfma_frac = alg["step_flops"] / step_s / (BF16_PEAK_TFLOPS * 1e12)
    t_roof = max(alg["step_bytes"] / (HBM_PEAK_GBS * 1e9), alg["step_flops"] / (BF16_PEAK_TFLOPS * 1e12))
    step_roof = {"bytes_alg": alg["step_bytes"], "flops_alg": alg["step_flops"],
                 "GB_per_s": round(alg["step_bytes"] / step_s / 1e9, 1),
                 "TFLOP_per_s": round(alg["step_flops"] / step_s / 1e12, 1),
                 "hbm_frac": round(hbm_frac, 4), "mfma_frac": round(mfma_frac, 4),
                 "frac": round(t_roof / step_s, 4)}
    if ATTAINABLE:
        t_att = max(alg["step_bytes"] / (ATTAINABLE["hbm"] * 1e9),
                    alg["step_flops"] / (ATTAINABLE["mfma"] * 1e12))
        step_roof["frac_of_attainable"] = round(t_att / step_s, 4)
    per_stage = {k: round(v / max(all_calls, 1), 4) for k, v in all_ms.items() if v > 0}
    return dict(value=cfg.T * steps / elapsed, ms_per_step=ms_step,
                ms_per_step_median=step_ms[len(step_ms) // 2], ms_per_step_min=step_ms[0],
                roofline=roof,
                step_roofline=step_roof, stage_ms=per_stage, path=path,
                max_load=int(counts.max()), counts=counts)


def load_summary(counts):
    """Tokens per expert of the timed batch: active experts and the spread of their loads."""
    import numpy as np
    c = np.asarray(counts)
    nz = np.sort(c[c > 0])
    if nz.size == 0:
        return {"active_experts": 0}
    return {"active_experts": int(nz.size), "min": int(nz[0]), "median": float(np.median(nz)),
            "max": int(nz[-1]), "p90": float(np.percentile(nz, 90))}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


class _HostExperts:
    """Host copies (bf16 bits) of the device expert weights the oracle needs."""

    def __init__(self, cfg, tin):
        import workloads
        self.cfg, self.tin = cfg, tin
        self.gu, self.dn = {}, {}
        self.shared = ([workloads.torch_to_host(tin[n]) for n in ("shared_gate", "shared_up",
                                                                  "shared_down")]
                       if cfg.Is else [None, None, None])

    def lists(self, experts):
        import workloads
        for e in experts:
            if e not in self.gu:
                self.gu[e] = workloads.torch_to_host(self.tin["gate_up"][e])
                self.dn[e] = workloads.torch_to_host(self.tin["down"][e])
        return ([self.gu.get(e) for e in range(self.cfg.E)],
                [self.dn.get(e) for e in range(self.cfg.E)])


def _oracle_seconds(cfg, small, hosts, rows):
    """Oracle time of the full forward (norm, router, selection, the selected experts and
    the shared expert, combine) on the given rows of the batch; weight copies to the host
    happen before the clock starts."""
    import numpy as np
    import oracle
    dt = oracle.DTYPES[cfg.dtype]
    xs = small["x"][rows]
    pre = oracle.route(xs, small["norm_w"], small["router_w"], small["corr_bias"], cfg.k,
                       cfg.routed_scale, dt, cfg.eps)
    gu, dn = hosts.lists(np.unique(pre["idx"]))
    sh = hosts.shared
    t0 = time.perf_counter()
    r = oracle.route(xs, small["norm_w"], small["router_w"], small["corr_bias"], cfg.k,
                     cfg.routed_scale, dt, cfg.eps)
    oracle.experts(np.arange(len(rows)), xs, r["h"], r["idx"], r["w"], gu, dn, sh[0], sh[1],
                   sh[2], dt)
    return time.perf_counter() - t0


def cpu_baseline(cfg, tin, small, seconds):
    """The CPU oracle, as it stands, timed on this machine's host cores.

    Headline: the same decode batch, in chunks of 8 tokens taken in order and from the
    start again when the batch ends, until about `seconds` of oracle time, on the
    oracle's OpenMP threads (the process's CPU share).  Beside it: single-thread rates on the tiny fp32 workload (whole batch)
    and on 4 decode tokens; and per-token rates on 16 tokens of the 4096-token prefill
    and of the mid-size workload, extrapolated to their whole batches."""
    import numpy as np
    import torch
    import oracle
    import workloads

    threads = oracle.num_threads()
    hosts = _HostExperts(cfg, tin)
    spent, done, chunk = 0.0, 0, 8
    pos = 0
    while spent < seconds or done == 0:
        rows = np.arange(pos, min(cfg.T, pos + chunk))
        spent += _oracle_seconds(cfg, small, hosts, rows)
        done += len(rows)
        pos = (pos + len(rows)) % cfg.T
        log("cpu oracle: %d tokens in %.1f s" % (done, spent))
    if done >= cfg.T:
        what = "%d tokens (%.2f passes over the %d %s tokens)" % (done, done / cfg.T, cfg.T,
                                                                  cfg.name)
    else:
        what = "first %d of the %d %s tokens" % (done, cfg.T, cfg.name)
    res = {"value": round(done / spent, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": "%s, full forward (norm, router, %d experts + shared, combine), "
                     "%.1f s on %d OpenMP threads" % (what, cfg.k, spent, threads),
           "cpu_model": cpu_model(), "cores_available": len(os.sched_getaffinity(0))}

    # single thread: the tiny fp32 workload in full, and 4 decode tokens
    single = {}
    tiny = workloads.config("tiny_fp32")
    host = workloads.make_host(tiny, 0)
    for n in (1, threads):
        oracle.set_num_threads(n)
        t0 = time.perf_counter()
        oracle.forward(host)
        dt_s = time.perf_counter() - t0
        single["tiny_fp32_%dthread%s" % (n, "" if n == 1 else "s")] = {
            "tokens": tiny.T, "seconds": round(dt_s, 4), "tokens_per_s": round(tiny.T / dt_s, 1)}
    oracle.set_num_threads(1)
    t1 = _oracle_seconds(cfg, small, hosts, np.arange(4))
    oracle.set_num_threads(threads)
    single["%s_1thread" % cfg.name] = {"tokens": 4, "seconds": round(t1, 3),
                                       "tokens_per_s": round(4 / t1, 3)}
    log("cpu oracle, 1 thread: %s 4 tokens in %.2f s" % (cfg.name, t1))
    res["single_thread"] = single

    # per-token time on 16 tokens of the prefill workloads, times their batch size
    extra = {}
    for name in ("glm5_prefill", "mid_prefill"):
        c2 = workloads.config(name)
        s2 = workloads.draw_small(c2, 0)
        same = (c2.d, c2.E, c2.I, c2.Is, c2.dtype) == (cfg.d, cfg.E, cfg.I, cfg.Is, cfg.dtype)
        t2 = tin if same else workloads.make_torch(c2, 0, device="cuda", weights="device")
        h2 = hosts if same else _HostExperts(c2, t2)
        n = 16
        sec = _oracle_seconds(c2, s2, h2, np.arange(n))
        extra[name] = {"tokens_timed": n, "seconds": round(sec, 3), "tokens_per_s": round(n / sec, 3),
                       "batch_tokens": c2.T, "batch_seconds_extrapolated": round(sec / n * c2.T, 1),
                       "threads": threads}
        log("cpu oracle: %s %d tokens in %.2f s (batch of %d: %.0f s extrapolated)" % (
            name, n, sec, c2.T, sec / n * c2.T))
        if not same:
            del h2, t2
            torch.cuda.empty_cache()
    res["extrapolated"] = extra
    return res


def measure_norms(launches):
    """Standalone RMSNorm entry point at the widths of the block's other norms: HBM
    roofline of each (algorithmic bytes = rows*width read + rows*width written + the
    gain, in bf16), timed with HIP events over `launches` calls on the current stream."""
    import torch
    import workloads
    import mixture_experts_transformer_rmsnorm_amd as moe
    out = {}
    g = torch.Generator(device="cuda")
    for name, c in workloads.NORM_CASES.items():
        g.manual_seed(1234)
        x = torch.randn((c.rows, c.stride), generator=g, device="cuda").to(torch.bfloat16)
        w = (1.0 + 0.1 * torch.randn((c.width,), generator=g, device="cuda")).to(torch.bfloat16)
        o = torch.empty_like(x)
        for _ in range(3):
            moe.moe_rmsnorm(None, moe.MOE_DTYPE_BF16, c.rows, c.width, c.eps, x, c.stride, w, o, c.stride)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(launches):
            moe.moe_rmsnorm(None, moe.MOE_DTYPE_BF16, c.rows, c.width, c.eps, x, c.stride, w, o, c.stride)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / launches
        nbytes = 2 * c.rows * c.width * 2 + c.width * 2
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"rows": c.rows, "width": c.width, "row_stride": c.stride, "ms": round(ms, 4),
                     "algorithmic_bytes": nbytes, "GB_per_s": round(gbs, 1),
                     "frac_of_hbm_peak": round(gbs / 8000.0, 4)}
        log("rmsnorm %s: %d x %d, %.4f ms, %.1f GB/s" % (name, c.rows, c.width, ms, gbs))
        del x, w, o
    return out


def measure_dense(launches):
    """Dense block (RMSNorm + SwiGLU MLP + residual; moe_dense_block_forward) at the
    GLM-5 hidden size with a synthetic MLP width: tokens/s and the step against
    max(bytes_alg / 8 TB/s, flops_alg / 2.5 PFLOP/s), bytes_alg = the three weight
    matrices + x read + out written, flops_alg = 6 T d Id."""
    import torch
    import workloads
    import mixture_experts_transformer_rmsnorm_amd as moe
    out = {}
    for name, c in workloads.DENSE_CASES.items():
        tin, _ = workloads.make_dense_torch(c, 0, "cuda", weights="device")
        blk = moe.DenseBlock({k: tin[k] for k in ("norm_w", "gate", "up", "down")}, max_tokens=c.T,
                             eps=c.eps)
        y = torch.empty_like(tin["x"])
        for _ in range(3):
            blk.forward(tin["x"], out=y)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(launches):
            blk.forward(tin["x"], out=y)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / launches
        b = 2 if c.dtype == "bf16" else 4
        nbytes = 3 * c.d * c.Id * b + 2 * c.T * c.d * b
        flops = 6 * c.T * c.d * c.Id
        t_hbm, t_mfma = nbytes / 8e12, flops / 2.5e15
        out[name] = {"tokens": c.T, "dim": c.d, "mlp_width": c.Id, "ms": round(ms, 4),
                     "tokens_per_s": round(c.T / (ms * 1e-3), 1),
                     "bound": "hbm" if t_hbm >= t_mfma else "mfma",
                     "GB_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "TFLOP_per_s": round(flops / (ms * 1e-3) / 1e12, 1),
                     "frac_of_max_roofline": round(max(t_hbm, t_mfma) / (ms * 1e-3), 4)}
        log("dense %s: %.4f ms, %.1f tokens/s, %.1f%% of the max roofline" % (
            name, ms, c.T / (ms * 1e-3), 100 * out[name]["frac_of_max_roofline"]))
        blk.close()
        del tin, blk, y
    return out


def measure_configs(cfg, tin, steps, names=("glm5_prefill_zipf", "mid_prefill")):
    """The MFMA-bound prefill workloads (Zipf-skewed routing at 16384 tokens on the GLM-5
    weights; the mid-size block at 8192 tokens): tokens/s, the step against the max
    roofline with its HBM and MFMA fractions, and the dominant kernel's roofline."""
    import torch
    import workloads
    out = {}
    for name in names:
        c2 = workloads.config(name)
        if tin is not None and (c2.d, c2.E, c2.I, c2.Is, c2.dtype) == (cfg.d, cfg.E, cfg.I, cfg.Is, cfg.dtype):
            t2 = dict(tin)
            small2 = workloads.draw_small(c2, 0)
            for key in ("x", "norm_w", "router_w"):
                t2[key] = workloads.host_to_torch(small2[key], c2.dtype, "cuda")
            t2["corr_bias"] = torch.from_numpy(small2["corr_bias"]).cuda()
        else:
            t2 = workloads.make_torch(c2, 0, device="cuda", weights="device")
        torch.cuda.synchronize()
        r = run_workload(c2, t2, steps, 2)
        out[name] = {"tokens": c2.T, "value": round(r["value"], 1), "unit": "tokens/s",
                     "ms_per_step": round(r["ms_per_step"], 4),
                     "kernel_path": "stream" if r["path"] == 1 else "mfma",
                     "max_expert_load": r["max_load"], "roofline": r["roofline"],
                     "step_roofline": r["step_roofline"]}
        log("%s: %.1f tokens/s, %.3f ms/step, step %.1f%% of the max roofline (MFMA %.1f%%)" % (
            name, r["value"], r["ms_per_step"], 100 * r["step_roofline"]["frac"],
            100 * r["step_roofline"]["mfma_frac"]))
        del t2
        torch.cuda.empty_cache()
    return out


def measure_sweep(cfg, tin, steps, warmup, tokens=(1, 2, 4, 8, 16, 32, 128, 256),
                  fused_tokens=(1, 8, 64)):
    """The MoE block at other batch sizes on the same weights (decode-sized batches use
    the streaming kernels): ms per step, tokens/s and the gate_up kernel's HBM rate;
    and the fused single-launch decode kernel (MOE_PATH_FUSED) at decode batch sizes."""
    import torch
    import workloads
    out = {}
    for T in tokens:
        c = workloads.config(cfg, T=T)
        t2 = dict(tin)
        sm = workloads.draw_small(c, 0)
        for key in ("x", "norm_w", "router_w"):
            t2[key] = workloads.host_to_torch(sm[key], c.dtype, "cuda")
        t2["corr_bias"] = torch.from_numpy(sm["corr_bias"]).cuda()
        r = run_workload(c, t2, steps, warmup)
        out["T%d" % T] = {"tokens": T, "ms_per_step": round(r["ms_per_step"], 4),
                          "ms_per_step_median": round(r["ms_per_step_median"], 4),
                          "tokens_per_s": round(r["value"], 1),
                          "kernel_path": "stream" if r["path"] == 1 else "mfma",
                          "gate_up_ms": r["roofline"]["kernel_ms"],
                          "gate_up_" + r["roofline"]["unit"].replace("/", "_per_"):
                              r["roofline"]["achieved"],
                          "gate_up_frac": r["roofline"]["frac"],
                          "active_experts": r["roofline"]["active_experts"]}
        if T <= 8:
            # per-stage breakdown (a separate pass with every stage between HIP events;
            # a stage whose work another stage's launch does is absent)
            out["T%d" % T]["stage_ms"] = r["stage_ms"]
        log("sweep T=%d: %.4f ms/step, %.1f tokens/s" % (T, r["ms_per_step"], r["value"]))
        del t2
    import mixture_experts_transformer_rmsnorm_amd as moe
    for T in fused_tokens:
        c = workloads.config(cfg, T=T)
        t2 = dict(tin)
        sm = workloads.draw_small(c, 0)
        for key in ("x", "norm_w", "router_w"):
            t2[key] = workloads.host_to_torch(sm[key], c.dtype, "cuda")
        t2["corr_bias"] = torch.from_numpy(sm["corr_bias"]).cuda()
        r = run_workload(c, t2, steps, warmup, path=moe.MOE_PATH_FUSED)
        out["fused_T%d" % T] = {"tokens": T, "ms_per_step": round(r["ms_per_step"], 4),
                                "ms_per_step_median": round(r["ms_per_step_median"], 4),
                                "tokens_per_s": round(r["value"], 1), "kernel_path": "fused",
                                "step_GB_per_s": r["step_roofline"]["GB_per_s"],
                                "step_frac": r["step_roofline"]["frac"]}
        log("sweep fused T=%d: %.4f ms/step, %.1f tokens/s" % (T, r["ms_per_step"], r["value"]))
        del t2
    return out


def measure_pack(launches, experts=32):
    """Expert layout conversion (moe_pack_expert / moe_unpack_expert) at the GLM-5 expert
    shape (d 6144, I 2048, bf16): HBM roofline with algorithmic bytes = each expert's
    three matrices read once and written once, over `experts` experts per pass."""
    import torch
    import mixture_experts_transformer_rmsnorm_amd as moe
    d, I = 6144, 2048
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    hf = [torch.randn((experts, I, d), generator=g, device="cuda").to(torch.bfloat16),
          torch.randn((experts, I, d), generator=g, device="cuda").to(torch.bfloat16),
          torch.randn((experts, d, I), generator=g, device="cuda").to(torch.bfloat16)]
    gu = torch.empty((experts, d, 2 * I), dtype=torch.bfloat16, device="cuda")
    dn = torch.empty((experts, I, d), dtype=torch.bfloat16, device="cuda")
    back = [torch.empty_like(t) for t in hf]
    out = {}
    nbytes = 2 * 3 * experts * d * I * 2
    for name in ("pack", "unpack"):
        def one_pass():
            for e in range(experts):
                if name == "pack":
                    moe.moe_pack_expert(None, moe.MOE_DTYPE_BF16, d, I, hf[0][e], hf[1][e], hf[2][e],
                                        gu[e], dn[e])
                else:
                    moe.moe_unpack_expert(None, moe.MOE_DTYPE_BF16, d, I, gu[e], dn[e], back[0][e],
                                          back[1][e], back[2][e])
        one_pass()
        passes = max(2, launches // 10)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(passes):
            one_pass()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / passes
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"experts": experts, "dim": d, "moe_inter": I, "ms_per_pass": round(ms, 4),
                     "algorithmic_bytes": nbytes, "GB_per_s": round(gbs, 1),
                     "frac_of_hbm_peak": round(gbs / 8000.0, 4)}
        log("%s %d experts: %.3f ms, %.1f GB/s" % (name, experts, ms, gbs))
    ok = all(torch.equal(a, b) for a, b in zip(hf, back))
    out["round_trip_identical"] = bool(ok)
    del hf, gu, dn, back
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="glm5_decode")
    ap.add_argument("--tokens", type=int, default=0,
                    help="run the --config workload at this many tokens instead (named "
                         "<config>_<tokens>tok), e.g. to profile a small decode batch")
    ap.add_argument("--secondary", default="glm5_prefill",
                    help="second workload of the same shape family reported in the line ('' = none)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring the attainable HBM-read and MFMA rates")
    ap.add_argument("--extras", default="norms,dense,pack,sweep,configs",
                    help="comma list of extra measurements put into the line's 'extras' "
                         "('norms', 'dense', 'pack', 'sweep': the block at other batch "
                         "sizes on the headline weights, 'configs': the MFMA-bound prefill "
                         "workloads; '' = none)")
    ap.add_argument("--only-extras", action="store_true",
                    help="measure only the extras and print them as one JSON line (profiling)")
    ap.add_argument("--calib-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size "
                         "kernel for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads

    torch.cuda.set_device(0)
    if args.calib_mib:
        n = args.calib_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: %d bytes read, %d bytes written" % (n, n))
        del src, dst
    extras_req = [e for e in args.extras.split(",") if e]
    peaks = None if args.no_peaks else measure_peaks()

    def run_extras(cfg=None, tin=None):
        ext = {}
        if "sweep" in extras_req and tin is not None:
            ext["batch_sweep"] = measure_sweep(cfg, tin, max(args.steps // 5, 5), 2)
        if "norms" in extras_req:
            ext["rmsnorm"] = measure_norms(max(args.steps // 2, 5))
        if "dense" in extras_req:
            ext["dense_block"] = measure_dense(max(args.steps // 2, 5))
        if "pack" in extras_req:
            ext["expert_pack"] = measure_pack(max(args.steps // 2, 5))
        if "configs" in extras_req:
            ext["prefill_configs"] = measure_configs(cfg, tin, max(args.steps // 5, 5))
        return ext

    if args.only_extras:
        print(json.dumps({"extras": run_extras()}), flush=True)
        return
    cfg = workloads.config(args.config)
    if args.tokens:
        cfg = workloads.config(cfg, T=args.tokens, name="%s_%dtok" % (cfg.name, args.tokens))
    log("drawing %s inputs on the device" % cfg.name)
    tin = workloads.make_torch(cfg, 0, device="cuda", weights="device")
    small = workloads.draw_small(cfg, 0)
    torch.cuda.synchronize()
    log("timing %s: %d warmup + %d steps" % (cfg.name, args.warmup, args.steps))
    res = run_workload(cfg, tin, args.steps, args.warmup)
    log("%s: %.1f tokens/s, %.3f ms/step, gate_up %.3f ms (%s %.1f%%), path %d" % (
        cfg.name, res["value"], res["ms_per_step"], res["roofline"]["kernel_ms"],
        res["roofline"]["bound"], 100 * res["roofline"]["frac"], res["path"]))
    line = {
        "metric": METRIC, "value": round(res["value"], 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 4),
        "ms_per_step_median": round(res["ms_per_step_median"], 4),
        "ms_per_step_min": round(res["ms_per_step_min"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded; random-init weights of the GLM-5 MoE-block shapes)",
        "config": {"workload": cfg.name, "tokens": cfg.T, "dim": cfg.d, "n_experts": cfg.E,
                   "moe_inter": cfg.I, "shared_inter": cfg.Is, "top_k": cfg.k,
                   "routed_scale": cfg.routed_scale, "active_experts": res["roofline"]["active_experts"],
                   "max_expert_load": res["max_load"],
                   "kernel_path": "stream" if res["path"] == 1 else "mfma"},
        "roofline": res["roofline"],
        "step_roofline": res["step_roofline"],
        "stage_ms": res["stage_ms"],
    }
    if peaks:
        line["attainable"] = peaks
    line["expert_load"] = load_summary(res["counts"])
    props = torch.cuda.get_device_properties(0)
    line["env"] = {"device": props.name, "compute_units": props.multi_processor_count,
                   "torch": torch.__version__, "hip": torch.version.hip}
    if args.secondary:
        cfg2 = workloads.config(args.secondary)
        if (cfg2.d, cfg2.E, cfg2.I, cfg2.Is, cfg2.dtype) == (cfg.d, cfg.E, cfg.I, cfg.Is, cfg.dtype):
            tin2 = dict(tin)
            small2 = workloads.draw_small(cfg2, 0)
            for key in ("x", "norm_w", "router_w"):
                tin2[key] = workloads.host_to_torch(small2[key], cfg2.dtype, "cuda")
            tin2["corr_bias"] = torch.from_numpy(small2["corr_bias"]).cuda()
            log("timing %s" % cfg2.name)
            r2 = run_workload(cfg2, tin2, max(args.steps // 2, 5), args.warmup)
            log("%s: %.1f tokens/s, %.3f ms/step, gate_up %.3f ms (%s %.1f%%)" % (
                cfg2.name, r2["value"], r2["ms_per_step"], r2["roofline"]["kernel_ms"],
                r2["roofline"]["bound"], 100 * r2["roofline"]["frac"]))
            line["secondary"] = {"workload": cfg2.name, "tokens": cfg2.T,
                                 "value": round(r2["value"], 1), "unit": "tokens/s",
                                 "ms_per_step": round(r2["ms_per_step"], 4),
                                 "ms_per_step_median": round(r2["ms_per_step_median"], 4),
                                 "ms_per_step_min": round(r2["ms_per_step_min"], 4),
                                 "kernel_path": "stream" if r2["path"] == 1 else "mfma",
                                 "roofline": r2["roofline"], "step_roofline": r2["step_roofline"],
                                 "stage_ms": r2["stage_ms"],
                                 "expert_load": load_summary(r2["counts"])}
            del tin2
    if extras_req:
        line["extras"] = run_extras(cfg, tin)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(cfg, tin, small, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
