#!/usr/bin/env python3
"""Throughput of the flow-matching denoise loop on one MI355X.

One bench step is one fm_denoise call: the whole T-step Euler loop of the action expert
over one batch of seeded synthetic inputs already resident in HBM (weights, bound prefix
K/V, x0), run as one launch of the persistent loop kernel where it applies (batch x
horizon <= 64 rows) or else replayed as one hipGraph of per-operation kernels. The default
workload is the pi0.5-shaped expert at batch 1, prefix 816, horizon 50, 10 Euler steps.
Prints one JSON line.

Besides chunks/s it reports: a linear fit of latency over the step count T (the model
latency P + T E of the vla.cpp paper, Sec. III-B Eq. (3)); the whole loop's algorithmic
HBM rate; a roofline entry for the dominant kernel (the loop kernel's one launch, or the
per-operation role that takes the most time), timed with HIP events around its launches on
the context stream; and the CPU oracle timed on the host cores on a bounded sample of the
same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3
METRIC = "action chunks/sec (10-step denoise) + per-step latency; % HBM / MFMA peak"

DESCRIPTIONS = {
    "tiny_fp32": "tiny fp32 expert: 2 layers, hidden 256, 4x64 q heads, 1 KV head, prefix 64, horizon 16, dim 7, 4 steps",
    "pi05_b1": "pi0.5-shaped action expert: 18 layers, hidden 1024, 8x256 q heads, 1 KV head, gated-GELU 4096, RoPE, prefix 816, horizon 50, dim 32, batch 1, 10 Euler steps",
    "pi05_b8": "pi0.5-shaped action expert, batch 8, prefix 816, 10 Euler steps",
    "dit_b1": "DiT action head: 32 blocks, hidden 1536, 24x64 heads, AdaLN, cross-attention to 600x2048 context, horizon 40 + 1 state token, batch 1, 4 Euler steps",
    "pi05_b64": "pi0.5-shaped action expert, batch 64, prefix 1024, 10 Euler steps",
}


def role_bytes_flops(cfg, role):
    """Algorithmic bytes and flops of one launch of a role at one Euler step: weights (and the
    bound K/V for attention) read once, plus the modulation vectors; activations between
    kernels are not counted (they can stay on chip)."""
    e = 2 if cfg["dtype"] == 1 else 4
    D, F, L = cfg["hidden"], cfg["mlp_dim"], cfg["n_layers"]
    w8 = cfg.get("w8", False)   # FP8 per-layer matrices: 1 byte per weight + a 4-byte scale per row
    B, H, da = cfg["batch"], cfg["action_horizon"], cfg["action_dim"]
    nq, dh = cfg["n_heads"], cfg["head_dim"]
    st = cfg.get("state_tokens", 0)
    M = B * (st + H)
    if cfg["arch"] == 0:
        qd = nq * dh
        keys = cfg["prefix_len"] + H
        nup = 2 * F if cfg["mlp_gated"] else F
        shapes = {   # (weights, modulation floats, weight rows)
            "qkv": ((qd + 2 * dh) * D, 2 * D, qd + 2 * dh), "oproj": (D * qd, D, D), "mlp_up": (nup * D, 2 * D, nup),
            "mlp_down": (D * F, D, D), "out": (da * D, 2 * D, 0), "inproj": (D * da, 0, 0),
        }
        if role == "attn":
            return B * keys * dh * 2 * e, B * 4 * nq * H * keys * dh
        w, mod, rows = shapes[role]
        Mr = B * H
        wb = w + 4 * rows if (w8 and rows) else w * e
        return wb + mod * 4, 2 * w * Mr
    # DiT: per-role averages over the two block kinds
    S = cfg["ctx_len"]
    if role == "qkv":
        w, rows = (D * D + 3 * D * D) / 2, (D + 3 * D) / 2
        return (w + 4 * rows if w8 else w * e) + 2 * D * 4, 2 * w * M
    if role == "attn":
        kv = (B * S * D * 2 * e + 0) / 2
        fl = (4 * B * (st + H) * S * D + 4 * B * (st + H) ** 2 * D) / 2
        return kv, fl
    w, rows = {"oproj": (D * D, D), "mlp_up": (F * D, F), "mlp_down": (D * F, D), "out": (da * D, 0),
               "inproj": (D * da, 0)}[role]
    return (w + 4 * rows if (w8 and rows) else w * e), 2 * w * M


def step_bytes_flops(cfg):
    """Algorithmic bytes / flops of one Euler step (all layers)."""
    L = cfg["n_layers"]
    tb, tf = 0.0, 0.0
    for r in ("qkv", "attn", "oproj", "mlp_up", "mlp_down"):
        b, f = role_bytes_flops(cfg, r)
        tb += L * b
        tf += L * f
    for r in ("out", "inproj"):
        b, f = role_bytes_flops(cfg, r)
        tb += b
        tf += f
    return tb, tf


HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(HERE, "profiles", "{}_loop_kernel_hbm_traffic.txt")
MFMA_FILE = os.path.join(HERE, "profiles", "{}_mfma_counters.txt")


def loop_traffic(workload):
    """HBM bytes per loop-kernel launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary of this workload, or None when there is none or the kernel source has changed
    since those counters were taken (the summary records the source hash)."""
    from flow_matching_vla_amd import profiling
    path = TRAFFIC_FILE.format(workload)
    if not os.path.exists(path):
        return None
    vals = {}
    for ln in open(path):
        if ":" in ln and not ln.startswith("#"):
            k, v = ln.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != profiling.loop_source_hash() or "traffic_bytes_per_launch" not in vals:
        return None
    return int(float(vals["traffic_bytes_per_launch"]))


def measured_ceilings():
    """Ceilings measured on this device with the platform's own routines, beside the nominal
    peaks: a 1 GiB device-to-device copy (bytes read + written per second) and a bf16
    8192 x 8192 x 8192 matrix product (torch.matmul), each the best of 20 timed runs."""
    import torch
    nb = 1 << 30
    src = torch.empty(nb, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)

    def best(fn, n=20):
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) * 1e-3)
        return min(out)
    t_copy = best(lambda: dst.copy_(src))
    t_mm = best(lambda: torch.matmul(a, b))
    r = {"copy_GBps": round(2 * nb / t_copy / 1e9, 1), "bf16_gemm_TFLOPs": round(2 * 8192 ** 3 / t_mm / 1e12, 1),
         "how": "1 GiB device copy (read + write) and torch.matmul bf16 8192^3, best of 20"}
    del src, dst, a, b
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return r


def mfma_counters(workload):
    """MFMA busy share of the per-operation kernels from the committed rocprofv3 counter
    summary of this workload (time-weighted over the kernels that issue MFMAs), or None when
    there is none or the kernel sources have changed since the counters were taken."""
    from flow_matching_vla_amd import profiling
    path = MFMA_FILE.format(workload)
    if not os.path.exists(path):
        return None
    vals = {}
    for ln in open(path):
        if ":" in ln and not ln.startswith("#") and not ln.startswith("void") and not ln.startswith("_Z"):
            k, v = ln.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != profiling.graph_source_hash() or "mfma_busy_pct_time_weighted" not in vals:
        return None
    return {"busy_frac_time_weighted": round(float(vals["mfma_busy_pct_time_weighted"]) / 100, 4),
            "counters": "SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16", "file": os.path.relpath(path, HERE)}


def cpu_baseline(cfg, W, I, budget_s=12.0):
    """The oracle as it stands, timed on the host in float32 (numpy, BLAS threads = the
    visible cores): Euler steps of the same workload, whole chunks one after another, until
    about budget_s of CPU work has been done (at least one step). chunks/s = batch / (mean
    step time x T); when the budget ends inside the first chunk the figure is extrapolated
    from the steps done, and the sample says so. The schedule table and the binding are
    computed before the timed region."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
        blas = ",".join(sorted({p.get("internal_api", "?") for p in threadpool_info() if p.get("user_api") == "blas"}))
    except Exception:
        threads, blas = os.cpu_count(), "unknown"
    T, B = cfg["steps"], cfg["batch"]
    f32 = np.float32
    w = oracle.cast_weights(W, f32)
    bound = oracle.bind(cfg, w, I, dtype=f32)
    tau = oracle.schedule(T, dtype=f32)
    table, tb = oracle.modulation_table(cfg, w, tau)
    x = np.array(I["x0"], dtype=f32)
    n = 0
    t0 = time.perf_counter()
    while True:
        k = n % T
        if k == 0:
            x = np.array(I["x0"], dtype=f32)
        x = x + (tau[k + 1] - tau[k]) * oracle.velocity(cfg, w, bound, x, table, tb, k)
        n += 1
        if time.perf_counter() - t0 > budget_s and (n % T == 0 or n < T):
            break
    dt = time.perf_counter() - t0
    whole = n // T
    how = (f"{whole} whole chunk(s)" if n % T == 0 else
           f"{n} of the {T} Euler steps of one chunk, extrapolated to the chunk")
    return {
        "value": round(B / (dt / n * T), 4), "unit": "chunks/s", "cores": int(threads), "kind": "oracle",
        "sample": f"{how} of {cfg['name']} (batch {B}), float32 numpy ({blas}, {threads} threads; "
                  f"{os.cpu_count()} CPUs visible), table and bind excluded, {dt:.1f} s",
    }


def time_calls(ctx, x0, T, out, n, stream):
    """n back-to-back fm_denoise calls with a HIP event on the context stream before each call
    and after the last: per-call latencies (ms) between consecutive events, and the wall time
    of the whole bracket (synchronized on both sides)."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        evs[i].record(stream)
        ctx.denoise(x0, T, out)
    evs[n].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [evs[i].elapsed_time(evs[i + 1]) for i in range(n)], wall


def latency_summary(lat):
    import numpy as np
    a = np.asarray(lat, float)
    return {"p50_ms": round(float(np.percentile(a, 50)), 4), "p90_ms": round(float(np.percentile(a, 90)), 4),
            "mean_ms": round(float(a.mean()), 4), "calls": int(a.size)}


def bound_of(cfg, seconds_per_step):
    """Fraction of the Euler step's own roofline bound: algorithmic bytes over 8 TB/s or flops
    over the dtype's dense MFMA peak, whichever bound is larger."""
    b, f = step_bytes_flops(cfg)
    peak_f = (BF16_PEAK_TFLOPS if cfg["dtype"] == 1 else FP32_PEAK_TFLOPS) * 1e12
    t_hbm, t_mfma = b / (HBM_PEAK_GBS * 1e9), f / peak_f
    kind = "hbm" if t_hbm >= t_mfma else "mfma"
    return {"bound": kind, "frac": round((t_hbm if kind == "hbm" else t_mfma) / seconds_per_step, 4),
            "hbm_frac": round(t_hbm / seconds_per_step, 4), "mfma_frac": round(t_mfma / seconds_per_step, 4),
            "alg_bytes_per_euler_step": int(b), "alg_flops_per_euler_step": int(f),
            "floor_us_per_euler_step": round(max(t_hbm, t_mfma) * 1e6, 2)}


def make_context(cfg, W, I, fmt_fp8=False):
    """Context with weights loaded, the seeded prefix (or context and state) bound and the
    schedule set; returns (ctx, bind callable)."""
    import torch
    from flow_matching_vla_amd import fm
    dt, B = cfg["dtype"], cfg["batch"]
    ctx = fm.Context(cfg)
    if fmt_fp8:
        ctx.set_weight_format(fm.WEIGHTS_FP8_E4M3)
    wt = {n: fm.to_device(a, dt) for n, a in W.items()}
    ctx.load_weights(wt)
    del wt
    if cfg["arch"] == 0:
        L = cfg["n_layers"]
        kk = [fm.to_device(I[f"prefix.k.{l}"], dt) for l in range(L)]
        vv = [fm.to_device(I[f"prefix.v.{l}"], dt) for l in range(L)]

        def bind():
            ctx.bind_prefix_kv(B, cfg["prefix_len"], kk, vv)
    else:
        zc, st = fm.to_device(I["context"], dt), fm.to_device(I["state"], fm.F32)

        def bind():
            ctx.bind_prefix_kv(B, cfg["ctx_len"], context=zc, state=st)
    bind()
    torch.cuda.synchronize()
    ctx.set_schedule(cfg["steps"], B)
    return ctx, bind


def dominant_role(ctx, cfg, x0, out):
    """Per-operation roles timed with events around every launch (eager replay); the role with
    the largest time per chunk and its fraction of its own bound."""
    from flow_matching_vla_amd import fm
    T, dt = cfg["steps"], cfg["dtype"]
    roles = {}
    for r in ("inproj", "qkv", "attn", "oproj", "mlp_up", "mlp_down", "out"):
        tot, nl = 0.0, 0
        for _ in range(3):
            m, n = fm.profile_loop(ctx, x0, T, r, out)
            tot += m
            nl += n
        roles[r] = (tot / nl, nl // 3)
    dom = max(roles, key=lambda r: roles[r][0] * roles[r][1])
    nbytes, nflops = role_bytes_flops(cfg, dom)
    avg_s = roles[dom][0] * 1e-3
    ridge = (BF16_PEAK_TFLOPS * 1e12) / (HBM_PEAK_GBS * 1e9)
    if nflops / max(nbytes, 1) < ridge:
        ach = nbytes / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "kernel_role": dom,
                "alg_bytes_per_launch": int(nbytes), "avg_launch_us": round(avg_s * 1e6, 2),
                "launches_per_chunk": roles[dom][1]}
    else:
        peak = BF16_PEAK_TFLOPS if dt == 1 else FP32_PEAK_TFLOPS
        ach = nflops / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "traffic": None, "kernel_role": dom,
                "alg_flops_per_launch": int(nflops), "avg_launch_us": round(avg_s * 1e6, 2),
                "launches_per_chunk": roles[dom][1]}
    return {r: round(v[0] * 1000, 2) for r, v in roles.items()}, roof


def bench_other(name, calls, cpu_budget):
    """One of the other workloads, in the same run: chunks/s, p50 / p90 chunk latency, the
    Euler step against its own roofline bound, the dominant kernel role where the per-operation
    graph serves it, and the oracle on a bounded sample. Every device object is released
    before returning."""
    import torch
    from flow_matching_vla_amd import workloads as wl
    cfg = wl.workload(name)
    T, B = cfg["steps"], cfg["batch"]
    print(f"[bench] {name}: generating seeded inputs", file=sys.stderr, flush=True)
    W, I = wl.make_weights(cfg), wl.make_inputs(cfg)
    ctx, _ = make_context(cfg, W, I)
    x0 = torch.from_numpy(I["x0"]).cuda()
    out = torch.empty_like(x0)
    for _ in range(5):
        ctx.denoise(x0, T, out)
    lat, wall = time_calls(ctx, x0, T, out, calls, ctx.stream)
    summ = latency_summary(lat)
    persistent, _ = ctx.loop_status()
    r = {"workload": f"{name}: {DESCRIPTIONS[name]}", "chunks_per_s": round(B * calls / wall, 3),
         "latency": summ, "per_euler_step_us": round(1000 * summ["p50_ms"] / T, 2),
         "path": "loop kernel (one launch per chunk)" if persistent else "hipGraph of per-operation kernels",
         "step_roofline": bound_of(cfg, summ["p50_ms"] * 1e-3 / T)}
    if not persistent:
        roles, roof = dominant_role(ctx, cfg, x0, out)
        r["roles_us_per_launch"], r["roofline"] = roles, roof
        mc = mfma_counters(name)
        if mc is not None:
            r["mfma_counters"] = mc
    print(f"[bench] {name}: {summ['p50_ms']:.3f} ms per chunk (p50), {r['chunks_per_s']:.1f} chunks/s",
          file=sys.stderr, flush=True)
    ctx.close()
    del x0, out, ctx
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if cpu_budget > 0:
        r["cpu_baseline"] = cpu_baseline(cfg, W, I, cpu_budget)
    return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="timed fm_denoise calls")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="pi05_b1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fit", action="store_true")
    ap.add_argument("--no-roles", action="store_true")
    ap.add_argument("--no-visibility", action="store_true")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8-weights line of bf16 workloads")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads' entries")
    ap.add_argument("--weights", choices=("as-given", "fp8"), default="as-given",
                    help="fp8: the expert's per-layer matrices as FP8 E4M3 codes with per-row scales")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="for rocprofv3 --pmc runs: a plain 512 MiB device copy (3x, the counter scale) "
                         "then 3 chunk calls; prints no JSON")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build runs on one GPU only (asked for {max(args.gpus, world)}); "
              "the loop shards by request with no exchange, see the design notes.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from flow_matching_vla_amd import fm, workloads as wl

    cfg = wl.workload(args.workload)
    if args.weights == "fp8":
        cfg["w8"] = True
    T, B = cfg["steps"], cfg["batch"]
    dt = cfg["dtype"]
    print(f"[bench] {cfg['name']}: generating seeded inputs", file=sys.stderr, flush=True)
    W, I = wl.make_weights(cfg), wl.make_inputs(cfg)
    torch.cuda.set_device(0)
    ctx, bind = make_context(cfg, W, I, fmt_fp8=args.weights == "fp8")
    x0 = torch.from_numpy(I["x0"]).cuda()
    out = torch.empty_like(x0)
    stream = ctx.stream
    if args.pmc_probe:
        nb = 512 << 20
        src = torch.ones(nb, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        for _ in range(3):
            ctx.denoise(x0, T, out)
        torch.cuda.synchronize()
        ctx.close()
        print(f"[bench] pmc probe done: copy {nb} bytes x3, {cfg['name']} x3", file=sys.stderr, flush=True)
        return
    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        ctx.denoise(x0, T, out)
    torch.cuda.synchronize()

    lat, wall = time_calls(ctx, x0, T, out, args.steps, stream)
    ms = sum(lat) / len(lat)
    value = B * args.steps / wall
    print(f"[bench] {ms:.3f} ms per chunk call ({value:.1f} chunks/s)", file=sys.stderr, flush=True)

    step_b, step_f = step_bytes_flops(cfg)
    res = {
        "metric": METRIC, "value": round(value, 3), "unit": "chunks/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if dt == 1 else "f32", "data": "synthetic (seeded, random-init)",
        "config": {"workload": f"{cfg['name']}: {DESCRIPTIONS[cfg['name']]}", "batch": B, "euler_steps": T,
                   "prefix_len": cfg["prefix_len"], "action_horizon": cfg["action_horizon"],
                   "action_dim": cfg["action_dim"], "parallelism": "none (1 GPU)",
                   "weights": "fp8-e4m3, per-row power-of-two scale" if args.weights == "fp8" else "as given"},
        "per_euler_step_us": round(1000 * ms / T, 2),
        "latency": latency_summary(lat),
        "loop": {"alg_bytes_per_euler_step": int(step_b), "alg_flops_per_euler_step": int(step_f),
                 "achieved_GBps": round(step_b * T / (ms * 1e-3) / 1e9, 1),
                 "hbm_frac": round(step_b * T / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "achieved_TFLOPs": round(step_f * T / (ms * 1e-3) / 1e12, 2),
                 "mfma_frac": round(step_f * T / (ms * 1e-3) / 1e12 / (BF16_PEAK_TFLOPS if dt == 1 else FP32_PEAK_TFLOPS), 4)},
    }
    # latency vs step count: L(T) = P + T E
    if not args.no_fit and T > 1:
        pts = []
        for t in sorted({1, 2, max(1, T // 2), T}):
            ctx.set_schedule(t, B)
            for _ in range(5):
                ctx.denoise(x0, t, out)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(20):
                ctx.denoise(x0, t, out)
            b.record(stream)
            torch.cuda.synchronize()
            pts.append((t, a.elapsed_time(b) / 20))
        ts = np.array([p[0] for p in pts], float)
        ls = np.array([p[1] for p in pts], float)
        E, P0 = np.polyfit(ts, ls, 1)
        res["latency_fit"] = {"points_ms": [[int(t), round(l, 4)] for t, l in pts], "P_ms": round(float(P0), 4),
                              "E_us_per_step": round(float(E) * 1000, 2)}
        ctx.set_schedule(T, B)
    persistent, _ = ctx.loop_status()
    res["loop_kernel"] = bool(persistent)
    # kernel time inside the loop, with HIP events on the context stream: the loop kernel's
    # single launch when it serves the workload, else each per-operation role (eager)
    if not args.no_roles and persistent:
        tot, nl = 0.0, 0
        for _ in range(5):
            m, n = fm.profile_loop(ctx, x0, T, "loop", out)
            tot += m
            nl += n
        avg_s = tot / nl * 1e-3
        nbytes, nflops = step_b * T, step_f * T
        ach = nbytes / avg_s / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": loop_traffic(cfg["name"] + ("_fp8" if args.weights == "fp8" else "")), "kernel": "k_xloop",
                           "alg_bytes_per_launch": int(nbytes), "avg_launch_us": round(avg_s * 1e6, 2),
                           "launches_per_chunk": 1, "mfma_TFLOPs": round(nflops / avg_s / 1e12, 2)}
    if not args.no_roles and not persistent:
        roles, roof = dominant_role(ctx, cfg, x0, out)
        res["roles_us_per_launch"] = roles
        res["roofline_kernel_role"] = roof["kernel_role"]
        res["roofline"] = roof
    mc = mfma_counters(cfg["name"]) if args.weights == "as-given" and not persistent else None
    if mc is not None:
        res["mfma_counters"] = mc
    # per-request visibility: the workload's seeded mixed batch (ragged compact prefixes for
    # pi0.5, text / image masks for DiT), same binding, timed like the main loop
    vis = None if args.no_visibility else wl.make_visibility(cfg)
    if vis is not None and (cfg["arch"] != 0 or bool(np.any(vis["prefix_lens"] < cfg["prefix_len"]))):
        if cfg["arch"] == 0:
            ctx.bind_prefix_lengths(vis["prefix_lens"])
            desc = {"prefix_lens_mean": round(float(vis["prefix_lens"].mean()), 1), "prefix_len": cfg["prefix_len"]}
        else:
            ctx.bind_context_masks(vis["text_mask"], vis["image_mask"])
            desc = {"text_visible_mean": round(float(vis["text_mask"].sum(1).mean()), 1),
                    "image_visible_mean": round(float(vis["image_mask"].sum(1).mean()), 1), "ctx_len": cfg["ctx_len"]}
        for _ in range(3):
            ctx.denoise(x0, T, out)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(20):
            ctx.denoise(x0, T, out)
        b.record(stream)
        torch.cuda.synchronize()
        vms = a.elapsed_time(b) / 20
        res["visibility"] = dict(desc, ms_per_chunk=round(vms, 4), chunks_per_s=round(B / (vms * 1e-3), 2),
                                 ms_per_chunk_whole_binding=round(ms, 4))
        if cfg["arch"] == 0:
            ctx.bind_prefix_lengths(None)
        else:
            ctx.bind_context_masks(None, None)
    # the same workload with the per-layer matrices as FP8 codes (a separate model: reported
    # beside the bf16 line, never as its value)
    if dt == 1 and args.weights == "as-given" and not args.no_fp8:
        c8, _ = make_context(cfg, W, I, fmt_fp8=True)
        o8 = torch.empty_like(x0)
        for _ in range(5):
            c8.denoise(x0, T, o8)
        torch.cuda.synchronize()
        a8, b8 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a8.record(c8.stream)
        for _ in range(args.steps):
            c8.denoise(x0, T, o8)
        b8.record(c8.stream)
        torch.cuda.synchronize()
        ms8 = a8.elapsed_time(b8) / args.steps
        ctx.denoise(x0, T, out)   # the bf16 model's chunk on the whole binding
        torch.cuda.synchronize()
        b8y, _ = step_bytes_flops(dict(cfg, w8=True))
        res["fp8_weights"] = {"chunks_per_s": round(B / (ms8 * 1e-3), 2), "per_euler_step_us": round(1000 * ms8 / T, 2),
                              "alg_bytes_per_euler_step": int(b8y), "loop_kernel": bool(c8.loop_status()[0]),
                              "traffic": loop_traffic(cfg["name"] + "_fp8"),
                              "chunk_e_rel_vs_bf16_weights": round(float(torch.linalg.vector_norm(o8 - out) / torch.linalg.vector_norm(out)), 5)}
        c8.close()
        del o8, c8
    # the step after the path: the chunk back to robot units (LIBERO width 7; GR00T's policy
    # keeps 16 of the model's 40 steps), timed with HIP events on the context stream
    post_kind = fm.UNNORM_QUANTILE_EPS if cfg["arch"] == 0 else fm.UNNORM_QUANTILE_CLIP
    post_h = cfg["action_horizon"] if cfg["arch"] == 0 else min(16, cfg["action_horizon"])
    post_d = min(7, cfg["action_dim"])
    q01 = -np.linspace(1.0, 2.0, post_d, dtype=np.float32)
    q99 = np.linspace(1.0, 3.0, post_d, dtype=np.float32)
    ctx.set_action_stats(post_kind, post_h, post_d, q01, q99)
    ctx.denoise(x0, T, out)
    robot = ctx.unnormalize(out, post_h, post_d)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(200):
        ctx.unnormalize(out, post_h, post_d, robot)
    b.record(stream)
    torch.cuda.synchronize()
    post_us = a.elapsed_time(b) / 200 * 1000
    post_bytes = 2 * B * post_h * post_d * 4 + 2 * post_d * 4
    res["post"] = {"kernel": "k_unnormalize", "kind": "quantile+eps (pi0.5)" if post_kind == 0 else "quantile clip (GR00T)",
                   "robot_horizon": post_h, "robot_dim": post_d, "us_per_chunk": round(post_us, 2),
                   "alg_bytes": int(post_bytes), "achieved_GBps": round(post_bytes / (post_us * 1e-6) / 1e9, 2)}
    # off the step path: the per-observation binding (prefix K/V copy into the pool, or the
    # DiT context projected to every cross block's K / V) and the per-schedule table; each
    # call synchronizes the stream before returning
    def per_call_ms(fn, n):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return round((time.perf_counter() - t0) / n * 1e3, 3)
    res["bind_ms"] = per_call_ms(bind, 5)
    res["measured_ceilings"] = measured_ceilings()
    res["schedule_ms"] = per_call_ms(lambda: ctx.set_schedule(T, B), 3)
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(cfg, W, I)
        import oracle
        chunk = out.cpu().numpy()
        t1 = time.perf_counter()
        for _ in range(100):
            oracle.quantile_unnormalize(chunk, q01, q99, post_kind, post_h, post_d)
        res["post"]["oracle_us"] = round((time.perf_counter() - t1) / 100 * 1e6, 2)
    # release every device object of this workload before the next one (and before exit: the
    # interpreter then tears down nothing of this library's)
    ctx.close()
    del ctx, bind, x0, out, robot
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_configs and args.workload == "pi05_b1" and args.weights == "as-given":
        res["configs"] = {}
        for name, calls, cb in (("tiny_fp32", 100, 3.0), ("pi05_b8", 100, 4.0), ("dit_b1", 100, 4.0), ("pi05_b64", 100, 6.0)):
            res["configs"][name] = bench_other(name, calls, 0.0 if args.no_cpu_baseline else cb)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
