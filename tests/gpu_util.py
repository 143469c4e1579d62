"""Shared set-up of the GPU parity tests: seeded inputs from the workload generator go
both to the CPU oracle (float64) and, through the C-ABI binding, to the HIP library."""
import sys

import numpy as np

import oracle
from flow_matching_vla_amd import workloads as wl


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


class Case:
    """One workload: host weights/inputs, the oracle's bound state, and a GPU context."""

    def __init__(self, cfg, W=None, I=None, steps=None, tau=None, vis=None):
        import torch
        from flow_matching_vla_amd import fm

        self.cfg = cfg
        self.W = wl.make_weights(cfg) if W is None else W
        self.I = wl.make_inputs(cfg) if I is None else I
        self.steps = cfg["steps"] if steps is None else steps
        self.tau = tau
        dt = cfg["dtype"]
        say("case", cfg["name"], {k: cfg[k] for k in ("n_layers", "hidden", "batch", "prefix_len", "ctx_len", "steps")})
        self.ctx = fm.Context(cfg)
        wt = {n: fm.to_device(a, dt) for n, a in self.W.items()}
        self.ctx.load_weights(wt)
        B = cfg["batch"]
        if cfg["arch"] == wl.ARCH_PREFIX_JOINT:
            L = cfg["n_layers"]
            k = [fm.to_device(self.I[f"prefix.k.{l}"], dt) for l in range(L)]
            v = [fm.to_device(self.I[f"prefix.v.{l}"], dt) for l in range(L)]
            self.ctx.bind_prefix_kv(B, cfg["prefix_len"], k, v)
        else:
            self.ctx.bind_prefix_kv(B, cfg["ctx_len"], context=fm.to_device(self.I["context"], dt),
                                    state=fm.to_device(self.I["state"], fm.F32))
        self.ctx.set_schedule(self.steps, B, tau)
        torch.cuda.synchronize()
        del wt
        self.x0 = torch.from_numpy(self.I["x0"]).cuda()
        # oracle state (float64)
        self.w64 = oracle.cast_weights(self.W)
        self.set_visibility(vis)
        self.tau64 = oracle.schedule(self.steps, tau)
        self.table, self.tb = oracle.modulation_table(cfg, self.w64, self.tau64) if self.steps else (None, None)

    def set_visibility(self, vis):
        """Per-request visibility on both sides: {"prefix_lens"} or {"text_mask", "image_mask"}
        (None: the whole binding)."""
        vis = vis or {}
        if self.cfg["arch"] == wl.ARCH_PREFIX_JOINT:
            self.ctx.bind_prefix_lengths(vis.get("prefix_lens"))
        else:
            self.ctx.bind_context_masks(vis.get("text_mask"), vis.get("image_mask"))
        self.vis = vis
        self.bound = oracle.bind(self.cfg, self.w64, dict(self.I, **vis))

    def oracle_velocity(self, x, k, trace=None, requests=None):
        if requests is None:
            return oracle.velocity(self.cfg, self.w64, self.bound, np.asarray(x, np.float64), self.table, self.tb, k, trace)
        cfg = dict(self.cfg, batch=len(requests))
        bound = {}
        for key, val in self.bound.items():
            if isinstance(val, list):
                bound[key] = [a[requests] for a in val]
            elif isinstance(val, dict):
                bound[key] = {i: a[requests] for i, a in val.items()}
            elif isinstance(val, np.ndarray):
                bound[key] = val[requests]
            else:
                bound[key] = val
        return oracle.velocity(cfg, self.w64, bound, np.asarray(x, np.float64)[requests], self.table, self.tb, k, trace)

    def gpu_velocity(self, x_np, k):
        import torch
        x = torch.from_numpy(np.ascontiguousarray(x_np, dtype=np.float32)).cuda()
        v = self.ctx.step_velocity(x, k)
        torch.cuda.synchronize()
        return v.cpu().numpy()

    def gpu_denoise(self):
        import torch
        out = self.ctx.denoise(self.x0, self.steps)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def close(self):
        self.ctx.close()


def teacher_forced(case, tol_v, requests=None, layers_trace=False):
    """GPU velocity at the GPU's own trajectory x_k vs the oracle velocity at the same x_k."""
    x = case.I["x0"].astype(np.float32)
    worst = 0.0
    for k in range(case.steps):
        v_gpu = case.gpu_velocity(x, k)
        v_ref = case.oracle_velocity(x, k, requests=requests)
        vg = v_gpu if requests is None else v_gpu[requests]
        e = oracle.e_rel(vg, v_ref)
        say(f"  step {k}: velocity e_rel {e:.3e} e_inf {oracle.e_inf(vg, v_ref):.3e}")
        worst = max(worst, e)
        x = (x + np.float32(case.tau64[k + 1] - case.tau64[k]) * v_gpu).astype(np.float32)
    assert worst <= tol_v, worst
    return worst


def chunk(case, tol_x, requests=None):
    x_gpu = case.gpu_denoise()
    I = case.I
    if requests is not None:
        x_ref = oracle.denoise(dict(case.cfg, batch=len(requests)), case.w64,
                               {k: ([a[requests] for a in v] if isinstance(v, list) else
                                    ({i: a[requests] for i, a in v.items()} if isinstance(v, dict) else
                                     (v[requests] if isinstance(v, np.ndarray) else v)))
                                for k, v in case.bound.items()},
                               I["x0"][requests], case.steps, tau=case.tau)
        x_gpu = x_gpu[requests]
    else:
        x_ref = oracle.denoise(case.cfg, case.w64, case.bound, I["x0"], case.steps, tau=case.tau)
    e = oracle.e_rel(x_gpu, x_ref)
    say(f"  chunk e_rel {e:.3e} e_inf {oracle.e_inf(x_gpu, x_ref):.3e}")
    assert e <= tol_x, e
    return x_gpu
