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

    def __init__(self, cfg, W=None, I=None, steps=None, tau=None):
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
        self.bound = oracle.bind(cfg, self.w64, self.I)
        self.tau64 = oracle.schedule(self.steps, tau)
        self.table, self.tb = oracle.modulation_table(cfg, self.w64, self.tau64) if self.steps else (None, None)

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
