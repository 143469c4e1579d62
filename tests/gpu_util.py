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

    def __init__(self, cfg, W=None, I=None, steps=None, tau=None, vis=None, oracle_dtype=np.float64):
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
        # oracle state (float64; float32 for the largest batches, whose oracle agrees with the
        # float64 one to ~1e-6, far inside the 1e-2 bar)
        self.odt = oracle_dtype
        self.w64 = oracle.cast_weights(self.W, oracle_dtype)
        self.set_visibility(vis)
        self.tau64 = oracle.schedule(self.steps, tau, dtype=self.odt)
        self.table, self.tb = oracle.modulation_table(cfg, self.w64, self.tau64) if self.steps else (None, None)
        self._table_r = None   # the bf16 reading's table, on first use

    def set_visibility(self, vis):
        """Per-request visibility on both sides: {"prefix_lens"} or {"text_mask", "image_mask"}
        (None: the whole binding)."""
        vis = vis or {}
        if self.cfg["arch"] == wl.ARCH_PREFIX_JOINT:
            self.ctx.bind_prefix_lengths(vis.get("prefix_lens"))
        else:
            self.ctx.bind_context_masks(vis.get("text_mask"), vis.get("image_mask"))
        self.vis = vis
        self.bound = oracle.bind(self.cfg, self.w64, dict(self.I, **vis), dtype=self.odt)

    def oracle_velocity(self, x, k, trace=None, requests=None, round_acts=False):
        """The oracle's velocity at x for step k (of the given requests only); round_acts: the
        bf16 reading (its own modulation table, computed on first use)."""
        table, tb = self.table, self.tb
        if round_acts:
            if self._table_r is None:
                self._table_r = oracle.modulation_table(self.cfg, self.w64, self.tau64, round_acts=True)
            table, tb = self._table_r
        x = np.asarray(x, self.odt)
        if requests is None:
            return oracle.velocity(self.cfg, self.w64, self.bound, x, table, tb, k, trace, round_acts=round_acts)
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
        return oracle.velocity(cfg, self.w64, bound, x[requests], table, tb, k, trace, round_acts=round_acts)

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


def per_request(got, ref, tol_rel, tol_inf, what):
    """e_rel (vla.cpp Eq. (5)) of every request on its own, each within tol_rel, and its largest
    element error within tol_inf of the request's largest reference magnitude; returns the
    worst (e_rel, e_inf / max|ref|)."""
    worst_rel, worst_inf = 0.0, 0.0
    for b in range(ref.shape[0]):
        er = oracle.e_rel(got[b], ref[b])
        ei = oracle.e_inf(got[b], ref[b]) / float(np.max(np.abs(ref[b])))
        worst_rel, worst_inf = max(worst_rel, er), max(worst_inf, ei)
        assert er <= tol_rel, (what, b, er)
        assert ei <= tol_inf, (what, b, ei)
    return worst_rel, worst_inf


def teacher_forced(case, tol_v, requests=None, layers_trace=False, steps=None, tol_inf=None, round_acts=False):
    """GPU velocity at the GPU's own trajectory x_k vs the oracle velocity at the same x_k, for
    the first `steps` steps (all by default). With tol_inf, every request is checked on its
    own (per_request); else the compared requests together."""
    x = case.I["x0"].astype(np.float32)
    worst = 0.0
    for k in range(case.steps if steps is None else steps):
        v_gpu = case.gpu_velocity(x, k)
        v_ref = case.oracle_velocity(x, k, requests=requests, round_acts=round_acts)
        vg = v_gpu if requests is None else v_gpu[requests]
        e = oracle.e_rel(vg, v_ref)
        say(f"  step {k}: velocity e_rel {e:.3e} e_inf {oracle.e_inf(vg, v_ref):.3e}")
        if tol_inf is not None:
            wr, wi = per_request(vg, v_ref, tol_v, tol_inf, f"velocity step {k}")
            say(f"  step {k}: worst request e_rel {wr:.3e}, worst e_inf / max|v| {wi:.3e}")
            e = wr
        worst = max(worst, e)
        x = (x + np.float32(case.tau64[k + 1] - case.tau64[k]) * v_gpu).astype(np.float32)
    assert worst <= tol_v, worst
    return worst


def chunk(case, tol_x, requests=None, tol_inf=None):
    x_gpu = case.gpu_denoise()
    I = case.I
    if requests is not None:
        x_ref = oracle.denoise(dict(case.cfg, batch=len(requests)), case.w64,
                               {k: ([a[requests] for a in v] if isinstance(v, list) else
                                    ({i: a[requests] for i, a in v.items()} if isinstance(v, dict) else
                                     (v[requests] if isinstance(v, np.ndarray) else v)))
                                for k, v in case.bound.items()},
                               I["x0"][requests], case.steps, tau=case.tau, dtype=case.odt)
        x_gpu = x_gpu[requests]
    else:
        x_ref = oracle.denoise(case.cfg, case.w64, case.bound, I["x0"], case.steps, tau=case.tau, dtype=case.odt)
    e = oracle.e_rel(x_gpu, x_ref)
    say(f"  chunk e_rel {e:.3e} e_inf {oracle.e_inf(x_gpu, x_ref):.3e}")
    if tol_inf is not None:
        wr, wi = per_request(x_gpu, x_ref, tol_x, tol_inf, "chunk")
        say(f"  chunk: worst request e_rel {wr:.3e}, worst e_inf / max|x| {wi:.3e}")
    assert e <= tol_x, e
    return x_gpu
