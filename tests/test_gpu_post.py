"""The step after the path on the GPU against the CPU oracle: the denoised chunk mapped back
to robot units with quantile statistics and cut to the robot's horizon and width (pi0.5
Design, "Embodiment adapters"; GR00T N1.7, "Policy contract"), and GR00T's increasing
(0 -> 1) schedule through the whole loop.

The unnormalization is elementwise fp32 on the GPU against float64 in the oracle, applied to
the same chunk (the GPU's own): errors stay at fp32 rounding of a few operations."""
import numpy as np
import pytest

import oracle
from flow_matching_vla_amd import fm, workloads as wl
from gpu_util import Case, say

pytestmark = pytest.mark.gpu

TOL_UNNORM = 2e-6   # relative to the larger of |y| and the statistics' range


def _stats(rng, dr, degenerate=()):
    q01 = rng.normal(size=dr).astype(np.float32) - 0.5
    q99 = (q01 + rng.uniform(0.2, 3.0, size=dr)).astype(np.float32)
    for j in degenerate:
        q99[j] = q01[j]
    return q01, q99


def _check(case, kind, hr, dr, degenerate=(), scale=1.0):
    import torch
    rng = np.random.default_rng(100 + 10 * kind + dr)
    chunk = case.gpu_denoise() * scale
    x = torch.from_numpy(np.ascontiguousarray(chunk, np.float32)).cuda()
    q01, q99 = _stats(rng, dr, degenerate)
    case.ctx.set_action_stats(kind, hr, dr, q01, q99)
    y = case.ctx.unnormalize(x, hr, dr)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    ref = oracle.quantile_unnormalize(chunk.astype(np.float32), q01, q99, kind, hr, dr)
    assert y.shape == ref.shape == (case.cfg["batch"], hr, dr)
    err = np.abs(y - ref) / np.maximum(np.maximum(np.abs(ref), np.abs(q99 - q01)), 1.0)
    say(f"  kind {kind} horizon {hr} width {dr}: max scaled error {err.max():.2e}, "
        f"|x| > 1 in {np.mean(np.abs(chunk[:, :hr, :dr]) > 1):.0%} of the kept values")
    assert err.max() <= TOL_UNNORM, err.max()
    return chunk, y, q01, q99


def test_unnormalize_pi05_width_slice():
    # LIBERO-style: 32 padded model dims, the robot's 7 kept, the whole horizon
    c = Case(wl.workload("pi05_b1", n_layers=2, steps=2, batch=2))
    _check(c, fm.UNNORM_QUANTILE_EPS, c.cfg["action_horizon"], 7)
    # every model dim and step kept
    _check(c, fm.UNNORM_QUANTILE_EPS, c.cfg["action_horizon"], c.cfg["action_dim"])
    c.close()


def test_unnormalize_gr00t_clip_horizon_and_degenerate_groups():
    # GR00T LIBERO policy: 16 of the model's 40 steps, 7 dims, clip to [-1, 1] (the chunk is
    # scaled so that a share of values falls outside), two degenerate groups (no guard)
    c = Case(wl.workload("dit_b1", n_layers=2, steps=2))
    chunk, y, q01, q99 = _check(c, fm.UNNORM_QUANTILE_CLIP, 16, 7, degenerate=(2, 5), scale=3.0)
    assert np.all(y[..., 2] == q01[2]) and np.all(y[..., 5] == q01[5])
    assert np.all(y >= np.minimum(q01, q99) - 1e-6) and np.all(y <= np.maximum(q01, q99) + 1e-6)
    c.close()


def test_unnormalize_errors():
    c = Case(wl.workload("pi05_b1", n_layers=1, steps=1))
    H, da = c.cfg["action_horizon"], c.cfg["action_dim"]
    import torch
    x = torch.zeros((1, H, da), dtype=torch.float32, device="cuda")
    with pytest.raises(fm.FMError) as e:
        c.ctx.unnormalize(x, H, 7)
    assert e.value.status == 3   # FM_ERR_STATE: no statistics yet
    q = np.zeros(da + 1, np.float32)
    with pytest.raises(fm.FMError) as e:
        c.ctx.set_action_stats(fm.UNNORM_QUANTILE_EPS, H, da + 1, q, q)
    assert e.value.status == 1   # FM_ERR_INVALID_ARG: wider than the model
    with pytest.raises(fm.FMError) as e:
        c.ctx.set_action_stats(fm.UNNORM_QUANTILE_EPS, H + 1, 7, q[:7], q[:7])
    assert e.value.status == 1   # longer than the model's horizon
    with pytest.raises(fm.FMError) as e:
        c.ctx.set_action_stats(5, H, 7, q[:7], q[:7])
    assert e.value.status == 1   # unknown kind
    c.close()


def test_increasing_schedule_dit():
    # GR00T integrates tau 0 -> 1: the direction is the tau array given to fm_set_schedule
    cfg = wl.workload("dit_b1", n_layers=2)
    T = cfg["steps"]
    tau = (np.arange(T + 1) / T).astype(np.float32)
    c = Case(cfg, tau=tau)
    x_gpu = c.gpu_denoise()
    x_ref = oracle.denoise(cfg, c.w64, c.bound, c.I["x0"], T, tau=tau)
    e = oracle.e_rel(x_gpu, x_ref)
    moved = oracle.e_rel(x_ref, c.I["x0"].astype(np.float64))
    say(f"  tau 0 -> 1, {T} steps: chunk e_rel {e:.3e} (the chunk moved {moved:.3f} from x0)")
    assert e <= 2e-2, e
    c.close()
