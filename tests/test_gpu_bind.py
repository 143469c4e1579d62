"""The step before the path on the GPU.

  * In-place binding: a producer writes every layer's prefix K/V straight into the library's
    pool through fm_prefix_kv_slot, in the layout fm_pool_k_col / fm_pool_v_slot give, and
    fm_bind_prefix_inplace binds it without a copy (pi0.5 Design, "Attention and the K/V
    pool"). The result must equal the copying bind bit for bit: the pool holds the same bytes
    either way. The producer's rows must be unchanged after the loop.
  * DiT context projection: every cross block's K_c = Z W_K^T and V_c = Z W_V^T come from two
    GEMMs over the stacked weights at bind (GR00T N1.7, "vl_backbone"). Checked against the
    oracle with a bound context shorter than the capacity and several requests, in fp32
    (relative L2 <= 1e-4) and bf16 (<= 1e-2 per teacher-forced step, <= 2e-2 on the chunk)."""
import numpy as np
import pytest

from flow_matching_vla_amd import fm, workloads as wl
from gpu_util import Case, say, teacher_forced, chunk

pytestmark = pytest.mark.gpu


def _write_prefix(ctx, cfg, I):
    """The producer: layer l's prefix keys / values written into the pool views in place."""
    import torch
    B, P, dh, L = cfg["batch"], cfg["prefix_len"], cfg["head_dim"], cfg["n_layers"]
    tdt = torch.bfloat16 if cfg["dtype"] == wl.DTYPE_BF16 else torch.float32
    src = torch.from_numpy(fm.pool_k_col(np.arange(dh), dh, cfg["rope_base"] > 0)).argsort().cuda()
    slots = torch.from_numpy(fm.pool_v_slot(np.arange(P), cfg["dtype"]).astype(np.int64)).cuda()
    views = []
    for l in range(L):
        kv, vv = ctx.prefix_pool_views(l)
        k = torch.from_numpy(I[f"prefix.k.{l}"][:, :, 0, :]).to(tdt).cuda()   # [B, P, dh]
        v = torch.from_numpy(I[f"prefix.v.{l}"][:, :, 0, :]).to(tdt).cuda()
        kv[:B, :P, :] = k[:, :, src]                       # column c holds key dim src[c]
        vv[:B, :, slots] = v.transpose(1, 2)               # key j at its slot
        views.append((kv, vv))
    torch.cuda.synchronize()
    return views


@pytest.mark.parametrize("name,over", [
    ("tiny_fp32", dict(batch=2)),
    ("pi05_b1", dict(n_layers=2, steps=2)),                  # the loop kernel
    ("pi05_b8", dict(n_layers=2, steps=2, batch=3)),         # the per-operation graph
])
def test_inplace_bind_equals_copy_bind(name, over):
    import torch
    cfg = wl.workload(name, **over)
    c = Case(cfg)
    x_copy = c.gpu_denoise()
    ctx = fm.Context(cfg)
    wt = {n: fm.to_device(a, cfg["dtype"]) for n, a in c.W.items()}
    ctx.load_weights(wt)
    views = _write_prefix(ctx, cfg, c.I)
    B, P = cfg["batch"], cfg["prefix_len"]
    before = [(kv[:B, :P].clone(), vv[:B].clone()) for kv, vv in views]
    ctx.bind_prefix_inplace(B, P)
    ctx.set_schedule(c.steps, B)
    x_in = ctx.denoise(c.x0, c.steps)
    torch.cuda.synchronize()
    x_in = x_in.cpu().numpy()
    say(f"  {name}: in-place vs copying bind, max |diff| {np.max(np.abs(x_in - x_copy)):.3e}")
    np.testing.assert_array_equal(x_in, x_copy)
    slots = torch.from_numpy(fm.pool_v_slot(np.arange(P), cfg["dtype"]).astype(np.int64)).cuda()
    for (k0, v0), (kv, vv) in zip(before, views):   # the loop never writes the prefix rows
        assert torch.equal(k0, kv[:B, :P])
        assert torch.equal(v0[:, :, slots], vv[:B][:, :, slots])
    ctx.close()
    c.close()


def test_inplace_bind_errors():
    cfg = wl.workload("tiny_fp32")
    ctx = fm.Context(cfg)
    with pytest.raises(fm.FMError) as e:
        ctx.bind_prefix_inplace(1, cfg["prefix_len"])
    assert e.value.status == 3            # FM_ERR_STATE: no weights
    with pytest.raises(fm.FMError) as e:
        ctx.prefix_kv_slot(cfg["n_layers"])
    assert e.value.status == 1
    ctx.close()
    d = fm.Context(wl.workload("dit_b1", n_layers=2))
    with pytest.raises(fm.FMError) as e:
        d.prefix_kv_slot(0)
    assert e.value.status == 5            # FM_ERR_UNSUPPORTED: the DiT head has no prefix pool
    d.close()


def test_dit_context_projection_fp32_short_context():
    cfg = wl.workload("dit_b1", dtype=wl.DTYPE_F32, n_layers=4, hidden=256, n_heads=4, n_kv_heads=4,
                      head_dim=64, mlp_dim=1024, action_horizon=16, action_dim=7, ctx_len=50, ctx_len_max=70,
                      ctx_dim=96, steps=2, batch=3)
    c = Case(cfg)
    teacher_forced(c, 1e-4)
    chunk(c, 1e-4)
    c.close()


def test_dit_context_projection_bf16_two_requests():
    cfg = wl.workload("dit_b1", n_layers=6, steps=2, batch=2, ctx_len=480, ctx_len_max=600)
    c = Case(cfg)
    teacher_forced(c, 1e-2)
    chunk(c, 2e-2)
    c.close()
