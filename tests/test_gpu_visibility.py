"""Per-request key visibility on the GPU against the CPU oracle.

  * pi0.5 expert: compact prefixes of different lengths in one batch. Request b attends to
    its first P_b prefix keys and its own chunk, which sits at RoPE positions P_b + i (pi0.5
    Design, "Component contract": the filled length after the append is per request).
  * DiT head: the text and image masks of the cross blocks, the additive mask of vla.cpp
    Eq. (2). Block i reads the text mask when i % 4 == 0 and the image mask otherwise
    (GR00T N1.7, section "action").

Tolerances are those of the parity tests: relative L2 <= 1e-4 in fp32; in bf16 <= 1e-2 per
teacher-forced step velocity and <= 2e-2 on the final chunk. Both the per-operation graph and
the loop kernel are covered, including requests with an empty prefix, a prefix that ends
inside a key tile, and key splits that hold no visible key."""
import numpy as np
import pytest

from flow_matching_vla_amd import fm, workloads as wl
from gpu_util import Case, say, teacher_forced, chunk

pytestmark = pytest.mark.gpu


def _lens(*v):
    return {"prefix_lens": np.array(v, dtype=np.int32)}


def test_ragged_prefix_fp32_graph():
    cfg = wl.workload("tiny_fp32", batch=4)
    P = cfg["prefix_len"]
    c = Case(cfg, vis=_lens(P, 37, 0, 32))   # whole, ends inside a tile, empty, tile edge
    teacher_forced(c, 1e-4)
    chunk(c, 1e-4)
    # back to the whole prefix on the same binding (the captured loop is reused)
    c.set_visibility(None)
    chunk(c, 1e-4)
    c.close()


def test_ragged_prefix_bf16_graph_split_keys():
    # 4 requests x 400 folded rows: the attention splits its 866 keys over 8 workgroups, so
    # the short requests leave whole splits without a visible key
    cfg = wl.workload("pi05_b8", n_layers=2, steps=2, batch=4)
    vis = wl.make_visibility(cfg)
    vis["prefix_lens"][3] = 1
    say("  prefix lengths", vis["prefix_lens"].tolist())
    c = Case(cfg, vis=vis)
    assert not c.ctx.loop_status()[0]
    teacher_forced(c, 1e-2)
    chunk(c, 2e-2)
    c.close()


@pytest.mark.parametrize("B,H,lens", [(1, 50, (300,)), (1, 50, (0,)), (1, 50, (815,)), (3, 20, (816, 401, 0))])
def test_ragged_prefix_loop_kernel(B, H, lens):
    cfg = wl.workload("pi05_b1", n_layers=2, steps=2, batch=B, action_horizon=H)
    c = Case(cfg, vis=_lens(*lens))
    assert c.ctx.loop_status()[0], "the loop kernel should serve this shape"
    teacher_forced(c, 1e-2)
    chunk(c, 2e-2)
    assert c.ctx.loop_status()[1] == 0
    c.close()


def test_dit_masks_bf16():
    # four blocks: cross block 0 reads the text mask, cross block 2 the image mask
    cfg = wl.workload("dit_b1", n_layers=4, steps=2, batch=2)
    vis = wl.make_visibility(cfg)
    say("  visible text / image tokens", vis["text_mask"].sum(1).tolist(), vis["image_mask"].sum(1).tolist())
    c = Case(cfg, vis=vis)
    teacher_forced(c, 1e-2)
    chunk(c, 2e-2)
    c.close()


def test_dit_masks_fp32():
    cfg = wl.workload("dit_b1", dtype=wl.DTYPE_F32, n_layers=4, hidden=256, n_heads=4, n_kv_heads=4,
                      head_dim=64, mlp_dim=1024, action_horizon=16, action_dim=7, ctx_len=70, ctx_dim=96,
                      steps=2, batch=3)
    vis = wl.make_visibility(cfg)
    vis["text_mask"][2] = False
    vis["text_mask"][2, 69] = True    # one visible token, in the ragged last key tile
    c = Case(cfg, vis=vis)
    teacher_forced(c, 1e-4)
    chunk(c, 1e-4)
    c.set_visibility(None)
    chunk(c, 1e-4)
    c.close()


def test_visibility_errors():
    c = Case(wl.workload("tiny_fp32", batch=2))
    P = c.cfg["prefix_len"]
    for bad in ((P + 1, 0), (-1, 3)):
        with pytest.raises(fm.FMError) as e:
            c.ctx.bind_prefix_lengths(np.array(bad, np.int32))
        assert e.value.status == 1   # FM_ERR_INVALID_ARG
    with pytest.raises(fm.FMError) as e:
        c.ctx.bind_context_masks(None, None)
    assert e.value.status == 5       # FM_ERR_UNSUPPORTED: masks belong to the DiT head
    chunk(c, 1e-4)                   # a refused call changed nothing
    c.close()
    d = Case(wl.workload("dit_b1", n_layers=4, steps=1, batch=2))
    S = d.cfg["ctx_len"]
    ok = np.ones((2, S), bool)
    empty = ok.copy()
    empty[1] = False
    for text, image in ((empty, ok), (ok, empty)):
        with pytest.raises(fm.FMError) as e:
            d.ctx.bind_context_masks(text, image)
        assert e.value.status == 1
    with pytest.raises(fm.FMError) as e:
        d.ctx.bind_prefix_lengths(None)
    assert e.value.status == 5
    d.close()
    # a two-block head reads only the text mask: an empty image mask is accepted
    d2 = Case(wl.workload("dit_b1", n_layers=2, steps=1, batch=2))
    d2.ctx.bind_context_masks(ok, empty)
    d2.close()
