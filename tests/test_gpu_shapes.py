"""Seeded random shapes through the C ABI against the CPU oracle.

Each case draws one expert from its own seed: the pi0.5-shaped AdaRMS expert (pi0.5 Design,
action expert; the shared-KV-head attention of Eq. (2) in vla.cpp) or the DiT head with
alternating self / cross blocks (GR00T N1.7, "Action head"), in fp32 or bf16. The draws
cover what a fixed workload does not:
  * horizons and action widths that leave ragged tiles (1 row, 1 action dim, odd counts);
  * 1 to 8 query heads per K/V head, head dims 64 / 128 / 256, hidden 256 to 1024;
  * batches from 1 to 12, so both the skinny (M <= 64) and the large-M GEMMs run;
  * ragged per-request prefixes (some of length 0) and random DiT text / image masks;
  * batch-1 bf16 experts of the loop kernel's shapes (hidden 512 / 1024, head dim 256).
Bars as everywhere: fp32 relative L2 <= 1e-4; bf16 <= 1e-2 per teacher-forced step velocity
and <= 2e-2 on the chunk."""
import numpy as np
import pytest

import oracle
from flow_matching_vla_amd import workloads as wl
from gpu_util import Case, say

N_CASES = 16


def draw(i):
    """Case i: (workload, visibility or None), from a generator seeded by i alone."""
    rng = np.random.default_rng(4099 + i)
    kind = i % 3                      # 0 pi0.5-shaped, 1 DiT, 2 the loop kernel's shapes
    fp32 = kind != 2 and rng.random() < 0.3
    if kind == 2:
        cfg = wl.workload("pi05_b1", n_layers=int(rng.integers(1, 3)), hidden=int(rng.choice([512, 1024])),
                          n_heads=int(rng.choice([1, 2, 4, 8])), mlp_dim=int(rng.choice([1024, 2048])),
                          action_horizon=int(rng.integers(1, 60)), action_dim=4 * int(rng.integers(1, 9)),
                          prefix_len=int(rng.integers(1, 500)), steps=int(rng.integers(1, 3)))
        plen = int(rng.integers(0, cfg["prefix_len"] + 1))
        vis = {"prefix_lens": np.array([plen], np.int32)} if (i // 3) % 2 else None   # every other one ragged
    elif kind == 0:
        dh = int(rng.choice([64, 128] if fp32 else [64, 128, 256]))
        B = int(rng.integers(1, 13))
        cfg = wl.workload("tiny_fp32" if fp32 else "pi05_b1", n_layers=int(rng.integers(1, 3)),
                          hidden=int(rng.choice([256, 512, 1024])), n_heads=int(rng.choice([1, 2, 4, 8])),
                          head_dim=dh, mlp_dim=int(rng.choice([512, 1024, 2048])),
                          action_horizon=int(rng.integers(1, 60)), action_dim=int(rng.integers(1, 33)),
                          prefix_len=int(rng.integers(1, 500)), batch=B, steps=int(rng.integers(1, 3)))
        vis = {"prefix_lens": rng.integers(0, cfg["prefix_len"] + 1, size=B).astype(np.int32)} \
            if rng.random() < 0.7 else None
    else:
        B = int(rng.integers(1, 5))
        D = int(rng.choice([256, 512]))
        cfg = wl.workload("dit_b1", dtype=wl.DTYPE_F32 if fp32 else wl.DTYPE_BF16, n_layers=int(rng.integers(1, 6)),
                          hidden=D, n_heads=D // 64, n_kv_heads=D // 64, head_dim=64,
                          mlp_dim=int(rng.choice([512, 1024])), action_horizon=int(rng.integers(1, 41)),
                          action_dim=int(rng.integers(1, 33)), state_dim=int(rng.integers(1, 33)),
                          ctx_len=int(rng.integers(1, 300)), ctx_dim=int(rng.choice([64, 96, 128])),
                          batch=B, steps=int(rng.integers(1, 3)))
        S = cfg["ctx_len"]
        text = rng.random((B, S)) < rng.uniform(0.05, 1.0)
        image = rng.random((B, S)) < rng.uniform(0.05, 1.0)
        text[:, int(rng.integers(0, S))] = True     # a request sees at least one token of each
        image[:, int(rng.integers(0, S))] = True
        vis = {"text_mask": text, "image_mask": image} if rng.random() < 0.7 else None
    return cfg, vis


def test_draws_cover_the_families():
    """The fixed draws hold every family, both dtypes, ragged prefixes, masks and batches > 1."""
    cases = [draw(i) for i in range(N_CASES)]
    assert {c["arch"] for c, _ in cases} >= {wl.ARCH_PREFIX_JOINT, wl.ARCH_DIT_CROSS}
    assert {c["dtype"] for c, _ in cases} == {wl.DTYPE_F32, wl.DTYPE_BF16}
    assert any(v and "prefix_lens" in v for _, v in cases)
    assert any(v and "text_mask" in v for _, v in cases)
    assert any(c["batch"] > 1 for c, _ in cases)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    cfg, vis = draw(i)
    keys = ("arch", "dtype", "n_layers", "hidden", "n_heads", "head_dim", "mlp_dim", "action_horizon",
            "action_dim", "prefix_len", "ctx_len", "batch", "steps")
    say(f"  case {i}: {[cfg[k] for k in keys]} visibility {None if vis is None else sorted(vis)}")
    fp32 = cfg["dtype"] == wl.DTYPE_F32
    c = Case(cfg, vis=vis)
    x = c.I["x0"].astype(np.float32)
    worst = 0.0
    for k in range(c.steps):
        v = c.gpu_velocity(x, k)
        worst = max(worst, oracle.e_rel(v, c.oracle_velocity(x, k)))
        x = (x + np.float32(c.tau64[k + 1] - c.tau64[k]) * v).astype(np.float32)
    xg = c.gpu_denoise()
    ex = oracle.e_rel(xg, oracle.denoise(cfg, c.w64, c.bound, c.I["x0"], c.steps))
    loop = c.ctx.loop_status()[0]
    c.close()
    say(f"  loop kernel {bool(loop)}: worst velocity e_rel {worst:.2e}, chunk e_rel {ex:.2e}")
    if i % 3 == 2:
        assert loop   # the loop kernel's family: its draws must not fall back to the graph
    assert worst <= (1e-4 if fp32 else 1e-2), worst
    assert ex <= (1e-4 if fp32 else 2e-2), ex
