"""Bitwise determinism over 100 replays of one chunk (vla.cpp Sec. III-E: every figure is a
replay of the same chunk, so a replay must reproduce it exactly). Every reduction order in the
library is fixed, with no atomics in arithmetic, so any difference between replays would be a
race: the loop kernel's cross-XCD exchanges, the split-K exchanges of the GEMMs, the
attention splits, or a graph replay that reads a buffer before it is written."""
import numpy as np
import pytest
import torch

from flow_matching_vla_amd import workloads as wl
from gpu_util import Case, say

pytestmark = pytest.mark.gpu
REPLAYS = 100


@pytest.mark.parametrize("name", ["pi05_b1", "pi05_b8", "dit_b1"])
def test_hundred_replays_are_bitwise_equal(name):
    cfg = wl.workload(name)
    c = Case(cfg)
    loop = c.ctx.loop_status()[0]
    say(f"  {name}: {REPLAYS} replays ({'loop kernel' if loop else 'graph'})")
    first = c.gpu_denoise()
    assert np.isfinite(first).all()
    out = torch.empty_like(c.x0)
    mismatches = 0
    for _ in range(REPLAYS - 1):
        c.ctx.denoise(c.x0, c.steps, out)
        torch.cuda.synchronize()
        mismatches += int(not np.array_equal(out.cpu().numpy(), first))
    _, fault = c.ctx.loop_status()
    c.close()
    assert fault == 0
    assert mismatches == 0, f"{mismatches} of {REPLAYS - 1} replays differ from the first"
