"""Page-stated constants (tests/golden/page_constants.txt, each line citing its passage)
recomputed from the seeded workloads' shapes and the library's sizing rules. No GPU."""
import os

import numpy as np
import pytest

from flow_matching_vla_amd import fm, workloads as wl

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    out = {}
    for ln in open(os.path.join(HERE, "golden", "page_constants.txt")):
        if ln.startswith("#") or not ln.strip():
            continue
        key, vals, cite = (f.strip() for f in ln.split("|"))
        assert cite, key
        out.setdefault(key, []).append([float(v) for v in vals.split()])
    return out


G = _golden()


def test_pi05_modulation_table_shape_and_bytes():
    shp = wl.weight_shapes(wl.workload("pi05_b1"))
    S, O, D = shp["mod.w"]
    assert S == G["pi05_mod_sites"][0][0] and O == G["pi05_mod_row_width"][0][0]
    assert abs(S * O * D * 2 / 1e6 - G["pi05_mod_dense_mb_fp16"][0][0]) < 0.05


def test_pi05_expert_parameter_count():
    shp = wl.weight_shapes(wl.workload("pi05_b1"))
    n = sum(np.prod(s) for k, s in shp.items() if k.startswith("layers.") or k == "mod.w")
    assert abs(n / 1e6 - G["pi05_expert_params_m"][0][0]) < 0.5


def test_gr00t_modulation_table_bytes():
    # the page's projections give (scale, shift), 2 x 1536 wide; the gate block that this
    # design's DiT adds for its gated attention residual is a reading, not counted here
    shp = wl.weight_shapes(wl.workload("dit_b1"))
    S, O, D = shp["mod.w"]
    assert S == G["gr00t_mod_sites"][0][0] and O == 3 * D
    assert abs(S * 2 * D * D * 2 / 1e6 - G["gr00t_mod_dense_mb_fp16"][0][0]) < 0.5


@pytest.mark.parametrize("row", G["pool_capacity"])
def test_pool_capacity(row):
    if not os.path.exists(fm.LIB_PATH):
        from flow_matching_vla_amd import build
        build.build(verbose=False)
    P, H, cap = (int(v) for v in row)
    assert fm.query(wl.workload("pi05_b1", prefix_len=P, action_horizon=H))["pool_capacity"] == cap
