"""Host-side checks of the C ABI: the library loads, exports every function include/fm.h
declares, validates configs, derives the pool capacity the pages' rule gives, and lists
the weight tensors the seeded workloads draw. No compute calls: these run without a GPU."""
import ctypes as C
import os

import numpy as np
import pytest

from flow_matching_vla_amd import fm, workloads as wl


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fm.LIB_PATH):
        from flow_matching_vla_amd import build
        build.build(verbose=False)
    return fm.lib()


def test_exports_every_header_symbol(lib):
    syms = fm.header_symbols()
    assert len(syms) >= 11
    for s in ("fm_load_weights", "fm_bind_prefix_kv", "fm_set_schedule", "fm_denoise"):
        assert s in syms
    for s in syms:
        assert hasattr(lib, s), s


@pytest.mark.parametrize("idx", range(5))
def test_weight_spec_matches_workload_shapes(lib, idx):
    cfg = wl.workload(idx)
    spec = dict(fm.weight_spec(cfg))
    assert spec == {k: tuple(v) for k, v in wl.weight_shapes(cfg).items()}


def test_pool_capacity_rule(lib):
    # pi0.5 Design, "Attention and the K/V pool": capacity = max prefix + horizon rounded up
    # to 256 keys; a 976-token prefix gives 1024 for horizons 10 and 15, 1280 for 50.
    for H, cap in ((10, 1024), (15, 1024), (50, 1280)):
        cfg = wl.workload("pi05_b1", prefix_len=976, action_horizon=H)
        assert fm.query(cfg)["pool_capacity"] == cap
    assert fm.query(wl.workload("pi05_b1"))["pool_capacity"] == 1024


def test_plan_info_sizes(lib):
    q = fm.query(wl.workload("pi05_b1"))
    assert q["n_sites"] == 37 and q["n_weights"] == 18 * 7 + 10
    assert q["weight_bytes"] == 2 * wl.param_count(wl.workload("pi05_b1"))
    assert fm.query(wl.workload("dit_b1"))["n_sites"] == 33


@pytest.mark.parametrize("field,value,status", [
    ("n_kv_heads", 2, fm.STATUS[5]), ("dtype", 7, fm.STATUS[1]), ("hidden", 100, fm.STATUS[5]),
    ("head_dim", 96, fm.STATUS[5]), ("max_batch", 0, fm.STATUS[1]), ("arch", 3, fm.STATUS[1]),
    ("norm_eps", -1.0, fm.STATUS[1]),
])
def test_config_validation(lib, field, value, status):
    cfg = dict(wl.workload("pi05_b1"), **{field: value})
    with pytest.raises(fm.FMError) as e:
        fm.query(cfg)
    assert str(e.value).startswith(status)


@pytest.mark.parametrize("field", ["n_layers", "n_heads", "mlp_dim", "action_horizon", "action_dim", "max_batch",
                                   "max_steps", "max_prefix_len"])
def test_config_fields_are_bounded(lib, field):
    # every field has an upper limit, so that a config cannot make the host build a weight list
    # or size arithmetic of billions of entries (found by the AddressSanitizer sweep)
    import time
    t0 = time.perf_counter()
    with pytest.raises(fm.FMError) as e:
        fm.query(dict(wl.workload("pi05_b1"), **{field: 1 << 30}))
    assert str(e.value).startswith(fm.STATUS[1])
    assert time.perf_counter() - t0 < 1.0
    fm.query(dict(wl.workload("pi05_b1"), n_layers=1024))   # the limit itself is accepted


def test_dit_config_validation(lib):
    with pytest.raises(fm.FMError):
        fm.query(dict(wl.workload("dit_b1"), n_kv_heads=1))
    with pytest.raises(fm.FMError):
        fm.query(dict(wl.workload("dit_b1"), rope_base=10000.0))
    fm.query(wl.workload("dit_b1"))


def test_null_and_range_arguments_fail_cleanly(lib):
    assert lib.fm_query(None, None, None, 0) == 1
    assert lib.fm_destroy(None) == 0
    assert lib.fm_load_weights(None, None, 0) == 1
    assert lib.fm_set_schedule(None, 1, 1, None) == 1
    assert lib.fm_denoise(None, None, 1, None) == 1
    cfg = fm.make_config(wl.workload("tiny_fp32"))
    name = C.c_char_p()
    assert lib.fm_weight_spec(C.byref(cfg), 10_000, C.byref(name), None, None) == 1
    assert lib.fm_op_linear(0, 4, 4, 7, None, None, None, 0, None, 0, None) == 1


def test_binding_refuses_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fm, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(fm, "_lib", None)
    with pytest.raises(RuntimeError):
        fm.lib()


def test_pool_layout_helpers_are_permutations():
    # where a prefix producer writes key dims and key slots (fm_pool_k_col / fm_pool_v_slot):
    # each a permutation, RoPE pairs (d, d + dh/2) side by side, slots permuted within 32-key tiles
    for dh in (64, 128, 256):
        cols = fm.pool_k_col(np.arange(dh), dh, True)
        assert sorted(cols.tolist()) == list(range(dh))
        assert np.all(cols[dh // 2:] == cols[:dh // 2] + 1)
        assert np.array_equal(fm.pool_k_col(np.arange(dh), dh, False), np.arange(dh))
    j = np.arange(1280)
    s = fm.pool_v_slot(j, fm.BF16)
    assert sorted(s.tolist()) == j.tolist()
    assert np.array_equal(s // 32, j // 32)
    assert np.array_equal(fm.pool_v_slot(j, fm.F32), j)


# ----------------------------------------------------------------------------- argument checks
def test_check_tensor_rejects_what_a_pointer_cannot_show(lib):
    """The binding's argument check (runs before any library call that takes a pointer)."""
    import torch
    from flow_matching_vla_amd import fm
    x = torch.zeros((2, 50, 32), dtype=torch.float32)
    # host memory is refused outright
    with pytest.raises(ValueError, match="device tensor"):
        fm.check_tensor(x, "x0", torch.float32, (2, 50, 32))
    # the remaining checks, independent of where the tensor lives
    fm.check_tensor(x, "x0", torch.float32, (2, 50, 32), on_device=False)
    with pytest.raises(ValueError, match="dtype"):
        fm.check_tensor(x.to(torch.bfloat16), "x0", torch.float32, (2, 50, 32), on_device=False)
    with pytest.raises(ValueError, match="shape"):
        fm.check_tensor(x[:1], "x0", torch.float32, (2, 50, 32), on_device=False)   # a batch-1 x0 on a batch-2 binding
    with pytest.raises(ValueError, match="shape"):
        fm.check_tensor(x, "x0", torch.float32, (2, 50, 7), on_device=False)
    with pytest.raises(ValueError, match="contiguous"):
        fm.check_tensor(x.transpose(0, 1).contiguous().transpose(0, 1), "x0", torch.float32, (2, 50, 32), on_device=False)
    with pytest.raises(ValueError, match="torch tensor"):
        fm.check_tensor(np.zeros((2, 50, 32), np.float32), "x0", torch.float32, (2, 50, 32), on_device=False)
    # prefix K of one layer: [batch, prefix_len, 1, head_dim] in the config dtype
    k = torch.zeros((1, 816, 1, 256), dtype=torch.bfloat16)
    fm.check_tensor(k, "k", fm.torch_dtype(fm.BF16), (1, 816, 1, 256), on_device=False)
    with pytest.raises(ValueError, match="shape"):
        fm.check_tensor(k[:, :800], "k", fm.torch_dtype(fm.BF16), (1, 816, 1, 256), on_device=False)


def test_kernel_level_helpers_refuse_host_tensors(lib):
    import torch
    from flow_matching_vla_amd import fm
    a = torch.zeros((64, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        fm.op_linear(a, a)
    q = torch.zeros((1, 4, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        fm.op_attention(q, q, q)
    with pytest.raises(ValueError, match="device tensor"):
        fm.quantize_fp8(a)


@pytest.mark.parametrize("arch,xcc,cus,ok", [
    ("gfx950", 8, 256, True),
    ("gfx950:sramecc+:xnack-", 8, 256, True),
    ("gfx950", 1, 32, False),    # a compute partition of one XCD: the exchanges' placement does not hold
    ("gfx950", 4, 128, False),
    ("gfx942", 8, 304, False),
    ("gfx950", 8, 252, False),
])
def test_device_precondition(lib, arch, xcc, cus, ok):
    from flow_matching_vla_amd import fm
    got, msg = fm.device_supported(arch, xcc, cus)
    assert got == ok, msg
    if not ok:
        assert msg
