"""FP8 weight streaming on the GPU against the CPU oracle.

The expert's per-layer matrices are stored as FP8 E4M3 codes with one power-of-two scale per
row (the oracle's quantize_fp8_rows, pinned in test_oracle.py; vla.cpp Sec. IV-D quantized
weights, pi0.5 Design FP8 for the expert).

  * The quantizer: codes and scales bit-exact with the oracle (a quantized code is an
    integer decision, taken in the same precision on both sides: the scaled value is exact).
  * The loop: the FP8 context computes the model whose weights are the dequantized values.
    A bf16 context loaded with exactly those values must give bit-identical chunks, since a
    power-of-two row scale commutes with every fp32 rounding and the codes convert to bf16
    exactly. This holds on the loop kernel and on the per-operation graph's weight-streaming
    GEMMs (64 rows, or 64-row groups that fit one round on the CUs), which stream the codes,
    and on the large-M GEMMs, which read dequantized bf16 copies; for the pi0.5-shaped expert
    and the DiT head (whose cross blocks' context projections stay bf16). Against the oracle on the dequantized weights the tolerances are
    the bf16 ones: <= 1e-2 per teacher-forced step velocity, <= 2e-2 on the chunk."""
import numpy as np
import pytest

import oracle
from flow_matching_vla_amd import fm, workloads as wl
from gpu_util import Case, say, teacher_forced, chunk

pytestmark = pytest.mark.gpu


def test_quantizer_codes_and_scales_bit_exact():
    import torch
    rng = np.random.default_rng(5)
    N, K = 40, 192
    w = rng.standard_normal((N, K)) * np.exp(rng.uniform(-12, 6, size=(N, 1)))
    w[3] = 0.0                                   # all-zero row: scale 1, zero codes
    w[4, 10] = 448 * 2.0 ** -5                   # a row max exactly 448 2^e
    w[5, :50] = rng.standard_normal(50) * 1e-9   # values far below the row's quantum (signed zeros)
    w[6] = -np.abs(w[6])
    w = wl.round_bf16(w.astype(np.float32)).astype(np.float64)
    codes, e, deq = oracle.quantize_fp8_rows(w)
    g_codes, g_scale, g_deq = fm.quantize_fp8(torch.from_numpy(w.astype(np.float32)).to(torch.bfloat16).cuda())
    torch.cuda.synchronize()
    g_codes = g_codes.cpu().numpy()
    bad = np.argwhere(g_codes != codes)
    say(f"  {N}x{K}: {len(bad)} code mismatches; exponents {e.min()}..{e.max()}")
    np.testing.assert_array_equal(g_codes, codes)
    np.testing.assert_array_equal(g_scale.cpu().numpy(), np.ldexp(1.0, e).astype(np.float32))
    np.testing.assert_array_equal(g_deq.float().cpu().numpy(), deq.astype(np.float32))


def _context(cfg, W, I, fp8, steps):
    """A context with the given weights, the case's prefix bound and the schedule set."""
    import torch
    dt = cfg["dtype"]
    ctx = fm.Context(cfg)
    if fp8:
        ctx.set_weight_format(fm.WEIGHTS_FP8_E4M3)
    ctx.load_weights({n: fm.to_device(a, dt) for n, a in W.items()})
    L, B = cfg["n_layers"], cfg["batch"]
    if cfg["arch"] == wl.ARCH_PREFIX_JOINT:
        ctx.bind_prefix_kv(B, cfg["prefix_len"], [fm.to_device(I[f"prefix.k.{l}"], dt) for l in range(L)],
                           [fm.to_device(I[f"prefix.v.{l}"], dt) for l in range(L)])
    else:
        ctx.bind_prefix_kv(B, cfg["ctx_len"], context=fm.to_device(I["context"], dt),
                           state=fm.to_device(I["state"], fm.F32))
    ctx.set_schedule(steps, B)
    torch.cuda.synchronize()
    return ctx


@pytest.mark.parametrize("name,over,graph", [
    ("pi05_b1", dict(n_layers=2, steps=2), False),            # the loop kernel streams the codes
    ("pi05_b1", dict(n_layers=2, steps=2), True),             # graph GEMMs of 50 rows stream them
    ("pi05_b8", dict(n_layers=2, steps=2, batch=3), False),   # 150 rows: codes streamed in 64-row groups, gate/up on bf16 copies
    ("dit_b1", dict(n_layers=4, steps=2), False),             # DiT head, 41 rows: codes streamed
    ("dit_b1", dict(n_layers=2, steps=2, batch=2), False),    # two requests, 82 rows: bf16 copies
])
def test_fp8_context_equals_dequantized_bf16(name, over, graph):
    import torch
    cfg = wl.workload(name, **over)
    W = wl.make_weights(cfg)
    Wq = oracle.fp8_weights(cfg, W)          # the model an FP8 context computes (exact in bf16)
    c = Case(cfg, W=Wq)                       # bf16 context holding the dequantized weights
    a8 = _context(cfg, W, c.I, True, c.steps)
    if graph:
        a8.set_loop_mode(fm.LOOP_GRAPH)
        c.ctx.set_loop_mode(fm.LOOP_GRAPH)
    assert a8.loop_status()[0] == c.ctx.loop_status()[0]
    x8 = a8.denoise(c.x0, c.steps)
    torch.cuda.synchronize()
    x8 = x8.cpu().numpy()
    xq = c.gpu_denoise()
    say(f"  {name}: FP8 context vs dequantized bf16, max |diff| {np.max(np.abs(x8 - xq)):.3e}")
    np.testing.assert_array_equal(x8, xq)
    # the FP8 context against the oracle on the dequantized weights
    x = c.I["x0"].astype(np.float32)
    worst = 0.0
    for k in range(c.steps):
        v = a8.step_velocity(torch.from_numpy(x).cuda(), k)
        torch.cuda.synchronize()
        v = v.cpu().numpy()
        worst = max(worst, oracle.e_rel(v, c.oracle_velocity(x, k)))
        x = (x + np.float32(c.tau64[k + 1] - c.tau64[k]) * v).astype(np.float32)
    chunk(c, 2e-2)
    # what quantization does to the model (context only, like the pages' Table V e_rel)
    xb = oracle.denoise(cfg, oracle.cast_weights(W), oracle.bind(cfg, oracle.cast_weights(W), c.I), c.I["x0"], c.steps)
    say(f"  worst step velocity e_rel {worst:.3e}; FP8 model vs bf16 model chunk e_rel {oracle.e_rel(x8, xb):.3e}")
    assert worst <= 1e-2, worst
    a8.close()
    c.close()


def _fp8_exact(cfg, W, seed):
    """The same weights with every matrix the format covers replaced by FP8-exact rows: random
    finite E4M3 codes of either sign times a per-row power of two, each row holding a code of
    value 448 (so the quantizer's exponent is that power and its codes are these). The
    dequantized weights are then these weights themselves: no full-size quantization on the
    host is needed (the quantizer is pinned against the oracle above)."""
    rng = np.random.default_rng(seed)
    table = oracle.fp8_e4m3_value(np.arange(256))          # value of every code byte
    out = dict(W)
    for key in oracle.fp8_weight_names(cfg):
        N, K = W[key].shape
        codes = rng.integers(0x18, 0x7F, size=(N, K), dtype=np.int64)   # exponent field >= 3, no NaN
        codes |= rng.integers(0, 2, size=(N, K), dtype=np.int64) << 7
        codes[:, 0] = 0x7E | (codes[:, 0] & 0x80)                         # |value| 448 in every row
        e = rng.integers(-13, -11, size=(N, 1))
        out[key] = np.ldexp(table[codes], e).astype(np.float32)
    return out


@pytest.mark.parametrize("name", ["dit_b1", "pi05_b1"])
def test_fp8_full_size_equals_bf16_on_fp8_exact_weights(name):
    # the whole head at its bench size: the FP8 context (codes streamed by the skinny GEMMs for
    # DiT, by the loop kernel for pi0.5) against a bf16 context on the same FP8-exact weights,
    # bitwise, and against the oracle over two teacher-forced steps
    import torch
    cfg = wl.workload(name, steps=2)
    W8 = _fp8_exact(cfg, wl.make_weights(cfg), seed=17)
    say(f"  {name}: FP8-exact weights built")
    c = Case(cfg, W=W8)
    a8 = _context(cfg, W8, c.I, True, c.steps)
    assert a8.loop_status()[0] == c.ctx.loop_status()[0]
    x8 = a8.denoise(c.x0, c.steps)
    torch.cuda.synchronize()
    x8 = x8.cpu().numpy()
    xq = c.gpu_denoise()
    say(f"  {name}: FP8 context vs bf16 on the same weights, max |diff| {np.max(np.abs(x8 - xq)):.3e}")
    np.testing.assert_array_equal(x8, xq)
    x = c.I["x0"].astype(np.float32)
    worst = 0.0
    for k in range(c.steps):
        v = a8.step_velocity(torch.from_numpy(x).cuda(), k)
        torch.cuda.synchronize()
        v = v.cpu().numpy()
        worst = max(worst, oracle.e_rel(v, c.oracle_velocity(x, k)))
        x = (x + np.float32(c.tau64[k + 1] - c.tau64[k]) * v).astype(np.float32)
    say(f"  worst step velocity e_rel {worst:.3e}")
    assert worst <= 1e-2, worst
    a8.close()
    c.close()


def test_fp8_weight_format_errors():
    # fp32 configurations, and an MLP width that is not a multiple of 64
    for cfg in (wl.workload("tiny_fp32"), wl.workload("dit_b1", n_layers=2, dtype=wl.DTYPE_F32),
                wl.workload("dit_b1", n_layers=2, mlp_dim=6144 + 32)):
        ctx = fm.Context(cfg)
        with pytest.raises(fm.FMError) as e:
            ctx.set_weight_format(fm.WEIGHTS_FP8_E4M3)
        assert e.value.status == 5      # FM_ERR_UNSUPPORTED
        ctx.close()
    ctx = fm.Context(wl.workload("pi05_b1", n_layers=1))
    with pytest.raises(fm.FMError) as e:
        ctx.set_weight_format(7)
    assert e.value.status == 1
    ctx.set_weight_format(fm.WEIGHTS_AS_GIVEN)
    ctx.close()
