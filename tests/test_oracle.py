"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each check is chosen so that a plausible slip in the oracle (a dropped term, a wrong
sign or index, a transposed operand) fails it: library routines (torch, float64),
closed forms of the Euler loop, invariants of RoPE / attention / norms, page-printed
sizes, and a scalar brute-force re-implementation on micro shapes.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from flow_matching_vla_amd import workloads as wl

RNG = np.random.default_rng(12345)


def t64(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


# ----------------------------------------------------------------------------- schedule / Euler
def test_schedule_uniform_one_to_zero():
    # vla.cpp Eq. (1) schedule; pi0.5 Design loop runs t from 1 to 0.
    np.testing.assert_array_equal(oracle.schedule(4), [1.0, 0.75, 0.5, 0.25, 0.0])
    np.testing.assert_array_equal(oracle.schedule(0), [1.0])
    with pytest.raises(ValueError):
        oracle.schedule(3, tau=[1.0, 0.0])


def _tiny(**kw):
    return wl.workload("tiny_fp32", **kw)


def test_steps_zero_returns_x0():
    cfg = _tiny()
    W, I = wl.make_weights(cfg), wl.make_inputs(cfg)
    x = oracle.run(cfg, W, I, steps=0)
    np.testing.assert_array_equal(x, I["x0"].astype(np.float64))


def test_dt_zero_returns_x0_bitwise():
    # a constant schedule gives dt = 0, and x + 0 * v == x exactly for finite v
    cfg = _tiny()
    W, I = wl.make_weights(cfg), wl.make_inputs(cfg)
    x = oracle.run(cfg, W, I, steps=3, tau=[0.4, 0.4, 0.4, 0.4])
    np.testing.assert_array_equal(x, I["x0"].astype(np.float64))


@pytest.mark.parametrize("name", ["tiny_fp32", "dit_b1"])
def test_constant_velocity_field_closed_form(name):
    # W_out = 0, b_out = c makes v == c at every step: X^T = X^0 + (tau_T - tau_0) c = X^0 - c.
    cfg = wl.workload(name, n_layers=2) if name == "dit_b1" else _tiny()
    if name == "dit_b1":
        cfg.update(ctx_len=8)
    W, I = wl.make_weights(cfg), wl.make_inputs(cfg)
    c = RNG.standard_normal(cfg["action_dim"])
    W["action_out.w"] = np.zeros_like(W["action_out.w"])
    W["action_out.b"] = c.astype(np.float32)
    x = oracle.run(cfg, W, I, steps=cfg["steps"])
    ref = I["x0"].astype(np.float64) - c.astype(np.float32).astype(np.float64)
    np.testing.assert_allclose(x, ref, rtol=0, atol=1e-12)


def test_linear_velocity_field_closed_form():
    # v = a x integrates by Euler to prod_k (1 + a dt_k) x0 = (1 - a/T)^T x0 on the uniform 1->0 grid.
    cfg = _tiny()
    x0 = RNG.standard_normal((2, 5, 3))
    a, T = 0.7, 6
    x = oracle.denoise(cfg, None, None, x0, T, field=lambda x, k, t: a * x)
    np.testing.assert_allclose(x, (1.0 - a / T) ** T * x0, rtol=1e-13)
    # a time-dependent field sees tau_k at the left end of each interval
    seen = []
    oracle.denoise(cfg, None, None, x0, 4, field=lambda x, k, t: seen.append(t) or 0 * x)
    assert seen == [1.0, 0.75, 0.5, 0.25]


# ----------------------------------------------------------------------------- elementwise
def test_gelu_tanh_and_silu_match_torch():
    x = np.linspace(-8, 8, 4001)
    np.testing.assert_allclose(oracle.gelu_tanh(x), F.gelu(t64(x), approximate="tanh").numpy(), rtol=1e-14, atol=1e-15)
    # the tanh form stays within its known approximation error of the exact erf GELU
    exact = 0.5 * x * (1 + np.vectorize(math.erf)(x / math.sqrt(2)))
    assert np.max(np.abs(oracle.gelu_tanh(x) - exact)) < 1e-3
    np.testing.assert_allclose(oracle.silu(x), F.silu(t64(x)).numpy(), rtol=1e-14, atol=1e-15)


def test_linear_matches_torch():
    x, w, b = RNG.standard_normal((3, 4, 7)), RNG.standard_normal((5, 7)), RNG.standard_normal(5)
    np.testing.assert_allclose(oracle.linear(x, w, b), F.linear(t64(x), t64(w), t64(b)).numpy(), rtol=1e-13)


# ----------------------------------------------------------------------------- norms
def test_rms_norm_matches_torch_and_invariants():
    h = RNG.standard_normal((4, 6, 64)) * 3 + 0.5
    eps = 1e-6
    np.testing.assert_allclose(oracle.rms_norm(h, eps), F.rms_norm(t64(h), (64,), eps=eps).numpy(), rtol=1e-13)
    n = oracle.rms_norm(h, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(n * n, axis=-1)), 1.0, rtol=1e-13)
    np.testing.assert_allclose(oracle.rms_norm(5.0 * h, 0.0), n, rtol=1e-13)


def test_layer_norm_matches_torch_and_invariants():
    h = RNG.standard_normal((4, 6, 48)) * 2 - 1.5
    eps = 1e-6
    np.testing.assert_allclose(oracle.layer_norm(h, eps), F.layer_norm(t64(h), (48,), eps=eps).numpy(), rtol=1e-12, atol=1e-13)
    n = oracle.layer_norm(h, 0.0)
    np.testing.assert_allclose(n.mean(-1), 0.0, atol=1e-13)
    np.testing.assert_allclose(n.var(-1), 1.0, rtol=1e-12)


def test_modulate_and_site_split():
    D = 4
    row = np.arange(3 * D, dtype=np.float64)
    s, sh, g = oracle.split_site(row, D)
    np.testing.assert_array_equal(s, [0, 1, 2, 3])
    np.testing.assert_array_equal(sh, [4, 5, 6, 7])
    np.testing.assert_array_equal(g, [8, 9, 10, 11])
    n = RNG.standard_normal((2, D))
    np.testing.assert_allclose(oracle.modulate(n, 0 * s, 0 * sh), n)
    np.testing.assert_allclose(oracle.modulate(n, s, sh), n + n * s + sh)


# ----------------------------------------------------------------------------- RoPE
def test_rope_matches_complex_rotation():
    # independent formulation: z_j = x_j + i x_{j+d/2} multiplied by exp(i p theta_j)
    d, base = 16, 10000.0
    x = RNG.standard_normal((2, 5, d))
    pos = np.array([0, 3, 7, 100, 1023])
    out = oracle.rope(x, pos, base)
    theta = base ** (-np.arange(d // 2) * 2.0 / d)
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * pos[:, None] * theta[None, :])
    np.testing.assert_allclose(out, np.concatenate([z.real, z.imag], -1), rtol=1e-12, atol=1e-12)


def test_rope_invariants():
    d = 32
    q, k = RNG.standard_normal((1, 1, d)), RNG.standard_normal((1, 1, d))
    np.testing.assert_array_equal(oracle.rope(q, [0], 1e4), q)          # position 0 is the identity
    np.testing.assert_allclose(np.linalg.norm(oracle.rope(q, [57], 1e4)), np.linalg.norm(q), rtol=1e-13)
    # <R_m q, R_n k> depends only on m - n
    def dot(m, n):
        return float(np.sum(oracle.rope(q, [m], 1e4) * oracle.rope(k, [n], 1e4)))
    assert abs(dot(10, 3) - dot(817, 810)) < 1e-10
    assert abs(dot(10, 3) - dot(3, 10)) > 1e-6


# ----------------------------------------------------------------------------- attention
def test_attention_matches_torch_sdpa_head_fold():
    # one K/V head shared by all query heads == MHA with K/V replicated per head
    B, nq, Tq, Tk, d = 2, 4, 5, 9, 8
    q = RNG.standard_normal((B, nq, Tq, d))
    k, v = RNG.standard_normal((B, 1, Tk, d)), RNG.standard_normal((B, 1, Tk, d))
    out = oracle.attention(q, k, v)
    ref = F.scaled_dot_product_attention(t64(q), t64(k).expand(B, nq, Tk, d), t64(v).expand(B, nq, Tk, d)).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    kk, vv = RNG.standard_normal((B, nq, Tk, d)), RNG.standard_normal((B, nq, Tk, d))
    ref = F.scaled_dot_product_attention(t64(q), t64(kk), t64(vv)).numpy()
    np.testing.assert_allclose(oracle.attention(q, kk, vv), ref, rtol=1e-12, atol=1e-13)


def test_attention_brute_force_and_special_cases():
    d, Tq, Tk = 3, 2, 4
    q, k, v = RNG.standard_normal((1, 1, Tq, d)), RNG.standard_normal((1, 1, Tk, d)), RNG.standard_normal((1, 1, Tk, d))
    out = oracle.attention(q, k, v)
    for i in range(Tq):
        w = [math.exp(sum(q[0, 0, i, c] * k[0, 0, j, c] for c in range(d)) / math.sqrt(d)) for j in range(Tk)]
        z = sum(w)
        for c in range(d):
            assert abs(out[0, 0, i, c] - sum(w[j] * v[0, 0, j, c] for j in range(Tk)) / z) < 1e-12
    # a single key returns its value; q = 0 averages the values uniformly
    np.testing.assert_allclose(oracle.attention(q, k[:, :, :1], v[:, :, :1]), np.broadcast_to(v[:, :, :1], out.shape), rtol=1e-14)
    np.testing.assert_allclose(oracle.attention(0 * q, k, v), np.broadcast_to(v.mean(2, keepdims=True), out.shape), rtol=1e-13)
    # permuting keys and values jointly changes nothing; huge logits are stable
    perm = RNG.permutation(Tk)
    np.testing.assert_allclose(oracle.attention(q, k[:, :, perm], v[:, :, perm]), out, rtol=1e-13)
    big = oracle.attention(1e4 * q, k, v)
    assert np.all(np.isfinite(big))


# ----------------------------------------------------------------------------- time conditioning
def test_sinusoidal_embedding_invariants():
    D = 64
    e0 = oracle.sinusoidal_embedding(np.array([0.0]), D)
    np.testing.assert_array_equal(e0[0, : D // 2], 0.0)
    np.testing.assert_array_equal(e0[0, D // 2:], 1.0)
    tau = np.array([0.1, 0.37, 0.9])
    e = oracle.sinusoidal_embedding(tau, D)
    np.testing.assert_allclose(e[:, : D // 2] ** 2 + e[:, D // 2:] ** 2, 1.0, rtol=1e-14)
    # angular frequencies 2 pi / p_j: p_0 = 4e-3 and p_last = 4.0, geometric in between
    h = 1e-7
    slope = oracle.sinusoidal_embedding(np.array([h]), D)[0, : D // 2] / h
    np.testing.assert_allclose(slope[0], 2 * math.pi / 4e-3, rtol=1e-6)
    np.testing.assert_allclose(slope[-1], 2 * math.pi / 4.0, rtol=1e-9)
    ratios = slope[1:] / slope[:-1]
    np.testing.assert_allclose(ratios, ratios[0], rtol=1e-5)


def test_modulation_table_sites_and_page_sizes():
    # pi0.5 Design: 37 AdaRMS Denses [3072, 1024] hoisted, 232.8 MB in fp16.
    shp = wl.weight_shapes(wl.workload("pi05_b1"))
    assert shp["mod.w"] == (37, 3072, 1024)
    assert abs(np.prod(shp["mod.w"]) * 2 / 1e6 - 232.8) < 0.05
    # GR00T N1.7 Build-time constants: 33 AdaLayerNorm projections [1536, 3072], 311 MB fp16.
    shp = wl.weight_shapes(wl.workload("dit_b1"))
    assert shp["mod.w"][0] == 33 and shp["mod.w"][2] == 1536
    assert abs(33 * 1536 * 3072 * 2 / 1e6 - 311) < 0.5
    # pi0.5 Design architecture diagram: action expert of 428M (blocks + AdaRMS Denses)
    cfg = wl.workload("pi05_b1")
    shp = wl.weight_shapes(cfg)
    n = sum(np.prod(s) for k, s in shp.items() if k.startswith("layers.") or k == "mod.w")
    assert abs(n / 1e6 - 428) < 0.5


def test_modulation_table_is_per_site_dense_of_time_conditioning():
    cfg = _tiny()
    W = oracle.cast_weights(wl.make_weights(cfg))
    tau = oracle.schedule(4)
    table, tb = oracle.modulation_table(cfg, W, tau)
    assert table.shape == (4, 5, 768) and tb is None
    c = oracle.time_conditioning(W, tau[:4])
    for k in range(4):
        for s in range(5):
            ref = F.linear(t64(c[k]), t64(W["mod.w"][s]), t64(W["mod.b"][s])).numpy()
            np.testing.assert_allclose(table[k, s], ref, rtol=1e-12, atol=1e-14)
    # zero weights leave only the bias; the time MLP is two SiLU(Linear) layers
    Z = dict(W)
    Z["mod.w"] = np.zeros_like(W["mod.w"])
    np.testing.assert_array_equal(oracle.modulation_table(cfg, Z, tau)[0][2], W["mod.b"])
    e = oracle.sinusoidal_embedding(tau[:4], 256)
    ref = F.silu(F.linear(F.silu(F.linear(t64(e), t64(W["time_in.w"]), t64(W["time_in.b"]))), t64(W["time_out.w"]), t64(W["time_out.b"])))
    np.testing.assert_allclose(c, ref.numpy(), rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------- whole-network pins
def _zero_gates(cfg, W):
    W = dict(W)
    D = cfg["hidden"]
    mw, mb = W["mod.w"].copy(), W["mod.b"].copy()
    mw[:, 2 * D:3 * D, :] = 0
    mb[:, 2 * D:3 * D] = 0
    W["mod.w"], W["mod.b"] = mw, mb
    return W


def test_all_gates_zero_makes_blocks_identity_pi05():
    cfg = _tiny()
    W, I = oracle.cast_weights(_zero_gates(cfg, wl.make_weights(cfg))), wl.make_inputs(cfg)
    bound = oracle.bind(cfg, W, I)
    tau = oracle.schedule(4)
    table, tb = oracle.modulation_table(cfg, W, tau)
    x = I["x0"].astype(np.float64)
    v = oracle.velocity(cfg, W, bound, x, table, tb, 2)
    h = oracle.linear(x, W["action_in.w"], W["action_in.b"])
    s, sh, _ = oracle.split_site(table[2, -1], cfg["hidden"])
    ref = oracle.linear(oracle.modulate(oracle.rms_norm(h, 1e-6), s, sh), W["action_out.w"], W["action_out.b"])
    np.testing.assert_allclose(v, ref, rtol=1e-12, atol=1e-13)


def test_all_gates_zero_dit_blocks_identity_when_ff_zero():
    cfg = wl.workload("dit_b1", n_layers=2, ctx_len=8)
    W = _zero_gates(cfg, wl.make_weights(cfg))
    for i in range(2):
        W[f"blocks.{i}.ff2.w"] = np.zeros_like(W[f"blocks.{i}.ff2.w"])
    W, I = oracle.cast_weights(W), wl.make_inputs(cfg)
    bound = oracle.bind(cfg, W, I)
    tau = oracle.schedule(4)
    table, tb = oracle.modulation_table(cfg, W, tau)
    x = I["x0"].astype(np.float64)
    v = oracle.velocity(cfg, W, bound, x, table, tb, 1)
    h = oracle.linear(x, W["action_in.w"], W["action_in.b"]) + tb[1]
    s, sh, _ = oracle.split_site(table[1, -1], cfg["hidden"])
    ref = oracle.linear(oracle.modulate(oracle.layer_norm(h, 1e-6), s, sh), W["action_out.w"], W["action_out.b"])
    np.testing.assert_allclose(v, ref, rtol=1e-11, atol=1e-12)


def test_prefix_kv_is_never_written_and_reused():
    cfg = _tiny()
    W, I = oracle.cast_weights(wl.make_weights(cfg)), wl.make_inputs(cfg)
    bound = oracle.bind(cfg, W, I)
    snap = [a.copy() for a in bound["k"] + bound["v"]]
    with pytest.raises(ValueError):
        bound["k"][0][0, 0, 0, 0] = 1.0
    x1 = oracle.denoise(cfg, W, bound, I["x0"], 4)
    x2 = oracle.denoise(cfg, W, bound, I["x0"], 4)
    for a, b in zip(snap, bound["k"] + bound["v"]):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(x1, x2)


def test_requests_are_independent():
    cfg = _tiny(batch=3)
    W, I = wl.make_weights(cfg), wl.make_inputs(cfg)
    xb = oracle.run(cfg, W, I)
    for b in range(3):
        Ib = {k: v[b:b + 1] for k, v in I.items()}
        np.testing.assert_allclose(oracle.run(dict(cfg, batch=1), W, Ib), xb[b:b + 1], rtol=1e-12, atol=1e-13)


def test_joint_prefix_permutation_invariance():
    cfg = _tiny()
    W, I = wl.make_weights(cfg), wl.make_inputs(cfg)
    perm = RNG.permutation(cfg["prefix_len"])
    Ip = dict(I)
    for l in range(cfg["n_layers"]):
        Ip[f"prefix.k.{l}"] = I[f"prefix.k.{l}"][:, perm]
        Ip[f"prefix.v.{l}"] = I[f"prefix.v.{l}"][:, perm]
    np.testing.assert_allclose(oracle.run(cfg, W, Ip), oracle.run(cfg, W, I), rtol=1e-12, atol=1e-13)


def test_float32_oracle_agrees_with_float64():
    for cfg in (_tiny(), wl.workload("pi05_b1", n_layers=2, prefix_len=40, action_horizon=12),
                wl.workload("dit_b1", n_layers=2, ctx_len=24)):
        W, I = wl.make_weights(cfg), wl.make_inputs(cfg)
        x64, tr64 = oracle.run(cfg, W, I, return_trace=True)
        x32, tr32 = oracle.run(cfg, W, I, dtype=np.float32, return_trace=True)
        assert oracle.e_rel(x32, x64) < 1e-5
        for (_, v64), (_, v32) in zip(tr64, tr32):
            assert oracle.e_rel(v32, v64) < 1e-4


def test_metrics():
    a, r = np.array([1.0, 2.0, 3.0]), np.array([1.0, 2.5, 3.0])
    assert oracle.e_inf(a, r) == 0.5
    assert abs(oracle.e_rel(a, r) - 0.5 / math.sqrt(1 + 6.25 + 9)) < 1e-15
    assert oracle.e_rel(a, 0 * r) is None


# ----------------------------------------------------------------------------- scalar brute force
def _brute_velocity_pi05(cfg, W, I, x, row, rq=None):
    """Scalar-loop re-statement of one expert step on micro shapes (pure Python floats).
    rq: optional rounding of a list of values (the bf16 reading): applied to the norm's scaled
    input h (1 + scale) and shift, the chunk's queries and keys after RoPE, its values, the
    attention output and the gated-GELU activation."""
    rounding = rq is not None
    rq = rq or (lambda vec: vec)
    D, L, nq, dh, F_, eps = cfg["hidden"], cfg["n_layers"], cfg["n_heads"], cfg["head_dim"], cfg["mlp_dim"], cfg["norm_eps"]
    H, da, P, base = cfg["action_horizon"], cfg["action_dim"], cfg["prefix_len"], cfg["rope_base"]

    def mv(Wm, vec):
        return [sum(Wm[o][i] * vec[i] for i in range(len(vec))) for o in range(len(Wm))]

    def rot(vec, p):
        out = list(vec)
        for j in range(dh // 2):
            th = p * base ** (-2.0 * j / dh)
            a, b = vec[j], vec[j + dh // 2]
            out[j] = a * math.cos(th) - b * math.sin(th)
            out[j + dh // 2] = b * math.cos(th) + a * math.sin(th)
        return out

    def nm(vec, site):
        r = math.sqrt(sum(t * t for t in vec) / D + eps)
        if rounding:
            hs = rq([vec[i] * (1 + row[site][i]) for i in range(D)])
            sh = rq([row[site][D + i] for i in range(D)])
            return [hs[i] / r + sh[i] for i in range(D)]
        return [vec[i] / r * (1 + row[site][i]) + row[site][D + i] for i in range(D)]

    h = [[sum(W["action_in.w"][o][i] * x[t][i] for i in range(da)) + W["action_in.b"][o] for o in range(D)] for t in range(H)]
    for l in range(L):
        p = f"layers.{l}."
        u = [nm(h[t], 2 * l) for t in range(H)]
        q = [mv(W[p + "q.w"], u[t]) for t in range(H)]
        ks = [rq(rot(mv(W[p + "k.w"], u[t]), P + t)) for t in range(H)]
        vs = [rq(mv(W[p + "v.w"], u[t])) for t in range(H)]
        keys = I[f"prefix.k.{l}"][0, :, 0].astype(np.float64).tolist() + ks
        vals = I[f"prefix.v.{l}"][0, :, 0].astype(np.float64).tolist() + vs
        o = [[0.0] * (nq * dh) for _ in range(H)]
        for t in range(H):
            for n in range(nq):
                qq = rq(rot(q[t][n * dh:(n + 1) * dh], P + t))
                sc = [sum(qq[c] * kk[c] for c in range(dh)) / math.sqrt(dh) for kk in keys]
                m = max(sc)
                e = [math.exp(s - m) for s in sc]
                z = sum(e)
                for c in range(dh):
                    o[t][n * dh + c] = sum(e[j] * vals[j][c] for j in range(len(keys))) / z
        o = [rq(o[t]) for t in range(H)]
        for t in range(H):
            y = mv(W[p + "o.w"], o[t])
            h[t] = [h[t][i] + row[2 * l][2 * D + i] * y[i] for i in range(D)]
        for t in range(H):
            u2 = nm(h[t], 2 * l + 1)
            g, up = mv(W[p + "gate.w"], u2), mv(W[p + "up.w"], u2)
            a = rq([0.5 * g[f] * (1 + math.tanh(math.sqrt(2 / math.pi) * (g[f] + 0.044715 * g[f] ** 3))) * up[f] for f in range(F_)])
            y = mv(W[p + "down.w"], a)
            h[t] = [h[t][i] + row[2 * l + 1][2 * D + i] * y[i] for i in range(D)]
    out = []
    for t in range(H):
        u = nm(h[t], 2 * L)
        out.append([sum(W["action_out.w"][o][i] * u[i] for i in range(D)) + W["action_out.b"][o] for o in range(da)])
    return out


def test_scalar_brute_force_pi05_micro():
    cfg = wl.workload("tiny_fp32", n_layers=2, hidden=8, n_heads=2, head_dim=4, mlp_dim=6,
                      action_horizon=3, action_dim=2, prefix_len=4, weight_std=0.5)
    W, I = oracle.cast_weights(wl.make_weights(cfg)), wl.make_inputs(cfg)
    bound = oracle.bind(cfg, W, I)
    tau = oracle.schedule(2)
    table, tb = oracle.modulation_table(cfg, W, tau)
    x = I["x0"].astype(np.float64)
    v = oracle.velocity(cfg, W, bound, x, table, tb, 1)
    Wl = {k: np.asarray(a).tolist() for k, a in W.items()}
    ref = _brute_velocity_pi05(cfg, Wl, I, x[0].tolist(), table[1].tolist())
    np.testing.assert_allclose(v[0], np.array(ref), rtol=1e-10, atol=1e-12)


def _brute_velocity_dit(cfg, W, I, x, row, tb, text=None, image=None):
    """text / image: visible context indices of the request for the cross blocks that read
    each mask (block i reads text when i % 4 == 0, else image); None = all visible."""
    D, L, nh, dh, F_, eps = cfg["hidden"], cfg["n_layers"], cfg["n_heads"], cfg["head_dim"], cfg["mlp_dim"], cfg["norm_eps"]
    H, da = cfg["action_horizon"], cfg["action_dim"]
    ctx = I["context"][0].astype(np.float64).tolist()
    st = I["state"][0, 0].astype(np.float64).tolist()

    def mv(Wm, vec):
        return [sum(Wm[o][i] * vec[i] for i in range(len(vec))) for o in range(len(Wm))]

    def ln(vec):
        mu = sum(vec) / D
        var = sum((t - mu) ** 2 for t in vec) / D
        return [(t - mu) / math.sqrt(var + eps) for t in vec]

    def gelu(g):
        return 0.5 * g * (1 + math.tanh(math.sqrt(2 / math.pi) * (g + 0.044715 * g ** 3)))

    h = [[a + b for a, b in zip(mv(W["state_in.w"], st), W["state_in.b"])]]
    for t in range(H):
        h.append([a + b + c for a, b, c in zip(mv(W["action_in.w"], x[t]), W["action_in.b"], tb)])
    T = len(h)
    for i in range(L):
        p = f"blocks.{i}."
        u = [[n * (1 + row[i][c]) + row[i][D + c] for c, n in enumerate(ln(h[t]))] for t in range(T)]
        q = [mv(W[p + "q.w"], u[t]) for t in range(T)]
        src = ctx if i % 2 == 0 else u
        if i % 2 == 0:
            keep = text if i % 4 == 0 else image
            if keep is not None:
                src = [ctx[j] for j in keep]
        ks = [mv(W[p + "k.w"], s) for s in src]
        vs = [mv(W[p + "v.w"], s) for s in src]
        o = [[0.0] * D for _ in range(T)]
        for t in range(T):
            for n in range(nh):
                sl = slice(n * dh, (n + 1) * dh)
                sc = [sum(a * b for a, b in zip(q[t][sl], kk[sl])) / math.sqrt(dh) for kk in ks]
                m = max(sc)
                e = [math.exp(s - m) for s in sc]
                z = sum(e)
                for c in range(n * dh, (n + 1) * dh):
                    o[t][c] = sum(e[j] * vs[j][c] for j in range(len(ks))) / z
        for t in range(T):
            y = mv(W[p + "o.w"], o[t])
            h[t] = [h[t][c] + row[i][2 * D + c] * y[c] for c in range(D)]
        for t in range(T):
            y = mv(W[p + "ff2.w"], [gelu(g) for g in mv(W[p + "ff1.w"], ln(h[t]))])
            h[t] = [a + b for a, b in zip(h[t], y)]
    out = []
    for t in range(1, T):
        u = [n * (1 + row[L][c]) + row[L][D + c] for c, n in enumerate(ln(h[t]))]
        out.append([a + b for a, b in zip(mv(W["action_out.w"], u), W["action_out.b"])])
    return out


def test_scalar_brute_force_dit_micro():
    cfg = wl.workload("dit_b1", n_layers=2, hidden=8, n_heads=2, head_dim=4, n_kv_heads=2, mlp_dim=12,
                      action_horizon=3, action_dim=2, state_dim=3, ctx_len=5, ctx_dim=6, weight_std=0.5)
    W, I = oracle.cast_weights(wl.make_weights(cfg)), wl.make_inputs(cfg)
    bound = oracle.bind(cfg, W, I)
    tau = oracle.schedule(2)
    table, tb = oracle.modulation_table(cfg, W, tau)
    x = I["x0"].astype(np.float64)
    v = oracle.velocity(cfg, W, bound, x, table, tb, 0)
    Wl = {k: np.asarray(a).tolist() for k, a in W.items()}
    ref = _brute_velocity_dit(cfg, Wl, I, x[0].tolist(), table[0].tolist(), tb[0].tolist())
    np.testing.assert_allclose(v[0], np.array(ref), rtol=1e-10, atol=1e-12)


def test_scalar_brute_force_dit_micro_masked():
    # four blocks: cross block 0 reads the text mask, cross block 2 the image mask; the
    # brute force drops the hidden keys instead of adding -inf to their scores
    cfg = wl.workload("dit_b1", n_layers=4, hidden=8, n_heads=2, head_dim=4, n_kv_heads=2, mlp_dim=12,
                      action_horizon=3, action_dim=2, state_dim=3, ctx_len=7, ctx_dim=6, weight_std=0.5)
    W, I = oracle.cast_weights(wl.make_weights(cfg)), dict(wl.make_inputs(cfg))
    text, image = [0, 3, 4], [1, 2, 4, 6]
    I["text_mask"] = np.isin(np.arange(7), text)[None]
    I["image_mask"] = np.isin(np.arange(7), image)[None]
    bound = oracle.bind(cfg, W, I)
    tau = oracle.schedule(2)
    table, tb = oracle.modulation_table(cfg, W, tau)
    x = I["x0"].astype(np.float64)
    v = oracle.velocity(cfg, W, bound, x, table, tb, 1)
    Wl = {k: np.asarray(a).tolist() for k, a in W.items()}
    ref = _brute_velocity_dit(cfg, Wl, I, x[0].tolist(), table[1].tolist(), tb[1].tolist(), text, image)
    np.testing.assert_allclose(v[0], np.array(ref), rtol=1e-10, atol=1e-12)
    # the masks swapped give another result: each block reads its own mask
    ref_sw = _brute_velocity_dit(cfg, Wl, I, x[0].tolist(), table[1].tolist(), tb[1].tolist(), image, text)
    assert np.max(np.abs(v[0] - np.array(ref_sw))) > 1e-6


# ----------------------------------------------------------------------------- masks and ragged prefixes
def test_masked_attention_is_attention_over_visible_keys():
    # vla.cpp Eq. (2): M = -inf on a key removes it from the softmax
    B, nq, Tq, Tk, d = 3, 2, 4, 11, 5
    q = RNG.standard_normal((B, nq, Tq, d))
    k, v = RNG.standard_normal((B, 1, Tk, d)), RNG.standard_normal((B, 1, Tk, d))
    vis = RNG.random((B, 1, Tq, Tk)) < 0.6
    vis[..., 0] = True
    vis[1, 0, 2] = False
    vis[1, 0, 2, 7] = True          # a row with one visible key
    out = oracle.attention(q, k, v, vis)
    for b in range(B):
        for i in range(Tq):
            j = np.flatnonzero(vis[b, 0, i])
            ref = oracle.attention(q[b:b + 1, :, i:i + 1], k[b:b + 1, :, j], v[b:b + 1, :, j])
            np.testing.assert_allclose(out[b:b + 1, :, i:i + 1], ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(out[1, :, 2], np.broadcast_to(v[1, 0, 7], (nq, d)), rtol=1e-14)
    # torch's boolean-mask attention (True takes part), K/V replicated over the query heads
    ref = F.scaled_dot_product_attention(t64(q), t64(k).expand(B, nq, Tk, d), t64(v).expand(B, nq, Tk, d),
                                         attn_mask=torch.from_numpy(vis)).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    # all visible is M = 0; no visible key has no defined result
    np.testing.assert_array_equal(oracle.attention(q, k, v, np.ones((B, 1, 1, Tk), bool)), oracle.attention(q, k, v))
    assert np.all(np.isnan(oracle.attention(q, k, v, np.zeros((B, 1, 1, Tk), bool))))


def test_ragged_prefix_equals_compact_single_request():
    # pi0.5 Design, "Component contract": request b's filled length is P_b + H with its chunk
    # just past its own prefix, so a ragged batch equals each request run alone on its
    # compact prefix (positions P_b + i); prefix rows past P_b are never read
    cfg = _tiny(batch=3, n_layers=2)
    W, I = wl.make_weights(cfg), dict(wl.make_inputs(cfg))
    P = cfg["prefix_len"]
    lens = np.array([P, 37, 0])
    Ir = dict(I, prefix_lens=lens)
    xr = oracle.run(cfg, W, Ir, steps=3)
    Ig = dict(Ir)
    for l in range(cfg["n_layers"]):
        for nm in (f"prefix.k.{l}", f"prefix.v.{l}"):
            g = I[nm].copy()
            for b in range(3):
                g[b, lens[b]:] = 1e3 * RNG.standard_normal(g[b, lens[b]:].shape)
            Ig[nm] = g
    np.testing.assert_array_equal(oracle.run(cfg, W, Ig, steps=3), xr)
    for b in range(3):
        Ib = {nm: a[b:b + 1, :lens[b]] if nm.startswith("prefix.") else a[b:b + 1] for nm, a in I.items()}
        xb = oracle.run(dict(cfg, batch=1, prefix_len=int(lens[b])), W, Ib, steps=3)
        np.testing.assert_allclose(xr[b:b + 1], xb, rtol=1e-12, atol=1e-13)
    # the positions follow P_b: the same rows at the full length differ
    assert np.max(np.abs(xr[1] - oracle.run(cfg, W, I, steps=3)[1])) > 1e-6
    with pytest.raises(ValueError):
        oracle.bind(cfg, oracle.cast_weights(W), dict(I, prefix_lens=np.array([P + 1, 0, 0])))


def test_dit_mask_reaches_only_its_blocks():
    # GR00T N1.7, section "action": cross block i reads the text mask when i % 4 == 0 and the
    # image mask otherwise. Context rows hidden from the text mask cannot move the residual
    # after block 0; rows the image mask shows move it after block 2; rows hidden from both
    # cannot move the velocity.
    cfg = wl.workload("dit_b1", n_layers=4, hidden=64, n_heads=2, head_dim=32, n_kv_heads=2, mlp_dim=128,
                      action_horizon=6, action_dim=5, state_dim=4, ctx_len=24, ctx_dim=16, weight_std=0.2)
    W, I = wl.make_weights(cfg), dict(wl.make_inputs(cfg))
    S = cfg["ctx_len"]
    text = np.zeros((1, S), bool); text[0, :10] = True
    image = np.zeros((1, S), bool); image[0, 6:18] = True
    I.update(text_mask=text, image_mask=image)
    W64 = oracle.cast_weights(W)
    table, tb = oracle.modulation_table(cfg, W64, oracle.schedule(2))
    x0 = I["x0"].astype(np.float64)

    def step(inputs):
        tr = []   # residual after the in-projection, then after every block
        v = oracle.velocity(cfg, W64, oracle.bind(cfg, W64, inputs), x0, table, tb, 0, tr)
        return v, tr

    base, tr0 = step(I)

    def moved(rows):
        z = I["context"].copy()
        z[0, rows] += 3.0 * RNG.standard_normal((len(rows), z.shape[2]))
        v, tr = step(dict(I, context=z))
        return v, [float(np.max(np.abs(a - b))) for a, b in zip(tr, tr0)]

    v, d = moved([12, 15])          # shown by the image mask only
    assert d[1] == 0.0 and d[2] == 0.0 and d[3] > 1e-6
    v, d = moved([2, 5])            # shown by the text mask only
    assert d[1] > 1e-6
    v, d = moved([19, 23])          # hidden from both
    np.testing.assert_array_equal(v, base)


def test_dit_shared_mask_equals_compacted_context():
    # masking keys == dropping them: with one mask for every cross block, a request equals
    # its run on the compacted context
    cfg = wl.workload("dit_b1", batch=2, n_layers=2, hidden=64, n_heads=2, head_dim=32, n_kv_heads=2, mlp_dim=128,
                      action_horizon=5, action_dim=4, state_dim=3, ctx_len=20, ctx_dim=12, weight_std=0.2)
    W, I = wl.make_weights(cfg), dict(wl.make_inputs(cfg))
    m = RNG.random((2, 20)) < 0.5
    m[:, 0] = True
    xr = oracle.run(cfg, W, dict(I, text_mask=m, image_mask=m), steps=2)
    for b in range(2):
        j = np.flatnonzero(m[b])
        Ib = {nm: a[b:b + 1] for nm, a in I.items()}
        Ib["context"] = I["context"][b:b + 1, j]
        xb = oracle.run(dict(cfg, batch=1, ctx_len=len(j)), W, Ib, steps=2)
        np.testing.assert_allclose(xr[b:b + 1], xb, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------- low-bit weights
def test_fp8_e4m3_codes_match_torch_and_brute_force():
    # the format's 256 codes: 254 values and two NaN; encoding picks the nearest value, ties to
    # an even mantissa (brute force over every code), and agrees with torch's float8_e4m3fn
    vals = oracle.fp8_e4m3_value(np.arange(256))
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF]) and np.sum(np.isnan(vals)) == 2
    assert np.nanmax(vals) == 448.0 and vals[1] == 2.0 ** -9 and vals[8] == 2.0 ** -6
    finite = np.array([c for c in range(256) if not np.isnan(vals[c])])
    x = np.concatenate([RNG.standard_normal(3000) * 40, RNG.standard_normal(3000) * 3e-3,
                        (vals[finite][:, None] + np.array([0.0])).ravel(),
                        0.5 * (np.sort(vals[finite])[1:] + np.sort(vals[finite])[:-1])])   # every midpoint
    x = np.clip(x, -448, 448)
    codes = oracle.fp8_e4m3_encode(x)
    got = oracle.fp8_e4m3_value(codes)
    d = np.abs(vals[finite][None, :] - x[:, None])
    best = d.min(axis=1)
    assert np.all(np.abs(got - x) == best)                      # nearest
    tie = (d == best[:, None]).sum(axis=1) > 1
    assert tie.sum() > 200
    assert np.all((codes[tie] & 1) == 0)                        # ties: even mantissa
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes, ref)
    with pytest.raises(ValueError):
        oracle.fp8_e4m3_encode(np.array([449.0]))


def test_fp8_row_scales_and_error_bound():
    # per row the smallest power of two that brings max |w| within 448; the dequantized
    # weight is within half a quantum of w (relative 2^-4 for normal values)
    w = np.stack([RNG.standard_normal(256) * s for s in (1e-3, 0.02, 1.0, 300.0)] + [np.zeros(256)])
    w[1, 7] = 448 * 2.0 ** -8   # a row max exactly 448 2^e: e = -8, not -7
    codes, e, deq = oracle.quantize_fp8_rows(w)
    amax = np.abs(w).max(axis=1)
    for r in range(4):
        assert amax[r] <= 448 * 2.0 ** e[r] and amax[r] > 448 * 2.0 ** (e[r] - 1)
        q = np.ldexp(w[r], -e[r])
        assert np.all(np.abs(q) <= 448)
        quantum = np.ldexp(1.0, np.maximum(np.frexp(np.abs(q))[1] - 1, -6) - 3)
        assert np.all(np.abs(np.ldexp(deq[r], -e[r]) - q) <= quantum / 2)
    assert e[4] == 0 and np.all(deq[4] == 0)
    # dequantized values are exact in bf16 (at most 4 significant bits times a power of two)
    np.testing.assert_array_equal(wl.round_bf16(deq[:4].astype(np.float32)), deq[:4].astype(np.float32))
    # the result is a function of the row alone: scaling a row by 2^k scales e by k
    c2, e2, d2 = oracle.quantize_fp8_rows(np.ldexp(w[:4], 5))
    np.testing.assert_array_equal(c2, codes[:4])
    np.testing.assert_array_equal(e2, e[:4] + 5)


def _fp8_expected(cfg, key):
    """The matrices the low-bit format covers, listed by hand: every per-layer matrix of the
    pi0.5-shaped expert; in the DiT head q, o, ff1, ff2 of every block and k, v of the
    self-attention (odd) blocks only."""
    parts = key.split(".")
    if cfg["arch"] == wl.ARCH_PREFIX_JOINT:
        return parts[0] == "layers" and parts[2] in ("q", "k", "v", "o", "gate", "up", "down") and parts[3] == "w"
    if parts[0] != "blocks" or parts[3] != "w":
        return False
    return parts[2] in ("q", "o", "ff1", "ff2") or (parts[2] in ("k", "v") and int(parts[1]) % 2 == 1)


@pytest.mark.parametrize("name", ["tiny_fp32", "dit_b1"])
def test_fp8_weights_replace_only_layer_matrices(name):
    cfg = _tiny() if name == "tiny_fp32" else wl.workload(name, n_layers=4, hidden=64, n_heads=2, head_dim=32,
                                                          n_kv_heads=2, mlp_dim=128, ctx_dim=48)
    W = wl.make_weights(cfg)
    Q = oracle.fp8_weights(cfg, W)
    n = 0
    for k in W:
        if _fp8_expected(cfg, k):
            n += 1
            assert not np.array_equal(Q[k], W[k])
            e = oracle.fp8_row_exponents(W[k])[:, None]   # half a quantum: relative 2^-4, or 2^(e-10) for subnormals
            assert np.all(np.abs(Q[k] - W[k]) <= np.maximum(np.abs(W[k]) / 16, np.ldexp(1.0, e - 10)))
        else:
            np.testing.assert_array_equal(Q[k], W[k])
    L = cfg["n_layers"]
    assert n == (7 * L if cfg["arch"] == wl.ARCH_PREFIX_JOINT else 4 * L + 2 * (L // 2))


# ----------------------------------------------------------------------------- after the path
def test_quantile_unnormalize_inverts_openpi_normalization():
    # pi0.5 Design, "Embodiment adapters": the normalization with its epsilon, inverted
    rng = np.random.default_rng(7)
    q01 = rng.normal(size=7) - 1.0
    q99 = q01 + rng.uniform(0.1, 3.0, size=7)
    x = rng.uniform(q01 - 0.5, q99 + 0.5, size=(2, 5, 7))
    y = oracle.quantile_normalize(x, q01, q99, oracle.UNNORM_QUANTILE_EPS)
    pad = np.concatenate([y, rng.normal(size=(2, 5, 25))], axis=2)   # model width 32
    back = oracle.quantile_unnormalize(pad, q01, q99, oracle.UNNORM_QUANTILE_EPS, robot_dim=7)
    np.testing.assert_allclose(back, x, rtol=0, atol=1e-12)
    # the ends of the model range: -1 -> q01, +1 -> q99 + 1e-6 (the epsilon is part of the formula)
    ends = np.stack([-np.ones(7), np.ones(7)])[None]
    u = oracle.quantile_unnormalize(ends, q01, q99, oracle.UNNORM_QUANTILE_EPS)
    np.testing.assert_array_equal(u[0, 0], q01)
    np.testing.assert_allclose(u[0, 1], q99 + 1e-6, rtol=0, atol=1e-15)


def test_quantile_unnormalize_gr00t_clip_and_slice():
    # GR00T N1.7, "Policy contract": clip to [-1, 1], no epsilon, no guard; the policy keeps
    # a horizon shorter than the model's 40 and the robot's width
    q01 = np.array([-2.0, 0.0, 1.0, 5.0, -1.0, 0.5, 0.0])
    q99 = np.array([2.0, 1.0, 3.0, 5.0, 1.0, 0.5, 4.0])   # dims 3 and 5 degenerate
    x = np.zeros((1, 40, 32))
    x[0, 0, :7] = [-1.0, 1.0, 0.0, 0.3, 7.0, -9.0, 0.5]
    x[0, 1, :7] = [3.0, -3.0, 1.0, 1.0, -1.0, 1.0, -0.5]
    x[0, 20, :] = 99.0                                     # past the kept horizon
    u = oracle.quantile_unnormalize(x, q01, q99, oracle.UNNORM_QUANTILE_CLIP, robot_horizon=16, robot_dim=7)
    assert u.shape == (1, 16, 7)
    np.testing.assert_allclose(u[0, 0], [-2.0, 1.0, 2.0, 5.0, 1.0, 0.5, 3.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(u[0, 1], [2.0, 0.0, 3.0, 5.0, -1.0, 0.5, 1.0], rtol=0, atol=1e-15)
    # x = 0 -> midpoint of (q01, q99) for every kept step without a planted value
    np.testing.assert_allclose(u[0, 2:], np.broadcast_to((q01 + q99) / 2, (14, 7)), rtol=0, atol=1e-15)
    # normalization maps a degenerate group to zero and clips the rest
    y = oracle.quantile_normalize(np.array([5.0, 9.0]), np.array([5.0, 0.0]), np.array([5.0, 4.0]),
                                  oracle.UNNORM_QUANTILE_CLIP)
    np.testing.assert_array_equal(y, [0.0, 1.0])
    # round trip inside the bounds (non-degenerate groups)
    rng = np.random.default_rng(3)
    lo = rng.normal(size=4); hi = lo + rng.uniform(0.5, 2.0, size=4)
    v = rng.uniform(lo, hi, size=(3, 6, 4))
    back = oracle.quantile_unnormalize(oracle.quantile_normalize(v, lo, hi, oracle.UNNORM_QUANTILE_CLIP),
                                       lo, hi, oracle.UNNORM_QUANTILE_CLIP)
    np.testing.assert_allclose(back, v, rtol=0, atol=1e-12)


def test_increasing_schedule_constant_field():
    # GR00T integrates tau 0 -> 1 (vla.cpp Eq. (1) with the schedule reversed): the direction
    # is the tau array alone; with a constant field x_T = x_0 + (tau_T - tau_0) c
    T = 4
    tau = np.arange(T + 1) / T
    sched = oracle.schedule(T, tau)
    np.testing.assert_allclose(np.diff(sched), 1.0 / T)
    cfg = _tiny()
    w, I = wl.make_weights(cfg), wl.make_inputs(cfg)
    c = np.linspace(-1.0, 1.0, cfg["action_dim"]).astype(np.float32)
    w["action_out.w"] = np.zeros_like(w["action_out.w"])
    w["action_out.b"] = c
    xT = oracle.run(cfg, w, I, steps=T, tau=tau)
    np.testing.assert_allclose(xT, I["x0"].astype(np.float64) + c.astype(np.float64), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- bf16 operand reading
def _torch_bf16(vec):
    """float32, then bfloat16, both round-to-nearest-even, by torch's own conversions."""
    return torch.tensor(vec, dtype=torch.float64).to(torch.float32).to(torch.bfloat16).to(torch.float64).tolist()


def test_round_bf16_matches_torch_including_ties():
    # exact ties (lower 16 bits 0x8000) on both parities of the kept bit, both signs, and the
    # binade edges where rounding up carries into the exponent
    hi = np.array([0x3F80, 0x3F81, 0x4049, 0xC2F7, 0x3F7F, 0x7F7E, 0x0080, 0x8001], dtype=np.uint32)
    lo = np.array([0x0000, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    pats = (hi[:, None] << 16 | lo[None, :]).ravel()
    x32 = pats.view(np.float32)
    got = oracle.round_bf16(x32)
    ref = torch.from_numpy(x32.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(got, ref)
    # float64 input is held in float32 first, as the kernels' fp32 accumulators hold it
    x64 = RNG.standard_normal(4096) * np.exp(RNG.uniform(-20, 20, 4096))
    np.testing.assert_array_equal(oracle.round_bf16(x64), np.array(_torch_bf16(x64.tolist())))
    # a tie goes to the even neighbour: 1 + 2^-8 (between 1 and 1 + 2^-7) rounds down to 1
    assert oracle.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert oracle.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


def test_round_acts_time_conditioning_rounds_the_mlp_operands():
    """The bf16 reading of the modulation table against torch with bf16 casts at the
    embedding and both time-MLP activations (the table itself stays exact)."""
    cfg = wl.workload("tiny_fp32")
    W = oracle.cast_weights(wl.make_weights(cfg))
    tau = oracle.schedule(4)
    table, _ = oracle.modulation_table(cfg, W, tau, round_acts=True)
    bf = lambda t: t.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    e = bf(t64(oracle.sinusoidal_embedding(tau[:4], cfg["hidden"])))
    c = bf(F.silu(e @ t64(W["time_in.w"]).T + t64(W["time_in.b"])))
    c = bf(F.silu(c @ t64(W["time_out.w"]).T + t64(W["time_out.b"])))
    S, O, D = W["mod.w"].shape
    ref = (c @ t64(W["mod.w"]).reshape(S * O, D).T).reshape(4, S, O) + t64(W["mod.b"])
    np.testing.assert_allclose(table, ref.numpy(), rtol=1e-12, atol=1e-12)
    exact, _ = oracle.modulation_table(cfg, W, tau)
    assert 0 < oracle.e_rel(table, exact) < 1e-2


def test_round_acts_rounds_bf16_tensors_where_formed():
    """round_acts against the scalar brute force with torch's bf16 rounding at the norm's scaled
    input and shift, the chunk's queries and keys after RoPE, its values, the attention output
    and the gated-GELU activation."""
    cfg = wl.workload("tiny_fp32", n_layers=2, hidden=8, n_heads=2, head_dim=4, mlp_dim=6,
                      action_horizon=3, action_dim=2, prefix_len=4, weight_std=0.5)
    W, I = oracle.cast_weights(wl.make_weights(cfg)), wl.make_inputs(cfg)
    bound = oracle.bind(cfg, W, I)
    table, tb = oracle.modulation_table(cfg, W, oracle.schedule(2))
    x = I["x0"].astype(np.float64)
    v = oracle.velocity(cfg, W, bound, x, table, tb, 1, round_acts=True)
    Wl = {k: np.asarray(a).tolist() for k, a in W.items()}
    ref = _brute_velocity_pi05(cfg, Wl, I, x[0].tolist(), table[1].tolist(), rq=_torch_bf16)
    np.testing.assert_allclose(v[0], np.array(ref), rtol=1e-10, atol=1e-12)
    exact = oracle.velocity(cfg, W, bound, x, table, tb, 1)
    e = oracle.e_rel(v, exact)
    assert 0 < e < 2e-2, e   # the reading moves the result by bf16-sized amounts, not more
