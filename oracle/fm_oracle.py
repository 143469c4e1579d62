"""Plain CPU oracle of the flow-matching denoise loop of a VLA action head.

TEST INFRASTRUCTURE ONLY. This module is the yardstick the HIP path is checked
against: tests, the package's smoke check and the benchmark's CPU-baseline leg may
call it; the product path never does. It shares no code with the HIP library and
imports nothing from it: only numpy. Every step is written out in the order the
pages state it, one tensor operation at a time, in float64 by default (float32 on
request), with no fusion, blocking or reordering.

Sources (pages as titled; sections, equations):
  * vla.cpp: A Unified Inference Runtime for Vision-Language-Action Models,
    Sec. III-A Eq. (1) (Euler integration over the schedule tau_0..tau_T),
    Sec. III-B Eq. (2) (softmax attention over cached keys/values),
    Sec. III-E Eq. (5) (e_inf, e_rel).
  * pi0.5 Design (TensorRT Edge-LLM): architecture diagram (expert 18 layers,
    hidden 1024, head_dim 256, one K/V head), sequence diagram (cond -> per-step
    modulation rows, loop t: 1 -> 0, x += dt * v), "Component contract"
    (adarms_modulation row layout and (scale, shift, gate) packing; action_pred is
    the velocity), "Attention and the K/V pool" (suffix K/V appended after the
    prefix; head fold of all query heads onto the single K/V head).
  * GR00T N1.7 (TensorRT Edge-LLM): section "action" (32 DiT blocks, odd blocks
    self-attend over state + action tokens, even blocks cross-attend into the VL
    context), "Build-time constants" (per-step modulation rows, timestep bias),
    "vl_backbone" (cross-attention K/V projected once and kept bound).
  * LoongForge GR00T-N1.7 training optimization blog, Sec. 3.3 (rotate_half RoPE,
    RMSNorm with fp32 reduction, gate * up MLP pattern).

Readings taken where the pages are silent (each is listed with its reason in the
design notes of the repository): sinusoid periods 4e-3..4.0 and a two-layer SiLU
time MLP; (1 + scale) modulation; RMS/Layer norm epsilon 1e-6 without a learned
weight; tanh-form GELU on the gate branch; RoPE base 10000 on queries and suffix
keys only (the prefix keys arrive already rotated); biases only on the time MLP,
modulation Denses and the action/state in/out projections; DiT feed-forward width
4 x hidden, ungated, behind a plain LayerNorm and an ungated residual.

Parity pins: every function here is checked by `tests/test_oracle.py` against
closed forms, invariants, library routines or brute force. The numerical values of
the time embedding and modulation table are "parity unpinned" beyond their
invariants, because the pages print no worked values for them.
"""
from __future__ import annotations

import math
import numpy as np

ARCH_PREFIX_JOINT = 0
ARCH_DIT_CROSS = 1

SINUSOID_MIN_PERIOD = 4e-3
SINUSOID_MAX_PERIOD = 4.0


# ----------------------------------------------------------------------------- schedule
def schedule(steps: int, tau=None, dtype=np.float64) -> np.ndarray:
    """Integration schedule tau_0..tau_T (vla.cpp Sec. III-A, Eq. (1); pi0.5 Design,
    sequence diagram: t runs from 1 to 0). Default: uniform, tau_k = 1 - k/T."""
    if tau is not None:
        tau = np.asarray(tau, dtype=dtype)
        if tau.shape != (steps + 1,):
            raise ValueError(f"schedule needs {steps + 1} values, got {tau.shape}")
        return tau
    return np.array([1.0 - k / steps for k in range(steps + 1)], dtype=dtype) if steps > 0 \
        else np.ones(1, dtype=dtype)


# ----------------------------------------------------------------------------- elementwise
def silu(x):
    return x / (1.0 + np.exp(-x))


def gelu_tanh(x):
    """GELU, tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    c = math.sqrt(2.0 / math.pi)
    return 0.5 * x * (1.0 + np.tanh(c * (x + 0.044715 * x * x * x)))


def linear(x, w, b=None):
    """y = x W^T (+ b), nn.Linear convention, W is [out, in]."""
    y = x @ w.T
    return y if b is None else y + b


# ----------------------------------------------------------------------------- norms
def rms_norm(h, eps):
    """h / sqrt(mean(h^2) + eps) over the last axis (LoongForge blog Sec. 3.3: RMSNorm with
    its reduction kept in full precision). No learned weight: the modulation supplies it."""
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)


def layer_norm(h, eps):
    """(h - mean) / sqrt(var + eps), biased variance, no affine (DiT AdaLN base norm)."""
    mu = np.mean(h, axis=-1, keepdims=True)
    d = h - mu
    return d / np.sqrt(np.mean(d * d, axis=-1, keepdims=True) + eps)


def modulate(n, scale, shift):
    """n * (1 + scale) + shift, scale/shift broadcast over tokens."""
    return n * (1.0 + scale) + shift


def split_site(row, D):
    """A modulation row packs (scale, shift, gate), each of width D (pi0.5 Design,
    "Component contract", adarms_modulation)."""
    return row[..., :D], row[..., D:2 * D], row[..., 2 * D:3 * D]


# ----------------------------------------------------------------------------- bf16 operands
def round_bf16(x):
    """x held in float32 (round to nearest, ties to even), then rounded to bfloat16 (1 sign,
    8 exponent, 7 stored mantissa bits), ties to even, as float64 (vla.cpp Sec. III-E: the
    reduced-precision model rounds to nearest even). bfloat16 is the upper half of a float32:
    adding 0x7FFF plus the lowest kept bit and clearing the lower 16 bits rounds to the
    nearest half, a tie going to the even one."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------- RoPE
def rope(x, positions, base):
    """Rotary embedding, rotate_half convention (LoongForge blog Sec. 3.3): for j < d/2,
    theta_j = base^(-2j/d), the pair (x_j, x_{j+d/2}) at position p rotates by p*theta_j:
    (a, b) -> (a cos - b sin, b cos + a sin). x: [..., T, d]; positions: [T]."""
    d = x.shape[-1]
    half = d // 2
    j = np.arange(half, dtype=np.float64)
    theta = base ** (-2.0 * j / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    cos = np.cos(ang).astype(x.dtype)
    sin = np.sin(ang).astype(x.dtype)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


# ----------------------------------------------------------------------------- attention
def attention(q, k, v, visible=None):
    """softmax(Q K^T / sqrt(d_k) + M) V (vla.cpp Eq. (2)), softmax over keys. The additive mask
    M is 0 where `visible` is true and -inf where it is false; visible=None is M = 0.

    q: [B, n_q, Tq, d]; k, v: [B, n_kv, Tk, d] with n_kv == 1 (the single K/V head shared by
    every query head, pi0.5 Design "Attention and the K/V pool") or n_kv == n_q; visible:
    booleans broadcastable to [B, n_q, Tq, Tk]. A query row with no visible key has no
    defined result (0 / 0); it comes out NaN here."""
    d = q.shape[-1]
    s = (q @ np.swapaxes(k, -1, -2)) / math.sqrt(d)
    if visible is not None:
        s = s + np.where(visible, 0.0, -np.inf).astype(s.dtype)
    with np.errstate(invalid="ignore"):
        s = s - np.max(s, axis=-1, keepdims=True)
        p = np.exp(s)
        p = p / np.sum(p, axis=-1, keepdims=True)
    return p @ v


# ----------------------------------------------------------------------------- time conditioning
def sinusoidal_embedding(tau, width, min_period=SINUSOID_MIN_PERIOD, max_period=SINUSOID_MAX_PERIOD):
    """e(tau) = [sin(2 pi tau / p_j)]_j ++ [cos(2 pi tau / p_j)]_j, j < width/2, with periods
    geometric from min_period to max_period. The time embedder that the pi0.5 cond component
    hoists out of the step (pi0.5 Design, cond paragraph); the constants are a reading."""
    tau = np.asarray(tau)
    half = width // 2
    frac = np.arange(half, dtype=np.float64) / max(half - 1, 1)
    period = min_period * (max_period / min_period) ** frac
    arg = tau[:, None].astype(np.float64) * (2.0 * math.pi / period)[None, :]
    return np.concatenate([np.sin(arg), np.cos(arg)], axis=-1).astype(tau.dtype)


def time_conditioning(w, tau_steps, round_acts=False):
    """c_k = SiLU(W_out SiLU(W_in e(tau_k) + b_in) + b_out) for each evaluated tau_k.
    round_acts: the bf16 model's reading, where the embedding and both activations are bf16
    tensors (each rounded where formed)."""
    rnd = round_bf16 if round_acts else (lambda a: a)
    D = w["time_in.w"].shape[0]
    e = rnd(sinusoidal_embedding(tau_steps, D))
    c = rnd(silu(linear(e, w["time_in.w"], w["time_in.b"])))
    return rnd(silu(linear(c, w["time_out.w"], w["time_out.b"])))


def modulation_table(cfg, w, tau, round_acts=False):
    """Per-step modulation rows, evaluated once per (steps, batch) off the step path
    (pi0.5 Design: the optional cond component, evaluated again only on a new step count or
    batch; GR00T N1.7 "Build-time constants"). Returns (table [T, S, 3D], time_bias [T, D] or None).

    table[k, s] = W_s c_k + b_s. The pages' tensor repeats each step's row once per
    request ([steps * batch, S, 3D]); every request shares tau_k, so the rows are equal
    across requests and one per step is kept here. round_acts: time_conditioning's reading
    (the rows themselves stay exact functions of the rounded c_k)."""
    T = len(tau) - 1
    if T == 0:
        return None, None
    c = time_conditioning(w, tau[:T], round_acts)          # [T, D]
    S, O, D = w["mod.w"].shape
    table = (w["mod.w"].reshape(S * O, D) @ c.T).T.reshape(T, S, O) + w["mod.b"][None]
    tb = None
    if cfg["arch"] == ARCH_DIT_CROSS:
        tb = linear(c, w["time_bias.w"], w["time_bias.b"])  # [T, D]
    return table, tb


# ----------------------------------------------------------------------------- bind
def bind(cfg, w, inputs, dtype=np.float64):
    """Per-observation conditioning, computed once and kept for the whole loop (vla.cpp
    Sec. III-B, observation reuse; GR00T N1.7 "Who runs what", vl_backbone row).

    pi0.5: the per-layer prefix K/V [B, P, 1, d_h] as given (already rotated by the
    prefix tower), and each request's compact prefix length P_b <= P ("prefix_lens", int
    [B]; default P for all): request b attends to its first P_b prefix keys and its chunk
    sits at positions P_b + i (pi0.5 Design, "Component contract": the filled length after
    the append is per request, and the prefix is compact). DiT: cross K/V of each even
    block, K_c = Z W_K^T, V_c = Z W_V^T, the state token W_s s + b_s, and the text and image
    masks over the context ("text_mask", "image_mask", bool [B, S]; default all visible;
    GR00T N1.7 section "action"). Arrays are returned read-only: the loop never writes them."""
    out = {}
    if cfg["arch"] == ARCH_PREFIX_JOINT:
        L = cfg["n_layers"]
        out["k"] = [np.asarray(inputs[f"prefix.k.{l}"], dtype=dtype)[:, :, 0, :][:, None] for l in range(L)]
        out["v"] = [np.asarray(inputs[f"prefix.v.{l}"], dtype=dtype)[:, :, 0, :][:, None] for l in range(L)]
        out["prefix_len"] = out["k"][0].shape[2] if L else 0
        B = out["k"][0].shape[0] if L else cfg["batch"]
        lens = inputs.get("prefix_lens")
        lens = np.full(B, out["prefix_len"], dtype=np.int64) if lens is None else np.asarray(lens, dtype=np.int64)
        if lens.shape != (B,) or np.any(lens < 0) or np.any(lens > out["prefix_len"]):
            raise ValueError("prefix_lens must be [B] within [0, prefix_len]")
        out["prefix_lens"] = lens
    else:
        nh, dh = cfg["n_heads"], cfg["head_dim"]
        z = np.asarray(inputs["context"], dtype=dtype)
        B, S, _ = z.shape
        out["k"], out["v"] = {}, {}
        for i in range(0, cfg["n_layers"], 2):
            kc = linear(z, w[f"blocks.{i}.k.w"].astype(dtype))
            vc = linear(z, w[f"blocks.{i}.v.w"].astype(dtype))
            out["k"][i] = kc.reshape(B, S, nh, dh).transpose(0, 2, 1, 3)
            out["v"][i] = vc.reshape(B, S, nh, dh).transpose(0, 2, 1, 3)
        s = np.asarray(inputs["state"], dtype=dtype)
        out["state_token"] = linear(s, w["state_in.w"].astype(dtype), w["state_in.b"].astype(dtype))
        for name in ("text_mask", "image_mask"):
            m = inputs.get(name)
            out[name] = np.ones((B, S), dtype=bool) if m is None else np.asarray(m, dtype=bool)
            if out[name].shape != (B, S):
                raise ValueError(f"{name} must be [B, S]")
    for key in ("k", "v"):
        vals = out[key].values() if isinstance(out[key], dict) else out[key]
        for a in vals:
            a.flags.writeable = False
    return out


# ----------------------------------------------------------------------------- velocity
def velocity_prefix_joint(cfg, w, bound, x, row, trace=None, round_acts=False):
    """One step of the pi0.5-shaped action expert: x [B, H, d_a] -> v [B, H, d_a].

    row: this step's modulation row [2L+1, 3D]; site 2l is layer l's input norm, 2l+1 its
    post-attention norm, the last site the final norm (pi0.5 Design, "Component contract").

    round_acts: a reading of the bf16 model rather than of the exact one, to tell rounding from
    bugs. Every activation that the bf16 model holds as a bf16 tensor is rounded to bfloat16
    (round_bf16) where it is formed, everything else stays exact:
      - the operand of each modulated norm's consumer: u = rinv * bf16(h (1 + scale)) +
        bf16(shift), rinv = 1 / sqrt(mean(h^2) + eps) of the unrounded h (the same u as
        n(h)(1 + scale) + shift, with the scaled input and the shift held in bf16);
      - the chunk's queries and keys after RoPE, its values, and the attention output;
      - the gated-GELU activation GELU(u W_gate^T) * (u W_up^T).
    The residual stream, the attention's scores and probabilities, x and v stay exact."""
    rnd = round_bf16 if round_acts else (lambda a: a)

    def norm_mod(h, site):
        scale, shift, _ = split_site(row[site], D)
        if not round_acts:
            return modulate(rms_norm(h, eps), scale, shift)
        rinv = 1.0 / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
        return (round_bf16(h * (1.0 + scale)) * rinv + round_bf16(shift)).astype(h.dtype)
    D, L = cfg["hidden"], cfg["n_layers"]
    nq, dh, eps = cfg["n_heads"], cfg["head_dim"], cfg["norm_eps"]
    B, H, _ = x.shape
    lens = bound["prefix_lens"]
    h = linear(x, w["action_in.w"], w["action_in.b"])
    if trace is not None:
        trace.append(h)
    for l in range(L):
        p = f"layers.{l}."
        gate = split_site(row[2 * l], D)[2]
        u = norm_mod(h, 2 * l)
        q = linear(u, w[p + "q.w"]).reshape(B, H, nq, dh).transpose(0, 2, 1, 3)
        k = linear(u, w[p + "k.w"]).reshape(B, H, 1, dh).transpose(0, 2, 1, 3)
        v = rnd(linear(u, w[p + "v.w"]).reshape(B, H, 1, dh).transpose(0, 2, 1, 3)).astype(h.dtype)
        o = np.empty((B, nq, H, dh), dtype=h.dtype)
        for b in range(B):   # each request: its compact prefix, then its own chunk
            P = lens[b]
            pos = P + np.arange(H)   # suffix positions continue after the compact prefix
            qb, kb = q[b:b + 1], k[b:b + 1]
            if cfg["rope_base"] > 0:
                qb = rope(qb, pos, cfg["rope_base"])
                kb = rope(kb, pos, cfg["rope_base"])
            qb, kb = rnd(qb).astype(h.dtype), rnd(kb).astype(h.dtype)
            K = np.concatenate([bound["k"][l][b:b + 1, :, :P], kb], axis=2)   # suffix after the prefix
            V = np.concatenate([bound["v"][l][b:b + 1, :, :P], v[b:b + 1]], axis=2)
            o[b] = attention(qb, K, V)[0]
        o = rnd(o.transpose(0, 2, 1, 3).reshape(B, H, nq * dh)).astype(h.dtype)
        h = h + gate * linear(o, w[p + "o.w"])
        gate = split_site(row[2 * l + 1], D)[2]
        u = norm_mod(h, 2 * l + 1)
        if cfg["mlp_gated"]:
            a = gelu_tanh(linear(u, w[p + "gate.w"])) * linear(u, w[p + "up.w"])
        else:
            a = gelu_tanh(linear(u, w[p + "gate.w"]))
        a = rnd(a).astype(h.dtype)
        h = h + gate * linear(a, w[p + "down.w"])
        if trace is not None:
            trace.append(h)
    u = norm_mod(h, 2 * L)
    return linear(u, w["action_out.w"], w["action_out.b"])


def velocity_dit_cross(cfg, w, bound, x, row, time_bias, trace=None):
    """One step of the DiT action head (GR00T N1.7, section "action"): the state token is
    prepended to the action tokens; 0-based even blocks cross-attend into the bound context
    K/V, odd blocks self-attend over state + action tokens; AdaLN-modulated LayerNorm with a
    gated attention residual, plain LayerNorm + GELU feed-forward; the output norm uses the
    last site and only action tokens are projected to the velocity. A cross block reads the
    text mask when its index is a multiple of 4 and the image mask otherwise (one cross block
    in two reads text)."""
    D, L = cfg["hidden"], cfg["n_layers"]
    nh, dh, eps = cfg["n_heads"], cfg["head_dim"], cfg["norm_eps"]
    B, H, _ = x.shape
    h_a = linear(x, w["action_in.w"], w["action_in.b"]) + time_bias
    h = np.concatenate([bound["state_token"], h_a], axis=1)
    T = h.shape[1]
    if trace is not None:
        trace.append(h)
    for i in range(L):
        p = f"blocks.{i}."
        scale, shift, gate = split_site(row[i], D)
        u = modulate(layer_norm(h, eps), scale, shift)
        q = linear(u, w[p + "q.w"]).reshape(B, T, nh, dh).transpose(0, 2, 1, 3)
        if i % 2 == 0:
            # cross block: the text mask when i % 4 == 0, else the image mask
            K, V = bound["k"][i], bound["v"][i]
            mask = bound["text_mask"] if i % 4 == 0 else bound["image_mask"]
            vis = mask[:, None, None, :]
        else:
            K = linear(u, w[p + "k.w"]).reshape(B, T, nh, dh).transpose(0, 2, 1, 3)
            V = linear(u, w[p + "v.w"]).reshape(B, T, nh, dh).transpose(0, 2, 1, 3)
            vis = None
        o = attention(q, K, V, vis).transpose(0, 2, 1, 3).reshape(B, T, D)
        h = h + gate * linear(o, w[p + "o.w"])
        h = h + linear(gelu_tanh(linear(layer_norm(h, eps), w[p + "ff1.w"])), w[p + "ff2.w"])
        if trace is not None:
            trace.append(h)
    scale, shift, _ = split_site(row[L], D)
    u = modulate(layer_norm(h[:, cfg["state_tokens"]:], eps), scale, shift)
    return linear(u, w["action_out.w"], w["action_out.b"])


def velocity(cfg, w, bound, x, table, time_bias, k, trace=None, round_acts=False):
    """v_theta(X^k, tau_k, C) of vla.cpp Eq. (1), for step k of the scheduled table.
    trace: optional list that receives the residual stream after the in-projection and
    after every layer (vla.cpp Sec. III-E: intermediate tensors localize discrepancies).
    round_acts: the bf16-operand reading of velocity_prefix_joint (pi0.5-shaped expert only)."""
    if cfg["arch"] == ARCH_PREFIX_JOINT:
        return velocity_prefix_joint(cfg, w, bound, x, table[k], trace, round_acts)
    if round_acts:
        raise ValueError("round_acts is a reading of the pi0.5-shaped expert only")
    return velocity_dit_cross(cfg, w, bound, x, table[k], time_bias[k], trace)


# ----------------------------------------------------------------------------- the loop
def cast_weights(w, dtype=np.float64):
    return {n: np.asarray(a, dtype=dtype) for n, a in w.items()}


def denoise(cfg, w, bound, x0, steps, tau=None, field=None, return_trace=False, dtype=np.float64):
    """Euler integration X^{k+1} = X^k + (tau_{k+1} - tau_k) v(X^k, tau_k) for k = 0..T-1
    (vla.cpp Sec. III-A, Eq. (1)); the update is applied to the float32-or-wider chunk and
    the velocity (not the updated chunk) is what one step of the network produces
    (pi0.5 Design, action_pred).

    field: optional callable (x, k, tau_k) -> v replacing the network, for closed-form checks.
    Returns X^T, and with return_trace the list of (X^k, v_k) pairs."""
    tau = schedule(steps, tau, dtype=dtype)
    x = np.array(x0, dtype=dtype, copy=True)
    trace = []
    if steps > 0 and field is None:
        table, tb = modulation_table(cfg, w, tau)
    for k in range(steps):
        if field is not None:
            v = field(x, k, tau[k])
        else:
            v = velocity(cfg, w, bound, x, table, tb, k)
        if return_trace:
            trace.append((x.copy(), v))
        x = x + (tau[k + 1] - tau[k]) * v
    return (x, trace) if return_trace else x


def run(cfg, weights, inputs, steps=None, tau=None, dtype=np.float64, return_trace=False, field=None):
    """Cast the seeded weights and inputs to the oracle precision, bind, and denoise x0."""
    steps = cfg["steps"] if steps is None else steps
    w = cast_weights(weights, dtype)
    bound = bind(cfg, w, inputs, dtype=dtype)
    return denoise(cfg, w, bound, inputs["x0"], steps, tau=tau, field=field,
                   return_trace=return_trace, dtype=dtype)


# ----------------------------------------------------------------------------- low-bit weights
# Weight streaming at half the bytes (vla.cpp Sec. IV-D, Table V: quantized GR00T weights; pi0.5
# Design: FP8 named as an option for the expert): each row of a per-layer matrix (one output
# feature) is stored as FP8 E4M3 codes times one power-of-two scale. The codes follow the OCP
# E4M3 ("fn") format: 1 sign, 4 exponent (bias 7) and 3 mantissa bits, subnormals below 2^-6,
# largest value 448, no infinity. The expert then computes with the dequantized weights.
FP8_E4M3_MAX = 448.0
FP8_LAYER_WEIGHTS = ("q.w", "k.w", "v.w", "o.w", "gate.w", "up.w", "down.w")


def fp8_e4m3_value(code):
    """Value of E4M3 code bytes (the format's definition; 0x7F / 0xFF are NaN)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e, m = (c >> 3) & 0xF, c & 7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def fp8_e4m3_encode(x):
    """Round to the nearest E4M3 value, ties to an even mantissa, for |x| <= 448; returns the
    code bytes. The quantum is 2^(E - 3) in binade [2^E, 2^(E+1)) for E >= -6, and 2^-9 below
    2^-6 (subnormals); x / quantum is exact, so the rounding is a half-to-even integer round."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > FP8_E4M3_MAX):
        raise ValueError("outside the E4M3 range")
    a = np.abs(x)
    _, ex = np.frexp(a)                       # a = f 2^ex, f in [0.5, 1)
    E = np.maximum(ex - 1, -6)                # binade exponent, subnormals share -6
    q = np.ldexp(1.0, E - 3)
    n = np.round(a / q)                       # half to even
    v = n * q                                 # may step up to the next binade: still exact
    _, ev = np.frexp(np.where(v > 0, v, 1.0))
    Ev = ev - 1
    normal = v >= 2.0 ** -6
    e_field = np.where(normal, Ev + 7, 0)
    m_field = np.where(normal, np.round(v / np.ldexp(1.0, Ev - 3)) - 8, np.round(v / 2.0 ** -9)).astype(np.int64)
    code = (e_field.astype(np.int64) << 3) | m_field
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)   # the sign kept on a zero too


def fp8_row_exponents(w):
    """Per row, the smallest e with max |w_row| <= 448 2^e (exact: with max = f 2^x, f in
    [0.5, 1), e = x - 9 + [f > 0.875], as 448 = 0.875 2^9); 0 for an all-zero row."""
    amax = np.max(np.abs(np.asarray(w, dtype=np.float64)), axis=-1)
    f, x = np.frexp(amax)
    return np.where(amax > 0, x - 9 + (f > 0.875), 0).astype(np.int64)


def quantize_fp8_rows(w):
    """w [N, K] -> (codes uint8 [N, K], exponents int [N], dequantized float64 [N, K]) with
    w_row ~ value(codes_row) 2^e_row."""
    w = np.asarray(w, dtype=np.float64)
    e = fp8_row_exponents(w)
    codes = fp8_e4m3_encode(np.ldexp(w, -e[:, None]))
    return codes, e, np.ldexp(fp8_e4m3_value(codes), e[:, None])


FP8_BLOCK_WEIGHTS = ("q.w", "o.w", "ff1.w", "ff2.w")        # every DiT block
FP8_SELF_BLOCK_WEIGHTS = ("k.w", "v.w")                      # self-attention blocks only


def fp8_weight_names(cfg):
    """Names of the matrices the low-bit format covers. pi0.5-shaped expert: q, k, v, o, gate,
    up, down of every layer. DiT head: the matrices applied to the action tokens inside the
    loop, namely q, o, ff1, ff2 of every block and k, v of the self-attention (odd) blocks; the
    cross blocks' k, v act on the context once per observation (bind), outside the loop, and
    keep the configured dtype (reading: the low-bit format serves the streamed weights of the
    denoise loop)."""
    keys = []
    for l in range(cfg["n_layers"]):
        if cfg["arch"] == ARCH_PREFIX_JOINT:
            keys += [f"layers.{l}.{nm}" for nm in FP8_LAYER_WEIGHTS]
        else:
            names = FP8_BLOCK_WEIGHTS + (FP8_SELF_BLOCK_WEIGHTS if l % 2 == 1 else ())
            keys += [f"blocks.{l}.{nm}" for nm in names]
    return keys


def fp8_weights(cfg, w):
    """The matrices fp8_weight_names lists replaced by their FP8-dequantized values, everything
    else unchanged."""
    out = dict(w)
    for key in fp8_weight_names(cfg):
        if key in out:
            out[key] = quantize_fp8_rows(out[key])[2].astype(np.asarray(w[key]).dtype)
    return out


# ----------------------------------------------------------------------------- after the path
# The chunk leaves the loop in normalized model space; the step after maps it back to robot
# units with the action statistics (q01, q99 per dimension) and keeps the robot's share.
UNNORM_QUANTILE_EPS = 0    # pi0.5 (openpi quantile normalization, epsilon included)
UNNORM_QUANTILE_CLIP = 1   # GR00T (clip to [-1, 1], no epsilon)
QUANTILE_EPS = 1e-6


def quantile_normalize(x, q01, q99, kind):
    """Normalization of robot values into [-1, 1]-ish model space, written to pin its inverse.
    pi0.5 Design, "Embodiment adapters": (x - q01) / (q99 - q01 + 1e-6) * 2 - 1.
    GR00T N1.7, "Policy contract": 2 (x - q01) / (q99 - q01) - 1 clipped to [-1, 1], a group
    whose q99 equals its q01 mapping to zero instead of dividing by its range."""
    x = np.asarray(x, np.float64)
    q01 = np.asarray(q01, np.float64)
    q99 = np.asarray(q99, np.float64)
    if kind == UNNORM_QUANTILE_EPS:
        return (x - q01) / (q99 - q01 + QUANTILE_EPS) * 2.0 - 1.0
    span = q99 - q01
    safe = np.where(span == 0, 1.0, span)
    y = np.clip(2.0 * (x - q01) / safe - 1.0, -1.0, 1.0)
    return np.where(span == 0, 0.0, y)


def quantile_unnormalize(x, q01, q99, kind, robot_horizon=None, robot_dim=None):
    """Model-space chunk [B, H, d_a] -> robot units [B, robot_horizon, robot_dim].
    pi0.5 Design, "Embodiment adapters": the openpi normalization above inverted,
    (x + 1) / 2 * (q99 - q01 + 1e-6) + q01, then the chunk sliced to the robot's width.
    GR00T N1.7, "Policy contract": (clip(x, -1, 1) + 1) / 2 * (q99 - q01) + q01 with no
    guard, the policy keeping its own horizon (shorter than the model's) and width.
    q01 / q99 hold robot_dim values (the first robot_dim model dimensions)."""
    x = np.asarray(x, np.float64)
    B, H, da = x.shape
    hr = H if robot_horizon is None else robot_horizon
    dr = da if robot_dim is None else robot_dim
    assert 0 < hr <= H and 0 < dr <= da
    q01 = np.asarray(q01, np.float64).reshape(dr)
    q99 = np.asarray(q99, np.float64).reshape(dr)
    xs = x[:, :hr, :dr]
    if kind == UNNORM_QUANTILE_EPS:
        return (xs + 1.0) / 2.0 * (q99 - q01 + QUANTILE_EPS) + q01
    return (np.clip(xs, -1.0, 1.0) + 1.0) / 2.0 * (q99 - q01) + q01


# ----------------------------------------------------------------------------- metrics
def e_inf(a, ref):
    """Maximum absolute error (vla.cpp Sec. III-E, Eq. (5))."""
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(ref, np.float64))))


def e_rel(a, ref):
    """||A - A_ref||_2 / ||A_ref||_2 over the flattened tensors (vla.cpp Eq. (5)); undefined
    (None) when the reference norm is zero, in which case e_inf is the figure to report."""
    a = np.asarray(a, np.float64).ravel()
    r = np.asarray(ref, np.float64).ravel()
    n = np.linalg.norm(r)
    return None if n == 0 else float(np.linalg.norm(a - r) / n)
