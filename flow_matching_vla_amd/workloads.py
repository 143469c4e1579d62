"""Seeded synthetic workloads for the flow-matching denoise loop.

This module only describes and draws inputs: the five model/workload shapes, the
names and shapes of every weight tensor, and seeded random draws (standard normal
times a width, rounded to bfloat16 where the workload is bf16). It contains none
of the method's arithmetic, so both the CPU oracle side (tests, bench baseline)
and the HIP path can take their inputs from it without sharing any computation.

Shapes follow the pages' models: the pi0.5 action expert (18 layers, hidden
1024, one 256-wide K/V head shared by all query heads; "pi0.5 Design" page,
architecture diagram) and a GR00T-style DiT action head (32 blocks alternating
self- and cross-attention; "GR00T N1.7" page, section "action").
"""
from __future__ import annotations

import copy
import numpy as np

ARCH_PREFIX_JOINT = 0  # pi0.5-style expert: joint attention over bound prefix K/V + suffix
ARCH_DIT_CROSS = 1     # GR00T-style DiT: alternating cross-attention (even blocks) and self-attention

DTYPE_F32 = 0
DTYPE_BF16 = 1

# The five workloads, in the order they are numbered (index = seed group).
_BASE_PI05 = dict(
    arch=ARCH_PREFIX_JOINT, dtype=DTYPE_BF16, n_layers=18, hidden=1024, n_heads=8, head_dim=256,
    n_kv_heads=1, mlp_dim=4096, mlp_gated=1, action_horizon=50, action_dim=32, state_tokens=0,
    state_dim=0, ctx_len=0, ctx_dim=0, prefix_len=816, batch=1, steps=10, rope_base=10000.0,
    norm_eps=1e-6, weight_std=0.02,
)

WORKLOADS = [
    dict(_BASE_PI05, name="tiny_fp32", dtype=DTYPE_F32, n_layers=2, hidden=256, n_heads=4,
         head_dim=64, mlp_dim=1024, action_horizon=16, action_dim=7, prefix_len=64, batch=1,
         steps=4),
    dict(_BASE_PI05, name="pi05_b1"),
    dict(_BASE_PI05, name="pi05_b8", batch=8),
    dict(name="dit_b1", arch=ARCH_DIT_CROSS, dtype=DTYPE_BF16, n_layers=32, hidden=1536,
         n_heads=24, head_dim=64, n_kv_heads=24, mlp_dim=6144, mlp_gated=0, action_horizon=40,
         action_dim=32, state_tokens=1, state_dim=32, ctx_len=600, ctx_dim=2048, prefix_len=0,
         batch=1, steps=4, rope_base=0.0, norm_eps=1e-6, weight_std=0.02),
    dict(_BASE_PI05, name="pi05_b64", batch=64, prefix_len=1024),
]
WORKLOAD_INDEX = {w["name"]: i for i, w in enumerate(WORKLOADS)}


def workload(name_or_index, **overrides) -> dict:
    """Return a copy of a workload description, optionally with fields overridden."""
    idx = name_or_index if isinstance(name_or_index, int) else WORKLOAD_INDEX[name_or_index]
    cfg = copy.deepcopy(WORKLOADS[idx])
    cfg["index"] = idx
    cfg.update(overrides)
    return cfg


def n_sites(cfg) -> int:
    """Modulation sites: two per layer plus the final norm (pi0.5), one per block plus the output (DiT)."""
    L = cfg["n_layers"]
    return 2 * L + 1 if cfg["arch"] == ARCH_PREFIX_JOINT else L + 1


def weight_shapes(cfg) -> dict:
    """Name -> shape of every weight tensor, nn.Linear convention ([out, in])."""
    D, L, F = cfg["hidden"], cfg["n_layers"], cfg["mlp_dim"]
    nq, dh, nkv, da = cfg["n_heads"], cfg["head_dim"], cfg["n_kv_heads"], cfg["action_dim"]
    S = n_sites(cfg)
    shp = {
        "time_in.w": (D, D), "time_in.b": (D,),
        "time_out.w": (D, D), "time_out.b": (D,),
        "mod.w": (S, 3 * D, D), "mod.b": (S, 3 * D),
        "action_in.w": (D, da), "action_in.b": (D,),
        "action_out.w": (da, D), "action_out.b": (da,),
    }
    if cfg["arch"] == ARCH_PREFIX_JOINT:
        for l in range(L):
            p = f"layers.{l}."
            shp[p + "q.w"] = (nq * dh, D)
            shp[p + "k.w"] = (nkv * dh, D)
            shp[p + "v.w"] = (nkv * dh, D)
            shp[p + "o.w"] = (D, nq * dh)
            shp[p + "gate.w"] = (F, D)
            if cfg["mlp_gated"]:
                shp[p + "up.w"] = (F, D)
            shp[p + "down.w"] = (D, F)
    else:
        shp["time_bias.w"] = (D, D)
        shp["time_bias.b"] = (D,)
        shp["state_in.w"] = (D, cfg["state_dim"])
        shp["state_in.b"] = (D,)
        for i in range(L):
            p = f"blocks.{i}."
            kin = cfg["ctx_dim"] if i % 2 == 0 else D
            shp[p + "q.w"] = (D, D)
            shp[p + "k.w"] = (D, kin)
            shp[p + "v.w"] = (D, kin)
            shp[p + "o.w"] = (D, D)
            shp[p + "ff1.w"] = (F, D)
            shp[p + "ff2.w"] = (D, F)
    return shp


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returned as float32."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(np.shape(a))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are already bf16-representable."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return (u >> 16).astype(np.uint16).reshape(np.shape(a))


def _draw(seed: int, shape, std: float, bf16: bool) -> np.ndarray:
    """Standard normal draws of one tensor from torch's CPU generator (Mersenne Twister,
    seeded per tensor), times std, rounded to bf16 (ties to even) when asked."""
    import torch

    g = torch.Generator().manual_seed(int(seed))
    t = torch.randn(tuple(int(d) for d in shape), generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(float(std))
    if bf16:
        t = t.to(torch.bfloat16).to(torch.float32)
    return t.numpy()


def input_shapes(cfg) -> dict:
    """Name -> shape of the per-observation inputs (prefix K/V or context + state) and x0."""
    B, H, da = cfg["batch"], cfg["action_horizon"], cfg["action_dim"]
    shp = {"x0": (B, H, da)}
    if cfg["arch"] == ARCH_PREFIX_JOINT:
        P, dh = cfg["prefix_len"], cfg["head_dim"]
        for l in range(cfg["n_layers"]):
            shp[f"prefix.k.{l}"] = (B, P, 1, dh)
            shp[f"prefix.v.{l}"] = (B, P, 1, dh)
    else:
        shp["context"] = (B, cfg["ctx_len"], cfg["ctx_dim"])
        shp["state"] = (B, cfg["state_tokens"], cfg["state_dim"])
    return shp


def make_weights(cfg, names=None) -> dict:
    """Seeded weights: N(0, weight_std) drawn in float32, rounded to bf16 for bf16 workloads.

    The seed of a tensor is 1000 * workload index + its position in the sorted name list,
    so any single tensor can be regenerated on its own.
    """
    shp = weight_shapes(cfg)
    order = sorted(shp)
    bf16 = cfg["dtype"] == DTYPE_BF16
    out = {}
    for ti, name in enumerate(order):
        if names is not None and name not in names:
            continue
        out[name] = _draw(1000 * cfg["index"] + ti, shp[name], cfg["weight_std"], bf16)
    return out


def make_inputs(cfg) -> dict:
    """Seeded per-observation inputs and initial noise, N(0, 1); K/V and context rounded to bf16
    for bf16 workloads, x0 and state kept in float32 (the loop state is float32)."""
    shp = input_shapes(cfg)
    bf16 = cfg["dtype"] == DTYPE_BF16
    base = 1000 * cfg["index"] + 500
    out = {}
    for ti, name in enumerate(sorted(shp)):
        rb = bf16 and name not in ("x0", "state")
        out[name] = _draw(base + ti, shp[name], 1.0, rb)
    return out


def param_count(cfg) -> int:
    return int(sum(int(np.prod(s)) for s in weight_shapes(cfg).values()))


def make_visibility(cfg, seed: int = 0) -> dict:
    """Seeded per-request key visibility for a mixed-request batch (no arithmetic of the
    method: lengths and booleans only).

    PREFIX_JOINT -> {"prefix_lens": int32 [B]}: request 0 keeps the whole bound prefix, the
    others a uniform draw in [P/2, P]: compact prefixes of different lengths sharing one
    binding.
    DIT_CROSS -> {"text_mask", "image_mask": bool [B, S]}: every context token is an image
    token (probability 3/4) or a text token, interleaved at random (the masks are arbitrary
    booleans, not spans); a uniform number in [0, S/4] of trailing tokens per request is
    padding, hidden from both. A request left with no visible token in a mask sees token 0
    in it."""
    rng = np.random.default_rng(7919 * (cfg["index"] + 1) + seed)
    B = cfg["batch"]
    if cfg["arch"] == ARCH_PREFIX_JOINT:
        P = cfg["prefix_len"]
        lens = rng.integers(P // 2, P + 1, size=B).astype(np.int32)
        lens[0] = P
        return {"prefix_lens": lens}
    S = cfg["ctx_len"]
    image = rng.random((B, S)) < 0.75
    valid = np.ones((B, S), dtype=bool)
    for b in range(B):
        pad = int(rng.integers(0, S // 4 + 1))
        if pad:
            valid[b, S - pad:] = False
    text_mask = valid & ~image
    image_mask = valid & image
    for m in (text_mask, image_mask):   # an empty mask shows token 0 (masks may overlap)
        m[~m.any(axis=1), 0] = True
    return {"text_mask": text_mask, "image_mask": image_mask}
