"""Seeded synthetic inputs for the KDN layer forward and decode step.

This module draws random numbers and rounds them to the storage dtype; it
holds none of the layer's arithmetic.  It is the one piece shared by the GPU
tests, the oracle tests and the benchmark, so that both sides read exactly
the same (already rounded) values.

Distributions (the workloads the pages' method is run on: projected,
L2-normalised queries and keys, Gaussian values, per-token decay and noise
scalars):
  q, k   ~ N(0, 1), L2-normalised along d_k per (b, h, t)
  v      ~ N(0, 1)
  a      = sigmoid(N(a_mu, 1))         (a_mu = 2, or 4 for long memory)
  nu     = softplus(N(-3, 1))          process-noise variance
  r      = softplus(N(0, 1))           observation-noise variance
  lambda0: ones, or U(0.5, 2) per key dimension (diagonal) / per head (isotropic)
  S0     : zeros, or N(0, variance 0.1)
Draw order from numpy's PCG64 stream: q, k, v, a, nu, r, lambda0, S0 (all in
float64), then one rounding to the storage dtype (bf16 round-to-nearest-even
through torch, or float32).  lambda0 and S0 are float32 state.
"""
from __future__ import annotations

import math

import numpy as np

DIAGONAL = "diagonal"
ISOTROPIC = "isotropic"


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 draws once to the storage dtype; returns float32 holding them."""
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
        return t.to(torch.bfloat16).to(torch.float32).numpy()
    raise ValueError(dtype)


def _unit_rows(rng, shape) -> np.ndarray:
    x = rng.standard_normal(shape)
    x /= np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.logaddexp(0.0, x)


def forward_inputs(B, H, T, dk, dv, *, variant=DIAGONAL, dtype="f32", gate_dtype=None,
                   seed=0, a_mu=2.0, lambda0="uniform", S0="normal") -> dict:
    """Inputs of one KDN forward call as float32 numpy arrays (bf16-exact if dtype='bf16').

    Returns dict with q, k [B,H,T,dk]; v [B,H,T,dv]; a, nu, r [B,H,T];
    lambda0 [B,H,dk] (diagonal) or [B,H] (isotropic); S0 [B,H,dv,dk]; and the
    metadata keys 'variant', 'dtype', 'gate_dtype'.
    """
    gate_dtype = gate_dtype or dtype
    rng = np.random.default_rng(seed)
    out = {}
    out["q"] = _round(_unit_rows(rng, (B, H, T, dk)), dtype)
    out["k"] = _round(_unit_rows(rng, (B, H, T, dk)), dtype)
    out["v"] = _round(rng.standard_normal((B, H, T, dv)), dtype)
    out["a"] = _round(_sigmoid(rng.normal(a_mu, 1.0, (B, H, T))), gate_dtype)
    out["nu"] = _round(_softplus(rng.normal(-3.0, 1.0, (B, H, T))), gate_dtype)
    out["r"] = _round(_softplus(rng.normal(0.0, 1.0, (B, H, T))), gate_dtype)
    lam_shape = (B, H, dk) if variant == DIAGONAL else (B, H)
    if lambda0 == "ones":
        out["lambda0"] = np.ones(lam_shape, np.float32)
    else:
        out["lambda0"] = rng.uniform(0.5, 2.0, lam_shape).astype(np.float32)
    if S0 == "zeros":
        out["S0"] = np.zeros((B, H, dv, dk), np.float32)
    else:
        out["S0"] = rng.normal(0.0, math.sqrt(0.1), (B, H, dv, dk)).astype(np.float32)
    out["variant"] = variant
    out["dtype"] = dtype
    out["gate_dtype"] = gate_dtype
    return out


def backward_cotangents(B, H, T, dk, dv, *, variant=DIAGONAL, dtype="f32", seed=0,
                        state_cotangents=True) -> dict:
    """Cotangents of one backward call: dO [B,H,T,dv] ~ N(0, 1) in the input
    dtype; dS_T [B,H,dv,dk] ~ N(0, variance 0.1) and dlambda_T ([B,H,dk] or
    [B,H]) ~ N(0, variance 0.01) as float32, or None with
    state_cotangents=False.  Drawn from their own PCG64 stream (seed + 7919),
    so the forward inputs of the same seed are unchanged."""
    rng = np.random.default_rng(seed + 7919)
    out = {"dO": _round(rng.standard_normal((B, H, T, dv)), dtype)}
    lam_shape = (B, H, dk) if variant == DIAGONAL else (B, H)
    if state_cotangents:
        out["dS_T"] = rng.normal(0.0, math.sqrt(0.1), (B, H, dv, dk)).astype(np.float32)
        out["dlambda_T"] = rng.normal(0.0, 0.1, lam_shape).astype(np.float32)
    else:
        out["dS_T"] = None
        out["dlambda_T"] = None
    return out


def decode_inputs(N, H, dk, dv, steps, *, variant=DIAGONAL, seed=0, qkv_dtype="bf16",
                  gate_dtype="f32", a_mu=2.0) -> dict:
    """Cached state plus per-step inputs of `steps` decode steps.

    Returns S0 [N,H,dv,dk] ~ N(0, var 0.1) and lambda0 [N,H,dk] (or [N,H])
    ~ U(0.5, 2) as float32, then per step q, k [steps,N,H,dk], v
    [steps,N,H,dv] (qkv_dtype) and a, nu, r [steps,N,H] (gate_dtype), drawn
    step after step from one PCG64 stream.
    """
    rng = np.random.default_rng(seed)
    out = {}
    out["S0"] = rng.normal(0.0, math.sqrt(0.1), (N, H, dv, dk)).astype(np.float32)
    lam_shape = (N, H, dk) if variant == DIAGONAL else (N, H)
    out["lambda0"] = rng.uniform(0.5, 2.0, lam_shape).astype(np.float32)
    per = {n: [] for n in ("q", "k", "v", "a", "nu", "r")}
    for _ in range(steps):
        per["q"].append(_round(_unit_rows(rng, (N, H, dk)), qkv_dtype))
        per["k"].append(_round(_unit_rows(rng, (N, H, dk)), qkv_dtype))
        per["v"].append(_round(rng.standard_normal((N, H, dv)), qkv_dtype))
        per["a"].append(_round(_sigmoid(rng.normal(a_mu, 1.0, (N, H))), gate_dtype))
        per["nu"].append(_round(_softplus(rng.normal(-3.0, 1.0, (N, H))), gate_dtype))
        per["r"].append(_round(_softplus(rng.normal(0.0, 1.0, (N, H))), gate_dtype))
    for n, lst in per.items():
        out[n] = np.stack(lst) if lst else np.zeros((0, N, H, dk if n in "qk" else dv), np.float32)
    out["variant"] = variant
    out["qkv_dtype"] = qkv_dtype
    out["gate_dtype"] = gate_dtype
    return out


# The five workloads.  Index i uses seed 1000 + i.
CONFIGS = [
    dict(name="iso_f32_B1_H2_T256_d32", kind="forward", variant=ISOTROPIC, dtype="f32",
         B=1, H=2, T=256, dk=32, dv=32, chunk=32, a_mu=2.0, lambda0="ones", S0="zeros"),
    dict(name="diag_f32_B2_H4_T2048_d64", kind="forward", variant=DIAGONAL, dtype="f32",
         B=2, H=4, T=2048, dk=64, dv=64, chunk=64, a_mu=2.0, lambda0="uniform", S0="normal"),
    dict(name="diag_bf16_B8_H16_T4096_d128", kind="forward", variant=DIAGONAL, dtype="bf16",
         B=8, H=16, T=4096, dk=128, dv=128, chunk=64, a_mu=2.0, lambda0="uniform",
         S0="normal"),
    dict(name="long_bf16_B1_H16_T65536_d128", kind="forward", variant=DIAGONAL, dtype="bf16",
         B=1, H=16, T=65536, dk=128, dv=128, chunk=64, a_mu=4.0, lambda0="uniform",
         S0="normal"),
    dict(name="decode_diag_N256_H16_d128_x128", kind="decode", variant=DIAGONAL,
         N=256, H=16, dk=128, dv=128, steps=128, qkv_dtype="bf16", gate_dtype="f32",
         a_mu=2.0),
]


def config_inputs(index: int, variant: str | None = None, **overrides) -> dict:
    """Inputs of workload `index` (seed 1000 + index); `variant` overrides the
    default (workload 3 runs both variants).  Size overrides (B, H, T, N,
    steps) keep the seed and distributions; they exist so that tests can draw
    a smaller slice with the same recipe."""
    cfg = dict(CONFIGS[index])
    cfg.update(overrides)
    seed = 1000 + index
    if cfg["kind"] == "forward":
        return forward_inputs(cfg["B"], cfg["H"], cfg["T"], cfg["dk"], cfg["dv"],
                              variant=variant or cfg["variant"], dtype=cfg["dtype"],
                              seed=seed, a_mu=cfg["a_mu"], lambda0=cfg["lambda0"],
                              S0=cfg["S0"])
    return decode_inputs(cfg["N"], cfg["H"], cfg["dk"], cfg["dv"], cfg["steps"],
                         variant=variant or cfg["variant"], seed=seed,
                         qkv_dtype=cfg["qkv_dtype"], gate_dtype=cfg["gate_dtype"],
                         a_mu=cfg["a_mu"])


def layer_inputs(B, T, H, D, dk, dv, *, variant=DIAGONAL, dtype="f32", seed=0) -> dict:
    """Inputs and random weights of one KDN layer call, as float32 numpy arrays
    (bf16-exact if dtype='bf16').

    x [B,T,D] standard normal; W_in [D, H(2dk+dv)+3H] and W_out [H*dv, D] with
    entries N(0, 1/fan_in); b_gate [3H] float32 = (2, -3, 0) per gate, so that
    with unit-variance logits the gates follow the layer workload's recipe
    (decay logits N(2, 1), process-noise logits N(-3, 1), observation-noise
    logits N(0, 1)); lambda0 and S0 as in forward_inputs.
    """
    rng = np.random.default_rng(seed)
    n_in = H * (2 * dk + dv) + 3 * H
    out = {
        "x": _round(rng.standard_normal((B, T, D)), dtype),
        "W_in": _round(rng.standard_normal((D, n_in)) / math.sqrt(D), dtype),
        "W_out": _round(rng.standard_normal((H * dv, D)) / math.sqrt(H * dv), dtype),
        "b_gate": np.concatenate([np.full(H, 2.0), np.full(H, -3.0), np.zeros(H)]).astype(
            np.float32),
    }
    lam_shape = (B, H, dk) if variant == DIAGONAL else (B, H)
    out["lambda0"] = rng.uniform(0.5, 2.0, lam_shape).astype(np.float32)
    out["S0"] = rng.normal(0.0, math.sqrt(0.1), (B, H, dv, dk)).astype(np.float32)
    out.update(variant=variant, dtype=dtype, H=H, dk=dk, dv=dv)
    return out

