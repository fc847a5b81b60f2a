"""Helpers of the GPU parity tests: device transfer of the seeded inputs and the
error metrics.

Error metrics: for o and S_T the normwise relative error of each (b, h) slice,
max|x - ref| / max|ref|, worst over slices (an elementwise ratio is
ill-posed near zeros of o); for lambda the elementwise relative error
(lambda > 0)."""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL_F32 = 1e-4    # o, S_T with float32 inputs
TOL_BF16 = 2e-2   # o, S_T with bfloat16 inputs and float32 state
TOL_LAMBDA = 1e-5


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def tdtype(name: str):
    return torch.bfloat16 if name == "bf16" else torch.float32


def to_dev(x: np.ndarray, dtype, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device=device,
                                                                          dtype=dtype)


def forward_tensors(inp: dict, device="cuda") -> dict:
    qd = tdtype(inp["dtype"])
    gd = tdtype(inp["gate_dtype"])
    out = {n: to_dev(inp[n], qd, device) for n in ("q", "k", "v")}
    out.update({n: to_dev(inp[n], gd, device) for n in ("a", "nu", "r")})
    out["lambda0"] = to_dev(inp["lambda0"], torch.float32, device)
    out["S0"] = to_dev(inp["S0"], torch.float32, device)
    return out


def host(x: torch.Tensor) -> np.ndarray:
    return x.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def normwise(x: np.ndarray, ref: np.ndarray, lead: int = 2) -> float:
    """worst over the leading `lead` axes of max|x-ref| / max|ref|"""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    sh = ref.shape[:lead] + (-1,)
    num = np.abs(x - ref).reshape(sh).max(axis=-1)
    den = np.abs(ref).reshape(sh).max(axis=-1)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max())


def elementwise(x: np.ndarray, ref: np.ndarray) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    return float((np.abs(x - ref) / np.abs(ref)).max())


def head_slice(inp: dict, heads):
    """The inputs of a list of (b, h) heads, stacked as B=len(heads), H=1."""
    out = {}
    for n in ("q", "k", "v", "a", "nu", "r", "lambda0", "S0"):
        out[n] = np.stack([inp[n][b, h] for b, h in heads])[:, None]
    for n in ("variant", "dtype", "gate_dtype"):
        out[n] = inp[n]
    return out


_CONFIG_CACHE: dict = {}


def cached_config(index: int, variant: str | None = None) -> dict:
    """config_inputs(index, variant), drawn once per test process (the full-size
    workloads take 10-20 s to draw and round)."""
    from kdn_inputs import config_inputs

    key = (index, variant)
    if key not in _CONFIG_CACHE:
        _CONFIG_CACHE[key] = config_inputs(index, variant=variant)
    return _CONFIG_CACHE[key]


def row_errors(x: np.ndarray, ref: np.ndarray, floor: float = 1e-2):
    """Per-row diagnostic beside the per-head metric: over the last axis (a
    token row of o, or a row of S), max|x - ref| / max|ref| of that row, for
    the rows whose own max|ref| is at least `floor` times the max of their
    head.  Returns (worst such row error, its flat row index, fraction of rows
    above 1e-2)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0, -1, 0.0
    rows = ref.reshape(ref.shape[0], ref.shape[1], -1, ref.shape[-1])
    xr = x.reshape(rows.shape)
    rmax = np.abs(rows).max(axis=-1)
    hmax = rmax.max(axis=-1, keepdims=True)
    keep = rmax >= floor * np.where(hmax > 0, hmax, 1.0)
    err = np.abs(xr - rows).max(axis=-1) / np.where(rmax > 0, rmax, 1.0)
    err = np.where(keep, err, 0.0)
    i = int(err.argmax())
    return float(err.reshape(-1)[i]), i, float((err > 1e-2).mean())
