"""GPU parity of the forward in the method's limiting and degenerate cases,
through the C ABI.  Each case stresses its own part of the kernels and is
checked both against the fp64 oracle and against what the mathematics fixes
independently of it:

* no decay and no process noise (a = 1, nu = 0) over 65,536 tokens: the
  precision is then lambda0 plus the summed evidence, lambda_T = lambda0 +
  sum_t b_t, with no forgetting (the Moebius products grow without bound and
  only their renormalisation keeps them finite);
* an observation noise of 1e30: the gain vanishes, so the memory only decays,
  S_T = (prod_t a_t) S0 and o_t = (prod_{s<=t} a_s) S0 q_t, and the precision
  follows the prediction step alone;
* decays of 1e-6 on every 7th token, inside the chunks: the chunk-local
  cumulative decay then underflows in single precision;
* the isotropic variant at the fixed point of its precision recursion, with
  constant gates and unit keys: the gain is then a constant multiple beta of
  the key, and the layer is the gated delta rule with that beta ("Kalman Delta
  Networks", English abstract: Delta-style updates are the special case of a
  token-wise isotropic surrogate);
* linearity of (o, S_T) in (v, S0) at fixed keys, gates and lambda0.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kalman_filter_memory_amd as kdn
import oracle
import textbook as tb
from gpu_util import (TOL_BF16, TOL_F32, TOL_LAMBDA, elementwise, forward_tensors, host,
                      normwise, say)
from kdn_inputs import forward_inputs

pytestmark = pytest.mark.gpu


def _tol(dtype):
    return TOL_BF16 if dtype == "bf16" else TOL_F32


def _run(inp, chunk):
    t = forward_tensors(inp)
    o, S_T, lam = kdn.forward(t["q"], t["k"], t["v"], t["a"], t["nu"], t["r"], t["lambda0"],
                              t["S0"], variant=inp["variant"], chunk=chunk)
    torch.cuda.synchronize()
    return host(o), host(S_T), host(lam)


def _oracle(inp):
    return oracle.forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["nu"], inp["r"],
                          inp["lambda0"], inp["S0"], inp["variant"])


def _evidence(inp):
    """b_t per token: k_i^2 / r (diagonal, per key dim) or |k|^2 / (d_k r)."""
    k = inp["k"].astype(np.float64)
    r = inp["r"].astype(np.float64)[..., None]
    if inp["variant"] == "diagonal":
        return k * k / r
    return (k * k).sum(-1) / (k.shape[-1] * r[..., 0])


def _set(inp, name, value):
    """Set a gate tensor to a constant, rounded to the storage dtype."""
    x = np.full_like(inp[name], value, dtype=np.float32)
    if inp["gate_dtype"] == "bf16":
        x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    inp[name] = x


@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_no_decay_no_process_noise_over_65536_tokens(variant):
    B, H, T, d = 1, 2, 65536, 128
    inp = forward_inputs(B, H, T, d, d, variant=variant, dtype="bf16", seed=501)
    _set(inp, "a", 1.0)
    _set(inp, "nu", 0.0)
    say(f"[gpu] a = 1, nu = 0, T = {T}, {variant}")
    o, S_T, lam = _run(inp, 64)
    lam_closed = inp["lambda0"].astype(np.float64) + _evidence(inp).sum(axis=2)
    ref = _oracle(inp)
    e_closed = elementwise(lam, lam_closed)
    e_o, e_s = normwise(o, ref["o"]), normwise(S_T, ref["S_T"])
    e_l = elementwise(lam, ref["lambda_T"])
    say(f"    lambda_T vs lambda0 + sum b: {e_closed:.2e}; vs oracle {e_l:.2e};  "
        f"o {e_o:.2e}  S_T {e_s:.2e}")
    assert np.all(np.isfinite(o))
    assert e_closed <= TOL_LAMBDA and e_l <= TOL_LAMBDA
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16


@pytest.mark.parametrize("variant,dtype", [("diagonal", "f32"), ("isotropic", "f32"),
                                           ("diagonal", "bf16"), ("isotropic", "bf16")])
def test_huge_observation_noise_leaves_only_decay(variant, dtype):
    B, H, T, dk, dv = 1, 3, 200, 64, 32
    inp = forward_inputs(B, H, T, dk, dv, variant=variant, dtype=dtype, seed=502)
    _set(inp, "r", 1e30)
    say(f"[gpu] r = 1e30, {variant} {dtype}")
    o, S_T, lam = _run(inp, 64)
    a = inp["a"].astype(np.float64)
    gam = np.cumprod(a, axis=2)                                   # [B,H,T]
    S0 = inp["S0"].astype(np.float64)
    o_closed = gam[..., None] * np.einsum("bhvk,bhtk->bhtv", S0, inp["q"].astype(np.float64))
    S_closed = gam[..., -1, None, None] * S0
    lam_pred = inp["lambda0"].astype(np.float64).copy()
    nu = inp["nu"].astype(np.float64)
    for t in range(T):
        at, nt = a[:, :, t], nu[:, :, t]
        if variant == "diagonal":
            at, nt = at[..., None], nt[..., None]
        lam_pred = lam_pred / (at * at + nt * lam_pred)
    ref = _oracle(inp)
    tol = _tol(dtype)
    e_oc, e_sc = normwise(o, o_closed), normwise(S_T, S_closed)
    e_lc = elementwise(lam, lam_pred)
    say(f"    vs closed form: o {e_oc:.2e}  S_T {e_sc:.2e}  lambda_T {e_lc:.2e}; vs oracle: o "
        f"{normwise(o, ref['o']):.2e}")
    assert e_oc <= tol and e_sc <= tol and e_lc <= TOL_LAMBDA
    assert normwise(o, ref["o"]) <= tol and normwise(S_T, ref["S_T"]) <= tol


@pytest.mark.parametrize("variant,dtype,dk,chunk", [("diagonal", "f32", 64, 64),
                                                    ("isotropic", "f32", 128, 32),
                                                    ("diagonal", "bf16", 128, 64),
                                                    ("isotropic", "bf16", 64, 64),
                                                    ("diagonal", "f32", 32, 16)])
def test_tiny_decays_inside_chunks(variant, dtype, dk, chunk):
    B, H, T, dv = 1, 3, 300, 64
    inp = forward_inputs(B, H, T, dk, dv, variant=variant, dtype=dtype, seed=503)
    a = inp["a"].copy()
    a[..., ::7] = 1e-6
    if inp["gate_dtype"] == "bf16":
        a = torch.from_numpy(a).to(torch.bfloat16).float().numpy()
    inp["a"] = a
    say(f"[gpu] a = 1e-6 on every 7th token, {variant} {dtype} d_k {dk} C {chunk}")
    o, S_T, lam = _run(inp, chunk)
    ref = _oracle(inp)
    e_o, e_s = normwise(o, ref["o"]), normwise(S_T, ref["S_T"])
    e_l = elementwise(lam, ref["lambda_T"])
    say(f"    err o {e_o:.2e}  S_T {e_s:.2e}  lambda_T {e_l:.2e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S_T))
    tol = _tol(dtype)
    assert e_o <= tol and e_s <= tol and e_l <= TOL_LAMBDA


@pytest.mark.parametrize("dtype,keys", [("f32", "unit"), ("bf16", "one-hot")])
def test_isotropic_fixed_point_is_the_gated_delta_rule(dtype, keys):
    """Constant a, nu, r and unit keys: b = 1 / (d_k r) is constant, lambda0 =
    lambda* stays put, and w = beta k with beta = 1 / (1 + r lambda*^-)."""
    B, H, T, dk, dv = 1, 2, 257, 64, 64
    a_c, nu_c, r_c = 0.9375, 0.0625, 0.5          # exact in bfloat16
    inp = forward_inputs(B, H, T, dk, dv, variant="isotropic", dtype=dtype, seed=504)
    if keys == "one-hot":
        rng = np.random.default_rng(505)
        k = np.zeros_like(inp["k"])
        idx = rng.integers(0, dk, (B, H, T))
        np.put_along_axis(k, idx[..., None], 1.0, axis=-1)
        inp["k"] = k
    _set(inp, "a", a_c)
    _set(inp, "nu", nu_c)
    _set(inp, "r", r_c)
    b = 1.0 / (dk * r_c)
    c = 1.0 + b * nu_c - a_c * a_c
    lam_star = (c + np.sqrt(c * c + 4.0 * nu_c * b * a_c * a_c)) / (2.0 * nu_c)
    inp["lambda0"] = np.full((B, H), lam_star, np.float32)
    lam_pred = lam_star / (a_c * a_c + nu_c * lam_star)
    say(f"[gpu] isotropic fixed point lambda* = {lam_star:.6f}, {dtype}, {keys} keys")
    o, S_T, lam = _run(inp, 64)
    kk = (inp["k"].astype(np.float64) ** 2).sum(-1)             # 1 up to rounding
    worst_o = worst_s = 0.0
    for h in range(H):
        beta = 1.0 / (kk[0, h] + r_c * lam_pred)
        o_ref, S_ref = tb.gated_delta(inp["q"][0, h], inp["k"][0, h], inp["v"][0, h],
                                      inp["a"][0, h], beta, inp["S0"][0, h])
        worst_o = max(worst_o, normwise(o[0:1, h:h + 1], o_ref[None, None]))
        worst_s = max(worst_s, normwise(S_T[0:1, h:h + 1], S_ref[None, None]))
    e_l = float(np.abs(lam / lam_star - 1.0).max())
    say(f"    vs gated delta rule: o {worst_o:.2e}  S_T {worst_s:.2e};  lambda_T vs lambda* "
        f"{e_l:.2e}")
    tol = _tol(dtype)
    assert worst_o <= tol and worst_s <= tol and e_l <= TOL_LAMBDA


@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_linear_in_values_and_initial_state(variant):
    B, H, T, dk, dv = 2, 2, 190, 64, 64
    x1 = forward_inputs(B, H, T, dk, dv, variant=variant, dtype="f32", seed=506)
    x2 = forward_inputs(B, H, T, dk, dv, variant=variant, dtype="f32", seed=507)
    al, be = 0.75, -1.5
    x3 = dict(x1)
    x3["v"] = (al * x1["v"].astype(np.float64) + be * x2["v"]).astype(np.float32)
    x3["S0"] = (al * x1["S0"].astype(np.float64) + be * x2["S0"]).astype(np.float32)
    x2 = dict(x1, v=x2["v"], S0=x2["S0"])
    say(f"[gpu] linearity in (v, S0), {variant}")
    o1, S1, _ = _run(x1, 64)
    o2, S2, _ = _run(x2, 64)
    o3, S3, _ = _run(x3, 64)
    e_o = normwise(o3, al * o1 + be * o2)
    e_s = normwise(S3, al * S1 + be * S2)
    ref = _oracle(x3)
    say(f"    o(a x1 + b x2) vs a o1 + b o2: {e_o:.2e}  S_T {e_s:.2e}; o3 vs oracle "
        f"{normwise(o3, ref['o']):.2e}")
    assert e_o <= 1e-5 and e_s <= 1e-5
    assert normwise(o3, ref["o"]) <= TOL_F32
