"""Pins of the oracle's backward (the vector-Jacobian product of the layer).

The pages print no gradient, so the backward is pinned against the forward
oracle by central finite differences, one input tensor at a time (a dropped
term, a wrong sign or a transposed operand in any one gradient moves that
tensor's directional derivative), and against a closed form: the derivative
of a Moebius map, which the uncertainty recurrence is ("Kalman Delta
Networks", English abstract).

Finite differences are taken along the perturbation the float32 inputs
actually received (x+ - x- computed in float64 after rounding), so the
comparison is limited only by the O(h^2) truncation of the central difference.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import textbook as tb
from kdn_inputs import backward_cotangents, forward_inputs

VARIANTS = ["diagonal", "isotropic"]
NAMES = ["q", "k", "v", "a", "nu", "r", "lambda0", "S0"]
GRAD = {"q": "dq", "k": "dk", "v": "dv", "a": "da", "nu": "dnu", "r": "dr",
        "lambda0": "dlambda0", "S0": "dS0"}


def _loss(x, cot):
    f = oracle.forward(x["q"], x["k"], x["v"], x["a"], x["nu"], x["r"], x["lambda0"],
                       x["S0"], variant=x["variant"])
    L = float(np.sum(f["o"] * cot["dO"]))
    if cot["dS_T"] is not None:
        L += float(np.sum(f["S_T"] * cot["dS_T"]))
        L += float(np.sum(f["lambda_T"] * cot["dlambda_T"]))
    return L


def _grads(x, cot):
    return oracle.backward(x["q"], x["k"], x["v"], x["a"], x["nu"], x["r"], cot["dO"],
                           x["lambda0"], x["S0"], cot["dS_T"], cot["dlambda_T"],
                           variant=x["variant"])


def _inputs(variant, B, H, T, dk, dv, seed):
    x = forward_inputs(B, H, T, dk, dv, variant=variant, seed=seed, a_mu=1.0)
    # keep the gates away from their domain edges so that +-h stays inside
    x["a"] = np.clip(x["a"], 0.2, 0.95).astype(np.float32)
    x["nu"] = (x["nu"] + 0.05).astype(np.float32)
    return x


def _directional_check(x, cot, g, name, rng, h=1e-3):
    base = x[name]
    d = rng.standard_normal(base.shape)
    if name in ("a", "nu", "r", "lambda0"):
        d = d * base  # relative steps keep positive inputs positive
    xp, xm = dict(x), dict(x)
    xp[name] = (base + h * d).astype(np.float32)
    xm[name] = (base - h * d).astype(np.float32)
    delta = xp[name].astype(np.float64) - xm[name].astype(np.float64)
    fd = _loss(xp, cot) - _loss(xm, cot)
    pred = float(np.sum(g[GRAD[name]] * delta))
    scale = float(np.sum(np.abs(g[GRAD[name]] * delta)))
    assert abs(fd - pred) <= 1e-5 * scale + 1e-12, (name, fd, pred, scale)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("shape", [(1, 2, 13, 5, 4), (2, 1, 7, 3, 6)])
def test_gradient_matches_finite_differences(variant, shape):
    B, H, T, dk, dv = shape
    x = _inputs(variant, B, H, T, dk, dv, seed=11 + T)
    cot = backward_cotangents(B, H, T, dk, dv, variant=variant, seed=5 + T)
    g = _grads(x, cot)
    rng = np.random.default_rng(3)
    for name in NAMES:
        _directional_check(x, cot, g, name, rng)


@pytest.mark.parametrize("variant", VARIANTS)
def test_gradient_of_read_out_only(variant):
    """No cotangent on the final state: only the read-outs drive the gradient."""
    x = _inputs(variant, 1, 1, 9, 4, 3, seed=2)
    cot = backward_cotangents(1, 1, 9, 4, 3, variant=variant, seed=4, state_cotangents=False)
    g = _grads(x, cot)
    rng = np.random.default_rng(8)
    for name in NAMES:
        _directional_check(x, cot, g, name, rng)


@pytest.mark.parametrize("variant", VARIANTS)
def test_single_coordinates_match_finite_differences(variant):
    """Every coordinate of every gradient, on a tiny head (brute force)."""
    x = _inputs(variant, 1, 1, 4, 2, 2, seed=21)
    cot = backward_cotangents(1, 1, 4, 2, 2, variant=variant, seed=22)
    g = _grads(x, cot)
    h = 1e-3
    for name in NAMES:
        base = x[name]
        for idx in np.ndindex(base.shape):
            xp, xm = dict(x), dict(x)
            xp[name] = base.copy()
            xm[name] = base.copy()
            step = h * max(abs(float(base[idx])), 0.1)
            xp[name][idx] = np.float32(base[idx] + step)
            xm[name][idx] = np.float32(base[idx] - step)
            delta = float(xp[name][idx]) - float(xm[name][idx])
            fd = (_loss(xp, cot) - _loss(xm, cot)) / delta
            ref = float(g[GRAD[name]][idx])
            assert abs(fd - ref) <= 1e-5 * (abs(ref) + 1.0), (name, idx, fd, ref)


def test_precision_gradient_is_moebius_derivative():
    """With only dlambda_T non-zero, dlambda0_i = dlambda_T_i * det(Pi) /
    (Pi21 lambda0 + Pi22)^2 for the composed token maps Pi of key dim i, and
    det(Pi) = prod_t a_t^2 (each token map has determinant a^2)."""
    B, H, T, dk, dv = 1, 1, 40, 3, 2
    x = _inputs("diagonal", B, H, T, dk, dv, seed=31)
    cot = {"dO": np.zeros((B, H, T, dv), np.float32),
           "dS_T": np.zeros((B, H, dv, dk), np.float32),
           "dlambda_T": np.ones((B, H, dk), np.float32)}
    g = _grads(x, cot)
    a, nu, r = (x[n][0, 0].astype(np.float64) for n in ("a", "nu", "r"))
    k = x["k"][0, 0].astype(np.float64)
    for i in range(dk):
        Pi = np.eye(2)
        for t in range(T):
            Pi = tb.mobius_step(a[t], nu[t], k[t, i] ** 2 / r[t]) @ Pi
        lam0 = float(x["lambda0"][0, 0, i])
        # det(Pi) from the product of the token determinants (the 2x2 formula
        # cancels catastrophically on a long product; it is checked on three maps)
        ref = np.prod(a * a) / (Pi[1, 0] * lam0 + Pi[1, 1]) ** 2
        np.testing.assert_allclose(g["dlambda0"][0, 0, i], ref, rtol=1e-10)
        P3 = np.eye(2)
        for t in range(3):
            P3 = tb.mobius_step(a[t], nu[t], k[t, i] ** 2 / r[t]) @ P3
        np.testing.assert_allclose(np.linalg.det(P3), np.prod(a[:3] ** 2), rtol=1e-10)
    # and nothing of the mean enters: the other gradients are driven only by
    # the precision path (dq and dv must vanish)
    assert np.all(g["dq"] == 0.0) and np.all(g["dv"] == 0.0) and np.all(g["dS0"] == 0.0)


def test_gated_delta_special_case_gradient_wrt_values():
    """dv is the adjoint of the linear map v -> o, so <dO, o(v)> with S0 = 0
    equals <dv, v>: the read-out is linear in the values."""
    x = _inputs("diagonal", 1, 2, 11, 4, 3, seed=41)
    x["S0"] = np.zeros_like(x["S0"])
    cot = backward_cotangents(1, 2, 11, 4, 3, seed=42, state_cotangents=False)
    g = _grads(x, cot)
    L = _loss(x, cot)
    np.testing.assert_allclose(np.sum(g["dv"] * x["v"].astype(np.float64)), L, rtol=1e-12)
    # and, with values and S0 both scaled, dS0 pairs with S0 the same way
    x2 = _inputs("diagonal", 1, 2, 11, 4, 3, seed=43)
    g2 = _grads(x2, cot)
    L2 = _loss(x2, cot)
    lin = np.sum(g2["dv"] * x2["v"]) + np.sum(g2["dS0"] * x2["S0"])
    np.testing.assert_allclose(lin, L2, rtol=1e-12)
