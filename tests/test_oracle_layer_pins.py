"""Pins of the layer oracle (oracle.layer: projections, per-head L2
normalisation, gate activations, output projection around the recurrence)
against what fixes them independently of its code:

* with W_in = I and W_out = [I 0] the layer is the recurrence on columns of x
  taken apart here by explicit loops, with scipy's logistic function and
  numpy's logaddexp as the gate activations (the layout and wiring);
* scaling one head's query or key columns by any positive factor leaves y
  unchanged (the normalisation is per head and per vector);
* with S0 = 0, y is linear in the value columns;
* relabelling the heads consistently (columns, gate biases, output rows,
  lambda0, S0) leaves y unchanged.
"""
from __future__ import annotations

import numpy as np
import pytest
from scipy.special import expit

import oracle
from oracle.layer import layer_forward
from kdn_inputs import layer_inputs


def _run(p, **kw):
    args = dict(lambda0=p["lambda0"], S0=p["S0"], variant=p["variant"])
    args.update(kw)
    return layer_forward(p["x"], p["W_in"], p["b_gate"], p["W_out"], p["H"], p["dk"], p["dv"],
                         **args)


@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_identity_weights_expose_the_wiring(variant):
    B, T, H, dk, dv = 2, 9, 3, 4, 2
    n_in = H * (2 * dk + dv) + 3 * H
    rng = np.random.default_rng(5)
    x = rng.standard_normal((B, T, n_in)).astype(np.float32)
    b_gate = rng.standard_normal(3 * H).astype(np.float32)
    W_in = np.eye(n_in, dtype=np.float32)
    W_out = np.zeros((H * dv, n_in), np.float32)
    W_out[:, :H * dv] = np.eye(H * dv)
    lam_shape = (B, H, dk) if variant == "diagonal" else (B, H)
    lam0 = rng.uniform(0.5, 2.0, lam_shape).astype(np.float32)
    S0 = rng.standard_normal((B, H, dv, dk)).astype(np.float32) * 0.3
    got = layer_forward(x, W_in, b_gate, W_out, H, dk, dv, lam0, S0, variant)
    q = np.zeros((B, H, T, dk))
    k = np.zeros((B, H, T, dk))
    v = np.zeros((B, H, T, dv))
    a, nu, r = (np.zeros((B, H, T)) for _ in range(3))
    g0 = H * (2 * dk + dv)
    for b in range(B):
        for t in range(T):
            for h in range(H):
                qv = x[b, t, h * dk:(h + 1) * dk].astype(np.float64)
                kv = x[b, t, H * dk + h * dk:H * dk + (h + 1) * dk].astype(np.float64)
                q[b, h, t] = qv / np.linalg.norm(qv)
                k[b, h, t] = kv / np.linalg.norm(kv)
                v[b, h, t] = x[b, t, 2 * H * dk + h * dv:2 * H * dk + (h + 1) * dv]
                a[b, h, t] = expit(float(x[b, t, g0 + h]) + float(b_gate[h]))
                nu[b, h, t] = np.logaddexp(0.0, float(x[b, t, g0 + H + h]) + float(b_gate[H + h]))
                r[b, h, t] = np.logaddexp(0.0, float(x[b, t, g0 + 2 * H + h])
                                          + float(b_gate[2 * H + h]))
    core = oracle.forward(q, k, v, a, nu, r, lam0, S0, variant)
    want = np.zeros((B, T, n_in))
    for b in range(B):
        for t in range(T):
            for h in range(H):
                want[b, t, h * dv:(h + 1) * dv] = core["o"][b, h, t]
    np.testing.assert_allclose(got["y"], want, rtol=0, atol=1e-6)
    np.testing.assert_allclose(got["S_T"], core["S_T"], rtol=0, atol=1e-6)
    np.testing.assert_allclose(got["lambda_T"], core["lambda_T"], rtol=1e-6)


def test_query_and_key_scale_per_head_leaves_y_unchanged():
    p = layer_inputs(2, 40, 3, 32, 8, 4, seed=6)
    H, dk = p["H"], p["dk"]
    base = _run(p)["y"]
    W = p["W_in"].astype(np.float64).copy()
    for h, c in enumerate((0.25, 3.0, 17.0)):
        W[:, h * dk:(h + 1) * dk] *= c               # q of head h
        W[:, H * dk + h * dk:H * dk + (h + 1) * dk] *= 1.0 / c + h  # k of head h
    got = _run(dict(p, W_in=W))["y"]
    np.testing.assert_allclose(got, base, rtol=0, atol=2e-6 * np.abs(base).max())


def test_y_is_linear_in_the_values_from_zero_state():
    p = layer_inputs(1, 30, 2, 32, 8, 8, seed=7)
    H, dk, dv = p["H"], p["dk"], p["dv"]
    S0 = np.zeros_like(p["S0"])
    base = _run(p, S0=S0)["y"]
    W = p["W_in"].astype(np.float64).copy()
    W[:, 2 * H * dk:2 * H * dk + H * dv] *= 2.5
    got = _run(dict(p, W_in=W), S0=S0)["y"]
    np.testing.assert_allclose(got, 2.5 * base, rtol=0, atol=2e-6 * np.abs(base).max())


@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_relabelling_heads_leaves_y_unchanged(variant):
    p = layer_inputs(2, 25, 3, 32, 8, 4, seed=8, variant=variant)
    H, dk, dv = p["H"], p["dk"], p["dv"]
    perm = np.array([2, 0, 1])
    W = p["W_in"]
    cols = []
    for lo, d in ((0, dk), (H * dk, dk), (2 * H * dk, dv)):
        cols += [np.arange(lo + h * d, lo + (h + 1) * d) for h in perm]
    g0 = H * (2 * dk + dv)
    cols += [g0 + g * H + perm for g in range(3)]
    W_p = W[:, np.concatenate(cols)]
    b_p = np.concatenate([p["b_gate"][g * H + perm] for g in range(3)])
    Wo_p = p["W_out"][np.concatenate([np.arange(h * dv, (h + 1) * dv) for h in perm])]
    q = dict(p, W_in=W_p, b_gate=b_p, W_out=Wo_p, lambda0=p["lambda0"][:, perm],
             S0=p["S0"][:, perm])
    a, b = _run(p), _run(q)
    np.testing.assert_allclose(b["y"], a["y"], rtol=0, atol=1e-9 * np.abs(a["y"]).max())
    np.testing.assert_allclose(b["S_T"], a["S_T"][:, perm], rtol=0, atol=1e-12)
