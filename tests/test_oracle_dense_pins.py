"""Pins of the oracle's exact (dense Riccati) KDN against what the pages and the
mathematics fix.  The exact filter is the one the two approximations replace
("Kalman Delta Networks", English abstract), so:

* it equals the textbook full-covariance Kalman filter (tests/textbook.py,
  Joseph-form covariance update: a different formulation of the same update);
* with axis-aligned keys the exact posterior stays diagonal and the diagonal
  variant is exact;
* with d_k = 1 it is the scalar Kalman filter;
* it is equivariant under a rotation of the key space (k, q -> R k, R q with
  S0 -> S0 R^T, P0 -> R P0 R^T), which the diagonal approximation is not.
A slip in the predict, gain or update step breaks at least one of these.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import textbook as tb
from kdn_inputs import forward_inputs


def _head(x):
    return x[None, None]


def _rand(seed, T, dk, dv):
    x = forward_inputs(1, 1, T, dk, dv, seed=seed, a_mu=1.0)
    out = {n: x[n][0, 0] for n in ("q", "k", "v", "a", "nu", "r", "lambda0", "S0")}
    # prior precisions that are powers of two, so that the prior covariance
    # diag(1 / lambda0) is exact in float32 and both filters start equal
    rng = np.random.default_rng(seed + 1)
    out["lambda0"] = (2.0 ** rng.integers(-1, 2, dk)).astype(np.float32)
    return out


def _dense(x, P0=None):
    return oracle.forward_dense(_head(x["q"]), _head(x["k"]), _head(x["v"]), _head(x["a"]),
                                _head(x["nu"]), _head(x["r"]),
                                None if P0 is None else _head(P0), _head(x["S0"]), debug=True)


def test_dense_equals_textbook_full_covariance_filter():
    x = _rand(5, 60, 7, 5)
    P0 = np.diag(1.0 / x["lambda0"]).astype(np.float32)
    out = _dense(x, P0)
    o, M, Sig, prior, gains = tb.dense_kalman(x["q"], x["k"], x["v"], x["a"], x["nu"], x["r"],
                                              x["lambda0"], x["S0"])
    # the two covariance updates (plain and Joseph form) are equal algebraically
    # and differ only in fp64 rounding
    sc = np.abs(o).max()
    np.testing.assert_allclose(out["o"][0, 0], o, rtol=0, atol=1e-11 * sc)
    np.testing.assert_allclose(out["S_T"][0, 0], M, rtol=0, atol=1e-11 * np.abs(M).max())
    np.testing.assert_allclose(out["P_T"][0, 0], Sig, rtol=0, atol=1e-11 * np.abs(Sig).max())
    np.testing.assert_allclose(out["w"][0, 0], gains, rtol=0, atol=1e-11 * np.abs(gains).max())


def test_dense_equals_diagonal_on_axis_aligned_keys():
    rng = np.random.default_rng(3)
    T, dk, dv = 40, 5, 3
    x = _rand(6, T, dk, dv)
    k = np.zeros((T, dk), np.float32)
    k[np.arange(T), rng.integers(0, dk, T)] = rng.uniform(0.5, 1.5, T).astype(np.float32)
    x["k"] = k
    P0 = np.diag(1.0 / x["lambda0"]).astype(np.float32)
    dense = _dense(x, P0)
    diag = oracle.forward(_head(x["q"]), _head(k), _head(x["v"]), _head(x["a"]),
                          _head(x["nu"]), _head(x["r"]), _head(x["lambda0"]), _head(x["S0"]),
                          "diagonal")
    np.testing.assert_allclose(dense["o"], diag["o"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dense["S_T"], diag["S_T"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(np.diagonal(dense["P_T"][0, 0]), 1.0 / diag["lambda_T"][0, 0],
                               rtol=1e-11)
    P = dense["P_T"][0, 0]
    assert np.abs(P - np.diag(np.diag(P))).max() < 1e-14


def test_dense_with_one_key_dimension_is_the_scalar_filter():
    x = _rand(7, 50, 1, 4)
    out = _dense(x)
    o, m, lam_T, lm, w = tb.scalar_kalman(x["q"][:, 0], x["k"][:, 0], x["v"], x["a"], x["nu"],
                                          x["r"], 1.0, x["S0"][:, 0])
    np.testing.assert_allclose(out["o"][0, 0], o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(out["P_T"][0, 0, 0, 0], 1.0 / lam_T, rtol=1e-11)


def test_dense_is_rotation_equivariant():
    x = _rand(8, 45, 6, 4)
    rng = np.random.default_rng(9)
    R, _ = np.linalg.qr(rng.standard_normal((6, 6)))
    P0 = np.diag(1.0 / x["lambda0"])
    # inputs are float32: rotate in float64 and compare the rotated run with the
    # float32-rounded rotated inputs it actually received
    y = dict(x)
    y["k"] = (x["k"].astype(np.float64) @ R.T).astype(np.float32)
    y["q"] = (x["q"].astype(np.float64) @ R.T).astype(np.float32)
    y["S0"] = (x["S0"].astype(np.float64) @ R.T).astype(np.float32)
    P0r = (R @ P0 @ R.T).astype(np.float32)
    a = _dense(x, P0.astype(np.float32))
    b = _dense(y, P0r)
    # the rotated run matches the original up to the float32 rounding of the
    # rotated inputs (relative 6e-8 per entry)
    np.testing.assert_allclose(b["o"], a["o"], rtol=0, atol=2e-5 * np.abs(a["o"]).max())
    np.testing.assert_allclose(b["P_T"][0, 0], R @ a["P_T"][0, 0] @ R.T,
                               atol=2e-5 * np.abs(a["P_T"]).max())
    # the diagonal approximation is not equivariant: the same rotation changes o
    d1 = oracle.forward(*(_head(x[n]) for n in ("q", "k", "v", "a", "nu", "r", "lambda0", "S0")),
                        "diagonal")
    d2 = oracle.forward(*(_head(y[n]) for n in ("q", "k", "v", "a", "nu", "r", "lambda0", "S0")),
                        "diagonal")
    assert np.abs(d1["o"] - d2["o"]).max() > 1e-3 * np.abs(d1["o"]).max()


def test_approximation_gap_of_diagonal_and_isotropic():
    """The gap study: o of the two approximations against the exact filter on
    the layer's input distribution (L2-normalised random keys), relative to
    max|o_exact|; both gaps are positive, and the exact filter's P stays
    symmetric positive definite."""
    x = forward_inputs(2, 4, 256, 32, 32, seed=17)
    iso = forward_inputs(2, 4, 256, 32, 32, variant="isotropic", seed=17)
    B, H, dk = 2, 4, 32
    P0 = np.zeros((B, H, dk, dk), np.float32)
    for b in range(B):
        for h in range(H):
            P0[b, h] = np.diag(1.0 / x["lambda0"][b, h])
    args = [x[n] for n in ("q", "k", "v", "a", "nu", "r")]
    dense = oracle.forward_dense(*args, P0, x["S0"])
    diag = oracle.forward(*args, x["lambda0"], x["S0"], "diagonal")
    # isotropic with the mean precision of each head's diagonal prior
    lam_iso = x["lambda0"].mean(axis=-1).astype(np.float32)
    isot = oracle.forward(*args, lam_iso, x["S0"], "isotropic")
    scale = np.abs(dense["o"]).max()
    gap_diag = np.abs(diag["o"] - dense["o"]).max() / scale
    gap_iso = np.abs(isot["o"] - dense["o"]).max() / scale
    print(f"approximation gap (max |o - o_exact| / max |o_exact|): diagonal {gap_diag:.3e}, "
          f"isotropic {gap_iso:.3e}")
    assert gap_diag > 0 and gap_iso > 0
    P = dense["P_T"]
    assert np.allclose(P, np.swapaxes(P, -1, -2), atol=1e-12)
    assert np.all(np.linalg.eigvalsh(P) > 0)
    _ = iso
