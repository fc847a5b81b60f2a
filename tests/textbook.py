"""Independent textbook references used to pin the oracle (numpy, float64).

None of these shares code with the oracle or with the GPU library.  Each is a
different formulation of something the KDN pages fix:

* ``scalar_kalman``: the textbook scalar Kalman filter in covariance form
  (predict variance a^2 P + nu, gain P k / (k^2 P + r), posterior variance
  (1 - K k) P).  With one key dimension the mean-field projection is exact, so
  both KDN variants must reduce to it ("Kalman Delta Networks", English
  abstract: for the linear-Gaussian memory model no recursive estimator
  beats the Kalman filter).
* ``dense_kalman``: the full-covariance Kalman filter (covariance form, Joseph
  update) that the pages call the exact, dense Riccati recursion.  With
  axis-aligned keys the exact posterior precision stays diagonal, so Diagonal
  KDN must equal it.
* ``gated_delta``: the gated delta rule S_t = a S_{t-1}(I - beta k k^T) +
  beta v k^T, which the pages present as the fixed-gain special case.
* ``chunk_forward``: the chunkwise (block) re-association of the state
  recurrence used by the GPU kernels, written from the block algebra of the
  recurrence S_t = a_t S_{t-1} + (v_t - a_t S_{t-1} k_t) w_t^T.
* Moebius helpers: 2x2 matrices acting by x -> (m11 x + m12) / (m21 x + m22),
  the structure the pages give for the uncertainty recurrence.
* ``gaussian_kl``: KL divergence between zero-mean Gaussians from its
  definition, for the mean-field projection pin.
"""
from __future__ import annotations

import numpy as np


def scalar_kalman(q, k, v, a, nu, r, lam0, s0):
    """One head with d_k = 1.  q, k: [T]; v: [T, dv]; a, nu, r: [T]; lam0: scalar
    precision; s0: [dv].  Returns o [T, dv], m_T [dv], precision_T, and per-token
    predictive precision and gain."""
    q, k, v, a, nu, r = (np.asarray(x, np.float64) for x in (q, k, v, a, nu, r))
    T, dv = v.shape
    P = 1.0 / lam0
    m = np.array(s0, np.float64)
    o = np.zeros((T, dv))
    lm = np.zeros(T)
    gain = np.zeros(T)
    for t in range(T):
        m = a[t] * m
        P = a[t] ** 2 * P + nu[t]
        lm[t] = 1.0 / P
        Sinn = k[t] ** 2 * P + r[t]
        K = P * k[t] / Sinn
        gain[t] = K
        m = m + K * (v[t] - k[t] * m)
        P = (1.0 - K * k[t]) * P
        o[t] = m * q[t]
    return o, m, 1.0 / P, lm, gain


def dense_kalman(q, k, v, a, nu, r, lam0, S0):
    """Full-covariance Kalman filter for one head; the d_v rows of the memory share
    one d_k x d_k covariance.  q, k: [T, dk]; v: [T, dv]; lam0: [dk] (diagonal
    prior precision); S0: [dv, dk].  Returns o, S_T, final covariance, and the
    per-token predictive covariances and gains."""
    q, k, v, a, nu, r = (np.asarray(x, np.float64) for x in (q, k, v, a, nu, r))
    T, dk = k.shape
    Sig = np.diag(1.0 / np.asarray(lam0, np.float64))
    M = np.array(S0, np.float64)
    I = np.eye(dk)
    o = np.zeros((T, v.shape[1]))
    prior = np.zeros((T, dk, dk))
    gains = np.zeros((T, dk))
    for t in range(T):
        kt = k[t].astype(np.float64)
        M = a[t] * M
        Sig = a[t] ** 2 * Sig + nu[t] * I
        prior[t] = Sig
        s = kt @ Sig @ kt + r[t]
        K = Sig @ kt / s
        gains[t] = K
        M = M + np.outer(v[t] - M @ kt, K)
        J = I - np.outer(K, kt)
        Sig = J @ Sig @ J.T + r[t] * np.outer(K, K)
        o[t] = M @ q[t]
    return o, M, Sig, prior, gains


def gated_delta(q, k, v, a, beta, S0):
    """Gated delta rule for one head with given write strengths beta [T]."""
    q, k, v, a, beta = (np.asarray(x, np.float64) for x in (q, k, v, a, beta))
    T, dk = k.shape
    S = np.array(S0, np.float64)
    o = np.zeros((T, v.shape[1]))
    I = np.eye(dk)
    for t in range(T):
        kt = k[t].astype(np.float64)
        S = a[t] * S @ (I - beta[t] * np.outer(kt, kt)) + beta[t] * np.outer(v[t], kt)
        o[t] = S @ q[t]
    return o, S


def chunk_forward(q, k, v, a, w, S0, C):
    """Chunkwise form of S_t = a_t S_{t-1} + (v_t - a_t S_{t-1} k_t) w_t^T, o_t = S_t q_t.

    Within a chunk with local cumulative decay gamma_t = prod_{s<=t} a_s:
      (I + A) U = V - diag(gamma) K S0^T,   A_ts = (gamma_t / gamma_s) k_t.w_s (s < t)
      O = diag(gamma) Q S0^T + (tril(Q W^T) * Gamma) U     (diagonal included)
      S_end = gamma_C S0 + U^T diag(gamma_C / gamma_s) W
    """
    T, dk = k.shape
    dv = v.shape[1]
    S = np.array(S0, np.float64)
    o = np.zeros((T, dv))
    for c0 in range(0, T, C):
        sl = slice(c0, min(c0 + C, T))
        K, W, Q, V = (x[sl].astype(np.float64) for x in (k, w, q, v))
        n = K.shape[0]
        g = np.cumsum(np.log(a[sl].astype(np.float64)))
        gam = np.exp(g)
        diff = g[:, None] - g[None, :]
        low = np.tril(np.ones((n, n), bool))
        Gam = np.where(low, np.exp(np.where(low, diff, 0.0)), 0.0)
        A = np.tril(K @ W.T * Gam, -1)
        U = np.linalg.solve(np.eye(n) + A, V - gam[:, None] * (K @ S.T))
        O = gam[:, None] * (Q @ S.T) + (np.tril(Q @ W.T) * Gam) @ U
        S = gam[-1] * S + U.T @ (np.exp(g[-1] - g)[:, None] * W)
        o[sl] = O
    return o, S


def mobius_step(a, nu, b):
    """Matrix of one token: predict then add evidence b (2x2, float64)."""
    return np.array([[1.0 + b * nu, b * a * a], [nu, a * a]], np.float64)


def mobius_predict(a, nu):
    return np.array([[1.0, 0.0], [nu, a * a]], np.float64)


def mobius_apply(M, x):
    return (M[0, 0] * x + M[0, 1]) / (M[1, 0] * x + M[1, 1])


def _norm(M):
    return M / np.abs(M).max()


def compose_sequential(mats):
    """Pi = M_T ... M_1 by a left fold (later tokens multiply on the left)."""
    P = np.eye(2)
    for M in mats:
        P = _norm(M @ P)
    return P


def compose_tree(mats):
    """Same product by balanced recursive halving."""
    if len(mats) == 1:
        return mats[0]
    h = len(mats) // 2
    return _norm(compose_tree(mats[h:]) @ compose_tree(mats[:h]))


def compose_random(mats, rng):
    """Same product by repeatedly merging a random adjacent pair."""
    items = list(mats)
    while len(items) > 1:
        i = int(rng.integers(0, len(items) - 1))
        items[i:i + 2] = [_norm(items[i + 1] @ items[i])]
    return items[0]


def gaussian_kl(Sig_q, Lam_p):
    """KL( N(m, Sig_q) || N(m, Lam_p^{-1}) ) for equal means, from the definition."""
    d = Sig_q.shape[0]
    _, logdet_q = np.linalg.slogdet(Sig_q)
    _, logdet_lam = np.linalg.slogdet(Lam_p)
    return 0.5 * (np.trace(Lam_p @ Sig_q) - d - logdet_lam - logdet_q)
