"""fp64 CPU oracle of the KDN layer around the recurrence (projections, per-head
L2 normalisation of queries and keys, gate activations, output projection).

TEST INFRASTRUCTURE ONLY, like the rest of this package: tests, the smoke
check and the benchmark's CPU-baseline leg may call it; the GPU library never
does.  The steps follow "Kalman Delta Networks" (English abstract: the layer
replaces linear attention in a language model) and the KDN summary (section
关键模块: queries, keys and values, the decay gate a in (0, 1] and the two
noise variances nu and r, positive), read as:

  Z = x W_in, columns [q (head-major) | k | v | logits of a | nu | r];
  q_h <- q_h / max(|q_h|, 1e-6), the same for k_h;
  a = sigmoid(z_a + b_a), nu = softplus(z_nu + b_nu), r = softplus(z_r + b_r);
  o = the recurrence (``oracle.forward``) over the B*H heads;
  y = [o_1 .. o_H] W_out.

The products are numpy matmuls in float64.  The recurrence's oracle takes
float32 inputs, so q, k, v and the gates are rounded to float32 on the way in
(relative 6e-8).
"""
from __future__ import annotations

import numpy as np

from . import forward


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.log1p(np.exp(x))


def layer_forward(x, W_in, b_gate, W_out, H, dk, dv, lambda0=None, S0=None,
                  variant="diagonal", debug=False) -> dict:
    """x [B,T,D] -> y [B,T,D] (float64), with S_T and lambda_T of the
    recurrence.  With debug=True also the recurrence's inputs q, k, v, a, nu, r
    ([B,H,T,.], float64) and its output o."""
    x = np.asarray(x, np.float64)
    W_in = np.asarray(W_in, np.float64)
    W_out = np.asarray(W_out, np.float64)
    b_gate = np.asarray(b_gate, np.float64)
    B, T, D = x.shape
    assert W_in.shape == (D, H * (2 * dk + dv) + 3 * H)
    assert W_out.shape == (H * dv, D) and b_gate.shape == (3 * H,)
    Z = x @ W_in

    def heads(lo, d):  # [B,T,H*d] columns from lo -> [B,H,T,d]
        return Z[..., lo:lo + H * d].reshape(B, T, H, d).transpose(0, 2, 1, 3)

    q, k, v = heads(0, dk), heads(H * dk, dk), heads(2 * H * dk, dv)
    q = q / np.maximum(np.sqrt((q * q).sum(-1, keepdims=True)), 1e-6)
    k = k / np.maximum(np.sqrt((k * k).sum(-1, keepdims=True)), 1e-6)
    g0 = H * (2 * dk + dv)
    logits = Z[..., g0:g0 + 3 * H].reshape(B, T, 3, H) + b_gate.reshape(3, H)
    logits = logits.transpose(2, 0, 3, 1)  # [3, B, H, T]
    a, nu, r = _sigmoid(logits[0]), _softplus(logits[1]), _softplus(logits[2])
    core = forward(q, k, v, a, nu, r, lambda0, S0, variant)
    o = core["o"]  # [B,H,T,dv]
    y = o.transpose(0, 2, 1, 3).reshape(B, T, H * dv) @ W_out
    out = {"y": y, "S_T": core["S_T"], "lambda_T": core["lambda_T"]}
    if debug:
        out.update(q=q, k=k, v=v, a=a, nu=nu, r=r, o=o)
    return out
