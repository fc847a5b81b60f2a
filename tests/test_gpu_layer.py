"""GPU parity of the KDN layer (kdn_layer_forward through the C ABI) against
the layer oracle: projections, per-head L2 normalisation, gates, recurrence
and output projection on random weights."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kalman_filter_memory_amd as kdn
from gpu_util import TOL_BF16, TOL_F32, elementwise, host, normwise, say
from kdn_inputs import layer_inputs
from oracle.layer import layer_forward as oracle_layer

pytestmark = pytest.mark.gpu

# bf16 bar of y: the recurrence's own bf16 bar (2e-2), plus the layer's three
# extra roundings to bf16 (the projection Z, the read-out o and y itself, each
# up to 2^-9 relative, 6e-3 together), rounded up
TOL_LAYER_BF16 = 3e-2


def _tensors(p):
    """Device copies of the layer inputs.  The oracle takes the weights
    input-features major (Z = x W_in); the library takes them out-features
    major (Z = x W_in^T), so they go to the GPU transposed."""
    dt = torch.bfloat16 if p["dtype"] == "bf16" else torch.float32
    t = {"x": torch.from_numpy(p["x"]).cuda().to(dt)}
    t.update({n: torch.from_numpy(np.ascontiguousarray(p[n].T)).cuda().to(dt)
              for n in ("W_in", "W_out")})
    t.update({n: torch.from_numpy(p[n]).cuda() for n in ("b_gate", "lambda0", "S0")})
    return t


def _gpu(p, chunk=64, t=None):
    t = t or _tensors(p)
    y, S_T, lam_T = kdn.layer_forward(t["x"], t["W_in"], t["b_gate"], t["W_out"], p["H"], p["dk"],
                                      p["dv"], t["lambda0"], t["S0"], variant=p["variant"],
                                      chunk=chunk)
    torch.cuda.synchronize()
    return host(y), host(S_T), host(lam_T)


CASES = [
    # B, T, H, D, dk, dv, variant, dtype, chunk
    (2, 100, 2, 64, 32, 32, "diagonal", "f32", 64),
    (1, 130, 4, 128, 64, 32, "isotropic", "f32", 32),
    (2, 77, 2, 96, 32, 64, "diagonal", "bf16", 16),
    (1, 64, 2, 256, 128, 128, "isotropic", "bf16", 64),
    (1, 1, 3, 32, 32, 32, "diagonal", "f32", 16),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}T{c[1]}H{c[2]}D{c[3]}dk{c[4]}dv{c[5]}"
                                              f"{c[6][:4]}{c[7]}" for c in CASES])
def test_layer_matches_oracle(case):
    B, T, H, D, dk, dv, variant, dtype, chunk = case
    p = layer_inputs(B, T, H, D, dk, dv, variant=variant, dtype=dtype, seed=31)
    say(f"[gpu] layer {case}")
    y, S_T, lam = _gpu(p, chunk)
    ref = oracle_layer(p["x"], p["W_in"], p["b_gate"], p["W_out"], H, dk, dv, p["lambda0"],
                       p["S0"], variant)
    e_y, e_s = normwise(y, ref["y"]), normwise(S_T, ref["S_T"])
    e_l = elementwise(lam, ref["lambda_T"])
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    tol_y = TOL_LAYER_BF16 if dtype == "bf16" else TOL_F32
    say(f"    err y {e_y:.2e}  S_T {e_s:.2e}  lambda_T {e_l:.2e}  (tol {tol_y:g}, {tol:g})")
    assert np.all(np.isfinite(y))
    # lambda_T follows the gates, which the layer rounds to bf16 (2^-9 relative)
    assert e_y <= tol_y and e_s <= tol and e_l <= (2e-2 if dtype == "bf16" else 1e-5)


def test_layer_empty_sequence_passes_the_state_through():
    p = layer_inputs(2, 0, 2, 64, 32, 32, seed=32)
    say("[gpu] layer T=0")
    y, S_T, lam = _gpu(p)
    assert y.shape == (2, 0, 64)
    np.testing.assert_array_equal(S_T, p["S0"])
    np.testing.assert_array_equal(lam, p["lambda0"])


def test_layer_workload_bf16_B8_T4096_H16_D2048_sampled_batch():
    """The layer at full size (B8 T4096 H16, d_model 2048, d 128, bf16) on the
    GPU; batch element 0 (all 16 heads, all 4096 tokens) against the oracle,
    which treats batch elements independently."""
    p = layer_inputs(8, 4096, 16, 2048, 128, 128, dtype="bf16", seed=33)
    say("[gpu] layer workload B8 T4096 H16 D2048 d128 bf16")
    y, S_T, lam = _gpu(p)
    ref = oracle_layer(p["x"][:1], p["W_in"], p["b_gate"], p["W_out"], 16, 128, 128,
                       p["lambda0"][:1], p["S0"][:1], "diagonal")
    e_y, e_s = normwise(y[:1], ref["y"]), normwise(S_T[:1], ref["S_T"])
    say(f"    batch 0: err y {e_y:.2e}  S_T {e_s:.2e}")
    assert np.all(np.isfinite(y))
    assert e_y <= TOL_LAYER_BF16 and e_s <= TOL_BF16


def test_layer_is_bitwise_deterministic():
    p = layer_inputs(2, 300, 4, 256, 64, 64, dtype="bf16", seed=34)
    t = _tensors(p)
    say("[gpu] layer determinism")
    a = _gpu(p, t=t)
    b = _gpu(p, t=t)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_layer_with_stage_events_matches_and_times_every_stage():
    """kdn_layer_forward_events (the benchmark's timing path): the same output,
    bit for bit, and a positive time for each of the five stages."""
    p = layer_inputs(2, 200, 4, 128, 32, 32, dtype="bf16", seed=35)
    t = _tensors(p)
    say("[gpu] layer with stage events")
    plain = _gpu(p, t=t)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(10)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    y, S_T, lam_T = kdn.layer_forward(t["x"], t["W_in"], t["b_gate"], t["W_out"], p["H"], p["dk"],
                                      p["dv"], t["lambda0"], t["S0"], variant=p["variant"],
                                      events=evs)
    torch.cuda.synchronize()
    for a, b in zip(plain, (host(y), host(S_T), host(lam_T))):
        np.testing.assert_array_equal(a, b)
    times = [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(5)]
    say(f"    stage ms {['%.3f' % x for x in times]}")
    assert all(x > 0 for x in times)
