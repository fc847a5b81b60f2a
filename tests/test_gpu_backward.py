"""GPU parity of the backward pass (kdn_backward, both variants) against the
fp64 oracle's vector-Jacobian product, through the C ABI.

Every gradient is compared per (b, h) slice with the normwise metric of the
forward tests (max|x - ref| / max|ref| over the slice).  Bars: TOL_BWD_F32 for
float32 inputs (the forward's float32 bar) and TOL_BWD_BF16 for bfloat16 inputs
(the MFMA operands -- the states, U, dU, dR -- are rounded to bfloat16, 2^-9
relative each, as in the forward; every gradient, dlambda0 included, is fed by
dW and so by those products).  The full-size workloads run in the launch
configuration of the benchmark, and the oracle checks every head of them.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kalman_filter_memory_amd as kdn
import oracle
from gpu_util import cached_config, forward_tensors, host, normwise, say, to_dev, tdtype
from kdn_inputs import backward_cotangents, config_inputs, forward_inputs

pytestmark = pytest.mark.gpu

TOL_BWD_F32 = 1e-4
TOL_BWD_BF16 = 3e-2
GRADS = ("dq", "dk", "dv", "da", "dnu", "dr", "dlambda0", "dS0")
KEYMAP = {"dnu": "dqnoise"}


def _gpu_backward(inp, cot, chunk):
    t = forward_tensors(inp)
    dO = to_dev(cot["dO"], tdtype(inp["dtype"]))
    dS_T = None if cot["dS_T"] is None else to_dev(cot["dS_T"], torch.float32)
    dl_T = None if cot["dlambda_T"] is None else to_dev(cot["dlambda_T"], torch.float32)
    g = kdn.backward(t["q"], t["k"], t["v"], t["a"], t["nu"], t["r"], dO, t["lambda0"],
                     t["S0"], dS_T, dl_T, variant=inp["variant"], chunk=chunk)
    torch.cuda.synchronize()
    return {n: host(g[KEYMAP.get(n, n)]) for n in GRADS}


def _oracle_backward(inp, cot):
    return oracle.backward(inp["q"], inp["k"], inp["v"], inp["a"], inp["nu"], inp["r"],
                           cot["dO"], inp["lambda0"], inp["S0"], cot["dS_T"], cot["dlambda_T"],
                           variant=inp["variant"])


def _errors(got, ref):
    """Normwise error per (b, h) slice.  A per-head scalar (the isotropic
    dlambda0, shape [B, H]) has one element per slice, where the normwise
    ratio degenerates into the elementwise one that is ill-posed near zero; it
    is taken over the H heads of each batch element instead (max over heads of
    |x - ref| divided by the max over heads of |ref|).  Its per-head relative
    errors are printed as a diagnostic."""
    err = {}
    for n in GRADS:
        x = got[n]
        if ref[n].ndim == 2:
            err[n] = normwise(x[None], ref[n][None])
            rel = np.abs(x - ref[n]) / np.maximum(np.abs(ref[n]), 1e-300)
            say(f"    {n} per head: worst relative {rel.max():.1e}, median {np.median(rel):.1e}, "
                f"|ref| from {np.abs(ref[n]).min():.2e} to {np.abs(ref[n]).max():.2e}")
        else:
            err[n] = normwise(x, ref[n])
    return err


def _assert(err, dtype):
    tol = TOL_BWD_BF16 if dtype == "bf16" else TOL_BWD_F32
    say("    " + "  ".join(f"{n} {e:.1e}" for n, e in err.items()) + f"  (tol {tol:g})")
    for n, e in err.items():
        assert e <= tol, (n, e)


SMALL = [
    # B, H, T, dk, dv, chunk, dtype
    (1, 1, 1, 32, 32, 16, "f32"),
    (1, 2, 37, 32, 64, 16, "f32"),
    (1, 2, 100, 64, 32, 32, "bf16"),
    (1, 2, 200, 64, 128, 64, "f32"),
    (1, 1, 97, 128, 64, 32, "f32"),
    (2, 2, 65, 128, 32, 64, "bf16"),
    (2, 1, 130, 128, 128, 64, "bf16"),
    (3, 1, 300, 128, 128, 16, "bf16"),
    (1, 3, 64, 32, 128, 64, "f32"),
]


@pytest.mark.parametrize("idx", range(len(SMALL)),
                         ids=["B{}H{}T{}k{}v{}C{}_{}".format(*c) for c in SMALL])
def test_backward_small_shapes(idx):
    B, H, T, dk, dv, C, dtype = SMALL[idx]
    inp = forward_inputs(B, H, T, dk, dv, dtype=dtype, seed=300 + idx)
    cot = backward_cotangents(B, H, T, dk, dv, dtype=dtype, seed=300 + idx)
    say(f"[gpu] backward B{B} H{H} T{T} dk{dk} dv{dv} C{C} {dtype}")
    got = _gpu_backward(inp, cot, C)
    for n, x in got.items():
        assert np.all(np.isfinite(x)), n
    _assert(_errors(got, _oracle_backward(inp, cot)), dtype)


SMALL_ISO = [
    # B, H, T, dk, dv, chunk, dtype
    (1, 1, 1, 32, 32, 16, "f32"),
    (2, 3, 37, 32, 64, 16, "f32"),
    (2, 1, 130, 128, 128, 64, "bf16"),
    (1, 3, 64, 32, 128, 64, "f32"),
    (1, 2, 100, 64, 32, 32, "bf16"),
]


@pytest.mark.parametrize("idx", range(len(SMALL_ISO)),
                         ids=["iso_B{}H{}T{}k{}v{}C{}_{}".format(*c) for c in SMALL_ISO])
def test_backward_isotropic_small_shapes(idx):
    B, H, T, dk, dv, C, dtype = SMALL_ISO[idx]
    inp = forward_inputs(B, H, T, dk, dv, variant="isotropic", dtype=dtype, seed=350 + idx)
    cot = backward_cotangents(B, H, T, dk, dv, variant="isotropic", dtype=dtype, seed=350 + idx)
    say(f"[gpu] backward isotropic B{B} H{H} T{T} dk{dk} dv{dv} C{C} {dtype}")
    got = _gpu_backward(inp, cot, C)
    for n, x in got.items():
        assert np.all(np.isfinite(x)), n
    _assert(_errors(got, _oracle_backward(inp, cot)), dtype)


def test_workload_iso_f32_B1_H2_T256_d32_backward():
    inp = config_inputs(0)
    cot = backward_cotangents(1, 2, 256, 32, 32, variant="isotropic", dtype="f32", seed=1000)
    say("[gpu] backward iso f32 [1,2,256,32]")
    _assert(_errors(_gpu_backward(inp, cot, 32), _oracle_backward(inp, cot)), "f32")


def test_backward_without_state_cotangents():
    inp = forward_inputs(1, 2, 150, 64, 64, dtype="bf16", seed=41)
    cot = backward_cotangents(1, 2, 150, 64, 64, dtype="bf16", seed=41, state_cotangents=False)
    say("[gpu] backward, read-out cotangent only")
    _assert(_errors(_gpu_backward(inp, cot, 64), _oracle_backward(inp, cot)), "bf16")


def test_backward_empty_sequence_passes_state_cotangents_through():
    inp = forward_inputs(1, 2, 0, 64, 64, seed=42)
    cot = backward_cotangents(1, 2, 0, 64, 64, seed=42)
    say("[gpu] backward T=0")
    got = _gpu_backward(inp, cot, 64)
    np.testing.assert_array_equal(got["dS0"], cot["dS_T"])
    np.testing.assert_array_equal(got["dlambda0"], cot["dlambda_T"])
    assert got["dq"].size == 0 and got["da"].size == 0


def test_workload_diag_f32_B2_H4_T2048_d64_backward():
    inp = config_inputs(1)
    cot = backward_cotangents(2, 4, 2048, 64, 64, dtype="f32", seed=1001)
    say("[gpu] backward diag f32 [2,4,2048,64]")
    _assert(_errors(_gpu_backward(inp, cot, 64), _oracle_backward(inp, cot)), "f32")


def _full_size_all_heads(index, B, H, T, d, variant=None):
    say(f"[gpu] generating workload {index}")
    inp = cached_config(index, variant)
    cot = backward_cotangents(B, H, T, d, d, variant=inp["variant"], dtype="bf16",
                              seed=1000 + index)
    say(f"[gpu] backward full size {inp['q'].shape}")
    got = _gpu_backward(inp, cot, 64)
    for n, x in got.items():
        assert np.all(np.isfinite(x)), n
    say(f"[cpu] oracle backward on all {B * H} heads")
    _assert(_errors(got, _oracle_backward(inp, cot)), "bf16")


def test_workload_diag_bf16_B8_H16_T4096_d128_backward_all_heads():
    _full_size_all_heads(2, 8, 16, 4096, 128)


@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_workload_long_bf16_B1_H16_T65536_d128_backward_all_heads(variant):
    _full_size_all_heads(3, 1, 16, 65536, 128, variant)


@pytest.mark.parametrize("variant,dtype", [("diagonal", "bf16"), ("isotropic", "f32")])
def test_forward_keep_then_backward_kept_matches_the_plain_calls(variant, dtype):
    """kdn_forward_keep returns what kdn_forward returns and kdn_backward_kept
    what kdn_backward returns (the same kernels on the same inputs: bitwise)."""
    B, H, T, dk, dv, C = 2, 2, 150, 64, 64, 64
    inp = forward_inputs(B, H, T, dk, dv, variant=variant, dtype=dtype, seed=61)
    cot = backward_cotangents(B, H, T, dk, dv, variant=variant, dtype=dtype, seed=61)
    say(f"[gpu] forward_keep + backward_kept {variant} {dtype}")
    t = forward_tensors(inp)
    dO = to_dev(cot["dO"], tdtype(dtype))
    dS_T = to_dev(cot["dS_T"], torch.float32)
    dl_T = to_dev(cot["dlambda_T"], torch.float32)
    args = (t["q"], t["k"], t["v"], t["a"], t["nu"], t["r"])
    o, S_T, lam = kdn.forward(*args, t["lambda0"], t["S0"], variant=variant, chunk=C)
    desc = kdn.make_desc(B, H, T, dk, dv, C, variant, kdn._dtype_code(t["q"].dtype),
                         kdn._dtype_code(t["a"].dtype))
    keep = torch.empty(kdn.backward_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    o2, S_T2, lam2 = kdn.forward(*args, t["lambda0"], t["S0"], variant=variant, chunk=C,
                                 keep=keep)
    g_kept = kdn.backward(*args, dO, t["lambda0"], t["S0"], dS_T, dl_T, variant=variant,
                          chunk=C, kept=keep)
    g = kdn.backward(*args, dO, t["lambda0"], t["S0"], dS_T, dl_T, variant=variant, chunk=C)
    torch.cuda.synchronize()
    for x, y in ((o, o2), (S_T, S_T2), (lam, lam2)):
        assert torch.equal(x, y)
    for n in g:
        assert torch.equal(g[n], g_kept[n]), n


@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_backward_is_bitwise_reproducible(variant):
    """No atomics in the gradient reductions: two calls give identical bits."""
    inp = forward_inputs(2, 3, 200, 128, 128, variant=variant, dtype="bf16", seed=71)
    cot = backward_cotangents(2, 3, 200, 128, 128, variant=variant, dtype="bf16", seed=71)
    say(f"[gpu] backward twice, {variant}")
    a = _gpu_backward(inp, cot, 64)
    b = _gpu_backward(inp, cot, 64)
    for n in GRADS:
        np.testing.assert_array_equal(a[n], b[n], err_msg=n)
