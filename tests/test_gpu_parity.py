"""GPU parity of libkdn against the fp64 oracle, through the C ABI.

Bars: o and S_T within 1e-4 (float32 inputs) or 2e-2 (bfloat16 inputs, float32
state) normwise per (b, h); lambda within 1e-5 elementwise relative.  The
full-size workloads run in the same launch configuration as the benchmark,
and the oracle checks every head of them."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kalman_filter_memory_amd as kdn
import oracle
from gpu_util import (TOL_BF16, TOL_F32, TOL_LAMBDA, cached_config, elementwise,
                      forward_tensors, host, normwise, row_errors, say)
from kdn_inputs import config_inputs, forward_inputs, decode_inputs

pytestmark = pytest.mark.gpu


def _tol(dtype):
    return TOL_BF16 if dtype == "bf16" else TOL_F32


def _gpu_forward(inp, chunk, variant=None):
    t = forward_tensors(inp)
    o, S_T, lam_T = kdn.forward(t["q"], t["k"], t["v"], t["a"], t["nu"], t["r"], t["lambda0"],
                                t["S0"], variant=variant or inp["variant"], chunk=chunk)
    torch.cuda.synchronize()
    return host(o), host(S_T), host(lam_T)


def _oracle_forward(inp, debug=False):
    return oracle.forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["nu"], inp["r"],
                          inp["lambda0"], inp["S0"], inp["variant"], debug=debug)


def _check_forward(inp, chunk, label):
    say(f"[gpu] forward {label}: {inp['variant']} {inp['dtype']} q{inp['q'].shape} C={chunk}")
    o, S_T, lam = _gpu_forward(inp, chunk)
    ref = _oracle_forward(inp)
    tol = _tol(inp["dtype"])
    e_o = normwise(o, ref["o"])
    e_s = normwise(S_T, ref["S_T"])
    e_l = elementwise(lam, ref["lambda_T"])
    say(f"    err o {e_o:.2e}  S_T {e_s:.2e}  lambda_T {e_l:.2e}  (tol {tol:g}, {TOL_LAMBDA:g})")
    assert np.all(np.isfinite(o))
    assert e_o <= tol and e_s <= tol and e_l <= TOL_LAMBDA
    return o, S_T, lam


# ------------------------------------------------------------- small shapes
SMALL = [
    # B, H, T, dk, dv, chunk, variant, dtype
    (1, 1, 1, 32, 32, 16, "diagonal", "f32"),
    (2, 3, 37, 32, 64, 16, "isotropic", "f32"),
    (1, 2, 100, 64, 32, 32, "diagonal", "bf16"),
    (2, 1, 130, 128, 128, 64, "isotropic", "bf16"),
    (1, 2, 200, 64, 128, 64, "diagonal", "f32"),
    (1, 1, 97, 128, 64, 32, "diagonal", "f32"),
    (2, 2, 65, 128, 32, 64, "diagonal", "bf16"),
    (1, 3, 64, 32, 128, 64, "isotropic", "f32"),
    (3, 1, 300, 128, 128, 16, "diagonal", "bf16"),
    # d_k < 64 with four 16-token sub-blocks: the gain's lanes past d_k are idle
    (1, 3, 64, 32, 128, 64, "diagonal", "f32"),
    (1, 3, 130, 32, 64, 64, "diagonal", "bf16"),
]


@pytest.mark.parametrize("idx", range(len(SMALL)),
                         ids=["B{}H{}T{}k{}v{}C{}_{}_{}".format(*c) for c in SMALL])
def test_forward_small_shapes(idx):
    B, H, T, dk, dv, C, variant, dtype = SMALL[idx]
    inp = forward_inputs(B, H, T, dk, dv, variant=variant, dtype=dtype, seed=100 + idx)
    _check_forward(inp, C, "small")


def test_forward_empty_sequence_returns_initial_state():
    inp = forward_inputs(1, 2, 0, 64, 64, seed=5)
    o, S_T, lam = _gpu_forward(inp, 64)
    assert o.shape == (1, 2, 0, 64)
    np.testing.assert_array_equal(S_T, inp["S0"])
    np.testing.assert_array_equal(lam, inp["lambda0"])


def test_forward_no_heads_is_a_no_op():
    inp = forward_inputs(0, 4, 16, 32, 32, seed=6)
    o, S_T, lam = _gpu_forward(inp, 16)
    assert o.size == 0 and S_T.size == 0


# ------------------------------------------- the segmented state pass
# Few heads, many chunks: the state pass is cut into sequence segments (each
# segment's affine map, their composition, then the read-out).  Shapes with a
# ragged last chunk, several segment counts, both variants and dtypes.
SEGMENTED = [
    # B, H, T, dk, dv, chunk, variant, dtype
    (1, 1, 16 * 64 + 37, 64, 64, 64, "diagonal", "f32"),
    (1, 2, 40 * 32 + 5, 128, 64, 32, "isotropic", "f32"),
    (2, 1, 24 * 16 + 9, 32, 128, 16, "diagonal", "bf16"),
    (1, 3, 20 * 64, 128, 128, 64, "diagonal", "bf16"),
    (1, 1, 70 * 64 + 63, 128, 32, 64, "isotropic", "bf16"),
    (1, 2, 33 * 32, 32, 32, 32, "diagonal", "f32"),
]


@pytest.mark.parametrize("idx", range(len(SEGMENTED)),
                         ids=["seg_B{}H{}T{}k{}v{}C{}_{}_{}".format(*c) for c in SEGMENTED])
def test_segmented_state_pass_matches_oracle(idx):
    B, H, T, dk, dv, C, variant, dtype = SEGMENTED[idx]
    inp = forward_inputs(B, H, T, dk, dv, variant=variant, dtype=dtype, seed=150 + idx)
    td = kdn.BF16 if dtype == "bf16" else kdn.F32
    nseg = kdn.forward_segments(kdn.make_desc(B, H, T, dk, dv, C, variant, td, td))
    say(f"[gpu] segmented state pass: {nseg} segments")
    assert nseg > 1
    _check_forward(inp, C, f"segmented ({nseg} segments)")


# ------------------------------------------- the repeat timing aid
# kdn_forward_repeat relaunches a range of the forward's kernels on the
# workspace a forward left: every relaunch must leave the forward's outputs
# bit for bit (the plain state pass, the segmented one, both variants).
@pytest.mark.parametrize("shape", [(2, 2, 300, 128, 128, 64, "diagonal"),
                                   (2, 2, 300, 128, 128, 64, "isotropic"),
                                   (1, 1, 64 * 40 + 9, 128, 128, 64, "diagonal")],
                         ids=["plain_diag", "plain_iso", "segmented_diag"])
def test_forward_repeat_rewrites_the_same_results(shape):
    B, H, T, dk, dv, C, variant = shape
    inp = forward_inputs(B, H, T, dk, dv, variant=variant, dtype="bf16", seed=170)
    t = forward_tensors(inp)
    d = kdn.make_desc(B, H, T, dk, dv, C, variant, kdn.BF16, kdn.BF16)
    say(f"[gpu] repeat {shape}: {kdn.forward_segments(d)} segments")
    ws = torch.empty(kdn.forward_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    args = (t["q"], t["k"], t["v"], t["a"], t["nu"], t["r"], t["lambda0"], t["S0"], variant, C)
    out = kdn.forward(*args, workspace=ws)
    ref = [host(x).copy() for x in out]
    for first, last in [(0, 3), (0, 2), (1, 3), (2, 2), (3, 3), (0, 0)]:
        kdn.forward(*args, workspace=ws, out=out, repeat=(first, last, 3))
        torch.cuda.synchronize()
        for name, got, want in zip(("o", "S_T", "lambda_T"), out, ref):
            assert np.array_equal(host(got), want), (first, last, name)


# ---------------------------------------------------- the named workloads
def test_workload_iso_f32_B1_H2_T256_d32():
    _check_forward(config_inputs(0), 32, "iso f32 [1,2,256,32]")


def test_workload_diag_f32_B2_H4_T2048_d64():
    _check_forward(config_inputs(1), 64, "diag f32 [2,4,2048,64]")


def _full_size_all_heads(index, variant, chunk=64):
    """The full-size workload in the benchmark's launch configuration, every
    head compared with the oracle (which runs the whole workload on the host
    cores), plus a per-token-row diagnostic of o."""
    say(f"[gpu] generating workload {index} ({variant})")
    inp = cached_config(index, variant)
    say(f"[gpu] forward full size {inp['q'].shape} {variant}")
    o, S_T, lam = _gpu_forward(inp, chunk)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S_T)) and np.all(lam > 0)
    say(f"[cpu] oracle on all {inp['q'].shape[0] * inp['q'].shape[1]} heads")
    ref = _oracle_forward(inp)
    e_o = normwise(o, ref["o"])
    e_s = normwise(S_T, ref["S_T"])
    e_l = elementwise(lam, ref["lambda_T"])
    r_o, r_i, r_frac = row_errors(o, ref["o"])
    say(f"    all heads: err o {e_o:.2e}  S_T {e_s:.2e}  lambda_T {e_l:.2e}; worst token row "
        f"of o {r_o:.2e} (row {r_i}), rows above 1e-2: {r_frac:.1e}")
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16 and e_l <= TOL_LAMBDA


def test_workload_diag_bf16_B8_H16_T4096_d128_all_heads():
    _full_size_all_heads(2, "diagonal")


def test_workload_iso_bf16_B8_H16_T4096_d128_all_heads():
    """The isotropic forward at the layer workload (the benchmark times it too)."""
    _full_size_all_heads(2, "isotropic")


@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_workload_long_bf16_B1_H16_T65536_d128_all_heads(variant):
    _full_size_all_heads(3, variant)


def test_workload_decode_N256_H16_d128_128_steps_all_states():
    """128 in-place decode steps on all 256 x 16 cached states: o of every
    state at every step against the oracle's step, and the whole cache (S and
    lambda) after steps 1, 64 and 128."""
    d = cached_config(4)
    steps = d["q"].shape[0]
    S = torch.from_numpy(d["S0"]).cuda()
    lam = torch.from_numpy(d["lambda0"]).cuda()
    dev = {n: torch.from_numpy(d[n]).cuda().to(torch.bfloat16 if n in ("q", "k", "v")
                                               else torch.float32)
           for n in ("q", "k", "v", "a", "nu", "r")}
    Sr = d["S0"].astype(np.float64)
    lr = d["lambda0"].astype(np.float64)
    say(f"[gpu] decode {steps} steps on S{tuple(S.shape)}, every state checked")
    worst_o, worst_s, worst_l = 0.0, 0.0, 0.0
    for s in range(steps):
        o = kdn.decode_step(dev["q"][s], dev["k"][s], dev["v"][s], dev["a"][s], dev["nu"][s],
                            dev["r"][s], S, lam, "diagonal")
        o_ref = oracle.decode_step(*(d[n][s] for n in ("q", "k", "v", "a", "nu", "r")), Sr, lr,
                                   "diagonal")
        worst_o = max(worst_o, normwise(host(o), o_ref))
        if s in (0, 63, steps - 1):
            torch.cuda.synchronize()
            S_h, l_h = host(S), host(lam)
            assert np.all(np.isfinite(S_h))
            e_s, e_l = normwise(S_h, Sr), elementwise(l_h, lr)
            say(f"    after step {s + 1}: err o (worst so far) {worst_o:.2e}  S {e_s:.2e}  "
                f"lambda {e_l:.2e}")
            worst_s, worst_l = max(worst_s, e_s), max(worst_l, e_l)
    assert worst_o <= TOL_BF16 and worst_s <= TOL_BF16 and worst_l <= TOL_LAMBDA


# ----------------------------------------------------- the separate steps
@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mobius_scan_matches_oracle_precisions(variant, dtype):
    inp = forward_inputs(2, 2, 333, 64, 32, variant=variant, dtype=dtype, seed=21)
    say(f"[gpu] mobius_scan {variant} {dtype}")
    t = forward_tensors(inp)
    out = kdn.mobius_scan(t["k"], t["a"], t["nu"], t["r"], t["lambda0"], variant=variant,
                          chunk=32, lambda_minus=True, lambda_chunk=True)
    torch.cuda.synchronize()
    ref = _oracle_forward(inp, debug=True)
    e_lm = elementwise(host(out["lambda_minus"]), ref["lambda_minus"])
    e_lt = elementwise(host(out["lambda_T"]), ref["lambda_T"])
    say(f"    err lambda_minus {e_lm:.2e}  lambda_T {e_lt:.2e}")
    assert e_lm <= TOL_LAMBDA and e_lt <= TOL_LAMBDA
    lc = host(out["lambda_chunk"])
    np.testing.assert_array_equal(lc[:, :, 0], inp["lambda0"])
    np.testing.assert_array_equal(lc[:, :, -1], host(out["lambda_T"]))


@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
@pytest.mark.parametrize("T,chunk", [(200 * 16 + 7, 16), (20000, 16), (1500 * 64 + 5, 64)])
def test_mobius_scan_carry_over_many_chunks(variant, T, chunk):
    """The carry splits each scan into more segments as the chunk count grows
    (16 at 201 chunks, 64 at 1,250 and 1,501 chunks, where a segment no longer
    fits in registers and is read twice)."""
    inp = forward_inputs(1, 2, T, 32, 32, variant=variant, dtype="bf16", seed=29, a_mu=4.0)
    say(f"[gpu] mobius_scan carry, {variant}, T={T} chunk={chunk}")
    t = forward_tensors(inp)
    out = kdn.mobius_scan(t["k"], t["a"], t["nu"], t["r"], t["lambda0"], variant=variant,
                          chunk=chunk, lambda_minus=True, lambda_chunk=True)
    torch.cuda.synchronize()
    ref = _oracle_forward(inp, debug=True)
    e_lm = elementwise(host(out["lambda_minus"]), ref["lambda_minus"])
    e_lt = elementwise(host(out["lambda_T"]), ref["lambda_T"])
    say(f"    err lambda_minus {e_lm:.2e}  lambda_T {e_lt:.2e}")
    assert e_lm <= TOL_LAMBDA and e_lt <= TOL_LAMBDA


@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
@pytest.mark.parametrize("dtype,gain_dtype", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
def test_gain_matches_oracle(variant, dtype, gain_dtype):
    inp = forward_inputs(1, 3, 150, 128, 32, variant=variant, dtype=dtype, seed=22)
    ref = _oracle_forward(inp, debug=True)
    say(f"[gpu] gain {variant} {dtype}->{gain_dtype}")
    t = forward_tensors(inp)
    lm = torch.from_numpy(ref["lambda_minus"].astype(np.float32)).cuda()
    gd = torch.bfloat16 if gain_dtype == "bf16" else torch.float32
    w = kdn.gain(t["k"], t["r"], lm, variant=variant, gain_dtype=gd)
    torch.cuda.synchronize()
    err = normwise(host(w), ref["w"], lead=3)
    say(f"    err w {err:.2e}")
    assert err <= (4e-3 if gain_dtype == "bf16" else 1e-5)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_delta_with_given_gain_matches_oracle(dtype):
    inp = forward_inputs(2, 2, 190, 64, 64, variant="diagonal", dtype=dtype, seed=23)
    ref = _oracle_forward(inp, debug=True)
    say(f"[gpu] chunk_delta {dtype}")
    t = forward_tensors(inp)
    w = torch.from_numpy(ref["w"].astype(np.float32)).cuda().to(t["q"].dtype)
    o, S_T = kdn.chunk_delta(t["q"], t["k"], t["v"], t["a"], w, t["S0"], chunk=64)
    torch.cuda.synchronize()
    e_o, e_s = normwise(host(o), ref["o"]), normwise(host(S_T), ref["S_T"])
    say(f"    err o {e_o:.2e}  S_T {e_s:.2e}")
    assert e_o <= _tol(dtype) and e_s <= _tol(dtype)


# -------------------------------------------------------------- invariants
def test_chunk_size_does_not_change_the_result():
    inp = forward_inputs(1, 2, 250, 64, 64, variant="diagonal", dtype="f32", seed=24)
    res = [_gpu_forward(inp, c) for c in (16, 32, 64)]
    for o, S_T, lam in res[1:]:
        assert normwise(o, res[0][0]) < 1e-5
        assert normwise(S_T, res[0][1]) < 1e-5
        assert elementwise(lam, res[0][2]) < 1e-5


@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_resume_from_carried_state(variant):
    inp = forward_inputs(2, 1, 300, 32, 64, variant=variant, dtype="f32", seed=25)
    T1 = 129
    t = forward_tensors(inp)
    full = kdn.forward(t["q"], t["k"], t["v"], t["a"], t["nu"], t["r"], t["lambda0"], t["S0"],
                       variant=variant, chunk=32)
    sl = lambda x, a, b: x[:, :, a:b].contiguous()
    n = ("q", "k", "v", "a", "nu", "r")
    o1, S1, l1 = kdn.forward(*(sl(t[x], 0, T1) for x in n), t["lambda0"], t["S0"],
                             variant=variant, chunk=32)
    o2, S2, l2 = kdn.forward(*(sl(t[x], T1, 300) for x in n), l1, S1, variant=variant, chunk=32)
    torch.cuda.synchronize()
    assert normwise(host(torch.cat([o1, o2], 2)), host(full[0])) < 1e-5
    assert normwise(host(S2), host(full[1])) < 1e-5
    assert elementwise(host(l2), host(full[2])) < 1e-5


@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_decode_steps_equal_forward(variant):
    N, H, dk, dv, steps = 3, 2, 64, 32, 20
    d = decode_inputs(N, H, dk, dv, steps, variant=variant, seed=26, qkv_dtype="f32")
    dev = {n: torch.from_numpy(d[n]).cuda() for n in ("q", "k", "v", "a", "nu", "r")}
    S = torch.from_numpy(d["S0"]).cuda()
    lam = torch.from_numpy(d["lambda0"]).cuda()
    outs = [kdn.decode_step(dev["q"][s], dev["k"][s], dev["v"][s], dev["a"][s], dev["nu"][s],
                            dev["r"][s], S, lam, variant) for s in range(steps)]
    tr = lambda x: x.movedim(0, 2).contiguous()
    o_f, S_f, l_f = kdn.forward(*(tr(dev[n]) for n in ("q", "k", "v", "a", "nu", "r")),
                                torch.from_numpy(d["lambda0"]).cuda(),
                                torch.from_numpy(d["S0"]).cuda(), variant=variant, chunk=16)
    torch.cuda.synchronize()
    assert normwise(host(torch.stack(outs, 2)), host(o_f)) < 1e-5
    assert normwise(host(S), host(S_f)) < 1e-5
    assert elementwise(host(lam), host(l_f)) < 1e-5


DECODE_SHAPES = [(dk, dv) for dk in (32, 64, 128) for dv in (32, 64, 128)]


@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
@pytest.mark.parametrize("dk,dv", DECODE_SHAPES)
def test_decode_shapes_match_oracle(dk, dv, variant):
    """Every built (d_k, d_v) of the decode step (each has its own workgroup
    shape), alternating q/k/v and gate dtypes, three steps against the oracle."""
    i = DECODE_SHAPES.index((dk, dv))
    qkv = "bf16" if i % 2 else "f32"
    gate = "bf16" if (i // 2) % 2 else "f32"
    N, H, steps = 3, 5, 3
    d = decode_inputs(N, H, dk, dv, steps, variant=variant, seed=40 + i, qkv_dtype=qkv,
                      gate_dtype=gate)
    tdt = lambda name: torch.bfloat16 if (gate if name in ("a", "nu", "r") else qkv) == "bf16" \
        else torch.float32
    dev = {n: torch.from_numpy(d[n]).cuda().to(tdt(n)) for n in ("q", "k", "v", "a", "nu", "r")}
    S = torch.from_numpy(d["S0"]).cuda()
    lam = torch.from_numpy(d["lambda0"]).cuda()
    Sr = d["S0"].astype(np.float64)
    lr = d["lambda0"].astype(np.float64)
    say(f"[gpu] decode d_k={dk} d_v={dv} {variant} qkv {qkv} gates {gate}")
    tol = _tol(qkv)
    for s in range(steps):
        o = kdn.decode_step(dev["q"][s], dev["k"][s], dev["v"][s], dev["a"][s], dev["nu"][s],
                            dev["r"][s], S, lam, variant)
        o_ref = oracle.decode_step(*(d[n][s] for n in ("q", "k", "v", "a", "nu", "r")), Sr, lr,
                                   variant)
        e_o = normwise(host(o), o_ref)
        assert e_o <= tol, (s, e_o)
    torch.cuda.synchronize()
    e_s, e_l = normwise(host(S), Sr), elementwise(host(lam), lr)
    say(f"    err S {e_s:.2e}  lambda {e_l:.2e}")
    assert e_s <= tol and e_l <= TOL_LAMBDA


def test_forward_is_bitwise_deterministic():
    inp = forward_inputs(2, 2, 300, 128, 128, variant="diagonal", dtype="bf16", seed=27)
    a = _gpu_forward(inp, 64)
    b = _gpu_forward(inp, 64)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_axis_aligned_keys_follow_the_dense_kalman_filter():
    """One-hot keys (exact in bf16) keep the exact posterior diagonal: the GPU
    result must then follow the dense-covariance Kalman filter."""
    import textbook as tb
    rng = np.random.default_rng(28)
    T, dk, dv = 128, 32, 32
    k = np.zeros((1, 1, T, dk), np.float32)
    k[0, 0, np.arange(T), rng.integers(0, dk, T)] = 1.0
    inp = forward_inputs(1, 1, T, dk, dv, variant="diagonal", dtype="f32", seed=28)
    inp["k"] = k
    o, S_T, lam = _gpu_forward(inp, 32)
    o_ref, M, Sig, _, _ = tb.dense_kalman(inp["q"][0, 0], k[0, 0], inp["v"][0, 0], inp["a"][0, 0],
                                          inp["nu"][0, 0], inp["r"][0, 0], inp["lambda0"][0, 0],
                                          inp["S0"][0, 0])
    assert normwise(o, o_ref[None, None]) <= TOL_F32
    assert normwise(S_T, M[None, None]) <= TOL_F32
    assert elementwise(lam[0, 0], 1.0 / np.diag(Sig)) <= TOL_LAMBDA


@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_decode_indexed_cache_matches_oracle(variant):
    """Continuous batching: 24 active sequences on a cache of 40 slots, slots in
    a shuffled order, one sequence idle (slot -1) and one past the cache; the
    touched slots match the oracle's step, every other slot and the idle rows'
    outputs are left bit for bit as they were."""
    N, H, dk, dv, n_slots = 24, 4, 64, 128, 40
    rng = np.random.default_rng(7)
    cache = decode_inputs(n_slots, H, dk, dv, 1, variant=variant, seed=81)
    step = decode_inputs(N, H, dk, dv, 1, variant=variant, seed=82)
    slots = rng.permutation(n_slots)[:N].astype(np.int32)
    slots[3] = -1
    slots[10] = n_slots + 5
    say(f"[gpu] decode_step_indexed {variant}: N={N} slots={n_slots}")
    S = torch.from_numpy(cache["S0"]).cuda()
    lam = torch.from_numpy(cache["lambda0"]).cuda()
    x = {n: torch.from_numpy(step[n][0]).cuda().to(torch.bfloat16 if n in ("q", "k", "v")
                                                     else torch.float32)
         for n in ("q", "k", "v", "a", "nu", "r")}
    o = torch.full((N, H, dv), 7.0, dtype=torch.bfloat16, device="cuda")
    kdn.decode_step_indexed(x["q"], x["k"], x["v"], x["a"], x["nu"], x["r"], S, lam,
                            torch.from_numpy(slots).cuda(), variant, out=o)
    torch.cuda.synchronize()
    active = [n for n in range(N) if 0 <= slots[n] < n_slots]
    Sr = cache["S0"][slots[active]].astype(np.float64).copy()
    lr = cache["lambda0"][slots[active]].astype(np.float64).copy()
    sub = {n: step[n][0][active] for n in ("q", "k", "v", "a", "nu", "r")}
    o_ref = oracle.decode_step(sub["q"], sub["k"], sub["v"], sub["a"], sub["nu"], sub["r"],
                               Sr, lr, variant)
    o_h, S_h, l_h = host(o), host(S), host(lam)
    e_o = normwise(o_h[active], o_ref)
    e_s = normwise(S_h[slots[active]], Sr)
    e_l = elementwise(l_h[slots[active]], lr)
    say(f"    err o {e_o:.2e}  S {e_s:.2e}  lambda {e_l:.2e}")
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16 and e_l <= TOL_LAMBDA
    untouched = sorted(set(range(n_slots)) - set(slots[active].tolist()))
    np.testing.assert_array_equal(S_h[untouched], cache["S0"][untouched])
    np.testing.assert_array_equal(l_h[untouched], cache["lambda0"][untouched])
    assert np.all(o_h[[3, 10]] == 7.0)


@pytest.mark.parametrize("variant,dtype,chunk", [("diagonal", "bf16", 64),
                                                 ("isotropic", "f32", 32),
                                                 ("diagonal", "f32", 16)])
def test_forward_varlen_matches_oracle_per_sequence(variant, dtype, chunk):
    """A packed batch of sequences of lengths 0, 1, ragged, exact chunk multiples
    and several chunks: each sequence's o, S_T and lambda_T are the oracle's
    for that sequence alone."""
    lens = [37, 0, 64, 1, 200, 130, 65, 5]
    H, dk, dv = 3, 64, 32
    N, T = len(lens), sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    say(f"[gpu] forward_varlen {variant} {dtype} C={chunk} lens={lens}")
    # one draw of a [1, H, T] batch, cut into the sequences
    inp = forward_inputs(1, H, T, dk, dv, variant=variant, dtype=dtype, seed=91)
    init = forward_inputs(N, H, 1, dk, dv, variant=variant, dtype=dtype, seed=92)
    t = forward_tensors(inp)
    lam0 = torch.from_numpy(init["lambda0"]).cuda()
    S0 = torch.from_numpy(init["S0"]).cuda()
    o, S_T, lam_T = kdn.forward_varlen(t["q"][0], t["k"][0], t["v"][0], t["a"][0], t["nu"][0],
                                       t["r"][0], torch.from_numpy(cu).cuda(), max(lens),
                                       lam0, S0, variant=variant, chunk=chunk)
    torch.cuda.synchronize()
    o_h, S_h, l_h = host(o), host(S_T), host(lam_T)
    tol = _tol(dtype)
    for s_, L in enumerate(lens):
        sl = slice(cu[s_], cu[s_ + 1])
        sub = {n: inp[n][:, :, sl] for n in ("q", "k", "v", "a", "nu", "r")}
        ref = oracle.forward(sub["q"], sub["k"], sub["v"], sub["a"], sub["nu"], sub["r"],
                             init["lambda0"][s_:s_ + 1], init["S0"][s_:s_ + 1], variant)
        e_o = normwise(o_h[:, sl][None], ref["o"]) if L else 0.0
        e_s = normwise(S_h[s_:s_ + 1], ref["S_T"])
        e_l = elementwise(l_h[s_:s_ + 1], ref["lambda_T"])
        say(f"    seq {s_} (L={L}): err o {e_o:.2e}  S_T {e_s:.2e}  lambda_T {e_l:.2e}")
        assert e_o <= tol and e_s <= tol and e_l <= TOL_LAMBDA
    # an empty sequence passes its state through unchanged
    np.testing.assert_array_equal(S_h[1], init["S0"][1])
    np.testing.assert_array_equal(l_h[1], init["lambda0"][1])


@pytest.mark.parametrize("variant,dtype,chunk,dk,lens,H", [
    ("diagonal", "bf16", 64, 128, [3000, 0, 1, 700, 64 * 20 + 5], 2),
    ("isotropic", "f32", 32, 64, [2100, 33, 0], 1),
], ids=["diag_bf16_C64", "iso_f32_C32"])
def test_forward_varlen_long_sequences_take_the_segmented_state_pass(variant, dtype, chunk, dk,
                                                                     lens, H):
    """Few (sequence, head) slabs with a long sequence: the packed forward cuts
    every slab into the same number of segments (short and empty sequences get
    empty ones, which act as identity maps); each sequence still matches the
    oracle on its own."""
    N, T = len(lens), sum(lens)
    td = kdn.BF16 if dtype == "bf16" else kdn.F32
    nseg = kdn.forward_segments(kdn.make_desc(N, H, max(lens), dk, dk, chunk, variant, td, td))
    say(f"[gpu] forward_varlen {variant} {dtype} C={chunk} lens={lens}: {nseg} segments")
    assert nseg > 1
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    inp = forward_inputs(1, H, T, dk, dk, variant=variant, dtype=dtype, seed=93)
    init = forward_inputs(N, H, 1, dk, dk, variant=variant, dtype=dtype, seed=94)
    t = forward_tensors(inp)
    o, S_T, lam_T = kdn.forward_varlen(t["q"][0], t["k"][0], t["v"][0], t["a"][0], t["nu"][0],
                                       t["r"][0], torch.from_numpy(cu).cuda(), max(lens),
                                       torch.from_numpy(init["lambda0"]).cuda(),
                                       torch.from_numpy(init["S0"]).cuda(), variant=variant,
                                       chunk=chunk)
    torch.cuda.synchronize()
    o_h, S_h, l_h = host(o), host(S_T), host(lam_T)
    tol = _tol(dtype)
    for s_, L in enumerate(lens):
        sl = slice(cu[s_], cu[s_ + 1])
        sub = {n: inp[n][:, :, sl] for n in ("q", "k", "v", "a", "nu", "r")}
        ref = oracle.forward(sub["q"], sub["k"], sub["v"], sub["a"], sub["nu"], sub["r"],
                             init["lambda0"][s_:s_ + 1], init["S0"][s_:s_ + 1], variant)
        e_o = normwise(o_h[:, sl][None], ref["o"]) if L else 0.0
        e_s = normwise(S_h[s_:s_ + 1], ref["S_T"])
        e_l = elementwise(l_h[s_:s_ + 1], ref["lambda_T"])
        say(f"    seq {s_} (L={L}): err o {e_o:.2e}  S_T {e_s:.2e}  lambda_T {e_l:.2e}")
        assert e_o <= tol and e_s <= tol and e_l <= TOL_LAMBDA
        if L == 0:  # an empty sequence passes its state through unchanged
            np.testing.assert_array_equal(S_h[s_], init["S0"][s_])


@pytest.mark.parametrize("dk,dtype,T,chunk", [(32, "f32", 300, 64), (64, "f32", 257, 64),
                                              (64, "bf16", 200, 64), (128, "f32", 96, 32),
                                              (128, "bf16", 150, 64), (32, "bf16", 5, 16)])
def test_dense_exact_kdn_matches_oracle(dk, dtype, T, chunk):
    """Exact KDN (dense Riccati gain, then the chunkwise write): gains, o, S_T
    and P_T against the oracle's dense filter, from a random SPD P0."""
    B, H, dv = 1, 3, 32
    inp = forward_inputs(B, H, T, dk, dv, dtype=dtype, seed=95)
    rng = np.random.default_rng(96)
    X = rng.standard_normal((B, H, dk, dk)) / np.sqrt(dk)
    P0 = (X @ np.swapaxes(X, -1, -2) + 0.5 * np.eye(dk)).astype(np.float32)
    say(f"[gpu] exact KDN dk={dk} {dtype} T={T}")
    t = forward_tensors(inp)
    o, S_T, P_T = kdn.forward_dense(t["q"], t["k"], t["v"], t["a"], t["nu"], t["r"],
                                    torch.from_numpy(P0).cuda(), t["S0"], chunk=chunk)
    w, _ = kdn.dense_gain(t["k"], t["a"], t["nu"], t["r"], torch.from_numpy(P0).cuda(),
                          want_P=False)
    torch.cuda.synchronize()
    ref = oracle.forward_dense(inp["q"], inp["k"], inp["v"], inp["a"], inp["nu"], inp["r"], P0,
                               inp["S0"], debug=True)
    e_w = normwise(host(w), ref["w"])
    e_o = normwise(host(o), ref["o"])
    e_s = normwise(host(S_T), ref["S_T"])
    e_p = normwise(host(P_T), ref["P_T"])
    say(f"    err w {e_w:.2e}  o {e_o:.2e}  S_T {e_s:.2e}  P_T {e_p:.2e}")
    tol = _tol(dtype)
    assert e_w <= tol and e_o <= tol and e_s <= tol and e_p <= 1e-4


def test_dense_exact_kdn_empty_sequence_keeps_prior():
    """T = 0: no gains, P_T equals P0 (identity when P0 is omitted)."""
    say("[gpu] exact KDN T=0")
    k = torch.empty((2, 2, 0, 64), device="cuda")
    g = torch.empty((2, 2, 0), device="cuda")
    P0 = torch.randn((2, 2, 64, 64), device="cuda")
    w, P_T = kdn.dense_gain(k, g, g, g, P0)
    _, P_I = kdn.dense_gain(k, g, g, g, None)
    torch.cuda.synchronize()
    assert w.numel() == 0
    assert torch.equal(P_T, P0)
    assert torch.equal(P_I, torch.eye(64, device="cuda").expand(2, 2, 64, 64))


@pytest.mark.parametrize("dk", [32, 128])
def test_dense_exact_kdn_extreme_decays(dk):
    """Decays of 1e-6 (the running scale of the covariance is folded back on
    that token), 1e-3 and exactly one, against the oracle's dense filter."""
    B, H, T, dv = 1, 2, 64, 32
    inp = forward_inputs(B, H, T, dk, dv, dtype="f32", seed=97)
    rng = np.random.default_rng(98)
    a = rng.uniform(0.02, 1.0, (B, H, T)).astype(np.float32)
    a[..., ::7] = 1e-6
    a[..., 1::9] = 1e-3
    a[..., 2::11] = 1.0
    inp["a"] = a
    say(f"[gpu] exact KDN extreme decays dk={dk}")
    t = forward_tensors(inp)
    o, S_T, P_T = kdn.forward_dense(t["q"], t["k"], t["v"], t["a"], t["nu"], t["r"], None,
                                    t["S0"], chunk=32)
    torch.cuda.synchronize()
    ref = oracle.forward_dense(inp["q"], inp["k"], inp["v"], inp["a"], inp["nu"], inp["r"], None,
                               inp["S0"])
    e_o, e_s, e_p = (normwise(host(x), ref[n]) for x, n in ((o, "o"), (S_T, "S_T"), (P_T, "P_T")))
    say(f"    err o {e_o:.2e}  S_T {e_s:.2e}  P_T {e_p:.2e}")
    assert e_o <= TOL_F32 and e_s <= TOL_F32 and e_p <= 1e-4


def test_dense_exact_kdn_workload_bf16_B8_H16_T4096_d128_all_heads():
    """The exact forward at the layer workload's full size, in the launch
    configuration the benchmark times (P0 = I, chunk 64); every head against
    the oracle's dense filter."""
    say("[gpu] generating workload 2 for the exact filter")
    inp = cached_config(2)
    t = forward_tensors(inp)
    say(f"[gpu] exact forward full size {inp['q'].shape}")
    o, S_T, P_T = kdn.forward_dense(t["q"], t["k"], t["v"], t["a"], t["nu"], t["r"], None,
                                    t["S0"], chunk=64)
    torch.cuda.synchronize()
    o, S_T, P_T = host(o), host(S_T), host(P_T)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(P_T))
    say("[cpu] dense oracle on all heads")
    ref = oracle.forward_dense(inp["q"], inp["k"], inp["v"], inp["a"], inp["nu"], inp["r"],
                               None, inp["S0"])
    e_o = normwise(o, ref["o"])
    e_s = normwise(S_T, ref["S_T"])
    e_p = normwise(P_T, ref["P_T"])
    say(f"    all heads: err o {e_o:.2e}  S_T {e_s:.2e}  P_T {e_p:.2e}")
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16 and e_p <= 1e-4
