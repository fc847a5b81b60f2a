"""Pins of the fp64 oracle against what the pages and the mathematics fix.

The pages print no worked example for the KDN layer, so every pin below is a
special case, closed form, invariant or independent formulation (see
tests/textbook.py).  Each is chosen so that a plausible slip in the oracle (a
dropped noise term, a instead of a^2, the posterior instead of the predictive
gain, a sum instead of a mean in the isotropic projection, a read-out before
the write, a transposed memory) breaks at least one of them.
"""
from __future__ import annotations

import numpy as np
import pytest
import scipy.optimize

import oracle
import textbook as tb
from kdn_inputs import forward_inputs, decode_inputs

VARIANTS = ["diagonal", "isotropic"]


def _rand_gates(rng, T, a_lo=0.3):
    a = rng.uniform(a_lo, 1.0, T).astype(np.float32)
    nu = rng.uniform(0.0, 0.3, T).astype(np.float32)
    r = rng.uniform(0.2, 2.0, T).astype(np.float32)
    return a, nu, r


def _one_head(x):
    return x[None, None]


@pytest.mark.parametrize("variant", VARIANTS)
def test_scalar_kalman_filter_when_dk_is_one(variant):
    """d_k = 1: the projection is exact and both variants are the scalar Kalman filter."""
    rng = np.random.default_rng(1)
    T, dv = 40, 3
    q = rng.standard_normal(T).astype(np.float32)
    k = rng.standard_normal(T).astype(np.float32)
    v = rng.standard_normal((T, dv)).astype(np.float32)
    a, nu, r = _rand_gates(rng, T)
    lam0 = np.float32(0.7)
    s0 = rng.standard_normal(dv).astype(np.float32)
    lam_arr = np.array([[[lam0]]], np.float32) if variant == "diagonal" else np.array([[lam0]])
    out = oracle.forward(q[None, None, :, None], k[None, None, :, None], v[None, None],
                         a[None, None], nu[None, None], r[None, None], lam_arr,
                         s0[None, None, :, None], variant=variant, debug=True)
    o, m, lamT, lm, gain = tb.scalar_kalman(q, k, v, a, nu, r, float(lam0), s0)
    np.testing.assert_allclose(out["o"][0, 0], o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["S_T"][0, 0, :, 0], m, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["lambda_T"].ravel()[0], lamT, rtol=1e-12)
    np.testing.assert_allclose(out["lambda_minus"].reshape(T), lm, rtol=1e-12)
    np.testing.assert_allclose(out["w"].reshape(T), gain, rtol=1e-12, atol=1e-14)


def test_diagonal_equals_dense_kalman_on_axis_aligned_keys():
    """Axis-aligned keys keep the exact posterior precision diagonal, so Diagonal KDN
    must equal the full-covariance (dense Riccati) Kalman filter exactly."""
    rng = np.random.default_rng(2)
    T, dk, dv = 50, 6, 4
    idx = rng.integers(0, dk, T)
    scale = rng.uniform(0.5, 1.5, T) * rng.choice([-1.0, 1.0], T)
    k = np.zeros((T, dk), np.float32)
    k[np.arange(T), idx] = scale
    q = rng.standard_normal((T, dk)).astype(np.float32)
    v = rng.standard_normal((T, dv)).astype(np.float32)
    a, nu, r = _rand_gates(rng, T)
    lam0 = rng.uniform(0.5, 2.0, dk).astype(np.float32)
    S0 = rng.standard_normal((dv, dk)).astype(np.float32)
    out = oracle.forward(_one_head(q), _one_head(k), _one_head(v), _one_head(a), _one_head(nu),
                         _one_head(r), _one_head(lam0), _one_head(S0), "diagonal", debug=True)
    o, M, Sig, prior, gains = tb.dense_kalman(q, k, v, a, nu, r, lam0, S0)
    assert np.abs(Sig - np.diag(np.diag(Sig))).max() < 1e-13
    np.testing.assert_allclose(out["o"][0, 0], o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(out["S_T"][0, 0], M, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(out["lambda_T"][0, 0], 1.0 / np.diag(Sig), rtol=1e-11)
    np.testing.assert_allclose(out["lambda_minus"][0, 0],
                               1.0 / np.diagonal(prior, axis1=1, axis2=2), rtol=1e-11)
    np.testing.assert_allclose(out["w"][0, 0], gains, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("variant", VARIANTS)
def test_gain_is_posterior_precision_solve(variant):
    """Sherman-Morrison: the Kalman gain of the projected prior equals
    (Lambda^- + k k^T / r)^{-1} k / r, a dense solve with the exact one-step
    posterior precision.  Checked for general random keys at every token."""
    inp = forward_inputs(1, 2, 24, 8, 5, variant=variant, seed=3)
    out = oracle.forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["nu"], inp["r"],
                         inp["lambda0"], inp["S0"], variant, debug=True)
    for h in range(2):
        for t in range(24):
            kt = inp["k"][0, h, t].astype(np.float64)
            rt = float(inp["r"][0, h, t])
            lm = out["lambda_minus"][0, h, t]
            Lm = np.diag(lm) if variant == "diagonal" else lm * np.eye(8)
            w_ref = np.linalg.solve(Lm + np.outer(kt, kt) / rt, kt) / rt
            np.testing.assert_allclose(out["w"][0, h, t], w_ref, rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("variant", VARIANTS)
def test_projection_is_reverse_kl_optimum(variant):
    """The precision after one token is the reverse-KL (mean-field VI) projection of the
    exact one-step posterior onto diagonal / isotropic Gaussians, found here by
    numerical minimisation of the Gaussian KL divergence from its definition."""
    dk = 5
    for seed in range(4):
        inp = forward_inputs(1, 1, 1, dk, 3, variant=variant, seed=10 + seed)
        out = oracle.forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["nu"], inp["r"],
                             inp["lambda0"], inp["S0"], variant, debug=True)
        kt = inp["k"][0, 0, 0].astype(np.float64)
        rt = float(inp["r"][0, 0, 0])
        lm = out["lambda_minus"][0, 0, 0]
        Lm = np.diag(lm) if variant == "diagonal" else lm * np.eye(dk)
        Lam_post = Lm + np.outer(kt, kt) / rt
        if variant == "diagonal":
            f = lambda x: tb.gaussian_kl(np.diag(np.exp(-x)), Lam_post)
            x0 = np.zeros(dk)
        else:
            f = lambda x: tb.gaussian_kl(np.exp(-x[0]) * np.eye(dk), Lam_post)
            x0 = np.zeros(1)
        res = scipy.optimize.minimize(f, x0, method="BFGS", options={"gtol": 1e-12})
        lam_opt = np.exp(res.x)
        np.testing.assert_allclose(np.ravel(out["lambda_T"]), lam_opt, rtol=2e-6)


@pytest.mark.parametrize("variant", VARIANTS)
def test_uncertainty_recurrence_is_a_moebius_map_in_any_bracketing(variant):
    """lambda_T equals the product of per-token 2x2 Moebius matrices applied to
    lambda_0, whatever the bracketing (sequential, balanced tree, random), and each
    lambda^-_t is the predict-only Moebius map applied to lambda_{t-1}."""
    T, dk = 96, 4
    inp = forward_inputs(1, 1, T, dk, 2, variant=variant, seed=4)
    out = oracle.forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["nu"], inp["r"],
                         inp["lambda0"], inp["S0"], variant, debug=True)
    a, nu, r = (inp[n][0, 0].astype(np.float64) for n in ("a", "nu", "r"))
    k = inp["k"][0, 0].astype(np.float64)
    rng = np.random.default_rng(0)
    lanes = range(dk) if variant == "diagonal" else [None]
    for i in lanes:
        if i is None:
            b = np.sum(k * k, axis=1) / (dk * r)
            lam0 = float(inp["lambda0"][0, 0])
            lamT = float(out["lambda_T"][0, 0])
            lm = out["lambda_minus"][0, 0]
        else:
            b = k[:, i] ** 2 / r
            lam0 = float(inp["lambda0"][0, 0, i])
            lamT = float(out["lambda_T"][0, 0, i])
            lm = out["lambda_minus"][0, 0, :, i]
        mats = [tb.mobius_step(a[t], nu[t], b[t]) for t in range(T)]
        for P in (tb.compose_sequential(mats), tb.compose_tree(mats),
                  tb.compose_random(mats, rng)):
            np.testing.assert_allclose(tb.mobius_apply(P, lam0), lamT, rtol=1e-12)
        lam = lam0
        for t in range(T):
            np.testing.assert_allclose(lm[t], tb.mobius_apply(tb.mobius_predict(a[t], nu[t]), lam),
                                       rtol=1e-12)
            lam = tb.mobius_apply(mats[t], lam)


@pytest.mark.parametrize("variant", VARIANTS)
def test_fixed_point_of_constant_gates(variant):
    """Constant (a, nu, b) with nu > 0 has the stationary precision
    lambda* = [(1 + b nu - a^2) + sqrt((1 + b nu - a^2)^2 + 4 nu b a^2)] / (2 nu):
    started there, lambda stays there; started elsewhere it converges to it."""
    T, dk, dv = 400, 3, 2
    a0, nu0, r0 = 0.9, 0.05, 0.7
    kvec = np.array([0.6, -0.3, 0.74], np.float32)
    rng = np.random.default_rng(5)
    k = np.tile(kvec, (T, 1))
    if variant == "diagonal":
        b = kvec.astype(np.float64) ** 2 / np.float64(np.float32(r0))
    else:
        b = np.array([np.sum(kvec.astype(np.float64) ** 2) / (dk * np.float64(np.float32(r0)))])
    a64, nu64 = np.float64(np.float32(a0)), np.float64(np.float32(nu0))
    c = 1 + b * nu64 - a64 ** 2
    lam_star = (c + np.sqrt(c * c + 4 * nu64 * b * a64 ** 2)) / (2 * nu64)
    gates = [np.full(T, x, np.float32) for x in (a0, nu0, r0)]
    q = rng.standard_normal((T, dk)).astype(np.float32)
    v = rng.standard_normal((T, dv)).astype(np.float32)
    for start, tol in ((lam_star, 1e-12), (np.full_like(lam_star, 5.0), 1e-10)):
        lam0 = start.astype(np.float32) if variant == "diagonal" else np.float32(start[0])
        lam0 = np.asarray(lam0, np.float32).reshape((1, 1, dk) if variant == "diagonal" else (1, 1))
        out = oracle.forward(_one_head(q), _one_head(k), _one_head(v), *(map(_one_head, gates)),
                             lam0, None, variant, debug=True)
        # float32 storage of lambda0 perturbs the start by ~1e-7; the map is a
        # contraction in log space so the end state is within rounding of lambda*.
        np.testing.assert_allclose(np.ravel(out["lambda_T"]), lam_star, rtol=max(tol, 1e-9))


@pytest.mark.parametrize("variant", VARIANTS)
def test_no_decay_no_process_noise_accumulates_evidence(variant):
    """a = 1, nu = 0: lambda_T = lambda_0 + sum_t b_t (pure accumulation of evidence)."""
    T, dk = 64, 5
    inp = forward_inputs(1, 1, T, dk, 2, variant=variant, seed=6)
    inp["a"][:] = 1.0
    inp["nu"][:] = 0.0
    out = oracle.forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["nu"], inp["r"],
                         inp["lambda0"], inp["S0"], variant)
    k = inp["k"][0, 0].astype(np.float64)
    r = inp["r"][0, 0].astype(np.float64)
    if variant == "diagonal":
        expect = inp["lambda0"][0, 0].astype(np.float64) + np.sum(k * k / r[:, None], axis=0)
    else:
        expect = float(inp["lambda0"][0, 0]) + np.sum(np.sum(k * k, 1) / (dk * r))
    np.testing.assert_allclose(np.ravel(out["lambda_T"]), np.ravel(expect), rtol=1e-13)


@pytest.mark.parametrize("variant", VARIANTS)
def test_uncertainty_invariants(variant):
    """lambda^- < 1/nu (prediction adds variance nu), b <= lambda_t < 1/nu + b, and
    lambda, lambda^-, w do not depend on v, q or S0."""
    T, dk, dv = 128, 8, 6
    inp = forward_inputs(2, 2, T, dk, dv, variant=variant, seed=7)
    out = oracle.forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["nu"], inp["r"],
                         inp["lambda0"], inp["S0"], variant, debug=True)
    nu = inp["nu"].astype(np.float64)
    lm = out["lambda_minus"]
    bound = (1.0 / nu)[..., None] if variant == "diagonal" else 1.0 / nu
    assert np.all(lm < bound)
    assert np.all(lm > 0)
    rng = np.random.default_rng(8)
    alt = oracle.forward(rng.standard_normal(inp["q"].shape), inp["k"],
                         rng.standard_normal(inp["v"].shape), inp["a"], inp["nu"], inp["r"],
                         inp["lambda0"], rng.standard_normal(inp["S0"].shape), variant,
                         debug=True)
    for name in ("lambda_T", "lambda_minus", "w"):
        np.testing.assert_array_equal(out[name], alt[name])


@pytest.mark.parametrize("variant", VARIANTS)
def test_mean_is_jointly_linear_in_values_and_initial_memory(variant):
    T, dk, dv = 50, 6, 5
    inp = forward_inputs(1, 2, T, dk, dv, variant=variant, seed=9)
    rng = np.random.default_rng(9)
    v2 = rng.standard_normal(inp["v"].shape).astype(np.float32)
    S2 = rng.standard_normal(inp["S0"].shape).astype(np.float32)
    run = lambda v, S: oracle.forward(inp["q"], inp["k"], v, inp["a"], inp["nu"], inp["r"],
                                      inp["lambda0"], S, variant)
    al, be = 0.75, -1.5
    f1 = run(inp["v"], inp["S0"])
    f2 = run(v2, S2)
    fc = run((al * inp["v"].astype(np.float64) + be * v2).astype(np.float32),
             (al * inp["S0"].astype(np.float64) + be * S2).astype(np.float32))
    # the combination is rounded to float32 on input; compare with a matching tolerance
    for name in ("o", "S_T"):
        np.testing.assert_allclose(fc[name], al * f1[name] + be * f2[name], rtol=0, atol=5e-6)


def test_isotropic_fixed_point_is_gated_delta_rule():
    """Isotropic KDN with constant (a, nu, r), unit-norm keys and lambda_0 = lambda*
    keeps a constant gain w = beta k, beta = p / (p |k|^2 + r) with p = 1/lambda^-:
    the gated delta rule with constant beta, for general (non-aligned) keys."""
    T, dk, dv = 200, 16, 8
    rng = np.random.default_rng(11)
    k = rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    k = k.astype(np.float32)
    q = rng.standard_normal((T, dk)).astype(np.float32)
    v = rng.standard_normal((T, dv)).astype(np.float32)
    S0 = rng.standard_normal((dv, dk)).astype(np.float32)
    a0, nu0, r0 = (np.float64(np.float32(x)) for x in (0.93, 0.02, 0.5))
    b = 1.0 / (dk * r0)
    c = 1 + b * nu0 - a0 ** 2
    lam_star = (c + np.sqrt(c * c + 4 * nu0 * b * a0 ** 2)) / (2 * nu0)
    p = 1.0 / (lam_star - b)
    beta = p / (p * 1.0 + r0)
    gates = [np.full(T, x, np.float32) for x in (a0, nu0, r0)]
    out = oracle.forward(_one_head(q), _one_head(k), _one_head(v), *map(_one_head, gates),
                         np.array([[lam_star]], np.float32), _one_head(S0), "isotropic")
    o_ref, S_ref = tb.gated_delta(q, k, v, gates[0].astype(np.float64), np.full(T, beta), S0)
    # |k|^2 = 1 and lambda* hold to float32 rounding only, hence the tolerance
    np.testing.assert_allclose(out["o"][0, 0], o_ref, rtol=0, atol=2e-5)
    np.testing.assert_allclose(out["S_T"][0, 0], S_ref, rtol=0, atol=2e-5)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("C", [1, 2, 4, 8, 16])
def test_chunkwise_form_equals_recurrence(variant, C):
    """The block (chunkwise) re-association reaches the token-by-token result, also
    when T is not a multiple of the chunk (tail chunk)."""
    T, dk, dv = 45, 8, 6
    inp = forward_inputs(1, 1, T, dk, dv, variant=variant, seed=12)
    out = oracle.forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["nu"], inp["r"],
                         inp["lambda0"], inp["S0"], variant, debug=True)
    o, S = tb.chunk_forward(inp["q"][0, 0], inp["k"][0, 0], inp["v"][0, 0], inp["a"][0, 0],
                            out["w"][0, 0], inp["S0"][0, 0], C)
    np.testing.assert_allclose(o, out["o"][0, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, out["S_T"][0, 0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("variant", VARIANTS)
def test_mean_update_is_information_form_posterior(variant):
    """Each token's write is the exact Bayesian posterior mean of every memory row
    under the projected Gaussian prior: s_j = (Lambda^- + k k^T/r)^{-1}
    (Lambda^- a s_j^prev + k v_j / r).  Checked for the first few tokens by running
    the oracle on growing prefixes."""
    T, dk, dv = 5, 6, 4
    inp = forward_inputs(1, 1, T, dk, dv, variant=variant, seed=13)
    prev = inp["S0"][0, 0].astype(np.float64)
    for t in range(1, T + 1):
        sl = lambda x: x[:, :, :t]
        out = oracle.forward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["a"]),
                             sl(inp["nu"]), sl(inp["r"]), inp["lambda0"], inp["S0"], variant,
                             debug=True)
        kt = inp["k"][0, 0, t - 1].astype(np.float64)
        rt = float(inp["r"][0, 0, t - 1])
        at = float(inp["a"][0, 0, t - 1])
        lm = out["lambda_minus"][0, 0, t - 1]
        Lm = np.diag(lm) if variant == "diagonal" else lm * np.eye(dk)
        Lpost = Lm + np.outer(kt, kt) / rt
        vt = inp["v"][0, 0, t - 1].astype(np.float64)
        S_ref = np.linalg.solve(Lpost, (Lm @ (at * prev).T) + np.outer(kt, vt) / rt).T
        np.testing.assert_allclose(out["S_T"][0, 0], S_ref, rtol=1e-11, atol=1e-12)
        qt = inp["q"][0, 0, t - 1].astype(np.float64)
        np.testing.assert_allclose(out["o"][0, 0, t - 1], S_ref @ qt, rtol=1e-11, atol=1e-12)
        prev = out["S_T"][0, 0]


@pytest.mark.parametrize("variant", VARIANTS)
def test_resume_from_carried_state(variant):
    T, T1 = 70, 29
    inp = forward_inputs(2, 1, T, 8, 5, variant=variant, seed=14)
    names = ("q", "k", "v", "a", "nu", "r")
    full = oracle.forward(*(inp[n] for n in names), inp["lambda0"], inp["S0"], variant)
    first = oracle.forward(*(inp[n][:, :, :T1] for n in names), inp["lambda0"], inp["S0"],
                           variant)
    second = oracle.forward(*(inp[n][:, :, T1:] for n in names),
                            first["lambda_T"].astype(np.float32),
                            first["S_T"].astype(np.float32), variant)
    # the carried state is rounded to float32 at the hand-over
    np.testing.assert_allclose(np.concatenate([first["o"], second["o"]], 2), full["o"],
                               rtol=0, atol=2e-6)
    np.testing.assert_allclose(second["S_T"], full["S_T"], rtol=0, atol=2e-6)
    np.testing.assert_allclose(second["lambda_T"], full["lambda_T"], rtol=1e-6)


@pytest.mark.parametrize("variant", VARIANTS)
def test_decode_steps_equal_forward(variant):
    N, H, dk, dv, steps = 3, 2, 8, 6, 9
    d = decode_inputs(N, H, dk, dv, steps, variant=variant, seed=15)
    S = d["S0"].astype(np.float64)
    lam = d["lambda0"].astype(np.float64)
    outs = []
    for s in range(steps):
        outs.append(oracle.decode_step(d["q"][s], d["k"][s], d["v"][s], d["a"][s], d["nu"][s],
                                       d["r"][s], S, lam, variant))
    tr = lambda x: np.moveaxis(x, 0, 2)  # [steps,N,H,...] -> [N,H,steps,...]
    full = oracle.forward(tr(d["q"]), tr(d["k"]), tr(d["v"]), tr(d["a"]), tr(d["nu"]),
                          tr(d["r"]), d["lambda0"], d["S0"], variant)
    np.testing.assert_allclose(np.stack(outs, 2), full["o"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(S, full["S_T"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lam, full["lambda_T"], rtol=1e-14)


@pytest.mark.parametrize("variant", VARIANTS)
def test_unreliable_observations_write_nothing(variant):
    """r -> infinity: the gain vanishes, the memory only decays (S_T = prod a * S0)
    and the precision follows prediction alone."""
    T = 30
    inp = forward_inputs(1, 1, T, 4, 3, variant=variant, seed=16)
    inp["r"][:] = 1e30
    out = oracle.forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["nu"], inp["r"],
                         inp["lambda0"], inp["S0"], variant, debug=True)
    assert np.abs(out["w"]).max() < 1e-25
    decay = np.prod(inp["a"][0, 0].astype(np.float64))
    np.testing.assert_allclose(out["S_T"][0, 0], decay * inp["S0"][0, 0], rtol=1e-12, atol=1e-30)
    lam = inp["lambda0"][0, 0].astype(np.float64)
    for t in range(T):
        lam = tb.mobius_apply(tb.mobius_predict(float(inp["a"][0, 0, t]), float(inp["nu"][0, 0, t])),
                              lam)
    np.testing.assert_allclose(np.ravel(out["lambda_T"]), np.ravel(lam), rtol=1e-12)


def test_variants_agree_when_dk_is_one():
    inp = forward_inputs(2, 2, 33, 1, 4, variant="diagonal", seed=17)
    names = ("q", "k", "v", "a", "nu", "r")
    d = oracle.forward(*(inp[n] for n in names), inp["lambda0"], inp["S0"], "diagonal")
    i = oracle.forward(*(inp[n] for n in names), inp["lambda0"][..., 0], inp["S0"], "isotropic")
    np.testing.assert_allclose(d["o"], i["o"], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(d["lambda_T"][..., 0], i["lambda_T"], rtol=1e-14)


def test_oracle_rejects_out_of_domain_values():
    inp = forward_inputs(1, 1, 4, 2, 2, seed=18)
    names = ("q", "k", "v", "a", "nu", "r")
    for name, bad in (("a", 0.0), ("a", 1.5), ("nu", -0.1), ("r", 0.0)):
        x = {n: inp[n].copy() for n in names}
        x[name][0, 0, 1] = bad
        with pytest.raises(ValueError):
            oracle.forward(*(x[n] for n in names), inp["lambda0"], inp["S0"], "diagonal")
    lam = inp["lambda0"].copy()
    lam[0, 0, 0] = 0.0
    with pytest.raises(ValueError):
        oracle.forward(*(inp[n] for n in names), lam, inp["S0"], "diagonal")


def test_empty_sequence_returns_initial_state():
    inp = forward_inputs(1, 2, 0, 4, 3, seed=19)
    out = oracle.forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["nu"], inp["r"],
                         inp["lambda0"], inp["S0"], "diagonal")
    assert out["o"].shape == (1, 2, 0, 3)
    np.testing.assert_array_equal(out["S_T"], inp["S0"])
    np.testing.assert_array_equal(out["lambda_T"], inp["lambda0"])
