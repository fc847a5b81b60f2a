"""A seeded sweep of forward shapes on the GPU against the fp64 oracle,
through the C ABI: batch and head counts, lengths around and between chunk
boundaries, every supported (d_k, d_v) pair, the three chunk sizes, both
variants and both input dtypes, drawn once from a fixed seed.  The few
combinations the chunk kernels do not take (float32 inputs with d_k = 128 and
64-token chunks: their LDS) are checked to be refused instead.  Bars as in the
other parity tests: o and S_T normwise per (b, h) within 1e-4 (float32) or
2e-2 (bfloat16), lambda_T within 1e-5.  The backward is swept the same way
against the oracle's vector-Jacobian product, and the packed variable-length
forward over random mixes of sequence lengths, sequence by sequence."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import kalman_filter_memory_amd as kdn
import oracle
from gpu_util import TOL_BF16, TOL_F32, TOL_LAMBDA, elementwise, forward_tensors, host, normwise, say
from kdn_inputs import forward_inputs

pytestmark = pytest.mark.gpu


def _cases(n=32, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        C = int(rng.choice([16, 32, 64]))
        # lengths: short, just below / at / above a chunk multiple, or several chunks
        kind = int(rng.integers(0, 4))
        m = int(rng.integers(1, 9))
        T = {0: int(rng.integers(1, C)), 1: m * C - 1, 2: m * C, 3: m * C + int(rng.integers(1, C))}[kind]
        out.append((int(rng.integers(1, 4)), int(rng.integers(1, 5)), T,
                    int(rng.choice([32, 64, 128])), int(rng.choice([32, 64, 128])), C,
                    str(rng.choice(["diagonal", "isotropic"])), str(rng.choice(["f32", "bf16"]))))
    return out


CASES = _cases()


@pytest.mark.parametrize("idx", range(len(CASES)),
                         ids=["B{}H{}T{}k{}v{}C{}_{}_{}".format(*c) for c in CASES])
def test_forward_sweep_matches_oracle(idx):
    case = CASES[idx]
    B, H, T, dk, dv, C, variant, dtype = case
    code = kdn.BF16 if dtype == "bf16" else kdn.F32
    d = kdn.make_desc(B, H, T, dk, dv, C, variant, code, code)
    st = kdn.validate(d)
    if dtype == "f32" and dk == 128 and C == 64:
        assert st == 3  # KDN_ERR_UNSUPPORTED: refused on the host, nothing launched
        return
    assert st == 0
    inp = forward_inputs(B, H, T, dk, dv, variant=variant, dtype=dtype, seed=5000 + idx)
    say(f"[gpu] sweep forward {case}")
    t = forward_tensors(inp)
    o, S_T, lam = kdn.forward(t["q"], t["k"], t["v"], t["a"], t["nu"], t["r"], t["lambda0"],
                              t["S0"], variant=variant, chunk=C)
    torch.cuda.synchronize()
    ref = oracle.forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["nu"], inp["r"],
                         inp["lambda0"], inp["S0"], variant)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    e_o = normwise(host(o), ref["o"])
    e_s = normwise(host(S_T), ref["S_T"])
    e_l = elementwise(host(lam), ref["lambda_T"])
    say(f"    err o {e_o:.2e}  S_T {e_s:.2e}  lambda_T {e_l:.2e}  (tol {tol:g}, {TOL_LAMBDA:g})")
    assert np.all(np.isfinite(host(o)))
    assert e_o <= tol and e_s <= tol and e_l <= TOL_LAMBDA


BWD_CASES = _cases(n=20, seed=20261205)


def _bwd_supported(B, H, T, dk, dv, C, variant, code):
    d = kdn.make_desc(B, H, T, dk, dv, C, variant, code, code)
    return kdn.load_library().kdn_backward_workspace_bytes(ctypes.byref(d)) > 0


@pytest.mark.parametrize("idx", range(len(BWD_CASES)),
                         ids=["B{}H{}T{}k{}v{}C{}_{}_{}".format(*c) for c in BWD_CASES])
def test_backward_sweep_matches_oracle(idx):
    """The backward over the same kind of sweep against the oracle's
    vector-Jacobian product (bars of the backward parity tests); a shape the
    backward kernels do not take is refused before any launch."""
    from test_gpu_backward import _assert, _errors, _gpu_backward, _oracle_backward
    from kdn_inputs import backward_cotangents

    case = BWD_CASES[idx]
    B, H, T, dk, dv, C, variant, dtype = case
    code = kdn.BF16 if dtype == "bf16" else kdn.F32
    inp = forward_inputs(B, H, T, dk, dv, variant=variant, dtype=dtype, seed=6000 + idx)
    cot = backward_cotangents(B, H, T, dk, dv, variant=variant, dtype=dtype, seed=6100 + idx)
    if not _bwd_supported(B, H, T, dk, dv, C, variant, code):
        say(f"[gpu] sweep backward {case}: not taken by the backward kernels, refused")
        with pytest.raises(kdn.KdnError):
            _gpu_backward(inp, cot, C)
        return
    say(f"[gpu] sweep backward {case}")
    got = _gpu_backward(inp, cot, C)
    ref = _oracle_backward(inp, cot)
    _assert(_errors(got, ref), dtype)


def _varlen_cases(n=10, seed=20261206):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        C = int(rng.choice([16, 32, 64]))
        N = int(rng.integers(1, 7))
        # lengths: empty, single tokens, ragged, chunk multiples, several chunks
        lens = [int(rng.choice([0, 1, C - 1, C, C + 1, 3 * C + 5, int(rng.integers(2, 400))]))
                for _ in range(N)]
        dtype = str(rng.choice(["f32", "bf16"]))
        dk = int(rng.choice([32, 64] if (dtype == "f32" and C == 64) else [32, 64, 128]))
        out.append((tuple(lens), int(rng.integers(1, 4)), dk, int(rng.choice([32, 64, 128])), C,
                    str(rng.choice(["diagonal", "isotropic"])), dtype))
    return out


VARLEN_CASES = _varlen_cases()


@pytest.mark.parametrize("idx", range(len(VARLEN_CASES)),
                         ids=["L{}_H{}k{}v{}C{}_{}_{}".format("-".join(map(str, c[0])), *c[1:])
                              for c in VARLEN_CASES])
def test_forward_varlen_sweep_matches_oracle_per_sequence(idx):
    """Packed batches of random length mixes (the serving prefill): each
    sequence's o, S_T and lambda_T equal the oracle's for that sequence alone."""
    lens, H, dk, dv, C, variant, dtype = VARLEN_CASES[idx]
    N, T = len(lens), sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    say(f"[gpu] sweep forward_varlen {variant} {dtype} C={C} H={H} d_k={dk} d_v={dv} lens={list(lens)}")
    inp = forward_inputs(1, H, T, dk, dv, variant=variant, dtype=dtype, seed=7000 + idx)
    init = forward_inputs(N, H, 1, dk, dv, variant=variant, dtype=dtype, seed=7100 + idx)
    t = forward_tensors(inp)
    lam0 = torch.from_numpy(init["lambda0"]).cuda()
    S0 = torch.from_numpy(init["S0"]).cuda()
    o, S_T, lam_T = kdn.forward_varlen(t["q"][0], t["k"][0], t["v"][0], t["a"][0], t["nu"][0],
                                       t["r"][0], torch.from_numpy(cu).cuda(), max(max(lens), 1),
                                       lam0, S0, variant=variant, chunk=C)
    torch.cuda.synchronize()
    o_h, S_h, l_h = host(o), host(S_T), host(lam_T)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
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
