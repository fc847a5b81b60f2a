"""The forward and the decode step captured in a HIP graph (torch.cuda.graph
around the binding, which launches on torch's current stream, the capture
stream there) and replayed: every replay equals the eager call bit for bit
(same kernels, same inputs), with eager work and synchronisations of the
program's own between the replays.  The library records nothing but kernel
launches (no memsets, allocations or synchronisations), so a captured forward
is its four kernels (six with the segmented state pass); the backward and
the layer (whose GEMMs hipBLASLt records) are captured the same way."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import kalman_filter_memory_amd as kdn
import oracle
from gpu_util import TOL_BF16, TOL_LAMBDA, forward_tensors, host, normwise, say
from kdn_inputs import decode_inputs, forward_inputs, layer_inputs

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _outputs_like(ref):
    return tuple(torch.empty_like(x) for x in ref)


def _poison(outs):
    for x in outs:
        x.fill_(float("nan"))


# (variant, B, H, T, d_k, d_v, noalloc): the layer-shaped kernels, the isotropic
# scan and prep, the segmented state pass (few heads, many chunks: maps pass,
# composition and read-out pass), and the allocation-free entry point
CASES = [
    ("diagonal", 2, 4, 1000, 128, 128, False),
    ("isotropic", 2, 4, 1000, 128, 128, False),
    ("diagonal", 1, 2, 4096, 128, 64, False),
    ("diagonal", 2, 4, 1000, 128, 128, True),
]


@pytest.mark.parametrize("variant,B,H,T,dk,dv,noalloc", CASES)
def test_forward_graph_replays_equal_eager(variant, B, H, T, dk, dv, noalloc):
    inp = forward_inputs(B, H, T, dk, dv, variant=variant, dtype="bf16", seed=911)
    other = forward_inputs(B, H, T, dk, dv, variant=variant, dtype="bf16", seed=912)
    say(f"[gpu] graph forward: {variant} B{B} H{H} T{T} d_k {dk} d_v {dv} noalloc={noalloc}")
    t = forward_tensors(inp)
    t2 = forward_tensors(other)
    args = (t["q"], t["k"], t["v"], t["a"], t["nu"], t["r"], t["lambda0"], t["S0"])
    args2 = (t2["q"], t2["k"], t2["v"], t2["a"], t2["nu"], t2["r"], t2["lambda0"], t2["S0"])
    fwd = kdn.forward_noalloc if noalloc else kdn.forward
    d = kdn.make_desc(B, H, T, dk, dv, 64, variant, kdn.BF16, kdn.BF16)
    if (B, H, T) == (1, 2, 4096):
        assert kdn.forward_segments(d) > 1  # the case exercises the segmented pass

    ref = fwd(*args, variant=variant, chunk=64)
    torch.cuda.synchronize()
    outs = _outputs_like(ref)
    kw = {} if noalloc else {
        "workspace": torch.empty(kdn.forward_workspace_bytes(d), dtype=torch.uint8,
                                 device="cuda")}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(*args, variant=variant, chunk=64, out=outs, **kw)
    other_outs = _outputs_like(ref)
    for i in range(REPLAYS):
        _poison(outs)
        g.replay()
        # eager work of the program's own between replays (a forward on other
        # inputs; for the allocation-free call it reuses the same static array)
        fwd(*args2, variant=variant, chunk=64, out=other_outs)
        torch.cuda.synchronize()
        for name, x, y in zip(("o", "S_T", "lambda_T"), outs, ref):
            assert torch.equal(x, y), f"replay {i}: {name} differs from the eager call"
    # and the eager result itself against the oracle
    ro = oracle.forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["nu"], inp["r"],
                        inp["lambda0"], inp["S0"], variant)
    eo = normwise(host(outs[0]), ro["o"])
    es = normwise(host(outs[1]), ro["S_T"])
    el = float((np.abs(host(outs[2]) - ro["lambda_T"]) / ro["lambda_T"]).max())
    say(f"        replayed o {eo:.2e}, S_T {es:.2e}, lambda {el:.2e} against the oracle")
    assert eo <= TOL_BF16 and es <= TOL_BF16 and el <= TOL_LAMBDA


def test_decode_graph_replays_equal_eager_steps():
    """One decode step captured once and replayed for consecutive tokens: each
    replay advances the cache in place exactly as the eager steps do."""
    N, H, d = 64, 16, 128
    inp = decode_inputs(N, H, d, d, steps=REPLAYS, seed=913)
    say(f"[gpu] graph decode: {N} sequences x {H} heads, d {d}, {REPLAYS} steps")
    S_e = torch.from_numpy(inp["S0"]).cuda()
    lam_e = torch.from_numpy(inp["lambda0"]).cuda()
    S_g, lam_g = S_e.clone(), lam_e.clone()
    # q, k, v in bf16 and the gates in float32, as drawn
    dt = {"q": torch.bfloat16, "k": torch.bfloat16, "v": torch.bfloat16,
          "a": torch.float32, "nu": torch.float32, "r": torch.float32}
    toks = [{n: torch.from_numpy(np.ascontiguousarray(inp[n][s], np.float32)).cuda().to(dt[n])
             for n in dt} for s in range(REPLAYS)]
    eager_o = []
    for s in range(REPLAYS):
        x = toks[s]
        eager_o.append(kdn.decode_step(x["q"], x["k"], x["v"], x["a"], x["nu"], x["r"], S_e,
                                       lam_e).clone())
    torch.cuda.synchronize()
    # the graph reads the token from fixed buffers, refilled before each replay
    cur = {n: torch.empty_like(toks[0][n]) for n in toks[0]}
    o_g = torch.empty_like(eager_o[0])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kdn.decode_step(cur["q"], cur["k"], cur["v"], cur["a"], cur["nu"], cur["r"], S_g, lam_g,
                        out=o_g)
    for s in range(REPLAYS):
        for n in cur:
            cur[n].copy_(toks[s][n])
        o_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, eager_o[s]), f"step {s}: o differs from the eager step"
    assert torch.equal(S_g, S_e) and torch.equal(lam_g, lam_e)


@pytest.mark.parametrize("variant", ["diagonal", "isotropic"])
def test_backward_graph_replays_equal_eager(variant):
    """The backward (recompute and the three gradient stages) captured and
    replayed: every gradient equals the eager call's bit for bit."""
    B, H, T, dk, dv = 2, 2, 300, 128, 64
    inp = forward_inputs(B, H, T, dk, dv, variant=variant, dtype="bf16", seed=914)
    say(f"[gpu] graph backward: {variant} B{B} H{H} T{T} d_k {dk} d_v {dv}")
    t = forward_tensors(inp)
    gen = torch.Generator(device="cpu").manual_seed(915)
    dO = torch.randn((B, H, T, dv), generator=gen).cuda().to(torch.bfloat16)
    args = (t["q"], t["k"], t["v"], t["a"], t["nu"], t["r"], dO)
    kw = dict(lambda0=t["lambda0"], S0=t["S0"], variant=variant, chunk=64)
    ref = kdn.backward(*args, **kw)
    torch.cuda.synchronize()
    d = kdn.make_desc(B, H, T, dk, dv, 64, variant, kdn.BF16, kdn.BF16)
    lib = kdn.load_library()
    ws = torch.empty(lib.kdn_backward_workspace_bytes(ctypes.byref(d)), dtype=torch.uint8,
                     device="cuda")
    out = {n: torch.empty_like(x) for n, x in ref.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kdn.backward(*args, **kw, workspace=ws, out=out)
    for i in range(REPLAYS):
        for x in out.values():
            x.fill_(float("nan"))
        g.replay()
        kdn.backward(*args, **kw)  # eager work between the replays
        torch.cuda.synchronize()
        for n in ref:
            assert torch.equal(out[n], ref[n]), f"replay {i}: {n} differs from the eager call"


def test_layer_graph_replays_equal_eager():
    """The layer (two hipBLASLt GEMMs around the library's kernels) captured
    after one eager call with the same shapes (which chooses and keeps the
    GEMM algorithms) and replayed: y, S_T and lambda_T equal the eager call's."""
    p = layer_inputs(1, 200, 2, 128, 64, 64, dtype="bf16", seed=916)
    say("[gpu] graph layer: B1 T200 H2 D128 d 64 bf16")
    bf = torch.bfloat16
    x = torch.from_numpy(p["x"]).cuda().to(bf)
    W_in = torch.from_numpy(np.ascontiguousarray(p["W_in"].T)).cuda().to(bf)
    W_out = torch.from_numpy(np.ascontiguousarray(p["W_out"].T)).cuda().to(bf)
    b, lam0, S0 = (torch.from_numpy(p[n]).cuda() for n in ("b_gate", "lambda0", "S0"))
    ref = kdn.layer_forward(x, W_in, b, W_out, 2, 64, 64, lam0, S0)
    torch.cuda.synchronize()
    d = kdn.make_layer_desc(1, 200, 2, 128, 64, 64, 64, "diagonal", kdn.BF16)
    ws = torch.empty(kdn.layer_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        got = kdn.layer_forward(x, W_in, b, W_out, 2, 64, 64, lam0, S0, workspace=ws)
    for i in range(REPLAYS):
        for y in got:
            y.fill_(float("nan"))
        g.replay()
        kdn.layer_forward(x, W_in, b, W_out, 2, 64, 64, lam0, S0)
        torch.cuda.synchronize()
        for name, a_, b_ in zip(("y", "S_T", "lambda_T"), got, ref):
            assert torch.equal(a_, b_), f"replay {i}: {name} differs from the eager call"
