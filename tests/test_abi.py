"""Host-side checks of libkdn: the library loads, exports every function that
include/kdn.h declares, and validates descriptors and arguments on the host
before any GPU work (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import kalman_filter_memory_amd as kdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "kdn.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kdn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kdn.LIB_PATH):
        from kalman_filter_memory_amd import build
        build.build()
    return kdn.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(kdn.EXPORTS)


def _desc(**kw):
    base = dict(B=2, H=4, T=100, d_k=64, d_v=64, chunk=64, variant="diagonal",
                qkv_dtype=kdn.BF16, gate_dtype=kdn.BF16)
    base.update(kw)
    return kdn.make_desc(base["B"], base["H"], base["T"], base["d_k"], base["d_v"],
                         base["chunk"], base["variant"], base["qkv_dtype"], base["gate_dtype"])


def test_validate_accepts_supported_and_rejects_the_rest(lib):
    assert kdn.validate(_desc()) == 0
    for dk in (32, 64, 128):
        for dv in (32, 64, 128):
            for c in (16, 32, 64):
                assert kdn.validate(_desc(d_k=dk, d_v=dv, chunk=c)) == 0
    assert kdn.validate(_desc(d_k=128, chunk=64, qkv_dtype=kdn.F32)) == 3  # LDS budget
    assert kdn.validate(_desc(d_k=128, chunk=32, qkv_dtype=kdn.F32)) == 0
    assert kdn.validate(_desc(d_k=48)) == 3
    assert kdn.validate(_desc(chunk=128)) == 3
    assert kdn.validate(_desc(chunk=24)) == 3
    assert kdn.validate(_desc(T=-1)) == 2
    assert kdn.validate(_desc(B=-2)) == 2
    assert kdn.validate(_desc(B=300, H=300)) == 3  # heads index grid.y
    d = _desc()
    d.variant = 7
    assert kdn.validate(d) == 3
    d = _desc()
    d.qkv_dtype = 5
    assert kdn.validate(d) == 3
    assert lib.kdn_validate(None) == 1


def test_workspace_sizes(lib):
    d = _desc(B=8, H=16, T=4096, d_k=128, d_v=128, chunk=64)
    ws = kdn.forward_workspace_bytes(d)
    bh, nc = 128, 64
    expect = (bh * nc * 4 * 128 * 16 + bh * (nc + 1) * 128 * 4 + bh * 4096 * 128 * 2
              + bh * nc * 64 * 64 * 2 + bh * nc * 64 * 4)
    assert expect <= ws <= expect + 5 * 256
    assert kdn.forward_workspace_bytes(_desc(d_k=48)) == 0
    assert lib.kdn_mobius_scan_workspace_bytes(ctypes.byref(d)) < ws
    assert lib.kdn_chunk_delta_workspace_bytes(ctypes.byref(d)) == bh * nc * 64 * 64 * 2 + bh * nc * 64 * 4


def test_status_strings(lib):
    for code in range(7):
        s = kdn.status_string(code)
        assert isinstance(s, str) and s
    assert "unknown" in kdn.status_string(99)


def test_host_side_errors_return_before_any_launch(lib):
    d = _desc()
    fake = ctypes.c_void_p(0x1000)
    ws = ctypes.c_void_p(0x2000)
    need = kdn.forward_workspace_bytes(d)
    P = lambda: fake
    # NULL descriptor
    assert lib.kdn_forward(None, *([fake] * 11), ws, need, None) == 1
    # missing input pointer
    assert lib.kdn_forward(ctypes.byref(d), None, *([fake] * 10), ws, need, None) == 1
    # workspace too small
    assert lib.kdn_forward(ctypes.byref(d), *([fake] * 11), ws, need - 1, None) == 4
    # misaligned q
    assert lib.kdn_forward(ctypes.byref(d), ctypes.c_void_p(0x1002), *([fake] * 10), ws, need,
                           None) == 5
    # unsupported size
    bad = _desc(d_k=40)
    assert lib.kdn_forward(ctypes.byref(bad), *([fake] * 11), ws, need, None) == 3
    # decode: NULL state
    dd = _desc(T=1, chunk=0)
    assert lib.kdn_decode_step(ctypes.byref(dd), *([fake] * 6), None, fake, fake, None) == 1
    assert lib.kdn_decode_step(ctypes.byref(_desc(d_v=96)), *([fake] * 9), None) == 3
    # chunk_delta needs gain dtype == qkv dtype
    g = _desc()
    g.gain_dtype = kdn.F32
    assert lib.kdn_chunk_delta(ctypes.byref(g), *([fake] * 8), ws, 1 << 30, None) == 3
    # the repeat timing aid: kernel index, repeat count and aliasing outputs
    # are refused, and its other checks are the forward's
    rep = lib.kdn_forward_repeat
    c = ctypes.c_void_p
    # q k v a nu r, then lambda0, S0, o, S_T, lambda_T at distinct addresses
    ok = [fake] * 6 + [c(0x3000), c(0x4000), c(0x5000), c(0x6000), c(0x7000)]
    assert rep(ctypes.byref(d), *ok, ws, need, None, 0, 4, 1) == 2
    assert rep(ctypes.byref(d), *ok, ws, need, None, -1, 3, 1) == 2
    assert rep(ctypes.byref(d), *ok, ws, need, None, 2, 1, 1) == 2
    assert rep(ctypes.byref(d), *ok, ws, need, None, 3, 3, -1) == 2
    assert rep(ctypes.byref(d), *(ok[:9] + [ok[7], ok[10]]), ws, need, None, 3, 3, 1) == 2
    assert rep(ctypes.byref(d), *(ok[:10] + [ok[6]]), ws, need, None, 0, 1, 1) == 2
    assert rep(ctypes.byref(d), *ok, ws, need - 1, None, 0, 3, 1) == 4
    assert rep(ctypes.byref(d), None, *ok[1:], ws, need, None, 0, 0, 1) == 1
    # empty problems are a no-op success without touching the GPU
    e = _desc(B=0)
    assert lib.kdn_forward(ctypes.byref(e), *([None] * 11), None, 0, None) == 0
    assert lib.kdn_decode_step(ctypes.byref(_desc(B=0, T=1)), *([None] * 9), None) == 0
    _ = P


def test_backward_host_side_checks(lib):
    """kdn_backward: workspace query and argument errors, all before any launch."""
    fake = ctypes.c_void_p(0x1000)
    ws = ctypes.c_void_p(0x2000)
    d = _desc(B=8, H=16, T=4096, d_k=128, d_v=128, chunk=64)
    need = kdn.backward_workspace_bytes(d)
    bh, nc, n = 128, 64, 8 * 16 * 4096
    # forward workspace, then 1/D, chunk-start states and chunk-end adjoints
    # (bf16), dW (bf16), s, d(ln a), chunk maps and G
    states = bh * nc * 128 * 128 * 2
    expect = (kdn.forward_workspace_bytes(d) + n * 4 + 2 * states + n * 128 * 2 + 2 * n * 4
              + bh * nc * 128 * 12)
    assert expect <= need <= expect + 9 * 256
    iso = _desc(B=1, H=1, T=16, d_k=32, d_v=32, chunk=16)
    iso.variant = kdn.ISOTROPIC
    assert kdn.backward_workspace_bytes(iso) > 0
    bad = _desc(d_k=48)
    assert kdn.backward_workspace_bytes(bad) == 0
    args = [fake] * 19
    assert lib.kdn_backward(ctypes.byref(bad), *args, ws, 1 << 40, None) == 3
    assert lib.kdn_backward(ctypes.byref(d), None, *args[1:], ws, need, None) == 1
    assert lib.kdn_backward(ctypes.byref(d), *args, ws, need - 1, None) == 4
    assert lib.kdn_backward(ctypes.byref(d), *args[:9], ctypes.c_void_p(0x1004), *args[10:],
                            ws, need, None) == 5
    assert lib.kdn_backward(ctypes.byref(_desc(B=0)), *([None] * 19), None, 0, None) == 0


def test_dense_gain_host_side_checks(lib):
    """kdn_dense_gain: unsupported d_k and mixed gain dtype are refused before
    any launch; no heads is a no-op."""
    fake = ctypes.c_void_p(0x1000)
    args = [fake] * 4 + [None, fake, None]
    assert lib.kdn_dense_gain(ctypes.byref(_desc(d_k=48)), *args, None) == 3
    mixed = _desc(d_k=64)
    mixed.gain_dtype = kdn.F32
    assert lib.kdn_dense_gain(ctypes.byref(mixed), *args, None) == 3
    assert lib.kdn_dense_gain(ctypes.byref(_desc(d_k=64)), None, *args[1:], None) == 1
    odd = [ctypes.c_void_p(0x1002)] + args[1:]
    assert lib.kdn_dense_gain(ctypes.byref(_desc(d_k=64)), *odd, None) == 5
    assert lib.kdn_dense_gain(ctypes.byref(_desc(B=0, d_k=64)), *([None] * 7), None) == 0


def test_layer_host_side_checks(lib):
    """kdn_layer_workspace_bytes: the documented layout at the layer workload
    (Z, q, k, v, the three gates, o, the GEMMs' 32 MiB and the recurrence's
    workspace); 0 for shapes the layer does not take; argument errors before
    any launch."""
    d = kdn.make_layer_desc(8, 4096, 16, 2048, 128, 128, 64, "diagonal", kdn.BF16)
    need = kdn.layer_workspace_bytes(d)
    M, BH, T = 8 * 4096, 128, 4096
    n_in = 16 * (2 * 128 + 128) + 48
    ldz = (n_in + 15) // 16 * 16
    core = kdn.forward_workspace_bytes(_desc(B=8, H=16, T=4096, d_k=128, d_v=128, chunk=64))
    expect = (M * ldz * 2 + 2 * BH * T * 128 * 2 + BH * T * 128 * 2 + 3 * BH * T * 2
              + BH * T * 128 * 2 + (32 << 20) + core)
    assert expect <= need <= expect + 10 * 256
    assert kdn.layer_workspace_bytes(
        kdn.make_layer_desc(1, 16, 2, 100, 32, 32, 16, "diagonal", kdn.F32)) == 0
    assert kdn.layer_workspace_bytes(
        kdn.make_layer_desc(1, 16, 90, 64, 32, 32, 16, "diagonal", kdn.F32)) == 0
    assert kdn.layer_workspace_bytes(
        kdn.make_layer_desc(1, 16, 2, 64, 48, 32, 16, "diagonal", kdn.F32)) == 0
    assert kdn.layer_workspace_bytes(
        kdn.make_layer_desc(1 << 16, 1 << 16, 2, 64, 32, 32, 16, "diagonal", kdn.F32)) == 0
    fake = ctypes.c_void_p(0x1000)
    args = [fake] * 4 + [None, None, fake, None, None, fake]
    small = kdn.make_layer_desc(1, 16, 2, 64, 32, 32, 16, "diagonal", kdn.F32)
    n = kdn.layer_workspace_bytes(small)
    assert lib.kdn_layer_forward(ctypes.byref(small), None, *args, n, None) == 1
    assert lib.kdn_layer_forward(ctypes.byref(small), fake, *args, n - 1, None) == 4
    odd = [ctypes.c_void_p(0x1004)] + args[1:]
    assert lib.kdn_layer_forward(ctypes.byref(small), fake, *odd, n, None) == 5
    none = kdn.make_layer_desc(0, 16, 2, 64, 32, 32, 16, "diagonal", kdn.F32)
    assert lib.kdn_layer_forward(ctypes.byref(none), None, *([None] * 10), 0, None) == 0


def test_smoke_cases_are_supported(lib):
    """The smoke check's forward calls are shapes the library builds."""
    import __graft_entry__ as g
    for variant, dtype, _, chunk in g.SMOKE_CASES:
        code = kdn.BF16 if dtype == "bf16" else kdn.F32
        d = kdn.make_desc(2, 2, 150, 128, 64, chunk, variant, code, code)
        assert kdn.validate(d) == 0, (variant, dtype, chunk)


def test_python_binding_refuses_cpu_tensors(lib):
    import torch
    x = torch.zeros(1, 1, 4, 32)
    g = torch.ones(1, 1, 4)
    with pytest.raises(kdn.KdnError):
        kdn.forward(x, x, x, g, g, g)


def test_state_pass_segments_follow_the_head_count(lib):
    """Enough heads to fill the GPU: one sequential pass.  Few heads with many
    chunks: the pass is cut into the segment count with the least estimated
    time (at B1 H16 T65536: segment 0 beside two rounds of the other segments'
    maps on 224 CUs, one read-out round on 256, hence 9), and the workspace
    grows by the segments' start states and maps (fp32)."""
    big = _desc(B=8, H=16, T=4096, d_k=128, d_v=128, chunk=64)
    assert kdn.forward_segments(big) == 1
    long = _desc(B=1, H=16, T=65536, d_k=128, d_v=128, chunk=64)
    nseg = kdn.forward_segments(long)
    assert nseg == 9
    plain = 16 * 1024 * (4 * 128 * 16 + 128 * 4 + 64 * 128 * 2 + 64 * 64 * 2 + 64 * 4) + 16 * 128 * 4
    seg_bytes = 16 * nseg * (128 * 128 + 128 * 128) * 4
    assert plain + seg_bytes <= kdn.forward_workspace_bytes(long) <= plain + seg_bytes + 8 * 256
    few_chunks = _desc(B=1, H=2, T=15 * 64, d_k=64, d_v=64, chunk=64)
    assert kdn.forward_segments(few_chunks) == 1
    ragged = _desc(B=1, H=1, T=16 * 64 + 37, d_k=64, d_v=64, chunk=64)
    n = kdn.forward_segments(ragged)
    assert n == 4          # 17 chunks: segment 0 of 2, three of 5
    assert kdn.forward_segments(_desc(d_k=48)) == 0
    # the stage call (given gains) keeps the plain pass and its workspace
    assert lib.kdn_chunk_delta_workspace_bytes(ctypes.byref(long)) == 16 * 1024 * (
        64 * 64 * 2 + 64 * 4)
