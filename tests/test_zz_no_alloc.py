"""The allocation-free forward (kdn_forward_noalloc) through the C ABI: its
output equals kdn_forward's (same kernels, same inputs: bit for bit) on two
calls in a row, the second with a smaller input, and a size whose workspace
exceeds the static array is refused before anything runs."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import kalman_filter_memory_amd as kdn
from gpu_util import forward_tensors, say
from kdn_inputs import forward_inputs

pytestmark = pytest.mark.gpu


def _both(inp, chunk):
    t = forward_tensors(inp)
    args = (t["q"], t["k"], t["v"], t["a"], t["nu"], t["r"], t["lambda0"], t["S0"])
    ref = kdn.forward(*args, variant=inp["variant"], chunk=chunk)
    got = kdn.forward_noalloc(*args, variant=inp["variant"], chunk=chunk)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("variant,dtype", [("diagonal", "bf16"), ("isotropic", "f32")])
def test_noalloc_forward_equals_forward_on_two_calls(variant, dtype):
    big = forward_inputs(2, 4, 1000, 128, 64, variant=variant, dtype=dtype, seed=601)
    small = forward_inputs(1, 3, 77, 64, 32, variant=variant, dtype=dtype, seed=602)
    for label, inp in (("first", big), ("second, smaller", small)):
        say(f"[gpu] noalloc forward, {label} call: {variant} {dtype} q{inp['q'].shape}")
        ref, got = _both(inp, 32 if dtype == "f32" else 64)
        for x, y in zip(ref, got):
            assert torch.equal(x, y)


def test_noalloc_forward_refuses_a_workspace_beyond_the_array():
    lib = kdn.load_library()
    cap = lib.kdn_noalloc_scratch_bytes()
    assert cap == 320 << 20
    d = kdn.make_desc(1, 16, 65536, 128, 128, 64, "diagonal", kdn.BF16, kdn.BF16)
    assert kdn.forward_workspace_bytes(d) > cap
    # refused on the host before any pointer is touched (NULL pointers suffice)
    rc = lib.kdn_forward_noalloc(ctypes.byref(d), *([None] * 11), None)
    assert rc == 4
    d2 = kdn.make_desc(8, 16, 4096, 128, 128, 64, "diagonal", kdn.BF16, kdn.BF16)
    assert kdn.forward_workspace_bytes(d2) <= cap
