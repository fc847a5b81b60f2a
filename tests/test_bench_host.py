"""Host-side checks of bench.py (no GPU): the refusal of several GPUs, and the
algorithmic byte counts that the roofline's achieved rate divides by, at the
layer workload (B8 H16 T4096, d 128, chunk 64, bf16)."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_forward_algorithmic_bytes_at_the_layer_workload():
    B, H, T, d, C = 8, 16, 4096, 128, 64
    by, _ = bench.algorithmic(B, H, T, d, d, C)
    n, bh, nc = B * H * T, B * H, T // C
    # keys (bf16) and three bf16 gates in, four fp32 Moebius products (4 floats
    # each: the prefixes after 16, 32, 48 and 64 tokens) per (head, chunk, key
    # dim) out
    assert by["scan_reduce"] == n * d * 2 + 3 * n * 2 + bh * nc * 4 * d * 16
    # per token-head: k 256 + gates 6 + w 256 + T 128 + g 4 + boundary precision 8
    # + three sub-block prefixes 96
    assert by["chunk_prep"] == pytest.approx(n * (256 + 6 + 256 + 128 + 4 + 8 + 96), rel=1e-3)
    # q, k, w, v 1024 + T 128 + g 4 + o 256 per token-head, plus S0 and S_T
    assert by["chunk_state"] == pytest.approx(n * (1024 + 128 + 4 + 256)
                                              + 2 * bh * d * d * 4, rel=1e-3)
    assert round(by["chunk_state"] / 1e6, 1) == 757.1


def test_backward_algorithmic_bytes_cover_every_stage():
    by, fl = bench.algorithmic_backward(8, 16, 4096, 128, 128, 64)
    assert set(by) == set(bench.BWD_STAGES)
    assert all(v > 0 for v in by.values())
    # the gradient stages move more than the forward's state pass
    assert by["bwd_grad"] > by["bwd_state"] > bench.algorithmic(8, 16, 4096, 128, 128, 64)[0][
        "chunk_state"]


def test_chunk_stage_roofline_bytes_follow_the_per_unit_figure():
    """The headline roofline divides by the chunk stage's per-unit bytes: q, k,
    v, w (bf16, 1024 B), a (2 B), o (256 B) and S0 / S_T amortised (32 B at
    T 4096): 1,314 B per token-head, 688.9 MB at the layer workload; 1,346 MB
    at the long workload (B1 H16 T65536)."""
    B, H, T, d = 8, 16, 4096, 128
    assert bench.bytes_8d(B, H, T, d, d) == B * H * T * 1314
    assert round(bench.bytes_8d(B, H, T, d, d) / 1e6, 1) == 688.9
    assert round(bench.bytes_8d(1, 16, 65536, d, d) / 1e6) == 1346


def test_isotropic_scan_bytes_hold_one_precision_per_chunk():
    by_d, _ = bench.algorithmic(1, 16, 65536, 128, 128, 64, "diagonal")
    by_i, _ = bench.algorithmic(1, 16, 65536, 128, 128, 64, "isotropic")
    n, nc = 16 * 65536, 1024
    assert by_d["scan_reduce"] - by_i["scan_reduce"] == 16 * nc * (4 * 128 - 1) * 16
    assert by_i["scan_carry"] < by_d["scan_carry"] / 100
    assert bench.scan_bytes_8d(1, 16, 65536, 128, "isotropic") == n * (256 + 6 + 4)
