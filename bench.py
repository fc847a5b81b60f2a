"""Benchmark of the KDN layer forward (and decode step) on one MI355X.

Default run (no flags): the diagonal KDN forward with bf16 q/k/v/a/nu/r and
float32 state at B=8, H=16, T=4096, d_k=d_v=128, chunk 64 -- one step is one
full layer forward over that batch (scan, gain, chunk prep, chunk state).
Prints ONE JSON line with tokens/s (tokens = B*T positions, all 16 heads),
the roofline of the dominant kernel timed with HIP events on the stream the
kernels run on, the per-kernel breakdown, the decode step's bandwidth, and
the fp64 CPU oracle timed on a bounded sample of the same workload.
Before the W warmup steps the forward runs untimed for --ramp-ms of wall time
(default 0.2 s), so that the K timed steps see the clocks of a GPU that is
running continuously rather than one just out of idle.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_TFLOPS = 157.3

WL = dict(B=8, H=16, T=4096, dk=128, dv=128, chunk=64)
KERNELS = ("scan_reduce", "scan_carry", "chunk_prep", "chunk_state")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


_HIP = None


def _hip():
    """The HIP runtime this process already runs on (the one torch loaded)."""
    global _HIP
    if _HIP is None:
        import ctypes

        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        _HIP = ctypes.CDLL(path)
    return _HIP


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence:
    recording it performs no system-scope fence, so it neither writes back and
    invalidates the caches between the timed kernels (which slows the kernel
    that follows) nor adds that flush to the measured interval.  Same use as
    torch.cuda.Event: record(), elapsed_time(end) in ms, and .cuda_event (the
    hipEvent_t), which the binding hands to the library's timed entry points.
    Read elapsed times only after a device synchronisation."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes

        h = ctypes.c_void_p()
        rc = _hip().hipEventCreateWithFlags(ctypes.byref(h), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.cuda_event = h.value

    def record(self):
        import ctypes

        import torch

        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        rc = _hip().hipEventRecord(ctypes.c_void_p(self.cuda_event), stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end) -> float:
        import ctypes

        ms = ctypes.c_float()
        rc = _hip().hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.cuda_event),
                                        ctypes.c_void_p(end.cuda_event))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        import ctypes

        if getattr(self, "cuda_event", None) and _HIP is not None:
            _HIP.hipEventDestroy(ctypes.c_void_p(self.cuda_event))


def algorithmic(B, H, T, dk, dv, C, variant="diagonal"):
    """Design bytes and flops of each forward kernel (bf16 inputs): what this
    design's kernels read and write, the intermediates it passes between
    kernels through HBM (w, T) included.

    Bytes count every tensor a kernel must read or write once; flops count
    2 per multiply-add of the products the kernel performs, triangular ones at
    their triangular size."""
    n = B * H * T           # token-heads
    nc = -(-T // C)
    bh = B * H
    e = 2                   # bf16 bytes
    g = 3 * e               # a, nu, r per token-head
    nl = dk if variant == "diagonal" else 1  # precisions per token
    ns = C // 16 if variant == "diagonal" else 1  # products kept per (chunk, precision)
    by = {
        # read k and the three gates, write the float4 Moebius products per
        # (chunk, precision): the prefixes after every 16 tokens (diagonal), the
        # last being the chunk's product
        "scan_reduce": n * (dk * e + g) + bh * nc * ns * nl * 16,
        # read the chunk products, write chunk-boundary precisions
        "scan_carry": bh * nc * nl * 16 + bh * (nc + 1) * nl * 4 + bh * nl * 4 * 2,
        # read k, gates, boundary precisions and the sub-block prefixes; write w,
        # T and the log2 decays
        "chunk_prep": n * (dk * e + g) + bh * nc * nl * 4 + bh * nc * (ns - 1) * nl * 16
        + n * dk * e + bh * nc * C * C * e + n * 4,
        # read q, k, v, w, T, log2 decays, S0; write o, S_T
        "chunk_state": n * (3 * dk + dv) * e + n * 4 + bh * nc * C * C * e + n * dv * e
        + 2 * bh * dv * dk * 4,
    }
    fl = {
        # six multiply-adds per (token, precision) for the factorized Moebius
        # step (isotropic: plus |k|^2)
        "scan_reduce": n * nl * 12 + (0 if variant == "diagonal" else n * 2 * dk),
        "scan_carry": bh * nc * nl * 5,
        # gain (~8 per key dim), strict lower triangle of K W^T (C dk), triangular
        # inverse (~C^2/3)
        "chunk_prep": n * (8 * dk + C * dk + C * C // 3),
        # K S^T, Q S^T and the state update (2 dk dv each), lower triangle of
        # Q W^T (C dk), U = T R and the masked M U (C dv each)
        "chunk_state": n * (6 * dk * dv + C * dk + 2 * C * dv),
    }
    return by, fl


def chunk_flops_full(n, dk, dv, C):
    """Flops of the chunkwise form counted on full (not triangular) products:
    6 dk dv + C (6 dk + 4 dv) + C^2/3 per token-head (181,589 at d=128, C=64)."""
    return n * (6 * dk * dv + C * (6 * dk + 4 * dv) + C * C / 3)


# HBM bytes per launch of the state kernel from rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE passes, scaled by the same counters on a plain device copy of
# 512 MiB (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0), with the SHA-256 of the
# kernel source they were taken on: reported only while the source is unchanged.
TRAFFIC = {"kernel": "chunk_state",
           "src_sha256": "76fc65b5d085f14b38fe5a8532b7a1b7a236dc9044c2017d913391cd5f58a938",
           "fetch_bytes": 614620515, "write_bytes": 142606438}


def _traffic():
    import hashlib
    path = os.path.join(ROOT, "kalman_filter_memory_amd", "csrc", "kdn_chunk.hip")
    with open(path, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if TRAFFIC["src_sha256"] != sha or TRAFFIC["fetch_bytes"] is None:
        return None, sha
    return TRAFFIC["fetch_bytes"] + TRAFFIC["write_bytes"], sha


def bytes_8d(B, H, T, dk, dv):
    """The chunk stage's algorithmic bytes by its per-unit figure: per
    token-head, read q, k, v and the gain key w (bf16), the decay a (bf16),
    write o (bf16), and the head's S0 read and S_T write (fp32) amortised over
    its T tokens.  1,314 B per token-head at d_k = d_v = 128, T = 4096."""
    n = B * H * T
    e = 2
    return n * ((3 * dk + dv) * e + e + dv * e) + B * H * 2 * dv * dk * 4


def _stats(xs):
    import numpy as np

    if len(xs) == 0:
        return None
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "mean": round(float(a.mean()), 2),
            "n": int(a.size)}


def bench_forward(args, inp, variant, steps, cold_reps, label):
    """One forward workload: wall-clock mean over `steps` back-to-back steps;
    per-step times (warm: back to back; cold: each step after a 512 MiB write
    that evicts the L2 and Infinity caches) as median / p10 / p90 from HIP
    events; per-kernel times from HIP events around back-to-back passes over
    the forward's first kernels on the launch stream (kdn_forward_repeat), as
    differences of prefixes that end one kernel apart."""
    import numpy as np
    import torch

    import kalman_filter_memory_amd as kdn

    dev = torch.device("cuda:0")
    B, H, T, dk = inp["k"].shape
    dv = inp["v"].shape[-1]
    C = args.chunk
    bf = torch.bfloat16
    t = {n: torch.from_numpy(inp[n]).to(dev, bf) for n in ("q", "k", "v", "a", "nu", "r")}
    lam0 = torch.from_numpy(inp["lambda0"]).to(dev)
    S0 = torch.from_numpy(inp["S0"]).to(dev)
    d = kdn.make_desc(B, H, T, dk, dv, C, variant, kdn.BF16, kdn.BF16)
    ws = torch.empty(kdn.forward_workspace_bytes(d), dtype=torch.uint8, device=dev)
    lam_shape = (B, H, dk) if variant == "diagonal" else (B, H)
    out = (torch.empty((B, H, T, dv), dtype=bf, device=dev),
           torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev),
           torch.empty(lam_shape, dtype=torch.float32, device=dev))

    def step(events=None):
        kdn.forward(t["q"], t["k"], t["v"], t["a"], t["nu"], t["r"], lam0, S0, variant, C,
                    workspace=ws, out=out, events=events)

    ramp(step, args.ramp_ms)
    log(f"{label}: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"{label}: timing {steps} steps")
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps

    # warm per-step distribution (back to back, one event pair per step)
    ev = [(TimingEvent(), TimingEvent())
          for _ in range(steps)]
    for a0, a1 in ev:
        a0.record()
        step()
        a1.record()
    torch.cuda.synchronize()
    warm_us = [a0.elapsed_time(a1) * 1e3 for a0, a1 in ev]
    # cold: a 512 MiB write between the steps evicts every cache level
    flush = torch.empty(128 << 20, dtype=torch.float32, device=dev)
    cold_us = []
    for _ in range(cold_reps):
        flush.fill_(1.0)
        a0, a1 = TimingEvent(), TimingEvent()
        a0.record()
        step()
        a1.record()
        torch.cuda.synchronize()
        cold_us.append(a0.elapsed_time(a1) * 1e3)
    del flush

    # the same step captured once in a HIP graph and replayed back to back
    # (the library launches kernels only, so the graph holds the forward's
    # kernels and nothing else)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    g0, g1 = TimingEvent(), TimingEvent()
    g0.record()
    for _ in range(steps):
        g.replay()
    g1.record()
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1) / steps
    del g

    # per-kernel durations as they run in the forward: the forward's kernels
    # 0..i back to back, REPS passes between two events (kdn_forward_repeat on
    # the workspace the steps above left), and kernel i's time the difference
    # between the prefixes that end at i and at i - 1, in rounds.  Events
    # between the kernels of a step would add packets of the runtime's own
    # there and slow the kernel that follows; a kernel repeated alone would
    # find other data in the caches than the one before it in the forward left.
    # At least 10 rounds: a kernel of a few us is a small difference of two
    # prefixes whose run-to-run spread is of the same order.
    reps, rounds = 10, max(10, steps // 10)
    kern_us = {k: [] for k in KERNELS}
    for _ in range(rounds):
        pre = []
        for last in range(len(KERNELS)):
            a0, a1 = TimingEvent(), TimingEvent()
            a0.record()
            kdn.forward(t["q"], t["k"], t["v"], t["a"], t["nu"], t["r"], lam0, S0, variant, C,
                        workspace=ws, out=out, repeat=(0, last, reps))
            a1.record()
            torch.cuda.synchronize()
            pre.append(a0.elapsed_time(a1) * 1e3 / reps)
        for i, kname in enumerate(KERNELS):
            kern_us[kname].append(pre[i] - (pre[i - 1] if i else 0.0))
    kern_mean = {k: float(np.mean(v)) for k, v in kern_us.items()}
    by, fl = algorithmic(B, H, T, dk, dv, C, variant)
    kernels = {}
    for k in KERNELS:
        sec = kern_mean[k] * 1e-6
        kernels[k] = {"us": round(kern_mean[k], 2), "us_stats": _stats(kern_us[k]),
                      "GB/s": round(by[k] / sec / 1e9, 1),
                      "TFLOP/s": round(fl[k] / sec / 1e12, 2)}
    # the dominant kernel (the chunk state pass) against HBM, by the chunk
    # stage's per-unit bytes; the design's own bytes (which also count the w
    # and T this design passes from prep to state through HBM) beside it
    dom = max(KERNELS, key=lambda k: kern_mean[k])
    s_dom = kern_mean[dom] * 1e-6
    alg = bytes_8d(B, H, T, dk, dv) if dom == "chunk_state" else by[dom]
    ach = alg / s_dom / 1e9
    roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None, "kernel": dom,
                "bytes_per_launch": alg,
                "bytes_rule": "q, k, v, w, a read and o written once per token-head, S0 and S_T "
                              "amortised (1314 B per token-head at d 128, T 4096)"
                if dom == "chunk_state" else "design bytes",
                "us_per_launch": round(kern_mean[dom], 2),
                "design_bytes_per_launch": by[dom],
                "design_frac": round(by[dom] / s_dom / 1e9 / PEAK_HBM_GBS, 4)}
    n = B * H * T
    chunk_s = (kern_mean["chunk_prep"] + kern_mean["chunk_state"]) * 1e-6
    mfma = {"kernels": "chunk_prep+chunk_state", "us": round(chunk_s * 1e6, 2),
            "flops_full": chunk_flops_full(n, dk, dv, C),
            "frac_full": round(chunk_flops_full(n, dk, dv, C) / chunk_s / 1e12
                               / PEAK_BF16_TFLOPS, 4),
            "flops_performed": fl["chunk_prep"] + fl["chunk_state"],
            "frac_performed": round((fl["chunk_prep"] + fl["chunk_state"]) / chunk_s / 1e12
                                    / PEAK_BF16_TFLOPS, 4),
            "flops_recurrent": n * 6 * dk * dv,
            "peak_TFLOP/s": PEAK_BF16_TFLOPS}
    scan_s = (kern_mean["scan_reduce"] + kern_mean["scan_carry"]) * 1e-6
    scan_by = by["scan_reduce"] + by["scan_carry"]
    scan8 = scan_bytes_8d(B, H, T, dk, variant)
    res = {"workload": f"{'diag' if variant == 'diagonal' else 'iso'}_bf16_B{B}_H{H}_T{T}_d{dk}",
           "variant": variant, "ms_per_step": round(ms, 4),
           "tokens/s": round(B * T / (ms * 1e-3), 1),
           "step_us_warm": _stats(warm_us), "step_us_cold": _stats(cold_us),
           "graph": {"ms_per_step": round(graph_ms, 4),
                     "tokens/s": round(B * T / (graph_ms * 1e-3), 1), "replays": steps,
                     "what": "the step captured once in a HIP graph (torch.cuda.graph around "
                             "the binding), replayed back to back between two HIP events"},
           "roofline": roofline, "mfma_chunk": mfma,
           "scan_hbm": {"kernels": "scan_reduce+scan_carry", "us": round(scan_s * 1e6, 2),
                        "bytes": scan_by, "GB/s": round(scan_by / scan_s / 1e9, 1),
                        "frac": round(scan_by / scan_s / 1e9 / PEAK_HBM_GBS, 4),
                        "bytes_8d": scan8,
                        "note_8d": "bytes_8d counts a scan that also writes every predictive "
                                   "precision; this design's scan does not (the prep derives them "
                                   "inside each chunk), so bytes_8d over its time is no fraction "
                                   "of anything it moves"},
           "kernels": kernels}
    del t, ws, out
    torch.cuda.empty_cache()
    return res


def scan_bytes_8d(B, H, T, dk, variant):
    """The precision scan's per-unit bytes: read k (bf16) and the three gates
    per token, write one fp32 predictive precision per (token, key dim)
    (diagonal) or per token (isotropic)."""
    n = B * H * T
    return n * (dk * 2 + 6 + (dk * 4 if variant == "diagonal" else 4))


def run(args):
    import torch

    from kdn_inputs import config_inputs

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    B, T = WL["B"], WL["T"]
    log("generating inputs")
    inp = config_inputs(2)
    if args.copy_calibration_mb:
        dev = torch.device("cuda:0")
        nb = args.copy_calibration_mb << 20
        src = torch.empty(nb // 4, dtype=torch.float32, device=dev).uniform_()
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {nb} bytes read and written")
        del src, dst
    head = bench_forward(args, inp, "diagonal", args.steps, args.cold_reps, "forward")
    ms = head["ms_per_step"]
    traffic, sha = _traffic()
    roofline = dict(head["roofline"])
    if roofline["kernel"] == TRAFFIC["kernel"]:
        roofline["traffic"] = traffic
        if traffic is not None:
            roofline["traffic_src_sha256"] = sha
    res = {
        "metric": "KDN fwd tokens/s (B8 T4096 H16 d128); % MFMA peak; decode GB/s",
        "value": round(B * T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ramp_ms": args.ramp_ms,
        "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "diag_bf16_B8_H16_T4096_d128", "variant": "diagonal",
                   "B": B, "H": WL["H"], "T": T, "d_k": WL["dk"], "d_v": WL["dv"],
                   "chunk": args.chunk, "state_dtype": "f32"},
        "roofline": roofline,
        "step_us_warm": head["step_us_warm"], "step_us_cold": head["step_us_cold"],
        "graph": head["graph"],
        "mfma_chunk": head["mfma_chunk"],
        "scan_hbm": head["scan_hbm"],
        "kernels": head["kernels"],
    }
    if not args.no_isotropic:
        res["isotropic"] = bench_forward(args, config_inputs(2, variant="isotropic"),
                                         "isotropic", 50, args.cold_reps, "isotropic forward")
    if not args.no_long:
        res["long"] = {}
        for variant in ("diagonal", "isotropic"):
            log(f"generating the long workload ({variant})")
            li = config_inputs(3, variant=variant)
            res["long"][variant] = bench_forward(args, li, variant, 10, 5, f"long {variant}")
            del li
    if not args.no_backward:
        res["backward"] = bench_backward(args, inp)
    if not args.no_dense:
        res["dense"] = bench_dense(args, inp)
    if not args.no_layer:
        res["layer"] = bench_layer(args)
    if not args.no_decode:
        res["decode"] = bench_decode(args)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, args)
    print(json.dumps(res), flush=True)


BWD_STAGES = ("scan_reduce", "scan_carry", "chunk_prep", "chunk_state", "bwd_state",
              "bwd_grad", "bwd_gain")


def algorithmic_backward(B, H, T, dk, dv, C):
    """Algorithmic bytes and MFMA flops of each backward stage (bf16 inputs,
    float32 gradients).  The first four stages are the forward recompute
    (as in the forward, plus 1/D per token from the prep pass and the bf16
    state at every chunk start from the state pass)."""
    n = B * H * T
    nc = -(-T // C)
    bh = B * H
    e = 2
    g = 3 * e
    states = bh * nc * dv * dk * e
    fby, ffl = algorithmic(B, H, T, dk, dv, C)
    by = {
        "scan_reduce": fby["scan_reduce"],
        "scan_carry": fby["scan_carry"] - bh * dk * 4,  # no lambda_T
        "chunk_prep": fby["chunk_prep"] + n * 4,
        "chunk_state": fby["chunk_state"] + states - n * dv * e,  # no read-out
        # read q, k, w, dO, T, g, dS_T; write dv (= dR, f32), the chunk-end
        # adjoints (bf16) and dS0
        "bwd_state": n * (3 * dk + dv) * e + bh * nc * C * C * e + n * 4 + bh * dv * dk * 4
        + n * dv * 4 + states + bh * dv * dk * 4,
        # read q, k, w, v, dO, dR, T, g and both chunk states; write dq, dk
        # (f32), dW (bf16), s and d(ln a)
        "bwd_grad": n * (3 * dk + 2 * dv) * e + n * dv * 4 + bh * nc * C * C * e + n * 4
        + 2 * states + 2 * n * dk * 4 + n * dk * e + 2 * n * 4,
        # map pass: k, dW, gates, 1/D, s, boundary precisions -> chunk maps;
        # carry; apply pass: the same plus d(ln a), G, dk read and written,
        # da, dnu, dr
        "bwd_gain": (n * dk * 2 * e + n * (g + 8) + bh * nc * dk * (4 + 8))
        + bh * nc * dk * (8 + 4)
        + (n * dk * 2 * e + n * (g + 12) + bh * nc * dk * 8 + 2 * n * dk * 4 + 3 * n * 4),
    }
    fl = {
        "scan_reduce": ffl["scan_reduce"], "scan_carry": ffl["scan_carry"],
        "chunk_prep": ffl["chunk_prep"], "chunk_state": ffl["chunk_state"],
        # M (lower half), D W dS^T, M^T dO, T^T dU, the adjoint update (two products)
        "bwd_state": n * (6 * dk * dv + C * dk + 2 * C * dv),
        # X = K S^T, U = T R (half), dM and dA (halves), dO S, dR S, U dS', M and A
        # (halves), (dM G) W, (dA G) W and their transposed products with Q, K (halves)
        "bwd_grad": n * (8 * dk * dv + 3 * C * dv + 4 * C * dk),
        "bwd_gain": 0,
    }
    return by, fl


def bench_backward(args, inp):
    """Backward pass (kdn_backward) on the same workload: recompute plus the
    gradient kernels, per-stage times from dispatch-recorded events."""
    import numpy as np
    import torch

    import kalman_filter_memory_amd as kdn
    from kdn_inputs import backward_cotangents

    dev = torch.device("cuda:0")
    B, H, T, dk, dv, C = (WL[x] for x in ("B", "H", "T", "dk", "dv", "chunk"))
    bf = torch.bfloat16
    t = {n: torch.from_numpy(inp[n]).to(dev, bf) for n in ("q", "k", "v", "a", "nu", "r")}
    lam0 = torch.from_numpy(inp["lambda0"]).to(dev)
    S0 = torch.from_numpy(inp["S0"]).to(dev)
    log("generating backward cotangents")
    cot = backward_cotangents(B, H, T, dk, dv, dtype="bf16", seed=1002)
    dO = torch.from_numpy(cot["dO"]).to(dev, bf)
    dS_T = torch.from_numpy(cot["dS_T"]).to(dev)
    dl_T = torch.from_numpy(cot["dlambda_T"]).to(dev)
    d = kdn.make_desc(B, H, T, dk, dv, C, "diagonal", kdn.BF16, kdn.BF16)
    ws = torch.empty(kdn.backward_workspace_bytes(d), dtype=torch.uint8, device=dev)
    shapes = {"dq": (B, H, T, dk), "dk": (B, H, T, dk), "dv": (B, H, T, dv),
              "da": (B, H, T), "dqnoise": (B, H, T), "dr": (B, H, T),
              "dlambda0": (B, H, dk), "dS0": (B, H, dv, dk)}
    out = {n: torch.empty(sh, dtype=torch.float32, device=dev) for n, sh in shapes.items()}

    def step(events=None):
        kdn.backward(t["q"], t["k"], t["v"], t["a"], t["nu"], t["r"], dO, lam0, S0, dS_T, dl_T,
                     chunk=C, workspace=ws, out=out, events=events)

    steps = max(1, args.backward_steps)
    ramp(step, args.ramp_ms)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    log(f"timing {steps} backward steps")
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    evs = [[TimingEvent() for _ in range(2 * len(BWD_STAGES))]
           for _ in range(steps)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for row in evs:
        step(events=row)
    torch.cuda.synchronize()
    st_ms = {k: float(np.mean([row[2 * i].elapsed_time(row[2 * i + 1]) for row in evs]))
             for i, k in enumerate(BWD_STAGES)}
    by, fl = algorithmic_backward(B, H, T, dk, dv, C)
    stages = {}
    for k in BWD_STAGES:
        sec = st_ms[k] * 1e-3
        stages[k] = {"us": round(st_ms[k] * 1e3, 2), "GB/s": round(by[k] / sec / 1e9, 1)}
        if fl[k]:
            stages[k]["TFLOP/s"] = round(fl[k] / sec / 1e12, 2)
    grad_stages = ("bwd_state", "bwd_grad", "bwd_gain")
    dom = max(grad_stages, key=lambda k: st_ms[k])
    ach = by[dom] / (st_ms[dom] * 1e-3) / 1e9

    # training step: the forward keeping its intermediates, then the backward
    # without its recompute
    o = torch.empty((B, H, T, dv), dtype=bf, device=dev)
    S_T = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    lam_T = torch.empty((B, H, dk), dtype=torch.float32, device=dev)

    def fwd_keep():
        kdn.forward(t["q"], t["k"], t["v"], t["a"], t["nu"], t["r"], lam0, S0, "diagonal", C,
                    out=(o, S_T, lam_T), keep=ws)

    def bwd_kept():
        kdn.backward(t["q"], t["k"], t["v"], t["a"], t["nu"], t["r"], dO, lam0, S0, dS_T, dl_T,
                     chunk=C, out=out, kept=ws)

    def timed_ms(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t1) * 1e3 / steps

    ramp(lambda: (fwd_keep(), bwd_kept()), args.ramp_ms)
    train_ms = timed_ms(lambda: (fwd_keep(), bwd_kept()))
    fk_ms = timed_ms(fwd_keep)
    bk_ms = timed_ms(lambda: (fwd_keep(), bwd_kept())) - fk_ms
    train = {"ms_per_step": round(train_ms, 4),
             "tokens_per_s": round(B * T / (train_ms * 1e-3), 1),
             "forward_keep_ms": round(fk_ms, 4), "backward_kept_ms": round(bk_ms, 4),
             "what": "kdn_forward_keep (the forward, keeping what the backward needs) then "
                     "kdn_backward_kept (no recompute), back to back"}
    del t, ws, out, dO, o, S_T, lam_T
    torch.cuda.empty_cache()
    return {"workload": "diag_bf16_B8_H16_T4096_d128", "steps": steps,
            "ms_per_step": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1),
            "includes": "forward recompute (scan, prep, state keeping chunk states) "
                        "and the three gradient stages",
            "train_step": train,
            "stages": stages,
            "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(ach / PEAK_HBM_GBS, 4), "bytes_per_launch": by[dom],
                         "us_per_launch": round(st_ms[dom] * 1e3, 2), "traffic": None}}


def ramp(fn, ms):
    """Run fn back to back for about `ms` milliseconds of wall time, untimed.

    An idle GPU runs its first tens of milliseconds of work at lower clocks
    (measured on MI355X: 20 back-to-back forward steps after a pause take
    ~350 us each, the same steps after ~50 ms of work ~297 us), so the timed
    steps start from the state a continuously running layer is in."""
    import torch

    if ms <= 0:
        return
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def bench_dense(args, inp):
    """Exact KDN (dense Riccati gain, then the chunkwise write) on the same
    workload from P0 = I.  The gain kernel is a sequential recursion per head;
    it is reported by its time per token and its arithmetic rate: the
    algorithmic count per token and head is 5 d_k^2 flops (prediction d_k^2,
    P^- k 2 d_k^2, rank-one update 2 d_k^2)."""
    import torch

    import kalman_filter_memory_amd as kdn

    dev = torch.device("cuda:0")
    B, H, T, dk, C = (WL[x] for x in ("B", "H", "T", "dk", "chunk"))
    bf = torch.bfloat16
    t = {n: torch.from_numpy(inp[n]).to(dev, bf) for n in ("q", "k", "v", "a", "nu", "r")}
    S0 = torch.from_numpy(inp["S0"]).to(dev)

    def fwd():
        kdn.forward_dense(t["q"], t["k"], t["v"], t["a"], t["nu"], t["r"], None, S0, chunk=C)

    def gain():
        kdn.dense_gain(t["k"], t["a"], t["nu"], t["r"], None, want_P=False)

    steps = 10
    for _ in range(2):
        fwd()
    torch.cuda.synchronize()
    log(f"timing {steps} exact-KDN forward steps")
    t0 = time.perf_counter()
    for _ in range(steps):
        fwd()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    e0, e1 = TimingEvent(), TimingEvent()
    e0.record()
    for _ in range(steps):
        gain()
    e1.record()
    torch.cuda.synchronize()
    g_ms = e0.elapsed_time(e1) / steps
    flops = 5.0 * B * H * T * dk * dk
    tf = flops / (g_ms * 1e-3) / 1e12
    return {"ms_per_step": round(ms, 4), "tokens/s": round(B * T / (ms * 1e-3), 1),
            "gain_us": round(g_ms * 1e3, 1), "ns_per_token": round(g_ms * 1e6 / T, 1),
            "gain_TFLOP/s": round(tf, 2), "frac_fp32": round(tf / PEAK_FP32_TFLOPS, 4),
            "bound": "latency (sequential over tokens; one workgroup per head)"}


LAYER = dict(B=8, T=4096, H=16, D=2048, dk=128, dv=128, chunk=64)
LAYER_STAGES = ("gemm_in", "norm_gates", "recurrence", "readout_rows", "gemm_out")


def bench_layer(args):
    """The KDN layer on random weights (kdn_layer_forward): input GEMM (hipBLASLt),
    normalisation and gates, the recurrence, the read-out to token rows, output
    GEMM; per-stage times from events recorded between the stages."""
    import numpy as np
    import torch

    import kalman_filter_memory_amd as kdn
    from kdn_inputs import layer_inputs

    dev = torch.device("cuda:0")
    B, T, H, D, dk, dv, C = (LAYER[x] for x in ("B", "T", "H", "D", "dk", "dv", "chunk"))
    log("generating layer inputs")
    p = layer_inputs(B, T, H, D, dk, dv, dtype="bf16", seed=1003)
    bf = torch.bfloat16
    # the library takes the weights out-features major (y = x W^T)
    t = {"x": torch.from_numpy(p["x"]).to(dev, bf)}
    t.update({n: torch.from_numpy(np.ascontiguousarray(p[n].T)).to(dev, bf)
              for n in ("W_in", "W_out")})
    t.update({n: torch.from_numpy(p[n]).to(dev) for n in ("b_gate", "lambda0", "S0")})
    d = kdn.make_layer_desc(B, T, H, D, dk, dv, C, "diagonal", kdn.BF16)
    ws = torch.empty(kdn.layer_workspace_bytes(d), dtype=torch.uint8, device=dev)

    def step(events=None):
        kdn.layer_forward(t["x"], t["W_in"], t["b_gate"], t["W_out"], H, dk, dv, t["lambda0"],
                          t["S0"], chunk=C, workspace=ws, events=events)

    ramp(step, args.ramp_ms)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    steps = 20
    log(f"timing {steps} layer steps")
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    evs = [[TimingEvent() for _ in range(10)] for _ in range(steps)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for row in evs:
        step(events=row)
    torch.cuda.synchronize()
    st = {k: float(np.mean([row[2 * i].elapsed_time(row[2 * i + 1]) for row in evs]))
          for i, k in enumerate(LAYER_STAGES)}
    M, n_in = B * T, H * (2 * dk + dv) + 3 * H
    flops = {"gemm_in": 2.0 * M * D * n_in, "gemm_out": 2.0 * M * H * dv * D}
    nbytes = {"norm_gates": M * n_in * 2 + B * H * T * (2 * dk + dv + 3) * 2,
              "readout_rows": 2 * B * H * T * dv * 2}
    stages = {}
    for k in LAYER_STAGES:
        sec = st[k] * 1e-3
        stages[k] = {"us": round(st[k] * 1e3, 1)}
        if k in flops:
            tf = flops[k] / sec / 1e12
            stages[k].update({"TFLOP/s": round(tf, 1), "frac_bf16": round(tf / PEAK_BF16_TFLOPS, 4)})
        if k in nbytes:
            gbs = nbytes[k] / sec / 1e9
            stages[k].update({"GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)})
    return {"workload": f"layer_diag_bf16_B{B}_T{T}_H{H}_D{D}_d{dk}", "ms_per_step": round(ms, 4),
            "tokens/s": round(M / (ms * 1e-3), 1), "stages": stages,
            "gemm": "hipBLASLt matmul, weights out-features major (x W^T), bf16 in and out, fp32 accumulation",
            "weights": "random (kdn_inputs.layer_inputs), no trained checkpoint"}


def bench_decode(args):
    """Decode step at 256 sequences x 16 heads x d 128, 128 steps in place."""
    import numpy as np
    import torch

    import kalman_filter_memory_amd as kdn
    from kdn_inputs import config_inputs

    dev = torch.device("cuda:0")
    log("generating decode inputs")
    dd = config_inputs(4)
    steps, N, H, dk = dd["q"].shape
    dv = dd["v"].shape[-1]
    S = torch.from_numpy(dd["S0"]).to(dev)
    lam = torch.from_numpy(dd["lambda0"]).to(dev)
    x = {n: torch.from_numpy(dd[n]).to(dev, torch.bfloat16 if n in "qkv" else torch.float32)
         for n in ("q", "k", "v", "a", "nu", "r")}
    o = torch.empty((N, H, dv), dtype=torch.bfloat16, device=dev)

    def one(s):
        kdn.decode_step(x["q"][s], x["k"][s], x["v"][s], x["a"][s], x["nu"][s], x["r"][s], S,
                        lam, "diagonal", out=o)

    ramp(lambda: one(0), args.ramp_ms / 2)
    for s in range(4):
        one(s)
    torch.cuda.synchronize()
    e0, e1 = TimingEvent(), TimingEvent()
    e0.record()
    for s in range(steps):
        one(s)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    nbytes = N * H * (2 * dv * dk * 4 + 2 * dk * 4 + (2 * dk + 2 * dv) * 2 + 3 * 4)
    return {"workload": "decode_diag_N256_H16_d128", "steps": steps,
            "us_per_step": round(us, 2), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "tokens_per_s": round(N / (us * 1e-6), 1), "bytes_per_step": nbytes,
            "timing": "128 back-to-back launches between two HIP events"}


def cpu_baseline(inp, args):
    """The fp64 oracle, as it is, on the same workload: all heads and tokens,
    repeated until at least --cpu-seconds of wall time have passed."""
    import numpy as np

    import oracle

    threads = oracle.default_threads()
    heads = WL["B"] * WL["H"]
    sub = {n: inp[n] for n in ("q", "k", "v", "a", "nu", "r", "lambda0", "S0")}
    log(f"cpu baseline: oracle on the whole workload ({heads} heads x T={WL['T']}) "
        f"with {threads} threads, for at least {args.cpu_seconds} s")
    reps, sec = 0, 0.0
    while reps == 0 or sec < args.cpu_seconds:
        t0 = time.perf_counter()
        oracle.forward(sub["q"], sub["k"], sub["v"], sub["a"], sub["nu"], sub["r"],
                       sub["lambda0"], sub["S0"], "diagonal", threads=threads)
        sec += time.perf_counter() - t0
        reps += 1
    tokens = reps * WL["B"] * WL["T"]
    return {"value": round(tokens / sec, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the whole workload (B={WL['B']}, H={WL['H']}, T={WL['T']}, d=128, fp64 "
                      f"token-by-token recurrence over the same bf16-rounded inputs) run {reps} "
                      f"times in {sec:.1f} s; a token carries all {WL['H']} heads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--ramp-ms", type=float, default=200.0,
                    help="untimed back-to-back steps for this long before the warmup steps, "
                         "so that the GPU is out of its idle clock state (0: none)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum wall time of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-isotropic", action="store_true")
    ap.add_argument("--no-layer", action="store_true")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long-context workload (B1 H16 T65536, both variants)")
    ap.add_argument("--chunk", type=int, default=64)
    ap.add_argument("--cold-reps", type=int, default=20,
                    help="steps timed one by one after a 512 MiB cache-evicting write")
    ap.add_argument("--backward-steps", type=int, default=20)
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a known-size "
                         "kernel that HBM byte counters can be scaled against)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer shards over heads with no communication)",
              file=sys.stderr)
        sys.exit(2)
    run(args)


if __name__ == "__main__":
    main()
