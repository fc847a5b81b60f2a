"""Python binding of libkdn, the gfx950 KDN layer library (argument marshalling only).

Every step of the computation runs in the HIP kernels behind the C ABI of
include/kdn.h; this module checks tensors, allocates outputs and workspaces
with torch on the current device, and passes raw pointers and the current
torch stream.  There is no fallback: if libkdn.so is missing or the tensors
are not on a GPU, the calls raise.

Functions (same names as the C entry points):
  forward(q, k, v, a, qnoise, r, lambda0=None, S0=None, variant="diagonal", chunk=64)
      -> (o, S_T, lambda_T)
  decode_step(q, k, v, a, qnoise, r, S, lam, variant="diagonal") -> o   (S, lam in place)
  decode_step_indexed(q, k, v, a, qnoise, r, S_cache, lam_cache, slot, variant=...) -> o
  dense_gain(k, a, qnoise, r, P0=None) -> (w, P_T);  forward_dense(...) -> (o, S_T, P_T)
  layer_forward(x, W_in, b_gate, W_out, H, d_k, d_v, ...) -> (y, S_T, lambda_T)
  forward_varlen(q, k, v, a, qnoise, r, cu_seqlens, max_seqlen, lambda0=None, S0=None,
                 variant=..., chunk=64) -> (o, S_T, lambda_T)   (a packed batch)
  mobius_scan(k, a, qnoise, r, lambda0=None, variant=..., chunk=64) -> dict
  gain(k, r, lambda_minus, variant=..., gain_dtype=None) -> w
  chunk_delta(q, k, v, a, w, S0=None, chunk=64) -> (o, S_T)
  backward(q, k, v, a, qnoise, r, dO, lambda0=None, S0=None, dS_T=None, dlambda_T=None,
           variant="diagonal", chunk=64) -> dict of float32 gradients (dq, dk, dv, da, dqnoise, dr,
           dlambda0, dS0)
"""
from __future__ import annotations

import atexit
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkdn.so")

DIAGONAL, ISOTROPIC = 0, 1
F32, BF16 = 0, 1

EXPORTS = (
    "kdn_status_string", "kdn_validate", "kdn_forward_workspace_bytes", "kdn_forward",
    "kdn_forward_events", "kdn_forward_repeat", "kdn_forward_segments",
    "kdn_mobius_scan_workspace_bytes", "kdn_mobius_scan", "kdn_gain",
    "kdn_chunk_delta_workspace_bytes", "kdn_chunk_delta", "kdn_decode_step",
    "kdn_backward_workspace_bytes", "kdn_backward", "kdn_backward_events",
    "kdn_forward_keep", "kdn_backward_kept", "kdn_backward_kept_events",
    "kdn_decode_step_indexed", "kdn_forward_varlen_workspace_bytes", "kdn_forward_varlen",
    "kdn_dense_gain", "kdn_blas_create", "kdn_blas_destroy", "kdn_layer_workspace_bytes",
    "kdn_layer_forward", "kdn_layer_forward_events",
    "kdn_noalloc_scratch_bytes", "kdn_forward_noalloc",
)


class KdnDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "B", "H", "T", "d_k", "d_v", "chunk", "variant", "qkv_dtype", "gate_dtype",
        "gain_dtype")]


class KdnLayerDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "B", "T", "H", "d_model", "d_k", "d_v", "chunk", "variant", "dtype")]


class KdnError(RuntimeError):
    pass


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libkdn.so (built by kalman_filter_memory_amd.build) and declare its ABI."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise KdnError(f"{path} is not built; run `python -m kalman_filter_memory_amd.build`")
    lib = ctypes.CDLL(path)
    P, S, D = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(KdnDesc)
    I = ctypes.c_int
    lib.kdn_status_string.argtypes = [I]
    lib.kdn_status_string.restype = ctypes.c_char_p
    lib.kdn_validate.argtypes = [D]
    lib.kdn_validate.restype = I
    for n in ("kdn_forward_workspace_bytes", "kdn_mobius_scan_workspace_bytes",
              "kdn_chunk_delta_workspace_bytes"):
        getattr(lib, n).argtypes = [D]
        getattr(lib, n).restype = S
    lib.kdn_forward_segments.argtypes = [D]
    lib.kdn_forward_segments.restype = ctypes.c_int32
    lib.kdn_forward.argtypes = [D] + [P] * 11 + [P, S, P]
    lib.kdn_forward.restype = I
    lib.kdn_forward_events.argtypes = [D] + [P] * 11 + [P, S, P, ctypes.POINTER(P)]
    lib.kdn_forward_events.restype = I
    lib.kdn_forward_repeat.argtypes = [D] + [P] * 11 + [P, S, P] + [ctypes.c_int32] * 3
    lib.kdn_forward_repeat.restype = I
    lib.kdn_mobius_scan.argtypes = [D] + [P] * 8 + [P, S, P]
    lib.kdn_mobius_scan.restype = I
    lib.kdn_gain.argtypes = [D, P, P, P, P, P]
    lib.kdn_gain.restype = I
    lib.kdn_chunk_delta.argtypes = [D] + [P] * 8 + [P, S, P]
    lib.kdn_chunk_delta.restype = I
    lib.kdn_decode_step.argtypes = [D] + [P] * 9 + [P]
    lib.kdn_backward.argtypes = [D] + [P] * 19 + [P, S, P]
    lib.kdn_backward_events.argtypes = [D] + [P] * 19 + [P, S, P, ctypes.POINTER(P)]
    lib.kdn_forward_keep.argtypes = [D] + [P] * 11 + [P, S, P]
    lib.kdn_decode_step_indexed.argtypes = [D] + [P] * 9 + [ctypes.c_int32, P, P]
    lib.kdn_dense_gain.argtypes = [D] + [P] * 8
    L = ctypes.POINTER(KdnLayerDesc)
    lib.kdn_blas_create.argtypes = [ctypes.POINTER(P)]
    lib.kdn_blas_destroy.argtypes = [P]
    lib.kdn_layer_workspace_bytes.argtypes = [L]
    lib.kdn_layer_workspace_bytes.restype = S
    lib.kdn_layer_forward.argtypes = [L] + [P] * 11 + [S, P]
    lib.kdn_layer_forward_events.argtypes = [L] + [P] * 11 + [S, P, ctypes.POINTER(P)]
    lib.kdn_forward_varlen_workspace_bytes.argtypes = [D]
    lib.kdn_forward_varlen_workspace_bytes.restype = S
    lib.kdn_forward_varlen.argtypes = [D, P, ctypes.c_int32] + [P] * 12 + [S, P]
    lib.kdn_backward_kept.argtypes = [D] + [P] * 19 + [P, S, P]
    lib.kdn_backward_kept_events.argtypes = [D] + [P] * 19 + [P, S, P, ctypes.POINTER(P)]
    lib.kdn_decode_step.restype = I
    lib.kdn_noalloc_scratch_bytes.argtypes = []
    lib.kdn_noalloc_scratch_bytes.restype = S
    lib.kdn_forward_noalloc.argtypes = [D] + [P] * 11 + [P]
    lib.kdn_forward_noalloc.restype = I
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load_library().kdn_status_string(code).decode()


def _check(code: int, what: str):
    if code != 0:
        raise KdnError(f"{what}: {status_string(code)} (kdn_status {code})")


def _variant(v) -> int:
    if v in (DIAGONAL, "diagonal", "diag"):
        return DIAGONAL
    if v in (ISOTROPIC, "isotropic", "iso"):
        return ISOTROPIC
    raise ValueError(f"unknown variant {v!r}")


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t}; use float32 or bfloat16")


def _torch_dtype(code: int) -> torch.dtype:
    return torch.bfloat16 if code == BF16 else torch.float32


def _gpu(x: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not x.is_cuda:
        raise KdnError(f"{name} must be on a GPU (no CPU path exists)")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return x


def _ptr(x):
    return None if x is None else x.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def make_desc(B, H, T, d_k, d_v, chunk, variant, qkv_dtype, gate_dtype, gain_dtype=None):
    d = KdnDesc()
    d.B, d.H, d.T, d.d_k, d.d_v, d.chunk = B, H, T, d_k, d_v, chunk
    d.variant = _variant(variant)
    d.qkv_dtype = qkv_dtype
    d.gate_dtype = gate_dtype
    d.gain_dtype = qkv_dtype if gain_dtype is None else gain_dtype
    return d


def validate(desc: KdnDesc) -> int:
    return load_library().kdn_validate(ctypes.byref(desc))


def forward_segments(desc: KdnDesc) -> int:
    """Sequence segments of kdn_forward's state pass for this descriptor (1:
    the plain sequential pass; 0: invalid descriptor)."""
    return load_library().kdn_forward_segments(ctypes.byref(desc))


def forward_workspace_bytes(desc: KdnDesc) -> int:
    return load_library().kdn_forward_workspace_bytes(ctypes.byref(desc))


def _forward_desc(q, k, v, a, qnoise, r, variant, chunk):
    for n, x in (("q", q), ("k", k), ("v", v), ("a", a), ("qnoise", qnoise), ("r", r)):
        _gpu(x, n)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    if q.shape != k.shape or v.shape != (B, H, T, dv):
        raise ValueError("q, k must be [B,H,T,d_k] and v [B,H,T,d_v]")
    if a.shape != (B, H, T) or qnoise.shape != a.shape or r.shape != a.shape:
        raise ValueError("a, qnoise, r must be [B,H,T]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    if not (a.dtype == qnoise.dtype == r.dtype):
        raise TypeError("a, qnoise, r must share one dtype")
    return make_desc(B, H, T, dk, dv, chunk, variant, _dtype_code(q.dtype), _dtype_code(a.dtype))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def forward(q, k, v, a, qnoise, r, lambda0=None, S0=None, variant="diagonal", chunk=64,
            workspace: torch.Tensor | None = None, out=None, events=None,
            keep: torch.Tensor | None = None, repeat: tuple[int, int, int] | None = None):
    """KDN layer forward on the GPU.  Returns (o, S_T, lambda_T).

    out: optional preallocated (o, S_T, lambda_T); events: optional list of 8
    events (objects with a .cuda_event handle, already created): the start and
    stop of each of the four kernels, handed to the kernel dispatches.  keep: a
    uint8 tensor of backward_workspace_bytes: the forward keeps in it what
    backward(..., kept=keep) needs (kdn_forward_keep).  repeat: (first, last,
    reps): kernels first..last of the forward, in order, reps times over, back
    to back (kdn_forward_repeat; workspace must hold what a forward with the
    same arguments left)."""
    lib = load_library()
    d = _forward_desc(q, k, v, a, qnoise, r, variant, chunk)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    lam_shape = (B, H, dk) if d.variant == DIAGONAL else (B, H)
    if lambda0 is not None:
        _gpu(lambda0, "lambda0")
        if lambda0.dtype != torch.float32 or tuple(lambda0.shape) != lam_shape:
            raise ValueError(f"lambda0 must be float32 {lam_shape}")
    if S0 is not None:
        _gpu(S0, "S0")
        if S0.dtype != torch.float32 or tuple(S0.shape) != (B, H, dv, dk):
            raise ValueError("S0 must be float32 [B,H,d_v,d_k]")
    dev = k.device
    if out is not None:
        o, S_T, lam_T = out
    else:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
        S_T = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
        lam_T = torch.empty(lam_shape, dtype=torch.float32, device=dev)
    if keep is not None:
        args = (ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(qnoise), _ptr(r),
                _ptr(lambda0), _ptr(S0), _ptr(o), _ptr(S_T), _ptr(lam_T), _ptr(keep),
                keep.numel() * keep.element_size(), _stream())
        _check(lib.kdn_forward_keep(*args), "kdn_forward_keep")
        return o, S_T, lam_T
    need = lib.kdn_forward_workspace_bytes(ctypes.byref(d))
    if need == 0:
        _check(lib.kdn_validate(ctypes.byref(d)), "kdn_forward")
    ws = workspace if workspace is not None else _workspace(need, dev)
    args = (ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(qnoise), _ptr(r),
            _ptr(lambda0), _ptr(S0), _ptr(o), _ptr(S_T), _ptr(lam_T), _ptr(ws),
            ws.numel() * ws.element_size(), _stream())
    if repeat is not None:
        if workspace is None:
            raise ValueError("repeat needs the workspace of an earlier forward")
        first, last, reps = (int(x) for x in repeat)
        _check(lib.kdn_forward_repeat(*args, first, last, reps), "kdn_forward_repeat")
    elif events is None:
        _check(lib.kdn_forward(*args), "kdn_forward")
    else:
        if len(events) != 8:
            raise ValueError("events: 8 entries (start and stop of four kernels)")
        arr = (ctypes.c_void_p * 8)(*[None if e is None else e.cuda_event for e in events])
        _check(lib.kdn_forward_events(*args, arr), "kdn_forward_events")
    return o, S_T, lam_T


def forward_noalloc(q, k, v, a, qnoise, r, lambda0=None, S0=None, variant="diagonal", chunk=64,
                    out=None):
    """kdn_forward_noalloc: the forward with the library's static device
    scratch array as its workspace (the C call allocates nothing).  out:
    optional preallocated (o, S_T, lambda_T); otherwise they are allocated
    here, by torch, before the call.  Calls on one GPU share the array and must
    not overlap."""
    lib = load_library()
    d = _forward_desc(q, k, v, a, qnoise, r, variant, chunk)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    lam_shape = (B, H, dk) if d.variant == DIAGONAL else (B, H)
    for x, name, shape in ((lambda0, "lambda0", lam_shape), (S0, "S0", (B, H, dv, dk))):
        if x is not None:
            _gpu(x, name)
            if x.dtype != torch.float32 or tuple(x.shape) != shape:
                raise ValueError(f"{name} must be float32 {shape}")
    if out is not None:
        o, S_T, lam_T = out
    else:
        dev = k.device
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
        S_T = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
        lam_T = torch.empty(lam_shape, dtype=torch.float32, device=dev)
    _check(lib.kdn_forward_noalloc(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                   _ptr(qnoise), _ptr(r), _ptr(lambda0), _ptr(S0), _ptr(o),
                                   _ptr(S_T), _ptr(lam_T), _stream()), "kdn_forward_noalloc")
    return o, S_T, lam_T


def dense_gain(k, a, qnoise, r, P0=None, want_P=True):
    """Exact KDN gains (dense Riccati recursion): k [B,H,T,d_k]; a, qnoise, r
    [B,H,T]; P0 float32 [B,H,d_k,d_k] or None (identity).  Returns (w in k's
    dtype [B,H,T,d_k], P_T float32 [B,H,d_k,d_k] or None)."""
    lib = load_library()
    for n, x in (("k", k), ("a", a), ("qnoise", qnoise), ("r", r)):
        _gpu(x, n)
    B, H, T, dk = k.shape
    d = make_desc(B, H, T, dk, dk, 0, "diagonal", _dtype_code(k.dtype), _dtype_code(a.dtype))
    if P0 is not None:
        _gpu(P0, "P0")
        if P0.dtype != torch.float32 or tuple(P0.shape) != (B, H, dk, dk):
            raise ValueError("P0 must be float32 [B,H,d_k,d_k]")
    w = torch.empty_like(k)
    P_T = torch.empty((B, H, dk, dk), dtype=torch.float32, device=k.device) if want_P else None
    _check(lib.kdn_dense_gain(ctypes.byref(d), _ptr(k), _ptr(a), _ptr(qnoise), _ptr(r),
                              _ptr(P0), _ptr(w), _ptr(P_T), _stream()), "kdn_dense_gain")
    return w, P_T


def forward_dense(q, k, v, a, qnoise, r, P0=None, S0=None, chunk=64):
    """Exact KDN layer forward: kdn_dense_gain, then the memory write and
    read-out with those gains (kdn_chunk_delta).  Returns (o, S_T, P_T)."""
    w, P_T = dense_gain(k, a, qnoise, r, P0)
    o, S_T = chunk_delta(q, k, v, a, w, S0, chunk=chunk)
    return o, S_T, P_T


_blas = None


def blas_handle():
    """This process's hipBLASLt context for the layer's GEMMs (created on first use,
    freed at exit)."""
    global _blas
    if _blas is None:
        lib = load_library()
        h = ctypes.c_void_p()
        _check(lib.kdn_blas_create(ctypes.byref(h)), "kdn_blas_create")
        _blas = h
        atexit.register(lambda: lib.kdn_blas_destroy(h))
    return _blas


def make_layer_desc(B, T, H, d_model, d_k, d_v, chunk, variant, dtype) -> KdnLayerDesc:
    d = KdnLayerDesc()
    d.B, d.T, d.H, d.d_model, d.d_k, d.d_v, d.chunk = B, T, H, d_model, d_k, d_v, chunk
    d.variant = _variant(variant)
    d.dtype = dtype
    return d


def layer_workspace_bytes(d: KdnLayerDesc) -> int:
    return int(load_library().kdn_layer_workspace_bytes(ctypes.byref(d)))


def layer_forward(x, W_in, b_gate, W_out, H, d_k, d_v, lambda0=None, S0=None,
                  variant="diagonal", chunk=64, workspace=None, events=None):
    """KDN layer on given weights (kdn_layer_forward): x [B,T,D] -> y [B,T,D].
    W_in [H(2 d_k + d_v) + 3H, D] and W_out [D, H d_v], out-features major (a
    linear layer's weight layout: y = x W^T), b_gate float32 [3H]; all but
    b_gate in x's dtype.  Returns (y, S_T, lambda_T).  events: optional 10
    torch.cuda.Event around the five stages."""
    lib = load_library()
    for n, t in (("x", x), ("W_in", W_in), ("b_gate", b_gate), ("W_out", W_out)):
        _gpu(t, n)
    B, T, D = x.shape
    code = _dtype_code(x.dtype)
    n_in = H * (2 * d_k + d_v) + 3 * H
    if W_in.dtype != x.dtype or tuple(W_in.shape) != (n_in, D):
        raise ValueError(f"W_in must be {x.dtype} [{n_in}, {D}] (out-features major)")
    if W_out.dtype != x.dtype or tuple(W_out.shape) != (D, H * d_v):
        raise ValueError(f"W_out must be {x.dtype} [{D}, {H * d_v}] (out-features major)")
    if b_gate.dtype != torch.float32 or tuple(b_gate.shape) != (3 * H,):
        raise ValueError(f"b_gate must be float32 [{3 * H}]")
    d = make_layer_desc(B, T, H, D, d_k, d_v, chunk, variant, code)
    lam_shape = (B, H, d_k) if d.variant == DIAGONAL else (B, H)
    for n, t, sh in (("lambda0", lambda0, lam_shape), ("S0", S0, (B, H, d_v, d_k))):
        if t is not None:
            _gpu(t, n)
            if t.dtype != torch.float32 or tuple(t.shape) != sh:
                raise ValueError(f"{n} must be float32 {sh}")
    need = layer_workspace_bytes(d)
    if need == 0:
        raise KdnError("kdn_layer_forward: unsupported layer shape")
    dev = x.device
    ws = workspace if workspace is not None else _workspace(need, dev)
    y = torch.empty((B, T, D), dtype=x.dtype, device=dev)
    S_T = torch.empty((B, H, d_v, d_k), dtype=torch.float32, device=dev)
    lam_T = torch.empty(lam_shape, dtype=torch.float32, device=dev)
    args = (ctypes.byref(d), blas_handle(), _ptr(x), _ptr(W_in), _ptr(b_gate), _ptr(W_out),
            _ptr(lambda0), _ptr(S0), _ptr(y), _ptr(S_T), _ptr(lam_T), _ptr(ws),
            ws.numel() * ws.element_size(), _stream())
    if events is None:
        _check(lib.kdn_layer_forward(*args), "kdn_layer_forward")
    else:
        if len(events) != 10:
            raise ValueError("events: 10 entries (start and stop of five stages)")
        arr = (ctypes.c_void_p * 10)(*[None if e is None else e.cuda_event for e in events])
        _check(lib.kdn_layer_forward_events(*args, arr), "kdn_layer_forward_events")
    return y, S_T, lam_T


def forward_varlen(q, k, v, a, qnoise, r, cu_seqlens, max_seqlen, lambda0=None, S0=None,
                   variant="diagonal", chunk=64, workspace: torch.Tensor | None = None):
    """Forward of a packed batch: q, k [H,T,d_k]; v [H,T,d_v]; a, qnoise, r [H,T]
    with N sequences laid end to end along T (cu_seqlens: int32 [N+1] on the
    GPU; max_seqlen: an int at least the longest length).  Returns (o [H,T,d_v],
    S_T [N,H,d_v,d_k], lambda_T [N,H,d_k] or [N,H])."""
    lib = load_library()
    for n, x in (("q", q), ("k", k), ("v", v), ("a", a), ("qnoise", qnoise), ("r", r),
                 ("cu_seqlens", cu_seqlens)):
        _gpu(x, n)
    H, T, dk = k.shape
    dv = v.shape[-1]
    N = cu_seqlens.shape[0] - 1
    if q.shape != k.shape or v.shape != (H, T, dv) or a.shape != (H, T):
        raise ValueError("q, k [H,T,d_k]; v [H,T,d_v]; a, qnoise, r [H,T]")
    if cu_seqlens.dtype != torch.int32 or N < 0:
        raise ValueError("cu_seqlens must be int32 [N+1]")
    d = make_desc(N, H, T, dk, dv, chunk, variant, _dtype_code(q.dtype), _dtype_code(a.dtype))
    lam_shape = (N, H, dk) if d.variant == DIAGONAL else (N, H)
    for name, x, shape in (("lambda0", lambda0, lam_shape), ("S0", S0, (N, H, dv, dk))):
        if x is not None:
            _gpu(x, name)
            if x.dtype != torch.float32 or tuple(x.shape) != shape:
                raise ValueError(f"{name} must be float32 {shape}")
    dev = k.device
    o = torch.empty((H, T, dv), dtype=q.dtype, device=dev)
    S_T = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
    lam_T = torch.empty(lam_shape, dtype=torch.float32, device=dev)
    need = lib.kdn_forward_varlen_workspace_bytes(ctypes.byref(d))
    if need == 0:
        _check(lib.kdn_validate(ctypes.byref(d)), "kdn_forward_varlen")
    ws = workspace if workspace is not None else _workspace(need, dev)
    _check(lib.kdn_forward_varlen(ctypes.byref(d), _ptr(cu_seqlens), int(max_seqlen), _ptr(q),
                                  _ptr(k), _ptr(v), _ptr(a), _ptr(qnoise), _ptr(r),
                                  _ptr(lambda0), _ptr(S0), _ptr(o), _ptr(S_T), _ptr(lam_T),
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream()),
           "kdn_forward_varlen")
    return o, S_T, lam_T


def backward_workspace_bytes(desc: KdnDesc) -> int:
    return load_library().kdn_backward_workspace_bytes(ctypes.byref(desc))


def backward(q, k, v, a, qnoise, r, dO, lambda0=None, S0=None, dS_T=None, dlambda_T=None,
             variant="diagonal", chunk=64, workspace: torch.Tensor | None = None, out=None,
             events=None, kept: torch.Tensor | None = None) -> dict:
    """Gradients of <dO, o> + <dS_T, S_T> + <dlambda_T, lambda_T> with respect
    to q, k, v, a, qnoise, r, lambda0 and S0, as float32 tensors in a dict
    (keys dq, dk, dv, da, dqnoise, dr, dlambda0, dS0).

    out: optional dict of preallocated outputs with those keys; events:
    optional list of 14 torch.cuda.Event (already recorded once), start and
    stop of the seven stages.  kept: the workspace that forward(..., keep=)
    filled for these same inputs; the backward then skips its recompute
    (kdn_backward_kept)."""
    lib = load_library()
    d = _forward_desc(q, k, v, a, qnoise, r, variant, chunk)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    lam_shape = (B, H, dk) if d.variant == DIAGONAL else (B, H)
    _gpu(dO, "dO")
    if dO.dtype != q.dtype or tuple(dO.shape) != (B, H, T, dv):
        raise ValueError("dO must be [B,H,T,d_v] in the dtype of q, k, v")
    for name, x, shape in (("lambda0", lambda0, lam_shape), ("S0", S0, (B, H, dv, dk)),
                           ("dS_T", dS_T, (B, H, dv, dk)), ("dlambda_T", dlambda_T, lam_shape)):
        if x is not None:
            _gpu(x, name)
            if x.dtype != torch.float32 or tuple(x.shape) != shape:
                raise ValueError(f"{name} must be float32 {shape}")
    dev = k.device
    shapes = {"dq": (B, H, T, dk), "dk": (B, H, T, dk), "dv": (B, H, T, dv),
              "da": (B, H, T), "dqnoise": (B, H, T), "dr": (B, H, T),
              "dlambda0": lam_shape, "dS0": (B, H, dv, dk)}
    g = out if out is not None else {
        n: torch.empty(sh, dtype=torch.float32, device=dev) for n, sh in shapes.items()}
    need = lib.kdn_backward_workspace_bytes(ctypes.byref(d))
    if need == 0:
        _check(lib.kdn_validate(ctypes.byref(d)), "kdn_backward")
        raise KdnError("kdn_backward: shape not supported by the backward kernels")
    ws = kept if kept is not None else (workspace if workspace is not None
                                         else _workspace(need, dev))
    args = (ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(qnoise), _ptr(r),
            _ptr(lambda0), _ptr(S0), _ptr(dO), _ptr(dS_T), _ptr(dlambda_T),
            *(_ptr(g[n]) for n in ("dq", "dk", "dv", "da", "dqnoise", "dr", "dlambda0", "dS0")),
            _ptr(ws), ws.numel() * ws.element_size(), _stream())
    name = "kdn_backward_kept" if kept is not None else "kdn_backward"
    if events is None:
        _check(getattr(lib, name)(*args), name)
    else:
        if len(events) != 14:
            raise ValueError("events: 14 entries (start and stop of seven stages)")
        arr = (ctypes.c_void_p * 14)(*[None if e is None else e.cuda_event for e in events])
        _check(getattr(lib, name + "_events")(*args, arr), name + "_events")
    return g


def mobius_scan(k, a, qnoise, r, lambda0=None, variant="diagonal", chunk=64,
                lambda_minus=True, lambda_chunk=False):
    """Precision scan alone.  Returns dict with lambda_T and, if asked, lambda_minus
    [B,H,T,d_k] / [B,H,T] and lambda_chunk [B,H,nc+1,d_k] / [B,H,nc+1]."""
    lib = load_library()
    for n, x in (("k", k), ("a", a), ("qnoise", qnoise), ("r", r)):
        _gpu(x, n)
    B, H, T, dk = k.shape
    d = make_desc(B, H, T, dk, dk, chunk, variant, _dtype_code(k.dtype), _dtype_code(a.dtype))
    diag = d.variant == DIAGONAL
    dev = k.device
    nc = (T + chunk - 1) // chunk
    out = {"lambda_T": torch.empty((B, H, dk) if diag else (B, H), dtype=torch.float32,
                                   device=dev)}
    if lambda_minus:
        out["lambda_minus"] = torch.empty((B, H, T, dk) if diag else (B, H, T),
                                          dtype=torch.float32, device=dev)
    if lambda_chunk:
        out["lambda_chunk"] = torch.empty((B, H, nc + 1, dk) if diag else (B, H, nc + 1),
                                          dtype=torch.float32, device=dev)
    if lambda0 is not None:
        _gpu(lambda0, "lambda0")
    need = lib.kdn_mobius_scan_workspace_bytes(ctypes.byref(d))
    if need == 0:
        _check(3, "kdn_mobius_scan")
    ws = _workspace(need, dev)
    _check(lib.kdn_mobius_scan(ctypes.byref(d), _ptr(k), _ptr(a), _ptr(qnoise), _ptr(r),
                               _ptr(lambda0), _ptr(out.get("lambda_minus")),
                               _ptr(out.get("lambda_chunk")), _ptr(out["lambda_T"]), _ptr(ws),
                               ws.numel(), _stream()), "kdn_mobius_scan")
    return out


def gain(k, r, lambda_minus, variant="diagonal", gain_dtype=None):
    """Kalman gain keys w [B,H,T,d_k] from predictive precisions."""
    lib = load_library()
    _gpu(k, "k")
    _gpu(r, "r")
    _gpu(lambda_minus, "lambda_minus")
    B, H, T, dk = k.shape
    gdt = k.dtype if gain_dtype is None else gain_dtype
    d = make_desc(B, H, T, dk, dk, 64, variant, _dtype_code(k.dtype), _dtype_code(r.dtype),
                  _dtype_code(gdt))
    w = torch.empty((B, H, T, dk), dtype=gdt, device=k.device)
    _check(lib.kdn_gain(ctypes.byref(d), _ptr(k), _ptr(r), _ptr(lambda_minus), _ptr(w),
                        _stream()), "kdn_gain")
    return w


def chunk_delta(q, k, v, a, w, S0=None, chunk=64):
    """Chunkwise memory write / read-out with given gain keys w.  Returns (o, S_T)."""
    lib = load_library()
    for n, x in (("q", q), ("k", k), ("v", v), ("a", a), ("w", w)):
        _gpu(x, n)
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    d = make_desc(B, H, T, dk, dv, chunk, "diagonal", _dtype_code(q.dtype),
                  _dtype_code(a.dtype), _dtype_code(w.dtype))
    o = torch.empty((B, H, T, dv), dtype=q.dtype, device=k.device)
    S_T = torch.empty((B, H, dv, dk), dtype=torch.float32, device=k.device)
    need = lib.kdn_chunk_delta_workspace_bytes(ctypes.byref(d))
    if need == 0:
        _check(lib.kdn_validate(ctypes.byref(d)) or 3, "kdn_chunk_delta")
    ws = _workspace(need, k.device)
    if S0 is not None:
        _gpu(S0, "S0")
    _check(lib.kdn_chunk_delta(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(w),
                               _ptr(S0), _ptr(o), _ptr(S_T), _ptr(ws), ws.numel(), _stream()),
           "kdn_chunk_delta")
    return o, S_T


def decode_step(q, k, v, a, qnoise, r, S, lam, variant="diagonal", out=None):
    """One in-place decode step on cached (S, lam).  q, k [N,H,d_k]; v [N,H,d_v];
    a, qnoise, r [N,H]; S float32 [N,H,d_v,d_k]; lam float32 [N,H,d_k] or [N,H]."""
    lib = load_library()
    for n, x in (("q", q), ("k", k), ("v", v), ("a", a), ("qnoise", qnoise), ("r", r),
                 ("S", S), ("lam", lam)):
        _gpu(x, n)
    N, H, dk = k.shape
    dv = v.shape[-1]
    if S.dtype != torch.float32 or tuple(S.shape) != (N, H, dv, dk):
        raise ValueError("S must be float32 [N,H,d_v,d_k]")
    d = make_desc(N, H, 1, dk, dv, 0, variant, _dtype_code(q.dtype), _dtype_code(a.dtype))
    lam_shape = (N, H, dk) if d.variant == DIAGONAL else (N, H)
    if lam.dtype != torch.float32 or tuple(lam.shape) != lam_shape:
        raise ValueError(f"lam must be float32 {lam_shape}")
    o = out if out is not None else torch.empty((N, H, dv), dtype=q.dtype, device=k.device)
    _check(lib.kdn_decode_step(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                               _ptr(qnoise), _ptr(r), _ptr(S), _ptr(lam), _ptr(o), _stream()),
           "kdn_decode_step")
    return o


def decode_step_indexed(q, k, v, a, qnoise, r, S_cache, lam_cache, slot, variant="diagonal",
                        out=None):
    """Continuous-batching decode step: sequence n of the active batch (q, k
    [N,H,d_k]; v [N,H,d_v]; a, qnoise, r [N,H]) reads and updates its state at
    cache slot slot[n] (int32 [N] on the GPU; outside [0, n_slots): idle) of
    S_cache float32 [n_slots,H,d_v,d_k] and lam_cache [n_slots,H,d_k] or
    [n_slots,H].  Returns o [N,H,d_v] (rows of idle sequences are left as they
    were in `out`, or uninitialised)."""
    lib = load_library()
    for n, x in (("q", q), ("k", k), ("v", v), ("a", a), ("qnoise", qnoise), ("r", r),
                 ("S_cache", S_cache), ("lam_cache", lam_cache), ("slot", slot)):
        _gpu(x, n)
    N, H, dk = k.shape
    dv = v.shape[-1]
    n_slots = S_cache.shape[0]
    if S_cache.dtype != torch.float32 or tuple(S_cache.shape) != (n_slots, H, dv, dk):
        raise ValueError("S_cache must be float32 [n_slots,H,d_v,d_k]")
    if slot.dtype != torch.int32 or tuple(slot.shape) != (N,):
        raise ValueError("slot must be int32 [N]")
    d = make_desc(N, H, 1, dk, dv, 0, variant, _dtype_code(q.dtype), _dtype_code(a.dtype))
    lam_shape = (n_slots, H, dk) if d.variant == DIAGONAL else (n_slots, H)
    if lam_cache.dtype != torch.float32 or tuple(lam_cache.shape) != lam_shape:
        raise ValueError(f"lam_cache must be float32 {lam_shape}")
    o = out if out is not None else torch.empty((N, H, dv), dtype=q.dtype, device=k.device)
    _check(lib.kdn_decode_step_indexed(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                       _ptr(qnoise), _ptr(r), _ptr(S_cache), _ptr(lam_cache),
                                       _ptr(slot), n_slots, _ptr(o), _stream()),
           "kdn_decode_step_indexed")
    return o
