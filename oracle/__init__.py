"""fp64 CPU oracle of the KDN layer forward and decode step.

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's
CPU-baseline leg may call this package; the GPU library never does, and the
two share no code.  The arithmetic lives in ``kdn_oracle.c`` (plain C loops in
double precision, threads across independent heads); this module only builds
it with gcc and marshals numpy arrays through ctypes.

Which passage each step follows is stated in the header of ``kdn_oracle.c``
("Kalman Delta Networks: Uncertainty-aware Associative Memory", English
abstract; ai-feeds.com summary, section 方法, steps 1-3).  The layer around
the recurrence (projections, normalisation, gates) is ``oracle.layer``, in
numpy float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_kdn_oracle.so")
# another build of the same source (the sanitizer test loads an
# AddressSanitizer / UndefinedBehaviorSanitizer build this way)
_LIB_OVERRIDE = os.environ.get("KDN_ORACLE_LIB")
_lib = None

DIAGONAL = 0
ISOTROPIC = 1


def build(force: bool = True) -> str:
    """Compile kdn_oracle.c into a shared library next to it (gcc -O2)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.kdn_oracle_forward.argtypes = [I, I, I, I, I, I] + [P] * 13 + [I]
        lib.kdn_oracle_forward.restype = I
        lib.kdn_oracle_decode_step.argtypes = [I, I, I, I, I] + [P] * 9 + [I]
        lib.kdn_oracle_decode_step.restype = I
        lib.kdn_oracle_backward.argtypes = [I, I, I, I, I, I] + [P] * 19 + [I]
        lib.kdn_oracle_backward.restype = I
        lib.kdn_oracle_forward_dense.argtypes = [I, I, I, I, I] + [P] * 12 + [I]
        lib.kdn_oracle_forward_dense.restype = I
        _lib = lib
    return _lib


def _variant(variant) -> int:
    if variant in (DIAGONAL, "diagonal", "diag"):
        return DIAGONAL
    if variant in (ISOTROPIC, "isotropic", "iso"):
        return ISOTROPIC
    raise ValueError(f"unknown variant {variant!r}")


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _ptr(x):
    return None if x is None else x.ctypes.data


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def forward(q, k, v, a, nu, r, lambda0=None, S0=None, variant="diagonal",
            debug: bool = False, threads: int | None = None) -> dict:
    """Token-by-token fp64 KDN forward.

    q, k: [B,H,T,d_k]; v: [B,H,T,d_v]; a, nu, r: [B,H,T]; lambda0: [B,H,d_k]
    (diagonal) or [B,H] (isotropic) or None (ones); S0: [B,H,d_v,d_k] or None
    (zeros).  Values are taken as float32 (bf16 inputs widen exactly).
    Returns float64 arrays o [B,H,T,d_v], S_T, lambda_T and, with debug=True,
    lambda_minus ([B,H,T,d_k] or [B,H,T]) and w ([B,H,T,d_k]).
    """
    lib = _load()
    var = _variant(variant)
    q, k, v, a, nu, r = (_f32(x) for x in (q, k, v, a, nu, r))
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    assert q.shape == k.shape and v.shape == (B, H, T, dv)
    assert a.shape == (B, H, T) and nu.shape == a.shape and r.shape == a.shape
    lam_shape = (B, H, dk) if var == DIAGONAL else (B, H)
    if lambda0 is not None:
        lambda0 = _f32(lambda0)
        assert lambda0.shape == lam_shape, (lambda0.shape, lam_shape)
    if S0 is not None:
        S0 = _f32(S0)
        assert S0.shape == (B, H, dv, dk)
    o = np.empty((B, H, T, dv), np.float64)
    S_T = np.empty((B, H, dv, dk), np.float64)
    lam_T = np.empty(lam_shape, np.float64)
    lm = np.empty((B, H, T, dk) if var == DIAGONAL else (B, H, T), np.float64) if debug else None
    w = np.empty((B, H, T, dk), np.float64) if debug else None
    rc = lib.kdn_oracle_forward(B, H, T, dk, dv, var, _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                _ptr(nu), _ptr(r), _ptr(lambda0), _ptr(S0), _ptr(o),
                                _ptr(S_T), _ptr(lam_T), _ptr(lm), _ptr(w),
                                threads or default_threads())
    if rc != 0:
        raise ValueError(f"kdn_oracle_forward rejected its arguments (code {rc})")
    out = {"o": o, "S_T": S_T, "lambda_T": lam_T}
    if debug:
        out["lambda_minus"] = lm
        out["w"] = w
    return out


def decode_step(q, k, v, a, nu, r, S, lam, variant="diagonal", threads: int | None = None):
    """One in-place fp64 decode step on cached state.

    q, k: [N,H,d_k]; v: [N,H,d_v]; a, nu, r: [N,H]; S: float64 [N,H,d_v,d_k]
    and lam: float64 [N,H,d_k] (diagonal) or [N,H] (isotropic), both C-contiguous
    and updated in place.  Returns o as float64 [N,H,d_v].
    """
    lib = _load()
    var = _variant(variant)
    q, k, v, a, nu, r = (_f32(x) for x in (q, k, v, a, nu, r))
    N, H, dk = k.shape
    dv = v.shape[-1]
    assert S.dtype == np.float64 and S.flags.c_contiguous and S.shape == (N, H, dv, dk)
    assert lam.dtype == np.float64 and lam.flags.c_contiguous
    assert lam.shape == ((N, H, dk) if var == DIAGONAL else (N, H))
    o = np.empty((N, H, dv), np.float64)
    rc = lib.kdn_oracle_decode_step(N, H, dk, dv, var, _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                    _ptr(nu), _ptr(r), _ptr(S), _ptr(lam), _ptr(o),
                                    threads or default_threads())
    if rc != 0:
        raise ValueError(f"kdn_oracle_decode_step rejected its arguments (code {rc})")
    return o


def backward(q, k, v, a, nu, r, dO, lambda0=None, S0=None, dS_T=None, dlambda_T=None,
             variant="diagonal", threads: int | None = None) -> dict:
    """fp64 gradient of L = <dO, o> + <dS_T, S_T> + <dlambda_T, lambda_T> (the
    last two taken as zero when None) with respect to every input of
    ``forward``: returns float64 arrays dq, dk, dv, da, dnu, dr, dlambda0, dS0
    shaped like the inputs (dlambda0 and dS0 also when lambda0 / S0 were None,
    the defaults ones / zeros being the point of evaluation)."""
    lib = _load()
    var = _variant(variant)
    q, k, v, a, nu, r, dO = (_f32(x) for x in (q, k, v, a, nu, r, dO))
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    assert q.shape == k.shape and v.shape == (B, H, T, dv) and dO.shape == v.shape
    assert a.shape == (B, H, T) and nu.shape == a.shape and r.shape == a.shape
    lam_shape = (B, H, dk) if var == DIAGONAL else (B, H)
    if lambda0 is not None:
        lambda0 = _f32(lambda0)
        assert lambda0.shape == lam_shape
    if S0 is not None:
        S0 = _f32(S0)
        assert S0.shape == (B, H, dv, dk)
    if dS_T is not None:
        dS_T = _f32(dS_T)
        assert dS_T.shape == (B, H, dv, dk)
    if dlambda_T is not None:
        dlambda_T = _f32(dlambda_T)
        assert dlambda_T.shape == lam_shape
    out = {
        "dq": np.empty((B, H, T, dk)), "dk": np.empty((B, H, T, dk)),
        "dv": np.empty((B, H, T, dv)), "da": np.empty((B, H, T)),
        "dnu": np.empty((B, H, T)), "dr": np.empty((B, H, T)),
        "dlambda0": np.empty(lam_shape), "dS0": np.empty((B, H, dv, dk)),
    }
    rc = lib.kdn_oracle_backward(
        B, H, T, dk, dv, var, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(nu), _ptr(r),
        _ptr(lambda0), _ptr(S0), _ptr(dO), _ptr(dS_T), _ptr(dlambda_T),
        *(_ptr(out[n]) for n in ("dq", "dk", "dv", "da", "dnu", "dr", "dlambda0", "dS0")),
        threads or default_threads())
    if rc != 0:
        raise ValueError(f"kdn_oracle_backward rejected its arguments (code {rc})")
    return out


def forward_dense(q, k, v, a, nu, r, P0=None, S0=None, debug=False,
                  threads: int | None = None) -> dict:
    """Exact KDN (dense Riccati recursion, one d_k x d_k covariance per head),
    fp64.  P0: [B,H,d_k,d_k] prior covariance or None (identity).  Returns o,
    S_T, P_T and, with debug=True, the gains w [B,H,T,d_k]."""
    lib = _load()
    q, k, v, a, nu, r = (_f32(x) for x in (q, k, v, a, nu, r))
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    if P0 is not None:
        P0 = _f32(P0)
        assert P0.shape == (B, H, dk, dk)
    if S0 is not None:
        S0 = _f32(S0)
        assert S0.shape == (B, H, dv, dk)
    o = np.empty((B, H, T, dv))
    S_T = np.empty((B, H, dv, dk))
    P_T = np.empty((B, H, dk, dk))
    w = np.empty((B, H, T, dk)) if debug else None
    rc = lib.kdn_oracle_forward_dense(B, H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                      _ptr(nu), _ptr(r), _ptr(P0), _ptr(S0), _ptr(o), _ptr(S_T),
                                      _ptr(P_T), _ptr(w), threads or default_threads())
    if rc != 0:
        raise ValueError(f"kdn_oracle_forward_dense rejected its arguments (code {rc})")
    out = {"o": o, "S_T": S_T, "P_T": P_T}
    if debug:
        out["w"] = w
    return out
