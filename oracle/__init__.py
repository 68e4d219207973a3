"""CPU oracle for the Complex KDA (CKDA) recurrence -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  The product library never imports, links or calls it, and it
imports nothing from the product package.

The heavy lifting is the token-by-token fp64 recurrence in ``ckda_oracle.c``
(see that file's header for the update rule and where it is stated).  This
module loads it through ctypes and adds two small helpers built on it:

* :func:`backward` -- the reverse-mode gradient of the same recurrence (the
  adjoint steps are written out in ``ckda_oracle.c``).
* :func:`transition` -- the one-token transition matrix of the oracle itself,
  obtained by running it with S0 = I and v = 0 (then S_1 = A S0 = A).
* :mod:`oracle.chunked` -- a dense chunked (WY/UT) fp64 formulation in NumPy,
  used only to check on tiny inputs that the chunked algebra equals the
  sequential recurrence.

Inputs are taken as NumPy arrays of any float dtype and widened to fp64
exactly (bf16 and fp32 values are exactly representable in fp64).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ckda_oracle.c")
# CKDA_ORACLE_SANITIZE=1 builds and loads an AddressSanitizer + UBSan copy
# instead (the process must then preload gcc's libasan and libubsan).
_SANITIZE = os.environ.get("CKDA_ORACLE_SANITIZE") == "1"
_LIB_PATH = os.path.join(_HERE, "libckda_oracle_san.so" if _SANITIZE else "libckda_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/libckda_oracle.so`` (or the
    sanitizer copy, see above)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        flags = (["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=undefined"] if _SANITIZE else ["-O2"])
        subprocess.check_call(["gcc", *flags, "-std=c99", "-shared", "-fPIC", "-pthread",
                               _SRC, "-o", tmp])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        ci = ctypes.c_int
        lib.ckda_oracle_forward.argtypes = [dp, dp, dp, dp, dp, dp, i64p, ci, ci, ci, ci,
                                            ci, ci, dp, dp, ci]
        lib.ckda_oracle_forward.restype = ci
        lib.ckda_oracle_decode.argtypes = [dp, dp, dp, dp, dp, dp, dp, ci, ci, ci, ci, ci]
        lib.ckda_oracle_decode.restype = ci
        lib.ckda_oracle_backward.argtypes = [dp, dp, dp, dp, dp, dp, i64p, ci, ci, ci, ci, ci,
                                             ci, dp, dp, dp, dp, dp, dp, dp, dp, ci]
        lib.ckda_oracle_backward.restype = ci
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
               else (os.cpu_count() or 1))


def forward(q, k, v, g, beta, S0=None, cu_seqlens=None, nthreads: int | None = None):
    """Token-by-token CKDA forward in fp64.

    Shapes: q, k, g ``[B, T, H, dk]``; v ``[B, T, H, dv]``; beta ``[B, T, H]``;
    S0 ``[N, H, dk, dv]`` or None (zero state); cu_seqlens ``[N+1]`` or None.
    With cu_seqlens, B must be 1 and the sequences are the packed token ranges
    ``[cu[n], cu[n+1])``.  Returns ``(o [B, T, H, dv], S_T [N, H, dk, dv])``.
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or v.shape[:3] != (B, T, H) \
            or beta.shape != (B, T, H):
        raise ValueError("shape mismatch")
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N = cu.shape[0] - 1
        if B != 1:
            raise ValueError("packed sequences need B == 1")
    else:
        cu = None
        N = B
    S0a = None if S0 is None else _f64(S0)
    if S0a is not None and S0a.shape != (N, H, dk, dv):
        raise ValueError("S0 shape mismatch")
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    S_T = np.zeros((N, H, dk, dv), dtype=np.float64)
    cu_p = None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    rc = _load().ckda_oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(S0a), cu_p, B, T, H, dk, dv, N, _ptr(o),
                                     _ptr(S_T), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected the sizes")
    return o, S_T


def l2_normalise(x):
    """Each row (last axis) scaled by (sum x^2 + 1e-6)^(-1/2), in fp64: the
    key/query normalisation the fused forward option applies."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-6)


def backward(q, k, v, g, beta, do, S0=None, dS_T=None, cu_seqlens=None,
             nthreads: int | None = None, normalize_qk: bool = False):
    """Reverse-mode gradient of the token-by-token forward, in fp64.

    For upstream gradients ``do`` (``[B, T, H, dv]``, of o) and ``dS_T``
    (``[N, H, dk, dv]`` or None for zero, of the final states), returns the
    gradient of ``sum(do * o) + sum(dS_T * S_T)`` with respect to the inputs:
    ``(dq, dk, dv, dg, dbeta, dS0)``, shaped like q, k, v, g, beta and
    ``[N, H, dk, dv]``.  ``dg`` is the derivative with respect to the signed
    gate alpha itself.  Rows outside every packed sequence get zero gradients.

    ``normalize_qk``: the forward first replaces every row x of q and of k by
    x s with s = (sum x^2 + 1e-6)^(-1/2); the chain rule through that step
    (d x = s (d xh - xh (xh . d xh)) with xh = x s) follows the recurrence's
    gradient with respect to the normalised rows.
    """
    if normalize_qk:
        qh, kh = l2_normalise(q), l2_normalise(k)
        out = list(backward(qh, kh, v, g, beta, do, S0=S0, dS_T=dS_T, cu_seqlens=cu_seqlens,
                            nthreads=nthreads))
        for idx, (x, xh) in ((0, (q, qh)), (1, (k, kh))):
            x = _f64(x)
            s = 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-6)
            dxh = out[idx]
            out[idx] = s * (dxh - xh * np.sum(xh * dxh, axis=-1, keepdims=True))
        return tuple(out)
    q, k, v, g, beta, do = map(_f64, (q, k, v, g, beta, do))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or v.shape[:3] != (B, T, H) \
            or beta.shape != (B, T, H) or do.shape != v.shape:
        raise ValueError("shape mismatch")
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N = cu.shape[0] - 1
        if B != 1:
            raise ValueError("packed sequences need B == 1")
    else:
        cu = None
        N = B
    S0a = None if S0 is None else _f64(S0)
    dSTa = None if dS_T is None else _f64(dS_T)
    for a in (S0a, dSTa):
        if a is not None and a.shape != (N, H, dk, dv):
            raise ValueError("state shape mismatch")
    out = [np.zeros(x.shape, dtype=np.float64) for x in (q, k, v, g, beta)]
    dS0 = np.zeros((N, H, dk, dv), dtype=np.float64)
    cu_p = None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    rc = _load().ckda_oracle_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      _ptr(S0a), cu_p, B, T, H, dk, dv, N, _ptr(do),
                                      _ptr(dSTa), *[_ptr(x) for x in out], _ptr(dS0),
                                      nthreads or default_threads())
    if rc == -2:
        raise MemoryError("oracle backward ran out of host memory")
    if rc != 0:
        raise ValueError("oracle rejected the sizes")
    return (*out, dS0)


def decode_step(q, k, v, g, beta, S, nthreads: int | None = None):
    """One decode step.  ``S`` ([N, H, dk, dv], fp64, C-contiguous) is updated
    in place; returns o ``[N, H, dv]``."""
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    if S.dtype != np.float64 or not S.flags.c_contiguous:
        raise ValueError("S must be a C-contiguous float64 array (updated in place)")
    N, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((N, H, dv), dtype=np.float64)
    rc = _load().ckda_oracle_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(S), _ptr(o), N, H, dk, dv,
                                    nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected the sizes")
    return o


def transition(k, g, beta):
    """The oracle's own one-token transition matrix A (dk x dk).

    Runs the oracle on one token with S0 = I (so dv = dk) and v = 0; then
    S_1 = A S0 + beta k 0^T = A.
    """
    k = _f64(k).reshape(-1)
    g = _f64(g).reshape(-1)
    dk = k.shape[0]
    one = lambda a: a.reshape(1, 1, 1, -1)
    q = np.zeros(dk)
    v = np.zeros(dk)
    b = np.array(float(beta)).reshape(1, 1, 1)
    S0 = np.eye(dk).reshape(1, 1, dk, dk)
    _, S_T = forward(one(q), one(k), one(v), one(g), b, S0=S0, nthreads=1)
    return S_T[0, 0]


__all__ = ["build", "forward", "backward", "l2_normalise", "decode_step", "transition",
           "default_threads"]
