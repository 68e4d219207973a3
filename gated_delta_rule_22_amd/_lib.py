"""ctypes binding of ``libckda.so`` (declared in ``include/ckda.h``).

Argument marshalling only: shapes and dtypes are read from torch tensors,
outputs and the workspace are allocated with torch (device memory), and the
current HIP stream is passed through.  Every step of the computation runs in
the library's kernels.  There is no fallback: if the library is missing or a
call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# CKDA_LIB names another build of the same library (e.g. a host-sanitized one).
LIB_PATH = os.environ.get("CKDA_LIB") or os.path.join(_PKG, "libckda.so")

CKDA_BF16 = 0
CKDA_F32 = 1

_lib = None


class CkdaError(RuntimeError):
    pass


def library() -> ctypes.CDLL:
    """Load ``libckda.so`` once and declare its signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise CkdaError(f"{LIB_PATH} is not built; run `python -m gated_delta_rule_22_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, ci, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        lib.ckda_abi_version.argtypes = []
        lib.ckda_abi_version.restype = ci
        lib.ckda_status_string.argtypes = [ci]
        lib.ckda_status_string.restype = ctypes.c_char_p
        lib.ckda_forward_workspace_bytes.argtypes = [ci] * 7
        lib.ckda_forward_workspace_bytes.restype = sz
        lib.ckda_forward_ex_workspace_bytes.argtypes = [ci] * 8
        lib.ckda_forward_ex_workspace_bytes.restype = sz
        lib.ckda_forward.argtypes = [vp] * 7 + [ci] * 7 + [vp, vp, vp, sz, vp]
        lib.ckda_forward.restype = ci
        lib.kda_forward.argtypes = [vp] * 7 + [ci] * 7 + [vp, vp, vp, sz, vp]
        lib.kda_forward.restype = ci
        lib.ckda_forward_ex.argtypes = [vp] * 7 + [ci] * 8 + [vp, vp, vp, sz, vp]
        lib.ckda_forward_ex.restype = ci
        lib.ckda_forward_noalloc.argtypes = [vp] * 7 + [ci] * 8 + [vp, vp, vp]
        lib.ckda_forward_noalloc.restype = ci
        lib.ckda_forward_noalloc_max_bytes.argtypes = []
        lib.ckda_forward_noalloc_max_bytes.restype = sz
        lib.ckda_backward_workspace_bytes.argtypes = [ci] * 7
        lib.ckda_backward_workspace_bytes.restype = sz
        lib.ckda_backward.argtypes = [vp] * 7 + [ci] * 7 + [vp] * 8 + [vp, sz, vp]
        lib.ckda_backward.restype = ci
        lib.kda_backward.argtypes = [vp] * 7 + [ci] * 7 + [vp] * 8 + [vp, sz, vp]
        lib.kda_backward.restype = ci
        lib.ckda_backward_ex.argtypes = [vp] * 7 + [ci] * 8 + [vp] * 8 + [vp, sz, vp]
        lib.ckda_backward_ex.restype = ci
        lib.ckda_decode_step.argtypes = [vp] * 7 + [ci] * 5 + [vp]
        lib.ckda_decode_step.restype = ci
        _lib = lib
    return _lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return CKDA_BF16
    if t.dtype == torch.float32:
        return CKDA_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(status: int, what: str):
    if status != 0:
        msg = library().ckda_status_string(status).decode()
        raise CkdaError(f"{what} failed with status {status}: {msg}")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def forward_workspace_bytes(B, T, H, dk, dv, N, dtype, options=0) -> int:
    code = dtype if isinstance(dtype, int) else (CKDA_BF16 if dtype == torch.bfloat16 else CKDA_F32)
    if options:
        return int(library().ckda_forward_ex_workspace_bytes(B, T, H, dk, dv, N, code, options))
    return int(library().ckda_forward_workspace_bytes(B, T, H, dk, dv, N, code))


def _need(t, name, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


OPT_KDA, OPT_QK_L2NORM, OPT_O_BF16, OPT_SPLIT = 1, 2, 4, 8   # CKDA_OPT_* in include/ckda.h


def forward(q, k, v, g, beta, S0=None, cu_seqlens=None, *, out=None, final_state=None,
            workspace=None, output_final_state=True, normalize_qk=False,
            out_dtype=torch.float32, kda=False, no_alloc=False, split=False):
    """CKDA chunkwise forward.  Returns ``(o, S_T)`` (``S_T`` is None when
    ``output_final_state`` is False).  See ``ckda_forward`` in include/ckda.h
    for shapes; ``final_state`` may be ``S0`` itself to advance it in place.

    ``normalize_qk`` (L2-normalise q and k rows in the kernel), ``out_dtype``
    (``torch.bfloat16`` for a bf16 ``o``) and ``kda`` (gate signs ignored) map
    to the options of ``ckda_forward_ex``; with none of them set the call goes
    to ``ckda_forward``.  ``no_alloc=True`` calls ``ckda_forward_noalloc``,
    which uses the library's fixed scratch instead of a workspace (pass
    ``out``, and ``final_state`` or ``output_final_state=False``, so that
    nothing is allocated here either).  ``split=True`` runs the two-kernel
    hand-off (``CKDA_OPT_SPLIT``) in place of the fused kernel."""
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")
    opts = ((OPT_KDA if kda else 0) | (OPT_QK_L2NORM if normalize_qk else 0)
            | (OPT_O_BF16 if out_dtype == torch.bfloat16 else 0) | (OPT_SPLIT if split else 0))
    entry = "ckda_forward_noalloc" if no_alloc else (
        "ckda_forward_ex" if opts else "ckda_forward")
    return _forward(entry, q, k, v, g, beta, S0, cu_seqlens, out, final_state, workspace,
                    output_final_state, opts)


def kda_forward(q, k, v, g, beta, S0=None, cu_seqlens=None, *, out=None, final_state=None,
                workspace=None, output_final_state=True):
    """KDA mode of the forward (gate signs ignored, |g| used); same arguments and
    results as :func:`forward`.  See ``kda_forward`` in include/ckda.h."""
    return _forward("kda_forward", q, k, v, g, beta, S0, cu_seqlens, out, final_state,
                    workspace, output_final_state)


def _forward(entry, q, k, v, g, beta, S0, cu_seqlens, out, final_state, workspace,
             output_final_state, opts=0):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need(k, "k", shape=(B, T, H, dk))
    _need(v, "v", shape=(B, T, H, dv))
    _need(g, "g", torch.float32, (B, T, H, dk))
    _need(beta, "beta", torch.float32, (B, T, H))
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if S0 is not None:
        _need(S0, "S0", torch.float32, (N, H, dk, dv))
    dev = q.device
    o_dt = torch.bfloat16 if opts & OPT_O_BF16 else torch.float32
    o = out if out is not None else torch.empty((B, T, H, dv), dtype=o_dt, device=dev)
    _need(o, "out", o_dt, (B, T, H, dv))
    S_T = None
    if output_final_state:
        S_T = final_state if final_state is not None else torch.empty(
            (N, H, dk, dv), dtype=torch.float32, device=dev)
        _need(S_T, "final_state", torch.float32, (N, H, dk, dv))
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(cu_seqlens),
            B, T, H, dk, dv, N, code)
    if entry == "ckda_forward_noalloc":
        st = library().ckda_forward_noalloc(*head, opts, _ptr(o), _ptr(S_T), _stream(dev))
        _check(st, entry)
        return o, S_T
    ws_bytes = forward_workspace_bytes(B, T, H, dk, dv, N, code, opts)
    if workspace is None or workspace.numel() * workspace.element_size() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    tail = (_ptr(o), _ptr(S_T), _ptr(workspace), ws_bytes, _stream(dev))
    fn = getattr(library(), entry)
    st = fn(*head, opts, *tail) if entry == "ckda_forward_ex" else fn(*head, *tail)
    _check(st, entry)
    return o, S_T


def backward_workspace_bytes(B, T, H, dk, dv, N, dtype) -> int:
    code = dtype if isinstance(dtype, int) else (CKDA_BF16 if dtype == torch.bfloat16 else CKDA_F32)
    return int(library().ckda_backward_workspace_bytes(B, T, H, dk, dv, N, code))


def backward(q, k, v, g, beta, do, S0=None, dS_T=None, cu_seqlens=None, *, workspace=None,
             need_dS0=True, kda=False, normalize_qk=False):
    """Gradients of ``sum(do * o) + sum(dS_T * S_T)`` for the forward's inputs:
    returns ``(dq, dk, dv, dg, dbeta, dS0)`` as fp32 tensors (``dS0`` is None
    when ``need_dS0`` is False).  See ``ckda_backward`` in include/ckda.h;
    ``kda=True`` calls ``kda_backward`` (the backward of :func:`kda_forward`);
    ``normalize_qk=True`` is the backward of ``forward(..., normalize_qk=True)``
    (``ckda_backward_ex``)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need(k, "k", shape=(B, T, H, dk))
    _need(v, "v", shape=(B, T, H, dv))
    _need(g, "g", torch.float32, (B, T, H, dk))
    _need(beta, "beta", torch.float32, (B, T, H))
    _need(do, "do", torch.float32, (B, T, H, dv))
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    for t, n in ((S0, "S0"), (dS_T, "dS_T")):
        if t is not None:
            _need(t, n, torch.float32, (N, H, dk, dv))
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    dq = torch.empty((B, T, H, dk), **f32)
    dk_ = torch.empty((B, T, H, dk), **f32)
    dv_ = torch.empty((B, T, H, dv), **f32)
    dg = torch.empty((B, T, H, dk), **f32)
    db = torch.empty((B, T, H), **f32)
    dS0 = torch.empty((N, H, dk, dv), **f32) if need_dS0 else None
    ws_bytes = backward_workspace_bytes(B, T, H, dk, dv, N, code)
    if workspace is None or workspace.numel() * workspace.element_size() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(cu_seqlens),
            B, T, H, dk, dv, N, code)
    tail = (_ptr(do), _ptr(dS_T), _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dg), _ptr(db),
            _ptr(dS0), _ptr(workspace), ws_bytes, _stream(dev))
    if normalize_qk:
        entry = "ckda_backward_ex"
        st = library().ckda_backward_ex(*head, OPT_QK_L2NORM | (OPT_KDA if kda else 0), *tail)
    else:
        entry = "kda_backward" if kda else "ckda_backward"
        st = getattr(library(), entry)(*head, *tail)
    _check(st, entry)
    return dq, dk_, dv_, dg, db, dS0


def decode_step(q, k, v, g, beta, S, *, out=None):
    """One decode step; ``S`` ([N, H, dk, dv] fp32) is updated in place.
    Returns o ``[N, H, dv]`` fp32."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    _need(k, "k", shape=(N, H, dk))
    _need(v, "v", shape=(N, H, dv))
    _need(g, "g", torch.float32, (N, H, dk))
    _need(beta, "beta", torch.float32, (N, H))
    _need(S, "S", torch.float32, (N, H, dk, dv))
    o = out if out is not None else torch.empty((N, H, dv), dtype=torch.float32, device=q.device)
    _need(o, "out", torch.float32, (N, H, dv))
    st = library().ckda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S),
                                    _ptr(o), N, H, dk, dv, code, _stream(q.device))
    _check(st, "ckda_decode_step")
    return o
