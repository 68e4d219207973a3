"""Seeded synthetic workloads for the CKDA forward and decode paths.

This module only draws inputs.  It holds none of the recurrence's arithmetic,
so both the HIP path and the CPU oracle can consume the same arrays.

Every array is drawn in fp64 from ``numpy.random.Generator(PCG64(seed))`` in a
fixed order -- q, k, v, gate sign, gate magnitude, beta, S0, sequence lengths --
then cast.  Keys (and queries) are L2-normalised per head in fp64 before the
cast.  For bf16 workloads q, k and v are rounded to fp32 and then to bf16 with
round-to-nearest-even; they are returned as fp32 arrays that hold exactly the
bf16 values (NumPy has no bf16 type), and the GPU binding casts them to bf16
without further rounding.  Gates alpha, beta and states stay fp32.

The pages measure throughput on a 1.3B-parameter language-model layer shape
(H=16, dk=dv=128, 32k tokens per step, bf16); no dataset is used here, these
synthetic draws stand in for it.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int              # batch rows (1 for packed sequences)
    T: int              # tokens per row (total tokens when packed)
    H: int
    dk: int
    dv: int
    dtype: str          # "bf16" or "f32": dtype of q, k, v
    gate: str           # "signed_uniform" | "rotation" | "tanh"
    q_scale: bool       # multiply q by dk**-0.5 after normalising
    s0: str             # "zero" | "unit_frobenius"
    n_seqs: int = 0     # > 0: packed variable-length sequences
    seq_min: int = 0
    seq_max: int = 0
    steps: int = 0      # decode workloads: consecutive steps
    chunk: int = 64


WORKLOADS = {
    # Tiny forward, fp32 inputs; the oracle finishes it in well under a second.
    "tiny_f32": Workload("tiny_f32", B=1, T=256, H=2, dk=64, dv=64, dtype="f32",
                         gate="signed_uniform", q_scale=True, s0="zero"),
    # Orthogonal transitions: alpha in {-1, +1}, beta = 2, unit keys, random
    # unit-Frobenius initial state.
    "rotation_f32": Workload("rotation_f32", B=2, T=4096, H=4, dk=128, dv=128, dtype="f32",
                             gate="rotation", q_scale=False, s0="unit_frobenius"),
    # One layer shaped like a 1.3B-parameter LM (hidden 2048 = 16 heads x 128).
    "layer_1p3b_bf16": Workload("layer_1p3b_bf16", B=8, T=4096, H=16, dk=128, dv=128,
                                dtype="bf16", gate="tanh", q_scale=False, s0="zero"),
    # The same layer with every eighth key channel forgetting fast (|alpha| in
    # [0.01, 0.1]): those channels' gates fall by 2^-213 or more over a chunk.
    "layer_1p3b_fastdecay_bf16": Workload("layer_1p3b_fastdecay_bf16", B=8, T=4096, H=16,
                                          dk=128, dv=128, dtype="bf16", gate="tanh_fastdecay",
                                          q_scale=False, s0="zero"),
    # Every eighth key channel forgetting faster still (|alpha| in [0.001,
    # 0.01]): over the 15 later gates of a 16-token block those channels fall
    # by 2^-100 to 2^-150, so most blocks leave the range of the factored
    # block form and take the exact (log-space) block path.
    "layer_1p3b_rapiddecay_bf16": Workload("layer_1p3b_rapiddecay_bf16", B=8, T=4096, H=16,
                                           dk=128, dv=128, dtype="bf16", gate="tanh_rapiddecay",
                                           q_scale=False, s0="zero"),
    # 65536 packed tokens in 12 sequences of log-uniform length.
    "varlen_64k_bf16": Workload("varlen_64k_bf16", B=1, T=65536, H=16, dk=128, dv=128,
                                dtype="bf16", gate="rotation", q_scale=False, s0="zero",
                                n_seqs=12, seq_min=512, seq_max=16384),
    # 1024 consecutive decode steps of 256 sequences x 16 heads.
    "decode_256x16": Workload("decode_256x16", B=256, T=1, H=16, dk=128, dv=128,
                              dtype="bf16", gate="rotation", q_scale=False,
                              s0="unit_frobenius", steps=1024),
}


def round_bf16(x) -> np.ndarray:
    """Round to fp32, then to bf16 (round to nearest, ties to even); return
    the bf16 values as an fp32 array.  Inputs here are finite."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = f.view(np.uint32)
    # finite inputs: bits + 0x8000 stays below 2^32, so uint32 cannot wrap
    out = bits + (np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1)))
    out &= np.uint32(0xFFFF0000)
    return out.view(np.float32).reshape(f.shape)


def _normalise(x):
    x /= np.sqrt(np.einsum("...i,...i->...", x, x))[..., None]
    return x


def _cast_qkv(x, dtype):
    return round_bf16(x) if dtype == "bf16" else x.astype(np.float32)


def _gates(rng, shape, kind):
    """Signed per-channel gates alpha (fp64 before the cast)."""
    if kind == "signed_uniform":
        neg = rng.random(shape) < 0.3            # gate sign: negative w.p. 0.3
        mag = rng.uniform(0.05, 1.0, shape)      # gate magnitude
        return np.where(neg, -mag, mag)
    if kind == "rotation":
        neg = rng.random(shape) < 0.5            # gate sign only, |alpha| = 1
        return np.where(neg, -1.0, 1.0)
    if kind in ("tanh", "tanh_fastdecay", "tanh_rapiddecay"):
        a = np.tanh(rng.normal(0.0, 1.5, shape))  # std 1.5
        sgn = np.where(a < 0, -1.0, 1.0)          # sign(0) := +
        mag = np.maximum(np.abs(a), 1e-3)
        if kind == "tanh_fastdecay":
            # every eighth channel forgets fast: |alpha| uniform in [0.01, 0.1]
            fast = rng.uniform(0.01, 0.1, shape)
            mag = np.where(np.arange(shape[-1]) % 8 == 7, fast, mag)
        if kind == "tanh_rapiddecay":
            # every eighth channel: |alpha| uniform in [0.001, 0.01]
            fast = rng.uniform(0.001, 0.01, shape)
            mag = np.where(np.arange(shape[-1]) % 8 == 7, fast, mag)
        return sgn * mag
    raise ValueError(kind)


def _betas(rng, shape, kind):
    if kind == "rotation":
        return np.full(shape, 2.0)
    return 2.0 / (1.0 + np.exp(-rng.normal(0.0, 1.0, shape)))   # 2 * sigmoid(N(0,1))


def _unit_frobenius_states(rng, shape):
    s = rng.normal(0.0, 1.0, shape)
    return s / np.sqrt(np.sum(s * s, axis=(-2, -1), keepdims=True))


def packed_lengths(rng, n, total, lo, hi):
    """Sequence lengths: log-uniform weights in [lo, hi], scaled to sum to
    ``total``, clamped to [lo, hi], the remainder spread one token at a time
    over sequences not at a bound."""
    x = np.exp(rng.uniform(np.log(lo), np.log(hi), n))
    lens = np.floor(x * total / x.sum()).astype(np.int64)
    lens = np.clip(lens, lo, hi)
    i = 0
    while lens.sum() != total:
        step = 1 if lens.sum() < total else -1
        j = i % n
        if lo <= lens[j] + step <= hi:
            lens[j] += step
        i += 1
        if i > 100 * n * (hi - lo + 1):
            raise ValueError("cannot meet the total under the bounds")
    return lens


def forward_inputs(w: Workload | str, seed: int = 0) -> dict:
    """Draw one forward batch.  Returns q, k, v ([B,T,H,d], fp32 holding bf16
    values when ``dtype == 'bf16'``), g (= alpha, fp32), beta ([B,T,H] fp32),
    S0 ([N,H,dk,dv] fp32 or None) and cu_seqlens (int32 [N+1] or None)."""
    w = WORKLOADS[w] if isinstance(w, str) else w
    rng = np.random.Generator(np.random.PCG64(seed))
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    q = _normalise(rng.normal(0.0, 1.0, (B, T, H, dk)))
    if w.q_scale:
        q = q * dk ** -0.5
    k = _normalise(rng.normal(0.0, 1.0, (B, T, H, dk)))
    v = rng.normal(0.0, 1.0, (B, T, H, dv))
    g = _gates(rng, (B, T, H, dk), w.gate)
    beta = _betas(rng, (B, T, H), w.gate)
    N = w.n_seqs if w.n_seqs else B
    S0 = None
    if w.s0 == "unit_frobenius":
        S0 = _unit_frobenius_states(rng, (N, H, dk, dv)).astype(np.float32)
    cu = None
    if w.n_seqs:
        lens = packed_lengths(rng, w.n_seqs, T, w.seq_min, w.seq_max)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return dict(q=_cast_qkv(q, w.dtype), k=_cast_qkv(k, w.dtype), v=_cast_qkv(v, w.dtype),
                g=g.astype(np.float32), beta=beta.astype(np.float32), S0=S0,
                cu_seqlens=cu, dtype=w.dtype, workload=w)


def decode_state(w: Workload | str, seed: int = 0) -> np.ndarray:
    """Initial decode state [N, H, dk, dv] fp32, unit Frobenius per (n, h)."""
    w = WORKLOADS[w] if isinstance(w, str) else w
    rng = np.random.Generator(np.random.PCG64([seed, 0x5EED]))
    return _unit_frobenius_states(rng, (w.B, w.H, w.dk, w.dv)).astype(np.float32)


def decode_step_inputs(w: Workload | str, step: int, seed: int = 0, heads=None) -> dict:
    """Inputs of decode step ``step`` (each step has its own seeded stream).
    ``heads``: optional index array into the flattened N*H pairs, to draw the
    full step and return only those rows (for sampled checks)."""
    w = WORKLOADS[w] if isinstance(w, str) else w
    rng = np.random.Generator(np.random.PCG64([seed, step]))
    N, H, dk, dv = w.B, w.H, w.dk, w.dv
    q = _normalise(rng.normal(0.0, 1.0, (N, H, dk)))
    if w.q_scale:
        q = q * dk ** -0.5
    k = _normalise(rng.normal(0.0, 1.0, (N, H, dk)))
    v = rng.normal(0.0, 1.0, (N, H, dv))
    g = _gates(rng, (N, H, dk), w.gate)
    beta = _betas(rng, (N, H), w.gate)
    out = dict(q=_cast_qkv(q, w.dtype), k=_cast_qkv(k, w.dtype), v=_cast_qkv(v, w.dtype),
               g=g.astype(np.float32), beta=beta.astype(np.float32))
    if heads is not None:
        out = {key: a.reshape(N * H, *a.shape[2:])[heads] for key, a in out.items()}
    return out


def scaled(w: Workload | str, **changes) -> Workload:
    """A copy of a workload with some sizes changed (for smaller test cases)."""
    from dataclasses import replace
    w = WORKLOADS[w] if isinstance(w, str) else w
    return replace(w, **changes)


def decode_steps(w: Workload | str, steps, seed: int = 0, workers: int = 8):
    """Inputs of several decode steps, drawn in parallel threads (each step
    has its own stream, so the result does not depend on ``workers``)."""
    from concurrent.futures import ThreadPoolExecutor
    steps = list(steps)
    with ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        return list(ex.map(lambda s: decode_step_inputs(w, s, seed), steps))
