"""Brute-force check: the dense chunked (WY/UT) fp64 formulation equals the
token-by-token recurrence on tiny inputs, for several chunk sizes (the result
must not depend on the chunk size), packed sequences, a non-zero initial state,
and both ways of forming the gate ratios (running product, and sign parity
plus log2-magnitude cumulative sum)."""
import numpy as np
import pytest

import oracle
from oracle import chunked
from gated_delta_rule_22_amd import workloads as wl


def _inputs(seed=0, T=100, H=2, dk=8, dv=6, packed=True):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(1, T, H, dk))
    k = rng.normal(size=(1, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.normal(size=(1, T, H, dv))
    g = rng.uniform(0.3, 1.0, size=(1, T, H, dk)) * np.where(rng.random((1, T, H, dk)) < 0.4, -1, 1)
    beta = rng.uniform(0, 2, size=(1, T, H))
    cu = np.array([0, 23, 64, T]) if packed else None
    N = 3 if packed else 1
    S0 = rng.normal(size=(N, H, dk, dv))
    return q, k, v, g, beta, S0, cu


@pytest.mark.parametrize("chunk", [16, 37, 64])
@pytest.mark.parametrize("mode", ["product", "logsign"])
def test_chunked_equals_sequential(chunk, mode):
    q, k, v, g, beta, S0, cu = _inputs()
    o_ref, S_ref = oracle.forward(q, k, v, g, beta, S0=S0, cu_seqlens=cu)
    o, S = chunked.forward(q, k, v, g, beta, S0=S0, cu_seqlens=cu, chunk=chunk, mode=mode)
    scale = np.sqrt(np.mean(o_ref ** 2))
    assert np.max(np.abs(o - o_ref)) / scale < 1e-12
    assert np.max(np.abs(S - S_ref)) / np.sqrt(np.mean(S_ref ** 2)) < 1e-12


def test_chunked_on_tiny_workload_shape():
    """The tiny fp32 workload's own draw (dk = 64, T = 256, chunk 64), one head."""
    x = wl.forward_inputs(wl.scaled("tiny_f32", H=1))
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"])
    o, S = chunked.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], chunk=64, mode="logsign")
    assert np.max(np.abs(o - o_ref)) / np.sqrt(np.mean(o_ref ** 2)) < 1e-11
    assert np.max(np.abs(S - S_ref)) / np.sqrt(np.mean(S_ref ** 2)) < 1e-11


def test_chunked_catches_planted_mistake():
    """The comparison is sharp: flipping one sign in the chunked algebra (the
    parity of one token's gate) is caught."""
    q, k, v, g, beta, S0, cu = _inputs(packed=False, T=40)
    o_ref, _ = oracle.forward(q, k, v, g, beta, S0=S0)
    g2 = g.copy()
    g2[0, 17, 0, 3] *= -1
    o, _ = chunked.forward(q, k, v, g2, beta, S0=S0, chunk=16)
    assert np.max(np.abs(o - o_ref)) / np.sqrt(np.mean(o_ref ** 2)) > 1e-6
