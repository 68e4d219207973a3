"""Dense chunked (WY/UT) fp64 formulation of CKDA -- TEST INFRASTRUCTURE ONLY.

This is the algebra a chunkwise-parallel kernel implements, written densely in
NumPy so that a reader can check every step against the derivation below.  It
exists to confirm, by brute force on tiny inputs, that the chunked algebra
reaches the same result as the token-by-token recurrence of the C oracle.

No page prints these formulas (the CKDA pages only say the kernels are a
small change to the chunked KDA kernels of the FLA library); they follow from
unrolling the update rule of the blog post "One update, one quarter turn"
(section "ELI5", paragraph "The mirror") inside one chunk.

Derivation.  Inside a chunk with incoming state S and local tokens i = 1..n,
write each update as S_i = D_i S_{i-1} + k_i u_i^T with D_i = Diag(alpha_i)
and u_i = beta_i (v_i - S_{i-1}^T D_i k_i).  Unrolling with the per-channel
ratio r_ij = prod_{j < s <= i} alpha_s (so r_ii = 1) and gamma_i = r_i0:

    S_{i-1}^T D_i k_i = S^T (gamma_i * k_i) + sum_{j<i} u_j [k_j^T Diag(r_ij) k_i]

so (I + A) U = Diag(beta) (V - (gamma*K) S) with the strictly lower
A_ij = beta_i sum_c k_ic r_ij,c k_jc.  With T = (I + A)^{-1}:

    U   = T Diag(beta) V - T Diag(beta) (gamma*K) S
    o_i = S_i^T q_i = S^T (gamma_i * q_i) + sum_{j<=i} P_ij u_j,
          P_ij = sum_c q_ic r_ij,c k_jc   (j <= i)
    S_n = Diag(gamma_n) S + sum_j (k_j * r_nj) u_j^T

Two ways of forming r are offered:

* ``"product"`` -- the running product of the gates, as defined.
* ``"logsign"`` -- the signed-gate decomposition the CKDA paper's methodology
  calls for (sign kept apart from the log-space magnitude):
  r_ij = (-1)^(pi_i xor pi_j) * 2^(G_i - G_j) with G the in-chunk inclusive
  cumulative sum of log2|alpha| and pi the inclusive cumulative parity of
  negative gates.  It needs alpha != 0.
"""
from __future__ import annotations

import numpy as np


def _ratios(alpha, mode):
    """r[i, j, c] for j <= i (zero above the diagonal), plus gamma[i, c]."""
    n, dk = alpha.shape
    r = np.zeros((n, n, dk))
    if mode == "product":
        for j in range(n):
            acc = np.ones(dk)
            r[j, j] = acc
            for i in range(j + 1, n):
                acc = acc * alpha[i]
                r[i, j] = acc
        gamma = np.cumprod(alpha, axis=0)
    elif mode == "logsign":
        G = np.cumsum(np.log2(np.abs(alpha)), axis=0)
        pi = np.cumsum((alpha < 0).astype(np.int64), axis=0) % 2
        for i in range(n):
            for j in range(i + 1):
                sgn = np.where((pi[i] ^ pi[j]) == 1, -1.0, 1.0)
                r[i, j] = sgn * np.exp2(G[i] - G[j])
        gamma = np.where(pi == 1, -1.0, 1.0) * np.exp2(G)
    else:
        raise ValueError(mode)
    return r, gamma


def chunk_step(S, q, k, v, alpha, beta, mode="product"):
    """Apply one chunk (n tokens) to state S. Returns (o [n, dv], S_next)."""
    n, dk = k.shape
    r, gamma = _ratios(alpha, mode)
    A = np.zeros((n, n))
    P = np.zeros((n, n))
    for i in range(n):
        for j in range(i + 1):
            P[i, j] = np.sum(q[i] * r[i, j] * k[j])
            if j < i:
                A[i, j] = beta[i] * np.sum(k[i] * r[i, j] * k[j])
    I_A = np.eye(n) + A
    # W = T Diag(beta) (gamma*K) and Ubar = T Diag(beta) V, via a solve.
    W = np.linalg.solve(I_A, beta[:, None] * (gamma * k))
    Ubar = np.linalg.solve(I_A, beta[:, None] * v)
    U = Ubar - W @ S
    o = (gamma * q) @ S + P @ U
    K_end = k * r[n - 1]                      # rows k_j * r_{n,j}
    S_next = gamma[n - 1][:, None] * S + K_end.T @ U
    return o, S_next


def forward(q, k, v, g, beta, S0=None, cu_seqlens=None, chunk=64, mode="product"):
    """Chunked forward with the same signature and result layout as
    :func:`oracle.forward`.  Pure NumPy, fp64, for tiny inputs only."""
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        seqs = [(b, 0, T) for b in range(B)]
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        seqs = [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    o = np.zeros((B, T, H, dv))
    S_T = np.zeros((len(seqs), H, dk, dv))
    for n, (b, t0, t1) in enumerate(seqs):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[n, h], dtype=np.float64)
            for c0 in range(t0, t1, chunk):
                c1 = min(c0 + chunk, t1)
                sl = (b, slice(c0, c1), h)
                o_c, S = chunk_step(S, q[sl], k[sl], v[sl], g[sl], beta[sl], mode)
                o[sl] = o_c
            S_T[n, h] = S
    return o, S_T
