"""Pins of the oracle's backward pass (``oracle.backward``).

The backward is the reverse-mode gradient of the token recurrence (update rule:
blog post "One update, one quarter turn", section "ELI5", paragraph "The
mirror"; readout o_t = S_t^T q_t after the write).  It is checked here against
things other than itself:

* central finite differences of the *forward* oracle (itself pinned by the
  forward pins) on tiny inputs, for every input element: brute force that a
  dropped term, a wrong sign, a transposed operand or a wrong state in any
  adjoint step would fail;
* two closed forms: beta = 0 with alpha = 1 (the state never changes), and a
  single token from a zero state (o = beta (k . q) v).

The loss is L = sum(dO * o) + sum(dS_T * S_T), so the gradients are those of
the vector-Jacobian product with upstream gradients dO and dS_T.
"""
import numpy as np
import pytest

import oracle

H_FD = 1e-6


def _inputs(rng, B, T, H, dk, dv, N=None, expansive=False):
    N = B if N is None else N
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk)) / np.sqrt(dk)
    v = rng.standard_normal((B, T, H, dv))
    lim = 1.2 if expansive else 1.0
    sign = np.where(rng.uniform(size=(B, T, H, dk)) < 0.4, -1.0, 1.0)
    g = sign * rng.uniform(0.2, lim, (B, T, H, dk))
    beta = rng.uniform(0.0, 2.5 if expansive else 2.0, (B, T, H))
    S0 = rng.standard_normal((N, H, dk, dv))
    do = rng.standard_normal((B, T, H, dv))
    dST = rng.standard_normal((N, H, dk, dv))
    return [q, k, v, g, beta, S0], do, dST


def _loss(args, do, dST, cu):
    q, k, v, g, beta, S0 = args
    o, ST = oracle.forward(q, k, v, g, beta, S0=S0, cu_seqlens=cu, nthreads=1)
    return float((o * do).sum() + (ST * dST).sum())


def _fd_check(args, do, dST, cu=None, sample=None, rng=None):
    grads = oracle.backward(*args[:5], do, S0=args[5], dS_T=dST, cu_seqlens=cu, nthreads=1)
    names = ["q", "k", "v", "g", "beta", "S0"]
    for ai, (a, gan) in enumerate(zip(args, grads)):
        assert gan.shape == a.shape
        idxs = list(np.ndindex(a.shape))
        if sample is not None and len(idxs) > sample:
            pick = rng.choice(len(idxs), size=sample, replace=False)
            idxs = [idxs[i] for i in pick]
        scale = max(1.0, float(np.abs(gan).max()))
        for idx in idxs:
            ap = [x.copy() for x in args]
            am = [x.copy() for x in args]
            ap[ai][idx] += H_FD
            am[ai][idx] -= H_FD
            fd = (_loss(ap, do, dST, cu) - _loss(am, do, dST, cu)) / (2 * H_FD)
            assert abs(fd - gan[idx]) <= 1e-7 * scale, (names[ai], idx, fd, gan[idx])


def test_backward_matches_finite_differences_uniform():
    rng = np.random.default_rng(11)
    args, do, dST = _inputs(rng, B=2, T=5, H=2, dk=3, dv=2)
    _fd_check(args, do, dST)


def test_backward_matches_finite_differences_expansive():
    """|alpha| up to 1.2 and beta up to 2.5: the gradient is that of the
    definition, whatever the gate range."""
    rng = np.random.default_rng(12)
    args, do, dST = _inputs(rng, B=1, T=6, H=1, dk=4, dv=3, expansive=True)
    _fd_check(args, do, dST)


def test_backward_matches_finite_differences_packed():
    rng = np.random.default_rng(13)
    cu = np.array([0, 2, 2, 7, 9])            # includes an empty sequence
    args, do, dST = _inputs(rng, B=1, T=9, H=2, dk=2, dv=3, N=4)
    _fd_check(args, do, dST, cu=cu)


def test_backward_matches_finite_differences_long():
    """150 tokens: more than two of the oracle's recompute segments."""
    rng = np.random.default_rng(14)
    args, do, dST = _inputs(rng, B=1, T=150, H=1, dk=2, dv=2)
    _fd_check(args, do, dST, sample=25, rng=rng)


def test_backward_beta_zero_unit_gate_closed_form():
    """beta = 0, alpha = 1: S_t = S0 for every t, o_t = S0^T q_t.  Then
    dq_t = S0 dO_t, dk = dv = 0, dS0 = dS_T + sum_t q_t dO_t^T,
    dalpha_t = rowsum(G_t * S0) and dbeta_t = (v_t - S0^T k_t) . (G_t^T k_t)
    with G_t = dS_T + sum_{s >= t} q_s dO_s^T (the gradient reaching S_t)."""
    rng = np.random.default_rng(15)
    T, dk, dv = 7, 5, 4
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    S0 = rng.standard_normal((dk, dv))
    do = rng.standard_normal((T, dv))
    dST = rng.standard_normal((dk, dv))
    e = lambda x: x[None, :, None]
    dq, dk_, dv_, dg, db, dS0 = oracle.backward(
        e(q), e(k), e(v), e(np.ones((T, dk))), e(np.zeros(T)), e(do), S0=S0[None, None],
        dS_T=dST[None, None], nthreads=1)
    np.testing.assert_allclose(dq[0, :, 0], do @ S0.T, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(dk_, 0.0)
    np.testing.assert_array_equal(dv_, 0.0)
    np.testing.assert_allclose(dS0[0, 0], dST + q.T @ do, rtol=1e-13, atol=1e-12)
    for t in range(T):
        G = dST + q[t:].T @ do[t:]
        np.testing.assert_allclose(dg[0, t, 0], (G * S0).sum(axis=1), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(db[0, t, 0], (v[t] - S0.T @ k[t]) @ (G.T @ k[t]),
                                   rtol=1e-12, atol=1e-12)


def test_backward_first_token_from_zero_state_closed_form():
    """One token, S0 = 0: S_1 = beta k v^T and o = beta (k . q) v, so
    dq = beta (v . dO) k, dk = beta (v . dO) q + beta dS_T v,
    dv = beta (k . q) dO + beta dS_T^T k, dbeta = (k . q)(v . dO) + k^T dS_T v,
    dalpha = 0 and dS0 = Diag(alpha) (dS_T + q dO^T - beta k (dS_T^T k + (k.q) dO)^T)."""
    rng = np.random.default_rng(16)
    dk, dv = 6, 5
    q, k, a = rng.standard_normal(dk), rng.standard_normal(dk), rng.uniform(-1, 1, dk)
    v, do = rng.standard_normal(dv), rng.standard_normal(dv)
    dST = rng.standard_normal((dk, dv))
    b = 1.3
    e = lambda x: x.reshape(1, 1, 1, -1)
    dq, dk_, dv_, dg, db, dS0 = oracle.backward(
        e(q), e(k), e(v), e(a), np.full((1, 1, 1), b), e(do), S0=np.zeros((1, 1, dk, dv)),
        dS_T=dST[None, None], nthreads=1)
    kq, vd = k @ q, v @ do
    np.testing.assert_allclose(dq.ravel(), b * vd * k, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dk_.ravel(), b * vd * q + b * dST @ v, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dv_.ravel(), b * kq * do + b * dST.T @ k, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(db.ravel(), [kq * vd + k @ dST @ v], rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(dg, 0.0)
    G = dST + np.outer(q, do)                        # gradient reaching S_1
    dSp = G - b * np.outer(k, G.T @ k)               # through the erase
    np.testing.assert_allclose(dS0[0, 0], a[:, None] * dSp, rtol=1e-13, atol=1e-13)


def test_backward_rejects_bad_shapes():
    rng = np.random.default_rng(17)
    args, do, dST = _inputs(rng, B=1, T=3, H=1, dk=2, dv=2)
    with pytest.raises(ValueError):
        oracle.backward(*args[:5], do[..., :1], S0=args[5])


def test_backward_with_qk_normalisation_matches_finite_differences():
    """The gradient through the fused key/query L2 normalisation: central
    differences of forward(normalise(q), normalise(k), ...) for every element
    of q and k, and the other gradients unchanged by the option."""
    rng = np.random.default_rng(18)
    args, do, dST = _inputs(rng, B=1, T=6, H=2, dk=3, dv=2)
    q, k, v, g, beta, S0 = args
    grads = oracle.backward(q, k, v, g, beta, do, S0=S0, dS_T=dST, nthreads=1,
                            normalize_qk=True)

    def loss(qq, kk):
        o, ST = oracle.forward(oracle.l2_normalise(qq), oracle.l2_normalise(kk), v, g, beta,
                               S0=S0, nthreads=1)
        return float((o * do).sum() + (ST * dST).sum())

    for which, x in ((0, q), (1, k)):
        scale = max(1.0, float(np.abs(grads[which]).max()))
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += H_FD
            xm[idx] -= H_FD
            pair = lambda a: (a, k) if which == 0 else (q, a)
            fd = (loss(*pair(xp)) - loss(*pair(xm))) / (2 * H_FD)
            assert abs(fd - grads[which][idx]) <= 1e-7 * scale, (which, idx)
    plain = oracle.backward(oracle.l2_normalise(q), oracle.l2_normalise(k), v, g, beta, do,
                            S0=S0, dS_T=dST, nthreads=1)
    for a, b in zip(grads[2:], plain[2:]):
        np.testing.assert_array_equal(a, b)
