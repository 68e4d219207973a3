"""Pins of the CPU oracle to facts the pages and the mathematics fix.

Each test checks the oracle (``oracle.forward`` / ``oracle.transition``, the
token-by-token fp64 recurrence) against something other than itself: values
printed on the pages (fixtures under tests/golden/, each with its citation),
closed forms, spectral theorems the CKDA summary states, and exact identities.
They are chosen so that a plausible mistake in the oracle -- a dropped decay,
a wrong order of decay and erase, a wrong sign of the delta term, a transposed
state, a gate applied to the wrong axis, a readout taken before the write --
fails at least one of them.
"""
import numpy as np
import pytest

import oracle
from tests import _golden

RNG = np.random.default_rng(1234)


def _unit(x):
    return x / np.linalg.norm(x)


def _run(q, k, v, g, beta, S0):
    """Single sequence helper: q,k,g [T,dk], v [T,dv], beta [T], S0 [dk,dv]."""
    T, dk = k.shape
    dv = v.shape[1]
    o, S_T = oracle.forward(q[None, :, None], k[None, :, None], v[None, :, None],
                            g[None, :, None], beta[None, :, None],
                            S0=S0[None, None], nthreads=1)
    return o[0, :, 0], S_T[0, 0]


def _rot2(theta, alpha, beta=2.0):
    k = np.array([np.cos(theta), np.sin(theta)])
    return oracle.transition(k, np.array([alpha, 1.0]), beta)


# ---------------------------------------------------------------- the dial (beta)

@pytest.mark.parametrize("rec", _golden.load("householder_dial.txt"))
def test_householder_dial(rec):
    """Blog "One update, one quarter turn", ELI5 "The mirror": beta = 0, 1, 2."""
    dk = 6
    k = _unit(RNG.normal(size=dk))
    A = oracle.transition(k, np.ones(dk), rec["beta"])
    I = np.eye(dk)
    if rec["kind"] == 0:
        np.testing.assert_allclose(A, I, atol=1e-15)
    elif rec["kind"] == 1:
        np.testing.assert_allclose(A @ A, A, atol=1e-14)          # projection
        np.testing.assert_allclose(A @ k, 0.0, atol=1e-14)        # erases along k
        assert np.linalg.matrix_rank(A, tol=1e-10) == dk - 1
    else:
        np.testing.assert_allclose(A @ A, I, atol=1e-14)          # involution
        np.testing.assert_allclose(A @ k, -k, atol=1e-14)         # mirror flips k
        assert np.linalg.det(A) == pytest.approx(-1.0, abs=1e-13)


def test_beta_zero_keeps_state_and_reads_it():
    """beta = 0 and alpha = 1: the transition is the identity, so S_t = S_0 and
    o_t = S_0^T q_t.  A non-symmetric, non-square S_0 catches a transposed
    state or readout."""
    T, dk, dv = 7, 5, 3
    q, k = RNG.normal(size=(T, dk)), RNG.normal(size=(T, dk))
    v = RNG.normal(size=(T, dv))
    S0 = RNG.normal(size=(dk, dv))
    o, S_T = _run(q, k, v, np.ones((T, dk)), np.zeros(T), S0)
    np.testing.assert_allclose(S_T, S0, atol=1e-15)
    np.testing.assert_allclose(o, q @ S0, atol=1e-13)


def test_beta_zero_is_pure_gate_decay():
    """beta = 0: the transition is Diag(alpha) alone, so
    S_t = Diag(prod_{s<=t} alpha_s) S_0 -- the gate scales key-channel rows."""
    T, dk, dv = 6, 4, 3
    g = RNG.uniform(-1, 1, size=(T, dk))
    S0 = RNG.normal(size=(dk, dv))
    q = RNG.normal(size=(T, dk))
    o, S_T = _run(q, RNG.normal(size=(T, dk)), RNG.normal(size=(T, dv)), g, np.zeros(T), S0)
    cum = np.cumprod(g, axis=0)
    np.testing.assert_allclose(S_T, cum[-1][:, None] * S0, atol=1e-14)
    for t in range(T):
        np.testing.assert_allclose(o[t], (cum[t] * q[t]) @ S0, atol=1e-13)


def test_projection_erases_key_direction():
    """beta = 1, alpha = 1, unit key, v = 0: k_t^T S_t = 0 after every step."""
    T, dk, dv = 5, 6, 4
    k = np.stack([_unit(RNG.normal(size=dk)) for _ in range(T)])
    S = RNG.normal(size=(dk, dv))
    for t in range(T):
        _, S = _run(np.zeros((1, dk)), k[t:t + 1], np.zeros((1, dv)), np.ones((1, dk)),
                    np.ones(1), S)
        np.testing.assert_allclose(k[t] @ S, 0.0, atol=1e-14)


def test_first_token_from_zero_state():
    """From S_0 = 0 one token leaves S_1 = beta k v^T (decay and erase act on
    zero), and the readout after that write is o_1 = beta (k.q) v."""
    dk, dv = 5, 4
    q, k, v = RNG.normal(size=dk), RNG.normal(size=dk), RNG.normal(size=dv)
    g, b = RNG.uniform(-1, 1, size=dk), 1.37
    o, S_T = _run(q[None], k[None], v[None], g[None], np.array([b]), np.zeros((dk, dv)))
    np.testing.assert_allclose(S_T, b * np.outer(k, v), atol=1e-15)
    np.testing.assert_allclose(o[0], b * (k @ q) * v, atol=1e-14)


# ---------------------------------------------------------------- rotations

def test_quarter_turn_golden():
    rec = _golden.load("quarter_turn.txt")[0]
    A = oracle.transition(np.array(rec["k"]), np.array(rec["alpha"]), rec["beta"])
    ev = np.linalg.eigvals(A)
    ev = ev[np.argsort(-ev.imag)]
    np.testing.assert_allclose(ev.real, rec["eig_real"], atol=1e-15)
    np.testing.assert_allclose(ev.imag, rec["eig_imag"], atol=1e-15)
    # every vector turns by 90 degrees without changing length
    x = RNG.normal(size=2)
    y = A @ x
    ang = np.degrees(np.arccos(x @ y / (np.linalg.norm(x) * np.linalg.norm(y))))
    assert ang == pytest.approx(rec["rotation_degrees"], abs=1e-9)
    assert np.linalg.norm(y) == pytest.approx(np.linalg.norm(x), rel=1e-14)
    # the state comes back after `period` updates (v = 0), and not before
    p = int(rec["period"])
    T = 3 * p
    k = np.tile(rec["k"], (T, 1))
    g = np.tile(rec["alpha"], (T, 1))
    S0 = RNG.normal(size=(2, 3))
    S = S0
    for t in range(1, T + 1):
        _, S = _run(np.zeros((1, 2)), k[:1], np.zeros((1, 3)), g[:1], np.full(1, rec["beta"]), S)
        back = np.allclose(S, S0, atol=1e-12)
        assert back == (t % p == 0)


def test_quarter_turn_embedded_high_dim():
    """The same quarter turn inside dk = 128: k = (e1 + e2)/sqrt(2), gate -1 on
    channel 1 and +1 elsewhere.  Rows 1-2 of the state rotate (period 4),
    every other row stays fixed."""
    dk, dv, T = 128, 8, 12
    k = np.zeros(dk)
    k[:2] = np.sqrt(0.5)
    g = np.ones(dk)
    g[0] = -1.0
    S0 = RNG.normal(size=(dk, dv))
    ks, gs = np.tile(k, (T, 1)), np.tile(g, (T, 1))
    o, S_T = _run(np.zeros((T, dk)), ks, np.zeros((T, dv)), gs, np.full(T, 2.0), S0)
    np.testing.assert_allclose(S_T, S0, atol=1e-13)          # 12 = 3 full turns
    _, S1 = _run(np.zeros((1, dk)), ks[:1], np.zeros((1, dv)), gs[:1], np.full(1, 2.0), S0)
    np.testing.assert_allclose(S1[2:], S0[2:], atol=1e-15)
    np.testing.assert_allclose(S1[:2], np.array([[0, -1], [1, 0]]) @ S0[:2], atol=1e-14)


@pytest.mark.parametrize("rec", _golden.load("closed_form_rotation.txt"))
def test_closed_form_2x2(rec):
    theta = rec["theta_over_pi"] * np.pi
    A = _rot2(theta, rec["alpha"])
    np.testing.assert_allclose(A.reshape(-1), rec["a"], atol=2e-15)
    tr, det = np.trace(A), np.linalg.det(A)
    assert tr * tr - 4 * det == pytest.approx(rec["disc"], abs=1e-12)
    ev = np.linalg.eigvals(A)
    is_complex = bool(np.max(np.abs(ev.imag)) > 1e-9)
    assert is_complex == bool(rec["complex"])
    if is_complex:
        assert rec["alpha"] < 0
        np.testing.assert_allclose(np.abs(ev), rec["abs_lambda"], rtol=1e-12)


def test_rotation_by_twice_the_angle():
    """Main Findings (closed form): at alpha = -1 the transition is a rotation
    by 2t.  Check the eigen-angle for a sweep of t."""
    for t in np.linspace(0.05, 1.5, 13):
        A = _rot2(t, -1.0)
        np.testing.assert_allclose(A.T @ A, np.eye(2), atol=1e-14)
        assert np.linalg.det(A) == pytest.approx(1.0, abs=1e-14)
        ang = np.arctan2(A[1, 0], A[0, 0])
        assert np.cos(ang) == pytest.approx(np.cos(2 * t), abs=1e-13)
        assert np.sin(ang) == pytest.approx(np.sin(2 * t), abs=1e-13)


@pytest.mark.parametrize("rec", _golden.load("sign_condition.txt"))
def test_sign_condition(rec):
    theta = rec["theta_over_pi"] * np.pi
    k = np.array([np.cos(theta), np.sin(theta)])
    A = oracle.transition(k, np.array([-1.0, 1.0]), rec["beta"])
    ev = np.linalg.eigvals(A)
    is_complex = bool(np.max(np.abs(ev.imag)) > 1e-9)
    assert is_complex == bool(rec["complex"])
    if is_complex:
        np.testing.assert_allclose(np.abs(ev) ** 2, rec["abs_lambda_sq"], rtol=1e-12)


def test_clock_mod12():
    rec = _golden.load("clock_mod12.txt")[0]
    n = int(rec["n"])
    A = _rot2(rec["theta_over_pi"] * np.pi, rec["alpha"][0], rec["beta"])
    P = np.eye(2)
    for m in range(1, n + 1):
        P = A @ P
        assert np.allclose(P, np.eye(2), atol=1e-12) == (m == int(rec["period"]))


# ---------------------------------------------------------------- spectra

def _nonreal_pairs(A, tol=1e-8):
    ev = np.linalg.eigvals(A)
    return int(np.sum(ev.imag > tol))


def test_scalar_gate_real_spectrum():
    """Main Findings: a scalar gate gives alpha (I - beta k k^T), symmetric,
    real spectrum -- for either sign of alpha."""
    dk = 8
    for _ in range(50):
        k = _unit(RNG.normal(size=dk))
        a = RNG.uniform(-1, 1)
        A = oracle.transition(k, np.full(dk, a), RNG.uniform(0, 2))
        np.testing.assert_allclose(A, A.T, atol=1e-15)
        assert _nonreal_pairs(A) == 0


def test_positive_channel_gates_real_spectrum():
    """Main Findings: positive per-channel gates still give a real spectrum
    (H_k D is similar to D^1/2 H_k D^1/2), though A is no longer symmetric."""
    dk = 8
    asym = 0.0
    for _ in range(50):
        k = _unit(RNG.normal(size=dk))
        A = oracle.transition(k, RNG.uniform(0.01, 1, dk), RNG.uniform(0, 2))
        asym = max(asym, np.max(np.abs(A - A.T)))
        assert _nonreal_pairs(A) == 0
    assert asym > 1e-3


def test_commutator_entry():
    """Main Findings: (H_k D - D H_k)_ij = beta k_i k_j (alpha_i - alpha_j)
    with H_k = I - beta k k^T.  H_k D is the oracle's transition; D H_k is
    read off as the transpose of the transition (both factors symmetric)."""
    dk = 6
    k = _unit(RNG.normal(size=dk))
    a = RNG.uniform(-1, 1, dk)
    b = 1.3
    A = oracle.transition(k, a, b)
    comm = A - A.T
    np.testing.assert_allclose(comm, b * np.outer(k, k) * (a[:, None] - a[None, :]), atol=1e-14)


def test_at_most_one_complex_pair():
    """Main Findings (Theorems 8/9): a CKDA transition has at most one
    non-real conjugate pair, and one needs both beta > 1 and a negative gate."""
    dk = 8
    seen = 0
    for _ in range(400):
        k = _unit(RNG.normal(size=dk))
        a = RNG.uniform(-1, 1, dk)
        b = RNG.uniform(0, 2)
        m = _nonreal_pairs(oracle.transition(k, a, b))
        assert m <= 1
        if m:
            seen += 1
            assert b > 1 and np.any(a < 0)
        assert _nonreal_pairs(oracle.transition(k, np.abs(a), b)) == 0
        assert _nonreal_pairs(oracle.transition(k, a, RNG.uniform(0, 1))) == 0
    assert seen > 10


def test_orthogonal_and_non_expansive():
    """Theorem 1 direction (signed Householder is orthogonal) and the
    abstract's non-expansiveness: beta = 2, alpha in {+-1}, unit k gives
    A^T A = I; alpha in [-1, 1], beta in [0, 2] gives ||A||_2 <= 1."""
    dk = 10
    for _ in range(100):
        k = _unit(RNG.normal(size=dk))
        A = oracle.transition(k, RNG.choice([-1.0, 1.0], dk), 2.0)
        np.testing.assert_allclose(A.T @ A, np.eye(dk), atol=1e-14)
        B = oracle.transition(k, RNG.uniform(-1, 1, dk), RNG.uniform(0, 2))
        assert np.linalg.norm(B, 2) <= 1 + 1e-13


def test_norm_preserving_transition():
    """Rotation workload reading: with alpha = +-1, beta = 2 and unit keys the
    transition preserves the Frobenius norm, so ||S_t - beta k_t v_t^T|| =
    ||S_{t-1}|| at every step even though the write changes the norm."""
    dk, dv, T = 16, 8, 40
    S = RNG.normal(size=(dk, dv))
    for _ in range(T):
        k = _unit(RNG.normal(size=dk))
        v = RNG.normal(size=dv)
        g = RNG.choice([-1.0, 1.0], dk)
        _, S1 = _run(np.zeros((1, dk)), k[None], v[None], g[None], np.full(1, 2.0), S)
        assert np.linalg.norm(S1 - 2.0 * np.outer(k, v)) == pytest.approx(np.linalg.norm(S),
                                                                            rel=1e-13)
        S = S1


# ---------------------------------------------------------------- sign absorption

def test_sign_absorption_identity():
    """Methodology (ai.info summary): signed gates can be handled by absorbing
    cumulative signs into keys and queries.  With sigma_t = prod_{s<=t}
    sign(alpha_s) per channel (restarting per sequence),
    ckda(q, k, v, alpha) = kda(sigma q, sigma k, v, |alpha|) for o and
    S_T = sigma_T * S_T(kda).  A sign error anywhere in the oracle's gate
    handling breaks this."""
    T, H, dk, dv = 37, 2, 8, 5
    q = RNG.normal(size=(1, T, H, dk))
    k = RNG.normal(size=(1, T, H, dk)) / np.sqrt(dk)
    v = RNG.normal(size=(1, T, H, dv))
    g = RNG.uniform(-1, 1, size=(1, T, H, dk))
    beta = RNG.uniform(0, 2, size=(1, T, H))
    cu = np.array([0, 11, 30, 37])
    S0 = RNG.normal(size=(3, H, dk, dv))
    o, S_T = oracle.forward(q, k, v, g, beta, S0=S0, cu_seqlens=cu)
    sig = np.ones_like(g)
    for a, b in zip(cu[:-1], cu[1:]):
        sig[:, a:b] = np.cumprod(np.sign(g[:, a:b]), axis=1)
    o2, S2 = oracle.forward(sig * q, sig * k, v, np.abs(g), beta, S0=S0, cu_seqlens=cu)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    for n, b in enumerate(cu[1:]):
        np.testing.assert_allclose(S_T[n], sig[0, b - 1][:, :, None] * S2[n], atol=1e-13)


# ---------------------------------------------------------------- layout / packing

def test_packed_equals_separate_and_split_resume():
    """Packed sequences are independent, and the final state is a checkpoint:
    running [0, t1) then [t1, T) from its S_T equals one run over [0, T)."""
    T, H, dk, dv = 30, 2, 4, 3
    q, k, g = (RNG.normal(size=(1, T, H, dk)) for _ in range(3))
    g = np.tanh(g)
    v = RNG.normal(size=(1, T, H, dv))
    beta = RNG.uniform(0, 2, size=(1, T, H))
    cu = np.array([0, 9, 30])
    o, S_T = oracle.forward(q, k, v, g, beta, cu_seqlens=cu)
    for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        sl = slice(a, b)
        o1, S1 = oracle.forward(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl])
        np.testing.assert_allclose(o[:, sl], o1, atol=1e-14)
        np.testing.assert_allclose(S_T[n], S1[0], atol=1e-14)
    # split/resume on the second sequence
    a, m, b = 9, 20, 30
    oa, Sa = oracle.forward(q[:, a:m], k[:, a:m], v[:, a:m], g[:, a:m], beta[:, a:m])
    ob, Sb = oracle.forward(q[:, m:b], k[:, m:b], v[:, m:b], g[:, m:b], beta[:, m:b], S0=Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o[:, a:b], atol=1e-13)
    np.testing.assert_allclose(Sb[0], S_T[1], atol=1e-13)


def test_decode_equals_forward():
    """T decode steps equal a length-T forward."""
    T, N, H, dk, dv = 6, 3, 2, 5, 4
    q, k = RNG.normal(size=(N, T, H, dk)), RNG.normal(size=(N, T, H, dk)) / 3
    v, g = RNG.normal(size=(N, T, H, dv)), RNG.uniform(-1, 1, size=(N, T, H, dk))
    beta = RNG.uniform(0, 2, size=(N, T, H))
    S0 = RNG.normal(size=(N, H, dk, dv))
    o, S_T = oracle.forward(q, k, v, g, beta, S0=S0)
    S = S0.copy()
    for t in range(T):
        ot = oracle.decode_step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], S)
        np.testing.assert_allclose(ot, o[:, t], atol=1e-13)
    np.testing.assert_allclose(S, S_T, atol=1e-13)


# ---------------------------------------------------------------- fused q/k normalisation

def test_l2_normalise_hand_values():
    """The fused key/query normalisation (CKDA summary, "Methodology in Plain
    English": the Triton variant fuses the signs into the normalisation) as
    this build reads it: each row x becomes x (sum x^2 + 1e-6)^(-1/2).  Hand
    values: (3, 4) -> (3, 4) / sqrt(25 + 1e-6); a zero row stays zero; a row
    far below the epsilon is scaled by about 1000 instead of to unit norm."""
    got = oracle.l2_normalise(np.array([[3.0, 4.0], [0.0, 0.0], [1e-6, 0.0]]))
    den = np.sqrt(25.0 + 1e-6)
    np.testing.assert_array_equal(got[0], [3.0 / den, 4.0 / den])
    np.testing.assert_array_equal(got[1], [0.0, 0.0])
    assert got[2, 0] == pytest.approx(1e-6 / np.sqrt(1e-12 + 1e-6), rel=1e-15)
    assert got[2, 0] == pytest.approx(1e-3, rel=1e-6)


def test_l2_normalise_is_per_row_of_the_last_axis():
    """Unit norm along the last axis for every (token, head) row with sum x^2
    >> 1e-6, each row independently (a wrong axis or a shared norm fails),
    direction unchanged, and scale invariance up to the epsilon."""
    x = RNG.normal(size=(3, 5, 4, 16)) * RNG.uniform(0.1, 10.0, size=(3, 5, 4, 1))
    y = oracle.l2_normalise(x)
    norms = np.linalg.norm(y, axis=-1)
    eps_rel = 1e-6 / np.sum(x * x, axis=-1)
    np.testing.assert_allclose(norms, 1.0 / np.sqrt(1.0 + eps_rel), rtol=1e-14)
    cos = np.sum(x * y, axis=-1) / (np.linalg.norm(x, axis=-1) * norms)
    np.testing.assert_allclose(cos, 1.0, rtol=1e-14)
    ss = np.sum(x * x, axis=-1, keepdims=True)
    np.testing.assert_allclose(oracle.l2_normalise(7.0 * x),
                               y * 7.0 * np.sqrt(ss + 1e-6) / np.sqrt(49.0 * ss + 1e-6),
                               rtol=1e-14)
    # one row changed: only that row's output changes
    x2 = x.copy()
    x2[1, 2, 3] *= 3.0
    y2 = oracle.l2_normalise(x2)
    diff = np.any(y2 != y, axis=-1)
    assert diff[1, 2, 3] and diff.sum() == 1
