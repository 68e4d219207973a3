"""GPU-side invariants that need no oracle run: checkpoint/resume, packing,
decode-vs-forward agreement, determinism, and the exact special cases the
pages fix (quarter turn, orthogonal transitions preserve the state norm)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_22_amd as ck
from gated_delta_rule_22_amd import workloads as wl
from tests._gpu import TOL, rel_err, say, to_dev, upload
from tests.test_gpu_parity import _rand_forward

pytestmark = pytest.mark.gpu


def _fwd(d, **kw):
    o, S = ck.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d.get("S0"),
                      cu_seqlens=d.get("cu_seqlens"), **kw)
    torch.cuda.synchronize()
    return o, S


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_split_resume(dtype):
    """Forward over [0, T) equals [0, t1) followed by [t1, T) from its S_T
    (t1 = 100 is not a chunk boundary)."""
    x = _rand_forward(21, B=2, T=300, H=2, dk=128, dv=128, dtype=dtype)
    d = upload(x)
    say(f"[gpu] split/resume {dtype}")
    o, S = _fwd(d)
    t1 = 100
    a = {k_: (v_[:, :t1].contiguous() if k_ in ("q", "k", "v", "g", "beta") else v_)
         for k_, v_ in d.items()}
    b = {k_: (v_[:, t1:].contiguous() if k_ in ("q", "k", "v", "g", "beta") else v_)
         for k_, v_ in d.items()}
    oa, Sa = _fwd(a)
    b["S0"] = Sa
    ob, Sb = _fwd(b)
    tol = TOL[dtype]
    assert rel_err(torch.cat([oa, ob], 1).cpu().numpy(), o.cpu().numpy()) <= tol
    assert rel_err(Sb.cpu().numpy(), S.cpu().numpy()) <= tol


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_packed_equals_separate(dtype):
    lens = [70, 1, 129, 64]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = _rand_forward(22, B=1, T=int(cu[-1]), H=2, dk=128, dv=64, dtype=dtype, cu=cu)
    d = upload(x)
    say(f"[gpu] packed vs separate {dtype}")
    o, S = _fwd(d)
    for n, (s, e) in enumerate(zip(cu[:-1], cu[1:])):
        dn = {k_: d[k_][:, s:e].contiguous() for k_ in ("q", "k", "v", "g", "beta")}
        dn["S0"] = d["S0"][n:n + 1].contiguous()
        on, Sn = _fwd(dn)
        assert rel_err(on.cpu().numpy(), o[:, s:e].cpu().numpy()) <= TOL[dtype]
        assert rel_err(Sn.cpu().numpy(), S[n:n + 1].cpu().numpy()) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_steps_equal_forward(dtype):
    x = _rand_forward(23, B=4, T=20, H=3, dk=128, dv=128, dtype=dtype)
    d = upload(x)
    say(f"[gpu] decode x T vs forward {dtype}")
    o, S = _fwd(d)
    St = d["S0"].clone()
    for t in range(20):
        ot = ck.decode_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                            d["v"][:, t].contiguous(), d["g"][:, t].contiguous(),
                            d["beta"][:, t].contiguous(), St)
        assert rel_err(ot.cpu().numpy(), o[:, t].cpu().numpy()) <= TOL[dtype]
    assert rel_err(St.cpu().numpy(), S.cpu().numpy()) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_deterministic(dtype):
    """No atomics on the path: two runs are bitwise identical."""
    x = _rand_forward(24, B=2, T=200, H=4, dk=128, dv=128, dtype=dtype)
    d = upload(x)
    say(f"[gpu] determinism {dtype}")
    o1, S1 = _fwd(d)
    o2, S2 = _fwd(d)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_quarter_turn_at_real_shape():
    """Blog "One update, one quarter turn": gate (-1, 1), beta = 2,
    k = (e1 + e2)/sqrt(2) turns rows 1-2 of the state by 90 degrees and fixes
    the rest; v = 0, so after 4m tokens the state is back (fp32 inputs).
    beta k k^T is the same matrix for k = e1 + e2 and beta = 1, which fp32
    holds exactly (sqrt(1/2) it does not), so the turn is exact here."""
    dk = dv = 128
    T = 4 * 33
    k = np.zeros((1, T, 1, dk), np.float32)
    k[..., :2] = 1.0
    g = np.ones((1, T, 1, dk), np.float32)
    g[..., 0] = -1.0
    rng = np.random.default_rng(3)
    S0 = rng.normal(size=(1, 1, dk, dv)).astype(np.float32)
    q = rng.normal(size=(1, T, 1, dk)).astype(np.float32)
    x = dict(q=q, k=k, v=np.zeros((1, T, 1, dv), np.float32), g=g,
             beta=np.full((1, T, 1), 1.0, np.float32), S0=S0, cu_seqlens=None, dtype="f32")
    say("[gpu] quarter turn dk=128 T=132")
    o, S = _fwd(upload(x))
    S = S.cpu().numpy()[0, 0]
    assert rel_err(S, S0[0, 0]) <= 1e-6
    # readout after the first token: rows 1-2 rotated by 90 degrees
    S1 = S0[0, 0].astype(np.float64).copy()
    S1[:2] = np.array([[0.0, -1.0], [1.0, 0.0]]) @ S1[:2]
    assert rel_err(o.cpu().numpy()[0, 0, 0], q[0, 0, 0] @ S1) <= 1e-6


def test_rotation_norm_preserved():
    """Rotation workload with v = 0: every transition is orthogonal, so the
    state's Frobenius norm stays 1 over all 4096 tokens (fp32 inputs)."""
    x = wl.forward_inputs("rotation_f32")
    x["v"] = np.zeros_like(x["v"])
    say("[gpu] rotation_f32 with v = 0")
    _, S = _fwd(upload(x))
    n = np.linalg.norm(S.cpu().numpy().astype(np.float64), axis=(-2, -1))
    np.testing.assert_allclose(n, 1.0, atol=1e-5)


def test_zero_length_and_identity_state():
    """T = 0 leaves the state untouched; an empty packed sequence returns its
    S0."""
    rng = np.random.default_rng(4)
    S0 = torch.from_numpy(rng.normal(size=(2, 3, 64, 64)).astype(np.float32)).cuda()
    z = lambda *s: torch.zeros(*s, device="cuda")
    say("[gpu] T = 0")
    o, S = ck.forward(z(2, 0, 3, 64).bfloat16(), z(2, 0, 3, 64).bfloat16(),
                      z(2, 0, 3, 64).bfloat16(), z(2, 0, 3, 64), z(2, 0, 3), S0=S0)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 3, 64) and torch.equal(S, S0)


def test_exact_zero_gate_and_large_beta():
    """alpha = 0 exactly on some tokens (the state is wiped on those channels)
    and beta beyond 2 are computed per the definition."""
    import oracle
    x = _rand_forward(25, B=1, T=160, H=2, dk=128, dv=128, dtype="f32")
    x["g"][0, 40:43, :, :5] = 0.0
    x["g"][0, 100, 1, :] = 0.0
    x["beta"][0, 10:20] = 2.6
    say("[gpu] zero gates, beta 2.6")
    o, S = _fwd(upload(x))
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], S0=x["S0"])
    assert rel_err(o.cpu().numpy(), o_ref) <= 1e-5
    assert rel_err(S.cpu().numpy(), S_ref) <= 1e-5


def test_segment_transition_composes_at_real_shape():
    """The building block of sharding one long sequence over several GPUs, on
    one GPU at the rotation workload's real shape (fp32, T = 4096, H = 4,
    d = 128; gates +-1, beta = 2, unit keys): split at t1 = 2000 (not a chunk
    boundary).  Running the second segment from S0 = I with v = 0 extracts its
    transition M = prod A_t (dk x dk); from S0 = 0 with the real v, its offset
    R.  Then the full run's S_T = M S_mid + R, where S_mid is the first
    segment's final state, and M is orthogonal (every A_t is, at beta = 2,
    |alpha| = 1, |k| = 1)."""
    w = wl.scaled("rotation_f32", B=1)
    x = wl.forward_inputs(w)
    d = upload(x)
    dk = x["q"].shape[-1]
    t1 = 2000
    seg = lambda lo, hi: {k_: d[k_][:, lo:hi].contiguous() for k_ in ("q", "k", "v", "g", "beta")}
    say("[gpu] segment transition composition, rotation shape")
    _, S_full = _fwd(d)
    a = seg(0, t1)
    a["S0"] = d["S0"]
    _, S_mid = _fwd(a)
    b = seg(t1, x["q"].shape[1])
    H = x["q"].shape[2]
    eye = torch.eye(dk, device="cuda").expand(1, H, dk, dk).contiguous()
    bm = dict(b, v=torch.zeros_like(b["v"]), S0=eye)
    _, M = _fwd(bm)
    br = dict(b, S0=None)
    _, Rr = _fwd(br)
    composed = torch.matmul(M.double(), S_mid.double()) + Rr.double()
    assert rel_err(composed.cpu().numpy(), S_full.cpu().numpy()) <= TOL["f32"]
    Mt = M.double()
    gram = torch.matmul(Mt.transpose(-1, -2), Mt)
    err = (gram - torch.eye(dk, device="cuda", dtype=torch.float64)).abs().max().item()
    say(f"  |M^T M - I|_max = {err:.2e}")
    assert err <= 1e-4


def test_forward_is_linear_in_values_and_initial_state():
    """With q, k, alpha, beta fixed, (o, S_T) is linear in (v, S0).  Inputs on
    a 2^-8 grid so that the fp32 sums are exact; fp64 arithmetic inside."""
    x = _rand_forward(23, B=2, T=150, H=2, dk=64, dv=64, dtype="f32")
    rng = np.random.default_rng(23)
    grid = lambda shape: (rng.integers(-256, 257, size=shape) / 256.0).astype(np.float32)
    v1, v2 = grid(x["v"].shape), grid(x["v"].shape)
    s1, s2 = grid(x["S0"].shape), grid(x["S0"].shape)
    run = lambda v, s: _fwd(upload(dict(x, v=v, S0=s)))
    say("[gpu] linearity in (v, S0)")
    o1, S1 = run(v1, s1)
    o2, S2 = run(v2, s2)
    o3, S3 = run(v1 + v2, s1 + s2)
    for a, b, c in ((o1, o2, o3), (S1, S2, S3)):
        a, b, c = (t.double().cpu().numpy() for t in (a, b, c))
        bound = 2.0 ** -24 * (np.abs(a) + np.abs(b) + np.abs(c)) + 1e-12 * np.sqrt(np.mean(c * c))
        assert np.all(np.abs(a + b - c) <= 2 * bound)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_head_permutation_equivariance(dtype):
    """Heads are independent: permuting them in the inputs permutes the
    outputs, bit for bit."""
    x = _rand_forward(24, B=2, T=130, H=4, dk=128, dv=128, dtype=dtype)
    d = upload(x)
    perm = torch.tensor([2, 0, 3, 1], device="cuda")
    dp = {k_: (v_.index_select(2, perm).contiguous() if k_ in ("q", "k", "v", "g", "beta")
               else v_.index_select(1, perm).contiguous() if k_ == "S0" and v_ is not None
               else v_) for k_, v_ in d.items()}
    say(f"[gpu] head permutation {dtype}")
    o, S = _fwd(d)
    op, Sp = _fwd(dp)
    assert torch.equal(op, o.index_select(2, perm))
    assert torch.equal(Sp, S.index_select(1, perm))
