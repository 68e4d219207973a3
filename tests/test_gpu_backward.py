"""GPU parity of the backward (``ckda_backward`` through the C ABI) against the
fp64 CPU oracle's reverse-mode gradient (``oracle.backward``, itself pinned by
finite differences and closed forms) on the same seeded inputs.

Bound.  The library computes every gradient in fp64 from inputs that widen
exactly and rounds it once to fp32, so each element must satisfy

    |got - ref| <= 2^-23 |ref| + 1e-7 rms(ref)

(one fp32 rounding, plus a small allowance for the fp64 arithmetic).  The
gate gradient is dalpha = dln|alpha| / alpha with dln|alpha| a reverse sum
whose terms cancel pairwise, so its fp64 error grows like 1e-16 / |alpha|;
the configs keep |alpha| >= 1e-3, where that stays far below the bound, and
positions with alpha = 0 (differentiated at the log-magnitude floor) are not
compared for dalpha."""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_22_amd as ck
from gated_delta_rule_22_amd import workloads as wl
from tests._gpu import say, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


def _inputs(seed, B, T, H, dk, dv, dtype, cu=None, s0=True, dst=True, gmax=1.0, gmin=0.05,
            bmax=2.0):
    rng = np.random.default_rng(seed)
    N = len(cu) - 1 if cu is not None else B
    q = rng.normal(size=(B, T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.normal(size=(B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.normal(size=(B, T, H, dv))
    g = rng.uniform(gmin, gmax, size=(B, T, H, dk)) * np.where(
        rng.random((B, T, H, dk)) < 0.4, -1, 1)
    beta = rng.uniform(0, bmax, size=(B, T, H))
    S0 = rng.normal(size=(N, H, dk, dv)) / np.sqrt(dk) if s0 else None
    do = rng.normal(size=(B, T, H, dv))
    dST = rng.normal(size=(N, H, dk, dv)) if dst else None
    cast = wl.round_bf16 if dtype == "bf16" else (lambda a: a.astype(np.float32))
    f32 = lambda a: None if a is None else a.astype(np.float32)
    return dict(q=cast(q), k=cast(k), v=cast(v), g=f32(g), beta=f32(beta), S0=f32(S0),
                do=f32(do), dST=f32(dST), cu=None if cu is None else np.asarray(cu, np.int32),
                dtype=dtype)


def _gpu_backward(x, tag, need_dS0=True):
    dt = torch.bfloat16 if x["dtype"] == "bf16" else torch.float32
    cu = None if x["cu"] is None else torch.from_numpy(x["cu"]).to("cuda")
    say(f"[gpu] ckda_backward {tag} q{x['q'].shape} {x['dtype']}")
    out = ck.backward(to_dev(x["q"], dt), to_dev(x["k"], dt), to_dev(x["v"], dt), to_dev(x["g"]),
                      to_dev(x["beta"]), to_dev(x["do"]), S0=to_dev(x["S0"]),
                      dS_T=to_dev(x["dST"]), cu_seqlens=cu, need_dS0=need_dS0)
    torch.cuda.synchronize()
    return [None if t is None else t.cpu().numpy().astype(np.float64) for t in out]


def _oracle_backward(x):
    return oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"], S0=x["S0"],
                           dS_T=x["dST"], cu_seqlens=x["cu"])


def _assert_close(name, got, ref, mask=None):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if mask is not None:
        got, ref = got[mask], ref[mask]
    if ref.size == 0:
        return
    rms = float(np.sqrt(np.mean(ref * ref)))
    excess = np.abs(got - ref) - (2.0 ** -23 * np.abs(ref) + 1e-7 * rms)
    worst = float(np.max(np.abs(got - ref)) / rms) if rms > 0 else float(np.max(np.abs(got)))
    say(f"  {name}: max|d|/rms={worst:.2e}")
    assert np.all(np.isfinite(got)), name
    assert float(np.max(excess)) <= 0.0, (name, worst)


def _compare(x, tag, gate_mask=None):
    got = _gpu_backward(x, tag)
    ref = _oracle_backward(x)
    for name, a, b in zip(NAMES, got, ref):
        _assert_close(name, a, b, gate_mask if name == "dg" else None)
    return got


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_backward_small(dtype, dk, dv):
    """Three chunks per sequence, the last one partial (150 = 2 x 64 + 22)."""
    x = _inputs(21, B=2, T=150, H=2, dk=dk, dv=dv, dtype=dtype)
    _compare(x, f"dk={dk} dv={dv}")


def test_backward_packed_sequences():
    """Packed sequences with an empty one, ragged tails, zero S0 and a
    sequence shorter than one chunk."""
    cu = [0, 70, 70, 200, 333, 340]
    x = _inputs(22, B=1, T=340, H=3, dk=128, dv=128, dtype="bf16", cu=cu, s0=False)
    _compare(x, "packed")


def test_backward_expansive_regime():
    """|alpha| up to 1.1 and beta up to 2.5: the gradient of the definition."""
    x = _inputs(23, B=1, T=200, H=2, dk=64, dv=64, dtype="f32", gmax=1.1, gmin=0.3, bmax=2.5)
    _compare(x, "expansive")


def test_backward_small_gates():
    """|alpha| down to 1e-3, the smallest magnitude the layer workload draws."""
    x = _inputs(24, B=1, T=192, H=2, dk=128, dv=64, dtype="bf16", gmin=1e-3, gmax=0.05)
    _compare(x, "small gates")


def test_backward_zero_gates_take_the_exact_ratio_path():
    """Two zero gates in one chunk on 8 channels: the channel's log-magnitude
    range passes 2000 binary orders and its pair sums use exp2 per pair.  Every
    gradient but dalpha at the zero gates themselves is compared."""
    x = _inputs(25, B=1, T=130, H=1, dk=64, dv=64, dtype="f32")
    x["g"][0, [3, 40, 90], 0, :8] = 0.0
    mask = x["g"] != 0.0
    _compare(x, "zero gates", gate_mask=mask)


def test_backward_without_dS0_and_dS_T():
    x = _inputs(26, B=2, T=64, H=2, dk=64, dv=128, dtype="bf16", dst=False)
    ref = _gpu_backward(x, "with dS0")
    got = _gpu_backward(x, "without dS0", need_dS0=False)
    assert got[5] is None
    for name, a, b in zip(NAMES[:5], got, ref):
        np.testing.assert_array_equal(a, b, err_msg=name)
    orc = _oracle_backward(x)
    for name, a, b in zip(NAMES, ref, orc):
        _assert_close(name, a, b)


def test_backward_empty_sequence_passes_dS_T_through():
    """T = 0: no token, so dS0 = dS_T and every per-token gradient is empty."""
    x = _inputs(27, B=1, T=0, H=2, dk=64, dv=64, dtype="f32")
    got = _gpu_backward(x, "T=0")
    np.testing.assert_array_equal(got[5], x["dST"].astype(np.float64))
    for a in got[:5]:
        assert a.size == 0


def test_backward_full_size():
    """The 1.3B-layer shape (B=8, T=4096, H=16, d=128, bf16) as one call; the
    oracle recomputes every sequence and head, and every element of every
    gradient is compared."""
    w = wl.WORKLOADS["layer_1p3b_bf16"]
    x = wl.forward_inputs(w, seed=0)
    rng = np.random.default_rng(28)
    B, T, H, dk = x["q"].shape
    dv = x["v"].shape[-1]
    x = dict(q=x["q"], k=x["k"], v=x["v"], g=x["g"], beta=x["beta"], S0=x.get("S0"),
             do=rng.normal(size=(B, T, H, dv)).astype(np.float32),
             dST=rng.normal(size=(B, H, dk, dv)).astype(np.float32), cu=None, dtype="bf16")
    got = _gpu_backward(x, "layer_1p3b_bf16")
    ref = _oracle_backward(x)
    say(f"  all {B} sequences")
    for name, a, r in zip(NAMES, got, ref):
        _assert_close(name, a, r)


def test_kda_backward_uses_gate_magnitudes():
    """kda_backward is the backward of the recurrence on |g|: every gradient
    matches the oracle's on |g|, with dg = d/d|g| * sign(g)."""
    x = _inputs(29, B=1, T=140, H=2, dk=64, dv=128, dtype="bf16")
    dt = torch.bfloat16
    say("[gpu] kda_backward")
    got = ck.backward(to_dev(x["q"], dt), to_dev(x["k"], dt), to_dev(x["v"], dt), to_dev(x["g"]),
                      to_dev(x["beta"]), to_dev(x["do"]), S0=to_dev(x["S0"]),
                      dS_T=to_dev(x["dST"]), kda=True)
    torch.cuda.synchronize()
    got = [t.cpu().numpy().astype(np.float64) for t in got]
    ga = np.abs(x["g"])
    ref = list(oracle.backward(x["q"], x["k"], x["v"], ga, x["beta"], x["do"], S0=x["S0"],
                               dS_T=x["dST"]))
    ref[3] = ref[3] * np.sign(x["g"])
    for name, a, b in zip(NAMES, got, ref):
        _assert_close(name, a, b)


def test_kda_backward_equals_ckda_backward_on_nonnegative_gates():
    x = _inputs(30, B=2, T=100, H=2, dk=128, dv=64, dtype="f32")
    x["g"] = np.abs(x["g"])
    dt = torch.float32
    args = (to_dev(x["q"], dt), to_dev(x["k"], dt), to_dev(x["v"], dt), to_dev(x["g"]),
            to_dev(x["beta"]), to_dev(x["do"]))
    kw = dict(S0=to_dev(x["S0"]), dS_T=to_dev(x["dST"]))
    say("[gpu] kda_backward vs ckda_backward, alpha >= 0")
    a = ck.backward(*args, **kw)
    b = ck.backward(*args, **kw, kda=True)
    torch.cuda.synchronize()
    for name, u, w in zip(NAMES, a, b):
        assert torch.equal(u, w), name


def test_backward_is_deterministic():
    """No atomics or order-dependent reductions: two calls agree bit for bit."""
    x = _inputs(31, B=2, T=130, H=2, dk=128, dv=128, dtype="bf16")
    a = _gpu_backward(x, "call 1")
    b = _gpu_backward(x, "call 2")
    for name, u, w in zip(NAMES, a, b):
        np.testing.assert_array_equal(u, w, err_msg=name)


def test_backward_packed_equals_separate_calls():
    """Sequences packed with cu_seqlens give the same gradients, bit for bit,
    as each sequence run on its own (chunks restart at every sequence)."""
    lens = [70, 129, 64]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = _inputs(32, B=1, T=int(cu[-1]), H=2, dk=64, dv=64, dtype="f32", cu=cu)
    packed = _gpu_backward(x, "packed")
    for n, (s0, s1) in enumerate(zip(cu[:-1], cu[1:])):
        sub = dict(x)
        for key in ("q", "k", "v", "g", "beta", "do"):
            sub[key] = np.ascontiguousarray(x[key][:, s0:s1])
        sub["S0"] = np.ascontiguousarray(x["S0"][n:n + 1])
        sub["dST"] = np.ascontiguousarray(x["dST"][n:n + 1])
        sub["cu"] = None
        one = _gpu_backward(sub, f"sequence {n}")
        for name, a, b in zip(NAMES[:5], packed[:5], one[:5]):
            np.testing.assert_array_equal(a[:, s0:s1], b, err_msg=f"{name} seq {n}")
        np.testing.assert_array_equal(packed[5][n:n + 1], one[5], err_msg=f"dS0 seq {n}")


def test_backward_is_linear_in_the_upstream_gradients():
    """Every gradient is linear in (d_o, dS_T), up to the fp32 rounding of the
    three results compared (one half-ulp each) and the fp64 allowance."""
    x = _inputs(33, B=1, T=100, H=2, dk=64, dv=64, dtype="f32")
    rng = np.random.default_rng(34)
    # upstream gradients on a 2^-8 grid, so that their fp32 sums are exact
    grid = lambda shape: (rng.integers(-512, 513, size=shape) / 256.0).astype(np.float32)
    d1, d2 = grid(x["do"].shape), grid(x["do"].shape)
    s1, s2 = grid(x["dST"].shape), grid(x["dST"].shape)
    x = dict(x, do=d1, dST=s1)
    y = dict(x, do=d2, dST=s2)
    xs = dict(x, do=d1 + d2, dST=s1 + s2)
    a, b, s = _gpu_backward(x, "d1"), _gpu_backward(y, "d2"), _gpu_backward(xs, "d1 + d2")
    for name, u, w, z in zip(NAMES, a, b, s):
        rms = np.sqrt(np.mean(z * z))
        bound = 2.0 ** -24 * (np.abs(u) + np.abs(w) + np.abs(z)) + 1e-7 * rms
        ex = np.abs(u + w - z) - bound
        j = np.unravel_index(np.argmax(ex), ex.shape)
        assert ex[j] <= 0.0, (name, j, u[j], w[j], z[j], float(np.abs(u + w - z)[j]), rms)


def test_backward_packed_64k():
    """The packed 64K-token workload (12 sequences of 1167 to 16384 tokens, not
    chunk aligned, H = 16, d = 128, bf16) as one call; the oracle recomputes
    every sequence and head, and every element of every gradient is
    compared."""
    w = wl.WORKLOADS["varlen_64k_bf16"]
    x = wl.forward_inputs(w, seed=0)
    cu = np.asarray(x["cu_seqlens"], np.int64)
    N = len(cu) - 1
    _, T, H, dk = x["q"].shape
    dv = x["v"].shape[-1]
    rng = np.random.default_rng(35)
    x = dict(q=x["q"], k=x["k"], v=x["v"], g=x["g"], beta=x["beta"], S0=None,
             do=rng.normal(size=(1, T, H, dv)).astype(np.float32),
             dST=rng.normal(size=(N, H, dk, dv)).astype(np.float32),
             cu=cu.astype(np.int32), dtype="bf16")
    got = _gpu_backward(x, "varlen_64k_bf16")
    ref = _oracle_backward(x)
    say(f"  all {N} sequences")
    for name, a, r in zip(NAMES, got, ref):
        _assert_close(name, a, r)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kda", [False, True])
def test_backward_through_qk_normalisation(dtype, kda):
    """ckda_backward_ex with CKDA_OPT_QK_L2NORM (and KDA mode): the gradient
    with respect to the raw keys and queries, through the fused normalisation,
    against the oracle's chain rule.  Unnormalised inputs, so the Jacobian of
    the normalisation matters."""
    x = _inputs(36, B=2, T=140, H=2, dk=128, dv=64, dtype=dtype)
    rng = np.random.default_rng(36)
    cast = wl.round_bf16 if dtype == "bf16" else (lambda a: a.astype(np.float32))
    x["q"] = cast(rng.normal(size=x["q"].shape) * 0.7)
    x["k"] = cast(rng.normal(size=x["k"].shape) * 0.3)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    say(f"[gpu] ckda_backward_ex L2NORM kda={kda} {dtype}")
    got = ck.backward(to_dev(x["q"], dt), to_dev(x["k"], dt), to_dev(x["v"], dt), to_dev(x["g"]),
                      to_dev(x["beta"]), to_dev(x["do"]), S0=to_dev(x["S0"]),
                      dS_T=to_dev(x["dST"]), kda=kda, normalize_qk=True)
    torch.cuda.synchronize()
    got = [t.cpu().numpy().astype(np.float64) for t in got]
    g = np.abs(x["g"]) if kda else x["g"]
    ref = list(oracle.backward(x["q"], x["k"], x["v"], g, x["beta"], x["do"], S0=x["S0"],
                               dS_T=x["dST"], normalize_qk=True))
    if kda:
        ref[3] = ref[3] * np.sign(x["g"])
    for name, a, b in zip(NAMES, got, ref):
        _assert_close(name, a, b)
