"""Failure containment on the GPU, forced from the host: a NaN in one (sequence,
head) stays there, offsets in cu_seqlens that decrease or leave [0, T] never
make a kernel read or write outside its sequence, and the debug mode
(CKDA_DEBUG) rejects such offsets and poisons the workspace without changing
valid results.  No case here makes a kernel fault: every input is one the
kernels bound by construction."""
import os

import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_22_amd as ck
from tests._gpu import TOL, rel_err, say, to_dev, upload
from tests.test_gpu_parity import _rand_forward

pytestmark = pytest.mark.gpu


def _fwd(d):
    o, S = ck.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d.get("S0"),
                      cu_seqlens=d.get("cu_seqlens"))
    torch.cuda.synchronize()
    return o.cpu().numpy(), S.cpu().numpy()


def _monotone(cu, T):
    """The sequence boundaries the library uses: P_i = clamp(max(cu[0..i]), 0, T)."""
    return np.clip(np.maximum.accumulate(np.asarray(cu, np.int64)), 0, T)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("what", ["k", "g"])
def test_nan_in_one_head_stays_there(dtype, what):
    """A NaN in one token of one (row, head) -- in its key or its gate -- leaves
    every other (row, head) bit-identical to a clean run."""
    x = _rand_forward(71, B=2, T=200, H=3, dk=128, dv=128, dtype=dtype)
    d = upload(x)
    say(f"[gpu] NaN isolation {dtype} {what}: clean run")
    o0, S0 = _fwd(d)
    d[what][1, 70, 2, 5] = float("nan")
    say(f"[gpu] NaN isolation {dtype} {what}: poisoned run")
    o1, S1 = _fwd(d)
    mask_o = np.ones(o0.shape[:3], bool)
    mask_o[1, :, 2] = False
    assert np.array_equal(o1[mask_o], o0[mask_o])
    mask_s = np.ones(S0.shape[:2], bool)
    mask_s[1, 2] = False
    assert np.array_equal(S1[mask_s], S0[mask_s])
    # the poisoned pair itself: chunks before the NaN's chunk are untouched.  A
    # NaN key propagates; a NaN gate has no magnitude above the floor the
    # kernels clamp log2|alpha| to, so it acts as a gate of magnitude 2^-126
    # (fp32 inputs: 2^-1000) and the pair's later outputs change but stay finite.
    if what == "k":
        assert np.isnan(o1[1, 70:, 2]).any() and np.isnan(S1[1, 2]).any()
    else:
        assert not np.array_equal(o1[1, 70:, 2], o0[1, 70:, 2])
    assert np.array_equal(o1[1, :64, 2], o0[1, :64, 2])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_nan_in_one_packed_sequence_stays_there(dtype):
    """Packed sequences of one head: a NaN in sequence 1 leaves sequences 0 and
    2 (same head) bit-identical."""
    lens = [130, 90, 77]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = _rand_forward(72, B=1, T=int(cu[-1]), H=2, dk=128, dv=64, dtype=dtype, cu=cu)
    d = upload(x)
    say(f"[gpu] NaN isolation packed {dtype}")
    o0, S0 = _fwd(d)
    d["v"][0, 150, 0, 3] = float("nan")
    o1, S1 = _fwd(d)
    for n, (s, e) in enumerate(zip(cu[:-1], cu[1:])):
        if n == 1:
            assert np.isnan(o1[0, 150:e, 0]).any()
            continue
        assert np.array_equal(o1[0, s:e], o0[0, s:e])
        assert np.array_equal(S1[n], S0[n])
    assert np.array_equal(o1[0, cu[1]:cu[2], 1], o0[0, cu[1]:cu[2], 1])   # other head


def test_nan_in_one_head_stays_there_backward():
    """The backward: a NaN in one head's key leaves every gradient of the other
    heads bit-identical."""
    x = _rand_forward(73, B=1, T=150, H=3, dk=64, dv=64, dtype="f32")
    d = upload(x)
    rng = np.random.default_rng(5)
    do = to_dev(rng.normal(size=x["v"].shape).astype(np.float32))
    run = lambda: [t.cpu().numpy() for t in
                   ck.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], do, S0=d["S0"])]
    say("[gpu] NaN isolation backward")
    clean = run()
    d["k"][0, 40, 1, 2] = float("nan")
    bad = run()
    for name, a, b in zip(("dq", "dk", "dv", "dg", "dbeta", "dS0"), clean, bad):
        head_axis = 1 if name == "dS0" else 2
        keep = [h for h in range(3) if h != 1]
        assert np.array_equal(np.take(a, keep, axis=head_axis),
                              np.take(b, keep, axis=head_axis)), name


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("cu", [[0, 120, 50, 200, 180], [-5, 80, 300, 40, 150]])
def test_non_monotone_offsets_are_made_monotone(dtype, cu):
    """Offsets that decrease or leave [0, T] (T = 200): sequence n covers
    [P_n, P_{n+1}) with P_i = clamp(max(cu[0..i]), 0, T), so sequences never
    overlap (an overlap would let the fp32 path index chunk records past the
    workspace).  Checked against the oracle on those boundaries."""
    T = 200
    P = _monotone(cu, T)
    x = _rand_forward(74, B=1, T=T, H=2, dk=128, dv=128, dtype=dtype, cu=P)
    x["cu_seqlens"] = np.asarray(cu, np.int32)
    d = upload(x)
    say(f"[gpu] non-monotone cu_seqlens {cu} {dtype}")
    o, S = _fwd(d)
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], S0=x["S0"],
                                  cu_seqlens=P)
    rows = slice(int(P[0]), int(P[-1]))
    assert rel_err(o[:, rows], o_ref[:, rows]) <= TOL[dtype]
    assert rel_err(S, S_ref) <= TOL[dtype]


def test_non_monotone_offsets_backward():
    """The backward with overlapping offsets [0, T, 0, T] (T = 130): the second
    sequence is empty, so its dS0 is dS_T, and the first is the whole range."""
    T = 130
    cu = [0, T, 0, T]
    P = _monotone(cu, T)
    x = _rand_forward(75, B=1, T=T, H=2, dk=64, dv=64, dtype="f32", cu=P)
    rng = np.random.default_rng(6)
    do = rng.normal(size=x["v"].shape).astype(np.float32)
    dST = rng.normal(size=(3, 2, 64, 64)).astype(np.float32)
    d = upload(x)
    say(f"[gpu] non-monotone cu_seqlens backward {cu}")
    got = ck.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], to_dev(do), S0=d["S0"],
                      dS_T=to_dev(dST), cu_seqlens=torch.tensor(cu, dtype=torch.int32,
                                                                device="cuda"))
    torch.cuda.synchronize()
    ref = oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, S0=x["S0"],
                          dS_T=dST, cu_seqlens=P)
    for name, a, b in zip(("dq", "dk", "dv", "dg", "dbeta", "dS0"), got, ref):
        a = a.cpu().numpy().astype(np.float64)
        bound = 2.0 ** -23 * np.abs(b) + 1e-7 * np.sqrt(np.mean(b * b))
        assert np.all(np.abs(a - b) <= bound), name


@pytest.fixture
def debug_env():
    os.environ["CKDA_DEBUG"] = "1"
    yield
    os.environ.pop("CKDA_DEBUG", None)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_debug_mode_rejects_bad_offsets_and_keeps_results(dtype, debug_env):
    """CKDA_DEBUG=1: the host validator rejects offsets that are not
    non-decreasing from 0 to T (status CKDA_ERR_SHAPE, nothing launched), and
    a valid call -- with its workspace filled with NaN first -- returns
    exactly what it returns without the debug mode."""
    lens = [70, 0, 129, 64]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = _rand_forward(76, B=1, T=int(cu[-1]), H=2, dk=128, dv=128, dtype=dtype, cu=cu)
    d = upload(x)
    say(f"[gpu] debug mode {dtype}")
    o_dbg, S_dbg = _fwd(d)
    os.environ["CKDA_DEBUG"] = "0"
    o_ref, S_ref = _fwd(d)
    os.environ["CKDA_DEBUG"] = "1"
    assert np.array_equal(o_dbg, o_ref) and np.array_equal(S_dbg, S_ref)
    T = int(cu[-1])
    for bad in ([0, 70, 60, 199, T], [1, 70, 70, 199, T], [0, 70, 70, 199, T + 1]):
        d["cu_seqlens"] = torch.tensor(bad, dtype=torch.int32, device="cuda")
        with pytest.raises(ck.CkdaError, match="status 2"):
            _fwd(d)
