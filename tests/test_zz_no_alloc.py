"""ckda_forward_noalloc (the entry point that allocates nothing, for callers
that cannot allocate) against ckda_forward / ckda_forward_ex through the C ABI:
bit-identical results, twice in a row on the shared fixed scratch with the
second call smaller than the first, for bf16 packed sequences (the scratch
holds the sequence table) and fp32 inputs (the scratch holds the chunk
records), and agreement with the oracle within the parity bound."""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_22_amd as ck
from tests._gpu import TOL, rel_err, say, upload
from tests.test_gpu_parity import _rand_forward

pytestmark = pytest.mark.gpu


def _both(x, **kw):
    d = upload(x)
    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    N = B if d["cu_seqlens"] is None else d["cu_seqlens"].numel() - 1
    o_dt = torch.bfloat16 if kw.get("out_dtype") == torch.bfloat16 else torch.float32
    o_na = torch.full((B, T, H, dv), float("nan"), dtype=o_dt, device="cuda")
    S_na = torch.full((N, H, dk, dv), float("nan"), device="cuda")
    ck.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"],
               cu_seqlens=d["cu_seqlens"], out=o_na, final_state=S_na, no_alloc=True, **kw)
    o_ws, S_ws = ck.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"],
                            cu_seqlens=d["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    return o_na, S_na, o_ws, S_ws


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry_twice(dtype):
    cases = [([300, 1, 129, 64, 0, 77], 2), ([70, 50], 1)]   # second call smaller
    for n, (lens, H) in enumerate(cases):
        cu = np.concatenate([[0], np.cumsum(lens)])
        x = _rand_forward(80 + n, B=1, T=int(cu[-1]), H=H, dk=128, dv=128, dtype=dtype, cu=cu)
        say(f"[gpu] ckda_forward_noalloc {dtype} call {n} lens={lens} H={H}")
        o_na, S_na, o_ws, S_ws = _both(x)
        assert torch.equal(o_na, o_ws) and torch.equal(S_na, S_ws)
        o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], S0=x["S0"],
                                      cu_seqlens=x["cu_seqlens"])
        assert rel_err(o_na.cpu().numpy(), o_ref) <= TOL[dtype]
        assert rel_err(S_na.cpu().numpy(), S_ref) <= TOL[dtype]


def test_noalloc_with_options_uniform_rows():
    """Uniform rows (no table) with the KDA and bf16-output options."""
    for n, (B, T) in enumerate([(3, 200), (2, 65)]):
        x = _rand_forward(90 + n, B=B, T=T, H=2, dk=64, dv=128, dtype="bf16")
        say(f"[gpu] ckda_forward_noalloc options B={B} T={T}")
        o_na, S_na, o_ws, S_ws = _both(x, kda=True, out_dtype=torch.bfloat16)
        assert torch.equal(o_na, o_ws) and torch.equal(S_na, S_ws)


def test_noalloc_rejects_calls_beyond_its_scratch():
    x = _rand_forward(95, B=2, T=4096, H=4, dk=128, dv=128, dtype="f32")
    d = upload(x)
    say("[gpu] ckda_forward_noalloc too large")
    with pytest.raises(ck.CkdaError, match="status 8"):
        ck.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"], no_alloc=True)
