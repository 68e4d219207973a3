"""The library's calls inside a captured HIP graph: every entry point enqueues
kernels on the caller's stream only (no allocation, no memset, no
synchronisation), so a graph captured around it replays the same kernels.

Each case captures one call, then replays the graph several times with new
input values copied into the captured buffers, the program's own eager calls
and synchronisations between the replays, and checks every replay's outputs
bit for bit against an eager call on the same inputs (the kernels use no
atomics, so a rerun gives the same bits)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_22_amd as ck
from gated_delta_rule_22_amd import workloads as wl
from tests._gpu import say

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _draw(seed, B, T, H, dk, dv, dtype, N):
    """Device inputs of the forward: unit q/k rows, signed gates, beta in [0, 2]."""
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(B, T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.normal(size=(B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.normal(size=(B, T, H, dv))
    g = rng.uniform(0.05, 1, size=(B, T, H, dk)) * np.where(rng.random((B, T, H, dk)) < 0.4, -1, 1)
    beta = rng.uniform(0, 2, size=(B, T, H))
    S0 = rng.normal(size=(N, H, dk, dv)) / np.sqrt(dk * dv)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cast = wl.round_bf16 if dtype == "bf16" else (lambda a: a.astype(np.float32))

    def dev(a, t=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(t)

    return dict(q=dev(cast(q), dt), k=dev(cast(k), dt), v=dev(cast(v), dt),
                g=dev(g.astype(np.float32)), beta=dev(beta.astype(np.float32)),
                S0=dev(S0.astype(np.float32)))


def _refill(static, fresh):
    for name, t in fresh.items():
        static[name].copy_(t)


def _same(got, want, what):
    assert got.shape == want.shape and got.dtype == want.dtype, what
    assert torch.equal(got, want), f"{what}: replay differs from the eager call"


def _capture(fn):
    """Capture fn() on a side stream after one eager warm-up call there."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = fn()
    torch.cuda.synchronize()
    return graph, outs


@pytest.mark.parametrize("no_alloc", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("packed", [False, True])
def test_forward_replays_match_eager(dtype, packed, no_alloc):
    """``no_alloc`` captures ckda_forward_noalloc (outputs allocated before the
    capture, the library's fixed scratch in place of a workspace) and checks it
    against eager ckda_forward calls."""
    H, dk, dv = (2 if no_alloc else 4), 128, 128
    if packed:
        lens = [70, 1, 193, 0, 64]
        B, T = 1, sum(lens)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
        N = len(lens)
    else:
        B, T, cu, N = 2, 150, None, 2
    if no_alloc:   # host-side check that the case fits the fixed scratch
        need = ck.forward_workspace_bytes(
            B, T, H, dk, dv, N, torch.bfloat16 if dtype == "bf16" else torch.float32)
        assert need <= ck.library().ckda_forward_noalloc_max_bytes()
    say(f"[gpu] graph capture of ckda_forward{'_noalloc' if no_alloc else ''} {dtype} "
        f"packed={packed} B={B} T={T} H={H}")
    static = _draw(100, B, T, H, dk, dv, dtype, N)
    o_pre = torch.empty((B, T, H, dv), dtype=torch.float32, device="cuda")
    S_pre = torch.empty((N, H, dk, dv), dtype=torch.float32, device="cuda")

    def call(captured=True):
        if no_alloc and captured:
            return ck.forward(static["q"], static["k"], static["v"], static["g"], static["beta"],
                              S0=static["S0"], cu_seqlens=cu, out=o_pre, final_state=S_pre,
                              no_alloc=True)
        return ck.forward(static["q"], static["k"], static["v"], static["g"], static["beta"],
                          S0=static["S0"], cu_seqlens=cu)

    graph, (o_g, S_g) = _capture(call)
    for r in range(REPLAYS):
        _refill(static, _draw(200 + r, B, T, H, dk, dv, dtype, N))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_e, S_e = call(captured=False)    # eager ckda_forward, on the same inputs
        torch.cuda.synchronize()
        say(f"  replay {r}: |o|max={o_g.abs().max().item():.3f}")
        _same(o_g, o_e, f"o, replay {r}")
        _same(S_g, S_e, f"S_T, replay {r}")


def test_decode_replays_match_eager():
    N, H, dk, dv = 3, 5, 128, 128
    say(f"[gpu] graph capture of ckda_decode_step N={N} H={H} dk={dk} dv={dv}")
    rng = np.random.default_rng(5)
    S_init = torch.from_numpy((rng.normal(size=(N, H, dk, dv)) / np.sqrt(dk * dv))
                              .astype(np.float32)).cuda()

    def step_inputs(seed):
        r = np.random.default_rng(seed)
        f = lambda *s: torch.from_numpy(r.normal(size=s).astype(np.float32)).cuda()
        return dict(q=f(N, H, dk) / np.sqrt(dk), k=f(N, H, dk) / np.sqrt(dk), v=f(N, H, dv),
                    g=torch.from_numpy(r.uniform(-1, 1, size=(N, H, dk)).astype(np.float32)).cuda(),
                    beta=torch.from_numpy(r.uniform(0, 2, size=(N, H)).astype(np.float32)).cuda())

    static = step_inputs(0)
    S_graph = S_init.clone()
    o_static = torch.empty((N, H, dv), dtype=torch.float32, device="cuda")

    def call():
        return ck.decode_step(static["q"], static["k"], static["v"], static["g"],
                              static["beta"], S_graph, out=o_static)

    graph, _ = _capture(call)
    # the warm-up and the capture ran on S_graph: restart both chains from S_init
    S_graph.copy_(S_init)
    S_eager = S_init.clone()
    for r in range(REPLAYS):
        fresh = step_inputs(10 + r)
        _refill(static, fresh)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_e = ck.decode_step(fresh["q"], fresh["k"], fresh["v"], fresh["g"], fresh["beta"],
                             S_eager)
        torch.cuda.synchronize()
        _same(o_static, o_e, f"o, step {r}")
        _same(S_graph, S_eager, f"S, step {r}")


def test_backward_replays_match_eager():
    B, T, H, dk, dv = 1, 130, 3, 64, 64
    say(f"[gpu] graph capture of ckda_backward B={B} T={T} H={H} dk={dk} dv={dv}")
    static = _draw(300, B, T, H, dk, dv, "bf16", B)
    static["do"] = torch.randn((B, T, H, dv), device="cuda")

    def call():
        return ck.backward(static["q"], static["k"], static["v"], static["g"], static["beta"],
                           static["do"], S0=static["S0"])

    graph, grads = _capture(call)
    for r in range(REPLAYS):
        fresh = _draw(400 + r, B, T, H, dk, dv, "bf16", B)
        fresh["do"] = torch.from_numpy(np.random.default_rng(r).normal(size=(B, T, H, dv))
                                       .astype(np.float32)).cuda()
        _refill(static, fresh)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager = call()
        torch.cuda.synchronize()
        for name, got, want in zip(("dq", "dk", "dv", "dg", "dbeta", "dS0"), grads, eager):
            _same(got, want, f"{name}, replay {r}")
