"""Benchmark of the CKDA hot path on one MI355X.

One step = one chunkwise forward over the 1.3B-LM-shaped layer workload
(B=8, T=4096, H=16, dk=dv=128, bf16 q/k/v, fp32 gates and state, chunk 64):
32768 tokens.  The headline value is forward tokens/s.  The same run also
times the recurrent decode workload (256 sequences x 16 heads, 1024
consecutive in-place steps) and reports steps/s and HBM GB/s.

Inputs are seeded synthetic draws (gated_delta_rule_22_amd.workloads), already
resident in device memory when the timed region starts.  Timing uses HIP
events on the stream the library launches on.  The CPU baseline is the fp64
oracle (test infrastructure) on the same forward workload, on 16 host threads
(the host's share per GPU on the measurement boxes), with the CPU model and the
visible thread count recorded beside it.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CKDA fwd tokens/s (H=16,d=128,bf16) + %MFMA peak; decode steps/s + HBM GB/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
F64_PEAK_TFLOPS = 78.6         # MI355X fp64 (vector and matrix)
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix


def fwd_algorithmic(w):
    """Compulsory HBM bytes and dense chunked flops of one forward."""
    th = w.B * w.T * w.H
    in_sz = 2 if w.dtype == "bf16" else 4
    per_th = in_sz * (2 * w.dk + w.dv) + 4 * w.dk + 4 + 4 * w.dv   # q,k,v + alpha + beta + o
    state = w.B * w.H * w.dk * w.dv * 4                              # S_T written (S0 = 0)
    if w.s0 != "zero":
        state *= 2
    C = w.chunk
    flops = th * (2 * C * (3 * w.dk + 2 * w.dv) + 6 * w.dk * w.dv)
    return th * per_th + state, flops, per_th


def profiled_traffic(summary, source):
    """HBM bytes per launch from a committed rocprofv3 summary under profiles/,
    or None when the kernel source has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", "`")):
            key, _, val = line.partition(":")
            fields[key.strip()] = val.strip().split()[0] if val.strip() else ""
    try:
        digest = hashlib.sha256(open(os.path.join(ROOT, source), "rb").read()).hexdigest()
        if fields.get("source_sha256") != digest:
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError, OSError):
        return None


def bwd_algorithmic(w):
    """Compulsory HBM bytes of one backward (inputs and upstream gradients read
    once, gradients written once) and its fp64 flop count, both per launch.

    Flops per (64-token chunk, head), counting each product's nonzero work (a
    product with a triangular factor at half; the matrix-core kernels execute
    the full tiles) (C = 64, d = dk = dv): the chunk records (A, P, T, W, Ubar)
    4 C^2 d + C^3 / 3 + 2 C^2 d; the forward's state pass (U and the state
    update) 4 C d^2; the reverse state pass (dU, dS) 6 C d^2 + C^2 d; the
    chunk gradients (dX, dP, dA, three C x d x d products, pair sums)
    3 C^2 d + 6 C d^2 + 4 C^2 d."""
    th = w.B * w.T * w.H
    in_sz = 2 if w.dtype == "bf16" else 4
    per_th = (in_sz * (2 * w.dk + w.dv) + 4 * w.dk + 4 + 4 * w.dv        # q,k,v,alpha,beta,dO
              + 4 * (3 * w.dk + w.dv) + 4)                               # dq,dk,dalpha,dv,dbeta
    states = 2 * w.B * w.H * w.dk * w.dv * 4                             # dS_T read, dS0 written
    C, d = w.chunk, w.dk
    per_chunk = (4 * C * C * d + C ** 3 // 3 + 2 * C * C * d + 4 * C * d * d
                 + 6 * C * d * d + C * C * d + 3 * C * C * d + 6 * C * d * d + 4 * C * C * d)
    chunks = w.B * ((w.T + C - 1) // C) * w.H
    return th * per_th + states, chunks * per_chunk, per_th


def decode_algorithmic(w):
    nh = w.B * w.H
    per_head = 2 * w.dk * w.dv * 4 + 2 * (2 * w.dk + w.dv) + 4 * w.dk + 4 + 4 * w.dv
    return nh * per_head, per_head


def _cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo ("unknown" if absent)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU's clocks need about 50 forward launches (~30 ms) to reach their steady
    # state; the defaults warm up past that and time 100 steps (~55 ms).
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="seconds of untimed forward launches before the warm-up steps")
    ap.add_argument("--decode-steps", type=int, default=None,
                    help="decode steps to time (default: the workload's 1024)")
    ap.add_argument("--skip-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--skip-forward", action="store_true")
    ap.add_argument("--skip-backward", action="store_true")
    ap.add_argument("--bwd-steps", type=int, default=10)
    ap.add_argument("--skip-split", action="store_true",
                    help="skip timing the two-kernel hand-off variant of the forward")
    ap.add_argument("--skip-others", action="store_true",
                    help="skip timing the fp32 and packed-varlen forward configs")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB (a reference "
                         "kernel of known traffic for hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(heads and sequences would shard across GPUs with no exchange between them)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_22_amd as ck
    from gated_delta_rule_22_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ck.library()
    out = {"metric": METRIC, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}

    # ------------------------------------------------------------- forward
    w = wl.WORKLOADS["layer_1p3b_bf16"]
    fwd_bytes, fwd_flops, per_th = fwd_algorithmic(w)
    out["config"] = {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "dk": w.dk, "dv": w.dv,
                     "chunk": w.chunk, "tokens_per_step": w.B * w.T, "qkv": "bf16",
                     "gates_state_out": "fp32"}
    x = wl.forward_inputs(w)
    fwd_result = None
    if not args.skip_forward:
        print(f"[bench] forward {w.name}: uploading", file=sys.stderr, flush=True)
        bf = lambda a: torch.from_numpy(a).to(dev).to(torch.bfloat16)
        f32 = lambda a: torch.from_numpy(a).to(dev)
        q, k, v, g, beta = bf(x["q"]), bf(x["k"]), bf(x["v"]), f32(x["g"]), f32(x["beta"])
        o = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.float32, device=dev)
        S_T = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, ck.forward_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv, w.B,
                                                           torch.bfloat16)),
                         dtype=torch.uint8, device=dev)
        run = lambda: ck.forward(q, k, v, g, beta, out=o, final_state=S_T, workspace=ws)
        # The clocks ramp up over the first ~30 ms of load, whatever --warmup is:
        # settle them with untimed launches first, then run the W warm-up steps.
        t_settle = time.perf_counter()
        while time.perf_counter() - t_settle < args.settle_s:
            for _ in range(10):
                run()
            torch.cuda.synchronize()
        out["settle_s"] = round(time.perf_counter() - t_settle, 3)
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        print(f"[bench] forward: timing {args.steps} steps", file=sys.stderr, flush=True)
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(args.steps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = e0.elapsed_time(e1) / args.steps
        out["ms_per_step"] = ms
        out["value"] = w.B * w.T / (ms * 1e-3)
        gbs = fwd_bytes / (ms * 1e-3) / 1e9
        tflops = fwd_flops / (ms * 1e-3) / 1e12
        traffic = profiled_traffic("fwd_bf16_layer_1p3b_bf16.md", "gated_delta_rule_22_amd/csrc/fwd_bf16.hip")
        out["roofline"] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": gbs / HBM_PEAK_GBS, "traffic": traffic,
                           "kernel": "ckda forward (one launch per step for uniform batches)",
                           "bytes_per_launch": fwd_bytes, "bytes_per_token_head": per_th}
        out["mfma"] = {"algorithmic_tflops": tflops, "peak_tflops": BF16_PEAK_TFLOPS,
                       "frac": tflops / BF16_PEAK_TFLOPS, "flops_per_step": fwd_flops}
        out["wall_s_timed"] = wall
        if not args.skip_cpu:
            # the timed forward's outputs, checked against the oracle in the CPU leg
            fwd_result = (o.cpu().numpy(), S_T.cpu().numpy())
        # KDA mode on the same shape and gate magnitudes: the comparison the pages
        # quote for CKDA's kernel throughput (CKDA over KDA).  The two are timed in
        # alternating blocks of launches (CKDA first in even blocks, KDA first in
        # odd ones), so that the clock's drift over the run weighs on both alike.
        ga = g.abs()
        run_kda = lambda: ck.kda_forward(q, k, v, ga, beta, out=o, final_state=S_T, workspace=ws)
        for _ in range(max(3, args.warmup // 4)):
            run_kda()
        torch.cuda.synchronize()
        # at least 16 launches per block: the launches queued right after each
        # block's synchronisation would otherwise weigh on the average
        n_blk = 6
        per_blk = max(16, args.steps // n_blk)
        t_ckda = t_kda = 0.0
        for blk in range(n_blk):
            order = ((run, True), (run_kda, False)) if blk % 2 == 0 else ((run_kda, False), (run, True))
            for fn, is_ckda in order:
                e0.record(stream)
                for _ in range(per_blk):
                    fn()
                e1.record(stream)
                torch.cuda.synchronize()
                if is_ckda:
                    t_ckda += e0.elapsed_time(e1)
                else:
                    t_kda += e0.elapsed_time(e1)
        ms_ckda_alt = t_ckda / (n_blk * per_blk)
        ms_kda = t_kda / (n_blk * per_blk)
        out["kda"] = {"ms_per_step": ms_kda, "tokens_per_s": w.B * w.T / (ms_kda * 1e-3),
                      "ckda_ms_per_step_alternating": ms_ckda_alt,
                      "ckda_over_kda_throughput": ms_kda / ms_ckda_alt,
                      "timing": f"{n_blk} alternating blocks of {per_blk} launches each",
                      "gates": "|alpha| of the same workload"}
        if not args.skip_split:
            # The two-kernel hand-off the fused kernel replaced (CKDA_OPT_SPLIT: a
            # preparation kernel writes every prepared block, a state kernel reads
            # them), the same arithmetic, timed in alternating blocks against the
            # fused kernel.  Its results are checked bit-identical to the fused ones.
            from gated_delta_rule_22_amd import _lib
            ws_bytes = ck.forward_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv, w.B, torch.bfloat16,
                                                  _lib.OPT_SPLIT)
            ws_split = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
            o_split = torch.empty_like(o)
            S_split = torch.empty_like(S_T)
            run_split = lambda: ck.forward(q, k, v, g, beta, out=o_split, final_state=S_split,
                                           workspace=ws_split, split=True)
            run()
            for _ in range(max(3, args.warmup // 4)):
                run_split()
            torch.cuda.synchronize()
            identical = bool(torch.equal(o, o_split) and torch.equal(S_T, S_split))
            t_fused = t_split = 0.0
            for blk in range(n_blk):
                order = ((run, True), (run_split, False)) if blk % 2 == 0 else ((run_split, False), (run, True))
                for fn, is_fused in order:
                    e0.record(stream)
                    for _ in range(per_blk):
                        fn()
                    e1.record(stream)
                    torch.cuda.synchronize()
                    if is_fused:
                        t_fused += e0.elapsed_time(e1)
                    else:
                        t_split += e0.elapsed_time(e1)
            ms_fused = t_fused / (n_blk * per_blk)
            ms_split = t_split / (n_blk * per_blk)
            out["hand_off"] = {"ms_per_step": ms_split, "fused_ms_per_step_alternating": ms_fused,
                               "over_fused": ms_split / ms_fused,
                               "bit_identical_to_fused": identical,
                               "prepared_bytes": ws_bytes,
                               "timing": f"{n_blk} alternating blocks of {per_blk} launches each",
                               "what": "preparation kernel writing every prepared 16-token "
                                       "block, then the state-pass kernel reading them"}
            del ws_split, o_split, S_split
        del q, k, v, g, ga, beta, o, S_T, ws
        torch.cuda.empty_cache()

    # ------------------------------------------------------------- decode
    if not args.skip_decode:
        wd = wl.WORKLOADS["decode_256x16"]
        steps = args.decode_steps or wd.steps
        print(f"[bench] decode {wd.name}: drawing {steps} steps", file=sys.stderr, flush=True)
        xs = wl.decode_steps(wd, range(steps), workers=min(16, os.cpu_count() or 1))
        bf = lambda a: torch.from_numpy(a).to(dev).to(torch.bfloat16)
        f32 = lambda a: torch.from_numpy(a).to(dev)
        dq = torch.stack([bf(s["q"]) for s in xs])
        dk_ = torch.stack([bf(s["k"]) for s in xs])
        dv_ = torch.stack([bf(s["v"]) for s in xs])
        dg = torch.stack([f32(s["g"]) for s in xs])
        db = torch.stack([f32(s["beta"]) for s in xs])
        del xs
        S = torch.from_numpy(wl.decode_state(wd)).to(dev)
        do = torch.empty((steps, wd.B, wd.H, wd.dv), dtype=torch.float32, device=dev)
        step = lambda i: ck.decode_step(dq[i], dk_[i], dv_[i], dg[i], db[i], S, out=do[i])
        for i in range(min(3, steps)):          # warm-up (advances the state)
            step(i)
        torch.cuda.synchronize()
        print(f"[bench] decode: timing {steps} steps", file=sys.stderr, flush=True)
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_d = e0.elapsed_time(e1) / steps
        dbytes, per_head = decode_algorithmic(wd)
        dgbs = dbytes / (ms_d * 1e-3) / 1e9
        dtraffic = profiled_traffic("decode_256x16.md", "gated_delta_rule_22_amd/csrc/decode.hip")
        # what a plain device copy of the same state bytes reaches on this GPU (one
        # read and one write per byte, like the decode step): the practical ceiling
        S2 = torch.empty_like(S)
        S2.copy_(S)
        torch.cuda.synchronize()
        ncopy = 50
        e0.record(stream)
        for _ in range(ncopy):
            S2.copy_(S)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_c = e0.elapsed_time(e1) / ncopy
        cgbs = 2 * S.numel() * 4 / (ms_c * 1e-3) / 1e9
        del S2
        # the same step over four times the states (four copies of each sequence's
        # inputs and state, 1.07 GB of state, over four times the 256 MB Infinity
        # Cache): a rate that holds here comes from HBM, not from the cache
        rep = 4
        nbig = min(64, steps)
        tile = lambda a: a[:nbig].repeat(1, rep, *([1] * (a.dim() - 2))).contiguous()
        bq, bk, bv, bg, bb = tile(dq), tile(dk_), tile(dv_), tile(dg), tile(db)
        Sb = S.repeat(rep, *([1] * (S.dim() - 1))).contiguous()
        bo = torch.empty((nbig, rep * wd.B, wd.H, wd.dv), dtype=torch.float32, device=dev)
        bstep = lambda i: ck.decode_step(bq[i], bk[i], bv[i], bg[i], bb[i], Sb, out=bo[i])
        for i in range(min(3, nbig)):
            bstep(i)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(nbig):
            bstep(i)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_b = e0.elapsed_time(e1) / nbig
        bgbs = rep * dbytes / (ms_b * 1e-3) / 1e9
        Sb2 = torch.empty_like(Sb)
        Sb2.copy_(Sb)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(20):
            Sb2.copy_(Sb)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_bc = e0.elapsed_time(e1) / 20
        bcgbs = 2 * Sb.numel() * 4 / (ms_bc * 1e-3) / 1e9
        large = {"states": rep * wd.B * wd.H, "state_bytes": Sb.numel() * 4, "steps": nbig,
                 "us_per_step": ms_b * 1e3, "hbm_gbs": bgbs, "hbm_frac": bgbs / HBM_PEAK_GBS,
                 "copy_gbs": bcgbs, "what": f"{rep} copies of each state and its inputs"}
        del bq, bk, bv, bg, bb, Sb, Sb2, bo
        out["decode"] = {"workload": wd.name, "steps": steps, "us_per_step": ms_d * 1e3,
                         "traffic": dtraffic,
                         "steps_per_s": 1e3 / ms_d, "hbm_gbs": dgbs, "hbm_frac": dgbs / HBM_PEAK_GBS,
                         "bytes_per_step": dbytes, "bytes_per_state": per_head,
                         "copy_reference": {"gbs": cgbs, "us": ms_c * 1e3,
                                            "what": "torch copy_ of the fp32 state buffer "
                                                    f"({S.numel() * 4} B read + written)"},
                         "frac_of_copy": dgbs / cgbs, "large_state": large}
        if args.skip_forward:
            out["roofline"] = {"bound": "hbm", "achieved": dgbs, "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": dgbs / HBM_PEAK_GBS, "traffic": dtraffic,
                               "kernel": "decode step"}
        del dq, dk_, dv_, dg, db, S, do
        torch.cuda.empty_cache()

    # ------------------------------------------------------------- backward
    if not args.skip_backward:
        print(f"[bench] backward {w.name}: uploading", file=sys.stderr, flush=True)
        bf = lambda a: torch.from_numpy(a).to(dev).to(torch.bfloat16)
        f32 = lambda a: torch.from_numpy(a).to(dev)
        q, k, v, g, beta = bf(x["q"]), bf(x["k"]), bf(x["v"]), f32(x["g"]), f32(x["beta"])
        gen = torch.Generator(device=dev)
        gen.manual_seed(0)
        do = torch.randn((w.B, w.T, w.H, w.dv), generator=gen, device=dev)
        dST = torch.randn((w.B, w.H, w.dk, w.dv), generator=gen, device=dev)
        ws = torch.empty(ck.backward_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv, w.B,
                                                     torch.bfloat16), dtype=torch.uint8,
                         device=dev)
        run_b = lambda: ck.backward(q, k, v, g, beta, do, dS_T=dST, workspace=ws)
        for _ in range(3):
            run_b()
        torch.cuda.synchronize()
        print(f"[bench] backward: timing {args.bwd_steps} steps", file=sys.stderr, flush=True)
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # KDA mode of the backward on |alpha|: with the KDA forward, the pages'
        # forward-plus-backward throughput comparison.  CKDA and KDA are timed in
        # the block order CKDA, KDA, KDA, CKDA, so a steady clock drift cancels.
        ga = g.abs()
        run_bk = lambda: ck.backward(q, k, v, ga, beta, do, dS_T=dST, workspace=ws, kda=True)
        run_bk()
        torch.cuda.synchronize()
        per_blk = max(1, args.bwd_steps // 2)
        t_b = t_bk = 0.0
        for fn, is_ckda in ((run_b, True), (run_bk, False), (run_bk, False), (run_b, True)):
            e0.record(stream)
            for _ in range(per_blk):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            if is_ckda:
                t_b += e0.elapsed_time(e1)
            else:
                t_bk += e0.elapsed_time(e1)
        ms_b = t_b / (2 * per_blk)
        ms_bk = t_bk / (2 * per_blk)
        bbytes, bflops, bper_th = bwd_algorithmic(w)
        out["backward"] = {
            "ms_per_step": ms_b, "tokens_per_s": w.B * w.T / (ms_b * 1e-3),
            "fwd_plus_bwd_tokens_per_s": (w.B * w.T / ((ms_b + out["ms_per_step"]) * 1e-3)
                                          if "ms_per_step" in out else None),
            "steps": 2 * per_blk, "arithmetic": "f64",
            "kda_ms_per_step": ms_bk,
            "fwd_bwd_ckda_over_kda_throughput": (
                (out["kda"]["ms_per_step"] + ms_bk)
                / (out["kda"]["ckda_ms_per_step_alternating"] + ms_b)
                if "kda" in out else None),
            "f64_tflops": bflops / (ms_b * 1e-3) / 1e12, "f64_peak_tflops": F64_PEAK_TFLOPS,
            "f64_frac": bflops / (ms_b * 1e-3) / 1e12 / F64_PEAK_TFLOPS,
            "hbm_gbs_compulsory": bbytes / (ms_b * 1e-3) / 1e9,
            "flops_per_step": bflops, "compulsory_bytes_per_step": bbytes,
            "upstream": "do ~ N(0,1), dS_T ~ N(0,1)"}
        del q, k, v, g, ga, beta, do, dST, ws
        torch.cuda.empty_cache()

    # ------------------------------------------------------------- other configs (time only)
    if not args.skip_forward and not args.skip_others:
        others = {}
        for name in ("tiny_f32", "rotation_f32", "varlen_64k_bf16", "layer_1p3b_fastdecay_bf16",
                     "layer_1p3b_rapiddecay_bf16"):
            wo = wl.WORKLOADS[name]
            xo = wl.forward_inputs(wo)
            dt = torch.bfloat16 if wo.dtype == "bf16" else torch.float32
            t = lambda a, d=torch.float32: None if a is None else torch.from_numpy(a).to(dev).to(d)
            qo, ko, vo = t(xo["q"], dt), t(xo["k"], dt), t(xo["v"], dt)
            go, bo, so = t(xo["g"]), t(xo["beta"]), t(xo.get("S0"))
            cu = xo.get("cu_seqlens")
            cu = None if cu is None else torch.from_numpy(np.asarray(cu, np.int32)).to(dev)
            run_o = lambda: ck.forward(qo, ko, vo, go, bo, S0=so, cu_seqlens=cu)
            for _ in range(20):
                run_o()
            torch.cuda.synchronize()
            n_o = 30
            e0.record(stream)
            for _ in range(n_o):
                run_o()
            e1.record(stream)
            torch.cuda.synchronize()
            ms_o = e0.elapsed_time(e1) / n_o
            toks = int(xo["q"].shape[0] * xo["q"].shape[1])
            others[name] = {"ms_per_forward": ms_o, "tokens_per_s": toks / (ms_o * 1e-3)}
            if name.startswith("layer_1p3b_") and "ms_per_step" in out:
                # strongly forgetting channels against the headline layer
                others[name]["time_over_layer"] = ms_o / out["ms_per_step"]
            del qo, ko, vo, go, bo, so, cu
        out["other_configs"] = others
        torch.cuda.empty_cache()

    if args.copy_mib:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_reference_bytes"] = {"read": n * 4, "write": n * 4}
        del src, dst

    # ------------------------------------------------------------- CPU oracle baseline
    if not args.skip_cpu:
        import oracle
        nth = min(16, oracle.default_threads())     # one GPU's share of the host
        print(f"[bench] cpu oracle on {nth} threads", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], nthreads=nth)
        dt = time.perf_counter() - t0
        if fwd_result is not None:
            # parity of the timed forward at the full size: max |gpu - oracle| / rms(oracle)
            err = lambda got, ref: float(np.max(np.abs(got.astype(np.float64) - ref)) /
                                         np.sqrt(np.mean(ref * ref)))
            out["parity"] = {"workload": w.name, "err_o": err(fwd_result[0], o_ref),
                             "err_S_T": err(fwd_result[1], S_ref), "tol": 2e-3,
                             "reference": "the fp64 oracle on the same inputs"}
        del o_ref, S_ref
        out["cpu_baseline"] = {"value": w.B * w.T / dt, "unit": "tokens/s", "cores": nth,
                               "kind": "oracle", "cpu_model": _cpu_model(),
                               "host_threads_visible": oracle.default_threads(),
                               "sample": f"the whole {w.name} forward (B={w.B}, T={w.T}, H={w.H}), "
                                         f"fp64 token-by-token, {dt:.1f} s"}
        if "backward" in out:
            # the oracle's backward on one of the batch rows (all heads), with the
            # same kind of upstream gradients
            rng = np.random.default_rng(0)
            sl = slice(0, 1)
            do1 = rng.normal(size=(1, w.T, w.H, w.dv))
            dST1 = rng.normal(size=(1, w.H, w.dk, w.dv))
            t0 = time.perf_counter()
            oracle.backward(x["q"][sl], x["k"][sl], x["v"][sl], x["g"][sl], x["beta"][sl], do1,
                            dS_T=dST1, nthreads=nth)
            dtb = time.perf_counter() - t0
            out["backward"]["cpu_baseline"] = {
                "value": w.T / dtb, "unit": "tokens/s", "cores": min(nth, w.H), "kind": "oracle",
                "sample": f"one of the {w.B} sequences of {w.name} (T={w.T}, H={w.H}), fp64 "
                          f"reverse mode with recomputed states, {dtb:.1f} s"}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
