#!/usr/bin/env python3
"""Benchmark of the exact attention backward-over-backward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

One step = one pass of the whole hot path over one batch of synthetic inputs:
fbob_forward (O, L, D) then BoB Pass 1 and Pass 2 (the same kernels fbob_bob
launches, issued as fbob_bob_pass1 + fbob_bob_pass2 so that each kernel can be
bracketed by HIP events on the stream it runs on).  Inputs are resident in HBM
before the timed region starts.

FLOP formula (per (batch, query head), non-causal, fixed): forward 4 N^2 d,
Pass 1 22 N^2 d, Pass 2 16 N^2 d; BoB = 38 N^2 d; step = 42 N^2 d.  Causal
workloads count the N (N + 1) / 2 unmasked (i, j) pairs instead of N^2.

After the timed step, two related operations are timed on the same inputs
(reported under "extras", outside `value`): the first-order backward
(fbob_backward, algorithmic 10 N^2 d: the five products of the backward) and one
Hessian-vector step through the autograd layer (forward, first backward with
create_graph, then the BoB as the backward of the backward).

Prints ONE JSON line.  `value` is the step's TFLOP/s; the BoB-only ms/call and
TFLOP/s (the headline) are reported alongside, with the dominant kernel's
roofline (Pass 1 against the bf16 dense MFMA peak) and the fp64 CPU oracle
timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # MI355X dense MFMA peaks
METRIC = "BoB ms/call + TFLOP/s (% bf16 MFMA peak), H=12 d=64 at N=16K; max N on 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pass1_hbm_traffic.json")
KERNEL_SOURCES = ("fbob_device.hpp", "fbob_pass1.hip")


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_softmax_attention_fbob_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per Pass 1 launch from the committed rocprofv3 counter runs, if
    they were taken on the current Pass 1 source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_digest") != kernel_source_digest() or rec.get("workload") != workload:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, budget_s: float = 15.0, max_heads: int = 4):
    """Time the fp64 oracle on a bounded sample: blocks of 256 full-width rows
    (forward row state + all BoB row outputs + the block's share of dK~/dV~), head
    after head (at most ``max_heads``), until ``budget_s`` seconds have passed."""
    import numpy as np
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    H = w.H
    group = H // w.extra.get("Hkv", H)
    qs = list(range(min(max_heads, w.B * H)))          # flat query heads b * H + h
    kv = {f: (f // H) * H + (f % H) // group for f in qs}  # their key/value heads in the draw
    need = sorted(set(qs) | set(kv.values()))
    pos = {f: k for k, f in enumerate(need)}
    inp = {k: v.astype(np.float64) for k, v in workloads.make_inputs(w, heads=need).items()}

    def pairs(r0, r1):  # (i, j) pairs of rows r0 .. r1 - 1
        return (r1 * (r1 + 1) - r0 * (r0 + 1)) / 2.0 if w.causal else float(r1 - r0) * w.N

    block = 256
    rows_done, heads_touched, pair_count = 0, 0, 0.0
    t0 = time.perf_counter()
    for f in qs:
        if time.perf_counter() - t0 >= budget_s:
            break
        heads_touched += 1
        qh = {k: inp[k][pos[f]] for k in ("Q", "dO", "UQ")}
        kh = {k: inp[k][pos[kv[f]]] for k in ("K", "V", "UK", "UV")}
        r0 = 0
        while r0 < w.N and time.perf_counter() - t0 < budget_s:
            r1 = min(w.N, r0 + block)
            oracle.bob_row_block(qh["Q"], kh["K"], kh["V"], qh["dO"], qh["UQ"], kh["UK"],
                                 kh["UV"], w.tau, np.arange(r0, r1), w.causal)
            pair_count += pairs(r0, r1)
            rows_done += r1 - r0
            r0 = r1
    dt = time.perf_counter() - t0
    flops = 42.0 * pair_count * w.d  # the bench step's FLOP formula over the sampled pairs
    full = 42.0 * pairs(0, w.N) * w.d * w.B * w.H
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rows_done} rows in {heads_touched} of {w.B * w.H} heads, "
                      f"{w.N} rows per head ({flops:.3e} FLOP, {dt:.1f} s, fp64 numpy)",
            "extrapolated_full_step_s": dt * full / flops}


def time_extras(fb, lib, T, O, L, w, Hkv, n2d, bob_ms, fwd_ms, stream, steps):
    """Time fbob_backward (HIP events on `stream`) and one autograd Hessian-vector
    step on the bench inputs; O, L come from the timed forward."""
    import ctypes
    import torch
    from exact_softmax_attention_fbob_amd.autograd import attention
    B, H, N, d, tau, causal = w.B, w.H, w.N, w.d, w.tau, w.causal
    dev = O.device
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(dQ=torch.empty((B, H, N, d), **f32), dK=torch.empty((B, Hkv, N, d), **f32),
             dV=torch.empty((B, Hkv, N, d), **f32), D=torch.empty((B, H, N), **f32))
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    sp = ctypes.c_void_p(stream.cuda_stream)
    dt_code = 1 if w.dtype == "bf16" else 0

    def bwd():
        st = lib.fbob_backward(dt_code, B, H, Hkv, N, d, ctypes.c_float(tau), int(causal),
                               p(T["Q"]), p(T["K"]), p(T["V"]), p(T["dO"]), p(O), p(L),
                               p(g["dQ"]), p(g["dK"]), p(g["dV"]), p(g["D"]), sp)
        if st != 0:
            raise fb.FbobError(st)

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    bwd_ms = timed(bwd, steps)
    Q, K, V, dO = (T[k].clone().requires_grad_(True) for k in ("Q", "K", "V", "dO"))
    U = [T[k].float() for k in ("UQ", "UK", "UV")]

    def hvp():
        o = attention(Q, K, V, tau, causal)
        gr = torch.autograd.grad(o, (Q, K, V), grad_outputs=dO, create_graph=True)
        phi = sum((gi.float() * u).sum() for gi, u in zip(gr, U))
        torch.autograd.grad(phi, (Q, K, V, dO))

    hvp_ms = timed(hvp, max(2, steps // 4))
    peak = PEAK_TFLOPS[w.dtype]
    alg = 10 * n2d / (bwd_ms * 1e-3) / 1e12
    return {
        "first_backward": {
            "ms_per_call": round(bwd_ms, 4),
            "tflops_algorithmic": round(alg, 2),
            "pct_peak": round(100 * alg / peak, 2),
            "tflops_executed": round(14 * n2d / (bwd_ms * 1e-3) / 1e12, 2),
            "flop_formula": "algorithmic 10 N^2 d (S, dP, dV, dQ, dK); executed 14 N^2 d "
                            "(row pass S, dP, dQ; column pass S, dP, dK, dV)",
        },
        "autograd_hvp_step": {
            "ms": round(hvp_ms, 4),
            "kernels_only_ms": round(float(fwd_ms) + bwd_ms + float(bob_ms), 4),
            "what": "attention(Q,K,V) forward, grad with create_graph, grad of "
                    "<dQ,U_Q>+<dK,U_K>+<dV,U_V> w.r.t. (Q,K,V,dO)",
        },
    }


def max_n_sweep(args):
    """Sweep the sequence length of one long head (B=1 H=1 d=64 bf16, the
    long-context workload's shape) upward by powers of two while the next call
    is predicted (N^2 scaling) to stay under --max-seconds.  Each length runs the
    forward and one timed BoB call (its two passes issued one after the other with
    a progress line between them), then checks size-independent properties of
    the outputs: all finite, and the column sums of dK~ and dV~ vanish (Phi is
    invariant under K -> K + 1c^T and V -> V + 1c^T)."""
    import torch
    import exact_softmax_attention_fbob_amd as fb
    dev = torch.device("cuda:0")
    d = 64
    tau = 1.0 / math.sqrt(d)
    g = torch.Generator(device=dev)
    results = []
    n = args.max_n_start
    free, total_mem = torch.cuda.mem_get_info()
    # bytes per position: 7 bf16 inputs + O, dQ~, dK~, dV~, ddO~ (fp32) + L, D, alpha, E
    per_pos = 7 * d * 2 + 5 * d * 4 + 4 * 4
    while True:
        g.manual_seed(1005 + n)
        T = [torch.randn((1, 1, n, d), generator=g, device=dev).to(torch.bfloat16)
             for _ in range(7)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        O, L, D = fb.forward(T[0], T[1], T[2], T[3], tau)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        print(f"[max-n] N={n}: forward {t1 - t0:.3f} s", file=sys.stderr, flush=True)
        # The two passes fbob_bob launches, issued one by one so that a line is printed
        # between them (a call at the largest lengths runs for minutes).
        out = fb.bob_pass1(*T, O, L, D, tau)
        torch.cuda.synchronize()
        tp = time.perf_counter()
        print(f"[max-n] N={n}: Pass 1 {tp - t1:.3f} s", file=sys.stderr, flush=True)
        out.update(fb.bob_pass2(*T, L, D, out["alpha"], out["E"], tau))
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        ok = all(bool(torch.isfinite(v).all()) for v in out.values())
        ratios = {}
        for k in ("dKt", "dVt"):
            x = out[k][0, 0].double()
            ratios[k] = float((x.sum(0).abs() / x.abs().sum(0).clamp_min(1e-30)).max())
        ok = ok and all(r < 1e-2 for r in ratios.values())
        bob_s = t2 - t1
        rec = {"N": n, "forward_s": round(t1 - t0, 4), "bob_s": round(bob_s, 4),
               "bob_tflops": round(38.0 * n * n * d / bob_s / 1e12, 1),
               "colsum_ratio": {k: float(f"{v:.2e}") for k, v in ratios.items()}, "ok": ok}
        results.append(rec)
        print(f"[max-n] {json.dumps(rec)}", file=sys.stderr, flush=True)
        del T, O, L, D, out
        torch.cuda.empty_cache()
        if not ok or bob_s * 4 > args.max_seconds:
            break
        n *= 2
    verified = max((r["N"] for r in results if r["ok"]), default=0)
    line = {"metric": "max N on 1 GPU (exact BoB, B=1 H=1 d=64 bf16)", "value": verified,
            "unit": "positions", "higher_is_better": True, "n_gpus": 1,
            "sweep": results, "max_seconds_per_call": args.max_seconds,
            "memory_bound_N": int(total_mem // per_pos),
            "bytes_per_position": per_pos,
            "data": "synthetic (torch.randn on device, seeded)"}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=150)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip timing the first-order backward and the autograd HVP step")
    ap.add_argument("--max-n", action="store_true",
                    help="sweep N for one long head instead of the headline step")
    ap.add_argument("--max-n-start", type=int, default=1 << 18)
    ap.add_argument("--max-seconds", type=float, default=20.0,
                    help="stop before a BoB call predicted to exceed this many seconds")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on exactly one GPU (one head-parallel kernel set per "
              "device); --gpus N > 1 is not supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads
    import exact_softmax_attention_fbob_amd as fb

    if args.max_n:
        if not torch.cuda.is_available():
            print("bench.py: no GPU visible", file=sys.stderr)
            sys.exit(3)
        fb.load_library()
        max_n_sweep(args)
        return

    name = args.workload or workloads.HEADLINE
    w = workloads.WORKLOADS[name]
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(3)
    fb.load_library()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    torch.cuda.init()
    torch.cuda.reset_peak_memory_stats(dev)
    print(f"[bench] generating {name} inputs", file=sys.stderr, flush=True)
    inp = workloads.make_inputs(w)
    T = {k: torch.from_numpy(v).to(dev).to(td).contiguous() for k, v in inp.items()}
    del inp
    B, H, N, d, tau, causal = w.B, w.H, w.N, w.d, w.tau, w.causal
    Hkv = int(w.extra.get("Hkv", H))  # grouped-query workloads keep the first Hkv heads
    if Hkv != H:
        for k in ("K", "V", "UK", "UV"):
            T[k] = T[k][:, :Hkv].contiguous()
    f32 = dict(dtype=torch.float32, device=dev)
    O = torch.empty((B, H, N, d), **f32)
    L = torch.empty((B, H, N), **f32)
    D = torch.empty((B, H, N), **f32)
    qargs = (T["Q"], T["K"], T["V"], T["dO"], T["UQ"], T["UK"], T["UV"])

    lib = fb.load_library()
    import ctypes
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    out = {k: torch.empty((B, H if k in ("dQt", "ddOt") else Hkv, N, d), **f32)
           for k in ("dQt", "dKt", "dVt", "ddOt")}
    out.update(alpha=torch.empty((B, H, N), **f32), E=torch.empty((B, H, N), **f32))
    dt_code = 1 if w.dtype == "bf16" else 0
    ctau = ctypes.c_float(tau)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def check(st):
        if st != 0:
            raise fb.FbobError(st)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        check(lib.fbob_forward(dt_code, B, H, Hkv, N, d, ctau, int(causal), *map(p, qargs[:4]),
                               p(O), p(L), p(D), sp))
        if ev is not None:
            ev[1].record(stream)
        check(lib.fbob_bob_pass1(dt_code, B, H, Hkv, N, d, ctau, int(causal), *map(p, qargs),
                                 p(O), p(L), p(D), p(out["dQt"]), p(out["ddOt"]),
                                 p(out["alpha"]), p(out["E"]), sp))
        if ev is not None:
            ev[2].record(stream)
        check(lib.fbob_bob_pass2(dt_code, B, H, Hkv, N, d, ctau, int(causal), *map(p, qargs),
                                 p(L), p(D), p(out["alpha"]), p(out["E"]),
                                 p(out["dKt"]), p(out["dVt"]), sp))
        if ev is not None:
            ev[3].record(stream)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = np.mean([e[0].elapsed_time(e[1]) for e in evs])
    p1_ms = np.mean([e[1].elapsed_time(e[2]) for e in evs])
    p2_ms = np.mean([e[2].elapsed_time(e[3]) for e in evs])
    bob_ms = np.mean([e[1].elapsed_time(e[3]) for e in evs])
    med = {"fwd_stats": float(np.median([e[0].elapsed_time(e[1]) for e in evs])),
           "bob_pass1": float(np.median([e[1].elapsed_time(e[2]) for e in evs])),
           "bob_pass2": float(np.median([e[2].elapsed_time(e[3]) for e in evs])),
           "bob": float(np.median([e[1].elapsed_time(e[3]) for e in evs]))}
    ms_step = wall * 1e3 / args.steps

    peak_mib = round(torch.cuda.max_memory_allocated(dev) / 2**20, 1)  # the step's own peak
    heads = B * H
    # causal: only the (i, j) pairs with j <= i count, N (N + 1) / 2 of N^2
    pairs = N * (N + 1) / 2.0 if causal else float(N) * N
    n2d = pairs * d * heads
    f_fwd, f_p1, f_p2 = 4 * n2d, 22 * n2d, 16 * n2d
    peak = PEAK_TFLOPS[w.dtype]
    bob_tflops = (f_p1 + f_p2) / (bob_ms * 1e-3) / 1e12
    step_tflops = (f_fwd + f_p1 + f_p2) / (ms_step * 1e-3) / 1e12
    p1_tflops = f_p1 / (p1_ms * 1e-3) / 1e12

    line = {
        "metric": METRIC,
        "value": round(step_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": name, "B": B, "H": H, "Hkv": Hkv, "N": N, "d": d, "causal": causal,
                   "tau": tau, "inputs": "i.i.d. N(0,1), PCG64 seed %d" % w.seed,
                   "scale_u": w.scale_u, "scale_qk": w.scale_qk},
        "bob_ms_per_call": round(float(bob_ms), 4),
        "bob_tflops": round(bob_tflops, 2),
        "bob_pct_bf16_peak": round(100 * bob_tflops / PEAK_TFLOPS["bf16"], 2),
        "kernels_ms": {"fwd_stats": round(float(fwd_ms), 4), "bob_pass1": round(float(p1_ms), 4),
                       "bob_pass2": round(float(p2_ms), 4)},
        "median_ms": {k: round(v, 4) for k, v in med.items()},
        "flop_formula": "per (b,h): forward 4 N^2 d, pass1 22 N^2 d, pass2 16 N^2 d"
                        + ("; causal counts N(N+1)/2 of the N^2 pairs" if causal else ""),
        "peak_mem_mib": peak_mib,
        "roofline": {
            "kernel": "bob_pass1",
            "bound": "mfma",
            "achieved": round(p1_tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(p1_tflops / peak, 4),
            "traffic": measured_traffic(name),
        },
    }
    if not args.no_extras:
        print("[bench] extras: first-order backward, autograd HVP step", file=sys.stderr,
              flush=True)
        line["extras"] = time_extras(fb, lib, T, O, L, w, Hkv, n2d, bob_ms, fwd_ms, stream,
                                     args.steps)
    if not args.no_cpu:
        print("[bench] cpu baseline (fp64 oracle, bounded sample)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
