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

Prints ONE JSON line.  `value` is the BoB TFLOP/s the metric names (Pass 1 +
Pass 2, HIP-event time); the whole step's rate and ms/step (wall clock) are
reported alongside, with the dominant kernel's roofline (Pass 1 against the bf16
dense MFMA peak, also at the clock measured during the timed region) and the
fp64 CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # MI355X dense MFMA peaks
SPEC_SCLK_MHZ = 2400.0  # the engine clock those peaks are quoted at
METRIC = "BoB ms/call + TFLOP/s (% bf16 MFMA peak), H=12 d=64 at N=16K; max N on 1 GPU"
TRAFFIC_FILES = {"pass1_kernel": os.path.join(ROOT, "profiles", "pass1_hbm_traffic.json"),
                 "pass2_kernel": os.path.join(ROOT, "profiles", "pass2_hbm_traffic.json")}
KERNEL_SOURCES = {"pass1_kernel": ("fbob_device.hpp", "fbob_pass1.hip"),
                  "pass2_kernel": ("fbob_device.hpp", "fbob_pass2.hip")}


def _code_only(text: str) -> str:
    """C++ source without /* */ and // comments, blank lines or trailing spaces."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def kernel_source_digest(kernel: str = "pass1_kernel") -> str:
    """Digest of the kernel's sources with comments, blank lines and trailing spaces
    removed: a counter record stays valid across comment edits, and only across them."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "exact_softmax_attention_fbob_amd", "csrc", name)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str = "pass1_kernel"):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter runs, if
    they were taken on the kernel's current source and this workload; else None."""
    try:
        with open(TRAFFIC_FILES[kernel]) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if (rec.get("kernel_source_digest") != kernel_source_digest(kernel)
            or rec.get("workload") != workload):
        return None
    return rec.get("bytes_per_launch")


class ClockSampler:
    """Samples the GPU's graphics clock on a background thread every `period`
    seconds while a window of back-to-back kernel launches runs (the kernels are
    already queued, so the sampling does not perturb them).  Each sample records
    amdsmi's GPU-metrics readings: the current clock of every XCD
    (``current_gfxclks``) and the firmware's running average
    (``average_gfxclk_frequency``).  result() gives the median over the second half
    of the window (after the clock has settled under load) or None where the
    metrics cannot be read."""

    def __init__(self, device=0, period=0.01):
        import threading
        self.device, self.period, self.samples = device, period, []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self, handle):
        import amdsmi
        m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
        xcd = [float(x) for x in (m.get("current_gfxclks") or []) if isinstance(x, (int, float))]
        avg = m.get("average_gfxclk_frequency")
        return {"xcd_mean": sum(xcd) / len(xcd) if xcd else None,
                "average": float(avg) if isinstance(avg, (int, float)) else None}

    def _run(self):
        try:
            import torch
            handle = torch.cuda._get_amdsmi_handler(self.device)
            self._read(handle)
        except Exception:  # no amdsmi access on this host
            return
        while not self._stop.is_set():
            try:
                self.samples.append(self._read(handle))
            except Exception:
                return
            self._stop.wait(self.period)

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join(timeout=5)

    def result(self):
        half = self.samples[len(self.samples) // 2:]
        out = {"samples": len(self.samples)}
        for k in ("xcd_mean", "average"):
            v = sorted(x[k] for x in half if x[k])
            out[k] = v[len(v) // 2] if v else None
        return out


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
    flops = 38.0 * pair_count * w.d  # the BoB FLOP formula (the metric's) over the sampled pairs
    full = 38.0 * pairs(0, w.N) * w.d * w.B * w.H
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rows_done} rows in {heads_touched} of {w.B * w.H} heads, "
                      f"{w.N} rows per head ({flops:.3e} FLOP, {dt:.1f} s, fp64 numpy)",
            "extrapolated_full_bob_s": dt * full / flops}


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


def _sampled_row_errors(w, T, out, O, L, D, rows):
    """max|gpu - ref| / max|ref| per row output over the sampled rows, the fp64
    oracle (bob_rows) on host copies of the same inputs."""
    import numpy as np
    import oracle
    host = {k: T[k][0, 0].double().cpu().numpy() for k in ("Q", "K", "V", "dO", "UQ", "UK", "UV")}
    idx = __import__("torch").as_tensor(rows, device=O.device)
    gpu = {"dQt": out["dQt"][0, 0][idx], "ddOt": out["ddOt"][0, 0][idx],
           "alpha": out["alpha"][0, 0][idx], "E": out["E"][0, 0][idx],
           "O": O[0, 0][idx], "L": L[0, 0][idx], "D": D[0, 0][idx]}
    gpu = {k: v.double().cpu().numpy() for k, v in gpu.items()}
    ref = {k: [] for k in gpu}
    for c0 in range(0, len(rows), 4):  # 4 rows at a time bounds the host memory
        o = oracle.bob_rows(host["Q"], host["K"], host["V"], host["dO"], host["UQ"], host["UK"],
                            host["UV"], w.tau, rows[c0:c0 + 4], w.causal)
        for k in ref:
            ref[k].append(o[k])
    errs = {}
    for k in gpu:
        r = np.concatenate(ref[k], axis=0)
        errs[k] = float(np.max(np.abs(gpu[k] - r)) / np.max(np.abs(r)))
    return errs


def _full_tensor_checks(T, out, D):
    """Size-independent properties of the full GPU outputs (float64 on the device):
    column sums of dK~, dV~ against their magnitudes (and no zero column output)
    and E = dO . ddO~ - alpha D at every row."""
    import torch
    o = {k: v[0, 0].double() for k, v in out.items()}
    res = {}
    for k in ("dKt", "dVt"):
        m = o[k].abs().sum(0)
        res[f"colsum_{k}"] = float((o[k].sum(0).abs() / m.clamp_min(1e-300)).max()) \
            if bool((m > 0).all()) else float("inf")
    rhs = (T["dO"][0, 0].double() * o["ddOt"]).sum(1) - o["alpha"] * D[0, 0].double()
    res["E=dO.ddOt-alpha*D"] = float((o["E"] - rhs).abs().max() / rhs.abs().max())
    del o
    torch.cuda.empty_cache()
    return res


def _class_tiled_errors(n, d, p, seed, tau):
    """Forward + BoB on class-tiled inputs (every row a copy of one of p seeded class
    rows, each class used n / p times, random order: workloads.class_tiled); every
    element of every output against the fp64 oracle on the p class rows gathered by
    class, L shifted by ln(n / p) (the reduction is pinned on the CPU by
    test_class_tiled_inputs_reduce_to_the_small_problem)."""
    import numpy as np
    import torch
    import exact_softmax_attention_fbob_amd as fb
    import oracle
    import workloads
    small, sigma = workloads.class_tiled(1, 1, n, d, "bf16", p, seed)
    dev = torch.device("cuda:0")
    sig = torch.from_numpy(sigma).to(dev)
    full = {k: torch.from_numpy(v).to(dev).index_select(2, sig).to(torch.bfloat16).contiguous()
            for k, v in small.items()}
    O, L, D = fb.forward(full["Q"], full["K"], full["V"], full["dO"], tau)
    args = tuple(full[k] for k in workloads.TENSORS)
    out = fb.bob_pass1(*args, O, L, D, tau)
    torch.cuda.synchronize()
    print(f"[max-n] N={n}: class-tiled forward + Pass 1 done", file=sys.stderr, flush=True)
    out.update(fb.bob_pass2(*args, L, D, out["alpha"], out["E"], tau))
    out.update(O=O, L=L, D=D)
    torch.cuda.synchronize()
    del full, args
    a = [small[k][0, 0].astype(np.float64) for k in workloads.TENSORS]
    ref = oracle.bob(*a, tau)
    O_s, L_s, D_s = oracle.forward(*a[:4], tau)
    ref.update(O=O_s, L=L_s + math.log(n // p), D=D_s)
    errs = {}
    for k, g in out.items():
        rf = torch.from_numpy(ref[k]).to(dev).index_select(0, sig)
        errs[k] = float((g[0, 0].double() - rf).abs().max() / rf.abs().max())
        del rf
    del out, O, L, D
    torch.cuda.empty_cache()
    return errs


def max_n_sweep(args):
    """Sweep the sequence length of one long head (B=1 H=1 d=64 bf16, the
    long-context workload's shape) upward by powers of two while the next call
    is predicted (N^2 scaling) to stay under --max-seconds.  Each length draws
    seeded i.i.d. inputs on the device and runs the forward and one timed BoB call
    (its two passes issued one after the other with a progress line between them),
    then checks:
      * sampled rows (dQ~, ddO~, alpha, E, O, L, D) against the fp64 oracle's
        row-restricted evaluation (bob_rows) on the same inputs, bar 2e-2;
      * vanishing column sums of dK~, dV~ (bar 1e-2, no zero column output) and
        E = dO . ddO~ - alpha D at every row (bar 2e-2);
      * a second BoB at the same length on class-tiled inputs (1024 class rows,
        each used N / 1024 times): every element of every output, dK~ and dV~ at
        every column included, against the oracle on the class rows (bar 2e-2).
    The largest N that passes all of them is reported."""
    import numpy as np
    import torch
    import exact_softmax_attention_fbob_amd as fb
    import workloads
    dev = torch.device("cuda:0")
    d = 64
    results = []
    n = args.max_n_start
    free, total_mem = torch.cuda.mem_get_info()
    # bytes per position: 7 bf16 inputs + O, dQ~, dK~, dV~, ddO~ (fp32) + L, D, alpha, E
    per_pos = 7 * d * 2 + 5 * d * 4 + 4 * 4
    while True:
        w = workloads.small(f"long_head_n{n}", B=1, H=1, N=n, d=d, dtype="bf16", seed=1005 + n)
        T = workloads.make_inputs_device(w, dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        O, L, D = fb.forward(T["Q"], T["K"], T["V"], T["dO"], w.tau)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        print(f"[max-n] N={n}: forward {t1 - t0:.3f} s", file=sys.stderr, flush=True)
        qargs = tuple(T[k] for k in ("Q", "K", "V", "dO", "UQ", "UK", "UV"))
        # The two passes fbob_bob launches, issued one by one so that a line is printed
        # between them (a call at the largest lengths runs for minutes).
        out = fb.bob_pass1(*qargs, O, L, D, w.tau)
        torch.cuda.synchronize()
        tp = time.perf_counter()
        print(f"[max-n] N={n}: Pass 1 {tp - t1:.3f} s", file=sys.stderr, flush=True)
        out.update(fb.bob_pass2(*qargs, L, D, out["alpha"], out["E"], w.tau))
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        print(f"[max-n] N={n}: Pass 2 {t2 - tp:.3f} s", file=sys.stderr, flush=True)
        finite = all(bool(torch.isfinite(v).all()) for v in out.values())
        rng = np.random.default_rng(n)
        rows = np.sort(rng.choice(n, size=args.max_n_rows, replace=False))
        rows[-1] = n - 1
        tr = time.perf_counter()
        row_errs = _sampled_row_errors(w, T, out, O, L, D, rows)
        print(f"[max-n] N={n}: oracle rows {time.perf_counter() - tr:.1f} s", file=sys.stderr,
              flush=True)
        props = _full_tensor_checks(T, out, D)
        del T, O, L, D, out
        torch.cuda.empty_cache()
        tc = time.perf_counter()
        tiled = _class_tiled_errors(n, d, 1024, 7000 + n.bit_length(), w.tau)
        print(f"[max-n] N={n}: class-tiled BoB + full comparison {time.perf_counter() - tc:.1f} s",
              file=sys.stderr, flush=True)
        ok = (finite and all(v <= 2e-2 for v in row_errs.values())
              and all(v < (1e-2 if k.startswith("colsum") else 2e-2) for k, v in props.items())
              and all(v <= 2e-2 for v in tiled.values()))
        bob_s = t2 - t1
        rec = {"N": n, "forward_s": round(t1 - t0, 4), "bob_s": round(bob_s, 4),
               "bob_tflops": round(38.0 * n * n * d / bob_s / 1e12, 1),
               "oracle_rows": len(rows),
               "row_err": {k: float(f"{v:.2e}") for k, v in row_errs.items()},
               "properties": {k: float(f"{v:.2e}") for k, v in props.items()},
               "class_tiled_err": {k: float(f"{v:.2e}") for k, v in tiled.items()}, "ok": ok}
        results.append(rec)
        print(f"[max-n] {json.dumps(rec)}", file=sys.stderr, flush=True)
        if not ok or bob_s * 4 > args.max_seconds:
            break
        n *= 2
    verified = max((r["N"] for r in results if r["ok"]), default=0)
    line = {"metric": "max N on 1 GPU (exact BoB, B=1 H=1 d=64 bf16)", "value": verified,
            "unit": "positions", "higher_is_better": True, "n_gpus": 1,
            "sweep": results, "max_seconds_per_call": args.max_seconds,
            "memory_bound_N": int(total_mem // per_pos),
            "bytes_per_position": per_pos,
            "check": "i.i.d. inputs: sampled rows vs the fp64 oracle (bob_rows), column sums "
                     "and the E identity on the full tensors; class-tiled inputs: every "
                     "element of every output vs the oracle on the 1024 class rows",
            "data": "synthetic (seeded torch device generator, workloads.make_inputs_device)"}
    print(json.dumps(line), flush=True)


def fill_sweep(args):
    """How fast one tile sweep runs as a function of how many CUs are busy: the
    GPT-2-heads shape (B=1, N=4096, d=64, bf16) at H = 2 .. 24 heads, i.e. 32 H Pass 1
    row tiles and 16 H Pass 2 column tiles for 256 CUs (one work-group per CU).
    Each head count times Pass 1, Pass 2 and fbob_bob_ws where the split schedule
    applies, each as a HIP graph of back-to-back calls (medians of three replays), so
    that host launch overhead does not count.  One JSON line per head count.  (No clock
    column: the GPU metrics refresh too slowly for windows this short.)"""
    import json as _json
    import statistics
    import torch
    import exact_softmax_attention_fbob_amd as fb
    import workloads
    base = workloads.WORKLOADS["gpt2_heads_h12_n4096_d64_bf16"]

    def med(run):
        return statistics.median(run() for _ in range(3))

    for H in (2, 4, 6, 8, 12, 16, 24):
        w = base.with_(H=H, name=f"gpt2_shape_h{H}")
        print(f"[fill] H={H}", file=sys.stderr, flush=True)
        T = {k: torch.from_numpy(v).cuda().to(torch.bfloat16)
             for k, v in workloads.make_inputs(w).items()}
        args7 = tuple(T[k] for k in workloads.TENSORS)
        O, L, D = fb.forward(*args7[:4], w.tau)
        p1 = fb.bob_pass1(*args7, O, L, D, w.tau)
        reps = max(10, int(200 * 12 / H))
        t1 = med(graph_timed(lambda: fb.bob_pass1(*args7, O, L, D, w.tau), reps))
        t2 = med(graph_timed(lambda: fb.bob_pass2(*args7, L, D, p1["alpha"], p1["E"], w.tau),
                             reps))
        need = fb.bob_workspace_size(args7[0], args7[1], w.tau)
        tws = None
        if need:
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
            tws = med(graph_timed(lambda: fb.bob_ws(*args7, O, L, D, w.tau, workspace=ws), reps))
        print(_json.dumps({"H": H, "pass1_tiles": 32 * H, "pass1_us": round(t1, 1),
                           "pass2_tiles": 16 * H, "pass2_us": round(t2, 1),
                           "bob_ws_us": None if tws is None else round(tws, 1),
                           "workspace_bytes": need}), flush=True)
        del T, args7, O, L, D, p1
        torch.cuda.empty_cache()


def causal_ab(args):
    """Causal against non-causal at equal unmasked work, interleaved on one box: the
    pages' causal shape B=4 H=12 N=16384 d=64 (4 N (N + 1) / 2 unmasked pairs per head
    index) against the same shape without the mask at B=2 (2 N^2).  Six rounds, each
    timing Pass 1 and Pass 2 of both (HIP events, mean of 10 calls after 3); medians
    over the rounds.  One JSON line."""
    import json as _json
    import statistics
    import torch
    import exact_softmax_attention_fbob_amd as fb
    import workloads

    def prep(w):
        T = {k: torch.from_numpy(v).cuda().to(torch.bfloat16)
             for k, v in workloads.make_inputs(w).items()}
        a7 = tuple(T[k] for k in workloads.TENSORS)
        O, L, D = fb.forward(*a7[:4], w.tau, w.causal)
        p1 = fb.bob_pass1(*a7, O, L, D, w.tau, w.causal)
        return w, a7, O, L, D, p1

    def timed(fn, reps=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    causal = workloads.WORKLOADS["pages_causal_b4_h12_n16384_d64_bf16"]
    plain = causal.with_(name="noncausal_b2_h12_n16384_d64_bf16", B=2, causal=False)
    cases = {"causal_b4": prep(causal), "noncausal_b2": prep(plain)}
    res = {k: {"pass1": [], "pass2": []} for k in cases}
    for rnd in range(6):
        for k, (w, a7, O, L, D, p1) in cases.items():
            res[k]["pass1"].append(timed(lambda: fb.bob_pass1(*a7, O, L, D, w.tau, w.causal)))
            res[k]["pass2"].append(timed(
                lambda: fb.bob_pass2(*a7, L, D, p1["alpha"], p1["E"], w.tau, w.causal)))
        print(f"[causal-ab] round {rnd} done", file=sys.stderr, flush=True)
    med = {k: {p: statistics.median(v[p]) for p in v} for k, v in res.items()}
    n = causal.N
    flops = {"causal_b4": 38.0 * n * (n + 1) / 2 * causal.d * causal.B * causal.H,
             "noncausal_b2": 38.0 * n * n * plain.d * plain.B * plain.H}
    out = {"median_ms": {k: {p: round(v, 4) for p, v in m.items()} for k, m in med.items()},
           "bob_tflops": {k: round(flops[k] / ((m["pass1"] + m["pass2"]) * 1e-3) / 1e12, 1)
                          for k, m in med.items()},
           "causal_time_per_work_over_noncausal": {
               p: round(med["causal_b4"][p] / med["noncausal_b2"][p]
                        * flops["noncausal_b2"] / flops["causal_b4"], 4)
               for p in ("pass1", "pass2")}}
    out["bob_rate_ratio"] = round(out["bob_tflops"]["causal_b4"] / out["bob_tflops"]["noncausal_b2"], 4)
    print(_json.dumps(out), flush=True)


def graph_timed(fn, reps):
    """Mean time in us of one call of ``fn``, timed as a HIP graph that replays ``reps``
    back-to-back calls (one warm-up replay first), so that host-side launch overhead
    never counts, however short the call."""
    import torch
    fn()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    torch.cuda.synchronize()

    def run():
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3
    return run


def causal_split(args):
    """The split schedule on causal problems (d = 64 and 128, bf16): fbob_bob against fbob_bob_ws
    with the workspace the planner asks for, each timed as a HIP graph of back-to-back
    calls, interleaved over three rounds (median).  Small causal problems leave most CUs
    idle: one work-group per pair of tiles.  One JSON line per shape; the non-causal
    GPT-2-heads shape is included for comparison."""
    import json as _json
    import statistics
    import torch
    import exact_softmax_attention_fbob_amd as fb
    import workloads
    base = workloads.WORKLOADS["gpt2_heads_h12_n4096_d64_bf16"]
    shapes = ((1, 12, 4096, True, 64), (1, 12, 4096, False, 64), (1, 4, 4096, True, 64),
              (1, 12, 2048, True, 64), (1, 12, 1024, True, 64), (1, 12, 16384, True, 64),
              (2, 12, 8192, True, 64), (4, 12, 4096, True, 64), (8, 12, 1024, True, 64),
              (1, 12, 4096, True, 128), (1, 4, 4096, True, 128), (1, 2, 8192, True, 128))
    for (B, H, N, causal, d) in shapes:
        w = base.with_(B=B, H=H, N=N, d=d, causal=causal, name=f"b{B}_h{H}_n{N}_d{d}",
                       extra={"tau": 1.0 / d ** 0.5})
        print(f"[causal-split] B={B} H={H} N={N} d={d} causal={causal}", file=sys.stderr,
              flush=True)
        T = {k: torch.from_numpy(v).cuda().to(torch.bfloat16)
             for k, v in workloads.make_inputs(w).items()}
        a7 = tuple(T[k] for k in workloads.TENSORS)
        O, L, D = fb.forward(*a7[:4], w.tau, causal)
        need = fb.bob_workspace_size(a7[0], a7[1], w.tau, causal)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        reps = max(4, min(50, int(4e5 * 12 * 4096 * 64 / (B * H * N * N * d))))
        unsplit = graph_timed(lambda: fb.bob(*a7, O, L, D, w.tau, causal), reps)
        split = graph_timed(lambda: fb.bob_ws(*a7, O, L, D, w.tau, causal, workspace=ws), reps)
        tu, ts = [], []
        for _ in range(3):
            tu.append(unsplit())
            ts.append(split())
        u, sp = statistics.median(tu), statistics.median(ts)
        flops = 38.0 * (N * (N + 1) / 2 if causal else N * N) * w.d * B * H
        print(_json.dumps({"B": B, "H": H, "N": N, "d": w.d, "causal": causal,
                           "workspace_bytes": need, "graph_reps": reps,
                           "bob_us": round(u, 1), "bob_ws_us": round(sp, 1),
                           "speedup": round(u / sp, 3),
                           "bob_tflops": round(flops / u / 1e6, 1),
                           "bob_ws_tflops": round(flops / sp / 1e6, 1)}), flush=True)
        del T, a7, O, L, D, ws, unsplit, split
        torch.cuda.empty_cache()


def n_sweep(args):
    """BoB rate against sequence length at the headline's heads and head size (B=1, H=12,
    d=64, bf16, non-causal, inputs as the GPT-2-heads recipe): N = 1024 .. 65536.  Each
    length times fbob_bob and fbob_bob_ws (the workspace the planner asks for, or none)
    as HIP graphs of back-to-back calls, interleaved over three rounds (median), and reads
    the engine clock of the sustained load.  One JSON line per length."""
    import json as _json
    import statistics
    import torch
    import exact_softmax_attention_fbob_amd as fb
    import workloads
    base = workloads.WORKLOADS["gpt2_heads_h12_n4096_d64_bf16"]
    for N in (1024, 2048, 4096, 8192, 16384, 32768, 65536):
        w = base.with_(N=N, name=f"h12_n{N}_d64")
        print(f"[n-sweep] N={N}", file=sys.stderr, flush=True)
        T = {k: torch.from_numpy(v).cuda().to(torch.bfloat16)
             for k, v in workloads.make_inputs(w).items()}
        a7 = tuple(T[k] for k in workloads.TENSORS)
        O, L, D = fb.forward(*a7[:4], w.tau)
        need = fb.bob_workspace_size(a7[0], a7[1], w.tau)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        reps = max(2, min(50, int(50 * (4096 / N) ** 2)))
        unsplit = graph_timed(lambda: fb.bob(*a7, O, L, D, w.tau), reps)
        split = graph_timed(lambda: fb.bob_ws(*a7, O, L, D, w.tau, workspace=ws), reps)
        tu, ts = [], []
        for _ in range(3):
            tu.append(unsplit())
            ts.append(split())
        u, sp = statistics.median(tu), statistics.median(ts)
        with ClockSampler() as clk:
            t_end = time.perf_counter() + 1.0
            while time.perf_counter() < t_end:
                unsplit()
        mhz = clk.result().get("xcd_mean")
        flops = 38.0 * N * N * w.d * w.H
        best = min(u, sp)
        out = {"N": N, "B": 1, "H": 12, "d": 64, "workspace_bytes": need, "graph_reps": reps,
               "bob_us": round(u, 1), "bob_ws_us": round(sp, 1),
               "bob_tflops": round(flops / u / 1e6, 1),
               "best_pct_bf16_peak": round(100 * flops / best / 1e6 / PEAK_TFLOPS["bf16"], 2),
               "sclk_mhz_measured": mhz}
        if mhz:
            out["best_frac_at_measured_sclk"] = round(
                flops / best / 1e6 / (PEAK_TFLOPS["bf16"] * mhz / SPEC_SCLK_MHZ), 4)
        print(_json.dumps(out), flush=True)
        del T, a7, O, L, D, ws, unsplit, split
        torch.cuda.empty_cache()


def split_audit(args):
    """Check of the split planners: fbob_bob against fbob_bob_ws, fbob_backward against
    fbob_backward_ws and fbob_forward against fbob_forward_ws (the workspaces the planners
    ask for), on a grid of small and medium
    shapes (d = 64 and 128, with and
    without the mask, 1-20 heads, grouped heads, B up to 3, N 2048-32768), each timed
    as a HIP graph of back-to-back calls, interleaved over three rounds (median).  One
    JSON line per shape; "slower" marks a split that lost more than 2 %."""
    import json as _json
    import statistics
    import torch
    import exact_softmax_attention_fbob_amd as fb
    import workloads
    base = workloads.WORKLOADS["gpt2_heads_h12_n4096_d64_bf16"]
    grid = ((1, 2, 2, 4096), (1, 6, 6, 4096), (1, 12, 12, 4096), (1, 20, 20, 4096),
            (2, 12, 12, 4096), (1, 12, 4, 4096), (1, 12, 12, 8192), (1, 4, 4, 16384),
            (1, 1, 1, 32768), (1, 2, 2, 2048), (3, 4, 4, 2048))
    slower = 0
    for d in (64, 128):
        for causal in (False, True):
            for (B, H, Hkv, N) in grid:
                w = base.with_(B=B, H=H, N=N, d=d, causal=causal,
                               name=f"b{B}_h{H}_hkv{Hkv}_n{N}_d{d}",
                               extra={"tau": 1.0 / d ** 0.5, "Hkv": Hkv})
                print(f"[split-audit] {w.name} causal={causal}", file=sys.stderr, flush=True)
                T = workloads.make_inputs_device(w)
                for k in ("K", "V", "UK", "UV"):
                    T[k] = T[k][:, :Hkv].contiguous()
                a7 = tuple(T[k] for k in workloads.TENSORS)
                O, L, D = fb.forward(*a7[:4], w.tau, causal)
                need = fb.bob_workspace_size(a7[0], a7[1], w.tau, causal)
                out = {"B": B, "H": H, "Hkv": Hkv, "N": N, "d": d, "causal": causal,
                       "workspace_bytes": need}
                if need > 0:
                    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
                    pairs = N * (N + 1) / 2 if causal else N * N
                    reps = max(3, min(40, int(40 * 12 * 4096 ** 2 * 64 / (B * H * pairs * d))))
                    unsplit = graph_timed(lambda: fb.bob(*a7, O, L, D, w.tau, causal), reps)
                    split = graph_timed(lambda: fb.bob_ws(*a7, O, L, D, w.tau, causal,
                                                          workspace=ws), reps)
                    tu, ts = [], []
                    for _ in range(3):
                        tu.append(unsplit())
                        ts.append(split())
                    u, sp = statistics.median(tu), statistics.median(ts)
                    out.update(bob_us=round(u, 1), bob_ws_us=round(sp, 1),
                               speedup=round(u / sp, 3), slower=u / sp < 0.98)
                    slower += int(u / sp < 0.98)
                    del ws, unsplit, split
                # the first backward's planner (fbob_backward_ws) on the same shape
                gneed = fb.backward_workspace_size(a7[0], a7[1], w.tau, causal)
                out["grad_workspace_bytes"] = gneed
                if gneed > 0:
                    gws = torch.empty(gneed, dtype=torch.uint8, device="cuda")
                    pairs = N * (N + 1) / 2 if causal else N * N
                    reps = max(3, min(40, int(40 * 12 * 4096 ** 2 * 64 / (B * H * pairs * d))))
                    gu = graph_timed(lambda: fb.backward(*a7[:4], O, L, w.tau, causal), reps)
                    gs = graph_timed(lambda: fb.backward_ws(*a7[:4], O, L, w.tau, causal,
                                                            workspace=gws), reps)
                    tu, ts = [], []
                    for _ in range(3):
                        tu.append(gu())
                        ts.append(gs())
                    u, sp = statistics.median(tu), statistics.median(ts)
                    out.update(backward_us=round(u, 1), backward_ws_us=round(sp, 1),
                               grad_speedup=round(u / sp, 3), grad_slower=u / sp < 0.98)
                    slower += int(u / sp < 0.98)
                    del gws, gu, gs
                # the forward's planner (fbob_forward_ws) on the same shape
                fneed = fb.forward_workspace_size(a7[0], a7[1], w.tau, causal)
                out["fwd_workspace_bytes"] = fneed
                if fneed > 0:
                    fws = torch.empty(fneed, dtype=torch.uint8, device="cuda")
                    pairs = N * (N + 1) / 2 if causal else N * N
                    reps = max(3, min(100, int(100 * 12 * 4096 ** 2 * 64 / (B * H * pairs * d))))
                    fu = graph_timed(lambda: fb.forward(*a7[:4], w.tau, causal), reps)
                    fs = graph_timed(lambda: fb.forward_ws(*a7[:4], w.tau, causal,
                                                           workspace=fws), reps)
                    tu, ts = [], []
                    for _ in range(3):
                        tu.append(fu())
                        ts.append(fs())
                    u, sp = statistics.median(tu), statistics.median(ts)
                    out.update(forward_us=round(u, 1), forward_ws_us=round(sp, 1),
                               fwd_speedup=round(u / sp, 3), fwd_slower=u / sp < 0.98)
                    slower += int(u / sp < 0.98)
                    del fws, fu, fs
                print(_json.dumps(out), flush=True)
                del T, a7, O, L, D
                torch.cuda.empty_cache()
    print(_json.dumps({"split_audit_shapes": 2 * 2 * len(grid), "slower": slower}), flush=True)


def row_sums(args):
    """Cost of the fp32 row-sum option (fbob_bob_ex, FBOB_FLAG_FP32_ROW_SUMS) against the
    default row sums: both through fbob_bob_ex with the workspace the planner asks for,
    each timed as a HIP graph of back-to-back calls, interleaved over three rounds
    (median).  One JSON line per shape (bf16, d = 64)."""
    import json as _json
    import statistics
    import torch
    import exact_softmax_attention_fbob_amd as fb
    import workloads
    shapes = (("h12_n16384_d64_bf16_u01", False), ("gpt2_heads_h12_n4096_d64_bf16", False),
              ("gpt2_heads_h12_n4096_d64_bf16", True), ("pages_causal_b4_h12_n16384_d64_bf16", True))
    for wname, causal in shapes:
        w = workloads.WORKLOADS[wname].with_(causal=causal)
        print(f"[row-sums] {wname} causal={causal}", file=sys.stderr, flush=True)
        T = workloads.make_inputs_device(w)
        a7 = tuple(T[k] for k in workloads.TENSORS)
        O, L, D = fb.forward(*a7[:4], w.tau, causal)
        need = fb.bob_workspace_size(a7[0], a7[1], w.tau, causal)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        reps = max(3, min(40, int(40 * 12 * 4096 ** 2 / (w.B * w.H * w.N * w.N))))
        runs = {f: graph_timed(lambda f=f: fb.bob_ex(*a7, O, L, D, w.tau, causal, flags=f,
                                                     workspace=ws), reps)
                for f in (0, fb.FLAG_FP32_ROW_SUMS)}
        t = {f: [] for f in runs}
        for _ in range(3):
            for f, run in runs.items():
                t[f].append(run())
        d0, d1 = statistics.median(t[0]), statistics.median(t[fb.FLAG_FP32_ROW_SUMS])
        print(_json.dumps({"workload": wname, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                           "causal": causal, "workspace_bytes": need, "graph_reps": reps,
                           "default_us": round(d0, 1), "fp32_row_sums_us": round(d1, 1),
                           "cost": round(d1 / d0 - 1, 4)}), flush=True)
        del T, a7, O, L, D, ws, runs
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=150)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip timing the first-order backward and the autograd HVP step")
    ap.add_argument("--workspace", action="store_true",
                    help="time the BoB as one fbob_bob_ws call with a workspace (small "
                         "problems split their sweeps); per-pass times are then not reported")
    ap.add_argument("--max-n", action="store_true",
                    help="sweep N for one long head instead of the headline step")
    ap.add_argument("--fill-sweep", action="store_true",
                    help="time the passes at N=4096 d=64 for 2..24 heads (GPU fill level)")
    ap.add_argument("--causal-ab", action="store_true",
                    help="causal B=4 vs non-causal B=2 at H=12 N=16384 d=64, interleaved")
    ap.add_argument("--causal-split", action="store_true",
                    help="fbob_bob vs fbob_bob_ws on causal d=64 shapes (HIP-graph timing)")
    ap.add_argument("--n-sweep", action="store_true",
                    help="BoB rate against N at B=1 H=12 d=64 (HIP-graph timing)")
    ap.add_argument("--split-audit", action="store_true",
                    help="fbob_bob vs fbob_bob_ws on a grid of shapes (HIP graphs)")
    ap.add_argument("--row-sums", action="store_true",
                    help="cost of fbob_bob_ex's fp32 row sums against the default (HIP graphs)")
    ap.add_argument("--max-n-start", type=int, default=1 << 18)
    ap.add_argument("--max-n-rows", type=int, default=16,
                    help="rows per length checked against the fp64 oracle in the max-N sweep")
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
    if args.fill_sweep:
        if not torch.cuda.is_available():
            print("bench.py: no GPU visible", file=sys.stderr)
            sys.exit(3)
        fb.load_library()
        fill_sweep(args)
        return
    if args.causal_ab:
        if not torch.cuda.is_available():
            print("bench.py: no GPU visible", file=sys.stderr)
            sys.exit(3)
        fb.load_library()
        causal_ab(args)
        return
    if args.causal_split:
        if not torch.cuda.is_available():
            print("bench.py: no GPU visible", file=sys.stderr)
            sys.exit(3)
        fb.load_library()
        causal_split(args)
        return
    if args.n_sweep:
        if not torch.cuda.is_available():
            print("bench.py: no GPU visible", file=sys.stderr)
            sys.exit(3)
        fb.load_library()
        n_sweep(args)
        return
    if args.split_audit:
        if not torch.cuda.is_available():
            print("bench.py: no GPU visible", file=sys.stderr)
            sys.exit(3)
        fb.load_library()
        split_audit(args)
        return
    if args.row_sums:
        if not torch.cuda.is_available():
            print("bench.py: no GPU visible", file=sys.stderr)
            sys.exit(3)
        fb.load_library()
        row_sums(args)
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

    ws_bytes = fb.bob_workspace_size(T["Q"], T["K"], tau, causal) if args.workspace else 0
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        check(lib.fbob_forward(dt_code, B, H, Hkv, N, d, ctau, int(causal), *map(p, qargs[:4]),
                               p(O), p(L), p(D), sp))
        if ev is not None:
            ev[1].record(stream)
        if args.workspace:  # both passes (and any split reductions) in one call
            check(lib.fbob_bob_ws(dt_code, B, H, Hkv, N, d, ctau, int(causal), *map(p, qargs),
                                  p(O), p(L), p(D), p(out["dQt"]), p(out["dKt"]),
                                  p(out["dVt"]), p(out["ddOt"]), p(out["alpha"]), p(out["E"]),
                                  p(ws), ws.numel(), sp))
            if ev is not None:
                ev[2].record(stream)
                ev[3].record(stream)
            return
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
    # Engine clock under this load: a separate window of back-to-back steps (about
    # 1.5 s) with the clock sampled throughout; the timed steps above run unobserved.
    n_clk = max(20, int(1500.0 / max(wall * 1e3 / args.steps, 0.01)))
    print(f"[bench] clock window: {n_clk} steps", file=sys.stderr, flush=True)
    with ClockSampler(0) as clk:
        for _ in range(n_clk):
            step()
        torch.cuda.synchronize()
    clock = clk.result()
    sclk = clock["xcd_mean"] or clock["average"]
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
    if args.workspace:  # one call: the roofline is the whole BoB (passes + reductions)
        p1_tflops = bob_tflops
        p2_tflops = None
    else:
        p1_tflops = f_p1 / (p1_ms * 1e-3) / 1e12
        p2_tflops = f_p2 / (p2_ms * 1e-3) / 1e12
    # the dense peak scales with the clock: 2.5 PFLOP/s bf16 is quoted at 2.4 GHz
    peak_at_clk = peak * sclk / SPEC_SCLK_MHZ if sclk else None

    line = {
        "metric": METRIC,
        "value": round(bob_tflops, 2),
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
        "value_is": "BoB (Pass 1 + Pass 2) TFLOP/s: 38 N^2 d per head over the HIP-event "
                    "time of the two passes, mean over the timed steps"
                    + ("; one fbob_bob_ws call with a %d-byte workspace" % ws_bytes
                       if args.workspace else ""),
        "bob_ms_per_call": round(float(bob_ms), 4),
        "bob_tflops": round(bob_tflops, 2),
        "bob_pct_bf16_peak": round(100 * bob_tflops / PEAK_TFLOPS["bf16"], 2),
        "step_tflops": round(step_tflops, 2),
        "step_what": "forward + Pass 1 + Pass 2 (42 N^2 d per head) over the wall time per step",
        "kernels_ms": {"fwd_stats": round(float(fwd_ms), 4),
                       "bob_pass1": None if args.workspace else round(float(p1_ms), 4),
                       "bob_pass2": None if args.workspace else round(float(p2_ms), 4)},
        "median_ms": {k: round(v, 4) for k, v in med.items()},
        "flop_formula": "per (b,h): forward 4 N^2 d, pass1 22 N^2 d, pass2 16 N^2 d"
                        + ("; causal counts N(N+1)/2 of the N^2 pairs" if causal else ""),
        "peak_mem_mib": peak_mib,
        "roofline": {
            "kernel": "bob (fbob_bob_ws)" if args.workspace else "bob_pass1",
            "bound": "mfma",
            "achieved": round(p1_tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(p1_tflops / peak, 4),
            "traffic": None if args.workspace else measured_traffic(name, "pass1_kernel"),
            "sclk_mhz_measured": round(sclk, 1) if sclk else None,
            "peak_at_measured_sclk": round(peak_at_clk, 1) if sclk else None,
            "frac_at_measured_sclk": round(p1_tflops / peak_at_clk, 4) if sclk else None,
            "sclk_readings": clock,
            "sclk_source": "amdsmi GPU metrics (per-XCD current GFX clock, mean over XCDs; "
                           "median over the second half of a ~1.5 s window of back-to-back "
                           "steps); peak scaled from 2.5 PFLOP/s at 2400 MHz",
        },
        "pass2": None if args.workspace else {
            "achieved": round(p2_tflops, 2), "frac": round(p2_tflops / peak, 4),
            "frac_at_measured_sclk": round(p2_tflops / peak_at_clk, 4) if sclk else None,
            "traffic": measured_traffic(name, "pass2_kernel")},
        "library": "libfbob.so (one kernel variant per problem class; reads no environment)",
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
