"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path through
the C ABI binding, and compare per output tensor with the fp64 oracle.

Error metric (per output tensor, over all compared entries):
    max |gpu - ref| / max |ref|
bars: 1e-3 for float32 inputs, 2e-2 for bfloat16 inputs.
"""

from __future__ import annotations

import sys

import numpy as np

import oracle
import workloads

TOL = {"f32": 1e-3, "bf16": 2e-2}
ROW_KEYS = ("dQt", "ddOt", "alpha", "E")
ALL_KEYS = ("dQt", "dKt", "dVt", "ddOt", "alpha", "E")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp: dict, dtype: str, device="cuda"):
    import torch
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    return {k: torch.from_numpy(v).to(device).to(td).contiguous() for k, v in inp.items()}


def run_gpu(dev: dict, tau: float, causal: bool):
    import exact_softmax_attention_fbob_amd as fb
    import torch
    O, L, D = fb.forward(dev["Q"], dev["K"], dev["V"], dev["dO"], tau, causal)
    out = fb.bob(dev["Q"], dev["K"], dev["V"], dev["dO"], dev["UQ"], dev["UK"], dev["UV"],
                 O, L, D, tau, causal)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()}
    res.update(O=O.cpu().numpy().astype(np.float64), L=L.cpu().numpy().astype(np.float64),
               D=D.cpu().numpy().astype(np.float64))
    return res


def class_tiled_errors(B, H, N, d, dtype, p, seed, tau):
    """Run forward + BoB on class-tiled inputs (workloads.class_tiled: every row a
    copy of one of p class rows, each class used N / p times) and compare EVERY
    element of every output with the fp64 oracle on the p class rows, gathered by
    class (L shifted by ln(N / p)): the reduction pinned on the CPU by
    test_class_tiled_inputs_reduce_to_the_small_problem.  Comparison on the device
    in float64.  Returns {output: max|gpu - ref| / max|ref|}."""
    import math
    import torch
    import exact_softmax_attention_fbob_amd as fb
    small, sigma = workloads.class_tiled(B, H, N, d, dtype, p, seed)
    dev = torch.device("cuda")
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    sig = torch.from_numpy(sigma).to(dev)
    full = {k: torch.from_numpy(v).to(dev).index_select(2, sig).to(td).contiguous()
            for k, v in small.items()}
    O, L, D = fb.forward(full["Q"], full["K"], full["V"], full["dO"], tau)
    out = fb.bob(full["Q"], full["K"], full["V"], full["dO"], full["UQ"], full["UK"], full["UV"],
                 O, L, D, tau)
    out.update(O=O, L=L, D=D)
    torch.cuda.synchronize()
    del full
    ref = {k: np.zeros((B, H, p) + ((d,) if k in ("dQt", "dKt", "dVt", "ddOt", "O") else ()))
           for k in out}
    for b in range(B):
        for h in range(H):
            a = [small[k][b, h].astype(np.float64) for k in workloads.TENSORS]
            r = oracle.bob(*a, tau)
            O_s, L_s, D_s = oracle.forward(*a[:4], tau)
            r.update(O=O_s, L=L_s + math.log(N // p), D=D_s)
            for k in ref:
                ref[k][b, h] = r[k]
    errs = {}
    for k, g in out.items():
        rf = torch.from_numpy(ref[k]).to(dev).index_select(2, sig)
        errs[k] = float((g.double() - rf).abs().max() / rf.abs().max())
        del rf
    return errs


def rel(a, b):
    den = np.max(np.abs(b)) if b.size else 0.0
    if den == 0.0:
        return float(np.max(np.abs(a))) if a.size else 0.0
    return float(np.max(np.abs(a - b)) / den)


def head_list(w):
    return [(b, h) for b in range(w.B) for h in range(w.H)]


def kv_index(w, h):
    hkv = w.extra.get("Hkv", w.H)
    return h // (w.H // hkv)


def split_inputs(inp, w):
    """Per-head 2-D float64 views: query-side [b, h], key-side [b, h // group]."""
    def q(name, b, h):
        return inp[name][b, h].astype(np.float64)

    def k(name, b, h):
        return inp[name][b, kv_index(w, h)].astype(np.float64)
    return q, k


def make_inputs(w):
    """Seeded inputs; for grouped-query workloads K, V, U_K, U_V have Hkv heads."""
    inp = workloads.make_inputs(w)
    hkv = w.extra.get("Hkv", w.H)
    if hkv != w.H:
        for name in ("K", "V", "UK", "UV"):
            inp[name] = np.ascontiguousarray(inp[name][:, :hkv])
    return inp


def oracle_full(inp, w, heads=None, blocked=False):
    """Full oracle outputs for the given (b, h) heads; column outputs of grouped
    heads are summed over the query heads of the group."""
    q, k = split_inputs(inp, w)
    tau = w.tau
    res = {}
    for (b, h) in heads or head_list(w):
        args = (q("Q", b, h), k("K", b, h), k("V", b, h), q("dO", b, h), q("UQ", b, h),
                k("UK", b, h), k("UV", b, h))
        fn = oracle.bob_blocked if blocked else oracle.bob
        out = fn(*args, tau, w.causal)
        O, L, D = oracle.forward(args[0], args[1], args[2], args[3], tau, w.causal)
        out.update(O=O, L=L, D=D)
        res[(b, h)] = out
    return res


def compare_full(gpu, ref, w, keys=ALL_KEYS + ("O", "L", "D")):
    """Per-tensor relative errors over the heads present in ``ref``."""
    errs = {}
    hkv = w.extra.get("Hkv", w.H)
    group = w.H // hkv
    for key in keys:
        a, bb = [], []
        if key in ("dKt", "dVt"):
            # grouped heads: sum the oracle over the query heads of each kv head
            kv = {}
            for (b, h), o in ref.items():
                kv.setdefault((b, h // group), []).append(o[key])
            for (b, g), parts in kv.items():
                if len(parts) != group:
                    continue
                a.append(gpu[key][b, g].ravel())
                bb.append(np.sum(parts, axis=0).ravel())
        else:
            for (b, h), o in ref.items():
                a.append(gpu[key][b, h].ravel())
                bb.append(o[key].ravel())
        errs[key] = rel(np.concatenate(a), np.concatenate(bb))
    return errs
