"""GPU parity on seeded random configurations: combinations of batch, grouped heads,
length (tiny, ragged, several tiles), head size, mask, tau, input scale and storage
type that the hand-picked cases do not cover one by one.  A second, wider draw of 150
runs every BoB entry point (the fp32 row-sum option and the static-scratch form too) and
the forward's and the first backward's split forms.

Every configuration runs the forward, the BoB (``fbob_bob``, and ``fbob_bob_ws`` with
the workspace the planner asks for) and the first backward through the C ABI and
compares every output element with the fp64 oracle at the usual bars (2e-2 of max|ref|
for bf16 inputs, 1e-3 for fp32).  The configurations come from a fixed seed, so the set
is the same on every run; each prints its parameters before it touches the GPU.
"""

import numpy as np
import pytest

import oracle
import workloads
from tests import _gpu_util as U

pytestmark = pytest.mark.gpu

N_CONFIGS = 24


def random_configs(n=N_CONFIGS, seed=20261203):
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for k in range(n):
        d = int(rng.choice([64, 128]))
        dtype = "f32" if rng.random() < 0.2 else "bf16"
        hkv = int(rng.choice([1, 2]))
        group = int(rng.choice([1, 2, 3]))
        B = int(rng.choice([1, 2]))
        # tiny, ragged and multi-tile lengths; longer ones only for bf16 (the oracle's
        # cost grows as N^2 per head).  Not N = 1: there dQ~, dK~ and dV~ are exactly zero
        # (P = 1), the relative metric has no scale, and the residual the bf16-rounded
        # alpha leaves (~2^-9 |F| |dO|) is checked by the dedicated N = 1 cases.
        lengths = [2, 17, 64, 100, 129, 257, 300] + ([520, 777] if dtype == "bf16" else [])
        N = int(rng.choice(lengths))
        causal = bool(rng.random() < 0.5)
        tau = float(rng.choice([1.0 / np.sqrt(d), 0.1, 0.3]))
        # score std up to ~14 (the near-one-hot extremes have cases of their own)
        scale_qk = float(rng.choice([1.0, 2.0]))
        scale_u = float(rng.choice([1.0, 0.1]))
        name = (f"rnd{k:02d}_b{B}_hq{hkv * group}_hkv{hkv}_n{N}_d{d}_{dtype}"
                f"{'_causal' if causal else ''}_tau{tau:.3f}_qk{scale_qk:g}_u{scale_u:g}")
        out.append(workloads.Workload(name, B=B, H=hkv * group, N=N, d=d, dtype=dtype,
                                      seed=5000 + k, causal=causal, scale_qk=scale_qk,
                                      scale_u=scale_u, extra={"Hkv": hkv, "tau": tau}))
    return out


CONFIGS = random_configs()


def wide_configs(n=150, seed=777):
    """A second, wider draw: three K/V heads, groups of four, B up to 3, lengths around
    every tile boundary up to 1300, tau from 0.05 to 0.3 and Q, K scaled up to x4 (score
    std up to ~38 at tau 0.3: rows effectively one-hot), U scaled down or up."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for k in range(n):
        d = int(rng.choice([64, 128]))
        dtype = "f32" if rng.random() < 0.15 else "bf16"
        hkv = int(rng.choice([1, 2, 3]))
        group = int(rng.choice([1, 2, 4]))
        B = int(rng.choice([1, 2, 3]))
        lengths = [2, 3, 15, 16, 31, 33, 63, 65, 127, 128, 191, 255, 256, 257, 383, 511, 513]
        if dtype == "bf16":
            lengths += [640, 1000, 1023, 1025, 1300]
        N = int(rng.choice(lengths))
        causal = bool(rng.random() < 0.5)
        tau = float(rng.choice([1.0 / np.sqrt(d), 0.125, 0.0625, 0.1, 0.3, 0.05]))
        scale_qk = float(rng.choice([0.5, 1.0, 2.0, 4.0]))
        scale_u = float(rng.choice([1.0, 0.1, 3.0]))
        name = (f"sw{k:03d}_b{B}_hq{hkv * group}_hkv{hkv}_n{N}_d{d}_{dtype}"
                f"{'_c' if causal else ''}_t{tau:.3f}_qk{scale_qk:g}_u{scale_u:g}")
        out.append(workloads.Workload(name, B=B, H=hkv * group, N=N, d=d, dtype=dtype,
                                      seed=9000 + k, causal=causal, scale_qk=scale_qk,
                                      scale_u=scale_u, extra={"Hkv": hkv, "tau": tau}))
    return out


WIDE = wide_configs()


@pytest.mark.parametrize("w", CONFIGS, ids=[w.name for w in CONFIGS])
def test_random_configuration_matches_oracle(w):
    import torch
    import exact_softmax_attention_fbob_amd as fb
    U.say(f"[random] {w.name}")
    inp = U.make_inputs(w)
    dev = U.to_device(inp, w.dtype)
    a7 = tuple(dev[k] for k in workloads.TENSORS)
    O, L, D = fb.forward(*a7[:4], w.tau, w.causal)
    out = fb.bob(*a7, O, L, D, w.tau, w.causal)
    ws = fb.bob_ws(*a7, O, L, D, w.tau, w.causal)
    g = fb.backward(*a7[:4], O, L, w.tau, w.causal)
    torch.cuda.synchronize()

    def host(x):
        return x.cpu().numpy().astype(np.float64)

    got = {k: host(v) for k, v in out.items()}
    got.update(O=host(O), L=host(L), D=host(D))
    ref = U.oracle_full(inp, w)
    errs = U.compare_full(got, ref, w)
    got_ws = {k: host(v) for k, v in ws.items()}
    errs.update({k + "_ws": v for k, v in U.compare_full(got_ws, ref, w, keys=U.ALL_KEYS).items()})

    # first backward: dQ per query head, dK and dV summed over a group's query heads
    q, k = U.split_inputs(inp, w)
    grads = {"dQ": [], "dK": {}, "dV": {}}
    for (b, h) in U.head_list(w):
        a = (q("Q", b, h), k("K", b, h), k("V", b, h), q("dO", b, h))
        dQ, dK, dV = oracle.first_backward(*a, w.tau, w.causal)
        grads["dQ"].append((b, h, dQ))
        key = (b, U.kv_index(w, h))
        grads["dK"][key] = grads["dK"].get(key, 0) + dK
        grads["dV"][key] = grads["dV"].get(key, 0) + dV
    gd = {kk: host(v) for kk, v in g.items()}
    errs["dQ"] = U.rel(np.stack([gd["dQ"][b, h] for b, h, _ in grads["dQ"]]),
                       np.stack([x for _, _, x in grads["dQ"]]))
    for kk in ("dK", "dV"):
        keys = sorted(grads[kk])
        errs[kk] = U.rel(np.stack([gd[kk][b, j] for b, j in keys]),
                         np.stack([grads[kk][key] for key in keys]))
    U.say(f"[random] {w.name}: " + " ".join(f"{kk}={v:.1e}" for kk, v in errs.items()))
    bad = {kk: v for kk, v in errs.items() if not (v <= U.TOL[w.dtype])}
    assert not bad, bad


@pytest.mark.parametrize("w", WIDE, ids=[w.name for w in WIDE])
def test_wide_random_configuration_every_bob_entry_point(w):
    """fbob_bob, fbob_bob_ws, fbob_bob_ex with fp32 row sums and fbob_bob_noalloc (where
    the split fits the static scratch), the forward through fbob_forward_ws and the first
    backward through fbob_backward_ws, against the oracle, every output element."""
    import torch
    import exact_softmax_attention_fbob_amd as fb
    U.say(f"[wide] {w.name}")
    inp = U.make_inputs(w)
    dev = U.to_device(inp, w.dtype)
    a7 = tuple(dev[k] for k in workloads.TENSORS)
    O, L, D = fb.forward(*a7[:4], w.tau, w.causal)
    runs = {"bob": fb.bob(*a7, O, L, D, w.tau, w.causal),
            "ws": fb.bob_ws(*a7, O, L, D, w.tau, w.causal),
            "ex": fb.bob_ex(*a7, O, L, D, w.tau, w.causal, flags=fb.FLAG_FP32_ROW_SUMS)}
    if fb.bob_workspace_size(a7[0], a7[1], w.tau, w.causal) <= 128 << 20:
        runs["noalloc"] = fb.bob_noalloc(*a7, O, L, D, w.tau, w.causal)
    torch.cuda.synchronize()
    ref = U.oracle_full(inp, w)
    errs = {}
    for kind, out in runs.items():
        got = {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()}
        got.update(O=O.cpu().numpy().astype(np.float64), L=L.cpu().numpy().astype(np.float64),
                   D=D.cpu().numpy().astype(np.float64))
        keys = U.ALL_KEYS + (("O", "L", "D") if kind == "bob" else ())
        errs.update({f"{kind}.{k}": v for k, v in U.compare_full(got, ref, w, keys=keys).items()})
    # the forward through fbob_forward_ws (split where its planner splits)
    fO, fL, fD = fb.forward_ws(*a7[:4], w.tau, w.causal)
    fgot = {"O": fO.cpu().numpy().astype(np.float64), "L": fL.cpu().numpy().astype(np.float64),
            "D": fD.cpu().numpy().astype(np.float64)}
    errs.update({f"fwd_ws.{k}": v
                 for k, v in U.compare_full(fgot, ref, w, keys=("O", "L", "D")).items()})
    # the first backward through fbob_backward_ws (split where its planner splits)
    g = fb.backward_ws(*a7[:4], O, L, w.tau, w.causal)
    gd = {kk: v.cpu().numpy().astype(np.float64) for kk, v in g.items()}
    q, k = U.split_inputs(inp, w)
    gq, gk, gv = [], {}, {}
    for (b, h) in U.head_list(w):
        dQ, dK, dV = oracle.first_backward(q("Q", b, h), k("K", b, h), k("V", b, h),
                                           q("dO", b, h), w.tau, w.causal)
        gq.append((b, h, dQ))
        key = (b, U.kv_index(w, h))
        gk[key] = gk.get(key, 0) + dK
        gv[key] = gv.get(key, 0) + dV
    errs["grad_ws.dQ"] = U.rel(np.stack([gd["dQ"][b, h] for b, h, _ in gq]),
                               np.stack([x for _, _, x in gq]))
    keys = sorted(gk)
    errs["grad_ws.dK"] = U.rel(np.stack([gd["dK"][b, j] for b, j in keys]),
                               np.stack([gk[kk] for kk in keys]))
    errs["grad_ws.dV"] = U.rel(np.stack([gd["dV"][b, j] for b, j in keys]),
                               np.stack([gv[kk] for kk in keys]))
    top = max(errs, key=errs.get)
    U.say(f"[wide] {w.name}: worst {top}={errs[top]:.2e}")
    bad = {kk: v for kk, v in errs.items() if not (v <= U.TOL[w.dtype])}
    assert not bad, bad
