"""GPU test of the allocation-free BoB entry point (C ABI ``fbob_bob_noalloc``).

``fbob_bob_noalloc`` runs the split schedule of ``fbob_bob_ws`` with the library's
static per-device scratch array in place of a caller-owned workspace.  Its outputs
are checked against ``fbob_bob_ws`` with a workspace of its own on two calls in a
row, the second on a smaller problem (so the scratch still holds the first call's
partial sums), and on a problem that needs no split against ``fbob_bob``.  Both
sides run the same kernels in the same order, so the comparison is bitwise; the
parity tolerance is asserted as well.  Every case prints its name before it
touches the GPU.
"""

import numpy as np
import pytest

import workloads
from tests import _gpu_util as U

pytestmark = pytest.mark.gpu


def small(name, B, H, N, d, seed, causal=False):
    return workloads.Workload(name, B=B, H=H, N=N, d=d, dtype="bf16", seed=seed,
                              causal=causal)


CALLS = [
    workloads.WORKLOADS["gpt2_heads_h12_n4096_d64_bf16"],   # 32.25 MiB: 4 heads in 2 parts
    small("noalloc_n1000_h2_ragged", 1, 2, 1000, 64, 71),      # 15.75 MiB, 8 + 8 parts
    small("noalloc_causal_n600_h2", 1, 2, 600, 64, 73, causal=True),  # 4.7 MiB, Pass 1 in 4
]


def prepared(w):
    import exact_softmax_attention_fbob_amd as fb
    dev = U.to_device(U.make_inputs(w), w.dtype)
    args = tuple(dev[k] for k in ("Q", "K", "V", "dO", "UQ", "UK", "UV"))
    O, L, D = fb.forward(*args[:4], w.tau, w.causal)
    return args, O, L, D


def outputs_like(ref):
    import torch
    return {k: torch.full_like(v, float("nan")) for k, v in ref.items()}


def assert_same(got, ref, name):
    import torch
    for k in ref:
        assert got[k].shape == ref[k].shape, k
        err = float((got[k].double() - ref[k].double()).abs().max()
                    / max(float(ref[k].double().abs().max()), 1e-30))
        assert np.isfinite(err) and err <= U.TOL["bf16"], (name, k, err)
        assert torch.equal(got[k], ref[k]), (name, k, err)


def test_noalloc_matches_bob_ws_on_two_calls_in_a_row():
    """Calls in a row, each smaller than the one before (the scratch keeps the previous
    call's partial sums), the last one causal."""
    import torch
    import exact_softmax_attention_fbob_amd as fb
    sizes = []
    for w in CALLS:
        U.say(f"[noalloc] {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal}")
        args, O, L, D = prepared(w)
        need = fb.bob_workspace_size(args[0], args[1], w.tau, w.causal)
        assert 0 < need <= 128 << 20, need
        sizes.append(need)
        ws = torch.empty(need, dtype=torch.uint8, device=args[0].device)
        ref = fb.bob_ws(*args, O, L, D, w.tau, w.causal, workspace=ws)
        out = outputs_like(ref)
        got = fb.bob_noalloc(*args, O, L, D, w.tau, w.causal, out=out)
        torch.cuda.synchronize()
        assert got is out
        assert_same(got, ref, w.name)
    assert sizes[2] < sizes[1] < sizes[0]


def test_noalloc_without_split_equals_fbob_bob():
    import torch
    import exact_softmax_attention_fbob_amd as fb
    w = small("noalloc_causal_n300_h2_d128", 1, 2, 300, 128, 72, causal=True)
    U.say(f"[noalloc] {w.name} (no split)")
    args, O, L, D = prepared(w)
    assert fb.bob_workspace_size(args[0], args[1], w.tau, True) == 0
    ref = fb.bob(*args, O, L, D, w.tau, True)
    got = fb.bob_noalloc(*args, O, L, D, w.tau, True, out=outputs_like(ref))
    torch.cuda.synchronize()
    assert_same(got, ref, w.name)


def test_split_and_noalloc_under_hip_graph_capture():
    """The callers the allocation-free entry point is for: forward + fbob_bob_ws (with a
    preallocated workspace) + fbob_bob_noalloc (preallocated outputs) captured in one
    HIP graph on a problem that splits.  New inputs are copied into the captured
    buffers before each of three replays, with eager work in between; every replay
    must equal the eager fbob_bob_ws result on the same inputs bitwise."""
    import torch
    import exact_softmax_attention_fbob_amd as fb
    names = ("Q", "K", "V", "dO", "UQ", "UK", "UV")
    ws_list = [small(f"noalloc_graph_n1000_h2_s{s}", 1, 2, 1000, 64, 80 + s) for s in range(3)]
    U.say("[noalloc] hip graph capture of the split schedule, 3 replays")
    inputs = [U.to_device(U.make_inputs(w), w.dtype) for w in ws_list]
    static = {k: inputs[0][k].clone() for k in names}
    tau = ws_list[0].tau
    need = fb.bob_workspace_size(static["Q"], static["K"], tau)
    assert 0 < need <= 128 << 20
    work = torch.empty(need, dtype=torch.uint8, device=static["Q"].device)

    def eager(t):
        O, L, D = fb.forward(t["Q"], t["K"], t["V"], t["dO"], tau)
        return fb.bob_ws(*(t[k] for k in names), O, L, D, tau, workspace=work)

    first = eager(static)
    out_na = outputs_like(first)

    def run(t):
        O, L, D = fb.forward(t["Q"], t["K"], t["V"], t["dO"], tau)
        a = fb.bob_ws(*(t[k] for k in names), O, L, D, tau, workspace=work)
        b = fb.bob_noalloc(*(t[k] for k in names), O, L, D, tau, out=out_na)
        return a, b

    run(static)  # warm-up outside the capture (the scratch address is looked up here)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap_ws, cap_na = run(static)
    torch.cuda.synchronize()
    for rep, t in enumerate(inputs):
        ref = eager(t)
        ref = {k: v.clone() for k, v in ref.items()}
        torch.cuda.synchronize()
        for k in names:
            static[k].copy_(t[k])
        graph.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(cap_ws[k], ref[k]), ("bob_ws", rep, k)
            assert torch.equal(cap_na[k], ref[k]), ("bob_noalloc", rep, k)
