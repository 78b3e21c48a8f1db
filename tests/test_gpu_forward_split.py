"""GPU tests of the split forward (C ABI ``fbob_forward_ws``): on problems whose 256-row
tiles leave work-group slots idle, each tile's key sweep is split over several
work-groups that keep their online-softmax state (unnormalised O, row sum, reference
maximum) in the workspace, and a reduction merges them.

* O, L and D of every row against the fp64 oracle at the bf16 bar (2e-2 of max|ref|),
  over the planner's part counts 2-8, with and without the mask (causal tiles whose late
  parts hold no key of the tile, and parts that hold no key of some rows), tau a power of
  two and not, grouped heads, d = 64 and 128, ragged tails, near-one-hot rows;
* ``dO = None`` gives the same O and L, bitwise;
* no workspace, too small a workspace or fp32 inputs run ``fbob_forward`` exactly
  (bitwise).
Every case prints its name and part count before it touches the GPU.
"""

import numpy as np
import pytest

import oracle
import workloads
from tests import _gpu_util as U

pytestmark = pytest.mark.gpu


def case(name, B, H, N, d, seed, Hkv=None, tau=None, dtype="bf16", **kw):
    extra = {"Hkv": Hkv} if Hkv else {}
    if tau is not None:
        extra["tau"] = tau
    return workloads.Workload(name, B=B, H=H, N=N, d=d, dtype=dtype, seed=seed, extra=extra,
                              **kw)


SPLIT = [
    case("fsplit_h1_n4096_d64", 1, 1, 4096, 64, 301),
    case("fsplit_h1_n4096_d64_causal", 1, 1, 4096, 64, 302, causal=True),
    case("fsplit_h2_n1000_d64_tau0.1_ragged", 1, 2, 1000, 64, 303, tau=0.1),
    case("fsplit_gqa_b2_hq4_hkv2_n2500_d64_causal", 2, 4, 2500, 64, 304, Hkv=2, causal=True),
    case("fsplit_h2_n1500_d128", 1, 2, 1500, 128, 305),
    case("fsplit_h1_n3000_d128_causal_tau0.3", 1, 1, 3000, 128, 306, causal=True, tau=0.3),
    case("fsplit_h1_n4000_d64_qk8_causal_sharp", 1, 1, 4000, 64, 307, causal=True,
         scale_qk=8.0),
    case("fsplit_h3_n2049_d64_u0.1", 1, 3, 2049, 64, 308, scale_u=0.1),
]


def run(w, workspace="auto", with_do=True):
    import torch
    import exact_softmax_attention_fbob_amd as fb
    inp = U.make_inputs(w)
    dev = U.to_device(inp, w.dtype)
    dO = dev["dO"] if with_do else None
    need = fb.forward_workspace_size(dev["Q"], dev["K"], w.tau, w.causal)
    ws = None if workspace == "auto" else workspace(dev["Q"].device, need)
    got = fb.forward_ws(dev["Q"], dev["K"], dev["V"], dO, w.tau, w.causal, workspace=ws)
    plain = fb.forward(dev["Q"], dev["K"], dev["V"], dO, w.tau, w.causal)
    torch.cuda.synchronize()
    return inp, need, got, plain


@pytest.mark.parametrize("w", SPLIT, ids=[w.name for w in SPLIT])
def test_split_forward_matches_oracle(w):
    U.say(f"[fsplit] {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal} "
          f"tau={w.tau:g}")
    inp, need, got, plain = run(w)
    rows = w.B * w.H * w.N
    parts = need // (rows * (w.d + 2) * 4)
    U.say(f"[fsplit] {w.name}: workspace {need} B = {parts} parts")
    assert need > 0 and need == parts * rows * (w.d + 2) * 4 and 2 <= parts <= 16
    q, k = U.split_inputs(inp, w)
    errs = {}
    for name, idx in (("O", 0), ("L", 1), ("D", 2)):
        g = got[idx].cpu().numpy().astype(np.float64)
        refs, gs = [], []
        for (b, h) in U.head_list(w):
            ref = oracle.forward(q("Q", b, h), k("K", b, h), k("V", b, h), q("dO", b, h),
                                 w.tau, w.causal)
            refs.append(ref[idx])
            gs.append(g[b, h])
        errs[name] = U.rel(np.stack(gs), np.stack(refs))
        errs[name + "_vs_unsplit"] = U.rel(g, plain[idx].cpu().numpy().astype(np.float64))
    U.say(f"[fsplit] {w.name}: " + " ".join(f"{kk}={v:.1e}" for kk, v in errs.items()))
    bad = {kk: v for kk, v in errs.items() if not kk.endswith("unsplit")
           and not (v <= U.TOL["bf16"])}
    assert not bad, bad
    assert np.isfinite(got[0].cpu().numpy()).all() and np.isfinite(got[1].cpu().numpy()).all()


def test_split_forward_without_do_gives_same_o_and_l():
    import torch
    w = SPLIT[1]
    U.say(f"[fsplit] {w.name}: dO = None")
    _, need, got, _ = run(w)
    _, need2, got2, _ = run(w, with_do=False)
    assert need == need2 > 0 and got2[2] is None
    assert torch.equal(got[0], got2[0]) and torch.equal(got[1], got2[1])


@pytest.mark.parametrize("kind", ["none", "small", "f32"])
def test_forward_ws_without_split_is_forward_bitwise(kind):
    import torch
    w = SPLIT[0] if kind != "f32" else case("fsplit_f32_h1_n1024_d64_causal", 1, 1, 1024, 64,
                                           309, dtype="f32", causal=True)
    U.say(f"[fsplit] {w.name}: workspace {kind}")
    if kind == "none":
        ws = lambda dev, need: torch.empty(0, dtype=torch.uint8, device=dev)  # noqa: E731
    elif kind == "small":
        ws = lambda dev, need: torch.empty(need - 16, dtype=torch.uint8, device=dev)  # noqa
    else:
        ws = "auto"
    _, need, got, plain = run(w, workspace=ws)
    assert (need == 0) == (kind == "f32")
    for a, b in zip(got, plain):
        assert torch.equal(a, b)
