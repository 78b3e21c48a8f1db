"""GPU parity of the split schedule for small problems (C ABI ``fbob_bob_ws``).

With a workspace, problems too small to fill the GPU split each Pass 1 row tile's
key sweep and each Pass 2 column tile's row sweep over several work-groups, which
write fp32 partial sums that a reduction kernel adds.  Where Pass 1's row tiles fill
whole rounds of the CUs and leave a partial one (either pass, with or without the mask),
the heads of the whole rounds run unsplit and only the rest split (a launch on each head
range).  With the causal mask (d = 64)
a work-group sweeps two tiles (row tiles n - 1 - p and p in Pass 1, column tiles p and
n - 1 - p in Pass 2), and the split cuts that joint sweep, so a part can end in one
tile and begin the other.  The outputs are checked against the fp64 oracle (same bars as the unsplit
path), against the unsplit ``fbob_bob`` (they differ only in the order of fp32
additions), and for bitwise determinism.  Every case prints its name before it
touches the GPU.
"""

import numpy as np
import pytest

import workloads
from tests import _gpu_util as U

pytestmark = pytest.mark.gpu


def case(name, B, H, N, d, dtype, seed, Hkv=None, **kw):
    extra = {"Hkv": Hkv} if Hkv else {}
    return workloads.Workload(name, B=B, H=H, N=N, d=d, dtype=dtype, seed=seed, extra=extra,
                              **kw)


SPLIT_CASES = [
    workloads.WORKLOADS["gpt2_heads_h12_n4096_d64_bf16"],       # 2 key parts, Pass 2 unsplit
    case("split_n1000_h2_ragged", 1, 2, 1000, 64, "bf16", 61),   # ragged tail, 8 parts each
    case("split_n560_h1_empty_parts", 1, 1, 560, 64, "bf16", 62),  # 4 + 4 parts, last ones empty
    case("split_gqa_hq8_hkv2_n700", 1, 8, 700, 64, "bf16", 63, Hkv=2),
    case("split_n1500_h2_d128", 1, 2, 1500, 128, "bf16", 64),
    case("split_n2048_b2_h3_qk2", 2, 3, 2048, 64, "bf16", 65, scale_qk=2.0),
    # causal, both passes in 8 parts: Pass 1 row-tile pairs of 18 joint key stages in
    # parts of 3 (part 5 crosses from the first tile into the second, parts 6 and 7 are
    # empty); Pass 2 column-tile pairs of 20 joint row steps (part 5 crosses, part 7 empty)
    case("split_causal_n1000_h2_ragged", 1, 2, 1000, 64, "bf16", 66, causal=True),
    # Pass 1 in 4 parts, Pass 2 in 8; 3 column tiles: a pair and an unpaired middle
    # tile (half the steps); 4 query heads per K/V head
    case("split_causal_gqa_hq8_hkv2_n700", 1, 8, 700, 64, "bf16", 67, Hkv=2, causal=True),
    case("split_causal_n2048_b2_h3_qk2", 2, 3, 2048, 64, "bf16", 68, causal=True,
         scale_qk=2.0),                                           # Pass 1 in 4, Pass 2 in 8
    # causal at d = 128: single tiles (longest first), each tile's own sweep cut, so the
    # first tiles' parts are short or empty; ragged, and grouped heads
    case("split_causal_d128_n1000_h2", 1, 2, 1000, 128, "bf16", 80, causal=True),
    case("split_causal_d128_gqa_hq6_hkv2_n600", 1, 6, 600, 128, "bf16", 81, Hkv=2,
         causal=True),
    # Pass 1 unsplit on the heads of whole rounds, split on the rest (384 row tiles: 256
    # in one round unsplit, 128 in two parts): grouped heads (the unsplit part ends on a
    # group boundary, the split part starts at K/V head 8), whole batches (batches 0-1
    # unsplit, batch 2 split), and d = 128 with a ragged N
    case("split_partial_hq24_hkv12_n2048", 1, 24, 2048, 64, "bf16", 74, Hkv=12),
    case("split_partial_b3_h8_n2048", 3, 8, 2048, 64, "bf16", 75),
    case("split_partial_h24_n2000_d128", 1, 24, 2000, 128, "bf16", 76),
]

# The GPT-2-heads shape with the causal mask: 96 Pass 2 work-groups (8 tile pairs x 12
# heads) on 256 CUs split in two, Pass 1 (192 pairs of row tiles) unsplit; checked
# against the oracle on two heads.
CAUSAL_C2 = workloads.WORKLOADS["gpt2_heads_h12_n4096_d64_bf16"].with_(
    name="split_causal_gpt2_heads_h12_n4096", causal=True)


def run_ws(dev, w):
    import torch
    import exact_softmax_attention_fbob_amd as fb
    args = tuple(dev[k] for k in ("Q", "K", "V", "dO", "UQ", "UK", "UV"))
    O, L, D = fb.forward(*args[:4], w.tau, w.causal)
    need = fb.bob_workspace_size(dev["Q"], dev["K"], w.tau, w.causal)
    ws = torch.empty(need, dtype=torch.uint8, device=dev["Q"].device)
    out = fb.bob_ws(*args, O, L, D, w.tau, w.causal, workspace=ws)
    ref = fb.bob(*args, O, L, D, w.tau, w.causal)
    torch.cuda.synchronize()
    return need, out, ref, (args, O, L, D, ws)


def check_against_unsplit(w, out, ref):
    # the same rounded products, fp32 sums in another order (dK~ and dV~ sum thousands
    # of rows with heavy cancellation, so the reordering shows at 1e-4 to 1e-3 of their
    # maximum; the bar is 7x under parity's)
    diff = {k: float((out[k] - ref[k]).abs().max() / ref[k].abs().max()) for k in out}
    U.say(f"[split] {w.name} vs unsplit: " + " ".join(f"{k}={v:.1e}" for k, v in diff.items()))
    assert all(v < 3e-3 for v in diff.values()), diff


@pytest.mark.parametrize("w", SPLIT_CASES, ids=[w.name for w in SPLIT_CASES])
def test_split_schedule_matches_oracle_and_unsplit(w):
    U.say(f"[split] {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal}")
    inp = U.make_inputs(w)
    dev = U.to_device(inp, w.dtype)
    need, out, ref, _ = run_ws(dev, w)
    assert need > 0, "the case is meant to take the split schedule"
    gpu = {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()}
    errs = U.compare_full(gpu, U.oracle_full(inp, w), w, keys=U.ALL_KEYS)
    U.say(f"[split] {w.name} vs oracle: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= U.TOL[w.dtype] for v in errs.values()), errs
    check_against_unsplit(w, out, ref)


def test_causal_split_at_the_gpt2_heads_shape():
    """Pass 2 in two parts (Pass 1 unsplit): every output against the unsplit call, and
    two heads (the first and the last) in full against the oracle."""
    w = CAUSAL_C2
    U.say(f"[split] {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal}")
    inp = U.make_inputs(w)
    dev = U.to_device(inp, w.dtype)
    need, out, ref, _ = run_ws(dev, w)
    assert need == 2 * w.H * w.N * 2 * w.d * 4, need
    check_against_unsplit(w, out, ref)
    gpu = {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()}
    ora = U.oracle_full(inp, w, heads=[(0, 0), (0, w.H - 1)])
    errs = U.compare_full(gpu, ora, w, keys=U.ALL_KEYS)
    U.say(f"[split] {w.name} vs oracle (2 heads): " +
          " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= U.TOL[w.dtype] for v in errs.values()), errs


# Pass 2, and the causal pairs of both passes, with the heads of whole rounds unsplit
# and the rest split: 40 heads at N = 2048 (Pass 1: 32 heads whole and 8 in two parts;
# Pass 2: 32 whole and 8 in four), the causal mask at N = 4096 (pairs of tiles: Pass 1
# 32 + 8 in two, Pass 2 32 + 8 in four) and 40 key/value heads shared by 80 query heads
# (Pass 2 over key/value head ranges: 32 whole, 8 in four).  The first and the last
# group of heads (one from each part) against the oracle, every head against the
# unsplit call.
PARTIAL = [
    case("split_partial_h40_n2048", 1, 40, 2048, 64, "bf16", 77),
    case("split_partial_causal_h40_n4096", 1, 40, 4096, 64, "bf16", 78, causal=True),
    case("split_partial_gqa_hq80_hkv40_n2048", 1, 80, 2048, 64, "bf16", 79, Hkv=40),
]


@pytest.mark.parametrize("w", PARTIAL, ids=[w.name for w in PARTIAL])
def test_partial_split_first_and_last_heads_against_oracle(w):
    U.say(f"[split] {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} causal={w.causal}")
    inp = U.make_inputs(w)
    dev = U.to_device(inp, w.dtype)
    need, out, ref, _ = run_ws(dev, w)
    assert need > 0, "the case is meant to take the split schedule"
    check_against_unsplit(w, out, ref)
    group = w.H // w.extra.get("Hkv", w.H)
    heads = [(0, h) for h in list(range(group)) + list(range(w.H - group, w.H))]
    gpu = {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()}
    errs = U.compare_full(gpu, U.oracle_full(inp, w, heads=heads), w, keys=U.ALL_KEYS)
    U.say(f"[split] {w.name} vs oracle (first and last groups): " +
          " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= U.TOL[w.dtype] for v in errs.values()), errs


@pytest.mark.parametrize("w", [SPLIT_CASES[1], SPLIT_CASES[6]],
                         ids=[SPLIT_CASES[1].name, SPLIT_CASES[6].name])
def test_split_schedule_is_deterministic(w):
    import torch
    import exact_softmax_attention_fbob_amd as fb
    U.say(f"[split] determinism {w.name}")
    dev = U.to_device(U.make_inputs(w), w.dtype)
    _, a, _, (args, O, L, D, ws) = run_ws(dev, w)
    b = fb.bob_ws(*args, O, L, D, w.tau, w.causal, workspace=ws)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_without_workspace_equals_fbob_bob():
    """No workspace (or a too small one): fbob_bob_ws is fbob_bob, bitwise."""
    import torch
    import exact_softmax_attention_fbob_amd as fb
    w = SPLIT_CASES[2]
    U.say(f"[split] small workspace {w.name}")
    dev = U.to_device(U.make_inputs(w), w.dtype)
    args = tuple(dev[k] for k in ("Q", "K", "V", "dO", "UQ", "UK", "UV"))
    O, L, D = fb.forward(*args[:4], w.tau)
    tiny = torch.empty(16, dtype=torch.uint8, device=dev["Q"].device)
    got = fb.bob_ws(*args, O, L, D, w.tau, workspace=tiny)
    ref = fb.bob(*args, O, L, D, w.tau)
    torch.cuda.synchronize()
    for k in got:
        assert torch.equal(got[k], ref[k]), k
