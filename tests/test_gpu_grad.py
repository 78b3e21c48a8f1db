"""GPU parity of the first-order backward (C ABI ``fbob_backward``) and of the
twice-differentiable autograd layer, against the fp64 oracle.

Every case prints its name before it touches the GPU.  Bars as for the BoB:
max|gpu - ref| / max|ref| per output tensor <= 1e-3 (fp32 inputs) or <= 2e-2
(bf16 inputs).  Key/value-side gradients of grouped heads are compared with the
oracle summed over the query heads of the group.
"""

import numpy as np
import pytest

import oracle
import workloads
from tests import _gpu_util as U

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS


def case(name, B, H, N, d, dtype, seed, causal=False, Hkv=None, tau=None, **kw):
    extra = {"Hkv": Hkv} if Hkv else {}
    if tau is not None:
        extra["tau"] = tau
    return workloads.Workload(name, B=B, H=H, N=N, d=d, dtype=dtype, seed=seed, causal=causal,
                              extra=extra, **kw)


CASES = [
    case("g_n1_bf16", 1, 1, 1, 64, "bf16", 41),
    case("g_n300_b2_h3_bf16_ragged", 2, 3, 300, 64, "bf16", 42),
    case("g_n129_d128_h2_bf16", 1, 2, 129, 128, "bf16", 43),
    case("g_n200_d64_f32", 1, 1, 200, 64, "f32", 44),
    case("g_n150_d128_h2_f32_causal", 1, 2, 150, 128, "f32", 45, causal=True),
    case("g_n333_h2_bf16_causal", 1, 2, 333, 64, "bf16", 46, causal=True),
    case("g_gqa_hq6_hkv2_n160_bf16_causal", 1, 6, 160, 64, "bf16", 47, causal=True, Hkv=2),
    case("g_mqa_hq3_hkv1_n96_d128_bf16", 1, 3, 96, 128, "bf16", 48, Hkv=1),
    case("g_n1000_qk2_bf16", 1, 1, 1000, 64, "bf16", 49, scale_qk=2.0),
    case("g_n210_h2_bf16_tau0.1_causal", 1, 2, 210, 64, "bf16", 52, causal=True, tau=0.1),
]


def run_grad(dev, tau, causal):
    import torch
    import exact_softmax_attention_fbob_amd as fb
    O, L, D0 = fb.forward(dev["Q"], dev["K"], dev["V"], None, tau, causal)
    assert D0 is None
    g = fb.backward(dev["Q"], dev["K"], dev["V"], dev["dO"], O, L, tau, causal)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy().astype(np.float64) for k, v in g.items()}


def oracle_grad(inp, w, heads=None, blocked=False):
    q, k = U.split_inputs(inp, w)
    res = {}
    for (b, h) in heads or U.head_list(w):
        a = (q("Q", b, h), k("K", b, h), k("V", b, h), q("dO", b, h))
        if blocked:
            res[(b, h)] = oracle.first_backward_blocked(*a, w.tau, w.causal)
        else:
            dQ, dK, dV = oracle.first_backward(*a, w.tau, w.causal)
            _, _, D = oracle.forward(*a, w.tau, w.causal)
            res[(b, h)] = dict(dQ=dQ, dK=dK, dV=dV, D=D)
    return res


def compare(gpu, ref, w, keys=("dQ", "dK", "dV", "D")):
    hkv = w.extra.get("Hkv", w.H)
    group = w.H // hkv
    errs = {}
    for key in keys:
        a, bb = [], []
        if key in ("dK", "dV"):
            kv = {}
            for (b, h), o in ref.items():
                kv.setdefault((b, h // group), []).append(o[key])
            for (b, g), parts in kv.items():
                if len(parts) == group:
                    a.append(gpu[key][b, g].ravel())
                    bb.append(np.sum(parts, axis=0).ravel())
        else:
            for (b, h), o in ref.items():
                a.append(gpu[key][b, h].ravel())
                bb.append(o[key].ravel())
        errs[key] = U.rel(np.concatenate(a), np.concatenate(bb))
    return errs


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_backward_small_cases_full_oracle(w):
    U.say(f"[grad] {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} causal={w.causal}")
    inp = U.make_inputs(w)
    gpu = run_grad(U.to_device(inp, w.dtype), w.tau, w.causal)
    errs = compare(gpu, oracle_grad(inp, w), w)
    U.say(f"[grad] {w.name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    tol = U.TOL[w.dtype]
    assert all(v <= tol for v in errs.values()), errs


DQ_VARIANTS = [("FBOB_TUNE_DQ", v) for v in (1, 2, 3, 4)] + \
    [("FBOB_TUNE_DQ_D128", v) for v in (1, 2)] + [("FBOB_TUNE_DKV", 1)]


@pytest.mark.parametrize("var,val", DQ_VARIANTS, ids=[f"{a}={b}" for a, b in DQ_VARIANTS])
def test_backward_row_pass_variants(var, val, monkeypatch, tuning_library):
    """Every compiled layout of the row pass (rows per wave, stage size, four-wave
    work-groups) and the column pass's four-wave layout against the oracle, on a ragged
    tail and on a causal grouped-query case."""
    d = 128 if var.endswith("D128") else 64
    monkeypatch.setenv(var, str(val))
    for w in (case(f"dqv_n300_b2_h2_d{d}", 2, 2, 300, d, "bf16", 81),
              case(f"dqv_gqa_hq4_hkv2_n200_d{d}_causal", 1, 4, 200, d, "bf16", 82, causal=True,
                   Hkv=2)):
        U.say(f"[grad] {var}={val} {w.name}")
        inp = U.make_inputs(w)
        gpu = run_grad(U.to_device(inp, w.dtype), w.tau, w.causal)
        errs = compare(gpu, oracle_grad(inp, w), w)
        U.say(f"[grad] {var}={val} {w.name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
        assert all(v <= U.TOL[w.dtype] for v in errs.values()), errs


def _check_column_sums(w, inp, gpu):
    """sum_j dK_j = 0 and sum_j dV_j = sum over the group's rows of dO (exact)."""
    hkv = w.extra.get("Hkv", w.H)
    group = w.H // hkv
    dK, dV = gpu["dK"], gpu["dV"]
    s = np.abs(dK.sum(axis=2))
    ratio = float(np.max(s / np.maximum(np.abs(dK).sum(axis=2), 1e-30)))
    dO = inp["dO"].astype(np.float64).reshape(w.B, hkv, group, w.N, w.d).sum(axis=(2, 3))
    err = U.rel(dV.sum(axis=2), dO)
    U.say(f"[grad] {w.name} column sums: dK ratio {ratio:.2e}, dV rel err {err:.2e}")
    assert ratio < 1e-2 and err < 1e-3, (ratio, err)


def test_backward_headline_two_heads_full_and_column_sums():
    w = W["h12_n16384_d64_bf16_u01"]
    U.say(f"[grad] {w.name}")
    inp = U.make_inputs(w)
    gpu = run_grad(U.to_device(inp, w.dtype), w.tau, w.causal)
    errs = compare(gpu, oracle_grad(inp, w, heads=[(0, 0), (0, 11)], blocked=True), w)
    U.say(f"[grad] {w.name} heads 0,11: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= U.TOL[w.dtype] for v in errs.values()), errs
    _check_column_sums(w, inp, gpu)


def test_backward_long_d128_sampled_rows_and_column_sums():
    w = W["h8_n65536_d128_bf16_qk2"]
    U.say(f"[grad] {w.name}")
    inp = U.make_inputs(w)
    gpu = run_grad(U.to_device(inp, w.dtype), w.tau, w.causal)
    q, k = U.split_inputs(inp, w)
    rng = np.random.default_rng(5)
    a = {"dQ": [], "D": []}
    r = {"dQ": [], "D": []}
    for (b, h) in U.head_list(w):
        rows = np.sort(rng.choice(w.N, size=8, replace=False))
        rows[-1] = w.N - 1
        o = oracle.first_backward_rows(q("Q", b, h), k("K", b, h), k("V", b, h), q("dO", b, h),
                                       w.tau, rows, w.causal)
        for key in a:
            a[key].append(gpu[key][b, h][rows].ravel())
            r[key].append(o[key].ravel())
    errs = {key: U.rel(np.concatenate(a[key]), np.concatenate(r[key])) for key in a}
    U.say(f"[grad] {w.name} sampled rows: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= U.TOL[w.dtype] for v in errs.values()), errs
    _check_column_sums(w, inp, gpu)


def test_forward_without_do_matches_forward_with_do():
    """O and L do not depend on whether D is requested; D from the backward agrees
    with D from the forward (two fp32 sums of the same products)."""
    import torch
    import exact_softmax_attention_fbob_amd as fb
    w = case("g_fwd_n500_h2_bf16", 1, 2, 500, 64, "bf16", 50)
    U.say(f"[grad] {w.name}")
    dev = U.to_device(U.make_inputs(w), w.dtype)
    O1, L1, D1 = fb.forward(dev["Q"], dev["K"], dev["V"], dev["dO"], w.tau)
    O2, L2, D2 = fb.forward(dev["Q"], dev["K"], dev["V"], None, w.tau)
    g = fb.backward(dev["Q"], dev["K"], dev["V"], dev["dO"], O2, L2, w.tau)
    torch.cuda.synchronize()
    assert D2 is None
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    err = (g["D"] - D1).abs().max().item() / D1.abs().max().item()
    assert err < 1e-5, err


def test_backward_bitwise_deterministic():
    import torch
    import exact_softmax_attention_fbob_amd as fb
    w = case("g_det_n700_hq4_hkv2_bf16", 1, 4, 700, 64, "bf16", 51, Hkv=2)
    U.say(f"[grad] {w.name}")
    dev = U.to_device(U.make_inputs(w), w.dtype)
    O, L, _ = fb.forward(dev["Q"], dev["K"], dev["V"], None, w.tau)
    a = fb.backward(dev["Q"], dev["K"], dev["V"], dev["dO"], O, L, w.tau)
    b = fb.backward(dev["Q"], dev["K"], dev["V"], dev["dO"], O, L, w.tau)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key


# ---------------------------------------------------------------------------
# autograd layer: attention(Q, K, V) differentiated once and twice
# ---------------------------------------------------------------------------

AUTOGRAD_CASES = [
    case("ag_n200_h2_bf16", 1, 2, 200, 64, "bf16", 61),
    case("ag_n130_f32_causal", 1, 1, 130, 64, "f32", 62, causal=True),
    case("ag_gqa_hq4_hkv2_n96_d128_bf16_causal", 1, 4, 96, 128, "bf16", 63, causal=True, Hkv=2),
    # small enough that the double backward takes the split schedule (Pass 1 in 4 parts)
    case("ag_n600_h2_bf16_causal_split", 1, 2, 600, 64, "bf16", 65, causal=True),
]


def _oracle_per_head(inp, w, fn):
    q, k = U.split_inputs(inp, w)
    return {(b, h): fn(q, k, b, h) for (b, h) in U.head_list(w)}


# the second derivative with the fp32 row-sum option on near-one-hot rows (Q, K x 8),
# unsplit and split
ROW_SUM_CASES = [
    case("ag_n200_h2_bf16_qk8_rowsums", 1, 2, 200, 64, "bf16", 30, scale_qk=8.0),
    case("ag_n600_h2_bf16_causal_split_rowsums", 1, 2, 600, 64, "bf16", 65, causal=True),
]


@pytest.mark.parametrize("w,row_sums", [(x, False) for x in AUTOGRAD_CASES]
                         + [(x, True) for x in ROW_SUM_CASES],
                         ids=[x.name for x in AUTOGRAD_CASES + ROW_SUM_CASES])
def test_autograd_first_and_second_derivatives(w, row_sums):
    """grad of O against dO is the first backward; the gradient of
    Phi = <dQ,U_Q> + <dK,U_K> + <dV,U_V> with respect to (Q, K, V, dO), taken by
    autograd through the first backward, is the BoB."""
    import torch
    from exact_softmax_attention_fbob_amd.autograd import attention
    U.say(f"[autograd] {w.name}")
    inp = U.make_inputs(w)
    dev = U.to_device(inp, w.dtype)
    Q, K, V, dO = (dev[n].clone().requires_grad_(True) for n in ("Q", "K", "V", "dO"))
    O = attention(Q, K, V, w.tau, w.causal, fp32_row_sums=row_sums)
    gQ, gK, gV = torch.autograd.grad(O, (Q, K, V), grad_outputs=dO, create_graph=True)
    phi = ((gQ.float() * dev["UQ"].float()).sum() + (gK.float() * dev["UK"].float()).sum()
           + (gV.float() * dev["UV"].float()).sum())
    hQ, hK, hV, hdO = torch.autograd.grad(phi, (Q, K, V, dO))
    torch.cuda.synchronize()
    got = {k: v.detach().float().cpu().numpy().astype(np.float64) for k, v in
           dict(O=O, dQ=gQ, dK=gK, dV=gV, dQt=hQ, dKt=hK, dVt=hV, ddOt=hdO).items()}

    def ref_fn(q, k, b, h):
        a = (q("Q", b, h), k("K", b, h), k("V", b, h), q("dO", b, h))
        u = (q("UQ", b, h), k("UK", b, h), k("UV", b, h))
        O_, _, _ = oracle.forward(*a, w.tau, w.causal)
        dQ, dK, dV = oracle.first_backward(*a, w.tau, w.causal)
        out = oracle.bob(*a, *u, w.tau, w.causal)
        out.update(O=O_, dQ=dQ, dK=dK, dV=dV)
        return out

    ref = _oracle_per_head(inp, w, ref_fn)
    errs = compare(got, ref, w, keys=("O", "dQ", "dK", "dV"))
    errs.update(U.compare_full(got, ref, w, keys=("dQt", "dKt", "dVt", "ddOt")))
    U.say(f"[autograd] {w.name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= U.TOL[w.dtype] for v in errs.values()), errs


def test_autograd_hessian_vector_product_of_squared_output():
    """HVP of loss = 0.5 ||O||^2 in direction (U_Q, U_K, U_V): here dO = O depends on
    (Q, K, V) too, so the product is the BoB at dO = O plus the first backward of
    the BoB's ddO~ (the path through dO)."""
    import torch
    from exact_softmax_attention_fbob_amd.autograd import attention
    w = case("ag_hvp_n160_h2_f32", 1, 2, 160, 64, "f32", 64)
    U.say(f"[autograd] {w.name}")
    inp = U.make_inputs(w)
    dev = U.to_device(inp, w.dtype)
    Q, K, V = (dev[n].clone().requires_grad_(True) for n in ("Q", "K", "V"))
    O = attention(Q, K, V, w.tau, w.causal)
    loss = 0.5 * (O * O).sum()
    g = torch.autograd.grad(loss, (Q, K, V), create_graph=True)
    s = sum((gi * dev[u]).sum() for gi, u in zip(g, ("UQ", "UK", "UV")))
    hv = torch.autograd.grad(s, (Q, K, V))
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy().astype(np.float64) for k, v in zip(("dQt", "dKt", "dVt"), hv)}

    def ref_fn(q, k, b, h):
        r = oracle.hvp_half_squared_output(q("Q", b, h), k("K", b, h), k("V", b, h),
                                           q("UQ", b, h), k("UK", b, h), k("UV", b, h),
                                           w.tau, w.causal)
        return dict(dQt=r["dQ"], dKt=r["dK"], dVt=r["dV"])

    ref = _oracle_per_head(inp, w, ref_fn)
    errs = U.compare_full(got, ref, w, keys=("dQt", "dKt", "dVt"))
    U.say(f"[autograd] {w.name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= U.TOL[w.dtype] for v in errs.values()), errs


# ---------------------------------------------------------------------------
# split schedule of the first backward (fbob_backward_ws) on problems too small to fill
# the GPU: against the oracle, against the unsplit call, and bitwise repeatable
# ---------------------------------------------------------------------------

SPLIT_GRAD = [
    case("gws_n1000_h2_ragged", 1, 2, 1000, 64, "bf16", 91),
    case("gws_gqa_hq8_hkv2_n700", 1, 8, 700, 64, "bf16", 92, Hkv=2),
    case("gws_n1500_h2_d128", 1, 2, 1500, 128, "bf16", 93),
    case("gws_causal_n1000_h2", 1, 2, 1000, 64, "bf16", 94, causal=True),
    case("gws_causal_gqa_hq6_hkv2_n600_d128", 1, 6, 600, 128, "bf16", 95, causal=True, Hkv=2),
]


@pytest.mark.parametrize("w", SPLIT_GRAD, ids=[w.name for w in SPLIT_GRAD])
def test_backward_split_schedule(w):
    import torch
    import exact_softmax_attention_fbob_amd as fb
    U.say(f"[grad] split {w.name}")
    inp = U.make_inputs(w)
    dev = U.to_device(inp, w.dtype)
    Q, K, V, dO = (dev[k] for k in ("Q", "K", "V", "dO"))
    O, L, _ = fb.forward(Q, K, V, None, w.tau, w.causal)
    need = fb.backward_workspace_size(Q, K, w.tau, w.causal)
    assert need > 0, "the case is meant to take the split schedule"
    ws = torch.empty(need, dtype=torch.uint8, device=Q.device)
    got = fb.backward_ws(Q, K, V, dO, O, L, w.tau, w.causal, workspace=ws)
    again = fb.backward_ws(Q, K, V, dO, O, L, w.tau, w.causal, workspace=ws)
    ref = fb.backward(Q, K, V, dO, O, L, w.tau, w.causal)
    torch.cuda.synchronize()
    for k in got:
        assert torch.equal(got[k], again[k]), k
    diff = {k: float((got[k] - ref[k]).abs().max() / ref[k].abs().max()) for k in got}
    U.say(f"[grad] split {w.name} vs unsplit: " + " ".join(f"{k}={v:.1e}" for k, v in diff.items()))
    assert all(v < 3e-3 for v in diff.values()), diff
    assert torch.equal(got["D"], ref["D"])
    gpu = {k: v.cpu().numpy().astype(np.float64) for k, v in got.items()}
    errs = compare(gpu, oracle_grad(inp, w), w)
    U.say(f"[grad] split {w.name} vs oracle: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= U.TOL[w.dtype] for v in errs.values()), errs
