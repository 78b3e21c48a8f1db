"""Pins of the fp64 oracle against things other than itself (CPU only).

Each check is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign, a transposed operand, a missing tau) fails at least one of them; the
mutation tests at the bottom plant such slips in a copy of the chain and confirm
that the finite-difference pin catches every one.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import fbob_oracle as fo
from workloads import round_to_bf16

OUT4 = ("dQt", "dKt", "dVt", "ddOt")


def rand_inputs(N, d, seed, scale_u=1.0, scale_qk=1.0):
    rng = np.random.default_rng(seed)
    t = {k: rng.standard_normal((N, d)) for k in ("Q", "K", "V", "dO", "UQ", "UK", "UV")}
    for k in ("UQ", "UK", "UV"):
        t[k] *= scale_u
    for k in ("Q", "K"):
        t[k] *= scale_qk
    return t


def args(t):
    return t["Q"], t["K"], t["V"], t["dO"], t["UQ"], t["UK"], t["UV"]


def central_fd(f, X, h=1e-5):
    """Central finite-difference gradient of scalar f with respect to array X."""
    G = np.zeros_like(X)
    for idx in np.ndindex(X.shape):
        old = X[idx]
        X[idx] = old + h
        fp = f()
        X[idx] = old - h
        fm = f()
        X[idx] = old
        G[idx] = (fp - fm) / (2 * h)
    return G


def rel_err(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ---------------------------------------------------------------------------
# first-order pieces
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,d,causal", [(5, 3, False), (9, 4, False), (7, 5, True)])
def test_first_backward_matches_fd_of_output_inner_product(N, d, causal):
    """dQ, dK, dV are the gradients of <O(Q,K,V), dO> (first backward, blog section 一)."""
    t = rand_inputs(N, d, seed=11 + N)
    tau = 1 / math.sqrt(d)
    dQ, dK, dV = fo.first_backward(t["Q"], t["K"], t["V"], t["dO"], tau, causal)

    def ell():
        O, _, _ = fo.forward(t["Q"], t["K"], t["V"], t["dO"], tau, causal)
        return float(np.sum(O * t["dO"]))

    for name, g in (("Q", dQ), ("K", dK), ("V", dV)):
        assert rel_err(g, central_fd(ell, t[name])) < 1e-8, name


def test_forward_rows_are_a_softmax_and_L_is_the_log_partition():
    t = rand_inputs(12, 6, seed=3)
    tau = 0.37
    P, L = fo.attention_probs(t["Q"], t["K"], tau)
    np.testing.assert_allclose(P.sum(1), 1.0, rtol=0, atol=1e-14)
    S = tau * t["Q"] @ t["K"].T
    # log-partition computed the naive way (no max shift) at this benign scale
    np.testing.assert_allclose(L, np.log(np.exp(S).sum(1)), rtol=1e-14)
    O, L2, D = fo.forward(t["Q"], t["K"], t["V"], t["dO"], tau)
    np.testing.assert_allclose(L2, L)
    dP = t["dO"] @ t["V"].T
    # D_i = dO_i . O_i equals sum_j P_ij dP_ij over all j (FlashBoB notes, "关键设计" 1)
    np.testing.assert_allclose(D, (P * dP).sum(1), rtol=1e-12, atol=1e-12)


def test_first_backward_matches_torch_autograd_fp64():
    torch = pytest.importorskip("torch")
    t = rand_inputs(10, 4, seed=5)
    tau = 0.5
    Q, K, V = (torch.tensor(t[k], requires_grad=True) for k in ("Q", "K", "V"))
    O = torch.softmax(tau * Q @ K.T, dim=-1) @ V
    gQ, gK, gV = torch.autograd.grad(O, (Q, K, V), torch.tensor(t["dO"]))
    dQ, dK, dV = fo.first_backward(t["Q"], t["K"], t["V"], t["dO"], tau)
    for a, b in ((dQ, gQ), (dK, gK), (dV, gV)):
        assert rel_err(a, b.numpy()) < 1e-13


# ---------------------------------------------------------------------------
# BoB outputs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,d,causal,su", [(6, 3, False, 1.0), (11, 4, False, 1.0),
                                           (16, 8, False, 0.1), (8, 5, True, 1.0)])
def test_bob_matches_central_fd_of_phi(N, d, causal, su):
    """The four BoB outputs are the gradient of Phi (FlashBoB notes, "整体框架")."""
    t = rand_inputs(N, d, seed=100 + N, scale_u=su)
    tau = 1 / math.sqrt(d)
    out = fo.bob(*args(t), tau, causal)

    def f():
        return fo.phi(*args(t), tau, causal)

    for name, key in (("Q", "dQt"), ("K", "dKt"), ("V", "dVt"), ("dO", "ddOt")):
        fd = central_fd(f, t[name])
        assert rel_err(out[key], fd) < 1e-7, (name, rel_err(out[key], fd))


def test_bob_matches_symbolic_derivation_2x2():
    """Pure calculus: sympy differentiates softmax attention twice, no printed formula used."""
    sp = pytest.importorskip("sympy")
    import mpmath

    N, d = 2, 2
    sym = {n: sp.Matrix(N, d, lambda i, j, n=n: sp.Symbol(f"{n}_{i}{j}"))
           for n in ("Q", "K", "V", "dO")}
    tau = sp.Rational(1, 2)
    S = tau * sym["Q"] * sym["K"].T
    P = sp.Matrix(N, N, lambda i, j: sp.exp(S[i, j]) / sum(sp.exp(S[i, k]) for k in range(N)))
    O = P * sym["V"]
    ell = sum(O[i, j] * sym["dO"][i, j] for i in range(N) for j in range(d))
    first = {n: sym[n].applyfunc(lambda x: sp.diff(ell, x)) for n in ("Q", "K", "V")}
    rq = np.array([[3, -2], [1, 4]]) / 7
    rk = np.array([[-5, 2], [2, 1]]) / 7
    rv = np.array([[1, -3], [-2, 6]]) / 7
    U = {"Q": rq, "K": rk, "V": rv}
    Phi = sum(first[n][i, j] * sp.Rational(int(round(U[n][i, j] * 7)), 7)
              for n in ("Q", "K", "V") for i in range(N) for j in range(d))
    flat = [s for n in ("Q", "K", "V", "dO") for s in sym[n]]
    grads = [sp.diff(Phi, s) for s in flat]
    point = {"Q": np.array([[0.4, -1.2], [0.8, 0.2]]), "K": np.array([[-0.6, 1.0], [1.4, -0.2]]),
             "V": np.array([[0.2, 1.6], [-1.0, 0.6]]), "dO": np.array([[1.2, -0.4], [0.6, 1.8]])}
    vals = [point[n][i, j] for n in ("Q", "K", "V", "dO") for i in range(N) for j in range(d)]
    mpmath.mp.dps = 30
    g = np.array([float(v) for v in sp.lambdify(flat, grads, "mpmath")(*vals)])
    out = fo.bob(point["Q"], point["K"], point["V"], point["dO"], rq, rk, rv, 0.5)
    ours = np.concatenate([out[k].ravel() for k in OUT4])
    np.testing.assert_allclose(ours, g, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_bob_matches_torch_double_backward_fp64(causal):
    """Independent library AD: torch differentiates the first backward again."""
    torch = pytest.importorskip("torch")
    N, d = 9, 4
    t = rand_inputs(N, d, seed=21)
    tau = 1 / math.sqrt(d)
    T = {k: torch.tensor(v, requires_grad=k in ("Q", "K", "V", "dO")) for k, v in t.items()}
    S = tau * T["Q"] @ T["K"].T
    if causal:
        S = S.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    O = torch.softmax(S, dim=-1) @ T["V"]
    dQ, dK, dV = torch.autograd.grad(O, (T["Q"], T["K"], T["V"]), T["dO"], create_graph=True)
    Phi = (dQ * T["UQ"]).sum() + (dK * T["UK"]).sum() + (dV * T["UV"]).sum()
    g = torch.autograd.grad(Phi, (T["Q"], T["K"], T["V"], T["dO"]))
    out = fo.bob(*args(t), tau, causal)
    for key, ref in zip(OUT4, g):
        assert rel_err(out[key], ref.detach().numpy()) < 1e-12, key


def test_bob_is_linear_in_U_and_zero_at_U_zero():
    t = rand_inputs(13, 6, seed=7)
    t2 = rand_inputs(13, 6, seed=8)
    tau = 1 / math.sqrt(6)
    a, b = 0.7, -1.9
    base = fo.bob(*args(t), tau)
    other = fo.bob(t["Q"], t["K"], t["V"], t["dO"], t2["UQ"], t2["UK"], t2["UV"], tau)
    mix = fo.bob(t["Q"], t["K"], t["V"], t["dO"], a * t["UQ"] + b * t2["UQ"],
                 a * t["UK"] + b * t2["UK"], a * t["UV"] + b * t2["UV"], tau)
    zero = fo.bob(t["Q"], t["K"], t["V"], t["dO"], 0 * t["UQ"], 0 * t["UK"], 0 * t["UV"], tau)
    for k in OUT4 + ("alpha", "E"):
        np.testing.assert_allclose(mix[k], a * base[k] + b * other[k], rtol=1e-11, atol=1e-12)
        assert np.all(zero[k] == 0.0), k


@pytest.mark.parametrize("causal", [False, True])
def test_affine_decomposition_equals_direct_chain(causal):
    """E = Edeg - alpha D, ddO~ = ddO~deg - alpha o, dQ~ = tau (Omega - alpha R - E B)."""
    t = rand_inputs(24, 7, seed=31)
    tau = 1 / math.sqrt(7)
    direct = fo.bob(*args(t), tau, causal)
    aff = fo.bob_affine(*args(t), tau, causal)
    for k in ("dQt", "ddOt", "alpha", "E"):
        assert rel_err(aff[k], direct[k]) < 1e-12, k


def test_exact_invariants():
    """Identities that follow from symmetries of Phi; they hold at any N."""
    N, d = 20, 6
    t = rand_inputs(N, d, seed=41)
    tau = 1 / math.sqrt(d)
    out = fo.bob(*args(t), tau)
    dQ, dK, dV = fo.first_backward(t["Q"], t["K"], t["V"], t["dO"], tau)
    Phi = fo.phi(*args(t), tau)
    scale = max(np.abs(out[k]).max() for k in OUT4)
    # K -> K + 1 c^T leaves P and sum_ij dS_ij F_ij unchanged
    assert np.abs(out["dKt"].sum(0)).max() < 1e-12 * scale * N
    # V -> V + 1 c^T leaves dS unchanged
    assert np.abs(out["dVt"].sum(0)).max() < 1e-12 * scale * N
    # Phi is linear (degree 1) in dO
    assert abs(np.sum(out["ddOt"] * t["dO"]) - Phi) < 1e-11 * max(1, abs(Phi))
    # dS is linear in V and dV does not depend on V
    lhs = np.sum(out["dVt"] * t["V"])
    rhs = np.sum(dQ * t["UQ"]) + np.sum(dK * t["UK"])
    assert abs(lhs - rhs) < 1e-11 * max(1, abs(rhs))
    # Q -> sQ, K -> K/s leaves the scores unchanged
    lhs = np.sum(out["dQt"] * t["Q"]) - np.sum(out["dKt"] * t["K"])
    rhs = np.sum(dK * t["UK"]) - np.sum(dQ * t["UQ"])
    assert abs(lhs - rhs) < 1e-11 * max(1, abs(rhs))


def test_E_is_dO_dot_ddO_minus_alpha_D():
    """E_i = sum_j P_ij dP~_ij equals dO_i . ddO~_i - alpha_i D_i: dP~ depends on dO
    only through dP = dO V^T and G = dO U_V^T, and the same sums of P-weighted V and
    U_V rows make up ddO~.  The oracle forms E from its definition and ddO~ from
    ddP V + P U_V, so a term dropped from either (G, the -alpha dP correction, the
    -D shift) breaks the identity.  The Pass 1 kernel forms E' this way instead of
    reducing P o dP~' over keys."""
    for causal in (False, True):
        N, d = 23, 7
        t = rand_inputs(N, d, seed=43)
        tau = 0.4
        out = fo.bob(*args(t), tau, causal=causal)
        _, _, D = fo.forward(t["Q"], t["K"], t["V"], t["dO"], tau, causal=causal)
        rhs = np.sum(t["dO"] * out["ddOt"], axis=1) - out["alpha"] * D
        assert np.abs(out["E"] - rhs).max() < 1e-12 * max(1.0, np.abs(out["E"]).max())


def test_softmax_adjoint_rows_sum_to_zero():
    t = rand_inputs(15, 4, seed=51)
    tau = 0.5
    r = fo._row_chain(t["Q"], t["dO"], t["UQ"], t["K"], t["V"], t["UK"], t["UV"], tau)
    assert np.abs(r["dSt"].sum(1)).max() < 1e-13 * np.abs(r["dSt"]).max() * 15
    assert np.abs(r["dS"].sum(1)).max() < 1e-13 * np.abs(r["dS"]).max() * 15


def test_special_case_only_UV_reduces_to_first_order_attention_backward():
    """U_Q = U_K = 0: Phi = <softmax(S) U_V, dO>, i.e. attention with V := U_V."""
    torch = pytest.importorskip("torch")
    N, d = 14, 5
    t = rand_inputs(N, d, seed=61)
    tau = 1 / math.sqrt(d)
    z = np.zeros((N, d))
    out = fo.bob(t["Q"], t["K"], t["V"], t["dO"], z, z, t["UV"], tau)
    Q, K, UV = (torch.tensor(t[k], requires_grad=True) for k in ("Q", "K", "UV"))
    Ostar = torch.softmax(tau * Q @ K.T, dim=-1) @ UV
    gQ, gK = torch.autograd.grad(Ostar, (Q, K), torch.tensor(t["dO"]))
    Ostar = Ostar.detach().numpy()
    assert rel_err(out["dQt"], gQ.numpy()) < 1e-12
    assert rel_err(out["dKt"], gK.numpy()) < 1e-12
    assert rel_err(out["ddOt"], Ostar) < 1e-13
    assert np.all(out["dVt"] == 0) and np.all(out["alpha"] == 0)
    np.testing.assert_allclose(out["E"], (t["dO"] * Ostar).sum(1), rtol=1e-12)


def test_special_case_single_position():
    """N = 1: P = 1, so (dQ~, dK~, dV~, ddO~) = (0, 0, 0, U_V), alpha = F, E = G - F dP."""
    d = 6
    t = rand_inputs(1, d, seed=71)
    tau = 0.3
    out = fo.bob(*args(t), tau)
    F = tau * (t["UQ"] @ t["K"].T + t["Q"] @ t["UK"].T)[0, 0]
    G = (t["dO"] @ t["UV"].T)[0, 0]
    dP = (t["dO"] @ t["V"].T)[0, 0]
    assert np.abs(out["dQt"]).max() < 1e-14 and np.abs(out["dKt"]).max() < 1e-14
    assert np.abs(out["dVt"]).max() < 1e-14
    np.testing.assert_allclose(out["ddOt"], t["UV"], rtol=1e-14)
    np.testing.assert_allclose(out["alpha"], [F], rtol=1e-14)
    np.testing.assert_allclose(out["E"], [G - F * dP], rtol=1e-12, atol=1e-14)


def test_u_scaling_scales_outputs():
    """The U x 0.1 workload gives exactly 0.1 x the outputs (linearity)."""
    t = rand_inputs(10, 4, seed=81)
    tau = 0.5
    a = fo.bob(*args(t), tau)
    b = fo.bob(t["Q"], t["K"], t["V"], t["dO"], 0.1 * t["UQ"], 0.1 * t["UK"], 0.1 * t["UV"], tau)
    for k in OUT4 + ("alpha", "E"):
        np.testing.assert_allclose(b[k], 0.1 * a[k], rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------------------
# row-, column- and block-restricted evaluations equal the plain one
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_rows_blocks_and_columns_agree_with_plain(causal):
    N, d = 70, 8
    t = rand_inputs(N, d, seed=91)
    tau = 1 / math.sqrt(d)
    full = fo.bob(*args(t), tau, causal)
    blk = fo.bob_blocked(*args(t), tau, causal, row_block=16)
    for k in OUT4 + ("alpha", "E"):
        assert rel_err(blk[k], full[k]) < 1e-13, k
    rows = np.array([0, 3, 17, 69])
    r = fo.bob_rows(*args(t), tau, rows, causal)
    for k in ("dQt", "ddOt", "alpha", "E"):
        assert rel_err(r[k], full[k][rows]) < 1e-13, k
    O, L, D = fo.forward(t["Q"], t["K"], t["V"], t["dO"], tau, causal)
    np.testing.assert_allclose(r["L"], L[rows], rtol=1e-14)
    np.testing.assert_allclose(r["D"], D[rows], rtol=1e-12)
    cols = np.array([1, 5, 64, 69])
    c = fo.bob_columns(*args(t), tau, cols, causal, row_block=32)
    for k in ("dKt", "dVt"):
        assert rel_err(c[k], full[k][cols]) < 1e-13, k


@pytest.mark.parametrize("N,d,causal", [(7, 4, False), (9, 3, True)])
def test_columns_from_row_scalars_match_fd_of_phi(N, d, causal):
    """dK~, dV~ at selected key positions from every row's (L, D, alpha, E) are the
    gradient of Phi with respect to those rows of K and V (central differences;
    nothing of ``bob`` is used)."""
    t = rand_inputs(N, d, seed=200 + N)
    tau = 0.55
    rs = fo.row_scalars(*args(t), tau, np.arange(N), causal)
    cols = np.array([0, 2, N - 1])
    c = fo.bob_columns_at(*args(t), tau, cols, rs["L"], rs["D"], rs["alpha"], rs["E"], causal)

    def f():
        return fo.phi(*args(t), tau, causal)

    for name, key in (("K", "dKt"), ("V", "dVt")):
        fd = central_fd(f, t[name])[cols]
        assert rel_err(c[key], fd) < 1e-7, (name, rel_err(c[key], fd))


@pytest.mark.parametrize("causal", [False, True])
def test_row_scalars_and_columns_agree_with_plain(causal):
    """The row-scalar pass equals the forward's L, D and the plain BoB's alpha, E; the
    columns built from it equal the plain BoB's dK~, dV~, and summed over all keys
    they vanish (Phi is invariant under K -> K + 1c^T and V -> V + 1c^T)."""
    N, d = 70, 8
    t = rand_inputs(N, d, seed=92)
    tau = 1 / math.sqrt(d)
    full = fo.bob(*args(t), tau, causal)
    _, L, D = fo.forward(t["Q"], t["K"], t["V"], t["dO"], tau, causal)
    rs = {k: np.empty(N) for k in ("L", "D", "alpha", "E")}
    for r0 in range(0, N, 16):  # row blocks: rows are independent
        rows = np.arange(r0, min(N, r0 + 16))
        part = fo.row_scalars(*args(t), tau, rows, causal)
        for k in rs:
            rs[k][rows] = part[k]
    np.testing.assert_allclose(rs["L"], L, rtol=1e-14)
    np.testing.assert_allclose(rs["D"], D, rtol=1e-12, atol=1e-13)
    for k in ("alpha", "E"):
        assert rel_err(rs[k], full[k]) < 1e-13, k
    allc = fo.bob_columns_at(*args(t), tau, np.arange(N), rs["L"], rs["D"], rs["alpha"],
                             rs["E"], causal)
    for k in ("dKt", "dVt"):
        assert rel_err(allc[k], full[k]) < 1e-12, k
        assert np.abs(allc[k].sum(axis=0)).max() < 1e-12 * np.abs(allc[k]).sum()
    cols = np.array([1, 5, 64, 69])
    c = fo.bob_columns_at(*args(t), tau, cols, rs["L"], rs["D"], rs["alpha"], rs["E"], causal)
    for k in ("dKt", "dVt"):
        assert rel_err(c[k], full[k][cols]) < 1e-12, k


@pytest.mark.parametrize("which", ["L", "D", "alpha", "E"])
def test_columns_depend_on_each_row_scalar(which):
    """A slip in any of the four row scalars handed to the column evaluation (here a
    shift of 0.05 in one of them) moves dK~ or dV~ well past the FD pin's bound, so
    that pin sees each scalar's role."""
    N, d = 8, 4
    t = rand_inputs(N, d, seed=301)
    tau = 0.5
    rs = fo.row_scalars(*args(t), tau, np.arange(N))
    bad = dict(rs)
    bad[which] = rs[which] + 0.05
    good = fo.bob_columns_at(*args(t), tau, np.arange(N), **rs)
    off = fo.bob_columns_at(*args(t), tau, np.arange(N), **bad)
    worst = max(rel_err(off[k], good[k]) for k in ("dKt", "dVt"))
    assert worst > 1e-3, (which, worst)


@pytest.mark.parametrize("p_rows,m", [(7, 5), (4, 9)])
def test_class_tiled_inputs_reduce_to_the_small_problem(p_rows, m):
    """If the N = m p rows of every input are copies of p class rows, each class used
    m times, then P_ij = P~_ab / m for classes a, b of i, j, and every BoB output (and
    O, D) of the full problem equals the p-row problem's output of the class, while
    L rises by ln m.  This lets a full-size GPU result be checked element by element
    against the oracle on the p class rows."""
    import workloads
    N, d = m * p_rows, 4
    small, sigma = workloads.class_tiled(1, 1, N, d, "f32", p_rows, seed=17)
    sm = {k: v[0, 0].astype(np.float64) for k, v in small.items()}
    full = {k: v[sigma] for k, v in sm.items()}
    assert sorted(np.bincount(sigma)) == [m] * p_rows
    tau = 0.7
    a_s = [sm[k] for k in ("Q", "K", "V", "dO", "UQ", "UK", "UV")]
    a_f = [full[k] for k in ("Q", "K", "V", "dO", "UQ", "UK", "UV")]
    ref, got = fo.bob(*a_s, tau), fo.bob(*a_f, tau)
    for k in OUT4 + ("alpha", "E"):
        assert rel_err(got[k], ref[k][sigma]) < 1e-12, k
    O_s, L_s, D_s = fo.forward(*a_s[:4], tau)
    O_f, L_f, D_f = fo.forward(*a_f[:4], tau)
    assert rel_err(O_f, O_s[sigma]) < 1e-13 and rel_err(D_f, D_s[sigma]) < 1e-12
    np.testing.assert_allclose(L_f, L_s[sigma] + math.log(m), rtol=1e-14)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3, 1.0 + 2 ** -8 + 2 ** -20],
                 dtype=np.float32)
    r = round_to_bf16(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa -> 1.0
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: even -> 1 + 2^-6
    np.testing.assert_array_equal(r[:4], np.array([1.0, 1.0, 1.015625, -2.5], np.float32))
    assert r[5] == np.float32(1.0 + 2 ** -7)
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    y = rng.standard_normal(10000).astype(np.float32)
    ref = torch.tensor(y).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(round_to_bf16(y), ref)


# ---------------------------------------------------------------------------
# the pins have teeth: plant slips in a copy of the chain, the FD pin must fail
# ---------------------------------------------------------------------------

def _mutant_bob(mutation):
    def chain(Qr, dOr, UQr, K, V, UK, UV, tau, causal=False, row_ids=None):
        S = tau * (Qr @ K.T)
        L = fo._logsumexp_rows(S)
        P = np.exp(S - L[:, None])
        O = P @ V
        D = (dOr * O).sum(1)
        dP = dOr @ V.T
        F = tau * (UQr @ K.T + Qr @ UK.T)
        if mutation == "F_transposed_term":
            F = tau * (UQr @ K.T + UK @ Qr.T)
        G = dOr @ UV.T
        if mutation == "drop_G":
            G = 0 * G
        dS = P * (dP - D[:, None])
        alpha = (P * F).sum(1)
        ddP = P * (F - alpha[:, None])
        if mutation == "ddP_without_D_path":
            ddP = P * F
        dPt = F * (dP - D[:, None]) + G - alpha[:, None] * dP
        if mutation == "alpha_sign":
            dPt = F * (dP - D[:, None]) + G + alpha[:, None] * dP
        E = (P * dPt).sum(1)
        dSt = P * (dPt - E[:, None])
        dQt = tau * (dSt @ K + dS @ UK)
        if mutation == "dQ_missing_tau":
            dQt = dSt @ K + dS @ UK
        ddOt = ddP @ V + P @ UV
        if mutation == "ddO_drop_PUV":
            ddOt = ddP @ V
        return dict(P=P, L=L, O=O, D=D, dS=dS, dSt=dSt, ddP=ddP, alpha=alpha, E=E,
                    dQt=dQt, ddOt=ddOt)
    return chain


@pytest.mark.parametrize("mutation", ["F_transposed_term", "drop_G", "ddP_without_D_path",
                                      "alpha_sign", "dQ_missing_tau", "ddO_drop_PUV"])
def test_fd_pin_catches_planted_mistakes(monkeypatch, mutation):
    N, d = 6, 6
    t = rand_inputs(N, d, seed=123)
    tau = 0.45
    monkeypatch.setattr(fo, "_row_chain", _mutant_bob(mutation))
    out = fo.bob(*args(t), tau)
    monkeypatch.undo()

    def f():
        return fo.phi(*args(t), tau)

    worst = 0.0
    for name, key in (("Q", "dQt"), ("K", "dKt"), ("V", "dVt"), ("dO", "ddOt")):
        worst = max(worst, rel_err(out[key], central_fd(f, t[name])))
    assert worst > 1e-3, f"mutation {mutation} not detected (worst rel err {worst})"


@pytest.mark.parametrize("mutation", ["drop_G", "ddP_without_D_path", "alpha_sign", "ddO_drop_PUV"])
def test_E_identity_catches_planted_mistakes(monkeypatch, mutation):
    """The identity E = dO . ddO~ - alpha D fails on every planted slip that touches E
    or ddO~ (a wrong F or a missing tau on dQ~ leaves it intact; the FD pin above
    catches those)."""
    N, d = 9, 5
    t = rand_inputs(N, d, seed=124)
    tau = 0.45
    monkeypatch.setattr(fo, "_row_chain", _mutant_bob(mutation))
    out = fo.bob(*args(t), tau)
    monkeypatch.undo()
    _, _, D = fo.forward(t["Q"], t["K"], t["V"], t["dO"], tau)
    rhs = np.sum(t["dO"] * out["ddOt"], axis=1) - out["alpha"] * D
    assert np.abs(out["E"] - rhs).max() > 1e-3 * max(1.0, np.abs(out["E"]).max()), mutation


@pytest.mark.parametrize("causal", [False, True])
def test_first_backward_rows_and_blocks_agree_with_plain(causal):
    """The row-restricted and row-blocked first backward equal the plain one, whose
    own pins are the finite differences and torch autograd above."""
    N, d = 75, 8
    t = rand_inputs(N, d, seed=93)
    tau = 1 / math.sqrt(d)
    dQ, dK, dV = fo.first_backward(t["Q"], t["K"], t["V"], t["dO"], tau, causal)
    _, _, D = fo.forward(t["Q"], t["K"], t["V"], t["dO"], tau, causal)
    blk = fo.first_backward_blocked(t["Q"], t["K"], t["V"], t["dO"], tau, causal, row_block=16)
    for k, ref in (("dQ", dQ), ("dK", dK), ("dV", dV), ("D", D)):
        assert rel_err(blk[k], ref) < 1e-13, k
    rows = np.array([0, 8, 40, 74])
    r = fo.first_backward_rows(t["Q"], t["K"], t["V"], t["dO"], tau, rows, causal)
    assert rel_err(r["dQ"], dQ[rows]) < 1e-13
    assert rel_err(r["D"], D[rows]) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_hvp_of_squared_output_matches_fd_of_gradient(causal):
    """The HVP composition against a central difference of the first-order gradient
    of 0.5 ||O||^2 (first backward at dO = O) along the direction U."""
    N, d = 9, 4
    t = rand_inputs(N, d, seed=95)
    tau = 0.6
    h = 1e-5

    def grad_at(s):
        Q, K, V = t["Q"] + s * t["UQ"], t["K"] + s * t["UK"], t["V"] + s * t["UV"]
        O, _, _ = fo.forward(Q, K, V, np.zeros_like(Q), tau, causal)
        return fo.first_backward(Q, K, V, O, tau, causal)

    gp, gm = grad_at(h), grad_at(-h)
    hv = fo.hvp_half_squared_output(*args(t)[:3], t["UQ"], t["UK"], t["UV"], tau, causal)
    for k, a, b in zip(("dQ", "dK", "dV"), gp, gm):
        assert rel_err(hv[k], (a - b) / (2 * h)) < 1e-7, k


def test_first_backward_column_sums():
    """Exact identities of the first backward at any size: sum_j dK_j = 0 (rows of
    dS sum to zero) and sum_j dV_j = sum_i dO_i (rows of P sum to one)."""
    N, d = 40, 6
    t = rand_inputs(N, d, seed=94)
    for causal in (False, True):
        out = fo.first_backward_blocked(t["Q"], t["K"], t["V"], t["dO"], 0.4, causal, row_block=7)
        assert np.max(np.abs(out["dK"].sum(axis=0))) < 1e-12 * np.abs(out["dK"]).sum()
        np.testing.assert_allclose(out["dV"].sum(axis=0), t["dO"].sum(axis=0), rtol=1e-12,
                                   atol=1e-12)


def test_oracle_package_exports():
    for name in ("forward", "first_backward", "first_backward_rows", "first_backward_blocked",
                 "phi", "bob", "bob_affine", "bob_rows", "hvp_half_squared_output",
                 "bob_blocked", "bob_columns", "attention_probs", "row_scalars",
                 "bob_columns_at"):
        assert callable(getattr(oracle, name))


def test_oracle_regression_fixture():
    """Frozen oracle output on a tiny case (tests/golden/bob_n6_d4.json)."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "bob_n6_d4.json")
    with open(path) as f:
        g = json.load(f)
    t = {k: np.array(v) for k, v in g["inputs"].items()}
    O, L, D = fo.forward(t["Q"], t["K"], t["V"], t["dO"], g["tau"])
    for k, v in (("O", O), ("L", L), ("D", D)):
        np.testing.assert_allclose(v, np.array(g["forward"][k]), rtol=1e-13, atol=1e-14)
    out = fo.bob(*args(t), g["tau"])
    for k, v in out.items():
        np.testing.assert_allclose(v, np.array(g["bob"][k]), rtol=1e-12, atol=1e-13)
