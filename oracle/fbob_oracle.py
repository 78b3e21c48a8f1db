"""fp64 CPU oracle: softmax attention forward, first backward and backward-over-backward.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see ``oracle/__init__.py``).  Only tests,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may call it.

Every function works on ONE head: 2-D float64 arrays of shape (N, d), rows are
query/key positions.  Nothing is tiled or fused; N x N matrices are materialised.
The only deviation from "all at once" is ``bob_blocked``/``bob_columns``, which
evaluate the same row formulas on blocks of full-width rows (rows are independent,
so this only splits the sum over rows that forms dK~ and dV~).

Notation (pages: FlashBoB notes, "整体框架" and "关键设计" item 1; FlashAttention
backward blog, section 一):

    S = tau Q K^T,  P = softmax_row(S),  O = P V                      (forward)
    dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij = dO_i . O_i
    dS = P o (dP - D),  dQ = tau dS K,  dK = tau dS^T Q                 (first backward)
    Phi = <dQ,U_Q> + <dK,U_K> + <dV,U_V>                               (BoB objective)
    F = tau (U_Q K^T + Q U_K^T),  alpha_i = sum_j P_ij F_ij
    E_i = sum_j P_ij dP~_ij,  dP~ = dP~deg - alpha dP                  (affine structure)

Readings where the pages leave a step open (each is listed again in the design doc):

* r1  tau multiplies the scores (S = tau Q K^T); F carries its own tau; dQ~ and dK~
      carry tau because dQ and dK do.
* r2  L is the natural-log log-sum-exp of the scaled scores of a row.
* r3  D_i sums over ALL columns of the row (not over one column tile).
* r4  O, L, D are functions of (Q, K, V, dO); derivatives flow through them.
* r11 G = dO U_V^T enters dP~deg: <dV, U_V> = sum_ij P_ij G_ij, so the adjoint of P
      picks up G.  The pages do not print this term; it follows from the chain rule.
* The names B, R, Omega, ddO~deg and E~deg are printed without definitions.  With the
  printed corrections E = Edeg - alpha D, ddO~ = ddO~deg - alpha o and
  dQ~ = tau (Omega - alpha R - E B), the only alpha- and E-free split is
      Edeg = rowsum(P o dP~deg)      B = P K         R = (P o dP) K
      Omega = (P o dP~deg) K + dS U_K                ddO~deg = (P o F) V + P U_V
* Causal masking (the pages' benchmark setting, FlashBoB notes, experiments table)
  sets P_ij = 0 for j > i; all formulas above are unchanged.

Parity pins (tests/test_oracle_pins.py): central finite differences of Phi and of
<O, dO>, a symbolic (sympy) derivation on a 2x2 case, torch autograd double
backward in float64, linearity in U, the affine identities, exact invariants (among
them E_i = dO_i . ddO~_i - alpha_i D_i, which ties E to ddO~) and the U_Q = U_K = 0
and N = 1 special cases.  No function here is "parity unpinned".
"""

from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _rowsum(x):
    return x.sum(axis=1)


def _col(v):
    """A length-N row scalar as an (N, 1) column so it broadcasts along j."""
    return v[:, None]


def _scores(Qr, K, tau, row_ids=None, causal=False):
    """S = tau Q K^T for the rows ``Qr``; causal masking puts -inf above the diagonal."""
    S = tau * (Qr @ K.T)
    if causal:
        n_rows = Qr.shape[0]
        rows = np.arange(n_rows) if row_ids is None else np.asarray(row_ids)
        cols = np.arange(K.shape[0])
        S = np.where(cols[None, :] > rows[:, None], -np.inf, S)
    return S


def _logsumexp_rows(S):
    """L_i = log sum_j exp(S_ij), computed with the row maximum subtracted."""
    m = S.max(axis=1)
    return m + np.log(np.exp(S - _col(m)).sum(axis=1))


def attention_probs(Q, K, tau, causal=False, row_ids=None):
    """P = softmax_row(tau Q K^T) and its log-partition L (FlashAttention blog, section 一)."""
    Q, K = _f64(Q), _f64(K)
    S = _scores(Q, K, tau, row_ids, causal)
    L = _logsumexp_rows(S)
    P = np.exp(S - _col(L))
    return P, L


def forward(Q, K, V, dO, tau, causal=False):
    """O = P V, L = log-sum-exp of the scaled scores, D_i = dO_i . O_i.

    FlashAttention blog, section 一 (forward formulas); FlashBoB notes, "关键设计" 1
    (D_i = do_i^T o_i); "关键设计" 2 (the row state kept for recomputation).
    """
    V, dO = _f64(V), _f64(dO)
    P, L = attention_probs(Q, K, tau, causal)
    O = P @ V
    D = _rowsum(dO * O)
    return O, L, D


def first_backward(Q, K, V, dO, tau, causal=False):
    """dQ, dK, dV of softmax attention for the upstream gradient dO.

    FlashAttention blog, section 一: dV = P^T dO, dP = dO V^T, D_i = sum_j dP_ij P_ij,
    dS = P o (dP - D), dQ = tau dS K, dK = tau dS^T Q.
    """
    Q, K, V, dO = map(_f64, (Q, K, V, dO))
    P, _ = attention_probs(Q, K, tau, causal)
    dV = P.T @ dO
    dP = dO @ V.T
    D = _rowsum(P * dP)
    dS = P * (dP - _col(D))
    dQ = tau * (dS @ K)
    dK = tau * (dS.T @ Q)
    return dQ, dK, dV


def first_backward_rows(Q, K, V, dO, tau, rows, causal=False):
    """dQ and D for the selected query rows only (same formulas as ``first_backward``).

    Exact: row i of dQ needs only row i of Q and dO and all of K, V.
    """
    rows = np.asarray(rows)
    Q, K, V, dO = map(_f64, (Q, K, V, dO))
    P, _ = attention_probs(Q[rows], K, tau, causal, row_ids=rows)
    dP = dO[rows] @ V.T
    D = _rowsum(P * dP)
    dS = P * (dP - _col(D))
    return dict(dQ=tau * (dS @ K), D=D)


def first_backward_blocked(Q, K, V, dO, tau, causal=False, row_block=1024):
    """dQ, dK, dV, D of ``first_backward`` with rows taken ``row_block`` at a time.

    Rows are independent; dK and dV are sums over rows, accumulated block by block.
    Memory O(row_block N) instead of O(N^2).
    """
    Q, K, V, dO = map(_f64, (Q, K, V, dO))
    N, d = Q.shape
    dQ, D = np.empty((N, d)), np.empty(N)
    dK, dV = np.zeros((N, d)), np.zeros((N, d))
    for r0 in range(0, N, row_block):
        rows = np.arange(r0, min(N, r0 + row_block))
        P, _ = attention_probs(Q[rows], K, tau, causal, row_ids=rows)
        dP = dO[rows] @ V.T
        Dr = _rowsum(P * dP)
        dS = P * (dP - _col(Dr))
        dQ[rows] = tau * (dS @ K)
        D[rows] = Dr
        dK += tau * (dS.T @ Q[rows])
        dV += P.T @ dO[rows]
    return dict(dQ=dQ, dK=dK, dV=dV, D=D)


def phi(Q, K, V, dO, UQ, UK, UV, tau, causal=False):
    """Phi = <dQ,U_Q> + <dK,U_K> + <dV,U_V> (FlashBoB notes, "整体框架")."""
    dQ, dK, dV = first_backward(Q, K, V, dO, tau, causal)
    return float(np.sum(dQ * _f64(UQ)) + np.sum(dK * _f64(UK)) + np.sum(dV * _f64(UV)))


def _row_chain(Qr, dOr, UQr, K, V, UK, UV, tau, causal=False, row_ids=None):
    """Reverse-mode chain of Phi for a set of full-width rows (every column j).

    Everything a row needs is row-local once its full width is seen: the forward
    row (P, O, L, D), the first backward row (dP, dS), and the adjoints below.

      alpha  = rowsum(P o F)                      FlashBoB notes, "关键设计" 1
      ddP    = P o (F - alpha)      adjoint of dP, including the path through D
      dPt    = F o (dP - D) + G - alpha dP        adjoint of P (affine form)
      E      = rowsum(P o dPt)                    FlashBoB notes, "关键设计" 1
      dSt    = P o (dPt - E)        adjoint of S through the softmax
      dQt_i  = tau (dSt K + dS U_K)_i
      ddOt_i = (ddP V + P U_V)_i
    """
    S = _scores(Qr, K, tau, row_ids, causal)
    L = _logsumexp_rows(S)
    P = np.exp(S - _col(L))
    O = P @ V
    D = _rowsum(dOr * O)
    dP = dOr @ V.T
    F = tau * (UQr @ K.T + Qr @ UK.T)
    G = dOr @ UV.T
    dS = P * (dP - _col(D))
    alpha = _rowsum(P * F)
    ddP = P * (F - _col(alpha))
    dPt = F * (dP - _col(D)) + G - _col(alpha) * dP
    E = _rowsum(P * dPt)
    dSt = P * (dPt - _col(E))
    dQt = tau * (dSt @ K + dS @ UK)
    ddOt = ddP @ V + P @ UV
    return dict(P=P, L=L, O=O, D=D, dS=dS, dSt=dSt, ddP=ddP,
                alpha=alpha, E=E, dQt=dQt, ddOt=ddOt)


def bob(Q, K, V, dO, UQ, UK, UV, tau, causal=False):
    """Exact BoB outputs (dQ~, dK~, dV~, ddO~, alpha, E) for one head, all at once.

    The column outputs are the transposed products of the same row adjoints:
      dK~ = tau (dS~^T Q + dS^T U_Q),   dV~ = ddP^T dO.
    Returns a dict with keys dQt, dKt, dVt, ddOt, alpha, E (float64).
    """
    Q, K, V, dO, UQ, UK, UV = map(_f64, (Q, K, V, dO, UQ, UK, UV))
    r = _row_chain(Q, dO, UQ, K, V, UK, UV, tau, causal)
    dKt = tau * (r["dSt"].T @ Q + r["dS"].T @ UQ)
    dVt = r["ddP"].T @ dO
    return dict(dQt=r["dQt"], dKt=dKt, dVt=dVt, ddOt=r["ddOt"],
                alpha=r["alpha"], E=r["E"])


def hvp_half_squared_output(Q, K, V, UQ, UK, UV, tau, causal=False):
    """Hessian-vector product of loss = 0.5 ||O||^2 in the direction (U_Q, U_K, U_V).

    The use the FlashBoB notes give for BoB (Sophia-H curvature estimates: the
    gradient of <grad loss, u>).  Here the upstream gradient dO = O depends on
    (Q, K, V) as well, so the product is the BoB at dO = O plus the first backward
    applied to the BoB's ddO~ (the path through dO).
    """
    Q, K, V, UQ, UK, UV = map(_f64, (Q, K, V, UQ, UK, UV))
    O, _, _ = forward(Q, K, V, np.zeros_like(Q), tau, causal)
    b = bob(Q, K, V, O, UQ, UK, UV, tau, causal)
    dQ2, dK2, dV2 = first_backward(Q, K, V, b["ddOt"], tau, causal)
    return dict(dQ=b["dQt"] + dQ2, dK=b["dKt"] + dK2, dV=b["dVt"] + dV2)


def bob_affine(Q, K, V, dO, UQ, UK, UV, tau, causal=False):
    """Row outputs through the hierarchical affine decomposition.

    FlashBoB notes, "关键设计" item 1: five alpha-free accumulators plus alpha, then
      E = Edeg - alpha D,  ddO~ = ddO~deg - alpha o,  dQ~ = tau (Omega - alpha R - E B).
    The accumulator definitions are the reading stated in this module's header.
    Returns dQt, ddOt, alpha, E and the accumulators themselves.
    """
    Q, K, V, dO, UQ, UK, UV = map(_f64, (Q, K, V, dO, UQ, UK, UV))
    P, L = attention_probs(Q, K, tau, causal)
    O = P @ V
    D = _rowsum(dO * O)
    dP = dO @ V.T
    F = tau * (UQ @ K.T + Q @ UK.T)
    G = dO @ UV.T
    dS = P * (dP - _col(D))
    dPt_deg = F * (dP - _col(D)) + G          # dP~ before the alpha correction
    alpha = _rowsum(P * F)
    E_deg = _rowsum(P * dPt_deg)
    B = P @ K
    R = (P * dP) @ K
    Omega = (P * dPt_deg) @ K + dS @ UK
    ddO_deg = (P * F) @ V + P @ UV
    E = E_deg - alpha * D
    ddOt = ddO_deg - _col(alpha) * O
    dQt = tau * (Omega - _col(alpha) * R - _col(E) * B)
    return dict(dQt=dQt, ddOt=ddOt, alpha=alpha, E=E, E_deg=E_deg, B=B, R=R,
                Omega=Omega, ddO_deg=ddO_deg)


def bob_rows(Q, K, V, dO, UQ, UK, UV, tau, rows, causal=False):
    """Row outputs (dQ~, ddO~, alpha, E, and L, D, O) for the selected rows only.

    Exact: each row's outputs depend only on that row of Q, dO, U_Q and on all of
    K, V, U_K, U_V.  Cost O(len(rows) N d).
    """
    rows = np.asarray(rows)
    Q, K, V, dO, UQ, UK, UV = map(_f64, (Q, K, V, dO, UQ, UK, UV))
    r = _row_chain(Q[rows], dO[rows], UQ[rows], K, V, UK, UV, tau, causal, rows)
    return dict(dQt=r["dQt"], ddOt=r["ddOt"], alpha=r["alpha"], E=r["E"],
                L=r["L"], D=r["D"], O=r["O"])


def bob_row_block(Q, K, V, dO, UQ, UK, UV, tau, rows, causal=False):
    """One block of full-width rows: its row outputs and its share of dK~, dV~.

    dK~ and dV~ are sums over rows; summing the returned dKt_part/dVt_part over a
    partition of the rows gives the full column outputs.
    """
    rows = np.asarray(rows)
    Q, K, V, dO, UQ, UK, UV = map(_f64, (Q, K, V, dO, UQ, UK, UV))
    r = _row_chain(Q[rows], dO[rows], UQ[rows], K, V, UK, UV, tau, causal, rows)
    return dict(dQt=r["dQt"], ddOt=r["ddOt"], alpha=r["alpha"], E=r["E"],
                dKt_part=tau * (r["dSt"].T @ Q[rows] + r["dS"].T @ UQ[rows]),
                dVt_part=r["ddP"].T @ dO[rows])


def bob_blocked(Q, K, V, dO, UQ, UK, UV, tau, causal=False, row_block=1024):
    """All BoB outputs for one head, rows taken ``row_block`` at a time.

    Same formulas as ``bob``; dK~ and dV~ are sums over rows, accumulated block by
    block.  Memory O(row_block N) instead of O(N^2).
    """
    Q, K, V, dO, UQ, UK, UV = map(_f64, (Q, K, V, dO, UQ, UK, UV))
    N, d = Q.shape
    out = dict(dQt=np.empty((N, d)), ddOt=np.empty((N, d)),
               dKt=np.zeros((N, d)), dVt=np.zeros((N, d)),
               alpha=np.empty(N), E=np.empty(N))
    for r0 in range(0, N, row_block):
        rows = np.arange(r0, min(N, r0 + row_block))
        r = bob_row_block(Q, K, V, dO, UQ, UK, UV, tau, rows, causal)
        for k in ("dQt", "ddOt", "alpha", "E"):
            out[k][rows] = r[k]
        out["dKt"] += r["dKt_part"]
        out["dVt"] += r["dVt_part"]
    return out


def bob_columns(Q, K, V, dO, UQ, UK, UV, tau, cols, causal=False, row_block=1024):
    """Column outputs dK~, dV~ for the selected key positions only.

    Every row contributes to every column, so all rows' row scalars are computed
    (a full pass over rows, O(N^2 d)), but only the selected columns are kept.
    """
    cols = np.asarray(cols)
    Q, K, V, dO, UQ, UK, UV = map(_f64, (Q, K, V, dO, UQ, UK, UV))
    N, d = Q.shape
    dKt = np.zeros((len(cols), d))
    dVt = np.zeros((len(cols), d))
    for r0 in range(0, N, row_block):
        rows = np.arange(r0, min(N, r0 + row_block))
        r = _row_chain(Q[rows], dO[rows], UQ[rows], K, V, UK, UV, tau, causal, rows)
        dKt += tau * (r["dSt"][:, cols].T @ Q[rows] + r["dS"][:, cols].T @ UQ[rows])
        dVt += r["ddP"][:, cols].T @ dO[rows]
    return dict(dKt=dKt, dVt=dVt)


def row_scalars(Q, K, V, dO, UQ, UK, UV, tau, rows, causal=False):
    """L, D, alpha and E of the selected full-width rows, from the score-shaped
    blocks S, dP, F, G alone (no d-wide contraction of P-shaped matrices).

    The same definitions as ``_row_chain`` (FlashAttention blog, section 一, for L
    and D = sum_j P_ij dP_ij over all columns; FlashBoB notes, "关键设计" 1, for
    alpha and E = sum_j P_ij dP~_ij), evaluated for ``rows`` only.  Cost
    10 len(rows) N d: five products with every key.  These four per-row numbers
    are all that a column of dK~ or dV~ needs from a row (``bob_columns_at``).
    """
    rows = np.asarray(rows)
    Q, K, V, dO, UQ, UK, UV = map(_f64, (Q, K, V, dO, UQ, UK, UV))
    Qr, dOr, UQr = Q[rows], dO[rows], UQ[rows]
    S = _scores(Qr, K, tau, rows, causal)
    L = _logsumexp_rows(S)
    P = np.exp(S - _col(L))
    dP = dOr @ V.T
    D = _rowsum(P * dP)
    F = tau * (UQr @ K.T + Qr @ UK.T)
    G = dOr @ UV.T
    alpha = _rowsum(P * F)
    dPt = F * (dP - _col(D)) + G - _col(alpha) * dP
    E = _rowsum(P * dPt)
    return dict(L=L, D=D, alpha=alpha, E=E)


def bob_columns_at(Q, K, V, dO, UQ, UK, UV, tau, cols, L, D, alpha, E, causal=False):
    """dK~ and dV~ at the selected key positions, given every row's L, D, alpha, E.

    Column j needs, for every row i, P_ij, dP_ij, F_ij and G_ij (products of row i
    with key j) and the row's four scalars; then, as in ``bob``,
      dS = P o (dP - D),  dP~ = F o (dP - D) + G - alpha dP,  dS~ = P o (dP~ - E),
      ddP = P o (F - alpha),  dK~_j = tau sum_i (dS~_ij Q_i + dS_ij U_Q,i),
      dV~_j = sum_i ddP_ij dO_i.
    The row scalars must be the oracle's own (``row_scalars`` over all rows).
    Cost O(N len(cols) d).
    """
    cols = np.asarray(cols)
    Q, K, V, dO, UQ, UK, UV = map(_f64, (Q, K, V, dO, UQ, UK, UV))
    L, D, alpha, E = map(_f64, (L, D, alpha, E))
    N = Q.shape[0]
    Kc, Vc, UKc, UVc = K[cols], V[cols], UK[cols], UV[cols]
    S = tau * (Q @ Kc.T)                                   # (N, c): rows i, columns j
    P = np.exp(S - _col(L))
    if causal:
        P = np.where(cols[None, :] > np.arange(N)[:, None], 0.0, P)
    dP = dO @ Vc.T
    F = tau * (UQ @ Kc.T + Q @ UKc.T)
    G = dO @ UVc.T
    dS = P * (dP - _col(D))
    dPt = F * (dP - _col(D)) + G - _col(alpha) * dP
    dSt = P * (dPt - _col(E))
    ddP = P * (F - _col(alpha))
    dKt = tau * (dSt.T @ Q + dS.T @ UQ)
    dVt = ddP.T @ dO
    return dict(dKt=dKt, dVt=dVt)
