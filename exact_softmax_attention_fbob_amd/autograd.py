"""Twice-differentiable softmax attention for torch autograd, on the library's kernels.

    from exact_softmax_attention_fbob_amd.autograd import attention
    O = attention(Q, K, V, tau=None, causal=False)      # O in Q's dtype
    O = attention(Q, K, V, fp32_row_sums=True)           # BoB with fp32 alpha, E'

* forward: ``fbob_forward_ws`` without dO (O and the log-partition L; a workspace from
  torch's allocator, so that small problems split their key sweeps);
* first backward (dQ, dK, dV for an upstream dO): ``fbob_backward_ws`` (a workspace
  from torch's allocator, so that small problems split their sweeps), which also
  returns the row scalar D;
* backward of that backward: for cotangents (U_Q, U_K, U_V) of (dQ, dK, dV) the
  vector-Jacobian product of the first backward is the gradient of
  Phi = <dQ,U_Q> + <dK,U_K> + <dV,U_V> with respect to (Q, K, V, dO), which is
  exactly the BoB of ``fbob_bob`` (FlashBoB notes, "整体框架").  This is what a
  Hessian-vector product through attention needs (the notes' Sophia-H
  integration: the gradient of <grad L, u> for a random direction u).  It runs
  through ``fbob_bob_ex`` with a workspace from torch's allocator, so problems too
  small to fill the GPU take the split schedule (the others run ``fbob_bob``);
  ``fp32_row_sums=True`` passes FBOB_FLAG_FP32_ROW_SUMS (bf16, d = 64: alpha and E'
  summed in fp32 from the unrounded products, for sharply peaked rows).

This module is an integration layer above the C ABI and uses torch autograd; the
arithmetic runs in the library's HIP kernels.  Conventions:

* Q, K, V are bf16 or fp32 GPU tensors [B, H, N, d] (K, V may have fewer heads,
  grouped-query attention).  Gradients are returned in the inputs' dtype; the
  kernels compute in fp32 and their fp32 outputs are rounded once at the end.
* O and L are saved from the forward and treated as functions of (Q, K, V): the
  BoB outputs already contain every derivative through O, L and D, so no separate
  gradient flows to them.
* Cotangents arriving in another dtype are rounded to the inputs' dtype before the
  BoB (the kernels take one storage type for all seven inputs).
* A third derivative is not provided (the BoB's own backward raises).
"""

from __future__ import annotations

import torch

from . import FLAG_FP32_ROW_SUMS as _FLAG_FP32_ROW_SUMS
from . import backward_ws as _backward
from . import bob_ex as _bob_ex
from . import forward_ws as _forward

__all__ = ["attention"]


def _contig(x):
    return x if x.is_contiguous() else x.contiguous()


class _AttentionBackward(torch.autograd.Function):
    """(Q, K, V, dO) -> (dQ, dK, dV); its backward is the BoB."""

    @staticmethod
    def forward(ctx, Q, K, V, dO, O, L, tau, causal, flags):
        g = _backward(Q, K, V, dO, O, L, tau, causal)
        ctx.save_for_backward(Q, K, V, dO, O, L, g["D"])
        ctx.tau, ctx.causal, ctx.flags = tau, causal, flags
        dt = Q.dtype
        return g["dQ"].to(dt), g["dK"].to(dt), g["dV"].to(dt)

    @staticmethod
    @torch.autograd.function.once_differentiable
    def backward(ctx, UQ, UK, UV):
        Q, K, V, dO, O, L, D = ctx.saved_tensors
        dt = Q.dtype

        def cot(u, like):
            return torch.zeros_like(like) if u is None else _contig(u.to(dt))

        r = _bob_ex(Q, K, V, dO, cot(UQ, Q), cot(UK, K), cot(UV, V), O, L, D, ctx.tau,
                    ctx.causal, flags=ctx.flags)
        return (r["dQt"].to(dt), r["dKt"].to(dt), r["dVt"].to(dt), r["ddOt"].to(dt),
                None, None, None, None, None)


class _Attention(torch.autograd.Function):
    """(Q, K, V) -> O = softmax(tau Q K^T) V."""

    @staticmethod
    def forward(ctx, Q, K, V, tau, causal, flags):
        O, L, _ = _forward(Q, K, V, None, tau, causal)
        ctx.save_for_backward(Q, K, V, O, L)
        ctx.tau, ctx.causal, ctx.flags = tau, causal, flags
        return O.to(Q.dtype) if Q.dtype != torch.float32 else O.clone()

    @staticmethod
    def backward(ctx, dO):
        Q, K, V, O, L = ctx.saved_tensors
        dO = _contig(dO.to(Q.dtype))
        dQ, dK, dV = _AttentionBackward.apply(Q, K, V, dO, O, L, ctx.tau, ctx.causal,
                                              ctx.flags)
        return dQ, dK, dV, None, None, None


def attention(Q, K, V, tau=None, causal=False, fp32_row_sums=False):
    """Softmax attention O = softmax_row(tau Q K^T) V, differentiable twice.

    ``tau`` defaults to 1/sqrt(d); ``causal`` masks key positions after the query's;
    ``fp32_row_sums`` selects the BoB's fp32 row-sum option for the second derivative.
    """
    d = Q.shape[-1]
    tau = float(1.0 / d ** 0.5 if tau is None else tau)
    flags = _FLAG_FP32_ROW_SUMS if fp32_row_sums else 0
    return _Attention.apply(_contig(Q), _contig(K), _contig(V), tau, bool(causal), flags)
