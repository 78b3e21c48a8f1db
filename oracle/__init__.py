"""Plain fp64 CPU oracle for exact backward-over-backward (BoB) of softmax attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import or
call anything in this package.  The HIP library never routes through it, and it
shares no code, table or helper with the HIP path.

Everything here materialises the N x N score-shaped matrices and follows the
definitions written out on the pages, in float64:

* forward and first backward of softmax attention: "FlashAttention 的反向传播设计"
  (bjdmk.com.cn), section 一 (the forward formulas and the chain dV, dP, D, dS, dQ, dK);
* the BoB objective Phi = <dQ,U_Q> + <dK,U_K> + <dV,U_V> and its four outputs:
  "FlashBoB: I/O-Efficient Exact Backward-over-Backward for Softmax Attention"
  (papernotes.org notes), section "整体框架" (overall framework);
* the row scalars D, alpha, E, the projected-gradient matrix F and the hierarchical
  affine decomposition: the same page, "关键设计" item 1 and its correction equation.

Parity status of each function is listed in ``oracle/fbob_oracle.py``'s header.
"""

from .fbob_oracle import (  # noqa: F401
    attention_probs,
    forward,
    first_backward,
    first_backward_rows,
    first_backward_blocked,
    phi,
    bob,
    bob_affine,
    hvp_half_squared_output,
    bob_rows,
    bob_row_block,
    bob_blocked,
    bob_columns,
    row_scalars,
    bob_columns_at,
)
