"""Products of MX-quantized operands (CPU oracle, test infrastructure only).

[Blog], section "1. End-to-End Block-Scaled GEMM Fusion": S = Q K^T (and every
other product of the path) is taken from the MX operands, their E8M0 block
scales applied inside the product.  The plain definition, and the only
expected value this oracle produces, is the exact sum of the dequantized
products rounded once to fp32 (``matmul_exact``).

The pages leave open how precisely the block-scaled matrix unit adds its
products.  A unit that aligns products to a shared exponent before adding them
returns a result near, not at, the exact sum, so a product is several-valued:
every result within ``product_error_bound`` of the exact sum is admissible.
That bound is a tolerance reading, stated once here:

    eps_ij = (2**-10 + ceil(K / 16) * 2**-22) * sum_d 2**(e(a_id) + e(b_jd))

where e(x) is an element's binade exponent -- its E4M3 (or FP6 / FP4)
exponent, the format's minimum exponent for subnormals, plus the exponent of
its block's E8M0 scale -- zero elements contribute nothing, and K is the
contraction length.  Derivation: products aligned in groups to the group's
largest binade and truncated no further than 13 bits below it lose less than
2**(E - 10) per group of 8, which is at most 2**-10 times the group's share of
the sum above; the partial sums of 16 products are then added in fp32, each
addition off by at most 2**-24 of a partial sum, which is below 4 times the sum
above.  Products and sums below fp32's normal range may flush to zero, which adds
(K + 1) 2**-126 to the bound.  The attention parity checks
propagate this bound through the method's steps (oracle/attention.py,
``forward_head_bounds`` and ``backward_bounds``); whether the matrix
instruction itself stays inside it is measured on the GPU by the tests.
"""
from __future__ import annotations

import numpy as np

BOUND_REL = 2.0 ** -10           # the alignment part of the bound (per unit of sum_d 2^(e_a + e_b))


def fl32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def matmul_exact(a, b):
    """fl32(a @ b^T) for a [M, K], b [N, K]: the exact sum (float64 is exact for products of
    E4M3 values with nearby scales; for far-apart scales it is the exact sum to 2^-53) rounded
    once to fp32."""
    return fl32(np.asarray(a, np.float64) @ np.asarray(b, np.float64).T)


def magnitudes(values, exponents):
    """2**e per element (e: binade exponent incl. the block scale), 0 where the value is 0."""
    values = np.asarray(values, np.float64)
    return np.where(values != 0, np.exp2(np.asarray(exponents, np.float64)), 0.0)


def bound_rel(K: int) -> float:
    """eps per unit of sum_d 2^(e_a + e_b) for a contraction of length K."""
    return BOUND_REL + -(-K // 16) * 2.0 ** -22


def product_error_bound(amag, bmag):
    """eps [M, N] for a [M, K] @ b[N, K]^T from the operands' element magnitudes."""
    amag, bmag = np.asarray(amag, np.float64), np.asarray(bmag, np.float64)
    K = amag.shape[-1]
    return bound_rel(K) * (amag @ bmag.T) + (K + 1) * 2.0 ** -126
