"""FP8 x FP8 GEMM with FP32-accumulation semantics, dequant to BF16, output amax
(oracle; test infrastructure only).

What the method computes ([P2] §五: the custom fp8 linear op quantises both
operands, multiplies them, and divides the product by the product of the two
scales; the per-tensor FBGEMM row: FP8 inputs, FP32 accumulate, BF16 output):

    acc[i, j] = sum_k a(i, k) * b(k, j)          a, b: decoded, unscaled FP8 values
    y[i, j]   = bf16( acc[i, j] / fl32(s_a * s_b) )
    amax_y    = max |y|                           (of the stored BF16 output)

``op(.)`` is N (as stored) or T (stored transposed), giving the three products of
the training step ([P2] §三: forward Y = X W, dX = dY W^T, dW = X^T dY).

The oracle takes the plain definition: ``acc`` is the exact sum, computed as an
fp64 matrix product of the decoded values.  E4M3 x E4M3 products are multiples of
2**-18 below 2**17.6 in magnitude, so for K <= 2**14 every partial sum fits in
53 bits and the fp64 product is exact whatever the summation order.  Products
involving E5M2 are multiples of 2**-25 (or 2**-32 for E5M2 x E5M2) and may not be
exact; their fp64 error is at most K * 2**-53 * sum_k |a b|, far inside the
1e-5 * sum_k |a b| tolerance.  ``gemm_int_exact`` gives the exact result in
int64 for small K (used as a pin and for the tiny configuration).

The GPU's own fp32 summation order is the one part that is bounded, not pinned:
its error is at most about (K / k_inst) * 2**-24 * sum_k |a b| for an instruction
of depth k_inst, and typically far less.
"""

from __future__ import annotations

import numpy as np

from . import bf16
from .fp8 import E4M3, E5M2, decode

# Subnormal quantum of each format: every finite value is an integer multiple.
QUANTUM_LOG2 = {E4M3: -9, E5M2: -16}

OP_N = 0
OP_T = 1


def op_view(stored: np.ndarray, op: int) -> np.ndarray:
    """``op(stored)``: the array as stored (N) or its transpose (T)."""
    return stored if op == OP_N else stored.T


def gemm_exact(a_codes, fa, opa, b_codes, fb, opb):
    """Return ``(acc, sum_abs)`` in fp64: ``op(A) @ op(B)`` and ``|op(A)| @ |op(B)|``."""
    a = op_view(decode(a_codes, fa), opa)
    b = op_view(decode(b_codes, fb), opb)
    acc = a @ b
    sum_abs = np.abs(a) @ np.abs(b)
    return acc, sum_abs


def gemm_int_exact(a_codes, fa, opa, b_codes, fb, opb):
    """Exact product as an int64 matrix and its power-of-two exponent.

    Every finite value of a format is an integer multiple of its subnormal
    quantum, so ``value = n * 2**q``; the product sum is ``(sum n_a n_b) * 2**(qa+qb)``.
    Valid while the int64 sum cannot overflow (small K; checked).
    """
    qa, qb = QUANTUM_LOG2[fa], QUANTUM_LOG2[fb]
    ia = np.rint(np.ldexp(decode(a_codes, fa), -qa)).astype(np.int64)
    ib = np.rint(np.ldexp(decode(b_codes, fb), -qb)).astype(np.int64)
    a = op_view(ia, opa)
    b = op_view(ib, opb)
    bound = np.abs(a).max(initial=0) * np.abs(b).max(initial=0) * a.shape[1]
    assert bound < 2**62, "int64 exact GEMM would overflow"
    return a @ b, qa + qb


def dequant_scale(scale_a, scale_b) -> np.float32:
    """``fl32(s_a * s_b)``: the product of the two fp32 scales, one fp32 rounding."""
    return np.float32(np.float32(scale_a) * np.float32(scale_b))


def dequant_to_bf16(acc: np.ndarray, scale_a, scale_b) -> np.ndarray:
    """``bf16(acc / fl32(s_a s_b))`` as uint16 bits (division in fp64, one bf16 rounding)."""
    d = np.float64(dequant_scale(scale_a, scale_b))
    return bf16.round_to_bf16_vec(np.asarray(acc, dtype=np.float64) / d)


def output_amax(y_bits: np.ndarray) -> np.float32:
    """``max |y|`` of a BF16 output given as uint16 bits (0.0 if empty)."""
    y = bf16.widen(y_bits)
    if y.size == 0:
        return np.float32(0.0)
    return np.float32(np.max(np.abs(y.astype(np.float64))))
