"""MXFP8: FP8 elements in blocks of 32 that share one power-of-two scale
(oracle; test infrastructure only).

What the pages fix ([P2] "FP8 混合精度训练工程实践" §九 "展望：Blackwell 的
Microscaling 与未来"; §三 "为什么权重梯度用 E5M2？" names micro-scaling with E4M3 as
the alternative to pure E5M2 gradients):

* a group of 32 FP8 elements shares one 8-bit scale of type E8M0;
* each block is scaled locally, which gives the elements more effective
  precision than one scale for the whole tensor.

The pages' figure of the format is garbled (it calls the shared scale both an
E8M0 byte and an FP32 factor, and its bit count does not add up), so the rest
is taken from the OCP Microscaling Formats (MX) specification v1.0, which
defines MXFP8:

* E8M0: an unsigned 8-bit exponent with bias 127; code ``e`` is ``2**(e - 127)``
  for ``e`` in 0..254, code 255 is NaN.  There is no sign and no zero.
* A block ``V_0 .. V_31`` (consecutive along the contraction dimension) is
  encoded as the scale ``X = 2**E`` with
  ``E = floor(log2(max_i |V_i|)) - emax_elem`` (``emax_elem`` = the exponent of
  the element format's largest normal value: 8 for E4M3, since 448 = 1.75 * 2**8;
  15 for E5M2, since 57344 = 1.75 * 2**15), and the elements
  ``P_i = encode(V_i / X)``, the element format's round-to-nearest-even
  conversion, saturating at its largest finite value.  The largest element of a
  block lands in the format's top binade, or on its maximum when it would
  round above it (e.g. 1.9 * 2**8 > 448 for E4M3).
* The value of element i is ``X * decode(P_i)``; the dot product of two blocks
  is ``X_a * X_b * sum_i decode(Pa_i) * decode(Pb_i)``.

Readings where the specification leaves a choice to the implementation (each
one written in the design notes):

* ``E`` is clamped to the E8M0 range [-127, 127].  A block of zeros takes code 0
  (its elements are zero whatever the scale).
* A block holding a NaN or an infinity takes the NaN scale (code 255) and the
  NaN code 0x7F for every element: its values, and every dot product that uses
  them, are NaN.
* ``V_i / X`` is exact (a power-of-two division of an fp32 value, far from fp32
  overflow); a quotient below fp32's normal range encodes to zero either way.

The MX GEMM ``C = A B^T`` contracts along K with A [M, K] and B [N, K] both
blocked along K; the exact sum is taken in fp64 (error at most
``K * 2**-53 * sum |ab|``), and the BF16 output is ``bf16(acc)`` -- the scales
live in the blocks, there is no per-tensor factor.
"""

from __future__ import annotations

import math

import numpy as np

from . import amax as oamax
from . import bf16
from .fp8 import E4M3, E5M2, decode, encode

BLOCK = 32
E8M0_BIAS = 127
E8M0_NAN = 0xFF
EMAX_ELEM = {E4M3: 8, E5M2: 15}


def e8m0_value(code: int) -> float:
    """The value of an E8M0 scale code (NaN for 255)."""
    code = int(code)
    if code == E8M0_NAN:
        return math.nan
    return math.ldexp(1.0, code - E8M0_BIAS)


def block_scale_code(a: float, fmt: int) -> int:
    """E8M0 code of the shared scale of a block whose amax is ``a``."""
    a = float(a)
    if math.isnan(a) or math.isinf(a):
        return E8M0_NAN
    if a == 0.0:
        return 0
    m, e = math.frexp(a)          # a = m * 2**e with 0.5 <= m < 1
    floor_log2 = e - 1            # exact floor(log2(a))
    E = floor_log2 - EMAX_ELEM[fmt]
    E = max(-E8M0_BIAS, min(E8M0_BIAS, E))
    return E + E8M0_BIAS


def quantize_block(v: np.ndarray, fmt: int):
    """One block of (up to) 32 fp32 values -> (element codes, E8M0 code)."""
    v32 = np.asarray(v, dtype=np.float32)
    code = block_scale_code(oamax.amax(v32), fmt)
    if code == E8M0_NAN:
        return np.full(v32.shape, 0x7F, dtype=np.uint8), code
    q = np.ldexp(v32.astype(np.float64), -(code - E8M0_BIAS))
    with np.errstate(under="ignore"):
        return encode(q.astype(np.float32), fmt), code


def mx_cast(x: np.ndarray, fmt: int):
    """MX-quantize a 2-D array along its rows (blocks of 32 consecutive elements
    of a row; the row length must be a multiple of 32).  Returns ``(codes [R, C]
    uint8, scales [R, C/32] uint8)``.

    The same steps as :func:`quantize_block`, taken for all blocks at once with
    array operations (the tests check the two against each other)."""
    x32 = np.asarray(x, dtype=np.float32)
    R, C = x32.shape
    assert C % BLOCK == 0, "row length must be a multiple of 32"
    blocks = x32.reshape(R, C // BLOCK, BLOCK).astype(np.float64)
    special = ~np.isfinite(blocks).all(axis=-1)              # NaN or Inf in the block
    amax = np.where(special[..., None], 0.0, np.abs(blocks)).max(axis=-1)
    _, e = np.frexp(amax)                                     # amax = m * 2**e, 0.5 <= m < 1
    E = np.clip(e.astype(np.int64) - 1 - EMAX_ELEM[fmt], -E8M0_BIAS, E8M0_BIAS)
    scales = np.where(amax == 0.0, 0, E + E8M0_BIAS)
    scales = np.where(special, E8M0_NAN, scales).astype(np.uint8)
    shift = np.where(special, 0, scales.astype(np.int64) - E8M0_BIAS)
    q = np.ldexp(np.where(special[..., None], 0.0, blocks), -shift[..., None])
    q32 = q.astype(np.float32).ravel()
    codes = np.empty(q32.size, dtype=np.uint8)
    step = 1 << 20  # elementwise: encoded in pieces to keep numpy's temporaries small
    for i in range(0, q32.size, step):
        codes[i:i + step] = encode(q32[i:i + step], fmt)
    codes = codes.reshape(R, C)
    codes = np.where(np.repeat(special, BLOCK, axis=1), np.uint8(0x7F), codes).astype(np.uint8)
    return codes, scales


def mx_dequant(codes: np.ndarray, scales: np.ndarray, fmt: int) -> np.ndarray:
    """Values of an MX-quantized 2-D array in fp64: ``X(block) * decode(code)``."""
    vals = decode(codes, fmt)
    sv = np.array([e8m0_value(s) for s in np.asarray(scales).ravel()],
                  dtype=np.float64).reshape(np.shape(scales))
    return vals * np.repeat(sv, BLOCK, axis=1)


def mx_gemm_nt(a_codes, a_scales, fa, b_codes, b_scales, fb):
    """``(acc, sum_abs)`` in fp64 for ``C = A B^T``, A [M, K], B [N, K] MX-blocked
    along K."""
    a = mx_dequant(a_codes, a_scales, fa)
    b = mx_dequant(b_codes, b_scales, fb)
    with np.errstate(invalid="ignore", over="ignore"):
        return a @ b.T, np.abs(a) @ np.abs(b).T


def to_bf16(acc: np.ndarray) -> np.ndarray:
    """``bf16(acc)`` as uint16 bits (one rounding from fp64)."""
    return bf16.round_to_bf16_vec(np.asarray(acc, dtype=np.float64))
