"""bfloat16 helpers (oracle; test infrastructure only).

bfloat16 is IEEE binary32 with the low 16 fraction bits dropped: 1 sign,
8 exponent (bias 127), 7 fraction bits, so 8 significant bits.  The Linear's
output is BF16 ([P2] §五, the per-tensor FP8 GEMM row: FP32 accumulate, BF16
out; [P2] §三: forward output kept in 16-bit).
"""

from __future__ import annotations

import math

import numpy as np


def widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (round to nearest, ties to even); returns uint16 bits.

    Written from the definition: the quantum of the binade ``[2**e, 2**(e+1))``
    is ``2**(e-7)`` for normals and ``2**-133`` below ``2**-126``; the value is
    divided by the quantum, rounded with ``rint`` (ties to even) and multiplied
    back.  Results of magnitude ``>= 2**128`` are infinities.  NaN gives the quiet
    NaN 0x7FC0 with the input's sign bit.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    flat_v = v.ravel()
    flat_o = out.ravel()
    for i, x in enumerate(flat_v):
        flat_o[i] = _round_one(float(x))
    return out


def _round_one(x: float) -> int:
    if math.isnan(x):
        return 0x7FC0 | (0x8000 if math.copysign(1.0, x) < 0 else 0)
    sign = 0x8000 if math.copysign(1.0, x) < 0 else 0
    a = abs(x)
    if a == 0.0:
        return sign
    if math.isinf(a):
        return sign | 0x7F80
    _, e = math.frexp(a)  # a = m * 2**e with m in [0.5, 1)
    e -= 1  # a in [2**e, 2**(e+1))
    q_exp = max(e, -126) - 7
    r = float(np.rint(a / 2.0**q_exp)) * 2.0**q_exp
    if r >= 2.0**128:
        return sign | 0x7F80
    b = int(np.array([r], dtype=np.float32).view(np.uint32)[0])
    assert b & 0xFFFF == 0
    return sign | (b >> 16)


def round_to_bf16_vec(v: np.ndarray) -> np.ndarray:
    """Vectorised form of :func:`round_to_bf16` (same definition, numpy ufuncs).

    Used for large arrays; pinned against the scalar form in the tests.
    """
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v)
    a = np.abs(v)
    nan = np.isnan(a)
    inf = np.isinf(a)
    zero = a == 0.0
    safe = np.where(nan | inf | zero, 1.0, a)
    _, e = np.frexp(safe)
    e = e.astype(np.int64) - 1
    q_exp = np.maximum(e, -126) - 7
    r = np.rint(np.ldexp(safe, -q_exp)) * np.ldexp(1.0, q_exp)
    over = r >= 2.0**128
    r32 = np.where(over, 0.0, r).astype(np.float32)
    bits = (r32.view(np.uint32) >> 16).astype(np.uint32)
    bits = np.where(over | inf, 0x7F80, bits)
    bits = np.where(zero, 0, bits)
    bits = np.where(nan, 0x7FC0, bits)
    bits = bits | np.where(sign, 0x8000, 0)
    return bits.astype(np.uint16)
