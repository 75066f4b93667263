"""Finer-grained FP8 scaling: current (just-in-time) per-tensor and per-row
scales, and the GEMM dequant with one scale per row of A and per column of B
(oracle; test infrastructure only).

What the pages fix:

* [P2] "FP8 混合精度训练工程实践：从 H100 到大模型训练的范式跃迁", §"FBGEMM_GPU 底层优化":
  besides the per-tensor FP8 GEMM, per-token (a scale per row of the activation
  operand) and per-channel (a scale per output channel of the weight) modes,
  all with FP8 inputs, FP32 accumulation and BF16 output.
* [P3] "LLM FP8 微调上线生产实战" §参考资料 lists current scaling beside delayed
  scaling; [P2] §四 "动态缩放" derives the scale from the tensor's own amax.
* The scale formula is the delayed one of [P3] §核心原理 "Scale 决定数值是否进入
  可表示区间": (FP8_MAX / amax) / 2**margin, applied to the amax of the tensor
  (current, per tensor) or of each row (per token / per channel) that is being
  cast -- no history.

Readings:

* Per-row scaling of an [R, C] matrix: row r is cast with
  ``scale_from_window(amax(row r), fmt, margin)`` (:mod:`oracle.scaling`: one
  fp32 division, exact power-of-two margin, 1.0 when the amax is 0, infinite or
  NaN).  Per-channel scaling of a weight W [K, N] (a scale per output channel n)
  is per-row scaling of its transpose [N, K]; per-token scaling of X [M, K] is
  per-row scaling of X.
* The inverse scales ``fl32(1 / s)`` are what a cast hands to a GEMM kernel
  that multiplies; the oracle does not use them for the dequant.
* GEMM with scale vectors: the pages' fp8 linear op divides the FP32 product by
  the product of the two scales ([P2] §五); with one scale per row of op(A) and
  per column of op(B) that is ``y[i, j] = bf16(acc[i, j] / fl32(s_a[i] * s_b[j]))``,
  ``acc`` the exact sum of products of the decoded codes, the scale product one
  fp32 multiply (as the per-tensor dequant of :mod:`oracle.gemm`), the division
  in fp64 and one rounding to BF16.
"""

from __future__ import annotations

import numpy as np

from . import amax as oamax
from . import bf16
from . import fp8 as ofp8
from .scaling import scale_from_window


def inv_scale(s) -> np.float32:
    """``fl32(1 / s)``."""
    with np.errstate(divide="ignore"):
        return np.float32(np.float32(1.0) / np.float32(s))


def current_cast(x: np.ndarray, fmt: int, margin: int):
    """Per-tensor current scaling: scale from this tensor's own amax.
    Returns ``(codes, scale, amax, saturated)``."""
    x32 = np.asarray(x, dtype=np.float32)
    a = oamax.amax(x32)
    s = scale_from_window(a, fmt, margin)
    codes, sat = ofp8.cast(x32.ravel(), s, fmt)
    return codes.reshape(x32.shape), s, a, sat


def rowwise_cast(x: np.ndarray, fmt: int, margin: int):
    """Per-row current scaling of a 2-D array.  Returns ``(codes [R, C],
    scale [R], scale_inv [R], amax [R])``."""
    x32 = np.asarray(x, dtype=np.float32)
    R = x32.shape[0]
    codes = np.zeros(x32.shape, dtype=np.uint8)
    scale = np.zeros(R, dtype=np.float32)
    sinv = np.zeros(R, dtype=np.float32)
    amax = np.zeros(R, dtype=np.float32)
    for r in range(R):
        a = oamax.amax(x32[r])
        s = scale_from_window(a, fmt, margin)
        codes[r] = ofp8.cast(x32[r], s, fmt)[0]
        scale[r], sinv[r], amax[r] = s, inv_scale(s), a
    return codes, scale, sinv, amax


def dequant_vec_to_bf16(acc: np.ndarray, scale_a: np.ndarray, scale_b: np.ndarray) -> np.ndarray:
    """``bf16(acc[i, j] / fl32(s_a[i] * s_b[j]))`` as uint16 bits (the scale product
    one fp32 multiply, the division in fp64, one bf16 rounding)."""
    sa = np.asarray(scale_a, dtype=np.float32)
    sb = np.asarray(scale_b, dtype=np.float32)
    prod = (sa[:, None] * sb[None, :]).astype(np.float32)  # fl32 of each pair
    y = np.asarray(acc, dtype=np.float64) / prod.astype(np.float64)
    return bf16.round_to_bf16_vec(y)
