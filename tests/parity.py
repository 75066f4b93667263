"""Helpers for GPU-vs-oracle parity tests (test infrastructure)."""

from __future__ import annotations

import numpy as np

from oracle import bf16 as obf16

# GEMM tolerances: the accumulator bound 1e-5 * sum_k |a_k b_k|; the BF16 output
# may also differ by one BF16 ulp of the reference (the device multiplies by the
# fp32 reciprocal of the scale product and rounds twice: fp32, then bf16).
ACC_REL = 1e-5


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (2**-133 below the normal range)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    safe = np.where(a > 0, a, 1.0)
    _, e = np.frexp(safe)
    e = np.maximum(e.astype(np.int64) - 1, -126)
    return np.where(a > 0, np.ldexp(1.0, e - 7), 2.0**-133)


def check_acc(acc_gpu: np.ndarray, acc_exact: np.ndarray, sum_abs: np.ndarray, what="",
              rel=ACC_REL):
    """|acc_gpu - acc_exact| <= rel * sum|ab| element by element (rel = 1e-5 by default)."""
    err = np.abs(acc_gpu.astype(np.float64) - acc_exact)
    bound = rel * sum_abs
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} elements out of tolerance; worst "
                           f"err {err[bad].max():.3e} bound {bound[bad].min():.3e}")


def check_bf16_out(y_gpu_bits: np.ndarray, acc_exact: np.ndarray, sum_abs: np.ndarray,
                   y_ref_bits: np.ndarray, d: float, what="", rel=ACC_REL):
    """|y_gpu - y_ref| <= ulp_bf16(y_ref) + rel * d * sum|ab| (rel = 1e-5 by default)."""
    yg = obf16.widen(y_gpu_bits).astype(np.float64)
    yr = obf16.widen(y_ref_bits).astype(np.float64)
    err = np.abs(yg - yr)
    bound = bf16_ulp(yr) + rel * d * sum_abs
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outputs out of tolerance; "
                           f"e.g. gpu {yg[bad][:3]} ref {yr[bad][:3]}")
    return int((yg != yr).sum())


def bf16_bits(t) -> np.ndarray:
    """uint16 bit patterns of a torch bf16 tensor (on any device)."""
    import torch

    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_bits(x) -> int:
    return int(np.array([x], dtype=np.float32).view(np.uint32)[0])
