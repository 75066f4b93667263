"""One training step of the FP8 delayed-scaling Linear (oracle; test infrastructure only).

The step in the pages' order ([P1] §"FP8 训练主路径图": scale metadata feeds the
casts and the backward GEMMs; [P2] §三 and §四 "自动混合精度与 FP8 的协同"):

1. cast X and W to E4M3 with their current (delayed) scales, recording each
   tensor's amax;
2. forward ``Y = Xq Wq`` (NN), dequantised by ``1/(s_X s_W)`` to BF16, with the
   output amax;
3. cast dY to E5M2 (HYBRID recipe, [P3] §核心原理 "E4M3 与 E5M2 承担不同职责");
4. ``dX = dYq Wq^T`` (NT) and ``dW = Xq^T dYq`` (TN), reusing the forward FP8
   bytes of X and W and the scales they were cast with;
5. push each tensor's amax into its history and compute the scales for the
   next step ([P3] §核心原理 "Scale 决定..." and "Delayed Scaling 用历史换取稳定性").

W is stored ``[in, out]`` (K x N), so the forward product is NN.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import amax as amax_mod
from . import fp8, gemm
from .scaling import ScalingState


@dataclass
class GemmResult:
    acc: np.ndarray  # exact accumulator (fp64)
    sum_abs: np.ndarray  # sum_k |a b| (fp64), for the tolerance
    y_bits: np.ndarray  # bf16 output bits
    amax_y: np.float32
    scale_a: np.float32
    scale_b: np.float32


def run_gemm(a_codes, fa, opa, b_codes, fb, opb, s_a, s_b) -> GemmResult:
    acc, sum_abs = gemm.gemm_exact(a_codes, fa, opa, b_codes, fb, opb)
    y = gemm.dequant_to_bf16(acc, s_a, s_b)
    return GemmResult(acc, sum_abs, y, gemm.output_amax(y), np.float32(s_a), np.float32(s_b))


@dataclass
class CastResult:
    codes: np.ndarray
    amax: np.float32
    scale_used: np.float32
    sat: int


def run_cast(x_f32: np.ndarray, state: ScalingState) -> CastResult:
    codes, sat = fp8.cast(x_f32, state.scale, state.fmt)
    return CastResult(codes, amax_mod.amax(x_f32), np.float32(state.scale), sat)


def train_step(x, w, dy, states: dict, algo: int, margin: int, backward: bool = True):
    """One fwd(+bwd) step.  ``x [M,K]``, ``w [K,N]``, ``dy [M,N]`` are fp32 arrays
    (bf16 inputs already widened).  ``states`` maps "x", "w", "dy" to ScalingState
    and is updated in place.  Returns a dict of per-tensor casts and GEMM results.
    """
    out = {}
    cx = run_cast(x, states["x"])
    cw = run_cast(w, states["w"])
    out["cast_x"], out["cast_w"] = cx, cw
    out["y"] = run_gemm(cx.codes, states["x"].fmt, gemm.OP_N,
                        cw.codes, states["w"].fmt, gemm.OP_N, cx.scale_used, cw.scale_used)
    if backward:
        cdy = run_cast(dy, states["dy"])
        out["cast_dy"] = cdy
        out["dx"] = run_gemm(cdy.codes, states["dy"].fmt, gemm.OP_N,
                             cw.codes, states["w"].fmt, gemm.OP_T, cdy.scale_used, cw.scale_used)
        out["dw"] = run_gemm(cx.codes, states["x"].fmt, gemm.OP_T,
                             cdy.codes, states["dy"].fmt, gemm.OP_N, cx.scale_used, cdy.scale_used)
    states["x"].update(cx.amax, algo, margin)
    states["w"].update(cw.amax, algo, margin)
    if backward:
        states["dy"].update(out["cast_dy"].amax, algo, margin)
    return out
