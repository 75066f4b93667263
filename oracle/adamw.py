"""AdamW step on FP32 master weights, and the FP8 cast of the updated weights
(oracle; test infrastructure only).

What the pages fix:

* [P1] "算子与编译器：FP8 训练与优化器 Kernel", §"FP8 训练主路径图": the master
  weights go through cast/scale to FP8 for the forward; the gradients go through
  unscale/clip into the fused optimizer, which writes the master weights back.
* [P1] §"Fused Optimizer 的意义" and §"优化器 kernel 的带宽账": one kernel reads the
  gradient, updates the first and second moments, applies the bias corrections
  and the weight decay and updates the parameter; AdamW reads and writes the
  parameter, the gradient, both moments and the master weight.
* [P2] "FP8 混合精度训练工程实践：从 H100 到大模型训练的范式跃迁", §"自动混合精度与 FP8
  的协同" (the precision flow of a training step): gradient un-scaling by the
  loss-scaling constant K, an FP32 AdamW step, then the updated weights cast to
  FP8 with scaling for the next forward; §三's precision table keeps the
  optimizer state in FP32.

The pages name AdamW without writing its update out.  The update taken here is
AdamW as published (Loshchilov & Hutter, "Decoupled Weight Decay
Regularization": the weight decay multiplies the weights and stays out of the
moments; moments and bias corrections as in Kingma & Ba, "Adam"), for step
t = 1, 2, ...::

    g  = grad * grad_scale                    (grad_scale: 1/K, times any clip factor)
    m  = beta1 * m + (1 - beta1) * g
    v  = beta2 * v + (1 - beta2) * g * g
    w  = w * (1 - lr * wd) - (lr / bc1) * m / (sqrt(v) / sqrt(bc2) + eps)
    bc1 = 1 - beta1^t,  bc2 = 1 - beta2^t

Precision (the pages fix FP32 for the step): every elementwise operation is one
correctly rounded fp32 operation, in exactly the order written in
:func:`adamw_update`; there is no fused multiply-add.  The per-step constants
(1 - lr*wd, 1 - beta1, 1 - beta2, lr/bc1, 1/sqrt(bc2)) are computed in float64
from the fp32 hyperparameters, with beta^t from the C library's ``pow``, and
rounded once to fp32.  Dividing by sqrt(bc2) is taken as a multiplication by
the rounded 1/sqrt(bc2) (the same value in exact arithmetic).

Skipped step: when the gradient holds an infinity or NaN (its amax, e.g. the
fused output amax of the dW product, is not finite), the update is skipped --
weights and moments stay as they are -- and the FP8 copy is made of the
unchanged weights ([P3] "第四步：建立 Amax 与低精度异常画像" counts skipped steps
among the gradient-health metrics; the loss-scaling practice of [P2] §四 skips
a step whose gradients overflowed).

The FP8 copy is :func:`oracle.fp8.cast` of the new weights with the delayed
scale of the weight tensor, and its amax is :func:`oracle.amax.amax` of them:
the same operations as casting the updated weights at the start of the next
forward.

Pins (tests/test_oracle_adamw.py): torch.optim.AdamW in float64 over many
steps; the first-step closed form w - lr*sign(g) (exact for dyadic settings);
zero gradients (pure decay); a constant gradient; an exact decimal evaluation
of one step; the skip rule.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from . import amax as oamax
from . import fp8 as ofp8

f32 = np.float32


@dataclass(frozen=True)
class StepConstants:
    beta1: np.float32
    beta2: np.float32
    one_minus_beta1: np.float32
    one_minus_beta2: np.float32
    eps: np.float32
    decay: np.float32         # 1 - lr * wd
    step_size: np.float32     # lr / (1 - beta1^t)
    inv_sqrt_bc2: np.float32  # 1 / sqrt(1 - beta2^t)
    grad_scale: np.float32


def step_constants(lr, beta1, beta2, eps, weight_decay, grad_scale, t: int) -> StepConstants:
    """The fp32 constants of step ``t`` (t >= 1) from fp32 hyperparameters."""
    if t < 1:
        raise ValueError("the step count starts at 1")
    lr, b1, b2, eps, wd, gs = (float(f32(x)) for x in (lr, beta1, beta2, eps, weight_decay,
                                                       grad_scale))
    bc1 = 1.0 - math.pow(b1, float(t))
    bc2 = 1.0 - math.pow(b2, float(t))
    return StepConstants(
        beta1=f32(b1), beta2=f32(b2),
        one_minus_beta1=f32(1.0 - b1), one_minus_beta2=f32(1.0 - b2),
        eps=f32(eps),
        decay=f32(1.0 - lr * wd),
        step_size=f32(lr / bc1),
        inv_sqrt_bc2=f32(1.0 / math.sqrt(bc2)),
        grad_scale=f32(gs),
    )


def adamw_update(w, grad, m, v, c: StepConstants, skip: bool = False):
    """One AdamW step, elementwise in fp32; returns new (w, m, v) as fp32 arrays.

    ``grad`` holds fp32 values (a BF16 gradient is widened exactly first)."""
    w = np.asarray(w, dtype=f32)
    m = np.asarray(m, dtype=f32)
    v = np.asarray(v, dtype=f32)
    if skip:
        return w.copy(), m.copy(), v.copy()
    g = np.asarray(grad, dtype=f32)
    with np.errstate(all="ignore"):
        g = f32(g * c.grad_scale)
        m1 = f32(f32(c.beta1 * m) + f32(c.one_minus_beta1 * g))
        v1 = f32(f32(c.beta2 * v) + f32(f32(c.one_minus_beta2 * g) * g))
        den = f32(f32(np.sqrt(v1) * c.inv_sqrt_bc2) + c.eps)
        u = f32(m1 / den)
        w1 = f32(f32(c.decay * w) - f32(c.step_size * u))
    return w1.astype(f32), m1.astype(f32), v1.astype(f32)


def grad_is_finite(grad) -> bool:
    """The skip test: the gradient's amax is finite (no NaN, no infinity)."""
    a = oamax.amax(np.asarray(grad, dtype=f32))
    return bool(np.isfinite(a))


def adamw_cast(w, grad, m, v, c: StepConstants, scale, fmt: int, skip_nonfinite: bool = True):
    """The fused step: AdamW, then the FP8 copy of the new weights.

    ``w`` is the [rows, cols] master weight.  Returns a dict with the new ``w``,
    ``m``, ``v``, the codes ``q`` [rows, cols] and ``q_t`` [cols, rows], the
    ``amax`` of the new weights, the saturation count ``sat`` and ``skipped``."""
    skip = skip_nonfinite and not grad_is_finite(grad)
    w1, m1, v1 = adamw_update(w, grad, m, v, c, skip)
    q, sat = ofp8.cast(w1, scale, fmt)
    q = q.reshape(w1.shape)
    return {"w": w1, "m": m1, "v": v1, "q": q, "q_t": q.T.copy() if q.ndim == 2 else None,
            "amax": oamax.amax(w1), "sat": int(sat), "skipped": skip}
