"""Delayed scaling: amax-history ring, window reduction and scale formula
(oracle; test infrastructure only).

* Scale formula, [P3] §核心原理 "Scale 决定数值是否进入可表示区间":
  ``scale = (FP8_MAX / amax) / 2**margin`` with ``margin`` an integer exponent.
* History and delayed use, [P3] §核心原理 "Delayed Scaling 用历史换取稳定性"
  (the table of ``max`` and ``most_recent``) and [P2] §四 "动态缩放": the scale
  used by a step comes from amax values recorded at earlier steps, never from
  the step's own amax.
* Ring buffer, [P2] §四 "Delayed Scaling 的工程细节": the new amax is written at
  the cursor and the cursor advances modulo the history length.

Readings taken where the pages are silent or disagree:

* The window is the whole history of ``amax_history_len`` entries ([P2] §二 and
  [P3] §工程落地 第三步 give the length as a recipe field); [P2] §四's
  last-8-entries slice and its 1.2 factor / 1e4 cap / 0.5 smoothing are a
  different formula and are not used.
* Initial state: history all zeros, cursor 0, scale 1.0.
* Fallback: if the window value is 0, NaN or infinite, or the quotient is not
  finite and positive, the next scale is 1.0 ([P2] §四 "Delayed Scaling 的工程细节"
  sets the scale to 1.0 when the history maximum is not positive).
* Arithmetic: the quotient ``FP8_MAX / w`` is one correctly rounded fp32 division;
  the division by ``2**margin`` is an exact power-of-two rescaling in fp32
  (``ldexp``), rounded only if the result is subnormal.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .fp8 import fmt_max

ALGO_MAX = 0
ALGO_MOST_RECENT = 1


def scale_from_window(w: np.float32, fmt: int, margin: int) -> np.float32:
    """``(FP8_MAX / w) / 2**margin`` in fp32 with the 1.0 fallback."""
    w = np.float32(w)
    if not np.isfinite(w) or w <= 0:
        return np.float32(1.0)
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        q = np.float32(np.float32(fmt_max(fmt)) / w)  # fp32 IEEE division
        s = np.float32(np.ldexp(q, -int(margin)))
    if not np.isfinite(s) or s <= 0:
        return np.float32(1.0)
    return s


def window_value(history: np.ndarray, newest: np.float32, algo: int) -> np.float32:
    """Window reduction of [P3]'s table: ``max`` over the history, or ``most_recent``.

    NaN anywhere in the window makes the ``max`` result NaN (then the scale falls
    back to 1.0).
    """
    if algo == ALGO_MOST_RECENT:
        return np.float32(newest)
    h = np.asarray(history, dtype=np.float32)
    if np.isnan(h).any():
        return np.float32(np.nan)
    return np.float32(np.max(h))


@dataclass
class ScalingState:
    """Per-tensor delayed-scaling state: history ring, cursor and current scale."""

    fmt: int
    hist_len: int
    history: np.ndarray = field(default=None)
    cursor: int = 0
    scale: np.float32 = np.float32(1.0)

    def __post_init__(self):
        if self.history is None:
            self.history = np.zeros(self.hist_len, dtype=np.float32)

    def copy(self) -> "ScalingState":
        return ScalingState(self.fmt, self.hist_len, self.history.copy(), self.cursor,
                            np.float32(self.scale))

    def update(self, amax_t: np.float32, algo: int, margin: int) -> np.float32:
        """Record this step's amax and produce the scale for the next step."""
        self.history[self.cursor] = np.float32(amax_t)
        self.cursor = (self.cursor + 1) % self.hist_len
        w = window_value(self.history, np.float32(amax_t), algo)
        self.scale = scale_from_window(w, self.fmt, margin)
        return self.scale


def scale_exact_rational(fmt_max_value: float, w: float, margin: int):
    """The real number ``(FP8_MAX / w) / 2**margin`` as an exact fraction (for pins)."""
    from fractions import Fraction

    return Fraction(fmt_max_value) / Fraction(w) / Fraction(2) ** margin


def f32_ulp(x: float) -> float:
    """Unit in the last place of an fp32 normal number ``x`` (for pins)."""
    m, e = math.frexp(abs(x))
    return 2.0 ** (e - 24)
