"""Host-side FP8 health monitoring over the counts of ``fp8ds_cast_health``.

The device pass (``fp8ds_cast_health``) gives, per cast, the input amax and the
counts of saturated values, NaN and infinite inputs, zero codes and top-binade
codes.  This module turns a series of them into decisions:

* :class:`AmaxSpikeDetector` -- [P2] §七 "陷阱 1：NaN/Inf 难以定位": once more than
  ten amax values of a tensor have been recorded, an amax above three times the
  mean of the nine values before it is a spike.
* :class:`HealthMonitor` -- the three alert levels of [P3] "第四步：建立 Amax 与
  低精度异常画像": *stop* on NaN or infinity, *degrade* (switch the layer to BF16)
  on saturation that persists over consecutive checks, *observe* on an amax
  spike or a jump of the share of zeros after quantization.  The pages give no
  numbers for "persistent" or "rising"; the thresholds are parameters, with the
  defaults stated below.
* :class:`PrecisionOverrides` -- [P3] "第五步：实现按层 BF16 回退": an auditable table
  module -> dtype, reason, step and the triggering metric.  The table records
  the decision; running that layer in BF16 belongs to the caller's model code.

Host logic only: no arithmetic of the cast or GEMM happens here.
"""

from __future__ import annotations

import math
from dataclasses import asdict, dataclass, field

OK, OBSERVE, DEGRADE, STOP = "ok", "observe", "degrade", "stop"
_RANK = {OK: 0, OBSERVE: 1, DEGRADE: 2, STOP: 3}


class AmaxSpikeDetector:
    """Per-tensor amax series with the spike rule of the pages' monitor."""

    def __init__(self, window: int = 9, factor: float = 3.0):
        self.window = window
        self.factor = factor
        self.series: dict[str, list[float]] = {}

    def push(self, name: str, amax: float) -> bool:
        """Record ``amax`` for ``name``; True when it is a spike."""
        s = self.series.setdefault(name, [])
        s.append(float(amax))
        if len(s) <= self.window + 1:
            return False
        prev = s[-self.window - 1:-1]
        mean = sum(prev) / len(prev)
        return math.isfinite(mean) and s[-1] > self.factor * mean


@dataclass
class Verdict:
    level: str
    reasons: list = field(default_factory=list)


class HealthMonitor:
    """Alert level of each check of a tensor's cast.

    ``sat_fraction`` (default 1e-3): share of saturated elements above which a
    check counts as saturated; ``sat_checks`` (default 3): consecutive saturated
    checks that make *degrade*; ``zero_jump`` (default 2.0): a share of zero codes
    above this factor times its mean over the previous ``window`` checks is an
    *observe*."""

    def __init__(self, window: int = 9, spike_factor: float = 3.0, sat_fraction: float = 1e-3,
                 sat_checks: int = 3, zero_jump: float = 2.0):
        self.spikes = AmaxSpikeDetector(window, spike_factor)
        self.window = window
        self.sat_fraction = sat_fraction
        self.sat_checks = sat_checks
        self.zero_jump = zero_jump
        self._sat_run: dict[str, int] = {}
        self._zero: dict[str, list[float]] = {}

    def check(self, name: str, amax: float, counts: dict, numel: int) -> Verdict:
        """``counts``: the names of ``HEALTH_NAMES`` (saturated, nan, inf, zero,
        near_max) of one cast of ``numel`` elements."""
        v = Verdict(OK)

        def raise_to(level, reason):
            if _RANK[level] > _RANK[v.level]:
                v.level = level
            v.reasons.append(reason)

        if counts["nan"] or counts["inf"]:
            raise_to(STOP, f"{counts['nan']} NaN and {counts['inf']} infinite inputs")
        n = max(int(numel), 1)
        sat = counts["saturated"] / n
        run = self._sat_run.get(name, 0) + 1 if sat > self.sat_fraction else 0
        self._sat_run[name] = run
        if run >= self.sat_checks:
            raise_to(DEGRADE, f"saturation {sat:.3g} over {run} consecutive checks")
        if self.spikes.push(name, amax):
            raise_to(OBSERVE, f"amax spike {amax:.4g}")
        zs = self._zero.setdefault(name, [])
        zf = counts["zero"] / n
        if len(zs) >= self.window:
            mean = sum(zs[-self.window:]) / self.window
            if zf > self.zero_jump * mean and zf > 0:
                raise_to(OBSERVE, f"zero share {zf:.3g} vs mean {mean:.3g}")
        zs.append(zf)
        return v


@dataclass
class Override:
    dtype: str
    reason: str
    activated_at_step: int
    metric: str = ""
    threshold: str = ""


class PrecisionOverrides:
    """Per-module precision overrides, kept as an auditable table."""

    def __init__(self):
        self.table: dict[str, Override] = {}

    def activate(self, module: str, step: int, reason: str, dtype: str = "bf16", metric: str = "",
                 threshold: str = "") -> Override:
        """Record a switch of ``module`` to ``dtype`` (the first activation of a
        module is kept: later calls do not rewrite its history)."""
        if module not in self.table:
            self.table[module] = Override(dtype, reason, int(step), metric, threshold)
        return self.table[module]

    def lookup(self, module: str):
        return self.table.get(module)

    def to_dict(self) -> dict:
        return {m: asdict(o) for m, o in self.table.items()}

    @classmethod
    def from_dict(cls, d: dict) -> "PrecisionOverrides":
        t = cls()
        for m, o in d.items():
            t.table[m] = Override(**o)
        return t
